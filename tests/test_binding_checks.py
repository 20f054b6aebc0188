"""Host-only checks of the Python binding: every tensor's shape, byte size
and device is checked before its pointer reaches the library (the C ABI sees
raw pointers only, so a wrong-sized tensor would otherwise become an
out-of-bounds access on the GPU).  No GPU is needed: the checks run before
anything touches a device, so CPU and meta tensors exercise them."""
import pytest
import torch

import iq4_xs_q8_amd as iq

M, N, K = 4, 64, 512
WB = K // 256 * 136


def _t(shape, dtype=torch.float32, device="cpu"):
    return torch.zeros(shape, dtype=dtype, device=device)


def test_gemm_shapes():
    W, X = _t((N, WB), torch.uint8), _t((M, K))
    with pytest.raises(ValueError, match="W must have shape"):
        iq.gemm(_t((N, WB + 8), torch.uint8), X)
    with pytest.raises(ValueError, match="Y must have shape"):
        iq.gemm(W, X, out=_t((M, N + 1)))
    with pytest.raises(ValueError, match="2-D"):
        iq.gemm(W, _t((M * K,)))
    with pytest.raises(ValueError, match="multiple of 256"):
        iq.gemm(W, _t((M, 300)))
    # well-formed CPU tensors get past the shape checks and stop at the device check
    with pytest.raises(TypeError, match="CUDA"):
        iq.gemm(W, X)


def test_gemm_q8_1_shapes():
    W = _t((N, WB), torch.uint8)
    with pytest.raises(ValueError, match="Xq must have shape"):
        iq.gemm_q8_1(W, _t((M, K // 32 * 36 - 4), torch.uint8), K)
    with pytest.raises(ValueError, match="Y must have shape"):
        iq.gemm_q8_1(W, _t((M, K // 32 * 36), torch.uint8), K, out=_t((N, M)))
    with pytest.raises(ValueError, match="W must have shape"):
        iq.gemm_q8_1(W, _t((M, K // 32 * 36), torch.uint8), 2 * K)


def test_prepared_activation_sizes():
    need = iq.act_bytes(M, K)
    with pytest.raises(ValueError, match="act holds"):
        iq.prepare_act(_t((M, K)), out=_t((need - 1,), torch.uint8))
    with pytest.raises(ValueError, match="act holds"):
        iq.gemm_act(_t((N, WB), torch.uint8), _t((need - 16,), torch.uint8), M, K)
    with pytest.raises(ValueError, match="Y must have shape"):
        iq.gemm_act(_t((N, WB), torch.uint8), _t((need,), torch.uint8), M, K, out=_t((M, N - 1)))


def test_quantize_and_dequantize_shapes():
    with pytest.raises(ValueError, match="Xq must have shape"):
        iq.quantize_q8_1(_t((M, K)), out=_t((M, K // 32 * 36 + 1), torch.uint8))
    with pytest.raises(ValueError, match="Wb must have shape"):
        iq.dequantize_bf16(_t((N, WB), torch.uint8), K, out=_t((N, K - 32), torch.bfloat16))


def test_group_shapes():
    Ws = [_t((N, WB), torch.uint8), _t((2 * N, WB), torch.uint8)]
    X = _t((M, K))
    with pytest.raises(ValueError, match=r"Y\[1\] must have shape"):
        iq.gemm_group(Ws, X, [_t((M, N)), _t((M, N))])
    with pytest.raises(ValueError, match="W must have shape"):
        iq.gemm_group([Ws[0], _t((N, WB - 136), torch.uint8)], X)
    with pytest.raises(ValueError, match="one output per weight matrix"):
        iq.gemm_group(Ws, X, [_t((M, N))])


def test_tensors_on_different_devices():
    W = _t((N, WB), torch.uint8, device="meta")
    with pytest.raises(ValueError, match="different devices"):
        iq.gemm(W, _t((M, K)))
    with pytest.raises(ValueError, match="different devices"):
        iq.gemm_group([W], _t((M, K)), [_t((M, N))])
