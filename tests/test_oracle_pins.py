"""The CPU oracle against its pins (see oracle_pins.py for what pins what)."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def o():
    return oracle.get()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(o, pin):
    pin(o)


def test_thread_count_does_not_change_results(o):
    import numpy as np
    import synth
    W = synth.weights((99, 33, 1024), 33, 1024)
    X = synth.activations((99, 5), 5, 1024)
    Xq = o.quantize_q8_1(X)
    o.set_threads(1)
    y1 = o.gemm_q8_1(W, Xq, 1024)
    o.set_threads(0)
    y8 = o.gemm_q8_1(W, Xq, 1024)
    assert np.array_equal(y1, y8)
