// abi.hip -- the extern "C" entry points of libiq4xs.so (declared and
// documented in include/iq4xs.h): validation, initialisation, the device
// check, stream-ordered scratch, and the launch sequence of each path.
//
// "SGLang MoE port thread" (lcz.me/post/31556), section on the torch bridge:
// the stream arrives as a plain handle and no framework header is included.
// "V100TPS engine log" (agent-report.daedalus.work/V100TPS/engine.html),
// section on the end-to-end concurrency test: a getenv on every matmul was
// suspected of costing time, so the environment is read once here.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <mutex>
#include <sstream>
#include <string>
#include <vector>

#include "common.hpp"
#include "dispatch.hpp"
#include "iq4xs.h"

using namespace iq4xs;

const TuneOverride &iq4xs::tune_override()
{
    static const TuneOverride t = [] {
        TuneOverride o;
        const char *m = getenv("IQ4XS_MMV");
        if (m && m[0] == '0')
            o.mmv = 0;
        const char *t = getenv("IQ4XS_TILE");
        if (t && t[0] == '0')
            o.tile = 0;
        return o;
    }();
    return t;
}

namespace {
int cus_of_current_device();
}

int iq4xs::device_cus() { return cus_of_current_device(); }

namespace {

thread_local std::string g_err;

struct Config {
    bool log = false;
    bool allow_bf16 = false;
    int init_status = IQ4XS_OK;
};

std::once_flag g_once;
Config g_cfg;
std::mutex g_mu;                       // guards g_table and g_dev_ok
Table g_table;
std::vector<int> g_dev_ok;             // per device: 0 unknown, 1 gfx950, -1 other
std::vector<int> g_dev_cus;            // per device: compute units (0 unknown)

int fail(int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    if (g_cfg.log)
        fprintf(stderr, "[iq4xs] error %d: %s\n", code, buf);
    return code;
}

int load_table_text(const std::string &text, const char *what)
{
    Table t;
    std::string err;
    if (!parse_table(text, &t, &err))
        return fail(IQ4XS_ETABLE, "%s: %s", what, err.c_str());
    std::lock_guard<std::mutex> lk(g_mu);
    g_table = t;
    return IQ4XS_OK;
}

int load_table_file(const char *path)
{
    std::ifstream f(path);
    if (!f)
        return fail(IQ4XS_ETABLE, "cannot read dispatch table %s", path);
    std::stringstream ss;
    ss << f.rdbuf();
    return load_table_text(ss.str(), path);
}

void do_init()
{
    const char *v = getenv("IQ4XS_LOG");
    g_cfg.log = v && v[0] == '1';
    v = getenv("IQ4XS_ALLOW_BF16");
    g_cfg.allow_bf16 = v && v[0] == '1';
    int st = load_table_text(default_table_text(), "built-in dispatch table");
    const char *path = getenv("IQ4XS_DISPATCH_TABLE");
    if (st == IQ4XS_OK && path && path[0])
        st = load_table_file(path);
    g_cfg.init_status = st;
}

int ensure_init()
{
    std::call_once(g_once, do_init);
    return g_cfg.init_status;
}

// The current device must be a gfx950 and the table must be for it.
int check_device()
{
    // (the built-in table, at least, is loaded by the first call of any entry
    // point, whichever path it names)
    ensure_init();
    int dev = -1, count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count < 1) {
        (void)hipGetLastError();
        return fail(IQ4XS_EDEVICE, "no HIP device");
    }
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= count) {
        (void)hipGetLastError();
        return fail(IQ4XS_EDEVICE, "no current HIP device");
    }
    std::lock_guard<std::mutex> lk(g_mu);
    if ((int)g_dev_ok.size() < count)
        g_dev_ok.resize(count, 0);
    if (g_dev_ok[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return fail(IQ4XS_EDEVICE, "cannot query device %d", dev);
        }
        g_dev_ok[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
        if ((int)g_dev_cus.size() < count)
            g_dev_cus.resize(count, 0);
        g_dev_cus[dev] = prop.multiProcessorCount;
        if (g_dev_ok[dev] == 1) {
            // keep freed scratch in the pool so steady-state calls do not
            // return memory to the driver
            hipMemPool_t pool;
            if (hipDeviceGetDefaultMemPool(&pool, dev) == hipSuccess) {
                uint64_t thr = UINT64_MAX;
                (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &thr);
            }
            (void)hipGetLastError();
        }
    }
    if (g_dev_ok[dev] != 1)
        return fail(IQ4XS_EDEVICE, "device %d is not gfx950", dev);
    if (g_table.arch != "gfx950")
        return fail(IQ4XS_ETABLE, "dispatch table is for %s, device is gfx950", g_table.arch.c_str());
    return IQ4XS_OK;
}

int cus_of_current_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return 256;
    }
    std::lock_guard<std::mutex> lk(g_mu);
    return dev >= 0 && dev < (int)g_dev_cus.size() && g_dev_cus[dev] > 0 ? g_dev_cus[dev] : 256;
}

// A call that asked for AUTO runs on a device (checked): the table's bands
// hold for it only if they were measured on as many compute units (a table
// that names no count applies to any).
int check_auto_cus(int requested_path)
{
    if (requested_path != IQ4XS_PATH_AUTO)
        return IQ4XS_OK;
    const int cus = cus_of_current_device();
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_table.cus > 0 && g_table.cus != cus)
        return fail(IQ4XS_ETABLE, "dispatch table measured on %d compute units, the device has %d", g_table.cus,
                    cus);
    return IQ4XS_OK;
}

// The scratch of iq4xs_gemm_noalloc.  In host code `scratch` names a host-side
// stand-in, not the device copy: the device address of the current device's
// copy is looked up once per device (with that device current) and only that
// address is ever passed to kernels.
static_assert(IQ4XS_STATIC_SCRATCH_BYTES % 256 == 0, "whole 256-byte units");
static __device__ __align__(256) char scratch[IQ4XS_STATIC_SCRATCH_BYTES];
std::vector<void *> g_scratch;         // per device: address of its copy of `scratch`

int static_scratch(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return fail(IQ4XS_EDEVICE, "no current HIP device");
    }
    std::lock_guard<std::mutex> lk(g_mu);
    if ((int)g_scratch.size() <= dev)
        g_scratch.resize(dev + 1, nullptr);
    if (g_scratch[dev] == nullptr) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return fail(IQ4XS_ELAUNCH, "static scratch of device %d: %s", dev, hipGetErrorString(e));
        }
        if ((uintptr_t)p % 256 != 0)
            return fail(IQ4XS_ELAUNCH, "static scratch of device %d is not 256-byte aligned", dev);
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return IQ4XS_OK;
}

bool mul_ok(int64_t a, int64_t b, int64_t *out)
{
    if (a < 0 || b < 0)
        return false;
    if (a != 0 && b > INT64_MAX / 4 / a)
        return false;
    *out = a * b;
    return true;
}

// M, N >= 1, K a positive multiple of 256, and every buffer size far from overflow.
int check_dims(int64_t M, int64_t N, int64_t K)
{
    int64_t t;
    if (M < 1 || N < 1 || K < QK || K % QK)
        return fail(IQ4XS_EINVAL, "need M >= 1, N >= 1, K a positive multiple of 256 (M=%lld N=%lld K=%lld)",
                    (long long)M, (long long)N, (long long)K);
    if (M > (1LL << 31) || N > (1LL << 31) || K > (1LL << 31) || !mul_ok(M, K, &t) ||
        !mul_ok(N, K, &t) || !mul_ok(M, N, &t) || !mul_ok(t, 4, &t))
        return fail(IQ4XS_EINVAL, "sizes overflow");
    // the matmul kernels address the activation planes (1.125 bytes per
    // element, rows padded to 4) with 32-bit offsets
    if (round_up(M, MPAD) * K / 8 * 9 >= (1LL << 31))
        return fail(IQ4XS_EINVAL, "M*K too large: the activation planes must stay below 2 GiB (M=%lld K=%lld)",
                    (long long)M, (long long)K);
    return IQ4XS_OK;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

struct Scratch {
    void *p = nullptr;
    hipStream_t s = nullptr;
    ~Scratch()
    {
        if (p)
            (void)hipFreeAsync(p, s);
    }
};

int launch_err(hipError_t e, const char *what)
{
    if (e == hipSuccess)
        return IQ4XS_OK;
    (void)hipGetLastError();
    return fail(IQ4XS_ELAUNCH, "%s: %s", what, hipGetErrorString(e));
}

int resolve_path(int path, int64_t M, int64_t N, int64_t K, int *out, int fmt = FMT_IQ4_XS)
{
    if (path < 0 || path >= IQ4XS_NUM_PATHS)
        return fail(IQ4XS_EINVAL, "unknown path %d", path);
    if (fmt != FMT_IQ4_XS && (path == IQ4XS_PATH_DEQ_BF16 || path == IQ4XS_PATH_BF16X3))
        return fail(IQ4XS_EPATH, "the bf16 paths read IQ4_XS weights only");
    ensure_init();
    if (path == IQ4XS_PATH_AUTO) {
        int st = ensure_init();
        if (st != IQ4XS_OK)
            return fail(st, "dispatch table not loaded: %s", g_err.c_str());
        {
            std::lock_guard<std::mutex> lk(g_mu);
            // (the bands were measured on IQ4_XS; for the 32-weight formats the
            // same GEMV / MMQ kernels run, and bf16 bands do not apply)
            path = table_lookup(g_table, M, N, K, g_cfg.allow_bf16 && fmt == FMT_IQ4_XS, fmt == FMT_IQ4_XS);
        }
        if (!path)
            return fail(IQ4XS_EPATH, "no dispatch band covers M=%lld N=%lld K=%lld", (long long)M,
                        (long long)N, (long long)K);
    }
    if (path == IQ4XS_PATH_GEMV && M > GEMV_MAX_M)
        return fail(IQ4XS_EPATH, "GEMV path handles M <= %d (M=%lld)", GEMV_MAX_M, (long long)M);
    if (g_cfg.log)
        fprintf(stderr, "[iq4xs] M=%lld N=%lld K=%lld -> %s\n", (long long)M, (long long)N,
                (long long)K, path_name(path));
    *out = path;
    return IQ4XS_OK;
}

// Scratch a path needs: activation planes (+ the split-K partial sums of
// MMQ), or for the bf16 paths the hi/lo bf16 activation planes.
size_t workspace_need(int path, int64_t M, int64_t N, int64_t K, int fmt = FMT_IQ4_XS)
{
    if (path == IQ4XS_PATH_GEMV || path == IQ4XS_PATH_MMQ)
        return (size_t)round_up((int64_t)xplanes_bytes(M, K), 256) +
               (path == IQ4XS_PATH_MMQ ? mmq_plan(M, N, K, fmt).workspace_bytes : 0);
    return fused_xs_bytes(M, K);
}

// Common tail of the gemm entry points.  Exactly one of X (fp32) and Xq (Q8_1
// blocks) is non-null.  With ws == nullptr the scratch comes from the
// device's default pool, stream-ordered; otherwise ws (ws_bytes, 256-byte
// aligned) is used and nothing is allocated.
int run_gemm(const void *W, const float *X, const void *Xq, float *Y, int64_t M, int64_t N, int64_t K,
             int path, void *ws, size_t ws_bytes, hipStream_t s, int fmt = FMT_IQ4_XS)
{
    const int requested = path;
    int st = resolve_path(path, M, N, K, &path, fmt);
    if (st != IQ4XS_OK)
        return st;
    if (path == IQ4XS_PATH_MMQ && !mmq_plan(M, N, K, fmt).ok)
        return fail(IQ4XS_EPATH, "no MMQ kernel takes a %s matrix of %lld x %lld (2 GiB or more)",
                    fmt == FMT_IQ4_NL ? "IQ4_NL" : "Q4_0", (long long)N, (long long)K);
    const size_t need = workspace_need(path, M, N, K, fmt);
    if (ws != nullptr) {
        if (!aligned(ws, 256))
            return fail(IQ4XS_EALIGN, "workspace must be 256-byte aligned");
        if (ws_bytes < need)
            return fail(IQ4XS_EINVAL, "workspace of %zu bytes, %zu needed", ws_bytes, need);
        if (overlaps(ws, ws_bytes, Y, (size_t)(M * N * 4)) ||
            overlaps(ws, ws_bytes, W, (size_t)(N * (K / QK) * sblk_bytes(fmt))) ||
            (X && overlaps(ws, ws_bytes, X, (size_t)(M * K * 4))) ||
            (Xq && overlaps(ws, ws_bytes, Xq, (size_t)(M * (K / SB) * XBLK))))
            return fail(IQ4XS_EINVAL, "workspace overlaps W, X or Y");
    }
    if ((st = check_device()) != IQ4XS_OK || (st = check_auto_cus(requested)) != IQ4XS_OK)
        return st;

    Scratch scr;
    scr.s = s;
    char *base = (char *)ws;
    if (base == nullptr) {
        if (hipMallocAsync(&scr.p, need, s) != hipSuccess) {
            (void)hipGetLastError();
            scr.p = nullptr;
            return fail(IQ4XS_ENOMEM, "scratch of %zu bytes", need);
        }
        base = (char *)scr.p;
    }
    if (path == IQ4XS_PATH_GEMV || path == IQ4XS_PATH_MMQ) {
        const size_t pbytes = (size_t)round_up((int64_t)xplanes_bytes(M, K), 256);
        const XPlanes xp = xplanes_at(base, M, K);
        // a matmul that adds partial tiles into Y gets them zeroed by the
        // quantizer: the shared tiles of the tile kernel, all of Y (M <= 32)
        // for the streaming kernel
        const MmqPlan mp = path == IQ4XS_PATH_MMQ ? mmq_plan(M, N, K, fmt) : MmqPlan();
        const bool zero = path == IQ4XS_PATH_MMQ && mp.zero_y;
        ZeroList zl;
        if (zero && mp.tile) {
            zl.tiles = mmqt_zero_tiles(mp.tp, M, N, K, Y);
        } else if (zero) {
            zl.p[0] = Y;
            zl.n[0] = M * N;
            zl.count = 1;
        }
        hipError_t e = X ? launch_quantize(X, nullptr, &xp, M, K, s, zl)
                         : launch_q8_1_convert(Xq, &xp, M, K, s, zl);
        if ((st = launch_err(e, "quantize")) != IQ4XS_OK)
            return st;
        e = path == IQ4XS_PATH_GEMV ? launch_gemv(W, xp, Y, N, s, fmt)
                                    : launch_mmq(W, xp, Y, N, base + pbytes, zero, s, fmt);
        return launch_err(e, path_name(path));
    }
    // BF16X3 and DEQ_BF16: the fused kernels, from the hi/lo activation planes
    // (DEQ_BF16 reads the hi parts only: the plain bf16 formulation)
    if (std::max(fused_grid(M, N), deq_grid(M, N)) > INT32_MAX || fused_xs_bytes(M, K) >= (size_t)INT32_MAX)
        return fail(IQ4XS_EPATH, "the bf16 paths take fewer than 2^31 workgroups and activation planes "
                    "below 2 GiB (M=%lld N=%lld K=%lld)", (long long)M, (long long)N, (long long)K);
    XSplit xsp;
    xsp.p = (uint16_t *)base;
    xsp.Ms = fused_ms(M);
    const hipError_t e = X ? launch_quantize(X, nullptr, nullptr, M, K, s, nullptr, 0, &xsp)
                           : launch_q8_1_convert(Xq, nullptr, M, K, s, nullptr, 0, &xsp);
    if ((st = launch_err(e, "quantize")) != IQ4XS_OK)
        return st;
    if (path == IQ4XS_PATH_BF16X3)
        return launch_err(launch_fused_x3(W, xsp.p, Y, M, N, K, s), "gemm_x3");
    return launch_err(launch_fused_deq(W, xsp.p, Y, M, N, K, s), "gemm_deq");
}

}  // namespace

extern "C" {

int iq4xs_weight_bytes(int64_t N, int64_t K, size_t *out)
{
    if (!out)
        return fail(IQ4XS_EINVAL, "null output pointer");
    if (N < 1 || K < QK || K % QK || N > (1LL << 40) || K > (1LL << 40))
        return fail(IQ4XS_EINVAL, "need N >= 1 and K a positive multiple of 256");
    *out = (size_t)N * (size_t)(K / QK) * WBLK;
    return IQ4XS_OK;
}

int iq4xs_q8_1_bytes(int64_t M, int64_t K, size_t *out)
{
    if (!out)
        return fail(IQ4XS_EINVAL, "null output pointer");
    if (M < 1 || K < SB || K % SB || M > (1LL << 40) || K > (1LL << 40))
        return fail(IQ4XS_EINVAL, "need M >= 1 and K a positive multiple of 32");
    *out = (size_t)M * (size_t)(K / SB) * XBLK;
    return IQ4XS_OK;
}

int iq4xs_init(void) { return ensure_init(); }

int iq4xs_quantize_q8_1(const float *X, void *Xq, int64_t M, int64_t K, void *stream)
{
    if (!X || !Xq)
        return fail(IQ4XS_EINVAL, "null pointer");
    if (M < 1 || K < SB || K % SB || M > (1LL << 31) || K > (1LL << 31) || M * K > (1LL << 60) / 4)
        return fail(IQ4XS_EINVAL, "need M >= 1 and K a positive multiple of 32");
    if (!aligned(X, 16) || !aligned(Xq, 4))
        return fail(IQ4XS_EALIGN, "X must be 16-byte and Xq 4-byte aligned");
    if (overlaps(X, (size_t)(M * K * 4), Xq, (size_t)(M * (K / SB) * XBLK)))
        return fail(IQ4XS_EINVAL, "X and Xq overlap");
    ensure_init();
    int st = check_device();
    if (st != IQ4XS_OK)
        return st;
    return launch_err(launch_quantize(X, Xq, nullptr, M, K, (hipStream_t)stream), "quantize");
}

int iq4xs_gemm_path(const void *W, const float *X, float *Y, int64_t M, int64_t N, int64_t K,
                    int path, void *stream)
{
    if (!W || !X || !Y)
        return fail(IQ4XS_EINVAL, "null pointer");
    int st = check_dims(M, N, K);
    if (st != IQ4XS_OK)
        return st;
    if (!aligned(W, 16) || !aligned(X, 16) || !aligned(Y, 16))
        return fail(IQ4XS_EALIGN, "W, X and Y must be 16-byte aligned");
    const size_t yb = (size_t)(M * N * 4);
    if (overlaps(Y, yb, W, (size_t)(N * (K / QK) * WBLK)) || overlaps(Y, yb, X, (size_t)(M * K * 4)))
        return fail(IQ4XS_EINVAL, "Y overlaps an input");
    return run_gemm(W, X, nullptr, Y, M, N, K, path, nullptr, 0, (hipStream_t)stream);
}

int iq4xs_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int path, size_t *out)
{
    if (!out)
        return fail(IQ4XS_EINVAL, "null output pointer");
    int st = check_dims(M, N, K);
    if (st != IQ4XS_OK)
        return st;
    if ((st = resolve_path(path, M, N, K, &path)) != IQ4XS_OK)
        return st;
    *out = workspace_need(path, M, N, K);
    return IQ4XS_OK;
}

int iq4xs_gemm_ws(const void *W, const float *X, float *Y, int64_t M, int64_t N, int64_t K, int path,
                  void *workspace, size_t workspace_bytes, void *stream)
{
    if (!W || !X || !Y || !workspace)
        return fail(IQ4XS_EINVAL, "null pointer");
    int st = check_dims(M, N, K);
    if (st != IQ4XS_OK)
        return st;
    if (!aligned(W, 16) || !aligned(X, 16) || !aligned(Y, 16))
        return fail(IQ4XS_EALIGN, "W, X and Y must be 16-byte aligned");
    const size_t yb = (size_t)(M * N * 4);
    if (overlaps(Y, yb, W, (size_t)(N * (K / QK) * WBLK)) || overlaps(Y, yb, X, (size_t)(M * K * 4)))
        return fail(IQ4XS_EINVAL, "Y overlaps an input");
    return run_gemm(W, X, nullptr, Y, M, N, K, path, workspace, workspace_bytes, (hipStream_t)stream);
}

int iq4xs_gemm_noalloc(const void *W, const float *X, float *Y, int64_t M, int64_t N, int64_t K, int path,
                       void *stream)
{
    if (!W || !X || !Y)
        return fail(IQ4XS_EINVAL, "null pointer");
    int st = check_dims(M, N, K);
    if (st != IQ4XS_OK)
        return st;
    if (!aligned(W, 16) || !aligned(X, 16) || !aligned(Y, 16))
        return fail(IQ4XS_EALIGN, "W, X and Y must be 16-byte aligned");
    const size_t yb = (size_t)(M * N * 4);
    if (overlaps(Y, yb, W, (size_t)(N * (K / QK) * WBLK)) || overlaps(Y, yb, X, (size_t)(M * K * 4)))
        return fail(IQ4XS_EINVAL, "Y overlaps an input");
    int resolved = 0;
    if ((st = resolve_path(path, M, N, K, &resolved)) != IQ4XS_OK)
        return st;
    const size_t need = workspace_need(resolved, M, N, K);
    if (need > IQ4XS_STATIC_SCRATCH_BYTES)
        return fail(IQ4XS_EINVAL, "M=%lld N=%lld K=%lld on %s needs %zu bytes of scratch; the static scratch holds %u",
                    (long long)M, (long long)N, (long long)K, path_name(resolved), need,
                    (unsigned)IQ4XS_STATIC_SCRATCH_BYTES);
    if ((st = check_device()) != IQ4XS_OK)
        return st;
    void *ws = nullptr;
    if ((st = static_scratch(&ws)) != IQ4XS_OK)
        return st;
    return run_gemm(W, X, nullptr, Y, M, N, K, path, ws, IQ4XS_STATIC_SCRATCH_BYTES, (hipStream_t)stream);
}

static bool fmt_ok(int fmt) { return fmt == FMT_IQ4_XS || fmt == FMT_IQ4_NL || fmt == FMT_Q4_0; }

int iq4xs_weight_bytes_fmt(int fmt, int64_t N, int64_t K, size_t *out)
{
    if (!out)
        return fail(IQ4XS_EINVAL, "null output pointer");
    if (!fmt_ok(fmt))
        return fail(IQ4XS_EINVAL, "unknown weight format %d", fmt);
    if (N < 1 || K < QK || K % QK || N > (1LL << 40) || K > (1LL << 40))
        return fail(IQ4XS_EINVAL, "need N >= 1 and K a positive multiple of 256");
    *out = (size_t)N * (size_t)(K / QK) * sblk_bytes(fmt);
    return IQ4XS_OK;
}

int iq4xs_gemm_fmt_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K, int path, size_t *out)
{
    if (!out)
        return fail(IQ4XS_EINVAL, "null output pointer");
    if (!fmt_ok(fmt))
        return fail(IQ4XS_EINVAL, "unknown weight format %d", fmt);
    int st = check_dims(M, N, K);
    if (st != IQ4XS_OK)
        return st;
    if ((st = resolve_path(path, M, N, K, &path, fmt)) != IQ4XS_OK)
        return st;
    *out = workspace_need(path, M, N, K, fmt);
    return IQ4XS_OK;
}

int iq4xs_gemm_fmt(int fmt, const void *W, const float *X, float *Y, int64_t M, int64_t N, int64_t K, int path,
                   void *workspace, size_t workspace_bytes, void *stream)
{
    if (!fmt_ok(fmt))
        return fail(IQ4XS_EINVAL, "unknown weight format %d", fmt);
    if (!W || !X || !Y)
        return fail(IQ4XS_EINVAL, "null pointer");
    int st = check_dims(M, N, K);
    if (st != IQ4XS_OK)
        return st;
    if (!aligned(W, 16) || !aligned(X, 16) || !aligned(Y, 16))
        return fail(IQ4XS_EALIGN, "W, X and Y must be 16-byte aligned");
    const size_t yb = (size_t)(M * N * 4);
    if (overlaps(Y, yb, W, (size_t)(N * (K / QK) * sblk_bytes(fmt))) || overlaps(Y, yb, X, (size_t)(M * K * 4)))
        return fail(IQ4XS_EINVAL, "Y overlaps an input");
    return run_gemm(W, X, nullptr, Y, M, N, K, path, workspace, workspace_bytes, (hipStream_t)stream, fmt);
}

int iq4xs_gemm(const void *W, const float *X, float *Y, int64_t M, int64_t N, int64_t K, void *stream)
{
    return iq4xs_gemm_path(W, X, Y, M, N, K, IQ4XS_PATH_AUTO, stream);
}

int iq4xs_gemm_q8_1(const void *W, const void *Xq, float *Y, int64_t M, int64_t N, int64_t K,
                    int path, void *stream)
{
    if (!W || !Xq || !Y)
        return fail(IQ4XS_EINVAL, "null pointer");
    int st = check_dims(M, N, K);
    if (st != IQ4XS_OK)
        return st;
    if (!aligned(W, 16) || !aligned(Y, 16) || !aligned(Xq, 4))
        return fail(IQ4XS_EALIGN, "W and Y must be 16-byte and Xq 4-byte aligned");
    const size_t yb = (size_t)(M * N * 4);
    if (overlaps(Y, yb, W, (size_t)(N * (K / QK) * WBLK)) ||
        overlaps(Y, yb, Xq, (size_t)(M * (K / SB) * XBLK)))
        return fail(IQ4XS_EINVAL, "Y overlaps an input");
    return run_gemm(W, nullptr, Xq, Y, M, N, K, path, nullptr, 0, (hipStream_t)stream);
}

int iq4xs_dequantize_bf16(const void *W, void *Wb, int64_t N, int64_t K, void *stream)
{
    if (!W || !Wb)
        return fail(IQ4XS_EINVAL, "null pointer");
    int st = check_dims(1, N, K);
    if (st != IQ4XS_OK)
        return st;
    if (!aligned(W, 16) || !aligned(Wb, 16))
        return fail(IQ4XS_EALIGN, "W and Wb must be 16-byte aligned");
    if (overlaps(Wb, (size_t)(N * K * 2), W, (size_t)(N * (K / QK) * WBLK)))
        return fail(IQ4XS_EINVAL, "W and Wb overlap");
    ensure_init();
    if ((st = check_device()) != IQ4XS_OK)
        return st;
    return launch_err(launch_dequant_bf16(W, (uint16_t *)Wb, N, K, (hipStream_t)stream), "dequant_bf16");
}

int iq4xs_act_bytes(int64_t M, int64_t K, size_t *out)
{
    if (!out)
        return fail(IQ4XS_EINVAL, "null output pointer");
    int st = check_dims(M, 1, K);
    if (st != IQ4XS_OK)
        return st;
    *out = xplanes_bytes(M, K);
    return IQ4XS_OK;
}

int iq4xs_prepare_act(const float *X, void *act, int64_t M, int64_t K, void *stream)
{
    if (!X || !act)
        return fail(IQ4XS_EINVAL, "null pointer");
    int st = check_dims(M, 1, K);
    if (st != IQ4XS_OK)
        return st;
    if (!aligned(X, 16) || !aligned(act, 256))
        return fail(IQ4XS_EALIGN, "X must be 16-byte and act 256-byte aligned");
    if (overlaps(X, (size_t)(M * K * 4), act, xplanes_bytes(M, K)))
        return fail(IQ4XS_EINVAL, "X and act overlap");
    ensure_init();
    if ((st = check_device()) != IQ4XS_OK)
        return st;
    const XPlanes xp = xplanes_at(act, M, K);
    return launch_err(launch_quantize(X, nullptr, &xp, M, K, (hipStream_t)stream), "quantize");
}

// The path a prepared-activation matmul runs: GEMV or MMQ.  The table's bf16
// bands do not apply to prepared activations: the integer kernel takes those
// shapes.
static int resolve_act_path(int path, int64_t M, int64_t N, int64_t K, int *out)
{
    const int requested = path;
    int st = resolve_path(path, M, N, K, &path);
    if (st != IQ4XS_OK)
        return st;
    if (requested == IQ4XS_PATH_AUTO && path == IQ4XS_PATH_BF16X3)
        path = IQ4XS_PATH_MMQ;
    if (path == IQ4XS_PATH_DEQ_BF16 || path == IQ4XS_PATH_BF16X3)
        return fail(IQ4XS_EPATH, "prepared activations feed the GEMV and MMQ paths only");
    *out = path;
    return IQ4XS_OK;
}

// Partial-result scratch of a prepared-activation matmul (the tile kernel
// with few tiles, the K-split fallback); 0 for every other shape.
static size_t act_workspace_need(int path, int64_t M, int64_t N, int64_t K)
{
    return path == IQ4XS_PATH_MMQ ? mmq_plan(M, N, K).workspace_bytes : 0;
}

// Common body of iq4xs_gemm_act (caller_ws false: scratch from the device's
// pool, stream-ordered) and iq4xs_gemm_act_ws (ws, ws_bytes from the caller;
// nothing allocated).
static int run_gemm_act(const void *W, const void *act, float *Y, int64_t M, int64_t N, int64_t K, int path,
                        bool caller_ws, void *ws, size_t ws_bytes, hipStream_t s)
{
    const bool y_zeroed = (path & IQ4XS_Y_ZEROED) != 0;
    path &= ~IQ4XS_Y_ZEROED;
    if (!W || !act || !Y)
        return fail(IQ4XS_EINVAL, "null pointer");
    int st = check_dims(M, N, K);
    if (st != IQ4XS_OK)
        return st;
    if (!aligned(W, 16) || !aligned(Y, 16) || !aligned(act, 256))
        return fail(IQ4XS_EALIGN, "W and Y must be 16-byte and act 256-byte aligned");
    const size_t yb = (size_t)(M * N * 4), wb = (size_t)(N * (K / QK) * WBLK), ab = xplanes_bytes(M, K);
    if (overlaps(Y, yb, W, wb) || overlaps(Y, yb, act, ab))
        return fail(IQ4XS_EINVAL, "Y overlaps an input");
    const int requested = path;
    if ((st = resolve_act_path(path, M, N, K, &path)) != IQ4XS_OK)
        return st;
    const size_t need = act_workspace_need(path, M, N, K);
    if (caller_ws && need > 0) {
        if (ws == nullptr)
            return fail(IQ4XS_EINVAL, "null workspace, %zu bytes needed", need);
        if (!aligned(ws, 256))
            return fail(IQ4XS_EALIGN, "workspace must be 256-byte aligned");
        if (ws_bytes < need)
            return fail(IQ4XS_EINVAL, "workspace of %zu bytes, %zu needed", ws_bytes, need);
        if (overlaps(ws, ws_bytes, Y, yb) || overlaps(ws, ws_bytes, W, wb) || overlaps(ws, ws_bytes, act, ab))
            return fail(IQ4XS_EINVAL, "workspace overlaps W, act or Y");
    }
    if ((st = check_device()) != IQ4XS_OK || (st = check_auto_cus(requested)) != IQ4XS_OK)
        return st;
    const XPlanes xp = xplanes_at((void *)act, M, K);
    if (path == IQ4XS_PATH_GEMV)
        return launch_err(launch_gemv(W, xp, Y, N, s), path_name(path));
    Scratch scr;   // partial-sum workspace when the shape splits K over workgroups
    scr.s = s;
    void *p = need > 0 ? ws : nullptr;
    if (!caller_ws && need > 0) {
        if (hipMallocAsync(&scr.p, need, s) != hipSuccess) {
            (void)hipGetLastError();
            scr.p = nullptr;
            return fail(IQ4XS_ENOMEM, "workspace of %zu bytes", need);
        }
        p = scr.p;
    }
    return launch_err(launch_mmq(W, xp, Y, N, p, y_zeroed, s), path_name(path));
}

int iq4xs_gemm_act(const void *W, const void *act, float *Y, int64_t M, int64_t N, int64_t K,
                   int path, void *stream)
{
    return run_gemm_act(W, act, Y, M, N, K, path, false, nullptr, 0, (hipStream_t)stream);
}

int iq4xs_gemm_act_workspace_bytes(int64_t M, int64_t N, int64_t K, int path, size_t *out)
{
    if (!out)
        return fail(IQ4XS_EINVAL, "null output pointer");
    int st = check_dims(M, N, K);
    if (st != IQ4XS_OK)
        return st;
    if ((st = resolve_act_path(path & ~IQ4XS_Y_ZEROED, M, N, K, &path)) != IQ4XS_OK)
        return st;
    *out = act_workspace_need(path, M, N, K);
    return IQ4XS_OK;
}

int iq4xs_gemm_act_ws(const void *W, const void *act, float *Y, int64_t M, int64_t N, int64_t K, int path,
                      void *workspace, size_t workspace_bytes, void *stream)
{
    return run_gemm_act(W, act, Y, M, N, K, path, true, workspace, workspace_bytes, (hipStream_t)stream);
}

static_assert(IQ4XS_MAX_GROUP == MAXGRP, "group bound of the header and the kernels");

// Scratch of a grouped call: the activation planes of the one-launch path,
// or the largest per-matrix need of the one-call-per-matrix path.
static int group_need(const int64_t *N, int G, int64_t M, int64_t K, bool *one_launch, size_t *need)
{
    const MmvPlan p = tune_override().mmv != 0 ? mmv_plan_group(M, N, G, K, device_cus()) : MmvPlan();
    *one_launch = p.ok;
    if (p.ok) {
        *need = xplanes_bytes(M, K);
        return IQ4XS_OK;
    }
    size_t most = 0;
    for (int g = 0; g < G; g++) {
        int path = IQ4XS_PATH_AUTO;
        const int st = resolve_path(path, M, N[g], K, &path);
        if (st != IQ4XS_OK)
            return st;
        most = std::max(most, workspace_need(path, M, N[g], K));
    }
    *need = most;
    return IQ4XS_OK;
}

static int check_group_sizes(const int64_t *N, int G, int64_t M, int64_t K)
{
    if (!N)
        return fail(IQ4XS_EINVAL, "null pointer");
    if (G < 1 || G > IQ4XS_MAX_GROUP)
        return fail(IQ4XS_EINVAL, "group of %d matrices (1..%d)", G, IQ4XS_MAX_GROUP);
    for (int g = 0; g < G; g++) {
        const int st = check_dims(M, N[g], K);
        if (st != IQ4XS_OK)
            return st;
    }
    return IQ4XS_OK;
}

int iq4xs_gemm_group_workspace_bytes(const int64_t *N, int G, int64_t M, int64_t K, size_t *out)
{
    if (!out)
        return fail(IQ4XS_EINVAL, "null output pointer");
    int st = check_group_sizes(N, G, M, K);
    if (st != IQ4XS_OK)
        return st;
    bool one = false;
    return group_need(N, G, M, K, &one, out);
}

int iq4xs_gemm_group(const void *const *W, float *const *Y, const int64_t *N, int G, const float *X,
                     int64_t M, int64_t K, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!W || !Y || !N || !X)
        return fail(IQ4XS_EINVAL, "null pointer");
    if (G < 1 || G > IQ4XS_MAX_GROUP)
        return fail(IQ4XS_EINVAL, "group of %d matrices (1..%d)", G, IQ4XS_MAX_GROUP);
    if (!aligned(X, 16))
        return fail(IQ4XS_EALIGN, "X must be 16-byte aligned");
    for (int g = 0; g < G; g++) {
        if (!W[g] || !Y[g])
            return fail(IQ4XS_EINVAL, "null pointer (matrix %d)", g);
        int st = check_dims(M, N[g], K);
        if (st != IQ4XS_OK)
            return st;
        if (!aligned(W[g], 16) || !aligned(Y[g], 16))
            return fail(IQ4XS_EALIGN, "W and Y must be 16-byte aligned (matrix %d)", g);
    }
    for (int g = 0; g < G; g++) {
        const size_t yb = (size_t)(M * N[g] * 4);
        if (overlaps(Y[g], yb, X, (size_t)(M * K * 4)))
            return fail(IQ4XS_EINVAL, "Y overlaps an input (matrix %d)", g);
        for (int h = 0; h < G; h++)
            if (overlaps(Y[g], yb, W[h], (size_t)(N[h] * (K / QK) * WBLK)) ||
                (h != g && overlaps(Y[g], yb, Y[h], (size_t)(M * N[h] * 4))))
                return fail(IQ4XS_EINVAL, "Y of matrix %d overlaps a weight matrix or another output", g);
    }
    if (workspace != nullptr) {
        if (!aligned(workspace, 256))
            return fail(IQ4XS_EALIGN, "workspace must be 256-byte aligned");
        if (overlaps(workspace, workspace_bytes, X, (size_t)(M * K * 4)))
            return fail(IQ4XS_EINVAL, "workspace overlaps X");
        for (int g = 0; g < G; g++)
            if (overlaps(workspace, workspace_bytes, Y[g], (size_t)(M * N[g] * 4)) ||
                overlaps(workspace, workspace_bytes, W[g], (size_t)(N[g] * (K / QK) * WBLK)))
                return fail(IQ4XS_EINVAL, "workspace overlaps W or Y (matrix %d)", g);
    }
    ensure_init();
    int st = check_device();
    if (st != IQ4XS_OK)
        return st;
    const hipStream_t s = (hipStream_t)stream;
    bool one_launch = false;
    size_t need = 0;
    if ((st = group_need(N, G, M, K, &one_launch, &need)) != IQ4XS_OK)
        return st;
    if (workspace != nullptr && workspace_bytes < need)
        return fail(IQ4XS_EINVAL, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    if (!one_launch) {
        // shapes the streaming kernel does not take: one call per matrix
        for (int g = 0; g < G; g++)
            if ((st = run_gemm(W[g], X, nullptr, Y[g], M, N[g], K, IQ4XS_PATH_AUTO, workspace,
                               workspace_bytes, s)) != IQ4XS_OK)
                return st;
        return IQ4XS_OK;
    }
    const MmvPlan p = mmv_plan_group(M, N, G, K, device_cus());
    Scratch scr;
    scr.s = s;
    void *base = workspace;
    if (base == nullptr) {
        if (hipMallocAsync(&scr.p, need, s) != hipSuccess) {
            (void)hipGetLastError();
            scr.p = nullptr;
            return fail(IQ4XS_ENOMEM, "scratch of %zu bytes", need);
        }
        base = scr.p;
    }
    const XPlanes xp = xplanes_at(base, M, K);
    ZeroList zl;
    if (p.zero_y) {
        zl.count = G;
        for (int g = 0; g < G; g++) {
            zl.p[g] = Y[g];
            zl.n[g] = M * N[g];
        }
    }
    if ((st = launch_err(launch_quantize(X, nullptr, &xp, M, K, s, zl), "quantize")) != IQ4XS_OK)
        return st;
    return launch_err(launch_mmv_group(mmv_group(W, Y, N, G), xp, p, s), "MMQ group");
}

int iq4xs_dispatch(int64_t M, int64_t N, int64_t K, int *path_out)
{
    if (!path_out)
        return fail(IQ4XS_EINVAL, "null output pointer");
    int st = check_dims(M, N, K);
    if (st != IQ4XS_OK)
        return st;
    int p = 0;
    if ((st = resolve_path(IQ4XS_PATH_AUTO, M, N, K, &p)) != IQ4XS_OK)
        return st;
    *path_out = p;
    return IQ4XS_OK;
}

int iq4xs_load_dispatch_table(const char *path)
{
    int st = ensure_init();
    (void)st;
    st = path ? load_table_file(path) : load_table_text(default_table_text(), "built-in dispatch table");
    if (st == IQ4XS_OK)
        g_cfg.init_status = IQ4XS_OK;
    return st;
}

const char *iq4xs_path_name(int path) { return path_name(path); }

const char *iq4xs_last_error(void) { return g_err.c_str(); }

}  // extern "C"
