// svdq_api.hip -- the C ABI declared in include/svdq.h: argument validation,
// the gfx950 device check, workspace carving and kernel launches.
//
// Order of checks: every argument first (no device call needed, so argument
// errors are reported on any host), then the device architecture, then the
// launches.  Nothing is written before all checks pass.  Unsupported hardware
// is refused with a clear error instead of running (the "Hardware support"
// section of the Nunchaku 4-bit in Diffusers blog does the same at load time).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "svdq.h"
#include "svdq_internal.h"

namespace {

thread_local char g_last_error[512] = "";

int32_t fail(int32_t status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Per-device cache of the architecture check: 0 unknown, 1 gfx950, 2 other.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];

int32_t check_device() {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0)
        return fail(SVDQ_ERR_UNSUPPORTED_DEVICE, "no HIP device available (%s)",
                    hipGetErrorString(e));
    if (dev < kMaxDevices) {
        int v = g_arch_ok[dev].load(std::memory_order_relaxed);
        if (v == 1) return SVDQ_OK;
        if (v == 2) return fail(SVDQ_ERR_UNSUPPORTED_DEVICE, "device %d is not gfx950", dev);
    }
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
        return fail(SVDQ_ERR_UNSUPPORTED_DEVICE, "hipGetDeviceProperties failed: %s",
                    hipGetErrorString(e));
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < kMaxDevices) g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    if (!ok)
        return fail(SVDQ_ERR_UNSUPPORTED_DEVICE,
                    "device %d is %s; this library is built for gfx950 (MI355X) only", dev,
                    prop.gcnArchName);
    return SVDQ_OK;
}

int32_t hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return SVDQ_OK;
    return fail(SVDQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int32_t check_k(int64_t K) {
    if (K < SVDQ_GROUP || K % SVDQ_GROUP != 0)
        return fail(SVDQ_ERR_UNSUPPORTED_SHAPE, "K must be a positive multiple of 64 (got %lld)",
                    (long long)K);
    if (K > SVDQ_MAX_K)
        return fail(SVDQ_ERR_UNSUPPORTED_SHAPE, "K = %lld exceeds the limit %d", (long long)K,
                    SVDQ_MAX_K);
    return SVDQ_OK;
}

// Token and output-row counts: >= 0 (0: nothing to do) and within the limit.
int32_t check_rows(int64_t n, const char *name) {
    if (n < 0) return fail(SVDQ_ERR_INVALID_ARG, "%s must be >= 0 (got %lld)", name, (long long)n);
    if (n > SVDQ_MAX_ROWS)
        return fail(SVDQ_ERR_UNSUPPORTED_SHAPE, "%s = %lld exceeds the limit %d", name,
                    (long long)n, SVDQ_MAX_ROWS);
    return SVDQ_OK;
}

// The MXFP4 variant: whole stages of two groups (128 values) along K.
int32_t check_k_mx(int64_t K) {
    if (K < 128 || K % 128 != 0)
        return fail(SVDQ_ERR_UNSUPPORTED_SHAPE,
                    "K must be a positive multiple of 128 for MXFP4 (got %lld)", (long long)K);
    return check_k(K);
}

int32_t check_r(int32_t r) {
    if (r < 0 || r > SVDQ_MAX_RANK || r % 16 != 0)
        return fail(SVDQ_ERR_UNSUPPORTED_SHAPE,
                    "rank r must be a multiple of 16 in [0, %d] (got %d)", SVDQ_MAX_RANK, r);
    return SVDQ_OK;
}

int32_t check_n(int64_t N) {
    if (N < 8 || N % 8 != 0)
        return fail(SVDQ_ERR_UNSUPPORTED_SHAPE, "N must be a positive multiple of 8 (got %lld)",
                    (long long)N);
    return check_rows(N, "N");
}

// A launch's work-items (workgroups x threads) must fit the 32-bit grid size
// of a dispatch.  Shapes inside the row and K limits can still exceed it
// (e.g. 2^28 tokens with a wide N); they are rejected here rather than
// launched with a truncated grid.
int32_t check_grid(int64_t workgroups, int64_t threads, const char *what) {
    if (workgroups > (int64_t)0xFFFFFFFF / threads)
        return fail(SVDQ_ERR_UNSUPPORTED_SHAPE,
                    "%s would need %lld workgroups of %lld threads, more than 2^32 - 1 work-items",
                    what, (long long)workgroups, (long long)threads);
    return SVDQ_OK;
}

#define SVDQ_TRY(expr)                       \
    do {                                     \
        int32_t _s = (expr);                 \
        if (_s != SVDQ_OK) return _s;        \
    } while (0)

// The activation step (at most one workgroup per 64 rows and two groups)
// and its partial-sum reduce; the GEMM's largest tile family (64 x 64 tiles
// of up to 512 threads).
int32_t check_down_grid(int64_t M, int64_t K, int32_t r) {
    SVDQ_TRY(check_grid((M + 63) / 64 * ((K / SVDQ_GROUP + 1) / 2), 256, "the activation step"));
    return check_grid((M * r / 4 + 63) / 64, 256, "the partial-sum reduce");
}

int32_t check_gemm_grid(int64_t M, int64_t N) {
    return check_grid((M + 63) / 64 * ((N + 63) / 64), 512, "the GEMM");
}

int32_t need_ptr(const void *p, const char *name) {
    if (!p) return fail(SVDQ_ERR_INVALID_ARG, "%s must not be NULL", name);
    if (!aligned16(p)) return fail(SVDQ_ERR_MISALIGNED, "%s is not 16-byte aligned", name);
    return SVDQ_OK;
}

int32_t lr_ptrs(const void *a, const char *an, const void *b, const char *bn, int32_t r) {
    if (r == 0) {
        if (a || b)
            return fail(SVDQ_ERR_INVALID_ARG, "%s and %s must be NULL when r == 0", an, bn);
        return SVDQ_OK;
    }
    SVDQ_TRY(need_ptr(a, an));
    return need_ptr(b, bn);
}

int32_t validate_down(const uint16_t *X, const float *lambda, const uint16_t *L1, int64_t M,
                      int64_t K, int32_t r, const uint8_t *qa, const void *sa,
                      const float *xl1, const void *ws, size_t ws_bytes) {
    SVDQ_TRY(check_rows(M, "M"));
    SVDQ_TRY(check_k(K));
    SVDQ_TRY(check_r(r));
    if (M == 0) return SVDQ_OK;
    SVDQ_TRY(check_down_grid(M, K, r));
    SVDQ_TRY(need_ptr(X, "X"));
    SVDQ_TRY(need_ptr(lambda, "lambda"));
    SVDQ_TRY(need_ptr(qa, "qa"));
    SVDQ_TRY(need_ptr(sa, "sa"));
    SVDQ_TRY(lr_ptrs(L1, "L1", xl1, "xl1", r));
    const size_t need = svdq::down_workspace_bytes(M, K, r);
    if (ws_bytes < need)
        return fail(SVDQ_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes < %zu needed",
                    ws_bytes, need);
    return need == 0 ? SVDQ_OK : need_ptr(ws, "workspace");
}

int32_t validate_gemm(const uint8_t *qa, const void *sa, const uint8_t *qw, const void *sw,
                      const float *xl1, const uint16_t *L2, const uint16_t *bias, int32_t act,
                      int64_t M, int64_t N, int64_t K, int32_t r, const uint16_t *Y) {
    SVDQ_TRY(check_rows(M, "M"));
    if (act != SVDQ_ACT_NONE && act != SVDQ_ACT_GELU)
        return fail(SVDQ_ERR_INVALID_ARG, "unknown activation %d", act);
    SVDQ_TRY(check_n(N));
    SVDQ_TRY(check_k(K));
    SVDQ_TRY(check_r(r));
    if (M == 0) return SVDQ_OK;
    SVDQ_TRY(check_gemm_grid(M, N));
    SVDQ_TRY(need_ptr(qa, "qa"));
    SVDQ_TRY(need_ptr(sa, "sa"));
    SVDQ_TRY(need_ptr(qw, "qw"));
    SVDQ_TRY(need_ptr(sw, "sw"));
    SVDQ_TRY(need_ptr(Y, "Y"));
    SVDQ_TRY(lr_ptrs(xl1, "xl1", L2, "L2", r));
    if (bias && !aligned16(bias)) return fail(SVDQ_ERR_MISALIGNED, "bias is not 16-byte aligned");
    return SVDQ_OK;
}

int32_t validate_qkv(const svdq_qkv_epilogue *e, int64_t M) {
    if (!e) return fail(SVDQ_ERR_INVALID_ARG, "epi must not be NULL");
    if (e->heads < 1) return fail(SVDQ_ERR_INVALID_ARG, "heads must be >= 1 (got %d)", e->heads);
    if (e->head_dim != 64 && e->head_dim != 128)
        return fail(SVDQ_ERR_UNSUPPORTED_SHAPE, "head_dim must be 64 or 128 (got %d)",
                    e->head_dim);
    if (((int64_t)e->heads * e->head_dim) % 128 != 0)
        return fail(SVDQ_ERR_UNSUPPORTED_SHAPE, "heads * head_dim must be a multiple of 128");
    if (e->seq < 1) return fail(SVDQ_ERR_INVALID_ARG, "seq must be >= 1");
    if (M % e->seq != 0)
        return fail(SVDQ_ERR_UNSUPPORTED_SHAPE, "M = %lld is not a multiple of seq = %lld",
                    (long long)M, (long long)e->seq);
    if (!(e->eps >= 0.0f) || e->eps > 3.0e38f)
        return fail(SVDQ_ERR_INVALID_ARG, "eps must be finite and >= 0");
    if (M == 0) return SVDQ_OK;
    SVDQ_TRY(need_ptr(e->gamma_q, "gamma_q"));
    SVDQ_TRY(need_ptr(e->gamma_k, "gamma_k"));
    SVDQ_TRY(need_ptr(e->cos_t, "cos_t"));
    SVDQ_TRY(need_ptr(e->sin_t, "sin_t"));
    SVDQ_TRY(need_ptr(e->q, "q"));
    SVDQ_TRY(need_ptr(e->k, "k"));
    return need_ptr(e->v, "v");
}

svdq::QkvArgs qkv_args(const svdq_qkv_epilogue *e) {
    svdq::QkvArgs a;
    a.H = e->heads;
    a.D = e->head_dim;
    a.S = e->seq;
    a.gq = e->gamma_q;
    a.gk = e->gamma_k;
    a.eps = e->eps;
    a.cos_t = e->cos_t;
    a.sin_t = e->sin_t;
    a.Q = e->q;
    a.K = e->k;
    a.V = e->v;
    return a;
}

struct LinearWorkspace {
    uint8_t *qa;
    float *sa;
    float *xl1;
    void *down;
    size_t bytes;
};

// mx: the scales are block-major E8M0 bytes [K/32][mx_scale_rows(M)] instead of fp32
// [M, K/64].
LinearWorkspace carve_linear(void *base, int64_t M, int64_t K, int32_t r, bool mx = false) {
    using svdq::align256;
    LinearWorkspace w{};
    char *p = static_cast<char *>(base);
    size_t off = 0;
    w.qa = reinterpret_cast<uint8_t *>(p + off);
    off += align256((size_t)((M + 1) / 2) * (size_t)K);   // row-pair codes
    w.sa = reinterpret_cast<float *>(p + off);
    off += align256(mx ? (size_t)svdq::mx_scale_rows(M) * (size_t)(K / 32)
                       : svdq::scale_floats(M, K / SVDQ_GROUP) * 4);
    w.xl1 = r > 0 ? reinterpret_cast<float *>(p + off) : nullptr;
    off += align256((size_t)M * (size_t)r * 4);
    w.down = p + off;
    off += svdq::down_workspace_bytes(M, K, r);
    w.bytes = off;
    return w;
}

}  // namespace

// Scratch of svdq_linear_noalloc: the layer's intermediates (codes, scales,
// x^ L1 and the down-projection's partial sums) for callers that cannot
// allocate.  Each device holds its own copy from module load to process end.
// Host code uses only the per-device address from hipGetSymbolAddress, never
// the array's name (which is a host-side stand-in).
static __device__ __align__(256) uint8_t scratch[SVDQ_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch`, looked up once per device (with
// that device current) on its first use.
int32_t scratch_address(void **out) {
    int dev = -1;
    SVDQ_TRY(hip_status(hipGetDevice(&dev), "hipGetDevice"));
    if (dev < 0 || dev >= kMaxDevices) return fail(SVDQ_ERR_HIP, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        SVDQ_TRY(hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)),
                            "hipGetSymbolAddress(scratch)"));
        if (!p) return fail(SVDQ_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SVDQ_OK;
}

}  // namespace

namespace {

int32_t check_awq_pack_shape(int64_t N, int64_t K) {
    SVDQ_TRY(check_rows(N, "N"));
    SVDQ_TRY(check_k(K));
    if (N > 0) SVDQ_TRY(check_n(N));
    const int64_t threads = (N + 15) / 16 * 16 * 4 * ((K / SVDQ_GROUP + 3) / 4);
    return check_grid((threads + 255) / 256, 256, "the W4A16 packer");
}

// Per-device cache of the per-workgroup LDS limit.
std::atomic<int64_t> g_lds_limit[kMaxDevices];

int32_t lds_limit(size_t *out) {
    int dev = -1;
    SVDQ_TRY(hip_status(hipGetDevice(&dev), "hipGetDevice"));
    if (dev < 0 || dev >= kMaxDevices) return fail(SVDQ_ERR_HIP, "device index %d out of range", dev);
    int64_t v = g_lds_limit[dev].load();
    if (v <= 0) {
        int bytes = 0;
        SVDQ_TRY(hip_status(
            hipDeviceGetAttribute(&bytes, hipDeviceAttributeMaxSharedMemoryPerBlock, dev),
            "hipDeviceGetAttribute(MaxSharedMemoryPerBlock)"));
        v = bytes;
        g_lds_limit[dev].store(v);
    }
    *out = (size_t)v;
    return SVDQ_OK;
}

}  // namespace

namespace {

size_t mlp_part_bytes(int64_t M, int64_t N, int32_t rn) {
    return rn > 0 ? svdq::align256((size_t)(N / 128) * (size_t)M * (size_t)rn * 4) : 0;
}

int32_t check_next_shape(int64_t N, int32_t rn) {
    if (N % 128 != 0)
        return fail(SVDQ_ERR_UNSUPPORTED_SHAPE,
                    "N must be a multiple of 128 for the fused activation step (got %lld)",
                    (long long)N);
    if (rn != 0 && rn != 16 && rn != 32)
        return fail(SVDQ_ERR_UNSUPPORTED_SHAPE,
                    "the fused activation step takes a next-layer rank of 0, 16 or 32 (got %d)", rn);
    return SVDQ_OK;
}

struct MlpWorkspace {
    LinearWorkspace up;
    uint8_t *qa_h;
    float *sa_h;
    float *xl1_h;
    float *part;
    size_t bytes;
};

MlpWorkspace carve_mlp(void *base, int64_t M, int64_t K, int64_t Nh, int32_t r_up, int32_t r_down) {
    using svdq::align256;
    MlpWorkspace w{};
    w.up = carve_linear(base, M, K, r_up);
    char *p = static_cast<char *>(base);
    size_t off = w.up.bytes;
    w.qa_h = reinterpret_cast<uint8_t *>(p + off);
    off += align256((size_t)((M + 1) / 2) * (size_t)Nh);   // row-pair codes
    w.sa_h = reinterpret_cast<float *>(p + off);
    off += align256(svdq::scale_floats(M, Nh / SVDQ_GROUP) * 4);
    w.xl1_h = r_down > 0 ? reinterpret_cast<float *>(p + off) : nullptr;
    off += align256((size_t)M * (size_t)r_down * 4);
    w.part = reinterpret_cast<float *>(p + off);
    off += mlp_part_bytes(M, Nh, r_down);
    w.bytes = off;
    return w;
}

}  // namespace

extern "C" {

int32_t svdq_abi_version(void) { return SVDQ_ABI_VERSION; }

const char *svdq_status_string(int32_t s) {
    switch (s) {
        case SVDQ_OK: return "ok";
        case SVDQ_ERR_INVALID_ARG: return "invalid argument";
        case SVDQ_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
        case SVDQ_ERR_MISALIGNED: return "misaligned pointer";
        case SVDQ_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case SVDQ_ERR_UNSUPPORTED_DEVICE: return "unsupported device";
        case SVDQ_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char *svdq_last_error(void) { return g_last_error; }

int32_t svdq_pack_weights(const float *R, int64_t N, int64_t K, uint8_t *qw, float *sw,
                          void *stream) {
    g_last_error[0] = 0;
    SVDQ_TRY(check_rows(N, "N"));
    SVDQ_TRY(check_k(K));
    if (N == 0) return SVDQ_OK;
    SVDQ_TRY(need_ptr(R, "R"));
    SVDQ_TRY(need_ptr(qw, "qw"));
    SVDQ_TRY(need_ptr(sw, "sw"));
    SVDQ_TRY(check_device());
    return hip_status(svdq::launch_pack_weights(R, N, K, qw, sw, (hipStream_t)stream),
                      "pack_weights launch");
}

int32_t svdq_repack_weights(const uint8_t *codes, const float *scales, int64_t N, int64_t K,
                            uint8_t *qw, float *sw, void *stream) {
    g_last_error[0] = 0;
    SVDQ_TRY(check_rows(N, "N"));
    SVDQ_TRY(check_k(K));
    if (N == 0) return SVDQ_OK;
    SVDQ_TRY(check_grid((N * (K / 16) + 255) / 256, 256, "the repack"));
    SVDQ_TRY(need_ptr(codes, "codes"));
    SVDQ_TRY(need_ptr(scales, "scales"));
    SVDQ_TRY(need_ptr(qw, "qw"));
    SVDQ_TRY(need_ptr(sw, "sw"));
    SVDQ_TRY(check_device());
    return hip_status(svdq::launch_repack_codes(codes, scales, N, K, qw, sw, (hipStream_t)stream),
                      "repack_weights launch");
}

size_t svdq_quantize_act_down_workspace_bytes(int64_t M, int64_t K, int32_t r) {
    if (M < 0 || K < 0 || r < 0) return 0;
    return svdq::down_workspace_bytes(M, K, r);
}

int32_t svdq_quantize_act_down(const uint16_t *X, const float *lambda, const uint16_t *L1,
                               int64_t M, int64_t K, int32_t r, uint8_t *qa, float *sa,
                               float *xl1, void *workspace, size_t ws_bytes, void *stream) {
    g_last_error[0] = 0;
    SVDQ_TRY(validate_down(X, lambda, L1, M, K, r, qa, sa, xl1, workspace, ws_bytes));
    if (M == 0) return SVDQ_OK;
    SVDQ_TRY(check_device());
    hipStream_t s = (hipStream_t)stream;
    const svdq::DownWorkspace dw = svdq::carve_down_workspace(workspace, M, K, r);
    return hip_status(svdq::launch_quant_down(X, lambda, L1, M, K, r, dw, qa, sa, xl1, s),
                      "quantize_act_down launch");
}

int32_t svdq_w4a4_lr_gemm(const uint8_t *qa, const float *sa, const uint8_t *qw,
                          const float *sw, const float *xl1, const uint16_t *L2,
                          const uint16_t *bias, int32_t act, int64_t M, int64_t N, int64_t K,
                          int32_t r, uint16_t *Y, void *stream) {
    g_last_error[0] = 0;
    SVDQ_TRY(validate_gemm(qa, sa, qw, sw, xl1, L2, bias, act, M, N, K, r, Y));
    if (M == 0) return SVDQ_OK;
    SVDQ_TRY(check_device());
    return hip_status(svdq::launch_w4a4_gemm(qa, sa, qw, sw, xl1, L2, bias, act, M, N, K, r, Y,
                                             (hipStream_t)stream),
                      "w4a4_lr_gemm launch");
}

int32_t svdq_w4a4_lr_gemm_qkv(const uint8_t *qa, const float *sa, const uint8_t *qw,
                              const float *sw, const float *xl1, const uint16_t *L2,
                              const uint16_t *bias, int64_t M, int64_t K, int32_t r,
                              const svdq_qkv_epilogue *epi, void *stream) {
    g_last_error[0] = 0;
    SVDQ_TRY(check_rows(M, "M"));
    SVDQ_TRY(validate_qkv(epi, M));
    const int64_t N = 3 * (int64_t)epi->heads * epi->head_dim;
    // the plain GEMM's checks, with a stand-in for the [M, N] output
    SVDQ_TRY(validate_gemm(qa, sa, qw, sw, xl1, L2, bias, SVDQ_ACT_NONE, M, N, K, r, epi->q));
    if (M == 0) return SVDQ_OK;
    SVDQ_TRY(check_device());
    return hip_status(svdq::launch_w4a4_gemm_qkv(qa, sa, qw, sw, xl1, L2, bias, M, K, r,
                                                 qkv_args(epi), (hipStream_t)stream),
                      "w4a4_lr_gemm_qkv launch");
}

size_t svdq_linear_workspace_bytes(int64_t M, int64_t K, int32_t r) {
    if (M < 0 || K < 0 || r < 0) return 0;
    return carve_linear(nullptr, M, K, r).bytes;
}

int32_t svdq_linear(const uint16_t *X, const float *lambda, const uint16_t *L1,
                    const uint8_t *qw, const float *sw, const uint16_t *L2,
                    const uint16_t *bias, int32_t act, int64_t M, int64_t N, int64_t K,
                    int32_t r, uint16_t *Y, void *workspace, size_t ws_bytes, void *stream) {
    g_last_error[0] = 0;
    SVDQ_TRY(check_rows(M, "M"));
    if (act != SVDQ_ACT_NONE && act != SVDQ_ACT_GELU)
        return fail(SVDQ_ERR_INVALID_ARG, "unknown activation %d", act);
    SVDQ_TRY(check_n(N));
    SVDQ_TRY(check_k(K));
    SVDQ_TRY(check_r(r));
    if (M == 0) return SVDQ_OK;
    SVDQ_TRY(check_down_grid(M, K, r));
    SVDQ_TRY(check_gemm_grid(M, N));
    SVDQ_TRY(need_ptr(X, "X"));
    SVDQ_TRY(need_ptr(lambda, "lambda"));
    SVDQ_TRY(need_ptr(qw, "qw"));
    SVDQ_TRY(need_ptr(sw, "sw"));
    SVDQ_TRY(need_ptr(Y, "Y"));
    SVDQ_TRY(lr_ptrs(L1, "L1", L2, "L2", r));
    if (bias && !aligned16(bias)) return fail(SVDQ_ERR_MISALIGNED, "bias is not 16-byte aligned");
    const size_t need = carve_linear(nullptr, M, K, r).bytes;
    if (ws_bytes < need)
        return fail(SVDQ_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes < %zu needed", ws_bytes,
                    need);
    SVDQ_TRY(need_ptr(workspace, "workspace"));
    SVDQ_TRY(check_device());
    hipStream_t s = (hipStream_t)stream;
    const LinearWorkspace w = carve_linear(workspace, M, K, r);
    const svdq::DownWorkspace dw = svdq::carve_down_workspace(w.down, M, K, r);
    SVDQ_TRY(hip_status(svdq::launch_quant_down(X, lambda, L1, M, K, r, dw, w.qa, w.sa, w.xl1,
                                                s),
                        "quantize_act_down launch"));
    return hip_status(svdq::launch_w4a4_gemm(w.qa, w.sa, qw, sw, w.xl1, L2, bias, act, M, N, K,
                                             r, Y, s),
                      "w4a4_lr_gemm launch");
}

int32_t svdq_linear_noalloc(const uint16_t *X, const float *lambda, const uint16_t *L1,
                            const uint8_t *qw, const float *sw, const uint16_t *L2,
                            const uint16_t *bias, int32_t act, int64_t M, int64_t N, int64_t K,
                            int32_t r, uint16_t *Y, void *stream) {
    g_last_error[0] = 0;
    SVDQ_TRY(check_rows(M, "M"));
    if (act != SVDQ_ACT_NONE && act != SVDQ_ACT_GELU)
        return fail(SVDQ_ERR_INVALID_ARG, "unknown activation %d", act);
    SVDQ_TRY(check_n(N));
    SVDQ_TRY(check_k(K));
    SVDQ_TRY(check_r(r));
    if (M == 0) return SVDQ_OK;
    SVDQ_TRY(check_down_grid(M, K, r));
    SVDQ_TRY(check_gemm_grid(M, N));
    SVDQ_TRY(need_ptr(X, "X"));
    SVDQ_TRY(need_ptr(lambda, "lambda"));
    SVDQ_TRY(need_ptr(qw, "qw"));
    SVDQ_TRY(need_ptr(sw, "sw"));
    SVDQ_TRY(need_ptr(Y, "Y"));
    SVDQ_TRY(lr_ptrs(L1, "L1", L2, "L2", r));
    if (bias && !aligned16(bias)) return fail(SVDQ_ERR_MISALIGNED, "bias is not 16-byte aligned");
    const size_t need = carve_linear(nullptr, M, K, r).bytes;
    if (need > (size_t)SVDQ_NOALLOC_SCRATCH_BYTES)
        return fail(SVDQ_ERR_WORKSPACE_TOO_SMALL,
                    "M = %lld, K = %lld, r = %d needs %zu bytes of scratch; the allocation-free "
                    "entry point holds %zu (use svdq_linear with a workspace)",
                    (long long)M, (long long)K, r, need, (size_t)SVDQ_NOALLOC_SCRATCH_BYTES);
    SVDQ_TRY(check_device());
    void *base = nullptr;
    SVDQ_TRY(scratch_address(&base));
    hipStream_t s = (hipStream_t)stream;
    const LinearWorkspace w = carve_linear(base, M, K, r);
    const svdq::DownWorkspace dw = svdq::carve_down_workspace(w.down, M, K, r);
    SVDQ_TRY(hip_status(svdq::launch_quant_down(X, lambda, L1, M, K, r, dw, w.qa, w.sa, w.xl1,
                                                s),
                        "quantize_act_down launch"));
    return hip_status(svdq::launch_w4a4_gemm(w.qa, w.sa, qw, sw, w.xl1, L2, bias, act, M, N, K,
                                             r, Y, s),
                      "w4a4_lr_gemm launch");
}

int32_t svdq_linear_qkv(const uint16_t *X, const float *lambda, const uint16_t *L1,
                        const uint8_t *qw, const float *sw, const uint16_t *L2,
                        const uint16_t *bias, int64_t M, int64_t K, int32_t r,
                        const svdq_qkv_epilogue *epi, void *workspace, size_t ws_bytes,
                        void *stream) {
    g_last_error[0] = 0;
    SVDQ_TRY(check_rows(M, "M"));
    SVDQ_TRY(validate_qkv(epi, M));
    SVDQ_TRY(check_k(K));
    SVDQ_TRY(check_r(r));
    if (M == 0) return SVDQ_OK;
    SVDQ_TRY(check_down_grid(M, K, r));
    SVDQ_TRY(check_gemm_grid(M, 3 * (int64_t)epi->heads * epi->head_dim));
    SVDQ_TRY(need_ptr(X, "X"));
    SVDQ_TRY(need_ptr(lambda, "lambda"));
    SVDQ_TRY(need_ptr(qw, "qw"));
    SVDQ_TRY(need_ptr(sw, "sw"));
    SVDQ_TRY(lr_ptrs(L1, "L1", L2, "L2", r));
    if (bias && !aligned16(bias)) return fail(SVDQ_ERR_MISALIGNED, "bias is not 16-byte aligned");
    const size_t need = carve_linear(nullptr, M, K, r).bytes;
    if (ws_bytes < need)
        return fail(SVDQ_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes < %zu needed", ws_bytes,
                    need);
    SVDQ_TRY(need_ptr(workspace, "workspace"));
    SVDQ_TRY(check_device());
    hipStream_t s = (hipStream_t)stream;
    const LinearWorkspace w = carve_linear(workspace, M, K, r);
    const svdq::DownWorkspace dw = svdq::carve_down_workspace(w.down, M, K, r);
    SVDQ_TRY(hip_status(svdq::launch_quant_down(X, lambda, L1, M, K, r, dw, w.qa, w.sa, w.xl1,
                                                s),
                        "quantize_act_down launch"));
    return hip_status(svdq::launch_w4a4_gemm_qkv(w.qa, w.sa, qw, sw, w.xl1, L2, bias, M, K, r,
                                                 qkv_args(epi), s),
                      "w4a4_lr_gemm_qkv launch");
}

size_t svdq_w4a4_lr_gemm_quant_down_workspace_bytes(int64_t M, int64_t N, int32_t r_next) {
    if (M < 0 || N < 0 || r_next < 0) return 0;
    return mlp_part_bytes(M, N, r_next);
}

int32_t svdq_w4a4_lr_gemm_quant_down(const uint8_t *qa, const float *sa, const uint8_t *qw,
                                     const float *sw, const float *xl1, const uint16_t *L2,
                                     const uint16_t *bias, int32_t act, int64_t M, int64_t N,
                                     int64_t K, int32_t r, const float *lambda_next,
                                     const uint16_t *L1_next, int32_t r_next, uint8_t *qa_next,
                                     float *sa_next, float *xl1_next, void *workspace,
                                     size_t ws_bytes, void *stream) {
    g_last_error[0] = 0;
    SVDQ_TRY(check_rows(M, "M"));
    SVDQ_TRY(check_n(N));
    SVDQ_TRY(check_next_shape(N, r_next));
    // the plain GEMM's checks, with the next layer's codes standing in for Y
    SVDQ_TRY(validate_gemm(qa, sa, qw, sw, xl1, L2, bias, act, M, N, K, r,
                           reinterpret_cast<const uint16_t *>(qa_next)));
    if (M == 0) return SVDQ_OK;
    SVDQ_TRY(check_down_grid(M, N, r_next));
    SVDQ_TRY(need_ptr(lambda_next, "lambda_next"));
    SVDQ_TRY(need_ptr(sa_next, "sa_next"));
    SVDQ_TRY(lr_ptrs(L1_next, "L1_next", xl1_next, "xl1_next", r_next));
    const size_t need = mlp_part_bytes(M, N, r_next);
    if (ws_bytes < need)
        return fail(SVDQ_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes < %zu needed", ws_bytes,
                    need);
    if (need > 0) SVDQ_TRY(need_ptr(workspace, "workspace"));
    SVDQ_TRY(check_device());
    hipStream_t s = (hipStream_t)stream;
    svdq::MlpArgs ma{lambda_next, L1_next, r_next, qa_next, sa_next,
                     static_cast<float *>(workspace)};
    SVDQ_TRY(hip_status(svdq::launch_w4a4_gemm_mlp(qa, sa, qw, sw, xl1, L2, bias, act, M, N, K, r,
                                                   ma, s),
                        "w4a4_lr_gemm_mlp launch"));
    if (r_next == 0) return SVDQ_OK;
    return hip_status(svdq::launch_xl1_reduce(ma.part, (int)(N / 128), M * (int64_t)r_next,
                                              xl1_next, s),
                      "xl1 reduce launch");
}

size_t svdq_mlp_workspace_bytes(int64_t M, int64_t K, int64_t N_hidden, int32_t r_up,
                                int32_t r_down) {
    if (M < 0 || K < 0 || N_hidden < 0 || r_up < 0 || r_down < 0) return 0;
    return carve_mlp(nullptr, M, K, N_hidden, r_up, r_down).bytes;
}

int32_t svdq_mlp(const uint16_t *X, const float *lambda_up, const uint16_t *L1_up,
                 const uint8_t *qw_up, const float *sw_up, const uint16_t *L2_up,
                 const uint16_t *bias_up, const float *lambda_down, const uint16_t *L1_down,
                 const uint8_t *qw_down, const float *sw_down, const uint16_t *L2_down,
                 const uint16_t *bias_down, int32_t act, int64_t M, int64_t K, int64_t N_hidden,
                 int32_t r_up, int32_t r_down, uint16_t *Y, void *workspace, size_t ws_bytes,
                 void *stream) {
    g_last_error[0] = 0;
    SVDQ_TRY(check_rows(M, "M"));
    if (act != SVDQ_ACT_NONE && act != SVDQ_ACT_GELU)
        return fail(SVDQ_ERR_INVALID_ARG, "unknown activation %d", act);
    SVDQ_TRY(check_k(K));
    SVDQ_TRY(check_n(K));            // the down layer's N
    SVDQ_TRY(check_k(N_hidden));
    SVDQ_TRY(check_n(N_hidden));
    SVDQ_TRY(check_r(r_up));
    SVDQ_TRY(check_r(r_down));
    SVDQ_TRY(check_next_shape(N_hidden, r_down));
    if (M == 0) return SVDQ_OK;
    SVDQ_TRY(check_down_grid(M, K, r_up));
    SVDQ_TRY(check_gemm_grid(M, N_hidden));
    SVDQ_TRY(check_down_grid(M, N_hidden, r_down));
    SVDQ_TRY(check_gemm_grid(M, K));
    SVDQ_TRY(need_ptr(X, "X"));
    SVDQ_TRY(need_ptr(lambda_up, "lambda_up"));
    SVDQ_TRY(need_ptr(qw_up, "qw_up"));
    SVDQ_TRY(need_ptr(sw_up, "sw_up"));
    SVDQ_TRY(lr_ptrs(L1_up, "L1_up", L2_up, "L2_up", r_up));
    SVDQ_TRY(need_ptr(lambda_down, "lambda_down"));
    SVDQ_TRY(need_ptr(qw_down, "qw_down"));
    SVDQ_TRY(need_ptr(sw_down, "sw_down"));
    SVDQ_TRY(lr_ptrs(L1_down, "L1_down", L2_down, "L2_down", r_down));
    SVDQ_TRY(need_ptr(Y, "Y"));
    if (bias_up && !aligned16(bias_up))
        return fail(SVDQ_ERR_MISALIGNED, "bias_up is not 16-byte aligned");
    if (bias_down && !aligned16(bias_down))
        return fail(SVDQ_ERR_MISALIGNED, "bias_down is not 16-byte aligned");
    const size_t need = carve_mlp(nullptr, M, K, N_hidden, r_up, r_down).bytes;
    if (ws_bytes < need)
        return fail(SVDQ_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes < %zu needed", ws_bytes,
                    need);
    SVDQ_TRY(need_ptr(workspace, "workspace"));
    SVDQ_TRY(check_device());
    hipStream_t s = (hipStream_t)stream;
    const MlpWorkspace w = carve_mlp(workspace, M, K, N_hidden, r_up, r_down);
    const svdq::DownWorkspace dw = svdq::carve_down_workspace(w.up.down, M, K, r_up);
    SVDQ_TRY(hip_status(svdq::launch_quant_down(X, lambda_up, L1_up, M, K, r_up, dw, w.up.qa,
                                                w.up.sa, w.up.xl1, s),
                        "quantize_act_down launch"));
    svdq::MlpArgs ma{lambda_down, L1_down, r_down, w.qa_h, w.sa_h, w.part};
    SVDQ_TRY(hip_status(svdq::launch_w4a4_gemm_mlp(w.up.qa, w.up.sa, qw_up, sw_up, w.up.xl1, L2_up,
                                                   bias_up, act, M, N_hidden, K, r_up, ma, s),
                        "w4a4_lr_gemm_mlp launch"));
    if (r_down > 0)
        SVDQ_TRY(hip_status(svdq::launch_xl1_reduce(w.part, (int)(N_hidden / 128),
                                                    M * (int64_t)r_down, w.xl1_h, s),
                            "xl1 reduce launch"));
    return hip_status(svdq::launch_w4a4_gemm(w.qa_h, w.sa_h, qw_down, sw_down, w.xl1_h, L2_down,
                                             bias_down, SVDQ_ACT_NONE, M, K, N_hidden, r_down, Y,
                                             s),
                      "w4a4_lr_gemm launch");
}

// ------------------------------------------------------------------ MXFP4

int32_t svdq_mx_pack_weights(const float *R, int64_t N, int64_t K, uint8_t *qw, uint8_t *sw,
                             void *stream) {
    g_last_error[0] = 0;
    SVDQ_TRY(check_rows(N, "N"));
    SVDQ_TRY(check_k_mx(K));
    if (N == 0) return SVDQ_OK;
    SVDQ_TRY(need_ptr(R, "R"));
    SVDQ_TRY(need_ptr(qw, "qw"));
    SVDQ_TRY(need_ptr(sw, "sw"));
    SVDQ_TRY(check_device());
    return hip_status(svdq::launch_pack_weights(R, N, K, qw, sw, (hipStream_t)stream, true),
                      "mx_pack_weights launch");
}

int32_t svdq_mx_quantize_act_down(const uint16_t *X, const float *lambda, const uint16_t *L1,
                                  int64_t M, int64_t K, int32_t r, uint8_t *qa, uint8_t *sa,
                                  float *xl1, void *workspace, size_t ws_bytes, void *stream) {
    g_last_error[0] = 0;
    SVDQ_TRY(check_k_mx(K));
    SVDQ_TRY(validate_down(X, lambda, L1, M, K, r, qa, sa, xl1, workspace, ws_bytes));
    if (M == 0) return SVDQ_OK;
    SVDQ_TRY(check_device());
    hipStream_t s = (hipStream_t)stream;
    const svdq::DownWorkspace dw = svdq::carve_down_workspace(workspace, M, K, r);
    return hip_status(svdq::launch_quant_down(X, lambda, L1, M, K, r, dw, qa, sa, xl1, s, true),
                      "mx_quantize_act_down launch");
}

int32_t svdq_mx_lr_gemm(const uint8_t *qa, const uint8_t *sa, const uint8_t *qw,
                        const uint8_t *sw, const float *xl1, const uint16_t *L2,
                        const uint16_t *bias, int32_t act, int64_t M, int64_t N, int64_t K,
                        int32_t r, uint16_t *Y, void *stream) {
    g_last_error[0] = 0;
    SVDQ_TRY(check_k_mx(K));
    SVDQ_TRY(validate_gemm(qa, sa, qw, sw, xl1, L2, bias, act, M, N, K, r, Y));
    if (M == 0) return SVDQ_OK;
    SVDQ_TRY(check_device());
    return hip_status(svdq::launch_w4a4_mx_gemm(qa, sa, qw, sw, xl1, L2, bias, act, M, N, K, r,
                                                Y, (hipStream_t)stream),
                      "mx_lr_gemm launch");
}

size_t svdq_mx_linear_workspace_bytes(int64_t M, int64_t K, int32_t r) {
    if (M < 0 || K < 0 || r < 0) return 0;
    return carve_linear(nullptr, M, K, r, true).bytes;
}

int32_t svdq_mx_linear(const uint16_t *X, const float *lambda, const uint16_t *L1,
                       const uint8_t *qw, const uint8_t *sw, const uint16_t *L2,
                       const uint16_t *bias, int32_t act, int64_t M, int64_t N, int64_t K,
                       int32_t r, uint16_t *Y, void *workspace, size_t ws_bytes, void *stream) {
    g_last_error[0] = 0;
    SVDQ_TRY(check_rows(M, "M"));
    if (act != SVDQ_ACT_NONE && act != SVDQ_ACT_GELU)
        return fail(SVDQ_ERR_INVALID_ARG, "unknown activation %d", act);
    SVDQ_TRY(check_n(N));
    SVDQ_TRY(check_k_mx(K));
    SVDQ_TRY(check_r(r));
    if (M == 0) return SVDQ_OK;
    SVDQ_TRY(check_down_grid(M, K, r));
    SVDQ_TRY(check_gemm_grid(M, N));
    SVDQ_TRY(need_ptr(X, "X"));
    SVDQ_TRY(need_ptr(lambda, "lambda"));
    SVDQ_TRY(need_ptr(qw, "qw"));
    SVDQ_TRY(need_ptr(sw, "sw"));
    SVDQ_TRY(need_ptr(Y, "Y"));
    SVDQ_TRY(lr_ptrs(L1, "L1", L2, "L2", r));
    if (bias && !aligned16(bias)) return fail(SVDQ_ERR_MISALIGNED, "bias is not 16-byte aligned");
    const size_t need = carve_linear(nullptr, M, K, r, true).bytes;
    if (ws_bytes < need)
        return fail(SVDQ_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes < %zu needed", ws_bytes,
                    need);
    SVDQ_TRY(need_ptr(workspace, "workspace"));
    SVDQ_TRY(check_device());
    hipStream_t s = (hipStream_t)stream;
    const LinearWorkspace w = carve_linear(workspace, M, K, r, true);
    const svdq::DownWorkspace dw = svdq::carve_down_workspace(w.down, M, K, r);
    uint8_t *sa = reinterpret_cast<uint8_t *>(w.sa);
    SVDQ_TRY(hip_status(svdq::launch_quant_down(X, lambda, L1, M, K, r, dw, w.qa, sa, w.xl1, s,
                                                true),
                        "mx_quantize_act_down launch"));
    return hip_status(svdq::launch_w4a4_mx_gemm(w.qa, sa, qw, sw, w.xl1, L2, bias, act, M, N, K,
                                                r, Y, s),
                      "mx_lr_gemm launch");
}

int32_t svdq_debug_group_sums(const uint8_t *qa, const float *sa, const uint8_t *qw,
                              const float *sw, int64_t M, int64_t N, int64_t K, int64_t m0,
                              int64_t n0, int64_t tm, int64_t tn, int32_t *S, void *stream) {
    g_last_error[0] = 0;
    if (M < 0 || N < 0 || m0 < 0 || n0 < 0 || tm < 0 || tn < 0 || m0 + tm > M || n0 + tn > N)
        return fail(SVDQ_ERR_INVALID_ARG, "block [%lld,+%lld) x [%lld,+%lld) outside %lld x %lld",
                    (long long)m0, (long long)tm, (long long)n0, (long long)tn, (long long)M,
                    (long long)N);
    SVDQ_TRY(check_k(K));
    SVDQ_TRY(check_rows(M, "M"));
    SVDQ_TRY(check_rows(N, "N"));
    if (tm == 0 || tn == 0) return SVDQ_OK;
    SVDQ_TRY(need_ptr(qa, "qa"));
    SVDQ_TRY(need_ptr(sa, "sa"));
    SVDQ_TRY(need_ptr(qw, "qw"));
    SVDQ_TRY(need_ptr(sw, "sw"));
    SVDQ_TRY(need_ptr(S, "S"));
    SVDQ_TRY(check_device());
    return hip_status(svdq::launch_group_sums(qa, sa, qw, sw, M, N, K, m0, n0, tm, tn, S,
                                              svdq::tile_policy() == SVDQ_TILES_QUARTER,
                                              (hipStream_t)stream),
                      "group_sums launch");
}


int32_t svdq_debug_set_tile_policy(int32_t policy) {
    g_last_error[0] = 0;
    if (policy < SVDQ_TILES_AUTO || policy > SVDQ_TILES_KSPLIT_QUARTER)
        return fail(SVDQ_ERR_INVALID_ARG, "tile policy %d is not one of 0 .. 4", (int)policy);
    svdq::set_tile_policy(policy);
    return SVDQ_OK;
}

int64_t svdq_awq_packed_bytes(int64_t N, int64_t K) {
    if (N < 0 || K < SVDQ_GROUP || K % SVDQ_GROUP != 0) return 0;
    return svdq::awq_packed_bytes(N, K);
}


int32_t svdq_awq_pack_weights(const float *W, int64_t N, int64_t K, uint8_t *packed, void *stream) {
    g_last_error[0] = 0;
    SVDQ_TRY(check_awq_pack_shape(N, K));
    if (N == 0) return SVDQ_OK;
    SVDQ_TRY(need_ptr(W, "W"));
    SVDQ_TRY(need_ptr(packed, "packed"));
    SVDQ_TRY(check_device());
    return hip_status(svdq::launch_awq_pack(W, N, K, packed, (hipStream_t)stream),
                      "awq_pack launch");
}

int32_t svdq_awq_repack(const uint8_t *codes, const float *scales, const uint8_t *zeros,
                        int64_t N, int64_t K, uint8_t *packed, void *stream) {
    g_last_error[0] = 0;
    SVDQ_TRY(check_awq_pack_shape(N, K));
    if (N == 0) return SVDQ_OK;
    SVDQ_TRY(need_ptr(codes, "codes"));
    SVDQ_TRY(need_ptr(scales, "scales"));
    if (!zeros) return fail(SVDQ_ERR_INVALID_ARG, "zeros must not be NULL");
    SVDQ_TRY(need_ptr(packed, "packed"));
    SVDQ_TRY(check_device());
    return hip_status(
        svdq::launch_awq_repack(codes, scales, zeros, N, K, packed, (hipStream_t)stream),
        "awq_repack launch");
}

int32_t svdq_awq_w4a16_linear(const uint16_t *X, const uint8_t *packed, const uint16_t *bias,
                              int64_t M, int64_t N, int64_t K, uint16_t *Y, void *stream) {
    g_last_error[0] = 0;
    SVDQ_TRY(check_rows(M, "M"));
    SVDQ_TRY(check_n(N));
    SVDQ_TRY(check_k(K));
    if (M == 0) return SVDQ_OK;
    SVDQ_TRY(need_ptr(X, "X"));
    SVDQ_TRY(need_ptr(packed, "packed"));
    SVDQ_TRY(need_ptr(Y, "Y"));
    if (bias && !aligned16(bias)) return fail(SVDQ_ERR_MISALIGNED, "bias is not 16-byte aligned");
    SVDQ_TRY(check_device());
    size_t limit = 0;
    SVDQ_TRY(lds_limit(&limit));
    const int MT = svdq::awq_rows_per_pass(K, limit);
    if (MT < 1)
        return fail(SVDQ_ERR_UNSUPPORTED_SHAPE,
                    "K = %lld: one activation row does not fit the %zu-byte workgroup LDS",
                    (long long)K, limit);
    SVDQ_TRY(check_grid((N + 15) / 16 * ((M + MT - 1) / MT), 256, "the W4A16 linear"));
    return hip_status(
        svdq::launch_awq_linear(X, packed, bias, M, N, K, MT, Y, (hipStream_t)stream),
        "awq_w4a16_linear launch");
}

}  // extern "C"
