// C ABI of the block-scaled GEMM library: argument validation (the pages'
// check_support()), status reporting and dispatch to the gfx950 kernels.
//
// Every host-detectable error is returned before anything is enqueued, as
// the "Grouped GEMM (SM100 BF16)" page requires of its launches
// (Scheduling, caching, and errors).  Device-resident values are not read.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <utility>

#include "../../include/bsg.h"
#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return status;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(int dt)
{
    switch (dt) {
    case BSG_F32: return 4;
    case BSG_F16:
    case BSG_BF16: return 2;
    default: return 1;
    }
}

bool is_float_out(int dt) { return dt == BSG_F32 || dt == BSG_F16 || dt == BSG_BF16; }

// Device check: the kernels are built for gfx950 only.
int check_device()
{
    static int cached[64];   // 0 unknown, 1 ok, 2 bad
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(BSG_ERR_DEVICE, "hipGetDevice failed");
    if (dev >= 0 && dev < 64 && cached[dev] == 1) return BSG_OK;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return fail(BSG_ERR_DEVICE, "hipGetDeviceProperties failed");
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
        if (dev >= 0 && dev < 64) cached[dev] = 2;
        return fail(BSG_ERR_DEVICE, "device %d is %s; this library is built for gfx950", dev,
                    prop.gcnArchName);
    }
    if (dev >= 0 && dev < 64) cached[dev] = 1;
    return BSG_OK;
}

int launch_status(hipError_t e, const char *what)
{
    if (e == hipSuccess) return BSG_OK;
    if (e == hipErrorNotSupported) return fail(BSG_ERR_UNSUPPORTED, "%s: not supported", what);
    return fail(BSG_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
}

int check_ab_sf(int ab_dtype, int sf_vec_size)
{
    if (ab_dtype != BSG_E4M3 && ab_dtype != BSG_E5M2 && ab_dtype != BSG_E2M1X2)
        return fail(BSG_ERR_DTYPE, "ab_dtype %d is not a block-scaled operand dtype", ab_dtype);
    if (sf_vec_size != 32) {
        if (sf_vec_size == 16)
            return fail(BSG_ERR_UNSUPPORTED, "sf_vec_size 16 is not built (32 is)");
        return fail(BSG_ERR_SHAPE, "sf_vec_size must be 32 (got %d)", sf_vec_size);
    }
    return BSG_OK;
}

int row_bytes(int ab_dtype, int64_t k) { return (int)(ab_dtype == BSG_E2M1X2 ? k / 2 : k); }

// Kernel operand format of a block-scaled ab_dtype (bsg::Fmt values).
int fmt_of(int ab_dtype) { return ab_dtype == BSG_E2M1X2 ? 1 : (ab_dtype == BSG_E5M2 ? 4 : 0); }

}  // namespace

extern "C" {

const char *bsg_status_string(int status)
{
    switch (status) {
    case BSG_OK: return "ok";
    case BSG_ERR_NULLPTR: return "required pointer is NULL";
    case BSG_ERR_SHAPE: return "invalid or inconsistent shape";
    case BSG_ERR_DTYPE: return "invalid dtype";
    case BSG_ERR_ALIGN: return "16-byte alignment violated";
    case BSG_ERR_UNSUPPORTED: return "combination not supported by this library";
    case BSG_ERR_DEVICE: return "device error (not gfx950 or HIP failure)";
    case BSG_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
    }
}

const char *bsg_last_error(void) { return g_err; }

int bsg_version(void) { return 100; }

// Opt-in check of the routing offsets' values (see the header): one copy of
// the num_experts ints to the host and a wait on the stream.
int bsg_check_padded_offsets(const int32_t *padded_offsets, int64_t num_experts, int64_t m, void *stream)
{
    if (!padded_offsets) return fail(BSG_ERR_NULLPTR, "padded_offsets is NULL");
    if (num_experts < 1 || num_experts > 1024)
        return fail(BSG_ERR_SHAPE, "num_experts=%lld must be in [1, 1024]", (long long)num_experts);
    if (m < 0 || m % 256) return fail(BSG_ERR_SHAPE, "m=%lld must be a non-negative multiple of 256", (long long)m);
    if (int r = check_device()) return r;
    int32_t host[1024];
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(host, padded_offsets, (size_t)num_experts * sizeof(int32_t), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(BSG_ERR_LAUNCH, "copying padded_offsets failed: %s", hipGetErrorString(e));
    int64_t prev = 0;
    for (int64_t g = 0; g < num_experts; ++g) {
        const int64_t v = host[g];
        if (v < 0) return fail(BSG_ERR_SHAPE, "padded_offsets[%lld]=%lld is negative", (long long)g, (long long)v);
        if (v % 256)
            return fail(BSG_ERR_SHAPE, "padded_offsets[%lld]=%lld is not a multiple of 256", (long long)g,
                        (long long)v);
        if (v < prev)
            return fail(BSG_ERR_SHAPE, "padded_offsets[%lld]=%lld is below padded_offsets[%lld]=%lld", (long long)g,
                        (long long)v, (long long)(g - 1), (long long)prev);
        if (v > m)
            return fail(BSG_ERR_SHAPE, "padded_offsets[%lld]=%lld exceeds m=%lld", (long long)g, (long long)v,
                        (long long)m);
        prev = v;
    }
    return BSG_OK;
}

// ---------------------------------------------------------------------------
// gemm_amax
// ---------------------------------------------------------------------------
// Launch-shape limits shared by every GEMM: one workgroup per 256x256 tile in
// a 1-D grid (under 2^24 workgroups of 256 threads), 32 output rows of at
// most 4 bytes per element addressable with 32-bit offsets.
static int check_tiles(int64_t m_tiles, int64_t n, int64_t l)
{
    const int64_t tiles = m_tiles * ((n + 255) / 256) * l;
    if (tiles >= (1ll << 24)) return fail(BSG_ERR_UNSUPPORTED, "%lld output tiles exceed the launch limit", (long long)tiles);
    if (n * 4 * 32 >= (1ll << 31)) return fail(BSG_ERR_UNSUPPORTED, "N=%lld too large for 32-bit row offsets", (long long)n);
    return BSG_OK;
}

int bsg_validate_gemm_amax(const void *a, const void *b, const uint8_t *sfa, const uint8_t *sfb,
                           void *c, float *amax, int64_t m, int64_t n, int64_t k, int64_t l,
                           int ab_dtype, int c_dtype, int sf_vec_size, int a_major, int b_major, int c_major)
{
    (void)amax;
    int st = check_ab_sf(ab_dtype, sf_vec_size);
    if (st) return st;
    if (m < 0 || n < 0 || k < 0 || l < 0) return fail(BSG_ERR_SHAPE, "negative size");
    if (k % 32) return fail(BSG_ERR_SHAPE, "K=%lld must be a multiple of sf_vec_size 32", (long long)k);
    if ((a_major != 'k' && a_major != 'm') || (b_major != 'k' && b_major != 'n') ||
        (c_major != 'n' && c_major != 'm'))
        return fail(BSG_ERR_SHAPE, "majors must be a_major 'k'/'m', b_major 'k'/'n', c_major 'n'/'m'");
    const bool fp8_c = c_dtype == BSG_E4M3 || c_dtype == BSG_E5M2, fp4_c = c_dtype == BSG_E2M1X2;
    if (fp8_c && ab_dtype != BSG_E2M1X2)
        return fail(BSG_ERR_UNSUPPORTED, "FP8 C with FP8 A/B is disabled (FP8 C takes FP4 A/B)");
    if (fp4_c && ab_dtype != BSG_E2M1X2) return fail(BSG_ERR_DTYPE, "FP4 C requires FP4 A/B");
    if (!is_float_out(c_dtype) && !fp8_c && !fp4_c)
        return fail(BSG_ERR_DTYPE, "c_dtype %d is not an output dtype", c_dtype);
    // "GEMM + Amax (SM100)", Layouts and strides: packed FP4 A/B are k-major, packed FP4 C n-major
    if (ab_dtype == BSG_E2M1X2 && (a_major != 'k' || b_major != 'k'))
        return fail(BSG_ERR_SHAPE, "packed FP4 A and B must be k-major");
    if (fp4_c && c_major != 'n') return fail(BSG_ERR_SHAPE, "packed FP4 C must be n-major");
    if (m * n * l == 0) return BSG_OK;   // nothing to read or write but amax
    if (!a || !b || !sfa || !sfb || !c) return fail(BSG_ERR_NULLPTR, "a, b, sfa, sfb and c are required");
    if (k > 0 && (!aligned16(a) || !aligned16(b))) return fail(BSG_ERR_ALIGN, "A and B must be 16-byte aligned");
    // C rows run along its contiguous dimension: N (n-major) or M (m-major)
    const int64_t c_row = c_major == 'n' ? n : m;
    if (!aligned16(c) || (fp4_c ? c_row % 32 : (c_row * elem_bytes(c_dtype)) % 16))
        return fail(BSG_ERR_ALIGN, "C must be 16-byte aligned with rows of a multiple of 16 bytes");
    if ((int64_t)row_bytes(ab_dtype, k) * 256 >= (1ll << 31))
        return fail(BSG_ERR_UNSUPPORTED, "K too large for 32-bit tile offsets");
    // MN-major operands: K rows of M (N) one-byte codes, 16-byte aligned, and
    // a batch's K + 256 rows within 32-bit offsets
    if (a_major == 'm' && m % 16) return fail(BSG_ERR_ALIGN, "m-major A needs M %% 16 == 0 (M=%lld)", (long long)m);
    if (b_major == 'n' && n % 16) return fail(BSG_ERR_ALIGN, "n-major B needs N %% 16 == 0 (N=%lld)", (long long)n);
    if ((a_major == 'm' && (k + 256) * m >= (1ll << 31)) || (b_major == 'n' && (k + 256) * n >= (1ll << 31)))
        return fail(BSG_ERR_UNSUPPORTED, "MN-major operand too large for 32-bit offsets");
    return c_major == 'n' ? check_tiles((m + 255) / 256, n, l) : check_tiles((n + 255) / 256, m, l);
}

int gemm_amax(const void *a, const void *b, const uint8_t *sfa, const uint8_t *sfb, void *c,
              float *amax, int64_t m, int64_t n, int64_t k, int64_t l, int ab_dtype, int c_dtype,
              int sf_vec_size, int a_major, int b_major, int c_major, void *stream)
{
    int st = bsg_validate_gemm_amax(a, b, sfa, sfb, c, amax, m, n, k, l, ab_dtype, c_dtype, sf_vec_size,
                                    a_major, b_major, c_major);
    if (st) return st;
    if ((st = check_device())) return st;
    bsg::GemmAmaxArgs args{static_cast<const uint8_t *>(a), static_cast<const uint8_t *>(b), sfa, sfb,
                           c, amax, m, n, k, l, fmt_of(ab_dtype), c_dtype};
    args.a_mn = a_major == 'm';
    args.b_mn = b_major == 'n';
    if (c_major == 'm') {
        // C stored m-major is C^T stored n-major: compute C^T = B A^T, with
        // B (and its scales) as the first operand
        std::swap(args.a, args.b);
        std::swap(args.sfa, args.sfb);
        std::swap(args.m, args.n);
        std::swap(args.a_mn, args.b_mn);
    }
    return launch_status(bsg::launch_gemm_amax(args, static_cast<hipStream_t>(stream)), "gemm_amax");
}

// ---------------------------------------------------------------------------
// Grouped: shared checks
// ---------------------------------------------------------------------------
// b is the weight tensor, or with `discrete` the device array of per-expert
// weight pointers (8-byte aligned; its targets are the caller's contract).
static int check_grouped_common(const void *a, const void *b, const int32_t *offsets,
                                const float *alpha, const float *prob, void *d, int64_t m, int64_t n,
                                int64_t k, int64_t num_experts, bool discrete = false)
{
    if (m < 0 || n < 0 || k < 0) return fail(BSG_ERR_SHAPE, "negative size");
    if (num_experts < 1 || num_experts > 1024)
        return fail(BSG_ERR_SHAPE, "expert count L=%lld must be in [1, 1024]", (long long)num_experts);
    if (m % 256) return fail(BSG_ERR_SHAPE, "M=%lld must be a multiple of 256", (long long)m);
    if (!offsets || !alpha) return fail(BSG_ERR_NULLPTR, "padded_offsets and alpha are required");
    if (!prob) return fail(BSG_ERR_NULLPTR, "prob is required");
    if (m * n == 0) return BSG_OK;
    if (!a || !b || !d) return fail(BSG_ERR_NULLPTR, discrete ? "a, b_ptrs and d are required" : "a, b and d are required");
    if (discrete && (reinterpret_cast<uintptr_t>(b) & 7u)) return fail(BSG_ERR_ALIGN, "b_ptrs must be 8-byte aligned");
    if (k > 0 && (!aligned16(a) || (!discrete && !aligned16(b))))
        return fail(BSG_ERR_ALIGN, "A and B must be 16-byte aligned");
    return check_tiles(m / 256, n, 1);
}

// ---------------------------------------------------------------------------
// grouped_gemm (BF16)
// ---------------------------------------------------------------------------
static int validate_grouped(const void *a, const void *b, const int32_t *padded_offsets,
                            const float *alpha, const float *prob, const void *bias, void *c,
                            void *d, int64_t m, int64_t n, int64_t k, int64_t num_experts,
                            int bias_dtype, int c_dtype, int d_dtype, bool discrete)
{
    int st = check_grouped_common(a, b, padded_offsets, alpha, prob, d, m, n, k, num_experts, discrete);
    if (st) return st;
    if (k % 8) return fail(BSG_ERR_ALIGN, "K=%lld: rows of bf16 A/B must be 16-byte multiples", (long long)k);
    if (!is_float_out(c_dtype) || !is_float_out(d_dtype))
        return fail(BSG_ERR_DTYPE, "C and D dtypes must be F32, F16 or BF16");
    if (bias && !is_float_out(bias_dtype)) return fail(BSG_ERR_DTYPE, "bias dtype must be F32, F16 or BF16");
    if (m * n == 0) return BSG_OK;
    if (!aligned16(d) || (n * elem_bytes(d_dtype)) % 16 || (c && (!aligned16(c) || (n * elem_bytes(c_dtype)) % 16)))
        return fail(BSG_ERR_ALIGN, "C/D must be 16-byte aligned with N*sizeof a multiple of 16");
    if ((int64_t)2 * k * 256 >= (1ll << 31)) return fail(BSG_ERR_UNSUPPORTED, "K too large");
    return BSG_OK;
}

static int run_grouped(const void *a, const void *b, const uint64_t *b_ptrs, const int32_t *padded_offsets,
                       const float *alpha, const float *prob, const void *bias, void *c, void *d,
                       int64_t m, int64_t n, int64_t k, int64_t num_experts, int bias_dtype, int c_dtype,
                       int d_dtype, void *stream, const char *name)
{
    int st = validate_grouped(a, b_ptrs ? static_cast<const void *>(b_ptrs) : b, padded_offsets, alpha, prob,
                              bias, c, d, m, n, k, num_experts, bias_dtype, c_dtype, d_dtype, b_ptrs != nullptr);
    if (st) return st;
    if ((st = check_device())) return st;
    bsg::GroupedArgs args{};
    args.a = static_cast<const uint8_t *>(a); args.b = static_cast<const uint8_t *>(b); args.b_ptrs = b_ptrs;
    args.offsets = padded_offsets; args.alpha = alpha; args.prob = prob; args.bias = bias;
    args.c = c; args.d = d; args.m = m; args.n = n; args.k = k; args.num_experts = num_experts;
    args.fmt = 2; args.c_dtype = c_dtype; args.d_dtype = d_dtype; args.bias_dtype = bias_dtype;
    return launch_status(bsg::launch_grouped_gemm(args, static_cast<hipStream_t>(stream)), name);
}

int bsg_validate_grouped_gemm(const void *a, const void *b, const int32_t *padded_offsets,
                              const float *alpha, const float *prob, const void *bias, void *c,
                              void *d, int64_t m, int64_t n, int64_t k, int64_t num_experts,
                              int bias_dtype, int c_dtype, int d_dtype)
{
    return validate_grouped(a, b, padded_offsets, alpha, prob, bias, c, d, m, n, k, num_experts,
                            bias_dtype, c_dtype, d_dtype, false);
}

int bsg_validate_grouped_gemm_discrete(const void *a, const uint64_t *b_ptrs,
                                       const int32_t *padded_offsets, const float *alpha,
                                       const float *prob, const void *bias, void *c, void *d,
                                       int64_t m, int64_t n, int64_t k, int64_t num_experts,
                                       int bias_dtype, int c_dtype, int d_dtype)
{
    return validate_grouped(a, b_ptrs, padded_offsets, alpha, prob, bias, c, d, m, n, k, num_experts,
                            bias_dtype, c_dtype, d_dtype, true);
}

int grouped_gemm(const void *a, const void *b, const int32_t *padded_offsets, const float *alpha,
                 const float *prob, const void *bias, void *c, void *d, int64_t m, int64_t n,
                 int64_t k, int64_t num_experts, int bias_dtype, int c_dtype, int d_dtype,
                 void *stream)
{
    return run_grouped(a, b, nullptr, padded_offsets, alpha, prob, bias, c, d, m, n, k, num_experts,
                       bias_dtype, c_dtype, d_dtype, stream, "grouped_gemm");
}

int grouped_gemm_discrete(const void *a, const uint64_t *b_ptrs, const int32_t *padded_offsets,
                          const float *alpha, const float *prob, const void *bias, void *c, void *d,
                          int64_t m, int64_t n, int64_t k, int64_t num_experts, int bias_dtype,
                          int c_dtype, int d_dtype, void *stream)
{
    if (!b_ptrs) return fail(BSG_ERR_NULLPTR, "b_ptrs is required");
    return run_grouped(a, nullptr, b_ptrs, padded_offsets, alpha, prob, bias, c, d, m, n, k, num_experts,
                       bias_dtype, c_dtype, d_dtype, stream, "grouped_gemm_discrete");
}

// ---------------------------------------------------------------------------
// grouped_gemm_srelu
// ---------------------------------------------------------------------------
static int validate_srelu(const void *a, const void *b, const uint8_t *sfa, const void *sfb,
                          const int32_t *padded_offsets, const float *alpha, const float *prob,
                          const float *norm_const, void *c, void *d, void *d_col, uint8_t *sfd_row,
                          uint8_t *sfd_col, float *amax, int64_t m, int64_t n, int64_t k,
                          int64_t num_experts, int ab_dtype, int c_dtype, int d_dtype, int sf_vec_size,
                          float tanh_clamp_scale, bool discrete)
{
    (void)amax;
    int st = check_ab_sf(ab_dtype, sf_vec_size);
    if (st) return st;
    if ((st = check_grouped_common(a, b, padded_offsets, alpha, prob, d, m, n, k, num_experts, discrete)))
        return st;
    if (k % 32) return fail(BSG_ERR_SHAPE, "K=%lld must be a multiple of sf_vec_size 32", (long long)k);
    if (n % 32) return fail(BSG_ERR_SHAPE, "N=%lld must be a multiple of 32", (long long)n);
    if (!(tanh_clamp_scale == tanh_clamp_scale)) return fail(BSG_ERR_SHAPE, "tanh_clamp_scale is NaN");
    // C: fp32 / fp16 / bf16, or an unscaled saturating FP8 / packed FP4 cast
    // ("Grouped GEMM + sReLU (SM100)", Input/Output tensors lists all six)
    const bool fp8_c = c_dtype == BSG_E4M3 || c_dtype == BSG_E5M2 || c_dtype == BSG_E2M1X2;
    if (c && !is_float_out(c_dtype) && !fp8_c)
        return fail(BSG_ERR_DTYPE, "C dtype must be F32, F16, BF16, E4M3, E5M2 or E2M1X2");
    // quantised D: E4M3 / E5M2 codes, or E2M1 codes two per byte
    const bool fp8_out = d_dtype == BSG_E4M3 || d_dtype == BSG_E5M2 || d_dtype == BSG_E2M1X2;
    if (!fp8_out && !is_float_out(d_dtype)) return fail(BSG_ERR_DTYPE, "D dtype %d invalid", d_dtype);
    if (fp8_out) {
        if (ab_dtype == BSG_E2M1X2)
            return fail(BSG_ERR_DTYPE, "quantised D requires FP8 A/B (FP4 inputs take fp16/bf16/fp32 D)");
        if (!norm_const || !sfd_row || !sfd_col || !d_col)
            return fail(BSG_ERR_NULLPTR, "quantised D needs norm_const, d_col, sfd_row and sfd_col");
    }
    if (m * n == 0) return BSG_OK;
    if (!sfa || !sfb) return fail(BSG_ERR_NULLPTR, discrete ? "sfa and sfb_ptrs are required" : "sfa and sfb are required");
    if (discrete && (reinterpret_cast<uintptr_t>(sfb) & 7u)) return fail(BSG_ERR_ALIGN, "sfb_ptrs must be 8-byte aligned");
    const int db = fp8_out ? 1 : elem_bytes(d_dtype);
    const int64_t c_row = c_dtype == BSG_E2M1X2 ? n / 2 : n * elem_bytes(c_dtype);
    if (!aligned16(d) || (n * db) % 16 || (d_col && !aligned16(d_col)) ||
        (c && (!aligned16(c) || c_row % 16)))
        return fail(BSG_ERR_ALIGN, "C/D/D_col must be 16-byte aligned with 16-byte rows");
    if (fp8_out && ((reinterpret_cast<uintptr_t>(sfd_row) | reinterpret_cast<uintptr_t>(sfd_col)) & 3u))
        return fail(BSG_ERR_ALIGN, "sfd_row and sfd_col must be 4-byte aligned");
    if ((int64_t)row_bytes(ab_dtype, k) * 256 >= (1ll << 31)) return fail(BSG_ERR_UNSUPPORTED, "K too large");
    return BSG_OK;
}

static int run_srelu(const void *a, const void *b, const uint64_t *b_ptrs, const uint8_t *sfa,
                     const uint8_t *sfb, const uint64_t *sfb_ptrs, const int32_t *padded_offsets,
                     const float *alpha, const float *prob, const float *norm_const, void *c, void *d,
                     void *d_col, uint8_t *sfd_row, uint8_t *sfd_col, float *amax, int64_t m, int64_t n,
                     int64_t k, int64_t num_experts, int ab_dtype, int c_dtype, int d_dtype,
                     int sf_vec_size, float tanh_clamp_scale, void *stream, const char *name)
{
    const bool discrete = b_ptrs != nullptr;
    int st = validate_srelu(a, discrete ? static_cast<const void *>(b_ptrs) : b, sfa,
                            discrete ? static_cast<const void *>(sfb_ptrs) : sfb, padded_offsets, alpha,
                            prob, norm_const, c, d, d_col, sfd_row, sfd_col, amax, m, n, k, num_experts,
                            ab_dtype, c_dtype, d_dtype, sf_vec_size, tanh_clamp_scale, discrete);
    if (st) return st;
    if ((st = check_device())) return st;
    bsg::GroupedArgs args{};
    args.a = static_cast<const uint8_t *>(a); args.b = static_cast<const uint8_t *>(b);
    args.b_ptrs = b_ptrs; args.sfb_ptrs = sfb_ptrs;
    args.sfa = sfa; args.sfb = sfb; args.offsets = padded_offsets; args.alpha = alpha;
    args.prob = prob; args.norm_const = norm_const; args.c = c; args.d = d; args.d_col = d_col;
    args.sfd_row = sfd_row; args.sfd_col = sfd_col;
    args.amax = (d_dtype == BSG_E4M3 || d_dtype == BSG_E5M2 || d_dtype == BSG_E2M1X2) ? nullptr : amax;
    args.m = m; args.n = n; args.k = k; args.num_experts = num_experts;
    args.fmt = fmt_of(ab_dtype); args.c_dtype = c_dtype; args.d_dtype = d_dtype;
    args.tanh_s = tanh_clamp_scale > 0.0f ? tanh_clamp_scale : 0.0f;
    return launch_status(bsg::launch_grouped_srelu(args, static_cast<hipStream_t>(stream)), name);
}

int bsg_validate_grouped_gemm_srelu(const void *a, const void *b, const uint8_t *sfa,
                                    const uint8_t *sfb, const int32_t *padded_offsets,
                                    const float *alpha, const float *prob, const float *norm_const,
                                    void *c, void *d, void *d_col, uint8_t *sfd_row,
                                    uint8_t *sfd_col, float *amax, int64_t m, int64_t n, int64_t k,
                                    int64_t num_experts, int ab_dtype, int c_dtype, int d_dtype,
                                    int sf_vec_size, float tanh_clamp_scale)
{
    return validate_srelu(a, b, sfa, sfb, padded_offsets, alpha, prob, norm_const, c, d, d_col, sfd_row,
                          sfd_col, amax, m, n, k, num_experts, ab_dtype, c_dtype, d_dtype, sf_vec_size,
                          tanh_clamp_scale, false);
}

int bsg_validate_grouped_gemm_srelu_discrete(const void *a, const uint64_t *b_ptrs,
                                             const uint8_t *sfa, const uint64_t *sfb_ptrs,
                                             const int32_t *padded_offsets, const float *alpha,
                                             const float *prob, const float *norm_const, void *c,
                                             void *d, void *d_col, uint8_t *sfd_row,
                                             uint8_t *sfd_col, float *amax, int64_t m, int64_t n,
                                             int64_t k, int64_t num_experts, int ab_dtype,
                                             int c_dtype, int d_dtype, int sf_vec_size,
                                             float tanh_clamp_scale)
{
    return validate_srelu(a, b_ptrs, sfa, sfb_ptrs, padded_offsets, alpha, prob, norm_const, c, d, d_col,
                          sfd_row, sfd_col, amax, m, n, k, num_experts, ab_dtype, c_dtype, d_dtype,
                          sf_vec_size, tanh_clamp_scale, true);
}

int grouped_gemm_srelu(const void *a, const void *b, const uint8_t *sfa, const uint8_t *sfb,
                       const int32_t *padded_offsets, const float *alpha, const float *prob,
                       const float *norm_const, void *c, void *d, void *d_col, uint8_t *sfd_row,
                       uint8_t *sfd_col, float *amax, int64_t m, int64_t n, int64_t k,
                       int64_t num_experts, int ab_dtype, int c_dtype, int d_dtype, int sf_vec_size,
                       float tanh_clamp_scale, void *stream)
{
    return run_srelu(a, b, nullptr, sfa, sfb, nullptr, padded_offsets, alpha, prob, norm_const, c, d, d_col,
                     sfd_row, sfd_col, amax, m, n, k, num_experts, ab_dtype, c_dtype, d_dtype, sf_vec_size,
                     tanh_clamp_scale, stream, "grouped_gemm_srelu");
}

int grouped_gemm_srelu_discrete(const void *a, const uint64_t *b_ptrs, const uint8_t *sfa,
                                const uint64_t *sfb_ptrs, const int32_t *padded_offsets,
                                const float *alpha, const float *prob, const float *norm_const,
                                void *c, void *d, void *d_col, uint8_t *sfd_row, uint8_t *sfd_col,
                                float *amax, int64_t m, int64_t n, int64_t k, int64_t num_experts,
                                int ab_dtype, int c_dtype, int d_dtype, int sf_vec_size,
                                float tanh_clamp_scale, void *stream)
{
    if (!b_ptrs) return fail(BSG_ERR_NULLPTR, "b_ptrs is required");
    return run_srelu(a, nullptr, b_ptrs, sfa, nullptr, sfb_ptrs, padded_offsets, alpha, prob, norm_const, c,
                     d, d_col, sfd_row, sfd_col, amax, m, n, k, num_experts, ab_dtype, c_dtype, d_dtype,
                     sf_vec_size, tanh_clamp_scale, stream, "grouped_gemm_srelu_discrete");
}

// ---------------------------------------------------------------------------
// grouped_gemm_dswiglu
// ---------------------------------------------------------------------------
int bsg_validate_grouped_gemm_dswiglu(const void *a, const void *b, const uint8_t *sfa, const uint8_t *sfb,
                                      const void *c, const int32_t *padded_offsets, const float *alpha,
                                      const float *beta, const float *prob, const float *norm_const,
                                      void *d_row, void *d_col, uint8_t *sfd_row, uint8_t *sfd_col,
                                      float *dprob, float *amax, int64_t m, int64_t n, int64_t k,
                                      int64_t num_experts, int ab_dtype, int c_dtype, int d_dtype,
                                      int sf_vec_size, int b_major)
{
    int st = check_ab_sf(ab_dtype, sf_vec_size);
    if (st) return st;
    // "Grouped GEMM + dSwiGLU (SM100)", Layouts and strides: B k-major or
    // n-major, k-major for FP4 inputs
    if (b_major != 'k' && b_major != 'n') return fail(BSG_ERR_SHAPE, "b_major must be 'k' or 'n'");
    if (b_major == 'n' && ab_dtype == BSG_E2M1X2) return fail(BSG_ERR_SHAPE, "packed FP4 B must be k-major");
    if ((st = check_grouped_common(a, b, padded_offsets, alpha, prob, d_row, m, n, k, num_experts)))
        return st;
    if (k % 32) return fail(BSG_ERR_SHAPE, "K=%lld must be a multiple of sf_vec_size 32", (long long)k);
    if (n % 32) return fail(BSG_ERR_SHAPE, "N=%lld must be a multiple of 32", (long long)n);
    const bool fp4 = ab_dtype == BSG_E2M1X2;
    if (c_dtype != BSG_BF16) {
        if (is_float_out(c_dtype) || c_dtype == BSG_E4M3 || c_dtype == BSG_E5M2)
            return fail(BSG_ERR_UNSUPPORTED, "C dtype %d is not built (BF16 is)", c_dtype);
        return fail(BSG_ERR_DTYPE, "C dtype %d invalid", c_dtype);
    }
    if (fp4) {
        // FP4 inputs: bf16 / fp32 D (d_col an optional copy), per-expert amax (L, 2) nullable
        if (d_dtype != BSG_BF16 && d_dtype != BSG_F32) return fail(BSG_ERR_DTYPE, "FP4 inputs take a bf16 or fp32 D");
    } else if (d_dtype != BSG_E4M3 && d_dtype != BSG_E5M2) {
        return fail(BSG_ERR_DTYPE, "FP8 inputs take an FP8 (E4M3 or E5M2) D");
    }
    if (!beta) return fail(BSG_ERR_NULLPTR, "beta is required");
    if (!dprob) return fail(BSG_ERR_NULLPTR, "dprob is required");
    if (!fp4 && (!norm_const || !d_col || !sfd_row || !sfd_col))
        return fail(BSG_ERR_NULLPTR, "FP8 D needs norm_const, d_col, sfd_row and sfd_col");
    if (m * n == 0) return BSG_OK;
    if (!c) return fail(BSG_ERR_NULLPTR, "c is required");
    if (!sfa || !sfb) return fail(BSG_ERR_NULLPTR, "sfa and sfb are required");
    if (!aligned16(c) || !aligned16(d_row) || (d_col && !aligned16(d_col)))
        return fail(BSG_ERR_ALIGN, "C, D_row and D_col must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(sfd_row) | reinterpret_cast<uintptr_t>(sfd_col) |
         reinterpret_cast<uintptr_t>(dprob) | reinterpret_cast<uintptr_t>(amax)) & 3u)
        return fail(BSG_ERR_ALIGN, "sfd_row, sfd_col, dprob and amax must be 4-byte aligned");
    if ((int64_t)row_bytes(ab_dtype, k) * 256 >= (1ll << 31) || m * 2 * n >= (1ll << 31))
        return fail(BSG_ERR_UNSUPPORTED, "K or M*2N too large");
    if (b_major == 'n' && (k + 256) * n >= (1ll << 31))
        return fail(BSG_ERR_UNSUPPORTED, "n-major B too large for 32-bit offsets");
    return BSG_OK;
}

int grouped_gemm_dswiglu(const void *a, const void *b, const uint8_t *sfa, const uint8_t *sfb, const void *c,
                         const int32_t *padded_offsets, const float *alpha, const float *beta,
                         const float *prob, const float *norm_const, void *d_row, void *d_col,
                         uint8_t *sfd_row, uint8_t *sfd_col, float *dprob, float *amax, int64_t m, int64_t n,
                         int64_t k, int64_t num_experts, int ab_dtype, int c_dtype, int d_dtype,
                         int sf_vec_size, int b_major, void *stream)
{
    int st = bsg_validate_grouped_gemm_dswiglu(a, b, sfa, sfb, c, padded_offsets, alpha, beta, prob, norm_const,
                                               d_row, d_col, sfd_row, sfd_col, dprob, amax, m, n, k, num_experts,
                                               ab_dtype, c_dtype, d_dtype, sf_vec_size, b_major);
    if (st) return st;
    if ((st = check_device())) return st;
    bsg::GroupedArgs args{};
    args.a = static_cast<const uint8_t *>(a); args.b = static_cast<const uint8_t *>(b);
    args.sfa = sfa; args.sfb = sfb; args.offsets = padded_offsets; args.alpha = alpha;
    args.prob = prob; args.norm_const = norm_const; args.d = d_row; args.d_col = d_col;
    args.sfd_row = sfd_row; args.sfd_col = sfd_col;
    args.m = m; args.n = n; args.k = k; args.num_experts = num_experts;
    args.fmt = fmt_of(ab_dtype); args.c_dtype = c_dtype; args.d_dtype = d_dtype;
    args.beta = beta; args.cfwd = static_cast<const uint16_t *>(c); args.dprob = dprob;
    args.amax = ab_dtype == BSG_E2M1X2 ? amax : nullptr;
    args.b_mn = b_major == 'n';
    return launch_status(bsg::launch_grouped_dswiglu(args, static_cast<hipStream_t>(stream)),
                         "grouped_gemm_dswiglu");
}

// ---------------------------------------------------------------------------
// gemm_proj_rope_mxfp8
// ---------------------------------------------------------------------------
int bsg_validate_gemm_proj_rope_mxfp8(const void *x, const void *w, const uint8_t *x_scale,
                                      const uint8_t *w_scale, const void *cos, const void *sin,
                                      uint8_t *out_fp8_row, uint8_t *out_scales_row,
                                      uint8_t *out_fp8_col, uint8_t *out_scales_col,
                                      int64_t tokens, int64_t q_lora, int64_t num_heads,
                                      int64_t head_dim, int64_t qk_rope, int in_dtype, int w_out_in)
{
    if (in_dtype != BSG_BF16 && in_dtype != BSG_E4M3) return fail(BSG_ERR_DTYPE, "x/w dtype must be BF16 or E4M3");
    const bool mx = in_dtype == BSG_E4M3;
    if (!mx && (x_scale || w_scale)) return fail(BSG_ERR_SHAPE, "x_scale/w_scale must be NULL for BF16 inputs");
    if (tokens < 0 || q_lora < 0 || num_heads < 0) return fail(BSG_ERR_SHAPE, "negative size");
    if (tokens % 128) return fail(BSG_ERR_SHAPE, "tokens=%lld must be a multiple of 128", (long long)tokens);
    if (q_lora % 32) return fail(BSG_ERR_SHAPE, "q_lora must be a multiple of 32");
    if (head_dim != 192 || qk_rope != 64)
        return fail(BSG_ERR_UNSUPPORTED, "only head_dim 192 with qk_rope 64 is built");
    if (w_out_in != 0 && w_out_in != 1) return fail(BSG_ERR_SHAPE, "w_out_in must be 0 or 1");
    // w as [in, out] (w_out_in = 0, the page's default layout): with MXFP8
    // inputs one head's w_scale columns are staged in LDS, which holds up to
    // 64 scale bytes per feature
    if (!w_out_in && mx && q_lora > 2048)
        return fail(BSG_ERR_UNSUPPORTED, "MXFP8 inputs with w as [in, out] need q_lora <= 2048");
    if (!w_out_in && (q_lora + 256) * (mx ? 1 : 2) * num_heads * head_dim >= (1ll << 31))
        return fail(BSG_ERR_UNSUPPORTED, "w as [in, out] too large for 32-bit offsets");
    if (mx && q_lora % 128)
        return fail(BSG_ERR_UNSUPPORTED, "MXFP8 inputs need q_lora to be a multiple of 128");
    if (tokens * num_heads == 0) return BSG_OK;
    if (mx && (!x_scale || !w_scale)) return fail(BSG_ERR_NULLPTR, "x_scale and w_scale are required for E4M3 inputs");
    if (mx && ((uintptr_t)x_scale % 4 || (uintptr_t)w_scale % 4))
        return fail(BSG_ERR_ALIGN, "x_scale and w_scale must be 4-byte aligned");
    if (!x || !w || !cos || !sin || !out_fp8_row || !out_scales_row || !out_fp8_col || !out_scales_col)
        return fail(BSG_ERR_NULLPTR, "all tensors are required");
    if (!aligned16(x) || !aligned16(w) || !aligned16(out_fp8_row) || !aligned16(out_fp8_col) ||
        !aligned16(cos) || !aligned16(sin))
        return fail(BSG_ERR_ALIGN, "x, w, cos, sin and the fp8 outputs must be 16-byte aligned");
    return BSG_OK;
}

int gemm_proj_rope_mxfp8(const void *x, const void *w, const uint8_t *x_scale, const uint8_t *w_scale,
                         const void *cos, const void *sin, uint8_t *out_fp8_row,
                         uint8_t *out_scales_row, uint8_t *out_fp8_col, uint8_t *out_scales_col,
                         int64_t tokens, int64_t q_lora, int64_t num_heads, int64_t head_dim,
                         int64_t qk_rope, int in_dtype, int w_out_in, void *stream)
{
    int st = bsg_validate_gemm_proj_rope_mxfp8(x, w, x_scale, w_scale, cos, sin, out_fp8_row,
                                               out_scales_row, out_fp8_col, out_scales_col, tokens,
                                               q_lora, num_heads, head_dim, qk_rope, in_dtype, w_out_in);
    if (st) return st;
    if ((st = check_device())) return st;
    bsg::ProjRopeArgs args{x, w, x_scale, w_scale,
                           static_cast<const uint16_t *>(cos), static_cast<const uint16_t *>(sin),
                           out_fp8_row, out_scales_row, out_fp8_col, out_scales_col,
                           tokens, q_lora, num_heads, head_dim, qk_rope, w_out_in,
                           in_dtype == BSG_E4M3 ? 1 : 0};
    return launch_status(bsg::launch_proj_rope(args, static_cast<hipStream_t>(stream)),
                         "gemm_proj_rope_mxfp8");
}

}  // extern "C"
