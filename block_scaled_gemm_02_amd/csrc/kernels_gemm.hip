// Dense and grouped block-scaled GEMM kernels for gfx950.
//
//   k_gemm_amax      "GEMM + Amax (SM100)": C = sum_k A_hat B_hat per batch,
//                    Amax = max |C| (one atomicMax per workgroup).
//   k_grouped        "Grouped GEMM (SM100 BF16)" and "Grouped GEMM + sReLU
//                    (SM100)": tiles of 256 rows never straddle an expert
//                    because every padded_offsets entry is a multiple of 256.
#include "device.hpp"
#include "launch.hpp"

namespace bsg {

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_E4M3 = 3 };

__device__ __forceinline__ void store_elem(void *base, int64_t idx, float v, int dtype)
{
    if (dtype == DT_F32) {
        static_cast<float *>(base)[idx] = v;
    } else if (dtype == DT_BF16) {
        static_cast<uint16_t *>(base)[idx] = f32_to_bf16_rne(v);
    } else {
        static_cast<uint16_t *>(base)[idx] = f32_to_f16_rne(v);
    }
}

__device__ __forceinline__ float load_elem(const void *base, int64_t idx, int dtype)
{
    if (dtype == DT_F32) return static_cast<const float *>(base)[idx];
    uint16_t h = static_cast<const uint16_t *>(base)[idx];
    if (dtype == DT_BF16) return __uint_as_float((uint32_t)h << 16);
    return (float)__builtin_bit_cast(_Float16, h);
}

__global__ void k_fill_zero(float *p, int64_t n)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

static hipError_t zero_floats(float *p, int64_t n, hipStream_t s)
{
    if (!p || n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

static inline uint32_t row_bytes_of(int fmt, int64_t k)
{
    return (uint32_t)(fmt == FMT_E2M1 ? k / 2 : (fmt == FMT_BF16 ? 2 * k : k));
}

// ---------------------------------------------------------------------------
// Dense batched GEMM + global amax
// ---------------------------------------------------------------------------
struct GemmAmaxParams {
    const uint8_t *a, *b, *sfa, *sfb;
    void *c;
    float *amax;
    int64_t m, n, k;
    int64_t m_t, n_t, k_t;   // ceil(M/128), ceil(N/128), ceil(K/128)
    uint32_t row_bytes;
    int c_dtype;
};

template <int F>
__global__ void __launch_bounds__(256) k_gemm_amax(GemmAmaxParams p)
{
    BSG_DECLARE_RING(F, ring);
    __shared__ float red[4];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6, wm = w >> 1, wn = w & 1;
    const int64_t batch = blockIdx.z;
    const int64_t m0 = (int64_t)blockIdx.y * kTileM, n0 = (int64_t)blockIdx.x * kTileN;
    const int64_t rows_a = p.m - m0 < kTileM ? p.m - m0 : kTileM;
    const int64_t rows_b = p.n - n0 < kTileN ? p.n - n0 : kTileN;

    OperandDesc A{p.a + (batch * p.m + m0) * p.row_bytes, (uint32_t)(rows_a * p.row_bytes),
                  p.row_bytes, p.sfa, batch, p.m_t, p.k_t, m0 / 128, p.m_t - 1};
    OperandDesc B{p.b + (batch * p.n + n0) * p.row_bytes, (uint32_t)(rows_b * p.row_bytes),
                  p.row_bytes, p.sfb, batch, p.n_t, p.k_t, n0 / 128, p.n_t - 1};
    f32x16 acc[4][4];
    mainloop_pipe<F>(acc, ring, A, B, p.k);

    float lmax = 0.0f;
    const int64_t cbase = batch * p.m * p.n;
    for_each_row_quad<4>(acc, wm, wn, lane, [&](auto, auto, auto, int row, int col0, float (&x)[4]) {
        const int64_t r = m0 + row, c = n0 + col0;
        if (r < p.m && c < p.n) {       // N is a multiple of 4: a quad is all in or all out
            store4(p.c, cbase + r * p.n + c, x, p.c_dtype);
            lmax = fmaxf(lmax, fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3]))));
        }
    });
    if (p.amax) block_amax_atomic(lmax, p.amax, red);
}

hipError_t launch_gemm_amax(const GemmAmaxArgs &a, hipStream_t s)
{
    hipError_t e = zero_floats(a.amax, 1, s);
    if (e != hipSuccess) return e;
    if (a.m == 0 || a.n == 0 || a.l == 0) return hipSuccess;
    GemmAmaxParams p;
    p.a = a.a; p.b = a.b; p.sfa = a.sfa; p.sfb = a.sfb; p.c = a.c; p.amax = a.amax;
    p.m = a.m; p.n = a.n; p.k = a.k;
    p.m_t = (a.m + 127) / 128; p.n_t = (a.n + 127) / 128; p.k_t = (a.k + 127) / 128;
    p.row_bytes = row_bytes_of(a.fmt, a.k);
    p.c_dtype = a.c_dtype;
    dim3 grid((unsigned)((a.n + kTileN - 1) / kTileN), (unsigned)((a.m + kTileM - 1) / kTileM),
              (unsigned)a.l);
    if (a.fmt == FMT_E4M3)
        hipLaunchKernelGGL(k_gemm_amax<FMT_E4M3>, grid, dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL(k_gemm_amax<FMT_E2M1>, grid, dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Grouped GEMM over padded_offsets expert ranges
// ---------------------------------------------------------------------------
enum : int { EPI_BF16_BIAS = 0, EPI_SRELU = 1, EPI_SRELU_FP8 = 2 };

struct GroupedParams {
    const uint8_t *a, *b, *sfa, *sfb;
    const int32_t *offsets;
    const float *alpha, *prob, *norm_const;
    const void *bias;
    void *c, *d, *d_col;
    uint8_t *sfd_row, *sfd_col;
    float *amax;
    int64_t m, n, k, num_experts;
    int64_t m_t, n_t, k_t;
    uint32_t row_bytes;
    int c_dtype, d_dtype, bias_dtype;
    float tanh_s, tanh_inv_s;
};

// Index of the expert whose range [offsets[g-1], offsets[g]) holds row r:
// the number of offsets <= r (offsets are nondecreasing).
__device__ __forceinline__ int expert_of(const int32_t *offsets, int num, int64_t r)
{
    int lo = 0, hi = num;   // first g with offsets[g] > r
    while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if ((int64_t)offsets[mid] > r) hi = mid;
        else lo = mid + 1;
    }
    return lo;
}

// sReLU value of one accumulator: alpha*acc -> relu -> optional tanh clamp
// -> prob * x^2 (fp32, "Grouped GEMM + sReLU (SM100)" Equations).
__device__ __forceinline__ float srelu_value(float gval, float pr, float s, float inv_s)
{
    float x = fmaxf(gval, 0.0f);
    if (s > 0.0f) x = s * fminf(1.0f, tanh_pos(x * inv_s));
    return pr * x * x;
}

// MXFP8 output: D quantised in 32-wide blocks along N (codes to d, scales to
// the SFD_row atoms over (M, N)) and in 32-tall blocks along M (codes to
// d_col, scales to the SFD_col atoms over (N, M)), with the quantiser of
// "Grouped GEMM + dSwiGLU (SM100)", Step 3 (rcp_max = 1/448).
//
// Works in the transposed accumulator layout, where a 32x32 block (i, j) of
// the wave holds, per lane, 4 columns of 4 rows: a column's 32 values sit in
// one quad of each half-wave, a row's 32 values in 8 lanes of one half-wave.
// C (pre-activation) is written first when requested.
__device__ __forceinline__ void epilogue_srelu_fp8(const GroupedParams &p, f32x16 (&acc)[4][4],
                                                   int64_t m0, int64_t n0, float alpha, int wm,
                                                   int wn, int lane)
{
    const float nc = *p.norm_const;
    const int64_t n = p.n;
    const int64_t row_kt = (n / 32 + 3) / 4;          // SFD_row: K' over N
    const int64_t col_kt = (p.m / 32 + 3) / 4;        // SFD_col: K' over M
    uint8_t *dq = static_cast<uint8_t *>(p.d);
    uint8_t *dc = static_cast<uint8_t *>(p.d_col);
    const int t = lane & 3, c32 = lane & 31, gh = lane >> 5;

    transpose_acc<4>(acc, lane);
    static_for<4>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t r = m0 + tr_row(wm, i, q, lane);
            const float pr = p.prob[r];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t c = n0 + tr_col<4>(wn, j, lane);
                float x[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) x[u] = alpha * acc[i][j][4 * q + u];
                if (p.c && c < n) store4(p.c, r * n + c, x, p.c_dtype);
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    acc[i][j][4 * q + u] = srelu_value(x[u], pr, p.tanh_s, p.tanh_inv_s);
            }
        }
    });

    uint32_t rword[4][4] = {};                        // SFD_row bytes j = 0..3 of each row
    static_for<4>([&](auto jj) {
        constexpr int j = decltype(jj)::value;
        const int64_t c = n0 + tr_col<4>(wn, j, lane);
        uint32_t cword = 0;                           // SFD_col bytes i = 0..3 of column c + t
        static_for<4>([&](auto ii) {
            constexpr int i = decltype(ii)::value;
            float cm[4], cinv[4];
            tr_col_absmax(acc[i][j], cm);
            uint32_t cb[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) cb[u] = mx_scale_byte(cm[u], nc, cinv[u]);
            cword |= (t == 0 ? cb[0] : t == 1 ? cb[1] : t == 2 ? cb[2] : cb[3]) << (8 * i);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float x[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                    acc[i][j][4 * q + 3]};
                float rm = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
                rm = row8_max(rm);
                float rinv;
                const uint32_t rb = mx_scale_byte(rm, nc, rinv);
                rword[i][q] |= rb << (8 * j);
                if (c < n) {
                    const int64_t r = m0 + tr_row(wm, i, q, lane);
                    *reinterpret_cast<uint32_t *>(dq + r * n + c) =
                        pack4_e4m3(x[0] * rinv, x[1] * rinv, x[2] * rinv, x[3] * rinv);
                    *reinterpret_cast<uint32_t *>(dc + r * n + c) =
                        pack4_e4m3(x[0] * cinv[0], x[1] * cinv[1], x[2] * cinv[2], x[3] * cinv[3]);
                }
            }
        });
        if (gh == 0 && c < n) {
            // column c + t, the wave's four 32-row blocks = one K' group of SFD_col
            const int64_t col = c + t;
            const int64_t mt = (m0 + 128 * wm) / 128;
            const int64_t off = (((col / 128) * col_kt + mt) * 32 + (col % 32)) * 16 + ((col % 128) / 32) * 4;
            *reinterpret_cast<uint32_t *>(p.sfd_col + off) = cword;
        }
    });
    if (c32 < 4 && n0 + 128 * wn < n) {
        // row r, the wave's four 32-column blocks = one K' group of SFD_row
        const int64_t kt = (n0 + 128 * wn) / 128;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t r = m0 + tr_row(wm, i, q, lane);
                const int64_t off = (((r / 128) * row_kt + kt) * 32 + (r % 32)) * 16 + ((r % 128) / 32) * 4;
                *reinterpret_cast<uint32_t *>(p.sfd_row + off) = rword[i][q];
            }
        }
    }
}

template <int F, int EPI>
__global__ void __launch_bounds__(256) k_grouped(GroupedParams p)
{
    BSG_DECLARE_RING(F, ring);
    __shared__ float red[4];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6, wm = w >> 1, wn = w & 1;
    const int64_t m0 = (int64_t)blockIdx.y * kTileM, n0 = (int64_t)blockIdx.x * kTileN;
    const int64_t valid_m = p.offsets[p.num_experts - 1];
    if (m0 >= valid_m) return;                      // uniform per workgroup
    const int g = expert_of(p.offsets, (int)p.num_experts, m0);
    const int64_t rows_b = p.n - n0 < kTileN ? p.n - n0 : kTileN;

    OperandDesc A{p.a + m0 * p.row_bytes, (uint32_t)(kTileM * p.row_bytes), p.row_bytes, p.sfa,
                  0, p.m_t, p.k_t, m0 / 128, p.m_t - 1};
    OperandDesc B{p.b + ((int64_t)g * p.n + n0) * p.row_bytes, (uint32_t)(rows_b * p.row_bytes),
                  p.row_bytes, p.sfb, g, p.n_t, p.k_t, n0 / 128, p.n_t - 1};
    f32x16 acc[4][4];
    mainloop_pipe<F>(acc, ring, A, B, p.k);

    const float alpha = p.alpha[g];
    if constexpr (EPI == EPI_SRELU_FP8) {
        epilogue_srelu_fp8(p, acc, m0, n0, alpha, wm, wn, lane);
    } else {
        float lmax = 0.0f;
        transpose_acc<4>(acc, lane);
        static_for<4>([&](auto ii) {
            constexpr int i = decltype(ii)::value;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t r = m0 + tr_row(wm, i, q, lane);
                const float pr = p.prob[r];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int64_t c = n0 + tr_col<4>(wn, j, lane);
                    if (c >= p.n) continue;         // N is a multiple of 8: runs of 4 are whole
                    const int64_t idx = r * p.n + c;
                    float cv[4], dv[4];
                    if constexpr (EPI == EPI_BF16_BIAS) {
                        // "Grouped GEMM (SM100 BF16)", Operation: with bias C = G + prob*bias,
                        // D = C; without bias C = G, D = prob*G.
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const float gval = alpha * acc[i][j][4 * q + u];
                            if (p.bias) {
                                cv[u] = gval + pr * load_elem(p.bias, (int64_t)g * p.n + c + u, p.bias_dtype);
                                dv[u] = cv[u];
                            } else {
                                cv[u] = gval;
                                dv[u] = pr * gval;
                            }
                        }
                        if (p.c) store4(p.c, idx, cv, p.c_dtype);
                        store4(p.d, idx, dv, p.d_dtype);
                    } else {
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            cv[u] = alpha * acc[i][j][4 * q + u];
                            dv[u] = srelu_value(cv[u], pr, p.tanh_s, p.tanh_inv_s);
                            lmax = fmaxf(lmax, fabsf(dv[u]));
                        }
                        if (p.c) store4(p.c, idx, cv, p.c_dtype);
                        store4(p.d, idx, dv, p.d_dtype);
                        if (p.d_col) store4(p.d_col, idx, dv, p.d_dtype);
                    }
                }
            }
        });
        if constexpr (EPI == EPI_SRELU) {
            if (p.amax) block_amax_atomic(lmax, p.amax + g, red);
        }
    }
}

static GroupedParams grouped_params(const GroupedArgs &a)
{
    GroupedParams p;
    p.a = a.a; p.b = a.b; p.sfa = a.sfa; p.sfb = a.sfb; p.offsets = a.offsets;
    p.alpha = a.alpha; p.prob = a.prob; p.norm_const = a.norm_const; p.bias = a.bias;
    p.c = a.c; p.d = a.d; p.d_col = a.d_col; p.amax = a.amax;
    p.sfd_row = a.sfd_row; p.sfd_col = a.sfd_col;
    p.m = a.m; p.n = a.n; p.k = a.k; p.num_experts = a.num_experts;
    p.m_t = (a.m + 127) / 128; p.n_t = (a.n + 127) / 128; p.k_t = (a.k + 127) / 128;
    p.row_bytes = row_bytes_of(a.fmt, a.k);
    p.c_dtype = a.c_dtype; p.d_dtype = a.d_dtype; p.bias_dtype = a.bias_dtype;
    p.tanh_s = a.tanh_s;
    p.tanh_inv_s = a.tanh_s > 0.0f ? 1.0f / a.tanh_s : 0.0f;
    return p;
}

hipError_t launch_grouped_gemm(const GroupedArgs &a, hipStream_t s)
{
    if (a.m == 0 || a.n == 0) return hipSuccess;
    GroupedParams p = grouped_params(a);
    dim3 grid((unsigned)((a.n + kTileN - 1) / kTileN), (unsigned)(a.m / kTileM));
    hipLaunchKernelGGL((k_grouped<FMT_BF16, EPI_BF16_BIAS>), grid, dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_grouped_srelu(const GroupedArgs &a, hipStream_t s)
{
    hipError_t e = zero_floats(a.amax, a.num_experts, s);
    if (e != hipSuccess) return e;
    if (a.m == 0 || a.n == 0) return hipSuccess;
    GroupedParams p = grouped_params(a);
    dim3 grid((unsigned)((a.n + kTileN - 1) / kTileN), (unsigned)(a.m / kTileM));
    if (a.d_dtype == DT_E4M3) {
        if (a.fmt != FMT_E4M3) return hipErrorNotSupported;
        hipLaunchKernelGGL((k_grouped<FMT_E4M3, EPI_SRELU_FP8>), grid, dim3(kThreads), 0, s, p);
    } else if (a.fmt == FMT_E4M3)
        hipLaunchKernelGGL((k_grouped<FMT_E4M3, EPI_SRELU>), grid, dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL((k_grouped<FMT_E2M1, EPI_SRELU>), grid, dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace bsg
