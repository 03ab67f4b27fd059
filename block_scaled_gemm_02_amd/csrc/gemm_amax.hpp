// "GEMM + Amax (SM100)": C = sum_k A_hat B_hat per batch, Amax = max |C|
// (one atomicMax per workgroup).  The kernel template is shared by
// kernels_amax.hip (k-major operands) and kernels_amax_mn.hip (m-major A
// and / or n-major B).
#pragma once
#include "kernels_common.hpp"

namespace bsg {

struct GemmAmaxParams {
    const uint8_t *a, *b, *sfa, *sfb;
    void *c;
    float *amax;
    int64_t m, n, k;
    int64_t m_t, n_t, k_t;   // ceil(M/128), ceil(N/128), ceil(K/128)
    uint32_t row_bytes;
    int c_dtype;
};

// CT: the C store type, a compile-time choice (one store path per kernel
// keeps the epilogue free of register spills).
template <int F, int CT>
__global__ void __launch_bounds__(256) k_gemm_amax(GemmAmaxParams p)
{
    BSG_DECLARE_RING(F, ring);
    __shared__ float red[4];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6, wm = w >> 1, wn = w & 1;
    const int64_t m_tiles = (p.m + kTileM - 1) / kTileM, n_tiles = (p.n + kTileN - 1) / kTileN;
    const TileCoord tc = tile_of(blockIdx.x, m_tiles, n_tiles, (int64_t)gridDim.x);
    const int64_t batch = tc.l;
    const int64_t m0 = tc.mt * kTileM, n0 = tc.nt * kTileN;
    const int64_t rows_a = p.m - m0 < kTileM ? p.m - m0 : kTileM;
    const int64_t rows_b = p.n - n0 < kTileN ? p.n - n0 : kTileN;

    OperandDesc A{p.a + (batch * p.m + m0) * p.row_bytes, (uint32_t)(rows_a * p.row_bytes),
                  p.row_bytes, p.sfa, batch, p.m_t, p.k_t, m0 / 128, p.m_t - 1};
    OperandDesc B{p.b + (batch * p.n + n0) * p.row_bytes, (uint32_t)(rows_b * p.row_bytes),
                  p.row_bytes, p.sfb, batch, p.n_t, p.k_t, n0 / 128, p.n_t - 1};
    if constexpr (a_t(F)) mn_major_operand(A, p.a, batch, p.m, m0, rows_a, p.k);
    if constexpr (b_t(F)) mn_major_operand(B, p.b, batch, p.n, n0, rows_b, p.k);
    f32x16 acc[4][4];
    mainloop_pipe<F>(acc, ring, A, B, p.k);

    // rows past M / columns past N (ragged last tiles) are computed from zero
    // rows of A / B and not stored
    float lmax = 0.0f;
    const int64_t qr = m0 + 128 * wm, qc = n0 + 128 * wn;
    auto val = [&](int, int, int, float a) {
        lmax = fmaxf(lmax, fabsf(a));
        return a;
    };
    if constexpr (CT == DT_E2M1) {
        // packed E2M1 C: N / 2 bytes per row (N % 32 == 0, checked on the host)
        char *const dst = static_cast<char *>(p.c) + ((batch * p.m + qr) * p.n + qc) / 2;
        store_quadrant_fp4<4>(wave_stage(ring, __builtin_amdgcn_readfirstlane(w)), dst, (uint32_t)(p.n / 2),
                              clamp_extent(p.m - qr), clamp_extent(p.n - qc), acc, lane, val);
    } else {
        constexpr int es = es_of<CT>();
        char *const dst = static_cast<char *>(p.c) + ((batch * p.m + qr) * p.n + qc) * es;
        store_quadrant<CT, 4>(wave_stage(ring, __builtin_amdgcn_readfirstlane(w)), dst, nullptr,
                              (uint32_t)(p.n * es), clamp_extent(p.m - qr), clamp_extent(p.n - qc), acc, lane, val);
    }
    if (p.amax) block_amax_atomic(lmax, p.amax, red);
}

template <int F>
static void launch_gemm_amax_fmt(const GemmAmaxParams &p, dim3 grid, hipStream_t s)
{
    if (p.c_dtype == DT_F32) hipLaunchKernelGGL((k_gemm_amax<F, DT_F32>), grid, dim3(kThreads), 0, s, p);
    else if (p.c_dtype == DT_BF16) hipLaunchKernelGGL((k_gemm_amax<F, DT_BF16>), grid, dim3(kThreads), 0, s, p);
    else if (p.c_dtype == DT_F16) hipLaunchKernelGGL((k_gemm_amax<F, DT_F16>), grid, dim3(kThreads), 0, s, p);
    else if constexpr (F == FMT_E2M1) {
        // FP8 and FP4 C: only with FP4 operands ("GEMM + Amax (SM100)", Dtypes)
        if (p.c_dtype == DT_E4M3) hipLaunchKernelGGL((k_gemm_amax<F, DT_E4M3>), grid, dim3(kThreads), 0, s, p);
        else if (p.c_dtype == DT_E5M2) hipLaunchKernelGGL((k_gemm_amax<F, DT_E5M2>), grid, dim3(kThreads), 0, s, p);
        else hipLaunchKernelGGL((k_gemm_amax<F, DT_E2M1>), grid, dim3(kThreads), 0, s, p);
    }
}

// MN-major FP8 operands (kernels_amax_mn.hip): fmt carries FMT_TA / FMT_TB.
void launch_gemm_amax_mn(const GemmAmaxParams &p, int fmt, dim3 grid, hipStream_t s);

}  // namespace bsg
