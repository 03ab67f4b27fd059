// Projection GEMM + per-head RoPE + dual-direction MXFP8 quantisation for
// gfx950 ("GEMM + RoPE + MXFP8 Projection (SM100)", Equations).
//
// One workgroup computes 256 tokens x one head (192 features) of
// Y = x W^T with the BF16 32x32x16 MFMA (fp32 accumulation); the waves are
// 2 (tokens) x 2 (features: 0..95 and 96..191).  The second feature wave
// holds the rotary part (features 128..191) in two 32-column accumulator
// blocks, applies the interleaved-in / halves-out rotation in registers
// (pair (2j, 2j+1) -> outputs j and 32+j, exchanged across lanes), then
// every wave quantises its blocks to E4M3 with E8M0 scales: 32-wide blocks
// along the head dimension (row) and 32-tall blocks along tokens (column).
#include "device.hpp"
#include "launch.hpp"

namespace bsg {

struct ProjParams {
    const uint8_t *x, *w;
    const uint16_t *cos, *sin;
    uint8_t *q_row, *s_row, *q_col, *s_col;
    int64_t tokens, q_lora, heads;
    uint32_t row_bytes;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__global__ void __launch_bounds__(256) k_proj_rope(ProjParams p)
{
    constexpr int HD = 192, NOPE = 128, HALF = 32, ROPE = 64, NBLK = HD / 32;
    BSG_DECLARE_RING(FMT_BF16, ring);
    const int t = threadIdx.x, lane = t & 63, w = t >> 6, wm = w >> 1, wn = w & 1;
    const int c32 = lane & 31, gh = lane >> 5;
    const int64_t h = blockIdx.x;
    const int64_t m0 = (int64_t)blockIdx.y * kTileM;
    const int64_t n_out = p.heads * HD;
    const int64_t rows_a = p.tokens - m0 < kTileM ? p.tokens - m0 : kTileM;

    OperandDesc A{p.x + m0 * p.row_bytes, (uint32_t)(rows_a * p.row_bytes), p.row_bytes, nullptr,
                  0, 0, 0, 0, 0};
    OperandDesc B{p.w + h * HD * p.row_bytes, (uint32_t)(HD * p.row_bytes), p.row_bytes, nullptr,
                  0, 0, 0, 0, 0};
    f32x16 acc[4][3];
    mainloop_pipe<FMT_BF16, 3>(acc, ring, A, B, p.q_lora);

    transpose_acc<3>(acc, lane);
    // Transposed layout: element 4q+u of block (i, j) in lane (k, t, g) is token
    // 32i + 8q + 4g + t of the wave's rows, feature 96wn + 32j + 4k + u.
    const int k4 = 4 * (c32 >> 2);

    // ---- RoPE on features 128..191 (wave wn = 1, blocks j = 1 and 2) ----
    // Output feature c of the rotated half pairs rope inputs 2c and 2c+1;
    // for output run 4k..4k+3 those are inputs 8k..8k+7 (mod 32), held by
    // lanes 2k and 2k+1 (mod 8) of the same row, in block 1 for k < 4 and
    // block 2 otherwise.
    if (wn == 1) {
        const int kk = c32 >> 2;
        const int src0 = 4 * ((2 * kk) & 7) + (lane & 3) + 32 * gh, src1 = src0 + 4;
        const bool lo = kk < 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float e[8];                               // rope inputs 8k'..8k'+7 of this row
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float x1 = __shfl(acc[i][1][4 * q + u], src0), x2 = __shfl(acc[i][2][4 * q + u], src0);
                    const float y1 = __shfl(acc[i][1][4 * q + u], src1), y2 = __shfl(acc[i][2][4 * q + u], src1);
                    e[u] = lo ? x1 : x2;
                    e[4 + u] = lo ? y1 : y2;
                }
                const int64_t row = m0 + tr_row(wm, i, q, lane);
                const int64_t tr = row < p.tokens ? row : 0;
                const uint2 cw0 = *reinterpret_cast<const uint2 *>(p.cos + tr * ROPE + k4);
                const uint2 sw0 = *reinterpret_cast<const uint2 *>(p.sin + tr * ROPE + k4);
                const uint2 cw1 = *reinterpret_cast<const uint2 *>(p.cos + tr * ROPE + HALF + k4);
                const uint2 sw1 = *reinterpret_cast<const uint2 *>(p.sin + tr * ROPE + HALF + k4);
                const float c0[4] = {bf16_lo(cw0.x), bf16_hi(cw0.x), bf16_lo(cw0.y), bf16_hi(cw0.y)};
                const float s0[4] = {bf16_lo(sw0.x), bf16_hi(sw0.x), bf16_lo(sw0.y), bf16_hi(sw0.y)};
                const float c1[4] = {bf16_lo(cw1.x), bf16_hi(cw1.x), bf16_lo(cw1.y), bf16_hi(cw1.y)};
                const float s1[4] = {bf16_lo(sw1.x), bf16_hi(sw1.x), bf16_lo(sw1.y), bf16_hi(sw1.y)};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float a = e[2 * u], b = e[2 * u + 1];
                    acc[i][1][4 * q + u] = a * c0[u] - b * s0[u];
                    acc[i][2][4 * q + u] = b * c1[u] + a * s1[u];
                }
            }
        }
    }
    (void)NOPE;

    // ---- dual MXFP8 quantisation (norm_const 1) ----
    static_for<3>([&](auto jj) {
        constexpr int j = decltype(jj)::value;
        const int blk = 3 * wn + j;                      // 32-feature block within the head
        const int64_t col = h * HD + 32 * blk + k4;      // first of this lane's 4 feature columns
        static_for<4>([&](auto ii) {
            constexpr int i = decltype(ii)::value;
            const int64_t rbase = m0 + 128 * wm + 32 * i;   // first token of this 32-token block
            const bool blk_ok = rbase < p.tokens;            // tokens % 128 == 0: blocks are whole
            // column direction: 32 tokens of one feature
            float cm[4], cinv[4];
            tr_col_absmax(acc[i][j], cm);
            uint32_t cb[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) cb[u] = mx_scale_byte(cm[u], 1.0f, cinv[u]);
            const int t = lane & 3;
            if (blk_ok && gh == 0)
                p.s_col[(rbase / 32) * n_out + col + t] =
                    (uint8_t)(t == 0 ? cb[0] : t == 1 ? cb[1] : t == 2 ? cb[2] : cb[3]);
            // row direction: 32 features of one token
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float x[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                    acc[i][j][4 * q + 3]};
                float rm = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
                rm = row8_max(rm);
                float rinv;
                const uint32_t rb = mx_scale_byte(rm, 1.0f, rinv);
                if (blk_ok) {
                    const int64_t row = m0 + tr_row(wm, i, q, lane);
                    *reinterpret_cast<uint32_t *>(p.q_row + row * n_out + col) =
                        pack4_e4m3(x[0] * rinv, x[1] * rinv, x[2] * rinv, x[3] * rinv);
                    *reinterpret_cast<uint32_t *>(p.q_col + row * n_out + col) =
                        pack4_e4m3(x[0] * cinv[0], x[1] * cinv[1], x[2] * cinv[2], x[3] * cinv[3]);
                    if (c32 < 4) p.s_row[(row * p.heads + h) * NBLK + blk] = (uint8_t)rb;
                }
            }
        });
    });
}

hipError_t launch_proj_rope(const ProjRopeArgs &a, hipStream_t s)
{
    if (a.tokens == 0 || a.heads == 0) return hipSuccess;
    if (!a.w_out_in) return hipErrorNotSupported;
    ProjParams p;
    p.x = reinterpret_cast<const uint8_t *>(a.x);
    p.w = reinterpret_cast<const uint8_t *>(a.w);
    p.cos = a.cos; p.sin = a.sin;
    p.q_row = a.q_row; p.s_row = a.s_row; p.q_col = a.q_col; p.s_col = a.s_col;
    p.tokens = a.tokens; p.q_lora = a.q_lora; p.heads = a.heads;
    p.row_bytes = (uint32_t)(2 * a.q_lora);
    dim3 grid((unsigned)a.heads, (unsigned)((a.tokens + kTileM - 1) / kTileM));
    hipLaunchKernelGGL(k_proj_rope, grid, dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace bsg
