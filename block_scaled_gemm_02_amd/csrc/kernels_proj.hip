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

__device__ __forceinline__ float bf16_val(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__global__ void __launch_bounds__(256) k_proj_rope(ProjParams p)
{
    constexpr int HD = 192, NOPE = 128, HALF = 32, ROPE = 64, NBLK = HD / 32;
    __shared__ __attribute__((aligned(16))) uint8_t lds[4 * kStageBytes];
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
    mainloop<FMT_BF16, 3>(acc, lds, A, B, p.q_lora);

    // ---- RoPE on features 128..191 (wave wn = 1, blocks j = 1 and 2) ----
    if (wn == 1) {
        const int src = ((2 * c32) & 31) + 32 * gh;     // lane of element 2c (mod 32)
        const bool lo = c32 < HALF / 2;                  // pair lives in block 1 (else 2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = m0 + acc_row(wm, i, v, lane);
                const float a1 = __shfl(acc[i][1][v], src), b1 = __shfl(acc[i][1][v], src + 1);
                const float a2 = __shfl(acc[i][2][v], src), b2 = __shfl(acc[i][2][v], src + 1);
                const float a = lo ? a1 : a2, b = lo ? b1 : b2;
                const int64_t tr = row < p.tokens ? row : 0;
                const float c0 = bf16_val(p.cos[tr * ROPE + c32]);
                const float s0 = bf16_val(p.sin[tr * ROPE + c32]);
                const float c1 = bf16_val(p.cos[tr * ROPE + HALF + c32]);
                const float s1 = bf16_val(p.sin[tr * ROPE + HALF + c32]);
                acc[i][1][v] = a * c0 - b * s0;
                acc[i][2][v] = b * c1 + a * s1;
            }
        }
    }
    (void)NOPE;

    // ---- dual MXFP8 quantisation (norm_const 1) ----
    static_for<12>([&](auto ij) {
        constexpr int i = decltype(ij)::value / 3, j = decltype(ij)::value % 3;
        const int blk = 3 * wn + j;                      // 32-feature block within the head
        const int64_t col = h * HD + 32 * blk + c32;     // feature column in [0, heads*192)
        const f32x16 dv = acc[i][j];
        const int64_t rbase = m0 + 128 * wm + 32 * i;    // first token of this 32-token block
        const bool blk_ok = rbase < p.tokens;            // tokens % 128 == 0: blocks are whole
        // column direction: 32 tokens of one feature
        float cm = 0.0f;
#pragma unroll
        for (int v = 0; v < 16; ++v) cm = fmaxf(cm, fabsf(dv[v]));
        cm = fmaxf(cm, __shfl_xor(cm, 32));
        float cinv;
        const uint32_t cbyte = mx_scale_byte(cm, 1.0f, cinv);
        if (blk_ok) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = m0 + acc_row(wm, i, v, lane);
                p.q_col[row * n_out + col] = (uint8_t)e4m3_code(dv[v] * cinv);
            }
            if (gh == 0) p.s_col[(rbase / 32) * n_out + col] = (uint8_t)cbyte;
        }
        // row direction: 32 features of one token
        uint32_t my_byte = 0;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float rm = half_wave_max(fabsf(dv[v]));
            float rinv;
            const uint32_t rbyte = mx_scale_byte(rm, 1.0f, rinv);
            if (c32 == v) my_byte = rbyte;
            if (blk_ok) {
                const int64_t row = m0 + acc_row(wm, i, v, lane);
                p.q_row[row * n_out + col] = (uint8_t)e4m3_code(dv[v] * rinv);
            }
        }
        if (blk_ok && c32 < 16) {
            const int64_t row = m0 + acc_row(wm, i, c32, lane);
            p.s_row[(row * p.heads + h) * NBLK + blk] = (uint8_t)my_byte;
        }
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
