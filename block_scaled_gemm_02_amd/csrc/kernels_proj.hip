// Projection GEMM + per-head RoPE + dual-direction MXFP8 quantisation for
// gfx950 ("GEMM + RoPE + MXFP8 Projection (SM100)", Equations).
//
// One workgroup computes 256 tokens x one head (192 features) of
// Y = x W^T (w as [out, in], or as [in, out] staged K-major and read with
// the transposing LDS reads) with the BF16 32x32x16 MFMA, or, for MXFP8 inputs (E4M3 codes
// with row-major E8M0 scales per 32 elements of a row), the scaled
// 32x32x64 f8f6f4 MFMA (fp32 accumulation either way); the waves are
// 4 (tokens, 64 each) x 2 (features: 0..95 and 96..191), two per SIMD, one
// of each feature half.  A wave of the second feature half holds the rotary
// part (features 128..191) in two 32-column accumulator blocks and applies
// the interleaved-in / halves-out rotation in registers (pair (2j, 2j+1) ->
// outputs j and 32+j), then every wave quantises its blocks to E4M3 with
// E8M0 scales: 32-wide blocks along the head dimension (row) and 32-tall
// blocks along tokens (column).  With eight waves a wave's two token blocks
// of cos/sin rows are loaded right after the K loop (held through it they
// would not fit in the 256 registers of a wave); with four waves the first
// two are loaded before the K loop and each later one a block ahead of its
// rotation.
#include "device.hpp"
#include "launch.hpp"

// Waves per workgroup: 8 (BSG_PROJ_MI 2, two waves of 64 tokens per SIMD)
// or 4 (BSG_PROJ_MI 4).  Eight waves run 2.5-4.5% faster on the DeepSeek-V3
// shape: the K loop takes the same time, and the two waves of a SIMD cover
// each other's epilogue waits.
#ifndef BSG_PROJ_MI
#define BSG_PROJ_MI 2
#endif

namespace bsg {

struct ProjParams {
    const uint8_t *x, *w;
    const uint8_t *x_scale, *w_scale;   // MXFP8 inputs only
    const uint16_t *cos, *sin;
    uint8_t *q_row, *s_row, *q_col, *s_col;
    int64_t tokens, q_lora, heads;
    uint32_t row_bytes;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Workgroup -> (head h, first token m0).  Launch index b runs on XCD b % 8,
// 32 workgroups per XCD at a time; when the shape allows, each XCD's 32
// concurrent tiles are 8 heads x 4 token tiles (the weights of 8 heads and
// the activations of 4 token tiles in its L2).  In the head-fastest launch
// order an XCD held 16 heads x 2 token tiles, and each head's weights were
// fetched again for every second token tile (2% slower).
__device__ __forceinline__ void proj_tile_of(int64_t &h, int64_t &m0)
{
    constexpr int HB = 8, TB = 4;
    const int64_t H = gridDim.x, TT = gridDim.y, b = (int64_t)blockIdx.y * H + blockIdx.x;
    h = blockIdx.x;
    int64_t tile = blockIdx.y;
    if (H % HB == 0 && TT % TB == 0 && (H * TT) % (kXcds * kCusPerXcd) == 0) {
        const int64_t x = b % kXcds, li = b / kXcds;
        const int64_t q = kXcds * (li / kCusPerXcd) + x, slot = li % kCusPerXcd, nhb = H / HB;
        h = (q % nhb) * HB + slot % HB;
        tile = (q / nhb) * TB + slot / HB;
    }
    m0 = tile * kTileM;
}

// MI = 4: four waves of 128 tokens x 96 features; MI = 2: eight waves of 64
// tokens x 96 features, two per SIMD (the eight-wave layout of
// mainloop_pipe), so that one wave's epilogue waits are covered by the
// other's work.
template <int F, int MI>
__global__ void __launch_bounds__(1024 / MI) k_proj_rope(ProjParams p)
{
    constexpr int HD = 192, HALF = 32, ROPE = 64, NBLK = HD / 32, NT = 1024 / MI;
    BSG_DECLARE_RING(F, ring);
    // MXFP8 inputs with w as [in, out]: the head's w_scale columns, as rows
    // of scale bytes per feature (up to 64 bytes, q_lora <= 2048)
    __shared__ __attribute__((aligned(16))) uint8_t wsc[b_static_sf<F>() ? 192 * 68 : 16];
    const int t = threadIdx.x, lane = t & 63, wall = t >> 6;
    const int w = MI == 2 ? (wall & 3) : wall, hh = MI == 2 ? (wall >> 2) : 0;
    const int wm = w >> 1, wn = MI == 2 ? ((w & 1) ^ hh) : (w & 1);
    const int row0 = 128 * wm + 64 * hh;                  // the wave's first token in the tile
    const int c32 = lane & 31, gh = lane >> 5;
    int64_t h, m0;
    proj_tile_of(h, m0);
    const int64_t n_out = p.heads * HD;
    const int64_t rows_a = p.tokens - m0 < kTileM ? p.tokens - m0 : kTileM;

    OperandDesc A{p.x + m0 * p.row_bytes, (uint32_t)(rows_a * p.row_bytes), p.row_bytes, nullptr,
                  0, 0, 0, 0, 0};
    // B: head h's 192 rows of w [out, in], or (FMT_BF16_BT) its 192 columns
    // of w [in, out], read K row by K row (K rows past q_lora read zeros)
    OperandDesc B{p.w + h * HD * p.row_bytes, (uint32_t)(HD * p.row_bytes), p.row_bytes, nullptr,
                  0, 0, 0, 0, 0};
    if constexpr (F == FMT_BF16_BT) {
        const uint32_t kstride = (uint32_t)(2 * n_out);
        B.base = p.w + 2 * HD * h;
        B.bytes = (uint32_t)(p.q_lora - 1) * kstride + 2u * HD;
        B.row_bytes = kstride;
    }
    if constexpr (b_static_sf<F>()) {
        // w [in, out] E4M3 codes: the head's 192 columns of each of the q_lora
        // K rows (n-major B); K rows past q_lora read zeros
        const uint32_t kstride = (uint32_t)n_out;
        B.base = p.w + HD * h;
        B.bytes = (uint32_t)(p.q_lora - 1) * kstride + (uint32_t)(n_out - HD * h);
        B.row_bytes = kstride;
        B.mn_valid = HD;
        // w_scale (q_lora/32, n_out): transpose the head's 192 columns into
        // LDS rows of kb bytes per feature, at an odd number of words per row
        // (the 32 rows one fragment read touches then hit distinct banks)
        const uint32_t kb_n = (uint32_t)(p.q_lora / 32);
        const uint32_t stride = (kb_n / 4) % 2 == 0 ? kb_n + 4 : kb_n;
        for (uint32_t wd = (uint32_t)t; wd < kb_n * (HD / 4); wd += NT) {
            const uint32_t kb = wd / (HD / 4), c4 = 4 * (wd % (HD / 4));
            const uint32_t v = *reinterpret_cast<const uint32_t *>(p.w_scale + (int64_t)kb * n_out + HD * h + c4);
#pragma unroll
            for (int e = 0; e < 4; ++e) wsc[(c4 + e) * stride + kb] = (uint8_t)(v >> (8 * e));
        }
        __syncthreads();
        B.sf = nullptr;
        B.sf_bytes = 0;
        B.sf_lds = wsc;
        B.sf_lds_stride = stride;
    }
    if constexpr (fmt_base(F) == FMT_E4M3_RM) {
        const uint32_t srow = (uint32_t)(p.q_lora / 32);          // scale bytes per row
        A.sf = p.x_scale + m0 * srow;
        A.sf_rm = srow;
        A.sf_bytes = (uint32_t)(rows_a * srow);
        if constexpr (!b_static_sf<F>()) {
            B.sf = p.w_scale + h * HD * srow;
            B.sf_rm = srow;
            B.sf_bytes = (uint32_t)(HD * srow);
        }
    }
    // Cos/sin rows for the rotation (waves of the second feature half only,
    // which hold the rotary features).  Four waves: those of the first two
    // 32-token blocks are loaded before the K loop, so they have landed by
    // the epilogue (loads complete in issue order, so the K loop's counted
    // waits stay correct), and block i + 2's once block i's rotation has used
    // its registers; two blocks' values (64 registers) are live at a time.
    // Eight waves: both of the wave's blocks after the K loop.
    uint2 tab[2][4][4];                                    // [block % 2][q][cos lo, sin lo, cos hi, sin hi]
    auto load_tab = [&](int i, uint2 (&t)[4][4]) {
        const int64_t row = m0 + row0 + 32 * i + c32;
        const int64_t tr = row < p.tokens ? row : 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int q8 = 8 * q + 4 * gh;
            t[q][0] = *reinterpret_cast<const uint2 *>(p.cos + tr * ROPE + q8);
            t[q][1] = *reinterpret_cast<const uint2 *>(p.sin + tr * ROPE + q8);
            t[q][2] = *reinterpret_cast<const uint2 *>(p.cos + tr * ROPE + HALF + q8);
            t[q][3] = *reinterpret_cast<const uint2 *>(p.sin + tr * ROPE + HALF + q8);
        }
    };
    if (MI == 4 && wn == 1) {
        load_tab(0, tab[0]);
        load_tab(1, tab[1]);
    }
    f32x16 acc[MI][3];
    mainloop_pipe<F, 3, MI>(acc, ring, A, B, p.q_lora);
    if (MI == 2 && wn == 1) {
        load_tab(0, tab[0]);
        load_tab(1, tab[1]);
    }
    // Block (i, j) lane (c, g) register 4q+u: token 32i + c of the wave's rows,
    // head feature 96wn + 32j + 8q + 4g + u.

    // ---- RoPE on features 128..191 (wave wn = 1, blocks j = 1 and 2) ----
    // Rotary position P of a token is held by block 1 + P/32, register group
    // (P%32)/8, half ((P%8)/4), element P%4.  Output position q8 = 8q + 4g + u
    // pairs inputs 2*q8 and 2*q8 + 1: block 1 + q/2, register group
    // 2(q%2) + g, half u/2, elements 2(u%2) and 2(u%2) + 1.  Each lane gets the
    // other half-wave's registers it needs with v_permlane32_swap (below).
    // RoPE of token block i: out[0] / out[1] are blocks 1 and 2 of the head
    // after the rotation.
    auto rope_block = [&](auto ii, float (&out)[2][16]) {
        constexpr int i = decltype(ii)::value;
        float cs0[16], sn0[16], cs1[16], sn1[16];          // cos/sin at q8 and 32 + q8
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint2 c0 = tab[i % 2][q][0], s0 = tab[i % 2][q][1], c1 = tab[i % 2][q][2], s1 = tab[i % 2][q][3];
            cs0[4 * q] = bf16_lo(c0.x); cs0[4 * q + 1] = bf16_hi(c0.x); cs0[4 * q + 2] = bf16_lo(c0.y); cs0[4 * q + 3] = bf16_hi(c0.y);
            sn0[4 * q] = bf16_lo(s0.x); sn0[4 * q + 1] = bf16_hi(s0.x); sn0[4 * q + 2] = bf16_lo(s0.y); sn0[4 * q + 3] = bf16_hi(s0.y);
            cs1[4 * q] = bf16_lo(c1.x); cs1[4 * q + 1] = bf16_hi(c1.x); cs1[4 * q + 2] = bf16_lo(c1.y); cs1[4 * q + 3] = bf16_hi(c1.y);
            sn1[4 * q] = bf16_lo(s1.x); sn1[4 * q + 1] = bf16_hi(s1.x); sn1[4 * q + 2] = bf16_lo(s1.y); sn1[4 * q + 3] = bf16_hi(s1.y);
        }
        // Rotary input pairs sit in registers 4q'+e (q' = 0, 2) of one half-wave
        // and 4q'+4+e of the other (see above).  v_permlane32_swap of
        // registers r and r + 4 (r = 0-3, 8-11) leaves in X[r] the value
        // that outputs with u < 2 use and in Y[r] the one that u >= 2 use, in
        // both half-waves: low lanes keep their register r in X and receive
        // the high lanes' register r in Y; high lanes receive the low lanes'
        // register r + 4 in X and keep their own in Y.
        float X[2][16], Y[2][16];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 12; ++r) {
                if ((r & 4) != 0) continue;
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[i][1 + b][r]),
                                                                 __float_as_uint(acc[i][1 + b][r + 4]), false, false);
                X[b][r] = __uint_as_float(sw[0]);
                Y[b][r] = __uint_as_float(sw[1]);
            }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int b = q / 2, r = 4 * (2 * (q % 2)) + 2 * (u % 2);
                const float ea = u < 2 ? X[b][r] : Y[b][r];
                const float eb = u < 2 ? X[b][r + 1] : Y[b][r + 1];
                const int v = 4 * q + u;
                out[0][v] = ea * cs0[v] - eb * sn0[v];
                out[1][v] = eb * cs1[v] + ea * sn1[v];
            }
        }
    };

    // ---- dual MXFP8 quantisation (norm_const 1) ----
    // One 32-token block at a time: both code arrays are staged in the wave's
    // LDS region (half a pair slot with four waves, a quarter with eight; the
    // K loop is over) and stored as whole 96-byte row segments; scale bytes
    // are written directly.
    typedef StageGeom<1, 3> G;
    // row codes, column codes and the 32-float exchange fit the wave's region
    static_assert(2 * 32 * G::RBP + 32 * 4 <= (MI == 2 ? (Ring<F>::kWaveStage / 2 & ~15) : Ring<F>::kWaveStage),
                  "projection staging exceeds the wave's LDS region");
    uint8_t *stage = MI == 2 ? wave_stage8(ring, __builtin_amdgcn_readfirstlane(wall))
                             : wave_stage(ring, __builtin_amdgcn_readfirstlane(w));
    uint8_t *sr = stage, *sc = stage + 32 * G::RBP;
    float *const xch = reinterpret_cast<float *>(stage + 2 * 32 * G::RBP);   // column-scale exchange
    uint8_t *wr = sr + c32 * G::RBP + 4 * gh, *wc = sc + c32 * G::RBP + 4 * gh;
    const int64_t col0 = h * HD + 96 * wn;              // the wave's first feature column
    // scale bytes: out_scales_row (tokens, heads, 6) and out_scales_col
    // (tokens/32, n_out); even lanes write the column scale of register
    // r = col_reg_of_lane(lane), column col0 + 32j + 8(r/4) + 4g + r%4
    const int rl = col_reg_of_lane(lane);
    uint8_t *const scol_lane = p.s_col + col0 + 8 * (rl >> 2) + 4 * gh + (rl & 3);
    static_for<MI>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
        __builtin_amdgcn_sched_barrier(0);
        const int64_t rbase = m0 + row0 + 32 * i;        // first token of this 32-token block
        const bool blk_ok = rbase < p.tokens;            // tokens % 128 == 0: blocks are whole
        const int64_t row = rbase + c32;
        uint8_t *const srow_i = p.s_row + (row * p.heads + h) * NBLK + 3 * wn;
        uint8_t *const scol_i = scol_lane + (rbase / 32) * n_out;
        float rot[2][16];                                // blocks 1 and 2 after RoPE (wave column 1)
        if (wn == 1) {
            rope_block(ii, rot);
            if constexpr (i + 2 < MI) load_tab(i + 2, tab[i % 2]);
        } else {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                rot[0][v] = acc[i][1][v];
                rot[1][v] = acc[i][2][v];
            }
        }
        static_for<3>([&](auto jj) {
            constexpr int j = decltype(jj)::value;
            float a[16];
#pragma unroll
            for (int v = 0; v < 16; ++v) a[v] = j == 0 ? acc[i][0][v] : rot[j - 1][v];
            // row direction: 32 features of one token (this lane and lane ^ 32)
            float rm = 0.0f;
#pragma unroll
            for (int v = 0; v < 16; ++v) rm = fmaxf(rm, fabsf(a[v]));
            rm = max_xor32(rm);
            float rinv;
            const uint32_t rb = mx_scale_byte(rm, 1.0f, rinv);
            const float rsf = sf_of_byte(rb);              // norm_const 1: codes are a / SF
            // column direction: 32 tokens of one feature (a register over the half-wave)
            float cinv[16];
            const uint32_t byte = col_scales_xch(a, 1.0f, cinv, lane, xch);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                *reinterpret_cast<uint32_t *>(wr + 32 * j + 8 * q) =
                    pack4_e4m3_sf(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3], rsf);
                *reinterpret_cast<uint32_t *>(wc + 32 * j + 8 * q) =
                    pack4_fp8_mx(a[4 * q] * cinv[4 * q], a[4 * q + 1] * cinv[4 * q + 1],
                                 a[4 * q + 2] * cinv[4 * q + 2], a[4 * q + 3] * cinv[4 * q + 3]);
            }
            if (blk_ok) {
                if (gh == 0) srow_i[j] = (uint8_t)rb;
                if ((lane & 1) == 0) scol_i[32 * j] = (uint8_t)byte;
            }
        });
        const int rows = blk_ok ? 32 : 0;
        stage_flush<1, 3>(sr, reinterpret_cast<char *>(p.q_row) + rbase * n_out + col0, (uint32_t)n_out, rows, 96, lane);
        stage_flush<1, 3>(sc, reinterpret_cast<char *>(p.q_col) + rbase * n_out + col0, (uint32_t)n_out, rows, 96, lane);
    });
}

hipError_t launch_proj_rope(const ProjRopeArgs &a, hipStream_t s)
{
    if (a.tokens == 0 || a.heads == 0) return hipSuccess;
    ProjParams p;
    p.x = reinterpret_cast<const uint8_t *>(a.x);
    p.w = reinterpret_cast<const uint8_t *>(a.w);
    p.x_scale = a.x_scale;
    p.w_scale = a.w_scale;
    p.cos = a.cos; p.sin = a.sin;
    p.q_row = a.q_row; p.s_row = a.s_row; p.q_col = a.q_col; p.s_col = a.s_col;
    p.tokens = a.tokens; p.q_lora = a.q_lora; p.heads = a.heads;
    p.row_bytes = (uint32_t)(a.mxfp8 ? a.q_lora : 2 * a.q_lora);
    dim3 grid((unsigned)a.heads, (unsigned)((a.tokens + kTileM - 1) / kTileM));
    constexpr int MI = BSG_PROJ_MI;
    const dim3 block(1024 / MI);
    if (a.mxfp8 && a.w_out_in) hipLaunchKernelGGL((k_proj_rope<FMT_E4M3_RM, MI>), grid, block, 0, s, p);
    else if (a.mxfp8) hipLaunchKernelGGL((k_proj_rope<FMT_E4M3_RM | FMT_TB, MI>), grid, block, 0, s, p);
    else if (a.w_out_in) hipLaunchKernelGGL((k_proj_rope<FMT_BF16, MI>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((k_proj_rope<FMT_BF16_BT, MI>), grid, block, 0, s, p);
    return hipGetLastError();
}

}  // namespace bsg
