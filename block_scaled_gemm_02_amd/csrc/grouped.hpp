// Grouped GEMM kernels for gfx950: "Grouped GEMM (SM100 BF16)", "Grouped
// GEMM + sReLU (SM100)" and "Grouped GEMM + dSwiGLU (SM100)".  Tiles of 256
// rows never straddle an expert because every padded_offsets entry is a
// multiple of 256.  The kernel template is instantiated by
// kernels_grouped.hip, kernels_srelu*.hip and kernels_dswiglu.hip.
//
// Epilogues work on the accumulator layout of mma_one: lane (c, g) of block
// (i, j) owns row 32i + c and the column runs 32j + 8q + 4g + [0, 4).  Every
// value a store depends on (prob, bias) is loaded before the first store:
// loads and stores share one counter, so a load issued after stores would
// wait for all of them.
#pragma once
#include "kernels_common.hpp"

namespace bsg {

enum : int { EPI_BF16_BIAS = 0, EPI_SRELU = 1, EPI_SRELU_FP8 = 2, EPI_BF16 = 3, EPI_DSWIGLU_FP8 = 4,
             EPI_DSWIGLU = 5 };

struct GroupedParams {
    const uint8_t *a, *b, *sfa, *sfb;
    const uint64_t *b_ptrs, *sfb_ptrs;   // discrete weights (else null)
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
    float tanh_s;
    TanhSqConst tq;      // constants of tanh(r/s)^2 (see tanh_sq)
    // dSwiGLU backward only: beta (L,), the forward tensor C (M, 2N) bf16, dprob (M,)
    const float *beta;
    const uint16_t *cfwd;
    float *dprob;
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

// sReLU value of one pre-activation value g = alpha*acc: relu, optional tanh
// clamp, times prob ("Grouped GEMM + sReLU (SM100)" Equations):
// D = prob * (s * tanh(relu(g) / s))^2, or prob * relu(g)^2 without clamp.
// prs2 = prob * s^2 (clamped form) or prob (plain form), per row.
template <bool CLAMP>
__device__ __forceinline__ float srelu_value(float gval, float prs2, const TanhSqConst &tq)
{
    const float r = fmaxf(gval, 0.0f);
    return prs2 * (CLAMP ? tanh_sq(r, tq) : r * r);
}
template <bool CLAMP>
__device__ __forceinline__ float srelu_row_factor(float pr, float s)
{
    return CLAMP ? pr * (s * s) : pr;
}

// BF16 bias epilogue and sReLU epilogue with 16/32-bit outputs: C, then D
// (and D_col, which equals D for unquantised outputs), each staged through
// the wave's LDS region with its own compile-time store type.
template <int F, int EPI, bool CLAMP, int OT>
__device__ __forceinline__ void epilogue_grouped(const GroupedParams &p, f32x16 (&acc)[4][4],
                                                 uint8_t *stage, int64_t m0, int64_t n0, int g, float alpha,
                                                 int wm, int wn, int lane, float *red, const float *prob_lds)
{
    const int64_t n = p.n;
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = prob_lds[acc_row(wm, i, lane)];
    // The bias of the wave's 128 columns goes to the last 512 bytes of its
    // staging region as floats (two per lane), and is read back per element:
    // held in registers it took 64 per lane.
    // (EPI_BF16_BIAS: the BF16 operation with bias; EPI_BF16: without.)
    constexpr bool kBf16 = EPI == EPI_BF16_BIAS || EPI == EPI_BF16, has_bias = EPI == EPI_BF16_BIAS;
    float *const bias_lds = reinterpret_cast<float *>(stage + Ring<F>::kWaveStage - 512);
    if constexpr (has_bias) {
        const int64_t c = n0 + 128 * wn + 2 * lane;          // N % 8 == 0: c + 1 < n with c
        float b0 = 0.0f, b1 = 0.0f;
        if (c < n) {
            b0 = load_elem(p.bias, (int64_t)g * n + c, p.bias_dtype);
            b1 = load_elem(p.bias, (int64_t)g * n + c + 1, p.bias_dtype);
        }
        *reinterpret_cast<float2 *>(bias_lds + 2 * lane) = make_float2(b0, b1);
    }
    const int gh = lane >> 5;
    auto bias_of = [&](int j, int v) { return bias_lds[32 * j + 8 * (v >> 2) + 4 * gh + (v & 3)]; };
    if constexpr (has_bias) wait_loads();
    // "Grouped GEMM (SM100 BF16)", Operation: with bias C = G + prob*bias,
    // D = C; without bias C = G, D = prob*G.  sReLU: C = G, D = sReLU(G).
    const int64_t qr = m0 + 128 * wm, qc = n0 + 128 * wn;
    const int cols = clamp_extent(n - qc);
    float prf[4];                                     // per-row sReLU factor
#pragma unroll
    for (int i = 0; i < 4; ++i) prf[i] = srelu_row_factor<CLAMP>(pr[i], p.tanh_s);
    float lmax = 0.0f;
    // C and D of one type, and both fit the staging slot: one pass
    const int es = OT >= 0 ? (OT == DT_F32 ? 4 : 2) : (p.d_dtype == DT_F32 ? 4 : 2);
    if (OT >= 0 || (p.c && p.c_dtype == p.d_dtype && 2 * 32 * (128 * es + 16) + 512 <= Ring<F>::kWaveStage)) {
        auto both = [&](int i, int j, int v, float a, float &cv, float &dv) {
            const float gval = alpha * a;
            if constexpr (has_bias) {
                cv = gval + pr[i] * bias_of(j, v);
                dv = cv;
            } else if constexpr (kBf16) {
                cv = gval;
                dv = pr[i] * gval;
            } else {
                cv = gval;
                dv = srelu_value<CLAMP>(gval, prf[i], p.tq);
                lmax = fmaxf(lmax, fabsf(dv));
                // (runtime-typed kernels: keep the running max here; left
                // free, the compiler moved the max chain into the amax branch
                // below, kept every D value live until then and spilled)
                if constexpr (OT < 0) asm volatile("" : "+v"(lmax));
            }
        };
        char *dd2 = kBf16 ? nullptr : static_cast<char *>(p.d_col);
        const size_t off = (size_t)(qr * n + qc) * es;
        const uint32_t rb = (uint32_t)(n * es);
        char *dc = static_cast<char *>(p.c) + off, *dd = static_cast<char *>(p.d) + off;
        dd2 = dd2 ? dd2 + off : nullptr;
        if constexpr (OT >= 0) store_quadrant2<OT, 4>(stage, dc, dd, dd2, rb, 128, cols, acc, lane, both);
        else if (p.d_dtype == DT_F32) store_quadrant2<DT_F32, 4>(stage, dc, dd, dd2, rb, 128, cols, acc, lane, both);
        else if (p.d_dtype == DT_BF16) store_quadrant2<DT_BF16, 4>(stage, dc, dd, dd2, rb, 128, cols, acc, lane, both);
        else store_quadrant2<DT_F16, 4>(stage, dc, dd, dd2, rb, 128, cols, acc, lane, both);
        if constexpr (EPI == EPI_SRELU) {
            if (p.amax) block_amax_atomic(lmax, p.amax + g, red);
        }
        return;
    }
    if constexpr (OT >= 0) return;
    if (p.c) {
        store_quadrant_rt<4>(p.c_dtype, stage, p.c, nullptr, n, qr, qc, 128, cols, acc, lane,
                             [&](int i, int j, int v, float a) {
            const float gval = alpha * a;
            if constexpr (has_bias) return gval + pr[i] * bias_of(j, v);
            else return gval;
        });
    }
    store_quadrant_rt<4>(p.d_dtype, stage, p.d, kBf16 ? nullptr : p.d_col, n, qr, qc, 128, cols,
                         acc, lane, [&](int i, int j, int v, float a) {
        const float gval = alpha * a;
        if constexpr (has_bias) {
            return gval + pr[i] * bias_of(j, v);
        } else if constexpr (kBf16) {
            return pr[i] * gval;
        } else {
            const float d = srelu_value<CLAMP>(gval, prf[i], p.tq);
            lmax = fmaxf(lmax, fabsf(d));
            asm volatile("" : "+v"(lmax));
            return d;
        }
    });
    if constexpr (EPI == EPI_SRELU) {
        if (p.amax) block_amax_atomic(lmax, p.amax + g, red);
    }
}

// MXFP8 output: D quantised in 32-wide blocks along N (codes to d, scales to
// the SFD_row atoms over (M, N)) and in 32-tall blocks along M (codes to
// d_col, scales to the SFD_col atoms over (N, M)), with the quantiser of
// "Grouped GEMM + dSwiGLU (SM100)", Step 3.  DF is the code format:
// DT_E4M3 (rcp_max = 1/448), DT_E5M2 (1/57344) or DT_E2M1 (1/6, two codes
// per byte with the even column in the low nibble, so D and D_col rows are
// N/2 bytes).
//
// A row's 32 values of block j sit in this lane (16) and lane ^ 32 (16); a
// column's 32 values of block i sit in one register of the 32 lanes of a
// half-wave.  C (pre-activation) is written first when requested.  Then, one
// 32-row block at a time, D is formed in registers, both code arrays are
// staged in the wave's LDS region and stored as whole rows, and the scale
// bytes are written: SFD_row as one word per row (the wave's four 32-column
// blocks are one K' group), SFD_col byte by byte.
template <bool CLAMP, int DF>
__device__ __forceinline__ void epilogue_srelu_fp8(const GroupedParams &p, f32x16 (&acc)[4][4],
                                                   uint8_t *stage, int64_t m0, int64_t n0, float alpha,
                                                   int wm, int wn, int lane, const float *prob_lds)
{
    constexpr bool FP4 = DF == DT_E2M1;
    constexpr int PB = FP4 ? 2 : 1;                   // codes per byte
    typedef StageGeom<1, 4 / PB> G;
    const float nc = *p.norm_const;
    const int64_t n = p.n;
    const int64_t row_kt = (n / 32 + 3) / 4;          // SFD_row: K' over N
    const int64_t col_kt = (p.m / 32 + 3) / 4;        // SFD_col: K' over M
    const int c32 = lane & 31, gh = lane >> 5;
    const int64_t qr = m0 + 128 * wm, qc = n0 + 128 * wn;
    const int cols = clamp_extent(n - qc);

    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = prob_lds[acc_row(wm, i, lane)];
    if (p.c) {
        store_quadrant_rt<4>(p.c_dtype, stage, p.c, nullptr, n, qr, qc, 128, cols, acc, lane,
                             [&](int, int, int, float a) { return alpha * a; });
    }

    uint8_t *sd = stage, *sdc = stage + 32 * G::RBP;
    uint8_t *wd = sd + c32 * G::RBP + (4 / PB) * gh, *wdc = sdc + c32 * G::RBP + (4 / PB) * gh;
    float *const xch = reinterpret_cast<float *>(stage + 2 * 32 * G::RBP);   // column-scale exchange
    const int64_t mt = qr / 128;
    // SFD_col: even lanes write the byte of register r = col_reg_of_lane(lane),
    // column qc + 32j + cl with cl = 8(r/4) + 4g + r%4 < 32; qc is a multiple
    // of 128, so its atom offset is ((qc/128 * col_kt + mt) * 32 + cl) * 16
    // + 4j, plus the row block i
    const int rl = col_reg_of_lane(lane), cl = 8 * (rl >> 2) + 4 * gh + (rl & 3);
    uint8_t *const sfc = p.sfd_col + (((qc / 128) * col_kt + mt) * 32 + cl) * 16;
    static_for<4>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
        __builtin_amdgcn_sched_barrier(0);
        uint32_t rword = 0u;                          // SFD_row bytes j = 0..3 of row 32i + c
        const float prf = srelu_row_factor<CLAMP>(pr[i], p.tanh_s);
        static_for<4>([&](auto jj) {
            constexpr int j = decltype(jj)::value;
            float d[16];
#pragma unroll
            for (int v = 0; v < 16; ++v) d[v] = srelu_value<CLAMP>(alpha * acc[i][j][v], prf, p.tq);
            // row block: this lane's 16 columns and the partner half's 16
            float rm = 0.0f;
#pragma unroll
            for (int v = 0; v < 16; ++v) rm = fmaxf(rm, fabsf(d[v]));
            rm = max_xor32(rm);
            float rinv;
            rword |= mx_scale_byte<DF>(rm, nc, rinv) << (8 * j);
            // column blocks: 32 rows of each column over the half-wave
            float cinv[16];
            const uint32_t byte = col_scales_xch<DF>(d, nc, cinv, lane, xch);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if constexpr (FP4) {
                    *reinterpret_cast<uint16_t *>(wd + 16 * j + 4 * q) = (uint16_t)pack4_e2m1(
                        d[4 * q] * rinv, d[4 * q + 1] * rinv, d[4 * q + 2] * rinv, d[4 * q + 3] * rinv);
                    *reinterpret_cast<uint16_t *>(wdc + 16 * j + 4 * q) = (uint16_t)pack4_e2m1(
                        d[4 * q] * cinv[4 * q], d[4 * q + 1] * cinv[4 * q + 1], d[4 * q + 2] * cinv[4 * q + 2],
                        d[4 * q + 3] * cinv[4 * q + 3]);
                } else {
                    *reinterpret_cast<uint32_t *>(wd + 32 * j + 8 * q) = pack4_fp8_mx<DF == DT_E5M2>(
                        d[4 * q] * rinv, d[4 * q + 1] * rinv, d[4 * q + 2] * rinv, d[4 * q + 3] * rinv);
                    *reinterpret_cast<uint32_t *>(wdc + 32 * j + 8 * q) = pack4_fp8_mx<DF == DT_E5M2>(
                        d[4 * q] * cinv[4 * q], d[4 * q + 1] * cinv[4 * q + 1], d[4 * q + 2] * cinv[4 * q + 2],
                        d[4 * q + 3] * cinv[4 * q + 3]);
                }
            }
            // (lane ^ 1 holds the same byte)
            if ((lane & 1) == 0 && 32 * j + cl < cols) sfc[4 * j + i] = (uint8_t)byte;
        });
        const uint32_t rb = (uint32_t)(n / PB);
        stage_flush<1, 4 / PB>(sd, static_cast<char *>(p.d) + ((qr + 32 * i) * n + qc) / PB, rb, 32, cols / PB, lane);
        stage_flush<1, 4 / PB>(sdc, static_cast<char *>(p.d_col) + ((qr + 32 * i) * n + qc) / PB, rb, 32, cols / PB,
                               lane);
        // SFD_row word of row r; columns past N carry the scale of an all-zero block
        if (gh == 0 && cols > 0) {
            const int64_t r = m0 + acc_row(wm, i, lane);
            const int64_t off = (((r / 128) * row_kt + qc / 128) * 32 + (r % 32)) * 16 + ((r % 128) / 32) * 4;
            *reinterpret_cast<uint32_t *>(p.sfd_row + off) = rword;
        }
    });
}

// dSwiGLU backward epilogue with MXFP8 output ("Grouped GEMM + dSwiGLU
// (SM100)", Steps 2 and 3).  ref = alpha_g^2 * acc; the forward tensor C
// holds, for ref columns [32b, 32b+32), the input in C columns [64b, 64b+32)
// and the gate in [64b+32, 64b+64), both scaled by beta_g;
//   swish = gate*sigmoid(gate),  ab = ref*prob*swish,
//   dswiglu = ref*prob*input*sigmoid(gate)*(1 + gate*(1 - sigmoid(gate))),
// written to D with the same pairing, and dprob[m] += sum swish*input*ref.
// The wave's 128 ref columns become 256 D columns (8 blocks of 32: ab of ref
// block j is D block 2j, dswiglu 2j+1), quantised along D (SFD_row atoms over
// (M, 2N)) and along M (SFD_col atoms over (2N, M)) as in the sReLU MXFP8
// epilogue (E5: E5M2 codes).  A lane's four C values of register group q
// are consecutive, one 8-byte load each for input and gate.
__device__ __forceinline__ float bf16_at(uint2 w, int u)
{
    const uint32_t x = (u < 2) ? w.x : w.y;
    return __uint_as_float((u & 1) ? (x & 0xFFFF0000u) : (x << 16));
}
// One ref element of the dSwiGLU backward, on the raw (unscaled) gate g and
// input x of the forward tensor: with gt = beta*g and sg = sigmoid(gt),
// t = g*sg = swish/beta and f = alpha^2 * prob * beta * scale (scale:
// norm_const for the MX outputs, whose quantiser then divides by the E8M0
// scale alone; 1 otherwise),
//   ab = f*a*t,  dswiglu = f*a*x*sg*(1 + gt - beta*t)  (= ... * (1 + gt*(1 - sg))),
// and t*x, which dprob accumulates times a; the row's dprob is that sum
// times beta^2 alpha^2.  kx = -log2(e)*beta.
struct DswigluTerms {
    float ab, ds, tx;
};
__device__ __forceinline__ DswigluTerms dswiglu_terms(float a, float g, float x, float f, float beta, float kx)
{
    const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(kx * g));
    const float t = g * sg;
    const float fa = f * a;
    return DswigluTerms{fa * t, fa * x * sg * fmaf(-beta, t, fmaf(beta, g, 1.0f)), t * x};
}
template <bool E5>
__device__ __forceinline__ void epilogue_dswiglu_fp8(const GroupedParams &p, f32x16 (&acc)[4][4], uint8_t *stage,
                                                     int64_t m0, int64_t n0, float alpha2, float beta, int wm,
                                                     int wn, int lane, const float *prob_lds)
{
    typedef StageGeom<1, 8> G;                       // 256 code bytes per staged row
    const float nc = *p.norm_const;
    const int64_t n = p.n, n2 = 2 * n;
    const int64_t row_kt = (n2 / 32 + 3) / 4;       // SFD_row: K' over 2N
    const int64_t col_kt = (p.m / 32 + 3) / 4;      // SFD_col: K' over M
    const int c32 = lane & 31, gh = lane >> 5;
    const int64_t qr = m0 + 128 * wm, qc = n0 + 128 * wn, dq = 2 * qc;
    const int cols = clamp_extent(n - qc);          // valid ref columns (a multiple of 32)
    const int dcols = 2 * cols;
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = prob_lds[acc_row(wm, i, lane)];
    uint8_t *sd = stage, *sdc = stage + 32 * G::RBP;
    uint8_t *wd = sd + c32 * G::RBP + 4 * gh, *wdc = sdc + c32 * G::RBP + 4 * gh;
    float *const xch = reinterpret_cast<float *>(stage + 2 * 32 * G::RBP);   // column-scale exchange
    const int64_t mt = qr / 128;
    // SFD_col: even lanes write the byte of register r = col_reg_of_lane(lane),
    // D column dq + 32 blk + cl with cl = 8(r/4) + 4g + r%4 < 32; dq is a
    // multiple of 256, so its atom offset is ((dq/128 + blk/4) * col_kt + mt)
    // * 512 + 16 cl + 4 (blk%4), plus the row block i
    const int rl = col_reg_of_lane(lane), cl = 8 * (rl >> 2) + 4 * gh + (rl & 3);
    uint8_t *const sfc = p.sfd_col + (((dq / 128) * col_kt + mt) * 32 + cl) * 16;
    const int64_t sfc_k4 = col_kt * 512;            // the next 128 D columns' atoms
    const float kx = -1.4426950408889634f * beta, cdp = beta * beta * alpha2;
    static_for<4>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
        __builtin_amdgcn_sched_barrier(0);
        const int64_t row = qr + 32 * i + c32;
        // input and gate of this lane's 64 ref columns (zero past N)
        uint2 cin[4][4], cgt[4][4];
        const uint16_t *crow = p.cfwd + row * n2 + 64 * (qc / 32) + 4 * gh;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const bool ok = 32 * j < cols;
                cin[j][q] = ok ? *reinterpret_cast<const uint2 *>(crow + 64 * j + 8 * q) : make_uint2(0u, 0u);
                cgt[j][q] = ok ? *reinterpret_cast<const uint2 *>(crow + 64 * j + 32 + 8 * q) : make_uint2(0u, 0u);
            }
        uint32_t rword[2] = {0u, 0u};                // SFD_row bytes of D blocks 0-3 and 4-7
        float dpr = 0.0f;
        // dv holds norm_const * D (see dswiglu_terms), so the scale step takes
        // norm_const 1, and a code is the value over the E8M0 scale: the row
        // codes by the scaled conversion, the column codes times 1/SF (both
        // exact power-of-two scalings of norm_const * D)
        auto quant_block = [&](const float (&dv)[16], int blk) {
            // row direction: 32 D columns of one row (this lane and lane ^ 32)
            float rm = 0.0f;
#pragma unroll
            for (int v = 0; v < 16; ++v) rm = fmaxf(rm, fabsf(dv[v]));
            rm = max_xor32(rm);
            float rinv;
            const uint32_t rb = mx_scale_byte<E5 ? DT_E5M2 : DT_E4M3>(rm, 1.0f, rinv);
            const float rsf = sf_of_byte(rb);
            rword[blk >> 2] |= rb << (8 * (blk & 3));
            // column direction: 32 rows of one D column over the half-wave
            float cinv[16];
            const uint32_t byte = col_scales_xch<E5 ? DT_E5M2 : DT_E4M3>(dv, 1.0f, cinv, lane, xch);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                *reinterpret_cast<uint32_t *>(wd + 32 * blk + 8 * q) =
                    pack4_fp8_sf<E5>(dv[4 * q], dv[4 * q + 1], dv[4 * q + 2], dv[4 * q + 3], rsf);
                *reinterpret_cast<uint32_t *>(wdc + 32 * blk + 8 * q) =
                    pack4_fp8_mx<E5>(dv[4 * q] * cinv[4 * q], dv[4 * q + 1] * cinv[4 * q + 1],
                               dv[4 * q + 2] * cinv[4 * q + 2], dv[4 * q + 3] * cinv[4 * q + 3]);
            }
            if ((lane & 1) == 0 && 32 * blk < dcols) sfc[(blk >> 2) * sfc_k4 + 4 * (blk & 3) + i] = (uint8_t)byte;
        };
        const float fi = alpha2 * pr[i] * beta * nc;
        static_for<4>([&](auto jj) {
            constexpr int j = decltype(jj)::value;
            float ab[16], ds[16];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const DswigluTerms r = dswiglu_terms(acc[i][j][v], bf16_at(cgt[j][v >> 2], v & 3),
                                                     bf16_at(cin[j][v >> 2], v & 3), fi, beta, kx);
                ab[v] = r.ab;
                ds[v] = r.ds;
                dpr = fmaf(r.tx, acc[i][j][v], dpr);
            }
            quant_block(ab, 2 * j);
            quant_block(ds, 2 * j + 1);
        });
        // dprob: this lane's 64 columns plus the other half-wave's 64 of the same row
        dpr = add_xor32(dpr) * cdp;
        if (gh == 0 && cols > 0) atomicAdd(p.dprob + row, dpr);
        const uint32_t rb = (uint32_t)n2;
        stage_flush<1, 8>(sd, static_cast<char *>(p.d) + (qr + 32 * i) * n2 + dq, rb, 32, dcols, lane);
        stage_flush<1, 8>(sdc, static_cast<char *>(p.d_col) + (qr + 32 * i) * n2 + dq, rb, 32, dcols, lane);
        // SFD_row words of this row: K' groups dq/128 and dq/128 + 1 (when they exist)
        if (gh == 0) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int64_t kg = dq / 128 + h;
                if (128 * h < dcols && kg < row_kt) {
                    const int64_t off = (((row / 128) * row_kt + kg) * 32 + (row % 32)) * 16 + ((row % 128) / 32) * 4;
                    *reinterpret_cast<uint32_t *>(p.sfd_row + off) = rword[h];
                }
            }
        }
    });
}

// dSwiGLU backward with an unquantised D (FP4 inputs: "Grouped GEMM + dSwiGLU
// (SM100)", Input/Output tensors: bf16 or fp32 D, per-expert amax (L, 2)).
// Same arithmetic as epilogue_dswiglu_fp8; D (and the optional D_col copy)
// is stored through the wave's staging rows, and amax[2g] / amax[2g+1] take
// max |ab| / max |dswiglu| (fp32 values) with one atomic each per workgroup.
template <int OT>
__device__ __forceinline__ void epilogue_dswiglu(const GroupedParams &p, f32x16 (&acc)[4][4], uint8_t *stage,
                                                 int64_t m0, int64_t n0, int g, float alpha2, float beta,
                                                 int wm, int wn, int lane, float *red, const float *prob_lds)
{
    constexpr int ES = OT == DT_F32 ? 4 : 2;
    typedef StageGeom<ES, 8> G;                     // the wave's 256 D columns per staged row
    const int64_t n = p.n, n2 = 2 * n;
    const int c32 = lane & 31, gh = lane >> 5;
    const int64_t qr = m0 + 128 * wm, qc = n0 + 128 * wn, dq = 2 * qc;
    const int cols = clamp_extent(n - qc);
    const int dcols = 2 * cols;
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = prob_lds[acc_row(wm, i, lane)];
    uint8_t *wd = stage + c32 * G::RBP + 4 * gh * ES;
    float mab = 0.0f, mds = 0.0f;
    const float kx = -1.4426950408889634f * beta, cdp = beta * beta * alpha2;
    static_for<4>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
        __builtin_amdgcn_sched_barrier(0);
        const int64_t row = qr + 32 * i + c32;
        const uint16_t *crow = p.cfwd + row * n2 + 64 * (qc / 32) + 4 * gh;
        float dpr = 0.0f;
        const float fi = alpha2 * pr[i] * beta;
        static_for<4>([&](auto jj) {
            constexpr int j = decltype(jj)::value;
            const bool ok = 32 * j < cols;
            uint2 ci[4], cg[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                ci[q] = ok ? *reinterpret_cast<const uint2 *>(crow + 64 * j + 8 * q) : make_uint2(0u, 0u);
                cg[q] = ok ? *reinterpret_cast<const uint2 *>(crow + 64 * j + 32 + 8 * q) : make_uint2(0u, 0u);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float ab[4], ds[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int v = 4 * q + u;
                    const DswigluTerms r = dswiglu_terms(acc[i][j][v], bf16_at(cg[q], u), bf16_at(ci[q], u), fi,
                                                         beta, kx);
                    ab[u] = r.ab;
                    ds[u] = r.ds;
                    dpr = fmaf(r.tx, acc[i][j][v], dpr);
                    mab = fmaxf(mab, fabsf(ab[u]));
                    mds = fmaxf(mds, fabsf(ds[u]));
                }
                *reinterpret_cast<typename Quad<ES>::T *>(wd + (64 * j + 8 * q) * ES) =
                    pack_quad<OT>(ab[0], ab[1], ab[2], ab[3]);
                *reinterpret_cast<typename Quad<ES>::T *>(wd + (64 * j + 32 + 8 * q) * ES) =
                    pack_quad<OT>(ds[0], ds[1], ds[2], ds[3]);
            }
        });
        dpr = add_xor32(dpr) * cdp;
        if (gh == 0 && cols > 0) atomicAdd(p.dprob + row, dpr);
        // Materialise both maxima per row block: otherwise the compiler sinks
        // their max chains into the amax branch at the end, keeping all 512
        // ab/dswiglu values of the lane live across the epilogue (~1 KB of
        // scratch per lane).
        asm volatile("" : "+v"(mab), "+v"(mds));
        const uint32_t rb = (uint32_t)(n2 * ES);
        stage_flush<ES, 8>(stage, static_cast<char *>(p.d) + ((qr + 32 * i) * n2 + dq) * ES, rb, 32, dcols * ES, lane);
        if (p.d_col)
            stage_flush<ES, 8>(stage, static_cast<char *>(p.d_col) + ((qr + 32 * i) * n2 + dq) * ES, rb, 32,
                               dcols * ES, lane);
    });
    if (p.amax) {
        // both maxima with one barrier: red[w] and red[4 + w]
        const float wab = wave_max(mab), wds = wave_max(mds);
        const int t = threadIdx.x;
        if ((t & 63) == 0) {
            red[t >> 6] = wab;
            red[4 + (t >> 6)] = wds;
        }
        __syncthreads();
        if (t == 0) {
            const float a0 = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
            const float a1 = fmaxf(fmaxf(red[4], red[5]), fmaxf(red[6], red[7]));
            if (a0 > 0.0f) atomicMax(reinterpret_cast<unsigned int *>(p.amax + 2 * g), __float_as_uint(a0));
            if (a1 > 0.0f) atomicMax(reinterpret_cast<unsigned int *>(p.amax + 2 * g + 1), __float_as_uint(a1));
        }
    }
}

template <int F, int EPI, bool CLAMP, int OT = -1>
__global__ void __launch_bounds__(256) k_grouped(GroupedParams p)
{
    BSG_DECLARE_RING(F, ring);
    __shared__ float red[8];
    __shared__ __attribute__((aligned(16))) float prob_lds[kTileM];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6, wm = w >> 1, wn = w & 1;
    const TileCoord tc = tile_of(blockIdx.x, p.m / kTileM, (p.n + kTileN - 1) / kTileN, (int64_t)gridDim.x);
    const int64_t m0 = tc.mt * kTileM, n0 = tc.nt * kTileN;
    const int64_t valid_m = p.offsets[p.num_experts - 1];
    if (m0 >= valid_m) return;                      // uniform per workgroup
    const int g = __builtin_amdgcn_readfirstlane(expert_of(p.offsets, (int)p.num_experts, m0));
    const int64_t rows_b = p.n - n0 < kTileN ? p.n - n0 : kTileN;

    OperandDesc A{p.a + m0 * p.row_bytes, (uint32_t)(kTileM * p.row_bytes), p.row_bytes, p.sfa,
                  0, p.m_t, p.k_t, m0 / 128, p.m_t - 1};
    // Expert g's weights: slice g of the (N,K,L) tensor and of its scale
    // atoms, or (discrete weights) the expert's own allocations, whose scale
    // atoms have L = 1.
    const uint8_t *bg = p.b_ptrs ? reinterpret_cast<const uint8_t *>(p.b_ptrs[g]) : p.b + (int64_t)g * p.n * p.row_bytes;
    const uint8_t *sfbg = p.sfb_ptrs ? reinterpret_cast<const uint8_t *>(p.sfb_ptrs[g]) : p.sfb;
    OperandDesc B{bg + n0 * p.row_bytes, (uint32_t)(rows_b * p.row_bytes), p.row_bytes, sfbg,
                  p.sfb_ptrs ? 0 : g, p.n_t, p.k_t, n0 / 128, p.n_t - 1};
    // n-major B ([L][K][N], FP8 only): expert g's K rows of N codes
    if constexpr (b_t(F)) mn_major_operand(B, p.b, g, p.n, n0, rows_b, p.k);
    const float alpha = p.alpha[g];
    // The tile's 256 prob values go straight to LDS ahead of the operand
    // loads (wave w: rows 64w..64w+63; M is a multiple of 256), so the K
    // loop's first wait and barrier cover them and the epilogue starts with
    // no global load.  (Issued after every scalar load above: the asm is a
    // memory clobber, and values loaded after it would not stay in SGPRs.)
    {
        const int wu = __builtin_amdgcn_readfirstlane(w);
        lds_load4(make_rsrc_words(p.prob + m0, kTileM * 4), reinterpret_cast<uint8_t *>(prob_lds) + 256 * wu,
                  4u * (64u * (uint32_t)wu + (uint32_t)lane));
    }
    f32x16 acc[4][4];
    mainloop_pipe<F>(acc, ring, A, B, p.k);

    if constexpr (EPI == EPI_SRELU_FP8) {
        epilogue_srelu_fp8<CLAMP, OT == -1 ? DT_E4M3 : OT>(p, acc, wave_stage(ring, __builtin_amdgcn_readfirstlane(w)), m0, n0, alpha,
                                  wm, wn, lane, prob_lds);
    } else if constexpr (EPI == EPI_DSWIGLU_FP8) {
        epilogue_dswiglu_fp8<OT == DT_E5M2>(p, acc, wave_stage(ring, __builtin_amdgcn_readfirstlane(w)), m0, n0, alpha * alpha,
                             p.beta[g], wm, wn, lane, prob_lds);
    } else if constexpr (EPI == EPI_DSWIGLU) {
        epilogue_dswiglu<OT>(p, acc, wave_stage(ring, __builtin_amdgcn_readfirstlane(w)), m0, n0, g, alpha * alpha,
                             p.beta[g], wm, wn, lane, red, prob_lds);
    } else {
        epilogue_grouped<F, EPI, CLAMP, OT>(p, acc, wave_stage(ring, __builtin_amdgcn_readfirstlane(w)), m0, n0, g,
                                            alpha, wm, wn, lane, red, prob_lds);
    }
}

inline GroupedParams grouped_params(const GroupedArgs &a)
{
    GroupedParams p;
    p.a = a.a; p.b = a.b; p.sfa = a.sfa; p.sfb = a.sfb; p.offsets = a.offsets;
    p.b_ptrs = a.b_ptrs; p.sfb_ptrs = a.sfb_ptrs;
    p.alpha = a.alpha; p.prob = a.prob; p.norm_const = a.norm_const; p.bias = a.bias;
    p.c = a.c; p.d = a.d; p.d_col = a.d_col; p.amax = a.amax;
    p.sfd_row = a.sfd_row; p.sfd_col = a.sfd_col;
    p.m = a.m; p.n = a.n; p.k = a.k; p.num_experts = a.num_experts;
    p.m_t = (a.m + 127) / 128; p.n_t = (a.n + 127) / 128; p.k_t = (a.k + 127) / 128;
    p.row_bytes = row_bytes_of(a.fmt, a.k);
    p.c_dtype = a.c_dtype; p.d_dtype = a.d_dtype; p.bias_dtype = a.bias_dtype;
    p.tanh_s = a.tanh_s;
    p.tq = tanh_sq_const(a.tanh_s);
    p.beta = a.beta;
    p.cfwd = a.cfwd;
    p.dprob = a.dprob;
    return p;
}

template <int F, int EPI, int OT = -1>
static void launch_srelu_variant(const GroupedParams &p, dim3 grid, hipStream_t s)
{
    // C and D both bf16: a kernel whose epilogue has one compile-time store
    // path (with every output type in one kernel the register allocator
    // spilled accumulators, and the spill reloads waited on the stores)
    if constexpr (EPI == EPI_SRELU) {
        if (p.c && p.c_dtype == DT_BF16 && p.d_dtype == DT_BF16) {
            if (p.tanh_s > 0.0f) hipLaunchKernelGGL((k_grouped<F, EPI, true, DT_BF16>), grid, dim3(kThreads), 0, s, p);
            else hipLaunchKernelGGL((k_grouped<F, EPI, false, DT_BF16>), grid, dim3(kThreads), 0, s, p);
            return;
        }
    }
    if (p.tanh_s > 0.0f) hipLaunchKernelGGL((k_grouped<F, EPI, true, OT>), grid, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((k_grouped<F, EPI, false, OT>), grid, dim3(kThreads), 0, s, p);
}

// grouped_gemm_dswiglu with FP8 operands and n-major B (kernels_dswiglu_mn.hip).
void launch_dswiglu_bn(const GroupedParams &p, int fmt, int d_dtype, dim3 grid, hipStream_t s);

// MX-quantised D of grouped_gemm_srelu (kernels_srelu_mx.hip).
void launch_grouped_srelu_mx(const GroupedParams &p, int fmt, int d_dtype, dim3 grid, hipStream_t s);

}  // namespace bsg
