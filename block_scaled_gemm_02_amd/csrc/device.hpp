// Device building blocks for the gfx950 block-scaled GEMM kernels.
//
// One workgroup = 4 wave64s computes a 256x256 output tile; each wave owns a
// 128x128 quadrant held as 4x4 fp32 32x32 accumulator blocks (256 values per
// lane, resident in AGPR/VGPR for the whole K loop).  K advances in steps of
// 128 bytes per row (E4M3: 128 elements, E2M1: 256, BF16: 64), double
// buffered in LDS through registers.
//
// Operand lane layouts of the CDNA4 32x32 MFMAs, measured on MI355X:
//   * v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 operands: lane (r = l%32,
//     g = l/32) holds row r, K elements [16g,16g+16) in bytes 0..15 and
//     [32+16g, 32+16g+16) in bytes 16..31 of its 8-dword operand.
//   * same instruction, E2M1 operands: lane (r,g) holds K elements
//     [32g, 32g+32) as 16 bytes, element 2j in the low nibble of byte j.
//   * v_mfma_f32_32x32x16_bf16: lane (r,g) holds K elements [8g, 8g+8).
//   * The E8M0 scale operand of lane (r,g) is the byte selected by op_sel of
//     its 32-bit register and scales row r over K elements [32g, 32g+32) of
//     the instruction's 64-wide K range.
//   * Accumulator: lane (c = l%32, g) register v holds row
//     8*(v/4) + 4*g + v%4, column c.
// In every format a lane therefore reads 16-byte chunks of the 128-byte
// K step: chunk 2s+g for sub-step s (E2M1: s<4, BF16: s<4), and chunks
// 4s+g (low half) and 4s+2+g (high half) for E4M3 (s<2).
//
// LDS rows are 128 bytes; chunk c of row r is stored at chunk c ^ (r % 8),
// which makes both the 8-lanes-per-row stores and the 32-rows-per-wave
// operand reads free of bank conflicts.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace bsg {

// Compile-time loop: f(std::integral_constant<int, 0>) ... f(<N-1>).  Used
// wherever an accumulator block is selected, so that no index into the
// accumulator array is ever a run-time value (which would move it to scratch).
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (N > 0) {
        static_for<N - 1>(f);
        f(std::integral_constant<int, N - 1>{});
    }
}

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

enum Fmt : int { FMT_E4M3 = 0, FMT_E2M1 = 1, FMT_BF16 = 2 };

constexpr int kTileM = 256;
constexpr int kTileN = 256;
constexpr int kRowBytes = 128;                  // bytes of one K step per row
constexpr int kThreads = 256;
constexpr int kStageBytes = kTileM * kRowBytes; // one operand, one stage
constexpr uint32_t kOOB = 0x80000000u;          // added to an offset: reads zeros

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ __forceinline__ i32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// ---------------------------------------------------------------------------
// Conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x)
{
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;   // NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint16_t f32_to_f16_rne(float x)
{
    _Float16 h = (_Float16)x;
    return __builtin_bit_cast(uint16_t, h);
}

// Two floats -> two E4M3 codes (round to nearest even).  The hardware
// conversion returns NaN beyond the format's range instead of saturating,
// so inputs are clamped to +-448 first.
__device__ __forceinline__ uint32_t pack2_e4m3(float a, float b)
{
    a = fminf(fmaxf(a, -448.0f), 448.0f);
    b = fminf(fmaxf(b, -448.0f), 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// E8M0 byte of the smallest power of two >= sigma (sigma >= 0), clamped to
// [0, 254]; sigma == 0 gives 0.
__device__ __forceinline__ uint32_t e8m0_ceil(float sigma)
{
    uint32_t u = __float_as_uint(sigma);
    if (!(sigma > 0.0f)) return 0u;
    uint32_t e = u >> 23;                 // biased exponent (sigma > 0, finite)
    uint32_t mant = u & 0x7FFFFFu;
    if (e == 0u) return mant > 0x400000u ? 1u : 0u;   // subnormal: 2^-126 or 2^-127
    if (mant != 0u) e += 1u;
    return e > 254u ? 254u : e;
}

// ---------------------------------------------------------------------------
// Scale-atom addressing: byte of (row r, k-block kb, batch l) lives at
// (((l*MN' + r/128)*K' + kb/4)*32 + r%32)*16 + ((r%128)/32)*4 + kb%4.
// A lane with row index r%32 loads the 16 bytes at atom + (r%32)*16:
// word j = rows 32j + r%32 of the atom, byte = k-block within the atom.
// ---------------------------------------------------------------------------
__device__ __forceinline__ const uint8_t *sf_atom(const uint8_t *sf, int64_t l, int64_t mn_t,
                                                 int64_t mt, int64_t k_t, int64_t kt)
{
    return sf + (((l * mn_t + mt) * k_t + kt) * 512);
}

// Replace bytes of k-blocks at or past `kblocks` (K padding) with 1.0.
__device__ __forceinline__ i32x4 sanitize_scales(i32x4 w, int kt, int kblocks)
{
    int valid = kblocks - 4 * kt;
    if (valid >= 4) return w;
    uint32_t keep = valid <= 0 ? 0u : (0xFFFFFFFFu >> (8 * (4 - valid)));
    uint32_t fill = 0x7F7F7F7Fu & ~keep;
    w.x = (int)(((uint32_t)w.x & keep) | fill);
    w.y = (int)(((uint32_t)w.y & keep) | fill);
    w.z = (int)(((uint32_t)w.z & keep) | fill);
    w.w = (int)(((uint32_t)w.w & keep) | fill);
    return w;
}

// ---------------------------------------------------------------------------
// Mainloop
// ---------------------------------------------------------------------------
struct OperandDesc {
    const uint8_t *base;   // first row of this tile (row 0 of the 256-row panel)
    uint32_t bytes;        // readable bytes from base (rows past the end read 0)
    uint32_t row_bytes;    // bytes per row (K, K/2 or 2K)
    const uint8_t *sf;     // scale atoms (nullptr for BF16)
    int64_t sf_l, sf_mn_t, sf_k_t;  // batch index, ceil(MN/128), ceil(K/128)
    int64_t sf_mt0;        // atom row-group index of this tile's row 0
    int64_t sf_mt_max;     // last valid atom row-group index
};

template <int F>
struct FmtTraits;
template <>
struct FmtTraits<FMT_E4M3> {
    static constexpr int kSub = 2;      // MFMAs along K per 128-byte step
    static constexpr int kAtoms = 1;    // scale atoms along K per step
    static constexpr int kCode = 0;     // cbsz / blgp code
};
template <>
struct FmtTraits<FMT_E2M1> {
    static constexpr int kSub = 4;
    static constexpr int kAtoms = 2;
    static constexpr int kCode = 4;
};
template <>
struct FmtTraits<FMT_BF16> {
    static constexpr int kSub = 4;
    static constexpr int kAtoms = 0;
    static constexpr int kCode = -1;
};

// Global -> registers: thread t fetches chunk (t % 8) of rows t/8 + 32i,
// for a panel of 32*R rows.
template <int R>
__device__ __forceinline__ void g2r(i32x4 (&r)[R], const OperandDesc &d, __amdgpu_buffer_rsrc_t rs,
                                    int ks, int t)
{
    const uint32_t c = t & 7;
    const uint32_t kb = (uint32_t)ks * kRowBytes + 16u * c;
    // chunks past the end of a row read zeros: push them past num_records
    // (rows * row_bytes < 2^31 is checked on the host, so this cannot wrap)
    const uint32_t koff = kb + (kb < d.row_bytes ? 0u : kOOB);
#pragma unroll
    for (int i = 0; i < R; ++i) {
        uint32_t row = (uint32_t)(t >> 3) + 32u * i;
        r[i] = buf_load16(rs, row * d.row_bytes + koff);
    }
}

template <int R>
__device__ __forceinline__ void r2lds(uint8_t *lds, const i32x4 (&r)[R], int t)
{
    const uint32_t c = t & 7, rr = t >> 3;
    const uint32_t pc = c ^ (rr & 7);
#pragma unroll
    for (int i = 0; i < R; ++i) {
        uint32_t row = rr + 32u * i;
        *reinterpret_cast<i32x4 *>(lds + row * kRowBytes + 16u * pc) = r[i];
    }
}

__device__ __forceinline__ i32x4 lds_chunk(const uint8_t *lds, uint32_t row, uint32_t chunk)
{
    return *reinterpret_cast<const i32x4 *>(lds + row * kRowBytes + 16u * (chunk ^ (row & 7)));
}

// Scale words for one operand and one 128-wide K atom: 4 words (row groups),
// byte = k-block in the atom; shifted so op_sel 2s picks k-block 2s + g.
__device__ __forceinline__ i32x4 load_scale_words(const OperandDesc &d, int wq, int kt, int kblocks,
                                                  int lane)
{
    int64_t mt = d.sf_mt0 + wq;
    if (mt > d.sf_mt_max) mt = d.sf_mt_max;
    int ktc = kt < (int)d.sf_k_t ? kt : (int)d.sf_k_t - 1;
    const uint8_t *p = sf_atom(d.sf, d.sf_l, d.sf_mn_t, mt, d.sf_k_t, ktc) + (lane & 31) * 16;
    i32x4 w = *reinterpret_cast<const i32x4 *>(p);
    w = sanitize_scales(w, kt, kblocks);
    if (lane >= 32) {
        w.x = (int)((uint32_t)w.x >> 8);
        w.y = (int)((uint32_t)w.y >> 8);
        w.z = (int)((uint32_t)w.z >> 8);
        w.w = (int)((uint32_t)w.w >> 8);
    }
    return w;
}

template <int F, int S, int NB>
__device__ __forceinline__ void mma_substep(f32x16 (&acc)[4][NB], const uint8_t *la, const uint8_t *lb,
                                            uint32_t arow, uint32_t brow, int g,
                                            const i32x4 (&sa)[2], const i32x4 (&sb)[2])
{
    if constexpr (F == FMT_E4M3) {
        i32x8 af[4], bf[NB];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            i32x4 lo = lds_chunk(la, arow + 32u * i, 4 * S + g);
            i32x4 hi = lds_chunk(la, arow + 32u * i, 4 * S + 2 + g);
            af[i] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            i32x4 blo = lds_chunk(lb, brow + 32u * j, 4 * S + g);
            i32x4 bhi = lds_chunk(lb, brow + 32u * j, 4 * S + 2 + g);
            bf[j] = i32x8{blo.x, blo.y, blo.z, blo.w, bhi.x, bhi.y, bhi.z, bhi.w};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    af[i], bf[j], acc[i][j], 0, 0, 2 * S, sa[0][i], 2 * S, sb[0][j]);
    } else if constexpr (F == FMT_E2M1) {
        i32x8 af[4], bf[NB];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            i32x4 a = lds_chunk(la, arow + 32u * i, 2 * S + g);
            af[i] = i32x8{a.x, a.y, a.z, a.w, 0, 0, 0, 0};
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            i32x4 b = lds_chunk(lb, brow + 32u * j, 2 * S + g);
            bf[j] = i32x8{b.x, b.y, b.z, b.w, 0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    af[i], bf[j], acc[i][j], 4, 4, 2 * (S & 1), sa[S >> 1][i], 2 * (S & 1),
                    sb[S >> 1][j]);
    } else {
        bf16x8 af[4], bf[NB];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            af[i] = __builtin_bit_cast(bf16x8, lds_chunk(la, arow + 32u * i, 2 * S + g));
#pragma unroll
        for (int j = 0; j < NB; ++j)
            bf[j] = __builtin_bit_cast(bf16x8, lds_chunk(lb, brow + 32u * j, 2 * S + g));
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
}

// Full K loop for one 256 x (64*NB) tile: 4 waves as 2 x 2, each wave owning
// 128 x (32*NB).  `lds` holds 2 stages x (A, B) x 32 KB.  NB = 4 for the
// block-scaled formats (a wave's columns must be one 128-row scale atom).
// On return every wave has passed a final barrier, so `lds` may be reused.
template <int F, int NB = 4>
__device__ __forceinline__ void mainloop(f32x16 (&acc)[4][NB], uint8_t *lds, const OperandDesc &A,
                                         const OperandDesc &B, int64_t k)
{
    static_assert(NB == 4 || F == FMT_BF16, "scaled formats need 128-column wave tiles");
    const int t = threadIdx.x, lane = t & 63, w = t >> 6, wm = w >> 1, wn = w & 1, g = lane >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int nks = (int)((A.row_bytes + kRowBytes - 1) / kRowBytes);
    const int kblocks = (int)(k / 32);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A.base, A.bytes);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(B.base, B.bytes);
    const uint32_t arow = 128u * wm + (lane & 31);
    const uint32_t brow = 32u * NB * wn + (lane & 31);
    constexpr int NA = FmtTraits<F>::kAtoms;

    i32x4 pa[8], pb[2 * NB];
    i32x4 sa[2] = {}, sb[2] = {}, na[2] = {}, nb[2] = {};
    if (nks > 0) {
        g2r(pa, A, ra, 0, t);
        g2r(pb, B, rb, 0, t);
        if constexpr (NA > 0) {
#pragma unroll
            for (int q = 0; q < NA; ++q) {
                sa[q] = load_scale_words(A, wm, NA * 0 + q, kblocks, lane);
                sb[q] = load_scale_words(B, wn, NA * 0 + q, kblocks, lane);
            }
        }
        r2lds(lds, pa, t);
        r2lds(lds + kStageBytes, pb, t);
    }
    __syncthreads();

    for (int ks = 0; ks < nks; ++ks) {
        uint8_t *cur = lds + (ks & 1) * 2 * kStageBytes;
        uint8_t *nxt = lds + ((ks + 1) & 1) * 2 * kStageBytes;
        const bool more = ks + 1 < nks;
        if (more) {
            g2r(pa, A, ra, ks + 1, t);
            g2r(pb, B, rb, ks + 1, t);
            if constexpr (NA > 0) {
#pragma unroll
                for (int q = 0; q < NA; ++q) {
                    na[q] = load_scale_words(A, wm, NA * (ks + 1) + q, kblocks, lane);
                    nb[q] = load_scale_words(B, wn, NA * (ks + 1) + q, kblocks, lane);
                }
            }
        }
        mma_substep<F, 0, NB>(acc, cur, cur + kStageBytes, arow, brow, g, sa, sb);
        mma_substep<F, 1, NB>(acc, cur, cur + kStageBytes, arow, brow, g, sa, sb);
        if constexpr (FmtTraits<F>::kSub == 4) {
            mma_substep<F, 2, NB>(acc, cur, cur + kStageBytes, arow, brow, g, sa, sb);
            mma_substep<F, 3, NB>(acc, cur, cur + kStageBytes, arow, brow, g, sa, sb);
        }
        if (more) {
            r2lds(nxt, pa, t);
            r2lds(nxt + kStageBytes, pb, t);
            if constexpr (NA > 0) {
#pragma unroll
                for (int q = 0; q < NA; ++q) { sa[q] = na[q]; sb[q] = nb[q]; }
            }
        }
        __syncthreads();
    }
}

// Row / column of accumulator element v of block (i, j) for this lane,
// relative to the tile origin.
__device__ __forceinline__ int acc_row(int wm, int i, int v, int lane)
{
    return 128 * wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}
__device__ __forceinline__ int acc_col(int wn, int j, int lane) { return 128 * wn + 32 * j + (lane & 31); }

// Max over the 32 lanes of each half-wave (lanes 0-31 and 32-63 separately):
// quad and row DPP steps reduce 16 lanes, a swizzle folds the two rows.
template <int CTRL>
__device__ __forceinline__ float dpp_max_c(float x)
{
    const int y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false);
    return fmaxf(x, __int_as_float(y));
}
__device__ __forceinline__ float half_wave_max(float x)
{
    x = dpp_max_c<0xB1>(x);    // quad_perm [1,0,3,2]
    x = dpp_max_c<0x4E>(x);    // quad_perm [2,3,0,1]
    x = dpp_max_c<0x141>(x);   // row_half_mirror
    x = dpp_max_c<0x140>(x);   // row_mirror
    const int y = __builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F);   // lane ^ 16
    return fmaxf(x, __int_as_float(y));
}

// E4M3 code of one value (round to nearest even, saturating to +-448).
__device__ __forceinline__ uint32_t e4m3_code(float x) { return pack2_e4m3(x, 0.0f) & 0xFFu; }

// The MX output quantiser's scale step for a block with max |D| = amax:
// SF = smallest power of two >= norm_const * amax / 448 (E8M0 byte), and
// the factor norm_const / SF that maps the block into E4M3 range.
__device__ __forceinline__ uint32_t mx_scale_byte(float amax, float norm_const, float &inv)
{
    const float sigma = (norm_const * amax) * (1.0f / 448.0f);
    const uint32_t byte = e8m0_ceil(sigma);
    inv = fminf(ldexpf(norm_const, 127 - (int)byte), 3.402823466e38f);
    return byte;
}

__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

// Workgroup max of non-negative values; one atomicMax on the float's bits.
__device__ __forceinline__ void block_amax_atomic(float local, float *dst, float *red4)
{
    const int t = threadIdx.x;
    float m = wave_max(local);
    if ((t & 63) == 0) red4[t >> 6] = m;
    __syncthreads();
    if (t == 0) {
        float r = fmaxf(fmaxf(red4[0], red4[1]), fmaxf(red4[2], red4[3]));
        if (r > 0.0f) atomicMax(reinterpret_cast<unsigned int *>(dst), __float_as_uint(r));
    }
}

// fp32 tanh for y >= 0: odd Taylor series below 1/16 (relative error
// < 1e-11 there), otherwise 1 - 2/(e^(2y) + 1) with e^(2y) = 2^(2y log2 e).
__device__ __forceinline__ float tanh_pos(float y)
{
    if (y < 0.0625f) {
        float y2 = y * y;
        // y - y^3/3 + 2y^5/15 - 17y^7/315
        float p = -17.0f / 315.0f;
        p = p * y2 + 2.0f / 15.0f;
        p = p * y2 - 1.0f / 3.0f;
        p = p * y2;
        return y + y * p;
    }
    float e = __builtin_amdgcn_exp2f(fminf(y * 2.8853900817779268f, 64.0f)); // 2*log2(e)
    return 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
}

}  // namespace bsg
