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
// Branch-free, so that it does not split the K step into basic blocks.
__device__ __forceinline__ i32x4 sanitize_scales(i32x4 w, int kt, int kblocks)
{
    const int valid = kblocks - 4 * kt;
    const int vc = valid < 0 ? 0 : (valid > 4 ? 4 : valid);
    const uint32_t keep = (uint32_t)(0xFFFFFFFFull >> (8 * (4 - vc)));
    const uint32_t fill = 0x7F7F7F7Fu & ~keep;
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

// ===========================================================================
// Pipelined mainloop: a 4-stage LDS ring filled by direct-to-LDS buffer loads
// ===========================================================================
// K advances 64 bytes per row per step.  A stage holds the A panel (256 rows
// x 64 B), the B panel (64*NB rows x 64 B) and, for the block-scaled formats,
// the four 512-byte scale atoms the tile needs for that step (A row groups 0
// and 1, B row groups 0 and 1; each padded to 1 KB).  Every lane of a
// direct-to-LDS load writes 16 bytes at M0 + 16*lane, so one instruction
// fills 16 rows; lane l fetches logical chunk (l%4) ^ ((row/4)%4) of row
// l/4, which stores chunk c of row r at chunk c ^ ((r/4)%4).  The gfx950 LDS
// serves a 128-bit read for 16 lanes (256 bytes, 64 banks) per cycle; the 16
// lanes read one chunk of 16 consecutive rows, and this swizzle puts them on
// 16 distinct bank groups (rows r, r+4, r+8, r+12 share row%4 and differ in
// (r/4)%4).  Loads past a row's end or past the panel read zeros (buffer
// range check).
//
// Step ks: wait until this wave's loads of stage ks+1 have landed, barrier
// (all waves: stage ks+1 ready, stage ks no longer read), read the fragments
// of stage ks+1 into the idle register set, issue the loads of stage ks+4
// into the slot stage ks used, and run the MFMAs of stage ks on the other
// register set.
constexpr int kKS = 64;                    // bytes per row per step
constexpr int kRing = 4;                   // stages in flight
constexpr int kStA = kTileM * kKS;         // 16 KB
constexpr int kStB = 256 * kKS;            // 16 KB (NB = 4)
constexpr int kStS = 4 * 1024;             // scale atoms
constexpr int kStageScaled = kStA + kStB + kStS;
constexpr int kStagePlain = kStA + kStB;

template <int F>
struct Ring {
    static constexpr bool kScaled = F != FMT_BF16;
    static constexpr int kStage = kScaled ? kStageScaled : kStagePlain;
    static constexpr int kBytes = kRing * kStage;
};

typedef __attribute__((address_space(3))) void lds_void;

// Buffer resource as four dwords for inline asm (raw buffer: stride 0).
__device__ __forceinline__ i32x4 make_rsrc_words(const void *base, uint32_t bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return i32x4{(int)(uint32_t)a, (int)(uint32_t)(a >> 32) & 0xFFFF, (int)bytes, 0x00020000};
}

// 16 bytes per lane from a buffer straight into LDS at dst + 16*lane.  Issued
// through asm so that the compiler, which cannot tell the ring slots apart,
// adds no waits of its own: completion is tracked explicitly with vmcnt and
// published to the other waves with a barrier.
__device__ __forceinline__ void lds_load16(const i32x4 &rsrc, uint8_t *dst, uint32_t voff)
{
    const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void *)dst;
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}

// Operand fragments of one step for one wave: two 16-byte chunks per
// 32-row block (E4M3: low/high halves of one MFMA operand; E2M1 and BF16:
// the operands of the step's two MFMAs), plus the scale words.
template <int NB>
struct Frags {
    i32x4 a[4][2];
    i32x4 b[NB][2];
    i32x4 sa, sb;
};

template <int N>
__device__ __forceinline__ void s_wait_vm()
{
    // vmcnt(N), expcnt and lgkmcnt untouched (gfx9 encoding)
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void s_wait_lgkm0()
{
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

struct PipeDesc {
    i32x4 ra, rb, rs;         // operand panels; this wave's scale atoms (buffer resources)
    uint32_t row_bytes;
    uint32_t va[4], vb[4];    // per-lane voffset of this wave's code loads (step 0)
    uint32_t lc16;            // 16 * logical chunk of this lane's loads
    uint32_t vs;              // per-lane voffset of this wave's scale atom (kt = 0)
    int kblocks;              // valid 32-wide K blocks
    int sf_kt;                // K atoms per row group (ceil(K/128))
};

// The four ring slots are distinct LDS objects, selected by compile-time
// index: the compiler can then see that a pending direct-to-LDS load into
// one slot does not alias the reads of another, and adds no waits of its own.
template <int F>
struct RingSlots {
    uint8_t *s0, *s1, *s2, *s3;
    template <int U>
    __device__ __forceinline__ uint8_t *at() const
    {
        if constexpr (U == 0) return s0;
        else if constexpr (U == 1) return s1;
        else if constexpr (U == 2) return s2;
        else return s3;
    }
};

// Declares the ring in the calling kernel's shared memory.
#define BSG_DECLARE_RING(F, name)                                                                    \
    __shared__ __attribute__((aligned(16))) uint8_t name##_0[Ring<F>::kStage];                      \
    __shared__ __attribute__((aligned(16))) uint8_t name##_1[Ring<F>::kStage];                      \
    __shared__ __attribute__((aligned(16))) uint8_t name##_2[Ring<F>::kStage];                      \
    __shared__ __attribute__((aligned(16))) uint8_t name##_3[Ring<F>::kStage];                      \
    const ::bsg::RingSlots<F> name{name##_0, name##_1, name##_2, name##_3}

template <int F, int NB>
__device__ __forceinline__ void issue_stage(const PipeDesc &d, uint8_t *st, int ks, int w)
{
    const uint32_t kb = (uint32_t)ks * kKS;
    const uint32_t oob = (kb + d.lc16 < d.row_bytes) ? 0u : kOOB;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        lds_load16(d.ra, st + 1024 * (4 * w + q), d.va[q] + kb + oob);
#pragma unroll
    for (int q = 0; q < NB; ++q)
        lds_load16(d.rb, st + kStA + 1024 * (NB * w + q), d.vb[q] + kb + oob);
    if constexpr (Ring<F>::kScaled) {
        // atom kt of this step: 128 K elements = 2 steps (E4M3) or 1 (E2M1)
        const int kt = F == FMT_E4M3 ? ks >> 1 : ks;
        const uint32_t so = kt < d.sf_kt ? d.vs + (uint32_t)kt * 512u : kOOB;
        lds_load16(d.rs, st + kStA + kStB + 1024 * w, so);
    }
}

template <int F, int NB>
__device__ __forceinline__ void read_frags(Frags<NB> &f, const uint8_t *st, int wm, int wn, int lane)
{
    const uint32_t r = lane & 31, g = lane >> 5;
    const uint32_t swz = (r >> 2) & 3;
    const uint32_t p0 = 16u * (g ^ swz), p1 = 16u * ((2u + g) ^ swz);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint8_t *row = st + (128u * wm + 32u * i + r) * kKS;
        f.a[i][0] = *reinterpret_cast<const i32x4 *>(row + p0);
        f.a[i][1] = *reinterpret_cast<const i32x4 *>(row + p1);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const uint8_t *row = st + kStA + (32u * NB * wn + 32u * j + r) * kKS;
        f.b[j][0] = *reinterpret_cast<const i32x4 *>(row + p0);
        f.b[j][1] = *reinterpret_cast<const i32x4 *>(row + p1);
    }
    if constexpr (Ring<F>::kScaled) {
        const uint8_t *sc = st + kStA + kStB;
        f.sa = *reinterpret_cast<const i32x4 *>(sc + 1024 * wm + 16 * r);
        f.sb = *reinterpret_cast<const i32x4 *>(sc + 1024 * (2 + wn) + 16 * r);
    }
}

// Byte of the scale word that an MFMA lane consumes is moved to byte 0
// (E4M3: k-block 2*(ks%2) + g of the atom) or byte 2s (E2M1: k-block 2s+g).
template <int F, int PAR>
__device__ __forceinline__ i32x4 prep_scales(i32x4 w, int kt, int kblocks, int g)
{
    w = sanitize_scales(w, kt, kblocks);
    const uint32_t sh = F == FMT_E4M3 ? 8u * (g + 2 * PAR) : 8u * g;
    w.x = (int)((uint32_t)w.x >> sh);
    w.y = (int)((uint32_t)w.y >> sh);
    w.z = (int)((uint32_t)w.z >> sh);
    w.w = (int)((uint32_t)w.w >> sh);
    return w;
}

template <int F, int NB, int PAR>
__device__ __forceinline__ void mma_step(f32x16 (&acc)[4][NB], const Frags<NB> &f, int ks, int kblocks,
                                         int g)
{
    if constexpr (F == FMT_E4M3) {
        const i32x4 sa = prep_scales<F, PAR>(f.sa, ks >> 1, kblocks, g);
        const i32x4 sb = prep_scales<F, PAR>(f.sb, ks >> 1, kblocks, g);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const i32x8 av{f.a[i][0].x, f.a[i][0].y, f.a[i][0].z, f.a[i][0].w,
                           f.a[i][1].x, f.a[i][1].y, f.a[i][1].z, f.a[i][1].w};
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const i32x8 bv{f.b[j][0].x, f.b[j][0].y, f.b[j][0].z, f.b[j][0].w,
                               f.b[j][1].x, f.b[j][1].y, f.b[j][1].z, f.b[j][1].w};
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    av, bv, acc[i][j], 0, 0, 0, sa[i], 0, sb[j]);
            }
        }
    } else if constexpr (F == FMT_E2M1) {
        const i32x4 sa = prep_scales<F, 0>(f.sa, ks, kblocks, g);
        const i32x4 sb = prep_scales<F, 0>(f.sb, ks, kblocks, g);
        static_for<2>([&](auto sc) {
            constexpr int S = decltype(sc)::value;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const i32x8 av{f.a[i][S].x, f.a[i][S].y, f.a[i][S].z, f.a[i][S].w, 0, 0, 0, 0};
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const i32x8 bv{f.b[j][S].x, f.b[j][S].y, f.b[j][S].z, f.b[j][S].w, 0, 0, 0, 0};
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        av, bv, acc[i][j], 4, 4, 2 * S, sa[i], 2 * S, sb[j]);
                }
            }
        });
    } else {
        static_for<2>([&](auto sc) {
            constexpr int S = decltype(sc)::value;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, f.a[i][S]), __builtin_bit_cast(bf16x8, f.b[j][S]),
                        acc[i][j], 0, 0, 0);
        });
    }
}

// Loads issued per wave per stage (codes + one scale atom).
template <int F, int NB>
constexpr int loads_per_stage() { return 4 + NB + (Ring<F>::kScaled ? 1 : 0); }

// MFMAs and fragment reads of one step, and how the scheduler interleaves
// them: a burst of LDS reads ahead of the MFMAs stalls the matrix pipe (the
// reads' returns and the MFMA operand fetches compete), one read after each
// MFMA keeps it busy.
template <int F, int NB>
constexpr int mfmas_per_step() { return (F == FMT_E4M3 ? 1 : 2) * 4 * NB; }
template <int F, int NB>
constexpr int reads_per_step() { return 8 + 2 * NB + (Ring<F>::kScaled ? 2 : 0); }

template <int F, int NB>
__device__ __forceinline__ void interleave_hint()
{
    constexpr int M = mfmas_per_step<F, NB>(), R = reads_per_step<F, NB>();
    static_for<R>([&](auto q) {
        constexpr int Q = decltype(q)::value;
        constexpr int m = (M * (Q + 1)) / R - (M * Q) / R;   // MFMAs before read Q
        if constexpr (m > 0) __builtin_amdgcn_sched_group_barrier(0x008, m, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    });
}

// One K step in ring slot U (K step ks = 4q + U): see the comment above.
template <int F, int NB, int U>
__device__ __forceinline__ void pipe_step(f32x16 (&acc)[4][NB], Frags<NB> &cur, Frags<NB> &nxt,
                                          const PipeDesc &d, const RingSlots<F> &ring, int ks, int w,
                                          int wm, int wn, int lane)
{
    constexpr int V = loads_per_stage<F, NB>();
    s_wait_vm<2 * V>();             // this wave's stage ks+1 has landed
    s_wait_lgkm0();                 // our reads of stage ks are complete
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue_stage<F, NB>(d, ring.template at<U>(), ks + kRing, w);
    __builtin_amdgcn_sched_barrier(0);
    read_frags<F, NB>(nxt, ring.template at<(U + 1) % kRing>(), wm, wn, lane);
    mma_step<F, NB, U & 1>(acc, cur, ks, d.kblocks, lane >> 5);
    interleave_hint<F, NB>();
}

// K loop over a 256 x (64*NB) tile, 4 waves as 2 x 2 (wave: 128 x 32*NB).
template <int F, int NB = 4>
__device__ __forceinline__ void mainloop_pipe(f32x16 (&acc)[4][NB], const RingSlots<F> &ring,
                                              const OperandDesc &A, const OperandDesc &B, int64_t k)
{
    static_assert(NB == 4 || F == FMT_BF16, "scaled formats need 128-column wave tiles");
    // the wave index is uniform: keep everything derived from it in SGPRs
    const int t = threadIdx.x, lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6), wm = w >> 1, wn = w & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    PipeDesc d;
    d.ra = make_rsrc_words(A.base, A.bytes);
    d.rb = make_rsrc_words(B.base, B.bytes);
    d.row_bytes = A.row_bytes;
    const uint32_t lrow = (uint32_t)lane >> 2;                       // row within a 16-row load
    const uint32_t lchunk = ((uint32_t)lane & 3) ^ ((lrow >> 2) & 3);
    d.lc16 = 16u * lchunk;
#pragma unroll
    for (int q = 0; q < 4; ++q) d.va[q] = (16u * (4 * w + q) + lrow) * A.row_bytes + d.lc16;
#pragma unroll
    for (int q = 0; q < NB; ++q) d.vb[q] = (16u * (NB * w + q) + lrow) * B.row_bytes + d.lc16;
    d.kblocks = (int)(k / 32);
    d.sf_kt = 0;
    d.rs = d.ra;
    d.vs = kOOB;
    if constexpr (Ring<F>::kScaled) {
        // wave w loads the K atom of atom row group w&1 of A (w < 2) or B (w >= 2)
        const OperandDesc &S = w < 2 ? A : B;
        const int64_t mt = S.sf_mt0 + (w & 1);
        const bool mt_ok = mt <= S.sf_mt_max;
        const uint8_t *base = S.sf + ((S.sf_l * S.sf_mn_t) * S.sf_k_t) * 512;
        d.rs = make_rsrc_words(base, (uint32_t)(S.sf_mn_t * S.sf_k_t * 512));
        d.vs = (lane < 32 && mt_ok) ? (uint32_t)(mt * S.sf_k_t * 512) + 16u * lane : kOOB;
        d.sf_kt = (int)S.sf_k_t;
    }

    const int nks = (int)((A.row_bytes + kKS - 1) / kKS);
    Frags<NB> fx, fy;
    issue_stage<F, NB>(d, ring.template at<0>(), 0, w);
    issue_stage<F, NB>(d, ring.template at<1>(), 1, w);
    issue_stage<F, NB>(d, ring.template at<2>(), 2, w);
    issue_stage<F, NB>(d, ring.template at<3>(), 3, w);
    constexpr int V = loads_per_stage<F, NB>();
    s_wait_vm<3 * V>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_frags<F, NB>(fx, ring.template at<0>(), wm, wn, lane);
    for (int ks = 0; ks < nks; ks += kRing) {
        pipe_step<F, NB, 0>(acc, fx, fy, d, ring, ks, w, wm, wn, lane);
        if (ks + 1 < nks) pipe_step<F, NB, 1>(acc, fy, fx, d, ring, ks + 1, w, wm, wn, lane);
        if (ks + 2 < nks) pipe_step<F, NB, 2>(acc, fx, fy, d, ring, ks + 2, w, wm, wn, lane);
        if (ks + 3 < nks) pipe_step<F, NB, 3>(acc, fy, fx, d, ring, ks + 3, w, wm, wn, lane);
    }
    s_wait_vm<0>();
    s_wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

// ===========================================================================
// Epilogue layout change: 4x4 transpose inside each lane quad
// ===========================================================================
// In the 32x32 accumulator layout, lane 4k+t holds column 4k+t of a block
// and registers 4q..4q+3 hold four consecutive rows 8q+4g+0..3.  Storing that
// directly writes 2-byte pieces of 64 different columns per instruction.  Two
// DPP butterfly stages (lane bit 0 with register bit 0, then lane bit 1 with
// register bit 1) transpose each 4x4 group so that lane 4k+t holds row
// 8q+4g+t, columns 4k..4k+3: 8 or 16 contiguous bytes per lane per store.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ void quad_swap_stage(float &x, float &y, bool hi)
{
    // hi lanes send x and take the partner's y into x; lo lanes send y and
    // take the partner's x into y
    const float recv = dpp_mov<CTRL>(hi ? x : y);
    x = hi ? recv : x;
    y = hi ? y : recv;
}

__device__ __forceinline__ void transpose4(float &a0, float &a1, float &a2, float &a3, int lane)
{
    const bool b0 = lane & 1, b1 = lane & 2;
    quad_swap_stage<0xB1>(a0, a1, b0);    // quad_perm [1,0,3,2]
    quad_swap_stage<0xB1>(a2, a3, b0);
    quad_swap_stage<0x4E>(a0, a2, b1);    // quad_perm [2,3,0,1]
    quad_swap_stage<0x4E>(a1, a3, b1);
}

// Calls f(i, j, q, row, col0, x) for every 4-row group q of accumulator block
// (i, j) after the quad transpose: this lane holds tile-relative row `row`,
// columns col0..col0+3 in x[0..3].  j is the innermost loop.
// i, j, q are passed as std::integral_constant so the callee can index
// per-block arrays with them.
template <int NB, class Fn>
__device__ __forceinline__ void for_each_row_quad(const f32x16 (&acc)[4][NB], int wm, int wn, int lane,
                                                  Fn &&f)
{
    const int t = lane & 3, g = lane >> 5, k4 = 4 * ((lane & 31) >> 2);
    static_for<16>([&](auto iq) {
        constexpr int i = decltype(iq)::value / 4, q = decltype(iq)::value % 4;
        const int row = 128 * wm + 32 * i + 8 * q + 4 * g + t;
        static_for<NB>([&](auto jj) {
            constexpr int j = decltype(jj)::value;
            float x[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            transpose4(x[0], x[1], x[2], x[3], lane);
            f(std::integral_constant<int, i>{}, jj, std::integral_constant<int, q>{}, row,
              32 * NB * wn + 32 * j + k4, x);
        });
    });
}

// Transposes every 4x4 quad of the accumulators in place.  Afterwards
// element 4q+u of block (i, j) in lane (k, t, g) -- k = (lane & 31) >> 2,
// t = lane & 3, g = lane >> 5 -- is row 32i + 8q + 4g + t, column 32j + 4k + u
// of the wave's sub-tile: each lane holds runs of 4 columns of one row.
template <int NB>
__device__ __forceinline__ void transpose_acc(f32x16 (&acc)[4][NB], int lane)
{
    static_for<4 * NB>([&](auto ij) {
        constexpr int i = decltype(ij)::value / NB, j = decltype(ij)::value % NB;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float a0 = acc[i][j][4 * q], a1 = acc[i][j][4 * q + 1], a2 = acc[i][j][4 * q + 2],
                  a3 = acc[i][j][4 * q + 3];
            transpose4(a0, a1, a2, a3, lane);
            acc[i][j][4 * q] = a0; acc[i][j][4 * q + 1] = a1;
            acc[i][j][4 * q + 2] = a2; acc[i][j][4 * q + 3] = a3;
        }
    });
}
// Row / first column of element 4q+u of block (i, j) in the transposed layout.
__device__ __forceinline__ int tr_row(int wm, int i, int q, int lane)
{
    return 128 * wm + 32 * i + 8 * q + 4 * (lane >> 5) + (lane & 3);
}
template <int NB>
__device__ __forceinline__ int tr_col(int wn, int j, int lane)
{
    return 32 * NB * wn + 32 * j + 4 * ((lane & 31) >> 2);
}

// max over the 4 lanes of a quad
__device__ __forceinline__ float quad_max(float x)
{
    x = fmaxf(x, dpp_mov<0xB1>(x));
    return fmaxf(x, dpp_mov<0x4E>(x));
}

// In the transposed layout: max |.| of each of this lane's 4 columns over the
// 32 rows of block (i, j) (in-lane over q, then the quad, then the two halves).
__device__ __forceinline__ void tr_col_absmax(const f32x16 &blk, float (&m)[4])
{
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        float x = fmaxf(fmaxf(fabsf(blk[u]), fabsf(blk[4 + u])), fmaxf(fabsf(blk[8 + u]), fabsf(blk[12 + u])));
        x = quad_max(x);
        m[u] = fmaxf(x, __shfl_xor(x, 32));
    }
}

// Four consecutive values of one row to global memory (8 bytes for 16-bit
// types, 16 bytes for fp32).  idx is a multiple of 4; rows are 16-byte
// multiples, so the access is naturally aligned.
__device__ __forceinline__ void store4(void *base, int64_t idx, const float (&x)[4], int dtype)
{
    if (dtype == 0) {            // fp32
        *reinterpret_cast<float4 *>(static_cast<float *>(base) + idx) = make_float4(x[0], x[1], x[2], x[3]);
    } else if (dtype == 2) {     // bf16
        const uint32_t lo = f32_to_bf16_rne(x[0]) | ((uint32_t)f32_to_bf16_rne(x[1]) << 16);
        const uint32_t hi = f32_to_bf16_rne(x[2]) | ((uint32_t)f32_to_bf16_rne(x[3]) << 16);
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(base) + idx) = make_uint2(lo, hi);
    } else {                     // fp16
        const uint32_t lo = f32_to_f16_rne(x[0]) | ((uint32_t)f32_to_f16_rne(x[1]) << 16);
        const uint32_t hi = f32_to_f16_rne(x[2]) | ((uint32_t)f32_to_f16_rne(x[3]) << 16);
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(base) + idx) = make_uint2(lo, hi);
    }
}

// Max over the 8 lanes holding the same row of a 32-column block after the
// quad transpose (lanes t, t+4, ..., t+28 of a half-wave).
__device__ __forceinline__ float row8_max(float x)
{
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x101F)));  // ^4
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x201F)));  // ^8
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F)));  // ^16
    return x;
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

// Four E4M3 codes, x0 in the lowest byte.
__device__ __forceinline__ uint32_t pack4_e4m3(float x0, float x1, float x2, float x3)
{
    return pack2_e4m3(x0, x1) | (pack2_e4m3(x2, x3) << 16);
}

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
