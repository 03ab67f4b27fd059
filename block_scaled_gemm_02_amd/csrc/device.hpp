// Device building blocks for the gfx950 block-scaled GEMM kernels.
//
// One workgroup = 4 wave64s computes a 256 x (64*NB) output tile (NB = 4:
// 256 x 256); the waves form a 2 x 2 grid and each owns a 128 x (32*NB)
// quadrant held as 4 x NB fp32 32x32 accumulator blocks (256 values per lane
// for NB = 4, resident in AGPRs for the whole K loop).
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
// A K step is 64 bytes of every row (E4M3: 64 elements, one MFMA per block;
// E2M1: 128 elements and BF16: 32 elements, two MFMAs per block), and a lane
// reads 16-byte chunks g and 2+g of it.
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

// FMT_E4M3_RM: E4M3 codes whose E8M0 scales are row-major, one byte per 32
// K elements of a row ("GEMM + RoPE + MXFP8 Projection (SM100)", x_scale and
// w_scale), instead of the scale-atom layout of the other block-scaled ops.
// FMT_E5M2: E5M2 codes (one byte each) with scale atoms, like FMT_E4M3.
// FMT_BF16_BT: BF16 whose B operand is stored [K][N] ("GEMM + RoPE + MXFP8
// Projection (SM100)", w as (Q_LORA, NUM_HEADS*HEAD_DIM) when w_out_in is
// false): each pair's B tile is staged K-major and its fragments are formed
// with the transposing LDS reads (see the B loads and read_one).
enum Fmt : int { FMT_E4M3 = 0, FMT_E2M1 = 1, FMT_BF16 = 2, FMT_E4M3_RM = 3, FMT_E5M2 = 4, FMT_BF16_BT = 5 };
// Layout flags added to FMT_E4M3 / FMT_E5M2: operand A is stored m-major
// (FMT_TA, memory [L][K][M]) or B n-major (FMT_TB, [L][K][N]) instead of
// k-major ("GEMM + Amax (SM100)", Input/Output tensors: the (1, M, M*K)
// strides).  Such an operand's pair tile is staged K-major in LDS and its
// fragments are formed with the 8-bit transposing LDS reads (see the
// constants kTRow... and read_one).
enum : int { FMT_TA = 8, FMT_TB = 16 };
constexpr int fmt_base(int f) { return f & 7; }
constexpr bool a_t(int f) { return (f & FMT_TA) != 0; }
constexpr bool b_t(int f) { return (f & FMT_TB) != 0; }
// one-byte codes: one 32x32x64 MFMA per block per 64-byte step
constexpr bool is_fp8(int f)
{
    return fmt_base(f) == FMT_E4M3 || fmt_base(f) == FMT_E4M3_RM || fmt_base(f) == FMT_E5M2;
}
constexpr bool is_bf16(int f) { return f == FMT_BF16 || f == FMT_BF16_BT; }
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2;

// K-major FP8 operand tile (FMT_TA / FMT_TB) in a pair slot: the pair's 128
// K rows, each holding the tile's 256 MN columns (one byte each) at a
// stride of 288 bytes (36 KB).  A transposing read has the 16 lanes of a
// group read 8 bytes each from 8 consecutive K rows (two lanes per row);
// the two groups of a half-wave cover 32 columns of those 8 rows, and with
// 288 = 256 + 32 the 8 row segments start 32 bytes apart in the 256-byte
// bank space, so the read is conflict-free.  9 direct-to-LDS loads per wave
// fill the 36 KB; lanes that fall in the 32 padding bytes of a row, or on
// columns past M (N), read zeros.
constexpr int kTRow = 288, kTData = 256, kTBytes = 128 * kTRow, kTLoads = kTBytes / 1024 / 4;

// K-major B tile of FMT_BF16_BT in a pair slot: the pair's 64 K rows, each
// holding the tile's (up to 192) BF16 columns in 384 bytes, at a stride of
// 448 bytes (28 KB).  The padding puts the four K rows that one 16-lane
// group of a transposing read touches on four different 64-byte bank groups
// (448 = 256 + 192), so the reads are conflict-free.
constexpr int kBtRow = 448, kBtData = 384, kBtLoads = 64 * kBtRow / 1024 / 4;   // 7 loads per wave

constexpr int kTileM = 256;
constexpr int kTileN = 256;
constexpr int kThreads = 256;
constexpr uint32_t kOOB = 0x80000000u;          // added to an offset: reads zeros

// ---------------------------------------------------------------------------
// Conversions
// ---------------------------------------------------------------------------
// Two floats -> two bf16 / fp16 values (a in the low half), one packed
// hardware conversion each (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32, round to
// nearest even).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b)
{
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint32_t pack2_f16(float a, float b)
{
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}

// Four codes from two packed conversions: the second writes the high half
// of the first one's result (word_sel), so no masking or shifting is needed.
// The first one's own high half (taken from its "old" operand) is
// overwritten, so x0's bits serve as that operand rather than a zero that
// would cost a register move.
template <bool E5>
__device__ __forceinline__ uint32_t cvt4_fp8(float x0, float x1, float x2, float x3)
{
    if constexpr (E5) {
        const int lo = __builtin_amdgcn_cvt_pk_bf8_f32(x0, x1, __float_as_int(x0), false);
        return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(x2, x3, lo, true);
    } else {
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, __float_as_int(x0), false);
        return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, lo, true);
    }
}

// Four E4M3 (E5 = false) or E5M2 (E5 = true) codes, x0 in the lowest byte,
// round to nearest even.  The conversion gives NaN from the midpoint past the
// largest finite value up instead of saturating, so the inputs are clamped to
// +-448 (E4M3) or +-57344 (E5M2) first.  (The two halves are converted
// separately and merged: the chained form of cvt4_fp8 made the register
// allocator spill in the FP8-D sReLU kernels, whose runtime-typed C store
// uses this cast.)
template <bool E5 = false>
__device__ __forceinline__ uint32_t pack4_fp8(float x0, float x1, float x2, float x3)
{
    constexpr float M = E5 ? 57344.0f : 448.0f;
    x0 = fminf(fmaxf(x0, -M), M);
    x1 = fminf(fmaxf(x1, -M), M);
    x2 = fminf(fmaxf(x2, -M), M);
    x3 = fminf(fmaxf(x3, -M), M);
    uint32_t lo, hi;
    if constexpr (E5) {
        lo = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(x0, x1, 0, false) & 0xFFFFu;
        hi = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(x2, x3, 0, false) & 0xFFFFu;
    } else {
        lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false) & 0xFFFFu;
        hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, 0, false) & 0xFFFFu;
    }
    return lo | (hi << 16);
}
__device__ __forceinline__ uint32_t pack4_e4m3(float x0, float x1, float x2, float x3)
{
    return pack4_fp8<false>(x0, x1, x2, x3);
}

// Four MX-scaled values -> four E4M3 (E5 = false) or E5M2 codes, round to
// nearest even, without the clamp of pack4_fp8.  A value x * (norm_const /
// SF) with SF from mx_scale_byte exceeds the format's largest finite value
// by at most a few ulp (the E8M0 decision is taken in fp32), and the hardware
// conversion rounds everything below the midpoint past it (464 for E4M3,
// 61440 for E5M2) to the largest finite code, as the plain clamp would.
template <bool E5 = false>
__device__ __forceinline__ uint32_t pack4_fp8_mx(float x0, float x1, float x2, float x3)
{
    return cvt4_fp8<E5>(x0, x1, x2, x3);
}

// Four values sharing one E8M0 scale -> four E4M3 codes of x / sf, with the
// scaled conversion (v_cvt_scalef32_pk_fp8_f32 divides by its scale operand
// exactly, a power of two here, and rounds to nearest even); sf is the
// scale as a float, 2^(byte - 127) (subnormal for byte 0, which the
// instruction also takes exactly).  Equal to pack4_fp8_mx(x * inv, ...) for
// inv = 1 / sf, in one instruction per two values.
typedef short s16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack4_e4m3_sf(float x0, float x1, float x2, float x3, float sf)
{
    // (the first conversion's high half is overwritten by the second, as in cvt4_fp8)
    const s16x2_t z = __builtin_bit_cast(s16x2_t, x0);
    const s16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, x0, x1, sf, false);
    const s16x2_t w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, x2, x3, sf, true);
    return __builtin_bit_cast(uint32_t, w);
}
// The same for E5M2 codes (v_cvt_scalef32_pk_bf8_f32).
__device__ __forceinline__ uint32_t pack4_e5m2_sf(float x0, float x1, float x2, float x3, float sf)
{
    const s16x2_t z = __builtin_bit_cast(s16x2_t, x0);
    const s16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(z, x0, x1, sf, false);
    const s16x2_t w = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(lo, x2, x3, sf, true);
    return __builtin_bit_cast(uint32_t, w);
}
template <bool E5>
__device__ __forceinline__ uint32_t pack4_fp8_sf(float x0, float x1, float x2, float x3, float sf)
{
    if constexpr (E5) return pack4_e5m2_sf(x0, x1, x2, x3, sf);
    else return pack4_e4m3_sf(x0, x1, x2, x3, sf);
}
__device__ __forceinline__ float sf_of_byte(uint32_t byte)
{
    return __uint_as_float(byte ? byte << 23 : 0x00400000u);
}

// E8M0 byte of the smallest power of two >= sigma (sigma >= 0), clamped to
// [0, 254]; sigma == 0 (or NaN) gives 0.  Branch-free: it runs once per
// quantisation block inside unrolled epilogues.
__device__ __forceinline__ uint32_t e8m0_ceil(float sigma)
{
    const uint32_t u = __float_as_uint(sigma);
    const uint32_t e = u >> 23, mant = u & 0x7FFFFFu;   // sign bit is 0 when sigma > 0
    // subnormal: 2^-127 (byte 0) or 2^-126 (byte 1); normal: exponent, + 1 if not a power of two.
    // Selected with masks: the compiler turns a select here into a branch.
    const uint32_t sub = (uint32_t)(mant > 0x400000u);
    const uint32_t nrm = e + (uint32_t)(mant != 0u);
    uint32_t b = sub ^ ((sub ^ nrm) & (0u - (uint32_t)(e != 0u)));
    b = min(b, 254u);
    return b & (0u - (uint32_t)(sigma > 0.0f));
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
// Tile order: XCD-aware
// ---------------------------------------------------------------------------
// MI355X has 8 XCDs of 32 CUs, each with its own L2; workgroup b of a launch
// goes to XCD b % 8, and (one 147 KB-LDS workgroup per CU) each XCD runs 32
// tiles at a time.  Launch index b is mapped to a tile sequence number s so
// that every XCD works through runs of 32 consecutive s, and s walks the
// tiles in groups of 4 m-tiles, column by column: an XCD's 32 concurrent
// tiles are then 4 m-tiles x 8 n-tiles and share 4 A panels and 8 B panels
// in its L2 (a row-major order gave each XCD 16 m-tiles x 2 n-tiles, with
// every A panel fetched by all 8 XCDs).  Groups of 4 beat groups of 8 by
// 0.5-1% on the grouped kernels once the outputs stopped filling the L2
// (non-temporal stores); 2 and 16 were slower.  The last partial round
// keeps b.
#ifndef BSG_GROUP_M
#define BSG_GROUP_M 4
#endif
constexpr int kXcds = 8, kCusPerXcd = 32, kGroupM = BSG_GROUP_M;

struct TileCoord {
    int64_t l, mt, nt;
};
__device__ __forceinline__ TileCoord tile_of(int64_t b, int64_t m_t, int64_t n_t, int64_t tiles)
{
    constexpr int64_t R = kXcds * kCusPerXcd;
    int64_t s = b;
    if (b < tiles - tiles % R) {
        const int64_t x = b % kXcds, li = b / kXcds;
        s = (li / kCusPerXcd) * R + x * kCusPerXcd + li % kCusPerXcd;
    }
    TileCoord t;
    const int64_t per_l = m_t * n_t;
    t.l = s / per_l;
    const int64_t sl = s % per_l;
    const int64_t grp = sl / (kGroupM * n_t), r = sl % (kGroupM * n_t);
    const int64_t gm = m_t - grp * kGroupM < kGroupM ? m_t - grp * kGroupM : kGroupM;
    t.mt = grp * kGroupM + r % gm;
    t.nt = r / gm;
    return t;
}

// ---------------------------------------------------------------------------
// K loop: a 4-stage LDS ring filled by direct-to-LDS buffer loads
// ---------------------------------------------------------------------------
// Scale-atom addressing ("Block-scaled GEMM + amax", scale factor layout):
// byte of (row r, k-block kb, batch l) lives at
// (((l*MN' + r/128)*K' + kb/4)*32 + r%32)*16 + ((r%128)/32)*4 + kb%4, so the
// 512-byte atom (l, r/128, kb/4) covers 128 rows x 4 k-blocks, and the 16
// bytes at atom + 16*(r%32) are rows r%32 + 32*w (word w) x 4 k-blocks.
struct OperandDesc {
    const uint8_t *base;   // first row of this tile (row 0 of the 256-row panel)
    uint32_t bytes;        // readable bytes from base (rows past the end read 0)
    uint32_t row_bytes;    // bytes per row (K, K/2 or 2K)
    const uint8_t *sf;     // scale atoms (nullptr for BF16)
    int64_t sf_l, sf_mn_t, sf_k_t;  // batch index, ceil(MN/128), ceil(K/128)
    int64_t sf_mt0;        // atom row-group index of this tile's row 0
    int64_t sf_mt_max;     // last valid atom row-group index
    // FMT_E4M3_RM only: sf is the scale row of this tile's row 0, sf_rm the
    // bytes per scale row (K/32, a multiple of 4), sf_bytes the readable bytes
    uint32_t sf_rm = 0, sf_bytes = 0;
    // MN-major operand (FMT_TA / FMT_TB): base is the tile's first column in
    // K row 0, row_bytes the stride between K rows (M or N), bytes ends at
    // the last K row's last column, and mn_valid columns of the tile exist
    uint32_t mn_valid = 0;
    // FMT_E4M3_RM with FMT_TB (B only): B's scales for the whole K range,
    // staged in LDS by the caller as rows of sf_lds_stride bytes, byte kb of
    // row n at sf_lds + n * sf_lds_stride + kb (the layout of row-major
    // scales); the ring's per-pair B scale loads then read nothing
    const uint8_t *sf_lds = nullptr;
    uint32_t sf_lds_stride = 0;
};
// Row-major E8M0 scales whose B operand has its scales staged in LDS (see
// OperandDesc::sf_lds): the projection's MXFP8 path with w stored [in, out].
template <int F>
constexpr bool b_static_sf() { return F == (FMT_E4M3_RM | FMT_TB); }

// The LDS holds two "pair slots"; a pair slot holds two consecutive K steps
// (128 bytes of every row): the A panel (256 rows x 128 B), the B panel
// (64*NB rows x 128 B) and, for the block-scaled formats, the scale atoms of
// those 128 bytes (A row groups 0 and 1, B row groups 0 and 1; 1 KB each, two
// sets for E2M1 whose atom covers one step).  Every lane of a direct-to-LDS
// load writes 16 bytes at M0 + 16*lane, so one instruction fills 8 rows x
// 128 B: each row is one whole 128-byte line of the operand, fetched with one
// request (64-byte rows per instruction took two requests per line and
// twice the miss-tracking entries of the L1).  Chunk c of row r is stored at
// chunk position c ^ s(r), s(r) = (r%8) ^ ((r/8)%2): load q of a wave covers
// rows with r/8 = q (mod 2) and r%8 = l/8, so lane l fetches logical chunk
// (l%8) ^ (l/8) ^ (q%2).  A 128-bit fragment read has every lane of a 32-row
// block read logical chunk c of its own row; two rows share a 256-byte bank
// line, and over any 16 consecutive rows the pairs (r%2, c ^ s(r)) are all
// distinct, so 16 lanes cover all 64 four-byte banks (and 8 lanes all 32).
// (s(r) = r%8 alone repeats every 8 rows and conflicted 2-way; the LDS bank
// conflict counter measured it at 0.94 conflict cycles per access.)
// Loads past a row's end or past the panel read zeros (buffer range check),
// which covers ragged M, N and K.
//
// Step ks uses pair slot (ks/2) % 2, half ks % 2.  Odd steps wait until this
// wave's loads of the next pair have landed and barrier (every wave's part of
// it is in LDS, and no wave still reads the other slot), then issue the loads
// of the pair after next into that slot; even steps need neither, and only
// prefetch A lines into L2 (see prefetch_a).  Every step interleaves its
// MFMAs on stage ks (held in registers) with the LDS reads of stage ks+1 into
// the idle register set and, on odd steps, the loads -- one MFMA, then its
// share of reads and loads, so that memory instructions issue while the
// matrix core is busy.
constexpr int kKS = 64;                    // bytes per row per step
constexpr int kPK = 2 * kKS;               // bytes per row per pair slot
constexpr int kPA = kTileM * kPK;          // 32 KB
constexpr int kPB = 256 * kPK;             // 32 KB (NB = 4)

// Bytes of a pair slot's A and B regions (the scale atoms follow them).
template <int F>
constexpr int a_region() { return a_t(F) ? kTBytes : kPA; }
template <int F>
constexpr int b_region() { return b_t(F) ? kTBytes : kPB; }

template <int F>
struct Ring {
    static constexpr bool kScaled = !is_bf16(F);
    static constexpr int kScaleSets = fmt_base(F) == FMT_E2M1 ? 2 : (is_fp8(F) ? 1 : 0);
    static constexpr int kSlot = a_region<F>() + b_region<F>() + kScaleSets * 4096;
    static constexpr int kBytes = 2 * kSlot;
    static constexpr int kWaveStage = kSlot / 2 & ~15;   // epilogue staging bytes per wave
};

typedef __attribute__((address_space(3))) void lds_void;

// Buffer resource as four dwords for inline asm (raw buffer: stride 0).
__device__ __forceinline__ i32x4 make_rsrc_words(const void *base, uint32_t bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return i32x4{(int)(uint32_t)a, (int)(uint32_t)(a >> 32) & 0xFFFF, (int)bytes, 0x00020000};
}

// 16 bytes per lane from a buffer straight into LDS at dst + 16*lane.  Issued
// through asm so that the compiler, which cannot tell the slots apart, adds
// no waits of its own: completion is tracked explicitly with vmcnt and
// published to the other waves with a barrier.  One wait state separates the
// M0 write from the load that reads it.
__device__ __forceinline__ void lds_load16(const i32x4 &rsrc, uint8_t *dst, uint32_t voff)
{
    const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void *)dst;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}

// 4 bytes per lane from a buffer into LDS at dst + 4*lane.
__device__ __forceinline__ void lds_load4(const i32x4 &rsrc, uint8_t *dst, uint32_t voff)
{
    const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void *)dst;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
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
    // vmcnt is split over bits 3:0 and 15:14; expcnt/lgkmcnt left at maximum
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void s_wait_lgkm0()
{
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

template <int NB>
struct PipeDesc {
    static constexpr int LB = 2 * NB;  // B loads per wave per pair (16*NB rows / 8)
    i32x4 ra, rb, rs;         // operand panels; this wave's scale atoms (buffer resources)
    uint32_t row_bytes;       // bytes of a k-major row along K (the K extent)
    static constexpr int LV = LB > kTLoads ? LB : kTLoads;   // >= kBtLoads
    uint32_t va[kTLoads], vb[LV];   // per-lane voffset of this wave's code loads (pair 0)
    uint32_t at_pair;         // FMT_TA: bytes of A per pair along K (128 K rows)
    uint32_t bt_pair;         // FMT_BF16_BT / FMT_TB: bytes of B per pair along K (64 / 128 K rows)
    uint32_t lc16;            // 16 * logical chunk of this lane's loads
    uint32_t vs;              // per-lane voffset of this wave's scale atom (kt = 0)
    uint32_t pa;              // per-lane voffset of the A line this lane prefetches (pair 0)
    uint32_t pb;              // same for B (BSG_PF_B)
    uint32_t vsr[2];          // row-major scales: per-lane voffsets of this wave's two scale loads (pair 0)
    int kblocks;              // valid 32-wide K blocks
    int sf_kt;                // K atoms per row group (ceil(K/128))
    const uint8_t *bsf;       // b_static_sf: this lane's row of B scales in LDS (block 0)
    uint32_t bsf_rm;          // b_static_sf: bytes between those rows
};

// The two pair slots are distinct LDS objects, selected by compile-time index.
template <int F>
struct RingSlots {
    uint8_t *s0, *s1;
    uint8_t *sink;            // 256 B per wave where the L2 prefetches land
    template <int S>
    __device__ __forceinline__ uint8_t *at() const
    {
        if constexpr (S == 0) return s0;
        else return s1;
    }
};

// Declares the ring in the calling kernel's shared memory.
#define BSG_DECLARE_RING(F, name)                                                                    \
    __shared__ __attribute__((aligned(16))) uint8_t name##_0[Ring<F>::kSlot];                       \
    __shared__ __attribute__((aligned(16))) uint8_t name##_1[Ring<F>::kSlot];                       \
    __shared__ __attribute__((aligned(16))) uint8_t name##_pf[1024];                                 \
    const ::bsg::RingSlots<F> name{name##_0, name##_1, name##_pf}

// After the K loop each wave stages epilogue output in half a pair slot
// (a quarter in the eight-wave layout).
template <int F>
__device__ __forceinline__ uint8_t *wave_stage(const RingSlots<F> &ring, int w)
{
    return (w < 2 ? ring.s0 : ring.s1) + (w & 1) * Ring<F>::kWaveStage;
}
template <int F>
__device__ __forceinline__ uint8_t *wave_stage8(const RingSlots<F> &ring, int w)
{
    return (w < 4 ? ring.s0 : ring.s1) + (w & 3) * (Ring<F>::kWaveStage / 2 & ~15);
}

// Per-pair / per-step instruction counts of one wave.  An E4M3 scale atom
// covers a whole pair (128 K elements): it is read with the even stage, and
// the odd stage reuses the even stage's scale words.
template <int F>
constexpr bool scales_in_stage(bool odd) { return Ring<F>::kScaled && !(is_fp8(F) && odd); }
template <int F>
constexpr int a_loads() { return a_t(F) ? kTLoads : 8; }
template <int F, int NB>
constexpr int b_loads() { return b_t(F) ? kTLoads : (F == FMT_BF16_BT ? kBtLoads : 2 * NB); }
template <int F, int NB>
constexpr int loads_per_pair()
{
    return a_loads<F>() + b_loads<F, NB>() + (fmt_base(F) == FMT_E4M3_RM ? 2 : Ring<F>::kScaleSets);
}
// MI: 32-row blocks per wave (4, or 2 in the eight-wave layout below).
template <int F, int NB, int MI = 4>
constexpr int mfmas_per_step() { return (is_fp8(F) ? 1 : 2) * MI * NB; }
// Reads of a stage: one 16-byte read per chunk, or (K-major staging) two
// 8-byte transposing reads per chunk
template <int F, int MI = 4>
constexpr int a_reads() { return a_t(F) ? 16 : 2 * MI; }
template <int F, int NB>
constexpr int b_reads() { return (b_t(F) || F == FMT_BF16_BT) ? 4 * NB : 2 * NB; }
// scale reads of a stage that has them: one word set per operand, or (B
// scales staged in LDS) one A read and one word per B block
template <int F, int NB>
constexpr int scale_reads() { return b_static_sf<F>() ? 1 + NB : 2; }
template <int F, int NB, int MI = 4>
constexpr int reads_in_stage(bool odd)
{
    return a_reads<F, MI>() + b_reads<F, NB>() + (scales_in_stage<F>(odd) ? scale_reads<F, NB>() : 0);
}

// Where this wave's loads of pair p go: code offset (K position, or out of
// range past the row end) and scale-atom offset of each atom set.
struct PairAddr {
    uint32_t kb_oob[2];       // added to va/vb of loads with even / odd index
    uint32_t so[2];           // scale-atom voffsets
    uint32_t kat, kbt;        // K-major staging: added to va / vb (K rows past K read zeros: range check)
};
template <int F, int NB>
__device__ __forceinline__ PairAddr pair_addr(const PipeDesc<NB> &d, int pair)
{
    PairAddr a;
    const uint32_t kb = (uint32_t)pair * kPK;
    a.kb_oob[0] = kb + ((kb + d.lc16 < d.row_bytes) ? 0u : kOOB);
    a.kb_oob[1] = kb + ((kb + (d.lc16 ^ 16u) < d.row_bytes) ? 0u : kOOB);
    a.kat = (uint32_t)pair * d.at_pair;
    a.kbt = (uint32_t)pair * d.bt_pair;
    if constexpr (fmt_base(F) == FMT_E4M3_RM) {
        // row-major scales: the pair's 4 bytes of a row follow its previous pair's
#pragma unroll
        for (int h = 0; h < 2; ++h) a.so[h] = pair < d.sf_kt ? d.vsr[h] + 4u * (uint32_t)pair : kOOB;
    } else {
        // an atom covers 128 K elements: one pair (E4M3) or one step (E2M1)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int kt = fmt_base(F) == FMT_E2M1 ? 2 * pair + h : pair;
            a.so[h] = kt < d.sf_kt ? d.vs + (uint32_t)kt * 512u : kOOB;
        }
    }
    return a;
}

// Load number L of this wave's share of a pair: A (8 loads of 8 rows, or 9
// KB of the K-major tile), B, then the scale atom(s).  Each load fills the
// 1 KB of the region that follows the wave's previous one.
template <int F, int NB, int L>
__device__ __forceinline__ void load_one(const PipeDesc<NB> &d, uint8_t *st, const PairAddr &a, int w)
{
    constexpr int LA = a_loads<F>(), LB = b_loads<F, NB>();
    constexpr int SC = a_region<F>() + b_region<F>();
    if constexpr (L < LA) {
        lds_load16(d.ra, st + 1024 * (LA * w + L), d.va[L] + (a_t(F) ? a.kat : a.kb_oob[L & 1]));
    } else if constexpr (L < LA + LB) {
        // K-major B (FMT_BF16_BT, FMT_TB): K rows past K and padding lanes read zeros
        constexpr int q = L - LA;
        constexpr bool kmaj = b_t(F) || F == FMT_BF16_BT;
        lds_load16(d.rb, st + a_region<F>() + 1024 * (LB * w + q), d.vb[q] + (kmaj ? a.kbt : a.kb_oob[q & 1]));
    } else if constexpr (fmt_base(F) == FMT_E4M3_RM) {
        constexpr int h = L - LA - LB;     // rows 0-15 (h = 0) or 16-31 (h = 1) of each 32-row block
        lds_load4(d.rs, st + SC + 1024 * w + 256 * h, a.so[h]);
    } else {
        constexpr int h = L - LA - LB;
        lds_load16(d.rs, st + SC + 4096 * h + 1024 * w, a.so[h]);
    }
}

template <int F, int NB>
__device__ __forceinline__ void issue_pair(const PipeDesc<NB> &d, uint8_t *st, int pair, int w)
{
    const PairAddr a = pair_addr<F, NB>(d, pair);
    static_for<loads_per_pair<F, NB>()>([&](auto l) { load_one<F, NB, decltype(l)::value>(d, st, a, w); });
}

// L2 prefetch of the A panel: each lane touches the 128-byte line of pair
// `pair` in one of this wave's 64 A rows, so that the pair's loads, issued one
// step later, find it in L2.  (An A panel is shared by fewer concurrent tiles
// than a B panel, so more of its lines miss; prefetching B as well cost more
// than it saved.)  The 4 bytes per lane land in the wave's sink; nothing
// reads them.
template <int F, int NB>
__device__ __forceinline__ void prefetch_a(const PipeDesc<NB> &d, const RingSlots<F> &ring, int pair, int w)
{
    if constexpr (a_t(F)) {
        // m-major A: the pair's 256 lines are 2 per K row (past K: range check)
        lds_load4(d.ra, ring.sink + 256 * w, d.pa + (uint32_t)pair * d.at_pair);
    } else {
        const uint32_t kb = (uint32_t)pair * kPK;
        lds_load4(d.ra, ring.sink + 256 * w, kb < d.row_bytes ? d.pa + kb : kOOB);
    }
#if BSG_PF_B
    if constexpr (!b_t(F) && F != FMT_BF16_BT) {
        const uint32_t kb = (uint32_t)pair * kPK;
        lds_load4(d.rb, ring.sink + 256 * w, kb < d.row_bytes ? d.pb + kb : kOOB);
    }
#endif
}
#ifndef BSG_PF_DIST
#define BSG_PF_DIST 2
#endif
#ifndef BSG_PF_B
#define BSG_PF_B 0
#endif
// Outstanding prefetch loads an odd step's wait leaves in flight.
template <int F>
constexpr int pf_loads() { return 1 + ((BSG_PF_B && !b_t(F) && F != FMT_BF16_BT) ? 1 : 0); }

// LDS read number R of a step's fragments: A chunks (R < 8), B chunks, then
// the two scale words.  In half H of a pair slot the lane reads logical
// chunks 4H+g and 4H+2+g of its row, stored at chunk ^ s(row).
struct ReadAddr {
    const uint8_t *a0, *b0;   // this lane's A / B row in block 0
    uint32_t p0, p1;          // byte offsets of its two chunks
    const uint8_t *sa, *sb;   // this lane's scale words
    uint32_t sb_blk;          // b_static_sf: bytes between the B scale words of blocks j and j + 1
};
// pair: K pair of the stage read (used by b_static_sf only); hh: the wave's
// half of its 128-row group in the eight-wave layout (MI = 2)
template <int F, int NB, int H, int MI = 4>
__device__ __forceinline__ ReadAddr read_addr(const uint8_t *st, int wm, int wn, int lane, const PipeDesc<NB> &d,
                                              int pair, int hh = 0)
{
    ReadAddr r;
    const uint32_t row = lane & 31, g = lane >> 5;
    const uint32_t swz = (row & 7) ^ ((row >> 3) & 1);
    r.p0 = 16u * ((4u * H + g) ^ swz);
    r.p1 = 16u * ((4u * H + 2u + g) ^ swz);
    // K-major FP8 tile (16-lane group G = lane / 16, lane s = lane % 16 in
    // it; the group holds MFMA rows 16(G%2) .. + 15 with K half g = G/2):
    // lane s reads 8 columns, 8(s%2) onwards, of K row 16(G/2) + s/2 of the
    // step (+ 32 for chunk 1, + 8 for a chunk's second read); lane j of the
    // group then holds 8 consecutive K values of column 16(G%2) + j
    const uint32_t G = (uint32_t)lane >> 4, s = (uint32_t)lane & 15;
    const uint32_t trow = (64u * H + 16u * (G >> 1) + (s >> 1)) * kTRow + 16u * (G & 1) + 8u * (s & 1);
    if constexpr (a_t(F)) r.a0 = st + trow + 128u * wm;
    else if constexpr (MI == 2) r.a0 = st + (128u * wm + 64u * hh + row) * kPK;
    else r.a0 = st + (128u * wm + row) * kPK;
    if constexpr (b_t(F)) {
        r.b0 = st + a_region<F>() + trow + 32u * NB * wn;
    } else if constexpr (F == FMT_BF16_BT) {
        // transposing reads (16-lane group G = lane / 16, lane s = lane % 16
        // in it): lane s reads 4 columns of K row 8(G/2) + s/4 (+ 4 for the
        // second read of a chunk, + 16 for chunk 1, + 32 in the pair's second
        // step), columns 16(G%2) + 4(s%4) of the block; lane j of the group
        // then holds 4 consecutive K values of column 16(G%2) + j
        r.b0 = st + a_region<F>() + (32u * H + 8u * (G >> 1) + (s >> 2)) * kBtRow +
               2u * (32u * NB * wn + 16u * (G & 1) + 4u * (s & 3));
    } else {
        r.b0 = st + a_region<F>() + (32u * NB * wn + row) * kPK;
    }
    const uint8_t *sc = st + a_region<F>() + b_region<F>() + (fmt_base(F) == FMT_E2M1 ? 4096 * H : 0);
    r.sa = sc + 1024 * wm + 16 * row + (MI == 2 ? 8 * hh : 0);   // word q: the lane's row of block q
    r.sb = sc + 1024 * (2 + wn) + 16 * row;
    r.sb_blk = 0;
    if constexpr (b_static_sf<F>()) {
        r.sb = d.bsf + 4u * (uint32_t)pair;
        r.sb_blk = 32u * d.bsf_rm;
    } else {
        (void)d;
        (void)pair;
    }
    return r;
}
// One 8-byte transposing read of a K-major FP8 tile into half e of chunk
// register c: K values [8e, 8e + 8) of the chunk's 16.
template <int E>
__device__ __forceinline__ void read_tr8(i32x4 &c, const uint8_t *p)
{
    const i32x2_t u = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(lds_void *)p);
    if constexpr (E == 0) {
        c.x = u.x;
        c.y = u.y;
    } else {
        c.z = u.x;
        c.w = u.y;
    }
}

template <int F, int NB, int R, int MI = 4>
__device__ __forceinline__ void read_one(Frags<NB> &f, const ReadAddr &r)
{
    constexpr int RA = a_reads<F, MI>();
    if constexpr (a_t(F) && R < RA) {
        // chunk h of block i: K [16g + 32h, +16) of the lane's column as two
        // reads of 8 K values each (e = 0, 1)
        constexpr int i = R / 4, h = (R / 2) % 2, e = R % 2;
        read_tr8<e>(f.a[i][h], r.a0 + (32 * h + 8 * e) * kTRow + 32 * i);
    } else if constexpr (R < RA) {
        constexpr int i = R / 2, h = R % 2;
        f.a[i][h] = *reinterpret_cast<const i32x4 *>(r.a0 + 32 * kPK * i + (h ? r.p1 : r.p0));
    } else if constexpr (b_t(F) && R < RA + 4 * NB) {
        constexpr int q = R - RA, j = q / 4, h = (q / 2) % 2, e = q % 2;
        read_tr8<e>(f.b[j][h], r.b0 + (32 * h + 8 * e) * kTRow + 32 * j);
    } else if constexpr (F == FMT_BF16_BT && R < RA + 4 * NB) {
        // chunk h of block j: K [8g + 16h, +8) of the lane's column as two
        // reads of 4 K values each (e = 0, 1)
        constexpr int q = R - RA, j = q / 4, h = (q / 2) % 2, e = q % 2;
        const uint8_t *p = r.b0 + (16 * h + 4 * e) * kBtRow + 64 * j;
        const auto v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(lds_void *)p);
        const i32x2_t u = __builtin_bit_cast(i32x2_t, v);
        if constexpr (e == 0) {
            f.b[j][h].x = u.x;
            f.b[j][h].y = u.y;
        } else {
            f.b[j][h].z = u.x;
            f.b[j][h].w = u.y;
        }
    } else if constexpr (R < RA + 2 * NB) {
        constexpr int j = (R - RA) / 2, h = (R - RA) % 2;
        f.b[j][h] = *reinterpret_cast<const i32x4 *>(r.b0 + 32 * kPK * j + (h ? r.p1 : r.p0));
    } else if constexpr (R == RA + b_reads<F, NB>() && MI == 2) {
        const i32x2_t v = *reinterpret_cast<const i32x2_t *>(r.sa);     // the wave's two row blocks
        f.sa = i32x4{v.x, v.y, 0, 0};
    } else if constexpr (R == RA + b_reads<F, NB>()) {
        f.sa = *reinterpret_cast<const i32x4 *>(r.sa);
    } else if constexpr (b_static_sf<F>()) {
        constexpr int j = R - RA - b_reads<F, NB>() - 1;
        f.sb[j] = *reinterpret_cast<const int *>(r.sb + j * r.sb_blk);
    } else {
        f.sb = *reinterpret_cast<const i32x4 *>(r.sb);
    }
}

template <int F, int NB, int MI = 4>
__device__ __forceinline__ void read_frags0(Frags<NB> &f, const uint8_t *st, int wm, int wn, int lane,
                                            const PipeDesc<NB> &d, int hh = 0)
{
    const ReadAddr r = read_addr<F, NB, 0, MI>(st, wm, wn, lane, d, 0, hh);
    static_for<reads_in_stage<F, NB, MI>(false)>([&](auto q) { read_one<F, NB, decltype(q)::value, MI>(f, r); });
}

// Byte of the scale word that an MFMA lane consumes is moved to byte 0
// (E4M3: k-block 2*(ks%2) + g of the atom) or byte 2s (E2M1: k-block 2s+g).
template <int F, int PAR>
__device__ __forceinline__ i32x4 prep_scales(i32x4 w, int kt, int kblocks, int g)
{
    w = sanitize_scales(w, kt, kblocks);
    const uint32_t sh = is_fp8(F) ? 8u * (g + 2 * PAR) : 8u * g;
    w.x = (int)((uint32_t)w.x >> sh);
    w.y = (int)((uint32_t)w.y >> sh);
    w.z = (int)((uint32_t)w.z >> sh);
    w.w = (int)((uint32_t)w.w >> sh);
    return w;
}

// MFMA number M of a step: block (i, j) = ((M % MI*NB) / NB, M % NB), sub-step
// S = M / (MI*NB) (E2M1, BF16).  The B fragment is the instruction's first
// operand and the A fragment its second, so the instruction computes the
// transposed block (B A^T): lane (c, g) register v of block (i, j) then holds
// C[32i + c][32j + 8(v/4) + 4g + v%4] -- one output row per lane with runs of
// four consecutive columns, the layout the epilogue stores.
template <int F, int NB, int M, int MI = 4>
__device__ __forceinline__ void mma_one(f32x16 (&acc)[MI][NB], const Frags<NB> &f, const i32x4 &sa,
                                        const i32x4 &sb)
{
    constexpr int S = M / (MI * NB), i = (M % (MI * NB)) / NB, j = M % NB;
    if constexpr (is_fp8(F)) {
        const i32x8 av{f.a[i][0].x, f.a[i][0].y, f.a[i][0].z, f.a[i][0].w,
                       f.a[i][1].x, f.a[i][1].y, f.a[i][1].z, f.a[i][1].w};
        const i32x8 bv{f.b[j][0].x, f.b[j][0].y, f.b[j][0].z, f.b[j][0].w,
                       f.b[j][1].x, f.b[j][1].y, f.b[j][1].z, f.b[j][1].w};
        // operand format: 0 = E4M3, 1 = E5M2 (for both operands)
        constexpr int fm = fmt_base(F) == FMT_E5M2 ? 1 : 0;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bv, av, acc[i][j], fm, fm, 0, sb[j], 0,
                                                                      sa[i]);
    } else if constexpr (fmt_base(F) == FMT_E2M1) {
        const i32x8 av{f.a[i][S].x, f.a[i][S].y, f.a[i][S].z, f.a[i][S].w, 0, 0, 0, 0};
        const i32x8 bv{f.b[j][S].x, f.b[j][S].y, f.b[j][S].z, f.b[j][S].w, 0, 0, 0, 0};
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bv, av, acc[i][j], 4, 4, 2 * S, sb[j],
                                                                      2 * S, sa[i]);
    } else {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f.b[j][S]),
                                                            __builtin_bit_cast(bf16x8, f.a[i][S]),
                                                            acc[i][j], 0, 0, 0);
    }
}

// Where in a step's MFMA sequence the fragment reads and the pair loads go.
#ifndef BSG_READ_SPAN_NUM
#define BSG_READ_SPAN_NUM 3     // reads over the first 3/4 of the MFMAs
#endif
template <int F, int NB, int MI = 4>
constexpr int read_span() { return mfmas_per_step<F, NB, MI>() * BSG_READ_SPAN_NUM / 4; }

// One K step, ks = 4q + U: see the comment above the pair-slot constants.
// LOADER: the wave issues its share of the loads (always, except waves 4-7
// of the eight-wave layout).
template <int F, int NB, int U, int MI = 4, bool LOADER = true>
__device__ __forceinline__ void pipe_step(f32x16 (&acc)[MI][NB], Frags<NB> &cur, Frags<NB> &nxt,
                                          const PipeDesc<NB> &d, const RingSlots<F> &ring, int ks, int w,
                                          int wm, int wn, int lane, int hh = 0)
{
    constexpr bool ODD = (U & 1) != 0;           // stage ks parity; stage ks+1 has the other
    constexpr int RS = ((U + 1) / 2) % 2;        // pair slot of stage ks+1 ...
    constexpr int RH = (U + 1) % 2;              // ... and its half
    constexpr int LSL = ((U + 3) / 2) % 2;       // slot the odd step refills
    constexpr int M = mfmas_per_step<F, NB, MI>(), R = reads_in_stage<F, NB, MI>(!ODD);
    constexpr int V = ODD && LOADER ? loads_per_pair<F, NB>() : 0;
    if constexpr (ODD) {
        // this wave's part of the pair holding stage ks+1 has landed (the
        // prefetch issued after it may still be in flight)
        s_wait_vm<pf_loads<F>()>();
        s_wait_lgkm0();             // our reads of stage ks are complete
        __builtin_amdgcn_s_barrier();
    } else {
        s_wait_lgkm0();             // our reads of stage ks are complete
    }
    __builtin_amdgcn_sched_barrier(0);
    const int g = lane >> 5;
    i32x4 sa{}, sb{};
    if constexpr (Ring<F>::kScaled) {
        const int kt = is_fp8(F) ? ks >> 1 : ks;
        sa = prep_scales<F, U & 1>(cur.sa, kt, d.kblocks, g);
        sb = prep_scales<F, U & 1>(cur.sb, kt, d.kblocks, g);
    }
    PairAddr la{};
    if constexpr (ODD) la = pair_addr<F, NB>(d, (ks + 3) >> 1);
    uint8_t *const lslot = ring.template at<LSL>();
    const ReadAddr ra = read_addr<F, NB, RH, MI>(ring.template at<RS>(), wm, wn, lane, d, (ks + 1) >> 1, hh);
    if constexpr (Ring<F>::kScaled && !scales_in_stage<F>(!ODD)) {
        nxt.sa = cur.sa;
        nxt.sb = cur.sb;
    }
    __builtin_amdgcn_sched_barrier(0);
    // Reads go out over the first MR MFMAs, so that the last of them has
    // landed by the next step's wait; loads over all MFMAs.
    constexpr int MR = read_span<F, NB, MI>();
    static_for<M>([&](auto mm) {
        constexpr int m = decltype(mm)::value;
        mma_one<F, NB, m, MI>(acc, cur, sa, sb);
        if constexpr (m < MR) {
            static_for<(R * (m + 1)) / MR - (R * m) / MR>([&](auto rr) {
                read_one<F, NB, (R * m) / MR + decltype(rr)::value, MI>(nxt, ra);
            });
        }
        if constexpr (V > 0) {
            static_for<(V * (m + 1)) / M - (V * m) / M>([&](auto ll) {
                load_one<F, NB, (V * m) / M + decltype(ll)::value>(d, lslot, la, w);
            });
        }
        // even step: prefetch the A lines of the pair after the one the next
        // (odd) step loads
        if constexpr (!ODD && m == 0 && LOADER) prefetch_a<F, NB>(d, ring, (ks + 2 * BSG_PF_DIST) >> 1, w);
        __builtin_amdgcn_sched_barrier(0);
    });
}

// K loop over a 256 x (64*NB) tile, 4 waves as 2 x 2 (wave: 128 x 32*NB).
//
// MI = 2 is the eight-wave layout (two waves per SIMD, 64 x 32*NB each) for
// kernels whose epilogue is long against their K loop: waves w and w + 4
// split the 128-row group of wave w's quadrant between them, and wave w + 4
// takes the other wave column, so that the two waves on one SIMD (w and
// w + 4) hold one quadrant half of each column.  Waves 0-3 issue every load
// exactly as in the four-wave layout (same LDS layout and counts); waves 4-7
// only read fragments and pass the same barriers.  Wave (wm, wn, hh) holds
// rows 128 wm + 64 hh .. + 63 and columns 32 NB wn .. of the tile.
template <int F, int NB = 4, int MI = 4>
__device__ __forceinline__ void mainloop_pipe(f32x16 (&acc)[MI][NB], const RingSlots<F> &ring,
                                              const OperandDesc &A, const OperandDesc &B, int64_t k)
{
    static_assert(MI == 4 || (MI == 2 && !a_t(F) && (is_bf16(F) || fmt_base(F) == FMT_E4M3_RM)),
                  "the eight-wave layout: k-major A, BF16 or row-major-scaled E4M3");
    static_assert(NB == 4 || is_bf16(F) || fmt_base(F) == FMT_E4M3_RM, "atom scales need 128-column wave tiles");
    static_assert(F != FMT_BF16_BT || 64 * NB <= kBtData / 2, "a K-major B row holds the tile's columns");
    static_assert(!(a_t(F) || b_t(F)) || (is_fp8(F) && (NB == 4 || b_static_sf<F>())),
                  "MN-major operands: FP8, 256 x 256 tiles (or the projection's [in, out] weights)");
    static_assert(!a_t(F) || fmt_base(F) != FMT_E4M3_RM, "row-major scales with an m-major A are not built");
    // the wave index is uniform: keep everything derived from it in SGPRs
    const int t = threadIdx.x, lane = t & 63;
    const int wall = __builtin_amdgcn_readfirstlane(t >> 6);
    const int w = MI == 2 ? (wall & 3) : wall;          // load role (waves 0-3)
    const int hh = MI == 2 ? (wall >> 2) : 0;
    const int wm = w >> 1, wn = MI == 2 ? ((w & 1) ^ hh) : (w & 1);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    PipeDesc<NB> d;
    d.ra = make_rsrc_words(A.base, A.bytes);
    d.rb = make_rsrc_words(B.base, B.bytes);
    // K extent of a row in bytes
    d.row_bytes = (uint32_t)(is_fp8(F) ? k : (fmt_base(F) == FMT_E2M1 ? k / 2 : 2 * k));
    const uint32_t lrow = (uint32_t)lane >> 3;                       // row within an 8-row load
    const uint32_t lchunk = ((uint32_t)lane & 7) ^ lrow;
    d.lc16 = 16u * lchunk;
    // MN-major operand: load q of wave w fills bytes 1024 (9w + q) .. of the
    // pair's K-major tile, 16 per lane, so a lane's byte o sits in K row
    // o / 288 at column o % 288 (zeros for the padding past 256 and for
    // columns past the operand's M or N)
    auto kmajor_off = [&](int q, const OperandDesc &X) {
        const uint32_t o = 1024u * (kTLoads * w + q) + 16u * (uint32_t)lane;
        const uint32_t kr = o / kTRow, cb = o % kTRow;
        return (cb < (uint32_t)kTData && cb < X.mn_valid) ? kr * X.row_bytes + cb : kOOB;
    };
#pragma unroll
    for (int q = 0; q < a_loads<F>(); ++q) {
        if constexpr (a_t(F)) d.va[q] = kmajor_off(q, A);
        else d.va[q] = (64u * w + 8u * q + lrow) * A.row_bytes + (d.lc16 ^ (16u * (q & 1)));
    }
#pragma unroll
    for (int q = 0; q < b_loads<F, NB>(); ++q) {
        if constexpr (b_t(F)) d.vb[q] = kmajor_off(q, B);
        else if constexpr (F != FMT_BF16_BT)
            d.vb[q] = (16u * NB * w + 8u * q + lrow) * B.row_bytes + (d.lc16 ^ (16u * (q & 1)));
    }
    d.at_pair = a_t(F) ? 128u * A.row_bytes : 0u;
    d.bt_pair = b_t(F) ? 128u * B.row_bytes : 0u;
    if constexpr (F == FMT_BF16_BT) {
        // B is [K][N] with B.row_bytes between K rows: load q of wave w fills
        // bytes 1024 (7w + q) .. of the pair's K-row block, 16 per lane, so a
        // lane's byte o sits in K row o / 448 at column byte o % 448 (zeros
        // for the padding past 384)
#pragma unroll
        for (int q = 0; q < kBtLoads; ++q) {
            const uint32_t o = 1024u * (kBtLoads * w + q) + 16u * (uint32_t)lane;
            const uint32_t kr = o / kBtRow, cb = o % kBtRow;
            d.vb[q] = cb < (uint32_t)kBtData ? kr * B.row_bytes + cb : kOOB;
        }
        d.bt_pair = 64u * B.row_bytes;
    }
    if constexpr (a_t(F)) {
        // lane (w, l) touches line (64w + l) % 2 of K row (64w + l) / 2
        const uint32_t tl = 64u * w + (uint32_t)lane, cb = 128u * (tl & 1);
        d.pa = cb < A.mn_valid ? (tl >> 1) * A.row_bytes + cb : kOOB;
    } else {
        d.pa = (64u * w + (uint32_t)lane) * A.row_bytes;
    }
    d.pb = (64u * w + (uint32_t)lane) * B.row_bytes;
    d.kblocks = (int)(k / 32);
    d.sf_kt = 0;
    d.rs = d.ra;
    d.vs = kOOB;
    d.vsr[0] = d.vsr[1] = kOOB;
    d.bsf = nullptr;
    d.bsf_rm = 0;
    if constexpr (fmt_base(F) == FMT_E4M3_RM) {
        // Row-major scales, staged in the layout the fragment reads expect:
        // wave w fills 512 bytes at 1 KB * w, where the 16 bytes at 16*r32 are
        // the pair's 4 scale bytes of the rows 32q + r32 (q = 0..3) of A row
        // group w (w < 2), or of the NB 32-row blocks of B wave column w - 2.
        // Each load moves 4 bytes per lane: lane l covers r32 = 16h + l/4 and
        // q = l%4 (load h = 0, 1); rows that do not exist read zeros.
        const OperandDesc &S = w < 2 ? A : B;
        d.rs = make_rsrc_words(S.sf, S.sf_bytes);
        const uint32_t q = (uint32_t)lane & 3;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t r32 = 16u * h + ((uint32_t)lane >> 2);
            const uint32_t row = (w < 2 ? 128u * (w & 1) : 32u * NB * (w & 1)) + 32u * q + r32;
            d.vsr[h] = (w < 2 || q < (uint32_t)NB) ? row * S.sf_rm : kOOB;
        }
        d.sf_kt = (int)((k + 127) / 128);
        if constexpr (b_static_sf<F>()) {
            // B's words come from the LDS copy; the ring's B scale loads read nothing
            if (w >= 2) d.vsr[0] = d.vsr[1] = kOOB;
            d.bsf = B.sf_lds + (32u * NB * wn + ((uint32_t)lane & 31u)) * B.sf_lds_stride;
            d.bsf_rm = B.sf_lds_stride;
        }
    } else if constexpr (Ring<F>::kScaled) {
        // wave w loads the K atom of atom row group w&1 of A (w < 2) or B (w >= 2)
        const OperandDesc &S = w < 2 ? A : B;
        const int64_t mt = S.sf_mt0 + (w & 1);
        const bool mt_ok = mt <= S.sf_mt_max;
        const uint8_t *base = S.sf + ((S.sf_l * S.sf_mn_t) * S.sf_k_t) * 512;
        d.rs = make_rsrc_words(base, (uint32_t)(S.sf_mn_t * S.sf_k_t * 512));
        d.vs = (lane < 32 && mt_ok) ? (uint32_t)(mt * S.sf_k_t * 512) + 16u * lane : kOOB;
        d.sf_kt = (int)S.sf_k_t;
    }

    const int nks = (int)((d.row_bytes + kKS - 1) / kKS);
    Frags<NB> fx, fy;
    if (MI == 4 || hh == 0) {
        issue_pair<F, NB>(d, ring.template at<0>(), 0, w);
        issue_pair<F, NB>(d, ring.template at<1>(), 1, w);
    }
    // pair 0 has landed, and with it any direct-to-LDS load the caller issued
    // before this call (loads complete in issue order); pair 1 may be in flight
    s_wait_vm<loads_per_pair<F, NB>()>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_frags0<F, NB, MI>(fx, ring.template at<0>(), wm, wn, lane, d, hh);
    auto kloop = [&](auto loader) {
        constexpr bool L = decltype(loader)::value;
        for (int ks = 0; ks < nks; ks += 4) {
            pipe_step<F, NB, 0, MI, L>(acc, fx, fy, d, ring, ks, w, wm, wn, lane, hh);
            if (ks + 1 < nks) pipe_step<F, NB, 1, MI, L>(acc, fy, fx, d, ring, ks + 1, w, wm, wn, lane, hh);
            if (ks + 2 < nks) pipe_step<F, NB, 2, MI, L>(acc, fx, fy, d, ring, ks + 2, w, wm, wn, lane, hh);
            if (ks + 3 < nks) pipe_step<F, NB, 3, MI, L>(acc, fy, fx, d, ring, ks + 3, w, wm, wn, lane, hh);
        }
    };
    if constexpr (MI == 4) {
        kloop(std::true_type{});
    } else {
        if (hh == 0) kloop(std::true_type{});
        else kloop(std::false_type{});
    }
    s_wait_vm<0>();
    s_wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

// ===========================================================================
// Epilogue helpers
// ===========================================================================
// Tile-relative row and first column of register group q (registers
// 4q..4q+3) of accumulator block (i, j) in this lane (see mma_one).
__device__ __forceinline__ int acc_row(int wm, int i, int lane) { return 128 * wm + 32 * i + (lane & 31); }
// The same in the eight-wave layout (mainloop_pipe with MI = 2).
__device__ __forceinline__ int acc_row8(int wm, int hh, int i, int lane)
{
    return 128 * wm + 64 * hh + 32 * i + (lane & 31);
}
template <int NB>
__device__ __forceinline__ int acc_col(int wn, int j, int q, int lane)
{
    return 32 * NB * wn + 32 * j + 8 * q + 4 * (lane >> 5);
}

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_E4M3 = 3, DT_E5M2 = 4, DT_E2M1 = 5 };

// ---------------------------------------------------------------------------
// Output staging through LDS
// ---------------------------------------------------------------------------
// After the K loop the ring is free.  Each wave stages one 32-row block of
// its 128 x (32*NB) quadrant at a time in its own ring slot, in the
// accumulator layout, then reads it back row-major, 16 bytes per lane, and
// stores whole row segments: every 128-byte line of the output is written by
// one instruction.  Storing straight from the accumulator layout writes 8- or
// 16-byte pieces of 32 rows per instruction, and those partial lines raised
// the HBM write traffic by half again.  ES is the output element size (1, 2
// or 4 bytes); staged rows are 16 bytes longer than the data so that the 32
// rows one write instruction touches start on different banks.
template <int ES, int NB>
struct StageGeom {
    static constexpr int RB = 32 * NB * ES;          // data bytes per row
    static constexpr int RBP = RB + 16;              // staged row stride
    static constexpr int LPR = RB / 16;              // lanes per row when reading back
    static constexpr int RPI = 64 / LPR;             // rows per read instruction
    static constexpr int NK = (32 + RPI - 1) / RPI;  // read instructions per 32 rows
    static_assert(RB % 16 == 0 && LPR <= 64, "rows are whole 16-byte chunks");
};

// Four consecutive output elements (columns 4k..4k+3 of a row) as stored.
template <int ES> struct Quad;
template <> struct Quad<1> { typedef uint32_t T; };
template <> struct Quad<2> { typedef uint2 T; };
template <> struct Quad<4> { typedef float4 T; };

// Stored bytes per element of output type DT.
template <int DT> constexpr int es_of() { return DT == DT_F32 ? 4 : ((DT == DT_E4M3 || DT == DT_E5M2) ? 1 : 2); }

// Packs four output values for output type DT.  The FP8 types are plain
// saturating casts (round to nearest even, clamped to the largest finite
// value of the format).
template <int DT>
__device__ __forceinline__ typename Quad<es_of<DT>()>::T pack_quad(float x0, float x1, float x2, float x3)
{
    if constexpr (DT == DT_F32) return make_float4(x0, x1, x2, x3);
    else if constexpr (DT == DT_BF16) return make_uint2(pack2_bf16(x0, x1), pack2_bf16(x2, x3));
    else if constexpr (DT == DT_E4M3) return pack4_fp8<false>(x0, x1, x2, x3);
    else if constexpr (DT == DT_E5M2) return pack4_fp8<true>(x0, x1, x2, x3);
    else return make_uint2(pack2_f16(x0, x1), pack2_f16(x2, x3));
}

// Stores the staged 32 rows: row r goes to dst + r*row_bytes, through a
// buffer resource over the valid rows (at most 32), so rows past M -- and the
// rows past 32 that a last partial read instruction covers -- fall outside its
// range and are dropped; lanes whose 16-byte chunk starts at or past
// col_bytes, or that hold no row, are pointed out of range as well.  The
// output rows are multiples of 16 bytes, so a chunk is all in or all out.
template <int ES, int NB>
__device__ __forceinline__ void stage_flush(const uint8_t *reg, char *dst, uint32_t row_bytes, int rows,
                                            int col_bytes, int lane)
{
    typedef StageGeom<ES, NB> G;
    if (rows <= 0) return;
    const int lr = lane / G::LPR, cb = (lane % G::LPR) * 16;
    const uint8_t *src = reg + lr * G::RBP + cb;
    // the destination and extent are wave-uniform: say so, so that the
    // resource is built once in SGPRs instead of in a loop over lane values
    const uint64_t base = (uint64_t)(uintptr_t)dst;
    char *const udst = (char *)(uintptr_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(base >> 32)) << 32) |
                                           (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base));
    const uint32_t nrec = (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(rows < 32 ? rows : 32) * row_bytes));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(udst, (short)0, (int)nrec, 0x00020000);
    const uint32_t voff = (cb < col_bytes && lr < G::RPI) ? (uint32_t)lr * row_bytes + (uint32_t)cb : kOOB;
    // Outputs are written once and not read back by the kernel: non-temporal
    // stores (nt, cache-policy bit 2) leave the L2 to the operand panels
    // (grouped MXFP8 + sReLU 2.7% faster, dense MXFP8 0.8%).  Only for row
    // segments of whole 128-byte lines: where two waves each write part of a
    // line (96-byte projection rows, 64-byte packed FP4 rows) streaming
    // stores reached HBM as partial lines, 25% more write traffic.
    constexpr int kStoreNT = G::RB % 128 == 0 ? 2 : 0;
#pragma unroll
    for (int k = 0; k < G::NK; ++k) {
        const i32x4 v = *reinterpret_cast<const i32x4 *>(src + k * G::RPI * G::RBP);
        __builtin_amdgcn_raw_buffer_store_b128(v, rs, voff + (uint32_t)(k * G::RPI) * row_bytes, 0, kStoreNT);
    }
}

// Writes one output of a wave's 128 x (32*NB) quadrant through LDS:
// value(i, j, v, acc) gives the element of register v of block (i, j).  dst
// (and dst2, if non-null) point at element (0, 0) of the quadrant;
// rows_valid and cols_valid bound it (ragged M / N).
template <int DT, int NB, class Fn>
__device__ __forceinline__ void store_quadrant(uint8_t *reg, char *dst, char *dst2, uint32_t row_bytes,
                                               int rows_valid, int cols_valid, f32x16 (&acc)[4][NB],
                                               int lane, Fn &&value)
{
    constexpr int ES = es_of<DT>();
    typedef StageGeom<ES, NB> G;
    const int c = lane & 31, g = lane >> 5;
    uint8_t *wrow = reg + c * G::RBP + 4 * g * ES;
    static_for<4>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
        // keep the scheduler from hoisting later blocks' accumulator reads
        // and arithmetic into this one (the register pressure spills)
        __builtin_amdgcn_sched_barrier(0);
        static_for<NB>([&](auto jj) {
            constexpr int j = decltype(jj)::value;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float x0 = value(i, j, 4 * q, acc[i][j][4 * q]);
                const float x1 = value(i, j, 4 * q + 1, acc[i][j][4 * q + 1]);
                const float x2 = value(i, j, 4 * q + 2, acc[i][j][4 * q + 2]);
                const float x3 = value(i, j, 4 * q + 3, acc[i][j][4 * q + 3]);
                *reinterpret_cast<typename Quad<ES>::T *>(wrow + (32 * j + 8 * q) * ES) =
                    pack_quad<DT>(x0, x1, x2, x3);
            }
        });
        const int rows = rows_valid - 32 * i;
        stage_flush<ES, NB>(reg, dst + (uint32_t)(32 * i) * row_bytes, row_bytes, rows, cols_valid * ES, lane);
        if (dst2)
            stage_flush<ES, NB>(reg, dst2 + (uint32_t)(32 * i) * row_bytes, row_bytes, rows, cols_valid * ES, lane);
    });
}

// Four E2M1 codes, x0 in the lowest nibble: round to nearest even,
// saturating at +-6, sign in bit 3 of each nibble.  gfx950's packed FP4
// conversion with a unit scale does exactly this (the byte its selector
// names takes the first value in its low nibble; the rest of the word is
// left at the given old value); its results equal a nearest-even,
// saturating E2M1 encode at every midpoint between codes, at the fp32
// neighbours of each midpoint, past 6 up to 1e30, and at signed zeros.
// The second conversion writes byte 1 of the first one's result; the two
// high bytes (x0's bits, standing in for an old value) are masked off.
__device__ __forceinline__ uint32_t pack4_e2m1(float x0, float x1, float x2, float x3)
{
    const uint32_t lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(__float_as_uint(x0), x0, x1, 1.0f, 0);
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, x2, x3, 1.0f, 1) & 0xFFFFu;
}

// store_quadrant for packed E2M1 output: two codes per byte, the even
// column in the low nibble.  A lane's four consecutive columns are two
// bytes; a staged row of 32*NB columns is 16*NB bytes (StageGeom<1, NB/2>).
template <int NB, class Fn>
__device__ __forceinline__ void store_quadrant_fp4(uint8_t *reg, char *dst, uint32_t row_bytes, int rows_valid,
                                                   int cols_valid, f32x16 (&acc)[4][NB], int lane, Fn &&value)
{
    static_assert(NB % 2 == 0, "whole 16-byte chunks per staged row");
    typedef StageGeom<1, NB / 2> G;
    const int c = lane & 31, g = lane >> 5;
    uint8_t *wrow = reg + c * G::RBP + 2 * g;
    static_for<4>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
        __builtin_amdgcn_sched_barrier(0);
        static_for<NB>([&](auto jj) {
            constexpr int j = decltype(jj)::value;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float x0 = value(i, j, 4 * q, acc[i][j][4 * q]);
                const float x1 = value(i, j, 4 * q + 1, acc[i][j][4 * q + 1]);
                const float x2 = value(i, j, 4 * q + 2, acc[i][j][4 * q + 2]);
                const float x3 = value(i, j, 4 * q + 3, acc[i][j][4 * q + 3]);
                *reinterpret_cast<uint16_t *>(wrow + 16 * j + 4 * q) = (uint16_t)pack4_e2m1(x0, x1, x2, x3);
            }
        });
        stage_flush<1, NB / 2>(reg, dst + (uint32_t)(32 * i) * row_bytes, row_bytes, rows_valid - 32 * i,
                               cols_valid / 2, lane);
    });
}

// Two outputs of the same type from one pass over the accumulators:
// value(i, j, v, acc, c, d) sets both elements; C is staged at reg, D at
// reg + 32 rows.  dst_d2, if non-null, receives a copy of D.
template <int DT, int NB, class Fn>
__device__ __forceinline__ void store_quadrant2(uint8_t *reg, char *dst_c, char *dst_d, char *dst_d2,
                                                uint32_t row_bytes, int rows_valid, int cols_valid,
                                                f32x16 (&acc)[4][NB], int lane, Fn &&value)
{
    constexpr int ES = DT == DT_F32 ? 4 : 2;
    typedef StageGeom<ES, NB> G;
    const int c = lane & 31, g = lane >> 5;
    uint8_t *reg_d = reg + 32 * G::RBP;
    uint8_t *wc = reg + c * G::RBP + 4 * g * ES, *wd = reg_d + c * G::RBP + 4 * g * ES;
    static_for<4>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
        __builtin_amdgcn_sched_barrier(0);
        static_for<NB>([&](auto jj) {
            constexpr int j = decltype(jj)::value;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float xc[4], xd[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) value(i, j, 4 * q + u, acc[i][j][4 * q + u], xc[u], xd[u]);
                *reinterpret_cast<typename Quad<ES>::T *>(wc + (32 * j + 8 * q) * ES) =
                    pack_quad<DT>(xc[0], xc[1], xc[2], xc[3]);
                *reinterpret_cast<typename Quad<ES>::T *>(wd + (32 * j + 8 * q) * ES) =
                    pack_quad<DT>(xd[0], xd[1], xd[2], xd[3]);
            }
        });
        const int rows = rows_valid - 32 * i;
        const uint32_t roff = (uint32_t)(32 * i) * row_bytes;
        stage_flush<ES, NB>(reg, dst_c + roff, row_bytes, rows, cols_valid * ES, lane);
        stage_flush<ES, NB>(reg_d, dst_d + roff, row_bytes, rows, cols_valid * ES, lane);
        if (dst_d2) stage_flush<ES, NB>(reg_d, dst_d2 + roff, row_bytes, rows, cols_valid * ES, lane);
    });
}

// max(x, x of lane l ^ 32) and x + (x of lane l ^ 32), identical in both
// lanes of the pair.  v_permlane32_swap of x with itself leaves x of the low
// half-wave in the first result and x of the high half-wave in the second,
// in every lane, with no LDS round trip (a shuffle goes through
// ds_bpermute); the sum is the same expression in both lanes, since
// addition is commutative.
__device__ __forceinline__ float max_xor32(float x)
{
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float add_xor32(float x)
{
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// The MX output quantiser's scale step for a block with max |D| = amax:
// SF = smallest power of two >= norm_const * amax / fmax (E8M0 byte), with
// fmax = 448 for E4M3 codes, 57344 for E5M2 and 6 for E2M1 (DF: DT_E4M3,
// DT_E5M2 or DT_E2M1), and the factor norm_const / SF that maps the block
// into the code format's range.
template <int DF = DT_E4M3>
__device__ __forceinline__ uint32_t mx_scale_byte(float amax, float norm_const, float &inv)
{
    const float rcp_max = DF == DT_E5M2 ? 1.0f / 57344.0f : (DF == DT_E2M1 ? 1.0f / 6.0f : 1.0f / 448.0f);
    const float sigma = (norm_const * amax) * rcp_max;
    const uint32_t byte = e8m0_ceil(sigma);
    inv = fminf(ldexpf(norm_const, 127 - (int)byte), 3.402823466e38f);
    return byte;
}

// Per-lane select with a wave-uniform lane mask: x1 in lanes whose mask bit
// is set, else x0 (one v_cndmask_b32).
__device__ __forceinline__ float lane_select(uint64_t mask, float x0, float x1)
{
    float r;
    asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(x0), "v"(x1), "s"(mask));
    return r;
}

// Column scales of one 32x32 block in the accumulator layout, by a
// transposing butterfly.  d[v] is register v of this lane; a column's 32
// values sit in one register over the 32 lanes of a half-wave.
// Each step pairs registers (2m, 2m+1); a lane keeps the one chosen by the
// lane bit in which it differs from its partner lane and takes the max with
// the partner's copy of it, so the register count halves per step.  The
// partners are l ^ 16 (v_permlane16_swap, which exchanges the pair between
// the two rows of a half-wave in one instruction: no selects), l ^ 15
// (row_mirror), l ^ 7 (row_half_mirror) and l ^ 2 (quad_perm), deciding on
// lane bits 4, 3, 2 and 1; a last max with l ^ 1 covers all 32 lanes.  Lane
// l then holds the column max of register col_reg_of_lane(l) = 8 b1 + 4 b2 +
// 2 b3 + b4 (so do l and l ^ 1), computes its E8M0 byte, and the 16 factors
// of each half-wave are broadcast back through xch (32 floats of LDS per
// wave, 16-byte aligned).  Returns this lane's byte.
__device__ __forceinline__ int col_reg_of_lane(int lane)
{
    return 8 * ((lane >> 1) & 1) + 4 * ((lane >> 2) & 1) + 2 * ((lane >> 3) & 1) + ((lane >> 4) & 1);
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}
// One butterfly step: lanes whose mask bit is set keep x1 and send x0 to
// their partner (DPP control CTRL), the others keep x0 and send x1.
template <int CTRL>
__device__ __forceinline__ uint32_t bfly_step(uint64_t mask, uint32_t x0, uint32_t x1)
{
    const uint32_t keep = __float_as_uint(lane_select(mask, __uint_as_float(x0), __uint_as_float(x1)));
    const uint32_t send = __float_as_uint(lane_select(mask, __uint_as_float(x1), __uint_as_float(x0)));
    return max(keep, dpp_mov<CTRL>(send));
}
template <int DF = DT_E4M3>
__device__ __forceinline__ uint32_t col_scales_xch(const float (&d)[16], float nc, float (&cinv)[16], int lane,
                                                   float *xch)
{
    uint32_t u[8], y[4], z[2];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(d[2 * m]) & 0x7FFFFFFFu,
                                                         __float_as_uint(d[2 * m + 1]) & 0x7FFFFFFFu, false, false);
        u[m] = max((uint32_t)sw[0], (uint32_t)sw[1]);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) y[m] = bfly_step<0x140>(0xFF00FF00FF00FF00ull, u[2 * m], u[2 * m + 1]);
#pragma unroll
    for (int m = 0; m < 2; ++m) z[m] = bfly_step<0x141>(0xF0F0F0F0F0F0F0F0ull, y[2 * m], y[2 * m + 1]);
    uint32_t t = bfly_step<0x4E>(0xCCCCCCCCCCCCCCCCull, z[0], z[1]);
    t = max(t, dpp_mov<0xB1>(t));
    float inv;
    const uint32_t byte = mx_scale_byte<DF>(__uint_as_float(t), nc, inv);
    const int half = lane >> 5;
    xch[16 * half + col_reg_of_lane(lane)] = inv;      // lanes l and l ^ 1 write the same value
    const float4 *src = reinterpret_cast<const float4 *>(xch + 16 * half);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float4 f = src[q];
        cinv[4 * q] = f.x;
        cinv[4 * q + 1] = f.y;
        cinv[4 * q + 2] = f.z;
        cinv[4 * q + 3] = f.w;
    }
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

// tanh(r/s)^2 for r >= 0, s > 0, in fp32.  Below r/s = 1/64 it is the
// series y^2 (1 - 2y^2/3) with y = r/s (the first omitted term, 17y^6/45, is
// below 1e-8 of the result there); otherwise (1 - 2/(e^(2y) + 1))^2 with
// e^(2y) = 2^(r * 2 log2(e) / s), which overflows to +inf for large r and then
// gives exactly 1.  Both forms are evaluated and one is selected, so the
// epilogue has no divergent branch per element.  t = 1 - 2/(e^(2y)+1) is
// within about 1e-7 absolute of tanh(y).  The per-call constants come from
// the host (tanh_sq_const) and live in scalar registers.
struct TanhSqConst {
    float is2;      // 1/s^2
    float c4;       // -(2/3)/s^4
    float k_exp;    // 2 log2(e)/s
    float thr;      // s/64: the series below it
};
inline TanhSqConst tanh_sq_const(float s)
{
    TanhSqConst t{0.0f, 0.0f, 0.0f, 0.0f};
    if (s > 0.0f) {
        const double is = 1.0 / (double)s;
        t.is2 = (float)(is * is);
        t.c4 = (float)(-(2.0 / 3.0) * is * is * is * is);
        t.k_exp = (float)(2.0 * 1.4426950408889634 * is);
        t.thr = (float)((double)s / 64.0);
    }
    return t;
}
__device__ __forceinline__ float tanh_sq(float r, const TanhSqConst &tq)
{
    const float r2 = r * r;
    const float series = r2 * fmaf(r2, tq.c4, tq.is2);
    const float t = fmaf(-2.0f, __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(r * tq.k_exp) + 1.0f), 1.0f);
    return r < tq.thr ? series : t * t;
}

}  // namespace bsg
