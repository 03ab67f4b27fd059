// Helpers shared by the GEMM kernel files: element loads, output stores
// through the wave's LDS staging rows with a run-time output type.
#pragma once
#include "device.hpp"
#include "launch.hpp"

namespace bsg {

__device__ __forceinline__ float load_elem(const void *base, int64_t idx, int dtype)
{
    if (dtype == DT_F32) return static_cast<const float *>(base)[idx];
    uint16_t h = static_cast<const uint16_t *>(base)[idx];
    if (dtype == DT_BF16) return __uint_as_float((uint32_t)h << 16);
    return (float)__builtin_bit_cast(_Float16, h);
}

// Zero-fills n floats on stream s (defined in kernels_amax.hip).
hipError_t zero_floats(float *p, int64_t n, hipStream_t s);

inline uint32_t row_bytes_of(int fmt, int64_t k)
{
    return (uint32_t)(fmt == FMT_E2M1 ? k / 2 : (fmt == FMT_BF16 ? 2 * k : k));
}

// One output of a wave's 128 x (32*NB) quadrant through the wave's LDS
// staging region: dispatches on the run-time output type (fp32 / fp16 /
// bf16, or the unscaled saturating E4M3 / E5M2 / packed E2M1 casts of an FP8
// or FP4 C).  (row0, col0) is the quadrant's first element; rows_valid /
// cols_valid bound it.  base2, if non-null, receives a copy (16-bit and
// 32-bit types only).
template <int NB, class Fn>
__device__ __forceinline__ void store_quadrant_rt(int dt, uint8_t *reg, void *base, void *base2, int64_t n,
                                                  int64_t row0, int64_t col0, int rows_valid, int cols_valid,
                                                  f32x16 (&acc)[4][NB], int lane, Fn &&value)
{
    if (dt == DT_E2M1) {
        char *dst = static_cast<char *>(base) + (row0 * n + col0) / 2;
        store_quadrant_fp4<NB>(reg, dst, (uint32_t)(n / 2), rows_valid, cols_valid, acc, lane, value);
        return;
    }
    const int es = dt == DT_F32 ? 4 : ((dt == DT_E4M3 || dt == DT_E5M2) ? 1 : 2);
    char *dst = static_cast<char *>(base) + (row0 * n + col0) * es;
    char *dst2 = base2 ? static_cast<char *>(base2) + (row0 * n + col0) * es : nullptr;
    const uint32_t rb = (uint32_t)(n * es);
    if (dt == DT_F32) store_quadrant<DT_F32, NB>(reg, dst, dst2, rb, rows_valid, cols_valid, acc, lane, value);
    else if (dt == DT_BF16) store_quadrant<DT_BF16, NB>(reg, dst, dst2, rb, rows_valid, cols_valid, acc, lane, value);
    else if (dt == DT_F16) store_quadrant<DT_F16, NB>(reg, dst, dst2, rb, rows_valid, cols_valid, acc, lane, value);
    else if (dt == DT_E4M3) store_quadrant<DT_E4M3, NB>(reg, dst, nullptr, rb, rows_valid, cols_valid, acc, lane, value);
    else store_quadrant<DT_E5M2, NB>(reg, dst, nullptr, rb, rows_valid, cols_valid, acc, lane, value);
}

// Waits for every outstanding vector-memory load before the epilogue's first
// store (see the file comment).
__device__ __forceinline__ void wait_loads() { s_wait_vm<0>(); }

__device__ __forceinline__ int clamp_extent(int64_t extent) { return extent < 0 ? 0 : (extent > 128 ? 128 : (int)extent); }

// Operand X stored MN-major (FP8, memory [L][K][MN]): the tile's columns
// [mn0, mn0 + cols) of every K row.  The readable range ends at the last K
// row's last column, so K rows past K read zeros; columns past MN in the
// other K rows are masked per lane (OperandDesc::mn_valid).
__device__ __forceinline__ void mn_major_operand(OperandDesc &X, const uint8_t *x, int64_t batch, int64_t mn,
                                                 int64_t mn0, int64_t cols, int64_t k)
{
    X.base = x + batch * mn * k + mn0;
    X.bytes = k > 0 ? (uint32_t)((k - 1) * mn + (mn - mn0)) : 0u;
    X.row_bytes = (uint32_t)mn;
    X.mn_valid = (uint32_t)cols;
}

}  // namespace bsg
