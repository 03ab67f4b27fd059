// "GEMM + Amax (SM100)" with k-major operands, and the launcher of every
// gemm_amax variant.
#include "gemm_amax.hpp"

namespace bsg {

__global__ void k_fill_zero(float *p, int64_t n)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

hipError_t zero_floats(float *p, int64_t n, hipStream_t s)
{
    if (!p || n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
    return hipGetLastError();
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
    dim3 grid((unsigned)(((a.n + kTileN - 1) / kTileN) * ((a.m + kTileM - 1) / kTileM) * a.l));
    if (a.a_mn || a.b_mn) {
        launch_gemm_amax_mn(p, a.fmt | (a.a_mn ? FMT_TA : 0) | (a.b_mn ? FMT_TB : 0), grid, s);
    } else if (a.fmt == FMT_E4M3) launch_gemm_amax_fmt<FMT_E4M3>(p, grid, s);
    else if (a.fmt == FMT_E5M2) launch_gemm_amax_fmt<FMT_E5M2>(p, grid, s);
    else launch_gemm_amax_fmt<FMT_E2M1>(p, grid, s);
    return hipGetLastError();
}

}  // namespace bsg
