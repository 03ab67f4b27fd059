// "GEMM + Amax (SM100)" with FP8 operands of which A is stored m-major
// and / or B n-major (the (1, M, M*K) and (1, N, N*K) strides of the page's
// Input/Output tensors).  Such operands are staged K-major in LDS and
// transposed into MFMA fragments by the LDS reads (device.hpp).
#include "gemm_amax.hpp"

namespace bsg {

template <int F>
static void launch_mn(const GemmAmaxParams &p, dim3 grid, hipStream_t s)
{
    if (p.c_dtype == DT_F32) hipLaunchKernelGGL((k_gemm_amax<F, DT_F32>), grid, dim3(kThreads), 0, s, p);
    else if (p.c_dtype == DT_BF16) hipLaunchKernelGGL((k_gemm_amax<F, DT_BF16>), grid, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((k_gemm_amax<F, DT_F16>), grid, dim3(kThreads), 0, s, p);
}

void launch_gemm_amax_mn(const GemmAmaxParams &p, int fmt, dim3 grid, hipStream_t s)
{
    switch (fmt) {
    case FMT_E4M3 | FMT_TA: launch_mn<FMT_E4M3 | FMT_TA>(p, grid, s); break;
    case FMT_E4M3 | FMT_TB: launch_mn<FMT_E4M3 | FMT_TB>(p, grid, s); break;
    case FMT_E4M3 | FMT_TA | FMT_TB: launch_mn<FMT_E4M3 | FMT_TA | FMT_TB>(p, grid, s); break;
    case FMT_E5M2 | FMT_TA: launch_mn<FMT_E5M2 | FMT_TA>(p, grid, s); break;
    case FMT_E5M2 | FMT_TB: launch_mn<FMT_E5M2 | FMT_TB>(p, grid, s); break;
    case FMT_E5M2 | FMT_TA | FMT_TB: launch_mn<FMT_E5M2 | FMT_TA | FMT_TB>(p, grid, s); break;
    default: break;   // rejected by the host validation
    }
}

}  // namespace bsg
