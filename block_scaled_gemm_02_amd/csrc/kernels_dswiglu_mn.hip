// "Grouped GEMM + dSwiGLU (SM100)" with FP8 operands and B stored n-major
// (the page's Input/Output tensors: B stride (1, N, N*K); Layouts and
// strides: FP4 B stays k-major).  B is staged K-major in LDS and transposed
// into MFMA fragments by the LDS reads (device.hpp).
#include "grouped.hpp"

namespace bsg {

void launch_dswiglu_bn(const GroupedParams &p, int fmt, int d_dtype, dim3 grid, hipStream_t s)
{
    constexpr int E4 = FMT_E4M3 | FMT_TB, E5 = FMT_E5M2 | FMT_TB;
    if (fmt == FMT_E4M3) {
        if (d_dtype == DT_E5M2) hipLaunchKernelGGL((k_grouped<E4, EPI_DSWIGLU_FP8, false, DT_E5M2>), grid, dim3(kThreads), 0, s, p);
        else hipLaunchKernelGGL((k_grouped<E4, EPI_DSWIGLU_FP8, false>), grid, dim3(kThreads), 0, s, p);
    } else {
        if (d_dtype == DT_E5M2) hipLaunchKernelGGL((k_grouped<E5, EPI_DSWIGLU_FP8, false, DT_E5M2>), grid, dim3(kThreads), 0, s, p);
        else hipLaunchKernelGGL((k_grouped<E5, EPI_DSWIGLU_FP8, false>), grid, dim3(kThreads), 0, s, p);
    }
}

}  // namespace bsg
