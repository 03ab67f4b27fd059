// "Grouped GEMM (SM100 BF16)" launcher.
#include "grouped.hpp"

namespace bsg {

hipError_t launch_grouped_gemm(const GroupedArgs &a, hipStream_t s)
{
    if (a.m == 0 || a.n == 0) return hipSuccess;
    GroupedParams p = grouped_params(a);
    dim3 grid((unsigned)(((a.n + kTileN - 1) / kTileN) * (a.m / kTileM)));
    const bool fast = p.c && p.c_dtype == DT_BF16 && p.d_dtype == DT_BF16;
    if (p.bias) {
        if (fast) hipLaunchKernelGGL((k_grouped<FMT_BF16, EPI_BF16_BIAS, false, DT_BF16>), grid, dim3(kThreads), 0, s, p);
        else hipLaunchKernelGGL((k_grouped<FMT_BF16, EPI_BF16_BIAS, false>), grid, dim3(kThreads), 0, s, p);
    } else {
        if (fast) hipLaunchKernelGGL((k_grouped<FMT_BF16, EPI_BF16, false, DT_BF16>), grid, dim3(kThreads), 0, s, p);
        else hipLaunchKernelGGL((k_grouped<FMT_BF16, EPI_BF16, false>), grid, dim3(kThreads), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace bsg
