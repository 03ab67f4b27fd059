// "Grouped GEMM + dSwiGLU (SM100)" launcher.
#include "grouped.hpp"

namespace bsg {

hipError_t launch_grouped_dswiglu(const GroupedArgs &a, hipStream_t s)
{
    if (a.fmt == FMT_E2M1) {
        // FP4 inputs: per-expert amax (L, 2), zero-filled first (also for an empty problem)
        hipError_t e = zero_floats(a.amax, 2 * a.num_experts, s);
        if (e != hipSuccess) return e;
    }
    if (a.m == 0 || a.n == 0) return hipSuccess;
    GroupedParams p = grouped_params(a);
    dim3 grid((unsigned)(((a.n + kTileN - 1) / kTileN) * (a.m / kTileM)));
    if (a.fmt == FMT_E2M1) {
        if (a.d_dtype == DT_F32) hipLaunchKernelGGL((k_grouped<FMT_E2M1, EPI_DSWIGLU, false, DT_F32>), grid, dim3(kThreads), 0, s, p);
        else hipLaunchKernelGGL((k_grouped<FMT_E2M1, EPI_DSWIGLU, false, DT_BF16>), grid, dim3(kThreads), 0, s, p);
    } else if (a.b_mn) {
        if (a.fmt != FMT_E4M3 && a.fmt != FMT_E5M2) return hipErrorNotSupported;
        launch_dswiglu_bn(p, a.fmt, a.d_dtype, grid, s);
    } else if (a.fmt == FMT_E4M3) {
        if (a.d_dtype == DT_E5M2) hipLaunchKernelGGL((k_grouped<FMT_E4M3, EPI_DSWIGLU_FP8, false, DT_E5M2>), grid, dim3(kThreads), 0, s, p);
        else hipLaunchKernelGGL((k_grouped<FMT_E4M3, EPI_DSWIGLU_FP8, false>), grid, dim3(kThreads), 0, s, p);
    } else if (a.fmt == FMT_E5M2) {
        if (a.d_dtype == DT_E5M2) hipLaunchKernelGGL((k_grouped<FMT_E5M2, EPI_DSWIGLU_FP8, false, DT_E5M2>), grid, dim3(kThreads), 0, s, p);
        else hipLaunchKernelGGL((k_grouped<FMT_E5M2, EPI_DSWIGLU_FP8, false>), grid, dim3(kThreads), 0, s, p);
    } else {
        return hipErrorNotSupported;
    }
    return hipGetLastError();
}

}  // namespace bsg
