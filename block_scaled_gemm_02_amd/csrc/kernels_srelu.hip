// "Grouped GEMM + sReLU (SM100)" launcher.
#include "grouped.hpp"

namespace bsg {

hipError_t launch_grouped_srelu(const GroupedArgs &a, hipStream_t s)
{
    hipError_t e = zero_floats(a.amax, a.num_experts, s);
    if (e != hipSuccess) return e;
    if (a.m == 0 || a.n == 0) return hipSuccess;
    GroupedParams p = grouped_params(a);
    dim3 grid((unsigned)(((a.n + kTileN - 1) / kTileN) * (a.m / kTileM)));
    if (a.d_dtype == DT_E4M3 || a.d_dtype == DT_E5M2 || a.d_dtype == DT_E2M1) {
        // MX-quantised D: FP8 operands only
        if (a.fmt != FMT_E4M3 && a.fmt != FMT_E5M2) return hipErrorNotSupported;
        launch_grouped_srelu_mx(p, a.fmt, a.d_dtype, grid, s);
    } else if (a.fmt == FMT_E4M3) {
        launch_srelu_variant<FMT_E4M3, EPI_SRELU>(p, grid, s);
    } else if (a.fmt == FMT_E5M2) {
        launch_srelu_variant<FMT_E5M2, EPI_SRELU>(p, grid, s);
    } else {
        launch_srelu_variant<FMT_E2M1, EPI_SRELU>(p, grid, s);
    }
    return hipGetLastError();
}

}  // namespace bsg
