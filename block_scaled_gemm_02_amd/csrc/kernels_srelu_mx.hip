// "Grouped GEMM + sReLU (SM100)" with MX-quantised D (FP8 or FP4 codes plus
// the SFD_row / SFD_col scale atoms).
#include "grouped.hpp"

namespace bsg {

void launch_grouped_srelu_mx(const GroupedParams &p, int fmt, int d_dtype, dim3 grid, hipStream_t s)
{
    if (d_dtype == DT_E4M3) {
        if (fmt == FMT_E4M3) launch_srelu_variant<FMT_E4M3, EPI_SRELU_FP8>(p, grid, s);
        else launch_srelu_variant<FMT_E5M2, EPI_SRELU_FP8>(p, grid, s);
    } else if (d_dtype == DT_E5M2) {
        if (fmt == FMT_E4M3) launch_srelu_variant<FMT_E4M3, EPI_SRELU_FP8, DT_E5M2>(p, grid, s);
        else launch_srelu_variant<FMT_E5M2, EPI_SRELU_FP8, DT_E5M2>(p, grid, s);
    } else {
        if (fmt == FMT_E4M3) launch_srelu_variant<FMT_E4M3, EPI_SRELU_FP8, DT_E2M1>(p, grid, s);
        else launch_srelu_variant<FMT_E5M2, EPI_SRELU_FP8, DT_E2M1>(p, grid, s);
    }
}

}  // namespace bsg
