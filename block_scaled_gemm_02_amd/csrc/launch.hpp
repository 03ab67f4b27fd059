// Host-side launch interface between the C ABI (api.cpp) and the kernels.
// Arguments have already been validated when these are called.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsg {

struct GemmAmaxArgs {
    const uint8_t *a, *b, *sfa, *sfb;
    void *c;
    float *amax;
    int64_t m, n, k, l;
    int fmt;       // bsg::Fmt: 0 = E4M3, 1 = E2M1, 4 = E5M2
    int c_dtype;   // bsg_dtype
    int a_mn = 0;  // A stored m-major ([L][K][M]; FP8 only)
    int b_mn = 0;  // B stored n-major ([L][K][N]; FP8 only)
};

struct GroupedArgs {
    const uint8_t *a, *b, *sfa, *sfb;   // sfa/sfb null for BF16
    const uint64_t *b_ptrs, *sfb_ptrs;  // discrete weights: per-expert B / SFB addresses (else null)
    const int32_t *offsets;
    const float *alpha, *prob, *norm_const;
    const void *bias;
    void *c, *d, *d_col;
    uint8_t *sfd_row, *sfd_col;
    float *amax;
    int64_t m, n, k, num_experts;
    int fmt;        // bsg::Fmt: 0 = E4M3, 1 = E2M1, 2 = BF16, 4 = E5M2
    int c_dtype, d_dtype, bias_dtype;
    float tanh_s;   // <= 0: no clamp
    // grouped_gemm_dswiglu only (else null): beta (L,), forward C (M, 2N) bf16, dprob (M,)
    const float *beta = nullptr;
    const uint16_t *cfwd = nullptr;
    float *dprob = nullptr;
    int b_mn = 0;   // B stored n-major ([L][K][N]; FP8 grouped_gemm_dswiglu only)
};

struct ProjRopeArgs {
    const void *x, *w;                  // bf16, or E4M3 codes when mxfp8
    const uint8_t *x_scale, *w_scale;   // row-major E8M0 (mxfp8 only)
    const uint16_t *cos, *sin;
    uint8_t *q_row, *s_row, *q_col, *s_col;
    int64_t tokens, q_lora, heads, head_dim, qk_rope;
    int w_out_in;
    int mxfp8;                          // 1: E4M3 inputs with x_scale / w_scale
};

hipError_t launch_gemm_amax(const GemmAmaxArgs &a, hipStream_t s);
hipError_t launch_grouped_gemm(const GroupedArgs &a, hipStream_t s);
hipError_t launch_grouped_srelu(const GroupedArgs &a, hipStream_t s);
hipError_t launch_proj_rope(const ProjRopeArgs &a, hipStream_t s);
hipError_t launch_grouped_dswiglu(const GroupedArgs &a, hipStream_t s);

}  // namespace bsg
