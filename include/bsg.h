/*
 * bsg.h -- block-scaled GEMM family for AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels.  Four operations, each the
 * problem statement of one cuDNN frontend "GEMM fusions" documentation page:
 *
 *   gemm_amax             "GEMM + Amax (SM100)"
 *   grouped_gemm          "Grouped GEMM (SM100 BF16)"
 *   grouped_gemm_srelu    "Grouped GEMM + sReLU (SM100)"
 *   grouped_gemm_dswiglu  "Grouped GEMM + dSwiGLU (SM100)"
 *   gemm_proj_rope_mxfp8  "GEMM + RoPE + MXFP8 Projection (SM100)"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer on the current HIP device;
 *    `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *  - All calls are asynchronous: arguments are validated on the host, then
 *    kernels are enqueued on `stream`; there is no host synchronisation.
 *    Every error the host can detect is returned BEFORE anything is
 *    enqueued ("Grouped GEMM (SM100 BF16)", Scheduling, caching, and errors).
 *  - The caller owns every buffer and keeps it alive and unmodified until
 *    the stream has completed the call ("Grouped GEMM (SM100 BF16)",
 *    Tensors and layouts).  The library allocates no device memory per call
 *    (same page, Using JAX arrays: workspaces belong to the caller).
 *  - Device-resident VALUES (padded_offsets, alpha, prob, ...) are the
 *    caller's responsibility and are not checked ("Grouped GEMM + dSwiGLU
 *    (SM100)", JAX execution: offsets are the caller's responsibility).
 *  - Operand layouts: A (M,K,L) and B (N,K,L) are k-major, i.e. memory
 *    order [L][rows][K], and C/D are n-major, memory order [L][M][N],
 *    except where an entry point takes a major argument (gemm_amax and the
 *    B operand of grouped_gemm_dswiglu).  Packed
 *    FP4 (E2M1X2) stores two codes per byte, element 2j in the low nibble,
 *    so a row holds K/2 bytes ("GEMM + Amax (SM100)", Layouts and strides).
 *  - Scale factors: one E8M0 byte per 32 consecutive K elements of a row
 *    (sf_vec_size = 32), stored in the scale-atom layout of the pages'
 *    Shapes sections: logical (32, 4, ceil(MN/128), 4, ceil(K/128), L),
 *    i.e. the C-contiguous physical buffer (L, ceil(MN/128), ceil(K/128),
 *    32, 4, 4).  The byte for row r, K-block kb = k/32, batch l sits at
 *        (((l*MN' + r/128)*K' + kb/4)*32 + r%32)*16 + ((r%128)/32)*4 + kb%4
 *    with MN' = ceil(MN/128), K' = ceil(K/128).  Bytes of padding rows and
 *    padding K-blocks are ignored.
 *  - Alignment: base pointers of A, B, C, D, D_col, x, w, cos, sin and the
 *    fp8 outputs must be 16-byte aligned and so must each row's byte length
 *    ("GEMM + Amax (SM100)": 16-byte alignment along the contiguous
 *    dimension); the sfd_row / sfd_col scale buffers must be 4-byte aligned.
 *  - Return value: BSG_OK (0) or a bsg_status; bsg_last_error() returns a
 *    thread-local message describing the most recent failure.
 */
#ifndef BSG_H
#define BSG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bsg_status {
    BSG_OK = 0,
    BSG_ERR_NULLPTR = 1,     /* a required pointer is NULL */
    BSG_ERR_SHAPE = 2,       /* negative or inconsistent sizes */
    BSG_ERR_DTYPE = 3,       /* dtype not valid for this argument */
    BSG_ERR_ALIGN = 4,       /* 16-byte alignment rule broken */
    BSG_ERR_UNSUPPORTED = 5, /* valid on the pages, not built here */
    BSG_ERR_DEVICE = 6,      /* current device is not gfx950 / HIP error */
    BSG_ERR_LAUNCH = 7       /* kernel launch failed */
} bsg_status;

typedef enum bsg_dtype {
    BSG_F32 = 0,
    BSG_F16 = 1,
    BSG_BF16 = 2,
    BSG_E4M3 = 3,   /* float8_e4m3fn (OCP) */
    BSG_E5M2 = 4,   /* float8_e5m2 */
    BSG_E2M1X2 = 5, /* float4_e2m1fn_x2: two E2M1 codes per byte */
    BSG_E8M0 = 6    /* float8_e8m0fnu */
} bsg_dtype;

/*
 * gemm_amax -- "GEMM + Amax (SM100)", Equations:
 *     C[m,n,l] = sum_k dequant(A)[m,k,l] * dequant(B)[n,k,l]
 *     Amax     = max_{m,n,l} |C[m,n,l]|
 * with dequant(X)[r,k,l] = X[r,k,l] * 2^(SF byte - 127) per 32-wide K block.
 *
 *  a     (M,K,L) codes; E4M3 / E5M2: M*K*L bytes; E2M1X2: M*(K/2)*L bytes.
 *        a_major 'k': k-major, memory [L][M][K] (stride (K, 1, M*K));
 *        a_major 'm': m-major, memory [L][K][M] (stride (1, M, M*K)),
 *        E4M3 / E5M2 only, M % 16 == 0 and (K + 256) * M < 2^31
 *  b     (N,K,L) codes, same dtype as a; b_major 'k': memory [L][N][K];
 *        b_major 'n': n-major, memory [L][K][N], under the same rules
 *        ("GEMM + Amax (SM100)", Input/Output tensors and Layouts and
 *        strides: packed FP4 A/B must be k-major)
 *  sfa   scale atoms over (M, K, L);  sfb: scale atoms over (N, K, L); the
 *        same layout whatever the operand majors
 *  c     (M,N,L) output; c_major 'n': n-major, memory [L][M][N]; c_major
 *        'm': m-major, memory [L][N][M] (the page's c_major; packed FP4 C
 *        must be n-major).  c_dtype in {F32, BF16, F16}; RNE cast
 *        of the fp32 accumulator.  With E2M1X2 A/B, c_dtype may also be
 *        E4M3 or E5M2 (the page's Dtypes allow FP8 C only with FP4 A/B): a
 *        plain RNE cast with no scale factor, saturated to +-448 / +-57344
 *        (never NaN or Inf).  Also with E2M1X2 A/B: c_dtype E2M1X2,
 *        packed FP4 C of (M, N/2, L) bytes, two codes per byte with the
 *        even column in the low nibble, an RNE cast saturated to +-6;
 *        N % 32 == 0.  FP8 C with FP8 A/B returns UNSUPPORTED; FP4 C with
 *        FP8 A/B returns DTYPE.  A row of C (along its contiguous
 *        dimension) must be a multiple of 16 bytes.
 *  amax  one float32 (nullable): max |C| of the fp32 accumulators (before
 *        the output cast); the library zero-fills it on `stream` first
 *  ab_dtype in {E4M3, E5M2, E2M1X2} (the page's float8_e4m3fn, float8_e5m2
 *  and float4_e2m1fn_x2 A/B); sf_vec_size must be 32.  a_major, b_major
 *  and c_major are the characters above; any other value, an MN-major
 *  packed FP4 operand or an m-major packed FP4 C returns SHAPE.
 *  Sizes: M, N, L >= 0; K >= 0 with K % 32 == 0.  M or N need not be tile
 *  multiples.  Accumulation is fp32 (the pages' only accumulator dtype).
 */
int gemm_amax(const void *a, const void *b, const uint8_t *sfa, const uint8_t *sfb,
              void *c, float *amax, int64_t m, int64_t n, int64_t k, int64_t l,
              int ab_dtype, int c_dtype, int sf_vec_size, int a_major, int b_major,
              int c_major, void *stream);

/*
 * grouped_gemm -- "Grouped GEMM (SM100 BF16)", Operation.  For expert g
 * with rows [begin_g, padded_offsets[g]) (begin_0 = 0, begin_g =
 * padded_offsets[g-1]):
 *     G = alpha[g] * A_g @ B_g^T                     (fp32 accumulation)
 *     with bias:    C = G + prob[m] * bias[n,g],  D = C
 *     without bias: C = G,                        D = prob[m] * G
 *
 *  a               (M,K) bf16, k-major
 *  b               (N,K,L) bf16, k-major: memory [L][N][K]
 *  padded_offsets  (L,) int32 cumulative padded ends, nondecreasing
 *                  multiples of 256 in [0, M]
 *  alpha (L,) fp32;  prob (M,) fp32
 *  bias            (N,L) with stride (1,N): memory [L][N]; nullable;
 *                  bias_dtype in {BF16, F16, F32}
 *  c               (M,N) n-major, nullable (no C output); c_dtype
 *  d               (M,N) n-major; d_dtype;  c/d dtypes in {BF16, F16, F32}
 *  Rows at or past padded_offsets[L-1] are not written.
 *  Sizes: M % 256 == 0, 1 <= L <= 1024, K % 8 == 0, N % 8 == 0.
 */
int grouped_gemm(const void *a, const void *b, const int32_t *padded_offsets,
                 const float *alpha, const float *prob, const void *bias,
                 void *c, void *d, int64_t m, int64_t n, int64_t k, int64_t num_experts,
                 int bias_dtype, int c_dtype, int d_dtype, void *stream);

/*
 * grouped_gemm_srelu -- "Grouped GEMM + sReLU (SM100)", Equations and
 * Tanh soft clamp.  For rows m of expert g:
 *     C[m,n] = alpha[g] * sum_k dequant(A)[m,k] * dequant(B)[n,k,g]
 *     D[m,n] = prob[m] * relu(C)^2                       (s <= 0)
 *     D[m,n] = prob[m] * (s * min(1, tanh(relu(C)/s)))^2  (s > 0)
 * evaluated in fp32 from the accumulator.
 *
 *  a, sfa          (M,K) codes, k-major, scale atoms over (M, K, 1)
 *  b, sfb          (N,K,L) codes [L][N][K]; scale atoms over (N, K, L)
 *  padded_offsets, alpha, prob   as for grouped_gemm
 *  c               (M,N) pre-activation alpha*acc, nullable; c_dtype in
 *                  {BF16, F16, F32} (RNE cast), or E4M3 / E5M2 (a round to
 *                  nearest even saturated to +-448 / +-57344, no scale
 *                  factor) or E2M1X2 ((M, N/2) bytes, two codes per byte,
 *                  the even column in the low nibble, saturated to +-6)
 *  d_dtype in {BF16, F16, F32}:
 *      d      (M,N) D, RNE cast;  d_col: nullable copy of d
 *      amax   (L,) fp32, nullable: amax[g] = max |D| over expert g's rows
 *             (fp32 values before the cast); zero-filled by the library;
 *             an expert with no rows reports 0
 *  d_dtype == E4M3, E5M2 or E2M1X2 (MX output, "Grouped GEMM + dSwiGLU
 *  (SM100)" Step 3 quantiser with rcp_max = 1/448 for E4M3 codes, 1/57344
 *  for E5M2 and 1/6 for E2M1; E2M1 codes are packed two per byte with the
 *  even column in the low nibble, so d and d_col are (M, N/2) bytes):
 *      d        (M,N) codes quantised in 32-wide blocks along N
 *      sfd_row  scale atoms over (M, N, 1)  (MN = M, "K" = N)
 *      d_col    (M,N) codes quantised in 32-tall blocks along M
 *      sfd_col  scale atoms over (N, M, 1)  (MN = N, "K" = M)
 *      norm_const (1,) fp32 device scalar, required
 *  tanh_clamp_scale: s; a value <= 0 means no clamp (the pages' None).
 *  ab_dtype in {E4M3, E5M2, E2M1X2}; sf_vec_size == 32.  A quantised D
 *  needs FP8 (E4M3 or E5M2) A/B.
 *  Sizes: M % 256 == 0, 1 <= L <= 1024, K % 32 == 0, N % 32 == 0.
 *  Rows at or past padded_offsets[L-1] are not written.
 */
int grouped_gemm_srelu(const void *a, const void *b, const uint8_t *sfa, const uint8_t *sfb,
                       const int32_t *padded_offsets, const float *alpha, const float *prob,
                       const float *norm_const, void *c, void *d, void *d_col,
                       uint8_t *sfd_row, uint8_t *sfd_col, float *amax,
                       int64_t m, int64_t n, int64_t k, int64_t num_experts,
                       int ab_dtype, int c_dtype, int d_dtype, int sf_vec_size,
                       float tanh_clamp_scale, void *stream);

/*
 * Discrete-weight forms -- "Grouped GEMM (SM100 BF16)", discrete mode of the
 * weight arguments, and "Grouped GEMM + sReLU (SM100)", Discrete-weight
 * wrapper and the b_ptrs / sfb_ptrs inputs.  The math is that of the dense
 * call; only the weight addressing differs: expert g's B is its own
 * allocation instead of slice g of one (N,K,L) tensor.
 *
 *  b_ptrs    (L,) contiguous device array of uint64: b_ptrs[g] is the
 *            device address of expert g's (N,K) k-major B (bf16 for
 *            grouped_gemm_discrete; E4M3 / packed E2M1 codes for
 *            grouped_gemm_srelu_discrete)
 *  sfb_ptrs  (L,) contiguous device array of uint64: sfb_ptrs[g] is expert
 *            g's scale atoms over (N, K, 1)
 *  Every other argument, size limit and status is that of grouped_gemm /
 *  grouped_gemm_srelu.  The pointer arrays must be non-null and 8-byte
 *  aligned (checked); each target must be 16-byte aligned and stay alive
 *  and unmodified until the stream completes (the caller's contract, as
 *  for padded_offsets: device values are not checked).  An expert with no
 *  rows has its pointers never read.
 */
int grouped_gemm_discrete(const void *a, const uint64_t *b_ptrs, const int32_t *padded_offsets,
                          const float *alpha, const float *prob, const void *bias,
                          void *c, void *d, int64_t m, int64_t n, int64_t k, int64_t num_experts,
                          int bias_dtype, int c_dtype, int d_dtype, void *stream);
int grouped_gemm_srelu_discrete(const void *a, const uint64_t *b_ptrs, const uint8_t *sfa,
                                const uint64_t *sfb_ptrs, const int32_t *padded_offsets,
                                const float *alpha, const float *prob, const float *norm_const,
                                void *c, void *d, void *d_col, uint8_t *sfd_row, uint8_t *sfd_col,
                                float *amax, int64_t m, int64_t n, int64_t k, int64_t num_experts,
                                int ab_dtype, int c_dtype, int d_dtype, int sf_vec_size,
                                float tanh_clamp_scale, void *stream);

/*
 * grouped_gemm_dswiglu -- "Grouped GEMM + dSwiGLU (SM100)", Equations.
 * For rows m of expert g (ranges as in grouped_gemm):
 *     ref[m,n] = alpha[g]^2 * sum_k dequant(A)[m,k] * dequant(B)[n,k,g]
 *     input, gate: C[m, 64b + o] and C[m, 64b + 32 + o] times beta[g],
 *                  for ref column n = 32b + o (32-column pairs)
 *     swish   = gate * sigmoid(gate)
 *     D[m, 64b + o]      = ref * prob[m] * swish                      (ab)
 *     D[m, 64b + 32 + o] = ref * prob[m] * input * sigmoid(gate)
 *                           * (1 + gate * (1 - sigmoid(gate)))         (dswiglu)
 *     dprob[m] += sum_n swish * input * ref
 * evaluated in fp32 from the accumulator.  With FP8 (E4M3 / E5M2) A/B, D is
 * MXFP8-quantised like the FP8 D of grouped_gemm_srelu (Step 3; d_dtype E4M3
 * with rcp_max = 1/448, or E5M2 with rcp_max = 1/57344):
 *  a, sfa, b, sfb, padded_offsets, alpha, prob   as for grouped_gemm_srelu
 *  c        (M, 2N) bf16, n-major: the forward input/gate tensor
 *  beta     (L,) fp32
 *  d_row    (M, 2N) FP8 codes in 32-wide blocks along 2N; sfd_row: scale
 *           atoms over (M, 2N, 1)
 *  d_col    (M, 2N) FP8 codes in 32-tall blocks along M; sfd_col: scale
 *           atoms over (2N, M, 1)
 *  norm_const (1,) fp32 device scalar
 *  dprob    (M,) fp32, accumulated with atomic adds: the caller zero-fills
 *           it (as the page requires); 4-byte aligned
 * With FP4 (E2M1X2) A/B, D is unquantised (the page's FP4-input form):
 *  d_row    (M, 2N) d_dtype BF16 or F32 (RNE cast); d_col: nullable copy
 *  amax     (L, 2) fp32, nullable: amax[g][0] = max |ab|, amax[g][1] =
 *           max |dswiglu| over expert g's rows (fp32 values before the
 *           cast); zero-filled by the library; norm_const and sfd_* unused
 *  c_dtype BF16; other C dtypes return UNSUPPORTED.
 *  b_major  'k': B k-major, memory [L][N][K]; 'n': B n-major, memory
 *           [L][K][N] (stride (1, N, N*K)), FP8 A/B only and
 *           (K + 256) * N < 2^31 ("Grouped GEMM + dSwiGLU (SM100)", Layouts
 *           and strides: FP4 B must be k-major; other values return SHAPE).
 *           Both give identical results.
 *  Sizes: M % 256 == 0, 1 <= L <= 1024, K % 32 == 0, N % 32 == 0.  Rows at
 *  or past padded_offsets[L-1] are not written.
 */
int grouped_gemm_dswiglu(const void *a, const void *b, const uint8_t *sfa, const uint8_t *sfb,
                         const void *c, const int32_t *padded_offsets, const float *alpha,
                         const float *beta, const float *prob, const float *norm_const,
                         void *d_row, void *d_col, uint8_t *sfd_row, uint8_t *sfd_col,
                         float *dprob, float *amax, int64_t m, int64_t n, int64_t k,
                         int64_t num_experts, int ab_dtype, int c_dtype, int d_dtype,
                         int sf_vec_size, int b_major, void *stream);

/*
 * gemm_proj_rope_mxfp8 -- "GEMM + RoPE + MXFP8 Projection (SM100)",
 * Equations:
 *     Y[t,h,:] = (x W) reshaped to [tokens, num_heads, head_dim]
 *     the trailing qk_rope features of each head get the interleaved-in /
 *     halves-out rotary embedding, pairs (2j, 2j+1) -> outputs j and
 *     qk_rope/2 + j:
 *        out[nope+j]      = a_j cos[t,j]        - b_j sin[t,j]
 *        out[nope+half+j] = b_j cos[t,half+j]   + a_j sin[t,half+j]
 *     then MXFP8 (E4M3, blocks of 32, E8M0 scales, norm_const 1) along
 *     head_dim (row) and along tokens (column).
 *
 *  x    (tokens, q_lora) row-major: bf16 (in_dtype BF16) or E4M3 codes
 *       (in_dtype E4M3, the page's MXFP8-input path)
 *  w    w_out_in = 1: (num_heads*head_dim, q_lora) [out, in], same dtype
 *       as x.  w_out_in = 0: (q_lora, num_heads*head_dim) [in, out], the
 *       page's default layout; with E4M3 inputs it needs q_lora <= 2048
 *       (else UNSUPPORTED).  Both layouts give identical results.
 *  x_scale  (tokens, q_lora/32) E8M0, row-major: byte (t, b) scales
 *           x[t, 32b .. 32b+31]                      (E4M3 inputs only)
 *  w_scale  E8M0, following w's layout ("GEMM + RoPE + MXFP8 Projection
 *           (SM100)", Shapes): (num_heads*head_dim, q_lora/32) when
 *           w_out_in = 1, (q_lora/32, num_heads*head_dim) when w_out_in = 0;
 *           byte (o, b) scales w[o, 32b .. 32b+31]   (E4M3 inputs only)
 *           The MXFP8 path contracts x[t,i]*2^(x_scale-127) with
 *           w[o,i]*2^(w_scale-127) in fp32; both must be NULL for BF16.
 *  cos, sin  (tokens, qk_rope) bf16
 *  out_fp8_row, out_fp8_col   (tokens, num_heads, head_dim) E4M3 codes
 *  out_scales_row             (tokens, num_heads, head_dim/32) E8M0
 *  out_scales_col             (tokens/32, num_heads, head_dim) E8M0
 *  Sizes: tokens % 128 == 0, q_lora % 32 == 0 (BF16) or % 128 == 0
 *  (E4M3), head_dim == 192, qk_rope == 64.  E4M3 inputs need 4-byte
 *  aligned x_scale/w_scale.  Violations return SHAPE / UNSUPPORTED / ALIGN
 *  before anything is enqueued.
 */
int gemm_proj_rope_mxfp8(const void *x, const void *w, const uint8_t *x_scale,
                         const uint8_t *w_scale, const void *cos, const void *sin,
                         uint8_t *out_fp8_row, uint8_t *out_scales_row,
                         uint8_t *out_fp8_col, uint8_t *out_scales_col,
                         int64_t tokens, int64_t q_lora, int64_t num_heads,
                         int64_t head_dim, int64_t qk_rope, int in_dtype, int w_out_in,
                         void *stream);

/* Host-only argument checks (the pages' check_support()): the same
 * arguments minus the stream; touch no device memory; return the status
 * the launch call would return before enqueueing anything. */
int bsg_validate_gemm_amax(const void *a, const void *b, const uint8_t *sfa,
                           const uint8_t *sfb, void *c, float *amax, int64_t m, int64_t n,
                           int64_t k, int64_t l, int ab_dtype, int c_dtype, int sf_vec_size,
                           int a_major, int b_major, int c_major);
int bsg_validate_grouped_gemm(const void *a, const void *b, const int32_t *padded_offsets,
                              const float *alpha, const float *prob, const void *bias,
                              void *c, void *d, int64_t m, int64_t n, int64_t k,
                              int64_t num_experts, int bias_dtype, int c_dtype, int d_dtype);
int bsg_validate_grouped_gemm_srelu(const void *a, const void *b, const uint8_t *sfa,
                                    const uint8_t *sfb, const int32_t *padded_offsets,
                                    const float *alpha, const float *prob,
                                    const float *norm_const, void *c, void *d, void *d_col,
                                    uint8_t *sfd_row, uint8_t *sfd_col, float *amax,
                                    int64_t m, int64_t n, int64_t k, int64_t num_experts,
                                    int ab_dtype, int c_dtype, int d_dtype, int sf_vec_size,
                                    float tanh_clamp_scale);
int bsg_validate_grouped_gemm_discrete(const void *a, const uint64_t *b_ptrs,
                                       const int32_t *padded_offsets, const float *alpha,
                                       const float *prob, const void *bias, void *c, void *d,
                                       int64_t m, int64_t n, int64_t k, int64_t num_experts,
                                       int bias_dtype, int c_dtype, int d_dtype);
int bsg_validate_grouped_gemm_srelu_discrete(const void *a, const uint64_t *b_ptrs,
                                             const uint8_t *sfa, const uint64_t *sfb_ptrs,
                                             const int32_t *padded_offsets, const float *alpha,
                                             const float *prob, const float *norm_const, void *c,
                                             void *d, void *d_col, uint8_t *sfd_row,
                                             uint8_t *sfd_col, float *amax, int64_t m, int64_t n,
                                             int64_t k, int64_t num_experts, int ab_dtype,
                                             int c_dtype, int d_dtype, int sf_vec_size,
                                             float tanh_clamp_scale);
int bsg_validate_grouped_gemm_dswiglu(const void *a, const void *b, const uint8_t *sfa,
                                      const uint8_t *sfb, const void *c,
                                      const int32_t *padded_offsets, const float *alpha,
                                      const float *beta, const float *prob,
                                      const float *norm_const, void *d_row, void *d_col,
                                      uint8_t *sfd_row, uint8_t *sfd_col, float *dprob,
                                      float *amax, int64_t m, int64_t n, int64_t k,
                                      int64_t num_experts, int ab_dtype, int c_dtype,
                                      int d_dtype, int sf_vec_size, int b_major);
int bsg_validate_gemm_proj_rope_mxfp8(const void *x, const void *w, const uint8_t *x_scale,
                                      const uint8_t *w_scale, const void *cos, const void *sin,
                                      uint8_t *out_fp8_row, uint8_t *out_scales_row,
                                      uint8_t *out_fp8_col, uint8_t *out_scales_col,
                                      int64_t tokens, int64_t q_lora, int64_t num_heads,
                                      int64_t head_dim, int64_t qk_rope, int in_dtype,
                                      int w_out_in);

/* Opt-in debug check of the routing offsets that the grouped entry points
 * take on the device without reading them ("Grouped GEMM + dSwiGLU (SM100)",
 * JAX execution: the offsets are the caller's responsibility).  Copies the
 * num_experts int32 values of padded_offsets (a device pointer) to the host
 * on `stream`, waits for the stream, and checks the contract the kernels
 * assume: every value a multiple of 256 in [0, m], nondecreasing ("Grouped
 * GEMM (SM100 BF16)", Tensors and layouts: each expert's rows padded to 256).
 * Returns BSG_OK, SHAPE naming the first violation (bsg_last_error), or
 * NULLPTR / DEVICE / LAUNCH.  Synchronises the stream: for debugging, not
 * for the hot path. */
int bsg_check_padded_offsets(const int32_t *padded_offsets, int64_t num_experts, int64_t m,
                             void *stream);

/* Static text for a status code. */
const char *bsg_status_string(int status);
/* Thread-local message for the most recent non-zero return on this thread. */
const char *bsg_last_error(void);
/* Library version: major*10000 + minor*100 + patch. */
int bsg_version(void);

#ifdef __cplusplus
}
#endif
#endif /* BSG_H */
