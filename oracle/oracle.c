/*
 * Plain, slow CPU oracle for the block-scaled GEMM family.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load this library.  It shares no code,
 * header, table or helper with the HIP path, and the HIP path never loads it.
 *
 * Everything is decoded exactly and accumulated in fp64; epilogues run in
 * fp64.  The one exception is the MX output quantiser, whose integer
 * decisions (scale byte, code) are taken in fp32 because that is the
 * precision the GPU kernels decide them in (documented per function).
 *
 * Sources (cuDNN frontend "GEMM fusions" documentation pages):
 *   [GA]  "GEMM + Amax (SM100)": Equations; Shapes; Input/Output tensors.
 *   [GS]  "Grouped GEMM + sReLU (SM100)": Equations; Tanh soft clamp;
 *         Shapes (SFD_row / SFD_col atom shapes).
 *   [GD]  "Grouped GEMM + dSwiGLU (SM100)": Steps 1-2 (dSwiGLU backward
 *         epilogue), Step 3 (output quantisation).
 *   [GB]  "Grouped GEMM (SM100 BF16)": Operation; Tensors and layouts.
 *   [PR]  "GEMM + RoPE + MXFP8 Projection (SM100)": Equations; Shapes.
 * Number formats follow the OCP Microscaling (MX) v1.0 definitions of
 * E4M3 ("fn", no infinities), E5M2 (IEEE-like, with Inf and NaN), E2M1 and
 * E8M0.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC oracle.c -o liboracle.so -lm
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Number formats                                                           */
/* ------------------------------------------------------------------------ */

/* E4M3 (fn flavour): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits.
 * Exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no Inf. */
double orc_dec_e4m3(uint32_t code)
{
    uint32_t s = (code >> 7) & 1u, e = (code >> 3) & 15u, m = code & 7u;
    double v;
    if (e == 15u && m == 7u) return NAN;
    if (e == 0u) v = ldexp((double)m / 8.0, -6);
    else v = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return s ? -v : v;
}

/* E5M2: 1 sign, 5 exponent bits (bias 15), 2 mantissa bits, IEEE-like:
 * exponent field 0 is subnormal (m/4 * 2^-14); field 31 is Inf (m = 0) or
 * NaN.  Largest finite magnitude 57344. */
double orc_dec_e5m2(uint32_t code)
{
    uint32_t s = (code >> 7) & 1u, e = (code >> 2) & 31u, m = code & 3u;
    double v;
    if (e == 31u) v = m ? NAN : INFINITY;
    else if (e == 0u) v = ldexp((double)m / 4.0, -14);
    else v = ldexp(1.0 + (double)m / 4.0, (int)e - 15);
    return s ? -v : v;
}

/* E2M1: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent field 0
 * is subnormal (m * 0.5).  Magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}. */
double orc_dec_e2m1(uint32_t nib)
{
    uint32_t s = (nib >> 3) & 1u, e = (nib >> 1) & 3u, m = nib & 1u;
    double v;
    if (e == 0u) v = 0.5 * (double)m;
    else v = ldexp(1.0 + (double)m / 2.0, (int)e - 1);
    return s ? -v : v;
}

/* fp64 -> E2M1 nibble: the nearest of the eight magnitudes (0, 0.5, 1, 1.5,
 * 2, 3, 4, 6), a tie going to the code whose mantissa bit is 0 (round to
 * nearest even); magnitudes past 6 saturate to 6.  Sign in bit 3. */
uint32_t orc_enc_e2m1(double x)
{
    uint32_t s = signbit(x) ? 8u : 0u, best = 0u, c;
    double a = fabs(x), bd = INFINITY;
    if (isnan(x)) return 7u;
    if (a >= 6.0) return s | 7u;
    for (c = 0u; c < 8u; ++c) {
        double dist = fabs(orc_dec_e2m1(c) - a);
        if (dist < bd || (dist == bd && (c & 1u) == 0u)) { bd = dist; best = c; }
    }
    return s | best;
}

/* E8M0: unsigned biased exponent 2^(b-127); 0xFF is NaN. */
double orc_dec_e8m0(uint32_t b)
{
    if ((b & 255u) == 255u) return NAN;
    return ldexp(1.0, (int)(b & 255u) - 127);
}

/* bf16 is the upper half of an IEEE binary32. */
double orc_dec_bf16(uint32_t h)
{
    uint32_t w = (h & 0xFFFFu) << 16;
    float f;
    memcpy(&f, &w, 4);
    return (double)f;
}

/* Round x to the nearest multiple of `step` (a power of two), ties to even. */
static double rne_to_step(double x, double step)
{
    double q = x / step;            /* exact: power-of-two division */
    double fl = floor(q);
    double r = q - fl;
    if (r > 0.5 || (r == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
    return fl * step;
}

/* fp64 -> E4M3 code: round to nearest, ties to even; magnitudes at or above
 * the largest finite value (448) saturate to it; never returns the NaN code.
 * Negative values that round to zero keep the sign bit (0x80). */
uint32_t orc_enc_e4m3(double x)
{
    uint32_t s = signbit(x) ? 0x80u : 0u;
    double a = fabs(x), q;
    int e2;
    if (isnan(x)) return 0x7Fu;
    if (a >= 448.0) return s | 0x7Eu;
    if (a == 0.0) return s;
    frexp(a, &e2);                         /* a in [2^(e2-1), 2^e2) */
    {
        int ulp_exp = e2 - 1 - 3;          /* 3 stored mantissa bits */
        if (ulp_exp < -9) ulp_exp = -9;    /* subnormal spacing 2^-9 */
        q = rne_to_step(a, ldexp(1.0, ulp_exp));
    }
    if (q >= 448.0) return s | 0x7Eu;
    if (q == 0.0) return s;
    if (q < ldexp(1.0, -6)) {              /* subnormal: m * 2^-9 */
        return s | (uint32_t)(q / ldexp(1.0, -9));
    }
    frexp(q, &e2);
    {
        int E = e2 - 1;                    /* q in [2^E, 2^(E+1)) */
        uint32_t m = (uint32_t)((q / ldexp(1.0, E) - 1.0) * 8.0);
        return s | ((uint32_t)(E + 7) << 3) | m;
    }
}

/* fp64 -> E5M2 code, round to nearest even; magnitudes at or above the
 * largest finite value (57344) saturate to it; never returns Inf or NaN. */
uint32_t orc_enc_e5m2(double x)
{
    uint32_t s = signbit(x) ? 0x80u : 0u;
    double a = fabs(x), q;
    int e2;
    if (isnan(x)) return 0x7Fu;
    if (a >= 57344.0) return s | 0x7Bu;
    if (a == 0.0) return s;
    frexp(a, &e2);
    {
        int ulp_exp = e2 - 1 - 2;          /* 2 stored mantissa bits */
        if (ulp_exp < -16) ulp_exp = -16;  /* subnormal spacing 2^-16 */
        q = rne_to_step(a, ldexp(1.0, ulp_exp));
    }
    if (q >= 57344.0) return s | 0x7Bu;
    if (q == 0.0) return s;
    if (q < ldexp(1.0, -14)) return s | (uint32_t)(q / ldexp(1.0, -16));   /* subnormal */
    frexp(q, &e2);
    {
        int E = e2 - 1;
        uint32_t m = (uint32_t)((q / ldexp(1.0, E) - 1.0) * 4.0);
        return s | ((uint32_t)(E + 15) << 2) | m;
    }
}

/* fp64 -> bf16 bits with a single round-to-nearest-even step. */
uint32_t orc_rne_bf16(double x)
{
    double a = fabs(x), q;
    int e2, ulp_exp;
    float f;
    uint32_t w;
    if (isnan(x)) return 0x7FC0u;
    if (a == 0.0) q = 0.0;
    else {
        frexp(a, &e2);
        ulp_exp = e2 - 1 - 7;              /* 7 stored mantissa bits */
        if (ulp_exp < -133) ulp_exp = -133;
        q = rne_to_step(a, ldexp(1.0, ulp_exp));
    }
    if (q >= ldexp(1.0, 128)) q = INFINITY;
    f = (float)(signbit(x) ? -q : q);      /* exact: q has <= 8 significant bits */
    memcpy(&w, &f, 4);
    return w >> 16;
}

void orc_rne_bf16_array(const double *x, uint16_t *out, int64_t n)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = (uint16_t)orc_rne_bf16(x[i]);
}

/* E8M0 byte of the smallest power of two >= sigma, clamped to [0, 254];
 * sigma <= 0 gives 0.  (Rounding of a computed scale: see the quantiser.) */
uint32_t orc_e8m0_ceil(double sigma)
{
    int e2, E;
    double f;
    if (!(sigma > 0.0)) return 0u;
    f = frexp(sigma, &e2);                 /* sigma = f * 2^e2, f in [0.5,1) */
    E = (f == 0.5) ? e2 - 1 : e2;
    E += 127;
    if (E < 0) E = 0;
    if (E > 254) E = 254;
    return (uint32_t)E;
}

/* ------------------------------------------------------------------------ */
/* Scale-factor atom addressing                                             */
/* ------------------------------------------------------------------------ */
/* [GA] Shapes / "Using JAX arrays": the logical scale tensor has shape
 * (32, 4, ceil(MN/128), 4, ceil(K/(4*sf)), L) and is the C-contiguous
 * physical buffer (L, ceil(MN/128), ceil(K/(4*sf)), 32, 4, 4) permuted by
 * (3,4,1,5,2,0).  Reading the hierarchical row mode (32,4,MN') first-mode
 * fastest, row r = 128*mt + 32*r4 + r32 and k-block kb = 4*kt + k4, so the
 * byte sits at physical index (l, mt, kt, r32, r4, k4). */
int64_t orc_sf_offset(int64_t r, int64_t kb, int64_t l, int64_t mn, int64_t kblocks)
{
    int64_t mt_n = (mn + 127) / 128;
    int64_t kt_n = (kblocks + 3) / 4;
    int64_t mt = r / 128, r4 = (r % 128) / 32, r32 = r % 32;
    int64_t kt = kb / 4, k4 = kb % 4;
    return ((((l * mt_n + mt) * kt_n + kt) * 32 + r32) * 4 + r4) * 4 + k4;
}

/* Offsets of rows [r0, r1) x k-blocks [0, nkb) of batch l, row-major. */
void orc_sf_offset_grid(int64_t r0, int64_t r1, int64_t nkb, int64_t l, int64_t mn,
                        int64_t kblocks, int64_t *out)
{
    for (int64_t r = r0; r < r1; ++r)
        for (int64_t kb = 0; kb < nkb; ++kb)
            out[(r - r0) * nkb + kb] = orc_sf_offset(r, kb, l, mn, kblocks);
}

/* ------------------------------------------------------------------------ */
/* Dequantisation ([GA] Equations: A_hat = dequantize(A, SFA, sf_vec_size)) */
/* ------------------------------------------------------------------------ */
/* fmt 0: one E4M3 code per byte.  fmt 1: E2M1, two per byte, element 2j in
 * the low nibble and 2j+1 in the high nibble.  fmt 2: one E5M2 code per byte. */
static double code_value(const uint8_t *row, int fmt, int64_t kk)
{
    if (fmt == 0) return orc_dec_e4m3(row[kk]);
    if (fmt == 2) return orc_dec_e5m2(row[kk]);
    {
        uint8_t byte = row[kk >> 1];
        return orc_dec_e2m1((kk & 1) ? (byte >> 4) : (byte & 15u));
    }
}

/* Row r of matrix `l` of an (MN, K) operand, dequantised into out[0..K). */
static void dequant_row(const uint8_t *codes, const uint8_t *sf, int fmt,
                        int64_t r, int64_t l, int64_t mn, int64_t k, double *out)
{
    int64_t rowbytes = fmt == 1 ? k / 2 : k;
    int64_t kblocks = (k + 31) / 32;
    const uint8_t *row = codes + (l * mn + r) * rowbytes;
    for (int64_t kk = 0; kk < k; ++kk) {
        double scale = orc_dec_e8m0(sf[orc_sf_offset(r, kk / 32, l, mn, kblocks)]);
        out[kk] = code_value(row, fmt, kk) * scale;
    }
}

/* acc = sum_k a[k]*b[k]; sabs = sum_k |a[k]*b[k]| */
static void dot(const double *a, const double *b, int64_t k, double *acc, double *sabs)
{
    double s = 0.0, t = 0.0;
    for (int64_t kk = 0; kk < k; ++kk) {
        double p = a[kk] * b[kk];
        s += p;
        t += fabs(p);
    }
    *acc = s;
    *sabs = t;
}

/* Error-bound statistic (not part of the result): sum over 32-wide K blocks
 * of the block's largest |a[k]*b[k]|. */
static double block_max_sum(const double *a, const double *b, int64_t k)
{
    double t = 0.0;
    for (int64_t k0 = 0; k0 < k; k0 += 32) {
        double mx = 0.0;
        for (int64_t kk = k0; kk < k0 + 32 && kk < k; ++kk) {
            double p = fabs(a[kk] * b[kk]);
            if (p > mx) mx = p;
        }
        t += mx;
    }
    return t;
}

/* Dequantise all N rows of B for batch/expert l: out is (N, K). */
static void dequant_matrix(const uint8_t *codes, const uint8_t *sf, int fmt,
                           int64_t l, int64_t rows, int64_t k, double *out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        dequant_row(codes, sf, fmt, r, l, rows, k, out + r * k);
}

/* ------------------------------------------------------------------------ */
/* [GA] C[m,n,l] = sum_k A_hat[m,k,l] * B_hat[n,k,l]                        */
/* ------------------------------------------------------------------------ */
/* Rows [r0, r1) of batch `batch`.  c and sabs (nullable) are (r1-r0, n). */
int orc_gemm_amax(const uint8_t *a, const uint8_t *b, const uint8_t *sfa, const uint8_t *sfb,
                  int64_t m, int64_t n, int64_t k, int64_t l, int fmt,
                  int64_t batch, int64_t r0, int64_t r1, double *c, double *sabs, double *bmax)
{
    double *bh, *ah;
    if (batch < 0 || batch >= l || r0 < 0 || r1 > m || r0 > r1) return 1;
    if (fmt == 1 && (k % 2)) return 2;
    bh = (double *)malloc(sizeof(double) * (size_t)(n * k));
    ah = (double *)malloc(sizeof(double) * (size_t)((r1 - r0) * k));
    if (!bh || !ah) { free(bh); free(ah); return 3; }
    dequant_matrix(b, sfb, fmt, batch, n, k, bh);
    #pragma omp parallel for schedule(static)
    for (int64_t i = r0; i < r1; ++i)
        dequant_row(a, sfa, fmt, i, batch, m, k, ah + (i - r0) * k);
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = r0; i < r1; ++i)
        for (int64_t j = 0; j < n; ++j) {
            double acc, t;
            dot(ah + (i - r0) * k, bh + j * k, k, &acc, &t);
            c[(i - r0) * n + j] = acc;
            if (sabs) sabs[(i - r0) * n + j] = t;
            if (bmax) bmax[(i - r0) * n + j] = block_max_sum(ah + (i - r0) * k, bh + j * k, k);
        }
    free(bh);
    free(ah);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Expert routing ([GB] Operation: rows [begin_g, padded_offsets[g]) with   */
/* begin_0 = 0 and begin_g = padded_offsets[g-1])                           */
/* ------------------------------------------------------------------------ */
/* The unique g whose range holds row r, or -1 when r >= padded_offsets[L-1].
 * Empty ranges (begin_g == end_g) hold no row. */
int32_t orc_expert_of_row(const int32_t *offsets, int64_t L, int64_t r)
{
    int64_t begin = 0;
    for (int64_t g = 0; g < L; ++g) {
        int64_t end = offsets[g];
        if (begin <= r && r < end) return (int32_t)g;
        begin = end;
    }
    return -1;
}

/* ------------------------------------------------------------------------ */
/* [GS] Equations and "Tanh soft clamp":                                    */
/*   C = alpha_g * sum_k A_hat * B_hat_g                                    */
/*   D = prob[m] * relu(C)^2                       (s <= 0: no clamp)       */
/*   D = prob[m] * (s * min(1, tanh(relu(C)/s)))^2 (s > 0; t capped at 1)   */
/* ------------------------------------------------------------------------ */
int orc_grouped_srelu(const uint8_t *a, const uint8_t *b, const uint8_t *sfa, const uint8_t *sfb,
                      const int32_t *offsets, const float *alpha, const float *prob,
                      int64_t m, int64_t n, int64_t k, int64_t L, int fmt, double s,
                      int64_t r0, int64_t r1,
                      double *c_out, double *d_out, double *sabs_out, int32_t *group_out,
                      double *bmax_out)
{
    double *bh = NULL, *ah;
    int64_t rows = r1 - r0, have = -1;
    if (r0 < 0 || r1 > m || r0 > r1) return 1;
    if (fmt == 1 && (k % 2)) return 2;
    ah = (double *)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1) * (size_t)(rows > 0 ? rows : 1));
    bh = (double *)malloc(sizeof(double) * (size_t)(n * k > 0 ? n * k : 1));
    if (!ah || !bh) { free(ah); free(bh); return 3; }
    for (int64_t i = r0; i < r1; ++i) group_out[i - r0] = orc_expert_of_row(offsets, L, i);
    #pragma omp parallel for schedule(static)
    for (int64_t i = r0; i < r1; ++i)
        dequant_row(a, sfa, fmt, i, 0, m, k, ah + (i - r0) * k);
    for (int64_t i = r0; i < r1; ++i) {
        int64_t g = group_out[i - r0];
        if (g < 0) {
            for (int64_t j = 0; j < n; ++j) {
                c_out[(i - r0) * n + j] = NAN;
                d_out[(i - r0) * n + j] = NAN;
                if (sabs_out) sabs_out[(i - r0) * n + j] = NAN;
                if (bmax_out) bmax_out[(i - r0) * n + j] = NAN;
            }
            continue;
        }
        if (g != have) { dequant_matrix(b, sfb, fmt, g, n, k, bh); have = g; }
        #pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < n; ++j) {
            double acc, t, cval, x;
            dot(ah + (i - r0) * k, bh + j * k, k, &acc, &t);
            cval = (double)alpha[g] * acc;
            x = cval > 0.0 ? cval : 0.0;
            if (s > 0.0) {
                double th = tanh(x / s);
                if (th > 1.0) th = 1.0;
                x = s * th;
            }
            c_out[(i - r0) * n + j] = cval;
            d_out[(i - r0) * n + j] = (double)prob[i] * x * x;
            if (sabs_out) sabs_out[(i - r0) * n + j] = fabs((double)alpha[g]) * t;
            if (bmax_out)
                bmax_out[(i - r0) * n + j] =
                    fabs((double)alpha[g]) * block_max_sum(ah + (i - r0) * k, bh + j * k, k);
        }
    }
    free(ah);
    free(bh);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* [GD] Step 1 and Step 2 (grouped GEMM + dSwiGLU backward epilogue):       */
/*   ref[m,n] = alpha_g^2 * sum_k dequant(A)[m,k] * dequant(B)[n,k,g]        */
/*   C (rows, 2N) holds 32-column blocks in pairs: columns [64b, 64b+32)    */
/*   are the input and [64b+32, 64b+64) the gate of ref columns             */
/*   [32b, 32b+32); both are scaled by beta_g.                              */
/*   swish = gate * sigmoid(gate)                                           */
/*   ab    = ref * prob * swish                                             */
/*   dsw   = ref * prob * input * sigmoid(gate) * (1 + gate*(1 - sigmoid))  */
/*   D has the same pairing: ab in [64b, 64b+32), dsw in [64b+32, 64b+64).  */
/*   dprob[m] = sum_n swish * input * ref                                   */
/* C is bf16 (bits).  Rows [r0, r1); ref_out (rows, N), d_out (rows, 2N),    */
/* dprob_out (rows); sabs_out / bmax_out (rows, N, nullable) carry          */
/* |alpha_g|^2 * sum|products| and the block-max sum of the GEMM.           */
/* ------------------------------------------------------------------------ */
int orc_grouped_dswiglu(const uint8_t *a, const uint8_t *b, const uint8_t *sfa, const uint8_t *sfb,
                        const int32_t *offsets, const float *alpha, const float *beta,
                        const float *prob, const uint16_t *c, int64_t m, int64_t n, int64_t k,
                        int64_t L, int fmt, int64_t r0, int64_t r1, double *ref_out, double *d_out,
                        double *dprob_out, double *sabs_out, double *bmax_out)
{
    double *bh = NULL, *ah;
    int64_t rows = r1 - r0, have = -1;
    if (r0 < 0 || r1 > m || r0 > r1 || n % 32) return 1;
    if (fmt == 1 && (k % 2)) return 2;
    ah = (double *)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1) * (size_t)(rows > 0 ? rows : 1));
    bh = (double *)malloc(sizeof(double) * (size_t)(n * k > 0 ? n * k : 1));
    if (!ah || !bh) { free(ah); free(bh); return 3; }
    #pragma omp parallel for schedule(static)
    for (int64_t i = r0; i < r1; ++i)
        dequant_row(a, sfa, fmt, i, 0, m, k, ah + (i - r0) * k);
    for (int64_t i = r0; i < r1; ++i) {
        int64_t g = orc_expert_of_row(offsets, L, i);
        double a2, bt, pr, dp = 0.0;
        if (g < 0) {
            for (int64_t j = 0; j < n; ++j) ref_out[(i - r0) * n + j] = NAN;
            for (int64_t j = 0; j < 2 * n; ++j) d_out[(i - r0) * 2 * n + j] = NAN;
            dprob_out[i - r0] = NAN;
            continue;
        }
        if (g != have) { dequant_matrix(b, sfb, fmt, g, n, k, bh); have = g; }
        a2 = (double)alpha[g] * (double)alpha[g];
        bt = (double)beta[g];
        pr = (double)prob[i];
        #pragma omp parallel for schedule(static) reduction(+ : dp)
        for (int64_t j = 0; j < n; ++j) {
            double acc, t, ref, in, gt, sg, sw;
            int64_t cin = 64 * (j / 32) + j % 32, cgt = cin + 32;
            dot(ah + (i - r0) * k, bh + j * k, k, &acc, &t);
            ref = a2 * acc;
            in = bt * orc_dec_bf16(c[i * 2 * n + cin]);
            gt = bt * orc_dec_bf16(c[i * 2 * n + cgt]);
            sg = 1.0 / (1.0 + exp(-gt));
            sw = gt * sg;
            ref_out[(i - r0) * n + j] = ref;
            d_out[(i - r0) * 2 * n + cin] = ref * pr * sw;
            d_out[(i - r0) * 2 * n + cgt] = ref * pr * in * sg * (1.0 + gt * (1.0 - sg));
            dp += sw * in * ref;
            if (sabs_out) sabs_out[(i - r0) * n + j] = a2 * t;
            if (bmax_out) bmax_out[(i - r0) * n + j] = a2 * block_max_sum(ah + (i - r0) * k, bh + j * k, k);
        }
        dprob_out[i - r0] = dp;
    }
    free(ah);
    free(bh);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* [GB] Operation:                                                          */
/*   G = alpha[g] * A_g @ B_g^T                                             */
/*   with bias:    C = G + prob * bias[:, g],  D = C                        */
/*   without bias: C = G,                      D = prob * G                 */
/* A (M,K) bf16; B stored [L][N][K] bf16; bias (N,L) stride (1,N) given     */
/* here already widened to fp64, memory [L][N].                             */
/* ------------------------------------------------------------------------ */
int orc_grouped_bf16(const uint16_t *a, const uint16_t *b, const int32_t *offsets,
                     const float *alpha, const float *prob, const double *bias,
                     int64_t m, int64_t n, int64_t k, int64_t L, int64_t r0, int64_t r1,
                     double *c_out, double *d_out, double *sabs_out, int32_t *group_out)
{
    double *bh, *ah;
    int64_t have = -1, rows = r1 - r0;
    if (r0 < 0 || r1 > m || r0 > r1) return 1;
    ah = (double *)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1) * (size_t)(rows > 0 ? rows : 1));
    bh = (double *)malloc(sizeof(double) * (size_t)(n * k > 0 ? n * k : 1));
    if (!ah || !bh) { free(ah); free(bh); return 3; }
    for (int64_t i = r0; i < r1; ++i) {
        group_out[i - r0] = orc_expert_of_row(offsets, L, i);
        for (int64_t kk = 0; kk < k; ++kk)
            ah[(i - r0) * k + kk] = orc_dec_bf16(a[i * k + kk]);
    }
    for (int64_t i = r0; i < r1; ++i) {
        int64_t g = group_out[i - r0];
        if (g < 0) {
            for (int64_t j = 0; j < n; ++j) {
                c_out[(i - r0) * n + j] = NAN;
                d_out[(i - r0) * n + j] = NAN;
                if (sabs_out) sabs_out[(i - r0) * n + j] = NAN;
            }
            continue;
        }
        if (g != have) {
            #pragma omp parallel for schedule(static)
            for (int64_t j = 0; j < n; ++j)
                for (int64_t kk = 0; kk < k; ++kk)
                    bh[j * k + kk] = orc_dec_bf16(b[(g * n + j) * k + kk]);
            have = g;
        }
        #pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < n; ++j) {
            double acc, t, G;
            dot(ah + (i - r0) * k, bh + j * k, k, &acc, &t);
            G = (double)alpha[g] * acc;
            if (bias) {
                double cval = G + (double)prob[i] * bias[g * n + j];
                c_out[(i - r0) * n + j] = cval;
                d_out[(i - r0) * n + j] = cval;
            } else {
                c_out[(i - r0) * n + j] = G;
                d_out[(i - r0) * n + j] = (double)prob[i] * G;
            }
            if (sabs_out) sabs_out[(i - r0) * n + j] = fabs((double)alpha[g]) * t;
        }
    }
    free(ah);
    free(bh);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* [PR] Equations: Y = x W reshaped to [tokens, heads, head_dim]; the        */
/* trailing qk_rope features of each head get the interleaved-in /          */
/* halves-out rotary embedding:                                             */
/*   a_j = Y[.., nope + 2j],  b_j = Y[.., nope + 2j + 1],  j < qk_rope/2      */
/*   out[nope + j]        = a_j cos[t, j]        - b_j sin[t, j]            */
/*   out[nope + half + j] = b_j cos[t, half + j] + a_j sin[t, half + j]     */
/* proj_rope_rows takes x rows [t0, t1) as xr (rows x q_lora) and the weight */
/* as wt [out][in], both already decoded to fp64, and frees them.           */
/* y_out and sabs_out (nullable) are (t1-t0, heads*head_dim).               */
/* ------------------------------------------------------------------------ */
static int proj_rope_rows(double *xr, double *wt, const uint16_t *cosv, const uint16_t *sinv,
                          int64_t q_lora, int64_t heads, int64_t head_dim, int64_t qk_rope,
                          int64_t t0, int64_t t1, double *y_out, double *sabs_out)
{
    int64_t nout = heads * head_dim, nope = head_dim - qk_rope, half = qk_rope / 2;
    int64_t rows = t1 - t0;
    double *yr = (double *)malloc(sizeof(double) * (size_t)(nout * (rows > 0 ? rows : 1)));
    double *sr = (double *)malloc(sizeof(double) * (size_t)(nout * (rows > 0 ? rows : 1)));
    if (!yr || !sr) { free(wt); free(xr); free(yr); free(sr); return 3; }
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t t = t0; t < t1; ++t)
        for (int64_t o = 0; o < nout; ++o) {
            double acc, s;
            dot(xr + (t - t0) * q_lora, wt + o * q_lora, q_lora, &acc, &s);
            yr[(t - t0) * nout + o] = acc;
            sr[(t - t0) * nout + o] = s;
        }
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t t = t0; t < t1; ++t)
        for (int64_t h = 0; h < heads; ++h) {
            const double *y = yr + (t - t0) * nout + h * head_dim;
            const double *sy = sr + (t - t0) * nout + h * head_dim;
            double *out = y_out + (t - t0) * nout + h * head_dim;
            double *so = sabs_out ? sabs_out + (t - t0) * nout + h * head_dim : NULL;
            for (int64_t d = 0; d < nope; ++d) {
                out[d] = y[d];
                if (so) so[d] = sy[d];
            }
            for (int64_t j = 0; j < half; ++j) {
                double av = y[nope + 2 * j], bv = y[nope + 2 * j + 1];
                double c0 = orc_dec_bf16(cosv[t * qk_rope + j]);
                double s0 = orc_dec_bf16(sinv[t * qk_rope + j]);
                double c1 = orc_dec_bf16(cosv[t * qk_rope + half + j]);
                double s1 = orc_dec_bf16(sinv[t * qk_rope + half + j]);
                out[nope + j] = av * c0 - bv * s0;
                out[nope + half + j] = bv * c1 + av * s1;
                if (so) {
                    double sa = sy[nope + 2 * j], sb = sy[nope + 2 * j + 1];
                    so[nope + j] = sa * fabs(c0) + sb * fabs(s0);
                    so[nope + half + j] = sb * fabs(c1) + sa * fabs(s1);
                }
            }
        }
    free(wt);
    free(xr);
    free(yr);
    free(sr);
    return 0;
}

/* [PR] BF16 inputs.  w_out_in = 1: w is [out, in]; 0: w is [in, out].      */
int orc_proj_rope(const uint16_t *x, const uint16_t *w, const uint16_t *cosv, const uint16_t *sinv,
                  int64_t tokens, int64_t q_lora, int64_t heads, int64_t head_dim,
                  int64_t qk_rope, int w_out_in, int64_t t0, int64_t t1,
                  double *y_out, double *sabs_out)
{
    int64_t nout = heads * head_dim, rows = t1 - t0;
    double *wt, *xr;
    if (t0 < 0 || t1 > tokens || t0 > t1 || qk_rope % 2 || qk_rope > head_dim) return 1;
    wt = (double *)malloc(sizeof(double) * (size_t)(nout * q_lora));
    xr = (double *)malloc(sizeof(double) * (size_t)(q_lora * (rows > 0 ? rows : 1)));
    if (!wt || !xr) { free(wt); free(xr); return 3; }
    /* weight as [out][in] */
    #pragma omp parallel for schedule(static)
    for (int64_t o = 0; o < nout; ++o)
        for (int64_t i = 0; i < q_lora; ++i)
            wt[o * q_lora + i] = orc_dec_bf16(w_out_in ? w[o * q_lora + i] : w[i * nout + o]);
    for (int64_t t = t0; t < t1; ++t)
        for (int64_t i = 0; i < q_lora; ++i)
            xr[(t - t0) * q_lora + i] = orc_dec_bf16(x[t * q_lora + i]);
    return proj_rope_rows(xr, wt, cosv, sinv, q_lora, heads, head_dim, qk_rope, t0, t1, y_out, sabs_out);
}

/* [PR] MXFP8 inputs (Shapes: x_scale (tokens, Q_LORA/BLOCK), w_scale       */
/* (heads*head_dim, Q_LORA/BLOCK) for the [out, in] weight; E8M0 row-wise    */
/* block scales, BLOCK = 32):                                               */
/*   x^[t, i] = dec_e4m3(x[t, i]) * dec_e8m0(x_scale[t, i / 32])            */
/*   w^[o, i] = dec_e4m3(w[o, i]) * dec_e8m0(w_scale[o, i / 32])            */
/* then the same projection and rotary embedding as the BF16 inputs.        */
int orc_proj_rope_mx(const uint8_t *x, const uint8_t *x_scale, const uint8_t *w,
                     const uint8_t *w_scale, const uint16_t *cosv, const uint16_t *sinv,
                     int64_t tokens, int64_t q_lora, int64_t heads, int64_t head_dim,
                     int64_t qk_rope, int64_t t0, int64_t t1, double *y_out, double *sabs_out)
{
    int64_t nout = heads * head_dim, rows = t1 - t0, nb = q_lora / 32;
    double *wt, *xr;
    if (t0 < 0 || t1 > tokens || t0 > t1 || qk_rope % 2 || qk_rope > head_dim || q_lora % 32) return 1;
    wt = (double *)malloc(sizeof(double) * (size_t)(nout * q_lora));
    xr = (double *)malloc(sizeof(double) * (size_t)(q_lora * (rows > 0 ? rows : 1)));
    if (!wt || !xr) { free(wt); free(xr); return 3; }
    #pragma omp parallel for schedule(static)
    for (int64_t o = 0; o < nout; ++o)
        for (int64_t i = 0; i < q_lora; ++i)
            wt[o * q_lora + i] = orc_dec_e4m3(w[o * q_lora + i]) * orc_dec_e8m0(w_scale[o * nb + i / 32]);
    for (int64_t t = t0; t < t1; ++t)
        for (int64_t i = 0; i < q_lora; ++i)
            xr[(t - t0) * q_lora + i] = orc_dec_e4m3(x[t * q_lora + i]) * orc_dec_e8m0(x_scale[t * nb + i / 32]);
    return proj_rope_rows(xr, wt, cosv, sinv, q_lora, heads, head_dim, qk_rope, t0, t1, y_out, sabs_out);
}

/* ------------------------------------------------------------------------ */
/* MX output quantiser ([GD] Step 3):                                       */
/*   SFD = norm_const * max_{k in block} |D| * rcp_max                      */
/*   D_q = D * norm_const / SFD                                             */
/* with rcp_max = 1/448 for E4M3 (1/57344 for E5M2, 1/6 for E2M1) and     */
/* blocks of 32 consecutive elements.                                       */
/* SFD is stored as E8M0: the smallest power of two >= the computed value   */
/* (so |D_q| <= 448 needs no clipping); codes are E4M3 by round to nearest  */
/* even, saturating.  The decisions are taken in binary32, in this order:   */
/*   v     = fp32(D)                                                         */
/*   amax  = max |v|                                                         */
/*   sigma = fp32(fp32(norm_const * amax) * fp32(1/448))                    */
/*   byte  = e8m0_ceil(sigma)                                               */
/*   inv   = min(norm_const * 2^(127 - byte), FLT_MAX)  (power-of-two step) */
/*   code  = e4m3_rne_sat(fp32(v * inv))                                    */
/* ------------------------------------------------------------------------ */
static void quant_block(const double *d, int64_t cnt, int64_t stride, float norm_const, int fmt,
                        uint8_t *codes, int64_t cstride, uint8_t *scale)
{
    float amax = 0.0f, sigma, inv;
    uint32_t byte;
    const float rcp_max = fmt == 2 ? 1.0f / 57344.0f : (fmt == 1 ? 1.0f / 6.0f : 1.0f / 448.0f);
    for (int64_t i = 0; i < cnt; ++i) {
        float v = fabsf((float)d[i * stride]);
        if (v > amax) amax = v;
    }
    sigma = (norm_const * amax) * rcp_max;
    byte = orc_e8m0_ceil((double)sigma);
    inv = ldexpf(norm_const, 127 - (int)byte);
    if (inv > FLT_MAX) inv = FLT_MAX;     /* tiny blocks with a large norm_const */
    for (int64_t i = 0; i < cnt; ++i) {
        float v = (float)d[i * stride];
        float y = v * inv;
        codes[i * cstride] = (uint8_t)(fmt == 2 ? orc_enc_e5m2((double)y)
                                                : (fmt == 1 ? orc_enc_e2m1((double)y) : orc_enc_e4m3((double)y)));
    }
    *scale = (uint8_t)byte;
}

/* Row direction: blocks of 32 along each row.  d is (rows, cols) with
 * leading dimension ld; codes (rows, cols); scales (rows, ceil(cols/32)). */
/* fmt 0: E4M3 codes; fmt 1: E2M1 codes (one nibble per byte); fmt 2: E5M2. */
void orc_mx_quant_rows(const double *d, int64_t rows, int64_t cols, int64_t ld,
                       float norm_const, int fmt, uint8_t *codes, uint8_t *scales)
{
    int64_t nb = (cols + 31) / 32;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            int64_t c0 = b * 32, cnt = cols - c0 < 32 ? cols - c0 : 32;
            quant_block(d + r * ld + c0, cnt, 1, norm_const, fmt, codes + r * cols + c0, 1,
                        scales + r * nb + b);
        }
}

/* Column direction: blocks of 32 consecutive rows in each column.
 * codes (rows, cols); scales (ceil(rows/32), cols). */
void orc_mx_quant_cols(const double *d, int64_t rows, int64_t cols, int64_t ld,
                       float norm_const, int fmt, uint8_t *codes, uint8_t *scales)
{
    int64_t nb = (rows + 31) / 32;
    #pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; ++c)
        for (int64_t b = 0; b < nb; ++b) {
            int64_t r0 = b * 32, cnt = rows - r0 < 32 ? rows - r0 : 32;
            quant_block(d + r0 * ld + c, cnt, ld, norm_const, fmt, codes + r0 * cols + c, cols,
                        scales + b * cols + c);
        }
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the following calls (n <= 0: leave as is); the baseline
 * timings use it to time one thread. */
void orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
