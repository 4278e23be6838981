/*
 * nf4_oracle.c -- plain, slow CPU oracle for the QLoRA NF4 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or constant with the
 * GPU library.
 *
 * Sources (page title, section):
 *   [BQ]  "Block-wise quantization in one page"   (zerotofrontier.app "sft/peft")
 *   [NF]  "NF4, derived from normal quantiles"     (same page)
 *   [DQ]  "Double quantization"                    (same page)
 *   [E2E] "Paged optimizers, and QLoRA end to end" (same page)
 *   [RW]  "The real way"                           (same page)
 *   [PT]  "Putting it together", forward formula   (prism.theerrors.in QLoRA explainer)
 *   AdamW: Kingma & Ba (2015) Algorithm 1 with Loshchilov & Hutter (2019)
 *          decoupled weight decay; the pages give only the paging and the rates
 *
 * Arithmetic conventions: fp32 operations are IEEE round-to-nearest-even,
 * compiled with -ffp-contract=off so that no multiply-add is silently fused.
 * Reductions that feed a floating-point result are done in float64.
 *
 * Readings where the pages are silent (all listed in the design notes):
 *   - level order ascending, code 0 = -1, code 7 = 0, code 15 = +1
 *   - x = fp32(w / c) by IEEE division; code = number of midpoints m_j with
 *     x > m_j (a value exactly on a midpoint takes the lower level)
 *   - zero block (c == 0): every code is 7 and the stored constant is 0
 *   - packing: element 2i in the low nibble of byte i, 2i+1 in the high
 *     nibble; an odd tail leaves the final high nibble 0
 *   - the "8-bit floats" of double quantization are OCP FP8 E4M3 (bias 7,
 *     max 448, no infinities) applied to s*448, s = (c1 - mean)/c2
 *   - one mean per tensor, summed in float64 by an aligned pairwise tree
 *
 * Parity of the codebook with the paper's printed appendix table is unpinned
 * (the table is not on the pages); so is bit parity of the 8-bit constant
 * format with the original implementation (the pages do not name it).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Inverse normal CDF: Wichura, "Algorithm AS 241: The percentage points of  */
/* the normal distribution", Applied Statistics 37 (1988), routine PPND16.   */
/* ------------------------------------------------------------------------ */
double orc_norm_ppf(double p)
{
    const double q = p - 0.5;
    if (fabs(q) <= 0.425) {
        const double r = 0.180625 - q * q;
        const double num =
            (((((((2.5090809287301226727e+3 * r + 3.3430575583588128105e+4) * r +
                  6.7265770927008700853e+4) * r + 4.5921953931549871457e+4) * r +
                1.3731693765509461125e+4) * r + 1.9715909503065514427e+3) * r +
              1.3314166789178437745e+2) * r + 3.3871328727963666080e+0);
        const double den =
            (((((((5.2264952788528545610e+3 * r + 2.8729085735721942674e+4) * r +
                  3.9307895800092710610e+4) * r + 2.1213794301586595867e+4) * r +
                5.3941960214247511077e+3) * r + 6.8718700749205790830e+2) * r +
              4.2313330701600911252e+1) * r + 1.0);
        return q * num / den;
    }
    double r = (q < 0.0) ? p : 1.0 - p;
    r = sqrt(-log(r));
    double val;
    if (r <= 5.0) {
        r -= 1.6;
        const double num =
            (((((((7.74545014278341407640e-4 * r + 2.27238449892691845833e-2) * r +
                  2.41780725177450611770e-1) * r + 1.27045825245236838258e+0) * r +
                3.64784832476320460504e+0) * r + 5.76949722146069140550e+0) * r +
              4.63033784615654529590e+0) * r + 1.42343711074968357734e+0);
        const double den =
            (((((((1.05075007164441684324e-9 * r + 5.47593808499534494600e-4) * r +
                  1.51986665636164571966e-2) * r + 1.48103976427480074590e-1) * r +
                6.89767334985100004550e-1) * r + 1.67638483018380384940e+0) * r +
              2.05319162663775882187e+0) * r + 1.0);
        val = num / den;
    } else {
        r -= 5.0;
        const double num =
            (((((((2.01033439929228813265e-7 * r + 2.71155556874348757815e-5) * r +
                  1.24266094738807843860e-3) * r + 2.65321895265761230930e-2) * r +
                2.96560571828504891230e-1) * r + 1.78482653991729133580e+0) * r +
              5.46378491116411436990e+0) * r + 6.65790464350110377720e+0);
        const double den =
            (((((((2.04426310338993978564e-15 * r + 1.42151175831644588870e-7) * r +
                  1.84631831751005468180e-5) * r + 7.86869131145613259100e-4) * r +
                1.48753612908506148525e-2) * r + 1.36929880922735805310e-1) * r +
              5.99832206555887937690e-1) * r + 1.0);
        val = num / den;
    }
    return (q < 0.0) ? -val : val;
}

/* ------------------------------------------------------------------------ */
/* [NF] NF4 codebook.  Probabilities run from p_max down towards 1/2, with   */
/* p_max the average of 1-1/30 and 1-1/32: 8 evenly spaced quantiles on the  */
/* positive side, 7 on the negative side, an exact zero, and a division by   */
/* the largest magnitude so that the table spans [-1, 1].  Every level is    */
/* computed in float64 and rounded to fp32 once.                             */
/* ------------------------------------------------------------------------ */
void orc_nf4_codebook(float out[16])
{
    const double pmax = ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0)) / 2.0;
    const double top = orc_norm_ppf(pmax);
    double v[16];
    int k = 0;
    /* negative half: 7 levels, probabilities pmax - i*(pmax-1/2)/7, i = 0..6 */
    for (int i = 0; i < 7; ++i)
        v[k++] = -orc_norm_ppf(pmax - (double)i * (pmax - 0.5) / 7.0);
    v[k++] = 0.0;
    /* positive half: 8 levels, probabilities pmax - i*(pmax-1/2)/8, i = 0..7 */
    for (int i = 0; i < 8; ++i)
        v[k++] = orc_norm_ppf(pmax - (double)i * (pmax - 0.5) / 8.0);
    /* ascending order (insertion sort: 16 values) */
    for (int i = 1; i < 16; ++i) {
        double t = v[i];
        int j = i - 1;
        while (j >= 0 && v[j] > t) { v[j + 1] = v[j]; --j; }
        v[j + 1] = t;
    }
    for (int i = 0; i < 16; ++i)
        out[i] = (float)(v[i] / top);
}

/* Widen a bf16 bit pattern exactly to fp32. */
static float bf16_bits_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* [BQ] nearest level by the threshold rule: code = #{j : x > m_j}, where    */
/* m_j = (q_j + q_{j+1})/2 is exact in float64.                              */
static int nearest_level(float x, const double mid[15])
{
    int code = 0;
    for (int j = 0; j < 15; ++j)
        if ((double)x > mid[j]) ++code;
    return code;
}

/* ------------------------------------------------------------------------ */
/* [BQ] blockwise absmax quantization with blocksize 64 onto any ascending   */
/* codebook of 16 levels (the page's comparison of NF4 with integer grids    */
/* and a Lloyd codebook quantizes the same blocks with each table).          */
/* w: n values, fp32 (is_bf16 == 0) or bf16 bit patterns (is_bf16 == 1).   */
/* codes: ceil(n/2) bytes.  absmax: ceil(n/64) fp32 constants.  A block     */
/* with absmax 0 takes the code of x = 0 under the same rule.                */
/* ------------------------------------------------------------------------ */
void orc_quantize_levels(const void* w, int is_bf16, int64_t n, const float lv[16], uint8_t* codes,
                         float* absmax)
{
    double mid[15];
    for (int j = 0; j < 15; ++j)
        mid[j] = ((double)lv[j] + (double)lv[j + 1]) / 2.0;
    const int zero_code = nearest_level(0.0f, mid);

    const int64_t nblk = (n + 63) / 64;
    const float* wf = (const float*)w;
    const uint16_t* wb = (const uint16_t*)w;
    memset(codes, 0, (size_t)((n + 1) / 2));

#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nblk; ++b) {
        const int64_t lo = b * 64;
        const int64_t hi = (lo + 64 < n) ? lo + 64 : n;
        float v[64];
        float c = 0.0f;
        for (int64_t i = lo; i < hi; ++i) {
            v[i - lo] = is_bf16 ? bf16_bits_to_f32(wb[i]) : wf[i];
            float a = fabsf(v[i - lo]);
            if (a > c) c = a;
        }
        absmax[b] = c;
        for (int64_t i = lo; i < hi; ++i) {
            int code;
            if (c == 0.0f) {
                code = zero_code;
            } else {
                volatile float x = v[i - lo] / c;  /* one IEEE fp32 division */
                code = nearest_level(x, mid);
            }
            /* each block covers 32 whole bytes, so threads never share a byte */
            if (i & 1) codes[i >> 1] |= (uint8_t)(code << 4);
            else       codes[i >> 1] |= (uint8_t)code;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* [BQ]+[NF]+[RW] blockwise absmax NF4 quantization with blocksize 64: the   */
/* NF4 table in the rule above (an all-zero block gets code 7, the exact     */
/* zero level).                                                              */
/* ------------------------------------------------------------------------ */
void orc_nf4_quantize(const void* w, int is_bf16, int64_t n, uint8_t* codes, float* absmax)
{
    float lv[16];
    orc_nf4_codebook(lv);
    orc_quantize_levels(w, is_bf16, n, lv, codes, absmax);
}

/* ------------------------------------------------------------------------ */
/* Statistics of a blockwise quantization with a 16-level codebook (the      */
/* page's comparison, "NF4, derived from normal quantiles"): per code, the   */
/* number of values and the sum of x = fp32(w / absmax) (a Lloyd step moves  */
/* each level to the mean x of its values); over all values, the squared    */
/* error sum of (w - fp32(level[code] * absmax))^2, in float64.  A block     */
/* with absmax 0 has x = 0 and no error.  Per-thread partial sums (static    */
/* schedule) are added in thread order.                                      */
/* ------------------------------------------------------------------------ */
void orc_codebook_stats(const void* w, int is_bf16, int64_t n, const uint8_t* codes, const float* absmax,
                        const float lv[16], int64_t count[16], double sum_x[16], double* sse)
{
    const float* wf = (const float*)w;
    const uint16_t* wb = (const uint16_t*)w;
    int nt = 1;
#ifdef _OPENMP
    nt = omp_get_max_threads();
#endif
    int64_t* pc = (int64_t*)calloc((size_t)nt * 16, sizeof(int64_t));
    double* px = (double*)calloc((size_t)nt * 16, sizeof(double));
    double* pe = (double*)calloc((size_t)nt, sizeof(double));
#pragma omp parallel
    {
        int t = 0;
#ifdef _OPENMP
        t = omp_get_thread_num();
#endif
#pragma omp for schedule(static)
        for (int64_t i = 0; i < n; ++i) {
            const float wi = is_bf16 ? bf16_bits_to_f32(wb[i]) : wf[i];
            const int code = (codes[i >> 1] >> (4 * (i & 1))) & 15;
            const float c = absmax[i / 64];
            pc[t * 16 + code] += 1;
            if (c != 0.0f) {
                volatile float x = wi / c;
                volatile float wq = lv[code] * c;
                const double e = (double)wi - (double)wq;
                px[t * 16 + code] += (double)x;
                pe[t] += e * e;
            }
        }
    }
    for (int j = 0; j < 16; ++j) {
        count[j] = 0;
        sum_x[j] = 0.0;
    }
    *sse = 0.0;
    for (int t = 0; t < nt; ++t) {
        for (int j = 0; j < 16; ++j) {
            count[j] += pc[t * 16 + j];
            sum_x[j] += px[t * 16 + j];
        }
        *sse += pe[t];
    }
    free(pc);
    free(px);
    free(pe);
}

/* ------------------------------------------------------------------------ */
/* OCP FP8 E4M3 (bias 7, largest finite 448, no infinities; 0x7F/0xFF NaN). */
/* ------------------------------------------------------------------------ */
double orc_e4m3_decode(uint8_t b)
{
    const int sign = b >> 7;
    const int e = (b >> 3) & 0xF;
    const int m = b & 7;
    double mag;
    if (e == 0) mag = ldexp((double)m, -9);            /* subnormal: m * 2^-9 */
    else        mag = ldexp((double)(8 + m), e - 10);  /* (1 + m/8) * 2^(e-7) */
    return sign ? -mag : mag;
}

/* Nearest E4M3 value to v by exhaustive search over the 127 finite non-    */
/* negative magnitudes; on a tie the even code (mantissa LSB 0) wins.  The   */
/* sign bit is the sign of v, so a negative v that rounds to zero gives 0x80.*/
/* |v| must not exceed 448.                                                  */
uint8_t orc_e4m3_encode(double v)
{
    const int neg = signbit(v) ? 1 : 0;
    const double a = fabs(v);
    int best = 0;
    double bestd = a;                      /* distance to code 0 (zero) */
    for (int code = 1; code <= 0x7E; ++code) {
        const double d = fabs(a - orc_e4m3_decode((uint8_t)code));
        if (d < bestd || (d == bestd && (code & 1) == 0 && (best & 1) == 1)) {
            best = code;
            bestd = d;
        }
    }
    return (uint8_t)((neg << 7) | best);
}

/* Aligned pairwise float64 sum: at every level neighbours 2i and 2i+1 are   */
/* added and an odd last element is carried up unchanged.                    */
double orc_pairwise_sum(const float* x, int64_t n)
{
    if (n == 0) return 0.0;
    double* buf = (double*)malloc((size_t)n * sizeof(double));
    for (int64_t i = 0; i < n; ++i) buf[i] = (double)x[i];
    int64_t len = n;
    while (len > 1) {
        const int64_t half = len / 2;
        for (int64_t i = 0; i < half; ++i) buf[i] = buf[2 * i] + buf[2 * i + 1];
        if (len & 1) { buf[half] = buf[len - 1]; len = half + 1; }
        else len = half;
    }
    const double s = buf[0];
    free(buf);
    return s;
}

/* ------------------------------------------------------------------------ */
/* [DQ] double quantization of the first-level constants c1 (n1 values):    */
/* subtract the tensor-wide mean, then per block of 256 take c2 = max|d|,   */
/* s = d / c2, and store the E4M3 code of s*448.                            */
/* q: n1 bytes.  c2: ceil(n1/256) fp32.  mean: 1 fp32.                      */
/* ------------------------------------------------------------------------ */
void orc_double_quantize(const float* c1, int64_t n1, uint8_t* q, float* c2, float* mean_out)
{
    const float mean = (n1 > 0) ? (float)(orc_pairwise_sum(c1, n1) / (double)n1) : 0.0f;
    *mean_out = mean;
    const int64_t nb = (n1 + 255) / 256;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nb; ++b) {
        const int64_t lo = b * 256;
        const int64_t hi = (lo + 256 < n1) ? lo + 256 : n1;
        float m = 0.0f;
        for (int64_t i = lo; i < hi; ++i) {
            volatile float d = c1[i] - mean;
            if (fabsf(d) > m) m = fabsf(d);
        }
        c2[b] = m;
        for (int64_t i = lo; i < hi; ++i) {
            if (m == 0.0f) { q[i] = 0x00; continue; }
            volatile float d = c1[i] - mean;
            volatile float s = d / m;
            q[i] = orc_e4m3_encode((double)s * 448.0);  /* exact product in fp64 */
        }
    }
}

/* [DQ] two-level constant decode: c1' = fma(E4M3(q), fp32(c2/448), mean)   */
/* with a single rounding (C99 fmaf).                                        */
void orc_double_dequantize(const uint8_t* q, const float* c2, const float* mean, int64_t n1,
                           float* c1_out)
{
    const float mu = *mean;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n1; ++i) {
        volatile float step = c2[i / 256] / 448.0f;
        const float e = (float)orc_e4m3_decode(q[i]);   /* exact: 4 significant bits */
        c1_out[i] = fmaf(e, step, mu);
    }
}

/* [BQ]+[RW] dequantization: w' = fp32(level[code] * c1'), c1' from the      */
/* double-dequantized constants.  out: n fp32 values.                        */
void orc_nf4_dequantize(const uint8_t* codes, const uint8_t* q, const float* c2, const float* mean,
                        int64_t n, float* out)
{
    float lv[16];
    orc_nf4_codebook(lv);
    const int64_t n1 = (n + 63) / 64;
    float* c1 = (float*)malloc((size_t)(n1 > 0 ? n1 : 1) * sizeof(float));
    orc_double_dequantize(q, c2, mean, n1, c1);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        const int code = (i & 1) ? (codes[i >> 1] >> 4) : (codes[i >> 1] & 0xF);
        out[i] = lv[code] * c1[i / 64];
    }
    free(c1);
}

/* ------------------------------------------------------------------------ */
/* [BQ] dequantization with plain first-level constants (double quantization    */
/* off): w' = fp32(level[code] * absmax[i/64]).                               */
void orc_nf4_dequantize_plain(const uint8_t* codes, const float* absmax, int64_t n, float* out)
{
    float lv[16];
    orc_nf4_codebook(lv);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        const int code = (codes[i >> 1] >> (4 * (i & 1))) & 15;
        volatile float v = lv[code] * absmax[i / 64];
        out[i] = v;
    }
}

/* ------------------------------------------------------------------------ */
/* [PT]+[E2E] QLoRA linear layer, float64 from the exact operand values.    */
/*   W' (N x K, row-major, the dequantized frozen weight), X (M x K),       */
/*   A (r x K), B (N x r), s = alpha / r.                                    */
/*   T = X A^T (M x r);  Y = X W'^T + s T B^T (M x N).                       */
/* Rows of Y are computed for the row list `rows` (nrows entries); pass      */
/* rows == NULL to compute every row.  T is always computed for all rows.   */
void orc_qlora_linear_fwd(const float* Wd, const float* X, const float* A, const float* B,
                          int64_t M, int64_t N, int64_t K, int64_t r, double alpha,
                          const int64_t* rows, int64_t nrows, double* Y, double* T)
{
    const double s = alpha / (double)r;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t j = 0; j < r; ++j) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += (double)X[m * K + k] * (double)A[j * K + k];
            T[m * r + j] = acc;
        }
    const int64_t nr = rows ? nrows : M;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nr; ++i) {
        const int64_t m = rows ? rows[i] : i;
        for (int64_t n = 0; n < N; ++n) {
            double base = 0.0;
            for (int64_t k = 0; k < K; ++k) base += (double)X[m * K + k] * (double)Wd[n * K + k];
            double lora = 0.0;
            for (int64_t j = 0; j < r; ++j) lora += T[m * r + j] * (double)B[n * r + j];
            Y[i * N + n] = base + s * lora;
        }
    }
}

/* [E2E] backward.  Gradients reach X through W' and the adapters; W' gets   */
/* none.  With G = dY (M x N) and U = G B (M x r):                           */
/*   dX = G W' + s U A        (rows from `rows`, or all rows if NULL)        */
/*   dA = s U^T X             (r x K)                                        */
/*   dB = s G^T (X A^T)       (N x r)                                        */
/* dX / dA / dB may be NULL to skip them.  Every sum runs over its           */
/* contraction index in ascending order; the loops are only nested so that  */
/* memory is walked contiguously.                                            */
void orc_qlora_linear_bwd(const float* Wd, const float* X, const float* dY, const float* A,
                          const float* B, int64_t M, int64_t N, int64_t K, int64_t r, double alpha,
                          const int64_t* rows, int64_t nrows, double* dX, double* dA, double* dB)
{
    const double s = alpha / (double)r;
    double* U = (double*)malloc((size_t)(M * r > 0 ? M * r : 1) * sizeof(double));
    double* T = (double*)malloc((size_t)(M * r > 0 ? M * r : 1) * sizeof(double));
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t j = 0; j < r; ++j) {
            double u = 0.0, t = 0.0;
            for (int64_t n = 0; n < N; ++n) u += (double)dY[m * N + n] * (double)B[n * r + j];
            for (int64_t k = 0; k < K; ++k) t += (double)X[m * K + k] * (double)A[j * K + k];
            U[m * r + j] = u;
            T[m * r + j] = t;
        }
    if (dX) {
        const int64_t nr = rows ? nrows : M;
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t i = 0; i < nr; ++i) {
            const int64_t m = rows ? rows[i] : i;
            double* out = dX + i * K;
            for (int64_t k = 0; k < K; ++k) out[k] = 0.0;
            for (int64_t n = 0; n < N; ++n) {          /* base = sum_n G[m,n] W'[n,k] */
                const double g = (double)dY[m * N + n];
                const float* wr = Wd + n * K;
                for (int64_t k = 0; k < K; ++k) out[k] += g * (double)wr[k];
            }
            for (int64_t k = 0; k < K; ++k) {
                double lora = 0.0;
                for (int64_t j = 0; j < r; ++j) lora += U[m * r + j] * (double)A[j * K + k];
                out[k] = out[k] + s * lora;
            }
        }
    }
    if (dA) {
#pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < r; ++j) {
            double* acc = dA + j * K;
            for (int64_t k = 0; k < K; ++k) acc[k] = 0.0;
            for (int64_t m = 0; m < M; ++m) {          /* sum_m U[m,j] X[m,k] */
                const double u = U[m * r + j];
                const float* xr = X + m * K;
                for (int64_t k = 0; k < K; ++k) acc[k] += u * (double)xr[k];
            }
            for (int64_t k = 0; k < K; ++k) acc[k] = s * acc[k];
        }
    }
    if (dB) {
        const int64_t nchunk = 64;
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t n0 = 0; n0 < N; n0 += nchunk) {
            const int64_t n1 = (n0 + nchunk < N) ? n0 + nchunk : N;
            double* acc = dB + n0 * r;
            for (int64_t i = 0; i < (n1 - n0) * r; ++i) acc[i] = 0.0;
            for (int64_t m = 0; m < M; ++m)            /* sum_m G[m,n] T[m,j] */
                for (int64_t n = n0; n < n1; ++n) {
                    const double g = (double)dY[m * N + n];
                    for (int64_t j = 0; j < r; ++j) acc[(n - n0) * r + j] += g * T[m * r + j];
                }
            for (int64_t i = 0; i < (n1 - n0) * r; ++i) acc[i] = s * acc[i];
        }
    }
    free(U);
    free(T);
}

/* ------------------------------------------------------------------------ */
/* One step of Adam with decoupled weight decay (AdamW) on the adapter       */
/* parameters.  The pages ("Paged optimizers, and QLoRA end to end",         */
/* zerotofrontier.app "sft/peft") keep the adapters' Adam states in paged    */
/* memory and give the learning rates; they do not restate the update, so   */
/* it is the published one: Kingma & Ba, "Adam: A Method for Stochastic      */
/* Optimization" (ICLR 2015), Algorithm 1, with the weight decay decoupled   */
/* from the gradient as in Loshchilov & Hutter, "Decoupled Weight Decay      */
/* Regularization" (ICLR 2019), Algorithm 2 (schedule multiplier folded into */
/* lr).  Step t >= 1, every value in float64 from the fp32 inputs:           */
/*   m' = b1 m + (1 - b1) g                                                  */
/*   v' = b2 v + (1 - b2) g^2                                                */
/*   p' = p - lr wd p - lr (m' / (1 - b1^t)) / (sqrt(v' / (1 - b2^t)) + eps) */
/* ------------------------------------------------------------------------ */
void orc_adamw_step(const float* p, const float* g, const float* m, const float* v, int64_t n,
                    double lr, double b1, double b2, double eps, double wd, int64_t t,
                    double* p_out, double* m_out, double* v_out)
{
    const double bc1 = 1.0 - pow(b1, (double)t);
    const double bc2 = 1.0 - pow(b2, (double)t);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        const double gi = (double)g[i];
        const double mi = b1 * (double)m[i] + (1.0 - b1) * gi;
        const double vi = b2 * (double)v[i] + (1.0 - b2) * gi * gi;
        const double mh = mi / bc1, vh = vi / bc2;
        const double pi = (double)p[i];
        p_out[i] = pi - lr * wd * pi - lr * mh / (sqrt(vh) + eps);
        m_out[i] = mi;
        v_out[i] = vi;
    }
}

/* Number of OpenMP threads the parallel loops above use. */
int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
