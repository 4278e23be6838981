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
 *   LoftQ: the pages ([E2E], closing remark) state only the goal, an adapter with
 *          dequant(W^NF4) + gamma B A close to W; the alternation of quantizing the
 *          residual and a rank-r truncated SVD of the quantization error is Li et
 *          al. (2023); the SVD here is one-sided Jacobi (Hestenes 1958)
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
/* Rank-r truncated SVD: the top r singular triplets of E (m x n, float64,   */
/* row-major), whose sum  sum_i S_i U_i Vt_i  is the best rank-r             */
/* approximation of E in Frobenius norm (Eckart-Young).  Computed by        */
/* one-sided Jacobi (Hestenes): the columns of a working copy of E (of E^T   */
/* when E has more columns than rows) are rotated pairwise, each rotation    */
/* making one pair orthogonal, with the rotations accumulated into V, until */
/* a whole sweep finds every pair orthogonal to working precision; then the */
/* column norms are the singular values, the normalised columns the left    */
/* singular vectors.  Pairs are visited in round-robin order (n/2 disjoint  */
/* pairs per round), so a round's rotations commute.                          */
/*   S: r values, descending; U: m x r; Vt: r x n (row-major).  r <= min(m,n). */
/* ------------------------------------------------------------------------ */
static void jacobi_columns(double* a, int64_t m, int64_t n, double* v)
{
    /* a: n columns of length m (column j at a + j*m); v: n x n, column j at v + j*n */
    for (int64_t j = 0; j < n * n; ++j) v[j] = 0.0;
    for (int64_t j = 0; j < n; ++j) v[j * n + j] = 1.0;
    const int64_t nn = n + (n & 1);          /* an odd count gets a dummy column */
    int64_t* slot = (int64_t*)malloc((size_t)nn * sizeof(int64_t));
    for (int sweep = 0; sweep < 60; ++sweep) {
        int rotated = 0;
        for (int64_t j = 0; j < nn; ++j) slot[j] = j;
        for (int64_t round = 0; round < nn - 1; ++round) {
#pragma omp parallel for schedule(dynamic, 1) reduction(| : rotated)
            for (int64_t k = 0; k < nn / 2; ++k) {
                int64_t p = slot[k], q = slot[nn - 1 - k];
                if (p >= n || q >= n) continue;
                if (p > q) { int64_t t = p; p = q; q = t; }
                double* ap = a + p * m;
                double* aq = a + q * m;
                double alpha = 0.0, beta = 0.0, gamma = 0.0;
                for (int64_t i = 0; i < m; ++i) {
                    alpha += ap[i] * ap[i];
                    beta += aq[i] * aq[i];
                    gamma += ap[i] * aq[i];
                }
                if (gamma == 0.0 || fabs(gamma) <= 1e-15 * sqrt(alpha * beta)) continue;
                rotated = 1;
                /* the rotation angle that zeroes the pair's inner product */
                const double zeta = (beta - alpha) / (2.0 * gamma);
                const double t = (zeta >= 0.0 ? 1.0 : -1.0) / (fabs(zeta) + sqrt(1.0 + zeta * zeta));
                const double c = 1.0 / sqrt(1.0 + t * t), sn = c * t;
                for (int64_t i = 0; i < m; ++i) {
                    const double x = ap[i], y = aq[i];
                    ap[i] = c * x - sn * y;
                    aq[i] = sn * x + c * y;
                }
                double* vp = v + p * n;
                double* vq = v + q * n;
                for (int64_t i = 0; i < n; ++i) {
                    const double x = vp[i], y = vq[i];
                    vp[i] = c * x - sn * y;
                    vq[i] = sn * x + c * y;
                }
            }
            /* round-robin: slot 0 stays, the others rotate by one */
            const int64_t last = slot[nn - 1];
            for (int64_t j = nn - 1; j > 1; --j) slot[j] = slot[j - 1];
            slot[1] = last;
        }
        if (!rotated) break;
    }
    free(slot);
}

void orc_svd_topr(const double* E, int64_t m, int64_t n, int64_t r, double* S, double* U, double* Vt)
{
    const int tr = n > m;                    /* work on E^T: more columns than rows */
    const int64_t rows = tr ? n : m, cols = tr ? m : n;
    double* a = (double*)malloc((size_t)(rows * cols) * sizeof(double));
    double* v = (double*)malloc((size_t)(cols * cols) * sizeof(double));
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            if (tr) a[i * n + j] = E[i * n + j];       /* column i of E^T = row i of E */
            else a[j * m + i] = E[i * n + j];          /* column j of E */
        }
    jacobi_columns(a, rows, cols, v);
    double* norm = (double*)malloc((size_t)cols * sizeof(double));
    int64_t* order = (int64_t*)malloc((size_t)cols * sizeof(int64_t));
    for (int64_t j = 0; j < cols; ++j) {
        double t = 0.0;
        for (int64_t i = 0; i < rows; ++i) t += a[j * rows + i] * a[j * rows + i];
        norm[j] = sqrt(t);
        order[j] = j;
    }
    for (int64_t i = 1; i < cols; ++i) {       /* descending singular values */
        const int64_t o = order[i];
        int64_t k = i;
        while (k > 0 && norm[order[k - 1]] < norm[o]) { order[k] = order[k - 1]; --k; }
        order[k] = o;
    }
    for (int64_t t = 0; t < r; ++t) {
        const int64_t j = order[t];
        S[t] = norm[j];
        const double inv = norm[j] > 0.0 ? 1.0 / norm[j] : 0.0;
        /* working matrix = (E or E^T) V: its normalised columns are the left singular
           vectors of that matrix, V's columns its right ones */
        for (int64_t i = 0; i < rows; ++i) {
            const double lu = a[j * rows + i] * inv;
            if (tr) Vt[t * n + i] = lu;        /* E^T = U' S V'^T  =>  E = V' S U'^T */
            else U[i * r + t] = lu;
        }
        for (int64_t i = 0; i < cols; ++i) {
            const double rv = v[j * cols + i];
            if (tr) U[i * r + t] = rv;
            else Vt[t * n + i] = rv;
        }
    }
    free(a);
    free(v);
    free(norm);
    free(order);
}

/* ------------------------------------------------------------------------ */
/* [E2E] LoftQ-style initialisation of the adapter of a quantized base: the  */
/* pages ask that dequant(W^NF4) + gamma B A start close to W ("Paged       */
/* optimizers, and QLoRA end to end", closing remark on LoftQ, Li et al.     */
/* 2023).  The published alternation, from B A = 0, repeated `iters` times:  */
/*   Q_t = NF4 + double quantization of the residual  W - gamma B A  (fp32); */
/*   E_t = W - dequant(Q_t)  (fp32, exact difference of two fp32 values     */
/*         rounded once);                                                     */
/*   U S V^T = the rank-r truncated SVD of E_t;                              */
/*   B = U S^(1/2) / sqrt(gamma),  A = S^(1/2) V^T / sqrt(gamma).            */
/* err[t] = || W - dequant(Q_t) - gamma B_t A_t ||_F, float64.  Outputs the  */
/* last Q (codes, q, c2, mean) and B (N x r), A (r x K) in float64.          */
/* ------------------------------------------------------------------------ */
void orc_loftq(const float* W, int64_t N, int64_t K, int64_t r, double gamma, int iters,
               uint8_t* codes, uint8_t* q, float* c2, float* mean, double* B, double* A, double* err)
{
    const int64_t n = N * K, n1 = (n + 63) / 64;
    float* R = (float*)malloc((size_t)n * sizeof(float));
    float* absmax = (float*)malloc((size_t)n1 * sizeof(float));
    float* Wd = (float*)malloc((size_t)n * sizeof(float));
    double* E = (double*)malloc((size_t)n * sizeof(double));
    double* S = (double*)malloc((size_t)r * sizeof(double));
    double* U = (double*)malloc((size_t)(N * r) * sizeof(double));
    double* Vt = (double*)malloc((size_t)(r * K) * sizeof(double));
    for (int64_t i = 0; i < N * r; ++i) B[i] = 0.0;
    for (int64_t i = 0; i < r * K; ++i) A[i] = 0.0;
    for (int t = 0; t < iters; ++t) {
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < N; ++i)
            for (int64_t k = 0; k < K; ++k) {
                double ba = 0.0;
                for (int64_t j = 0; j < r; ++j) ba += B[i * r + j] * A[j * K + k];
                R[i * K + k] = (float)((double)W[i * K + k] - gamma * ba);
            }
        orc_nf4_quantize(R, 0, n, codes, absmax);
        orc_double_quantize(absmax, n1, q, c2, mean);
        orc_nf4_dequantize(codes, q, c2, mean, n, Wd);
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < n; ++i) {
            volatile float e = W[i] - Wd[i];
            E[i] = (double)e;
        }
        orc_svd_topr(E, N, K, r, S, U, Vt);
        const double g = 1.0 / sqrt(gamma);
        for (int64_t i = 0; i < N; ++i)
            for (int64_t j = 0; j < r; ++j) B[i * r + j] = U[i * r + j] * sqrt(S[j]) * g;
        for (int64_t j = 0; j < r; ++j)
            for (int64_t k = 0; k < K; ++k) A[j * K + k] = sqrt(S[j]) * Vt[j * K + k] * g;
        double e2 = 0.0;
#pragma omp parallel for schedule(static) reduction(+ : e2)
        for (int64_t i = 0; i < N; ++i)
            for (int64_t k = 0; k < K; ++k) {
                double ba = 0.0;
                for (int64_t j = 0; j < r; ++j) ba += B[i * r + j] * A[j * K + k];
                const double d = E[i * K + k] - gamma * ba;
                e2 += d * d;
            }
        err[t] = sqrt(e2);
    }
    free(R);
    free(absmax);
    free(Wd);
    free(E);
    free(S);
    free(U);
    free(Vt);
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
