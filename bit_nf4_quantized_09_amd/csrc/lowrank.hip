// lowrank.hip -- rank-r truncated SVD and the LoftQ-style initialisation of the adapter
// (gfx950).
//
// "Paged optimizers, and QLoRA end to end" (zerotofrontier.app "sft/peft"), closing remark:
// LoftQ (Li et al. 2023) starts the adapter so that dequant(W^NF4) + gamma B A is close to
// W, gamma = alpha / r.  Its alternation, from B A = 0: quantize the residual W - gamma B A
// (NF4 with double quantization: the codec kernels), then take the rank-r truncated SVD
// U S V^T of the quantization error E = W - dequant(Q) and set B = U S^1/2 / sqrt(gamma),
// A = S^1/2 V^T / sqrt(gamma).
//
// The SVD of the N x K fp32 matrix E is randomized subspace iteration (Halko, Martinsson &
// Tropp, SIAM Review 2011: the range finder with power iterations, Algorithms 4.3/4.4, and
// the direct SVD, Algorithm 5.1): with a given Gaussian K x l test matrix Omega (l = r +
// oversampling), Y = orth(E Omega); q times Z = orth(E^T Y), Y = orth(E Z); then Z = E^T Y
// (= (Y^T E)^T), the eigen-decomposition Z^T Z = V diag(lambda) V^T of its l x l Gram matrix,
// sigma = sqrt(lambda), and
//     U_r = Y V_r,   W_r = Z V_r diag(1 / sigma_r)        (E ~ U_r diag(sigma_r) W_r^T),
// the top r columns of V.  orth() is Cholesky QR, twice: G = X^T X (fp64), G = L L^T,
// X <- X L^-T.  The residual norm follows from the projection: ||E - U_r S_r W_r^T||_F^2 =
// ||E||_F^2 - sum sigma_r^2.
//
// Kernels: the tall products op(E) X (fp32 FMA, LDS-tiled, split along the contraction with a
// fixed-order sum), Gram partial sums in fp64, one workgroup for the l x l problems (fp64
// Cholesky and its inverse, cyclic Jacobi in LDS), the residual W - gamma B A and the
// quantization error W - dequant(Q) with its squared norm.
#include "launch.h"

namespace nf4 {

constexpr int LR_TM = 128;      // rows of a tall-product tile
constexpr int LR_TP = 32;       // contraction values per staged chunk

// ---------------------------------------------------------------------------
// C = op(E) X: E is M x P row-major (TRANS false) or P x M row-major (TRANS true), X is
// P x l row-major, C is M x l.  Workgroup (row tile, contraction slice z): 128 rows x all
// l <= LR_MAX columns over contraction values [z pchunk, (z+1) pchunk); thread (ty, tx)
// owns rows 8 ty .. 8 ty + 7 and columns tx + 16 j (48 accumulators, 6 FMAs per LDS read).
// Sums over p in ascending order (fp32 FMA); the slice's sums go to part[z] (M x l), or
// straight to C when there is one slice.
// ---------------------------------------------------------------------------
template <bool TRANS>
__global__ __launch_bounds__(256) void k_tall(const float* __restrict__ E, int64_t M, int64_t P,
                                              const float* __restrict__ X, int l, int64_t pchunk,
                                              float* __restrict__ part) {
    __shared__ __attribute__((aligned(16))) float sA[LR_TP][LR_TM + 4];   // [p][m]
    __shared__ float sB[LR_TP][LR_MAX];                                   // [p][c]
    const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
    const int64_t m0 = (int64_t)blockIdx.x * LR_TM;
    const int64_t p0 = (int64_t)blockIdx.y * pchunk;
    const int64_t p1 = p0 + pchunk < P ? p0 + pchunk : P;
    float acc[8][LR_MAX / 16];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < LR_MAX / 16; ++j) acc[i][j] = 0.0f;
    for (int64_t pc = p0; pc < p1; pc += LR_TP) {
#pragma unroll
        for (int e = 0; e < LR_TM * LR_TP / 256; ++e) {
            const int idx = tid + 256 * e;
            int pp, mm;
            if (TRANS) { pp = idx / LR_TM; mm = idx % LR_TM; }   // E[p][m]: m contiguous
            else       { mm = idx / LR_TP; pp = idx % LR_TP; }   // E[m][p]: p contiguous
            const int64_t gm = m0 + mm, gp = pc + pp;
            float v = 0.0f;
            if (gm < M && gp < p1) v = TRANS ? E[gp * M + gm] : E[gm * P + gp];
            sA[pp][mm] = v;
        }
        for (int idx = tid; idx < LR_TP * LR_MAX; idx += 256) {
            const int pp = idx / LR_MAX, c = idx % LR_MAX;
            const int64_t gp = pc + pp;
            sB[pp][c] = (c < l && gp < p1) ? X[gp * l + c] : 0.0f;
        }
        __syncthreads();
#pragma unroll 4
        for (int pp = 0; pp < LR_TP; ++pp) {
            const float4 a0 = *reinterpret_cast<const float4*>(&sA[pp][8 * ty]);
            const float4 a1 = *reinterpret_cast<const float4*>(&sA[pp][8 * ty + 4]);
            const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
            for (int j = 0; j < LR_MAX / 16; ++j) {
                const float b = sB[pp][tx + 16 * j];
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i][j] = __fmaf_rn(av[i], b, acc[i][j]);
            }
        }
        __syncthreads();
    }
    float* out = part + (int64_t)blockIdx.y * M * l;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t m = m0 + 8 * ty + i;
#pragma unroll
        for (int j = 0; j < LR_MAX / 16; ++j) {
            const int c = tx + 16 * j;
            if (m < M && c < l) out[m * l + c] = acc[i][j];
        }
    }
}

// out[i] = sum over z < S of part[z][i], z ascending (n values per slice)
__global__ __launch_bounds__(256) void k_slices_sum(const float* __restrict__ part, int S, int64_t n,
                                                    float* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    float s = part[i];
    for (int z = 1; z < S; ++z) s += part[(int64_t)z * n + i];
    out[i] = s;
}

// ---------------------------------------------------------------------------
// Gram partial sums: gpart[b][a][c] = sum over the rows of chunk b of X[row][a] X[row][c]
// (fp64 products of the fp32 values, rows ascending).  Workgroup b covers LR_GROWS rows;
// thread t owns entries e = t + 256 k of the l x l matrix.
// ---------------------------------------------------------------------------
constexpr int LR_GROWS = 64;
__global__ __launch_bounds__(256) void k_gram_part(const float* __restrict__ Xm, int64_t rows, int l,
                                                   double* __restrict__ gpart) {
    constexpr int EPT = LR_MAX * LR_MAX / 256;   // entries per thread
    constexpr int SR = 32;                       // rows staged at a time
    __shared__ float sX[SR][LR_MAX + 1];
    const int tid = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.x * LR_GROWS;
    const int64_t r1 = r0 + LR_GROWS < rows ? r0 + LR_GROWS : rows;
    double acc[EPT];
    int ea[EPT], ec[EPT];
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        const int e = tid + 256 * k;
        ea[k] = e / LR_MAX;
        ec[k] = e % LR_MAX;
        acc[k] = 0.0;
    }
    for (int64_t rc = r0; rc < r1; rc += SR) {
        for (int idx = tid; idx < SR * LR_MAX; idx += 256) {
            const int rr = idx / LR_MAX, c = idx % LR_MAX;
            const int64_t g = rc + rr;
            sX[rr][c] = (g < r1 && c < l) ? Xm[g * l + c] : 0.0f;
        }
        __syncthreads();
        for (int rr = 0; rr < SR; ++rr) {
#pragma unroll
            for (int k = 0; k < EPT; ++k) acc[k] = fma((double)sX[rr][ea[k]], (double)sX[rr][ec[k]], acc[k]);
        }
        __syncthreads();
    }
    double* out = gpart + (int64_t)blockIdx.x * l * l;
#pragma unroll
    for (int k = 0; k < EPT; ++k)
        if (ea[k] < l && ec[k] < l) out[ea[k] * l + ec[k]] = acc[k];
}

// G[e] = sum over the nparts Gram partials of gpart[z][e], z ascending (one entry per thread).
__global__ __launch_bounds__(256) void k_gram_sum(const double* __restrict__ gpart, int nparts, int64_t n,
                                                  double* __restrict__ G) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= n) return;
    double s = 0.0;
    for (int z = 0; z < nparts; ++z) s += gpart[(int64_t)z * n + e];
    G[e] = s;
}

// ---------------------------------------------------------------------------
// The l x l problems, one workgroup, fp64 in LDS (dynamic: 2 LR_MAX (LR_MAX + 1) doubles).
// G: the Gram matrix (summed by k_gram_sum).
//   SMALL_CHOL: G = L L^T (a column whose pivot falls to 1e-12 of the largest diagonal entry
//     or below is dropped: its L column is zero); writes Minv = L^-T (l x l, fp32), whose
//     dropped rows are zero, so that X Minv has orthonormal columns (zero where dropped).
//   SMALL_EIG: cyclic Jacobi (circle-method order, n/2 disjoint rotations per round, a pair
//     skipped once its entry is below 1e-16 of the geometric mean of its diagonal entries;
//     sweeps until the off-diagonal mass falls below 1e-22 of the total, at most 40); sorts the
//     eigenvalues descending; sigma = sqrt(max(lambda, 0)); writes S[0..r) (fp32),
//     Mb = V_r diag(g sigma^eb) and Ma = V_r diag(g sigma^ea) (l x r, fp32; a zero sigma
//     gives a zero column when its exponent is negative) and, when err != null,
//     err = sqrt(max(||E||^2 - sum sigma_r^2, 0)) with ||E||^2 = the sum of the nnorm fp64
//     partials in `norm2`, in order.
// ---------------------------------------------------------------------------
enum SmallMode { SMALL_CHOL = 0, SMALL_EIG = 1 };
struct SmallArgs {
    const double* gpart;
    int nparts;
    int l, r;
    float* Minv;                  // SMALL_CHOL
    float* S;                     // SMALL_EIG
    float* Mb;
    float* Ma;
    float eb, ea, g;
    const double* norm2;
    int nnorm;
    double* err;
};

template <int MODE>
__global__ __launch_bounds__(256) void k_small(SmallArgs a) {
    extern __shared__ __attribute__((aligned(16))) double sm[];
    constexpr int LD = LR_MAX + 1;
    double* G = sm;                 // [LR_MAX][LD]
    double* V = sm + LR_MAX * LD;   // [LR_MAX][LD]
    __shared__ double s_red[256];
    __shared__ double s_c[LR_MAX / 2], s_s[LR_MAX / 2];
    __shared__ int s_p[LR_MAX / 2], s_q[LR_MAX / 2];
    __shared__ int s_order[LR_MAX];
    __shared__ int s_flag;
    const int tid = threadIdx.x, l = a.l;
    for (int e = tid; e < l * l; e += 256) G[(e / l) * LD + e % l] = a.gpart[e];   // the summed Gram matrix
    __syncthreads();
    // symmetrize (the partial sums of (a, c) and (c, a) are the same products, in the same
    // order, so this only guards the algorithms below against any asymmetry)
    for (int e = tid; e < l * l; e += 256) {
        const int i = e / l, j = e % l;
        if (i < j) {
            const double v = 0.5 * (G[i * LD + j] + G[j * LD + i]);
            G[i * LD + j] = v;
            G[j * LD + i] = v;
        }
    }
    __syncthreads();

    if constexpr (MODE == SMALL_CHOL) {
        double dmax = 0.0;
        for (int i = 0; i < l; ++i) dmax = fmax(dmax, G[i * LD + i]);
        const double tol = 1e-12 * dmax;
        // Cholesky, right-looking: at step j the pivot, then column j, then the rank-1
        // update of the trailing lower triangle; every entry receives its products in
        // ascending step order, as in the column-by-column form.  L overwrites the lower
        // triangle of G.
        for (int j = 0; j < l; ++j) {
            if (tid == 0) {
                const double d = G[j * LD + j];
                const double ljj = d > tol && d > 0.0 ? sqrt(d) : 0.0;
                G[j * LD + j] = ljj;
                s_red[0] = ljj;
            }
            __syncthreads();
            const double ljj = s_red[0];
            for (int i = j + 1 + tid; i < l; i += 256) G[i * LD + j] = ljj > 0.0 ? G[i * LD + j] / ljj : 0.0;
            __syncthreads();
            const int t = l - j - 1;
            for (int e = tid; e < t * t; e += 256) {
                const int i = j + 1 + e / t, k = j + 1 + e % t;
                if (k <= i) G[i * LD + k] -= G[i * LD + j] * G[k * LD + j];
            }
            __syncthreads();
        }
        // Linv = L^-1 (lower) into V, by rows: at step j row j is divided by its pivot
        // (a zero pivot gives a zero row), then eliminated from the rows below; each entry
        // receives its products in ascending order of j, then its one division
        for (int e = tid; e < l * l; e += 256) V[(e / l) * LD + e % l] = (e / l == e % l) ? 1.0 : 0.0;
        __syncthreads();
        for (int j = 0; j < l; ++j) {
            const double ljj = G[j * LD + j];
            for (int c = tid; c < l; c += 256) V[j * LD + c] = (j < c || ljj == 0.0) ? 0.0 : V[j * LD + c] / ljj;
            __syncthreads();
            const int t = l - j - 1, w = j + 1;
            for (int e = tid; e < t * w; e += 256) {
                const int i = j + 1 + e / w, c = e % w;
                V[i * LD + c] -= G[i * LD + j] * V[j * LD + c];
            }
            __syncthreads();
        }
        // Minv = Linv^T
        for (int e = tid; e < l * l; e += 256) {
            const int i = e / l, j = e % l;
            a.Minv[i * l + j] = (float)V[j * LD + i];
        }
        return;
    } else {
        for (int e = tid; e < l * l; e += 256) V[(e / l) * LD + e % l] = (e / l == e % l) ? 1.0 : 0.0;
        const int n = l + (l & 1);           // an odd order gets a dummy index
        const int np = n / 2;
        double total = 0.0;
        for (int i = 0; i < l; ++i)
            for (int j = 0; j < l; ++j) total += G[i * LD + j] * G[i * LD + j];
        __syncthreads();
        // this thread's (pair, index) work items of a round: e = tid + 256 m < np * l
        constexpr int WI = (LR_MAX / 2 * LR_MAX + 255) / 256;
        int wk[WI], wc[WI];
#pragma unroll
        for (int m = 0; m < WI; ++m) {
            const int e = tid + 256 * m;
            wk[m] = e < np * l ? e / l : -1;
            wc[m] = e < np * l ? e % l : 0;
        }
        for (int sweep = 0; sweep < 40; ++sweep) {
            // off-diagonal mass
            double off = 0.0;
            for (int e = tid; e < l * l; e += 256) {
                const int i = e / l, j = e % l;
                if (i != j) off += G[i * LD + j] * G[i * LD + j];
            }
            s_red[tid] = off;
            __syncthreads();
            for (int st = 128; st > 0; st >>= 1) {
                if (tid < st) s_red[tid] += s_red[tid + st];
                __syncthreads();
            }
            if (tid == 0) s_flag = !(s_red[0] > 1e-22 * total);
            __syncthreads();
            if (s_flag) break;
            for (int round = 0; round < n - 1; ++round) {
                // this round's pairs (circle method: index n - 1 meets `round`, the others
                // meet across the circle of n - 1) and rotations
                if (tid < np) {
                    int p = tid == 0 ? n - 1 : (round + tid) % (n - 1);
                    int q = tid == 0 ? round : (round - tid + (n - 1)) % (n - 1);
                    if (p > q) { const int t = p; p = q; q = t; }
                    double c = 1.0, s = 0.0;
                    if (q < l) {
                        const double gpq = G[p * LD + q];
                        // a pair already orthogonal to working precision is left as it is
                        if (fabs(gpq) > 1e-16 * sqrt(fabs(G[p * LD + p] * G[q * LD + q]))) {
                            const double tau = (G[q * LD + q] - G[p * LD + p]) / (2.0 * gpq);
                            const double t = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
                            c = 1.0 / sqrt(1.0 + t * t);
                            s = t * c;
                        }
                    }
                    s_p[tid] = p;
                    s_q[tid] = q;
                    s_c[tid] = c;
                    s_s[tid] = s;
                }
                __syncthreads();
                // G <- J^T G (rows p, q of every pair)
#pragma unroll
                for (int m = 0; m < WI; ++m) {
                    const int k = wk[m], col = wc[m];
                    if (k < 0) continue;
                    const int p = s_p[k], q = s_q[k];
                    if (q >= l) continue;
                    const double c = s_c[k], s = s_s[k];
                    const double gp = G[p * LD + col], gq = G[q * LD + col];
                    G[p * LD + col] = c * gp - s * gq;
                    G[q * LD + col] = s * gp + c * gq;
                }
                __syncthreads();
                // G <- G J and V <- V J (columns p, q of every pair)
#pragma unroll
                for (int m = 0; m < WI; ++m) {
                    const int k = wk[m], row = wc[m];
                    if (k < 0) continue;
                    const int p = s_p[k], q = s_q[k];
                    if (q >= l) continue;
                    const double c = s_c[k], s = s_s[k];
                    const double gp = G[row * LD + p], gq = G[row * LD + q];
                    G[row * LD + p] = c * gp - s * gq;
                    G[row * LD + q] = s * gp + c * gq;
                    const double vp = V[row * LD + p], vq = V[row * LD + q];
                    V[row * LD + p] = c * vp - s * vq;
                    V[row * LD + q] = s * vp + c * vq;
                }
                __syncthreads();
            }
        }
        // eigenvalues on the diagonal: order them descending (ties by index)
        if (tid < l) {
            const double v = G[tid * LD + tid];
            int rank = 0;
            for (int j = 0; j < l; ++j) {
                const double w = G[j * LD + j];
                rank += (w > v || (w == v && j < tid)) ? 1 : 0;
            }
            s_order[rank] = tid;
        }
        __syncthreads();
        for (int e = tid; e < l * a.r; e += 256) {
            const int row = e / a.r, t = e % a.r, j = s_order[t];
            const double sig = sqrt(fmax(G[j * LD + j], 0.0));
            const double fb = sig > 0.0 ? pow(sig, (double)a.eb) : (a.eb == 0.0f ? 1.0 : 0.0);
            const double fa = sig > 0.0 ? pow(sig, (double)a.ea) : (a.ea == 0.0f ? 1.0 : 0.0);
            a.Mb[row * a.r + t] = (float)(V[row * LD + j] * fb * (double)a.g);
            a.Ma[row * a.r + t] = (float)(V[row * LD + j] * fa * (double)a.g);
        }
        if (tid < a.r) a.S[tid] = (float)sqrt(fmax(G[s_order[tid] * LD + s_order[tid]], 0.0));
        if (a.err) {
            // ||E||^2: the nnorm <= 1024 partials, 4 per thread in order, then a fixed tree
            double e2 = 0.0;
            for (int z = 4 * tid; z < 4 * tid + 4; ++z) e2 += z < a.nnorm ? a.norm2[z] : 0.0;
            __syncthreads();
            s_red[tid] = e2;
            __syncthreads();
            for (int st = 128; st > 0; st >>= 1) {
                if (tid < st) s_red[tid] += s_red[tid + st];
                __syncthreads();
            }
            if (tid == 0) {
                double cap = 0.0;
                for (int t = 0; t < a.r; ++t) cap += fmax(G[s_order[t] * LD + s_order[t]], 0.0);
                *a.err = sqrt(fmax(s_red[0] - cap, 0.0));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// R = W - gamma (Bf AfT^T): Bf N x r, AfT K x r (fp32), tile 64 x 64, thread (ty, tx) owns
// rows 4 ty.., columns 4 tx..; the rank sum is fp32 FMA over j ascending, then one fp32
// multiply by gamma and one subtraction.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_residual(const float* __restrict__ W, int64_t N, int64_t K,
                                                  const float* __restrict__ Bf, const float* __restrict__ AfT,
                                                  int r, float gamma, float* __restrict__ R) {
    __shared__ __attribute__((aligned(16))) float sb[LR_MAX][68];   // [j][row]
    __shared__ __attribute__((aligned(16))) float sa[LR_MAX][68];   // [j][col]
    const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
    const int64_t ktiles = (K + 63) / 64;
    const int64_t n0 = ((int64_t)blockIdx.x / ktiles) * 64, k0 = ((int64_t)blockIdx.x % ktiles) * 64;
    for (int idx = tid; idx < 64 * r; idx += 256) {
        const int row = idx / r, j = idx % r;
        sb[j][row] = n0 + row < N ? Bf[(n0 + row) * r + j] : 0.0f;
        sa[j][row] = k0 + row < K ? AfT[(k0 + row) * r + j] : 0.0f;
    }
    __syncthreads();
    float acc[4][4] = {};
    for (int j = 0; j < r; ++j) {
        const float4 b = *reinterpret_cast<const float4*>(&sb[j][4 * ty]);
        const float4 c = *reinterpret_cast<const float4*>(&sa[j][4 * tx]);
        const float bv[4] = {b.x, b.y, b.z, b.w}, cv[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[i][q] = __fmaf_rn(bv[i], cv[q], acc[i][q]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t n = n0 + 4 * ty + i;
        if (n >= N) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t k = k0 + 4 * tx + q;
            if (k < K) R[n * K + k] = W[n * K + k] - gamma * acc[i][q];
        }
    }
}

// ---------------------------------------------------------------------------
// E = W - dequant(Q) elementwise, E[i] = fp32(W[i] - fp32(level[code_i] c1'[i/64])), and
// partial sums of E^2 in fp64: workgroup b strides over the tensor in 8-value groups and
// writes the sum of its own squares (groups ascending per thread, then a fixed tree).
// ---------------------------------------------------------------------------
constexpr int QE_GRID = 1024;
__global__ __launch_bounds__(256) void k_quant_error(const float* __restrict__ W, const uint8_t* __restrict__ codes,
                                                     const float* __restrict__ c1, int64_t n, Nf4Table tab,
                                                     float* __restrict__ E, double* __restrict__ norm2) {
    __shared__ float s_lv[16];
    __shared__ double s_red[256];
    if (threadIdx.x < 16) s_lv[threadIdx.x] = tab.lv[threadIdx.x];
    __syncthreads();
    double acc = 0.0;
    const int64_t groups = (n + 7) / 8;
    for (int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x; gi < groups; gi += (int64_t)gridDim.x * 256) {
        const int64_t i0 = gi * 8;
        if (i0 + 8 <= n) {
            const uint32_t w = *reinterpret_cast<const uint32_t*>(codes + i0 / 2);
            const float c = c1[i0 / 64];
            const float4 a0 = *reinterpret_cast<const float4*>(W + i0);
            const float4 a1 = *reinterpret_cast<const float4*>(W + i0 + 4);
            const float wv[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            float ev[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float deq = s_lv[(w >> (4 * e)) & 15u] * c;
                ev[e] = wv[e] - deq;
                acc = fma((double)ev[e], (double)ev[e], acc);
            }
            *reinterpret_cast<float4*>(E + i0) = make_float4(ev[0], ev[1], ev[2], ev[3]);
            *reinterpret_cast<float4*>(E + i0 + 4) = make_float4(ev[4], ev[5], ev[6], ev[7]);
        } else {
            for (int64_t i = i0; i < n; ++i) {
                const int code = (codes[i >> 1] >> (4 * (i & 1))) & 15;
                const float ev = W[i] - s_lv[code] * c1[i / 64];
                E[i] = ev;
                acc = fma((double)ev, (double)ev, acc);
            }
        }
    }
    s_red[threadIdx.x] = acc;
    __syncthreads();
    for (int st = 128; st > 0; st >>= 1) {
        if (threadIdx.x < st) s_red[threadIdx.x] += s_red[threadIdx.x + st];
        __syncthreads();
    }
    if (threadIdx.x == 0) norm2[blockIdx.x] = s_red[0];
}

// bf16 adapter factors for the layer: B = bf16(Bf) (N x r), A = bf16(AfT^T) (r x K)
__global__ __launch_bounds__(256) void k_factors_bf16(const float* __restrict__ Bf, const float* __restrict__ AfT,
                                                      int64_t N, int64_t K, int r, uint16_t* __restrict__ B,
                                                      uint16_t* __restrict__ A) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < N * r) B[i] = f32_to_bf16(Bf[i]);
    if (i < (int64_t)r * K) {
        const int64_t j = i / K, k = i % K;
        A[i] = f32_to_bf16(AfT[k * r + j]);
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// contraction slices of a tall product: enough workgroups to fill the chip
static int tall_slices(int64_t M, int64_t P) {
    const int64_t tiles = cdiv(M, LR_TM);
    int64_t S = cdiv(1024, tiles);
    const int64_t maxS = cdiv(P, LR_TP);
    if (S > maxS) S = maxS;
    if (S > LR_MAX_SLICES) S = LR_MAX_SLICES;
    return (int)(S < 1 ? 1 : S);
}

size_t lowrank_ws_bytes(int64_t N, int64_t K, int l, int r) {
    const int64_t big = N > K ? N : K;
    size_t b = 0;
    b += 2 * al256((size_t)N * l * 4);                       // Y, Y2
    b += 2 * al256((size_t)K * l * 4);                       // Z, Z2
    b += al256((size_t)LR_MAX_SLICES * big * l * 4);          // tall-product slices
    b += al256((size_t)cdiv(big, LR_GROWS) * l * l * 8);      // Gram partials
    b += al256((size_t)l * l * 8);                           // their sum
    b += al256((size_t)l * l * 4);                           // Minv
    b += 2 * al256((size_t)l * r * 4);                       // Mb, Ma
    return b;
}

struct LowrankWs {
    float *Y, *Y2, *Z, *Z2, *part;
    double* gpart;
    double* gsum;
    float *Minv, *Mb, *Ma;
};

static LowrankWs carve(void* ws, int64_t N, int64_t K, int l, int r) {
    const int64_t big = N > K ? N : K;
    char* p = (char*)ws;
    LowrankWs w;
    auto take = [&](size_t bytes) { char* q = p; p += al256(bytes); return (void*)q; };
    w.Y = (float*)take((size_t)N * l * 4);
    w.Y2 = (float*)take((size_t)N * l * 4);
    w.Z = (float*)take((size_t)K * l * 4);
    w.Z2 = (float*)take((size_t)K * l * 4);
    w.part = (float*)take((size_t)LR_MAX_SLICES * big * l * 4);
    w.gpart = (double*)take((size_t)cdiv(big, LR_GROWS) * l * l * 8);
    w.gsum = (double*)take((size_t)l * l * 8);
    w.Minv = (float*)take((size_t)l * l * 4);
    w.Mb = (float*)take((size_t)l * r * 4);
    w.Ma = (float*)take((size_t)l * r * 4);
    return w;
}

static size_t small_lds() { return (size_t)2 * LR_MAX * (LR_MAX + 1) * sizeof(double); }

static hipError_t small_attr() {
    static bool done = false;
    if (done) return hipSuccess;
    hipError_t e = hipFuncSetAttribute((const void*)k_small<SMALL_CHOL>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)small_lds());
    if (e == hipSuccess)
        e = hipFuncSetAttribute((const void*)k_small<SMALL_EIG>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)small_lds());
    if (e == hipSuccess) done = true;
    return e;
}

// C (M x l) = op(E) X, op(E) M x P
static hipError_t tall(bool trans, const float* E, int64_t M, int64_t P, const float* X, int l, float* C,
                       float* part, hipStream_t s) {
    const int S = tall_slices(M, P);
    const int64_t pchunk = cdiv(cdiv(P, S), LR_TP) * LR_TP;
    const int Sx = (int)cdiv(P, pchunk);
    dim3 grid((unsigned)cdiv(M, LR_TM), (unsigned)Sx);
    float* dst = Sx == 1 ? C : part;
    if (trans) hipLaunchKernelGGL(k_tall<true>, grid, dim3(256), 0, s, E, M, P, X, l, pchunk, dst);
    else hipLaunchKernelGGL(k_tall<false>, grid, dim3(256), 0, s, E, M, P, X, l, pchunk, dst);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || Sx == 1) return e;
    hipLaunchKernelGGL(k_slices_sum, dim3((unsigned)cdiv(M * l, 256)), dim3(256), 0, s, part, Sx, M * l, C);
    return hipGetLastError();
}

// G (l x l fp64, at gsum) = Xm^T Xm over `rows` rows: partial sums per 64 rows, then their
// fixed-order sum
static hipError_t gram(const float* Xm, int64_t rows, int l, double* gpart, double* gsum, hipStream_t s) {
    const int nparts = (int)cdiv(rows, LR_GROWS);
    hipLaunchKernelGGL(k_gram_part, dim3((unsigned)nparts), dim3(256), 0, s, Xm, rows, l, gpart);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_gram_sum, dim3((unsigned)cdiv((int64_t)l * l, 256)), dim3(256), 0, s, gpart, nparts,
                       (int64_t)l * l, gsum);
    return hipGetLastError();
}

// X <- orth(X) (rows x l) by Cholesky QR twice: X -> tmp -> X
static hipError_t orth(float* X, float* tmp, int64_t rows, int l, LowrankWs& w, hipStream_t s) {
    float* src = X;
    float* dst = tmp;
    for (int pass = 0; pass < 2; ++pass) {
        hipError_t e = gram(src, rows, l, w.gpart, w.gsum, s);
        if (e != hipSuccess) return e;
        SmallArgs a{};
        a.gpart = w.gsum;
        a.nparts = 1;
        a.l = l;
        a.Minv = w.Minv;
        hipLaunchKernelGGL(k_small<SMALL_CHOL>, dim3(1), dim3(256), small_lds(), s, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        e = tall(false, src, rows, l, w.Minv, l, dst, w.part, s);
        if (e != hipSuccess) return e;
        float* t = src;
        src = dst;
        dst = t;
    }
    return hipSuccess;
}

// Rank-r factors of E (N x K) by randomized subspace iteration: on return Lf = E-side
// factor (N x r) = Y V_r diag(g sigma^eb), Rf = (K x r) = Z V_r diag(g sigma^ea), S the
// top r singular values, err (if given) = sqrt(||E||^2 - sum sigma_r^2) from the norm2
// partials.
static hipError_t lowrank_factors(const float* E, int64_t N, int64_t K, int r, int l, int power,
                                  const float* omega, LowrankWs& w, float eb, float ea, float g, float* Lf,
                                  float* Rf, float* S, const double* norm2, int nnorm, double* err,
                                  hipStream_t s) {
    hipError_t e = small_attr();
    if (e != hipSuccess) return e;
    // Y = orth(E Omega)
    e = tall(false, E, N, K, omega, l, w.Y, w.part, s);
    if (e == hipSuccess) e = orth(w.Y, w.Y2, N, l, w, s);
    for (int it = 0; it < power && e == hipSuccess; ++it) {
        e = tall(true, E, K, N, w.Y, l, w.Z, w.part, s);           // Z = orth(E^T Y)
        if (e == hipSuccess) e = orth(w.Z, w.Z2, K, l, w, s);
        if (e == hipSuccess) e = tall(false, E, N, K, w.Z, l, w.Y, w.part, s);    // Y = orth(E Z)
        if (e == hipSuccess) e = orth(w.Y, w.Y2, N, l, w, s);
    }
    if (e != hipSuccess) return e;
    // Z = E^T Y, its Gram matrix, the eigen-decomposition and the factor matrices
    e = tall(true, E, K, N, w.Y, l, w.Z, w.part, s);
    if (e == hipSuccess) e = gram(w.Z, K, l, w.gpart, w.gsum, s);
    if (e != hipSuccess) return e;
    SmallArgs a{};
    a.gpart = w.gsum;
    a.nparts = 1;
    a.l = l;
    a.r = r;
    a.S = S;
    a.Mb = w.Mb;
    a.Ma = w.Ma;
    a.eb = eb;
    a.ea = ea;
    a.g = g;
    a.norm2 = norm2;
    a.nnorm = nnorm;
    a.err = err;
    hipLaunchKernelGGL(k_small<SMALL_EIG>, dim3(1), dim3(256), small_lds(), s, a);
    e = hipGetLastError();
    if (e == hipSuccess) e = tall(false, w.Y, N, l, w.Mb, r, Lf, w.part, s);
    if (e == hipSuccess) e = tall(false, w.Z, K, l, w.Ma, r, Rf, w.part, s);
    return e;
}

hipError_t launch_lowrank_svd(const float* E, int64_t N, int64_t K, int r, int l, int power, const float* omega,
                              float* U, float* S, float* V, void* ws, hipStream_t s) {
    LowrankWs w = carve(ws, N, K, l, r);
    // U = Y V_r, V = Z V_r diag(1 / sigma)
    return lowrank_factors(E, N, K, r, l, power, omega, w, 0.0f, -1.0f, 1.0f, U, V, S, nullptr, 0, nullptr, s);
}

size_t loftq_ws_bytes(int64_t N, int64_t K, int l, int r) {
    const int64_t n = N * K, n1 = cdiv(n, 64);
    size_t b = lowrank_ws_bytes(N, K, l, r);
    b += al256((size_t)n * 4);                     // E (also the residual)
    b += 2 * al256((size_t)n1 * 4);                // absmax, c1'
    b += al256(double_quantize_ws_bytes(n1));
    b += al256((size_t)QE_GRID * 8);               // ||E||^2 partials
    b += al256((size_t)N * r * 4) + al256((size_t)K * r * 4);   // Bf, AfT
    b += al256((size_t)r * 4);                     // singular values
    return b;
}

hipError_t launch_loftq(const float* W, int64_t N, int64_t K, int r, float gamma, int iters, int l, int power,
                        const float* omega, uint8_t* codes, uint8_t* q, float* c2, float* mean, uint16_t* A,
                        uint16_t* B, double* err, void* ws, const Nf4Table& tab, hipStream_t s) {
    const int64_t n = N * K, n1 = cdiv(n, 64);
    LowrankWs w = carve(ws, N, K, l, r);
    char* p = (char*)ws + lowrank_ws_bytes(N, K, l, r);
    auto take = [&](size_t bytes) { char* t = p; p += al256(bytes); return (void*)t; };
    float* E = (float*)take((size_t)n * 4);
    float* absmax = (float*)take((size_t)n1 * 4);
    float* c1 = (float*)take((size_t)n1 * 4);
    double* dqws = (double*)take(double_quantize_ws_bytes(n1));
    double* norm2 = (double*)take((size_t)QE_GRID * 8);
    float* Bf = (float*)take((size_t)N * r * 4);
    float* AfT = (float*)take((size_t)K * r * 4);
    float* S = (float*)take((size_t)r * 4);
    const float g = 1.0f / sqrtf(gamma);
    const unsigned qe_grid = (unsigned)(cdiv(cdiv(n, 8), 256) < QE_GRID ? cdiv(cdiv(n, 8), 256) : QE_GRID);
    hipError_t e = hipSuccess;
    for (int t = 0; t < iters && e == hipSuccess; ++t) {
        const float* R = W;                    // B A = 0 at the start: W itself is quantized
        if (t > 0) {
            hipLaunchKernelGGL(k_residual, dim3((unsigned)(cdiv(K, 64) * cdiv(N, 64))), dim3(256), 0, s, W, N, K,
                               Bf, AfT, r, gamma, E);
            e = hipGetLastError();
            R = E;
        }
        if (e == hipSuccess) e = launch_quantize(R, false, n, codes, absmax, tab, s);
        if (e == hipSuccess) e = launch_double_quantize(absmax, n1, q, c2, mean, dqws, s);
        if (e == hipSuccess) e = launch_double_dequantize(q, c2, mean, n1, c1, s);
        if (e != hipSuccess) break;
        hipLaunchKernelGGL(k_quant_error, dim3(qe_grid), dim3(256), 0, s, W, codes, c1, n, tab, E, norm2);
        e = hipGetLastError();
        // B = U_r S^1/2 / sqrt(gamma) = Y V_r diag(sigma^1/2 g), A^T = W_r S^1/2 / sqrt(gamma)
        //   = Z V_r diag(sigma^-1/2 g)
        if (e == hipSuccess)
            e = lowrank_factors(E, N, K, r, l, power, omega, w, 0.5f, -0.5f, g, Bf, AfT, S, norm2, (int)qe_grid,
                                err + t, s);
    }
    if (e != hipSuccess) return e;
    const int64_t most = N * r > (int64_t)r * K ? N * r : (int64_t)r * K;
    hipLaunchKernelGGL(k_factors_bf16, dim3((unsigned)cdiv(most, 256)), dim3(256), 0, s, Bf, AfT, N, K, r, B, A);
    return hipGetLastError();
}

}  // namespace nf4
