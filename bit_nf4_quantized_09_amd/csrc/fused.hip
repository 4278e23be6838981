// fused.hip -- NF4 dequantization fused into bf16 MFMA products (gfx950).
//
// "Paged optimizers, and QLoRA end to end" (zerotofrontier.app "sft/peft"):
// every frozen matrix is dequantized to bfloat16 block by block and multiplied
// in 16-bit precision, with the bf16 LoRA output added; gradients flow back
// through the dequantized weight.  "The real way": the dequantization is fused
// into the matrix multiply.  Layer formula: "Putting it together"
// (prism.theerrors.in QLoRA explainer).
//
// Forward  Y  = X W'^T + s T B^T   (NT product, contraction over K)
// Backward dX = dY W' + s U A      (NN product, contraction over N)
//
// Design for CDNA4: 256 x 256 output tile per workgroup of 4 waves (each wave
// 128 x 128 = 4 x 4 tiles of v_mfma_f32_32x32x16_bf16, 256 fp32 accumulators
// per lane), one NF4 block (64 values) of contraction per pipeline step, two
// LDS stages of 64 KB.  The packed codes of one (row, 64-block) are owned by
// one lane, which builds a 16-entry bf16 table scaled by the block's decoded
// constant and expands its 64 codes with byte permutes before writing them to
// LDS; every dequantized value is therefore computed once per workgroup and
// reused by 256 rows of the other operand.
#include "launch.h"

namespace nf4 {

constexpr int FT = 256;                 // output tile edge (M and N/K directions)
constexpr int FSTAGE = 65536;           // bytes per pipeline stage: 2 tiles of 256 x 64 bf16
constexpr int FLDS = 2 * FSTAGE;        // 128 KB of the 160 KB LDS

// Row-major [row][64 bf16] tile, 16-byte chunk c of row r stored at c ^ (r & 7).
__device__ __forceinline__ int tile_off(int row, int chunk) {
    return row * 128 + ((chunk ^ (row & 7)) << 4);
}

// Transposed tile for the backward W' operand: element (k, n) of a
// [256 k][64 n] tile; chunk n/8 of row k is stored at (n/8) ^ swz(k).
__device__ __forceinline__ int tt_swz(int k) { return (k & 7) ^ ((k >> 6) & 3); }
__device__ __forceinline__ int ttile_off(int k, int n) {
    return k * 128 + ((((n >> 3) ^ tt_swz(k)) & 7) << 4) + ((n & 7) << 1);
}

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_fused_fwd(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ qc,
                 const float* __restrict__ c2, const float* __restrict__ mean_p, int64_t N,
                 int64_t K, const uint16_t* __restrict__ X, int64_t M,
                 const uint16_t* __restrict__ Ts, const uint16_t* __restrict__ Bl, int r,
                 uint16_t* __restrict__ Y, Nf4Table tab) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t n0 = (int64_t)blockIdx.x * FT, m0 = (int64_t)blockIdx.y * FT;
    const int64_t KB = K >> 6;
    const float mean = *mean_p;

    // this lane dequantizes row n0 + tid of W
    const int64_t wrow = n0 + tid;
    const bool wvalid = wrow < N;
    const uint8_t* wcode = codes + wrow * (K >> 1);
    const int64_t cidx0 = wrow * KB;

    uint4 xr[8];
    uint4 wc0 = make_uint4(0, 0, 0, 0), wc1 = make_uint4(0, 0, 0, 0);
    uint32_t qb = 0;
    float c2v = 0.0f;

    auto load_step = [&](int64_t kb) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int qi = tid + 256 * i;
            const int row = qi >> 3, c = qi & 7;
            const int64_t gm = m0 + row;
            xr[i] = (gm < M) ? *reinterpret_cast<const uint4*>(X + gm * K + kb * 64 + c * 8)
                             : make_uint4(0, 0, 0, 0);
        }
        if (wvalid) {
            wc0 = *reinterpret_cast<const uint4*>(wcode + kb * 32);
            wc1 = *reinterpret_cast<const uint4*>(wcode + kb * 32 + 16);
            qb = qc[cidx0 + kb];
            c2v = c2[(cidx0 + kb) >> 8];
        }
    };
    auto store_step = [&](int stage) {
        uint8_t* sX = lds + stage * FSTAGE;
        uint8_t* sW = sX + 32768;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int qi = tid + 256 * i;
            const int row = qi >> 3, c = qi & 7;
            *reinterpret_cast<uint4*>(sX + tile_off(row, c)) = xr[i];
        }
        const float c1p = wvalid ? decode_c1(qb, c2_step(c2v), mean) : 0.0f;
        const ScaledTable st = make_scaled_table(tab, c1p);
        const uint32_t words[8] = {wc0.x, wc0.y, wc0.z, wc0.w, wc1.x, wc1.y, wc1.z, wc1.w};
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            uint32_t o[4];
            decode8(st, words[c], o);
            *reinterpret_cast<uint4*>(sW + tile_off(tid, c)) = make_uint4(o[0], o[1], o[2], o[3]);
        }
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

    auto mfma_step = [&](const uint8_t* sA, const uint8_t* sB, int nsub) {
#pragma unroll
        for (int sub = 0; sub < 4; ++sub) {
            if (sub < nsub) {
                const int ch = 2 * sub + (lane >> 5);
                bf16x8 a[4], b[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ra = wm * 128 + i * 32 + (lane & 31);
                    a[i] = *reinterpret_cast<const bf16x8*>(sA + tile_off(ra, ch));
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int rb = wn * 128 + j * 32 + (lane & 31);
                    b[j] = *reinterpret_cast<const bf16x8*>(sB + tile_off(rb, ch));
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
            }
        }
    };

    load_step(0);
    store_step(0);
    __syncthreads();
    for (int64_t kb = 0; kb < KB; ++kb) {
        const int stage = (int)(kb & 1);
        if (kb + 1 < KB) load_step(kb + 1);
        mfma_step(lds + stage * FSTAGE, lds + stage * FSTAGE + 32768, 4);
        if (kb + 1 < KB) store_step(stage ^ 1);
        __syncthreads();
    }

    // LoRA: acc += (s T) B^T, rank chunks of 64 staged through stage 0 (Ts holds s * T)
    if (r > 0) {
        for (int rc = 0; rc < r; rc += 64) {
            uint8_t* sT = lds;
            uint8_t* sB = lds + 32768;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int qi = tid + 256 * i;
                const int row = qi >> 3, c = qi & 7;
                const int col = rc + 8 * c;
                const int64_t gm = m0 + row, gn = n0 + row;
                uint4 tv = make_uint4(0, 0, 0, 0), bv = make_uint4(0, 0, 0, 0);
                if (col < r) {
                    if (gm < M) tv = *reinterpret_cast<const uint4*>(Ts + gm * r + col);
                    if (gn < N) bv = *reinterpret_cast<const uint4*>(Bl + gn * r + col);
                }
                *reinterpret_cast<uint4*>(sT + tile_off(row, c)) = tv;
                *reinterpret_cast<uint4*>(sB + tile_off(row, c)) = bv;
            }
            __syncthreads();
            const int left = r - rc;
            mfma_step(sT, sB, left >= 64 ? 4 : (left + 15) / 16);
            __syncthreads();
        }
    }

    // store bf16
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t col = n0 + wn * 128 + j * 32 + (lane & 31);
#pragma unroll
            for (int reg = 0; reg < 16; ++reg) {
                const int64_t row = m0 + wm * 128 + i * 32 + 8 * (reg >> 2) + 4 * (lane >> 5) + (reg & 3);
                if (row < M && col < N) Y[row * N + col] = f32_to_bf16(acc[i][j][reg]);
            }
        }
}

static bool g_fwd_attr = false, g_bwd_attr = false;

FusedEvents& fused_events() {
    static thread_local FusedEvents ev;
    return ev;
}

// Launch `fn` between the armed profiling events (if any), then disarm.
template <typename F>
static hipError_t with_events(hipStream_t st, F&& fn) {
    FusedEvents& ev = fused_events();
    const FusedEvents armed = ev;
    ev = FusedEvents{};
    if (armed.start) {
        hipError_t e = hipEventRecord(armed.start, st);
        if (e != hipSuccess) return e;
    }
    hipError_t e = fn();
    if (e != hipSuccess) return e;
    if (armed.stop) return hipEventRecord(armed.stop, st);
    return hipSuccess;
}

hipError_t launch_fused_fwd(const WeightView& W, const uint16_t* X, int64_t M, const uint16_t* Ts,
                            const uint16_t* Bl, int r, uint16_t* Y, const Nf4Table& tab,
                            hipStream_t st) {
    if (M == 0 || W.rows == 0) return hipSuccess;
    if (!g_fwd_attr) {
        hipError_t e = hipFuncSetAttribute((const void*)k_fused_fwd,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, FLDS);
        if (e != hipSuccess) return e;
        g_fwd_attr = true;
    }
    dim3 grid((unsigned)((W.rows + FT - 1) / FT), (unsigned)((M + FT - 1) / FT));
    return with_events(st, [&] {
        hipLaunchKernelGGL(k_fused_fwd, grid, dim3(256), FLDS, st, W.codes, W.q, W.c2, W.mean,
                           W.rows, W.cols, X, M, Ts, Bl, r, Y, tab);
        return hipGetLastError();
    });
}

// ---------------------------------------------------------------------------
// Backward dX: tile (256 tokens) x (256 input features), contraction over N in
// steps of 64 output rows of W.  Lane t dequantizes row n = 64-step + t/4,
// NF4 block (t % 4) of the tile's 4 K-blocks, and scatters the 64 bf16 values
// into the transposed tile so that MFMA B fragments are 16-byte LDS reads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_fused_bwd_dx(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ qc,
                    const float* __restrict__ c2, const float* __restrict__ mean_p, int64_t N,
                    int64_t K, const uint16_t* __restrict__ dY, int64_t M,
                    const uint16_t* __restrict__ Us, const uint16_t* __restrict__ Al, int r,
                    uint16_t* __restrict__ dX, Nf4Table tab) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t k0 = (int64_t)blockIdx.x * FT, m0 = (int64_t)blockIdx.y * FT;
    const int64_t KB = K >> 6;
    const int64_t NB = (N + 63) >> 6;
    const float mean = *mean_p;

    const int nl = tid >> 2, jb = tid & 3;          // this lane's (row in step, K-block in tile)
    const int64_t kbi = (k0 >> 6) + jb;

    uint4 gr[8];
    uint4 wc0 = make_uint4(0, 0, 0, 0), wc1 = make_uint4(0, 0, 0, 0);
    uint32_t qb = 0;
    float c2v = 0.0f;
    bool wvalid = false;

    auto load_step = [&](int64_t nb) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int qi = tid + 256 * i;
            const int row = qi >> 3, c = qi & 7;
            const int64_t gm = m0 + row, gn = nb * 64 + 8 * c;
            gr[i] = (gm < M && gn < N) ? *reinterpret_cast<const uint4*>(dY + gm * N + gn)
                                       : make_uint4(0, 0, 0, 0);
        }
        const int64_t n = nb * 64 + nl;
        wvalid = (n < N) && (kbi < KB);
        if (wvalid) {
            const uint8_t* p = codes + n * (K >> 1) + kbi * 32;
            wc0 = *reinterpret_cast<const uint4*>(p);
            wc1 = *reinterpret_cast<const uint4*>(p + 16);
            qb = qc[n * KB + kbi];
            c2v = c2[(n * KB + kbi) >> 8];
        } else {
            wc0 = make_uint4(0, 0, 0, 0);
            wc1 = make_uint4(0, 0, 0, 0);
        }
    };
    auto store_step = [&](int stage) {
        uint8_t* sG = lds + stage * FSTAGE;
        uint8_t* sW = sG + 32768;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int qi = tid + 256 * i;
            const int row = qi >> 3, c = qi & 7;
            *reinterpret_cast<uint4*>(sG + tile_off(row, c)) = gr[i];
        }
        const float c1p = wvalid ? decode_c1(qb, c2_step(c2v), mean) : 0.0f;
        const ScaledTable stb = make_scaled_table(tab, c1p);
        const uint32_t words[8] = {wc0.x, wc0.y, wc0.z, wc0.w, wc1.x, wc1.y, wc1.z, wc1.w};
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            uint32_t o[4];
            decode8(stb, words[c], o);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int k = jb * 64 + c * 8 + e;
                const uint16_t h = (uint16_t)(o[e >> 1] >> (16 * (e & 1)));
                *reinterpret_cast<uint16_t*>(sW + ttile_off(k, nl)) = h;
            }
        }
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

    // A fragments from a row-major [256][64] tile, B fragments from the transposed tile
    auto mfma_step = [&](const uint8_t* sA, const uint8_t* sBt, int nsub) {
#pragma unroll
        for (int sub = 0; sub < 4; ++sub) {
            if (sub < nsub) {
                const int ch = 2 * sub + (lane >> 5);
                bf16x8 a[4], b[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ra = wm * 128 + i * 32 + (lane & 31);
                    a[i] = *reinterpret_cast<const bf16x8*>(sA + tile_off(ra, ch));
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int kk = wn * 128 + j * 32 + (lane & 31);
                    b[j] = *reinterpret_cast<const bf16x8*>(sBt + ttile_off(kk, ch * 8));
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
            }
        }
    };

    load_step(0);
    store_step(0);
    __syncthreads();
    for (int64_t nb = 0; nb < NB; ++nb) {
        const int stage = (int)(nb & 1);
        if (nb + 1 < NB) load_step(nb + 1);
        mfma_step(lds + stage * FSTAGE, lds + stage * FSTAGE + 32768, 4);
        if (nb + 1 < NB) store_step(stage ^ 1);
        __syncthreads();
    }

    // LoRA: acc += (s U) A, Us [M x r] row-major holds s * U, A [r x K] row-major
    if (r > 0) {
        for (int rc = 0; rc < r; rc += 64) {
            uint8_t* sU = lds;
            uint8_t* sA = lds + 32768;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int qi = tid + 256 * i;
                // U tile: row = token, 8 chunks of 8 ranks
                {
                    const int row = qi >> 3, c = qi & 7;
                    const int col = rc + 8 * c;
                    const int64_t gm = m0 + row;
                    uint4 v = make_uint4(0, 0, 0, 0);
                    if (col < r && gm < M) v = *reinterpret_cast<const uint4*>(Us + gm * r + col);
                    *reinterpret_cast<uint4*>(sU + tile_off(row, c)) = v;
                }
                // A tile transposed: rank j = qi / 32, 8 features per chunk
                {
                    const int j = qi >> 5, c = qi & 31;
                    const int64_t gk = k0 + 8 * c;
                    uint4 v = make_uint4(0, 0, 0, 0);
                    if (rc + j < r && gk < K) v = *reinterpret_cast<const uint4*>(Al + (int64_t)(rc + j) * K + gk);
                    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const uint16_t h = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
                        *reinterpret_cast<uint16_t*>(sA + ttile_off(8 * c + e, j)) = h;
                    }
                }
            }
            __syncthreads();
            const int left = r - rc;
            mfma_step(sU, sA, left >= 64 ? 4 : (left + 15) / 16);
            __syncthreads();
        }
    }

#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t col = k0 + wn * 128 + j * 32 + (lane & 31);
#pragma unroll
            for (int reg = 0; reg < 16; ++reg) {
                const int64_t row = m0 + wm * 128 + i * 32 + 8 * (reg >> 2) + 4 * (lane >> 5) + (reg & 3);
                if (row < M && col < K) dX[row * K + col] = f32_to_bf16(acc[i][j][reg]);
            }
        }
}

hipError_t launch_fused_bwd_dx(const WeightView& W, const uint16_t* dY, int64_t M, const uint16_t* Us,
                               const uint16_t* Al, int r, uint16_t* dX, const Nf4Table& tab,
                               hipStream_t st) {
    if (M == 0 || W.cols == 0) return hipSuccess;
    if (!g_bwd_attr) {
        hipError_t e = hipFuncSetAttribute((const void*)k_fused_bwd_dx,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, FLDS);
        if (e != hipSuccess) return e;
        g_bwd_attr = true;
    }
    dim3 grid((unsigned)((W.cols + FT - 1) / FT), (unsigned)((M + FT - 1) / FT));
    return with_events(st, [&] {
        hipLaunchKernelGGL(k_fused_bwd_dx, grid, dim3(256), FLDS, st, W.codes, W.q, W.c2, W.mean,
                           W.rows, W.cols, dY, M, Us, Al, r, dX, tab);
        return hipGetLastError();
    });
}

// ---------------------------------------------------------------------------
// Few-token dequant-GEMV (M <= 16): HBM-bound stream over the packed weight.
// Workgroup = 16 rows of W x all of K; wave w takes NF4 blocks b = w mod 4.
// Per block a lane holds 16 codes of row n0 + lane%16 (k-group lane/16) and
// the matching X values; two v_mfma_f32_16x16x32_bf16 on the unscaled bf16
// levels (LDS table) give the block's partial dot, which the block's decoded
// constant then scales into the fp32 accumulator.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
constexpr int GV_ROWS = 16;
constexpr int GV_UNROLL = 4;
constexpr int GV_MAX_STEPS = 64;

__global__ __launch_bounds__(256) void k_fused_gemv(const uint8_t* __restrict__ codes,
                                                    const uint8_t* __restrict__ qc,
                                                    const float* __restrict__ c2,
                                                    const float* __restrict__ mean_p, int64_t N,
                                                    int64_t K, const uint16_t* __restrict__ X, int M,
                                                    const uint16_t* __restrict__ Ts,
                                                    const uint16_t* __restrict__ Bl, int r,
                                                    uint16_t* __restrict__ Y, Nf4Table tab) {
    __shared__ uint16_t s_lut[16];
    __shared__ float s_step[GV_MAX_STEPS];
    __shared__ float s_red[4][16][17];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t n0 = (int64_t)blockIdx.x * GV_ROWS;
    const int64_t KB = K >> 6;
    const int64_t n2 = (N * KB + 255) >> 8;
    const float mean = *mean_p;

#pragma unroll
    for (int j = 0; j < 16; ++j)
        if (tid == j) s_lut[j] = f32_to_bf16(tab.lv[j]);
    // second-level steps fp32(c2/448) for the 256-blocks this tile touches
    const int64_t sidx0 = (n0 * KB) >> 8;
    const int64_t nlast = (n0 + GV_ROWS < N ? n0 + GV_ROWS : N) - 1;
    const int64_t scount = ((nlast * KB + KB - 1) >> 8) - sidx0 + 1;
    const bool step_lds = scount <= GV_MAX_STEPS;
    if (step_lds)
        for (int i = tid; i < scount; i += 256)
            if (sidx0 + i < n2) s_step[i] = c2_step(c2[sidx0 + i]);
    __syncthreads();

    const int nl = lane & 15, g = lane >> 4;
    const int64_t n = n0 + nl;
    const bool nvalid = n < N;
    const uint8_t* rowc = codes + n * (K >> 1) + g * 8;
    const int m = lane & 15;
    const bool mvalid = m < M;
    const uint16_t* xrow = X + (int64_t)m * K + g * 16;

    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t b0 = wave; b0 < KB; b0 += 4 * GV_UNROLL) {
        uint2 cw[GV_UNROLL];
        uint4 xa[GV_UNROLL], xb[GV_UNROLL];
        uint32_t qv[GV_UNROLL];
        float stp[GV_UNROLL];
#pragma unroll
        for (int u = 0; u < GV_UNROLL; ++u) {
            const int64_t b = b0 + 4 * u;
            const bool ok = b < KB;
            cw[u] = (ok && nvalid) ? *reinterpret_cast<const uint2*>(rowc + b * 32) : make_uint2(0, 0);
            xa[u] = (ok && mvalid) ? *reinterpret_cast<const uint4*>(xrow + b * 64) : make_uint4(0, 0, 0, 0);
            xb[u] = (ok && mvalid) ? *reinterpret_cast<const uint4*>(xrow + b * 64 + 8) : make_uint4(0, 0, 0, 0);
            const int64_t ci = n * KB + b;
            qv[u] = (ok && nvalid) ? qc[ci] : 0u;
            stp[u] = (ok && nvalid) ? (step_lds ? s_step[(ci >> 8) - sidx0] : c2_step(c2[ci >> 8])) : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < GV_UNROLL; ++u) {
            uint32_t bw[8];
            const uint32_t words[2] = {cw[u].x, cw[u].y};
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t lo = s_lut[(words[h] >> (8 * e)) & 0xFu];
                    const uint32_t hi = s_lut[(words[h] >> (8 * e + 4)) & 0xFu];
                    bw[4 * h + e] = lo | (hi << 16);
                }
            const bf16x8v a0 = __builtin_bit_cast(bf16x8v, xa[u]);
            const bf16x8v a1 = __builtin_bit_cast(bf16x8v, xb[u]);
            const bf16x8v b0v = __builtin_bit_cast(bf16x8v, make_uint4(bw[0], bw[1], bw[2], bw[3]));
            const bf16x8v b1v = __builtin_bit_cast(bf16x8v, make_uint4(bw[4], bw[5], bw[6], bw[7]));
            f32x4 part = {0.0f, 0.0f, 0.0f, 0.0f};
            part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0v, part, 0, 0, 0);
            part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1v, part, 0, 0, 0);
            const float c1p = decode_c1(qv[u], stp[u], mean);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = __fmaf_rn(c1p, part[i], acc[i]);
        }
    }
    // lane holds rows 4g..4g+3 (tokens) of column nl
#pragma unroll
    for (int i = 0; i < 4; ++i) s_red[wave][4 * g + i][nl] = acc[i];
    __syncthreads();
    const int ti = tid >> 4, tj = tid & 15;
    const int64_t on = n0 + tj;
    if (ti < M && on < N) {
        float y = ((s_red[0][ti][tj] + s_red[1][ti][tj]) + s_red[2][ti][tj]) + s_red[3][ti][tj];
        const uint16_t* trow = Ts + (int64_t)ti * r;
        const uint16_t* brow = Bl + on * r;
        for (int q = 0; q < r; ++q) y += bf16_to_f32(trow[q]) * bf16_to_f32(brow[q]);
        Y[(int64_t)ti * N + on] = f32_to_bf16(y);
    }
}

hipError_t launch_fused_gemv(const WeightView& W, const uint16_t* X, int64_t M, const uint16_t* Ts,
                             const uint16_t* Bl, int r, uint16_t* Y, const Nf4Table& tab,
                             hipStream_t st) {
    if (M == 0 || W.rows == 0) return hipSuccess;
    dim3 grid((unsigned)((W.rows + GV_ROWS - 1) / GV_ROWS));
    return with_events(st, [&] {
        hipLaunchKernelGGL(k_fused_gemv, grid, dim3(256), 0, st, W.codes, W.q, W.c2, W.mean,
                           W.rows, W.cols, X, (int)M, Ts, Bl, r, Y, tab);
        return hipGetLastError();
    });
}

}  // namespace nf4
