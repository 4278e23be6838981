// lora.hip -- the rank-r adapter products of the QLoRA layer.
//
// "Paged optimizers, and QLoRA end to end" (zerotofrontier.app "sft/peft"):
// a bf16 LoRA adapter on every linear, r = 64, alpha = 16, gradients only into
// the adapters.  With s = alpha / r the layer needs
//   T = X A^T (forward, saved), U = dY B, dA = s U^T X, dB = s dY^T T.
// They are skinny products (one side is r <= 128), a few percent of the
// layer's flops, but they stream the big activations once more, so they must
// run at bandwidth.  One LDS-staged MFMA kernel covers all four: each operand
// is either contraction-contiguous in memory (16-byte chunks straight into
// LDS) or contraction-strided (8 x 8 blocks transposed in registers with byte
// permutes).  The contraction is split across workgroups so that the grid
// fills the chip; a second pass sums the fp32 slices in a fixed order, so the
// result is deterministic.
#include "launch.h"

namespace nf4 {

constexpr int SK_BM = 128;   // rows of C per workgroup (4 waves x 32)
constexpr int SK_BN = 64;    // columns of C per workgroup (2 MFMA tiles of 32)
constexpr int SK_PC = 64;    // contraction chunk per pipeline step
constexpr int SK_A_BYTES = SK_BM * 128;
constexpr int SK_B_BYTES = SK_BN * 128;
constexpr int SK_STAGE = SK_A_BYTES + SK_B_BYTES;

// LDS tile [rows][64 bf16], 16-byte chunk c of row i stored at c ^ (i & 7).
__device__ __forceinline__ int lds_off(int row, int chunk) {
    return row * 128 + ((chunk ^ (row & 7)) << 4);
}

// 8 x 8 transpose of 16-bit values: in[i] holds row i (8 values), out[j] column j.
__device__ __forceinline__ void transpose8x8(const uint4 in[8], uint4 out[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 lo = in[2 * q], hi = in[2 * q + 1];
            const uint32_t a = (j >> 1) == 0 ? lo.x : (j >> 1) == 1 ? lo.y : (j >> 1) == 2 ? lo.z : lo.w;
            const uint32_t b = (j >> 1) == 0 ? hi.x : (j >> 1) == 1 ? hi.y : (j >> 1) == 2 ? hi.z : hi.w;
            w[q] = __builtin_amdgcn_perm(b, a, sel);
        }
        out[j] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// Operand staging into an LDS tile [ROWS][64 contraction] for one chunk.
//   TRANS == false: element (i, p) at src[i * ld + p]   (16-byte chunks along p)
//   TRANS == true : element (i, p) at src[p * ld + i]   (8 x 8 blocks, transposed in registers)
// `slot` numbers this thread's share: slots [0, NSLOT) of a tile are spread over the
// workgroup; a thread owns at most one transposed block or CPT contiguous chunks.
template <int ROWS, bool TRANS>
struct Stager {
    static constexpr int NBLK = (ROWS / 8) * 8;          // 8x8 blocks per tile (transposed)
    static constexpr int CPT = ROWS * 8 / 256;           // 16-byte chunks per thread (direct)
    uint4 r[TRANS ? 8 : CPT];

    __device__ __forceinline__ void load(const uint16_t* __restrict__ src, int64_t ld, int64_t rows,
                                         int64_t P, int64_t i0, int64_t p0, int slot) {
        if constexpr (TRANS) {
            if (slot < NBLK) {
                const int rb = slot >> 3, pb = slot & 7;
                const int64_t gi = i0 + rb * 8;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int64_t gp = p0 + pb * 8 + e;
                    r[e] = (gp < P && gi < rows) ? *reinterpret_cast<const uint4*>(src + gp * ld + gi)
                                                 : make_uint4(0, 0, 0, 0);
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < CPT; ++t) {
                const int q = slot + 256 * t;
                const int a = q >> 3, c = q & 7;
                const int64_t gi = i0 + a, gp = p0 + 8 * c;
                r[t] = (gi < rows && gp < P) ? *reinterpret_cast<const uint4*>(src + gi * ld + gp)
                                             : make_uint4(0, 0, 0, 0);
            }
        }
    }
    __device__ __forceinline__ void store(uint8_t* sm, int slot) {
        if constexpr (TRANS) {
            if (slot < NBLK) {
                const int rb = slot >> 3, pb = slot & 7;
                uint4 t[8];
                transpose8x8(r, t);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    *reinterpret_cast<uint4*>(sm + lds_off(rb * 8 + j, pb)) = t[j];
            }
        } else {
#pragma unroll
            for (int t = 0; t < CPT; ++t) {
                const int q = slot + 256 * t;
                *reinterpret_cast<uint4*>(sm + lds_off(q >> 3, q & 7)) = r[t];
            }
        }
    }
};

// Partial C[i][j] = sum over this workgroup's contraction slice of Aop[i][p] * Bop[p][j],
// written as fp32 to part[z][i][j].  Grid: (col tiles, row tiles, slices).
template <bool ATR, bool BTR>
__global__ __launch_bounds__(256) void k_skinny(const uint16_t* __restrict__ A,
                                                const uint16_t* __restrict__ B, int64_t Mc,
                                                int64_t Nc, int64_t P, int64_t chunks_per_slice,
                                                float* __restrict__ part) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * SK_STAGE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t i0 = (int64_t)blockIdx.y * SK_BM, j0 = (int64_t)blockIdx.x * SK_BN;
    const int64_t nchunks = (P + SK_PC - 1) / SK_PC;
    const int64_t c0 = (int64_t)blockIdx.z * chunks_per_slice;
    const int64_t c1 = (c0 + chunks_per_slice < nchunks) ? c0 + chunks_per_slice : nchunks;
    const int64_t lda = ATR ? Mc : P;
    const int64_t ldb = BTR ? Nc : P;
    // thread roles: transposed A uses slots 0..127, transposed B slots 128..191
    const int aslot = tid;
    const int bslot = ATR ? tid - 128 : tid;

    Stager<SK_BM, ATR> sa;
    Stager<SK_BN, BTR> sb;
    f32x16 acc0 = {}, acc1 = {};

    auto load = [&](int64_t c) {
        sa.load(A, lda, Mc, P, i0, c * SK_PC, aslot);
        if (!BTR || bslot >= 0) sb.load(B, ldb, Nc, P, j0, c * SK_PC, BTR ? bslot : tid);
    };
    auto store = [&](int stage) {
        uint8_t* base = lds + stage * SK_STAGE;
        sa.store(base, aslot);
        if (!BTR || bslot >= 0) sb.store(base + SK_A_BYTES, BTR ? bslot : tid);
    };

    if (c0 < c1) {
        load(c0);
        store(0);
        __syncthreads();
        for (int64_t c = c0; c < c1; ++c) {
            const int stage = (int)((c - c0) & 1);
            if (c + 1 < c1) load(c + 1);
            const uint8_t* sA = lds + stage * SK_STAGE;
            const uint8_t* sB = sA + SK_A_BYTES;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int ch = 2 * s + (lane >> 5);
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(sA + lds_off(wave * 32 + (lane & 31), ch));
                const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(sB + lds_off(lane & 31, ch));
                const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(sB + lds_off(32 + (lane & 31), ch));
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, acc1, 0, 0, 0);
            }
            if (c + 1 < c1) store(stage ^ 1);
            __syncthreads();
        }
    }
    float* out = part + (int64_t)blockIdx.z * Mc * Nc;
#pragma unroll
    for (int reg = 0; reg < 16; ++reg) {
        const int64_t row = i0 + wave * 32 + 8 * (reg >> 2) + 4 * (lane >> 5) + (reg & 3);
        const int64_t col0 = j0 + (lane & 31), col1 = col0 + 32;
        if (row < Mc) {
            if (col0 < Nc) out[row * Nc + col0] = acc0[reg];
            if (col1 < Nc) out[row * Nc + col1] = acc1[reg];
        }
    }
}

// Fixed-order sum of the slices: v = sum_z part[z][i][j];  C = scale * v (bf16 or fp32,
// [i][j] or transposed [j][i]);  C2 = bf16(scale2 * v) when given.
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ part, int S,
                                                       int64_t Mc, int64_t Nc, float scale,
                                                       void* __restrict__ C, bool c_f32,
                                                       bool c_trans, uint16_t* __restrict__ C2,
                                                       float scale2) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = Mc * Nc;
    if (i >= total) return;
    float v = 0.0f;
    for (int z = 0; z < S; ++z) v += part[(int64_t)z * total + i];
    const int64_t row = i / Nc, col = i - row * Nc;
    const int64_t dst = c_trans ? col * Mc + row : i;
    if (c_f32) reinterpret_cast<float*>(C)[dst] = v * scale;
    else reinterpret_cast<uint16_t*>(C)[dst] = f32_to_bf16(v * scale);
    if (C2) C2[dst] = f32_to_bf16(v * scale2);
}

void skinny_plan(int64_t Mc, int64_t Nc, int64_t P, int* slices, int64_t* chunks_per_slice) {
    const int64_t tiles = ((Mc + SK_BM - 1) / SK_BM) * ((Nc + SK_BN - 1) / SK_BN);
    const int64_t nchunks = (P + SK_PC - 1) / SK_PC;
    if (tiles <= 0 || nchunks <= 0) {      // empty output or empty contraction: one slice
        *slices = 1;
        *chunks_per_slice = 0;
        return;
    }
    int64_t S = (512 + tiles - 1) / tiles;
    const int64_t smax = nchunks / 4 > 1 ? nchunks / 4 : 1;
    if (S > smax) S = smax;
    if (S < 1) S = 1;
    int64_t cps = nchunks > 0 ? (nchunks + S - 1) / S : 0;
    if (cps > 0) S = (nchunks + cps - 1) / cps;
    *slices = (int)S;
    *chunks_per_slice = cps;
}

size_t skinny_partial_bytes(int64_t Mc, int64_t Nc, int64_t P) {
    int S;
    int64_t cps;
    skinny_plan(Mc, Nc, P, &S, &cps);
    return ((size_t)S * (size_t)Mc * (size_t)Nc * 4 + 255) & ~(size_t)255;
}

hipError_t launch_lora_gemm(const uint16_t* A, bool a_trans, const uint16_t* B, bool b_trans,
                            int64_t Mc, int64_t Nc, int64_t P, float* part, float scale, void* C,
                            bool c_f32, bool c_trans, uint16_t* C2, float scale2, hipStream_t s) {
    if (Mc == 0 || Nc == 0) return hipSuccess;
    int S;
    int64_t cps;
    skinny_plan(Mc, Nc, P, &S, &cps);
    dim3 grid((unsigned)((Nc + SK_BN - 1) / SK_BN), (unsigned)((Mc + SK_BM - 1) / SK_BM), (unsigned)S);
    if (!a_trans && !b_trans)
        hipLaunchKernelGGL((k_skinny<false, false>), grid, dim3(256), 0, s, A, B, Mc, Nc, P, cps, part);
    else if (!a_trans && b_trans)
        hipLaunchKernelGGL((k_skinny<false, true>), grid, dim3(256), 0, s, A, B, Mc, Nc, P, cps, part);
    else if (a_trans && b_trans)
        hipLaunchKernelGGL((k_skinny<true, true>), grid, dim3(256), 0, s, A, B, Mc, Nc, P, cps, part);
    else
        hipLaunchKernelGGL((k_skinny<true, false>), grid, dim3(256), 0, s, A, B, Mc, Nc, P, cps, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t total = Mc * Nc;
    hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, part, S,
                       Mc, Nc, scale, C, c_f32, c_trans, C2, scale2);
    return hipGetLastError();
}

}  // namespace nf4
