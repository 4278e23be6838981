// lora.hip -- the rank-r adapter products of the QLoRA layer.
//
// "Paged optimizers, and QLoRA end to end" (zerotofrontier.app "sft/peft"):
// a bf16 LoRA adapter on every linear, r = 64, alpha = 16, gradients only into
// the adapters.  With s = alpha / r the layer needs
//   T = X A^T (forward, saved), U = dY B, dA = s U^T X, dB = s dY^T T.
// They are skinny products (one side is r <= 128), a few percent of the
// layer's flops.  One LDS-staged MFMA kernel covers all four: each operand is
// either contraction-contiguous in memory (copied to LDS in 16-byte chunks) or
// contraction-strided (transposed into LDS with 16-bit writes).
#include "launch.h"

namespace nf4 {

constexpr int LT = 64;      // output tile edge
constexpr int LKC = 64;     // contraction chunk

// LDS tile [64 rows][64 bf16], 16-byte chunk c of row i stored at c ^ (i & 7).
__device__ __forceinline__ int lds_off(int row, int chunk) {
    return row * 128 + ((chunk ^ (row & 7)) << 4);
}

// Stage rows [i0, i0+64) x contraction [p0, p0+64) of an operand into LDS.
//   trans == false: element (i, p) at src[i * ld + p]  (rows contiguous along p)
//   trans == true : element (i, p) at src[p * ld + i]  (rows contiguous along i)
__device__ __forceinline__ void stage_operand(uint8_t* sm, const uint16_t* __restrict__ src, bool trans,
                                              int64_t ld, int64_t rows, int64_t P, int64_t i0,
                                              int64_t p0, int tid) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int qi = tid + 256 * it;     // 512 chunks of 8 elements
        const int a = qi >> 3, c = qi & 7;
        if (!trans) {
            // row a, contraction chunk c
            const int64_t gi = i0 + a, gp = p0 + 8 * c;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (gi < rows && gp < P) v = *reinterpret_cast<const uint4*>(src + gi * ld + gp);
            *reinterpret_cast<uint4*>(sm + lds_off(a, c)) = v;
        } else {
            // contraction index a, rows 8c .. 8c+7
            const int64_t gp = p0 + a, gi = i0 + 8 * c;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (gp < P && gi < rows) v = *reinterpret_cast<const uint4*>(src + gp * ld + gi);
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int row = 8 * c + e;
                const uint16_t h = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
                *reinterpret_cast<uint16_t*>(sm + lds_off(row, a >> 3) + ((a & 7) << 1)) = h;
            }
        }
    }
}

__global__ __launch_bounds__(256) void k_lora_gemm(const uint16_t* __restrict__ A, bool a_trans,
                                                   const uint16_t* __restrict__ B, bool b_trans,
                                                   int64_t Mc, int64_t Nc, int64_t P, float scale,
                                                   void* __restrict__ C, bool c_f32,
                                                   uint16_t* __restrict__ C2, float scale2) {
    __shared__ __attribute__((aligned(16))) uint8_t sA[LT * 128];
    __shared__ __attribute__((aligned(16))) uint8_t sB[LT * 128];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wi = wave >> 1, wj = wave & 1;
    const int64_t i0 = (int64_t)blockIdx.y * LT, j0 = (int64_t)blockIdx.x * LT;
    const int64_t lda = a_trans ? Mc : P;
    const int64_t ldb = b_trans ? Nc : P;
    f32x16 acc = {};
    for (int64_t p0 = 0; p0 < P; p0 += LKC) {
        stage_operand(sA, A, a_trans, lda, Mc, P, i0, p0, tid);
        stage_operand(sB, B, b_trans, ldb, Nc, P, j0, p0, tid);
        __syncthreads();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int ra = wi * 32 + (lane & 31), rb = wj * 32 + (lane & 31);
            const int ch = 2 * s + (lane >> 5);
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(sA + lds_off(ra, ch));
            const bf16x8 b = *reinterpret_cast<const bf16x8*>(sB + lds_off(rb, ch));
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
        }
        __syncthreads();
    }
    const int64_t col = j0 + wj * 32 + (lane & 31);
#pragma unroll
    for (int reg = 0; reg < 16; ++reg) {
        const int64_t row = i0 + wi * 32 + 8 * (reg >> 2) + 4 * (lane >> 5) + (reg & 3);
        if (row < Mc && col < Nc) {
            const float v = acc[reg] * scale;
            if (c_f32) reinterpret_cast<float*>(C)[row * Nc + col] = v;
            else reinterpret_cast<uint16_t*>(C)[row * Nc + col] = f32_to_bf16(v);
            if (C2) C2[row * Nc + col] = f32_to_bf16(acc[reg] * scale2);
        }
    }
}

hipError_t launch_lora_gemm(const uint16_t* A, bool a_trans, const uint16_t* B, bool b_trans,
                            int64_t Mc, int64_t Nc, int64_t P, float scale, void* C, bool c_f32,
                            uint16_t* C2, float scale2, hipStream_t s) {
    if (Mc == 0 || Nc == 0) return hipSuccess;
    dim3 grid((unsigned)((Nc + LT - 1) / LT), (unsigned)((Mc + LT - 1) / LT));
    hipLaunchKernelGGL(k_lora_gemm, grid, dim3(256), 0, s, A, a_trans, B, b_trans, Mc, Nc, P, scale,
                       C, c_f32, C2, scale2);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// T = X A^T for M <= 16 tokens: one workgroup per adapter row j; lanes stride
// over K in 8-element chunks, then a fixed-order reduction across the block.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_lora_t_small(const uint16_t* __restrict__ X,
                                                      const uint16_t* __restrict__ A, int M,
                                                      int64_t K, int r, uint16_t* __restrict__ T,
                                                      uint16_t* __restrict__ Ts, float s) {
    const int j = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float acc[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) acc[m] = 0.0f;
    const uint16_t* arow = A + (int64_t)j * K;
    for (int64_t k = (int64_t)tid * 8; k < K; k += 256 * 8) {
        const uint4 av = *reinterpret_cast<const uint4*>(arow + k);
        const uint32_t aw[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            if (m < M) {
                const uint4 xv = *reinterpret_cast<const uint4*>(X + (int64_t)m * K + k);
                const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
                float s = acc[m];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    s += bf16_lo(xw[e]) * bf16_lo(aw[e]);
                    s += bf16_hi(xw[e]) * bf16_hi(aw[e]);
                }
                acc[m] = s;
            }
        }
    }
    __shared__ float red[4][16];
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        float v = acc[m];
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
        if (lane == 0) red[wave][m] = v;
    }
    __syncthreads();
    if (tid < M) {
        const float v = (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
        T[(int64_t)tid * r + j] = f32_to_bf16(v);
        Ts[(int64_t)tid * r + j] = f32_to_bf16(v * s);
    }
}

hipError_t launch_lora_t_small(const uint16_t* X, const uint16_t* A, int64_t M, int64_t K, int r,
                               uint16_t* T, uint16_t* Ts, float s, hipStream_t st) {
    if (M == 0) return hipSuccess;
    hipLaunchKernelGGL(k_lora_t_small, dim3((unsigned)r), dim3(256), 0, st, X, A, (int)M, K, r, T,
                       Ts, s);
    return hipGetLastError();
}

}  // namespace nf4
