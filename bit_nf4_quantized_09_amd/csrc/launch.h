// launch.h -- host-side launchers for the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "nf4_common.h"
#include "tile_map.h"

namespace nf4 {

// Device view of a double-quantized NF4 weight (N x K, row-major).
struct WeightView {
    const uint8_t* codes;
    const uint8_t* q;
    const float* c2;
    const float* mean;
    int64_t rows;   // N
    int64_t cols;   // K
    const float* absmax;   // plain first-level constants (no double quantization), or null
};

// ---- codec ----------------------------------------------------------------
hipError_t launch_quantize(const void* w, bool w_bf16, int64_t n, uint8_t* codes, float* absmax,
                           const Nf4Table& tab, hipStream_t s);
size_t double_quantize_ws_bytes(int64_t n1);
// A batch of tensors for double quantization (up to DQB_MAX per launch pair), each of at
// most 2048 x 2048 constants: device pointers, sizes and the prefix counts of their
// 2048-constant chunks and encode groups.
constexpr int DQB_MAX = 32;
struct DqBatch {
    int count;
    const float* c1[DQB_MAX];
    uint8_t* q[DQB_MAX];
    float* c2[DQB_MAX];
    float* mean[DQB_MAX];
    int64_t n1[DQB_MAX];
    int64_t chunk0[DQB_MAX + 1];
    int64_t group0[DQB_MAX + 1];
    double* ws;                // chunk sums, chunk0[count] of them
};
constexpr int64_t DQB_MAX_N1 = (int64_t)2048 * 2048;
size_t double_quantize_batch_ws_bytes(int count, const int64_t* n1);
hipError_t launch_double_quantize_batch(int count, const float* const* c1, const int64_t* n1, uint8_t* const* q,
                                        float* const* c2, float* const* mean, double* ws, hipStream_t s);
hipError_t launch_double_quantize(const float* c1, int64_t n1, uint8_t* q, float* c2, float* mean,
                                  double* ws, hipStream_t s);
hipError_t launch_double_dequantize(const uint8_t* q, const float* c2, const float* mean, int64_t n1,
                                    float* out, hipStream_t s);
hipError_t launch_dequantize(const WeightView& W, void* out, bool out_bf16, const Nf4Table& tab,
                             hipStream_t s);

// ---- LoRA side products (bf16 operands, fp32 accumulation) ----------------
// C[i][j] = scale * sum_p Aop[i][p] * Bop[p][j] over p < P, i < Mc, j < Nc.
// a_trans == false: Aop is row-major [Mc x P] (lda = P);  true: stored [P x Mc] (lda = Mc).
// b_trans == false: Bop^T is row-major [Nc x P] (ldb = P); true: Bop stored [P x Nc] (ldb = Nc).
// C is bf16 or fp32, stored [Mc x Nc] or (c_trans) [Nc x Mc]; C2, if given, receives
// bf16(scale2 * sum) in the same layout.  `part` is fp32 workspace of
// skinny_partial_bytes(Mc, Nc, P) bytes for the split-contraction slices.  `pack`, if given
// (A direct only), receives A in the fused product's fragment order (tile_map.h:
// 512-row token tiles x 64-value steps, ld = P), written from the tiles the product stages
// anyway; with pack_even_odd each 16-byte piece holds its 8 values in the order 0, 2, 4, 6,
// 1, 3, 5, 7 (the order of the forward product's decoded weights).
size_t skinny_partial_bytes(int64_t Mc, int64_t Nc, int64_t P);
// A two-level constant decode (as launch_double_dequantize) that rides on the slice-sum
// launch of a rank-r product: extra workgroups of that launch write out[0 .. n1).
struct DqDecode {
    const uint8_t* q;
    const float* c2;
    const float* mean;
    int64_t n1;
    float* out;
};
// A both-strided product C = scale * A^T B (fp32 out, C transposed when c_trans): A is
// P x Mc and B is P x Nc, both row-major with the contraction P as rows (Mc, Nc multiples
// of 8, below 2^23); part holds skinny_partial_bytes(Mc, Nc, P).
struct TtProduct {
    const uint16_t* A;
    const uint16_t* B;
    int64_t Mc, Nc, P;
    float* part;
    float scale;
    float* C;
    bool c_trans;
};
// Kernel argument of one both-strided product: its operands, slice length and grid.
struct TtProblem {
    const uint16_t* A;
    const uint16_t* B;
    int64_t Mc, Nc, P, cps;
    float* part;
    int64_t gx, gy;           // column tiles, row tiles (slices are the third dimension)
};
// Two both-strided products in one launch (two workgroups per CU), then the slice sum of
// each; their partial regions must not overlap.
hipError_t launch_lora_tt_pair(const TtProduct& d0, const TtProduct& d1, hipStream_t s);
hipError_t launch_lora_gemm(const uint16_t* A, bool a_trans, const uint16_t* B, bool b_trans,
                            int64_t Mc, int64_t Nc, int64_t P, float* part, float scale, void* C,
                            bool c_f32, bool c_trans, uint16_t* C2, float scale2, hipStream_t s,
                            uint16_t* pack = nullptr, bool pack_even_odd = false,
                            const DqDecode* dq = nullptr);

// ---- profiling hook: events around the next fused launch on this thread ----
struct FusedEvents {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};
FusedEvents& fused_events();

// Launch `fn` between the armed profiling events (if any), then disarm.
template <typename F>
inline hipError_t with_events(hipStream_t st, F&& fn) {
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

// ---- fused dequant products -------------------------------------------------
// Y = X W'^T + Ts B^T, Ts = s T   (MFMA GEMM, dequantization fused into the W operand load).
// c1: the decoded first-level constants of W (launch_double_dequantize), one per 64-block.
hipError_t launch_fused_fwd(const WeightView& W, const float* c1, const uint16_t* Xpk, int64_t M, const uint16_t* Ts,
                            const uint16_t* Bl, int r, uint16_t* Y, void* split_ws, const Nf4Table& tab,
                            hipStream_t st);
// Whole forward for M <= 16 tokens (HBM-bound dequant-GEMV): Y = X W'^T + s (X A^T) B^T and
// T = X A^T, through fp32 partial sums per contraction slice (part: gemv_partial_bytes).
int64_t gemv_slices(int64_t M, int64_t K);
size_t gemv_partial_bytes(int64_t M, int64_t N, int64_t K, int r);
hipError_t launch_fused_gemv(const WeightView& W, const uint16_t* X, int64_t M, const uint16_t* Al,
                             const uint16_t* Bl, int r, float s, uint16_t* Y, uint16_t* T, float* part,
                             const Nf4Table& tab, hipStream_t st);
// dX = dY W' + Us A, Us = s U   (contraction over N, W' used transposed)
hipError_t launch_fused_bwd_dx(const WeightView& W, const float* c1, const uint16_t* dYpk, int64_t M, const uint16_t* Us,
                               const uint16_t* Al, int r, uint16_t* dX, void* split_ws, const Nf4Table& tab,
                               hipStream_t st);

// ---- codebook statistics ----------------------------------------------------
// Layout shared with nf4_codebook_stats_t of the C ABI.
struct CodebookStats {
    int64_t count[16];
    double sum_x[16];
    double sse;
};
size_t codebook_stats_ws_bytes(int64_t n);
// part: codebook_stats_ws_bytes(n) bytes of workspace; out: device CodebookStats.
hipError_t launch_codebook_stats(const void* w, bool w_bf16, int64_t n, const uint8_t* codes,
                                 const float* absmax, const Nf4Table& tab, CodebookStats* part,
                                 CodebookStats* out, hipStream_t s);

// ---- adapter optimizer step (AdamW over fp32 state) -------------------------
// Scalars of one step, formed on the host: omb1 = 1 - b1, omb2 = 1 - b2,
// step_size = lr / (1 - b1^t), inv_sqrt_bc2 = 1 / sqrt(1 - b2^t), decay = 1 - lr wd.
struct AdamwScalars {
    float b1, omb1, b2, omb2, step_size, inv_sqrt_bc2, eps, decay;
};
// p, g, m, v: n fp32 values (16-byte aligned); pbf: bf16 copy of p or null (8-byte aligned).
hipError_t launch_adamw(float* p, const float* g, float* m, float* v, uint16_t* pbf, int64_t n,
                        const AdamwScalars& k, hipStream_t s);

// ---- rank-r truncated SVD (randomized subspace iteration) and LoftQ initialisation ----
constexpr int LR_MAX = 96;          // sketch width l at most (l >= r)
constexpr int LR_MAX_SLICES = 16;   // contraction slices of a tall product at most
size_t lowrank_ws_bytes(int64_t N, int64_t K, int l, int r);
// E (N x K fp32) ~ U diag(S) V^T: U N x r, S r, V K x r (fp32), from the K x l Gaussian omega
// and `power` subspace iterations
hipError_t launch_lowrank_svd(const float* E, int64_t N, int64_t K, int r, int l, int power, const float* omega,
                              float* U, float* S, float* V, void* ws, hipStream_t s);
size_t loftq_ws_bytes(int64_t N, int64_t K, int l, int r);
hipError_t launch_loftq(const float* W, int64_t N, int64_t K, int r, float gamma, int iters, int l, int power,
                        const float* omega, uint8_t* codes, uint8_t* q, float* c2, float* mean, uint16_t* A,
                        uint16_t* B, double* err, void* ws, const Nf4Table& tab, hipStream_t s);

}  // namespace nf4
