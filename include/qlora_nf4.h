/*
 * qlora_nf4.h -- C ABI of the MI355X (gfx950) QLoRA NF4 linear-layer library.
 *
 * The frozen weight of a linear layer is stored as blockwise-absmax NF4 with
 * double-quantized constants, and the layer runs
 *     Y = X dequant(W)^T + (alpha/r) (X A^T) B^T
 * forward, with dX, dA and dB backward (no gradient for W).
 *
 * Passages that define the operations (page title, section):
 *   [BQ]  zerotofrontier.app "sft/peft", "Block-wise quantization in one page"
 *   [NF]  same page, "NF4, derived from normal quantiles"
 *   [DQ]  same page, "Double quantization" (stubs double_quantize / double_dequantize)
 *   [E2E] same page, "Paged optimizers, and QLoRA end to end" (r, alpha, gradient flow)
 *   [RW]  same page, "The real way" (two codes per byte, dequant fused into the matmul)
 *   [PT]  prism.theerrors.in QLoRA explainer, "Putting it together" (layer formula)
 *   [PO]  zerotofrontier.app "sft/peft", "Paged optimizers, and QLoRA end to end"
 *         (only the adapters learn; their Adam states are paged between GPU and host
 *         RAM; learning rates).  The update itself is Adam (Kingma & Ba, ICLR 2015,
 *         Algorithm 1) with decoupled weight decay (Loshchilov & Hutter, ICLR 2019).
 *
 * Conventions shared by every entry point:
 *   - Memory: every pointer argument is device memory unless stated; the
 *     caller owns all buffers.  The library never allocates or frees device
 *     memory and keeps no pointer after a call returns.  (The one device memory
 *     of its own is the fixed scratch array of qlora_linear_fwd_noalloc, part of
 *     the library's code object on each GPU it runs on.)
 *   - Streams: `stream` is a hipStream_t (NULL = the default stream).  Calls
 *     only enqueue work; inputs must stay alive until the stream has run it.
 *     No call synchronizes the host.
 *   - Layouts: row-major, dense.  W is N x K (out x in); blocks of 64 run
 *     along the flattened row-major weight.  bf16 data is IEEE bfloat16.
 *   - Errors: arguments are checked on the host before any HIP call; on
 *     error nothing is enqueued and a status is returned, with a message
 *     from nf4_last_error().  Faults inside kernels surface at the next
 *     synchronizing HIP call, as for any HIP work.
 *   - Alignment: device pointers to arrays of 16-byte vectors (w, codes,
 *     X, A, B, dY, Y, T, dX, out) must be 16-byte aligned.
 *   - Concurrency: calls are reentrant; concurrent calls on different
 *     streams must not share output buffers or workspaces.
 *   - Narrowed from a broader interface sketch: the block sizes are fixed at
 *     64 (first level) and 256 (second level), the values QLoRA uses, so
 *     nf4_weight carries no block-size fields; it carries absmax instead, for
 *     the variant without double quantization; and four error statuses
 *     (argument, unsupported, workspace, HIP) stand for finer per-cause codes,
 *     the cause being spelled out by nf4_last_error().
 */
#ifndef QLORA_NF4_H
#define QLORA_NF4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nf4_status {
    NF4_OK = 0,
    NF4_ERR_ARG = 1,          /* null pointer, negative or inconsistent size, misalignment */
    NF4_ERR_UNSUPPORTED = 2,  /* valid for the method, outside what this library implements */
    NF4_ERR_WORKSPACE = 3,    /* workspace missing or smaller than nf4_workspace_bytes() */
    NF4_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed */
} nf4_status;

typedef enum nf4_dtype { NF4_F32 = 0, NF4_BF16 = 1 } nf4_dtype;

/* An NF4 weight: the storage tuple of [DQ] + [RW], double-quantized, or with the
 * first-level constants kept as plain fp32 ([DQ] off: 0.5 instead of about 0.127
 * bits of constants per value).  n = rows * cols values; n1 = ceil(n/64)
 * first-level constants.  q != NULL selects the double-quantized constants
 * (q, c2, mean; absmax ignored); q == NULL selects absmax (c2 and mean ignored,
 * may be NULL). */
typedef struct nf4_weight {
    const uint8_t* codes;  /* ceil(n/2) bytes; element 2i in the low nibble of byte i */
    const uint8_t* q;      /* n1 bytes: OCP FP8 E4M3 codes of 448*(c1 - mean)/c2, or NULL */
    const float* c2;       /* ceil(n1/256) fp32 second-level constants */
    const float* mean;     /* 1 fp32: mean of the first-level constants */
    int64_t rows;          /* N (out features) */
    int64_t cols;          /* K (in features) */
    const float* absmax;   /* with q == NULL: n1 fp32 first-level constants (nf4_quantize) */
} nf4_weight;

/* Workspace selectors for nf4_workspace_bytes(). */
#define NF4_OP_DOUBLE_QUANTIZE 1
#define NF4_OP_LINEAR_FWD 2
#define NF4_OP_LINEAR_BWD 3
#define NF4_OP_CODEBOOK_STATS 4
#define NF4_OP_LOWRANK_SVD 5     /* pass the sketch width l as M */
#define NF4_OP_LOFTQ 6           /* pass the sketch width l as M */

/* [BQ]+[NF]: blockwise absmax NF4 quantization (stub nf4_quantize(w, block=64)).
 * For each block of 64 consecutive values (the last may be partial):
 * absmax[b] = max|w|; each value becomes the code of the nearest NF4 level of
 * w/absmax (IEEE fp32 division; a value exactly between two levels takes the
 * lower code; an all-zero block gives code 7, the exact-zero level).
 *   w       n values, dtype NF4_F32 or NF4_BF16 (widened exactly to fp32)
 *   n       number of values, >= 0 (n == 0 enqueues nothing)
 *   blocksize  must be 64
 *   codes   out: ceil(n/2) bytes, two codes per byte, low nibble first; the
 *           high nibble past an odd n is 0
 *   absmax  out: ceil(n/64) fp32 first-level constants c1 */
nf4_status nf4_quantize(const void* w, nf4_dtype dtype, int64_t n, int32_t blocksize,
                        uint8_t* codes, float* absmax, void* stream);

/* [BQ]+[NF] comparison: the same quantization onto a caller's codebook of 16
 * ascending levels (the page compares NF4 with the integer grids {-7..7}/7 and
 * {-8..7}/8 and with a Lloyd codebook).  Each value becomes the code of the
 * nearest level of w/absmax (a value exactly between two levels takes the lower
 * code); an all-zero block takes the code of x = 0.  Arguments as for
 * nf4_quantize, plus
 *   levels  host array of 16 finite, strictly ascending fp32 levels.  Levels
 *           outside [-1, 1] are allowed (never nearest past the last one inside).
 * The kernel finds the nearest level through 1/32-wide buckets of [-1, 1] and an
 * exact division for normal quotients, so a codebook is rejected
 * (NF4_ERR_UNSUPPORTED) when two midpoints of adjacent levels fall within one
 * bucket [k/32, (k+1)/32), or a midpoint lies within the fp32 subnormal range
 * around 0. */
nf4_status nf4_quantize_codebook(const void* w, nf4_dtype dtype, int64_t n, int32_t blocksize,
                                 const float* levels, uint8_t* codes, float* absmax, void* stream);

/* Statistics of such a quantization (device struct, written by
 * nf4_codebook_stats): per code the number of values and the sum of
 * x = fp32(w / absmax) (a Lloyd step moves each level to sum_x / count), and the
 * float64 sum of (w - fp32(level[code] * absmax))^2.  Values of all-zero blocks
 * count, with x = 0 and no error. */
typedef struct nf4_codebook_stats_t {
    int64_t count[16];
    double sum_x[16];
    double sse;
} nf4_codebook_stats_t;

/* One pass over (w, codes, absmax) of nf4_quantize_codebook (or nf4_quantize
 * with the NF4 levels of nf4_codebook) into *out.  Sums are float64 in a fixed
 * order, so the result does not depend on timing.
 *   w, dtype, n, codes, absmax  as for nf4_quantize (blocksize 64)
 *   levels     host array of the 16 levels the codes index
 *   out        device nf4_codebook_stats_t, overwritten
 *   workspace  nf4_workspace_bytes(NF4_OP_CODEBOOK_STATS, 0, n, 0, 0) bytes,
 *              8-byte aligned */
nf4_status nf4_codebook_stats(const void* w, nf4_dtype dtype, int64_t n, const uint8_t* codes,
                              const float* absmax, const float* levels, nf4_codebook_stats_t* out,
                              void* workspace, size_t workspace_bytes, void* stream);

/* [DQ]: double quantization of the first-level constants (stub
 * double_quantize(c1, block=256)).  mean = fp32(S / n1), S the float64 sum of
 * c1 over an aligned pairwise tree; d = fp32(c1 - mean); per block of 256:
 * c2 = max|d|, q = E4M3 round-to-nearest-even of 448 * fp32(d / c2) (0 when
 * c2 == 0).  The mean never leaves the device.
 *   absmax  n1 fp32 values >= +0 (the output of nf4_quantize)
 *   blocksize2  must be 256
 *   q       out: n1 bytes;  c2 out: ceil(n1/256) fp32;  mean out: 1 fp32
 *   workspace   nf4_workspace_bytes(NF4_OP_DOUBLE_QUANTIZE, 0, n1, 0, 0) bytes,
 *               8-byte aligned (partial sums). */
nf4_status nf4_double_quantize(const float* absmax, int64_t n1, int32_t blocksize2, uint8_t* q,
                               float* c2, float* mean, void* workspace, size_t workspace_bytes,
                               void* stream);

/* [DQ] for many tensors at once (a model's weights quantized in bulk): the
 * result for tensor t is exactly nf4_double_quantize(absmax[t], n1[t], 256, q[t],
 * c2[t], mean[t]); the whole batch takes two kernel launches per 32 tensors
 * instead of two per tensor.
 *   count   number of tensors (0: nothing to do)
 *   absmax, n1, q, c2, mean   HOST arrays of `count` entries: device pointers
 *           (as for nf4_double_quantize) and sizes, 0 <= n1[t] <= 2048 * 2048
 *           (NF4_ERR_UNSUPPORTED above: use nf4_double_quantize for such a tensor)
 *   workspace   nf4_double_quantize_batch_workspace_bytes(count, n1) bytes,
 *               8-byte aligned (chunk sums).
 * The host arrays are read during the call only. */
size_t nf4_double_quantize_batch_workspace_bytes(int32_t count, const int64_t* n1);
nf4_status nf4_double_quantize_batch(int32_t count, const float* const* absmax, const int64_t* n1,
                                     uint8_t* const* q, float* const* c2, float* const* mean, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* [DQ]: two-level constant decode (stub double_dequantize(q, c2, mean)):
 * c1'[i] = fma(E4M3(q[i]), fp32(c2[i/256] / 448), mean), one rounding.
 *   c1_out  out: n1 fp32 */
nf4_status nf4_double_dequantize(const uint8_t* q, const float* c2, const float* mean, int64_t n1,
                                 int32_t blocksize2, float* c1_out, void* stream);

/* [BQ]+[DQ]: dequantization of a whole weight (stub nf4_dequantize(codes,
 * absmax, shape), with the double-quantized constants in place of absmax):
 * out[i] = fp32(level[code_i] * c1'[i/64]), c1' the decoded constant (or the
 * plain absmax when W->q is NULL); NF4_BF16 output rounds that value to nearest
 * even.
 *   out     rows*cols values of out_dtype */
nf4_status nf4_dequantize(const nf4_weight* W, void* out, nf4_dtype out_dtype, void* stream);

/* [PT]+[E2E]+[RW]: QLoRA linear forward.
 *   Y = X W'^T + s (X A^T) B^T,  s = alpha / r,  W' = dequant(W) rounded to bf16
 * with the dequantization fused into the matrix multiply.
 *   W       N x K weight, K a multiple of 64, N a multiple of 8, N*K < 2^32,
 *           N and K below 2^22 (the kernels' 32-bit buffer offsets)
 *   X       bf16 M x K;  0 <= M < 2^23 (M == 0 enqueues nothing); for M > 16 the
 *           product runs as ceil(M/512) * ceil(N/128) output tiles (plus split
 *           pieces), which must stay below 2^24 (backward: ceil(M/512) * ceil(K/128))
 *   A       bf16 r x K;  B  bf16 N x r;  1 <= r <= 128, r a multiple of 8
 *   Y       out: bf16 M x N
 *   T_out   out: bf16 M x r copy of X A^T for the backward, or NULL
 *   workspace  nf4_workspace_bytes(NF4_OP_LINEAR_FWD, M, N, K, r) bytes,
 *              256-byte aligned (may be NULL if that is 0) */
nf4_status qlora_linear_fwd(const nf4_weight* W, const void* X, int64_t M, const void* A,
                            const void* B, int32_t r, float alpha, void* Y, void* T_out,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Allocation-free variant of qlora_linear_fwd, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops (the few-token
 * forward), harnesses that forbid hipMalloc.  Same arguments, kernels and results as
 * qlora_linear_fwd, without the workspace: the forward's workspace is taken from a
 * fixed scratch array of NF4_NOALLOC_SCRATCH_BYTES (32 MiB) that the library keeps on
 * every GPU it runs on until the process ends.  It covers, for example, the few-token
 * forward (M <= 16) at every LLaMA-65B projection shape.
 *   Errors: a shape whose nf4_workspace_bytes(NF4_OP_LINEAR_FWD, M, N, K, r) exceeds the
 *           scratch returns NF4_ERR_WORKSPACE before anything is enqueued; other
 *           arguments are checked as for qlora_linear_fwd.  The first call on a device
 *           looks up that device's scratch address (NF4_ERR_HIP if that fails).
 *   Concurrency: every call on one GPU uses the same scratch, which keeps the contents
 *           of the last call (nothing in it needs to start at zero).  Calls that
 *           overlap in time on one GPU (other streams, or host threads without stream
 *           order between them) race on it and give wrong results. */
#define NF4_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
nf4_status qlora_linear_fwd_noalloc(const nf4_weight* W, const void* X, int64_t M, const void* A,
                                    const void* B, int32_t r, float alpha, void* Y, void* T_out,
                                    void* stream);

/* [E2E]+[PT]: QLoRA linear backward; the 4-bit weight receives no gradient.
 * With U = dY B:
 *   dX = dY W' + s U A   (bf16 M x K)
 *   dA = s U^T X         (fp32 r x K, overwritten)
 *   dB = s dY^T T        (fp32 N x r, overwritten), T = X A^T
 *   T       bf16 M x r from qlora_linear_fwd, or NULL to recompute it
 *   dX      may be NULL to skip the input gradient
 * Shapes and limits as for qlora_linear_fwd; M == 0 writes dA = dB = 0. */
nf4_status qlora_linear_bwd(const nf4_weight* W, const void* X, const void* dY, int64_t M,
                            const void* A, const void* B, int32_t r, float alpha, const void* T,
                            void* dX, float* dA, float* dB, void* workspace,
                            size_t workspace_bytes, void* stream);

/* [PO]: one AdamW step over n adapter parameters, in fp32 with no fused
 * multiply-add:
 *   m = b1 m + (1 - b1) g;   v = b2 v + (1 - b2) g^2
 *   p = p (1 - lr wd) - (lr / (1 - b1^t)) * m / (sqrt(v) / sqrt(1 - b2^t) + eps)
 * 1 - b1, 1 - b2, the bias corrections and 1 - lr wd are formed in double on the
 * host and rounded once to fp32; sqrt and the division are correctly rounded.
 *   p, m, v  n fp32 values each (master parameters, first and second moments),
 *            updated in place; 16-byte aligned
 *   g        n fp32 gradient values (dA or dB of qlora_linear_bwd); 16-byte aligned
 *   p_bf16   out: bf16 copy of the updated p (round to nearest even), the A or B
 *            operand of the layer; or NULL.  8-byte aligned
 *   step     t >= 1, the step being taken;  0 <= beta1, beta2 < 1;  eps > 0;
 *            lr and weight_decay finite
 * n == 0 enqueues nothing.  No buffer may overlap another. */
nf4_status nf4_adamw_step(float* p, const float* g, float* m, float* v, uint16_t* p_bf16, int64_t n,
                          float lr, float beta1, float beta2, float eps, float weight_decay,
                          int64_t step, void* stream);

/* [PO]: the same step for state paged out to host memory.  p_host, m_host and
 * v_host are page-locked host buffers (hipHostMalloc or equivalent); g and p_bf16
 * are device memory as above.  The state passes through the device buffer `stage`,
 * split in two halves of floor(stage_bytes / 1536) * 64 parameters that chunks use
 * in turn: a chunk is copied in and updated on `stream`, and copied back on a
 * helper stream of the library (one per device, created on first use, default
 * priority), so that one chunk's copy-back overlaps the next chunk's copy-in.
 * `stream` completes only after every copy-back.  The host buffers must stay
 * untouched until `stream` has run the work.  Results are bit-identical to
 * nf4_adamw_step on device-resident state.
 *   stage        device scratch, 256-byte aligned, stage_bytes >= 1536 */
nf4_status nf4_adamw_step_paged(float* p_host, const float* g, float* m_host, float* v_host,
                                uint16_t* p_bf16, int64_t n, float lr, float beta1, float beta2,
                                float eps, float weight_decay, int64_t step, void* stage,
                                size_t stage_bytes, void* stream);

/* Bytes of device workspace an operation needs (0 = none).  For
 * NF4_OP_DOUBLE_QUANTIZE pass n1 as N; for NF4_OP_CODEBOOK_STATS pass n as N.  The linear products keep their
 * intermediates there: the rank-r activations (s*T, T, s*U), the decoded
 * first-level constants c1' of W (4 bytes per 64-block, written before the
 * fused MFMA product; not needed by the M <= 16 forward) and fp32 partial sums
 * of the split-contraction adapter products and of the fused product's tail
 * tiles (when the last wave of 512 x 128 output tiles, tokens x features, would
 * leave most compute units idle, those tiles are computed in up to 4
 * contraction pieces: at most 64 MiB).  Contents are scratch: nothing
 * survives between calls, and two calls that overlap in time on one device
 * need separate workspaces. */
size_t nf4_workspace_bytes(int32_t op, int64_t M, int64_t N, int64_t K, int32_t r);

/* [DQ] storage accounting for n values: codes ceil(n/2) bytes, q ceil(n/64)
 * bytes, c2 4*ceil(n1/256) bytes -- 4 + 8/64 + 32/(64*256) ~ 4.127 bits per
 * value.  Host-only; any output pointer may be NULL. */
void nf4_storage_bytes(int64_t n, int32_t blocksize, int32_t blocksize2, size_t* codes_bytes,
                       size_t* q_bytes, size_t* c2_bytes);

/* [NF]: host copy of the 16 NF4 levels, ascending (code 7 = 0, 0 = -1, 15 = +1). */
void nf4_codebook(float out[16]);

/* Profiling hook: the next fused dequant kernel (forward GEMM, dequant-GEMV or
 * backward dX GEMM) that the calling thread launches records the hipEvent_t
 * `start` on its stream right before itself and `stop` right after, then the
 * hook disarms.  Events are created and owned by the caller; NULL, NULL
 * disarms without recording. */
void nf4_profile_next_fused(void* start_event, void* stop_event);

/* Message for the last error returned on the calling thread ("" if none). */
const char* nf4_last_error(void);

/* Rank-r truncated SVD of an fp32 matrix, E ~ U diag(S) V^T, the step of the LoftQ
 * initialisation below, exported for tests and reuse.  Randomized subspace iteration
 * (Halko, Martinsson & Tropp, SIAM Review 2011): Y = orth(E Omega), `power_iters` rounds of
 * Z = orth(E^T Y), Y = orth(E Z), then the eigen-decomposition of the l x l Gram matrix of
 * E^T Y.  It approaches the exact truncated SVD as power_iters grows; the error of the
 * approximation is what the test matrix and the gap between the r-th and (l+1)-th singular
 * values allow.
 *   E       fp32 N x K, row-major, 16-byte aligned (not modified); N, K < 2^22, N*K < 2^32
 *   r, l    1 <= r <= l <= 96, l <= N, l <= K (l: sketch width, r plus oversampling)
 *   power_iters  0 .. 16
 *   omega   fp32 K x l test matrix (the caller draws it, e.g. i.i.d. N(0, 1))
 *   U       out: fp32 N x r (orthonormal columns); S out: fp32 r, descending;
 *   V       out: fp32 K x r (the right singular vectors as columns)
 *   workspace  nf4_workspace_bytes(NF4_OP_LOWRANK_SVD, l, N, K, r) bytes, 256-byte aligned
 * A column direction that E does not reach (rank below r) comes out as zero. */
nf4_status nf4_lowrank_svd(const float* E, int64_t N, int64_t K, int32_t r, int32_t l, int32_t power_iters,
                           const float* omega, float* U, float* S, float* V, void* workspace,
                           size_t workspace_bytes, void* stream);

/* [E2E] LoftQ-style initialisation of the adapter of a quantized base (closing remark of
 * "Paged optimizers, and QLoRA end to end": start A and B so that dequant(W^NF4) + gamma B A
 * is close to W, gamma = alpha / r).  The alternation of Li et al. (2023), from B A = 0,
 * `iters` times: quantize the residual W - gamma B A with nf4_quantize and
 * nf4_double_quantize; take the rank-r truncated SVD U S V^T of the quantization error
 * E = W - dequant(Q) (nf4_lowrank_svd's method); B = U S^1/2 / sqrt(gamma),
 * A = S^1/2 V^T / sqrt(gamma).
 *   W       fp32 N x K (the full-precision weight), 16-byte aligned; N*K < 2^32
 *   r, l, power_iters, omega   as for nf4_lowrank_svd (omega K x l)
 *   alpha   > 0 (the layer's scale is alpha / r)
 *   iters   1 .. 64
 *   codes, q, c2, mean  out: the last quantization Q (the layer's frozen weight, as
 *           nf4_quantize + nf4_double_quantize lay it out)
 *   A       out: bf16 r x K;  B  out: bf16 N x r (round to nearest even of the fp32 factors)
 *   err     out: device float64[iters], err[t] = ||W - dequant(Q_t) - gamma B_t A_t||_F with
 *           the fp32 factors of alternation t (from ||E_t||_F^2 - sum S^2)
 *   workspace  nf4_workspace_bytes(NF4_OP_LOFTQ, l, N, K, r) bytes, 256-byte aligned */
nf4_status nf4_loftq_init(const float* W, int64_t N, int64_t K, int32_t r, float alpha, int32_t iters, int32_t l,
                          int32_t power_iters, const float* omega, uint8_t* codes, uint8_t* q, float* c2,
                          float* mean, void* A, void* B, double* err, void* workspace, size_t workspace_bytes,
                          void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_NF4_H */
