// api.hip -- the extern "C" entry points declared in include/qlora_nf4.h.
//
// Host side only: argument validation (before any HIP call), the NF4 table,
// workspace carving and kernel dispatch.  Every product step runs in the
// gfx950 kernels of codec.hip, lora.hip, fused.hip, gemv.hip, adamw.hip and codebook.hip.
#include <math.h>
#include <string.h>

#include <mutex>
#include <string>

#include "../../include/qlora_nf4.h"
#include "launch.h"

using nf4::Nf4Table;
using nf4::WeightView;

namespace {

thread_local std::string g_last_error;

nf4_status fail(nf4_status st, const std::string& msg) {
    g_last_error = msg;
    return st;
}

nf4_status hip_status(hipError_t e, const char* where) {
    if (e == hipSuccess) return NF4_OK;
    return fail(NF4_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// ---------------------------------------------------------------------------
// NF4 levels ("NF4, derived from normal quantiles", zerotofrontier.app
// "sft/peft"): probabilities from p_max = ((1-1/30)+(1-1/32))/2 down towards
// 1/2, 8 evenly spaced quantiles on the positive side and 7 on the negative
// side, an exact zero, normalised by the largest magnitude.  The inverse
// normal CDF is solved by bisection on erfcl in long double.
// ---------------------------------------------------------------------------
long double norm_cdf(long double x) { return 0.5L * erfcl(-x / sqrtl(2.0L)); }

long double norm_quantile(long double p) {
    long double lo = -40.0L, hi = 40.0L;
    for (int it = 0; it < 256; ++it) {
        const long double mid = 0.5L * (lo + hi);
        if (mid == lo || mid == hi) break;
        if (norm_cdf(mid) < p) lo = mid;
        else hi = mid;
    }
    return 0.5L * (lo + hi);
}

// Encode table of an ascending 16-level codebook ("Block-wise quantization in one
// page": the nearest level, a value exactly between two taking the lower one).  The
// quantize kernel compares x = w/absmax with th[j], the largest fp32 not above the
// float64 midpoint, which decides x > midpoint exactly for every fp32 x.  It finds the
// candidate threshold through 1/32-wide buckets of [-1, 1 + 1/32), so at most one
// threshold may fall in a bucket; and its division is exact for every normal quotient,
// so no threshold may lie within the subnormal range around 0 (there every quotient
// must fall on the same side as 0).  Returns false, with the reason, for a codebook
// outside these limits.
bool make_table(const float lv[16], Nf4Table& t, std::string& why) {
    for (int i = 0; i < 16; ++i) {
        if (!isfinite(lv[i])) { why = "levels must be finite"; return false; }
        if (i > 0 && !(lv[i] > lv[i - 1])) { why = "levels must be strictly ascending"; return false; }
        t.lv[i] = lv[i];
    }
    int zero_code = 0;
    int last_bucket = -1;
    for (int j = 0; j < 15; ++j) {
        // largest fp32 not above the (exact) midpoint: x > th[j] <=> x > midpoint
        const double mid = ((double)lv[j] + (double)lv[j + 1]) / 2.0;
        float th = (float)mid;
        if ((double)th > mid) th = nextafterf(th, -INFINITY);
        t.th[j] = th;
        if (fabsf(th) < 1.1754943508222875e-38f) { why = "a decision threshold lies in the subnormal range around 0"; return false; }
        if (th >= -1.0f && th < 1.0f + 1.0f / 32.0f) {
            const int b = (int)floorf(th * 32.0f) + 32;
            if (b == last_bucket) { why = "two decision thresholds lie within one 1/32-wide bucket"; return false; }
            last_bucket = b;
        }
        zero_code += th < 0.0f ? 1 : 0;
    }
    t.zero_word = 0x11111111u * (uint32_t)zero_code;
    return true;
}

Nf4Table build_table() {
    const long double pmax = ((1.0L - 1.0L / 30.0L) + (1.0L - 1.0L / 32.0L)) / 2.0L;
    const long double top = norm_quantile(pmax);
    long double v[16];
    for (int i = 0; i < 7; ++i) v[i] = -norm_quantile(pmax - (long double)i * (pmax - 0.5L) / 7.0L);
    v[7] = 0.0L;
    for (int i = 0; i < 8; ++i) v[8 + i] = norm_quantile(pmax - (long double)(7 - i) * (pmax - 0.5L) / 8.0L);
    float lv[16];
    for (int i = 0; i < 16; ++i) lv[i] = (float)(v[i] / top);
    lv[7] = 0.0f;
    Nf4Table t;
    std::string why;
    make_table(lv, t, why);
    return t;
}

const Nf4Table& table() {
    static Nf4Table t;
    static std::once_flag once;
    std::call_once(once, [] { t = build_table(); });
    return t;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Limits of the linear products, checked before anything is enqueued.  Buffer descriptors
// cap a range at 2^31 - 1 bytes and take 32-bit per-lane offsets: the adapter products
// address up to 128 rows (direct operands) or 64 contraction rows (strided operands) of a
// leading dimension N or K, 254 ld bytes at most, and the few-token forward 16 token rows
// of K or 128 adapter rows; with N, K below 2^22 every offset stays below 2^31.  (The fused
// products read their token operand through 64 KB fragment-order blocks and the packed
// weight within N * K / 2 < 2^31 bytes.)  A launch holds at most 2^24 workgroups of 256
// threads (2^32 work-items); the adapter products stack the token rows in 128-row
// workgroups along the grid's second dimension.
constexpr int64_t LINEAR_DIM_LIMIT = (int64_t)1 << 22;
constexpr int64_t LINEAR_M_LIMIT = (int64_t)1 << 23;
constexpr int64_t FUSED_GRID_LIMIT = (int64_t)1 << 24;

nf4_status check_weight(const nf4_weight* W, WeightView& v, bool linear) {
    if (!W) return fail(NF4_ERR_ARG, "weight descriptor is NULL");
    if (W->rows < 0 || W->cols < 0) return fail(NF4_ERR_ARG, "negative weight shape");
    if (W->cols > 0 && W->rows > INT64_MAX / W->cols) return fail(NF4_ERR_ARG, "rows * cols overflows 64 bits");
    const int64_t n = W->rows * W->cols;
    const bool plain = W->q == nullptr;
    if (plain) {
        if (n > 0 && (!W->codes || !W->absmax)) return fail(NF4_ERR_ARG, "weight has a NULL codes/absmax pointer");
        if (!aligned(W->absmax, 4)) return fail(NF4_ERR_ARG, "misaligned absmax");
    } else {
        if (n > 0 && (!W->codes || !W->c2 || !W->mean))
            return fail(NF4_ERR_ARG, "weight has a NULL codes/q/c2/mean pointer");
        if (!W->mean) return fail(NF4_ERR_ARG, "weight mean pointer is NULL");
    }
    if (linear) {
        if (W->cols % 64 != 0) return fail(NF4_ERR_UNSUPPORTED, "K (cols) must be a multiple of 64");
        if (W->rows % 8 != 0) return fail(NF4_ERR_UNSUPPORTED, "N (rows) must be a multiple of 8");
        if (W->rows == 0 || W->cols == 0) return fail(NF4_ERR_ARG, "empty weight");
        // the fused kernels address the packed weight through 32-bit buffer offsets
        if (n / 2 >= ((int64_t)1 << 31)) return fail(NF4_ERR_UNSUPPORTED, "weight larger than 2^32 values");
        if (W->rows >= LINEAR_DIM_LIMIT || W->cols >= LINEAR_DIM_LIMIT)
            return fail(NF4_ERR_UNSUPPORTED, "N (rows) and K (cols) must be below 2^22");
    }
    if (!aligned(W->codes, 16)) return fail(NF4_ERR_ARG, "codes must be 16-byte aligned");
    if (!plain && (!aligned(W->c2, 4) || !aligned(W->mean, 4))) return fail(NF4_ERR_ARG, "misaligned c2/mean");
    v.codes = W->codes;
    v.q = W->q;
    v.c2 = plain ? nullptr : W->c2;
    v.mean = plain ? nullptr : W->mean;
    v.rows = W->rows;
    v.cols = W->cols;
    v.absmax = plain ? W->absmax : nullptr;
    return NF4_OK;
}

nf4_status check_lora(const void* A, const void* B, int32_t r, float alpha) {
    if (r < 1 || r > 128) return fail(NF4_ERR_UNSUPPORTED, "rank r must be in [1, 128]");
    if (r % 8 != 0) return fail(NF4_ERR_UNSUPPORTED, "rank r must be a multiple of 8");
    if (!A || !B) return fail(NF4_ERR_ARG, "adapter A or B is NULL");
    if (!aligned(A, 16) || !aligned(B, 16)) return fail(NF4_ERR_ARG, "A and B must be 16-byte aligned");
    if (!isfinite(alpha)) return fail(NF4_ERR_ARG, "alpha must be finite");
    return NF4_OK;
}

size_t rank_buffer_bytes(int64_t M, int32_t r) { return align256((size_t)M * (size_t)r * 2); }

// Token counts up to this use the dequantize-GEMV forward; larger ones the fused MFMA product.
constexpr int64_t GEMV_MAX_M = 16;

// Decoded first-level constants c1' (fp32, one per 64-block) that the fused MFMA products
// read; the GEMV forward decodes them itself.
size_t c1_buffer_bytes(int32_t op, int64_t M, int64_t N, int64_t K) {
    const bool fused = op == NF4_OP_LINEAR_FWD ? M > GEMV_MAX_M : M > 0;
    return fused ? align256((size_t)(N * (K / 64)) * 4) : 0;
}

// The fused products' A operand (X forward, dY backward) in fragment order: one 64 KB block
// per (512-token tile, 64-value contraction step).
size_t pack_bytes(int32_t op, int64_t M, int64_t N, int64_t K) {
    const bool fused = op == NF4_OP_LINEAR_FWD ? M > GEMV_MAX_M : M > 0;
    if (!fused) return 0;
    const int64_t ld = op == NF4_OP_LINEAR_FWD ? K : N;
    return (size_t)((M + nf4::FUSED_TM - 1) / nf4::FUSED_TM) * (size_t)((ld + 63) / 64) * nf4::A_BLOCK_BYTES;
}

// Workspace layouts (256-byte aligned pieces):
//   forward : [s*T bf16 M x r][T bf16 M x r, when T_out is NULL][c1' fp32][fp32 partials][packed X]
//   backward: [s*U bf16 M x r][T bf16 M x r, when T is NULL][c1' fp32][fp32 partials][packed dY]
// The partials region serves, one after the other in stream order, the split-contraction
// slices of the rank-r products and the fp32 partial tiles of the fused product's split
// tail tiles.
size_t fwd_partial_bytes(int64_t M, int64_t N, int64_t K, int32_t r) {
    if (M <= GEMV_MAX_M) return align256(nf4::gemv_partial_bytes(M, N, K, r));
    const size_t a = nf4::skinny_partial_bytes(M, r, K), b = align256(nf4::fused_fwd_plan(M, N, K).bytes);
    return a > b ? a : b;
}
size_t bwd_partial_bytes(int64_t M, int64_t N, int64_t K, int32_t r) {
    size_t b = align256(nf4::fused_bwd_plan(M, N, K).bytes);
    b = nf4::skinny_partial_bytes(M, r, N) > b ? nf4::skinny_partial_bytes(M, r, N) : b;
    // dB and dA run in one launch, each with its own slices
    const size_t c[2] = {nf4::skinny_partial_bytes(M, r, K),
                         nf4::skinny_partial_bytes(N, r, M) + nf4::skinny_partial_bytes(K, r, M)};
    for (size_t x : c) b = x > b ? x : b;
    return b;
}

// Scratch of qlora_linear_fwd_noalloc: a file-scope device array (each GPU the library runs
// on holds its own copy, at its own address, until the process ends).  In host code its
// name is only a stand-in; the device address comes from hipGetSymbolAddress, looked up
// once per device with that device current, and that address is what the kernels get.
static __device__ __align__(256) uint8_t scratch[NF4_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

hipError_t noalloc_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p || !aligned(p, 256)) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

const char* nf4_last_error(void) { return g_last_error.c_str(); }

void nf4_profile_next_fused(void* start_event, void* stop_event) {
    nf4::FusedEvents& ev = nf4::fused_events();
    ev.start = (hipEvent_t)start_event;
    ev.stop = (hipEvent_t)stop_event;
}

void nf4_codebook(float out[16]) {
    if (!out) return;
    memcpy(out, table().lv, sizeof(float) * 16);
}

void nf4_storage_bytes(int64_t n, int32_t blocksize, int32_t blocksize2, size_t* codes_bytes,
                       size_t* q_bytes, size_t* c2_bytes) {
    if (n < 0 || blocksize <= 0 || blocksize2 <= 0) n = 0;
    if (blocksize <= 0) blocksize = 64;
    if (blocksize2 <= 0) blocksize2 = 256;
    const int64_t n1 = (n + blocksize - 1) / blocksize;
    const int64_t n2 = (n1 + blocksize2 - 1) / blocksize2;
    if (codes_bytes) *codes_bytes = (size_t)((n + 1) / 2);
    if (q_bytes) *q_bytes = (size_t)n1;
    if (c2_bytes) *c2_bytes = (size_t)n2 * 4;
}

size_t nf4_workspace_bytes(int32_t op, int64_t M, int64_t N, int64_t K, int32_t r) {
    if (M < 0 || N < 0 || K < 0 || r < 0) return 0;
    switch (op) {
        case NF4_OP_DOUBLE_QUANTIZE: return nf4::double_quantize_ws_bytes(N);
        case NF4_OP_CODEBOOK_STATS: return N > 0 ? nf4::codebook_stats_ws_bytes(N) : 0;
        case NF4_OP_LINEAR_FWD:
            return 2 * rank_buffer_bytes(M, r) + c1_buffer_bytes(op, M, N, K) + fwd_partial_bytes(M, N, K, r) +
                   pack_bytes(op, M, N, K);
        case NF4_OP_LINEAR_BWD:
            return 2 * rank_buffer_bytes(M, r) + c1_buffer_bytes(op, M, N, K) + bwd_partial_bytes(M, N, K, r) +
                   pack_bytes(op, M, N, K);
        case NF4_OP_LOWRANK_SVD:   // M carries the sketch width l
            return (N > 0 && K > 0 && M > 0 && M <= nf4::LR_MAX && r > 0) ? nf4::lowrank_ws_bytes(N, K, (int)M, r) : 0;
        case NF4_OP_LOFTQ:
            return (N > 0 && K > 0 && M > 0 && M <= nf4::LR_MAX && r > 0) ? nf4::loftq_ws_bytes(N, K, (int)M, r) : 0;
        default: return 0;
    }
}

nf4_status nf4_quantize(const void* w, nf4_dtype dtype, int64_t n, int32_t blocksize, uint8_t* codes,
                        float* absmax, void* stream) {
    if (blocksize != 64) return fail(NF4_ERR_UNSUPPORTED, "blocksize must be 64");
    if (dtype != NF4_F32 && dtype != NF4_BF16) return fail(NF4_ERR_ARG, "dtype must be NF4_F32 or NF4_BF16");
    if (n < 0) return fail(NF4_ERR_ARG, "n must be >= 0");
    if (n == 0) return NF4_OK;
    if (!w || !codes || !absmax) return fail(NF4_ERR_ARG, "NULL w/codes/absmax");
    if (!aligned(w, 16)) return fail(NF4_ERR_ARG, "w must be 16-byte aligned");
    if (!aligned(codes, 4) || !aligned(absmax, 4)) return fail(NF4_ERR_ARG, "codes/absmax must be 4-byte aligned");
    return hip_status(nf4::launch_quantize(w, dtype == NF4_BF16, n, codes, absmax, table(),
                                           (hipStream_t)stream),
                      "nf4_quantize");
}

nf4_status nf4_quantize_codebook(const void* w, nf4_dtype dtype, int64_t n, int32_t blocksize,
                                 const float* levels, uint8_t* codes, float* absmax, void* stream) {
    if (blocksize != 64) return fail(NF4_ERR_UNSUPPORTED, "blocksize must be 64");
    if (dtype != NF4_F32 && dtype != NF4_BF16) return fail(NF4_ERR_ARG, "dtype must be NF4_F32 or NF4_BF16");
    if (!levels) return fail(NF4_ERR_ARG, "levels is NULL");
    Nf4Table tab;
    std::string why;
    if (!make_table(levels, tab, why)) return fail(NF4_ERR_UNSUPPORTED, "codebook: " + why);
    if (n < 0) return fail(NF4_ERR_ARG, "n must be >= 0");
    if (n == 0) return NF4_OK;
    if (!w || !codes || !absmax) return fail(NF4_ERR_ARG, "NULL w/codes/absmax");
    if (!aligned(w, 16)) return fail(NF4_ERR_ARG, "w must be 16-byte aligned");
    if (!aligned(codes, 4) || !aligned(absmax, 4)) return fail(NF4_ERR_ARG, "codes/absmax must be 4-byte aligned");
    return hip_status(nf4::launch_quantize(w, dtype == NF4_BF16, n, codes, absmax, tab, (hipStream_t)stream),
                      "nf4_quantize_codebook");
}

nf4_status nf4_codebook_stats(const void* w, nf4_dtype dtype, int64_t n, const uint8_t* codes,
                              const float* absmax, const float* levels, nf4_codebook_stats_t* out,
                              void* workspace, size_t workspace_bytes, void* stream) {
    static_assert(sizeof(nf4_codebook_stats_t) == sizeof(nf4::CodebookStats), "stats layout");
    if (dtype != NF4_F32 && dtype != NF4_BF16) return fail(NF4_ERR_ARG, "dtype must be NF4_F32 or NF4_BF16");
    if (!levels) return fail(NF4_ERR_ARG, "levels is NULL");
    if (n < 0) return fail(NF4_ERR_ARG, "n must be >= 0");
    if (!out || !aligned(out, 8)) return fail(NF4_ERR_ARG, "out must be an 8-byte aligned device struct");
    Nf4Table tab;
    for (int i = 0; i < 16; ++i) {
        if (!isfinite(levels[i])) return fail(NF4_ERR_ARG, "levels must be finite");
        tab.lv[i] = levels[i];
    }
    if (n == 0)   // the reduction of no partials writes the zero statistics
        return hip_status(nf4::launch_codebook_stats(nullptr, false, 0, nullptr, nullptr, tab, nullptr,
                                                     (nf4::CodebookStats*)out, (hipStream_t)stream),
                          "nf4_codebook_stats");
    if (!w || !codes || !absmax) return fail(NF4_ERR_ARG, "NULL w/codes/absmax");
    if (!aligned(w, 16)) return fail(NF4_ERR_ARG, "w must be 16-byte aligned");
    if (!aligned(codes, 4) || !aligned(absmax, 4)) return fail(NF4_ERR_ARG, "codes/absmax must be 4-byte aligned");
    const size_t need = nf4::codebook_stats_ws_bytes(n);
    if (!workspace || workspace_bytes < need)
        return fail(NF4_ERR_WORKSPACE, "workspace smaller than nf4_workspace_bytes(NF4_OP_CODEBOOK_STATS)");
    if (!aligned(workspace, 8)) return fail(NF4_ERR_ARG, "workspace must be 8-byte aligned");
    return hip_status(nf4::launch_codebook_stats(w, dtype == NF4_BF16, n, codes, absmax, tab,
                                                 (nf4::CodebookStats*)workspace, (nf4::CodebookStats*)out,
                                                 (hipStream_t)stream),
                      "nf4_codebook_stats");
}

nf4_status nf4_double_quantize(const float* absmax, int64_t n1, int32_t blocksize2, uint8_t* q,
                               float* c2, float* mean, void* workspace, size_t workspace_bytes,
                               void* stream) {
    if (blocksize2 != 256) return fail(NF4_ERR_UNSUPPORTED, "blocksize2 must be 256");
    if (n1 < 0) return fail(NF4_ERR_ARG, "n1 must be >= 0");
    if (!mean) return fail(NF4_ERR_ARG, "mean is NULL");
    if (n1 > 0 && (!absmax || !q || !c2)) return fail(NF4_ERR_ARG, "NULL absmax/q/c2");
    if (!aligned(absmax, 16)) return fail(NF4_ERR_ARG, "absmax must be 16-byte aligned");
    if (!aligned(q, 4) || !aligned(c2, 4) || !aligned(mean, 4)) return fail(NF4_ERR_ARG, "misaligned q/c2/mean");
    const size_t need = nf4::double_quantize_ws_bytes(n1);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(NF4_ERR_WORKSPACE, "workspace smaller than nf4_workspace_bytes(NF4_OP_DOUBLE_QUANTIZE)");
    if (need > 0 && !aligned(workspace, 8)) return fail(NF4_ERR_ARG, "workspace must be 8-byte aligned");
    return hip_status(nf4::launch_double_quantize(absmax, n1, q, c2, mean, (double*)workspace,
                                                  (hipStream_t)stream),
                      "nf4_double_quantize");
}

size_t nf4_double_quantize_batch_workspace_bytes(int32_t count, const int64_t* n1) {
    if (count <= 0 || !n1) return 0;
    for (int32_t t = 0; t < count; ++t)
        if (n1[t] < 0) return 0;
    return nf4::double_quantize_batch_ws_bytes(count, n1);
}

nf4_status nf4_double_quantize_batch(int32_t count, const float* const* absmax, const int64_t* n1,
                                     uint8_t* const* q, float* const* c2, float* const* mean, void* workspace,
                                     size_t workspace_bytes, void* stream) {
    if (count < 0) return fail(NF4_ERR_ARG, "count must be >= 0");
    if (count == 0) return NF4_OK;
    if (!absmax || !n1 || !q || !c2 || !mean) return fail(NF4_ERR_ARG, "NULL array");
    for (int32_t t = 0; t < count; ++t) {
        if (n1[t] < 0) return fail(NF4_ERR_ARG, "n1 must be >= 0");
        if (n1[t] > nf4::DQB_MAX_N1)
            return fail(NF4_ERR_UNSUPPORTED, "a batched tensor holds at most 2048 x 2048 constants");
        if (!mean[t]) return fail(NF4_ERR_ARG, "mean is NULL");
        if (n1[t] > 0 && (!absmax[t] || !q[t] || !c2[t])) return fail(NF4_ERR_ARG, "NULL absmax/q/c2");
        if (!aligned(absmax[t], 16)) return fail(NF4_ERR_ARG, "absmax must be 16-byte aligned");
        if (!aligned(q[t], 4) || !aligned(c2[t], 4) || !aligned(mean[t], 4))
            return fail(NF4_ERR_ARG, "misaligned q/c2/mean");
    }
    const size_t need = nf4::double_quantize_batch_ws_bytes(count, n1);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(NF4_ERR_WORKSPACE, "workspace smaller than nf4_double_quantize_batch_workspace_bytes()");
    if (need > 0 && !aligned(workspace, 8)) return fail(NF4_ERR_ARG, "workspace must be 8-byte aligned");
    return hip_status(nf4::launch_double_quantize_batch(count, absmax, n1, q, c2, mean, (double*)workspace,
                                                        (hipStream_t)stream),
                      "nf4_double_quantize_batch");
}

nf4_status nf4_double_dequantize(const uint8_t* q, const float* c2, const float* mean, int64_t n1,
                                 int32_t blocksize2, float* c1_out, void* stream) {
    if (blocksize2 != 256) return fail(NF4_ERR_UNSUPPORTED, "blocksize2 must be 256");
    if (n1 < 0) return fail(NF4_ERR_ARG, "n1 must be >= 0");
    if (n1 == 0) return NF4_OK;
    if (!q || !c2 || !mean || !c1_out) return fail(NF4_ERR_ARG, "NULL q/c2/mean/c1_out");
    if (!aligned(c2, 4) || !aligned(mean, 4) || !aligned(c1_out, 4)) return fail(NF4_ERR_ARG, "misaligned fp32 pointer");
    return hip_status(nf4::launch_double_dequantize(q, c2, mean, n1, c1_out, (hipStream_t)stream),
                      "nf4_double_dequantize");
}

nf4_status nf4_dequantize(const nf4_weight* W, void* out, nf4_dtype out_dtype, void* stream) {
    WeightView v;
    nf4_status st = check_weight(W, v, false);
    if (st != NF4_OK) return st;
    if (out_dtype != NF4_F32 && out_dtype != NF4_BF16) return fail(NF4_ERR_ARG, "out_dtype must be NF4_F32 or NF4_BF16");
    if (v.rows * v.cols == 0) return NF4_OK;
    if (!out) return fail(NF4_ERR_ARG, "out is NULL");
    if (!aligned(out, 16)) return fail(NF4_ERR_ARG, "out must be 16-byte aligned");
    return hip_status(nf4::launch_dequantize(v, out, out_dtype == NF4_BF16, table(), (hipStream_t)stream),
                      "nf4_dequantize");
}

nf4_status qlora_linear_fwd(const nf4_weight* W, const void* X, int64_t M, const void* A,
                            const void* B, int32_t r, float alpha, void* Y, void* T_out,
                            void* workspace, size_t workspace_bytes, void* stream) {
    WeightView v;
    nf4_status st = check_weight(W, v, true);
    if (st != NF4_OK) return st;
    st = check_lora(A, B, r, alpha);
    if (st != NF4_OK) return st;
    if (M < 0) return fail(NF4_ERR_ARG, "M must be >= 0");
    if (M == 0) return NF4_OK;
    if (M >= LINEAR_M_LIMIT) return fail(NF4_ERR_UNSUPPORTED, "M must be below 2^23");
    if (M > GEMV_MAX_M && nf4::fused_fwd_plan(M, v.rows, v.cols).grid >= FUSED_GRID_LIMIT)
        return fail(NF4_ERR_UNSUPPORTED, "M x N needs more than 2^24 workgroups of 512 x 128 output tiles");
    if (!X || !Y) return fail(NF4_ERR_ARG, "X or Y is NULL");
    if (!aligned(X, 16) || !aligned(Y, 16) || !aligned(T_out, 16))
        return fail(NF4_ERR_ARG, "X, Y and T_out must be 16-byte aligned");
    const size_t rb = rank_buffer_bytes(M, r);
    const size_t cb = c1_buffer_bytes(NF4_OP_LINEAR_FWD, M, v.rows, v.cols);
    const size_t pb = fwd_partial_bytes(M, v.rows, v.cols, r);
    const size_t need = 2 * rb + cb + pb + pack_bytes(NF4_OP_LINEAR_FWD, M, v.rows, v.cols);
    if (!workspace || workspace_bytes < need)
        return fail(NF4_ERR_WORKSPACE, "workspace smaller than nf4_workspace_bytes(NF4_OP_LINEAR_FWD)");
    if (!aligned(workspace, 256)) return fail(NF4_ERR_ARG, "workspace must be 256-byte aligned");
    uint16_t* Ts = (uint16_t*)workspace;
    uint16_t* Tb = T_out ? (uint16_t*)T_out : (uint16_t*)((char*)workspace + rb);
    float* c1 = (float*)((char*)workspace + 2 * rb);
    float* part = (float*)((char*)workspace + 2 * rb + cb);
    uint16_t* xpk = (uint16_t*)((char*)workspace + 2 * rb + cb + pb);
    const float s = alpha / (float)r;
    hipStream_t hs = (hipStream_t)stream;
    const uint16_t* x = (const uint16_t*)X;
    hipError_t e;
    if (M <= GEMV_MAX_M) {
        e = nf4::launch_fused_gemv(v, x, M, (const uint16_t*)A, (const uint16_t*)B, r, s, (uint16_t*)Y,
                                   Tb, part, table(), hs);
        return hip_status(e, "qlora_linear_fwd (gemv)");
    }
    // T = X A^T (kept for the backward) and s*T for the epilogue of the fused product; the
    // same pass writes X in the fused product's fragment order
    // The block constants of W are decoded by extra workgroups of T's slice-sum launch (plain
    // constants are read as they are)
    const nf4::DqDecode dq{v.q, v.c2, v.mean, v.rows * (v.cols / 64), c1};
    e = nf4::launch_lora_gemm(x, false, (const uint16_t*)A, false, M, r, v.cols, part, 1.0f, Tb,
                              false, false, Ts, s, hs, xpk, true, v.absmax ? nullptr : &dq);
    if (e != hipSuccess) return hip_status(e, "qlora_linear_fwd (T)");
    if (v.absmax) c1 = (float*)v.absmax;
    e = nf4::launch_fused_fwd(v, c1, xpk, M, Ts, (const uint16_t*)B, r, (uint16_t*)Y, part, table(), hs);
    return hip_status(e, "qlora_linear_fwd (gemm)");
}

nf4_status qlora_linear_fwd_noalloc(const nf4_weight* W, const void* X, int64_t M, const void* A,
                                    const void* B, int32_t r, float alpha, void* Y, void* T_out,
                                    void* stream) {
    // the size check needs only the shape; everything else is checked by qlora_linear_fwd
    WeightView v;
    nf4_status st = check_weight(W, v, true);
    if (st != NF4_OK) return st;
    if (M < 0) return fail(NF4_ERR_ARG, "M must be >= 0");
    if (r < 0) return fail(NF4_ERR_UNSUPPORTED, "rank r must be in [1, 128]");
    const size_t need = nf4_workspace_bytes(NF4_OP_LINEAR_FWD, M, v.rows, v.cols, r);
    if (need > NF4_NOALLOC_SCRATCH_BYTES)
        return fail(NF4_ERR_WORKSPACE, "this shape's forward needs " + std::to_string(need) +
                                           " bytes of workspace, more than the 33554432-byte scratch of "
                                           "qlora_linear_fwd_noalloc");
    void* ws = nullptr;
    hipError_t e = noalloc_scratch(&ws);
    if (e != hipSuccess) return hip_status(e, "qlora_linear_fwd_noalloc (scratch address)");
    return qlora_linear_fwd(W, X, M, A, B, r, alpha, Y, T_out, ws, NF4_NOALLOC_SCRATCH_BYTES, stream);
}

nf4_status qlora_linear_bwd(const nf4_weight* W, const void* X, const void* dY, int64_t M,
                            const void* A, const void* B, int32_t r, float alpha, const void* T,
                            void* dX, float* dA, float* dB, void* workspace,
                            size_t workspace_bytes, void* stream) {
    WeightView v;
    nf4_status st = check_weight(W, v, true);
    if (st != NF4_OK) return st;
    st = check_lora(A, B, r, alpha);
    if (st != NF4_OK) return st;
    if (M < 0) return fail(NF4_ERR_ARG, "M must be >= 0");
    if (M >= LINEAR_M_LIMIT) return fail(NF4_ERR_UNSUPPORTED, "M must be below 2^23");
    if (M > 0 && dX && nf4::fused_bwd_plan(M, v.rows, v.cols).grid >= FUSED_GRID_LIMIT)
        return fail(NF4_ERR_UNSUPPORTED, "M x K needs more than 2^24 workgroups of 512 x 128 output tiles");
    if (!dA || !dB) return fail(NF4_ERR_ARG, "dA or dB is NULL");
    if (!aligned(dA, 4) || !aligned(dB, 4)) return fail(NF4_ERR_ARG, "dA/dB must be 4-byte aligned");
    if (M > 0 && (!X || !dY)) return fail(NF4_ERR_ARG, "X or dY is NULL");
    if (!aligned(X, 16) || !aligned(dY, 16) || !aligned(T, 16) || !aligned(dX, 16))
        return fail(NF4_ERR_ARG, "X, dY, T and dX must be 16-byte aligned");
    const size_t rb = rank_buffer_bytes(M, r);
    const size_t cb = c1_buffer_bytes(NF4_OP_LINEAR_BWD, M, v.rows, v.cols);
    const size_t pb = bwd_partial_bytes(M, v.rows, v.cols, r);
    const size_t need = 2 * rb + cb + pb + pack_bytes(NF4_OP_LINEAR_BWD, M, v.rows, v.cols);
    if (!workspace || workspace_bytes < need)
        return fail(NF4_ERR_WORKSPACE, "workspace smaller than nf4_workspace_bytes(NF4_OP_LINEAR_BWD)");
    if (!aligned(workspace, 256)) return fail(NF4_ERR_ARG, "workspace must be 256-byte aligned");
    const float s = alpha / (float)r;
    hipStream_t hs = (hipStream_t)stream;
    const uint16_t* x = (const uint16_t*)X;
    const uint16_t* g = (const uint16_t*)dY;
    const uint16_t* al = (const uint16_t*)A;
    const uint16_t* bl = (const uint16_t*)B;
    uint16_t* Us = (uint16_t*)workspace;       // s * dY B
    const uint16_t* Tb = (const uint16_t*)T;
    float* c1 = (float*)((char*)workspace + 2 * rb);
    float* part = (float*)((char*)workspace + 2 * rb + cb);
    uint16_t* gpk = (uint16_t*)((char*)workspace + 2 * rb + cb + pb);
    hipError_t e;
    if (M > 0) {
        // Us = s dY B   (B stored N x r: contraction-strided); with dX wanted, the same pass
        // writes dY in the fused product's fragment order
        // with dX wanted, extra workgroups of the slice-sum launch decode W's block constants
        const nf4::DqDecode dq{v.q, v.c2, v.mean, v.rows * (v.cols / 64), c1};
        e = nf4::launch_lora_gemm(g, false, bl, true, M, r, v.rows, part, s, Us, false, false,
                                  nullptr, 0.0f, hs, dX ? gpk : nullptr, false,
                                  (dX && !v.absmax) ? &dq : nullptr);
        if (e != hipSuccess) return hip_status(e, "qlora_linear_bwd (U)");
        if (!Tb) {
            uint16_t* Tw = (uint16_t*)((char*)workspace + rb);
            e = nf4::launch_lora_gemm(x, false, al, false, M, r, v.cols, part, 1.0f, Tw, false, false,
                                      nullptr, 0.0f, hs);
            if (e != hipSuccess) return hip_status(e, "qlora_linear_bwd (T)");
            Tb = Tw;
        }
        if (dX) {
            const float* c1b = v.absmax ? v.absmax : c1;   // plain constants: read as they are
            e = nf4::launch_fused_bwd_dx(v, c1b, gpk, M, Us, al, r, (uint16_t*)dX, part, table(), hs);
            if (e != hipSuccess) return hip_status(e, "qlora_linear_bwd (dX)");
        }
    }
    // dB = s dY^T T (N x r); dA^T = X^T (s U)  (K x r, stored transposed as dA r x K);
    // both contract over the M tokens (stored token-major: contraction-strided).  One launch
    // runs the two side by side, dB's workgroups first, each into its own partial slices.
    const nf4::TtProduct pb_dB{g, Tb, v.rows, r, M, part, s, dB, false};
    float* part_dA = (float*)((char*)part + nf4::skinny_partial_bytes(v.rows, r, M));
    const nf4::TtProduct pb_dA{x, Us, v.cols, r, M, part_dA, 1.0f, dA, true};
    e = nf4::launch_lora_tt_pair(pb_dB, pb_dA, hs);
    return hip_status(e, "qlora_linear_bwd (dA, dB)");
}

}  // extern "C"

namespace {

// Shared checks of the rank-r SVD and the LoftQ initialisation (host only).
nf4_status check_lowrank(const float* E, int64_t N, int64_t K, int32_t r, int32_t l, int32_t power_iters,
                         const float* omega) {
    if (!E || !omega) return fail(NF4_ERR_ARG, "matrix or omega is NULL");
    if (N < 1 || K < 1) return fail(NF4_ERR_ARG, "N and K must be >= 1");
    if (N >= ((int64_t)1 << 22) || K >= ((int64_t)1 << 22)) return fail(NF4_ERR_UNSUPPORTED, "N and K must be below 2^22");
    if (N * K >= ((int64_t)1 << 32)) return fail(NF4_ERR_UNSUPPORTED, "N*K must be below 2^32");
    if (r < 1 || l < r) return fail(NF4_ERR_ARG, "need 1 <= r <= l");
    if (l > nf4::LR_MAX) return fail(NF4_ERR_UNSUPPORTED, "sketch width l must be at most 96");
    if (l > N || l > K) return fail(NF4_ERR_ARG, "sketch width l must not exceed N or K");
    if (power_iters < 0 || power_iters > 16) return fail(NF4_ERR_ARG, "power_iters must be in [0, 16]");
    if (!aligned(E, 16) || !aligned(omega, 4)) return fail(NF4_ERR_ARG, "the matrix must be 16-byte aligned, omega 4-byte");
    return NF4_OK;
}

}  // namespace

extern "C" {

nf4_status nf4_lowrank_svd(const float* E, int64_t N, int64_t K, int32_t r, int32_t l, int32_t power_iters,
                           const float* omega, float* U, float* S, float* V, void* workspace,
                           size_t workspace_bytes, void* stream) {
    nf4_status st = check_lowrank(E, N, K, r, l, power_iters, omega);
    if (st != NF4_OK) return st;
    if (!U || !S || !V) return fail(NF4_ERR_ARG, "U, S or V is NULL");
    if (!aligned(U, 4) || !aligned(S, 4) || !aligned(V, 4)) return fail(NF4_ERR_ARG, "misaligned U, S or V");
    const size_t need = nf4::lowrank_ws_bytes(N, K, l, r);
    if (!workspace || workspace_bytes < need)
        return fail(NF4_ERR_WORKSPACE, "workspace smaller than nf4_workspace_bytes(NF4_OP_LOWRANK_SVD)");
    if (!aligned(workspace, 256)) return fail(NF4_ERR_ARG, "workspace must be 256-byte aligned");
    return hip_status(nf4::launch_lowrank_svd(E, N, K, r, l, power_iters, omega, U, S, V, workspace,
                                              (hipStream_t)stream),
                      "nf4_lowrank_svd");
}

nf4_status nf4_loftq_init(const float* W, int64_t N, int64_t K, int32_t r, float alpha, int32_t iters, int32_t l,
                          int32_t power_iters, const float* omega, uint8_t* codes, uint8_t* q, float* c2,
                          float* mean, void* A, void* B, double* err, void* workspace, size_t workspace_bytes,
                          void* stream) {
    nf4_status st = check_lowrank(W, N, K, r, l, power_iters, omega);
    if (st != NF4_OK) return st;
    if (!(alpha > 0.0f) || !isfinite(alpha)) return fail(NF4_ERR_ARG, "alpha must be positive and finite");
    if (iters < 1 || iters > 64) return fail(NF4_ERR_ARG, "iters must be in [1, 64]");
    if (!codes || !q || !c2 || !mean || !A || !B || !err) return fail(NF4_ERR_ARG, "an output is NULL");
    if (!aligned(codes, 4) || !aligned(q, 4) || !aligned(c2, 4) || !aligned(mean, 4) || !aligned(A, 2) ||
        !aligned(B, 2) || !aligned(err, 8))
        return fail(NF4_ERR_ARG, "misaligned output");
    const size_t need = nf4::loftq_ws_bytes(N, K, l, r);
    if (!workspace || workspace_bytes < need)
        return fail(NF4_ERR_WORKSPACE, "workspace smaller than nf4_workspace_bytes(NF4_OP_LOFTQ)");
    if (!aligned(workspace, 256)) return fail(NF4_ERR_ARG, "workspace must be 256-byte aligned");
    const float gamma = alpha / (float)r;
    return hip_status(nf4::launch_loftq(W, N, K, r, gamma, iters, l, power_iters, omega, codes, q, c2, mean,
                                        (uint16_t*)A, (uint16_t*)B, err, workspace, table(), (hipStream_t)stream),
                      "nf4_loftq_init");
}

}  // extern "C"

namespace {

// Hyperparameter checks and the per-step scalars of the AdamW update (bias
// corrections and the decay factor in double, rounded once to fp32).
nf4_status adamw_scalars(float lr, float beta1, float beta2, float eps, float weight_decay, int64_t step,
                         nf4::AdamwScalars& k) {
    if (step < 1) return fail(NF4_ERR_ARG, "step must be >= 1");
    if (!(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f))
        return fail(NF4_ERR_ARG, "beta1 and beta2 must lie in [0, 1)");
    if (!(eps > 0.0f) || !isfinite(eps)) return fail(NF4_ERR_ARG, "eps must be positive and finite");
    if (!isfinite(lr) || !isfinite(weight_decay)) return fail(NF4_ERR_ARG, "lr and weight_decay must be finite");
    const double bc1 = 1.0 - pow((double)beta1, (double)step);
    const double bc2 = 1.0 - pow((double)beta2, (double)step);
    if (!(bc1 > 0.0) || !(bc2 > 0.0)) return fail(NF4_ERR_ARG, "bias correction vanishes (beta = 0 with step 0?)");
    k.b1 = beta1;
    k.omb1 = (float)(1.0 - (double)beta1);
    k.b2 = beta2;
    k.omb2 = (float)(1.0 - (double)beta2);
    k.step_size = (float)((double)lr / bc1);
    k.inv_sqrt_bc2 = (float)(1.0 / sqrt(bc2));
    k.eps = eps;
    k.decay = (float)(1.0 - (double)lr * (double)weight_decay);
    return NF4_OK;
}

// Per device, for the copy-out of paged optimizer state: a helper stream (default
// priority) and the events that order it against the caller's stream, created on first
// use and kept for the life of the process.  Calls enqueue their work under the mutex,
// so every wait pairs with the record its own call made just before.
struct PagedResources {
    hipStream_t out = nullptr;
    hipEvent_t ready[2] = {nullptr, nullptr};
    hipEvent_t done[2] = {nullptr, nullptr};
};
std::mutex g_paged_mu;

hipError_t paged_resources(PagedResources** res) {
    static PagedResources per_dev[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    PagedResources& r = per_dev[dev];
    if (!r.out) {
        for (int b = 0; b < 2; ++b) {
            if (!r.ready[b]) e = hipEventCreateWithFlags(&r.ready[b], hipEventDisableTiming);
            if (e == hipSuccess && !r.done[b]) e = hipEventCreateWithFlags(&r.done[b], hipEventDisableTiming);
            if (e != hipSuccess) return e;
        }
        e = hipStreamCreateWithFlags(&r.out, hipStreamNonBlocking);
        if (e != hipSuccess) {
            r.out = nullptr;
            return e;
        }
    }
    *res = &r;
    return hipSuccess;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return a && b && x < y + nb && y < x + na;
}

}  // namespace

extern "C" {

nf4_status nf4_adamw_step(float* p, const float* g, float* m, float* v, uint16_t* p_bf16, int64_t n,
                          float lr, float beta1, float beta2, float eps, float weight_decay,
                          int64_t step, void* stream) {
    nf4::AdamwScalars k;
    nf4_status st = adamw_scalars(lr, beta1, beta2, eps, weight_decay, step, k);
    if (st != NF4_OK) return st;
    if (n < 0) return fail(NF4_ERR_ARG, "n must be >= 0");
    if (n == 0) return NF4_OK;
    if (!p || !g || !m || !v) return fail(NF4_ERR_ARG, "p, g, m or v is NULL");
    if (!aligned(p, 16) || !aligned(g, 16) || !aligned(m, 16) || !aligned(v, 16))
        return fail(NF4_ERR_ARG, "p, g, m and v must be 16-byte aligned");
    if (!aligned(p_bf16, 8)) return fail(NF4_ERR_ARG, "p_bf16 must be 8-byte aligned");
    const size_t b4 = (size_t)n * 4, b2 = (size_t)n * 2;
    const void* bufs[4] = {p, g, m, v};
    for (int i = 0; i < 4; ++i) {
        for (int j = i + 1; j < 4; ++j)
            if (overlaps(bufs[i], b4, bufs[j], b4)) return fail(NF4_ERR_ARG, "p, g, m and v must not overlap");
        if (overlaps(bufs[i], b4, p_bf16, b2)) return fail(NF4_ERR_ARG, "p_bf16 overlaps the state");
    }
    return hip_status(nf4::launch_adamw(p, g, m, v, p_bf16, n, k, (hipStream_t)stream), "nf4_adamw_step");
}

nf4_status nf4_adamw_step_paged(float* p_host, const float* g, float* m_host, float* v_host,
                                uint16_t* p_bf16, int64_t n, float lr, float beta1, float beta2,
                                float eps, float weight_decay, int64_t step, void* stage,
                                size_t stage_bytes, void* stream) {
    nf4::AdamwScalars k;
    nf4_status st = adamw_scalars(lr, beta1, beta2, eps, weight_decay, step, k);
    if (st != NF4_OK) return st;
    if (n < 0) return fail(NF4_ERR_ARG, "n must be >= 0");
    if (n == 0) return NF4_OK;
    if (!p_host || !g || !m_host || !v_host) return fail(NF4_ERR_ARG, "p, g, m or v is NULL");
    if (!aligned(g, 16)) return fail(NF4_ERR_ARG, "g must be 16-byte aligned");
    if (!aligned(p_bf16, 8)) return fail(NF4_ERR_ARG, "p_bf16 must be 8-byte aligned");
    if (!stage || !aligned(stage, 256)) return fail(NF4_ERR_ARG, "stage must be a 256-byte aligned buffer");
    if (stage_bytes < 1536) return fail(NF4_ERR_WORKSPACE, "stage must hold at least 1536 bytes");
    // two halves, each [p][m][v] of `chunk` parameters (a multiple of 64, so that every
    // staged vector stays 256-byte aligned): chunk c uses half c % 2
    const int64_t chunk = (int64_t)(stage_bytes / 1536) * 64;
    float* half[2] = {(float*)stage, (float*)stage + 3 * chunk};
    hipStream_t hs = (hipStream_t)stream;
    std::lock_guard<std::mutex> lock(g_paged_mu);
    PagedResources* res = nullptr;
    hipError_t e = paged_resources(&res);
    if (e != hipSuccess) return hip_status(e, "nf4_adamw_step_paged (helper stream)");
    hipStream_t out_stream = res->out;
    // ready[b]: half b updated (the copy-out may start); done[b]: half b copied out (the
    // next chunk of that half may be copied in)
    hipEvent_t* ready = res->ready;
    hipEvent_t* done = res->done;
    int64_t nchunks = 0;
    for (int64_t c0 = 0; c0 < n && e == hipSuccess; c0 += chunk, ++nchunks) {
        const int b = (int)(nchunks & 1);
        const int64_t cn = n - c0 < chunk ? n - c0 : chunk;
        const size_t nb = (size_t)cn * 4;
        float* sp = half[b];
        float* sm = sp + chunk;
        float* sv = sm + chunk;
        if (nchunks >= 2) e = hipStreamWaitEvent(hs, done[b], 0);
        if (e == hipSuccess) e = hipMemcpyAsync(sp, p_host + c0, nb, hipMemcpyHostToDevice, hs);
        if (e == hipSuccess) e = hipMemcpyAsync(sm, m_host + c0, nb, hipMemcpyHostToDevice, hs);
        if (e == hipSuccess) e = hipMemcpyAsync(sv, v_host + c0, nb, hipMemcpyHostToDevice, hs);
        if (e == hipSuccess) e = nf4::launch_adamw(sp, g + c0, sm, sv, p_bf16 ? p_bf16 + c0 : nullptr, cn, k, hs);
        if (e == hipSuccess) e = hipEventRecord(ready[b], hs);
        if (e == hipSuccess) e = hipStreamWaitEvent(out_stream, ready[b], 0);
        if (e == hipSuccess) e = hipMemcpyAsync(p_host + c0, sp, nb, hipMemcpyDeviceToHost, out_stream);
        if (e == hipSuccess) e = hipMemcpyAsync(m_host + c0, sm, nb, hipMemcpyDeviceToHost, out_stream);
        if (e == hipSuccess) e = hipMemcpyAsync(v_host + c0, sv, nb, hipMemcpyDeviceToHost, out_stream);
        if (e == hipSuccess) e = hipEventRecord(done[b], out_stream);
    }
    // the caller's stream completes after every copy-out
    for (int b = 0; b < 2 && b < nchunks && e == hipSuccess; ++b) e = hipStreamWaitEvent(hs, done[b], 0);
    return hip_status(e, "nf4_adamw_step_paged");
}

}  // extern "C"
