// codec.hip -- NF4 quantize, double quantization, constant decode and dequantize.
//
// zerotofrontier.app "sft/peft": "Block-wise quantization in one page" (absmax
// blocks of 64, nearest level), "NF4, derived from normal quantiles" (the
// levels), "Double quantization" (mean-subtracted 8-bit constants in blocks of
// 256 with fp32 second-level constants), "The real way" (two codes per byte).
// All of these kernels are HBM-bound streams.
#include <type_traits>

#include "launch.h"

namespace nf4 {

// ---------------------------------------------------------------------------
// Quantize.  One lane owns 16 consecutive values (64 bytes of fp32 or 32 of bf16);
// the 4 lanes of one 64-value block reduce the absmax with xor shuffles, then each
// lane encodes its values and writes 8 bytes of codes.  A workgroup takes 64 blocks
// per step and strides over the tensor.
//
// Division: for an absmax in [2^-126, 2^126), x = fp32(w / absmax) is formed from the
// correctly rounded reciprocal y = RN(1/absmax) (a normal number there; one IEEE
// division per lane) as q = RN(w y), r = w - absmax q (exact, fma), x = RN(q + r y).
// By Markstein's theorem (y within half an ulp of 1/absmax, q within one ulp of the
// quotient) this is the IEEE quotient whenever it is a normal number.  A quotient
// small enough to be subnormal lies far inside (-t, t) for the smallest encode
// threshold t ~ 0.04, so its code is the zero level whichever way it rounds: the
// codes equal those of the IEEE division.  Blocks with an absmax outside that range
// (subnormal, above 2^126, infinite) take the IEEE division itself.
//
// Encode: the code is the number of thresholds below x (nearest level, a value
// exactly between two levels taking the lower code).  |x| <= 1, so bucket
// b = floor(32 x) + 32 (exact: 32 x is exact) is in [0, 64]; bucket b covers
// [(b-32)/32, (b-31)/32).  The thresholds lie more than 1/32 apart, so a bucket
// holds at most one: code = (thresholds below the bucket) + (x > the bucket's
// threshold, +inf if none).  The same fp32 thresholds and strict comparisons as a
// search through all fifteen, in one LDS read, one compare and one add.
// ---------------------------------------------------------------------------
// floor(x) as an int in one v_cvt_flr_i32_f32 (for |x| < 2^31; (int)floorf(x) compiles to a
// v_floor_f32 and a v_cvt_i32_f32): quantize fp32 +3%, bf16 +3-5%
__device__ __forceinline__ int floor_to_int(float x) {
    int r;
    asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(r) : "v"(x));
    return r;
}

// values per lane: 64 bytes of fp32 or 32 of bf16 in flight per lane (8 values per lane
// measured 7% slower for fp32 and 20% for bf16; 32 per lane no faster)
constexpr int Q_EPL = 16;

template <typename T>
__global__ __launch_bounds__(256) void k_quantize(const T* __restrict__ w, int64_t n,
                                                  uint8_t* __restrict__ codes,
                                                  float* __restrict__ absmax, Nf4Table tab) {
    constexpr int EPL = Q_EPL;             // values per lane
    constexpr int LPB = 64 / EPL;          // lanes per 64-value block
    constexpr int QB = 256 / LPB;          // blocks per workgroup step
    constexpr int VPL = EPL * (int)sizeof(T) / 16;   // 16-byte loads per lane
    typedef uint32_t pack_t __attribute__((ext_vector_type(EPL / 8)));
    // {thresholds below, threshold bits}: entry 1 + b for bucket b; entry 0 takes a NaN
    // quotient (no threshold below it and none to pass: code 0)
    __shared__ uint2 s_bucket[66];
    if (threadIdx.x < 66) {
        const float lo = (float)((int)threadIdx.x - 33) * (1.0f / 32.0f);
        const float hi = lo + 1.0f / 32.0f;
        uint32_t below = 0;
        float th = __builtin_inff();
#pragma unroll
        for (int j = 0; j < 15; ++j) {
            below += tab.th[j] < lo ? 1u : 0u;
            th = (tab.th[j] >= lo && tab.th[j] < hi) ? tab.th[j] : th;
        }
        s_bucket[threadIdx.x] = threadIdx.x == 0 ? make_uint2(0u, 0x7F800000u)   // +inf
                                                 : make_uint2(below, __float_as_uint(th));
    }
    __syncthreads();

    const int64_t nblk = (n + 63) / 64;
    const int64_t steps = (nblk + QB - 1) / QB;
    const int sub = (int)(threadIdx.x % LPB);
    for (int64_t st = blockIdx.x; st < steps; st += gridDim.x) {
        const int64_t b = st * QB + threadIdx.x / LPB;
        if (b >= nblk) continue;           // whole 64-value groups leave together
        const int64_t base = b * 64 + (int64_t)sub * EPL;
        const bool full = (b * 64 + 64 <= n);

        float v[EPL];
        if (full) {
            uint4 raw[VPL];
#pragma unroll
            for (int i = 0; i < VPL; ++i) raw[i] = reinterpret_cast<const uint4*>(w + base)[i];
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const uint32_t r4[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
                if constexpr (sizeof(T) == 4) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[4 * i + j] = __uint_as_float(r4[j]);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) { v[8 * i + 2 * j] = bf16_lo(r4[j]); v[8 * i + 2 * j + 1] = bf16_hi(r4[j]); }
                }
            }
        } else {
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const int64_t idx = base + e;
                float x = 0.0f;
                if (idx < n) {
                    if constexpr (sizeof(T) == 4) x = __uint_as_float(w[idx]);
                    else x = bf16_to_f32(w[idx]);
                }
                v[e] = x;
            }
        }
        float m = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) m = fmaxf(m, fabsf(v[e]));
#pragma unroll
        for (int o = LPB / 2; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, LPB));
        if (sub == 0) absmax[b] = m;

        float x[EPL];
        if (__builtin_expect(m >= 0x1p-126f && m < 0x1p126f, 1)) {
            const float y = __fdiv_rn(1.0f, m);
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const float q = v[e] * y;
                const float r = __fmaf_rn(-m, q, v[e]);
                x[e] = __fmaf_rn(r, y, q);
            }
        } else {
            // a subnormal, huge or infinite absmax: the reciprocal would be subnormal,
            // infinite or zero, so the IEEE division itself
#pragma unroll
            for (int e = 0; e < EPL; ++e) x[e] = __fdiv_rn(v[e], m);
        }
        uint32_t packed[EPL / 8];
#pragma unroll
        for (int k = 0; k < EPL / 8; ++k) {
            uint32_t pw = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // table entry of the bucket, clamped in fp32 (|x| <= 1 puts every number in
                // entries 1..65): a NaN quotient (a NaN value, or an infinite one over an
                // infinite absmax) takes entry 0 and code 0, as the comparisons x > m_j all
                // fail for it (a zero block gives NaN too; its codes are replaced below)
                const float xe = x[8 * k + e];
                const int bi = floor_to_int(fminf(fmaxf(xe * 32.0f, -33.0f), 32.0f)) + 33;
                const uint2 bk = s_bucket[bi];
                const uint32_t code = bk.x + (xe > __uint_as_float(bk.y) ? 1u : 0u);
                pw |= code << (4 * e);
            }
            packed[k] = m == 0.0f ? tab.zero_word : pw;   // an all-zero block: the code of x = 0
        }
        uint8_t* dst = codes + base / 2;
        if (full) {
            pack_t pv;
#pragma unroll
            for (int k = 0; k < EPL / 8; ++k) pv[k] = packed[k];
            *reinterpret_cast<pack_t*>(dst) = pv;
        } else {
            const int64_t nbytes = (n + 1) / 2;
#pragma unroll
            for (int j = 0; j < EPL / 2; ++j) {
                if (base / 2 + j < nbytes) {
                    // codes past n are zero
                    uint32_t byte = (packed[j / 4] >> (8 * (j & 3))) & 0xFFu;
                    if (base + 2 * j + 1 >= n) byte &= 0x0Fu;
                    if (base + 2 * j >= n) byte = 0u;
                    dst[j] = (uint8_t)byte;
                }
            }
        }
    }
}

hipError_t launch_quantize(const void* w, bool w_bf16, int64_t n, uint8_t* codes, float* absmax,
                           const Nf4Table& tab, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const int64_t nblk = (n + 63) / 64;
    const int qb = 256 / (64 / Q_EPL);     // blocks per workgroup step
    const int64_t steps = (nblk + qb - 1) / qb;
    // enough workgroups to fill the chip several times over; each strides over the rest
    const unsigned grid = (unsigned)(steps < 8192 ? steps : 8192);
    if (w_bf16)
        hipLaunchKernelGGL(k_quantize<uint16_t>, dim3(grid), dim3(256), 0, s,
                           (const uint16_t*)w, n, codes, absmax, tab);
    else
        hipLaunchKernelGGL(k_quantize<uint32_t>, dim3(grid), dim3(256), 0, s,
                           (const uint32_t*)w, n, codes, absmax, tab);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Mean of the first-level constants.  S is the float64 sum over an aligned
// pairwise tree: neighbours 2i and 2i+1 are added at every level.  A workgroup
// reduces an aligned chunk of 2048 values (8 per lane in registers, then xor
// butterflies, then the 4 waves), which is exactly the tree restricted to that
// chunk; zero padding past the end leaves every sum unchanged because the
// constants are >= +0.  Chunks of chunks repeat the same step.
// ---------------------------------------------------------------------------
constexpr int SUM_CHUNK = 2048;

// Sum over the aligned pairwise tree of x[c0 .. c0 + 2048) (zeros past n), by the 256
// threads of a workgroup; the result is in every thread.
template <typename T>
__device__ __forceinline__ double chunk_tree_sum(const T* __restrict__ x, int64_t n, int64_t c0) {
    __shared__ double sw[4];
    const int64_t i0 = c0 + threadIdx.x * 8;
    double v[8];
    if (sizeof(T) == 4 && i0 + 8 <= n) {
        // fp32 constants (16-byte aligned; i0 is a multiple of 8): two 16-byte loads
        const float4 a = reinterpret_cast<const float4*>(x + i0)[0];
        const float4 b = reinterpret_cast<const float4*>(x + i0)[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (i0 + e < n) ? (double)x[i0 + e] : 0.0;
    }
    double s = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) s = s + __shfl_xor(s, o);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();                    // sw may still be read from a previous call
    if (lane == 0) sw[wave] = s;
    __syncthreads();
    return (sw[0] + sw[1]) + (sw[2] + sw[3]);
}

template <typename T>
__global__ __launch_bounds__(256) void k_pairwise_chunks(const T* __restrict__ x, int64_t n,
                                                         double* __restrict__ out, int64_t mean_n1,
                                                         float* __restrict__ mean) {
    const double r = chunk_tree_sum(x, n, (int64_t)blockIdx.x * SUM_CHUNK);
    if (threadIdx.x == 0) {
        if (mean_n1 >= 0) *mean = (mean_n1 > 0) ? (float)(r / (double)mean_n1) : 0.0f;
        else out[blockIdx.x] = r;
    }
}

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t double_quantize_ws_bytes(int64_t n1) {
    size_t total = 0;
    int64_t len = ceil_div(n1, SUM_CHUNK);
    if (len == 1) return sizeof(double);   // the single chunk sum
    while (len > 1) {
        total += (size_t)len;
        len = ceil_div(len, SUM_CHUNK);
    }
    return total * sizeof(double);
}

// Double quantization of a batch of tensors (a single tensor is a batch of one) in two
// launches: k_dqb_chunks sums every 2048-constant chunk of every tensor over the aligned
// pairwise tree (one workgroup per chunk, float64); k_dqb_encode re-sums a tensor's chunk
// sums over the same tree (the exact float64 sum S of all its constants; the group that
// starts the tensor stores mean = fp32(S / n1)) and encodes DQ_BLOCKS_PER_WG blocks of 256
// constants, one wave per block, 4 constants per lane.  A workgroup finds its tensor by a
// search over the batch's prefix counts (kernel arguments).  Tensors of up to 2048 chunks.
// ---------------------------------------------------------------------------
constexpr int DQ_BLOCKS_PER_WG = 16;

// The encode of block b (256 constants) of one tensor, by one wave.
__device__ __forceinline__ void dq_encode_block(const float* __restrict__ c1, int64_t n1, float mean, int64_t b,
                                                int lane, uint8_t* __restrict__ q, float* __restrict__ c2) {
    const int64_t base = b * 256 + lane * 4;
    const bool full = (b * 256 + 256 <= n1);
    float d[4];
    if (full) {
        const float4 c = *reinterpret_cast<const float4*>(c1 + base);
        d[0] = c.x - mean; d[1] = c.y - mean; d[2] = c.z - mean; d[3] = c.w - mean;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) d[e] = (base + e < n1) ? c1[base + e] - mean : 0.0f;
    }
    float m = fmaxf(fmaxf(fabsf(d[0]), fabsf(d[1])), fmaxf(fabsf(d[2]), fabsf(d[3])));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if (lane == 0) c2[b] = m;
    uint32_t packed = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t code = (m == 0.0f) ? 0u : e4m3_from_unit(__fdiv_rn(d[e], m));
        packed |= code << (8 * e);
    }
    if (full) {
        *reinterpret_cast<uint32_t*>(q + base) = packed;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (base + e < n1) q[base + e] = (uint8_t)(packed >> (8 * e));
    }
}

// Encode of a tensor past 2048 chunks (its mean already stored): one wave per block.
__global__ __launch_bounds__(64) void k_dq_encode(const float* __restrict__ c1, int64_t n1,
                                                  const float* __restrict__ mean_p,
                                                  uint8_t* __restrict__ q, float* __restrict__ c2) {
    dq_encode_block(c1, n1, *mean_p, blockIdx.x, threadIdx.x, q, c2);
}

// Tensor t of the batch holding item g of a prefix (first[t] <= g < first[t + 1]); the
// search is over kernel arguments, the same for every lane.
__device__ __forceinline__ int dqb_find(const int64_t* first, int count, int64_t g) {
    int lo = 0, hi = count - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (first[mid] <= g) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

__global__ __launch_bounds__(256) void k_dqb_chunks(DqBatch b) {
    const int64_t g = blockIdx.x;
    const int t = dqb_find(b.chunk0, b.count, g);
    const double r = chunk_tree_sum(b.c1[t], b.n1[t], (g - b.chunk0[t]) * SUM_CHUNK);
    if (threadIdx.x == 0) b.ws[g] = r;
}

__global__ __launch_bounds__(256) void k_dqb_encode(DqBatch b) {
    const int64_t g = blockIdx.x;
    const int t = dqb_find(b.group0, b.count, g);
    const int64_t n1 = b.n1[t];
    const double S = chunk_tree_sum(b.ws + b.chunk0[t], b.chunk0[t + 1] - b.chunk0[t], 0);
    const float mean = n1 > 0 ? (float)(S / (double)n1) : 0.0f;
    if (g == b.group0[t] && threadIdx.x == 0) *b.mean[t] = mean;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t nblk = (n1 + 255) / 256;
    for (int j = wave; j < DQ_BLOCKS_PER_WG; j += 4) {
        const int64_t blk = (g - b.group0[t]) * DQ_BLOCKS_PER_WG + j;
        if (blk >= nblk) break;
        dq_encode_block(b.c1[t], n1, mean, blk, lane, b.q[t], b.c2[t]);
    }
}

int64_t dqb_chunks(int64_t n1) { return ceil_div(n1, SUM_CHUNK); }
// encode groups of a tensor: at least one, which stores the mean of an empty tensor
int64_t dqb_groups(int64_t n1) {
    const int64_t g = ceil_div(ceil_div(n1, 256), DQ_BLOCKS_PER_WG);
    return g > 0 ? g : 1;
}

hipError_t launch_double_quantize_batch(int count, const float* const* c1, const int64_t* n1, uint8_t* const* q,
                                        float* const* c2, float* const* mean, double* ws, hipStream_t s) {
    for (int t0 = 0; t0 < count; t0 += DQB_MAX) {
        DqBatch b{};
        b.count = count - t0 < DQB_MAX ? count - t0 : DQB_MAX;
        b.ws = ws;
        b.chunk0[0] = 0;
        b.group0[0] = 0;
        for (int t = 0; t < b.count; ++t) {
            b.c1[t] = c1[t0 + t];
            b.n1[t] = n1[t0 + t];
            b.q[t] = q[t0 + t];
            b.c2[t] = c2[t0 + t];
            b.mean[t] = mean[t0 + t];
            b.chunk0[t + 1] = b.chunk0[t] + dqb_chunks(b.n1[t]);
            b.group0[t + 1] = b.group0[t] + dqb_groups(b.n1[t]);
        }
        if (b.chunk0[b.count] > 0) {
            hipLaunchKernelGGL(k_dqb_chunks, dim3((unsigned)b.chunk0[b.count]), dim3(256), 0, s, b);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(k_dqb_encode, dim3((unsigned)b.group0[b.count]), dim3(256), 0, s, b);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        ws += b.chunk0[b.count];
    }
    return hipSuccess;
}

size_t double_quantize_batch_ws_bytes(int count, const int64_t* n1) {
    size_t total = 0;
    for (int t = 0; t < count; ++t) total += (size_t)dqb_chunks(n1[t]);
    return total * sizeof(double);
}

hipError_t launch_double_quantize(const float* c1, int64_t n1, uint8_t* q, float* c2, float* mean,
                                  double* ws, hipStream_t s) {
    int64_t len = ceil_div(n1, SUM_CHUNK);
    if (n1 > 0 && len <= SUM_CHUNK) {
        // up to 2048^2 constants (2^28 weights): a batch of one (a single chunk's sum is the
        // whole tree's; the encode re-sums that one value)
        return launch_double_quantize_batch(1, &c1, &n1, &q, &c2, &mean, ws, s);
    }
    // larger tensors (and n1 = 0): repeated chunk reductions until one chunk is left; that
    // last pass writes the mean; then the encode
    if (len <= 1) {
        hipLaunchKernelGGL(k_pairwise_chunks<float>, dim3(1), dim3(256), 0, s, c1, n1,
                           (double*)nullptr, n1, mean);
    } else {
        hipLaunchKernelGGL(k_pairwise_chunks<float>, dim3((unsigned)len), dim3(256), 0, s, c1, n1,
                           ws, (int64_t)-1, (float*)nullptr);
        double* cur = ws;
        while (true) {
            const int64_t next = ceil_div(len, SUM_CHUNK);
            if (next <= 1) {
                hipLaunchKernelGGL(k_pairwise_chunks<double>, dim3(1), dim3(256), 0, s, cur, len,
                                   (double*)nullptr, n1, mean);
                break;
            }
            double* nxt = cur + len;
            hipLaunchKernelGGL(k_pairwise_chunks<double>, dim3((unsigned)next), dim3(256), 0, s,
                               cur, len, nxt, (int64_t)-1, (float*)nullptr);
            cur = nxt;
            len = next;
        }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || n1 == 0) return e;
    hipLaunchKernelGGL(k_dq_encode, dim3((unsigned)ceil_div(n1, 256)), dim3(64), 0, s, c1, n1,
                       mean, q, c2);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Two-level constant decode, one constant per lane.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_double_dequantize(const uint8_t* __restrict__ q,
                                                           const float* __restrict__ c2,
                                                           const float* __restrict__ mean_p,
                                                           int64_t n1, float* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n1) return;
    out[i] = decode_c1(q[i], c2_step(c2[i >> 8]), *mean_p);
}

hipError_t launch_double_dequantize(const uint8_t* q, const float* c2, const float* mean, int64_t n1,
                                    float* out, hipStream_t s) {
    if (n1 == 0) return hipSuccess;
    hipLaunchKernelGGL(k_double_dequantize, dim3((unsigned)ceil_div(n1, 256)), dim3(256), 0, s, q,
                       c2, mean, n1, out);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Dequantize.  Each wave handles chunks of 8 x 64 groups of E values (E = 4 for
// fp32 output, 8 for bf16, so one group is 16 bytes of output) in a grid-stride
// loop over the tensor's chunks; store j of lane l covers group 64 j + l of the
// chunk, so every store of a wave is one contiguous kilobyte.  The chunk's codes
// (256 E contiguous bytes) arrive in one or two 16-byte loads per lane, and its
// 8 E block constants in one load per lane, each lane decoding the constant of one
// block; both go through a wave-private LDS slot to the lanes that store them
// (LDS accesses of one wave execute in order, so no barrier is needed).  That is
// two or three requests per chunk where one request per store and operand cost
// most of the time; a wave requests its next chunk before storing the current one,
// so the requests of one chunk are in flight while the previous one is written.
// Levels come from a 256-entry LDS table of code byte -> the two fp32 levels.  The
// last chunk, when partial, takes a checked path with a request per group.
// ---------------------------------------------------------------------------
// s_waitcnt operand: vmcnt 0, expcnt and lgkmcnt unconstrained
constexpr int DQ_WAIT_VMCNT0 = 0x0F70;

template <bool OUT_BF16, bool PLAIN>
__global__ __launch_bounds__(256) void k_dequantize(const uint8_t* __restrict__ codes,
                                                    const uint8_t* __restrict__ q,
                                                    const float* __restrict__ c2,
                                                    const float* __restrict__ mean_p,
                                                    const float* __restrict__ absmax, int64_t n,
                                                    void* __restrict__ out, Nf4Table tab) {
    constexpr int E = OUT_BF16 ? 8 : 4;            // values per group (16 bytes of output)
    constexpr int WV = 8 * 64 * E;                 // values per wave chunk
    constexpr int WB = WV / 64;                    // its blocks: 32 or 64
    constexpr int WC = WV / 2;                     // its code bytes: 1 or 2 KB
    __shared__ float2 s_pair[256];                 // code byte -> (level of low nibble, of high nibble)
    __shared__ __attribute__((aligned(16))) uint8_t s_codes[4][WC];
    __shared__ float s_c1[4][WB];
    {
        float lo = 0.0f, hi = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            lo = (threadIdx.x & 15) == j ? tab.lv[j] : lo;
            hi = (threadIdx.x >> 4) == j ? tab.lv[j] : hi;
        }
        s_pair[threadIdx.x] = make_float2(lo, hi);
    }
    __syncthreads();
    const float mean = PLAIN ? 0.0f : *mean_p;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t nbytes = (n + 1) / 2;
    uint8_t* my_codes = s_codes[wave];
    float* my_c1 = s_c1[wave];

    // E levels of one group (codes cw, E/2 bytes) times its constant, stored at out + i0
    auto emit = [&](int64_t i0, uint32_t cw, float c1p, bool whole) {
        float v[E];
#pragma unroll
        for (int e = 0; e < E / 2; ++e) {
            const float2 l = s_pair[(cw >> (8 * e)) & 0xFFu];
            v[2 * e] = l.x * c1p;
            v[2 * e + 1] = l.y * c1p;
        }
        if constexpr (OUT_BF16) {
            uint16_t* o = reinterpret_cast<uint16_t*>(out) + i0;
            if (whole) {
                uint4 pk;
                pk.x = pack_bf16x2(v[0], v[1]); pk.y = pack_bf16x2(v[2], v[3]);
                pk.z = pack_bf16x2(v[4], v[5]); pk.w = pack_bf16x2(v[6], v[7]);
                *reinterpret_cast<uint4*>(o) = pk;
            } else {
                for (int e = 0; e < E; ++e)
                    if (i0 + e < n) o[e] = f32_to_bf16(v[e]);
            }
        } else {
            float* o = reinterpret_cast<float*>(out) + i0;
            if (whole) {
                *reinterpret_cast<float4*>(o) = make_float4(v[0], v[1], v[2], v[3]);
            } else {
                for (int e = 0; e < E; ++e)
                    if (i0 + e < n) o[e] = v[e];
            }
        }
    };
    auto constant_of = [&](int64_t blk) {
        if constexpr (PLAIN) return absmax[blk];
        else return decode_c1(q[blk], c2_step(c2[blk >> 8]), mean);
    };

    // a whole chunk's requests, made one chunk ahead of their use: the code bytes
    // 16 (64 k + lane) .. of the chunk, and block b0 + lane % WB (raw operands)
    auto fetch = [&](int64_t c, uint4& cw0, uint4& cw1, uint32_t& qb, float& cs) {
        const int64_t v0 = c * WV;
        const uint4* src = reinterpret_cast<const uint4*>(codes + v0 / 2);
        cw0 = src[lane];
        if constexpr (E == 8) cw1 = src[64 + lane];
        const int64_t blk = v0 / 64 + (lane & (WB - 1));
        if constexpr (PLAIN) {
            qb = 0;
            cs = absmax[blk];
        } else {
            qb = q[blk];
            cs = c2[blk >> 8];
        }
    };
    auto whole_chunk = [&](int64_t c, uint4 cw0, uint4 cw1, uint32_t qb, float cs) {
        const int64_t v0 = c * WV;
        const float c1p = PLAIN ? cs : decode_c1(qb, c2_step(cs), mean);
        *reinterpret_cast<uint4*>(my_codes + 16 * lane) = cw0;
        if constexpr (E == 8) *reinterpret_cast<uint4*>(my_codes + 16 * (64 + lane)) = cw1;
        if (lane < WB) my_c1[lane] = c1p;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int g = 64 * j + lane;
            uint32_t cw;
            if constexpr (E == 4) cw = *reinterpret_cast<const uint16_t*>(my_codes + 2 * g);
            else cw = *reinterpret_cast<const uint32_t*>(my_codes + 4 * g);
            emit(v0 + (int64_t)g * E, cw, my_c1[g * E / 64], true);
        }
    };

    // Whole chunks 0 .. nwhole-1 in a grid-stride loop over the waves, software-pipelined
    // over two register sets: each half waits for everything in flight (its own chunk's
    // operands and the previous chunk's stores), requests the next chunk (clamped to the
    // last whole one, so the request count never depends on a branch), then stores its
    // chunk.  The scheduling barriers keep the next half's work, which waits for the
    // requests just made, from moving in front of this half's stores.
    const int64_t gstride = (int64_t)gridDim.x * 4;
    const int64_t first = (int64_t)blockIdx.x * 4 + wave;
    const int64_t nwhole = n / WV;
    if (first < nwhole) {
        uint4 a0, a1 = {}, b0, b1 = {};
        uint32_t a_q, b_q;
        float a_c, b_c;
        fetch(first, a0, a1, a_q, a_c);
        int64_t c = first;
        while (true) {
            __builtin_amdgcn_s_waitcnt(DQ_WAIT_VMCNT0);
            __builtin_amdgcn_sched_barrier(0);
            fetch(c + gstride < nwhole ? c + gstride : nwhole - 1, b0, b1, b_q, b_c);
            whole_chunk(c, a0, a1, a_q, a_c);
            __builtin_amdgcn_sched_barrier(0);
            c += gstride;
            if (c >= nwhole) break;
            __builtin_amdgcn_s_waitcnt(DQ_WAIT_VMCNT0);
            __builtin_amdgcn_sched_barrier(0);
            fetch(c + gstride < nwhole ? c + gstride : nwhole - 1, a0, a1, a_q, a_c);
            whole_chunk(c, b0, b1, b_q, b_c);
            __builtin_amdgcn_sched_barrier(0);
            c += gstride;
            if (c >= nwhole) break;
        }
    }
    // the partial last chunk, by the wave whose sequence reaches it: groups past n store nothing
    if (nwhole * WV < n && nwhole >= first && (nwhole - first) % gstride == 0) {
        const int64_t v0 = nwhole * WV;
        for (int j = 0; j < 8; ++j) {
            const int64_t i0 = v0 + (int64_t)(64 * j + lane) * E;
            if (i0 >= n) continue;
            uint32_t cw = 0;
            for (int t = 0; t < E / 2; ++t)
                if (i0 / 2 + t < nbytes) cw |= (uint32_t)codes[i0 / 2 + t] << (8 * t);
            emit(i0, cw, constant_of(i0 / 64), i0 + E <= n);
        }
    }
}

hipError_t launch_dequantize(const WeightView& W, void* out, bool out_bf16, const Nf4Table& tab,
                             hipStream_t s) {
    const int64_t n = W.rows * W.cols;
    if (n == 0) return hipSuccess;
    const int64_t chunk = out_bf16 ? 256 * 8 * 8 : 256 * 8 * 4;
    const int64_t need = ceil_div(n, chunk);
    // up to 8192 workgroups (32 per CU): more in flight than 2048 measured 3-5% faster for
    // fp32 output; 16384 no faster
    const unsigned grid = (unsigned)(need < 8192 ? need : 8192);
    const bool plain = W.absmax != nullptr;
    if (out_bf16 && plain)
        hipLaunchKernelGGL((k_dequantize<true, true>), dim3(grid), dim3(256), 0, s, W.codes, W.q, W.c2,
                           W.mean, W.absmax, n, out, tab);
    else if (out_bf16)
        hipLaunchKernelGGL((k_dequantize<true, false>), dim3(grid), dim3(256), 0, s, W.codes, W.q, W.c2,
                           W.mean, W.absmax, n, out, tab);
    else if (plain)
        hipLaunchKernelGGL((k_dequantize<false, true>), dim3(grid), dim3(256), 0, s, W.codes, W.q, W.c2,
                           W.mean, W.absmax, n, out, tab);
    else
        hipLaunchKernelGGL((k_dequantize<false, false>), dim3(grid), dim3(256), 0, s, W.codes, W.q, W.c2,
                           W.mean, W.absmax, n, out, tab);
    return hipGetLastError();
}

}  // namespace nf4
