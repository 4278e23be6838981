// codebook.hip -- statistics of a blockwise quantization with any 16-level codebook (gfx950).
//
// "NF4, derived from normal quantiles" (zerotofrontier.app "sft/peft") compares NF4 with
// integer grids and with the codebook that minimises squared error (Lloyd's algorithm)
// on Gaussian blocks of 64, by RMS error and by the entropy of the codes.  One pass over
// (w, codes, absmax) gives what that comparison needs:
//   count[j]  values with code j                  (entropy)
//   sum_x[j]  sum of x = w / absmax over code j    (a Lloyd step: level j <- sum_x/count)
//   sse       sum of (w - fp32(level[code] absmax))^2, float64   (RMS error)
// A block with absmax 0 adds to count only (x = 0, no error).
//
// x is fp32(w / absmax) through the correctly rounded reciprocal and one correction
// (the IEEE quotient whenever that is a normal number); the sums are float64.
//
// Each lane owns one column of two LDS arrays, [16 codes][256 lanes] of u32 counts and
// of f64 sums: slot (j, lane) sits at j * 256 + lane, so the lanes of one LDS cycle hit
// distinct banks whatever their codes, and a slot is only ever touched by its own lane,
// in program order.  The workgroup then sums its 256 columns in a fixed tree, and a
// second kernel sums the workgroups in order: the result does not depend on timing.
#include "launch.h"

namespace nf4 {

constexpr int CB_THREADS = 256;
constexpr int CB_MAX_GRID = 1024;

int64_t codebook_stats_grid(int64_t n) {
    const int64_t chunks = (n + 7) / 8;
    int64_t g = (chunks + 8 * CB_THREADS - 1) / (8 * CB_THREADS);   // >= 8 chunks per lane
    if (g > CB_MAX_GRID) g = CB_MAX_GRID;
    if (g < 1) g = 1;
    return g;
}

size_t codebook_stats_ws_bytes(int64_t n) {
    return (size_t)codebook_stats_grid(n) * sizeof(CodebookStats);
}

template <typename T>
__device__ __forceinline__ float cb_value(const T* w, int64_t i) {
    if constexpr (sizeof(T) == 4) return __uint_as_float(w[i]);
    else return bf16_to_f32(w[i]);
}

template <typename T>
__global__ __launch_bounds__(CB_THREADS) void k_codebook_stats(const T* __restrict__ w, int64_t n,
                                                               const uint8_t* __restrict__ codes,
                                                               const float* __restrict__ absmax,
                                                               Nf4Table tab,
                                                               CodebookStats* __restrict__ part) {
    __shared__ uint32_t s_cnt[16 * CB_THREADS];
    __shared__ double s_sum[16 * CB_THREADS];
    __shared__ float s_lv[16];
    __shared__ double s_red[CB_THREADS];
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        s_cnt[j * CB_THREADS + tid] = 0u;
        s_sum[j * CB_THREADS + tid] = 0.0;
    }
    if (tid < 16) s_lv[tid] = tab.lv[tid];
    __syncthreads();

    uint32_t* my_cnt = s_cnt + tid;
    double* my_sum = s_sum + tid;
    double sse = 0.0;
    // LDS atomics without return: the lane does not wait for its previous update of the
    // same slot, and updates of one slot from one lane apply in issue order
    auto one = [&](float v, uint32_t code, float c, float y) {
        atomicAdd(my_cnt + code * CB_THREADS, 1u);
        if (c != 0.0f) {
            float x;
            if (__builtin_expect(c >= 0x1p-126f && c < 0x1p126f, 1)) {
                const float q = v * y;
                const float r = __fmaf_rn(-c, q, v);
                x = __fmaf_rn(r, y, q);
            } else {
                x = __fdiv_rn(v, c);      // reciprocal subnormal, zero or infinite
            }
            atomicAdd(my_sum + code * CB_THREADS, (double)x);
            const float wq = s_lv[code] * c;
            const double e = (double)v - (double)wq;
            sse += e * e;
        }
    };

    // chunk q: values 8q .. 8q+7, one 32-bit word of codes, inside block q / 8.  The
    // grid-stride loop is software-pipelined over two register sets: a chunk's requests
    // go out one iteration before its values are used (the next chunk index is clamped,
    // so the number of requests in flight never depends on a branch, and only loads are
    // in flight, so each wait covers exactly the chunk it needs).
    const int64_t n8 = n >> 3;
    auto fetch = [&](int64_t q, uint4& a, uint4& b, uint32_t& word, float& c) {
        if constexpr (sizeof(T) == 4) {
            a = reinterpret_cast<const uint4*>(w)[2 * q];
            b = reinterpret_cast<const uint4*>(w)[2 * q + 1];
        } else {
            a = reinterpret_cast<const uint4*>(w)[q];
        }
        word = reinterpret_cast<const uint32_t*>(codes)[q];
        c = absmax[q >> 3];
    };
    auto chunk = [&](uint4 a, uint4 b, uint32_t word, float c) {
        float v[8];
        if constexpr (sizeof(T) == 4) {
            v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
            v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y); v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
        } else {
            const uint32_t r4[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) { v[2 * j] = bf16_lo(r4[j]); v[2 * j + 1] = bf16_hi(r4[j]); }
        }
        const float y = __fdiv_rn(1.0f, c);
#pragma unroll
        for (int e = 0; e < 8; ++e) one(v[e], (word >> (4 * e)) & 15u, c, y);
    };
    const int64_t stride = (int64_t)gridDim.x * CB_THREADS;
    int64_t q = (int64_t)blockIdx.x * CB_THREADS + tid;
    if (q < n8) {
        uint4 a0, a1 = {}, b0, b1 = {};
        uint32_t aw, bw;
        float ac, bc;
        fetch(q, a0, a1, aw, ac);
        while (true) {
            int64_t qn = q + stride;
            fetch(qn < n8 ? qn : q, b0, b1, bw, bc);
            chunk(a0, a1, aw, ac);
            if (qn >= n8) break;
            q = qn;
            qn = q + stride;
            fetch(qn < n8 ? qn : q, a0, a1, aw, ac);
            chunk(b0, b1, bw, bc);
            if (qn >= n8) break;
            q = qn;
        }
    }
    // the last n % 8 values
    if (blockIdx.x == 0 && tid == 0) {
        for (int64_t i = n8 << 3; i < n; ++i) {
            const float c = absmax[i >> 6];
            one(cb_value(w, i), (codes[i >> 1] >> (4 * (i & 1))) & 15u, c, __fdiv_rn(1.0f, c));
        }
    }
    __syncthreads();

    // fixed-order sums over the 256 lanes: counts and per-code sums (one code per pass),
    // then the squared error
    auto tree = [&](double val) -> double {
        s_red[tid] = val;
        __syncthreads();
#pragma unroll
        for (int s = CB_THREADS / 2; s > 0; s >>= 1) {
            if (tid < s) s_red[tid] += s_red[tid + s];
            __syncthreads();
        }
        const double out = s_red[0];
        __syncthreads();
        return out;
    };
    CodebookStats* out = part + blockIdx.x;
    for (int j = 0; j < 16; ++j) {
        const double cj = tree((double)s_cnt[j * CB_THREADS + tid]);    // exact: < 2^53
        const double sj = tree(s_sum[j * CB_THREADS + tid]);
        if (tid == 0) {
            out->count[j] = (int64_t)cj;
            out->sum_x[j] = sj;
        }
    }
    const double se = tree(sse);
    if (tid == 0) out->sse = se;
}

// Sum of the workgroups' partial statistics (at most 1024) in a fixed order: thread t
// adds partials t, t + 256, t + 512, t + 768 in that order, then the 256 thread sums go
// through a fixed tree in LDS, one field at a time (16 counts, 16 sums, the squared
// error).  Every load is requested before the first add.
__global__ __launch_bounds__(CB_THREADS) void k_codebook_stats_reduce(const CodebookStats* __restrict__ part,
                                                                     int nparts,
                                                                     CodebookStats* __restrict__ out) {
    constexpr int F = 33;
    constexpr int PER = CB_MAX_GRID / CB_THREADS;
    __shared__ double s_red[CB_THREADS];
    const int tid = threadIdx.x;
    double acc[F];
#pragma unroll
    for (int f = 0; f < F; ++f) acc[f] = 0.0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int i = tid + CB_THREADS * k;
        if (i < nparts) {
            const CodebookStats& p = part[i];
            double v[F];
#pragma unroll
            for (int f = 0; f < 16; ++f) {
                v[f] = (double)p.count[f];
                v[16 + f] = p.sum_x[f];
            }
            v[32] = p.sse;
#pragma unroll
            for (int f = 0; f < F; ++f) acc[f] += v[f];
        }
    }
#pragma unroll
    for (int f = 0; f < F; ++f) {
        s_red[tid] = acc[f];
        __syncthreads();
#pragma unroll
        for (int s = CB_THREADS / 2; s > 0; s >>= 1) {
            if (tid < s) s_red[tid] += s_red[tid + s];
            __syncthreads();
        }
        if (tid == 0) {
            if (f < 16) out->count[f] = (int64_t)s_red[0];       // exact: counts < 2^53
            else if (f < 32) out->sum_x[f - 16] = s_red[0];
            else out->sse = s_red[0];
        }
        __syncthreads();
    }
}

hipError_t launch_codebook_stats(const void* w, bool w_bf16, int64_t n, const uint8_t* codes,
                                 const float* absmax, const Nf4Table& tab, CodebookStats* part,
                                 CodebookStats* out, hipStream_t s) {
    if (n == 0) {                   // no values: only the reduction, of no partials (zeros)
        hipLaunchKernelGGL(k_codebook_stats_reduce, dim3(1), dim3(CB_THREADS), 0, s, part, 0, out);
        return hipGetLastError();
    }
    const int64_t g = codebook_stats_grid(n);
    if (w_bf16)
        hipLaunchKernelGGL(k_codebook_stats<uint16_t>, dim3((unsigned)g), dim3(CB_THREADS), 0, s,
                           (const uint16_t*)w, n, codes, absmax, tab, part);
    else
        hipLaunchKernelGGL(k_codebook_stats<uint32_t>, dim3((unsigned)g), dim3(CB_THREADS), 0, s,
                           (const uint32_t*)w, n, codes, absmax, tab, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_codebook_stats_reduce, dim3(1), dim3(CB_THREADS), 0, s, part, (int)g, out);
    return hipGetLastError();
}

}  // namespace nf4
