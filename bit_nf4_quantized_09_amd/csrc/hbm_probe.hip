// Streaming probes of the HBM ceilings on gfx950: a linear read, a linear write and
// a copy of one buffer, each a grid-stride loop of 16-byte accesses with four in
// flight per lane.  They frame what the codec and few-token kernels can reach; no
// part of the NF4 path calls them.  Built into a library of their own.
#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace {

constexpr int PROBE_THREADS = 256;
constexpr int PROBE_UNROLL = 4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ u32x4 ld16(const u32x4* p) {
    if constexpr (NT) {
        return __builtin_nontemporal_load(p);
    } else {
        return *p;
    }
}

template <bool NT>
__device__ __forceinline__ void st16(u32x4* p, u32x4 v) {
    if constexpr (NT) {
        __builtin_nontemporal_store(v, p);
    } else {
        *p = v;
    }
}

// Reads n16 16-byte words and folds them into one xor; the fold is stored only when
// it equals a value no filled buffer gives, so the loads cannot be dropped.
template <bool NT>
__global__ __launch_bounds__(PROBE_THREADS) void k_probe_read(const u32x4* __restrict__ p, size_t n16,
                                                             uint32_t* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * PROBE_THREADS;
    size_t i = (size_t)blockIdx.x * PROBE_THREADS + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (PROBE_UNROLL - 1) * stride < n16; i += PROBE_UNROLL * stride) {
        u32x4 v[PROBE_UNROLL];
#pragma unroll
        for (int u = 0; u < PROBE_UNROLL; ++u) v[u] = ld16<NT>(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < PROBE_UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const u32x4 v = ld16<NT>(p + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9E3779B9u) sink[threadIdx.x] = acc;
}

template <bool NT>
__global__ __launch_bounds__(PROBE_THREADS) void k_probe_write(u32x4* __restrict__ p, size_t n16, uint32_t value) {
    const size_t stride = (size_t)gridDim.x * PROBE_THREADS;
    const u32x4 v = u32x4{value, value ^ 1u, value ^ 2u, value ^ 3u};
    size_t i = (size_t)blockIdx.x * PROBE_THREADS + threadIdx.x;
    for (; i + (PROBE_UNROLL - 1) * stride < n16; i += PROBE_UNROLL * stride) {
#pragma unroll
        for (int u = 0; u < PROBE_UNROLL; ++u) st16<NT>(p + i + u * stride, v);
    }
    for (; i < n16; i += stride) st16<NT>(p + i, v);
}

template <bool NT>
__global__ __launch_bounds__(PROBE_THREADS) void k_probe_copy(const u32x4* __restrict__ src,
                                                             u32x4* __restrict__ dst, size_t n16) {
    const size_t stride = (size_t)gridDim.x * PROBE_THREADS;
    size_t i = (size_t)blockIdx.x * PROBE_THREADS + threadIdx.x;
    for (; i + (PROBE_UNROLL - 1) * stride < n16; i += PROBE_UNROLL * stride) {
        u32x4 v[PROBE_UNROLL];
#pragma unroll
        for (int u = 0; u < PROBE_UNROLL; ++u) v[u] = ld16<NT>(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < PROBE_UNROLL; ++u) st16<NT>(dst + i + u * stride, v[u]);
    }
    for (; i < n16; i += stride) st16<NT>(dst + i, ld16<NT>(src + i));
}

int check(const void* a, size_t bytes, int grid) {
    if (a == nullptr || bytes == 0 || bytes % 16 != 0) return 1;
    if (grid < 1 || grid > (1 << 20)) return 1;
    return 0;
}

}  // namespace

extern "C" {

// kind: 0 read (sink: 256 uint32 of device memory), 1 write (dst), 2 copy (src -> dst).
// bytes: a multiple of 16; grid: workgroups of 256 lanes; nontemporal: 0 or 1.
// Returns 0, 1 for a bad argument, 2 when the launch fails.
int nf4probe_stream(int kind, const void* src, void* dst, size_t bytes, int grid, int nontemporal,
                    hipStream_t stream) {
    const size_t n16 = bytes / 16;
    const dim3 g(grid), b(PROBE_THREADS);
    const bool nt = nontemporal != 0;
    if (kind == 0) {
        if (check(src, bytes, grid) || dst == nullptr) return 1;
        auto* s = static_cast<const u32x4*>(src);
        auto* k = static_cast<uint32_t*>(dst);
        if (nt) hipLaunchKernelGGL(k_probe_read<true>, g, b, 0, stream, s, n16, k);
        else hipLaunchKernelGGL(k_probe_read<false>, g, b, 0, stream, s, n16, k);
    } else if (kind == 1) {
        if (check(dst, bytes, grid)) return 1;
        auto* d = static_cast<u32x4*>(dst);
        if (nt) hipLaunchKernelGGL(k_probe_write<true>, g, b, 0, stream, d, n16, 0x5A5A5A5Au);
        else hipLaunchKernelGGL(k_probe_write<false>, g, b, 0, stream, d, n16, 0x5A5A5A5Au);
    } else if (kind == 2) {
        if (check(src, bytes, grid) || check(dst, bytes, grid)) return 1;
        auto* s = static_cast<const u32x4*>(src);
        auto* d = static_cast<u32x4*>(dst);
        if (nt) hipLaunchKernelGGL(k_probe_copy<true>, g, b, 0, stream, s, d, n16);
        else hipLaunchKernelGGL(k_probe_copy<false>, g, b, 0, stream, s, d, n16);
    } else {
        return 1;
    }
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
