// bufio.h -- raw buffer loads for the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nf4 {

// Raw buffer access: a 128-bit descriptor in SGPRs, a per-lane 32-bit byte offset
// and a wave-uniform byte offset.  The hardware range check sees the per-lane offset
// (plus the instruction's immediate) only: a read whose per-lane offset reaches `bytes`
// returns zero, while the wave-uniform offset is added after the check.  Every
// wave-uniform offset below therefore stays inside the row it starts in, and offsets
// that can leave the valid region go into the per-lane offset or the descriptor.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const int64_t nrec = bytes <= 0 ? 0 : (bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nrec, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ float buf_loadf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}

// 16-bit store: dropped by the hardware when the per-lane offset reaches the range.
__device__ __forceinline__ void buf_store2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint16_t v) {
    __builtin_amdgcn_raw_buffer_store_b16(v, r, (int)voff, 0, 0);
}

}  // namespace nf4
