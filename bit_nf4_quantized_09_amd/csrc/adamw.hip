// adamw.hip -- the adapter's optimizer step (gfx950).
//
// "Paged optimizers, and QLoRA end to end" (zerotofrontier.app "sft/peft"): only the
// adapters learn, their Adam states live in paged memory and move between GPU and host
// RAM, and the step uses learning rates of 2e-4 (7B, 13B) and 1e-4 (33B, 65B).  The
// pages do not restate the update; it is the published one, Kingma & Ba, "Adam"
// (ICLR 2015) Algorithm 1, with the weight decay decoupled from the gradient as in
// Loshchilov & Hutter, "Decoupled Weight Decay Regularization" (ICLR 2019).
//
// The state is fp32 (master parameters p, moments m and v); the gradient g is the fp32
// dA or dB of the layer's backward.  Per element, in fp32 with no contraction:
//   m = b1 m + (1 - b1) g
//   v = b2 v + (1 - b2) g g
//   p = p (1 - lr wd) - (lr / bc1) (m / (sqrt(v) / sqrt(bc2) + eps))
// with bc1 = 1 - b1^t, bc2 = 1 - b2^t formed on the host in double.  An optional bf16
// copy of p (round to nearest even) is the operand the layer reads.
//
// The step is a stream over 28 bytes per parameter (30 with the bf16 copy): bound by HBM.
#include "launch.h"

namespace nf4 {

struct AdamwArgs {
    float* p;
    const float* g;
    float* m;
    float* v;
    uint16_t* pbf;        // bf16 copy of p, or null
    int64_t n;
    AdamwScalars k;
};

__device__ __forceinline__ void adamw_one(const AdamwScalars& k, float& p, float g, float& m, float& v) {
    m = k.b1 * m + k.omb1 * g;
    v = k.b2 * v + k.omb2 * (g * g);
    const float denom = __fsqrt_rn(v) * k.inv_sqrt_bc2 + k.eps;
    p = p * k.decay - k.step_size * __fdiv_rn(m, denom);
}

// Each lane updates 4 consecutive parameters per iteration (16-byte loads of p, g, m
// and v), two iterations at a time so that eight loads are in flight; the grid strides
// over the whole vector.  The last n % 4 parameters go to thread 0 of workgroup 0.
__global__ __launch_bounds__(256) void k_adamw(AdamwArgs a) {
    const int64_t n4 = a.n >> 2;
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + stride < n4; i += 2 * stride) {
        const int64_t j = i + stride;
        float4 p0 = reinterpret_cast<const float4*>(a.p)[i], p1 = reinterpret_cast<const float4*>(a.p)[j];
        const float4 g0 = reinterpret_cast<const float4*>(a.g)[i], g1 = reinterpret_cast<const float4*>(a.g)[j];
        float4 m0 = reinterpret_cast<const float4*>(a.m)[i], m1 = reinterpret_cast<const float4*>(a.m)[j];
        float4 v0 = reinterpret_cast<const float4*>(a.v)[i], v1 = reinterpret_cast<const float4*>(a.v)[j];
        adamw_one(a.k, p0.x, g0.x, m0.x, v0.x);
        adamw_one(a.k, p0.y, g0.y, m0.y, v0.y);
        adamw_one(a.k, p0.z, g0.z, m0.z, v0.z);
        adamw_one(a.k, p0.w, g0.w, m0.w, v0.w);
        adamw_one(a.k, p1.x, g1.x, m1.x, v1.x);
        adamw_one(a.k, p1.y, g1.y, m1.y, v1.y);
        adamw_one(a.k, p1.z, g1.z, m1.z, v1.z);
        adamw_one(a.k, p1.w, g1.w, m1.w, v1.w);
        reinterpret_cast<float4*>(a.p)[i] = p0;
        reinterpret_cast<float4*>(a.p)[j] = p1;
        reinterpret_cast<float4*>(a.m)[i] = m0;
        reinterpret_cast<float4*>(a.m)[j] = m1;
        reinterpret_cast<float4*>(a.v)[i] = v0;
        reinterpret_cast<float4*>(a.v)[j] = v1;
        if (a.pbf) {
            reinterpret_cast<uint2*>(a.pbf)[i] = make_uint2(pack_bf16x2(p0.x, p0.y), pack_bf16x2(p0.z, p0.w));
            reinterpret_cast<uint2*>(a.pbf)[j] = make_uint2(pack_bf16x2(p1.x, p1.y), pack_bf16x2(p1.z, p1.w));
        }
    }
    if (i < n4) {
        float4 p0 = reinterpret_cast<const float4*>(a.p)[i];
        const float4 g0 = reinterpret_cast<const float4*>(a.g)[i];
        float4 m0 = reinterpret_cast<const float4*>(a.m)[i];
        float4 v0 = reinterpret_cast<const float4*>(a.v)[i];
        adamw_one(a.k, p0.x, g0.x, m0.x, v0.x);
        adamw_one(a.k, p0.y, g0.y, m0.y, v0.y);
        adamw_one(a.k, p0.z, g0.z, m0.z, v0.z);
        adamw_one(a.k, p0.w, g0.w, m0.w, v0.w);
        reinterpret_cast<float4*>(a.p)[i] = p0;
        reinterpret_cast<float4*>(a.m)[i] = m0;
        reinterpret_cast<float4*>(a.v)[i] = v0;
        if (a.pbf)
            reinterpret_cast<uint2*>(a.pbf)[i] = make_uint2(pack_bf16x2(p0.x, p0.y), pack_bf16x2(p0.z, p0.w));
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        for (int64_t e = n4 << 2; e < a.n; ++e) {
            float p = a.p[e], m = a.m[e], v = a.v[e];
            adamw_one(a.k, p, a.g[e], m, v);
            a.p[e] = p;
            a.m[e] = m;
            a.v[e] = v;
            if (a.pbf) a.pbf[e] = f32_to_bf16(p);
        }
    }
}

hipError_t launch_adamw(float* p, const float* g, float* m, float* v, uint16_t* pbf, int64_t n,
                        const AdamwScalars& k, hipStream_t s) {
    if (n == 0) return hipSuccess;
    // up to 16 workgroups per CU, each lane with at least two iterations where n allows
    const int64_t n4 = n >> 2;
    int64_t grid = (n4 + 511) / 512;
    if (grid > 4096) grid = 4096;
    if (grid < 1) grid = 1;
    AdamwArgs a{p, g, m, v, pbf, n, k};
    hipLaunchKernelGGL(k_adamw, dim3((unsigned)grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace nf4
