// nf4_common.h -- device helpers shared by the gfx950 kernels of the library.
//
// Number formats (zerotofrontier.app "sft/peft" page):
//   NF4   -- 16-level codebook, "NF4, derived from normal quantiles"; the levels
//            and the 15 encode thresholds are computed on the host and passed by
//            value (Nf4Table), so they live in SGPRs / constant registers.
//   E4M3  -- the 8-bit float of "Double quantization", read as OCP FP8 E4M3
//            (bias 7, largest finite 448); stored codes are 448 * (c1-mean)/c2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nf4 {

// 16 levels (ascending) and the 15 fp32 thresholds t_j: x > t_j exactly when
// x lies above the float64 midpoint between levels j and j+1.
struct Nf4Table {
    float lv[16];          // levels, ascending
    float th[15];          // th[j]: the largest fp32 not above the midpoint of lv[j], lv[j+1]
    uint32_t zero_word;    // eight codes of x = 0 (the code an all-zero block takes)
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// bf16
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Two fp32 -> packed bf16 pair (round to nearest even; one v_cvt_pk_bf16_f32).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    __bf16 a = (__bf16)f;
    return __builtin_bit_cast(uint16_t, a);
}

// ---------------------------------------------------------------------------
// OCP FP8 E4M3
// ---------------------------------------------------------------------------
// Exact value of a code (no NaN codes are ever produced).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
    const uint32_t e = (b >> 3) & 0xFu;
    const uint32_t m = b & 7u;
    // normal: (8+m) * 2^(e-10) -> fp32 exponent e-7+127, mantissa m<<20
    float normal = __uint_as_float(((e + 120u) << 23) | (m << 20));
    float sub = (float)m * 0x1p-9f;
    float mag = (e == 0u) ? sub : normal;
    return (b & 0x80u) ? -mag : mag;
}

// Nearest E4M3 code of v = s * 448 (exact in float64), ties to even code; the
// sign bit follows s.  |s| <= 1.
__device__ __forceinline__ uint32_t e4m3_from_unit(float s) {
    const uint32_t sign = (__float_as_uint(s) >> 24) & 0x80u;
    const double a = fabs((double)s * 448.0);
    if (a < 0x1p-6) {                                   // subnormal grid, step 2^-9
        const double m = rint(a * 512.0);               // 0..8; 8 is the smallest normal
        return sign | (uint32_t)m;
    }
    int e = ilogb(a);                                    // -6 .. 8
    double m = rint(ldexp(a, 3 - e));                    // 8 .. 16
    uint32_t mi = (uint32_t)m;
    if (mi == 16u) { mi = 8u; e += 1; }
    return sign | ((uint32_t)(e + 7) << 3) | (mi - 8u);
}

// Two-level constant decode: c1' = fma(E4M3(q), step, mean), step = fp32(c2/448).
__device__ __forceinline__ float decode_c1(uint32_t q, float step, float mean) {
    return __fmaf_rn(e4m3_to_f32(q), step, mean);
}

// step = fp32(c2 / 448), correctly rounded.  For 2^-100 <= |c2| <= FLT_MAX the product
// with the rounded reciprocal is corrected once by its exact fma residual; over that
// range the result equals the IEEE quotient for every fp32 input (checked exhaustively
// on the host), and no intermediate is subnormal.  Other inputs take the division.
__device__ __forceinline__ float c2_step(float c2) {
    const float a = fabsf(c2);
    if (__builtin_expect(a >= 0x1p-100f && a <= 0x1.fffffep+127f, 1)) {
        constexpr float rcp = 1.0f / 448.0f;
        const float q0 = c2 * rcp;
        const float e = __fmaf_rn(-q0, 448.0f, c2);
        return __fmaf_rn(e, rcp, q0);
    }
    return __fdiv_rn(c2, 448.0f);
}

// ---------------------------------------------------------------------------
// NF4 encode: number of thresholds below x, by a 4-step branch-free search.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t nf4_encode(float x, const Nf4Table& t) {
    uint32_t i = (x > t.th[7]) ? 8u : 0u;
    const float t3 = i ? t.th[11] : t.th[3];
    i += (x > t3) ? 4u : 0u;
    const float t1 = (i & 8u) ? ((i & 4u) ? t.th[13] : t.th[9]) : ((i & 4u) ? t.th[5] : t.th[1]);
    i += (x > t1) ? 2u : 0u;
    float t0;
    if (i & 8u) {
        t0 = (i & 4u) ? ((i & 2u) ? t.th[14] : t.th[12]) : ((i & 2u) ? t.th[10] : t.th[8]);
    } else {
        t0 = (i & 4u) ? ((i & 2u) ? t.th[6] : t.th[4]) : ((i & 2u) ? t.th[2] : t.th[0]);
    }
    i += (x > t0) ? 1u : 0u;
    return i;
}

// ---------------------------------------------------------------------------
// NF4 decode of 8 packed codes through a per-lane scaled table.
//
// The two lanes that share one (row, 64-block), adjacent lanes 2i and 2i+1, build the 16
// scaled values bf16(fp32(level_j * c1')) together: lane h of the pair computes entries
// 8h .. 8h+7 and splits them into a low-byte and a high-byte table (2 registers each), and a
// quad permute (v_mov_b32 DPP quad_perm [1,0,3,2]) hands each lane its partner's two pairs.
// Lane 0 then holds entries 0-7 in registers 0-1 and 8-15 in 2-3; lane 1 holds them the other
// way round, which flipping bit 3 of every code (pair_code_flip) undoes.  v_perm_b32 looks up
// four 8-entry byte tables at a time; bit 3 of each code picks the half.
// ---------------------------------------------------------------------------
struct ScaledTable {
    uint32_t lo[4];   // low bytes of 16 entries, four per register
    uint32_t hi[4];   // high bytes
};

// lvh: this lane's 8 levels (entries 8h .. 8h+7 of the codebook, h = lane & 1).  Both lanes of
// the pair must be active.
__device__ __forceinline__ ScaledTable make_pair_table(const float lvh[8], float c1p) {
    uint32_t p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = pack_bf16x2(lvh[2 * j] * c1p, lvh[2 * j + 1] * c1p);
    ScaledTable s;
    // bytes of p[2k] = [e0.lo e0.hi e1.lo e1.hi], p[2k+1] = [e2.lo ...]
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        s.lo[k] = __builtin_amdgcn_perm(p[2 * k + 1], p[2 * k], 0x06040200u);
        s.hi[k] = __builtin_amdgcn_perm(p[2 * k + 1], p[2 * k], 0x07050301u);
    }
    constexpr int SWAP_PAIRS = 0xB1;   // quad_perm [1,0,3,2]
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        s.lo[2 + k] = (uint32_t)__builtin_amdgcn_mov_dpp((int)s.lo[k], SWAP_PAIRS, 0xF, 0xF, false);
        s.hi[2 + k] = (uint32_t)__builtin_amdgcn_mov_dpp((int)s.hi[k], SWAP_PAIRS, 0xF, 0xF, false);
    }
    return s;
}

// XOR mask for the code words of lane h of a pair (see make_pair_table)
__device__ __forceinline__ uint32_t pair_code_flip(int h) { return h ? 0x88888888u : 0u; }

// Byte lane k of `sel` holds a code 0..15 and byte lane k of `hi8` is 0xFF exactly
// where that code is >= 8; returns the table's low and high bytes for the 4 codes.
__device__ __forceinline__ void lookup4(const ScaledTable& s, uint32_t sel, uint32_t hi8, uint32_t& lo,
                                        uint32_t& hi) {
    const uint32_t s7 = sel & 0x07070707u;
    const uint32_t la = __builtin_amdgcn_perm(s.lo[1], s.lo[0], s7);
    const uint32_t lb = __builtin_amdgcn_perm(s.lo[3], s.lo[2], s7);
    const uint32_t ha = __builtin_amdgcn_perm(s.hi[1], s.hi[0], s7);
    const uint32_t hb = __builtin_amdgcn_perm(s.hi[3], s.hi[2], s7);
    lo = (lb & hi8) | (la & ~hi8);
    hi = (hb & hi8) | (ha & ~hi8);
}

// v_perm_b32 selector values 8..11 return 0x00 or 0xFF from the sign bit of byte 1 or
// 3 of either source: 8 -> src1 byte 1, 9 -> src1 byte 3, 10 -> src0 byte 1,
// 11 -> src0 byte 3.  With the bit of interest moved to those sign positions this
// spreads one bit per byte lane into a full byte mask in a single instruction.
constexpr uint32_t SIGN_SPREAD = 0x090B080Au;

// 8 codes (nibble i = element i) -> 8 bf16 in element order (4 registers), or with
// EVEN_ODD in the order 0, 2, 4, 6, 1, 3, 5, 7 (a product whose other operand is permuted
// the same way within every 8-value chunk contracts to the same sum).
template <bool EVEN_ODD>
__device__ __forceinline__ void decode8(const ScaledTable& s, uint32_t w, uint32_t out[4]) {
    const uint32_t ev = w & 0x0F0F0F0Fu;           // elements 0,2,4,6
    const uint32_t od = (w >> 4) & 0x0F0F0F0Fu;    // elements 1,3,5,7
    // bit 3 of element 2k sits at bit 8k+3 of w, of element 2k+1 at bit 8k+7
    const uint32_t ev_hi8 = __builtin_amdgcn_perm(w << 12, w << 4, SIGN_SPREAD);
    const uint32_t od_hi8 = __builtin_amdgcn_perm(w << 8, w, SIGN_SPREAD);
    uint32_t elo, ehi, olo, ohi;
    lookup4(s, ev, ev_hi8, elo, ehi);
    lookup4(s, od, od_hi8, olo, ohi);
    // bf16 pairs (e0,e2),(e4,e6) and (o1,o3),(o5,o7)
    const uint32_t e01 = __builtin_amdgcn_perm(ehi, elo, 0x05010400u);
    const uint32_t e23 = __builtin_amdgcn_perm(ehi, elo, 0x07030602u);
    const uint32_t o01 = __builtin_amdgcn_perm(ohi, olo, 0x05010400u);
    const uint32_t o23 = __builtin_amdgcn_perm(ohi, olo, 0x07030602u);
    if constexpr (EVEN_ODD) {
        // elements in the order 0, 2, 4, 6, 1, 3, 5, 7 (four byte permutes fewer)
        out[0] = e01;
        out[1] = e23;
        out[2] = o01;
        out[3] = o23;
    } else {
        out[0] = __builtin_amdgcn_perm(o01, e01, 0x05040100u);   // elements 0,1
        out[1] = __builtin_amdgcn_perm(o01, e01, 0x07060302u);   // 2,3
        out[2] = __builtin_amdgcn_perm(o23, e23, 0x05040100u);   // 4,5
        out[3] = __builtin_amdgcn_perm(o23, e23, 0x07060302u);   // 6,7
    }
}

// The within-chunk order of decode8<true>, applied to 8 bf16 values (16 bytes, element
// order): the even elements, then the odd ones.
__device__ __forceinline__ uint4 even_odd8(uint4 v) {
    return make_uint4(__builtin_amdgcn_perm(v.y, v.x, 0x05040100u), __builtin_amdgcn_perm(v.w, v.z, 0x05040100u),
                      __builtin_amdgcn_perm(v.y, v.x, 0x07060302u), __builtin_amdgcn_perm(v.w, v.z, 0x07060302u));
}

}  // namespace nf4
