// tile_map.h -- work units of the fused dequant products: which output tile, and which
// part of the contraction, each workgroup computes (host and device).
#pragma once

#include <stddef.h>
#include <stdint.h>

#ifndef __HIPCC__
#define __host__
#define __device__
#define __forceinline__ inline
#endif

namespace nf4 {

constexpr int FUSED_TM = 512;           // output tile: tokens
constexpr int FUSED_TN = 128;           //              x features
constexpr int TILE_FLOATS = 65536;      // TM x TN of every tile shape
constexpr int XCDS = 8;                 // accelerator complex dies, each with its own L2
constexpr int XCD_CUS = 32;             // compute units per XCD (256 / 8)
constexpr int GROUP_M = 2;              // token tiles per group of the tile order
constexpr int MAX_SPLIT = 4;            // pieces per tail tile at most
// Fragment-order layout of the fused products' A operand (X forward, dY backward), written
// by k_skinny (lora.hip) and read by k_fused: one 64 KB block per (512-row token tile, 64-value step),
// 4096 chunks of 16 bytes.  Chunk q = 1024 w + 64 (4 i + s) + l is the 16 bytes lane l of
// wave w loads for MFMA fragment (row tile i, substep s): tile row 128 w + 32 i + l % 32,
// 16-byte column 2 s + l / 32 of the step's 128 bytes (contraction values 16 s + 8 (l / 32)
// .. + 7, the v_mfma_f32_32x32x16_bf16 A-operand layout).
constexpr int A_BLOCK_BYTES = 65536;
__host__ __device__ __forceinline__ int a_pack_row(int q) {
    return 128 * (q >> 10) + 32 * ((q >> 8) & 3) + (q & 31);
}
__host__ __device__ __forceinline__ int a_pack_col(int q) { return 2 * ((q >> 6) & 3) + ((q >> 5) & 1); }

// Split of a launch's tail tiles along the contraction (S == 1: none).  A launch with
// S > 1 needs `bytes` of split workspace: `tails` x S fp32 partial tiles, summed by a
// second kernel.  A pure function of the shape.
struct FusedPlan {
    int S;
    int64_t chunk;            // contraction steps per piece
    int64_t grid;             // workgroups
    int64_t tails;            // tail tile slots (8 x the fuller XCDs' tail)
    size_t bytes;             // split workspace (0 when S == 1)
};

// Launch over an M x ncols output in tm x tn tiles with `steps` 64-deep contraction
// steps.  One workgroup fills a compute unit, so an XCD runs its tiles in waves of
// XCD_CUS; when the last wave of the fuller XCDs is at most half full, each of its
// tiles is cut into S = min(4, XCD_CUS / tail) pieces (every piece non-empty).
__host__ __device__ __forceinline__ FusedPlan fused_plan(int64_t M, int64_t ncols, int64_t steps,
                                                         int tm = FUSED_TM, int tn = FUSED_TN) {
    FusedPlan p{1, steps, 0, 0, 0};
    const int64_t T = ((ncols + tn - 1) / tn) * ((M + tm - 1) / tm);
    p.grid = T;
    if (T == 0 || steps < 2) return p;
    const int64_t q = T / XCDS, rem = T % XCDS;
    const int64_t n0 = q + (rem ? 1 : 0);
    const int64_t r0 = n0 % XCD_CUS;
    if (r0 == 0 || 2 * r0 > XCD_CUS) return p;
    int S = (int)(XCD_CUS / r0 < MAX_SPLIT ? XCD_CUS / r0 : MAX_SPLIT);
    int64_t chunk = (steps + S - 1) / S;
    while (S > 1 && (S - 1) * chunk >= steps) {
        --S;
        chunk = (steps + S - 1) / S;
    }
    if (S == 1) return p;
    p.S = S;
    p.chunk = chunk;
    p.grid = XCDS * ((n0 - r0) + S * r0);
    p.tails = XCDS * r0;
    p.bytes = (size_t)(XCDS * r0 * S) * TILE_FLOATS * sizeof(float);
    return p;
}
inline FusedPlan fused_fwd_plan(int64_t M, int64_t N, int64_t K) { return fused_plan(M, N, K >> 6); }
inline FusedPlan fused_bwd_plan(int64_t M, int64_t N, int64_t K) { return fused_plan(M, K, (N + 63) >> 6); }

// Work unit of workgroup `wg`: output tile (tm, tn) and, for a tail tile, the piece of
// the contraction it covers.
//
// Workgroups are handed to the XCDs in turn: workgroup i runs on XCD i % 8.  The map
// gives XCD x a contiguous range of the tile order, and walks that order in groups of
// 2 token tiles, so the ~32 workgroups an XCD holds at once cover a compact 2 x 16 block
// of output tiles and share their A tiles and W' tiles in that XCD's L2 instead of
// fetching them again (2 x 16 fetched a third less than 4 x 8 at the same speed; 8 x 4
// fetched twice as much).  With S > 1, the last (tiles mod XCD_CUS) tiles of each XCD's
// range are run as S pieces each, by workgroups that follow the whole tiles in launch
// order on the same XCD (so the pieces of a tile share its L2).  Returns false for a
// workgroup with no unit (XCDs with one tile fewer than the first).
struct Unit {
    int64_t tm, tn;
    int split;                // -1: whole tile; else piece index
    int64_t tail;             // tail tile index: partial slots tail*S .. tail*S + S-1
};

// Tile order position p -> output tile (groups of GROUP_M token tiles).
__host__ __device__ __forceinline__ void tile_at(int64_t p, int64_t tiles_m, int64_t tiles_n, int64_t& tm,
                                                 int64_t& tn) {
    const int64_t per_group = GROUP_M * tiles_n;
    const int64_t first_m = (p / per_group) * GROUP_M;
    const int64_t gm = tiles_m - first_m < GROUP_M ? tiles_m - first_m : GROUP_M;
    const int64_t in_group = p % per_group;
    tm = first_m + in_group % gm;
    tn = in_group / gm;
}

__host__ __device__ __forceinline__ bool unit_of(int64_t wg, int64_t tiles_m, int64_t tiles_n, int S,
                                                 Unit& u) {
    const int64_t T = tiles_m * tiles_n;
    const int64_t q = T / XCDS, rem = T % XCDS;
    const int64_t x = wg % XCDS, local = wg / XCDS;
    const int64_t nx = q + (x < rem ? 1 : 0);
    const int64_t r0 = (q + (rem ? 1 : 0)) % XCD_CUS;   // tail of the fuller XCDs
    const int64_t rx = S > 1 ? nx % XCD_CUS : 0;
    const int64_t fx = nx - rx;
    int64_t p = x * q + (x < rem ? x : rem);
    if (local < fx) {
        p += local;
        u.split = -1;
        u.tail = 0;
    } else {
        const int64_t v = local - fx, ti = v / S;
        if (ti >= rx) return false;
        p += fx + ti;
        u.split = (int)(v % S);
        u.tail = x * r0 + ti;
    }
    tile_at(p, tiles_m, tiles_n, u.tm, u.tn);
    return true;
}

// Output tile of tail slot `t` (the inverse of Unit::tail); false for a slot no tile uses
// (XCDs with one tile fewer than the first).
__host__ __device__ __forceinline__ bool tail_tile(int64_t t, int64_t tiles_m, int64_t tiles_n, int64_t& tm,
                                                   int64_t& tn) {
    const int64_t T = tiles_m * tiles_n;
    const int64_t q = T / XCDS, rem = T % XCDS;
    const int64_t r0 = (q + (rem ? 1 : 0)) % XCD_CUS;
    if (r0 == 0) return false;
    const int64_t x = t / r0, ti = t % r0;
    const int64_t nx = q + (x < rem ? 1 : 0);
    const int64_t rx = nx % XCD_CUS;
    if (x >= XCDS || ti >= rx) return false;
    tile_at(x * q + (x < rem ? x : rem) + (nx - rx) + ti, tiles_m, tiles_n, tm, tn);
    return true;
}

// Contraction steps sb .. sb + n - 1 of a unit (piece `split` of `chunk` steps, or all).
__host__ __device__ __forceinline__ void unit_steps(int64_t all_steps, int64_t chunk, int split, int64_t& sb,
                                                    int64_t& n) {
    sb = split < 0 ? 0 : split * chunk;
    n = split < 0 ? all_steps : (all_steps - sb < chunk ? all_steps - sb : chunk);
}

}  // namespace nf4
