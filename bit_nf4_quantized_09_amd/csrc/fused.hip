// fused.hip -- NF4 dequantization fused into bf16 MFMA products (gfx950).
//
// "Paged optimizers, and QLoRA end to end" (zerotofrontier.app "sft/peft"):
// every frozen matrix is dequantized to bfloat16 block by block and multiplied
// in 16-bit precision, with the bf16 LoRA output added; gradients flow back
// through the dequantized weight.  "The real way": the dequantization is fused
// into the matrix multiply.  Layer formula: "Putting it together"
// (prism.theerrors.in QLoRA explainer).
//
// Forward  Y  = X W'^T + s T B^T   (NT product, contraction over K)
// Backward dX = dY W' + s U A      (NN product, contraction over N)
//
// Design for CDNA4: a TM x TN output tile per workgroup of 4 waves (each wave
// 128 x 128 = 4 x 4 tiles of v_mfma_f32_32x32x16_bf16, 256 fp32 accumulators per
// lane), one NF4 block (64 values) of contraction per pipeline step, two LDS
// stages.  The packed codes of one (row, 64-block) are owned by a pair of lanes (TN =
// 128), which build the block's 16-entry bf16 table scaled by its decoded constant
// together (each computes half and takes the other half from its partner); each lane
// then expands its share of the codes with byte permutes before writing them to LDS;
// every dequantized value is therefore computed once per workgroup and reused by TM
// rows of the other operand.  The decode work per MFMA falls as TM grows: the
// 512 x 128 tile (2 x 80 KB stages, the whole 160 KB LDS) decodes half as much per
// MFMA as a 256 x 256 tile.
#include "bufio.h"
#include "launch.h"

namespace nf4 {

// Tile geometry of k_fused<BWD, TM, TN>.
template <int TM, int TN>
struct FusedTile {
    static_assert(TM * TN == TILE_FLOATS && TM % 128 == 0 && TN % 128 == 0, "tile");
    static constexpr int WN = TN / 128;                  // waves across the tile (4 waves)
    static constexpr int A_BYTES = TM * 128;             // A tile: TM tokens x 64 bf16
    static constexpr int W_BYTES = TN * 128;             // W' tile: TN x 64 (fwd) or 64 x TN (bwd)
    static constexpr int STAGE = A_BYTES + W_BYTES;
    static constexpr int LDS = 2 * STAGE;
    static constexpr int ACH = TM / 32;                  // A tile 16-byte chunks per lane per step
    static constexpr int LPP = 256 / TN;                 // lanes per (row, 64-block) of W'
    static constexpr int CPL = 64 / LPP;                 // codes per lane per step
    static constexpr int NCH = CPL / 8;                  // 8-code chunks per lane per step
    static constexpr int NW = CPL / 32;                  // 16-byte code words per lane
    // A-tile register sets: two (8 chunks: loaded in step it for step it+2, written at the
    // end of step it+1), or one (16 chunks: chunks 2r, 2r+1 written in region r of step
    // it+1, reloaded for step it+2 two regions later)
    static constexpr int DEPTH = ACH <= 8 ? 2 : 1;
};

// [rows][64 bf16] tile with 128-byte rows: 16-byte chunk c of row r sits at chunk
// position c ^ g(r), g(r) = (r ^ (r >> 3)) & 7.  Any 16 consecutive rows reading the
// same chunk (one b128 pass of 16 lanes) then cover all 64 banks exactly once, and so
// do 8 consecutive rows (32-bank view).
__device__ __forceinline__ int tile_off(int row, int chunk) {
    return row * 128 + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4);
}

// Stage layout of the 160 KB of LDS (512 x 128 tiles): the A tiles [512 rows][128 B] of the
// two stages are interleaved by halves (rows 0-255 of stages 0 and 1 at 0 and 32 KB, rows
// 256-511 at 64 and 96 KB), then the W' tiles of stages 0 and 1 (16 KB each) at 128 and
// 144 KB.  Every stage offset (32 KB, 16 KB) then fits the 16-bit immediate of a DS
// instruction, so with the stage known at compile time each address is a loop-invariant
// per-lane base plus an immediate.
constexpr int A_STAGE_OFF = 32768;
constexpr int W_REGION = 131072;
constexpr int W_STAGE_OFF = 16384;
__device__ __forceinline__ int a_off(int row, int chunk) { return tile_off(row, chunk) + ((row >> 8) << 15); }

// Backward W' tile [64 n][TN k] with 2 TN-byte rows, read by ds_read_b64_tr_b16:
// 32-byte segment u (16 k values) of row r sits at u ^ 2(r & 3), so the 4 rows x 2
// segments that 32 lanes read in one pass land on distinct banks.
template <int TN>
__device__ __forceinline__ int wt_off(int row, int k) {
    return row * (2 * TN) + (((k >> 4) ^ ((row & 3) << 1)) << 5) + ((k & 15) << 1);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Transposing LDS read (gfx950 ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i receives element (i & 3) of the 4-element vectors addressed by lanes
// 4e + (i >> 2), e = 0..3.  With lane j addressing row (j >> 2), columns 4(j & 3)..+3
// of a 4 x 16 block, lane i receives column i of rows 0..3.
__device__ __forceinline__ uint2 ds_read_tr16(const uint8_t* p) {
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(const __attribute__((address_space(3))) uint8_t*)(p));
    return __builtin_bit_cast(uint2, v);
}

struct FusedArgs {
    const uint8_t* codes;
    const float* c1;          // decoded first-level constant of every 64-block (N * K/64)
    int64_t N, K;             // frozen weight rows (out features) and columns (in features)
    const uint16_t* A;        // X [M x K] (forward) or dY [M x N] (backward)
    int64_t M;
    const uint16_t* Rk;       // forward: s*T [M x r]; backward: s*U [M x r]
    const uint16_t* Lr;       // forward: B [N x r];   backward: A [r x K]
    int r;
    uint16_t* out;            // forward: Y [M x N];   backward: dX [M x K]
    // split contraction of the tail tiles (S == 1: none)
    int S;                    // pieces per tail tile
    int64_t chunk;            // contraction steps per piece
    float* spart;             // fp32 partial tiles, 65536 floats per (tail tile, piece)
};

// One lane's 16-byte chunks of an A tile (indexed with constants only, so that they
// stay in registers).
template <int N>
struct XRegs {
    uint4 r[N];
};

// This lane's packed codes of one (row, 64-block) and its decoded constant (zero past
// the last row).
template <int NW>
struct BlockCodes {
    uint4 w[NW];
    float c1;
};

template <bool BWD, int TM, int TN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_fused(FusedArgs a, Nf4Table tab) {
    using G = FusedTile<TM, TN>;
    static_assert(G::A_BYTES == 2 * A_STAGE_OFF && G::W_BYTES == W_STAGE_OFF && G::LDS == W_REGION + 2 * W_STAGE_OFF,
                  "stage layout");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / G::WN, wn = wave % G::WN;
    // forward tiles (tokens, out features); backward tiles (tokens, in features)
    Unit u;
    if (!unit_of(blockIdx.x, (a.M + TM - 1) / TM, ((BWD ? a.K : a.N) + TN - 1) / TN, a.S, u)) return;
    const int64_t c0 = u.tn * TN, m0 = u.tm * TM;
    const int64_t KB = a.K >> 6;
    const int64_t ldA = BWD ? a.N : a.K;                 // row length of the A operand
    const int64_t all_steps = BWD ? (a.N + 63) >> 6 : KB;   // 64-deep contraction steps
    int64_t sb, steps;                                    // this unit's steps sb .. sb + steps - 1
    unit_steps(all_steps, a.chunk, u.split, sb, steps);

    // ---- this lane's share of the packed weight: CPL codes of one (row, 64-block) per step ----
    // pair = tid / LPP, part = tid % LPP (codes part*CPL .. of the block).
    // forward: row c0 + pair, block = step; backward: row 64*step + pair / (TN/64), block
    // c0/64 + pair % (TN/64).  Rows past N fall outside the buffers' range and read zero
    // codes and a zero constant, so their dequantized values are zero.  The forward
    // advances by a wave-uniform offset inside the row; the backward moves the
    // descriptors down by 64 rows per step.
    const int pair = tid / G::LPP, part = tid % G::LPP;
    const int nl = BWD ? pair / (TN / 64) : pair;         // row of the W' tile (bwd: of 64)
    const int jb = BWD ? pair % (TN / 64) : 0;            // block of the tile (bwd)
    const int64_t kblk_b = (c0 >> 6) + jb < KB ? (c0 >> 6) + jb : KB - 1;
    const int64_t my_row0 = BWD ? nl : c0 + pair;         // row at step 0
    const uint32_t code_voff = (uint32_t)(my_row0 * (a.K >> 1) + (BWD ? kblk_b * 32 : 0) + part * (G::CPL / 2));
    const uint32_t c1_voff = (uint32_t)((my_row0 * KB + (BWD ? kblk_b : 0)) * 4);
    // The constant is requested first: it is needed first (scaled table), then the
    // codes, then the A tile (LDS write at the end of the step).
    auto load_codes = [&](int64_t lstep) {
        const int64_t step = sb + lstep;
        BlockCodes<G::NW> bc;
        if constexpr (BWD) {
            const int64_t r0 = step * 64;                  // first weight row of the step
            const __amdgpu_buffer_rsrc_t rs_c1 = make_rsrc(a.c1 + r0 * KB, (a.N - r0) * KB * 4);
            const __amdgpu_buffer_rsrc_t rs_codes = make_rsrc(a.codes + r0 * (a.K >> 1), (a.N - r0) * (a.K >> 1));
            bc.c1 = buf_loadf(rs_c1, c1_voff, 0);
#pragma unroll
            for (int i = 0; i < G::NW; ++i) bc.w[i] = buf_load16(rs_codes, code_voff + 16 * i, 0);
        } else {
            const __amdgpu_buffer_rsrc_t rs_c1 = make_rsrc(a.c1, a.N * KB * 4);
            const __amdgpu_buffer_rsrc_t rs_codes = make_rsrc(a.codes, a.N * (a.K >> 1));
            bc.c1 = buf_loadf(rs_c1, c1_voff, (uint32_t)(step * 4));
#pragma unroll
            for (int i = 0; i < G::NW; ++i) bc.w[i] = buf_load16(rs_codes, code_voff + 16 * i, (uint32_t)(step * 32));
        }
        return bc;
    };
    // LDS position of this lane's decoded chunk c (8 codes)
    auto w_off = [&](int c) {
        if constexpr (BWD) return wt_off<TN>(nl, jb * 64 + part * G::CPL + c * 8);
        else return tile_off(pair, part * G::NCH + c);
    };
    auto word = [&](const BlockCodes<G::NW>& bc, int c) {
        const uint4 v = bc.w[c >> 2];
        return (c & 3) == 0 ? v.x : (c & 3) == 1 ? v.y : (c & 3) == 2 ? v.z : v.w;
    };
    // the two lanes of a (row, 64-block) pair (tid 2i, 2i+1) build its scaled table together:
    // lane `part` computes entries 8 part .. 8 part + 7, and its codes are flipped to match
    static_assert(G::LPP == 2, "pair lanes");
    float lvh[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) lvh[i] = part ? tab.lv[8 + i] : tab.lv[i];
    const uint32_t flip = pair_code_flip(part);
    auto half_table = [&](float c) { return make_pair_table(lvh, c); };
    auto dequant_store = [&](uint8_t* sW, const BlockCodes<G::NW>& bc) {
        const ScaledTable st = half_table(bc.c1);
#pragma unroll
        for (int c = 0; c < G::NCH; ++c) {
            uint32_t o[4];
            decode8(st, word(bc, c) ^ flip, o);
            *reinterpret_cast<uint4*>(sW + w_off(c)) = make_uint4(o[0], o[1], o[2], o[3]);
        }
    };

    // ---- A operand tile: TM tokens x 64 contraction values, ACH chunks per lane ----
    // chunk i of this lane: tile row (tid >> 3) + 32 i, contraction chunk (tid & 7).  The
    // descriptor of a step starts at the step's first contraction value of the tile's
    // first row and ends with the tile's last row, so rows past M, and columns of the
    // last row past its end, read zero.  Backward columns past N of the other rows read
    // finite data of the next row and meet zeroed W' rows.
    // (the ABI bounds ldA so that every offset, a_chunk_offset(tid, i, ldA) + 16 bytes,
    // stays inside the descriptor's 2^31 - 1 byte range)
    static_assert(TM == FUSED_TM && G::ACH == A_CHUNKS, "A-tile offsets of tile_map.h");
    const int achunk = tid & 7;
    const int64_t arows = a.M - m0 < TM ? a.M - m0 : TM;
    const uint32_t a_voff0 = (uint32_t)a_chunk_offset(tid, 0, ldA);
    const uint32_t a_rstride = (uint32_t)(a_chunk_offset(tid, 1, ldA) - a_chunk_offset(tid, 0, ldA));
    auto a_rsrc = [&](int64_t lstep) {
        const int64_t step = sb + lstep;
        return make_rsrc(a.A + m0 * ldA + step * 64, arows * ldA * 2 - step * 128);
    };
    auto load_a = [&](XRegs<G::ACH>& X, int64_t lstep) {
        const __amdgpu_buffer_rsrc_t rs_a = a_rsrc(lstep);
#pragma unroll
        for (int i = 0; i < G::ACH; ++i) X.r[i] = buf_load16(rs_a, a_voff0 + i * a_rstride, 0);
    };
    auto store_a = [&](const XRegs<G::ACH>& X, uint8_t* sA) {
#pragma unroll
        for (int i = 0; i < G::ACH; ++i)
            *reinterpret_cast<uint4*>(sA + a_off((tid >> 3) + 32 * i, achunk)) = X.r[i];
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

    // B fragment of MFMA column tile j, substep sub (16 contraction values).  Backward: the
    // swizzle of wt_off depends on row & 3 only, so rows 16 sub + r and r + 4 sit at fixed
    // distances from row r: one per-lane base per column tile, the rest immediates.
    // (the bases hold the W' region's offset, which exceeds an immediate; the stage, substep
    // and second-read offsets do not)
    int bt_abs[4] = {0, 0, 0, 0};
    if constexpr (BWD) {
        const int g = lane >> 4, jl = lane & 15;
        const int row0 = 8 * (g >> 1) + (jl >> 2);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            bt_abs[j] = W_REGION + wt_off<TN>(row0, wn * 128 + j * 32 + 16 * (g & 1) + 4 * (jl & 3));
    }
    auto read_b = [&](const uint8_t* sB, int j, int sub) -> bf16x8 {
        if constexpr (BWD) {
            const int soff = (int)(sB - (lds + W_REGION));      // the stage's offset (0 or 16 KB)
            const uint8_t* p = lds + bt_abs[j] + (soff + sub * 16 * (2 * TN));
            const uint2 lo = ds_read_tr16(p);
            const uint2 hi = ds_read_tr16(p + 4 * (2 * TN));
            return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
        } else {
            const int rb = wn * 128 + j * 32 + (lane & 31);
            return *reinterpret_cast<const bf16x8*>(sB + tile_off(rb, 2 * sub + (lane >> 5)));
        }
    };
    auto mfma_step = [&](const uint8_t* sA, const uint8_t* sB, int nsub) {
#pragma unroll
        for (int sub = 0; sub < 4; ++sub) {
            if (sub < nsub) {
                const int ch = 2 * sub + (lane >> 5);
                bf16x8 fa[4], fb[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    fa[i] = *reinterpret_cast<const bf16x8*>(sA + a_off(wm * 128 + i * 32 + (lane & 31), ch));
#pragma unroll
                for (int j = 0; j < 4; ++j) fb[j] = read_b(sB, j, sub);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
            }
        }
    };

    // ---- main loop: the MFMAs of step `it` overlap the dequantization of step it+1 ----
    // The body is laid out by hand as 8 regions fenced by sched_barrier: region r
    // issues MFMAs 8r..8r+7 of this step (substep r/2), one slice of the
    // dequantization of the next step (region 0: block constant and scaled table;
    // region r > 0: chunk r-1 of this lane's codes and its LDS write), half of the
    // fragment reads of the following substep and a share of the A tile traffic.  Inside
    // a region, each MFMA is followed by a few VALU instructions, so the VALU work
    // executes while the matrix core is busy.
    // step `it` (stage it & 1): xn receives the A tile of step it+2 and xw holds that of
    // step it+1, to be written to the other stage.  Two sets: one chunk loaded per region,
    // xw written at the end.  One set (xn == xw): region r writes chunks 2r, 2r+1 and
    // reloads chunks 2r-4, 2r-3; chunks 12-15 are reloaded after the last region, so
    // every chunk has six regions to arrive.  With one set the decode of the next W'
    // tile runs in regions 3-7, away from the A-tile writes of the first regions.
    BlockCodes<G::NW> wcur;
    // (stage_tag: the stage of step `it`, it & 1, as a compile-time constant)
    auto step_body = [&](auto stage_tag, int64_t it, XRegs<G::ACH>& xn, const XRegs<G::ACH>& xw) {
        constexpr int st = decltype(stage_tag)::value;
        const int64_t n2 = it + 2 < steps ? it + 2 : steps - 1;
        const BlockCodes<G::NW> wnxt = load_codes(n2);
        const __amdgpu_buffer_rsrc_t rs_an = a_rsrc(n2);
        const uint8_t* sA = lds + st * A_STAGE_OFF;
        uint8_t* sAn = lds + (st ^ 1) * A_STAGE_OFF;
        const uint8_t* sB = lds + W_REGION + st * W_STAGE_OFF;
        uint8_t* sWn = lds + W_REGION + (st ^ 1) * W_STAGE_OFF;

        bf16x8 fa[2][4], fb[2][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            fa[0][i] = *reinterpret_cast<const bf16x8*>(sA + a_off(wm * 128 + i * 32 + (lane & 31), (lane >> 5)));
#pragma unroll
        for (int j = 0; j < 4; ++j) fb[0][j] = read_b(sB, j, 0);
        __builtin_amdgcn_sched_barrier(0);

        ScaledTable tbl;
#pragma unroll
        for (int rg = 0; rg < 8; ++rg) {
            const int sub = rg >> 1, half = rg & 1, fc = sub & 1;
            // next-substep fragments: region 2s loads A, region 2s+1 loads B
            if (sub < 3) {
                const int ch = 2 * (sub + 1) + (lane >> 5);
                if (half == 0) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        fa[fc ^ 1][i] = *reinterpret_cast<const bf16x8*>(sA + a_off(wm * 128 + i * 32 + (lane & 31), ch));
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) fb[fc ^ 1][j] = read_b(sB, j, sub + 1);
                }
            }
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int i = (half * 8 + t) >> 2, j = t & 3;
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[fc][i], fb[fc][j], acc[i][j], 0, 0, 0);
            }
            // A tile chunks, spread over the regions: a burst of wide loads at the top of
            // the step would stall the wave at the texture unit
            if constexpr (G::DEPTH == 2) {
                xn.r[rg] = buf_load16(rs_an, a_voff0 + rg * a_rstride, 0);
            } else {
                // region r writes chunks 2r, 2r+1 and (r >= 2) reloads chunks 2r-4, 2r-3
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int i = 2 * rg + q;
                    *reinterpret_cast<uint4*>(sAn + a_off((tid >> 3) + 32 * i, achunk)) = xw.r[i];
                }
                if (rg >= 2) {
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const int i = 2 * rg - 4 + q;
                        xn.r[i] = buf_load16(rs_an, a_voff0 + i * a_rstride, 0);
                    }
                }
            }
            // decode window: regions 0.. (two register sets) or 3.. (one set: the first
            // half carries the A tile writes)
            constexpr int D0 = G::DEPTH == 2 ? 0 : 3;
            if (rg == D0) {
                tbl = half_table(wcur.c1);
            } else if (rg > D0 && rg - D0 - 1 < G::NCH && rg - D0 - 1 < 7 - D0) {
                const int c = rg - D0 - 1;
                uint32_t o[4];
                decode8(tbl, word(wcur, c) ^ flip, o);
                *reinterpret_cast<uint4*>(sWn + w_off(c)) = make_uint4(o[0], o[1], o[2], o[3]);
            }
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);     // VALU
                if (t < (BWD && half ? 8 : 4) && sub < 3)
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); // DS read
                if (G::DEPTH == 2 ? t == 2 : (rg >= 2 && (t == 2 || t == 6)))
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
                if (G::DEPTH == 1 && (t == 4 || t == 7))
                    __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int c = (G::DEPTH == 2 ? 7 : 4); c < G::NCH; ++c) {
            uint32_t o[4];
            decode8(tbl, word(wcur, c) ^ flip, o);
            *reinterpret_cast<uint4*>(sWn + w_off(c)) = make_uint4(o[0], o[1], o[2], o[3]);
        }
        if constexpr (G::DEPTH == 2) {
            store_a(xw, sAn);
        } else {
            // the last four chunks of the A tile of step it+2
#pragma unroll
            for (int i = 12; i < 16; ++i) xn.r[i] = buf_load16(rs_an, a_voff0 + i * a_rstride, 0);
        }
        wcur = wnxt;
        __syncthreads();
    };

    // ---- prologue: stage 0 <- step 0; codes of step 1 (and, DEPTH 2, the A tile of step 1) ----
    XRegs<G::ACH> xa, xb;
    {
        load_a(xa, 0);
        const BlockCodes<G::NW> b0 = load_codes(0);
        store_a(xa, lds);
        dequant_store(lds + W_REGION, b0);
    }
    if constexpr (G::DEPTH == 2) {
        load_a(xb, steps > 1 ? 1 : 0);
        wcur = load_codes(steps > 1 ? 1 : 0);
    } else {
        // the loop's own request order (codes of a step, then the A tile of the step
        // before it), so that its waits need no slack for a different order
        wcur = load_codes(steps > 1 ? 1 : 0);
        load_a(xa, steps > 1 ? 1 : 0);
    }
    __syncthreads();

    if constexpr (G::DEPTH == 2) {
        int64_t it = 0;
        for (; it + 1 < steps; it += 2) {
            step_body(std::integral_constant<int, 0>{}, it, xa, xb);
            step_body(std::integral_constant<int, 1>{}, it + 1, xb, xa);
        }
        if (it < steps) step_body(std::integral_constant<int, 0>{}, it, xa, xb);
    } else {
        int64_t it = 0;
        for (; it + 1 < steps; it += 2) {
            step_body(std::integral_constant<int, 0>{}, it, xa, xa);
            step_body(std::integral_constant<int, 1>{}, it + 1, xa, xa);
        }
        if (it < steps) step_body(std::integral_constant<int, 0>{}, it, xa, xa);
    }

    // ---- rank-r adapter term, staged through stage 0 in rank chunks of 64 ----
    //   forward : acc += (s T) B^T   (A operand s*T [M x r], B operand rows of B [N x r])
    //   backward: acc += (s U) A     (A operand s*U [M x r], B operand A [r x K], transposed read)
    // (piece 0 only, for a split tile)
    const int rr = u.split <= 0 ? a.r : 0;
    for (int rc = 0; rc < rr; rc += 64) {
        uint8_t* sR = lds;                 // stage 0 of the layout above
        uint8_t* sL = lds + W_REGION;
#pragma unroll
        for (int i = 0; i < TM * 8 / 256; ++i) {
            const int qi = tid + 256 * i;
            const int row = qi >> 3, c = qi & 7;
            const int col = rc + 8 * c;
            const int64_t gm = m0 + row;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (col < a.r && gm < a.M) v = *reinterpret_cast<const uint4*>(a.Rk + gm * a.r + col);
            *reinterpret_cast<uint4*>(sR + a_off(row, c)) = v;
        }
#pragma unroll
        for (int i = 0; i < TN * 8 / 256; ++i) {
            const int qi = tid + 256 * i;
            if constexpr (BWD) {
                const int j = qi / (TN / 8), c = qi % (TN / 8);   // rank row j, 8 features per chunk
                const int64_t gk = c0 + 8 * c;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (rc + j < a.r && gk < a.K) v = *reinterpret_cast<const uint4*>(a.Lr + (int64_t)(rc + j) * a.K + gk);
                *reinterpret_cast<uint4*>(sL + wt_off<TN>(j, 8 * c)) = v;
            } else {
                const int row = qi >> 3, c = qi & 7;
                const int col = rc + 8 * c;
                const int64_t gn = c0 + row;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (col < a.r && gn < a.N) v = *reinterpret_cast<const uint4*>(a.Lr + gn * a.r + col);
                *reinterpret_cast<uint4*>(sL + tile_off(row, c)) = v;
            }
        }
        __syncthreads();
        const int left = a.r - rc;
        mfma_step(sR, sL, left >= 64 ? 4 : (left + 15) / 16);
        __syncthreads();
    }

    // ---- piece of a split tile: fp32 partial tile, row-major TM x TN, summed later ----
    if (u.split >= 0) {
        float* slot = a.spart + (u.tail * a.S + u.split) * (int64_t)TILE_FLOATS;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = wn * 128 + j * 32 + (lane & 31);
#pragma unroll
                for (int reg = 0; reg < 16; ++reg) {
                    const int row = wm * 128 + i * 32 + 8 * (reg >> 2) + 4 * (lane >> 5) + (reg & 3);
                    slot[row * TN + col] = acc[i][j][reg];
                }
            }
        return;
    }

    // ---- store bf16 ----
    const int64_t ncols = BWD ? a.K : a.N;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t col = c0 + wn * 128 + j * 32 + (lane & 31);
#pragma unroll
            for (int reg = 0; reg < 16; ++reg) {
                const int64_t row = m0 + wm * 128 + i * 32 + 8 * (reg >> 2) + 4 * (lane >> 5) + (reg & 3);
                if (row < a.M && col < ncols) a.out[row * ncols + col] = f32_to_bf16(acc[i][j][reg]);
            }
        }
}

FusedEvents& fused_events() {
    static thread_local FusedEvents ev;
    return ev;
}

// Sum of the S fp32 partial tiles of every split tail tile, in piece order, to bf16.
// Workgroup (slot t, part b) of a TM x TN tile: 256 runs of 8 columns, row-major.
template <int TN>
__global__ __launch_bounds__(256) void k_split_reduce(const float* __restrict__ spart, int S, int64_t M,
                                                      int64_t ncols, int64_t tiles_m, int64_t tiles_n,
                                                      uint16_t* __restrict__ out) {
    constexpr int TM = TILE_FLOATS / TN;
    const int64_t t = blockIdx.x >> 5;
    int64_t tm, tn;
    if (!tail_tile(t, tiles_m, tiles_n, tm, tn)) return;
    const int q = ((blockIdx.x & 31) << 8) + threadIdx.x;      // run of 8 floats in the tile
    const int row = q / (TN / 8), col = (q % (TN / 8)) * 8;
    const float* p = spart + t * S * (int64_t)TILE_FLOATS + row * TN + col;
    float4 lo = *reinterpret_cast<const float4*>(p), hi = *reinterpret_cast<const float4*>(p + 4);
    for (int pc = 1; pc < S; ++pc) {
        const float4 l2 = *reinterpret_cast<const float4*>(p + pc * (int64_t)TILE_FLOATS);
        const float4 h2 = *reinterpret_cast<const float4*>(p + pc * (int64_t)TILE_FLOATS + 4);
        lo.x += l2.x; lo.y += l2.y; lo.z += l2.z; lo.w += l2.w;
        hi.x += h2.x; hi.y += h2.y; hi.z += h2.z; hi.w += h2.w;
    }
    const int64_t grow = tm * TM + row, gcol = tn * TN + col;
    if (grow >= M || gcol >= ncols) return;
    const float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    uint16_t* o = out + grow * ncols + gcol;
    if ((ncols & 7) == 0) {
        uint4 w;
        w.x = f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
        w.y = f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
        w.z = f32_to_bf16(v[4]) | ((uint32_t)f32_to_bf16(v[5]) << 16);
        w.w = f32_to_bf16(v[6]) | ((uint32_t)f32_to_bf16(v[7]) << 16);
        *reinterpret_cast<uint4*>(o) = w;
    } else {
        for (int e = 0; e < 8 && gcol + e < ncols; ++e) o[e] = f32_to_bf16(v[e]);
    }
}

template <bool BWD>
static hipError_t launch_fused(FusedArgs fa, int64_t ncols, int64_t steps, void* split_ws,
                               const Nf4Table& tab, hipStream_t st) {
    constexpr int TM = FUSED_TM, TN = FUSED_TN;
    using G = FusedTile<TM, TN>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)k_fused<BWD, TM, TN>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, G::LDS);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const FusedPlan p = fused_plan(fa.M, ncols, steps);
    fa.S = p.S;
    fa.chunk = p.chunk;
    fa.spart = (float*)split_ws;
    if (p.S > 1 && !split_ws) return hipErrorInvalidValue;
    // the profiling events cover the product and, for split tail tiles, their sum
    return with_events(st, [&] {
        hipLaunchKernelGGL((k_fused<BWD, TM, TN>), dim3((unsigned)p.grid), dim3(256), G::LDS, st, fa, tab);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || p.S == 1) return e;
        hipLaunchKernelGGL(k_split_reduce<TN>, dim3((unsigned)(p.tails * 32)), dim3(256), 0, st, fa.spart, p.S,
                           fa.M, ncols, (fa.M + TM - 1) / TM, (ncols + TN - 1) / TN, fa.out);
        return hipGetLastError();
    });
}

hipError_t launch_fused_fwd(const WeightView& W, const float* c1, const uint16_t* X, int64_t M, const uint16_t* Ts,
                            const uint16_t* Bl, int r, uint16_t* Y, void* split_ws, const Nf4Table& tab,
                            hipStream_t st) {
    if (M == 0 || W.rows == 0) return hipSuccess;
    FusedArgs fa{W.codes, c1, W.rows, W.cols, X, M, Ts, Bl, r, Y, 1, 0, nullptr};
    return launch_fused<false>(fa, W.rows, W.cols >> 6, split_ws, tab, st);
}

hipError_t launch_fused_bwd_dx(const WeightView& W, const float* c1, const uint16_t* dY, int64_t M, const uint16_t* Us,
                               const uint16_t* Al, int r, uint16_t* dX, void* split_ws, const Nf4Table& tab,
                               hipStream_t st) {
    if (M == 0 || W.cols == 0) return hipSuccess;
    FusedArgs fa{W.codes, c1, W.rows, W.cols, dY, M, Us, Al, r, dX, 1, 0, nullptr};
    return launch_fused<true>(fa, W.cols, (W.rows + 63) >> 6, split_ws, tab, st);
}

}  // namespace nf4
