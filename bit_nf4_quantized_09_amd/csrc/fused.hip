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
// Design for CDNA4: a 512 x 128 output tile (tokens x features) per workgroup of 4 waves.
// Wave w owns token rows 128 w .. 128 w + 127 of the tile and all 128 features: 4 x 4 tiles
// of v_mfma_f32_32x32x16_bf16, 256 fp32 accumulators per lane.  One NF4 block (64 values)
// of contraction per pipeline step.
//
// The A operand (X forward, dY backward) is private to a wave, so it goes from global
// memory straight into MFMA operand registers and never through LDS.  The rank-r product
// that reads the operand anyway (T = X A^T forward, U = dY B backward: k_skinny in
// lora.hip) also writes it in fragment order: for each 512-row token tile and
// 64-value contraction step, 64 KB holding, per wave and MFMA fragment (row tile i,
// substep s), the 16 bytes of each of the 64 lanes (row 128 w + 32 i + l % 32, contraction
// values 16 s + 8 (l / 32) .. + 7) contiguously, so that every fragment load is one
// coalesced kilobyte, with zeros past the last token row and past the contraction's end.
// The W' decode leaves each 8-value chunk in the order 0, 2, 4, 6, 1, 3, 5, 7, which saves
// its last four byte permutes (decode8<true>).  In the forward the chunk runs along the
// contraction, and every 16-byte piece of the packed X holds its 8 values in the same order (a
// contraction is blind to the order its pairs come in).  In the backward it runs along the
// output features: the rank-r operand A is staged in the same order, and the stores put each
// accumulator column back at its feature.
// (Loaded from the row-major operand, each lane of a fragment load would touch its own
// row: four times the cache lines per load instruction.)  Two register sets of A fragments
// (steps of even and odd index) are reloaded two steps ahead, each fragment as soon as its
// last MFMA of the step has issued.
//
// The W' tile is shared by the 4 waves and goes through LDS, decoded once per workgroup: the
// packed codes of one (row, 64-block) are owned by a pair of lanes, which build the block's
// 16-entry bf16 table scaled by its decoded constant together (each computes half and takes
// the other half from its partner); each lane then expands its 32 codes with byte permutes
// and writes them to one of two 16 KB LDS stages.  Every dequantized value is used by the
// tile's 512 token rows.
#include "bufio.h"
#include "launch.h"

namespace nf4 {

// W' tiles: [128 rows][64 bf16] forward (128-byte rows, XOR-swizzled 16-byte chunks) or
// [64 rows][128 bf16] backward (256-byte rows, read transposed); two stages.
constexpr int W_STAGE_BYTES = 16384;
constexpr int FUSED_LDS_BYTES = 2 * W_STAGE_BYTES;

// [rows][64 bf16] tile with 128-byte rows: 16-byte chunk c of row r sits at chunk
// position c ^ g(r), g(r) = (r ^ (r >> 3)) & 7.  Any 16 consecutive rows reading the
// same chunk (one b128 pass of 16 lanes) then cover all 64 banks exactly once.
__device__ __forceinline__ int tile_off(int row, int chunk) {
    return row * 128 + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4);
}

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
    const uint16_t* A;        // X [M x K] (forward) or dY [M x N] (backward), in fragment order
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

// One step's A fragments of a lane: [row tile i][substep s], 8 bf16 each (indexed with
// constants only, so that they stay in registers).
struct AFrags {
    uint4 f[4][4];
};

// This lane's packed codes of one (row, 64-block) and its decoded constant (zero past
// the last row).
struct BlockCodes {
    uint4 w;
    float c1;
};

template <bool BWD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_fused(FusedArgs a, Nf4Table tab) {
    constexpr int TM = FUSED_TM, TN = FUSED_TN;
    static_assert(TM == 512 && TN == 128 && TM * TN == TILE_FLOATS, "tile");
    __shared__ __attribute__((aligned(16))) uint8_t lds[FUSED_LDS_BYTES];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, rl = lane & 31;
    // forward tiles (tokens, out features); backward tiles (tokens, in features)
    Unit u;
    if (!unit_of(blockIdx.x, (a.M + TM - 1) / TM, ((BWD ? a.K : a.N) + TN - 1) / TN, a.S, u)) return;
    const int64_t c0 = u.tn * TN, m0 = u.tm * TM;
    const int64_t KB = a.K >> 6;
    const int64_t all_steps = BWD ? (a.N + 63) >> 6 : KB;   // 64-deep contraction steps
    int64_t sb64, steps64;                                // this unit's steps sb .. sb + steps - 1
    unit_steps(all_steps, a.chunk, u.split, sb64, steps64);
    // 32-bit and wave-uniform (said so), so that the step arithmetic, the buffer offsets and
    // the descriptors stay in scalar registers (steps < 2^16: N, K < 2^22)
    const int sb = __builtin_amdgcn_readfirstlane((int)sb64);
    const int steps = __builtin_amdgcn_readfirstlane((int)steps64);

    // ---- this lane's share of the packed weight: 32 codes of one (row, 64-block) per step ----
    // pair = tid / 2, part = tid % 2 (codes 32 part .. of the block).
    // forward: row c0 + pair, block = step; backward: row 64*step + pair / 2, block
    // c0/64 + pair % 2.  Rows past N fall outside the buffers' range and read zero
    // codes and a zero constant, so their dequantized values are zero.  The forward
    // advances by a wave-uniform offset inside the row; the backward moves the
    // descriptors down by 64 rows per step.
    const int pair = tid >> 1, part = tid & 1;
    const int nl = BWD ? pair >> 1 : pair;                // row of the W' tile (bwd: of 64)
    const int jb = BWD ? pair & 1 : 0;                    // block of the tile (bwd)
    const int64_t kblk_b = (c0 >> 6) + jb < KB ? (c0 >> 6) + jb : KB - 1;
    const int64_t my_row0 = BWD ? nl : c0 + pair;         // row at step 0
    const uint32_t code_voff = (uint32_t)(my_row0 * (a.K >> 1) + (BWD ? kblk_b * 32 : 0) + part * 16);
    const uint32_t c1_voff = (uint32_t)((my_row0 * KB + (BWD ? kblk_b : 0)) * 4);
    // The constant is requested first: it is needed first (scaled table), then the codes.
    auto load_codes = [&](int lstep) {
        const int step = sb + lstep;
        BlockCodes bc;
        if constexpr (BWD) {
            const int64_t r0 = (int64_t)step * 64;         // first weight row of the step
            const __amdgpu_buffer_rsrc_t rs_c1 = make_rsrc(a.c1 + r0 * KB, (a.N - r0) * KB * 4);
            const __amdgpu_buffer_rsrc_t rs_codes = make_rsrc(a.codes + r0 * (a.K >> 1), (a.N - r0) * (a.K >> 1));
            bc.c1 = buf_loadf(rs_c1, c1_voff, 0);
            bc.w = buf_load16(rs_codes, code_voff, 0);
        } else {
            const __amdgpu_buffer_rsrc_t rs_c1 = make_rsrc(a.c1, a.N * KB * 4);
            const __amdgpu_buffer_rsrc_t rs_codes = make_rsrc(a.codes, a.N * (a.K >> 1));
            bc.c1 = buf_loadf(rs_c1, c1_voff, (uint32_t)(step * 4));
            bc.w = buf_load16(rs_codes, code_voff, (uint32_t)(step * 32));
        }
        return bc;
    };
    // LDS position (in a stage) of this lane's decoded chunk c (8 codes)
    auto w_off = [&](int c) {
        if constexpr (BWD) return wt_off<TN>(nl, jb * 64 + part * 32 + c * 8);
        else return tile_off(pair, part * 4 + c);
    };
    auto word = [&](const BlockCodes& bc, int c) {
        return c == 0 ? bc.w.x : c == 1 ? bc.w.y : c == 2 ? bc.w.z : bc.w.w;
    };
    // the two lanes of a (row, 64-block) pair (tid 2i, 2i+1) build its scaled table together:
    // lane `part` computes entries 8 part .. 8 part + 7, and its codes are flipped to match
    float lvh[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) lvh[i] = part ? tab.lv[8 + i] : tab.lv[i];
    const uint32_t flip = pair_code_flip(part);
    auto decode_chunk = [&](uint8_t* sW, const ScaledTable& st, const BlockCodes& bc, int c) {
        uint32_t o[4];
        decode8<true>(st, word(bc, c) ^ flip, o);
        *reinterpret_cast<uint4*>(sW + w_off(c)) = make_uint4(o[0], o[1], o[2], o[3]);
    };

    // ---- A operand: 16 fragments per lane and step, from the packed operand ----
    // The step's 64 KB block of this token tile: wave w's fragment (i, s) is the kilobyte at
    // 16 KB w + 1 KB (4 i + s), lane l's 16 bytes at 16 l of it.
    uint32_t a_voff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a_voff[i] = (uint32_t)(wave * 16384 + 4096 * i + lane * 16);
    const uint16_t* a_tile = a.A + u.tm * all_steps * (int64_t)(A_BLOCK_BYTES / 2);
    auto a_rsrc = [&](int lstep) {
        return make_rsrc(a_tile + (int64_t)(sb + lstep) * (A_BLOCK_BYTES / 2), A_BLOCK_BYTES);
    };
    auto load_frag = [&](__amdgpu_buffer_rsrc_t rs, int i, int s) {
        return buf_load16(rs, a_voff[i] + 1024 * s, 0);
    };
    auto load_all = [&](AFrags& F, int lstep) {
        const __amdgpu_buffer_rsrc_t rs = a_rsrc(lstep);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) F.f[i][s] = load_frag(rs, i, s);
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

    // W' fragment of MFMA column tile j, substep s, from stage `st` (contraction values
    // 16 s + 8 h .. + 7 of the step).  Forward: row 32 j + rl, chunk 2 s + h.  Backward: the
    // swizzle of wt_off depends on row & 3 only, so rows 16 s + 8 h + r and r + 4 sit at fixed
    // distances from row 8 h + r: one per-lane base per column tile, the rest immediates.
    int bt_abs[4] = {0, 0, 0, 0};
    if constexpr (BWD) {
        const int g = lane >> 4, jl = lane & 15;
        const int row0 = 8 * (g >> 1) + (jl >> 2);
#pragma unroll
        for (int j = 0; j < 4; ++j) bt_abs[j] = wt_off<TN>(row0, j * 32 + 16 * (g & 1) + 4 * (jl & 3));
    }
    auto read_b = [&](int st, int j, int s) -> bf16x8 {
        if constexpr (BWD) {
            const uint8_t* p = lds + st * W_STAGE_BYTES + bt_abs[j] + s * 16 * (2 * TN);
            const uint2 lo = ds_read_tr16(p);
            const uint2 hi = ds_read_tr16(p + 4 * (2 * TN));
            return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
        } else {
            return *reinterpret_cast<const bf16x8*>(lds + st * W_STAGE_BYTES + tile_off(j * 32 + rl, 2 * s + h));
        }
    };
    auto mfma = [&](int i, int j, uint4 af, bf16x8 bf) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af), bf, acc[i][j], 0, 0, 0);
    };

    // ---- main loop: the MFMAs of step `it` overlap the dequantization of step it+1 ----
    // The body is laid out by hand as 8 regions fenced by sched_barrier: region r issues
    // MFMAs 8r..8r+7 of this step (substep r/2, row tiles 2(r%2), 2(r%2)+1), then reloads the
    // two A fragments they consumed for step it+2, reads the next substep's W' fragments
    // (even regions) and carries one slice of the decode of the next step's W' tile (region
    // 0: block constant and scaled table; regions 1-4: one 8-code chunk each, decoded and
    // written to the other stage).  The last region's MFMAs run after the step's barrier,
    // behind the first W' reads of the next step, so that those reads' latency is hidden.
    BlockCodes wcur;
    bf16x8 fb[2][4];
    // (stage_tag: the stage of step `it`, it & 1, as a compile-time constant; `cur` holds the
    // A fragments of step it and receives those of step it + 2)
    auto step_body = [&](auto stage_tag, int it, AFrags& cur) {
        constexpr int st = decltype(stage_tag)::value;
        const int n2 = it + 2 < steps ? it + 2 : steps - 1;
        const BlockCodes wnxt = load_codes(n2);
        const __amdgpu_buffer_rsrc_t rs_an = a_rsrc(n2);
        uint8_t* sWn = lds + (st ^ 1) * W_STAGE_BYTES;
        ScaledTable tbl;
#pragma unroll
        for (int rg = 0; rg < 7; ++rg) {
            const int s = rg >> 1, half = rg & 1, fc = s & 1;
            if (half == 0 && s < 3) {
#pragma unroll
                for (int j = 0; j < 4; ++j) fb[fc ^ 1][j] = read_b(st, j, s + 1);
            }
#pragma unroll
            for (int t = 0; t < 8; ++t) mfma(2 * half + (t >> 2), t & 3, cur.f[2 * half + (t >> 2)][s], fb[fc][t & 3]);
#pragma unroll
            for (int q = 0; q < 2; ++q) cur.f[2 * half + q][s] = load_frag(rs_an, 2 * half + q, s);
            if (rg == 0) {
                tbl = make_pair_table(lvh, wcur.c1);
            } else if (rg <= 4) {
                decode_chunk(sWn, tbl, wcur, rg - 1);
            }
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
                if (rg <= 4) __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
                else __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
                if (half == 0 && s < 3 && t < 4)
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0); // DS read
                if (t == 2 || t == 5 || (rg == 0 && (t == 0 || t == 1)))
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
                if (rg >= 1 && rg <= 4 && t == 6)
                    __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        wcur = wnxt;
        __syncthreads();
        // the next step's first W' fragments, then the last 8 MFMAs of this step behind them
#pragma unroll
        for (int j = 0; j < 4; ++j) fb[0][j] = read_b(st ^ 1, j, 0);
#pragma unroll
        for (int t = 0; t < 8; ++t) mfma(2 + (t >> 2), t & 3, cur.f[2 + (t >> 2)][3], fb[1][t & 3]);
#pragma unroll
        for (int q = 0; q < 2; ++q) cur.f[2 + q][3] = load_frag(rs_an, 2 + q, 3);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
            if (t < 4) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);     // DS read
            if (t == 2 || t == 5) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- prologue ----
    // The rank-r adapter term goes first, in rank chunks of 64 (piece 0 only, for a split
    // tile), through stage 1 of the W' buffer, which the main loop first writes after the
    // prologue's barrier:
    //   forward : acc += (s T) B^T   (A operand s*T [M x r], stage: rows of B [N x r])
    //   backward: acc += (s U) A     (A operand s*U [M x r], stage: A [r x K], read transposed)
    // Its operands are requested before the main loop's first A fragments (those of step 0;
    // the step-1 fragments follow the term), so that its MFMAs run while those are in flight.  The A operand comes straight from global memory (it is
    // small: M x r); rank values past r are zero on both sides.
    // Then stage 0 <- W' of step 0, with the A fragments of steps 0 and 1 and the codes of
    // step 1 requested.
    AFrags fa0, fa1;
    const BlockCodes b0 = load_codes(0);
    wcur = load_codes(steps > 1 ? 1 : 0);
    const int rr = u.split <= 0 ? a.r : 0;
    const int64_t arows = a.M - m0 < TM ? a.M - m0 : TM;
    for (int rc = 0; rc < rr; rc += 64) {
        if (rc > 0) __syncthreads();        // every wave is done with the previous chunk
        // stage operand, through buffer loads that read zero out of range (no branch, so
        // that nothing waits for them before the other loads are issued)
        uint4 rv[TN * 8 / 256];
        {
            const __amdgpu_buffer_rsrc_t rs =
                BWD ? make_rsrc(a.Lr + (int64_t)rc * a.K, (int64_t)(a.r - rc) * a.K * 2)
                    : make_rsrc(a.Lr + c0 * a.r, (a.N - c0 < TN ? a.N - c0 : TN) * a.r * 2);
#pragma unroll
            for (int i = 0; i < TN * 8 / 256; ++i) {
                const int qi = tid + 256 * i;
                uint32_t off;
                if constexpr (BWD) {
                    const int j = qi / (TN / 8), c = qi % (TN / 8);   // rank row rc + j, 8 features per chunk
                    off = c0 + 8 * c < a.K ? (uint32_t)(((int64_t)j * a.K + 8 * c) * 2) + (uint32_t)(c0 * 2) : 0x80000000u;
                } else {
                    const int row = qi >> 3, c = qi & 7;             // feature c0 + row, rank rc + 8 c
                    off = rc + 8 * c < a.r ? (uint32_t)((row * a.r + rc + 8 * c) * 2) : 0x80000000u;
                }
                rv[i] = buf_load16(rs, off, 0);
            }
        }
        AFrags R;
        {
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.Rk + m0 * a.r + rc, arows * a.r * 2 - rc * 2);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bool live = rc + 16 * s + 8 * h < a.r;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t off = (uint32_t)((128 * wave + 32 * i + rl) * a.r * 2 + 32 * s + 16 * h);
                    R.f[i][s] = buf_load16(rs, live ? off : 0x80000000u, 0);
                }
            }
        }
        if (rc == 0) load_all(fa0, 0);
#pragma unroll
        for (int i = 0; i < TN * 8 / 256; ++i) {
            const int qi = tid + 256 * i;
            if constexpr (BWD) {
                const int j = qi / (TN / 8), c = qi % (TN / 8);
                *reinterpret_cast<uint4*>(lds + W_STAGE_BYTES + wt_off<TN>(j, 8 * c)) = even_odd8(rv[i]);
            } else {
                *reinterpret_cast<uint4*>(lds + W_STAGE_BYTES + tile_off(qi >> 3, qi & 7)) = rv[i];
            }
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8 b[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = read_b(1, j, s);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) mfma(i, j, R.f[i][s], b[j]);
        }
    }
    if (rr <= 0) load_all(fa0, 0);
    load_all(fa1, steps > 1 ? 1 : 0);
    {
        const ScaledTable t0 = make_pair_table(lvh, b0.c1);
#pragma unroll
        for (int c = 0; c < 4; ++c) decode_chunk(lds, t0, b0, c);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[0][j] = read_b(0, j, 0);

    {
        int it = 0;
        for (; it + 1 < steps; it += 2) {
            step_body(std::integral_constant<int, 0>{}, it, fa0);
            step_body(std::integral_constant<int, 1>{}, it + 1, fa1);
        }
        if (it < steps) step_body(std::integral_constant<int, 0>{}, it, fa0);
    }

    // The output column of accumulator column rl: forward, the feature itself; backward, the
    // W' tile holds each 8-feature chunk in even/odd order (decode8<true>; the rank-r operand A
    // is staged the same way), so position p of a chunk is feature 2p (p < 4) or 2p - 7.
    const int rl_col = BWD ? (rl & ~7) | ((rl & 7) < 4 ? 2 * (rl & 7) : 2 * (rl & 7) - 7) : rl;

    // ---- piece of a split tile: fp32 partial tile, row-major TM x TN, summed later ----
    if (u.split >= 0) {
        float* slot = a.spart + (u.tail * a.S + u.split) * (int64_t)TILE_FLOATS;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = j * 32 + rl_col;
#pragma unroll
                for (int reg = 0; reg < 16; ++reg) {
                    const int row = wave * 128 + i * 32 + 8 * (reg >> 2) + 4 * h + (reg & 3);
                    slot[row * TN + col] = acc[i][j][reg];
                }
            }
        return;
    }

    // ---- store bf16 ----
    // One buffer range per group of 8 rows (fragment row tile i, register group g): a group
    // with rows past M gets a shorter range, and a lane whose column is past the last takes
    // an offset beyond every range, so the hardware drops those stores with no branch.  The
    // per-lane offsets hold the row in the group and the column; nothing goes through the
    // wave-uniform offset, which the range check does not see.  Ranges and offsets stay
    // below 2^27 (8 rows of fewer than 2^22 columns).
    const int64_t ncols = BWD ? a.K : a.N;
    const uint32_t rstride = (uint32_t)(ncols * 2);       // bytes per output row
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    uint32_t voff[4][4];                                  // [row of the group][j]
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const bool col_ok = c0 + j * 32 + rl_col < ncols;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            voff[k][j] = col_ok ? (uint32_t)(4 * h + k) * rstride + (uint32_t)(j * 32 + rl_col) * 2 : 0x80000000u;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int64_t grow = wv * 128 + i * 32 + 8 * g;     // first row of the group in the tile
            const int64_t live = arows - grow < 8 ? (arows - grow > 0 ? arows - grow : 0) : 8;
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.out + (m0 + grow) * ncols + c0, live * rstride);
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int k = 0; k < 4; k += 2) {
                    const uint32_t pk = pack_bf16x2(acc[i][j][4 * g + k], acc[i][j][4 * g + k + 1]);
                    buf_store2(rs, voff[k][j], (uint16_t)pk);
                    buf_store2(rs, voff[k + 1][j], (uint16_t)(pk >> 16));
                }
        }
}

// ---------------------------------------------------------------------------
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
    const FusedPlan p = fused_plan(fa.M, ncols, steps);
    fa.S = p.S;
    fa.chunk = p.chunk;
    fa.spart = (float*)split_ws;
    if (p.S > 1 && !split_ws) return hipErrorInvalidValue;
    // the profiling events cover the product and, for split tail tiles, their sum
    return with_events(st, [&] {
        hipLaunchKernelGGL((k_fused<BWD>), dim3((unsigned)p.grid), dim3(256), 0, st, fa, tab);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || p.S == 1) return e;
        hipLaunchKernelGGL(k_split_reduce<TN>, dim3((unsigned)(p.tails * 32)), dim3(256), 0, st, fa.spart, p.S,
                           fa.M, ncols, (fa.M + TM - 1) / TM, (ncols + TN - 1) / TN, fa.out);
        return hipGetLastError();
    });
}

hipError_t launch_fused_fwd(const WeightView& W, const float* c1, const uint16_t* Xpk, int64_t M, const uint16_t* Ts,
                            const uint16_t* Bl, int r, uint16_t* Y, void* split_ws, const Nf4Table& tab,
                            hipStream_t st) {
    if (M == 0 || W.rows == 0) return hipSuccess;
    FusedArgs fa{W.codes, c1, W.rows, W.cols, Xpk, M, Ts, Bl, r, Y, 1, 0, nullptr};
    return launch_fused<false>(fa, W.rows, W.cols >> 6, split_ws, tab, st);
}

hipError_t launch_fused_bwd_dx(const WeightView& W, const float* c1, const uint16_t* dYpk, int64_t M, const uint16_t* Us,
                               const uint16_t* Al, int r, uint16_t* dX, void* split_ws, const Nf4Table& tab,
                               hipStream_t st) {
    if (M == 0 || W.cols == 0) return hipSuccess;
    FusedArgs fa{W.codes, c1, W.rows, W.cols, dYpk, M, Us, Al, r, dX, 1, 0, nullptr};
    return launch_fused<true>(fa, W.cols, (W.rows + 63) >> 6, split_ws, tab, st);
}

}  // namespace nf4
