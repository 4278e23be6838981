// gemv.hip -- few-token forward of the QLoRA NF4 linear layer (gfx950).
//
// "Paged optimizers, and QLoRA end to end" (zerotofrontier.app "sft/peft"): every
// frozen matrix is dequantized block by block and multiplied in 16-bit precision,
// with the bf16 LoRA output added.  Layer formula: "Putting it together"
// (prism.theerrors.in QLoRA explainer).  For a handful of tokens the product is a
// stream over the packed weight, bound by HBM.
#include "bufio.h"
#include "launch.h"

namespace nf4 {

// ---------------------------------------------------------------------------
// Few-token forward (M <= 16): an HBM-bound stream over the packed weight, in two
// launches.
//
// k_gemv_part<RB, MT>: workgroup (contraction slice, row group) = 64 rows (MT = 4) or
// 128 rows (MT = 16) x RB NF4 blocks; wave w owns one or two tiles of 16 consecutive
// rows.  The slice's token inputs X[0:MT, slice]
// (MT = 4 or 16 staged token rows, rows past M reading zero) are staged once into
// LDS, rows padded by 16 bytes for the banks.  Every wave then requests all of its
// codes at once, so the whole slice is in flight and no later request waits behind an
// earlier one (the vector-memory counter retires in order).
//
// Codes move as 16 bytes per lane: lane (n = lane % 16, g = lane / 16) reads bytes
// 16g..16g+15 of the 64-byte block pair (2p, 2p+1) of row n, so one request covers
// 64 contiguous bytes of each of 16 rows (the 8-byte-per-lane form, 32 bytes per row,
// streams at about three quarters of the rate).  Lanes 0-31 then hold block 2p and
// lanes 32-63 block 2p+1; one v_permlane32_swap per register pair trades the second
// half of the first with the first half of the second, after which every lane holds
// 16 codes of each block: codes kA(g)..kA(g)+15, kA = 0, 32, 16, 48 for g = 0..3.
// Two v_mfma_f32_16x16x32_bf16 per block on the unscaled bf16 levels, against the
// inputs of the same contraction indices from LDS, give the block's partial dot
// products, which the block's decoded constant c1' scales into the fp32 accumulator.
// Levels come from a 256-entry LDS table that maps one code byte to its two bf16
// levels, held in 16 copies so that lanes with different bytes mostly read different
// banks; c1' from an E4M3 table, the row's 8-bit constants (one aligned window) and
// at most two second-level steps per row and slice.  Row groups past the weight run
// the adapter rows A (bf16, no scale): partial sums of T = X A^T from the same pass.
// Partial sums go to part[slice][token][row] (rows N.. hold T).
//
// k_gemv_reduce: per 32 weight rows, sums the slices in slice order, forms T
// (the sum of its slices) and s T (bf16), and Y = sum + (s T) B^T (bf16), with every
// load of a thread requested before the first is used.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));


// NF4 blocks per contraction slice (16: more, smaller workgroups measured faster than
// 32 even at 16 tokens, where the slices double the partial-sum traffic)
constexpr int GV_RB = 16;
int64_t gemv_slices(int64_t M, int64_t K) {
    (void)M;
    return ((K >> 6) + GV_RB - 1) / GV_RB;
}
size_t gemv_partial_bytes(int64_t M, int64_t N, int64_t K, int r) {
    return (size_t)gemv_slices(M, K) * (size_t)M * (size_t)(N + r) * 4;
}

struct GvArgs {
    const uint8_t* codes;
    const uint8_t* qc;
    const float* c2;
    const float* mean;
    int64_t N, K;
    const uint16_t* X;
    int M;
    const uint16_t* Al;      // adapter A [r x K]
    const uint16_t* Bl;      // adapter B [N x r]
    int r;
    float s;
    float* part;             // [slices][M][N + r]
    uint16_t* Y;             // [M x N]
    uint16_t* T;             // [M x r]
    const float* absmax;     // plain first-level constants (no double quantization), or null
};

// Four code bytes (8 codes) -> the MFMA operand of their 8 unscaled bf16 levels.  The
// table holds CP copies of each entry, copy c of entry b at dword CP b + c; lane l reads
// copy l % CP (s_lane = table + l % CP), so that the lanes of one LDS cycle mostly read
// distinct banks whatever their code bytes (all of them for CP = 32).
template <int CP>
__device__ __forceinline__ bf16x8v lookup8(const uint32_t* s_lane, uint32_t w) {
    return __builtin_bit_cast(bf16x8v, make_uint4(s_lane[(w & 0xFFu) * CP], s_lane[((w >> 8) & 0xFFu) * CP],
                                                  s_lane[((w >> 16) & 0xFFu) * CP], s_lane[(w >> 24) * CP]));
}

constexpr int GV_WV = 4;                   // waves per workgroup of k_gemv_part
constexpr int GV_AROWS = 16;               // adapter rows per workgroup
// 16-row tiles per wave: with 16 staged tokens two tiles share each input operand read
// from LDS (the reads cost as much LDS time as the level lookups); with 4, one tile
// keeps more, smaller workgroups in flight
constexpr int gv_tiles(int MT) { return MT == 16 ? 2 : 1; }
constexpr int gv_rows(int MT) { return 16 * gv_tiles(MT) * GV_WV; }   // weight rows per workgroup
// copies of the level table (16 KB): lane l reads copy l % 16.  32 copies make the lookups
// conflict-free but cost a workgroup slot per CU, which measured slower.
constexpr int GV_CP = 16;

// Dynamic LDS of k_gemv_part: the staged inputs (the level and E4M3 tables are static, at
// fixed addresses; adapter workgroups keep their cross-wave sums in the level table's
// space, which they do not use).
constexpr int gv_lds_bytes(int MT) { return MT * (GV_RB * 128 + 16); }

// One workgroup of k_gemv_part: gv_rows(MT) weight rows (ADAPTER false), or GV_AROWS adapter
// rows A (bf16, no scale) whose slice is split among the waves (wave w: blocks
// w RB/WV ..) and summed across the waves in LDS, so that an adapter workgroup moves
// about as many bytes as a weight workgroup.  Straight-line code from the first
// request to the last wait, so that every wait names exactly the requests it needs.
template <int RB, int MT, bool ADAPTER, bool PLAIN>
__device__ __forceinline__ void gemv_part_body(const GvArgs& a, const Nf4Table& tab, int64_t slice,
                                               int64_t group, uint32_t* s_pair, float* s_e4m3) {
    constexpr int CP = GV_CP;
    extern __shared__ __attribute__((aligned(16))) uint8_t gv_lds[];
    constexpr int NT = 64 * GV_WV;                     // threads
    constexpr int XSTRIDE = RB * 128 + 16;             // bytes per staged token row
    constexpr int RBW = RB / GV_WV;                    // adapter blocks per wave
    constexpr int TT = ADAPTER ? 1 : gv_tiles(MT);     // row tiles of this wave
    static_assert(GV_WV * 64 * 16 <= 256 * CP * 4, "adapter sums fit in the table space");
    uint8_t* s_x = gv_lds;                                         // [MT][XSTRIDE] token inputs
    f32x4* s_red = reinterpret_cast<f32x4*>(s_pair);               // [WV][64] adapter partials

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t KB = a.K >> 6;
    const int64_t b0 = slice * RB;                      // first block of the slice
    const int nb = KB - b0 < RB ? (int)(KB - b0) : RB;  // blocks of the slice inside the row
    const int nl = lane & 15, g = lane >> 4;
    // row of this lane in tile t: n0 + 16 t
    const int64_t n0 = ADAPTER ? group * GV_AROWS + nl : group * gv_rows(MT) + 16 * TT * wave + nl;

    // ---- requests: token inputs of the slice first, then this wave's rows ----
    const __amdgpu_buffer_rsrc_t rs_x = make_rsrc(a.X + b0 * 64, (int64_t)a.M * a.K * 2 - b0 * 128);
    constexpr int XCH = MT * RB * 8 / NT;               // chunks per thread
    uint4 xs[XCH];
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
        const int q = tid + NT * i, m = q / (RB * 8), c = q % (RB * 8);
        const uint32_t vo = (m < a.M && c < nb * 8) ? (uint32_t)((int64_t)m * a.K * 2 + c * 16) : 0x80000000u;
        xs[i] = buf_load16(rs_x, vo, 0);
    }
    uint4 cw[TT][RB / 2];
    uint32_t qw[TT][RB / 4 + 1];
    uint4 al[RBW][2];
    float mean = 0.0f, c2f[TT], c2l[TT];
    float cpl[PLAIN ? TT : 1][PLAIN ? RB : 1];           // plain constants of the slice
    if constexpr (!ADAPTER && PLAIN) {
        // the row's RB constants of the slice; past the row: the next row's (finite, given
        // a zero factor below); past the last row: zero
        const __amdgpu_buffer_rsrc_t rs_a = make_rsrc(a.absmax, a.N * KB * 4);
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            const uint32_t ca = (uint32_t)(((n0 + 16 * t) * KB + b0) * 4);
#pragma unroll
            for (int j = 0; j < RB; ++j) cpl[t][j] = buf_loadf(rs_a, ca + 4 * j, 0);
        }
    }
    if constexpr (!ADAPTER && !PLAIN) {
        mean = *a.mean;
        // second-level constants: a row's slice meets at most two 256-blocks
        const int64_t n2 = (a.N * KB + 255) >> 8;
        const __amdgpu_buffer_rsrc_t rs_q = make_rsrc(a.qc, a.N * KB);
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            const int64_t ci0 = (n0 + 16 * t) * KB + b0;
            const int64_t gf = ci0 >> 8, gl = (ci0 + nb - 1) >> 8;
            c2f[t] = a.c2[gf < n2 ? gf : n2 - 1];
            c2l[t] = a.c2[gl < n2 ? gl : n2 - 1];
            // 8-bit constants of the slice (aligned window); past the last row: zero
            const uint32_t qa = (uint32_t)ci0 & ~3u;
#pragma unroll
            for (int i = 0; i < RB / 4 + 1; ++i) qw[t][i] = buf_load4(rs_q, qa + 4 * i, 0);
        }
    }
    if constexpr (!ADAPTER) {
        // the codes, block pair by block pair (the order they are used in).  A pair past
        // the row reads the next row (finite codes, given a zero constant below) or, past
        // the last row, zero.
        const __amdgpu_buffer_rsrc_t rs_codes = make_rsrc(a.codes, a.N * (a.K >> 1));
        const uint32_t c_voff = (uint32_t)(n0 * (a.K >> 1) + b0 * 32 + 16 * g);
        const uint32_t t_step = (uint32_t)(16 * (a.K >> 1));
#pragma unroll
        for (int p = 0; p < RB / 2; ++p)
#pragma unroll
            for (int t = 0; t < TT; ++t) cw[t][p] = buf_load16(rs_codes, c_voff + t * t_step + 64 * p, 0);
    } else {
        // this wave's blocks of the adapter rows; lane (n, g) takes contraction indices
        // 16g..16g+15 of each block (block index clamped into the row: the wave-uniform
        // offset is not range-checked; blocks past the row are skipped below)
        const __amdgpu_buffer_rsrc_t rs_al = make_rsrc(a.Al, (int64_t)a.r * a.K * 2);
        const uint32_t a_voff = n0 < a.r ? (uint32_t)(n0 * a.K * 2 + 32 * g) : 0x80000000u;
#pragma unroll
        for (int u = 0; u < RBW; ++u) {
            const int64_t j = b0 + wave * RBW + u;
            const uint32_t so = (uint32_t)((j < KB ? j : KB - 1) * 128);
            al[u][0] = buf_load16(rs_al, a_voff, so);
            al[u][1] = buf_load16(rs_al, a_voff + 16, so);
        }
    }

    // ---- tables and staged inputs ----
    {
        float lo = 0.0f, hi = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            lo = (tid & 15) == j ? tab.lv[j] : lo;
            hi = (tid >> 4) == j ? tab.lv[j] : hi;
        }
        if constexpr (!ADAPTER) {
            // entry tid, all CP copies; the rotation spreads one instruction's lanes over the banks
            const uint32_t pv = pack_bf16x2(lo, hi);
            const uint4 p4 = make_uint4(pv, pv, pv, pv);
#pragma unroll
            for (int i = 0; i < CP / 4; ++i)
                *reinterpret_cast<uint4*>(s_pair + tid * CP + 4 * ((tid + i) & (CP / 4 - 1))) = p4;
        }
        s_e4m3[tid] = e4m3_to_f32((uint32_t)tid);
    }
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
        const int q = tid + NT * i, m = q / (RB * 8), c = q % (RB * 8);
        *reinterpret_cast<uint4*>(s_x + m * XSTRIDE + c * 16) = xs[i];
    }
    __syncthreads();

    // MFMA A operand rows: token m = lane % 16 (rows past MT repeat rows below MT; their
    // outputs are never stored)
    const uint8_t* xtok = s_x + (lane & (MT - 1)) * XSTRIDE;
    const uint32_t* s_lane = s_pair + (lane & (CP - 1));
    f32x4 acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (!ADAPTER) {
        float st_first[TT], st_last[TT];
        int jsplit[TT];
        uint32_t q4[TT][RB / 4];
#pragma unroll
        for (int t = 0; t < TT && !PLAIN; ++t) {
            st_first[t] = c2_step(c2f[t]);
            st_last[t] = c2_step(c2l[t]);
            const int64_t ci0 = (n0 + 16 * t) * KB + b0;  // constant index of the slice's first block
            // blocks j >= jsplit of this row's slice belong to the next second-level block
            jsplit[t] = 256 - (int)(ci0 & 255);
            // the slice's 8-bit constants, realigned: byte j of q4[] is block j's
            const uint32_t sh = ((uint32_t)ci0 & 3u) * 8;
#pragma unroll
            for (int i = 0; i < RB / 4; ++i) q4[t][i] = (uint32_t)__builtin_amdgcn_alignbit(qw[t][i + 1], qw[t][i], sh);
        }
        const int kA = 32 * (g & 1) + 16 * (g >> 1);     // first contraction index of the lane
        // valid: blocks past the row contribute zero (a factor, not a branch: the decoded
        // constant of any byte is finite)
        auto c1_of = [&](int t, int j, bool all_valid) {
            float c;
            if constexpr (PLAIN) {
                c = cpl[t][j];
            } else {
                const uint32_t qbyte = (q4[t][j / 4] >> (8 * (j & 3))) & 0xFFu;
                c = __fmaf_rn(s_e4m3[qbyte], j < jsplit[t] ? st_first[t] : st_last[t], mean);
            }
            return all_valid ? c : c * (float)(j < nb);
        };
        auto run = [&](bool all_valid) {
#pragma unroll
            for (int p = 0; p < RB / 2; ++p) {
                const uint8_t* xa = xtok + (2 * p) * 128 + kA * 2;
                const uint8_t* xb = xa + 128;
                const bf16x8v xa0 = *reinterpret_cast<const bf16x8v*>(xa);
                const bf16x8v xa1 = *reinterpret_cast<const bf16x8v*>(xa + 16);
                const bf16x8v xb0 = *reinterpret_cast<const bf16x8v*>(xb);
                const bf16x8v xb1 = *reinterpret_cast<const bf16x8v*>(xb + 16);
#pragma unroll
                for (int t = 0; t < TT; ++t) {
                    // lanes 0-31: bytes of block 2p, lanes 32-63: block 2p+1 -> both blocks per lane
                    uint32_t x = cw[t][p].x, y = cw[t][p].y, z = cw[t][p].z, w = cw[t][p].w;
                    const auto xz = __builtin_amdgcn_permlane32_swap(x, z, false, false);
                    const auto yw = __builtin_amdgcn_permlane32_swap(y, w, false, false);
                    x = xz[0]; z = xz[1]; y = yw[0]; w = yw[1];
                    f32x4 pa = {0.0f, 0.0f, 0.0f, 0.0f}, pb = {0.0f, 0.0f, 0.0f, 0.0f};
                    pa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa0, lookup8<CP>(s_lane, x), pa, 0, 0, 0);
                    pa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa1, lookup8<CP>(s_lane, y), pa, 0, 0, 0);
                    pb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb0, lookup8<CP>(s_lane, z), pb, 0, 0, 0);
                    pb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb1, lookup8<CP>(s_lane, w), pb, 0, 0, 0);
                    const float ca = c1_of(t, 2 * p, all_valid), cb = c1_of(t, 2 * p + 1, all_valid);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[t][i] = __fmaf_rn(cb, pb[i], __fmaf_rn(ca, pa[i], acc[t][i]));
                }
            }
        };
        // a whole slice (all but a row's last), or the last, with blocks past the row
        if (nb == RB) run(true);
        else run(false);
    } else {
        const uint8_t* xrow = xtok + 32 * g;
#pragma unroll
        for (int u = 0; u < RBW; ++u) {
            const int j = wave * RBW + u;
            if (j < nb) {
                const bf16x8v x0 = *reinterpret_cast<const bf16x8v*>(xrow + j * 128);
                const bf16x8v x1 = *reinterpret_cast<const bf16x8v*>(xrow + j * 128 + 16);
                acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x0, __builtin_bit_cast(bf16x8v, al[u][0]), acc[0], 0, 0, 0);
                acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x1, __builtin_bit_cast(bf16x8v, al[u][1]), acc[0], 0, 0, 0);
            }
        }
        // sum over the waves, in wave order
        s_red[wave * 64 + lane] = acc[0];
        __syncthreads();
        if (wave != 0) return;
        acc[0] = s_red[lane];
#pragma unroll
        for (int w = 1; w < GV_WV; ++w) {
            const f32x4 v = s_red[w * 64 + lane];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[0][i] += v[i];
        }
    }
    // lane holds tokens 4g..4g+3 of row n
    const int64_t nrows = ADAPTER ? a.r : a.N;
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        const int64_t n = n0 + 16 * t;
        if (n < nrows) {
            const int64_t col = ADAPTER ? a.N + n : n;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * g + i < a.M) a.part[(slice * a.M + 4 * g + i) * (a.N + a.r) + col] = acc[t][i];
        }
    }
}

// grid: one dimension, workgroup b = (row group) x slices + slice; the slices of one row
// group are dispatched together, so the workgroups in flight read whole rows of codes
// (long runs within one DRAM page); the adapter row groups come first.  (One dimension
// holds the 2^22 / 64 row groups of the longest weight, which the second grid dimension
// of a launch could not.)
template <int RB, int MT, bool PLAIN>
__global__ __launch_bounds__(64 * GV_WV) __attribute__((amdgpu_waves_per_eu(3, 8)))
void k_gemv_part(GvArgs a, Nf4Table tab) {
    __shared__ __attribute__((aligned(16))) uint32_t s_pair[256 * GV_CP];   // code byte -> two bf16 levels
    __shared__ float s_e4m3[256];                      // 8-bit constant -> E4M3 value
    const int64_t nag = (a.r + GV_AROWS - 1) / GV_AROWS;
    const int64_t nsl = ((a.K >> 6) + RB - 1) / RB;      // slices of a row (gemv_slices)
    const int64_t b = blockIdx.x, slice = b % nsl, group = b / nsl;
    if (group < nag) gemv_part_body<RB, MT, true, PLAIN>(a, tab, slice, group, s_pair, s_e4m3);
    else gemv_part_body<RB, MT, false, PLAIN>(a, tab, slice, group - nag, s_pair, s_e4m3);
}

// k_gemv_reduce<ROWS, NO, NT>: workgroup of ROWS weight rows; thread (row n = n0 + tid %
// ROWS, token group tg = tid / ROWS) owns outputs (tg + (256/ROWS) i, n), i < NO, and T
// entries tid + 256 t, t < NT (all M x r of them, in every workgroup: they are few and
// L2-resident).  Slices are added in slice order, 8 at a time with every load of the
// eight requested before the first add.
template <int ROWS, int NO, int NT>
__global__ __launch_bounds__(256) void k_gemv_reduce(GvArgs a, int64_t slices) {
    constexpr int TG = 256 / ROWS;
    constexpr int NE = NO + NT;
    // s T (rounded to bf16), tokens x rank; the lanes of a wave share a token, so each read
    // is a broadcast, four ranks at a time
    __shared__ __attribute__((aligned(16))) float s_ts[16][128];
    const int tid = threadIdx.x;
    const int64_t ld = a.N + a.r;
    const int64_t sstride = (int64_t)a.M * ld;        // one slice of partial sums
    const int64_t n = (int64_t)blockIdx.x * ROWS + tid % ROWS;
    const int tg = tid / ROWS;
    // this thread's row of B, requested first
    uint4 bv[16];
    const bool row_ok = n < a.N;
#pragma unroll
    for (int q8 = 0; q8 < 16; ++q8)
        bv[q8] = (row_ok && q8 < a.r / 8) ? reinterpret_cast<const uint4*>(a.Bl + n * a.r)[q8] : make_uint4(0, 0, 0, 0);
    // partial-sum byte offsets of the outputs and T entries in slice 0 (all slices span
    // slices x M x (N + r) x 4 < 2^28 bytes); an entry that does not exist, or a slice past
    // the last, requests an offset past the range, which reads zero and touches no memory
    constexpr uint32_t OOR = 0x80000000u;
    const __amdgpu_buffer_rsrc_t rs_part = make_rsrc(a.part, slices * sstride * 4);
    uint32_t off[NE];
#pragma unroll
    for (int i = 0; i < NO; ++i) {
        const int m = tg + TG * i;
        off[i] = (row_ok && m < a.M) ? (uint32_t)(((int64_t)m * ld + n) * 4) : OOR;
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int e = tid + 256 * t;
        off[NO + t] = e < a.M * a.r ? (uint32_t)(((int64_t)(e / a.r) * ld + a.N + e % a.r) * 4) : OOR;
    }
    float sum[NE];
#pragma unroll
    for (int i = 0; i < NE; ++i) sum[i] = 0.0f;
    for (int64_t s0 = 0; s0 < slices; s0 += 8) {
        float v[8][NE];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const bool su = s0 + u < slices;
            const uint32_t so = (uint32_t)((s0 + u) * sstride * 4);
#pragma unroll
            for (int i = 0; i < NE; ++i) v[u][i] = buf_loadf(rs_part, su && off[i] != OOR ? off[i] + so : OOR, 0);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int i = 0; i < NE; ++i) sum[i] += v[u][i];
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if (off[NO + t] != OOR) {
            const int e = tid + 256 * t, m = e / a.r, q = e % a.r;
            s_ts[m][q] = bf16_to_f32(f32_to_bf16(a.s * sum[NO + t]));
            if (blockIdx.x == 0) a.T[(int64_t)m * a.r + q] = f32_to_bf16(sum[NO + t]);
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NO; ++i) {
        if (off[i] == OOR) continue;
        const int m = tg + TG * i;
        float l = 0.0f;
#pragma unroll
        for (int q8 = 0; q8 < 16; ++q8) {
            if (q8 < a.r / 8) {
                const uint32_t bw[4] = {bv[q8].x, bv[q8].y, bv[q8].z, bv[q8].w};
                const float4 t0 = *reinterpret_cast<const float4*>(&s_ts[m][8 * q8]);
                const float4 t1 = *reinterpret_cast<const float4*>(&s_ts[m][8 * q8 + 4]);
                const float tv[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    l = __fmaf_rn(tv[2 * e], bf16_lo(bw[e]), l);
                    l = __fmaf_rn(tv[2 * e + 1], bf16_hi(bw[e]), l);
                }
            }
        }
        a.Y[(int64_t)m * a.N + n] = f32_to_bf16(sum[i] + l);
    }
}

template <int MT, bool PLAIN>
static hipError_t launch_gemv_part(dim3 grid, const GvArgs& ga, const Nf4Table& tab, hipStream_t st) {
    const int lds = gv_lds_bytes(MT);
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)k_gemv_part<GV_RB, MT, PLAIN>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL((k_gemv_part<GV_RB, MT, PLAIN>), grid, dim3(64 * GV_WV), lds, st, ga, tab);
    return hipGetLastError();
}

hipError_t launch_fused_gemv(const WeightView& W, const uint16_t* X, int64_t M, const uint16_t* Al,
                             const uint16_t* Bl, int r, float s, uint16_t* Y, uint16_t* T, float* part,
                             const Nf4Table& tab, hipStream_t st) {
    if (M == 0) return hipSuccess;
    const int64_t slices = gemv_slices(M, W.cols);
    GvArgs ga{W.codes, W.q, W.c2, W.mean, W.rows, W.cols, X, (int)M, Al, Bl, r, s, part, Y, T, W.absmax};
    const bool small = M <= 4;
    const int64_t wrows = small ? gv_rows(4) : gv_rows(16);
    dim3 g1((unsigned)(slices * ((r + GV_AROWS - 1) / GV_AROWS + (W.rows + wrows - 1) / wrows)));
    // reduce: 32 rows x 8 token groups, one output per thread for up to 4 tokens, two
    // above (64-row workgroups with four outputs each left half the chip idle on the
    // 8192-row weights and measured 1% slower at 16 tokens)
    const int64_t rrows = 32;
    dim3 g2((unsigned)((W.rows + rrows - 1) / rrows > 0 ? (W.rows + rrows - 1) / rrows : 1));
    return with_events(st, [&] {
        if (g1.x > 0) {
            const bool plain = W.absmax != nullptr;
            hipError_t e = small ? (plain ? launch_gemv_part<4, true>(g1, ga, tab, st)
                                          : launch_gemv_part<4, false>(g1, ga, tab, st))
                                 : (plain ? launch_gemv_part<16, true>(g1, ga, tab, st)
                                          : launch_gemv_part<16, false>(g1, ga, tab, st));
            if (e != hipSuccess) return e;
        }
        // T entries per thread: just enough for the M x r of them (every reduce workgroup
        // forms all of T, so unused slots would only add requests)
        const int64_t mr = M * r;
        if (small && mr <= 256) hipLaunchKernelGGL((k_gemv_reduce<32, 1, 1>), g2, dim3(256), 0, st, ga, slices);
        else if (small) hipLaunchKernelGGL((k_gemv_reduce<32, 1, 2>), g2, dim3(256), 0, st, ga, slices);
        else if (mr <= 1024) hipLaunchKernelGGL((k_gemv_reduce<32, 2, 4>), g2, dim3(256), 0, st, ga, slices);
        else hipLaunchKernelGGL((k_gemv_reduce<32, 2, 8>), g2, dim3(256), 0, st, ga, slices);
        return hipGetLastError();
    });
}

}  // namespace nf4
