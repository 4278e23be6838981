// lora.hip -- the rank-r adapter products of the QLoRA layer.
//
// "Paged optimizers, and QLoRA end to end" (zerotofrontier.app "sft/peft"):
// a bf16 LoRA adapter on every linear, r = 64, alpha = 16, gradients only into
// the adapters.  With s = alpha / r the layer needs
//   T = X A^T (forward, saved), U = dY B, dA = s U^T X, dB = s dY^T T.
// They are skinny products (one side is r <= 128), a few percent of the
// layer's flops, but they stream the big activations once more, so they must
// run at bandwidth.  One LDS-staged MFMA kernel covers T and U: each operand
// is either contraction-contiguous in memory (16-byte chunks straight into
// LDS) or contraction-strided (8 x 8 blocks transposed in registers with byte
// permutes).  dA and dB, whose operands are both contraction-strided, have a
// kernel of their own that stages rows as they lie and reads the MFMA operands
// out of LDS transposed (k_skinny_tt).  The contraction is split across
// workgroups so that the grid fills the chip; a second pass sums the fp32
// slices in a fixed order, so the result is deterministic.
#include "bufio.h"
#include "launch.h"

namespace nf4 {

constexpr int SK_BM = 128;   // rows of C per workgroup (4 waves x 32)
constexpr int SK_BN = 64;    // columns of C per workgroup (2 MFMA tiles of 32)
constexpr int SK_PC = 64;    // contraction chunk per pipeline step
constexpr int SK_A_BYTES = SK_BM * 128;
constexpr int SK_B_BYTES = SK_BN * 128;
constexpr int SK_STAGE = SK_A_BYTES + SK_B_BYTES;

// LDS tile [rows][64 bf16], 16-byte chunk c of row i stored at c ^ (i & 7).
__device__ __forceinline__ int lds_off(int row, int chunk) {
    return row * 128 + ((chunk ^ (row & 7)) << 4);
}

// 8 x 8 transpose of 16-bit values: in[i] holds row i (8 values), out[j] column j.
__device__ __forceinline__ void transpose8x8(const uint4 in[8], uint4 out[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 lo = in[2 * q], hi = in[2 * q + 1];
            const uint32_t a = (j >> 1) == 0 ? lo.x : (j >> 1) == 1 ? lo.y : (j >> 1) == 2 ? lo.z : lo.w;
            const uint32_t b = (j >> 1) == 0 ? hi.x : (j >> 1) == 1 ? hi.y : (j >> 1) == 2 ? hi.z : hi.w;
            w[q] = __builtin_amdgcn_perm(b, a, sel);
        }
        out[j] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// Operand staging.  Each LDS stage holds the A tile [128 rows][64 contraction] and the
// B tile [64 cols][64 contraction] of one contraction chunk:
//   direct operand    : element (i, p) at src[i * ld + p]  (16-byte pieces along p)
//   transposed operand: element (i, p) at src[p * ld + i]  (8 x 8 blocks, one contraction
//                       row per piece, transposed in registers with byte permutes)
// A thread stages up to 8 pieces of one chunk, all of one operand except in the
// all-direct case; which pieces is fixed per wave:
//   A T, B T : waves 0-1 one A block each, wave 2 one B block each, wave 3 none
//   A D, B T : waves 0-2 A pieces tid + 192 t (t < 6), wave 3 one B block each
//   A T, B D : waves 0-1 one A block each, waves 2-3 B pieces (tid - 128) + 128 t (t < 4)
//   A D, B D : every thread A pieces tid + 256 t (t < 4) and B pieces tid + 256 (t - 4)
// A piece's byte offset is the same for every chunk: the chunk moves the descriptor
// instead (direct: src + r0 * ld + p0, transposed: src + p0 * ld + r0, with r0 the tile's
// first row and p0 the chunk's first contraction index).  Pieces the thread does not own,
// or whose rows lie past the operand, get an offset past any descriptor range and read
// zero; so do pieces past the contraction end P, tested per chunk (direct pieces never
// straddle P, which is a multiple of 8 for them).  The loads are straight-line code.
constexpr uint32_t SK_OOB = 0x80000000u;

template <bool ATR, bool BTR>
struct SkStage {
    static constexpr int NR = (!ATR && !BTR) ? 6 : 8;
    uint4 r[NR];
};

// Partial C[i][j] = sum over this workgroup's contraction slice of Aop[i][p] * Bop[p][j],
// written as fp32 to part[z][i][j].  Grid: (col tiles, row tiles, slices).
//
// Three register sets of staged chunks: chunk c+3 is requested during step c and
// written to LDS at the start of step c+2, so every request has two steps to arrive.
template <bool ATR, bool BTR>
__global__ __launch_bounds__(256) void k_skinny(const uint16_t* __restrict__ A,
                                                const uint16_t* __restrict__ B, int64_t Mc,
                                                int64_t Nc, int64_t P, int64_t chunks_per_slice,
                                                float* __restrict__ part, uint16_t* __restrict__ pack,
                                                bool pack_even_odd) {
    using St = SkStage<ATR, BTR>;
    constexpr int NR = St::NR;
    constexpr bool DD = !ATR && !BTR;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * SK_STAGE];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t i0 = (int64_t)blockIdx.y * SK_BM, j0 = (int64_t)blockIdx.x * SK_BN;
    const int64_t nchunks = (P + SK_PC - 1) / SK_PC;
    const int64_t c0 = (int64_t)blockIdx.z * chunks_per_slice;
    const int64_t c1 = (c0 + chunks_per_slice < nchunks) ? c0 + chunks_per_slice : nchunks;
    const int64_t lda = ATR ? Mc : P;
    const int64_t ldb = BTR ? Nc : P;

    // this wave's operand and layout (wave-uniform); B in the all-direct case is pieces 4-5
    const bool a_wave = DD || (ATR ? wave < 2 : (BTR ? wave < 3 : true));
    const bool b_wave = !DD && (ATR ? (wave >= 2 && (!BTR || wave == 2)) : wave == 3);
    const bool w_trans = a_wave ? ATR : BTR;
    // piece t: tile row (direct) or 8-row group start (transposed), contraction index in chunk
    auto piece_row = [&](int t) -> int {
        if constexpr (DD) return (tid >> 3) + 32 * (t & 3);
        if (w_trans) return (((a_wave ? tid : tid - (ATR ? 128 : 192)) >> 3) & 15) * 8;
        return a_wave ? (tid + 192 * t) >> 3 : ((tid - 128) + 128 * t) >> 3;
    };
    auto piece_pc = [&](int t) -> int { return 8 * (tid & 7) + ((!DD && w_trans) ? t : 0); };
    auto piece_own = [&](int t) -> bool {
        if constexpr (DD) return t < 4 || (tid >> 3) + 32 * (t - 4) < SK_BN;
        if (!a_wave && !b_wave) return false;
        if (w_trans) return true;
        return a_wave ? (t < 6 && tid + 192 * t < SK_BM * 8) : t < 4;
    };
    uint32_t off[NR];
#pragma unroll
    for (int t = 0; t < NR; ++t) {
        const bool ob = DD ? t >= 4 : !a_wave;
        const int64_t rows = ob ? Nc : Mc, r0 = ob ? j0 : i0, ld = ob ? ldb : lda;
        const int row = piece_row(t), pc = piece_pc(t);
        const bool tr = DD ? false : w_trans;
        const bool ok = piece_own(t) && r0 + row < rows;
        off[t] = ok ? (uint32_t)(tr ? ((int64_t)pc * ld + row) * 2 : ((int64_t)row * ld + pc) * 2) : SK_OOB;
    }
    auto rsrc_at = [&](const uint16_t* src, bool tr, int64_t ld, int64_t rows, int64_t r0, int64_t nmax,
                       int64_t p0) {
        if (tr) return make_rsrc(src + p0 * ld + r0, (P - p0) * ld * 2 - r0 * 2);
        const int64_t nr = rows - r0 < nmax ? rows - r0 : nmax;
        return make_rsrc(src + r0 * ld + p0, (nr * ld - p0) * 2);
    };
    auto load = [&](St& S, int64_t c) {
        const int64_t cc = c < c1 ? c : c1 - 1;            // past the slice: a repeat, never used
        const int64_t p0 = cc * SK_PC;
        const int rem = (int)(P - p0 < SK_PC ? P - p0 : SK_PC);
        const __amdgpu_buffer_rsrc_t ra = rsrc_at(A, ATR, lda, Mc, i0, SK_BM, p0);
        const __amdgpu_buffer_rsrc_t rb = rsrc_at(B, BTR, ldb, Nc, j0, SK_BN, p0);
#pragma unroll
        for (int t = 0; t < NR; ++t) {
            const bool ob = DD ? t >= 4 : !a_wave;
            const uint32_t o = piece_pc(t) < rem ? off[t] : SK_OOB;
            S.r[t] = buf_load16(ob ? rb : ra, o, 0);
        }
    };
    auto store = [&](const St& S, int stage) {
        uint8_t* sA = lds + stage * SK_STAGE;
        uint8_t* sB = sA + SK_A_BYTES;
        if constexpr (DD) {
#pragma unroll
            for (int t = 0; t < NR; ++t) {
                if (piece_own(t))
                    *reinterpret_cast<uint4*>((t < 4 ? sA : sB) + lds_off(piece_row(t), tid & 7)) = S.r[t];
            }
        } else {
            if (!a_wave && !b_wave) return;
            uint8_t* dst = a_wave ? sA : sB;
            if (w_trans) {
                const int rb = piece_row(0);
                uint4 tr[8];
                transpose8x8(S.r, tr);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    *reinterpret_cast<uint4*>(dst + lds_off(rb + j, tid & 7)) = tr[j];
            } else {
#pragma unroll
                for (int t = 0; t < 6; ++t)
                    if (piece_own(t))
                        *reinterpret_cast<uint4*>(dst + lds_off(piece_row(t), tid & 7)) = S.r[t];
            }
        }
    };
    f32x16 acc0 = {}, acc1 = {};
    auto compute = [&](int stage) {
        const uint8_t* sA = lds + stage * SK_STAGE;
        const uint8_t* sB = sA + SK_A_BYTES;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int ch = 2 * s + (lane >> 5);
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(sA + lds_off(wave * 32 + (lane & 31), ch));
            const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(sB + lds_off(lane & 31, ch));
            const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(sB + lds_off(32 + (lane & 31), ch));
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, acc1, 0, 0, 0);
        }
    };
    // The A tile of a chunk, staged in LDS, in the fused product's fragment order (tile_map.h):
    // sub-block (token tile i0 / 512, contraction step c, row quarter (i0 / 128) % 4), whose
    // 1024 16-byte pieces this workgroup writes contiguously, each piece's 8 values in the
    // even/odd order of the forward product's decoded weights when pack_even_odd is set.
    // Only the first column tile writes it; rows past Mc and contraction values past P are
    // the zeros staged for them.
    uint16_t* const pk = (ATR || blockIdx.x != 0) ? nullptr : pack;
    auto write_pack = [&](int stage, int64_t c) {
        const uint8_t* sA = lds + stage * SK_STAGE;
        uint8_t* dst = reinterpret_cast<uint8_t*>(pk) + ((i0 >> 9) * nchunks + c) * (int64_t)A_BLOCK_BYTES +
                       ((i0 >> 7) & 3) * (A_BLOCK_BYTES / 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + 256 * i;
            const uint4 v = *reinterpret_cast<const uint4*>(sA + lds_off(a_pack_row(q), a_pack_col(q)));
            *reinterpret_cast<uint4*>(dst + 16 * q) = pack_even_odd ? even_odd8(v) : v;
        }
    };
    St s0, s1, s2;
    // step k (chunk c0 + k) with register sets cur (chunk k's, already in LDS) and nx (chunk
    // k+1's): write nx to the free stage, request chunk k+3 into cur, multiply stage k & 1
    auto step = [&](int64_t k, St& cur, const St& nx) {
        store(nx, (int)((k + 1) & 1));
        load(cur, c0 + k + 3);
        compute((int)(k & 1));
        if (pk) write_pack((int)(k & 1), c0 + k);
        __syncthreads();
    };

    const int64_t n = c1 - c0;
    if (n > 0) {
        load(s0, c0);
        store(s0, 0);
        load(s1, c0 + 1);
        load(s2, c0 + 2);
        __syncthreads();
        int64_t k = 0;
        for (; k + 3 <= n; k += 3) {
            step(k, s0, s1);
            step(k + 1, s1, s2);
            step(k + 2, s2, s0);
        }
        if (k < n) step(k, s0, s1);
        if (k + 1 < n) step(k + 1, s1, s2);
    }
    float* out = part + (int64_t)blockIdx.z * Mc * Nc;
#pragma unroll
    for (int reg = 0; reg < 16; ++reg) {
        const int64_t row = i0 + wave * 32 + 8 * (reg >> 2) + 4 * (lane >> 5) + (reg & 3);
        const int64_t col0 = j0 + (lane & 31), col1 = col0 + 32;
        if (row < Mc) {
            if (col0 < Nc) out[row * Nc + col0] = acc0[reg];
            if (col1 < Nc) out[row * Nc + col1] = acc1[reg];
        }
    }
}


// ---------------------------------------------------------------------------
// Both operands contraction-strided (dA = U^T X, dB = dY^T T: the contraction runs over
// the token rows): the chunk's rows of each source go into LDS as they lie in memory,
// [64 contraction rows][128 or 64 columns] in 16-byte pieces (every lane a piece, every
// load of a wave one run of whole rows), and the MFMA operands are read out transposed
// with ds_read_b64_tr_b16.  A 32-byte segment u of row p sits at u ^ (swizzle of p), so
// that the 4 rows x 64 bytes that 32 lanes read in one pass meet 64 distinct banks.
// Against the register transposes of k_skinny, whose staging used 3 of the 4 waves:
// 26.6 against 30.4 us per launch on average over the LLaMA-65B layer's dA and dB.
template <int COLS>
__device__ __forceinline__ int tt_off(int row, int col) {
    // COLS = 128: 256-byte rows, u ^ 2 (row & 3); COLS = 64: 128-byte rows (two per bank
    // row), u ^ 2 ((row >> 1) & 1)
    const int sw = COLS == 128 ? ((row & 3) << 1) : (((row >> 1) & 1) << 1);
    return row * (2 * COLS) + (((col >> 4) ^ sw) << 5) + ((col & 15) << 1);
}

typedef short tt_i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) tt_i16x4 tt_lds_i16x4;
// Within each group of 16 lanes, lane i receives column i of the 4 x 16 block whose rows
// the lanes 4e + (i >> 2) address (e = 0..3).
__device__ __forceinline__ uint2 tt_read_tr16(const uint8_t* p) {
    const tt_i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (tt_lds_i16x4*)(const __attribute__((address_space(3))) uint8_t*)(p));
    return __builtin_bit_cast(uint2, v);
}

// Workgroup (bx, by, bz) of one both-strided product: output tile (by, bx), slice bz.
__device__ __forceinline__ void skinny_tt_unit(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                               int64_t Mc, int64_t Nc, int64_t P, int64_t chunks_per_slice,
                                               float* __restrict__ part, int64_t bx, int64_t by, int64_t bz) {
    constexpr int NA = SK_BM * SK_PC * 2 / 16 / 256;   // A pieces per thread: 4
    constexpr int NB = SK_BN * SK_PC * 2 / 16 / 256;   // B pieces per thread: 2
    static_assert(SK_BM == 128 && SK_BN == 64 && SK_PC == 64, "tile");
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * SK_STAGE];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t i0 = by * SK_BM, j0 = bx * SK_BN;
    const int64_t nchunks = (P + SK_PC - 1) / SK_PC;
    const int64_t c0 = bz * chunks_per_slice;
    const int64_t c1 = (c0 + chunks_per_slice < nchunks) ? c0 + chunks_per_slice : nchunks;
    // element (i, p) of the A operand at A[p * Mc + i], (j, p) of the B operand at B[p * Nc + j]
    uint32_t offa[NA], offb[NB];
    int pa[NA], pb[NB];
#pragma unroll
    for (int t = 0; t < NA; ++t) {
        const int q = tid + 256 * t, p = q >> 4, c = q & 15;
        pa[t] = p;
        offa[t] = i0 + 8 * c < Mc ? (uint32_t)(((int64_t)p * Mc + 8 * c) * 2) : SK_OOB;
    }
#pragma unroll
    for (int t = 0; t < NB; ++t) {
        const int q = tid + 256 * t, p = q >> 3, c = q & 7;
        pb[t] = p;
        offb[t] = j0 + 8 * c < Nc ? (uint32_t)(((int64_t)p * Nc + 8 * c) * 2) : SK_OOB;
    }
    struct Stage { uint4 a[NA], b[NB]; };
    auto load = [&](Stage& S, int64_t c) {
        const int64_t cc = c < c1 ? c : c1 - 1;            // past the slice: a repeat, never used
        const int64_t p0 = cc * SK_PC;
        const int rem = (int)(P - p0 < SK_PC ? P - p0 : SK_PC);
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + p0 * Mc + i0, (P - p0) * Mc * 2 - i0 * 2);
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + p0 * Nc + j0, (P - p0) * Nc * 2 - j0 * 2);
#pragma unroll
        for (int t = 0; t < NA; ++t) S.a[t] = buf_load16(ra, pa[t] < rem ? offa[t] : SK_OOB, 0);
#pragma unroll
        for (int t = 0; t < NB; ++t) S.b[t] = buf_load16(rb, pb[t] < rem ? offb[t] : SK_OOB, 0);
    };
    auto store = [&](const Stage& S, int stage) {
        uint8_t* sA = lds + stage * SK_STAGE;
        uint8_t* sB = sA + SK_A_BYTES;
#pragma unroll
        for (int t = 0; t < NA; ++t) {
            const int q = tid + 256 * t;
            *reinterpret_cast<uint4*>(sA + tt_off<SK_BM>(q >> 4, 8 * (q & 15))) = S.a[t];
        }
#pragma unroll
        for (int t = 0; t < NB; ++t) {
            const int q = tid + 256 * t;
            *reinterpret_cast<uint4*>(sB + tt_off<SK_BN>(q >> 3, 8 * (q & 7))) = S.b[t];
        }
    };
    // lane l reads, for column tile `ct` (32 columns), column 32 ct + l % 32 at contraction
    // rows 16 s + 8 (l / 32) .. + 7: rows row0 .. row0 + 3 and row0 + 4 .. row0 + 7
    const int g = lane >> 4, jl = lane & 15;
    const int row0 = 8 * (g >> 1) + (jl >> 2);
    const int a_base = tt_off<SK_BM>(row0, wave * 32 + 16 * (g & 1) + 4 * (jl & 3));
    const int b_base0 = tt_off<SK_BN>(row0, 16 * (g & 1) + 4 * (jl & 3));
    const int b_base1 = tt_off<SK_BN>(row0, 32 + 16 * (g & 1) + 4 * (jl & 3));
    auto frag = [&](const uint8_t* p, int rowbytes) {
        const uint2 lo = tt_read_tr16(p);
        const uint2 hi = tt_read_tr16(p + 4 * rowbytes);
        return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
    };
    f32x16 acc0 = {}, acc1 = {};
    auto compute = [&](int stage) {
        const uint8_t* sA = lds + stage * SK_STAGE;
        const uint8_t* sB = sA + SK_A_BYTES;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const bf16x8 a = frag(sA + a_base + s * 16 * (2 * SK_BM), 2 * SK_BM);
            const bf16x8 b0 = frag(sB + b_base0 + s * 16 * (2 * SK_BN), 2 * SK_BN);
            const bf16x8 b1 = frag(sB + b_base1 + s * 16 * (2 * SK_BN), 2 * SK_BN);
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, acc1, 0, 0, 0);
        }
    };
    Stage s0, s1, s2;
    auto step = [&](int64_t k, Stage& cur, const Stage& nx) {
        store(nx, (int)((k + 1) & 1));
        load(cur, c0 + k + 3);
        compute((int)(k & 1));
        __syncthreads();
    };
    const int64_t n = c1 - c0;
    if (n > 0) {
        load(s0, c0);
        store(s0, 0);
        load(s1, c0 + 1);
        load(s2, c0 + 2);
        __syncthreads();
        int64_t k = 0;
        for (; k + 3 <= n; k += 3) {
            step(k, s0, s1);
            step(k + 1, s1, s2);
            step(k + 2, s2, s0);
        }
        if (k < n) step(k, s0, s1);
        if (k + 1 < n) step(k + 1, s1, s2);
    }
    float* out = part + bz * Mc * Nc;
#pragma unroll
    for (int reg = 0; reg < 16; ++reg) {
        const int64_t row = i0 + wave * 32 + 8 * (reg >> 2) + 4 * (lane >> 5) + (reg & 3);
        const int64_t col0 = j0 + (lane & 31), col1 = col0 + 32;
        if (row < Mc) {
            if (col0 < Nc) out[row * Nc + col0] = acc0[reg];
            if (col1 < Nc) out[row * Nc + col1] = acc1[reg];
        }
    }
}

// One launch runs two both-strided products side by side (dA and dB of the backward, each
// of which fills the chip with about one workgroup per CU; together they hold two per CU,
// so twice the loads are in flight): workgroups below blocks0 belong to p0, the rest to p1.
// A single product passes itself twice with blocks0 = its workgroup count.
__global__ __launch_bounds__(256) void k_skinny_tt(TtProblem p0, TtProblem p1, int64_t blocks0) {
    const bool second = (int64_t)blockIdx.x >= blocks0;
    const int64_t b = second ? (int64_t)blockIdx.x - blocks0 : (int64_t)blockIdx.x;
    const int64_t gx = second ? p1.gx : p0.gx, gy = second ? p1.gy : p0.gy;
    skinny_tt_unit(second ? p1.A : p0.A, second ? p1.B : p0.B, second ? p1.Mc : p0.Mc, second ? p1.Nc : p0.Nc,
                   second ? p1.P : p0.P, second ? p1.cps : p0.cps, second ? p1.part : p0.part, b % gx,
                   (b / gx) % gy, b / (gx * gy));
}

// Fixed-order sum of the slices: v = sum_z part[z][i][j];  C = scale * v (bf16 or fp32,
// [i][j] or transposed [j][i]);  C2 = bf16(scale2 * v) when given.  Workgroups from
// `sum_blocks` on decode the weight's block constants instead (dq.n1 of them, one per
// thread), so that the decode the next fused product needs costs no launch of its own.
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ part, int S,
                                                       int64_t Mc, int64_t Nc, float scale,
                                                       void* __restrict__ C, bool c_f32,
                                                       bool c_trans, uint16_t* __restrict__ C2,
                                                       float scale2, int64_t sum_blocks, DqDecode dq) {
    if ((int64_t)blockIdx.x >= sum_blocks) {
        const int64_t i = ((int64_t)blockIdx.x - sum_blocks) * 256 + threadIdx.x;
        if (i < dq.n1) dq.out[i] = decode_c1(dq.q[i], c2_step(dq.c2[i >> 8]), *dq.mean);
        return;
    }
    const int64_t total = Mc * Nc;
    const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i4 >= total) return;
    float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (i4 + 4 <= total) {
        for (int z = 0; z < S; ++z) {
            const float4 p = *reinterpret_cast<const float4*>(part + (int64_t)z * total + i4);
            v[0] += p.x; v[1] += p.y; v[2] += p.z; v[3] += p.w;
        }
    } else {
        for (int z = 0; z < S; ++z)
            for (int e = 0; e < 4; ++e)
                if (i4 + e < total) v[e] += part[(int64_t)z * total + i4 + e];
    }
    for (int e = 0; e < 4; ++e) {
        const int64_t i = i4 + e;
        if (i >= total) break;
        const int64_t row = i / Nc, col = i - row * Nc;
        const int64_t dst = c_trans ? col * Mc + row : i;
        if (c_f32) reinterpret_cast<float*>(C)[dst] = v[e] * scale;
        else reinterpret_cast<uint16_t*>(C)[dst] = f32_to_bf16(v[e] * scale);
        if (C2) C2[dst] = f32_to_bf16(v[e] * scale2);
    }
}

void skinny_plan(int64_t Mc, int64_t Nc, int64_t P, int* slices, int64_t* chunks_per_slice) {
    const int64_t tiles = ((Mc + SK_BM - 1) / SK_BM) * ((Nc + SK_BN - 1) / SK_BN);
    const int64_t nchunks = (P + SK_PC - 1) / SK_PC;
    if (tiles <= 0 || nchunks <= 0) {      // empty output or empty contraction: one slice
        *slices = 1;
        *chunks_per_slice = 0;
        return;
    }
    // About one workgroup per CU: more slices would add fp32 partial traffic (S times the
    // output, written once and read once) faster than they add bandwidth.  When that leaves
    // the CUs unevenly loaded (the busiest one runs ceil(tiles S / 256) workgroups of 1/S
    // of a tile each), another S up to 8 is taken if a cost estimate puts it 5% lower: the
    // busiest CU's share of the operands at 1/256 of 5 TB/s, 3 us per workgroup it runs,
    // and the partial sums written and read at 5 TB/s.
    const int64_t smax = nchunks / 4 > 1 ? nchunks / 4 : 1;
    int64_t S = (256 + tiles - 1) / tiles;
    if (S > smax) S = smax;
    if (S < 1) S = 1;
    auto cost = [&](int64_t c) {
        const double rounds = (double)((tiles * c + 255) / 256);
        return rounds / (double)c * (double)P * (SK_BM + SK_BN) * 2.0 / 19.5e9 + rounds * 3e-6 +
               (double)c * (double)Mc * (double)Nc * 8.0 / 5e12;
    };
    const double base = cost(S);
    double best = base;
    for (int64_t c = 1; c <= 8 && c <= smax; ++c) {
        const double t = cost(c);
        if (t < 0.95 * base && t < best) {
            best = t;
            S = c;
        }
    }
    int64_t cps = nchunks > 0 ? (nchunks + S - 1) / S : 0;
    if (cps > 0) S = (nchunks + cps - 1) / cps;
    *slices = (int)S;
    *chunks_per_slice = cps;
}

size_t skinny_partial_bytes(int64_t Mc, int64_t Nc, int64_t P) {
    int S;
    int64_t cps;
    skinny_plan(Mc, Nc, P, &S, &cps);
    return ((size_t)S * (size_t)Mc * (size_t)Nc * 4 + 255) & ~(size_t)255;
}

hipError_t launch_lora_gemm(const uint16_t* A, bool a_trans, const uint16_t* B, bool b_trans,
                            int64_t Mc, int64_t Nc, int64_t P, float* part, float scale, void* C,
                            bool c_f32, bool c_trans, uint16_t* C2, float scale2, hipStream_t s,
                            uint16_t* pack, bool pack_even_odd, const DqDecode* dq) {
    if (Mc == 0 || Nc == 0) return hipSuccess;
    if (pack && a_trans) return hipErrorInvalidValue;
    // per-lane buffer offsets are 32-bit: a direct operand spans 128 rows of its leading
    // dimension P, a transposed one 64 contraction rows of its leading dimension
    if ((!a_trans || !b_trans) && P >= ((int64_t)1 << 22)) return hipErrorInvalidValue;
    if ((a_trans && Mc >= ((int64_t)1 << 23)) || (b_trans && Nc >= ((int64_t)1 << 23)))
        return hipErrorInvalidValue;
    // a strided operand is read in 16-byte pieces along its rows: 8 | its row length
    if ((a_trans && (Mc & 7)) || (b_trans && (Nc & 7))) return hipErrorInvalidValue;
    int S;
    int64_t cps;
    skinny_plan(Mc, Nc, P, &S, &cps);
    // with a packed copy of A to write, the row tiles cover whole 512-row token tiles, so
    // that the rows past Mc are written too (as zeros)
    const int64_t row_tiles = pack ? ((Mc + 511) / 512) * (512 / SK_BM) : (Mc + SK_BM - 1) / SK_BM;
    dim3 grid((unsigned)((Nc + SK_BN - 1) / SK_BN), (unsigned)row_tiles, (unsigned)S);
    if (!a_trans && !b_trans)
        hipLaunchKernelGGL((k_skinny<false, false>), grid, dim3(256), 0, s, A, B, Mc, Nc, P, cps, part, pack, pack_even_odd);
    else if (!a_trans && b_trans)
        hipLaunchKernelGGL((k_skinny<false, true>), grid, dim3(256), 0, s, A, B, Mc, Nc, P, cps, part, pack, pack_even_odd);
    else if (a_trans && b_trans) {
        const TtProblem p{A, B, Mc, Nc, P, cps, part, (int64_t)grid.x, (int64_t)grid.y};
        const int64_t blocks = (int64_t)grid.x * grid.y * grid.z;
        hipLaunchKernelGGL(k_skinny_tt, dim3((unsigned)blocks), dim3(256), 0, s, p, p, blocks);
    }
    else
        hipLaunchKernelGGL((k_skinny<true, false>), grid, dim3(256), 0, s, A, B, Mc, Nc, P, cps, part, nullptr, false);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t total = Mc * Nc;
    const int64_t sum_blocks = (total + 1023) / 1024;
    const DqDecode none{nullptr, nullptr, nullptr, 0, nullptr};
    const DqDecode& d = dq ? *dq : none;
    const int64_t blocks = sum_blocks + (d.n1 + 255) / 256;
    hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)blocks), dim3(256), 0, s, part, S, Mc, Nc, scale, C,
                       c_f32, c_trans, C2, scale2, sum_blocks, d);
    return hipGetLastError();
}

hipError_t launch_lora_tt_pair(const TtProduct& d0, const TtProduct& d1, hipStream_t s) {
    const TtProduct* d[2] = {&d0, &d1};
    TtProblem p[2];
    int S[2];
    int64_t blocks[2];
    for (int i = 0; i < 2; ++i) {
        const TtProduct& q = *d[i];
        if (q.Mc >= ((int64_t)1 << 23) || q.Nc >= ((int64_t)1 << 23) || (q.Mc & 7) || (q.Nc & 7))
            return hipErrorInvalidValue;
        int64_t cps;
        skinny_plan(q.Mc, q.Nc, q.P, &S[i], &cps);
        p[i] = TtProblem{q.A, q.B, q.Mc, q.Nc, q.P, cps, q.part, (q.Nc + SK_BN - 1) / SK_BN,
                         (q.Mc + SK_BM - 1) / SK_BM};
        blocks[i] = q.Mc == 0 || q.Nc == 0 ? 0 : p[i].gx * p[i].gy * S[i];
    }
    if (blocks[0] + blocks[1] > 0)
        hipLaunchKernelGGL(k_skinny_tt, dim3((unsigned)(blocks[0] + blocks[1])), dim3(256), 0, s, p[0], p[1],
                           blocks[0]);
    hipError_t e = hipGetLastError();
    const DqDecode none{nullptr, nullptr, nullptr, 0, nullptr};
    for (int i = 0; i < 2 && e == hipSuccess; ++i) {
        const TtProduct& q = *d[i];
        if (blocks[i] == 0) continue;
        const int64_t sum_blocks = (q.Mc * q.Nc + 1023) / 1024;
        hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)sum_blocks), dim3(256), 0, s, q.part, S[i], q.Mc, q.Nc,
                           q.scale, q.C, true, q.c_trans, (uint16_t*)nullptr, 0.0f, sum_blocks, none);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace nf4
