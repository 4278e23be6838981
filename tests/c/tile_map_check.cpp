// Host check of the fused products' work units (tile_map.h) over many launch shapes.
//
// For each shape it runs the workgroup -> unit map over the whole grid and checks that
// every output tile is computed exactly once, either whole or as pieces 0 .. S-1 whose
// contraction ranges partition all steps; that the pieces of a tile run on one XCD
// after that XCD's whole tiles and own S partial slots inside the planned workspace;
// that the summing kernel's slot -> tile lookup inverts the map (and rejects unused
// slots); and that tail waves fit the XCD.  It also checks that the fragment-order packing
// of the A operand is a bijection onto the MFMA operand layout.  Prints "<shapes> <failures>".
#include <cstdio>
#include <map>
#include <set>
#include <vector>

#include "tile_map.h"

using namespace nf4;

static int check(int64_t M, int64_t ncols, int64_t steps, int TM, int TN) {
    const FusedPlan p = fused_plan(M, ncols, steps, TM, TN);
    const int64_t tm_n = (M + TM - 1) / TM, tn_n = (ncols + TN - 1) / TN, T = tm_n * tn_n;
    if (p.S < 1 || p.S > MAX_SPLIT) return 1;
    if (p.S == 1 && (p.grid != T || p.bytes != 0)) return 2;
    if (p.S > 1 && p.bytes != (size_t)(p.tails * p.S) * TILE_FLOATS * 4) return 3;
    std::vector<int> whole(T, 0);
    std::vector<std::vector<int>> pieces(T, std::vector<int>(p.S, 0));
    std::map<int64_t, int64_t> tail_of_tile;     // tile -> tail index
    std::map<int64_t, int64_t> xcd_of_tile;
    std::vector<int64_t> last_whole_local(XCDS, -1), first_piece_local(XCDS, INT64_MAX);
    std::vector<int64_t> units_per_xcd(XCDS, 0);
    for (int64_t wg = 0; wg < p.grid; ++wg) {
        Unit u;
        if (!unit_of(wg, tm_n, tn_n, p.S, u)) continue;
        if (u.tm < 0 || u.tm >= tm_n || u.tn < 0 || u.tn >= tn_n) return 4;
        const int64_t t = u.tm * tn_n + u.tn, x = wg % XCDS, local = wg / XCDS;
        units_per_xcd[x]++;
        int64_t sb, n;
        unit_steps(steps, p.chunk, u.split, sb, n);
        if (u.split < 0) {
            whole[t]++;
            if (sb != 0 || n != steps) return 5;
            if (local > last_whole_local[x]) last_whole_local[x] = local;
            continue;
        }
        if (p.S == 1 || u.split >= p.S) return 6;
        pieces[t][u.split]++;
        if (n < 1 || sb + n > steps || sb != u.split * p.chunk) return 7;
        if (u.split == p.S - 1 && sb + n != steps) return 8;
        if (u.tail < 0 || u.tail >= p.tails) return 9;
        if ((size_t)(u.tail * p.S + p.S) * TILE_FLOATS * 4 > p.bytes) return 10;
        auto it = tail_of_tile.find(t);
        if (it == tail_of_tile.end()) {
            tail_of_tile[t] = u.tail;
            xcd_of_tile[t] = x;
        } else if (it->second != u.tail || xcd_of_tile[t] != x) {
            return 11;
        }
        if (local < first_piece_local[x]) first_piece_local[x] = local;
    }
    std::set<int64_t> tails;
    for (auto& kv : tail_of_tile)
        if (!tails.insert(kv.second).second) return 12;   // distinct tiles, distinct tails
    for (int64_t t = 0; t < p.tails; ++t) {
        int64_t tm, tn;
        const bool used = tail_tile(t, tm_n, tn_n, tm, tn);
        if (used != (tails.count(t) == 1)) return 17;
        if (used && tail_of_tile[tm * tn_n + tn] != t) return 18;
    }
    for (int64_t t = 0; t < T; ++t) {
        int np = 0;
        for (int s = 0; s < p.S; ++s) {
            if (pieces[t][s] > 1) return 13;
            np += pieces[t][s];
        }
        if (!((whole[t] == 1 && np == 0) || (whole[t] == 0 && np == p.S))) return 14;
    }
    for (int x = 0; x < XCDS; ++x) {
        if (first_piece_local[x] != INT64_MAX && first_piece_local[x] < last_whole_local[x]) return 15;
        // the units of an XCD beyond its full waves fit one wave
        if (p.S > 1) {
            const int64_t tail_units = units_per_xcd[x] - (last_whole_local[x] + 1);
            if (tail_units > XCD_CUS) return 16;
        }
    }
    return 0;
}

int main() {
    const int64_t Ms[] = {1, 17, 255, 256, 257, 512, 1000, 2048, 4096, 4097, 8192};
    const int64_t Ns[] = {64, 256, 320, 1088, 4096, 8192, 11008, 22016, 65600};
    const int64_t Ss[] = {1, 2, 3, 4, 5, 7, 8, 64, 128, 129, 172, 344};
    long shapes = 0, bad = 0;
    for (int64_t M : Ms)
        for (int64_t N : Ns)
            for (int64_t S : Ss) {
                for (int shape = 0; shape < 2; ++shape) {
                    ++shapes;
                    const int e = shape ? check(M, N, S, 512, 128) : check(M, N, S, 256, 256);
                    if (e) {
                        ++bad;
                        if (bad < 10) std::printf("# M=%lld ncols=%lld steps=%lld shape %d code %d\n",
                                                  (long long)M, (long long)N, (long long)S, shape, e);
                    }
                }
            }
    // every tile count up to 600 (one token tile), with a few step counts
    for (int64_t T = 1; T <= 600; ++T)
        for (int64_t S : {2, 3, 9, 128}) {
            ++shapes;
            const int e = check(FUSED_TM, T * FUSED_TN, S, FUSED_TM, FUSED_TN);
            if (e) {
                ++bad;
                if (bad < 10) std::printf("# tiles=%lld steps=%lld code %d\n", (long long)T, (long long)S, e);
            }
        }
    // fragment-order packing: the 4096 chunks of a block cover the 512 rows x 8 chunk columns
    // of a step once each, and chunk q of the block is what lane q % 64 of wave q / 1024
    // loads for fragment (i, s) = ((q / 256) % 4, (q / 64) % 4): row 128 w + 32 i + l % 32,
    // column 2 s + l / 32 (the 32x32x16 bf16 MFMA A-operand layout)
    {
        std::vector<int> seen(FUSED_TM * 8, 0);
        ++shapes;
        for (int q = 0; q < A_BLOCK_BYTES / 16; ++q) {
            const int row = a_pack_row(q), col = a_pack_col(q);
            if (row < 0 || row >= FUSED_TM || col < 0 || col >= 8) { ++bad; break; }
            seen[row * 8 + col]++;
            const int w = q >> 10, l = q & 63, frag = (q >> 6) & 15, i = frag >> 2, s = frag & 3;
            if (16 * q != w * 16384 + 4096 * i + 1024 * s + 16 * l) ++bad;
            if (row != 128 * w + 32 * i + (l & 31) || col != 2 * s + (l >> 5)) ++bad;
        }
        for (int v : seen)
            if (v != 1) { ++bad; break; }
    }
    std::printf("%ld %ld\n", shapes, bad);
    return 0;
}
