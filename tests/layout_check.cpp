// Host-side check of the matrix-core kernel's LDS stage layouts
// (dense_fp32_matrix_amd/csrc/lds_layout.hpp, compiled here as plain C++).
//
// For every layout the kernel instantiates (KC and KM, R = 64/128/256 rows,
// BK = 16/32, 16- or 4-byte load lanes) it walks every direct-load
// instruction and lane of one K-step and checks that
//   * each element (r, k) of the R x BK block is fetched exactly once,
//   * it lands where the fragment reads look for it (at(r, k)), and
//   * the stage offsets stay inside the stage (FLOATS) and never collide;
// then it prints, for every tile and operand layout, the LDS byte offsets
// each lane of each wave reads in one K-step (fragment reads) and writes
// (direct loads), for the bank model in tests/test_lds_layout.py.
//
// Output lines:  "ok <layout>"  /  "FAIL <layout>: <reason>"
//                "read <tile> <ops> <wave> <width> <64 byte offsets>"
//                "write <tile> <ops> <wave> <width> <64 byte offsets>"
#include <cstdio>
#include <set>
#include <string>
#include <vector>

#include "lds_layout.hpp"
#include "tile_order.hpp"

using namespace sgemm_impl;

static int failures = 0;

template <class L>
void check_layout(const char* kind, int R, int BK, int W) {
    char name[96];
    std::snprintf(name, sizeof(name), "%s R=%d BK=%d W=%d", kind, R, BK, W);
    std::vector<int> hits(R * BK, 0);
    std::set<int> offsets;
    std::string why;
    for (int ins = 0; ins < L::INSTR && why.empty(); ++ins) {
        for (int lane = 0; lane < 64 && why.empty(); ++lane) {
            int r0, k0;
            L::elem(ins, lane, r0, k0);
            for (int sub = 0; sub < W; ++sub) {
                const int r = L::KC ? r0 : r0 + sub;       // a lane's W floats run along k (KC) or r (KM)
                const int k = L::KC ? k0 + sub : k0;
                const int off = L::dst(ins) + W * lane + sub;
                if (r < 0 || r >= R || k < 0 || k >= BK) { why = "element outside the block"; break; }
                if (off < 0 || off >= L::FLOATS) { why = "offset outside the stage"; break; }
                if (!offsets.insert(off).second) { why = "two elements at one offset"; break; }
                if (L::at(r, k) != off) { why = "fragment read looks elsewhere"; break; }
                ++hits[r * BK + k];
            }
        }
    }
    if (why.empty())
        for (int e = 0; e < R * BK; ++e)
            if (hits[e] != 1) { why = "element fetched " + std::to_string(hits[e]) + " times"; break; }
    if (why.empty() && L::INSTR * L::SEG != R * BK) why = "instructions do not cover the block";
    if (why.empty()) std::printf("ok %s\n", name);
    else { std::printf("FAIL %s: %s\n", name, why.c_str()); ++failures; }
}

// Edge clamp: for every matrix extent lim along the non-K dimension (a
// multiple of 4 for a 16-byte KM lane) and every tile start r0 < lim, the
// W-float read of every lane of a tile's block stays inside [0, lim).
template <class L>
void check_clamp(const char* kind, int R, int W) {
    const int lanew = L::KC ? 1 : W;
    for (int lim = 1; lim <= 3 * R; ++lim) {
        if (lim % lanew) continue;
        for (int r0 = 0; r0 < lim; r0 += R) {
            for (int ins = 0; ins < L::INSTR; ++ins)
                for (int lane = 0; lane < 64; ++lane) {
                    int r, k;
                    L::elem(ins, lane, r, k);
                    const int rr = clamp_index<L>(r0 + r, lim);
                    if (rr < 0 || rr + lanew > lim || (r0 + r < lim && rr != r0 + r)) {
                        std::printf("FAIL clamp %s R=%d W=%d lim=%d r0=%d r=%d -> %d\n", kind, R, W, lim, r0, r, rr);
                        ++failures;
                        return;
                    }
                }
        }
    }
    std::printf("ok clamp %s R=%d W=%d\n", kind, R, W);
}

template <int R, int BK>
void check_rbk() {
    check_clamp<KcLayout<R, BK, 4>>("KC", R, 4);
    check_clamp<KcLayout<R, BK, 1>>("KC", R, 1);
    check_clamp<KmLayout<R, BK, 4>>("KM", R, 4);
    check_clamp<KmLayout<R, BK, 1>>("KM", R, 1);
    check_layout<KcLayout<R, BK, 4>>("KC", R, BK, 4);
    check_layout<KcLayout<R, BK, 1>>("KC", R, BK, 1);
    check_layout<KmLayout<R, BK, 4>>("KM", R, BK, 4);
    check_layout<KmLayout<R, BK, 1>>("KM", R, BK, 1);
}

// The fragment reads of one K-step of one wave, as the kernel issues them
// (mfma_tile_dtl's read_frags): lane l holds op(A)[m][k] and op(B)[k][n] for
// m, n = l % 32 within the block and k = 8 kg + 4 (l / 32) + q.
template <int BM, int BN, int BK, int WGM, int WGN, int OPS>
void dump_tile(int tile) {
    using LA = ALayout<(OPS & 1) != 0, BM, BK, 4>;
    using LB = BLayout<(OPS & 2) != 0, BN, BK, 4>;
    constexpr int WM = BM / WGM, WN = BN / WGN, MB = WM / 32, NB = WN / 32, KG = BK / 8;
    constexpr bool IB = !LB::KC && LA::KC && NB == 4;      // interleaved columns
    for (int wave = 0; wave < WGM * WGN; ++wave) {
        const int wm = wave / WGN, wn = wave % WGN;
        auto emit = [&](const char* what, int width, auto addr) {
            std::printf("%s %d %d %d %d", what, tile, OPS, wave, width);
            for (int lane = 0; lane < 64; ++lane) std::printf(" %d", 4 * addr(lane % 32, lane / 32));
            std::printf("\n");
        };
        for (int kg = 0; kg < KG; ++kg) {
            for (int mb = 0; mb < MB; ++mb) {
                if constexpr (LA::KC) {
                    emit("read", 16, [&](int l32, int lh) { return LA::chunk(wm * WM + mb * 32 + l32, 2 * kg + lh); });
                } else {
                    for (int q = 0; q < 4; ++q)
                        emit("read", 4, [&](int l32, int lh) { return LA::krow(8 * kg + 4 * lh + q) + wm * WM + l32 + mb * 32; });
                }
            }
            if constexpr (IB) {
                for (int q = 0; q < 4; ++q)
                    emit("read", 16, [&](int l32, int lh) { return LA::FLOATS + LB::krow(8 * kg + 4 * lh + q) + wn * WN + 4 * l32; });
            } else {
                for (int nb = 0; nb < NB; ++nb) {
                    if constexpr (LB::KC) {
                        emit("read", 16, [&](int l32, int lh) {
                            return LA::FLOATS + LB::chunk(wn * WN + nb * 32 + l32, 2 * kg + lh);
                        });
                    } else {
                        for (int q = 0; q < 4; ++q)
                            emit("read", 4, [&](int l32, int lh) {
                                return LA::FLOATS + LB::krow(8 * kg + 4 * lh + q) + wn * WN + l32 + nb * 32;
                            });
                    }
                }
            }
        }
        // direct loads: instruction i * waves + wave of each operand, lane l at dst + 4 l floats
        for (int i = 0; i < LA::INSTR / (WGM * WGN); ++i)
            emit("write", 16, [&](int l32, int lh) { return LA::dst(i * WGM * WGN + wave) + 4 * (l32 + 32 * lh); });
        for (int i = 0; i < LB::INSTR / (WGM * WGN); ++i)
            emit("write", 16, [&](int l32, int lh) {
                return LA::FLOATS + LB::dst(i * WGM * WGN + wave) + 4 * (l32 + 32 * lh);
            });
    }
}

template <int BM, int BN, int BK, int WGM, int WGN>
void dump_all_ops(int tile) {
    dump_tile<BM, BN, BK, WGM, WGN, 0>(tile);
    dump_tile<BM, BN, BK, WGM, WGN, 1>(tile);
    dump_tile<BM, BN, BK, WGM, WGN, 2>(tile);
    dump_tile<BM, BN, BK, WGM, WGN, 3>(tile);
}

// Tile order: for every grid of tiles (and the raster group heights the
// dispatcher uses), workgroup ids 0 .. tiles - 1 map one to one onto the
// output tiles.
void check_tile_order() {
    for (int tm_n = 1; tm_n <= 48; ++tm_n)
        for (int tn_n = 1; tn_n <= 48; ++tn_n)
            for (int gm : {0, 1, tm_n < 8 ? tm_n : 8}) {
                std::vector<int> seen(tm_n * tn_n, 0);
                for (int b = 0; b < tm_n * tn_n; ++b) {
                    int tm, tn;
                    tile_coords(b, tm_n, tn_n, gm, &tm, &tn);
                    if (tm < 0 || tm >= tm_n || tn < 0 || tn >= tn_n || seen[tm * tn_n + tn]++) {
                        std::printf("FAIL tile order %d x %d group %d: id %d -> (%d, %d)\n", tm_n, tn_n, gm, b, tm, tn);
                        ++failures;
                        return;
                    }
                }
            }
    std::printf("ok tile order\n");
}

int main() {
    check_tile_order();
    check_rbk<256, 16>();
    check_rbk<128, 16>();
    check_rbk<64, 32>();
    check_rbk<64, 16>();
    check_rbk<128, 32>();
    // the matrix-core tile table: 256 x 256 x 16 (4 x 2 waves, two tiles),
    // 128 x 128 x 16 (2 x 4 waves), 64 x 64 x 16 (2 x 2 waves)
    dump_all_ops<256, 256, 16, 4, 2>(0);
    dump_all_ops<128, 128, 16, 2, 4>(2);
    dump_all_ops<64, 64, 16, 2, 2>(3);
    return failures == 0 ? 0 : 1;
}
