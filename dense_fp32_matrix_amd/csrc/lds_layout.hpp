// LDS stage layouts of the matrix-core kernel (mfma.hip), shared with the
// host-side layout check (tests/layout_check.cpp), which compiles this
// header as plain C++.
//
// One K-step of one operand is an R x BK block (R = BM for A, BN for B).
// Direct-to-LDS loads write it: instruction `ins` of a wave writes SEG
// consecutive floats at dst(ins), lane l's W floats at dst(ins) + W * l, and
// elem(ins, lane) names the element (r, k) that lane fetches (its W floats
// run along k for a KC stage and along r for a KM stage).  The fragment
// reads then find element (r, k) at at(r, k).
//  KC: R rows of BK floats (k contiguous within a row), the 16-byte chunks of
//      row r at XOR-swizzled positions; fragments are read as 16-byte
//      chunks.  A stored M x K and B stored N x K (transposed) use it.
//  KM: BK rows of R floats (k-major), in blocks of 256 / R rows whose starts
//      are GS floats apart; fragments are read one float per k row (four
//      adjacent floats with interleaved columns).  B stored K x N and A
//      stored K x M (transposed) use it.
#pragma once

#include <type_traits>

#if defined(__HIPCC__)
#define SGEMM_HD __host__ __device__ __forceinline__
#else
#define SGEMM_HD inline
#endif

namespace sgemm_impl {

// Chunk-position swizzle of row r of a KC stage (BK/4 chunks of 16 bytes
// per row): logical chunk c is stored at chunk c ^ swz(r).
// A fragment read (ds_read_b128) has lane l read chunk 2 kg + l / 32 of row
// base + l % 32.  gfx950 serves such a read in 4 phases of 16 lanes -- lane
// l in phase (l >> 5, parity of bits 2-4 of l) -- each over one 256-byte row
// of 64 banks, so the 16 rows of a phase must land on 16 different 16-byte
// bank slots.  With 64-byte rows (BK = 16) row r sits in slot 4 (r & 3) +
// chunk, and the rows of a phase that share r & 3 differ in (r >> 2) & 3,
// which the swizzle XORs into the chunk; with 128-byte rows (BK = 32) the slot
// is 8 (r & 1) + chunk and bit 1 of r is XORed in as well.  (The bank model
// and the measurements behind it are in tests/test_lds_layout.py.)
template <int BK>
SGEMM_HD int a_swizzle(int r) {
    if constexpr (BK == 16) return (r >> 2) & 3;
    else return ((r >> 2) & 3) | (((r >> 1) & 1) << 2);
}

template <int R, int BK, int W>
struct KcLayout {
    static constexpr bool KC = true;
    static constexpr int EXTENT = R;                      // rows (the non-K dimension) of the stage
    static constexpr int SEG = 64 * W;                    // floats one instruction writes
    static constexpr int FLOATS = R * BK;
    static constexpr int INSTR = FLOATS / SEG;
    static_assert(SEG % BK == 0, "an instruction fills whole rows");
    static SGEMM_HD void elem(int ins, int lane, int& r, int& k) {
        const int p = ins * SEG + W * lane;
        r = p / BK;
        k = 4 * (((p % BK) / 4) ^ a_swizzle<BK>(r)) + p % 4;
    }
    static SGEMM_HD int dst(int ins) { return ins * SEG; }
    // 16-byte chunk c (k = 4c .. 4c + 3) of row r
    static SGEMM_HD int chunk(int r, int c) { return r * BK + 4 * (c ^ a_swizzle<BK>(r)); }
    static SGEMM_HD int at(int r, int k) { return chunk(r, k / 4) + k % 4; }
};

template <int R, int BK, int W>
struct KmLayout {
    static constexpr bool KC = false;
    static constexpr int EXTENT = R;                      // floats per k row (the non-K dimension)
    static constexpr int SEG = 64 * W;
    static constexpr int ROWS = 256 / R;                  // k rows per 1 KB block
    static constexpr int GS = 256 + 8 * ROWS;            // floats between blocks
    static constexpr int SEGS = 256 / SEG;                // instructions per block
    static constexpr int INSTR = BK / ROWS * SEGS;
    static constexpr int FLOATS = BK / ROWS * GS;
    static_assert(R == 64 || R == 128 || R == 256, "blocks hold one, two or four rows");
    static_assert((4 / ROWS) * GS % 64 == 32, "lane halves of a fragment read 32 banks apart");
    static SGEMM_HD void elem(int ins, int lane, int& r, int& k) {
        const int f = (ins % SEGS) * SEG + W * lane;       // float within the block
        k = ins / SEGS * ROWS + f / R;
        r = f % R;
    }
    static SGEMM_HD int dst(int ins) { return ins / SEGS * GS + ins % SEGS * SEG; }
    // k row k starts at this offset
    static SGEMM_HD int krow(int k) { return (k / ROWS) * GS + (k % ROWS) * R; }
    static SGEMM_HD int at(int r, int k) { return krow(k) + r; }
};

// The stored index along the non-K dimension that a load lane reads for
// tile index idx of a matrix with lim of them: past the end, a KC lane reads
// the last row instead, and a KM lane (SEG / 64 consecutive columns) the
// last whole group of columns, so that every lane's read stays inside the
// matrix (a 16-byte KM lane needs lim to be a multiple of 4, which the
// 16-byte loaders require); those values only reach outputs that are never
// written.
template <class L>
SGEMM_HD int clamp_index(int idx, int lim) {
    constexpr int lanew = L::SEG / 64;
    const int last = L::KC ? lim - 1 : (lim - 1) & ~(lanew - 1);
    return idx < last ? idx : last;
}

// A stored as is (M x K) is k-contiguous, stored transposed k-major; B the
// other way round.
template <bool TA, int BM, int BK, int W>
using ALayout = std::conditional_t<TA, KmLayout<BM, BK, W>, KcLayout<BM, BK, W>>;
template <bool TB, int BN, int BK, int W>
using BLayout = std::conditional_t<TB, KcLayout<BN, BK, W>, KmLayout<BN, BK, W>>;

// Floats per stage: the A region, then the B region (the same for both lane
// widths).
template <int OPS, int BM, int BN, int BK>
struct DtlStageFloats {
    static constexpr int value =
        ALayout<(OPS & 1) != 0, BM, BK, 4>::FLOATS + BLayout<(OPS & 2) != 0, BN, BK, 4>::FLOATS;
};

}  // namespace sgemm_impl
