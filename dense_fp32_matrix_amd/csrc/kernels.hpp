// Internal interface between the host dispatcher and the gfx950 kernels.
// Not installed; the public C interface is include/sgemm.h.
#pragma once

#include <cstdint>
#include <hip/hip_runtime.h>

#include "tile_order.hpp"

namespace sgemm_impl {

// One launch of a tiled product kernel.  The kernel computes, for every
// output tile (tm, tn) and slice z < gridDim.z,
//   Sz[i][j] = sum_{k in [z*k_chunk, min(K, (z+1)*k_chunk))} op(A)[i][k] op(B)[k][j]
// with op(A)[i][k] = A[i*lda + k] (or A[k*lda + i] when A is stored
// transposed) and op(B)[k][j] = B[k*ldb + j] (or B[j*ldb + k]).  With one
// slice (c_slice == 0) it writes C[i][j] = alpha * S[i][j] + beta * C[i][j]
// where i < M, j < N (C read only when beta != 0); with several, the raw
// partial Sz goes to C + z * c_slice and the reduction applies alpha, beta.
struct GemmArgs {
    const float* A;
    const float* B;
    float* C;
    int32_t M, N, K;
    float alpha, beta;
    int32_t trans_a, trans_b;   // the naive kernel reads these; the tiled ones are instantiated per layout
    int32_t k_chunk;    // K elements per slice (a multiple of the tile's BK)
    int64_t lda, ldb, ldc;
    int64_t c_slice;    // elements between consecutive slices' outputs
    int32_t tiles_m, tiles_n;
    int32_t group_m;    // tile rows per raster group of the XCD-aware order, or 0 for row-major order
    // stream-K decomposition (MFMA and skinny paths; sk_iters == 0 disables it)
    int32_t sk_grid;    // persistent workgroups
    int32_t dp_tiles;   // tiles computed whole, before the stream-K tiles
    int32_t k_steps;    // K-steps per tile, ceil(K / BK)
    int64_t sk_iters;   // (tile, K-step) units of the stream-K tiles
    int64_t sk_ipw;     // units per workgroup
    float* ws;          // partial-tile slots, 2 per workgroup, BM * BN floats each
};

// The final write of one output element: alpha * v + beta * (*p), one
// rounding for alpha * v and one for the fused add; *p is read only when
// beta != 0 (so whatever C held, NaN included, does not matter then).
__device__ __forceinline__ void store_scaled(float* p, float v, float alpha, float beta) {
    v = alpha * v;
    if (beta != 0.f) v = __builtin_fmaf(beta, *p, v);
    *p = v;
}

// Tile shapes of each path.  The kernels are instantiated for exactly these;
// the dispatcher and sgemm_tile_info read the same table.
struct TileShape {
    int bm, bn, bk;
    int waves_m, waves_n;   // waves per workgroup along M and N
    int waves_per_simd;     // occupancy the register budget is sized for
    int stages = 0;         // matrix-core tiles: LDS stages filled by direct global -> LDS loads
    bool narrow = false;    // matrix-core tiles: also built with 4-byte load lanes (unaligned operands)
    bool prio = false;      // matrix-core tiles: raise the wave's priority while it issues a K-step's
                            // MFMAs after its direct loads, back to normal before the barrier
};

// Matrix-core tiles.  Every one reads its operands with direct global -> LDS
// loads and is built for the four operand layouts (A and B each as stored or
// stored transposed).  The 256 x 256 tiles are built for 16-byte load lanes
// only: with 4-byte lanes their four times as many load offsets do not fit
// the registers left next to 128 accumulators per lane, so unaligned
// operands take the 128 x 128 or 64 x 64 tile, or are packed.
constexpr TileShape kMfmaTiles[] = {
    {256, 256, 16, 4, 2, 2, 2},               // 0: 8 waves (two per SIMD) of 64 x 128; step s + 1 loads during step s
    {256, 256, 16, 4, 2, 2, 3},               // 1: as 0 with three stages (faster when both operands are k-contiguous)
    {128, 128, 16, 2, 4, 2, 4, true, true},   // 2: 8 waves of 64 x 32, four stages (three with 4-byte lanes):
                                              //    fewer tiles than CUs at 256 x 256, long K
    {64, 64, 16, 2, 2, 2, 4, true, true},     // 3: 4 waves of 32 x 32, four stages (three with 4-byte lanes):
                                              //    small products, thin M or N
};
constexpr int kNumMfmaTiles = sizeof(kMfmaTiles) / sizeof(kMfmaTiles[0]);

constexpr TileShape kValuTiles[] = {
    {128, 128, 8, 2, 2, 2},    // 0: 8x8 outputs per lane, 8x8 lanes per wave
};
constexpr int kNumValuTiles = sizeof(kValuTiles) / sizeof(kValuTiles[0]);

// The one-thread-per-output kernel: a 64 x 4 thread block.
constexpr TileShape kNaiveTiles[] = {{4, 64, 1, 1, 1, 4}};
constexpr int kNumNaiveTiles = 1;

// Skinny products (M <= 32): a workgroup of 4 waves owns 16 (or 32) rows x
// 64 columns and one K slice, split over its waves; K slices are multiples
// of bk = 64, the stream-K unit.  Built for the four operand layouts.
constexpr TileShape kSkinnyTiles[] = {
    {16, 64, 64, 1, 4, 2},     // 0: one 16-row block of A (M <= 16)
    {32, 64, 64, 1, 4, 2},     // 1: two 16-row blocks of A (M <= 32)
};
constexpr int kNumSkinnyTiles = sizeof(kSkinnyTiles) / sizeof(kSkinnyTiles[0]);

hipError_t launch_naive(const GemmArgs& g, hipStream_t stream);
// ops: bit 0 = A stored transposed, bit 1 = B stored transposed.  vec == false
// (4-byte lanes) only for the tiles marked `narrow`.
hipError_t launch_mfma(int tile, bool vec, int ops, const GemmArgs& g, int splits, hipStream_t stream);
hipError_t launch_valu(int tile, bool vec, const GemmArgs& g, int splits, hipStream_t stream);
hipError_t launch_skinny(int tile, bool vec, int ops, const GemmArgs& g, int splits, hipStream_t stream);

// C[i][j] = sum_{z=0}^{splits-1} W[z*w_slice + i*ldw + j], summed in order z = 0, 1, ...
hipError_t launch_splitk_reduce(const float* W, int64_t ldw, int64_t w_slice, int splits,
                                float* C, int64_t ldc, int32_t M, int32_t N, float alpha, float beta,
                                hipStream_t stream);

// Stream-K fix-up: for each stream-K tile split over several workgroups, sum
// its partial slots in workgroup order and write the tile to C.
hipError_t launch_streamk_fixup(const GemmArgs& g, int bm, int bn, int sk_tiles, hipStream_t stream);

// C[i][j] = +0.0 for i < M, j < N (the empty sum, K == 0).
// C = beta * C (C not read when beta == 0): the whole product when alpha == 0 or K == 0.
hipError_t launch_scale(float* C, int64_t ldc, int32_t M, int32_t N, float beta, hipStream_t stream);
// The read-rate probe: reads x[0 .. n) once (n % 4 == 0, x 16-byte aligned)
// and writes kReadGrid per-workgroup sums to partial.
constexpr int kReadGrid = 4096;
hipError_t launch_read_probe(const float* x, int64_t n, float* partial, hipStream_t stream);
// The FMA-rate probe: `workgroups` x 256 lanes, each 16 x 8 x iters scalar
// FP32 FMAs; one float per lane to out.
constexpr int kFmaPerLanePerIter = 16 * 8;
hipError_t launch_fma_probe(int iters, int workgroups, float* out, hipStream_t stream);

// dst (rows_p x cols_p, leading dimension ldd >= cols_p, both multiples of 4,
// 16-byte aligned) = src (rows x cols, leading dimension ld) zero-padded.
// One operand to pack: rows x cols at src (leading dimension ld) into the
// zero-padded rows_p x cols_p copy at dst (leading dimension ldd).
struct PackJob {
    const float* src;
    int64_t ld;
    int32_t rows, cols;
    float* dst;
    int64_t ldd;
    int32_t rows_p, cols_p;
    // set by launch_pack: workgroups of this job, the 16-byte groups each
    // moves, and how each covers its part (whole rows per workgroup when a
    // row has at most that many groups, else pieces per row)
    int64_t blocks;
    int32_t groups, rows_per_block, pieces_per_row;
};
struct PackJobs {
    PackJob job[2];
    int32_t count;   // 1 or 2, packed in one launch
};
hipError_t launch_pack(const PackJobs& jobs, hipStream_t stream);

// Sixteen zero bytes in device memory, defined once per kernel source.  A
// masked-off load (outside the matrix, or past the end of a K slice) reads
// from here instead of being followed by a select, so no instruction waits on
// the load until its data is consumed.  The block is externally visible and
// never written, so the compiler cannot fold the loads into selects.
#define SGEMM_DEFINE_ZERO_BLOCK(name) __device__ __attribute__((aligned(16))) float name[4] = {0.f, 0.f, 0.f, 0.f}

}  // namespace sgemm_impl
