// Internal interface between the host dispatcher and the gfx950 kernels.
// Not installed; the public C interface is include/sgemm.h.
#pragma once

#include <cstdint>
#include <hip/hip_runtime.h>

namespace sgemm_impl {

// One launch of a tiled product kernel.  The kernel computes, for every
// output tile (tm, tn) and slice z < gridDim.z,
//   Cz[i][j] = sum_{k in [z*k_chunk, min(K, (z+1)*k_chunk))} A[i][k] B[k][j]
// with Cz = C + z * c_slice, and writes it (overwrite) where i < M, j < N.
struct GemmArgs {
    const float* A;
    const float* B;
    float* C;
    int32_t M, N, K;
    int32_t k_chunk;    // K elements per slice (a multiple of the tile's BK)
    int64_t lda, ldb, ldc;
    int64_t c_slice;    // elements between consecutive slices' outputs
    int32_t tiles_m, tiles_n;
};

// Tile shapes of each path.  The kernels are instantiated for exactly these;
// the dispatcher and sgemm_tile_info read the same table.
struct TileShape {
    int bm, bn, bk;
    int waves_m, waves_n;   // waves per workgroup along M and N
    int waves_per_simd;     // occupancy the register budget is sized for
};

constexpr TileShape kMfmaTiles[] = {
    {256, 128, 16, 2, 2, 2},   // 0: large products
    {128, 256, 16, 2, 2, 2},   // 1: large products, wide N
    {128, 128, 16, 2, 2, 2},   // 2: medium
    {256, 256, 16, 2, 2, 1},   // 3: one workgroup per CU
    {64, 64, 16, 2, 2, 4},     // 4: small products / split-K
    {128, 128, 32, 2, 2, 2},   // 5: medium, deeper K-step
};
constexpr int kNumMfmaTiles = sizeof(kMfmaTiles) / sizeof(kMfmaTiles[0]);

constexpr TileShape kValuTiles[] = {
    {128, 128, 8, 2, 2, 2},    // 0: 8x8 outputs per lane, 8x8 lanes per wave
    {128, 128, 16, 2, 2, 2},   // 1: same, deeper K-step
};
constexpr int kNumValuTiles = sizeof(kValuTiles) / sizeof(kValuTiles[0]);

// The one-thread-per-output kernel: a 64 x 4 thread block.
constexpr TileShape kNaiveTiles[] = {{4, 64, 1, 1, 1, 4}};
constexpr int kNumNaiveTiles = 1;

// Skinny products (M <= 16): a workgroup owns 16 rows x 64 columns and one K
// slice, split over its 4 waves; K slices are multiples of bk = 64.
constexpr TileShape kSkinnyTiles[] = {{16, 64, 64, 1, 4, 2}};
constexpr int kNumSkinnyTiles = 1;

hipError_t launch_naive(const GemmArgs& g, hipStream_t stream);
hipError_t launch_mfma(int tile, bool vec, const GemmArgs& g, int splits, hipStream_t stream);
hipError_t launch_valu(int tile, bool vec, const GemmArgs& g, int splits, hipStream_t stream);
hipError_t launch_skinny(int tile, bool vec, const GemmArgs& g, int splits, hipStream_t stream);

// C[i][j] = sum_{z=0}^{splits-1} W[z*w_slice + i*ldw + j], summed in order z = 0, 1, ...
hipError_t launch_splitk_reduce(const float* W, int64_t ldw, int64_t w_slice, int splits,
                                float* C, int64_t ldc, int32_t M, int32_t N, hipStream_t stream);

// C[i][j] = +0.0 for i < M, j < N (the empty sum, K == 0).
hipError_t launch_fill_zero(float* C, int64_t ldc, int32_t M, int32_t N, hipStream_t stream);

}  // namespace sgemm_impl
