// Skinny SGEMM (M <= 32) on FP32 matrix cores.
//
// With few rows of A every element of B is used at most M times, so the
// product is bound by reading B once from HBM, not by arithmetic -- the
// GEMV / decode regime of "GEMM from naive to tiled", section 十.2, and the
// GEMV example of "如何让计算受限问题真正达到计算受限", section 7.  The kernel
// is therefore built to stream B with deep memory-level parallelism and no
// LDS staging:
//   * a wave owns 64 columns of C and a quarter of the workgroup's K range;
//     a workgroup (4 waves) owns a 64-column strip and one K slice, whose
//     partial sums across workgroups the split-K reduction adds, or (stream-K)
//     an equal share of all (strip, K-step) units, partial strips being added
//     by the stream-K fix-up;
//   * lane l = 16 * kk + jj loads B[k][n + 4jj .. 4jj+3] as one 16-byte read
//     for k = k0 + 4kk + t (t = 0..3): 16 lanes cover a 256-byte run of a row;
//   * component c of that vector is the B operand of v_mfma_f32_16x16x4_f32
//     number c, whose 16 output columns are n + 4j + c (j = 0..15): the four
//     instructions together cover the 64 columns, and lane jj of each stores
//     its 4 outputs of a row as 4 consecutive columns;
//   * A (M x K, at most 16 MT rows) is read from L2 as 16-byte runs of one
//     row; with two 16-row blocks (MT = 2, M <= 32) each B vector feeds the
//     MFMAs of both blocks, so B is still read once;
//   * B stored transposed (N x K, k-contiguous, the weight layout of a
//     linear layer): lane l = 16 * kk + jj instead loads row n + 16g + jj of
//     the stored B at k = k0 + 4kk .. 4kk+3 for each column group g = 0..3,
//     and component t of that vector is the B operand of MFMA (t, g): the
//     four components are the MFMA's k = 4kk + t, the 16 lanes jj its 16
//     columns; MFMA (t, g) accumulates columns n + 16g + j.  A stored
//     transposed (K x M) is read as single floats (A is small and cached);
//   * masked-off elements (rows >= M, columns >= N, k past the slice) load
//     from a 16-byte zero block, so loads are never followed by a select;
//   * two register stages of 2 k-groups of 16 each keep 2 x 2 x 4 = 16 16-byte
//     B loads per lane in flight while the previous stage is contracted
//     (measured: 4 groups per stage are 2-4 % slower with one row block and
//     spill with two, 9-14 % slower; 3 are 3-12 % slower and 1 is 6 % slower
//     with two row blocks);
//   * the waves' partial tiles are summed through LDS in wave order.
// Operand layout of v_mfma_f32_16x16x4_f32 (wave64):
//   A: lane l holds A[i = l % 16][kk = l / 16];  B: lane l holds B[kk = l / 16][j = l % 16];
//   D: lane l, register r holds D[4 * (l / 16) + r][l % 16].
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace sgemm_impl {

SGEMM_DEFINE_ZERO_BLOCK(kZeroSkinny);

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kStageK = 64;                // K elements of one stream-K unit
constexpr int kGroups = 2;                 // k-groups of 16 per register stage
constexpr int kRegK = 16 * kGroups;        // K elements per register stage per wave

// One segment: the 64-column strip of B starting at column n_w over
// k in [kb, ke), split in K across the waves (quarters rounded up to 16),
// contracted with all rows of A, summed over the waves in wave order, and
// written as alpha * sum + beta * out to out[i * ldo + c] for rows i < M and
// strip columns c < col_lim.  MT: 16-row blocks of A (M <= 16 MT); every B
// vector feeds MT x 4 MFMAs.
// OPS: bit 0 = A stored transposed (K x M), bit 1 = B stored transposed (N x K).
template <bool VEC, int WAVES, int MT, int OPS>
__device__ __forceinline__ void skinny_segment(const GemmArgs& g, float (&red)[WAVES][16 * MT][64], int n_w,
                                               int kb, int ke, float* out, int64_t ldo, int col_lim, float alpha,
                                               float beta) {
    constexpr bool TA = (OPS & 1) != 0;
    constexpr bool TB = (OPS & 2) != 0;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int jj = lane & 15;
    const int kk = lane >> 4;

    const int kq = ((ke - kb + WAVES - 1) / WAVES + 15) / 16 * 16;
    const int wkb = min(ke, kb + wave * kq);
    const int wke = min(ke, wkb + kq);

    // this lane's row of A in each row block: element k of it at a_row[b][k * a_step]
    bool a_row_ok[MT];
    const float* a_row[MT];
    const int64_t a_step = TA ? g.lda : 1;
#pragma unroll
    for (int b = 0; b < MT; ++b) {
        a_row_ok[b] = 16 * b + jj < g.M;
        const int64_t row = a_row_ok[b] ? 16 * b + jj : 0;
        a_row[b] = g.A + (TA ? row : row * g.lda);
    }
    const int ncol = n_w + 4 * jj;               // B as stored: first of this lane's 4 columns

    static_assert(MT == 1 || MT == 2, "one or two row blocks");
    f32x4 ra[2][MT][kGroups];
    f32x4 rb[2][kGroups][4];

    auto load_stage = [&](int buf, int k0) {
#pragma unroll
        for (int gi = 0; gi < kGroups; ++gi) {
            // this lane's 4 k's; with B transposed, a lane's two k-groups are
            // adjacent, so the 4 lanes of a column read 128 contiguous bytes
            // of its row per stage (A follows the same k order)
            const int ka = TB ? k0 + 8 * kk + 4 * gi : k0 + 16 * gi + 4 * kk;
#pragma unroll
            for (int b = 0; b < MT; ++b) {
                if constexpr (VEC && !TA) {
                    const bool ok = a_row_ok[b] && ka < wke;
                    ra[buf][b][gi] = *reinterpret_cast<const f32x4*>(ok ? a_row[b] + ka : kZeroSkinny);
                } else {
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const bool ok = a_row_ok[b] && ka + t < wke;
                        ra[buf][b][gi][t] = *(ok ? a_row[b] + (int64_t)(ka + t) * a_step : kZeroSkinny);
                    }
                }
            }
            if constexpr (TB) {
                // rb[buf][gi][q]: stored row n_w + 16q + jj of B, k = ka .. ka + 3
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int n = n_w + 16 * q + jj;
                    const float* bcol = g.B + (int64_t)n * g.ldb;
                    if constexpr (VEC) {
                        const bool ok = n < g.N && ka < wke;
                        rb[buf][gi][q] = *reinterpret_cast<const f32x4*>(ok ? bcol + ka : kZeroSkinny);
                    } else {
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            const bool ok = n < g.N && ka + t < wke;
                            rb[buf][gi][q][t] = *(ok ? bcol + ka + t : kZeroSkinny);
                        }
                    }
                }
            } else {
                // rb[buf][gi][q]: row k = ka + q of B, this lane's 4 columns
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int k = ka + t;
                    const float* brow = g.B + (int64_t)k * g.ldb;
                    if constexpr (VEC) {
                        const bool ok = k < wke && ncol < g.N;
                        rb[buf][gi][t] = *reinterpret_cast<const f32x4*>(ok ? brow + ncol : kZeroSkinny);
                    } else {
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const bool ok = k < wke && ncol + c < g.N;
                            rb[buf][gi][t][c] = *(ok ? brow + ncol + c : kZeroSkinny);
                        }
                    }
                }
            }
        }
    };

    f32x4 acc[MT][4];
#pragma unroll
    for (int b = 0; b < MT; ++b)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[b][c] = f32x4{0.f, 0.f, 0.f, 0.f};

    // MFMA (t, c): A component t (k = 4kk + t); as stored, B vector t
    // component c (columns 4j + c) into acc[c]; B transposed, B vector c
    // component t (columns 16c + j) into acc[c]
    auto compute_stage = [&](int buf) {
#pragma unroll
        for (int gi = 0; gi < kGroups; ++gi)
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int b = 0; b < MT; ++b)
                        acc[b][c] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                            ra[buf][b][gi][t], TB ? rb[buf][gi][c][t] : rb[buf][gi][t][c], acc[b][c], 0, 0, 0);
    };

    const int nst = (wke - wkb + kRegK - 1) / kRegK;
    if (nst > 0) {
        load_stage(0, wkb);
        int s = 0;
        for (; s + 2 <= nst; s += 2) {
            load_stage(1, wkb + (s + 1) * kRegK);
            compute_stage(0);
            if (s + 2 < nst) load_stage(0, wkb + (s + 2) * kRegK);
            compute_stage(1);
        }
        if (s < nst) compute_stage(0);
    }

    // wave partials -> LDS: row block b, MFMA c, register r is row 16b + 4kk + r,
    // column 4jj + c (B as stored) or 16c + jj (B transposed)
#pragma unroll
    for (int b = 0; b < MT; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if constexpr (TB) {
#pragma unroll
                for (int c = 0; c < 4; ++c) red[wave][16 * b + 4 * kk + r][16 * c + jj] = acc[b][c][r];
            } else {
                *reinterpret_cast<f32x4*>(&red[wave][16 * b + 4 * kk + r][4 * jj]) =
                    f32x4{acc[b][0][r], acc[b][1][r], acc[b][2][r], acc[b][3][r]};
            }
        }
    __syncthreads();

    // sum the wave partials in wave order and write rows < M, columns < col_lim
    // (16 MT rows x 16 groups of 4 columns)
    for (int e = tid; e < 16 * MT * 16; e += 64 * WAVES) {
        const int i = e >> 4;
        const int c4 = (e & 15) * 4;
        f32x4 s4 = *reinterpret_cast<const f32x4*>(&red[0][i][c4]);
#pragma unroll
        for (int w = 1; w < WAVES; ++w) s4 += *reinterpret_cast<const f32x4*>(&red[w][i][c4]);
        if (i < g.M) {
            float* crow = out + (int64_t)i * ldo;
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (c4 + c < col_lim) store_scaled(crow + c4 + c, s4[c], alpha, beta);
        }
    }
}

// Two work decompositions, as in the matrix-core kernel:
//  * one (strip, K slice) per workgroup (sk_iters == 0): strip blockIdx.x,
//    slice blockIdx.z; slices go to C + z * c_slice as raw partial sums;
//  * stream-K (sk_iters > 0): the (strip, 64-deep K-step) units, strip-major,
//    cut into equal ranges of sk_ipw units, one per workgroup, so that every
//    CU streams the same share of B whatever the strip count.  A segment
//    covering a whole strip writes C; a partial strip goes to the
//    workgroup's slot 2 * wg + (0 for its first segment, 1 afterwards), and
//    the stream-K fix-up kernel sums each strip's slots in workgroup order.
//    Strip j of the unit order is tile_coords' column of tile j, as the
//    fix-up kernel maps it.
template <bool VEC, int WAVES, int MT, int OPS>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WAVES, 64 * WAVES), amdgpu_waves_per_eu(2, 2)))
void skinny_gemm_kernel(GemmArgs g) {
    __shared__ __attribute__((aligned(16))) float red[WAVES][16 * MT][64];
    int64_t it = (int64_t)blockIdx.x * g.sk_ipw;
    const int64_t it_end = min(it + g.sk_ipw, g.sk_iters);
    bool first = true;
    int which = 0;
    while (true) {
        int n_w, kb, ke, col_lim;
        float* out;
        int64_t ldo, step = 0;
        float alpha, beta;
        if (g.sk_iters == 0) {
            if (!first) break;
            n_w = blockIdx.x * 64;
            kb = blockIdx.z * g.k_chunk;
            ke = min(g.K, kb + g.k_chunk);
            out = g.C + (int64_t)blockIdx.z * g.c_slice + n_w;
            ldo = g.ldc;
            col_lim = g.N - n_w;
            alpha = g.c_slice ? 1.f : g.alpha;    // slices are raw partial sums
            beta = g.c_slice ? 0.f : g.beta;
        } else {
            if (it >= it_end) break;
            const int j = (int)(it / g.k_steps);
            const int q0 = (int)(it - (int64_t)j * g.k_steps);
            const int q1 = (int)min<int64_t>(g.k_steps, q0 + (it_end - it));
            int tm, tn;
            tile_coords(j, 1, g.tiles_n, g.group_m, &tm, &tn);
            n_w = tn * 64;
            kb = q0 * kStageK;
            ke = min(g.K, q1 * kStageK);
            if (q0 == 0 && q1 == g.k_steps) {
                out = g.C + n_w;
                ldo = g.ldc;
                col_lim = g.N - n_w;
                alpha = g.alpha;
                beta = g.beta;
            } else {
                out = g.ws + (int64_t)(2 * blockIdx.x + which) * (16 * MT * 64);
                ldo = 64;
                col_lim = 64;
                alpha = 1.f;
                beta = 0.f;
            }
            which = 1;
            step = q1 - q0;
        }
        if (!first) __syncthreads();       // the previous segment is done with the LDS
        first = false;
        skinny_segment<VEC, WAVES, MT, OPS>(g, red, n_w, kb, ke, out, ldo, col_lim, alpha, beta);
        it += step;
    }
}

template <int WAVES, int MT, int OPS>
hipError_t launch_ops(bool vec, const GemmArgs& g, int splits, hipStream_t stream) {
    dim3 grid(g.sk_iters > 0 ? (unsigned)g.sk_grid : (unsigned)g.tiles_n, 1, g.sk_iters > 0 ? 1u : (unsigned)splits);
    if (vec)
        hipLaunchKernelGGL((skinny_gemm_kernel<true, WAVES, MT, OPS>), grid, dim3(64 * WAVES), 0, stream, g);
    else
        hipLaunchKernelGGL((skinny_gemm_kernel<false, WAVES, MT, OPS>), grid, dim3(64 * WAVES), 0, stream, g);
    return hipGetLastError();
}

template <int WAVES, int MT>
hipError_t launch_waves(bool vec, int ops, const GemmArgs& g, int splits, hipStream_t stream) {
    switch (ops) {
        case 0: return launch_ops<WAVES, MT, 0>(vec, g, splits, stream);
        case 1: return launch_ops<WAVES, MT, 1>(vec, g, splits, stream);
        case 2: return launch_ops<WAVES, MT, 2>(vec, g, splits, stream);
        case 3: return launch_ops<WAVES, MT, 3>(vec, g, splits, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_skinny(int tile, bool vec, int ops, const GemmArgs& g, int splits, hipStream_t stream) {
    switch (tile) {
        case 0: return launch_waves<kSkinnyTiles[0].waves_n, kSkinnyTiles[0].bm / 16>(vec, ops, g, splits, stream);
        case 1: return launch_waves<kSkinnyTiles[1].waves_n, kSkinnyTiles[1].bm / 16>(vec, ops, g, splits, stream);
        default: return hipErrorInvalidValue;
    }
}
static_assert(kNumSkinnyTiles == 2, "launch_skinny covers every skinny tile");

}  // namespace sgemm_impl
