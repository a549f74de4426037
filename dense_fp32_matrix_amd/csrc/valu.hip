// FP32 SGEMM on the vector ALU: per-lane register tiles updated by rank-1
// (outer-product) steps.
//
// This is the CUDA-core design of "GEMM from naive to tiled" (sections 五 and
// 六: 8x8 outputs per thread, A stored transposed in shared memory, 16-byte
// fragment reads, register prefetch with two shared buffers and one barrier
// per K-step) and of "SGEMM 纯 CUDA 优化总结" (ex8/ex9), re-laid for wave64:
//   * workgroup = 256 lanes = 4 waves in a 2 x 2 grid; tile 128 x 128 x BK;
//   * wave tile 64 x 64; the 64 lanes form an 8 x 8 grid (square, so both
//     operands are reused in two dimensions -- the 4x8-over-1x32 argument of
//     "SGEMM 纯 CUDA 优化总结", Q8, at 64 lanes);
//   * lane (lr, lc) owns rows {4lr..4lr+3} u {32+4lr..32+4lr+3} and the same
//     pattern of columns with lc: each of its A and B fragments is two
//     16-byte runs 32 floats apart, so the 8 lanes that read different runs
//     of one operand cover 128 consecutive bytes (the split-column fix of
//     section 九.2) and the other 56 lanes read the same addresses again;
//   * per k each lane issues 4 16-byte LDS reads and 64 FP32 FMAs,
//     acc[i][j] += a[i] * b[j] (the outer-product update, section 五.1).
// Each k-step's FMAs are scalar v_fmac_f32 (packed FP32 is not used).  On
// gfx950 these issue at the full FP32 vector rate when at least two waves
// per SIMD have FMAs ready (measured with the library's FMA-rate probe: 69
// TFLOP/s with one wave per SIMD, 123 with two, 145-150 with four or more);
// this kernel's 214 VGPRs allow two, so a wave waiting on LDS or at the
// barrier halves its SIMD's rate, which is where most of the gap to the
// peak goes.  Four waves per SIMD would need at most 128 VGPRs: the 64
// accumulators, the fragments and the prefetch registers then spill.
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace sgemm_impl {

SGEMM_DEFINE_ZERO_BLOCK(kZeroValu);

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int BM, int BN, int BK, bool VEC>
struct ValuCfg {
    static constexpr int T = 256;
    static constexpr int LDA_S = BM + 4;     // As_t[BK][BM + 4]: A transposed (k-major)
    static constexpr int LDB_S = BN + 4;     // Bs[BK][BN + 4]
    static constexpr int A_STAGE = BK * LDA_S;
    static constexpr int B_STAGE = BK * LDB_S;
    static constexpr int STAGE = A_STAGE + B_STAGE;
    static constexpr int A_PER = BM * BK / T;
    static constexpr int B_PER = BK * BN / T;
    static_assert(BM == 128 && BN == 128, "lane mapping assumes a 128 x 128 tile");
    static_assert(A_PER * T == BM * BK && B_PER * T == BK * BN, "loader must cover the tile");
    static_assert(!VEC || (A_PER % 4 == 0 && B_PER % 4 == 0), "vector loader must cover the tile");
};

template <int BM, int BN, int BK, bool VEC>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void valu_gemm_kernel(GemmArgs g) {
    using P = ValuCfg<BM, BN, BK, VEC>;
    __shared__ __attribute__((aligned(16))) float smem[2 * P::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1;
    const int wn = wave & 1;
    const int lr = lane >> 3;
    const int lc = lane & 7;

    int tm, tn;
    tile_coords(blockIdx.x, g.tiles_m, g.tiles_n, g.group_m, &tm, &tn);
    const int m0 = tm * BM;
    const int n0 = tn * BN;

    const int kb = blockIdx.z * g.k_chunk;
    const int ke = min(g.K, kb + g.k_chunk);
    const int steps = (ke - kb + BK - 1) / BK;

    constexpr int AN = VEC ? P::A_PER / 4 : P::A_PER;
    constexpr int BNL = VEC ? P::B_PER / 4 : P::B_PER;
    constexpr int W = VEC ? 4 : 1;
    constexpr int A_COLS = BK / W;
    constexpr int B_COLS = BN / W;

    int64_t a_off[AN];
    int a_kc[AN];
    bool a_rok[AN];
    int a_lds[AN];      // As_t[kc][row]; the W elements go to rows kc..kc+W-1 of the transposed tile
#pragma unroll
    for (int r = 0; r < AN; ++r) {
        const int q = tid + r * P::T;
        const int row = q / A_COLS;
        const int col = (q % A_COLS) * W;
        const int gm = m0 + row;
        a_rok[r] = gm < g.M;
        a_off[r] = (int64_t)(a_rok[r] ? gm : 0) * g.lda + col;
        a_kc[r] = col;
        a_lds[r] = col * P::LDA_S + row;
    }
    int64_t b_off[BNL];
    int b_kr[BNL];
    bool b_cok[BNL];
    int b_lds[BNL];
#pragma unroll
    for (int r = 0; r < BNL; ++r) {
        const int q = tid + r * P::T;
        const int row = q / B_COLS;
        const int col = (q % B_COLS) * W;
        const int gn = n0 + col;
        b_cok[r] = gn < g.N;
        b_off[r] = (int64_t)row * g.ldb + (b_cok[r] ? gn : 0);
        b_kr[r] = row;
        b_lds[r] = P::A_STAGE + row * P::LDB_S + col;
    }

    f32x4 va[VEC ? AN : 1], vb[VEC ? BNL : 1];
    float sa[VEC ? 1 : AN], sb[VEC ? 1 : BNL];

    // masked-off elements load from kZeroValu (no select after the load)
    auto load = [&](int k0) {
#pragma unroll
        for (int r = 0; r < AN; ++r) {
            const bool ok = a_rok[r] && (k0 + a_kc[r] < ke);
            const float* p = ok ? g.A + a_off[r] + k0 : kZeroValu;
            if constexpr (VEC) va[r] = *reinterpret_cast<const f32x4*>(p);
            else sa[r] = *p;
        }
#pragma unroll
        for (int r = 0; r < BNL; ++r) {
            const bool ok = b_cok[r] && (k0 + b_kr[r] < ke);
            const float* p = ok ? g.B + b_off[r] + (int64_t)k0 * g.ldb : kZeroValu;
            if constexpr (VEC) vb[r] = *reinterpret_cast<const f32x4*>(p);
            else sb[r] = *p;
        }
    };
    auto store = [&](int buf) {
        float* s = smem + buf * P::STAGE;
#pragma unroll
        for (int r = 0; r < AN; ++r) {
            if constexpr (VEC) {
#pragma unroll
                for (int c = 0; c < 4; ++c) s[a_lds[r] + c * P::LDA_S] = va[r][c];
            } else {
                s[a_lds[r]] = sa[r];
            }
        }
#pragma unroll
        for (int r = 0; r < BNL; ++r) {
            if constexpr (VEC) *reinterpret_cast<f32x4*>(s + b_lds[r]) = vb[r];
            else s[b_lds[r]] = sb[r];
        }
    };

    float acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;

    const int a_frag = wm * 64 + 4 * lr;                // + 32 for the second run
    const int b_frag = P::A_STAGE + wn * 64 + 4 * lc;

    auto compute = [&](int buf) {
        const float* s = smem + buf * P::STAGE;
#pragma unroll
        for (int k = 0; k < BK; ++k) {
            const f32x4 a0 = *reinterpret_cast<const f32x4*>(s + k * P::LDA_S + a_frag);
            const f32x4 a1 = *reinterpret_cast<const f32x4*>(s + k * P::LDA_S + a_frag + 32);
            const f32x4 b0 = *reinterpret_cast<const f32x4*>(s + k * P::LDB_S + b_frag);
            const f32x4 b1 = *reinterpret_cast<const f32x4*>(s + k * P::LDB_S + b_frag + 32);
            float a[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            float b[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        }
    };

    if (steps > 0) {
        load(kb);
        store(0);
        __syncthreads();
        for (int s = 0; s < steps; ++s) {
            const bool more = s + 1 < steps;
            if (more) load(kb + (s + 1) * BK);
            compute(s & 1);
            if (more) store((s & 1) ^ 1);
            __syncthreads();
        }
    }

    float* C = g.C + (int64_t)blockIdx.z * g.c_slice;
    const float alpha = g.c_slice ? 1.f : g.alpha;    // slices are raw partial sums
    const float beta = g.c_slice ? 0.f : g.beta;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int gi = m0 + wm * 64 + (i < 4 ? 4 * lr + i : 32 + 4 * lr + (i - 4));
        if (gi >= g.M) continue;
        float* crow = C + (int64_t)gi * g.ldc;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int gj = n0 + wn * 64 + (j < 4 ? 4 * lc + j : 32 + 4 * lc + (j - 4));
            if (gj < g.N) store_scaled(crow + gj, acc[i][j], alpha, beta);
        }
    }
}

template <int BM, int BN, int BK>
hipError_t launch_one(bool vec, const GemmArgs& g, int splits, hipStream_t stream) {
    dim3 grid((unsigned)((int64_t)g.tiles_m * g.tiles_n), 1, (unsigned)splits);
    if (vec)
        hipLaunchKernelGGL((valu_gemm_kernel<BM, BN, BK, true>), grid, dim3(256), 0, stream, g);
    else
        hipLaunchKernelGGL((valu_gemm_kernel<BM, BN, BK, false>), grid, dim3(256), 0, stream, g);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_valu(int tile, bool vec, const GemmArgs& g, int splits, hipStream_t stream) {
    switch (tile) {
        case 0:
            return launch_one<kValuTiles[0].bm, kValuTiles[0].bn, kValuTiles[0].bk>(vec, g, splits, stream);
        default:
            return hipErrorInvalidValue;
    }
}
static_assert(kNumValuTiles == 1, "launch_valu covers every VALU tile");

}  // namespace sgemm_impl
