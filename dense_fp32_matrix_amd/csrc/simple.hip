// Small kernels: the one-thread-per-output product, the split-K reduction,
// the stream-K fix-up, operand packing, the C = beta * C scaling used when
// alpha == 0 or K == 0, and the read-rate and FMA-rate probes.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "kernels.hpp"

namespace sgemm_impl {

namespace {

// One thread per C element, operands read straight from global memory
// ("GEMM from naive to tiled", section 三; the first rung of "SGEMM 纯 CUDA
// 优化总结").  threadIdx.x runs along N so a wave reads 64 consecutive B
// floats and one broadcast A float per k.  The sum runs in ascending k with
// one rounding per fused multiply-add.  Kept as the bring-up and
// cross-check kernel, not a performance path.  Operands stored transposed
// only change the strides: op(A)[i][k] steps by 1 in k (lda when
// transposed), op(B)[k][j] by ldb in k (1 when transposed).
constexpr int kNaiveX = 64;
constexpr int kNaiveY = 4;

__global__ __launch_bounds__(kNaiveX * kNaiveY)
void naive_gemm_kernel(GemmArgs g) {
    const int64_t tiles_n = g.tiles_n;
    const int64_t t = blockIdx.x;
    const int64_t i = (t / tiles_n) * kNaiveY + threadIdx.y;
    const int64_t j = (t % tiles_n) * kNaiveX + threadIdx.x;
    if (i >= g.M || j >= g.N) return;
    const float* a = g.trans_a ? g.A + i : g.A + i * g.lda;
    const int64_t sa = g.trans_a ? g.lda : 1;
    const float* b = g.trans_b ? g.B + j * g.ldb : g.B + j;
    const int64_t sb = g.trans_b ? 1 : g.ldb;
    float acc = 0.f;
    for (int k = 0; k < g.K; ++k) acc = __builtin_fmaf(a[k * sa], b[k * sb], acc);
    store_scaled(g.C + i * g.ldc + j, acc, g.alpha, g.beta);
}

// Deterministic split-K reduction: each output is the sum of the slices'
// partial products taken in slice order (the workspace variant of "GEMM from
// naive to tiled", section 十.1, which, unlike atomic adds, always yields the
// same bits).  The workspace rows are padded to a multiple of 4 floats and
// 16-byte aligned, so each thread reads 4 consecutive outputs of every slice
// with one 16-byte load.
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256)
void splitk_reduce_kernel(const float* __restrict__ W, int64_t ldw, int64_t w_slice, int splits,
                          float* __restrict__ C, int64_t ldc, int32_t M, int32_t N, float alpha, float beta) {
    const int64_t groups_per_row = ldw / 4;
    const int64_t total = (int64_t)M * groups_per_row;
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < total;
         v += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = v / groups_per_row;
        const int64_t j = (v - i * groups_per_row) * 4;
        if (j >= N) continue;
        const float* w = W + i * ldw + j;
        f32x4 s = *reinterpret_cast<const f32x4*>(w);
        for (int z = 1; z < splits; ++z) s += *reinterpret_cast<const f32x4*>(w + z * w_slice);
        float* c = C + i * ldc + j;
        store_scaled(c, s[0], alpha, beta);
        if (j + 1 < N) store_scaled(c + 1, s[1], alpha, beta);
        if (j + 2 < N) store_scaled(c + 2, s[2], alpha, beta);
        if (j + 3 < N) store_scaled(c + 3, s[3], alpha, beta);
    }
}

__global__ __launch_bounds__(256)
void scale_kernel(float* __restrict__ C, int64_t ldc, int32_t M, int32_t N, float beta) {
    const int64_t total = (int64_t)M * N;
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < total;
         v += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = v / N;
        const int64_t j = v - i * N;
        float* p = C + i * ldc + j;
        *p = beta != 0.f ? beta * *p : 0.f;
    }
}

// Packing: the rows x cols matrix src (leading dimension ld, any 4-byte
// alignment) is copied into the rows_p x cols_p row-major dst (leading
// dimension ldd >= cols_p, both multiples of 4; dst 16-byte aligned; columns
// from cols_p to ldd are left alone, nothing reads them), with zeros in the
// padding rows and columns.  The copy is exact, and the zeros only add +0
// terms to the product, so the matrix kernel's 16-byte loaders can then run
// on operands that were not aligned.  One launch packs both operands when
// both need it: workgroups [0, job[0].blocks) copy the first, the rest the
// second, so no workgroup is idle whatever the two shapes.  A workgroup
// moves `groups` 16-byte groups (256 to kPackGroups, fewer for small copies
// so that they still spread over every CU): whole rows when a row holds at
// most that many (narrow rows: one workgroup copies several), else one piece
// of a row.  Each thread first loads all its groups (up to kPackU, 4 loads
// each, the source having no alignment), then stores them.
constexpr int kPackU = 4;
constexpr int kPackGroups = 256 * kPackU;
constexpr int64_t kPackMinBlocks = 2048;

__global__ __launch_bounds__(256)
void pack_kernel(PackJobs jobs) {
    const bool second = (int64_t)blockIdx.x >= jobs.job[0].blocks;
    const PackJob& j = jobs.job[second ? 1 : 0];
    const int64_t b = (int64_t)blockIdx.x - (second ? jobs.job[0].blocks : 0);
    const int32_t cols4 = j.cols_p / 4;
    int32_t row[kPackU], c4[kPackU];
    if (j.pieces_per_row > 0) {
        // one piece of one row: groups [p * groups, (p + 1) * groups)
        const int32_t r = (int32_t)(b / j.pieces_per_row);
        const int32_t c0 = (int32_t)(b - (int64_t)r * j.pieces_per_row) * j.groups;
#pragma unroll
        for (int u = 0; u < kPackU; ++u) {
            const int32_t l = u * 256 + (int32_t)threadIdx.x;
            row[u] = l < j.groups ? r : j.rows_p;                   // past the piece: nothing
            c4[u] = c0 + l;
        }
    } else {
        // rows_per_block whole rows, flattened
        const int32_t r0 = (int32_t)b * j.rows_per_block;
#pragma unroll
        for (int u = 0; u < kPackU; ++u) {
            const int32_t l = u * 256 + (int32_t)threadIdx.x;
            const int32_t rl = l / cols4;
            row[u] = rl < j.rows_per_block ? r0 + rl : j.rows_p;     // past the block's rows: nothing
            c4[u] = l - rl * cols4;
        }
    }
    float4 v[kPackU];
#pragma unroll
    for (int u = 0; u < kPackU; ++u) {
        v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (row[u] < j.rows && c4[u] < cols4) {
            const float* s = j.src + (int64_t)row[u] * j.ld + 4 * c4[u];
            const int32_t left = j.cols - 4 * c4[u];
            if (left > 0) v[u].x = s[0];
            if (left > 1) v[u].y = s[1];
            if (left > 2) v[u].z = s[2];
            if (left > 3) v[u].w = s[3];
        }
    }
#pragma unroll
    for (int u = 0; u < kPackU; ++u)
        if (row[u] < j.rows_p && c4[u] < cols4)
            *reinterpret_cast<float4*>(j.dst + (int64_t)row[u] * j.ldd + 4 * c4[u]) = v[u];
}

// Stream-K fix-up (see the stream-K decomposition of the MFMA kernel):
// workgroup (j, part) handles elements [part * 1024 U, (part + 1) * 1024 U)
// of stream-K tile j, U 16-byte groups per thread; the loop over the
// contributing slots is unrolled so that several loads per thread are in
// flight (the sum itself stays in slot order).  U = 4 when a tile has few
// contributors, U = 1 (four times the workgroups) when it has many.  A tile
// whose K-steps fall in one workgroup's range was written whole; otherwise
// its partial slots, from workgroups w0..w1 in that order, are summed and the
// tile is written to C.
constexpr bool fixup_chunks_fit() {
    for (const TileShape& t : kMfmaTiles)
        if ((t.bm * t.bn) % 4096 != 0) return false;
    return true;
}
static_assert(fixup_chunks_fit(), "every MFMA tile splits into whole fix-up chunks");

template <int U>
__global__ __launch_bounds__(256)
void streamk_fixup_kernel(GemmArgs g, int bm, int bn) {
    const int j = blockIdx.x;
    const int64_t first = (int64_t)j * g.k_steps;
    const int64_t last = first + g.k_steps - 1;
    const int w0 = (int)(first / g.sk_ipw);
    const int w1 = (int)(last / g.sk_ipw);
    if (w0 == w1) return;
    int tm, tn;
    tile_coords(g.dp_tiles + j, g.tiles_m, g.tiles_n, g.group_m, &tm, &tn);
    const int m0 = tm * bm;
    const int n0 = tn * bn;
    const int64_t slot = (int64_t)bm * bn;
    const bool vec_c = (g.ldc % 4 == 0) && (reinterpret_cast<uintptr_t>(g.C) % 16 == 0);
    f32x4 s[U];
    int es[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        es[u] = (int)blockIdx.y * (1024 * U) + 4 * ((int)threadIdx.x + 256 * u);
        s[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll 4
    for (int w = w0; w <= w1; ++w) {
        const int which = (int64_t)w * g.sk_ipw >= first ? 0 : 1;
        const float* src = g.ws + (int64_t)(2 * w + which) * slot;
#pragma unroll
        for (int u = 0; u < U; ++u) s[u] += *reinterpret_cast<const f32x4*>(src + es[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int i = es[u] / bn;
        const int c = es[u] - i * bn;
        if (m0 + i >= g.M || n0 + c >= g.N) continue;
        float* crow = g.C + (int64_t)(m0 + i) * g.ldc + n0 + c;
        if (vec_c && n0 + c + 3 < g.N) {
            f32x4 v = g.alpha * s[u];
            if (g.beta != 0.f) {
                const f32x4 old = *reinterpret_cast<const f32x4*>(crow);
#pragma unroll
                for (int q = 0; q < 4; ++q) v[q] = __builtin_fmaf(g.beta, old[q], v[q]);
            }
            *reinterpret_cast<f32x4*>(crow) = v;
        } else {
            store_scaled(crow, s[u][0], g.alpha, g.beta);
            if (n0 + c + 1 < g.N) store_scaled(crow + 1, s[u][1], g.alpha, g.beta);
            if (n0 + c + 2 < g.N) store_scaled(crow + 2, s[u][2], g.alpha, g.beta);
            if (n0 + c + 3 < g.N) store_scaled(crow + 3, s[u][3], g.alpha, g.beta);
        }
    }
}

// Read-rate probe, the yardstick of the streaming (skinny) path: the rate
// at which the chip reads a buffer it uses once, measured rather than taken
// from the data sheet (the "realistic machine model" of the GEMV example in
// "如何让计算受限问题真正达到计算受限", section 7).  x[0 .. 4 n4) is cut into
// kReadGrid contiguous chunks, one per workgroup (16 per CU), each read with
// 16-byte loads, kReadU in flight per lane (a wave's load covers 1 KB);
// each workgroup writes its sum to partial[blockIdx.x], so no load is dead.
// Of grid-stride and chunked reads with 1024-16384 workgroups and 4-16 loads
// in flight, chunks over 4096 workgroups with 4 loads read a 4 GiB buffer
// fastest (6.16 TB/s in the sweep, 6.2 in later runs; grid-stride at most 5.96).
constexpr int kReadU = 4;

__global__ __launch_bounds__(256)
void read_probe_kernel(const f32x4* __restrict__ x, int64_t n4, float* __restrict__ partial) {
    __shared__ float red[4];
    const int64_t per = (n4 + gridDim.x - 1) / gridDim.x;
    const int64_t b = (int64_t)blockIdx.x * per;
    const int64_t e = b + per < n4 ? b + per : n4;
    int64_t i = b + threadIdx.x;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (; i + (kReadU - 1) * 256 < e; i += kReadU * 256) {
        f32x4 v[kReadU];
#pragma unroll
        for (int u = 0; u < kReadU; ++u) v[u] = x[i + u * 256];
#pragma unroll
        for (int u = 0; u < kReadU; ++u) acc += v[u];
    }
    for (; i < e; i += 256) acc += x[i];
    float s = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    for (int off = 32; off > 0; off >>= 1) s += __shfl_down(s, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) partial[blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
}

// FMA-rate probe, the yardstick of the VALU path: each lane runs kFmaChains
// independent chains acc = x * y + acc of `iters` x 8 scalar FP32 FMAs
// (v_fmac_f32; packed FP32 is off in this build, as for the VALU kernel),
// x and y lane-dependent so nothing folds, and writes the chains' sum, so no
// FMA is dead.  With kFmaChains chains per lane and several waves per SIMD,
// issue, not the FMA latency, is the limit.
constexpr int kFmaChains = 16;

__global__ __launch_bounds__(256)
void fma_probe_kernel(int iters, float* __restrict__ out) {
    const float x = 1.0f + 1e-7f * (float)threadIdx.x;
    const float y = 1.0f - 1e-7f * (float)blockIdx.x;
    float acc[kFmaChains];
#pragma unroll
    for (int c = 0; c < kFmaChains; ++c) acc[c] = (float)c;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int c = 0; c < kFmaChains; ++c) acc[c] = __builtin_fmaf(x, y, acc[c]);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kFmaChains; ++c) s += acc[c];
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

unsigned grid_for(int64_t items, int64_t per_block) {
    int64_t blocks = (items + per_block - 1) / per_block;
    if (blocks > 256 * 16) blocks = 256 * 16;   // grid-stride beyond 16 workgroups per CU
    if (blocks < 1) blocks = 1;
    return (unsigned)blocks;
}

}  // namespace

hipError_t launch_naive(const GemmArgs& g, hipStream_t stream) {
    dim3 grid((unsigned)((int64_t)g.tiles_m * g.tiles_n));
    dim3 block(kNaiveX, kNaiveY);
    hipLaunchKernelGGL(naive_gemm_kernel, grid, block, 0, stream, g);
    return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float* W, int64_t ldw, int64_t w_slice, int splits,
                                float* C, int64_t ldc, int32_t M, int32_t N, float alpha, float beta,
                                hipStream_t stream) {
    const int64_t items = (int64_t)M * (ldw / 4);
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3(grid_for(items, 256)), dim3(256), 0, stream,
                       W, ldw, w_slice, splits, C, ldc, M, N, alpha, beta);
    return hipGetLastError();
}

hipError_t launch_streamk_fixup(const GemmArgs& g, int bm, int bn, int sk_tiles, hipStream_t stream) {
    // every tile shape holds a whole number of 1024-element chunks
    if ((bm * bn) % 1024 != 0) return hipErrorInvalidValue;
    // workgroups contributing to one tile (at most): many -> smaller chunks, more
    // workgroups; tiles that are no whole number of 4096-element chunks (the
    // skinny strips) take 1024-element chunks as well
    const int64_t contributors = (g.k_steps + g.sk_ipw - 1) / g.sk_ipw + 1;
    if (contributors > 8 || (bm * bn) % 4096 != 0)
        hipLaunchKernelGGL(streamk_fixup_kernel<1>, dim3((unsigned)sk_tiles, (unsigned)(bm * bn / 1024)), dim3(256),
                           0, stream, g, bm, bn);
    else
        hipLaunchKernelGGL(streamk_fixup_kernel<4>, dim3((unsigned)sk_tiles, (unsigned)(bm * bn / 4096)), dim3(256),
                           0, stream, g, bm, bn);
    return hipGetLastError();
}

hipError_t launch_pack(const PackJobs& in, hipStream_t stream) {
    if (in.count < 1 || in.count > 2) return hipErrorInvalidValue;
    PackJobs jobs = in;
    int64_t all_groups = 0;
    for (int i = 0; i < jobs.count; ++i) {
        const PackJob& j = jobs.job[i];
        if (j.ldd < j.cols_p || j.ldd % 4 != 0 || j.cols_p % 4 != 0 || j.cols_p <= 0 || j.rows_p <= 0 ||
            j.rows > j.rows_p || j.cols > j.cols_p)
            return hipErrorInvalidValue;
        all_groups += (int64_t)j.rows_p * (j.cols_p / 4);
    }
    // groups per workgroup: the most that still gives kPackMinBlocks workgroups, at least 256
    int32_t groups = kPackGroups;
    while (groups > 256 && all_groups / groups < kPackMinBlocks) groups /= 2;
    int64_t total = 0;
    for (int i = 0; i < 2; ++i) {
        PackJob& j = jobs.job[i];
        j.blocks = 0;
        j.groups = groups;
        j.rows_per_block = 0;
        j.pieces_per_row = 0;
        if (i >= jobs.count) continue;
        const int32_t cols4 = j.cols_p / 4;
        if (cols4 > groups) {
            j.pieces_per_row = (cols4 + groups - 1) / groups;
            j.blocks = (int64_t)j.rows_p * j.pieces_per_row;
        } else {
            j.rows_per_block = groups / cols4;
            j.blocks = (j.rows_p + j.rows_per_block - 1) / j.rows_per_block;
        }
        total += j.blocks;
    }
    if (total > 0xffffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)total), dim3(256), 0, stream, jobs);
    return hipGetLastError();
}

hipError_t launch_scale(float* C, int64_t ldc, int32_t M, int32_t N, float beta, hipStream_t stream) {
    hipLaunchKernelGGL(scale_kernel, dim3(grid_for((int64_t)M * N, 256)), dim3(256), 0, stream, C, ldc, M, N, beta);
    return hipGetLastError();
}

hipError_t launch_fma_probe(int iters, int workgroups, float* out, hipStream_t stream) {
    if (iters < 0 || workgroups < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fma_probe_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream, iters, out);
    return hipGetLastError();
}

hipError_t launch_read_probe(const float* x, int64_t n, float* partial, hipStream_t stream) {
    if (n < 0 || n % 4 != 0 || reinterpret_cast<uintptr_t>(x) % 16 != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(read_probe_kernel, dim3(kReadGrid), dim3(256), 0, stream, reinterpret_cast<const f32x4*>(x),
                       n / 4, partial);
    return hipGetLastError();
}

}  // namespace sgemm_impl
