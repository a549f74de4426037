// FP32 matrix-core SGEMM for gfx950.
//
// Structure (the block -> wave -> lane tiling of "GEMM from naive to tiled",
// sections 四-六, carried onto CDNA4 matrix cores):
//   * Each workgroup owns one BM x BN tile of C (output-stationary, as in the
//     throughput-matching page "如何让计算受限问题真正达到计算受限", section 1.2)
//     and walks K in steps of BK.
//   * Per K-step, the A tile (BM x BK) and B tile (BK x BN) reach LDS
//     straight from global memory (direct-to-LDS loads, see mfma_tile_dtl);
//     elements past the end of K are zero-filled (the padding argument of
//     section 七: a zero term leaves the sum alone).
//   * DS LDS stages: the loads of step s + DS - 1 are issued while step s is
//     computed, and one barrier per K-step makes a stage visible (section 六;
//     "SGEMM 纯 CUDA 优化总结", ex9).
//   * Each wave owns a WM x WN sub-tile as (WM/32) x (WN/32) blocks of
//     v_mfma_f32_32x32x2_f32: true FP32 products, FP32 accumulation.
//
// Operand layout of v_mfma_f32_32x32x2_f32 (wave64):
//   A operand: lane l holds A[i = l % 32][kk = l / 32]           (32 x 2)
//   B operand: lane l holds B[kk = l / 32][j = l % 32]           (2 x 32)
//   D        : lane l, register r holds D[i][j] with j = l % 32,
//              i = 8 * (r / 4) + 4 * (l / 32) + (r % 4)          (32 x 32)
// A k-group of 8 is split so that lane half h = l / 32 takes k = 4h + q for
// q = 0..3 and instruction q contracts k in {q, 4 + q}: every k of the group
// is used once, and the fragment of a lane is 4 k's of one row or column,
// read from a k-contiguous stage as a single 16-byte LDS read.
#include <hip/hip_runtime.h>

#include "kernels.hpp"
#include "lds_layout.hpp"

namespace sgemm_impl {

SGEMM_DEFINE_ZERO_BLOCK(kZeroMfma);

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <bool V>
struct BoolC {
    static constexpr bool value = V;
};

template <int V>
struct IntC {
    static constexpr int value = V;
};

template <int BM, int BN, int BK, int WGM, int WGN>
struct MfmaCfg {
    static constexpr int WM = BM / WGM;
    static constexpr int WN = BN / WGN;
    static constexpr int MB = WM / 32;
    static constexpr int NB = WN / 32;
    static constexpr int KG = BK / 8;           // k-groups of 8 per K-step
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(BK == 16 || BK == 32, "the chunk swizzle is defined for BK = 16 and 32");
    static_assert(KG % 2 == 0, "the fragment sets alternate within a K-step");
};

// Scheduling hints for one K-loop iteration of KG groups of NM MFMAs each:
// in every group one LDS read (the next group's fragments, NR of them) is
// placed after each of the first MFMAs.  __builtin_amdgcn_sched_group_barrier
// needs constant arguments, hence the recursion over template parameters.
constexpr int kMaskMfma = 0x008, kMaskDsRead = 0x100;

template <int I, int NM, int NR>
__device__ __forceinline__ void interleave_group() {
    if constexpr (I < NM) {
        __builtin_amdgcn_sched_group_barrier(kMaskMfma, 1, 0);
        if constexpr (I < NR) __builtin_amdgcn_sched_group_barrier(kMaskDsRead, 1, 0);
        interleave_group<I + 1, NM, NR>();
    }
}

template <int NM, int NR, int KG, int G = 0>
__device__ __forceinline__ void interleave_hints() {
    if constexpr (G < KG) {
        interleave_group<0, NM, NR>();
        interleave_hints<NM, NR, KG, G + 1>();
    }
}

// Where a tile's result goes: element (i, j) of the tile (tile-local
// coordinates) is written to out[(row0 + i) * ldo + col0 + j] when
// row0 + i < row_lim and col0 + j < col_lim.
struct TileOut {
    float* out;
    int64_t ldo;
    int row0, col0, row_lim, col_lim;
    float alpha = 1.f, beta = 0.f;   // out = alpha * sum + beta * out (partial sums: 1, 0)
};

// The epilogue: each wave writes its MB x NB blocks of 32 x 32 (lane l,
// register r of a block holds row 8 (r / 4) + 4 (l / 32) + r % 4, column
// l % 32), masked at the tile's limits, as alpha * sum + beta * out.  With
// beta != 0 the old values are read one block at a time (the fence keeps the
// scheduler from hoisting all of them next to the live accumulators).
// IB (interleaved columns, NB == 4): column c of block nb is wave column
// 4c + nb instead of 32 nb + c, so a lane holds 4 adjacent columns of each
// row, written as one 16-byte store where the output allows it.
template <int MB, int NB, int WM, int WN, bool IB = false>
__device__ __forceinline__ void write_tile(const TileOut& o, const f32x16 (&acc)[MB][NB], int wm, int wn, int l32,
                                           int lh) {
    if constexpr (IB) {
        static_assert(NB == 4, "interleaved columns come in groups of four blocks");
        const bool vec_out = ((reinterpret_cast<uintptr_t>(o.out) | (uintptr_t)(o.ldo * 4)) & 15) == 0;
        const int j0 = o.col0 + wn * WN + 4 * l32;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int ib = o.row0 + wm * WM + mb * 32 + 4 * lh;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = ib + 8 * (r >> 2) + (r & 3);
                if (i >= o.row_lim) continue;
                float* p = o.out + (int64_t)i * o.ldo + j0;
                f32x4 v = {o.alpha * acc[mb][0][r], o.alpha * acc[mb][1][r], o.alpha * acc[mb][2][r],
                           o.alpha * acc[mb][3][r]};
                if (vec_out && j0 + 3 < o.col_lim) {
                    if (o.beta != 0.f) {
                        const f32x4 c = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
                        for (int q = 0; q < 4; ++q) v[q] = __builtin_fmaf(o.beta, c[q], v[q]);
                    }
                    *reinterpret_cast<f32x4*>(p) = v;
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (j0 + q < o.col_lim) p[q] = o.beta == 0.f ? v[q] : __builtin_fmaf(o.beta, p[q], v[q]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        return;
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int j = o.col0 + wn * WN + nb * 32 + l32;
            const int ib = o.row0 + wm * WM + mb * 32 + 4 * lh;
            if (o.beta == 0.f) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int i = ib + 8 * (r >> 2) + (r & 3);
                    if (i < o.row_lim && j < o.col_lim) o.out[(int64_t)i * o.ldo + j] = o.alpha * acc[mb][nb][r];
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int i = ib + 8 * (r >> 2) + (r & 3);
                    if (i < o.row_lim && j < o.col_lim) {
                        float* p = o.out + (int64_t)i * o.ldo + j;
                        *p = __builtin_fmaf(o.beta, *p, o.alpha * acc[mb][nb][r]);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// ---------------------------------------------------------------------------
// One output tile, loaded direct-to-LDS.
//
// gfx950's global_load_lds_dwordx4 moves 16 bytes per lane from global
// memory straight into LDS: lane l of a wave lands at (wave-uniform base) +
// 16 * l, so one instruction fills 1 KB of LDS in lane order while the
// source address of each lane is free.  global_load_lds_dword does the same
// with 4 bytes per lane (256 B per instruction); it serves operands whose
// rows are not 16-byte aligned and builds exactly the same stage layout.
// There are no staging registers and no LDS write instructions (the direct
// global -> shared copy that "GEMM from naive to tiled" section 六.2
// describes for cp.async, and the register-free prefetch of "SGEMM 纯 CUDA
// 优化总结" Q10), and DS stages of LDS can be in flight at once:
//   * A stage [BM][BK]: an instruction fills whole rows, and the lane that
//     lands in physical 4-float chunk c of row r fetches logical chunk
//     c ^ swz(r), so the stage holds the swizzled layout;
//   * B stage: blocks of R = 256 / BN whole rows (1 KB, one 16-byte-lane
//     instruction or four 4-byte-lane ones), GS floats apart, GS chosen so
//     that the fragment reads of rows k and k + 4 (the two lane halves) fall
//     32 banks apart.
// Schedule: the loads of step s + DS - 1 are issued during step s into the
// stage that step s - 1 used; each wave waits (vmcnt) until its own loads
// of step s have landed, and the barrier makes every wave's part visible.
// The stages are separate __shared__ arrays and the loop is unrolled by DS,
// so each access names its stage statically.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void glb_void_t;

// The direct loads of one operand that one wave issues per K-step: PER
// instructions, ins = i * waves + wave.  Each lane's element of load i sits
// at a fixed byte offset off[i] from a wave-uniform base, the tile's first
// element at the current K-step, which an issue moves on by one K-step with
// a scalar add (steps are issued in order).  Inside the K range the loads
// take the scalar-base form of global_load_lds (the base in scalar
// registers, one 32-bit offset register per lane); a per-lane 64-bit pointer
// per load, advanced with a 64-bit vector add every step, measured 1.8 %
// slower for the 256 x 256 tile at 4096^3, 3 % for the 128 x 128 tile and
// 6.5 % for the 64 x 64 tile.  The offsets are 32-bit: the dispatcher runs
// a tile only where the farthest element of its K-step lies within 2^32
// bytes of the base (for a k-contiguous operand a row stride below about
// 2^30 / (R - 1) floats, R the tile's extent outside K).
// r0 is the tile's first non-K index and lim its bound (M or N): lanes past
// it read the last valid row (k-contiguous layout), or the last whole lane
// group of columns (k-major layout: a lane fetches L::SEG / 64 consecutive
// columns, so the clamp keeps its first column a multiple of that width and
// its last one inside the stored row), instead; that data only reaches
// outputs outside C that are never written.  The clamped index is never
// below r0, so no offset is negative.  Only the K range needs the zero
// block, on the steps that cross its end (checked()).
template <class L, int PER>
struct DtlLoads {
    const float* base;
    uint32_t off[PER];
    int kk[PER];
    int64_t step;
    __device__ __forceinline__ void init(const float* X, int64_t ld, int wave, int waves, int lane, int r0, int lim,
                                         int kb, int bk) {
        base = X + (L::KC ? (int64_t)r0 * ld + kb : (int64_t)kb * ld + r0);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            int r, k;
            L::elem(i * waves + wave, lane, r, k);
            const int d = clamp_index<L>(r0 + r, lim) - r0;
            off[i] = (uint32_t)((L::KC ? (int64_t)d * ld + k : (int64_t)k * ld + d) * 4);
            kk[i] = k;
        }
        step = L::KC ? (int64_t)bk : (int64_t)bk * ld;
    }
    // this lane's source of load i at the current K-step
    __device__ __forceinline__ const float* src(int i) const {
        return reinterpret_cast<const float*>(reinterpret_cast<const char*>(base) + off[i]);
    }
    // source of load i for the step starting at k0, zero block past ke
    __device__ __forceinline__ const float* checked(int i, int k0, int ke) const {
        return k0 + kk[i] < ke ? src(i) : kZeroMfma;
    }
    __device__ __forceinline__ void advance() { base += step; }
};

// s_waitcnt that waits for vmcnt <= N and nothing else (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Barrier for the direct-to-LDS pipeline: wait until at most N of this
// wave's direct loads are outstanding and all its LDS reads have returned,
// then s_barrier.  Written as one asm statement with a memory clobber: the
// workgroup fence of __syncthreads() would also wait for the loads that are
// meant to stay in flight.
template <int N>
__device__ __forceinline__ void dtl_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// One direct load of W floats per lane from src to LDS byte address
// lds + 4 * W * lane.  Issued as asm so that the compiler's LDS-DMA
// tracking, which cannot tell the stages apart across the unrolled loop and
// would wait for every load in flight, stays out of it: dtl_barrier's
// explicit vmcnt is the only wait.  M0 holds the LDS base; the s_nop is the
// wait state the hardware needs between an M0 write and an LDS DMA reading it.
template <int W>
__device__ __forceinline__ void dma_lanes(const float* src, const float* lds) {
    const uint32_t base = (uint32_t)(uintptr_t)(lds_void_t*)lds;
    if constexpr (W == 4)
        asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(base));
    else
        asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "{m0}"(base));
}

// The same load with a wave-uniform source base in scalar registers and a
// 32-bit byte offset per lane (global_load_lds with saddr).
template <int W>
__device__ __forceinline__ void dma_lanes_s(uint32_t off, const float* src_base, const float* lds) {
    const uint32_t base = (uint32_t)(uintptr_t)(lds_void_t*)lds;
    if constexpr (W == 4)
        asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(src_base), "{m0}"(base));
    else
        asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(src_base), "{m0}"(base));
}

// Race check (built with SGEMM_LDS_POISON=1, never in the product library):
// before each refill of a stage, every wave writes NaN into exactly the LDS
// bytes its own direct loads of that refill will fill, and waits for those
// writes, so that the loads land on top of them.  A wave that still read the
// stage after the barrier that freed it, or read a refill before its loads
// had landed, would see NaN, which the parity tests catch.
#ifndef SGEMM_LDS_POISON
#define SGEMM_LDS_POISON 0
#endif
constexpr bool kLdsPoison = SGEMM_LDS_POISON != 0;

template <int W>
__device__ __forceinline__ void poison_lanes(float* lds, int lane) {
    const float nan = __builtin_nanf("");
    if constexpr (W == 4)
        *reinterpret_cast<f32x4*>(lds + 4 * lane) = f32x4{nan, nan, nan, nan};
    else
        lds[lane] = nan;
}

template <int BM, int BN, int BK, int WGM, int WGN, int DS, int W, int OPS, bool PRIO>
__device__ __forceinline__ void mfma_tile_dtl(const GemmArgs& g, float* st0, float* st1, float* st2, float* st3,
                                              int tm, int tn, int kb, int ke, const TileOut& o) {
    float* const stg[4] = {st0, st1, st2, st3};
    using P = MfmaCfg<BM, BN, BK, WGM, WGN>;
    using LA = ALayout<(OPS & 1) != 0, BM, BK, W>;
    using LB = BLayout<(OPS & 2) != 0, BN, BK, W>;
    // a k-major B with four column blocks per wave reads the four blocks'
    // values of one k row as one 16-byte chunk (interleaved columns); with
    // A k-major as well this measured slower (139.8 against 145.2 TFLOP/s
    // at 4096^3), so it is kept to a k-contiguous A
    constexpr bool IB = !LB::KC && LA::KC && P::NB == 4;
    constexpr int WAVES = WGM * WGN;
    constexpr int A_PER = LA::INSTR / WAVES;
    constexpr int B_PER = LB::INSTR / WAVES;
    constexpr int LOADS = A_PER + B_PER;                 // per lane per K-step
    static_assert(A_PER * WAVES == LA::INSTR && B_PER * WAVES == LB::INSTR, "instructions per wave");
    static_assert(DS >= 2 && DS <= 4, "two to four stages");
    static_assert((DS - 2) * LOADS < 64, "loads in flight fit the vmcnt counter");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN;
    const int wn = wave % WGN;
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const int steps = (ke - kb + BK - 1) / BK;

    DtlLoads<LA, A_PER> la;
    DtlLoads<LB, B_PER> lb;
    la.init(g.A, g.lda, wave, WAVES, lane, m0, g.M, kb, BK);
    lb.init(g.B, g.ldb, wave, WAVES, lane, n0, g.N, kb, BK);

    // issue the direct loads of the next K-step (`step`) into stage `st`;
    // FULL: the whole step lies inside [kb, ke), so no lane needs the check
    // (the scalar-base form)
    auto issue = [&](int step, float* st, auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        const int k0 = kb + step * BK;
        if constexpr (kLdsPoison) {
#pragma unroll
            for (int i = 0; i < A_PER; ++i) poison_lanes<W>(st + LA::dst(i * WAVES + wave), lane);
#pragma unroll
            for (int i = 0; i < B_PER; ++i) poison_lanes<W>(st + LA::FLOATS + LB::dst(i * WAVES + wave), lane);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
        if constexpr (FULL) {
#pragma unroll
            for (int i = 0; i < A_PER; ++i) dma_lanes_s<W>(la.off[i], la.base, st + LA::dst(i * WAVES + wave));
#pragma unroll
            for (int i = 0; i < B_PER; ++i)
                dma_lanes_s<W>(lb.off[i], lb.base, st + LA::FLOATS + LB::dst(i * WAVES + wave));
        } else {
#pragma unroll
            for (int i = 0; i < A_PER; ++i) dma_lanes<W>(la.checked(i, k0, ke), st + LA::dst(i * WAVES + wave));
#pragma unroll
            for (int i = 0; i < B_PER; ++i)
                dma_lanes<W>(lb.checked(i, k0, ke), st + LA::FLOATS + LB::dst(i * WAVES + wave));
        }
        la.advance();
        lb.advance();
    };

    f32x16 acc[P::MB][P::NB];
#pragma unroll
    for (int mb = 0; mb < P::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < P::NB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.f;

    const int l32 = lane & 31;
    const int lh = lane >> 5;
    // Fragments: lane l holds op(A)[m = l % 32][k] and op(B)[k][n = l % 32] for
    // k = 8 kg + 4 (l / 32) + q, q < 4 (the MFMA's two k of step q are 4
    // apart; A and B agree on that order).  A KC operand reads its four k as
    // one 16-byte chunk, a KM operand one float per k row.
    int a_frag[P::KG][P::MB];
    int b_frag[P::KG][P::NB];
#pragma unroll
    for (int kg = 0; kg < P::KG; ++kg) {
#pragma unroll
        for (int mb = 0; mb < P::MB; ++mb) {
            if constexpr (LA::KC) a_frag[kg][mb] = LA::chunk(wm * P::WM + mb * 32 + l32, 2 * kg + lh);
            else a_frag[kg][mb] = 0;
        }
#pragma unroll
        for (int nb = 0; nb < P::NB; ++nb) {
            if constexpr (LB::KC) b_frag[kg][nb] = LA::FLOATS + LB::chunk(wn * P::WN + nb * 32 + l32, 2 * kg + lh);
            else b_frag[kg][nb] = 0;
        }
    }
    const int a_col = wm * P::WM + l32;
    const int b_col = wn * P::WN + l32;
    const int b_col4 = wn * P::WN + 4 * l32;

    f32x4 fa[2][P::MB];
    float fb[2][P::NB][4];
    auto read_frags = [&](const float* st, int kg, int set) {
#pragma unroll
        for (int mb = 0; mb < P::MB; ++mb) {
            if constexpr (LA::KC) {
                fa[set][mb] = *reinterpret_cast<const f32x4*>(st + a_frag[kg][mb]);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) fa[set][mb][q] = st[LA::krow(8 * kg + 4 * lh + q) + a_col + mb * 32];
            }
        }
#pragma unroll
        for (int nb = 0; nb < P::NB; ++nb) {
            if constexpr (LB::KC) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(st + b_frag[kg][nb]);
#pragma unroll
                for (int q = 0; q < 4; ++q) fb[set][nb][q] = v[q];
            } else if constexpr (!IB) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    fb[set][nb][q] = st[LA::FLOATS + LB::krow(8 * kg + 4 * lh + q) + b_col + nb * 32];
            }
        }
        if constexpr (IB) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 v =
                    *reinterpret_cast<const f32x4*>(st + LA::FLOATS + LB::krow(8 * kg + 4 * lh + q) + b_col4);
#pragma unroll
                for (int nb = 0; nb < P::NB; ++nb) fb[set][nb][q] = v[nb];
            }
        }
    };
    auto mfmas = [&](int set) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int mb = 0; mb < P::MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < P::NB; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[set][mb][q], fb[set][nb][q],
                                                                       acc[mb][nb], 0, 0, 0);
    };
    if (steps > 0) {
#pragma unroll
        for (int j = 0; j + 1 < DS; ++j) issue(j, stg[j], BoolC<false>{});
        dtl_barrier<(DS - 2) * LOADS>();
        read_frags(stg[0], 0, 0);
        issue(DS - 1, stg[DS - 1], BoolC<false>{});
#pragma unroll
        for (int kg = 0; kg + 1 < P::KG; ++kg) {
            read_frags(stg[0], kg + 1, (kg + 1) & 1);
            mfmas(kg & 1);
        }
        // iteration s uses stage s % DS and refills stage (s - 1) % DS with step s + DS - 1
        auto iter = [&](int s, auto j_tag, auto full_tag) {
            constexpr int J = decltype(j_tag)::value;
            dtl_barrier<(DS - 2) * LOADS>();
            read_frags(stg[J], 0, 0);
            mfmas(1);
            issue(s + DS - 1, stg[(J + DS - 1) % DS], full_tag);
            // PRIO: the wave that has issued its loads wins issue arbitration
            // for the rest of its MFMAs (measured +2 to +4 % on the 128x128
            // eight-wave and the 64x64 tiles, -1 % on the others)
            if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int kg = 0; kg + 1 < P::KG; ++kg) {
                read_frags(stg[J], kg + 1, (kg + 1) & 1);
                mfmas(kg & 1);
            }
            if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
            interleave_hints<P::MB * P::NB * 4, P::MB + 2 * P::NB, P::KG>();
        };
        // Unrolled by DS so that every iteration names its stages statically.
        // The first loop runs whole trips of iterations whose refill step lies
        // inside the K range (s + DS - 1 < full_steps); the second finishes
        // with the checked loads (and the loads past the end, which read zeros).
        // 4-byte lanes, with four times the loads, gain most from the first
        // loop's scalar-base loads: 497 -> 419 us for the 128 x 128 tile at
        // 4096 x 3008 x 2052, 195 -> 134 us for the 64 x 64 tile at 2048^3.
        int s = 1;
        {
            const int full_steps = (ke - kb) / BK;
            const int fast_trips = full_steps > DS ? (full_steps - DS) / DS : 0;
            for (int t = 0; t < fast_trips; ++t) {
                iter(s++, IntC<1>{}, BoolC<true>{});
                if constexpr (DS > 2) iter(s++, IntC<2>{}, BoolC<true>{});
                if constexpr (DS > 3) iter(s++, IntC<3>{}, BoolC<true>{});
                iter(s++, IntC<0>{}, BoolC<true>{});
            }
        }
        while (true) {
            if (s >= steps) break;
            iter(s++, IntC<1>{}, BoolC<false>{});
            if constexpr (DS > 2) {
                if (s >= steps) break;
                iter(s++, IntC<2>{}, BoolC<false>{});
            }
            if constexpr (DS > 3) {
                if (s >= steps) break;
                iter(s++, IntC<3>{}, BoolC<false>{});
            }
            if (s >= steps) break;
            iter(s++, IntC<0>{}, BoolC<false>{});
        }
        mfmas(1);
        wait_vmcnt<0>();                     // loads issued past the end land before the LDS is reused
    }

    write_tile<P::MB, P::NB, P::WM, P::WN, IB>(o, acc, wm, wn, l32, lh);
}

// The kernel has two work decompositions.
//  * One tile per workgroup (sk_iters == 0): workgroup x owns tile x (in the
//    XCD-aware order) and slice z = blockIdx.z of K; the slices' partial
//    products go to C + z * c_slice (split-K, summed by a second kernel).
//  * Stream-K (sk_iters > 0), a persistent grid of P workgroups: first the
//    dp_tiles "data-parallel" tiles, tile t on workgroup t % P, each over all
//    of K; then the remaining tiles' K-steps, flattened to sk_iters
//    (tile, K-step) units and cut into P equal ranges of sk_ipw units.  A
//    range covering a whole tile writes C; a partial tile is written to the
//    workspace slot 2 * wg + (0 for the range's first tile, 1 for its last)
//    and the stream-K fix-up kernel sums the slots of each tile in range
//    order.  The cut depends only on the shapes, so the sums always happen in
//    the same order (the work-splitting of "GEMM from naive to tiled", 十.1).
template <int BM, int BN, int BK, int WGM, int WGN, bool VEC, int WPE, int DS, int OPS, bool PRIO>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WGM * WGN, 64 * WGM * WGN),
                          amdgpu_waves_per_eu(WPE, WPE)))
void mfma_gemm_kernel(GemmArgs g) {
    // LDS: DSE separate stage arrays (16-byte lanes when the operands are
    // 16-byte aligned, else 4-byte lanes, which keep at most three stages so
    // that the loads in flight fit the vmcnt counter)
    static_assert(DS >= 2 && DS <= 4, "two to four stages");
    constexpr int DSE = VEC || DS < 3 ? DS : 3;
    constexpr int W = VEC ? 4 : 1;
    constexpr int QS = DtlStageFloats<OPS, BM, BN, BK>::value;
    __shared__ __attribute__((aligned(16))) float lds0[QS];
    __shared__ __attribute__((aligned(16))) float lds1[QS];
    __shared__ __attribute__((aligned(16))) float lds2[DSE > 2 ? QS : 4];
    __shared__ __attribute__((aligned(16))) float lds3[DSE > 3 ? QS : 4];
    // One call site for every work item, so that a single copy of the tile
    // code serves all decompositions: (tile, slice) in the one-tile mode;
    // the data-parallel tiles, then the K-step ranges, in stream-K mode.
    int64_t it = (int64_t)blockIdx.x * g.sk_ipw;                // stream-K: next (tile, K-step) unit
    const int64_t it_end = min(it + g.sk_ipw, g.sk_iters);
    int t = blockIdx.x;                                          // stream-K: next data-parallel tile
    int which = 0;                                               // stream-K: partial slot 0, then 1
    bool first = true;
    while (true) {
        int tile, kb, ke;
        TileOut o;
        int64_t step = 0;                                        // K-steps this item covers (stream-K ranges)
        bool slot = false;                                       // a partial tile, written to its slot
        if (g.sk_iters == 0) {
            if (!first) break;
            tile = blockIdx.x;
            kb = blockIdx.z * g.k_chunk;
            ke = min(g.K, kb + g.k_chunk);
            // one slice writes alpha * sum + beta * C; several write raw partial sums
            o = TileOut{g.C + (int64_t)blockIdx.z * g.c_slice, g.ldc, 0, 0, g.M, g.N,
                        g.c_slice ? 1.f : g.alpha, g.c_slice ? 0.f : g.beta};
        } else if (t < g.dp_tiles) {
            tile = t;
            t += gridDim.x;
            kb = 0;
            ke = g.K;
            o = TileOut{g.C, g.ldc, 0, 0, g.M, g.N, g.alpha, g.beta};
        } else if (it < it_end) {
            const int j = (int)(it / g.k_steps);
            const int ks0 = (int)(it - (int64_t)j * g.k_steps);
            const int ks1 = (int)min((int64_t)g.k_steps, ks0 + (it_end - it));
            tile = g.dp_tiles + j;
            kb = ks0 * BK;
            ke = min(g.K, ks1 * BK);
            if (ks0 == 0 && ks1 == g.k_steps) {
                o = TileOut{g.C, g.ldc, 0, 0, g.M, g.N, g.alpha, g.beta};
            } else {
                // slot 0 for the range's first tile, 1 for its last (the
                // fix-up picks the slot the same way)
                o = TileOut{g.ws + (int64_t)(2 * blockIdx.x + which) * (BM * BN), BN, 0, 0, BM, BN};
                slot = true;
            }
            which = 1;
            step = ks1 - ks0;
        } else {
            break;
        }
        int tm, tn;
        tile_coords(tile, g.tiles_m, g.tiles_n, g.group_m, &tm, &tn);
        if (!slot) {
            o.row0 = tm * BM;                                    // C (or a split-K slice): the tile's place
            o.col0 = tn * BN;
        }
        if (!first) __syncthreads();                             // the next tile's prologue overwrites LDS
        first = false;
        mfma_tile_dtl<BM, BN, BK, WGM, WGN, DSE, W, OPS, PRIO>(g, lds0, lds1, lds2, lds3, tm, tn, kb, ke, o);
        it += step;
    }
}

template <int BM, int BN, int BK, int WGM, int WGN, int WPE, int DS, bool NARROW, bool PRIO, int OPS>
hipError_t launch_ops(bool vec, const GemmArgs& g, int splits, hipStream_t stream) {
    dim3 grid(g.sk_iters > 0 ? (unsigned)g.sk_grid : (unsigned)((int64_t)g.tiles_m * g.tiles_n), 1,
              g.sk_iters > 0 ? 1u : (unsigned)splits);
    dim3 block(64 * WGM * WGN);
    if (vec) {
        hipLaunchKernelGGL((mfma_gemm_kernel<BM, BN, BK, WGM, WGN, true, WPE, DS, OPS, PRIO>), grid, block, 0, stream,
                           g);
    } else {
        if constexpr (!NARROW) return hipErrorInvalidValue;   // not built with 4-byte lanes
        else
            hipLaunchKernelGGL((mfma_gemm_kernel<BM, BN, BK, WGM, WGN, false, WPE, DS, OPS, PRIO>), grid, block, 0,
                               stream, g);
    }
    return hipGetLastError();
}

// ops: bit 0 = A stored transposed, bit 1 = B stored transposed.
template <int BM, int BN, int BK, int WGM, int WGN, int WPE, int DS, bool NARROW, bool PRIO>
hipError_t launch_one(bool vec, int ops, const GemmArgs& g, int splits, hipStream_t stream) {
    switch (ops) {
        case 0: return launch_ops<BM, BN, BK, WGM, WGN, WPE, DS, NARROW, PRIO, 0>(vec, g, splits, stream);
        case 1: return launch_ops<BM, BN, BK, WGM, WGN, WPE, DS, NARROW, PRIO, 1>(vec, g, splits, stream);
        case 2: return launch_ops<BM, BN, BK, WGM, WGN, WPE, DS, NARROW, PRIO, 2>(vec, g, splits, stream);
        case 3: return launch_ops<BM, BN, BK, WGM, WGN, WPE, DS, NARROW, PRIO, 3>(vec, g, splits, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_mfma(int tile, bool vec, int ops, const GemmArgs& g, int splits, hipStream_t stream) {
#define SGEMM_MFMA_CASE(ID)                                                                          \
    case ID:                                                                                         \
        return launch_one<kMfmaTiles[ID].bm, kMfmaTiles[ID].bn, kMfmaTiles[ID].bk, kMfmaTiles[ID].waves_m, \
                          kMfmaTiles[ID].waves_n, kMfmaTiles[ID].waves_per_simd, kMfmaTiles[ID].stages,      \
                          kMfmaTiles[ID].narrow, kMfmaTiles[ID].prio>(vec, ops, g, splits, stream);
    switch (tile) {
        SGEMM_MFMA_CASE(0)
        SGEMM_MFMA_CASE(1)
        SGEMM_MFMA_CASE(2)
        SGEMM_MFMA_CASE(3)
        default:
            return hipErrorInvalidValue;
    }
#undef SGEMM_MFMA_CASE
}
static_assert(kNumMfmaTiles == 4, "launch_mfma covers every MFMA tile");

}  // namespace sgemm_impl
