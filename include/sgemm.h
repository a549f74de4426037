/*
 * sgemm.h -- row-major FP32 matrix product C = A.B on one AMD Instinct
 * MI355X (gfx950), C-ABI.
 *
 * Operation (the plain definition of the product, "CUDA 算子优化：GEMM",
 * section "矩阵乘法"; notation of "GEMM from naive to tiled", section 一.2):
 *
 *     C[i][j] = sum_{k=0}^{K-1} A[i][k] * B[k][j],   0 <= i < M, 0 <= j < N
 *
 * with A an M x K, B a K x N and C an M x N matrix, all row-major binary32:
 *     A[i][k] is at A[i*lda + k],  B[k][j] at B[k*ldb + j],  C[i][j] at C[i*ldc + j].
 * Leading dimensions are passed separately from the widths (the advice of
 * the inner/outer-product GEMM page on hotelren.com, section 4.2), so
 * sub-matrices and padded rows work; the gap between a row's width and its
 * leading dimension is never read or written.
 *
 * Arithmetic: every product and sum is IEEE binary32 with round-to-nearest-
 * even and one rounding per fused multiply-add; there is no reduced-precision
 * mode.  The summation order over k is the library's and may differ between
 * kernels, tiles and split counts, but a given call (same shapes, alignment,
 * options) always produces the same bits.  On inputs whose products and
 * partial sums are exact in binary32 (small integers) every kernel returns
 * the exact result.
 *
 * Semantics: C is overwritten (no alpha/beta).  M == 0 or N == 0 is a no-op.
 * K == 0 writes +0.0 to every element of C (the empty sum).
 *
 * Memory and streams: A, B and C are device pointers owned by the caller, on
 * the device that is current when the call is made.  The library keeps no
 * reference to them after the call returns.  All work is enqueued on
 * `stream` (0 = the null stream) and the call returns without waiting;
 * the caller synchronises.  Calls on one stream run in order.  When a plan
 * needs scratch memory (packed operand copies, split-K or stream-K
 * partials) and the caller passes none (`sgemm_ex` can take one), the
 * library uses a buffer it keeps for the (device, stream) pair, grown
 * stream-ordered (hipMallocAsync / hipFreeAsync) and held until the process
 * ends, at most 512 MiB each for up to 8 streams per device; larger requests,
 * further streams and calls under graph capture allocate and free their own,
 * stream-ordered.  Because the kept buffer belongs to the stream handle,
 * synchronise a stream before destroying it if a call of this library may
 * still be running on it.
 *
 * Errors: every argument check below runs on the host before any HIP call;
 * on failure nothing is enqueued and C is untouched.  No exception crosses
 * this interface.
 */
#ifndef DENSE_FP32_MATRIX_AMD_SGEMM_H
#define DENSE_FP32_MATRIX_AMD_SGEMM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sgemm_status {
    SGEMM_OK = 0,
    SGEMM_ERR_INVALID_ARG = 1,  /* negative size, ld too small, NULL pointer with a
                                   nonzero extent, C overlapping A or B, bad option */
    SGEMM_ERR_UNSUPPORTED = 2,  /* a size beyond the kernels' index range, or a forced
                                   matrix-core plan whose leading dimensions are too long
                                   for its loads' 32-bit offsets (see sgemm_ex) */
    SGEMM_ERR_HIP = 3,          /* a HIP runtime call or kernel launch failed */
    SGEMM_ERR_ALLOC = 4,        /* scratch allocation failed, or the caller's
                                   workspace is too small */
    SGEMM_ERR_SCRATCH_LIMIT = 5 /* sgemm_gemm_noalloc: no plan of the call fits the
                                   static scratch buffer */
} sgemm_status;

/*
 * C = A.B (see the file comment).
 *   M, N, K : sizes, each >= 0 and < 2^30 (larger sizes: SGEMM_ERR_UNSUPPORTED).
 *   A, lda  : M x K, lda >= max(1, K).   May be NULL when M == 0 or K == 0.
 *   B, ldb  : K x N, ldb >= max(1, N).   May be NULL when K == 0 or N == 0.
 *   C, ldc  : M x N, ldc >= max(1, N).   May be NULL when M == 0 or N == 0.
 * Pointers need only 4-byte alignment; 16-byte aligned rows take a faster
 * loader.  The byte ranges of C and of A or B must not overlap.
 */
sgemm_status sgemm(int64_t M, int64_t N, int64_t K,
                   const float* A, int64_t lda,
                   const float* B, int64_t ldb,
                   float* C, int64_t ldc,
                   hipStream_t stream);

/* Kernel families ("paths"). */
typedef enum sgemm_path {
    SGEMM_PATH_AUTO = 0,    /* per-shape choice */
    SGEMM_PATH_NAIVE = 1,   /* one thread per output, operands straight from memory */
    SGEMM_PATH_VALU = 2,    /* LDS-tiled, per-lane 8x8 outer-product update on FP32 FMA */
    SGEMM_PATH_MFMA = 3,    /* LDS-tiled, FP32 matrix-core contraction (v_mfma_f32_32x32x2_f32) */
    SGEMM_PATH_SKINNY = 4   /* M <= 32: streams B once, FP32 matrix cores (16x16x4) */
} sgemm_path;

/* Work decompositions of the tiled paths. */
typedef enum sgemm_decomposition {
    SGEMM_DECOMP_AUTO = 0,      /* per-shape choice */
    SGEMM_DECOMP_TILES = 1,     /* one output tile (and K slice) per workgroup */
    SGEMM_DECOMP_STREAM_K = 2   /* persistent workgroups share the tiles' K-steps evenly
                                   (MFMA and skinny paths) */
} sgemm_decomposition;

/*
 * Options for sgemm_ex.  Zero-initialised options mean "same as sgemm".
 * The matrix-core tiles address each load lane by a 32-bit byte offset from
 * its tile's first element, so a tile runs only where its K-step spans less
 * than 2^32 bytes: for A stored as is (and B stored transposed) a row stride
 * below about 2^30 / (rows of the tile - 1) floats, for the other layouts
 * below about 2^30 / 15.  The automatic choice then takes a smaller tile or
 * packed copies, and where neither fits (K itself that long) the vector-ALU
 * path (operands as stored) or the naive path; forcing the matrix-core path
 * on such operands is SGEMM_ERR_UNSUPPORTED.
 *   path          : an sgemm_path.
 *   tile          : index into the path's tile table (sgemm_tile_info), or -1 to choose;
 *                   ignored when path is SGEMM_PATH_AUTO.
 *   split_k       : 0 = choose, 1 = no split, S >= 2 = split K into S slices whose
 *                   partial products are summed in slice order 0..S-1 by a second
 *                   kernel (one-tile-per-workgroup decomposition only).
 *   vector        : 0 = choose (16-byte loads when the operands allow them),
 *                   1 = force 4-byte loads.  The 256 x 256 matrix-core tiles are
 *                   built for 16-byte loads only: forcing one of them with 4-byte
 *                   loads, or on unaligned operands with pack = 1, is
 *                   SGEMM_ERR_INVALID_ARG (with pack = 0 or 2 it runs on packed
 *                   copies).
 *   decomposition : an sgemm_decomposition.
 *   pack          : operands whose rows are not 16-byte aligned (or K, N not multiples
 *                   of 4) can first be copied into zero-padded, aligned workspace
 *                   copies (the "packing" of blocked GEMMs) so that the 16-byte
 *                   loaders apply: 0 = when the time model favours it, 1 = never,
 *                   2 = whenever an operand is misaligned.  Ignored when vector = 1.
 *                   Packing copies values exactly, so results are those of the
 *                   16-byte path on the same values.
 *   workspace     : 256-byte aligned device buffer of workspace_bytes for packed
 *                   operands and split-K or stream-K partials, or NULL to let the
 *                   library provide it (see "Memory and streams").  The caller keeps
 *                   it alive until the work completes.
 *   tile_order    : order in which workgroups take the matrix-core path's output
 *                   tiles: 0 = XCD-aware (each of the 8 XCDs, with its own L2, takes
 *                   one contiguous range of tiles, walked in groups of 8 tile rows;
 *                   the rasterisation of "如何让计算受限问题真正达到计算受限" section
 *                   5.2), 1 = plain row-major (for comparison).  Results are the
 *                   same bits either way.
 *   row_tail      : matrix-core path, any operand layout, M 1 to 32 rows past a
 *                   multiple of 64: run those last rows through the skinny kernel
 *                   after the main kernel has done the rows above, instead of a row
 *                   of output tiles that is mostly padding (the edge handling of
 *                   "GEMM from naive to tiled" section 七 moved to a kernel sized
 *                   for it).  0 = when the time model favours it, 1 = never,
 *                   2 = whenever possible (and the scratch fits).  The tail rows'
 *                   sums are those of the skinny path.
 */
typedef struct sgemm_options {
    int32_t path;
    int32_t tile;
    int32_t split_k;
    int32_t vector;
    int32_t decomposition;
    int32_t pack;
    void* workspace;
    size_t workspace_bytes;
    int32_t tile_order;
    int32_t row_tail;
} sgemm_options;

/* sgemm with explicit options (tests and benchmarks).  opts may be NULL. */
sgemm_status sgemm_ex(int64_t M, int64_t N, int64_t K,
                      const float* A, int64_t lda,
                      const float* B, int64_t ldb,
                      float* C, int64_t ldc,
                      hipStream_t stream, const sgemm_options* opts);

/* The launch plan a call would use.  Host only: validates the arguments
 * exactly as sgemm_ex does and fills *plan, without any HIP call. */
typedef struct sgemm_plan {
    int32_t path;            /* sgemm_path actually used */
    int32_t tile;            /* tile table index */
    int32_t split_k;         /* K slices (1 = no split) */
    int32_t vector;          /* 1 if the 16-byte loaders are used */
    int32_t bm, bn, bk;      /* block tile */
    int32_t threads;         /* threads per workgroup */
    int64_t tiles_m, tiles_n;/* output tiles along M and N */
    int64_t k_chunk;         /* K elements per slice */
    int64_t workgroups;      /* workgroups of the main kernel */
    size_t workspace_bytes;  /* split-K / stream-K scratch (0 if none) */
    int32_t launches;        /* kernels enqueued by the call (0 to 5: one packing copy of the
                                misaligned operands, the matrix kernel, a split-K reduction or
                                stream-K fix-up, and for a row tail the skinny kernel and its
                                reduction or fix-up) */
    int32_t decomposition;   /* sgemm_decomposition actually used */
    int64_t dp_tiles;        /* stream-K: tiles computed whole first */
    int64_t sk_tiles;        /* stream-K: tiles whose K-steps are shared out */
    int64_t sk_units_per_wg; /* stream-K: (tile, K-step) units per workgroup */
    int32_t packed;          /* bit 0: A, bit 1: B copied to aligned workspace first */
    int32_t k_padded;        /* K as the matrix kernel sees it (a multiple of 4 when
                                packed; K otherwise) */
    int32_t tail_rows;       /* last rows computed by the skinny kernel after the main
                                kernel (0: none; tiles_m and workgroups describe the main
                                kernel's M - tail_rows rows) */
} sgemm_plan;

sgemm_status sgemm_plan_query(int64_t M, int64_t N, int64_t K,
                              const float* A, int64_t lda,
                              const float* B, int64_t ldb,
                              const float* C, int64_t ldc,
                              const sgemm_options* opts, sgemm_plan* plan);

/*
 * The library-call form ("GEMM from naive to tiled", section 二.2, which
 * follows torch.matmul down to the BLAS call with operation flags, alpha
 * and beta; the epilogue of section 九.2 applies alpha and beta):
 *
 *     C = alpha * op(A) * op(B) + beta * C,     op(X) = X or X^T,
 *
 * all matrices row-major, op(A) M x K, op(B) K x N, C M x N:
 *   op_a = SGEMM_OP_N: A stored M x K, op(A)[i][k] = A[i*lda + k], lda >= max(1, K)
 *   op_a = SGEMM_OP_T: A stored K x M, op(A)[i][k] = A[k*lda + i], lda >= max(1, M)
 *   op_b = SGEMM_OP_N: B stored K x N, op(B)[k][j] = B[k*ldb + j], ldb >= max(1, N)
 *   op_b = SGEMM_OP_T: B stored N x K, op(B)[k][j] = B[j*ldb + k], ldb >= max(1, K)
 * (so nn.Linear's X . W^T is op_a = N, op_b = T with W stored N x K).
 * Scalars follow BLAS: with beta == 0, C is not read (whatever it holds,
 * NaN included, is overwritten); with alpha == 0 or K == 0, A and B are not
 * read (they may be NULL) and C = beta * C.  The arithmetic is that of
 * sgemm for the sum, then one rounding for alpha * sum and one for the
 * fused beta * C + (alpha * sum).  sgemm(...) is sgemm_gemm(N, N, ..., 1,
 * ..., 0, ...).  C may not overlap A or B when they are read; errors,
 * streams and workspace as for sgemm / sgemm_ex.  Operands stored
 * transposed are read by the matrix-core path, by the skinny path (M <= 32)
 * and by the naive path when forced; forcing the VALU path with them is
 * SGEMM_ERR_INVALID_ARG.
 */
typedef enum sgemm_op {
    SGEMM_OP_N = 0,   /* the operand as stored */
    SGEMM_OP_T = 1    /* the transpose of the stored operand */
} sgemm_op;

sgemm_status sgemm_gemm(int32_t op_a, int32_t op_b, int64_t M, int64_t N, int64_t K, float alpha,
                        const float* A, int64_t lda, const float* B, int64_t ldb, float beta,
                        float* C, int64_t ldc, hipStream_t stream);

/* sgemm_gemm with explicit options (opts may be NULL). */
sgemm_status sgemm_gemm_ex(int32_t op_a, int32_t op_b, int64_t M, int64_t N, int64_t K, float alpha,
                           const float* A, int64_t lda, const float* B, int64_t ldb, float beta,
                           float* C, int64_t ldc, hipStream_t stream, const sgemm_options* opts);

/*
 * sgemm_gemm_ex for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, and harnesses that forbid
 * hipMalloc.  It computes exactly what sgemm_gemm_ex computes with the same
 * arguments, but allocates and frees nothing: the scratch its kernels need
 * (packed operand copies, split-K slices, stream-K partial tiles) lives in
 * one static device array of SGEMM_NOALLOC_SCRATCH_BYTES that each device the
 * library runs on holds until the process ends (its address is looked up
 * once per device, on the first call there).
 *   - The automatic plan is the fastest one whose scratch fits the array (so
 *     it can differ from sgemm_gemm's plan, and with it the rounding order;
 *     results stay within the same bound).  Options that force a plan needing
 *     more return SGEMM_ERR_SCRATCH_LIMIT, with nothing enqueued.
 *   - opts->workspace must be NULL (and workspace_bytes 0): SGEMM_ERR_INVALID_ARG
 *     otherwise.
 *   - Every call on a device shares that device's array and leaves its last
 *     contents there; nothing in it needs to start at zero.  Calls that overlap
 *     on one device (different streams, or several host threads without
 *     ordering) race on it: order them on one stream or synchronise.
 * Arguments, semantics and the other errors are those of sgemm_gemm_ex.  No
 * device memory is allocated or freed (the host-side plan cache may grow on
 * the first call of a new shape).
 */
#define SGEMM_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

sgemm_status sgemm_gemm_noalloc(int32_t op_a, int32_t op_b, int64_t M, int64_t N, int64_t K, float alpha,
                                const float* A, int64_t lda, const float* B, int64_t ldb, float beta,
                                float* C, int64_t ldc, hipStream_t stream, const sgemm_options* opts);

/* The plan sgemm_gemm_ex would use.  Host only, no HIP call. */
sgemm_status sgemm_gemm_plan_query(int32_t op_a, int32_t op_b, int64_t M, int64_t N, int64_t K, float alpha,
                                   const float* A, int64_t lda, const float* B, int64_t ldb, float beta,
                                   const float* C, int64_t ldc, const sgemm_options* opts,
                                   sgemm_plan* plan);

/* Scratch bytes the default plan of sgemm_gemm would need for 16-byte
 * aligned base pointers and these leading dimensions.  Host only. */
size_t sgemm_gemm_workspace_size(int32_t op_a, int32_t op_b, int64_t M, int64_t N, int64_t K,
                                 int64_t lda, int64_t ldb, int64_t ldc);

/* Scratch bytes the default plan of sgemm would need for 16-byte aligned
 * base pointers and these leading dimensions (0 when it neither packs nor
 * splits K).  Host only. */
size_t sgemm_workspace_size(int64_t M, int64_t N, int64_t K,
                            int64_t lda, int64_t ldb, int64_t ldc);

/* Tile table of a path: returns SGEMM_OK and fills bm/bn/bk/threads for a
 * valid (path, tile), SGEMM_ERR_INVALID_ARG otherwise.  *count receives the
 * number of tiles of the path (any out-parameter may be NULL). */
sgemm_status sgemm_tile_info(int32_t path, int32_t tile, int32_t* count,
                             int32_t* bm, int32_t* bn, int32_t* bk, int32_t* threads);

/* Measurement helper, outside the product path: reads the n floats at x
 * once and writes SGEMM_READ_PROBE_PARTIALS per-workgroup sums to partial,
 * enqueued on `stream`.  Timing it gives the rate at which the chip streams
 * a buffer it reads once -- the measured machine model against which a
 * bandwidth-bound product (the skinny path, which reads B once) is judged,
 * as the GEMV example of "如何让计算受限问题真正达到计算受限", section 7,
 * weighs a kernel against the attainable, not the data-sheet, bandwidth.
 * x: device, 16-byte aligned, n >= 0 and a multiple of 4 (SGEMM_ERR_INVALID_ARG
 * otherwise, nothing enqueued); partial: device, SGEMM_READ_PROBE_PARTIALS
 * floats, caller-owned.  Nothing is allocated. */
#define SGEMM_READ_PROBE_PARTIALS 4096
sgemm_status sgemm_read_probe(const float* x, int64_t n, float* partial, hipStream_t stream);

/* Measurement helper, outside the product path: the rate of scalar FP32
 * fused multiply-adds (v_fmac_f32, no packed FP32), the ceiling of the VALU
 * path's rank-1 updates ("GEMM from naive to tiled", section 五: the inner
 * loop is nothing but such FMAs).  Enqueues `workgroups` x 256 lanes, each
 * running 16 independent chains of SGEMM_FMA_PROBE_FMAS_PER_ITER x iters
 * FMAs in total, and writing one float per lane to out (device, caller-owned,
 * workgroups x 256 floats).  FLOPs = 2 x 256 x workgroups x iters x
 * SGEMM_FMA_PROBE_FMAS_PER_ITER.  SGEMM_ERR_INVALID_ARG for iters < 0,
 * workgroups < 1 or a null out; nothing is allocated. */
#define SGEMM_FMA_PROBE_FMAS_PER_ITER 128
sgemm_status sgemm_fma_probe(int32_t iters, int32_t workgroups, float* out, hipStream_t stream);

/* Static string naming a status code. */
const char* sgemm_status_string(sgemm_status status);

/* Library version as "major.minor.patch". */
const char* sgemm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DENSE_FP32_MATRIX_AMD_SGEMM_H */
