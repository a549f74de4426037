// C interface of the SGEMM library: argument checks, per-shape planning and
// dispatch.  Everything up to the first HIP call is plain host code, so an
// invalid call returns before touching the device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <limits>

#include "../../include/sgemm.h"
#include "kernels.hpp"

using namespace sgemm_impl;

namespace {

constexpr int64_t kMaxDim = (int64_t(1) << 30) - 1;   // kernels index tiles in 32-bit
constexpr int kNumCUs = 256;                          // MI355X: 8 XCDs x 32 CUs

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Byte range [lo, hi) a row-major rows x cols matrix with leading dimension ld occupies.
struct Range {
    uintptr_t lo = 0, hi = 0;
    bool empty() const { return hi <= lo; }
};
Range span(const float* p, int64_t rows, int64_t cols, int64_t ld) {
    Range r;
    if (p == nullptr || rows <= 0 || cols <= 0) return r;
    r.lo = reinterpret_cast<uintptr_t>(p);
    r.hi = r.lo + (uintptr_t)(((rows - 1) * ld + cols) * (int64_t)sizeof(float));
    return r;
}
bool overlap(const Range& a, const Range& b) {
    return !a.empty() && !b.empty() && a.lo < b.hi && b.lo < a.hi;
}

// (rows - 1) * ld + cols must fit comfortably in int64 bytes.
bool extent_ok(int64_t rows, int64_t cols, int64_t ld) {
    if (rows <= 0 || cols <= 0) return true;
    const int64_t lim = std::numeric_limits<int64_t>::max() / 8;
    return (rows - 1) <= (lim - cols) / ld;
}

struct Plan {
    sgemm_plan pub;
    int64_t ldw = 0;       // split-K workspace leading dimension (floats)
};

const TileShape& tile_of(int path, int tile) {
    switch (path) {
        case SGEMM_PATH_MFMA: return kMfmaTiles[tile];
        case SGEMM_PATH_VALU: return kValuTiles[tile];
        case SGEMM_PATH_SKINNY: return kSkinnyTiles[tile];
        default: return kNaiveTiles[0];
    }
}

int tile_count(int path) {
    switch (path) {
        case SGEMM_PATH_NAIVE: return kNumNaiveTiles;
        case SGEMM_PATH_VALU: return kNumValuTiles;
        case SGEMM_PATH_MFMA: return kNumMfmaTiles;
        case SGEMM_PATH_SKINNY: return kNumSkinnyTiles;
        default: return 0;
    }
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

// Relative throughput of a workgroup tile on the matrix cores, and how many
// of its workgroups one CU holds at once (from the register and LDS budgets).
// Used only to rank candidate plans.
double mfma_tile_efficiency(int tile) {
    switch (tile) {
        case 0: case 1: return 1.00;
        case 3: return 1.00;
        case 2: case 5: return 0.90;
        default: return 0.60;
    }
}

// Modelled time (arbitrary units) of an MFMA plan: waves of workgroups times
// the per-workgroup work, plus the reduction's traffic and launch when split.
double mfma_cost(int tile, int64_t M, int64_t N, int64_t K, int64_t splits, int64_t k_chunk) {
    const TileShape& t = kMfmaTiles[tile];
    const int64_t tiles = cdiv(M, t.bm) * cdiv(N, t.bn);
    const int64_t per_cu = t.waves_per_simd * 4 / (t.waves_m * t.waves_n);   // WGs resident per CU
    const int64_t slots = kNumCUs * std::max<int64_t>(per_cu, 1);
    const int64_t waves = cdiv(tiles * splits, slots);
    // one resident set shares the CU: each of its WGs takes per_cu times as long
    const double wg_work = (double)t.bm * t.bn * round_up(std::min(k_chunk, K), t.bk);
    const double cu_rate = 128.0 * 2.4e9 * 0.8;    // MACs/s per CU at ~80% of peak
    double time = waves * wg_work * per_cu / (cu_rate * mfma_tile_efficiency(tile));
    if (splits > 1) {
        const double bytes = 2.0 * splits * M * N * 4 + M * N * 4.0;
        time += bytes / 5e12 + 4e-6;              // reduction pass + one more launch
    }
    return time;
}

void choose_split(int64_t tiles, int64_t K, int bk, int64_t target_wgs, int64_t max_splits,
                  int64_t* splits, int64_t* k_chunk) {
    int64_t s = 1;
    if (tiles < target_wgs) s = cdiv(target_wgs, tiles);
    s = std::min(s, std::max<int64_t>(1, K / (4 * bk)));   // at least 4 K-steps per slice
    s = std::min(s, max_splits);
    int64_t kc = round_up(cdiv(K, s), bk);
    s = cdiv(K, kc);
    *splits = std::max<int64_t>(s, 1);
    *k_chunk = kc;
}

sgemm_status validate(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B,
                      int64_t ldb, const float* C, int64_t ldc) {
    if (M < 0 || N < 0 || K < 0) return SGEMM_ERR_INVALID_ARG;
    if (lda < std::max<int64_t>(1, K) || ldb < std::max<int64_t>(1, N) || ldc < std::max<int64_t>(1, N))
        return SGEMM_ERR_INVALID_ARG;
    if (M > 0 && K > 0 && A == nullptr) return SGEMM_ERR_INVALID_ARG;
    if (K > 0 && N > 0 && B == nullptr) return SGEMM_ERR_INVALID_ARG;
    if (M > 0 && N > 0 && C == nullptr) return SGEMM_ERR_INVALID_ARG;
    if (!aligned(A, 4) || !aligned(B, 4) || !aligned(C, 4)) return SGEMM_ERR_INVALID_ARG;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return SGEMM_ERR_UNSUPPORTED;
    if (!extent_ok(M, K, lda) || !extent_ok(K, N, ldb) || !extent_ok(M, N, ldc)) return SGEMM_ERR_UNSUPPORTED;
    const Range rc = span(C, M, N, ldc);
    if (overlap(rc, span(A, M, K, lda)) || overlap(rc, span(B, K, N, ldb))) return SGEMM_ERR_INVALID_ARG;
    return SGEMM_OK;
}

sgemm_status make_plan(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B,
                       int64_t ldb, const float* C, int64_t ldc, const sgemm_options* opts, Plan* out) {
    sgemm_status st = validate(M, N, K, A, lda, B, ldb, C, ldc);
    if (st != SGEMM_OK) return st;
    sgemm_options o{};
    if (opts) o = *opts;
    if (o.path < SGEMM_PATH_AUTO || o.path > SGEMM_PATH_SKINNY) return SGEMM_ERR_INVALID_ARG;
    if (o.split_k < 0 || o.vector < 0 || o.vector > 1) return SGEMM_ERR_INVALID_ARG;
    if (o.workspace != nullptr && !aligned(o.workspace, 256)) return SGEMM_ERR_INVALID_ARG;

    Plan p;
    std::memset(&p.pub, 0, sizeof(p.pub));
    sgemm_plan& q = p.pub;
    q.split_k = 1;
    if (M == 0 || N == 0) {          // nothing to write
        q.path = o.path == SGEMM_PATH_AUTO ? SGEMM_PATH_MFMA : o.path;
        q.launches = 0;
        *out = p;
        return SGEMM_OK;
    }
    if (K == 0) {                    // the empty sum: C = 0
        q.path = o.path == SGEMM_PATH_AUTO ? SGEMM_PATH_MFMA : o.path;
        q.launches = 1;
        *out = p;
        return SGEMM_OK;
    }

    const bool vec_ok = aligned(A, 16) && aligned(B, 16) && lda % 4 == 0 && ldb % 4 == 0 &&
                        K % 4 == 0 && N % 4 == 0;
    q.vector = (vec_ok && o.vector == 0) ? 1 : 0;

    int path = o.path;
    if (path == SGEMM_PATH_AUTO) path = (M <= 16) ? SGEMM_PATH_SKINNY : SGEMM_PATH_MFMA;
    if (path == SGEMM_PATH_SKINNY && M > 16) return SGEMM_ERR_INVALID_ARG;
    const int ntiles = tile_count(path);
    if (o.tile < -1 || o.tile >= ntiles) return SGEMM_ERR_INVALID_ARG;
    if (path == SGEMM_PATH_NAIVE && o.split_k > 1) return SGEMM_ERR_INVALID_ARG;

    int tile = o.tile;
    int64_t splits = 1, k_chunk = K;
    if (path == SGEMM_PATH_NAIVE) {
        tile = 0;
    } else if (path == SGEMM_PATH_SKINNY) {
        tile = 0;
        const TileShape& t = kSkinnyTiles[0];
        const int64_t tiles = cdiv(N, t.bn);
        if (o.split_k > 0) {
            splits = std::min<int64_t>(o.split_k, cdiv(K, t.bk));
            k_chunk = round_up(cdiv(K, splits), t.bk);
            splits = cdiv(K, k_chunk);
        } else {
            // enough workgroups to keep every CU streaming: about 4 per CU
            choose_split(tiles, K, t.bk / 4, 4 * kNumCUs, 64, &splits, &k_chunk);
            k_chunk = round_up(k_chunk, t.bk);
            splits = cdiv(K, k_chunk);
        }
    } else if (path == SGEMM_PATH_MFMA && tile < 0) {
        // rank candidate (tile, split) plans with the cost model
        double best = 0;
        for (int cand : {0, 1, 2, 3, 4}) {
            const TileShape& t = kMfmaTiles[cand];
            const int64_t tiles = cdiv(M, t.bm) * cdiv(N, t.bn);
            int64_t s = 1, kc = K;
            if (o.split_k > 0) {
                s = std::min<int64_t>(o.split_k, cdiv(K, t.bk));
                kc = round_up(cdiv(K, s), t.bk);
                s = cdiv(K, kc);
            } else {
                const int64_t per_cu = t.waves_per_simd * 4 / (t.waves_m * t.waves_n);
                choose_split(tiles, K, t.bk, kNumCUs * per_cu, 32, &s, &kc);
            }
            const double c = mfma_cost(cand, M, N, K, s, kc);
            if (tile < 0 || c < best) {
                best = c;
                tile = cand;
                splits = s;
                k_chunk = kc;
            }
        }
    } else {
        if (tile < 0) tile = 0;
        const TileShape& t = tile_of(path, tile);
        const int64_t tiles = cdiv(M, t.bm) * cdiv(N, t.bn);
        if (o.split_k > 0) {
            splits = std::min<int64_t>(o.split_k, cdiv(K, t.bk));
            k_chunk = round_up(cdiv(K, splits), t.bk);
            splits = cdiv(K, k_chunk);
        } else {
            const int64_t per_cu = std::max(1, t.waves_per_simd * 4 / (t.waves_m * t.waves_n));
            choose_split(tiles, K, t.bk, kNumCUs * per_cu, 32, &splits, &k_chunk);
        }
    }

    const TileShape& t = tile_of(path, tile);
    q.path = path;
    q.tile = tile;
    q.bm = t.bm;
    q.bn = t.bn;
    q.bk = t.bk;
    q.threads = 64 * t.waves_m * t.waves_n;
    if (path == SGEMM_PATH_NAIVE) q.threads = 256;
    q.tiles_m = cdiv(M, t.bm);
    q.tiles_n = cdiv(N, t.bn);
    q.split_k = (int32_t)splits;
    q.k_chunk = k_chunk;
    q.workgroups = q.tiles_m * q.tiles_n * splits;
    if (q.tiles_m * q.tiles_n * (int64_t)q.threads >= (int64_t(1) << 32) || splits > 65535)
        return SGEMM_ERR_UNSUPPORTED;
    if (splits > 1) {
        p.ldw = round_up(N, 4);
        q.workspace_bytes = (size_t)(splits * M * p.ldw * (int64_t)sizeof(float));
        q.launches = 2;
    } else {
        q.launches = 1;
    }
    *out = p;
    return SGEMM_OK;
}

sgemm_status run(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B, int64_t ldb,
                 float* C, int64_t ldc, hipStream_t stream, const sgemm_options* opts) {
    Plan p;
    sgemm_status st = make_plan(M, N, K, A, lda, B, ldb, C, ldc, opts, &p);
    if (st != SGEMM_OK) return st;
    const sgemm_plan& q = p.pub;
    if (q.launches == 0) return SGEMM_OK;
    if (K == 0) {
        return launch_fill_zero(C, ldc, (int32_t)M, (int32_t)N, stream) == hipSuccess ? SGEMM_OK
                                                                                     : SGEMM_ERR_HIP;
    }

    void* ws = nullptr;
    bool owned = false;
    if (q.split_k > 1) {
        if (opts != nullptr && opts->workspace != nullptr) {
            if (opts->workspace_bytes < q.workspace_bytes) return SGEMM_ERR_ALLOC;
            ws = opts->workspace;
        } else {
            if (hipMallocAsync(&ws, q.workspace_bytes, stream) != hipSuccess || ws == nullptr) {
                (void)hipGetLastError();
                return SGEMM_ERR_ALLOC;
            }
            owned = true;
        }
    }

    GemmArgs g;
    g.A = A;
    g.B = B;
    g.M = (int32_t)M;
    g.N = (int32_t)N;
    g.K = (int32_t)K;
    g.k_chunk = (int32_t)q.k_chunk;
    g.lda = lda;
    g.ldb = ldb;
    g.tiles_m = (int32_t)q.tiles_m;
    g.tiles_n = (int32_t)q.tiles_n;
    // 8 tile rows per raster group: the 64 workgroups one XCD holds at a time
    // (32 CUs x 2) then cover about an 8 x 8 block of tiles
    g.group_m = (int32_t)std::min<int64_t>(q.tiles_m, 8);
    if (q.split_k > 1) {
        g.C = static_cast<float*>(ws);
        g.ldc = p.ldw;
        g.c_slice = M * p.ldw;
    } else {
        g.C = C;
        g.ldc = ldc;
        g.c_slice = 0;
    }

    hipError_t e;
    switch (q.path) {
        case SGEMM_PATH_NAIVE: e = launch_naive(g, stream); break;
        case SGEMM_PATH_VALU: e = launch_valu(q.tile, q.vector != 0, g, q.split_k, stream); break;
        case SGEMM_PATH_SKINNY: e = launch_skinny(q.tile, q.vector != 0, g, q.split_k, stream); break;
        default: e = launch_mfma(q.tile, q.vector != 0, g, q.split_k, stream); break;
    }
    if (e == hipSuccess && q.split_k > 1)
        e = launch_splitk_reduce(static_cast<const float*>(ws), p.ldw, M * p.ldw, q.split_k, C, ldc,
                                 (int32_t)M, (int32_t)N, stream);
    if (owned) {
        if (hipFreeAsync(ws, stream) != hipSuccess && e == hipSuccess) e = hipErrorUnknown;
    }
    return e == hipSuccess ? SGEMM_OK : SGEMM_ERR_HIP;
}

}  // namespace

extern "C" {

sgemm_status sgemm(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B, int64_t ldb,
                   float* C, int64_t ldc, hipStream_t stream) {
    return run(M, N, K, A, lda, B, ldb, C, ldc, stream, nullptr);
}

sgemm_status sgemm_ex(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B,
                      int64_t ldb, float* C, int64_t ldc, hipStream_t stream, const sgemm_options* opts) {
    return run(M, N, K, A, lda, B, ldb, C, ldc, stream, opts);
}

sgemm_status sgemm_plan_query(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B,
                              int64_t ldb, const float* C, int64_t ldc, const sgemm_options* opts,
                              sgemm_plan* plan) {
    if (plan == nullptr) return SGEMM_ERR_INVALID_ARG;
    Plan p;
    sgemm_status st = make_plan(M, N, K, A, lda, B, ldb, C, ldc, opts, &p);
    if (st == SGEMM_OK) *plan = p.pub;
    return st;
}

size_t sgemm_workspace_size(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc) {
    // A plan for 16-byte aligned stand-in pointers far apart; only shapes matter.
    const float* A = reinterpret_cast<const float*>(uintptr_t(1) << 44);
    const float* B = reinterpret_cast<const float*>(uintptr_t(2) << 44);
    const float* C = reinterpret_cast<const float*>(uintptr_t(3) << 44);
    Plan p;
    if (make_plan(M, N, K, A, lda, B, ldb, C, ldc, nullptr, &p) != SGEMM_OK) return 0;
    return p.pub.workspace_bytes;
}

sgemm_status sgemm_tile_info(int32_t path, int32_t tile, int32_t* count, int32_t* bm, int32_t* bn, int32_t* bk,
                             int32_t* threads) {
    const int n = tile_count(path);
    if (count) *count = n;
    if (n == 0 || tile < 0 || tile >= n) return SGEMM_ERR_INVALID_ARG;
    const TileShape& t = tile_of(path, tile);
    if (bm) *bm = t.bm;
    if (bn) *bn = t.bn;
    if (bk) *bk = t.bk;
    if (threads) *threads = path == SGEMM_PATH_NAIVE ? 256 : 64 * t.waves_m * t.waves_n;
    return SGEMM_OK;
}

const char* sgemm_status_string(sgemm_status s) {
    switch (s) {
        case SGEMM_OK: return "SGEMM_OK";
        case SGEMM_ERR_INVALID_ARG: return "SGEMM_ERR_INVALID_ARG: invalid argument";
        case SGEMM_ERR_UNSUPPORTED: return "SGEMM_ERR_UNSUPPORTED: size beyond the kernels' index range";
        case SGEMM_ERR_HIP: return "SGEMM_ERR_HIP: HIP runtime or launch failure";
        case SGEMM_ERR_ALLOC: return "SGEMM_ERR_ALLOC: scratch allocation failed or workspace too small";
        default: return "unknown sgemm_status";
    }
}

const char* sgemm_version(void) { return "0.1.0"; }

}  // extern "C"
