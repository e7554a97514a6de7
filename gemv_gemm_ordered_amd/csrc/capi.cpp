// C-ABI shim: argument checks, launch geometry, error reporting.
// The GEMM entry points choose their tile from the weight's shape and the operands' alignment, never
// from M. The GEMV entry points choose, from M, how many rows of x a workgroup stages (and, for the
// ordered GEMV, 64- or 128-k stages): instances that compute every output's chains, order and tree
// identically. ggo_test_gemv_instance runs any instance at any M, so the tests compare them bit for bit.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "kernels.hpp"

#ifndef GGO_BUILD_INFO
#define GGO_BUILD_INFO "unknown build"
#endif

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return GGO_OK;
}

constexpr int64_t I32MAX = 0x7fffffff;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_mnk(const char* fn, int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0) return fail(GGO_EINVAL, "%s: negative size (M=%lld N=%lld K=%lld)", fn, (long long)M, (long long)N, (long long)K);
    if (M > I32MAX || N > I32MAX || K > I32MAX) return fail(GGO_EUNSUPPORTED, "%s: a size exceeds 2^31-1", fn);
    return GGO_OK;
}

int launched(const char* fn, hipError_t e) {
    if (e != hipSuccess) return fail(GGO_ELAUNCH, "%s: %s", fn, hipGetErrorString(e));
    return ok();
}

// Fill an [M, N] binary32 matrix with +0.0 (the value of an empty fold).
__global__ void k_fill_zero(float* C, int64_t ldc, int M, int N) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t total = static_cast<int64_t>(M) * N;
    if (i < total) {
        const int64_t m = i / N, n = i - m * N;
        C[m * ldc + n] = 0.0f;
    }
}

hipError_t fill_zero(float* C, int64_t ldc, int64_t M, int64_t N, hipStream_t s) {
    const int64_t total = M * N;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(k_fill_zero, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, C, ldc, (int)M, (int)N);
    return hipGetLastError();
}

// The value of an empty fold (+0) passed through a fused epilogue.
__global__ void k_epi_zero(void* C, int64_t ldc, int M, int N, Epi ep) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t total = static_cast<int64_t>(M) * N;
    if (i < total) {
        const int64_t m = i / N, n = i - m * N;
        epi_store(ep, C, ldc, m, n, 0.0f);
    }
}

hipError_t epi_zero(void* C, int64_t ldc, int64_t M, int64_t N, const Epi& ep, hipStream_t s) {
    if (epi_identity(ep)) return fill_zero(static_cast<float*>(C), ldc, M, N, s);
    const int64_t blocks = (M * N + 255) / 256;
    hipLaunchKernelGGL(k_epi_zero, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, C, ldc, static_cast<int>(M),
                       static_cast<int>(N), ep);
    return hipGetLastError();
}

Epi no_epi() { return Epi{nullptr, nullptr, 0, GGO_ACT_NONE, 0}; }

// Check a caller's epilogue (NULL means none) and turn it into the kernels' form.
int make_epi(const char* fn, const ggo_epilogue* e, int64_t N, Epi* out) {
    *out = no_epi();
    if (!e) return GGO_OK;
    if (e->act < GGO_ACT_NONE || e->act > GGO_ACT_GELU_TANH) return fail(GGO_EINVAL, "%s: unknown activation %d", fn, e->act);
    if (e->out_dtype != GGO_F32 && e->out_dtype != GGO_BF16) return fail(GGO_EINVAL, "%s: out_dtype must be GGO_F32 or GGO_BF16", fn);
    if (e->residual && e->ldr < N) return fail(GGO_EINVAL, "%s: residual row stride below N", fn);
    out->bias = e->bias;
    out->res = e->residual;
    out->ldr = e->residual ? e->ldr : 0;
    out->act = e->act;
    out->out_bf16 = e->out_dtype == GGO_BF16;
    return GGO_OK;
}

int fill_problem(const char* fn, const ggo_problem& q, int a_dtype, int kind, OrdProblem& p, int64_t& tiles) {
    int rc = check_mnk(fn, q.M, q.N, q.K);
    if (rc) return rc;
    if (q.batch < 0) return fail(GGO_EINVAL, "%s: negative batch", fn);
    if (q.M && q.N && q.batch) {
        if (!q.C || (q.K && (!q.A || !q.W))) return fail(GGO_EINVAL, "%s: null pointer", fn);
        if (q.lda < q.K || q.ldw < q.N || q.ldc < q.N)
            return fail(GGO_EINVAL, "%s: row stride below extent (lda=%lld K=%lld ldw=%lld ldc=%lld N=%lld)", fn,
                        (long long)q.lda, (long long)q.K, (long long)q.ldw, (long long)q.ldc, (long long)q.N);
        if (q.batch > 1 && (q.stride_a < 0 || q.stride_w < 0 || q.stride_c < 0))
            return fail(GGO_EINVAL, "%s: negative batch stride", fn);
    }
    int bm, bn;
    ordered_tile_shape(kind, &bm, &bn);
    p.A = q.A;
    p.W = q.W;
    p.C = q.C;
    p.lda = q.lda;
    p.ldw = q.ldw;
    p.ldc = q.ldc;
    p.sa = q.stride_a;
    p.sw = q.stride_w;
    p.sc = q.stride_c;
    p.M = (int32_t)q.M;
    p.N = (int32_t)q.N;
    p.K = (int32_t)q.K;
    p.batch = (int32_t)q.batch;
    p.tiles_m = (int32_t)((q.M + bm - 1) / bm);
    p.tiles_n = (int32_t)((q.N + bn - 1) / bn);
    const size_t esz = a_dtype == GGO_F32 ? 4 : 2;
    const int64_t avec = a_dtype == GGO_F32 ? 4 : 8;
    p.vec = 0;
    if (aligned(q.A, 16) && q.lda % avec == 0 && (q.batch <= 1 || (q.stride_a * (int64_t)esz) % 16 == 0)) p.vec |= VEC_A;
    if (aligned(q.W, 16) && q.ldw % 8 == 0 && (q.batch <= 1 || q.stride_w % 8 == 0)) p.vec |= VEC_W;
    if (aligned(q.C, 16) && q.ldc % 4 == 0 && (q.batch <= 1 || q.stride_c % 4 == 0)) p.vec |= VEC_C;
    tiles = (q.M && q.N) ? q.batch * (int64_t)p.tiles_m * p.tiles_n : 0;
    if (q.batch > I32MAX) return fail(GGO_EUNSUPPORTED, "%s: batch exceeds 2^31-1", fn);
    return GGO_OK;
}

// Tile of the ordered kernel, for gemm_ordered: 16 x 16 (one output per lane) on a weight of at most
// 2^20 elements, 64 x 32 (4 x 2 per lane) on one of at most 2^22, else 64 x 64 (4 x 4 per lane): the
// smaller the weight, the more outputs a tile gives up so that the weight still fills the chip at small
// M. A grouped launch (the value product) counts the weight elements of all its problems and batch
// entries: 64 x 32 up to 2^22, else 64 x 64 (32 heads of d = 128: 64 x 32 at L = 256 took 17 - 19 us
// against 24 - 26 on 64 x 64, level at L = 1024, 6% slower at L = 5000; the 16 x 16 tile was no faster
// than 64 x 64 at L = 256). The choice depends on the entry point and the weights' shapes, never on M;
// every output's chain, and so its bits, is the same under every tile.
constexpr int64_t ORDERED_SMALL_WEIGHT = int64_t(1) << 20, ORDERED_MID_WEIGHT = int64_t(1) << 22;

// Weight elements of a launch, counted up to just past ORDERED_MID_WEIGHT (problems that validation will
// reject count as nothing, and nothing here can overflow)
int64_t launch_weight(const ggo_problem* qs, int64_t count) {
    const int64_t cap = ORDERED_MID_WEIGHT + 1;
    int64_t w = 0;
    for (int64_t i = 0; i < count && w < cap; ++i) {
        const ggo_problem& q = qs[i];
        if (q.batch <= 0 || q.N <= 0 || q.K <= 0) continue;
        if (q.batch >= cap || q.N >= cap || q.K >= cap || q.N * q.K >= cap) return cap;
        w += q.batch * (q.N * q.K);   // each factor below 2^23: no overflow
    }
    return w < cap ? w : cap;
}

int run_group(const char* fn, const ggo_problem* qs, int64_t count, int a_dtype, int small_ok, hipStream_t s,
              int force_kind = -1) {
    if (a_dtype != GGO_BF16 && a_dtype != GGO_F32) return fail(GGO_EINVAL, "%s: a_dtype must be GGO_BF16 or GGO_F32", fn);
    if (!qs) return fail(GGO_EINVAL, "%s: null problem array", fn);
    if (count < 1 || count > GGO_MAX_PROBLEMS) return fail(GGO_EINVAL, "%s: count must be 1..%d", fn, GGO_MAX_PROBLEMS);
    OrdGroup g;
    std::memset(&g, 0, sizeof g);
    int64_t total = 0;
    int n = 0;
    const bool single = small_ok && count == 1 && qs[0].batch == 1;
    const int64_t wsum = launch_weight(qs, count);
    const int kind = force_kind >= 0                            ? force_kind
                   : single && wsum <= ORDERED_SMALL_WEIGHT ? ORD_TILE_SMALL
                   : wsum <= ORDERED_MID_WEIGHT             ? ORD_TILE_MID
                                                            : ORD_TILE_BIG;
    int wide = 1;   // the launch takes the wide loads only if every problem allows them
    for (int64_t i = 0; i < count; ++i) {
        int64_t tiles = 0;
        OrdProblem p;
        int rc = fill_problem(fn, qs[i], a_dtype, kind, p, tiles);
        if (rc) return rc;
        if (qs[i].K == 0 && qs[i].M && qs[i].N) {
            // empty folds: +0.0 for every output of every batch entry
            for (int64_t b = 0; b < qs[i].batch; ++b) {
                hipError_t e = fill_zero(qs[i].C + b * qs[i].stride_c, qs[i].ldc, qs[i].M, qs[i].N, s);
                if (e != hipSuccess) return launched(fn, e);
            }
            continue;
        }
        if (tiles == 0) continue;
        const int64_t max_ld = ordered_wide_max_ld(kind, a_dtype == GGO_F32);
        if (!((p.vec & VEC_A) && (p.vec & VEC_W) && p.K % 8 == 0 && p.N % 8 == 0 && p.lda <= max_ld && p.ldw <= max_ld))
            wide = 0;
        g.p[n] = p;
        g.tile_start[n] = (int32_t)total;
        total += tiles;
        if (total > I32MAX) return fail(GGO_EUNSUPPORTED, "%s: more than 2^31-1 tiles", fn);
        ++n;
    }
    if (n == 0) return ok();
    g.count = n;
    g.tile_start[n] = (int32_t)total;
    return launched(fn, launch_gemm_ordered(g, (int)total, a_dtype == GGO_F32, kind, wide, s));
}

// Tile of the matrix-core GEMM, from the weight's shape and the operands' alignment, never from M.
// "Wide" operands are 16-byte aligned with row strides that are multiples of 8 (and below 2^22: buffer
// offsets are 32-bit) and K and N multiples of 8: the direct-to-LDS instances load 16-byte chunks through
// range-checked buffer descriptors that end at the caller's last element, and the range check drops a
// whole dword that straddles that end, so no chunk may straddle it. With wide operands:
//  - a weight of at most 2^20 elements: 64x128 tiles, so that a small weight still fills more CUs at
//    small M;
//  - up to 2^24 elements with K <= 1024: 128x128 tiles (few k-steps per workgroup: the first loads' latency
//    and the stores weigh more than a larger tile's efficiency);
//  - up to 2^24 elements with a longer K: 256x128;
//  - from 2^24 elements: 256x256.
// Other operands take the register-staged instances: 64x64 tiles for weights of at most 2^20 elements,
// else 128x128.
// Every instance gives every output the same bits (the same opcode, the same operand values in the same
// groups of 32 k, ascending), so the choice moves no bit. `force` (a MFMA_TILE_* value, or -1) lets the
// test hook run any instance.
enum {
    MFMA_TILE_256x128 = 0, MFMA_TILE_128x128 = 1, MFMA_TILE_64x64 = 2, MFMA_TILE_256x256 = 3,
    MFMA_TILE_128x128_LDS = 4, MFMA_TILE_64x128_LDS = 5
};
constexpr int64_t MFMA_SMALL_WEIGHT = int64_t(1) << 20, MFMA_LARGE_WEIGHT = int64_t(1) << 24;
constexpr int64_t MFMA_SHORT_K = 1024;

// The direct-to-LDS tile of a weight N x K (operands that allow its loads), by the rule above
static int mfma_wide_tile(int64_t N, int64_t K) {
    return N * K <= MFMA_SMALL_WEIGHT ? MFMA_TILE_64x128_LDS
         : N * K >= MFMA_LARGE_WEIGHT ? MFMA_TILE_256x256
         : K <= MFMA_SHORT_K          ? MFMA_TILE_128x128_LDS
                                      : MFMA_TILE_256x128;
}

// Its shape
static void mfma_wide_shape(int tile, int* bm, int* bn) {
    if (tile == MFMA_TILE_256x256) mfma_tile_shape_t256x256(bm, bn);
    else if (tile == MFMA_TILE_128x128_LDS) mfma_tile_shape_lds128(bm, bn);
    else if (tile == MFMA_TILE_64x128_LDS) mfma_tile_shape_lds64x128(bm, bn);
    else mfma_tile_shape(bm, bn);
}

int run_mfma(const char* fn, const uint16_t* A, int64_t lda, const uint16_t* W, int64_t ldw, void* C, int64_t ldc,
             int64_t M, int64_t N, int64_t K, hipStream_t s, int force, const Epi& ep) {
    int rc = check_mnk(fn, M, N, K);
    if (rc) return rc;
    if (M == 0 || N == 0) return ok();
    if (!C || (K && (!A || !W))) return fail(GGO_EINVAL, "%s: null pointer", fn);
    if (lda < K || ldw < N || ldc < N) return fail(GGO_EINVAL, "%s: row stride below extent", fn);
    if (K == 0) return launched(fn, epi_zero(C, ldc, M, N, ep, s));
    const bool wide_ok = aligned(A, 16) && lda % 8 == 0 && aligned(W, 16) && ldw % 8 == 0 &&
                         lda < (int64_t(1) << 22) && ldw < (int64_t(1) << 22) && K % 8 == 0 && N % 8 == 0;
    // the tile follows the weight (and what the operands allow), never M
    const int tile = force >= 0 ? force
                   : !wide_ok ? (N * K <= MFMA_SMALL_WEIGHT ? MFMA_TILE_64x64 : MFMA_TILE_128x128)
                   : mfma_wide_tile(N, K);
    static const char* const names[] = {"256x128", "128x128", "64x64", "256x256", "128x128 direct-to-LDS",
                                        "64x128 direct-to-LDS"};
    const bool needs_wide = tile == MFMA_TILE_256x128 || tile == MFMA_TILE_256x256 || tile == MFMA_TILE_128x128_LDS ||
                            tile == MFMA_TILE_64x128_LDS;
    if (needs_wide && !wide_ok)
        return fail(GGO_EUNSUPPORTED, "%s: the %s instance needs 16-byte aligned operands with row strides and K, N "
                    "multiples of 8", fn, names[tile]);
    int bm, bn;
    if (tile == MFMA_TILE_256x128)
        mfma_tile_shape(&bm, &bn);
    else if (tile == MFMA_TILE_256x256)
        mfma_tile_shape_t256x256(&bm, &bn);
    else if (tile == MFMA_TILE_128x128_LDS)
        mfma_tile_shape_lds128(&bm, &bn);
    else if (tile == MFMA_TILE_64x128_LDS)
        mfma_tile_shape_lds64x128(&bm, &bn);
    else if (tile == MFMA_TILE_128x128)
        mfma_tile_shape_t128(&bm, &bn);
    else
        mfma_tile_shape_t64(&bm, &bn);
    MfmaArgs a;
    a.A = A;
    a.W = W;
    a.C = C;
    a.lda = lda;
    a.ldw = ldw;
    a.ldc = ldc;
    a.M = (int32_t)M;
    a.N = (int32_t)N;
    a.K = (int32_t)K;
    const int64_t tm = (M + bm - 1) / bm, tn = (N + bn - 1) / bn;
    if (tm * tn > I32MAX) return fail(GGO_EUNSUPPORTED, "%s: too many tiles", fn);
    a.tiles_m = (int32_t)tm;
    a.tiles_n = (int32_t)tn;
    a.vec = 0;
    if (aligned(A, 16) && lda % 8 == 0) a.vec |= VEC_A;
    if (aligned(W, 8) && ldw % 4 == 0) a.vec |= VEC_W;
    if (aligned(C, 16) && ldc % 4 == 0) a.vec |= VEC_C;
    a.ep = ep;
    // 64x64 tile, branch-free loads: 16-byte chunks of A and 8-byte pieces of W never straddle a row's end,
    // and every offset into the A panel (64 rows) and the W panel (K rows) stays below 2^31 bytes
    if (aligned(A, 16) && lda % 8 == 0 && aligned(W, 8) && ldw % 8 == 0 && K % 8 == 0 && N % 4 == 0 &&
        64 * lda * 2 < (int64_t(1) << 31) && K * ldw * 2 < (int64_t(1) << 31))
        a.vec |= VEC_WIDE64;
    if ((!ep.bias || aligned(ep.bias, 16)) && (!ep.res || (aligned(ep.res, 16) && ep.ldr % 4 == 0)) &&
        aligned(C, ep.out_bf16 ? 8 : 16) && ldc % 4 == 0)
        a.vec |= VEC_EP;
    return launched(fn, tile == MFMA_TILE_256x128       ? launch_gemm_mfma_invariant(a, s)
                        : tile == MFMA_TILE_256x256     ? launch_gemm_mfma_invariant_256(a, s)
                        : tile == MFMA_TILE_128x128_LDS ? launch_gemm_mfma_lds128(a, s)
                        : tile == MFMA_TILE_64x128_LDS  ? launch_gemm_mfma_lds64x128(a, s)
                        : tile == MFMA_TILE_128x128     ? launch_gemm_mfma_t128(a, s)
                                                        : launch_gemm_mfma_t64(a, s));
}

}  // namespace

extern "C" {

int gemm_ordered(const void* A, int a_dtype, int64_t lda, const uint16_t* W, int64_t ldw, float* C, int64_t ldc,
                 int64_t M, int64_t N, int64_t K, void* stream) {
    ggo_problem q;
    q.A = A;
    q.W = W;
    q.C = C;
    q.lda = lda;
    q.ldw = ldw;
    q.ldc = ldc;
    q.batch = 1;
    q.stride_a = q.stride_w = q.stride_c = 0;
    q.M = M;
    q.N = N;
    q.K = K;
    return run_group("gemm_ordered", &q, 1, a_dtype, 1, static_cast<hipStream_t>(stream));
}

int gemm_ordered_grouped(const ggo_problem* problems, int64_t count, int a_dtype, void* stream) {
    return run_group("gemm_ordered_grouped", problems, count, a_dtype, 0, static_cast<hipStream_t>(stream));
}

int ggo_test_gemm_ordered_tile(int tile, const void* A, int a_dtype, int64_t lda, const uint16_t* W, int64_t ldw, float* C,
                               int64_t ldc, int64_t M, int64_t N, int64_t K, void* stream) {
    const char* fn = "ggo_test_gemm_ordered_tile";
    if (tile != GGO_TEST_ORDERED_TILE_64x64 && tile != GGO_TEST_ORDERED_TILE_16x16 && tile != GGO_TEST_ORDERED_TILE_64x32)
        return fail(GGO_EINVAL, "%s: unknown tile %d", fn, tile);
    const int kind = tile == GGO_TEST_ORDERED_TILE_16x16 ? ORD_TILE_SMALL
                   : tile == GGO_TEST_ORDERED_TILE_64x32 ? ORD_TILE_MID
                                                         : ORD_TILE_BIG;
    ggo_problem q;
    q.A = A;
    q.W = W;
    q.C = C;
    q.lda = lda;
    q.ldw = ldw;
    q.ldc = ldc;
    q.batch = 1;
    q.stride_a = q.stride_w = q.stride_c = 0;
    q.M = M;
    q.N = N;
    q.K = K;
    return run_group(fn, &q, 1, a_dtype, 1, static_cast<hipStream_t>(stream), kind);
}

}  // extern "C"

// gemv_ordered (wt = 0, W [K, N]) and gemv_ordered_wt (wt = 1, W^T [N, K]); form as in GemvArgs.
static int run_gemv_ordered(const char* fn, int wt, const uint16_t* x, int64_t ldx, const uint16_t* W, int64_t ldw,
                            float* y, int64_t ldy, int64_t M, int64_t N, int64_t K, hipStream_t s, int form,
                            int rows = 0) {
    int rc = check_mnk(fn, M, N, K);
    if (rc) return rc;
    if (M > GGO_GEMV_MAX_M) return fail(GGO_EUNSUPPORTED, "%s: M=%lld exceeds %d (gemm_ordered gives the same bits)", fn, (long long)M, GGO_GEMV_MAX_M);
    if (M == 0 || N == 0) return ok();
    if (!y || (K && (!x || !W))) return fail(GGO_EINVAL, "%s: null pointer", fn);
    if (ldx < K || ldw < (wt ? K : N) || ldy < N) return fail(GGO_EINVAL, "%s: row stride below extent", fn);
    if (K == 0) return launched(fn, fill_zero(y, ldy, M, N, s));
    GemvArgs a;
    a.x = x;
    a.W = W;
    a.y = y;
    a.ldx = ldx;
    a.ldw = ldw;
    a.ldy = ldy;
    a.M = (int32_t)M;
    a.N = (int32_t)N;
    a.K = (int32_t)K;
    a.wt = wt;
    a.form = form;
    a.rows = rows;
    if (wt) {
        // 8-byte loads of 4 k from rows of x and W^T: no load may straddle the end of a row
        if (!aligned(x, 8) || ldx % 4 || !aligned(W, 8) || ldw % 4 || K % 4)
            return fail(GGO_EUNSUPPORTED,
                        "%s: x and W^T must be 8-byte aligned with row strides and K multiples of 4 "
                        "(gemv_ordered on W [K, N] takes any operands and gives the same bits)", fn);
        if (ldw > gemv_ordered_wt_max_ldw())
            return fail(GGO_EUNSUPPORTED, "%s: ldwt=%lld too large for 32-bit buffer offsets", fn, (long long)ldw);
        a.vec = VEC_W | VEC_A;
        if (aligned(x, 16) && ldx % 8 == 0 && aligned(W, 16) && ldw % 8 == 0 && K % 8 == 0) a.vec |= VEC_W16;
    } else {
        if (ldw > gemv_ordered_max_ldw() || K >= (int64_t(1) << 30))
            return fail(GGO_EUNSUPPORTED, "%s: ldw=%lld or K=%lld too large for 32-bit buffer offsets (gemm_ordered gives the same bits)",
                        fn, (long long)ldw, (long long)K);
        // wide loads: W as 4-byte column pairs at even n, x as 8-byte runs of 4 k
        // (same arithmetic and bits either way; only the load width differs)
        a.vec = 0;
        if (aligned(W, 4) && ldw % 2 == 0 && N % 2 == 0 && aligned(x, 8) && ldx % 4 == 0 && K % 4 == 0)
            a.vec |= VEC_W | VEC_A;
    }
    if (form == 2 && !gemv_ordered_k128_ok(a))
        return fail(GGO_EUNSUPPORTED, "%s: the 128-k instance needs 4-byte column pairs of W (or W^T) and ldw "
                    "small enough for its stage ranges", fn);
    if (form == 4 && !gemv_ordered_mr_ok(a))
        return fail(GGO_EUNSUPPORTED, "%s: the MR-row instance serves W^T with 16-byte aligned x and W^T and row "
                    "strides and K multiples of 8", fn);
    if (form == 3 && !gemv_ordered_m1_ok(a))
        return fail(GGO_EUNSUPPORTED, "%s: the 512-k instance serves M = 1 with W^T, 16-byte aligned x and W^T and "
                    "row strides and K multiples of 8", fn);
    return launched(fn, launch_gemv_ordered(a, s));
}

static int run_tree(const char* fn, const uint16_t* x, int64_t ldx, const uint16_t* WT, int64_t ldwt, void* y, int64_t ldy,
                    int64_t M, int64_t N, int64_t K, hipStream_t s, const Epi& ep, int rows = 0, int form = 0) {
    int rc = check_mnk(fn, M, N, K);
    if (rc) return rc;
    if (M > GGO_GEMV_MAX_M) return fail(GGO_EUNSUPPORTED, "%s: M=%lld exceeds %d", fn, (long long)M, GGO_GEMV_MAX_M);
    if (M == 0 || N == 0) return ok();
    if (!y || (K && (!x || !WT))) return fail(GGO_EINVAL, "%s: null pointer", fn);
    if (ldx < K || ldwt < K || ldy < N) return fail(GGO_EINVAL, "%s: row stride below extent", fn);
    if (K == 0) return launched(fn, epi_zero(y, ldy, M, N, ep, s));
    if (K > gemv_tree_max_k())
        return fail(GGO_EUNSUPPORTED, "%s: K=%lld too large for 32-bit byte offsets along a row", fn, (long long)K);
    TreeArgs a;
    a.x = x;
    a.WT = WT;
    a.y = y;
    a.ldx = ldx;
    a.ldwt = ldwt;
    a.ldy = ldy;
    a.M = (int32_t)M;
    a.N = (int32_t)N;
    a.K = (int32_t)K;
    // 16-byte tile loads when no tile can straddle the end of a row (same arithmetic and bits either way)
    a.wide = aligned(x, 16) && ldx % 8 == 0 && aligned(WT, 16) && ldwt % 8 == 0 && K % 8 == 0;
    a.ep = ep;
    a.rows = rows;
    a.form = form;
    if (form == 1 && !(a.wide && K <= gemv_tree_persistent_max_k() && rows <= 8))
        return fail(GGO_EUNSUPPORTED, "%s: the persistent instance needs 16-byte operands, K <= %d and at most 8 staged rows",
                    fn, gemv_tree_persistent_max_k());
    return launched(fn, launch_gemv_tree(a, s));
}

extern "C" {

int gemv_ordered(const uint16_t* x, int64_t ldx, const uint16_t* W, int64_t ldw, float* y, int64_t ldy, int64_t M,
                 int64_t N, int64_t K, void* stream) {
    return run_gemv_ordered("gemv_ordered", 0, x, ldx, W, ldw, y, ldy, M, N, K, static_cast<hipStream_t>(stream), 0);
}

int gemv_ordered_wt(const uint16_t* x, int64_t ldx, const uint16_t* WT, int64_t ldwt, float* y, int64_t ldy, int64_t M,
                    int64_t N, int64_t K, void* stream) {
    return run_gemv_ordered("gemv_ordered_wt", 1, x, ldx, WT, ldwt, y, ldy, M, N, K, static_cast<hipStream_t>(stream), 0);
}

int gemv_tree(const uint16_t* x, int64_t ldx, const uint16_t* WT, int64_t ldwt, float* y, int64_t ldy, int64_t M,
              int64_t N, int64_t K, void* stream) {
    return run_tree("gemv_tree", x, ldx, WT, ldwt, y, ldy, M, N, K, static_cast<hipStream_t>(stream), no_epi());
}

int gemv_tree_ep(const uint16_t* x, int64_t ldx, const uint16_t* WT, int64_t ldwt, const ggo_epilogue* ep, void* y,
                 int64_t ldy, int64_t M, int64_t N, int64_t K, void* stream) {
    Epi e;
    int rc = make_epi("gemv_tree_ep", ep, N, &e);
    if (rc) return rc;
    return run_tree("gemv_tree_ep", x, ldx, WT, ldwt, y, ldy, M, N, K, static_cast<hipStream_t>(stream), e);
}

int gemm_mfma_invariant_ep(const uint16_t* A, int64_t lda, const uint16_t* W, int64_t ldw, const ggo_epilogue* ep,
                           void* C, int64_t ldc, int64_t M, int64_t N, int64_t K, void* stream) {
    Epi e;
    int rc = make_epi("gemm_mfma_invariant_ep", ep, N, &e);
    if (rc) return rc;
    return run_mfma("gemm_mfma_invariant_ep", A, lda, W, ldw, C, ldc, M, N, K, static_cast<hipStream_t>(stream), -1, e);
}

int gemm_mfma_invariant(const uint16_t* A, int64_t lda, const uint16_t* W, int64_t ldw, float* C, int64_t ldc,
                        int64_t M, int64_t N, int64_t K, void* stream) {
    return run_mfma("gemm_mfma_invariant", A, lda, W, ldw, C, ldc, M, N, K, static_cast<hipStream_t>(stream), -1, no_epi());
}

int gemm_mfma_invariant_wt(const uint16_t* A, int64_t lda, const uint16_t* WT, int64_t ldwt, float* C, int64_t ldc,
                           int64_t M, int64_t N, int64_t K, void* stream) {
    const char* fn = "gemm_mfma_invariant_wt";
    hipStream_t s = static_cast<hipStream_t>(stream);
    int rc = check_mnk(fn, M, N, K);
    if (rc) return rc;
    if (M == 0 || N == 0) return ok();
    if (!C || (K && (!A || !WT))) return fail(GGO_EINVAL, "%s: null pointer", fn);
    if (lda < K || ldwt < K || ldc < N) return fail(GGO_EINVAL, "%s: row stride below extent", fn);
    if (K == 0) return launched(fn, fill_zero(C, ldc, M, N, s));
    // 16-byte chunks through range-checked descriptors: no chunk may straddle the end of a row of A or W^T
    if (!aligned(A, 16) || lda % 8 || !aligned(WT, 16) || ldwt % 8 || lda >= (int64_t(1) << 22) ||
        ldwt >= (int64_t(1) << 22) || K % 8)
        return fail(GGO_EUNSUPPORTED,
                    "%s: A and W^T must be 16-byte aligned with row strides that are multiples of 8 and below 2^22, "
                    "and K a multiple of 8 (gemm_mfma_invariant takes any W [K, N] and gives the same bits)", fn);
    int bm, bn;
    mfma_wide_shape(mfma_wide_tile(N, K), &bm, &bn);   // the weight's tile, as for gemm_mfma_invariant
    MfmaArgs a;
    a.A = A;
    a.W = WT;
    a.C = C;
    a.lda = lda;
    a.ldw = ldwt;
    a.ldc = ldc;
    a.M = (int32_t)M;
    a.N = (int32_t)N;
    a.K = (int32_t)K;
    const int64_t tm = (M + bm - 1) / bm, tn = (N + bn - 1) / bn;
    if (tm * tn > I32MAX) return fail(GGO_EUNSUPPORTED, "%s: too many tiles", fn);
    a.tiles_m = (int32_t)tm;
    a.tiles_n = (int32_t)tn;
    a.vec = VEC_A | VEC_W;
    if (aligned(C, 16) && ldc % 4 == 0) a.vec |= VEC_C;
    a.ep = no_epi();
    return launched(fn, launch_gemm_mfma_invariant_wt(a, bm, bn, s));
}

}  // extern "C"

static int run_gemv_mfma(const char* fn, const uint16_t* x, int64_t ldx, const uint16_t* WT, int64_t ldwt, void* y,
                         int64_t ldy, int64_t M, int64_t N, int64_t K, hipStream_t s, const Epi& ep, int rows = 0) {
    int rc = check_mnk(fn, M, N, K);
    if (rc) return rc;
    if (M > GGO_GEMV_MAX_M) return fail(GGO_EUNSUPPORTED, "%s: M=%lld exceeds %d", fn, (long long)M, GGO_GEMV_MAX_M);
    if (M == 0 || N == 0) return ok();
    if (!y || (K && (!x || !WT))) return fail(GGO_EINVAL, "%s: null pointer", fn);
    if (ldx < K || ldwt < K || ldy < N) return fail(GGO_EINVAL, "%s: row stride below extent", fn);
    if (K == 0) return launched(fn, epi_zero(y, ldy, M, N, ep, s));
    // 16-byte chunks through range-checked row descriptors: no chunk may straddle the end of a row
    if (!aligned(x, 16) || ldx % 8 || !aligned(WT, 16) || ldwt % 8 || K % 8)
        return fail(GGO_EUNSUPPORTED,
                    "%s: x and W^T must be 16-byte aligned with row strides and K multiples of 8 "
                    "(gemm_mfma_invariant takes any operands and gives the same bits)", fn);
    if (K > gemv_mfma_max_k())
        return fail(GGO_EUNSUPPORTED, "%s: K=%lld too large for 32-bit byte offsets along a row", fn, (long long)K);
    GemvMfmaArgs a;
    a.x = x;
    a.WT = WT;
    a.y = y;
    a.ldx = ldx;
    a.ldwt = ldwt;
    a.ldy = ldy;
    a.M = (int32_t)M;
    a.N = (int32_t)N;
    a.K = (int32_t)K;
    a.ep = ep;
    a.rows = rows;
    return launched(fn, launch_gemv_mfma(a, s));
}

extern "C" {

int gemv_mfma_invariant(const uint16_t* x, int64_t ldx, const uint16_t* WT, int64_t ldwt, float* y, int64_t ldy,
                        int64_t M, int64_t N, int64_t K, void* stream) {
    return run_gemv_mfma("gemv_mfma_invariant", x, ldx, WT, ldwt, y, ldy, M, N, K, static_cast<hipStream_t>(stream),
                         no_epi());
}

int gemv_mfma_invariant_ep(const uint16_t* x, int64_t ldx, const uint16_t* WT, int64_t ldwt, const ggo_epilogue* ep,
                           void* y, int64_t ldy, int64_t M, int64_t N, int64_t K, void* stream) {
    Epi e;
    int rc = make_epi("gemv_mfma_invariant_ep", ep, N, &e);
    if (rc) return rc;
    return run_gemv_mfma("gemv_mfma_invariant_ep", x, ldx, WT, ldwt, y, ldy, M, N, K, static_cast<hipStream_t>(stream), e);
}

int ggo_test_gemm_mfma_tile128(const uint16_t* A, int64_t lda, const uint16_t* W, int64_t ldw, float* C, int64_t ldc,
                               int64_t M, int64_t N, int64_t K, void* stream) {
    return run_mfma("ggo_test_gemm_mfma_tile128", A, lda, W, ldw, C, ldc, M, N, K, static_cast<hipStream_t>(stream),
                    MFMA_TILE_128x128, no_epi());
}

int ggo_test_gemm_mfma_tile(int tile, const uint16_t* A, int64_t lda, const uint16_t* W, int64_t ldw, float* C,
                            int64_t ldc, int64_t M, int64_t N, int64_t K, void* stream) {
    if (tile < GGO_TEST_MFMA_TILE_256x128 || tile > GGO_TEST_MFMA_TILE_64x128_LDS)
        return fail(GGO_EINVAL, "ggo_test_gemm_mfma_tile: unknown tile %d", tile);
    static_assert(GGO_TEST_MFMA_TILE_256x128 == MFMA_TILE_256x128 && GGO_TEST_MFMA_TILE_128x128 == MFMA_TILE_128x128 &&
                  GGO_TEST_MFMA_TILE_64x64 == MFMA_TILE_64x64 && GGO_TEST_MFMA_TILE_256x256 == MFMA_TILE_256x256 &&
                  GGO_TEST_MFMA_TILE_128x128_LDS == MFMA_TILE_128x128_LDS &&
                  GGO_TEST_MFMA_TILE_64x128_LDS == MFMA_TILE_64x128_LDS, "");
    return run_mfma("ggo_test_gemm_mfma_tile", A, lda, W, ldw, C, ldc, M, N, K, static_cast<hipStream_t>(stream), tile,
                    no_epi());
}

int ggo_test_gemv_instance(int kind, int rows, int form, const uint16_t* x, int64_t ldx, const uint16_t* W, int64_t ldw,
                           float* y, int64_t ldy, int64_t M, int64_t N, int64_t K, void* stream) {
    const char* fn = "ggo_test_gemv_instance";
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool tiered = kind == GGO_TEST_GEMV_TREE || kind == GGO_TEST_GEMV_MFMA;
    if (kind < GGO_TEST_GEMV_TREE || kind > GGO_TEST_GEMV_MFMA) return fail(GGO_EINVAL, "%s: unknown kind %d", fn, kind);
    if (tiered && !(rows == 1 || rows == 2 || rows == 4 || rows == 8 || rows == 16))
        return fail(GGO_EINVAL, "%s: rows must be 1, 2, 4, 8 or 16", fn);
    if (tiered && rows < M) return fail(GGO_EUNSUPPORTED, "%s: an instance staging %d rows cannot serve M=%lld", fn, rows, (long long)M);
    if (kind == GGO_TEST_GEMV_MFMA ? form != 0
        : kind == GGO_TEST_GEMV_TREE ? (form != 1 && form != 2)
        : kind == GGO_TEST_GEMV_ORDERED ? (form != 1 && form != 2)
                                        : (form < 1 || form > 4))
        return fail(GGO_EINVAL, "%s: form %d is not an instance of kind %d", fn, form, kind);
    // the ordered GEMV stages rows only in its MR-row instance (form 4): 2, 4 or 8 rows per workgroup, any M
    if (!tiered && form == 4 ? !(rows == 0 || rows == 2 || rows == 4 || rows == 8) : (!tiered && rows != 0))
        return fail(GGO_EINVAL, "%s: rows must be 0 for the ordered GEMV (or 0, 2, 4 or 8 for form 4)", fn);
    switch (kind) {
    case GGO_TEST_GEMV_TREE: return run_tree(fn, x, ldx, W, ldw, y, ldy, M, N, K, s, no_epi(), rows, form);
    case GGO_TEST_GEMV_ORDERED: return run_gemv_ordered(fn, 0, x, ldx, W, ldw, y, ldy, M, N, K, s, form);
    case GGO_TEST_GEMV_ORDERED_WT: return run_gemv_ordered(fn, 1, x, ldx, W, ldw, y, ldy, M, N, K, s, form, rows);
    default: return run_gemv_mfma(fn, x, ldx, W, ldw, y, ldy, M, N, K, s, no_epi(), rows);
    }
}

const char* ggo_build_info(void) { return GGO_BUILD_INFO; }

const char* ggo_last_error(void) { return g_err; }

}  // extern "C"
