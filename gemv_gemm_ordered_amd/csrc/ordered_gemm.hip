// Ordered GEMM (and its grouped launch for the attention value product).
//
// Order contract ("Reproducible GPU inference", section "Three interventions,
// and what each was worth"): every output is one chain over ascending k of
// acc = acc + a*w with the product and the sum rounded separately; one lane
// owns each output; parallelism is only across outputs. Because the chain of an
// output never depends on which lane, tile or workgroup computes it, the bits
// cannot depend on M, on the tile size or on the number of compute units
// ("Taming Bitwise Behavior in GPU Kernels with Tensor Core", section 3.1: the
// dependence tree of each output is a left fold held in one thread's registers).
//
// Design for gfx950: a 64x64 output tile per 256-lane workgroup; each lane holds
// a 4x4 register micro-tile (16 independent chains, which keeps the VALU busy
// while each chain stays sequential). A and W tiles are read from HBM with
// 16-byte loads, widened to binary32 once, and staged in LDS (A transposed so a
// lane's four rows sit in one 16-byte LDS read). Tiles move through registers
// one step ahead of the arithmetic (prefetch), which moves loads but no adds.
// Built with -ffp-contract=off and the pragma below, so no mul/add pair is ever
// fused; packed binary32 ops are disabled at build time.
#include "common.hpp"
#include "kernels.hpp"

#pragma clang fp contract(off)

namespace {

constexpr int BM = 64, BN = 64, BK = 32, TM = 4, TN = 4, THREADS = 256;
constexpr int APAD = 4;

struct ATile { float v[8]; };
struct WTile { float v[8]; };

template <int AF32>
GGO_DEV void load_a(const OrdProblem& P, const void* Abase, int m0, int k0, int t, ATile& out) {
    const int r = t >> 2, kc = (t & 3) * 8;
    const int row = m0 + r, k = k0 + kc;
    const bool rowok = row < P.M;
    if (AF32) {
        const float* A = static_cast<const float*>(Abase) + static_cast<int64_t>(row) * P.lda + k;
        if (rowok && k + 8 <= P.K && (P.vec & VEC_A)) {
            const float4 a0 = reinterpret_cast<const float4*>(A)[0];
            const float4 a1 = reinterpret_cast<const float4*>(A)[1];
            out.v[0] = a0.x; out.v[1] = a0.y; out.v[2] = a0.z; out.v[3] = a0.w;
            out.v[4] = a1.x; out.v[5] = a1.y; out.v[6] = a1.z; out.v[7] = a1.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) out.v[i] = (rowok && k + i < P.K) ? A[i] : 0.0f;
        }
    } else {
        const uint16_t* A = static_cast<const uint16_t*>(Abase) + static_cast<int64_t>(row) * P.lda + k;
        if (rowok && k + 8 <= P.K && (P.vec & VEC_A)) {
            const uint4 q = *reinterpret_cast<const uint4*>(A);
            out.v[0] = bf16_lo(q.x); out.v[1] = bf16_hi(q.x); out.v[2] = bf16_lo(q.y); out.v[3] = bf16_hi(q.y);
            out.v[4] = bf16_lo(q.z); out.v[5] = bf16_hi(q.z); out.v[6] = bf16_lo(q.w); out.v[7] = bf16_hi(q.w);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) out.v[i] = (rowok && k + i < P.K) ? bf16_one(A[i]) : 0.0f;
        }
    }
}

GGO_DEV void load_w(const OrdProblem& P, const uint16_t* Wb, int n0, int k0, int t, WTile& out) {
    const int kr = t >> 3, nc = (t & 7) * 8;
    const int k = k0 + kr, n = n0 + nc;
    const uint16_t* W = Wb + static_cast<int64_t>(k) * P.ldw + n;
    if (k < P.K && n + 8 <= P.N && (P.vec & VEC_W)) {
        const uint4 q = *reinterpret_cast<const uint4*>(W);
        out.v[0] = bf16_lo(q.x); out.v[1] = bf16_hi(q.x); out.v[2] = bf16_lo(q.y); out.v[3] = bf16_hi(q.y);
        out.v[4] = bf16_lo(q.z); out.v[5] = bf16_hi(q.z); out.v[6] = bf16_lo(q.w); out.v[7] = bf16_hi(q.w);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) out.v[i] = (k < P.K && n + i < P.N) ? bf16_one(W[i]) : 0.0f;
    }
}

GGO_DEV void store_tiles(float (*As)[BM + APAD], float (*Ws)[BN], int t, const ATile& a, const WTile& w) {
    const int r = t >> 2, kc = (t & 3) * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) As[kc + i][r] = a.v[i];
    const int kr = t >> 3, nc = (t & 7) * 8;
    *reinterpret_cast<float4*>(&Ws[kr][nc]) = make_float4(w.v[0], w.v[1], w.v[2], w.v[3]);
    *reinterpret_cast<float4*>(&Ws[kr][nc + 4]) = make_float4(w.v[4], w.v[5], w.v[6], w.v[7]);
}

// One step of every chain the lane owns: acc[i][j] = acc[i][j] + (a[i] * w[j]).
GGO_DEV void fold_step(float (&acc)[TM][TN], const float (*As)[BM + APAD], const float (*Ws)[BN],
                       int kk, int ty, int tx) {
    const float4 a4 = *reinterpret_cast<const float4*>(&As[kk][ty * TM]);
    const float4 w4 = *reinterpret_cast<const float4*>(&Ws[kk][tx * TN]);
    const float a[TM] = {a4.x, a4.y, a4.z, a4.w};
    const float w[TN] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const float p = a[i] * w[j];   // first rounding
            acc[i][j] = acc[i][j] + p;     // second rounding
        }
}

template <int AF32>
__global__ __launch_bounds__(THREADS) void k_gemm_ordered(const OrdGroup g) {
    __shared__ __attribute__((aligned(16))) float As[BK][BM + APAD];
    __shared__ __attribute__((aligned(16))) float Ws[BK][BN];

    // which problem, which batch entry, which tile
    const int tile = xcd_contiguous(blockIdx.x, gridDim.x);
    int pi = 0;
    while (pi + 1 < g.count && tile >= g.tile_start[pi + 1]) ++pi;
    const OrdProblem& P = g.p[pi];
    const int local = tile - g.tile_start[pi];
    const int per_batch = P.tiles_m * P.tiles_n;
    const int b = local / per_batch, tt = local - b * per_batch;
    const int tm = tt / P.tiles_n, tn = tt - tm * P.tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;

    const void* Ab = AF32 ? static_cast<const void*>(static_cast<const float*>(P.A) + b * P.sa)
                          : static_cast<const void*>(static_cast<const uint16_t*>(P.A) + b * P.sa);
    const uint16_t* Wb = P.W + b * P.sw;
    float* Cb = P.C + b * P.sc;

    const int t = threadIdx.x, tx = t & 15, ty = t >> 4;
    float acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = 0.0f;   // +0.0: the chain's start

    const int nkt = (P.K + BK - 1) / BK;
    ATile ra;
    WTile rw;
    if (nkt > 0) {
        load_a<AF32>(P, Ab, m0, 0, t, ra);
        load_w(P, Wb, n0, 0, t, rw);
        store_tiles(As, Ws, t, ra, rw);
    }
    __syncthreads();
    for (int kt = 0; kt < nkt; ++kt) {
        const int k0 = kt * BK;
        if (kt + 1 < nkt) {                       // next tile in flight while this one folds
            load_a<AF32>(P, Ab, m0, k0 + BK, t, ra);
            load_w(P, Wb, n0, k0 + BK, t, rw);
        }
        const int kb = P.K - k0 < BK ? P.K - k0 : BK;
        if (kb == BK) {
#pragma unroll 8
            for (int kk = 0; kk < BK; ++kk) fold_step(acc, As, Ws, kk, ty, tx);
        } else {
            for (int kk = 0; kk < kb; ++kk) fold_step(acc, As, Ws, kk, ty, tx);
        }
        __syncthreads();
        if (kt + 1 < nkt) {
            store_tiles(As, Ws, t, ra, rw);
            __syncthreads();
        }
    }

#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int row = m0 + ty * TM + i;
        if (row >= P.M) break;
        const int col = n0 + tx * TN;
        float* c = Cb + static_cast<int64_t>(row) * P.ldc + col;
        if (col + TN <= P.N && (P.vec & VEC_C)) {
            *reinterpret_cast<float4*>(c) = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
        } else {
#pragma unroll
            for (int j = 0; j < TN; ++j)
                if (col + j < P.N) c[j] = acc[i][j];
        }
    }
}

}  // namespace

void ordered_tile_shape(int* bm, int* bn) { *bm = BM; *bn = BN; }

hipError_t launch_gemm_ordered(const OrdGroup& g, int total_tiles, int a_f32, hipStream_t stream) {
    if (a_f32)
        hipLaunchKernelGGL(k_gemm_ordered<1>, dim3(total_tiles), dim3(THREADS), 0, stream, g);
    else
        hipLaunchKernelGGL(k_gemm_ordered<0>, dim3(total_tiles), dim3(THREADS), 0, stream, g);
    return hipGetLastError();
}
