// Ordered GEMV for decode shapes (few rows of x against a large W).
//
// Same order contract and bits as the ordered GEMM ("Reproducible GPU
// inference", section "Three interventions, and what each was worth"): lane
// (m, n) folds acc = acc + x[m,k]*W[k,n] over k = 0, 1, ..., K-1, product and
// sum rounded separately, starting from +0.0.
//
// Design for gfx950: every output is a K-long dependent chain, so one wave
// (64 lanes = 64 consecutive columns) owns one row m, and the grid spreads
// (64-column slice, group of 4 rows) over workgroups so that all M*N chains run
// at once. The four waves of a workgroup read the same W slice (coalesced
// 128-byte rows, shared through the CU's L1); their x rows are staged in LDS
// as binary32 and read as broadcasts.
#include "common.hpp"
#include "kernels.hpp"

#pragma clang fp contract(off)

namespace {

constexpr int THREADS = 256, ROWS = 4, COLS = 64;
constexpr int KCH = 1024;   // x staged in LDS in chunks of KCH k per row

__global__ __launch_bounds__(THREADS) void k_gemv_ordered(const GemvArgs a) {
    __shared__ float xs[ROWS][KCH];
    const int t = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
    const int m = blockIdx.y * ROWS + wv;
    const int n = blockIdx.x * COLS + (t & 63);
    const bool live = (m < a.M) && (n < a.N);
    const int rows_here = a.M - blockIdx.y * ROWS < ROWS ? a.M - blockIdx.y * ROWS : ROWS;
    const uint16_t* wcol = a.W + (n < a.N ? n : 0);
    float acc = 0.0f;

    for (int k0 = 0; k0 < a.K; k0 += KCH) {
        const int kb = a.K - k0 < KCH ? a.K - k0 : KCH;
        __syncthreads();
        for (int i = t; i < rows_here * KCH; i += THREADS) {
            const int r = i / KCH, kk = i - r * KCH;
            const int64_t row = blockIdx.y * ROWS + r;
            xs[r][kk] = kk < kb ? bf16_one(a.x[row * a.ldx + k0 + kk]) : 0.0f;
        }
        __syncthreads();
        if (live) {
            const uint16_t* wp = wcol + static_cast<int64_t>(k0) * a.ldw;
#pragma unroll 8
            for (int kk = 0; kk < kb; ++kk) {
                const float w = bf16_one(wp[static_cast<int64_t>(kk) * a.ldw]);
                const float p = xs[wv][kk] * w;   // first rounding
                acc = acc + p;                    // second rounding
            }
        }
    }
    if (live) a.y[static_cast<int64_t>(m) * a.ldy + n] = acc;
}

}  // namespace

hipError_t launch_gemv_ordered(const GemvArgs& a, hipStream_t stream) {
    const dim3 grid((a.N + COLS - 1) / COLS, (a.M + ROWS - 1) / ROWS);
    hipLaunchKernelGGL(k_gemv_ordered, grid, dim3(THREADS), 0, stream, a);
    return hipGetLastError();
}
