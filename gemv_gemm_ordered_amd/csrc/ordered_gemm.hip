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
// while each chain stays sequential). Small weights take a 16x16 tile with one
// output per lane instead (see Tile below). A and W tiles are read from HBM with
// 16-byte loads, widened to binary32 once, and staged in LDS (A transposed so a
// lane's four rows sit in one 16-byte LDS read; on the one-output tile A by rows
// and W by columns, so a lane's four k do). Tiles move through registers
// one step ahead of the arithmetic (prefetch), which moves loads but no adds.
// Built with -ffp-contract=off and the pragma below, so no mul/add pair is ever
// fused; packed binary32 ops are disabled at build time.
#include "common.hpp"
#include "kernels.hpp"

#pragma clang fp contract(off)

namespace {

constexpr int THREADS = 256, APAD = 4;

// Tile shapes. All give every output the same chain, so the same bits; which one a launch uses
// depends only on the weight's shape and the entry point, never on M.
//   Big:   64 x 64 outputs, 32-k steps, a 4 x 4 micro-tile per lane (16 chains: the VALU stays busy).
//   Mid:   64 x 32 outputs, 32-k steps, a 4 x 2 micro-tile (8 chains), for weights of 2^20 < N K <=
//          2^22: twice the workgroups of the big tile at every M, so at M = 256 on a 1024 x 4096 weight
//          each SIMD holds two waves instead of one (one wave alone issues binary32 operations at
//          about half the rate two waves reach).
//   Small: 16 x 16 outputs, 128-k steps, one output per lane, for small weights (N K <= 2^20): at
//          M <= 64 the big tile leaves most CUs idle (12 workgroups for a 768 x 768 weight) and each
//          lane's 16 chains run one after another.
// DEPTH: k-steps of A and W in flight in registers ahead of the one being folded.
template <int BM_, int BN_, int BK_, int TM_, int TN_, int DEPTH_> struct Tile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, TM = TM_, TN = TN_, DEPTH = DEPTH_;
    static constexpr int CA = BK / 8, CW = BN / 8;   // 8-element chunks per A row / per W k-row
    static constexpr int WCH = BK * CW;               // W chunks per k-step: threads 0 .. WCH-1 load one each
    static_assert(BM * CA == THREADS && WCH <= THREADS && WCH % 64 == 0,
                  "each thread loads one chunk of A; whole waves load one chunk of W each");
    static_assert((BM / TM) * (BN / TN) == THREADS, "one micro-tile per lane");
};
// two k-steps in flight on the micro-tile instances (with two LDS stages; MLP weight M = 256 / 512 /
// 2048 and 4096 x 4096 at M = 2048: 3-9% faster than one step, three steps level with two)
using BigTile = Tile<64, 64, 32, 4, 4, 2>;
using MidTile = Tile<64, 32, 32, 4, 2, 2>;
using SmallTile = Tile<16, 16, 128, 1, 1, 1>;   // deeper rings measured no faster

// One 8-element chunk as loaded: bf16 pairs in u[0..3] (element 2i in the low half of u[i]) or eight
// binary32 in u[0..7]. It is widened only when stored to LDS, so the loads of the next k-step stay in
// flight while the current one is folded (widening at load time made every load wait at once).
struct Chunk { uint32_t u[8]; };

template <class T, int AF32>
GGO_DEV void load_a(const OrdProblem& P, const void* Abase, int m0, int k0, int t, Chunk& out) {
    const int r = t / T::CA, kc = (t % T::CA) * 8;
    const int row = m0 + r, k = k0 + kc;
    const bool rowok = row < P.M;
    if (AF32) {
        const float* A = static_cast<const float*>(Abase) + static_cast<int64_t>(row) * P.lda + k;
        if (rowok && k + 8 <= P.K && (P.vec & VEC_A)) {
            const uint4 a0 = reinterpret_cast<const uint4*>(A)[0];
            const uint4 a1 = reinterpret_cast<const uint4*>(A)[1];
            out.u[0] = a0.x; out.u[1] = a0.y; out.u[2] = a0.z; out.u[3] = a0.w;
            out.u[4] = a1.x; out.u[5] = a1.y; out.u[6] = a1.z; out.u[7] = a1.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) out.u[i] = (rowok && k + i < P.K) ? __float_as_uint(A[i]) : 0u;
        }
    } else {
        const uint16_t* A = static_cast<const uint16_t*>(Abase) + static_cast<int64_t>(row) * P.lda + k;
        if (rowok && k + 8 <= P.K && (P.vec & VEC_A)) {
            const uint4 q = *reinterpret_cast<const uint4*>(A);
            out.u[0] = q.x; out.u[1] = q.y; out.u[2] = q.z; out.u[3] = q.w;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t lo = (rowok && k + 2 * i < P.K) ? A[2 * i] : 0u;
                const uint32_t hi = (rowok && k + 2 * i + 1 < P.K) ? A[2 * i + 1] : 0u;
                out.u[i] = lo | (hi << 16);
            }
        }
    }
}

template <class T>
GGO_DEV void load_w(const OrdProblem& P, const uint16_t* Wb, int n0, int k0, int t, Chunk& out) {
    if (T::WCH < THREADS && t >= T::WCH) return;   // uniform per wave: this wave loads no W
    const int kr = t / T::CW, nc = (t % T::CW) * 8;
    const int k = k0 + kr, n = n0 + nc;
    const uint16_t* W = Wb + static_cast<int64_t>(k) * P.ldw + n;
    if (k < P.K && n + 8 <= P.N && (P.vec & VEC_W)) {
        const uint4 q = *reinterpret_cast<const uint4*>(W);
        out.u[0] = q.x; out.u[1] = q.y; out.u[2] = q.z; out.u[3] = q.w;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = (k < P.K && n + 2 * i < P.N) ? W[2 * i] : 0u;
            const uint32_t hi = (k < P.K && n + 2 * i + 1 < P.N) ? W[2 * i + 1] : 0u;
            out.u[i] = lo | (hi << 16);
        }
    }
}

// Wide form: every operand 16-byte aligned with row strides, K and N multiples of 8, so no chunk
// straddles the end of a row. Loads go through range-checked buffer descriptors: rows past M (A) or
// past K (W) lie past the range and read 0, and chunks past K (A) or past N (W) inside a row get an
// offset past every range. No per-lane branch surrounds a load, so nothing forces it to land before
// the k-step that needs it.
constexpr int BUF_DWORD3 = 0x00020000;   // buffer descriptor word 3: raw 32-bit data, range checked
constexpr int OUT_OF_RANGE = 0x7ffffff0;

template <class T, int AF32>
GGO_DEV void load_a_wide(const OrdProblem& P, const void* Abase, int m0, int k0, int t, Chunk& out) {
    constexpr int ESZ = AF32 ? 4 : 2;
    const int r = t / T::CA, kc = (t % T::CA) * 8;
    const int rows = P.M - m0 < T::BM ? P.M - m0 : T::BM;
    const char* base = static_cast<const char*>(Abase) + static_cast<int64_t>(m0) * P.lda * ESZ;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(base), 0, ((rows - 1) * static_cast<int>(P.lda) + P.K) * ESZ, BUF_DWORD3);
    const int off = (r < rows && k0 + kc < P.K) ? (r * static_cast<int>(P.lda) + k0 + kc) * ESZ : OUT_OF_RANGE;
    const auto q0 = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    out.u[0] = q0[0]; out.u[1] = q0[1]; out.u[2] = q0[2]; out.u[3] = q0[3];
    if (AF32) {
        const auto q1 = __builtin_amdgcn_raw_buffer_load_b128(rs, off == OUT_OF_RANGE ? OUT_OF_RANGE : off + 16, 0, 0);
        out.u[4] = q1[0]; out.u[5] = q1[1]; out.u[6] = q1[2]; out.u[7] = q1[3];
    }
}

template <class T>
GGO_DEV void load_w_wide(const OrdProblem& P, const uint16_t* Wb, int n0, int k0, int t, Chunk& out) {
    if (T::WCH < THREADS && t >= T::WCH) return;   // uniform per wave: this wave loads no W
    const int kr = t / T::CW, nc = (t % T::CW) * 8;
    const int krows = P.K - k0 < T::BK ? P.K - k0 : T::BK;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(Wb) + static_cast<int64_t>(k0) * P.ldw + n0, 0,
        ((krows - 1) * static_cast<int>(P.ldw) + (P.N - n0)) * 2, BUF_DWORD3);
    const int off = (kr < krows && n0 + nc < P.N) ? (kr * static_cast<int>(P.ldw) + nc) * 2 : OUT_OF_RANGE;
    const auto q = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    out.u[0] = q[0]; out.u[1] = q[1]; out.u[2] = q[2]; out.u[3] = q[3];
}

// Element i of a chunk as binary32 (bf16 widening is exact).
template <int F32>
GGO_DEV float elem(const Chunk& c, int i) {
    if (F32) return __uint_as_float(c.u[i]);
    return (i & 1) ? bf16_hi(c.u[i >> 1]) : bf16_lo(c.u[i >> 1]);
}

template <class T, int AF32>
GGO_DEV void store_tiles(float (*As)[T::BM + APAD], float (*Ws)[T::BN], int t, const Chunk& a, const Chunk& w) {
    const int r = t / T::CA, kc = (t % T::CA) * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) As[kc + i][r] = elem<AF32>(a, i);
    if (T::WCH < THREADS && t >= T::WCH) return;   // uniform per wave
    const int kr = t / T::CW, nc = (t % T::CW) * 8;
    *reinterpret_cast<float4*>(&Ws[kr][nc]) = make_float4(elem<0>(w, 0), elem<0>(w, 1), elem<0>(w, 2), elem<0>(w, 3));
    *reinterpret_cast<float4*>(&Ws[kr][nc + 4]) = make_float4(elem<0>(w, 4), elem<0>(w, 5), elem<0>(w, 6), elem<0>(w, 7));
}

// One-output tile: LDS holds the rows of A and the columns of W with k contiguous (each row padded by 4
// floats, so the 4 rows of A and the 16 columns of W a wave reads fall on distinct banks), and a lane takes
// 4 k of its row and of its column with one 16-byte read each. The thread's chunk of A (one row, 8 k)
// goes into its row with two 16-byte writes; its chunk of W (one k-row, 8 columns) into 8 columns.
template <class T, int AF32>
GGO_DEV void store_rows(float (*A1)[T::BK + 4], float (*W1)[T::BK + 4], int t, const Chunk& a, const Chunk& w) {
    const int r = t / T::CA, kc = (t % T::CA) * 8;
    *reinterpret_cast<float4*>(&A1[r][kc]) = make_float4(elem<AF32>(a, 0), elem<AF32>(a, 1), elem<AF32>(a, 2), elem<AF32>(a, 3));
    *reinterpret_cast<float4*>(&A1[r][kc + 4]) = make_float4(elem<AF32>(a, 4), elem<AF32>(a, 5), elem<AF32>(a, 6), elem<AF32>(a, 7));
    if (T::WCH < THREADS && t >= T::WCH) return;   // uniform per wave
    const int kr = t / T::CW, nc = (t % T::CW) * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) W1[nc + i][kr] = elem<0>(w, i);
}

// 4 x 2 tile: LDS holds the rows of A and the columns of W with k contiguous, so a lane reads 4 k of
// each of its 4 rows and 2 columns with 6 16-byte reads (8 with one k per read). Column n of W sits in row
// (n & 1) BN/2 + n/2 (rows padded by 4 floats): the 16 columns a wave reads together, and the 4 rows of A,
// then fall on distinct banks.
template <class T, int AF32>
GGO_DEV void store_rows2(float (*A2)[T::BK + 4], float (*W2)[T::BK + 4], int t, const Chunk& a, const Chunk& w) {
    const int r = t / T::CA, kc = (t % T::CA) * 8;
    *reinterpret_cast<float4*>(&A2[r][kc]) = make_float4(elem<AF32>(a, 0), elem<AF32>(a, 1), elem<AF32>(a, 2), elem<AF32>(a, 3));
    *reinterpret_cast<float4*>(&A2[r][kc + 4]) = make_float4(elem<AF32>(a, 4), elem<AF32>(a, 5), elem<AF32>(a, 6), elem<AF32>(a, 7));
    if (T::WCH < THREADS && t >= T::WCH) return;   // uniform per wave
    const int kr = t / T::CW, nc = (t % T::CW) * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int n = nc + i;
        W2[(n & 1) * (T::BN / 2) + (n >> 1)][kr] = elem<0>(w, i);
    }
}

// One step of every chain the lane owns: acc[i][j] = acc[i][j] + (a[i] * w[j]).
template <class T>
GGO_DEV void fold_step(float (&acc)[T::TM][T::TN], const float (*As)[T::BM + APAD], const float (*Ws)[T::BN],
                       int kk, int ty, int tx) {
    float a[T::TM], w[T::TN];
    if constexpr (T::TM == 4) {
        const float4 a4 = *reinterpret_cast<const float4*>(&As[kk][ty * 4]);
        a[0] = a4.x; a[1] = a4.y; a[2] = a4.z; a[3] = a4.w;
    } else {
#pragma unroll
        for (int i = 0; i < T::TM; ++i) a[i] = As[kk][ty * T::TM + i];
    }
    if constexpr (T::TN == 4) {
        const float4 w4 = *reinterpret_cast<const float4*>(&Ws[kk][tx * 4]);
        w[0] = w4.x; w[1] = w4.y; w[2] = w4.z; w[3] = w4.w;
    } else if constexpr (T::TN == 2) {
        const float2 w2 = *reinterpret_cast<const float2*>(&Ws[kk][tx * 2]);
        w[0] = w2.x; w[1] = w2.y;
    } else {
#pragma unroll
        for (int j = 0; j < T::TN; ++j) w[j] = Ws[kk][tx * T::TN + j];
    }
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
            const float p = a[i] * w[j];   // first rounding
            acc[i][j] = acc[i][j] + p;     // second rounding
        }
}

template <class T, int AF32, bool WIDE>
__global__ __launch_bounds__(THREADS) void k_gemm_ordered(const OrdGroup g) {
    constexpr int BM = T::BM, BN = T::BN, BK = T::BK, TM = T::TM, TN = T::TN;
    // Two LDS stages: step kt + 1 is stored into the other stage while the slower lanes may still be
    // folding step kt, so a k-step needs one barrier instead of two (MLP weight M = 256 / 512: 32.3 -> 34.2
    // / 39.1 -> 41.2 TFLOP/s; 4096 x 4096 at M = 2048 52.2 -> 54.6; the one-output tile's GPT-2 projection
    // 9.0 - 9.8 -> 8.8 - 9.4 us at M <= 64, 27.0 -> 26.6 at M = 512).
    constexpr int NSTG = 2;
    __shared__ __attribute__((aligned(16))) float AsB[NSTG][BK][BM + APAD];
    __shared__ __attribute__((aligned(16))) float WsB[NSTG][BK][BN];
    // the one-output tile's rows of A and columns of W (store_rows); the arrays an instance never touches
    // take no LDS
    constexpr bool ONE = T::TM * T::TN == 1;
    __shared__ __attribute__((aligned(16))) float A1S[ONE ? NSTG : 1][ONE ? BM : 1][BK + 4];
    __shared__ __attribute__((aligned(16))) float W1S[ONE ? NSTG : 1][ONE ? BN : 1][BK + 4];
    // the 4 x 2 tile's rows of A and columns of W (store_rows2)
    constexpr bool ROWS2 = T::TM == 4 && T::TN == 2;
    __shared__ __attribute__((aligned(16))) float A2S[ROWS2 ? NSTG : 1][ROWS2 ? BM : 1][BK + 4];
    __shared__ __attribute__((aligned(16))) float W2S[ROWS2 ? NSTG : 1][ROWS2 ? BN : 1][BK + 4];

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

    const int t = threadIdx.x, tx = t % (BN / TN), ty = t / (BN / TN);
    float acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = 0.0f;   // +0.0: the chain's start

    // Register ring of DEPTH k-steps: step kt sits in slot kt % DEPTH until it is stored to LDS; the
    // k loop is unrolled by DEPTH so every slot index is static. Loads move ahead; the adds do not.
    constexpr int D = T::DEPTH;
    const int nkt = (P.K + BK - 1) / BK;
    Chunk ra[D], rw[D];
#pragma unroll
    for (int d = 0; d < D; ++d)
        if (d < nkt) {
            if constexpr (WIDE) {
                load_a_wide<T, AF32>(P, Ab, m0, d * BK, t, ra[d]);
                load_w_wide<T>(P, Wb, n0, d * BK, t, rw[d]);
            } else {
                load_a<T, AF32>(P, Ab, m0, d * BK, t, ra[d]);
                load_w<T>(P, Wb, n0, d * BK, t, rw[d]);
            }
        }
    if (nkt > 0) {
        if constexpr (ONE) store_rows<T, AF32>(A1S[0], W1S[0], t, ra[0], rw[0]);
        else if constexpr (ROWS2) store_rows2<T, AF32>(A2S[0], W2S[0], t, ra[0], rw[0]);
        else store_tiles<T, AF32>(AsB[0], WsB[0], t, ra[0], rw[0]);
    }
    __syncthreads();
    for (int kt0 = 0; kt0 < nkt; kt0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int kt = kt0 + d;
            if (kt >= nkt) break;                 // uniform
            const int k0 = kt * BK;
            if (kt + D < nkt) {                   // slot d is free: step kt is in LDS
                if constexpr (WIDE) {
                    load_a_wide<T, AF32>(P, Ab, m0, k0 + D * BK, t, ra[d]);
                    load_w_wide<T>(P, Wb, n0, k0 + D * BK, t, rw[d]);
                } else {
                    load_a<T, AF32>(P, Ab, m0, k0 + D * BK, t, ra[d]);
                    load_w<T>(P, Wb, n0, k0 + D * BK, t, rw[d]);
                }
            }
            const int kb = P.K - k0 < BK ? P.K - k0 : BK;
            const auto& As = AsB[kt & (NSTG - 1)];
            const auto& Ws = WsB[kt & (NSTG - 1)];
            const auto& A1 = A1S[ONE ? (kt & (NSTG - 1)) : 0];
            const auto& W1 = W1S[ONE ? (kt & (NSTG - 1)) : 0];
            const auto& A2 = A2S[ROWS2 ? (kt & (NSTG - 1)) : 0];
            const auto& W2 = W2S[ROWS2 ? (kt & (NSTG - 1)) : 0];
            if (kb == BK) {
                if constexpr (T::TM * T::TN == 1) {
                    // One output per lane and one wave per SIMD: nothing else hides the LDS latency, so
                    // the reads of the next 8 k (two 16-byte reads of the lane's row of A, two of its
                    // column of W) are issued before the adds of the current 8. With a 4-byte read per
                    // operand and k the GPT-2 projection took 13.0 - 13.3 us at M = 1 - 64 and 55 us at
                    // M = 512, against 9.1 - 9.8 and 27 (same bits).
                    constexpr int CH = 8, NCH = BK / CH;
                    float4 av[2][2], wv[2][2];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        av[0][h] = *reinterpret_cast<const float4*>(&A1[ty][4 * h]);
                        wv[0][h] = *reinterpret_cast<const float4*>(&W1[tx][4 * h]);
                    }
#pragma unroll
                    for (int c = 0; c < NCH; ++c) {
                        if (c + 1 < NCH) {
#pragma unroll
                            for (int h = 0; h < 2; ++h) {
                                av[(c + 1) & 1][h] = *reinterpret_cast<const float4*>(&A1[ty][(c + 1) * CH + 4 * h]);
                                wv[(c + 1) & 1][h] = *reinterpret_cast<const float4*>(&W1[tx][(c + 1) * CH + 4 * h]);
                            }
                        }
#pragma unroll
                        for (int h = 0; h < 2; ++h) {   // ascending k
                            const float4 a = av[c & 1][h], w = wv[c & 1][h];
                            float p = a.x * w.x;
                            acc[0][0] = acc[0][0] + p;
                            p = a.y * w.y;
                            acc[0][0] = acc[0][0] + p;
                            p = a.z * w.z;
                            acc[0][0] = acc[0][0] + p;
                            p = a.w * w.w;
                            acc[0][0] = acc[0][0] + p;
                        }
                    }
                } else if constexpr (T::TN == 4) {
                    // 4 x 4 micro-tile: the next k's two 16-byte reads are issued before this k's 32
                    // operations (the same reasoning at small M, where a CU holds one workgroup). Taking A
                    // through a DPP row broadcast instead (the 16 lanes of a row share their rows of A, so
                    // one 4-byte read per lane covers four k) measured slower: 36.7 against 50.2 TFLOP/s at
                    // M = 2048 on the 1024 x 4096 weight, same bits.
                    static_assert(T::TM == 4, "");
                    float4 a4[2], w4[2];
                    a4[0] = *reinterpret_cast<const float4*>(&As[0][ty * 4]);
                    w4[0] = *reinterpret_cast<const float4*>(&Ws[0][tx * 4]);
#pragma unroll
                    for (int kk = 0; kk < BK; ++kk) {
                        if (kk + 1 < BK) {
                            a4[(kk + 1) & 1] = *reinterpret_cast<const float4*>(&As[kk + 1][ty * 4]);
                            w4[(kk + 1) & 1] = *reinterpret_cast<const float4*>(&Ws[kk + 1][tx * 4]);
                        }
                        const float a[4] = {a4[kk & 1].x, a4[kk & 1].y, a4[kk & 1].z, a4[kk & 1].w};
                        const float w[4] = {w4[kk & 1].x, w4[kk & 1].y, w4[kk & 1].z, w4[kk & 1].w};
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                const float p = a[i] * w[j];   // first rounding
                                acc[i][j] = acc[i][j] + p;     // second rounding
                            }
                    }
                } else {
                    // 4 x 2 micro-tile, rows of A and columns of W: the next 4 k's six 16-byte reads are
                    // issued before this 4 k's 32 operations. With one k per read (a 16-byte read of A, an
                    // 8-byte read of W) the MLP weight took 50.3 / 61.7 / 102 / 343 us at M = 64 / 256 /
                    // 512 / 2048, against 48.0 / 54.2 / 94.9 / 325 (same bits).
                    static_assert(T::TM == 4 && T::TN == 2, "");
                    float4 a4[2][4], w4[2][2];
#pragma unroll
                    for (int i = 0; i < 4; ++i) a4[0][i] = *reinterpret_cast<const float4*>(&A2[ty * 4 + i][0]);
#pragma unroll
                    for (int j = 0; j < 2; ++j) w4[0][j] = *reinterpret_cast<const float4*>(&W2[j * (BN / 2) + tx][0]);
#pragma unroll
                    for (int k4 = 0; k4 < BK / 4; ++k4) {
                        if (k4 + 1 < BK / 4) {
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                a4[(k4 + 1) & 1][i] = *reinterpret_cast<const float4*>(&A2[ty * 4 + i][4 * (k4 + 1)]);
#pragma unroll
                            for (int j = 0; j < 2; ++j)
                                w4[(k4 + 1) & 1][j] = *reinterpret_cast<const float4*>(&W2[j * (BN / 2) + tx][4 * (k4 + 1)]);
                        }
#pragma unroll
                        for (int e = 0; e < 4; ++e) {   // ascending k
                            float a[4], w[2];
#pragma unroll
                            for (int i = 0; i < 4; ++i) a[i] = (&a4[k4 & 1][i].x)[e];
#pragma unroll
                            for (int j = 0; j < 2; ++j) w[j] = (&w4[k4 & 1][j].x)[e];
#pragma unroll
                            for (int i = 0; i < 4; ++i)
#pragma unroll
                                for (int j = 0; j < 2; ++j) {
                                    const float p = a[i] * w[j];   // first rounding
                                    acc[i][j] = acc[i][j] + p;     // second rounding
                                }
                        }
                    }
                }
            } else if constexpr (ROWS2) {
                for (int kk = 0; kk < kb; ++kk)   // the partial last step, ascending k
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 2; ++j) {
                            const float p = A2[ty * 4 + i][kk] * W2[j * (BN / 2) + tx][kk];
                            acc[i][j] = acc[i][j] + p;
                        }
            } else if constexpr (ONE) {
                for (int kk = 0; kk < kb; ++kk) {   // the partial last step, ascending k
                    const float p = A1[ty][kk] * W1[tx][kk];
                    acc[0][0] = acc[0][0] + p;
                }
            } else {
                for (int kk = 0; kk < kb; ++kk) fold_step<T>(acc, As, Ws, kk, ty, tx);
            }
            // the other stage was last read in step kt - 1, before the barrier that ended it
            if (kt + 1 < nkt) {
                if constexpr (ONE) store_rows<T, AF32>(A1S[(kt + 1) & 1], W1S[(kt + 1) & 1], t, ra[(d + 1) % D], rw[(d + 1) % D]);
                else if constexpr (ROWS2) store_rows2<T, AF32>(A2S[(kt + 1) & 1], W2S[(kt + 1) & 1], t, ra[(d + 1) % D], rw[(d + 1) % D]);
                else store_tiles<T, AF32>(AsB[(kt + 1) & 1], WsB[(kt + 1) & 1], t, ra[(d + 1) % D], rw[(d + 1) % D]);
            }
            __syncthreads();
        }
    }

#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int row = m0 + ty * TM + i;
        if (row >= P.M) break;
        const int col = n0 + tx * TN;
        float* c = Cb + static_cast<int64_t>(row) * P.ldc + col;
        bool done = false;
        if constexpr (TN == 4) {
            if (col + TN <= P.N && (P.vec & VEC_C)) {
                *reinterpret_cast<float4*>(c) = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
                done = true;
            }
        } else if constexpr (TN == 2) {
            if (col + TN <= P.N && (P.vec & VEC_C)) {
                *reinterpret_cast<float2*>(c) = make_float2(acc[i][0], acc[i][1]);
                done = true;
            }
        }
        if (!done) {
#pragma unroll
            for (int j = 0; j < TN; ++j)
                if (col + j < P.N) c[j] = acc[i][j];
        }
    }
}

}  // namespace

void ordered_tile_shape(int kind, int* bm, int* bn) {
    *bm = kind == ORD_TILE_SMALL ? SmallTile::BM : kind == ORD_TILE_MID ? MidTile::BM : BigTile::BM;
    *bn = kind == ORD_TILE_SMALL ? SmallTile::BN : kind == ORD_TILE_MID ? MidTile::BN : BigTile::BN;
}

template <class T>
void launch_tile(const OrdGroup& g, int total_tiles, int a_f32, int wide, hipStream_t stream) {
    const dim3 grid(total_tiles), block(THREADS);
    if (wide) {
        if (a_f32) hipLaunchKernelGGL((k_gemm_ordered<T, 1, true>), grid, block, 0, stream, g);
        else hipLaunchKernelGGL((k_gemm_ordered<T, 0, true>), grid, block, 0, stream, g);
    } else {
        if (a_f32) hipLaunchKernelGGL((k_gemm_ordered<T, 1, false>), grid, block, 0, stream, g);
        else hipLaunchKernelGGL((k_gemm_ordered<T, 0, false>), grid, block, 0, stream, g);
    }
}

hipError_t launch_gemm_ordered(const OrdGroup& g, int total_tiles, int a_f32, int kind, int wide, hipStream_t stream) {
    if (kind == ORD_TILE_SMALL) launch_tile<SmallTile>(g, total_tiles, a_f32, wide, stream);
    else if (kind == ORD_TILE_MID) launch_tile<MidTile>(g, total_tiles, a_f32, wide, stream);
    else launch_tile<BigTile>(g, total_tiles, a_f32, wide, stream);
    return hipGetLastError();
}

// Largest row stride (elements) the wide form takes: its byte ranges and offsets stay below 2^30.
int64_t ordered_wide_max_ld(int kind, int a_f32) {
    const int64_t rows = kind == ORD_TILE_SMALL ? (SmallTile::BK > SmallTile::BM ? SmallTile::BK : SmallTile::BM)
                       : kind == ORD_TILE_MID   ? (MidTile::BK > MidTile::BM ? MidTile::BK : MidTile::BM)
                                                : (BigTile::BK > BigTile::BM ? BigTile::BK : BigTile::BM);
    return (int64_t(1) << 30) / ((rows + 1) * (a_f32 ? 4 : 2));
}
