// Ordered GEMV for decode shapes (few rows of x against a large W).
//
// Same order contract and bits as the ordered GEMM ("Reproducible GPU
// inference", section "Three interventions, and what each was worth"): lane
// (m, n) folds acc = acc + x[m,k]*W[k,n] over k = 0, 1, ..., K-1, product and
// sum rounded separately, starting from +0.0.
//
// Why the kernel is split into producers and a consumer. Every output is a
// K-long chain of dependent binary32 adds held in one lane, and a gfx950 wave
// issues about one VALU instruction every 4.5 clocks, so the chain costs at
// least K * 4.5 clocks and every other instruction the owning wave issues per
// k (the multiply, the bf16 widening, the loads) lengthens it. Here the owning
// wave issues nothing per k but the add, plus one 16-byte LDS read per four k;
// separate producer waves stream W, widen it, multiply it by x and leave the
// rounded products in LDS. A product is the same binary32 value whichever
// lane rounds it, so moving the multiply to another wave moves no bits
// ("Taming Bitwise Behavior in GPU Kernels with Tensor Core", section 3.1:
// warp specialisation and pipelining leave the dependence tree unchanged).
//
// Workgroup = 16 output columns x 8 output rows, six waves:
//   waves 0, 1   consumers: lane (r, c) = (lane / 16, lane % 16) of wave w owns
//                y[m0 + 4w + r, n0 + c]
//   waves 2 - 5  producers: lane q owns the 4(k) x 2(n) block (kq, np) of each
//                64-k stage, for rows 4h .. 4h+3 (h = 0 for waves 2-3, 1 for 4-5)
// Stages of products rotate through NBUF LDS buffers; the consumers run two
// stages behind the producers so their LDS reads overlap the previous stage's
// adds. W and x are prefetched DEPTH stages ahead in registers. Waves whose
// rows all lie past M only keep the barrier count.
//
// Operands are read with raw buffer loads whose descriptors end exactly at the
// last element the caller owns, so a load past that end returns 0 without
// touching memory. That pads K to whole stages with W = 0 and x = 0: the
// padded products are +0 (0 * 0), and acc + (+0) == acc for every value a
// +0-started fold can hold (it is never -0), so the padding changes no bit.
// Columns past N only feed chains that are never stored. The grid is
// ceil(N/16) x ceil(M/8) workgroups, and each workgroup's column slice is
// mapped XCD-contiguously so that slices sharing an L2 line run under one L2.
//
// W^T form (WT): the weight arrives as W^T [N, K], k contiguous, as a linear
// layer stores it. A producer lane then loads 4 consecutive k of each of its
// two weight rows with one 8-byte load per row, so a workgroup's 16 rows are
// read in 128-byte runs per stage instead of the 32-byte column slices of
// W [K, N]. One descriptor covers the workgroup's slab of rows; a load for a
// row past N or a k past K gets an offset beyond that range and returns 0.
// The products, their order and the consumers are those of the W [K, N] form,
// and so are the bits.
#include <type_traits>


#include "common.hpp"
#include "kernels.hpp"

#pragma clang fp contract(off)

namespace {

constexpr int NS = 16;                 // output columns per workgroup
constexpr int RG = 8;                  // output rows per workgroup
constexpr int KC = 64;                 // k per stage
constexpr int NBUF = 4;                // product stages resident in LDS
constexpr int RUN = KC;                // floats per (row, column) run of products
constexpr int NQ = KC / 4;             // 16-byte consumer reads per stage
constexpr int CONSUMERS = RG / 4;      // consumer waves (4 rows x 16 columns each)
constexpr int THREADS = 64 * CONSUMERS + 256;
constexpr int TASKS = (KC / 4) * (NS / 2);   // 4(k) x 2(n) product blocks per stage
constexpr int BUF_DWORD3 = 0x00020000; // buffer descriptor word 3: raw 32-bit data, range checked

static_assert(2 * TASKS == 256, "two producer lanes (row halves) per block");

// Position of the 4 products (k4*4 .. k4*4+3) of run `run` (= row*NS + column)
// inside a stage buffer. The 16-byte slot index is XOR-swizzled so that both
// the producers' writes (8 lanes: one kq, columns 0,2,..,14 or 1,3,..,15) and
// the consumers' reads (8 lanes: 8 consecutive runs, one k4) fall in 8
// distinct groups of 4 banks.
GGO_DEV int slot(int run, int k4) { return run * RUN + ((k4 ^ ((run + (run >> 3)) & 7)) << 2); }

// One stage of one producer lane, as loaded: W[k+i][n .. n+1] and
// x[m0+4h+j][k .. k+3]. WIDE: one 4-byte load per W pair and one 8-byte load
// per x quad (8 loads). Otherwise one 2-byte load per element (24 loads), for
// operands whose alignment or extents rule the wide loads out.
template <bool WIDE> struct Fetch;
template <> struct Fetch<true> {
    uint32_t w[4];
    uint2 x[4];
};
template <> struct Fetch<false> {
    uint16_t w[4][2];
    uint16_t x[4][4];
};

// W^T form: rows n and n+1 of W^T at the lane's 4 k, one 8-byte load each, and x as in Fetch<true>.
struct FetchT {
    uint2 w[2];
    uint2 x[4];
};

// Per-lane constants: byte offsets of the lane's W elements inside a stage,
// the lane's byte offset into a row of x, and the descriptors of its x rows.
// W^T form: the slab descriptor, the byte offsets of the lane's two rows at
// k = 4 kq (relative to the slab), the lane's first k, and which rows are live.
struct Lane {
    int wof[4][2];
    int xof;
    __amdgpu_buffer_rsrc_t xr[4];
    __amdgpu_buffer_rsrc_t wt;
    int tof[2];
    int k4;
    bool tlive[2];
};

constexpr int OUT_OF_RANGE = 0x7ffffff0;   // a buffer offset past every slab range: the load returns 0

// W descriptor of one stage: it starts at row stage*KC and ends right after
// column N-1 of the stage's last row, so nothing past the elements the caller
// owns is read (lanes of columns past N in that row, and rows past K, read 0);
// stages wholly past K have an empty range.
GGO_DEV __amdgpu_buffer_rsrc_t w_rsrc(const GemvArgs& a, int stage) {
    const int rows_left = a.K - stage * KC;
    const int rows_in = rows_left < KC ? rows_left : KC;
    const int nrec = rows_left <= 0 ? 0 : ((rows_in - 1) * static_cast<int>(a.ldw) + a.N) * 2;
    const int64_t row0 = rows_left <= 0 ? 0 : static_cast<int64_t>(stage) * KC;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.W) + row0 * a.ldw, 0, nrec, BUF_DWORD3);
}

GGO_DEV void fetch(const GemvArgs& a, const Lane& L, int stage, Fetch<true>& f) {
    const __amdgpu_buffer_rsrc_t wr = w_rsrc(a, stage);
#pragma unroll
    for (int i = 0; i < 4; ++i) f.w[i] = __builtin_amdgcn_raw_buffer_load_b32(wr, L.wof[i][0], 0, 0);
    const int xo = L.xof + stage * KC * 2;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(L.xr[j], xo, 0, 0);
        f.x[j] = make_uint2(v[0], v[1]);
    }
}

GGO_DEV void fetch(const GemvArgs& a, const Lane& L, int stage, Fetch<false>& f) {
    const __amdgpu_buffer_rsrc_t wr = w_rsrc(a, stage);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) f.w[i][j] = __builtin_amdgcn_raw_buffer_load_b16(wr, L.wof[i][j], 0, 0);
    const int xo = L.xof + stage * KC * 2;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) f.x[j][i] = __builtin_amdgcn_raw_buffer_load_b16(L.xr[j], xo + 2 * i, 0, 0);
}

GGO_DEV void fetch(const GemvArgs& a, const Lane& L, int stage, FetchT& f) {
    const bool kin = stage * KC + L.k4 < a.K;   // K % 4 == 0: the lane's 4 k lie wholly inside or past K
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int off = (kin && L.tlive[j]) ? L.tof[j] + stage * KC * 2 : OUT_OF_RANGE;
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(L.wt, off, 0, 0);
        f.w[j] = make_uint2(v[0], v[1]);
    }
    const int xo = L.xof + stage * KC * 2;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(L.xr[j], xo, 0, 0);
        f.x[j] = make_uint2(v[0], v[1]);
    }
}

GGO_DEV void unpack_w(const FetchT& f, float (&w0)[4], float (&w1)[4]) {
    w0[0] = bf16_lo(f.w[0].x);
    w0[1] = bf16_hi(f.w[0].x);
    w0[2] = bf16_lo(f.w[0].y);
    w0[3] = bf16_hi(f.w[0].y);
    w1[0] = bf16_lo(f.w[1].x);
    w1[1] = bf16_hi(f.w[1].x);
    w1[2] = bf16_lo(f.w[1].y);
    w1[3] = bf16_hi(f.w[1].y);
}
GGO_DEV void unpack_x(const FetchT& f, int j, float (&xv)[4]) {
    xv[0] = bf16_lo(f.x[j].x);
    xv[1] = bf16_hi(f.x[j].x);
    xv[2] = bf16_lo(f.x[j].y);
    xv[3] = bf16_hi(f.x[j].y);
}

GGO_DEV void unpack_w(const Fetch<true>& f, float (&w0)[4], float (&w1)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        w0[i] = bf16_lo(f.w[i]);
        w1[i] = bf16_hi(f.w[i]);
    }
}
GGO_DEV void unpack_w(const Fetch<false>& f, float (&w0)[4], float (&w1)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        w0[i] = bf16_one(f.w[i][0]);
        w1[i] = bf16_one(f.w[i][1]);
    }
}
GGO_DEV void unpack_x(const Fetch<true>& f, int j, float (&xv)[4]) {
    xv[0] = bf16_lo(f.x[j].x);
    xv[1] = bf16_hi(f.x[j].x);
    xv[2] = bf16_lo(f.x[j].y);
    xv[3] = bf16_hi(f.x[j].y);
}
GGO_DEV void unpack_x(const Fetch<false>& f, int j, float (&xv)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) xv[i] = bf16_one(f.x[j][i]);
}

// Products of one 4(k) x 2(n) block for the lane's live rows, written as
// 16-byte runs of 4 ascending k.
template <typename F>
GGO_DEV void produce(const F& f, float* ps, int kq, int np, int r0, int rows) {
    float w0[4], w1[4];
    unpack_w(f, w0, w1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = r0 + j;
        if (r >= rows) break;   // uniform across the wave
        float xv[4];
        unpack_x(f, j, xv);
        const float4 p0 = make_float4(xv[0] * w0[0], xv[1] * w0[1], xv[2] * w0[2], xv[3] * w0[3]);
        const float4 p1 = make_float4(xv[0] * w1[0], xv[1] * w1[1], xv[2] * w1[2], xv[3] * w1[3]);
        const int run = r * NS + 2 * np;
        *reinterpret_cast<float4*>(ps + slot(run, kq)) = p0;
        *reinterpret_cast<float4*>(ps + slot(run + 1, kq)) = p1;
    }
}

template <bool WIDE, bool WT = false>
__global__ __launch_bounds__(THREADS) void k_gemv_ordered(const GemvArgs a) {
    static_assert(!WT || WIDE, "the W^T form loads 8 bytes per row");
    using F = typename std::conditional<WT, FetchT, Fetch<WIDE>>::type;
    // prefetch distance of W and x in stages (the wide ring keeps 64 loads in
    // flight, the element ring 48), and an unroll that makes every ring index static
    constexpr int DEPTH = WIDE ? 8 : 2;
    constexpr int UNROLL = WIDE ? 8 : 4;
    static_assert(UNROLL % NBUF == 0 && UNROLL % DEPTH == 0 && UNROLL % 2 == 0, "");

    __shared__ __attribute__((aligned(16))) float ps[NBUF][RG * NS * RUN];

    const int t = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int n0 = xcd_contiguous(blockIdx.x, gridDim.x) * NS;
    const int m0 = blockIdx.y * RG;
    const int rows = a.M - m0 < RG ? a.M - m0 : RG;
    const int nst = (a.K + KC - 1) / KC;
    // Iteration s (one barrier each): producers form stage s, the consumers
    // read stage s-1 and fold stage s-2. The count is nst + 2 rounded up to a
    // whole unroll, so ring indices stay static and the loop body has no early
    // exit; iterations past the data skip the products and the adds.
    const int iters = (nst + 2 + UNROLL - 1) / UNROLL * UNROLL;

    // The consumers' stages -2 and -1 (their two-stage lag) read zeros: each
    // chain's first two steps add +0 to +0.
    for (int i = t; i < NBUF * RG * NS * RUN / 4; i += THREADS)
        reinterpret_cast<float4*>(&ps[0][0])[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);

    // Every role runs its own loop with the same number of barriers (iters,
    // plus one before the loop). Inside a loop every iteration issues the same
    // loads and reads (no conditional loads), so no register versions have to
    // be merged and the prefetch ring stays in flight across barriers.
    const bool consumer = wave < CONSUMERS;
    const int first_row = consumer ? 4 * wave : 4 * __builtin_amdgcn_readfirstlane((t - 64 * CONSUMERS) / TASKS);
    if (first_row >= rows) {   // no live row in this wave
        __syncthreads();
        for (int s = 0; s < iters; ++s) __syncthreads();
    } else if (!consumer) {
        const int q = t - 64 * CONSUMERS;
        const int task = q % TASKS;
        const int kq = task >> 3, np = task & 7, n = n0 + 2 * np;
        Lane L;
        if (WT) {
            const int slab_rows = a.N - n0 < NS ? a.N - n0 : NS;
            L.wt = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.W) + static_cast<int64_t>(n0) * a.ldw, 0,
                                                     ((slab_rows - 1) * static_cast<int>(a.ldw) + a.K) * 2, BUF_DWORD3);
            L.k4 = 4 * kq;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                L.tof[j] = ((2 * np + j) * static_cast<int>(a.ldw) + 4 * kq) * 2;
                L.tlive[j] = n + j < a.N;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) L.wof[i][j] = ((4 * kq + i) * static_cast<int>(a.ldw) + n + j) * 2;
        }
        L.xof = 8 * kq;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = first_row + j;
            const bool live = r < rows;
            L.xr[j] = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t*>(a.x) + (live ? static_cast<int64_t>(m0 + r) * a.ldx : 0), 0,
                live ? a.K * 2 : 0, BUF_DWORD3);
        }
        F f[DEPTH];
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) fetch(a, L, d, f[d]);
        __syncthreads();
        for (int s0 = 0; s0 < iters; s0 += UNROLL) {
#pragma unroll
            for (int d = 0; d < UNROLL; ++d) {
                const int s = s0 + d;
                if (s < nst) produce(f[d % DEPTH], ps[d % NBUF], kq, np, first_row, rows);   // uniform
                fetch(a, L, s + DEPTH, f[d % DEPTH]);   // empty range past the end: zeros, no memory access
                __syncthreads();
            }
        }
    } else {
        const int run = t;   // = (4 * wave + lane / 16) * NS + lane % 16
        float acc = 0.0f;    // +0.0: the chain's start
        float4 cb[2][NQ];
#pragma unroll
        for (int j = 0; j < NQ; ++j) cb[0][j] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        __syncthreads();
        for (int s0 = 0; s0 < iters; s0 += UNROLL) {
#pragma unroll
            for (int d = 0; d < UNROLL; ++d) {
                const int s = s0 + d;
                const float* src = ps[(d + NBUF - 1) % NBUF];
#pragma unroll
                for (int j = 0; j < NQ; ++j) cb[(d + 1) & 1][j] = *reinterpret_cast<const float4*>(src + slot(run, j));
                if (s < nst + 2) {   // uniform
#pragma unroll
                    for (int j = 0; j < NQ; ++j) {     // ascending k
                        const float4 v = cb[d & 1][j];
                        acc = acc + v.x;
                        acc = acc + v.y;
                        acc = acc + v.z;
                        acc = acc + v.w;
                    }
                }
                __syncthreads();
            }
        }
        const int r = t >> 4, nn = n0 + (t & 15);
        if (r < rows && nn < a.N) a.y[static_cast<int64_t>(m0 + r) * a.ldy + nn] = acc;
    }
}


// ---------------------------------------------------------------------------
// The same contract with 128-k stages, for M > 4 (16-byte-capable operands only). A producer lane
// covers all eight rows of its 4(k) x 2(n) block, so each weight pair is loaded once for the eight
// rows instead of once per half, and a stage is twice as long, so there are half as many barriers;
// two product buffers suffice because the consumers read stage s-1 and fold it in the same
// iteration. Products, their positions in each chain and the consumers' order are those of
// k_gemv_ordered, so the bits are too (the tests compare every M against the oracle). Measured on
// the 4096 x 4096 decode weight: M = 8 42 -> 35 us, M = 13 73 -> 62 us; at M <= 4 the 64-k form is
// as fast or faster, so it stays there.
constexpr int KC2 = 128, NBUF2 = 2, RUN2 = KC2, NQ2 = KC2 / 4, TASKS2 = (KC2 / 4) * (NS / 2);
static_assert(TASKS2 == 256, "one 4(k) x 2(n) block per producer lane");

// slot() for 128-k runs: both the producers' writes and the consumers' reads keep 8 distinct groups
// of 4 banks per 8 lanes.
GGO_DEV int slot2(int run, int k4) { return run * RUN2 + ((k4 ^ ((run + (run >> 3)) & 7)) << 2); }

template <bool WT> struct Fetch2;
template <> struct Fetch2<true> {    // W^T rows n, n+1 at the lane's 4 k; x rows 0 .. RG-1 at the same k
    uint2 w[2];
    uint2 x[RG];
};
template <> struct Fetch2<false> {   // W [K, N]: the pair (n, n+1) of each of the lane's 4 k-rows
    uint32_t w[4];
    uint2 x[RG];
};

struct Lane2 {
    __amdgpu_buffer_rsrc_t wt;   // W^T: the workgroup's slab of rows
    int tof[2];
    bool tlive[2];
    int wof[4][2];               // W [K, N]: offsets inside a stage
    int k4;
    int xof;
    __amdgpu_buffer_rsrc_t xr[RG];
};

// W [K, N] descriptor of one 128-k stage (w_rsrc for KC2 rows; launched only for ldw small enough that the range fits 31 bits).
GGO_DEV __amdgpu_buffer_rsrc_t w_rsrc2(const GemvArgs& a, int stage) {
    const int rows_left = a.K - stage * KC2;
    const int rows_in = rows_left < KC2 ? rows_left : KC2;
    const int nrec = rows_left <= 0 ? 0 : ((rows_in - 1) * static_cast<int>(a.ldw) + a.N) * 2;
    const int64_t row0 = rows_left <= 0 ? 0 : static_cast<int64_t>(stage) * KC2;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.W) + row0 * a.ldw, 0, nrec, BUF_DWORD3);
}

template <bool WT>
GGO_DEV void fetch2(const GemvArgs& a, const Lane2& L, int stage, Fetch2<WT>& f) {
    if constexpr (WT) {
        const bool kin = stage * KC2 + L.k4 < a.K;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int off = (kin && L.tlive[j]) ? L.tof[j] + stage * KC2 * 2 : OUT_OF_RANGE;
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(L.wt, off, 0, 0);
            f.w[j] = make_uint2(v[0], v[1]);
        }
    } else {
        const __amdgpu_buffer_rsrc_t wr = w_rsrc2(a, stage);
#pragma unroll
        for (int i = 0; i < 4; ++i) f.w[i] = __builtin_amdgcn_raw_buffer_load_b32(wr, L.wof[i][0], 0, 0);
    }
    const int xo = L.xof + stage * KC2 * 2;
#pragma unroll
    for (int j = 0; j < RG; ++j) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(L.xr[j], xo, 0, 0);
        f.x[j] = make_uint2(v[0], v[1]);
    }
}

GGO_DEV void unpack_w2(const Fetch2<true>& f, float (&w0)[4], float (&w1)[4]) {
    w0[0] = bf16_lo(f.w[0].x); w0[1] = bf16_hi(f.w[0].x); w0[2] = bf16_lo(f.w[0].y); w0[3] = bf16_hi(f.w[0].y);
    w1[0] = bf16_lo(f.w[1].x); w1[1] = bf16_hi(f.w[1].x); w1[2] = bf16_lo(f.w[1].y); w1[3] = bf16_hi(f.w[1].y);
}
GGO_DEV void unpack_w2(const Fetch2<false>& f, float (&w0)[4], float (&w1)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        w0[i] = bf16_lo(f.w[i]);
        w1[i] = bf16_hi(f.w[i]);
    }
}

// Products of the lane's 4(k) x 2(n) block for every live row, as 16-byte runs of 4 ascending k.
template <bool WT>
GGO_DEV void produce2(const Fetch2<WT>& f, float* ps, int kq, int np, int rows) {
    float w0[4], w1[4];
    unpack_w2(f, w0, w1);
#pragma unroll
    for (int r = 0; r < RG; ++r) {
        if (r >= rows) break;   // uniform across the workgroup
        const float xv[4] = {bf16_lo(f.x[r].x), bf16_hi(f.x[r].x), bf16_lo(f.x[r].y), bf16_hi(f.x[r].y)};
        const float4 p0 = make_float4(xv[0] * w0[0], xv[1] * w0[1], xv[2] * w0[2], xv[3] * w0[3]);
        const float4 p1 = make_float4(xv[0] * w1[0], xv[1] * w1[1], xv[2] * w1[2], xv[3] * w1[3]);
        const int run = r * NS + 2 * np;
        *reinterpret_cast<float4*>(ps + slot2(run, kq)) = p0;
        *reinterpret_cast<float4*>(ps + slot2(run + 1, kq)) = p1;
    }
}

template <bool WT>
__global__ __launch_bounds__(THREADS) void k_gemv_ordered_k128(const GemvArgs a) {
    constexpr int DEPTH = 2, UNROLL = 2;   // prefetch distance in 128-k stages (deeper measured slower)
    static_assert(UNROLL % NBUF2 == 0 && UNROLL % DEPTH == 0, "");
    __shared__ __attribute__((aligned(16))) float ps[NBUF2][RG * NS * RUN2];

    const int t = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int n0 = xcd_contiguous(blockIdx.x, gridDim.x) * NS;
    const int m0 = blockIdx.y * RG;
    const int rows = a.M - m0 < RG ? a.M - m0 : RG;
    const int nst = (a.K + KC2 - 1) / KC2;
    // Iteration s (one barrier each): the producers form stage s, the consumers read and fold stage
    // s-1. Iterations past the data skip the products and the adds.
    const int iters = (nst + 1 + UNROLL - 1) / UNROLL * UNROLL;

    const bool consumer = wave < CONSUMERS;
    if (consumer && 4 * wave >= rows) {   // no live row in this consumer wave
        for (int s = 0; s < iters + 1; ++s) __syncthreads();
    } else if (!consumer) {
        const int q = t - 64 * CONSUMERS;
        const int kq = q >> 3, np = q & 7, n = n0 + 2 * np;
        Lane2 L;
        if (WT) {
            const int slab_rows = a.N - n0 < NS ? a.N - n0 : NS;
            L.wt = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.W) + static_cast<int64_t>(n0) * a.ldw, 0,
                                                     ((slab_rows - 1) * static_cast<int>(a.ldw) + a.K) * 2, BUF_DWORD3);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                L.tof[j] = ((2 * np + j) * static_cast<int>(a.ldw) + 4 * kq) * 2;
                L.tlive[j] = n + j < a.N;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) L.wof[i][j] = ((4 * kq + i) * static_cast<int>(a.ldw) + n + j) * 2;
        }
        L.k4 = 4 * kq;
        L.xof = 8 * kq;
#pragma unroll
        for (int j = 0; j < RG; ++j) {
            const bool live = j < rows;
            L.xr[j] = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t*>(a.x) + (live ? static_cast<int64_t>(m0 + j) * a.ldx : 0), 0, live ? a.K * 2 : 0,
                BUF_DWORD3);
        }
        Fetch2<WT> f[DEPTH];
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) fetch2<WT>(a, L, d, f[d]);
        __syncthreads();
        for (int s0 = 0; s0 < iters; s0 += UNROLL) {
#pragma unroll
            for (int d = 0; d < UNROLL; ++d) {
                const int s = s0 + d;
                if (s < nst) produce2<WT>(f[d % DEPTH], ps[d % NBUF2], kq, np, rows);   // uniform
                fetch2<WT>(a, L, s + DEPTH, f[d % DEPTH]);   // past the end: empty ranges, zeros
                __syncthreads();
            }
        }
    } else {
        const int run = t;   // = (4 * wave + lane / 16) * NS + lane % 16
        float acc = 0.0f;    // +0.0: the chain's start
        __syncthreads();
        for (int s0 = 0; s0 < iters; s0 += UNROLL) {
#pragma unroll
            for (int d = 0; d < UNROLL; ++d) {
                const int s = s0 + d;
                if (s >= 1 && s <= nst) {   // uniform: stage s - 1, formed in the previous iteration
                    const float* src = ps[(d + NBUF2 - 1) % NBUF2];
                    float4 cb[NQ2];
#pragma unroll
                    for (int j = 0; j < NQ2; ++j) cb[j] = *reinterpret_cast<const float4*>(src + slot2(run, j));
#pragma unroll
                    for (int j = 0; j < NQ2; ++j) {   // ascending k
                        acc = acc + cb[j].x;
                        acc = acc + cb[j].y;
                        acc = acc + cb[j].z;
                        acc = acc + cb[j].w;
                    }
                }
                __syncthreads();
            }
        }
        const int r = t >> 4, nn = n0 + (t & 15);
        if (r < rows && nn < a.N) a.y[static_cast<int64_t>(m0 + r) * a.ldy + nn] = acc;
    }
}
// ---------------------------------------------------------------------------
// M = 1 with the weight as W^T (16-byte operands): 512-k stages. The one-lane chain costs at least
// K x 4.5 clocks whatever the kernel does; what the 64-k kernel adds on top is a barrier every 64 adds.
// Here a stage is 512 k, so a 4096-long chain meets 8 barriers instead of 64, and every producer load
// instruction reads 1 KiB of one weight row (lane l: k = 8 l .. 8 l + 7 of the stage), the access pattern
// of the tree GEMV's weight stream.
//   wave 0        consumer: lane c < 16 owns y[0, n0 + c] and folds the stage's 512 products of its
//                 column in ascending k (16-byte LDS reads, four adds each)
//   waves 1 - P1  producers: wave q forms the products of rows n0 + RW1 (q - 1) .. + RW1 - 1 of W^T
//                 (P1 = 2 waves of 8 rows; 1 or 4 waves measured the same)
// Products, their places in the chain and the adds are those of k_gemv_ordered, so the bits are too.
// Clock stamps at K = 4096 put the time in three parts: about 5,600 clocks until stage 0 is formed (the
// first loads' latency), 3,400 per stage (512 dependent adds at 4.5 plus about 6 for each 16-byte LDS
// read), and 350 per barrier.
constexpr int NS1 = 16, SL1 = 512, P1 = 2, NBUF1 = 2, DEPTH1 = 3, RW1 = NS1 / P1;
constexpr int THREADS1 = 64 * (1 + P1);
constexpr int NQ1 = SL1 / 4;   // 16-byte chunks of one column's products per stage

// Position (in floats) of chunk k4 (products 4 k4 .. 4 k4 + 3) of column c in a stage buffer: the chunk
// index is XORed with c, so the 16 consumer lanes reading chunk k4 of their columns, and a producer wave
// writing one column's chunks, fall on distinct groups of 4 banks.
GGO_DEV int slot1(int c, int k4) { return c * SL1 + ((k4 ^ c) << 2); }

struct Fetch1 {
    uint4 w[RW1];   // k = 8 l .. 8 l + 7 of the stage, for the wave's RW1 rows of W^T
    uint4 x;        // the same 8 k of x
};

__global__ __launch_bounds__(THREADS1) void k_gemv_ordered_m1(const GemvArgs a) {
    __shared__ __attribute__((aligned(16))) float ps[NBUF1][NS1 * SL1];
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int n0 = xcd_contiguous(blockIdx.x, gridDim.x) * NS1;
    const int nst = (a.K + SL1 - 1) / SL1;
    // Iteration s (one barrier each): the producers form stage s, the consumer folds stage s - 1. The
    // count is padded to a whole number of DEPTH1 groups so the producers' loop has no exit or skip
    // inside it: a branch there made the compiler wait for every load in flight, the prefetched stages
    // too. Stages past the last are formed from zeros into the buffer no one reads next.
    const int iters = (nst + DEPTH1) / DEPTH1 * DEPTH1;
    const int kbytes = a.K * 2;
    if (wave > 0) {
        const int q = wave - 1;
        __amdgpu_buffer_rsrc_t wr[RW1];
#pragma unroll
        for (int r = 0; r < RW1; ++r) {
            const int64_t n = n0 + RW1 * q + r;
            wr[r] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.W) + n * a.ldw, 0, n < a.N ? kbytes : 0,
                                                      BUF_DWORD3);
        }
        const auto xr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.x), 0, kbytes, BUF_DWORD3);
        auto fetch1 = [&](int stage, Fetch1& f) {   // past K (or past the last stage): zeros, no memory access
            const int off = stage * SL1 * 2 + lane * 16;
#pragma unroll
            for (int r = 0; r < RW1; ++r) {
                const auto v = __builtin_amdgcn_raw_buffer_load_b128(wr[r], off, 0, 0);
                f.w[r] = make_uint4(v[0], v[1], v[2], v[3]);
            }
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
            f.x = make_uint4(v[0], v[1], v[2], v[3]);
        };
        Fetch1 f[DEPTH1];
#pragma unroll
        for (int d = 0; d < DEPTH1; ++d) {
            fetch1(d, f[d]);
            __builtin_amdgcn_sched_barrier(0);   // issued stage by stage, so stage 0's loads are the oldest
        }
        for (int s0 = 0; s0 < iters; s0 += DEPTH1) {
#pragma unroll
            for (int d = 0; d < DEPTH1; ++d) {
                const int s = s0 + d;
                {
                    float* buf = ps[s % NBUF1];
                    const float xv[8] = {bf16_lo(f[d].x.x), bf16_hi(f[d].x.x), bf16_lo(f[d].x.y), bf16_hi(f[d].x.y),
                                         bf16_lo(f[d].x.z), bf16_hi(f[d].x.z), bf16_lo(f[d].x.w), bf16_hi(f[d].x.w)};
#pragma unroll
                    for (int r = 0; r < RW1; ++r) {
                        const uint4 w = f[d].w[r];
                        const float wv[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                                             bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
                        const int c = RW1 * q + r;
                        *reinterpret_cast<float4*>(buf + slot1(c, 2 * lane)) =
                            make_float4(xv[0] * wv[0], xv[1] * wv[1], xv[2] * wv[2], xv[3] * wv[3]);
                        *reinterpret_cast<float4*>(buf + slot1(c, 2 * lane + 1)) =
                            make_float4(xv[4] * wv[4], xv[5] * wv[5], xv[6] * wv[6], xv[7] * wv[7]);
                    }
                }
                fetch1(s + DEPTH1, f[d]);
                __syncthreads();
                // keep each stage's conversions after its own barrier: hoisted ahead, they made the
                // loads of later stages complete first
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    } else {
        float acc = 0.0f;   // +0.0: the chain's start
        const int c = lane & (NS1 - 1);
        // The output pointer's scalar load completes here: outstanding inside the loop, it made each
        // stage's first LDS wait a wait for every read in flight (scalar loads return out of order).
        float* const y = a.y;
        asm volatile("" ::"s"(y));
        // The reads of the next 64 k are issued before the adds of the current 64. Measured against
        // this: 8 or 4 chunks per burst (more bursts, each with a fixed cost), one read every four adds
        // 12 chunks ahead (each read inside the chain costs more than in a burst), and all 64 lanes
        // reading 16 k of 16 columns with the quad's products taken by DPP broadcasts in the adds
        // (a quarter of the reads, but a dependent DPP add costs twice a plain one).
        constexpr int G = 16, NG = NQ1 / G;
        for (int s = 0; s < iters; ++s) {
            if (s >= 1 && s <= nst && lane < NS1) {   // stage s - 1, formed in the previous iteration
                const float* src = ps[(s - 1) % NBUF1];
                float4 cb[2][G];
#pragma unroll
                for (int j = 0; j < G; ++j) cb[0][j] = *reinterpret_cast<const float4*>(src + slot1(c, j));
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) {
                    if (gi + 1 < NG) {
#pragma unroll
                        for (int j = 0; j < G; ++j)
                            cb[(gi + 1) & 1][j] = *reinterpret_cast<const float4*>(src + slot1(c, (gi + 1) * G + j));
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int j = 0; j < G; ++j) {   // ascending k
                        const float4 v = cb[gi & 1][j];
                        acc = acc + v.x;
                        acc = acc + v.y;
                        acc = acc + v.z;
                        acc = acc + v.w;
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            __syncthreads();
        }
        if (lane < NS1 && n0 + c < a.N) y[n0 + c] = acc;
    }
}

// ---------------------------------------------------------------------------
// Two to eight rows of x, weight as W^T (16-byte operands): the structure of k_gemv_ordered_m1 for MR
// rows. One consumer wave: lane m NSC + c folds y[m0 + m, n0 + c] (MR NSC <= 64 chains). Two producer
// waves stream the workgroup's NSC weight rows, SL k per stage: a load instruction covers 64 / LPR rows,
// LPR = SL / 8 lanes per row (lane l: row l / LPR of the load, k = 8 (l mod LPR) .. + 7 of the stage),
// and each lane forms the MR products of each of its weight elements with the same 8 k of every row of x.
// A stage holds MR NSC SL products. Products, their places in the chain and the adds are those of
// k_gemv_ordered, so the bits are too.
template <int MR, int NSC, int SL, int P_>
struct MrGeo {
    static constexpr int P = P_, CH = MR * NSC;            // producer waves, chains
    static constexpr int LPR = SL / 8, RPL = 64 / LPR;     // lanes per weight row, rows per load instruction
    static constexpr int RW = NSC / P, WL = RW / RPL;      // weight rows per producer wave, loads per stage
    static constexpr int NQ = SL / 4;                      // 16-byte product chunks per chain and stage
    static constexpr int SWZ = (NQ < 16 ? NQ : 16) - 1;    // chunk XOR: 16 consecutive chains on distinct banks
    static constexpr int NBUF = 2, DEPTH = 3, THREADS = 64 * (1 + P);
    static_assert(CH <= 64 && RW % RPL == 0 && WL >= 1 && NQ % 16 == 0, "MrGeo");
};
constexpr int OFF_PAST_MR = 0x7ffffff0;   // a buffer offset past every range used here: the load returns 0

template <class G>
GGO_DEV int slot_mr(int ch, int k4) { return ch * (G::NQ * 4) + ((k4 ^ (ch & G::SWZ)) << 2); }

template <int MR, int NSC, int SL, int P>
__global__ __launch_bounds__(64 * (1 + P)) void k_gemv_ordered_mr(const GemvArgs a) {
    using G = MrGeo<MR, NSC, SL, P>;
    __shared__ __attribute__((aligned(16))) float ps[G::NBUF][G::CH * SL];
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int n0 = xcd_contiguous(blockIdx.x, gridDim.x) * NSC, m0 = blockIdx.y * MR;
    const int nst = (a.K + SL - 1) / SL;
    // Iteration s (one barrier each): the producers form stage s, the consumer folds stage s - 1; the
    // count is padded to whole rounds of DEPTH stages, as in k_gemv_ordered_m1 (no exit or skip inside the
    // producers' loop; stages past the last are formed from zeros into the buffer no one reads next).
    const int iters = (nst + G::DEPTH) / G::DEPTH * G::DEPTH;
    if (wave > 0) {
        const int q = wave - 1, kq = lane % G::LPR, rl = lane / G::LPR;
        // one range for the workgroup's weight rows and one for its rows of x; a lane past K or past the
        // last row gets an offset past the range (K is a multiple of 8: a lane's 8 k are all in or all out)
        const int wrows = a.N - n0 < NSC ? a.N - n0 : NSC, xrows = a.M - m0 < MR ? a.M - m0 : MR;
        const auto wr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.W) + static_cast<int64_t>(n0) * a.ldw,
                                                          0, ((wrows - 1) * static_cast<int>(a.ldw) + a.K) * 2, BUF_DWORD3);
        const auto xr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.x) + static_cast<int64_t>(m0) * a.ldx,
                                                          0, ((xrows - 1) * static_cast<int>(a.ldx) + a.K) * 2, BUF_DWORD3);
        struct Fetch {
            uint4 w[G::WL];   // k = 8 kq .. 8 kq + 7 of the stage, weight rows q RW + i RPL + rl
            uint4 x[MR];      // the same 8 k of each row of x
        };
        auto fetch = [&](int stage, Fetch& f) {
            const int k = stage * SL + 8 * kq;
#pragma unroll
            for (int i = 0; i < G::WL; ++i) {
                const int r = q * G::RW + i * G::RPL + rl;
                const int off = (k < a.K && r < wrows) ? (r * static_cast<int>(a.ldw) + k) * 2 : OFF_PAST_MR;
                const auto v = __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, 0);
                f.w[i] = make_uint4(v[0], v[1], v[2], v[3]);
            }
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const int off = (k < a.K && m < xrows) ? (m * static_cast<int>(a.ldx) + k) * 2 : OFF_PAST_MR;
                const auto v = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
                f.x[m] = make_uint4(v[0], v[1], v[2], v[3]);
            }
        };
        Fetch f[G::DEPTH];
#pragma unroll
        for (int d = 0; d < G::DEPTH; ++d) {
            fetch(d, f[d]);
            __builtin_amdgcn_sched_barrier(0);   // issued stage by stage, so stage 0's loads are the oldest
        }
        for (int s0 = 0; s0 < iters; s0 += G::DEPTH) {
#pragma unroll
            for (int d = 0; d < G::DEPTH; ++d) {
                const int s = s0 + d;
                float* buf = ps[s % G::NBUF];
                float xv[MR][8];
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    const uint4 x = f[d].x[m];
                    xv[m][0] = bf16_lo(x.x); xv[m][1] = bf16_hi(x.x); xv[m][2] = bf16_lo(x.y); xv[m][3] = bf16_hi(x.y);
                    xv[m][4] = bf16_lo(x.z); xv[m][5] = bf16_hi(x.z); xv[m][6] = bf16_lo(x.w); xv[m][7] = bf16_hi(x.w);
                }
#pragma unroll
                for (int i = 0; i < G::WL; ++i) {
                    const uint4 w = f[d].w[i];
                    const float wv[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                                         bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
                    const int r = q * G::RW + i * G::RPL + rl;
#pragma unroll
                    for (int m = 0; m < MR; ++m) {
                        const int ch = m * NSC + r;
                        *reinterpret_cast<float4*>(buf + slot_mr<G>(ch, 2 * kq)) =
                            make_float4(xv[m][0] * wv[0], xv[m][1] * wv[1], xv[m][2] * wv[2], xv[m][3] * wv[3]);
                        *reinterpret_cast<float4*>(buf + slot_mr<G>(ch, 2 * kq + 1)) =
                            make_float4(xv[m][4] * wv[4], xv[m][5] * wv[5], xv[m][6] * wv[6], xv[m][7] * wv[7]);
                    }
                }
                fetch(s + G::DEPTH, f[d]);
                __syncthreads();
                __builtin_amdgcn_sched_barrier(0);   // each stage's conversions after its own barrier
            }
        }
    } else {
        float acc = 0.0f;   // +0.0: the chain's start
        const int ch = lane, m = lane / NSC, c = lane % NSC;
        float* const y = a.y;
        asm volatile("" ::"s"(y));   // the output pointer's scalar load completes before the loop
        constexpr int GR = 16, NGR = G::NQ / GR;   // reads of the next 64 k before the adds of the current 64
        for (int s = 0; s < iters; ++s) {
            if (s >= 1 && s <= nst && ch < G::CH) {   // stage s - 1, formed in the previous iteration
                const float* src = ps[(s - 1) % G::NBUF];
                float4 cb[2][GR];
#pragma unroll
                for (int j = 0; j < GR; ++j) cb[0][j] = *reinterpret_cast<const float4*>(src + slot_mr<G>(ch, j));
#pragma unroll
                for (int gi = 0; gi < NGR; ++gi) {
                    if (gi + 1 < NGR) {
#pragma unroll
                        for (int j = 0; j < GR; ++j)
                            cb[(gi + 1) & 1][j] = *reinterpret_cast<const float4*>(src + slot_mr<G>(ch, (gi + 1) * GR + j));
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int j = 0; j < GR; ++j) {   // ascending k
                        const float4 v = cb[gi & 1][j];
                        acc = acc + v.x;
                        acc = acc + v.y;
                        acc = acc + v.z;
                        acc = acc + v.w;
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            __syncthreads();
        }
        if (ch < G::CH && m0 + m < a.M && n0 + c < a.N) y[static_cast<int64_t>(m0 + m) * a.ldy + n0 + c] = acc;
    }
}

template <int MR, int NSC, int SL, int P>
hipError_t launch_mr(const GemvArgs& a, hipStream_t stream) {
    using G = MrGeo<MR, NSC, SL, P>;
    hipLaunchKernelGGL((k_gemv_ordered_mr<MR, NSC, SL, P>), dim3((a.N + NSC - 1) / NSC, (a.M + MR - 1) / MR),
                       dim3(G::THREADS), 0, stream, a);
    return hipGetLastError();
}

// rows of x per workgroup for the MR instance: M rounded up to 2, 4 or 8, and 8-row groups above 8 rows
// (two workgroups per CU; the 4-row shape's 64 KiB stages hold one, and at M = 12 / 16 its row groups ran
// in rounds: 53.7 / 71.0 us against 54.7 / 55.2), or the caller's forced value
int mr_rows(const GemvArgs& a) { return a.rows ? a.rows : a.M <= 2 ? 2 : a.M <= 4 ? 4 : 8; }

}  // namespace

// M = 1, W^T, 16-byte loads that never straddle the end of a row, byte offsets within 32 bits
bool gemv_ordered_m1_ok(const GemvArgs& a) {
    return a.wt && a.M == 1 && (a.vec & VEC_W16) && a.K <= (1 << 29) - 4 * DEPTH1 * SL1;
}

// 2 <= M (per workgroup: 2, 4 or 8 rows), W^T, 16-byte loads; a 16-row slab of W^T and 8 rows of x in
// 32-bit byte offsets below the past-the-end offset
bool gemv_ordered_mr_ok(const GemvArgs& a) {
    return a.wt && (a.vec & VEC_W16) && a.ldw <= (OFF_PAST_MR / 2 - a.K) / 16 && a.ldx <= (OFF_PAST_MR / 2 - a.K) / 8;
}

bool gemv_ordered_k128_ok(const GemvArgs& a) {
    return a.wt || ((a.vec & VEC_W) && a.ldw <= ((1 << 30) - (1 << 16)) / (KC2 + 1));   // 32-bit stage ranges
}

hipError_t launch_gemv_ordered(const GemvArgs& a, hipStream_t stream) {
    const dim3 grid((a.N + NS - 1) / NS, (a.M + RG - 1) / RG);
    // With operands it can take, the 128-k form (same bits; see k_gemv_ordered_k128) from M = 2 on W [K, N]
    // (4096 x 4096: 20.5 / 22.5 us at M = 2 / 4 against 21.5 / 28.3 with 64-k stages; level at M = 1) and
    // above M = 4 on W^T where the MR-row instance cannot serve; form 1 or 2 forces the 64-k or the 128-k
    // form (the caller has checked that the latter can serve)
    const bool k128 = a.form == 2 || (a.form == 0 && a.M > (a.wt ? 4 : 1) && gemv_ordered_k128_ok(a));
    if (a.form == 3 || (a.form == 0 && a.M == 1 && gemv_ordered_m1_ok(a))) {
        hipLaunchKernelGGL(k_gemv_ordered_m1, dim3((a.N + NS1 - 1) / NS1), dim3(THREADS1), 0, stream, a);
    } else if (a.form == 4 || (a.form == 0 && a.M >= 2 && gemv_ordered_mr_ok(a))) {
        // rows x columns x k per stage, producer waves: 2 x 16 x 512 and 4 x 16 x 256 (64 KiB stages, one
        // workgroup per CU), 8 x 8 x 128 with two workgroups per CU (32 KiB stages). Measured on 4096 x 4096
        // against these: 256-k stages at two rows (18.9 against 17.1 us), 128-k stages or two producer waves
        // at four rows (21.6 / 20.5 against 19.5), 256-k stages at eight rows (37-42 against 27.9: one
        // workgroup per CU, two rounds of the 512 workgroups)
        const int mr = mr_rows(a);
        return mr == 2 ? launch_mr<2, 16, 512, 2>(a, stream) : mr == 4 ? launch_mr<4, 16, 256, 4>(a, stream)
                                                                       : launch_mr<8, 8, 128, 2>(a, stream);
    } else if (k128 && a.wt)
        hipLaunchKernelGGL((k_gemv_ordered_k128<true>), grid, dim3(THREADS), 0, stream, a);
    else if (k128)
        hipLaunchKernelGGL((k_gemv_ordered_k128<false>), grid, dim3(THREADS), 0, stream, a);
    else if (a.wt)
        hipLaunchKernelGGL((k_gemv_ordered<true, true>), grid, dim3(THREADS), 0, stream, a);
    else if (a.vec & VEC_W)
        hipLaunchKernelGGL(k_gemv_ordered<true>, grid, dim3(THREADS), 0, stream, a);
    else
        hipLaunchKernelGGL(k_gemv_ordered<false>, grid, dim3(THREADS), 0, stream, a);
    return hipGetLastError();
}

int gemv_ordered_max_ldw() { return ((1 << 30) - (1 << 16)) / (KC + 1); }

// The W^T slab range, (NS - 1) * ldw + K elements of 2 bytes, stays below OUT_OF_RANGE.
int gemv_ordered_wt_max_ldw() { return ((1 << 30) - (1 << 16)) / NS; }
