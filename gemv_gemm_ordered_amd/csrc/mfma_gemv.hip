// Decode GEMV on the gfx950 matrix cores, with the bits of gemm_mfma_invariant:
// y[m, n] = sum_k x[m, k] * WT[n, k] for M <= 16, the weight given as a linear layer stores it.
//
// "Taming Bitwise Behavior in GPU Kernels with Tensor Core", sections 3.2.1 and 3.2.2: what fixes
// an output's bits on a matrix-instruction path is the opcode (its group of k and internal fold),
// the accumulator carried from one instruction to the next through the instruction's C input, and
// where the last short group of K falls -- not the tile. This kernel keeps all three of
// gemm_mfma_invariant's: one v_mfma_f32_16x16x32_bf16 per 32 k, groups in ascending k from k = 0,
// the binary32 accumulator passed through srcC from +0, k past K fed as zeros. So every output
// equals the GEMM's bit for bit, at any M: a decode step and a prefill of the same rows agree.
//
// Shape. One instruction covers 16 outputs n (its A rows: weight rows) by 16 rows m of x (its B
// columns), so a workgroup owns one block of 16 consecutive n and runs the whole k chain of that
// block in one wave; with no split of K there are N / 16 chains, one workgroup each (256 for a
// 4096-wide weight, one per CU). Eight producer waves keep the weight stream in flight: the block's
// 16 weight rows (and the MT staged rows of x) move HBM -> LDS with direct-to-LDS 16-byte loads, one
// 1 KiB contiguous run of one row per load instruction, through a ring of NST stages of 512 k. Per
// stage every producer waits for its own loads, the workgroup meets at one barrier, the stage
// NST - 1 ahead is requested into the buffer freed by the previous stage, and wave 0 folds the
// stage: its 32 fragment reads, then a chain of 16 dependent MFMAs (one wave issues them back to
// back at the instruction's full rate, about 7.6 ns each).
//
// Wave 0 issues no loads of its own. The compiler puts a wait for every outstanding load before
// each LDS read that might alias a direct-to-LDS load still in flight; a wave that also loaded would
// wait there for the stages requested ahead, which drained the pipeline every stage (1 us per call).
//
// Measured on the 4096 x 4096 decode weight: loads and barriers alone take 7.3 us per call, the whole
// kernel 7.8 - 8.0 us at M = 1 ... 8. Four producers or a ring of 3 or 6 stages were slower.
//
// LDS layout: a row's 64 chunks of 16 bytes are stored with chunk c at slot c xor (row mod 16),
// by letting the lane that fills slot l fetch chunk l xor (row mod 16); the fragment reads (lane l
// reads chunk 4g + l / 16 of row l mod 16) then fall on 16 distinct bank groups.
//
// Range: one raw buffer descriptor per row whose range is exactly K elements (empty for rows past
// M or N), so loads past K write zeros without touching memory; no stage past the last is requested. Operands must be 16-byte aligned with row strides and K multiples of 8, so no 16-byte
// chunk straddles the end of a row.
#include "common.hpp"
#include "kernels.hpp"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_t;

constexpr int NB = 16;                 // outputs per workgroup: the instruction's 16 rows
constexpr int PRODUCERS = 8;           // waves 1 .. PRODUCERS load; wave 0 folds and issues no loads
constexpr int RW = NB / PRODUCERS;     // weight rows per producer and stage
constexpr int THREADS = 64 * (PRODUCERS + 1);
constexpr int SK = 512;                // k per stage (16 groups of 32)
constexpr int GROUPS = SK / 32;
constexpr int NST = 4;                 // stages in the ring
constexpr int BUF_DWORD3 = 0x00020000; // buffer descriptor word 3: raw 32-bit data, range checked
constexpr int AUX_STREAM = 2;          // weight loads: nontemporal (each weight byte is read once)

// s_waitcnt vmcnt(n) for the constant n (expcnt and lgkmcnt left at their maxima)
template <int N>
GGO_DEV void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

GGO_DEV __amdgpu_buffer_rsrc_t row_rsrc(const uint16_t* row, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(row), 0, bytes, BUF_DWORD3);
}

// Stage buffer: NB weight rows, then MT rows of x, each SK bf16 (1 KiB) in swizzled chunk order.
template <int MT> struct Ring {
    static constexpr int ROW = SK;                       // elements per staged row
    static constexpr int STAGE = (NB + MT) * ROW;        // elements per stage
    // Loads per producer and stage: RW weight rows, plus the rows of x p, p + PRODUCERS, ... below MT.
    static constexpr int XROWS_PER_WAVE = MT > PRODUCERS ? MT / PRODUCERS : 1;
    static_assert(NB % PRODUCERS == 0, "weight rows spread evenly over the producers");
    static_assert(MT <= PRODUCERS || MT % PRODUCERS == 0, "rows of x spread evenly over the producers");
};

// Producer p's loads of stage s into buffer `buf`: weight rows RW p .. RW p + RW - 1 and its rows of x.
template <int MT>
GGO_DEV void issue_stage(const GemvMfmaArgs& a, int64_t n0, int p, int lane, int s, uint16_t* buf) {
    using R = Ring<MT>;
    const int kbytes = a.K * 2;
    const int base = s * SK * 2;   // byte offset of the stage along a row
#pragma unroll
    for (int j = 0; j < RW; ++j) {
        const int r = RW * p + j;
        const int64_t n = n0 + r;
        const auto rs = row_rsrc(a.WT + n * a.ldwt, n < a.N ? kbytes : 0);
        const int off = base + ((lane ^ (r & 15)) << 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_t*)(buf + r * R::ROW), 16, off, 0, 0, AUX_STREAM);
    }
#pragma unroll
    for (int j = 0; j < R::XROWS_PER_WAVE; ++j) {
        const int m = p + j * PRODUCERS;
        if (m < MT) {
            const auto rs = row_rsrc(a.x + m * a.ldx, m < a.M ? kbytes : 0);
            const int off = base + ((lane ^ (m & 15)) << 4);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_t*)(buf + (NB + m) * R::ROW), 16, off, 0, 0, 0);
        }
    }
}

// Wait until producer p's loads of the current stage have landed; the `ahead` stages requested after
// it (NST - 2 in the steady state, fewer near the end, where nothing past the last stage is requested)
// may stay in flight. Loads per stage differ between producers (rows of x), so the count is chosen per
// producer; the branches are uniform within a wave.
template <int MT, int AHEAD>
GGO_DEV void wait_ahead(int p) {
    using R = Ring<MT>;
    constexpr int LX = (MT < PRODUCERS ? 1 : R::XROWS_PER_WAVE);
    if (p < MT) wait_vm<(RW + LX) * AHEAD>();
    else wait_vm<RW * AHEAD>();
}

template <int MT>
GGO_DEV void wait_stage(int p, int ahead) {
    static_assert(NST == 4, "the cases below cover up to NST - 2 = 2 stages ahead");
    if (ahead >= 2) wait_ahead<MT, 2>(p);
    else if (ahead == 1) wait_ahead<MT, 1>(p);
    else wait_ahead<MT, 0>(p);
}

// Wave 0's fold of one stage: every fragment read of the stage first, then its chain of 16 MFMAs,
// groups in ascending k (the chain waits for each group's reads as they land; reading a few groups ahead
// of each MFMA instead measured 0.1 us slower per call). xrow is this lane's row of x in the stage, or a
// row of zeros for lanes whose row is not staged (l mod 16 >= MT). TAIL: the last stage, whose groups
// from gmax on lie wholly past K and are skipped.
template <bool TAIL>
GGO_DEV void fold_stage(const uint16_t* __restrict__ wrow, const uint16_t* __restrict__ xrow, int c, int gmax,
                        f32x4& acc) {
    bf16x8 wf[GROUPS], xf[GROUPS];
    // chunk 4g + l/16 of a row sits at slot (4g + l/16) xor (l mod 16) = 4g xor c, c = (l/16) xor (l mod 16)
#pragma unroll
    for (int g = 0; g < GROUPS; ++g) {
        if (!TAIL || g < gmax) {
            wf[g] = *reinterpret_cast<const bf16x8*>(wrow + ((4 * g) ^ c) * 8);
            xf[g] = *reinterpret_cast<const bf16x8*>(xrow + ((4 * g) ^ c) * 8);
        }
    }
    __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of the chain
#pragma unroll
    for (int g = 0; g < GROUPS; ++g)
        if (!TAIL || g < gmax) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[g], xf[g], acc, 0, 0, 0);
}

template <int MT, bool EPI>
__global__ __launch_bounds__(THREADS) void k_gemv_mfma(const GemvMfmaArgs a) {
    using R = Ring<MT>;
    __shared__ __attribute__((aligned(16))) uint16_t ring[NST * R::STAGE];
    __shared__ __attribute__((aligned(16))) uint16_t zero_row[SK];   // the x operand of unstaged rows
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * NB;
    const int groups = (a.K + 31) / 32;
    const int stages = (groups + GROUPS - 1) / GROUPS;

    const int p = wave - 1;   // producer index (wave 0 is the consumer)
    if (wave > 0) {
#pragma unroll
        for (int s = 0; s < NST - 1; ++s)
            if (s < stages) issue_stage<MT>(a, n0, p, lane, s, ring + s * R::STAGE);
    }

    if (MT < 16)   // read by wave 0 only after the first barrier below
        for (int i = threadIdx.x; i < SK / 2; i += THREADS) reinterpret_cast<uint32_t*>(zero_row)[i] = 0u;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const int lr = lane & 15, lq = lane >> 4, c = lq ^ lr;
    for (int s = 0; s < stages; ++s) {
        if (wave > 0) wait_stage<MT>(p, min(NST - 2, stages - 1 - s));
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): wave 0's reads of the previous stage are done
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
        if (wave > 0) {
            // the buffer of stage s - 1 is free: request stage s + NST - 1 into it
            if (s + NST - 1 < stages)
                issue_stage<MT>(a, n0, p, lane, s + NST - 1, ring + ((s + NST - 1) % NST) * R::STAGE);
        } else {
            // wave 0 has no loads of its own in flight, so the wait for outstanding loads that the
            // compiler puts before these LDS reads (it cannot tell the direct-to-LDS loads of later
            // stages from this stage's data) costs nothing
            const uint16_t* buf = ring + (s % NST) * R::STAGE;
            const uint16_t* wrow = buf + lr * R::ROW;
            const uint16_t* xrow = lr < MT ? buf + (NB + lr) * R::ROW : zero_row;
            if (s + 1 < stages) fold_stage<false>(wrow, xrow, c, GROUPS, acc);
            else fold_stage<true>(wrow, xrow, c, groups - s * GROUPS, acc);
        }
    }
    if (wave == 0) {
        // lane l holds D[4 (l / 16) + r][l mod 16]: outputs n0 + 4 (l / 16) + r of row m = l mod 16
        const int m = lr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t n = n0 + 4 * lq + r;
            if (m < a.M && n < a.N) {
                if constexpr (EPI) epi_store(a.ep, a.y, a.ldy, m, n, acc[r]);
                else static_cast<float*>(a.y)[m * a.ldy + n] = acc[r];
            }
        }
    }
}

template <int MT>
hipError_t launch_mt(const GemvMfmaArgs& a, hipStream_t stream) {
    const int64_t blocks = (a.N + NB - 1) / NB;
    if (epi_identity(a.ep))
        hipLaunchKernelGGL((k_gemv_mfma<MT, false>), dim3(static_cast<unsigned>(blocks)), dim3(THREADS), 0, stream, a);
    else
        hipLaunchKernelGGL((k_gemv_mfma<MT, true>), dim3(static_cast<unsigned>(blocks)), dim3(THREADS), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

// Stage offsets along a row are 32-bit byte offsets: (stages + NST) * 1 KiB must stay below 2^31.
int gemv_mfma_max_k() { return (1 << 29) - (NST + 1) * SK; }

hipError_t launch_gemv_mfma(const GemvMfmaArgs& a, hipStream_t stream) {
    // MT (rows of x staged per stage: M rounded up to a power of two, or the caller's forced value) only
    // sets how many rows are loaded; the instruction always covers 16, and no output's operands or order
    // depend on it.
    const int mt = a.rows ? a.rows : a.M <= 1 ? 1 : a.M <= 2 ? 2 : a.M <= 4 ? 4 : a.M <= 8 ? 8 : 16;
    switch (mt) {
    case 1: return launch_mt<1>(a, stream);
    case 2: return launch_mt<2>(a, stream);
    case 4: return launch_mt<4>(a, stream);
    case 8: return launch_mt<8>(a, stream);
    default: return launch_mt<16>(a, stream);
    }
}
