// Tree-ordered GEMV for decode shapes: y[m, n] = sum_k x[m, k] * WT[n, k], with the weight given
// transposed ([N, K], k contiguous: the layout of a linear layer's weight).
//
// The order ("Taming Bitwise Behavior in GPU Kernels with Tensor Core", section 3.2.2, the GEMV
// paragraph and Figure 2(d); section 5.1 for the pinned butterfly). It depends on K alone, never on
// M, N, the workgroup shape or the launch:
//   * the k axis is cut into tiles of 8; chain p (0 <= p < 256) takes the tiles p, p + 256,
//     p + 512, ... and folds their k in ascending order with one fused multiply-add per k,
//     acc = fma(x, w, acc), starting from +0;
//   * the 256 chain totals are added by a balanced pairwise tree that pairs neighbours first
//     (chains 2i and 2i+1, then neighbouring pairs, ...).
// bfloat16 products are exact in binary32, so each fused step rounds only the sum.
//
// Mapping. A workgroup is four waves and owns R consecutive outputs n, for every row m of x (MT is
// M rounded up to a power of two; rows past M read as zero and are not stored). Lane l of wave w
// is chain p = 64 w + l. Step j of the lane loads tile p + 256 j of its R weight rows and of the
// MT rows of x, 16 bytes each (a wave reads 1 KiB of one weight row per load), and folds the tile
// into R x MT accumulators. The steps of a lane never wait on another lane.
//
// The tree then runs on the lanes. Within a wave the first six levels pair lanes l and l xor 1,
// then l xor 2, ..., l xor 32, the count-up tree of section 5.1's wave reduction; since every lane
// holds R x MT accumulators, each level also hands half of them to the partner lane, so a level
// costs half the adds of the one before (a reduce-scatter). The last two levels add the four wave
// totals, (w0 + w1) + (w2 + w3), read back from LDS.
//
// Loads go through raw buffer descriptors, one per row, whose range is exactly the K elements of
// that row (empty for rows past M or N): a load past K returns 0 without touching memory, and a
// +0 product leaves every accumulator's bits unchanged (a chain started at +0 never holds -0).
// The wide instances load 16 bytes per row and tile and need K, both row strides multiples of 8
// and 16-byte aligned operands (then no load straddles the end of a row); the narrow instances load
// 2 bytes per element and take any operands. The result of each output goes through the fused
// epilogue (epilogue.hpp) on its way out.
#include <algorithm>
#include <atomic>

#include "common.hpp"
#include "kernels.hpp"

#pragma clang fp contract(off)

namespace {

constexpr int TILE = 8;                 // k per tile
constexpr int CHAINS = 256;             // chains per output
constexpr int WAVES = CHAINS / 64;      // one chain per lane
constexpr int THREADS = 64 * WAVES;
constexpr int STEP_BYTES = TILE * CHAINS * 2;   // bytes of a row covered by one step of all chains
constexpr int BUF_DWORD3 = 0x00020000;  // buffer descriptor word 3: raw 32-bit data, range checked

using rsrc_t = __amdgpu_buffer_rsrc_t;

GGO_DEV rsrc_t row_rsrc(const uint16_t* row, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(row), 0, bytes, BUF_DWORD3);
}

// Cache policy of the weight loads: nontemporal (each weight byte is read once per call).
constexpr int AUX_STREAM = 2;

// One tile (8 bf16) of one row, as 4 dwords: dword i holds k0 + 2i (low half) and k0 + 2i + 1.
template <bool WIDE, int AUX = 0>
GGO_DEV void load_tile(rsrc_t r, int off, uint32_t (&d)[4]) {
    if constexpr (WIDE) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
        d[0] = v[0];
        d[1] = v[1];
        d[2] = v[2];
        d[3] = v[3];
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(r, off + 4 * i, 0, 0);
            const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(r, off + 4 * i + 2, 0, 0);
            d[i] = lo | (hi << 16);
        }
    }
}

template <int MT, int R, bool WIDE>
GGO_DEV void load_step(const rsrc_t (&wr)[R], const rsrc_t (&xr)[MT], int off, uint32_t (&w)[R][4],
                       uint32_t (&x)[MT][4]) {
    // x first: a wait for the x tiles (hits in L2) then never waits behind weight rows from HBM
#pragma unroll
    for (int m = 0; m < MT; ++m) load_tile<WIDE>(xr[m], off, x[m]);
#pragma unroll
    for (int r = 0; r < R; ++r) load_tile<WIDE, AUX_STREAM>(wr[r], off, w[r]);
}

GGO_DEV float elem(const uint32_t (&d)[4], int e) { return (e & 1) ? bf16_hi(d[e >> 1]) : bf16_lo(d[e >> 1]); }

// Fold one tile into the accumulators: k ascending inside the tile, one fma per k.
template <int MT, int R>
GGO_DEV void fold_tile(float (&acc)[R][MT], const uint32_t (&w)[R][4], const uint32_t (&x)[MT][4]) {
#pragma unroll
    for (int e = 0; e < TILE; ++e) {
        float xf[MT], wf[R];
#pragma unroll
        for (int m = 0; m < MT; ++m) xf[m] = elem(x[m], e);
#pragma unroll
        for (int r = 0; r < R; ++r) wf[r] = elem(w[r], e);
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[r][m] = __builtin_fmaf(xf[m], wf[r], acc[r][m]);
    }
}

template <int CTRL>
GGO_DEV float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// The value lane (l xor D) holds. DPP for partners inside a row of 16 lanes: quad_perm [1,0,3,2]
// and [2,3,0,1] for D = 1, 2; for D = 4 the quad mirror followed by the half-row mirror
// (l -> l^3 -> (l^3)^7 = l^4); row_ror:8 for D = 8. D = 16 and 32 go through ds_bpermute.
template <int D>
GGO_DEV float xor_lane(float v) {
    if constexpr (D == 1) return dpp<0xb1>(v);
    else if constexpr (D == 2) return dpp<0x4e>(v);
    else if constexpr (D == 4) return dpp<0x141>(dpp<0x1b>(v));
    else if constexpr (D == 8) return dpp<0x128>(v);
    else return __shfl_xor(v, D);
}

// Count-up tree over the 64 lanes of a wave for each of the C values a lane holds (v[0 .. C)),
// one level per lane bit D = 1, 2, 4, ..., 32: the partial sums over aligned blocks of D lanes are
// added in pairs, (block) + (block next to it), exactly the tree of the DPP row_shr 1, 2, 4, 8 and
// row_bcast 15, 31 reduction. While a lane still holds several values, each level also halves
// them (a reduce-scatter): the lane with bit D clear keeps the lower half of the indices, its
// partner the upper half, and each adds the partner's copy of what it keeps. After the C = 2^a
// values are down to one, the remaining levels add the partner's value. At the end lane l holds
// the total of value index bitrev_a(l mod C), the same in every lane with the same low a bits.
template <int C, int D, int N>
GGO_DEV void wave_tree_scatter(float (&v)[N], int lane) {
    if constexpr (D < 64) {
        if constexpr (C > 1) {
            const bool upper = (lane & D) != 0;
#pragma unroll
            for (int i = 0; i < C / 2; ++i) {
                const float keep = upper ? v[C / 2 + i] : v[i];
                const float send = upper ? v[i] : v[C / 2 + i];
                v[i] = keep + xor_lane<D>(send);
            }
            wave_tree_scatter<C / 2, 2 * D>(v, lane);
        } else {
            v[0] = v[0] + xor_lane<D>(v[0]);
            wave_tree_scatter<1, 2 * D>(v, lane);
        }
    }
}

template <int C>
GGO_DEV int scatter_index(int lane) {
    int idx = 0;
#pragma unroll
    for (int b = 1; b < C; b <<= 1) idx = (idx << 1) | ((lane & b) ? 1 : 0);
    return idx;
}

template <int MT, int R, bool WIDE, bool EPI>
__global__ __launch_bounds__(THREADS) void k_gemv_tree(TreeArgs a) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int p = wave * 64 + lane;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * R;
    const int kbytes = a.K * 2;

    rsrc_t wr[R], xr[MT];
#pragma unroll
    for (int r = 0; r < R; ++r) wr[r] = row_rsrc(a.WT + (n0 + r) * a.ldwt, n0 + r < a.N ? kbytes : 0);
#pragma unroll
    for (int m = 0; m < MT; ++m) xr[m] = row_rsrc(a.x + m * a.ldx, m < a.M ? kbytes : 0);

    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;

    // Two steps in flight: step j + 1 is requested before step j is folded. Steps past K (the
    // padding to an even count, and the one requested after the last) read as zero.
    const int steps = (a.K + TILE * CHAINS - 1) / (TILE * CHAINS);
    int off = p * TILE * 2;
    uint32_t wA[R][4], xA[MT][4], wB[R][4], xB[MT][4];
    load_step<MT, R, WIDE>(wr, xr, off, wA, xA);
    // (The scheduling barriers keep each request ahead of the fold that precedes it in the source;
    // left alone, the scheduler sinks the loads of step j + 1 below the fold of step j.)
    for (int j = 0; j < steps; j += 2) {
        load_step<MT, R, WIDE>(wr, xr, off + STEP_BYTES, wB, xB);
        __builtin_amdgcn_sched_barrier(0);
        fold_tile<MT, R>(acc, wA, xA);
        __builtin_amdgcn_sched_barrier(0);
        load_step<MT, R, WIDE>(wr, xr, off + 2 * STEP_BYTES, wA, xA);
        __builtin_amdgcn_sched_barrier(0);
        fold_tile<MT, R>(acc, wB, xB);
        __builtin_amdgcn_sched_barrier(0);
        off += 2 * STEP_BYTES;
    }

    constexpr int V = R * MT;
    static_assert(V <= 64 && (V & (V - 1)) == 0, "one wave total per lane at most, a power of two");
    float v[V];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) v[r * MT + m] = acc[r][m];
    wave_tree_scatter<V, 1>(v, lane);
    __shared__ float red[WAVES][V];
    if (lane < V) red[wave][scatter_index<V>(lane)] = v[0];
    __syncthreads();
    for (int i = threadIdx.x; i < R * MT; i += THREADS) {
        const int r = i / MT, m = i % MT;
        if (m < a.M && n0 + r < a.N) {
            const float v = (red[0][i] + red[1][i]) + (red[2][i] + red[3][i]);
            if constexpr (EPI) epi_store(a.ep, a.y, a.ldy, m, n0 + r, v);
            else static_cast<float*>(a.y)[m * a.ldy + n0 + r] = v;
        }
    }
}

// The same arithmetic in persistent form, for 16-byte operands with K <= S * 2048 (S steps per
// chain) and M <= 8. A lane's x tiles are the same for every output n (chain p always takes the
// tiles p, p + 256, ...), so they are loaded once, widened to binary32 and kept in registers. The
// workgroup then walks groups of R outputs (consecutive groups, or with CONTIG false the groups
// blockIdx.x, blockIdx.x + gridDim.x, ...), with the weight rows of the next NB - 1 groups in flight while a
// group is folded: the weight stream and the
// FMAs overlap, and the x tiles are not fetched again for every R rows. (In the form above a
// workgroup owns one group: all of its loads, then all of its FMAs, in step with the other
// workgroups on its CU.) Every output's chains, their order and the tree are those of k_gemv_tree,
// so the bits are too.
template <int MT, int R, int S>
GGO_DEV void load_group(const TreeArgs& a, int g, int gend, int off, uint32_t (&w)[S][R][4]) {
    const int kbytes = a.K * 2;
    rsrc_t wr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t n = static_cast<int64_t>(g) * R + r;
        // past the workgroup's last group (or past N): empty
        wr[r] = row_rsrc(a.WT + n * a.ldwt, g < gend && n < a.N ? kbytes : 0);
    }
#pragma unroll
    for (int j = 0; j < S; ++j)
#pragma unroll
        for (int r = 0; r < R; ++r) load_tile<true, AUX_STREAM>(wr[r], off + j * STEP_BYTES, w[j][r]);
}

// The wave levels of the tree for one group (levels 1-6, a reduce-scatter over the lanes), left in
// LDS for the cross-wave levels: red[wave][i] is this wave's total of value i (i = r * MT + m).
template <int MT, int R>
GGO_DEV void wave_partials(float (&acc)[R][MT], float (&red)[WAVES][R * MT], int lane, int wave) {
    constexpr int V = R * MT;
    static_assert(V <= 64 && (V & (V - 1)) == 0, "one wave total per lane at most, a power of two");
    float v[V];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) v[r * MT + m] = acc[r][m];
    wave_tree_scatter<V, 1>(v, lane);
    if (lane < V) red[wave][scatter_index<V>(lane)] = v[0];
}

// Levels 7-8 of the tree, (w0 + w1) + (w2 + w3), for the cnt groups whose wave totals sit in red[0 .. cnt),
// the groups of ordinals j0 .. j0 + cnt - 1 of this workgroup (group g = first + ordinal * step), and the
// store. Called by every thread after a barrier.
template <int MT, int R, int RB, bool EPI>
GGO_DEV void finish_groups(const TreeArgs& a, const float (&red)[RB][WAVES][R * MT], int first, int step, int j0,
                           int cnt) {
    constexpr int V = R * MT;
    for (int i = threadIdx.x; i < cnt * V; i += THREADS) {
        const int q = i / V, iv = i - q * V, r = iv / MT, m = iv % MT;
        const int64_t n = (static_cast<int64_t>(first) + static_cast<int64_t>(j0 + q) * step) * R + r;
        if (m < a.M && n < a.N) {
            const float y = (red[q][0][iv] + red[q][1][iv]) + (red[q][2][iv] + red[q][3][iv]);
            if constexpr (EPI) epi_store(a.ep, a.y, a.ldy, m, n, y);
            else static_cast<float*>(a.y)[m * a.ldy + n] = y;
        }
    }
}

// fold_tile with the x tile already widened to binary32.
template <int MT, int R, int S>
GGO_DEV void fold_group(float (&acc)[R][MT], const uint32_t (&w)[S][R][4], const float (&xf)[S][MT][TILE]) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;
#pragma unroll
    for (int j = 0; j < S; ++j)          // the chain's tiles in ascending order, k ascending in each
#pragma unroll
        for (int e = 0; e < TILE; ++e) {
            float wf[R];
#pragma unroll
            for (int r = 0; r < R; ++r) wf[r] = elem(w[j][r], e);
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < MT; ++m) acc[r][m] = __builtin_fmaf(xf[j][m][e], wf[r], acc[r][m]);
        }
}

// CONTIG: workgroup b walks the gpw consecutive groups from b gpw, else the groups b, b + gridDim.x, ...
template <int MT, int R, int S, int NB, bool EPI, int RB, bool CONTIG>
__global__ __launch_bounds__(THREADS) void k_gemv_tree_p(TreeArgs a, int gpw) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int p = wave * 64 + lane;
    const int off = p * TILE * 2;
    const int groups = static_cast<int>((a.N + R - 1) / R);
    const int kbytes = a.K * 2;

    float x[S][MT][TILE];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const rsrc_t xr = row_rsrc(a.x + m * a.ldx, m < a.M ? kbytes : 0);
#pragma unroll
        for (int j = 0; j < S; ++j) {
            uint32_t d[4];
            load_tile<true>(xr, off + j * STEP_BYTES, d);
#pragma unroll
            for (int e = 0; e < TILE; ++e) x[j][m][e] = elem(d, e);
        }
    }
    // NB weight buffers in rotation. The cross-wave levels of the tree wait for a batch of RB groups
    // (RB = 1: a barrier per group):
    // each wave leaves its totals of a group in the batch's LDS slot and goes on to the next group, and
    // the workgroup meets once per batch (or at its last group) to add the four waves' totals of every
    // group in the batch. Two batch buffers alternate, so the next batch's totals never overwrite a
    // buffer that is still being read. The arithmetic is that of one barrier per group.
    __shared__ float red[2][RB][WAVES][R * MT];
    uint32_t w[NB][S][R][4];
    float acc[R][MT];
    const int first = CONTIG ? static_cast<int>(blockIdx.x) * gpw : static_cast<int>(blockIdx.x);   // < groups
    const int stride = CONTIG ? 1 : static_cast<int>(gridDim.x);
    const int gend = CONTIG ? min(groups, first + gpw) : groups;
    int g = first;
    int j = 0;                                // ordinal of the current group in this workgroup
#pragma unroll
    for (int b = 0; b + 1 < NB; ++b) load_group<MT, R, S>(a, g + b * stride, gend, off, w[b]);
    for (;;) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int gb = g + b * stride;
            load_group<MT, R, S>(a, gb + (NB - 1) * stride, gend, off, w[(b + NB - 1) % NB]);
            __builtin_amdgcn_sched_barrier(0);    // the requests stay ahead of this fold
            fold_group<MT, R, S>(acc, w[b], x);
            const int h = (j / RB) & 1, q = j % RB;
            wave_partials<MT, R>(acc, red[h][q], lane, wave);
            const bool last = gb + stride >= gend;   // uniform across the workgroup
            if (last || q == RB - 1) {
                __syncthreads();
                finish_groups<MT, R, RB, EPI>(a, red[h], first, stride, j - q, q + 1);
            }
            ++j;
            if (last) goto done;
        }
        g += NB * stride;
    }
done:
    // the loads of the groups past the end (empty ranges) return zeros to registers nobody reads;
    // they have landed before the wave ends
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
}

// Compute units of the current device (the persistent grid is a few workgroups per CU).
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v <= 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

// Persistent launch: R outputs per group, NB groups in rotation, two workgroups per CU (8 waves).
// Measured on the decode shape (N = K = 4096): two outputs per group at M <= 4 (M = 1: 6.8 us against
// 7.0 with four), one at M = 8, where the fold per group is largest. Slower, each measured at M = 8 in
// the same process: deeper rotation (NB = 3, 4: 9.5, 9.9 against 9.0 us; again with the prologue's loads
// kept in order, so that the loop waits for the oldest group only, and the groups in whole rounds with
// one batch: 10.0 - 10.4, 9.6 - 10.1 against 8.8 - 9.0, and with NB = 2 level); three workgroups per CU
// or one (9.6, 11.3); issuing the first groups' weight loads before the x tiles are widened (no change);
// raising the wave priority around the weight loads (no change); splitting the rows of x over twice or
// four times the waves, each set fetching the same weight tiles (10.8-17.7); producer waves streaming
// the weight into an LDS ring with direct-to-LDS loads and four folding waves (12.3-15.2: a barrier per
// group exposes one stage's latency to the whole workgroup).
template <int MT, int S>
hipError_t launch_persistent(const TreeArgs& a, hipStream_t stream) {
    // RB: groups per cross-wave batch. At M = 8 a barrier per group kept the waves in step and the folds
    // from overlapping the stream (R = 2: 9.6 us; batches of 4: 9.2 us; one output per group in batches
    // of 8: 8.9 us). At M <= 2 (four groups per workgroup) one batch, so one barrier, per workgroup: M = 1
    // 6.70 against 6.92 - 7.09 us with a barrier per group, M = 2 level; at M = 4 the batch was level to
    // 0.1 us slower, and it keeps a barrier per group.
    // CONTIG: each workgroup walks consecutive groups, so the rows it has in flight are neighbours (one
    // advancing window per wave instead of rows gridDim.x groups apart): M = 4 / 8 7.42 / 8.93 us against
    // 7.74 / 9.18 strided, M = 1 level (alternated three times; the same bits). With contiguous groups a
    // third group in flight gained nothing at M = 8 and a fourth lost 0.7 us.
    // RB_EP: the fused epilogue's instances take one batch at M = 4 too. Its code then runs once per
    // workgroup instead of once per group, each time on the critical path of the next barrier: M = 4 7.8 -
    // 8.0 us against 9.0 - 9.2 with a barrier per group (and 9.8 - 10.2 before that form loaded each group's
    // bias and residual a group ahead; same bits throughout).
    constexpr int R = MT >= 8 ? 1 : 2, NB = 2, PER_CU = 2, RB = MT >= 8 ? 8 : MT <= 2 ? 4 : 1;
    constexpr int RB_EP = MT >= 8 ? 8 : 4;
    constexpr bool CONTIG = true;
    const int64_t groups = (a.N + R - 1) / R;
    int64_t blocks = std::min<int64_t>(groups, static_cast<int64_t>(device_cus()) * PER_CU);
    const int gpw = static_cast<int>((groups + blocks - 1) / blocks);
    if (CONTIG) blocks = (groups + gpw - 1) / gpw;   // every workgroup has at least one group
    if (epi_identity(a.ep))
        hipLaunchKernelGGL((k_gemv_tree_p<MT, R, S, NB, false, RB, CONTIG>), dim3(static_cast<unsigned>(blocks)), dim3(THREADS), 0,
                           stream, a, gpw);
    else
        hipLaunchKernelGGL((k_gemv_tree_p<MT, R, S, NB, true, RB_EP, CONTIG>), dim3(static_cast<unsigned>(blocks)), dim3(THREADS), 0,
                           stream, a, gpw);
    return hipGetLastError();
}

template <int MT, bool WIDE>
hipError_t launch_mt(const TreeArgs& a, hipStream_t stream) {
    // Rows per workgroup: 4 keeps more workgroups (and loads) in flight; at MT = 8 the x tiles,
    // reloaded once per R rows, cost more than that, and 8 rows still fit the registers.
    constexpr int R = MT == 8 ? 8 : 4;
    const int64_t blocks = (a.N + R - 1) / R;
    if (epi_identity(a.ep))
        hipLaunchKernelGGL((k_gemv_tree<MT, R, WIDE, false>), dim3(static_cast<unsigned>(blocks)), dim3(THREADS), 0, stream, a);
    else
        hipLaunchKernelGGL((k_gemv_tree<MT, R, WIDE, true>), dim3(static_cast<unsigned>(blocks)), dim3(THREADS), 0, stream, a);
    return hipGetLastError();
}

// The instance for MT staged rows: the persistent form for 16-byte operands with at most two steps per
// chain (MT <= 8), unless the caller forces one group per workgroup (form 2), else one group per workgroup.
template <int MT>
hipError_t launch_any(const TreeArgs& a, hipStream_t stream) {
    if constexpr (MT <= 8) {
        const int steps = (a.K + TILE * CHAINS - 1) / (TILE * CHAINS);
        if (a.form != 2 && a.wide && steps <= 1) return launch_persistent<MT, 1>(a, stream);
        if (a.form != 2 && a.wide && steps == 2) return launch_persistent<MT, 2>(a, stream);
    }
    return a.wide ? launch_mt<MT, true>(a, stream) : launch_mt<MT, false>(a, stream);
}

}  // namespace

int gemv_tree_max_k() { return (1 << 29) - 3 * TILE * CHAINS; }

int gemv_tree_persistent_max_k() { return 2 * TILE * CHAINS; }

// MT, the rows of x a workgroup stages, is M rounded up to a power of two (or the caller's forced
// value): it sets how many x rows ride in registers, never an output's chains, order or tree.
hipError_t launch_gemv_tree(const TreeArgs& a, hipStream_t stream) {
    const int mt = a.rows ? a.rows : a.M <= 1 ? 1 : a.M <= 2 ? 2 : a.M <= 4 ? 4 : a.M <= 8 ? 8 : 16;
    switch (mt) {
    case 1: return launch_any<1>(a, stream);
    case 2: return launch_any<2>(a, stream);
    case 4: return launch_any<4>(a, stream);
    case 8: return launch_any<8>(a, stream);
    default: return launch_any<16>(a, stream);
    }
}
