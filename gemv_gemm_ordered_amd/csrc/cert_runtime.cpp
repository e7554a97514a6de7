// Certificate engine for a decode loop ("Same Bits on the CPU and the GPU", section "The CPU as a
// checker: a float Freivalds certificate", and the costs it lists as unpaid: hooking the check into
// the engine through asynchronous copies on the launch path, and checking more than one sign vector
// or matrix per token, because a fault whose contributions cancel under one r escapes with
// probability 1/2).
//
// Per registered matrix the engine holds t independent sign vectors r_1..r_t over the output index
// and, in binary64, s_i = W r_i, q_k = ||W[k,:]||_2 and a_k = sum_n |w_kn| (freivalds_prepare's
// quantities). A submit copies one sampled row x (K bf16) and its output row y (N binary32) from the
// device into a pinned host slot, on the engine's own stream after an event recorded on the caller's
// stream, so the caller's next kernels do not wait for the copy. Worker threads wait for each slot's
// copy, run freivalds_check once per sign vector (the check fails if any vector rejects) and return
// the slot. When every slot is in use, submit waits for a worker (back pressure), so the ring bounds
// both host memory and how far the checks may trail the GPU.
//
// A worker learns that its slot's copy has landed from the slot's flag: a word of pinned host memory
// that a small kernel on the engine's stream sets to the slot's sequence number after the copy. The
// worker polls that word (no runtime call on the way, so the workers never contend with the thread
// that launches the decode kernels) and falls back to synchronising the copy stream, which also
// reports a failed copy, only when the flag is late.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <condition_variable>
#include <cstring>
#include <deque>
#include <memory>
#include <mutex>
#include <thread>
#include <vector>

#include "../../include/ggo.h"
#include "kernels.hpp"

namespace {

struct Matrix {
    int64_t K = 0, N = 0;
    int nr = 0;
    std::vector<int8_t> r;     // nr x N
    std::vector<double> s;     // nr x K
    std::vector<double> q, a;  // K
};

struct Slot {
    uint16_t* x = nullptr;     // pinned, max_K
    float* y = nullptr;        // pinned, max_N
    uint16_t* x_dev = nullptr; // the same memory as the GPU addresses it
    float* y_dev = nullptr;
    uint32_t* flag = nullptr;  // pinned; set to seq on the engine's stream once the copy has landed
    uint32_t* flag_dev = nullptr;
    uint32_t seq = 0;          // sequence number of the submit that filled the slot
    int matrix = -1;
    int64_t token = 0;
    bool device = true;        // false: filled from host memory by ggo_cert_submit_host
};

}  // namespace

struct ggo_cert {
    int64_t max_K = 0, max_N = 0;
    double c_f = 0.125;
    bool host_only = false;            // slots in ordinary memory; only ggo_cert_submit_host
    std::mutex submit_mu;              // one submit at a time uses ready_evt
    hipStream_t copy_stream = nullptr;
    hipEvent_t ready_evt = nullptr;    // recorded on the caller's stream, waited on by copy_stream
    uint32_t* flags = nullptr;         // pinned, one 64-byte line per slot (Slot::flag)
    uint32_t next_seq = 0;             // under submit_mu
    // Registered matrices. A matrix is built, stored in its own entry and only then counted (release
    // store); readers load the count (acquire) before touching an entry, and entries never move, so a
    // matrix may be added while checks of earlier ones run.
    std::unique_ptr<Matrix> mats[GGO_CERT_MAX_MATRICES];
    std::atomic<int> nmats{0};
    std::mutex add_mu;                 // one ggo_cert_add_matrix at a time
    std::vector<Slot> slots;
    std::mutex mu;
    std::condition_variable cv_work, cv_free, cv_idle;
    std::deque<int> free_slots, queued;
    int64_t in_flight = 0;             // submitted and not yet checked
    bool stop = false;
    std::vector<std::thread> workers;
    // statistics (under mu)
    int64_t submitted = 0, checked = 0, failed = 0;
    double max_ratio = 0.0, check_seconds = 0.0, wait_seconds = 0.0, submit_wait_seconds = 0.0;
    std::atomic<int64_t> submit_ns{0};   // launching thread's time inside ggo_cert_submit_rows
    std::vector<std::pair<int64_t, int>> failures;   // (token, matrix), oldest first
    int copy_error = 0;
};

namespace {

using Clock = std::chrono::steady_clock;

// Wait until the copy into slot s has landed. Poll the slot's flag: with pause instructions between
// looks for the first SPIN, then yielding the core between looks, for up to POLL; past that (a copy stuck behind a long kernel, or one that failed) synchronise the
// engine's copy stream, which finishes at or after this slot's copy and returns the error of a failed
// one. (No per-slot event: recording one per row cost a runtime call per row on the launch path.)
bool wait_copy(hipStream_t copy_stream, Slot& s) {
    constexpr auto SPIN = std::chrono::microseconds(100);   // a copy normally lands within tens of us
    constexpr auto POLL = std::chrono::milliseconds(2);
    const auto t0 = Clock::now();
    for (;;) {
        if (__atomic_load_n(s.flag, __ATOMIC_ACQUIRE) == s.seq) return true;
        const auto waited = Clock::now() - t0;
        if (waited > POLL) break;
        if (waited < SPIN) {
            for (int i = 0; i < 32; ++i) __builtin_ia32_pause();   // no system call while the copy is due
        } else {
            std::this_thread::yield();
        }
    }
    if (hipStreamSynchronize(copy_stream) != hipSuccess) return false;
    return __atomic_load_n(s.flag, __ATOMIC_ACQUIRE) == s.seq;
}

void worker_loop(ggo_cert* c) {
    std::vector<double> out(4 * FREIVALDS_MAX_T);
    for (;;) {
        int id;
        bool more;
        {
            std::unique_lock<std::mutex> lk(c->mu);
            c->cv_work.wait(lk, [&] { return c->stop || !c->queued.empty(); });
            if (c->queued.empty()) return;   // stop requested and nothing left
            id = c->queued.front();
            c->queued.pop_front();
            more = !c->queued.empty();
        }
        if (more) c->cv_work.notify_one();   // pass the wake-up on: the submitting thread wakes one worker only
        Slot& sl = c->slots[id];
        bool copy_ok = true;
        const auto tw = Clock::now();
        if (sl.device) copy_ok = wait_copy(c->copy_stream, sl);
        const Matrix& m = *c->mats[sl.matrix];
        bool pass = true;
        double worst = 0.0;
        const auto t0 = Clock::now();
        const double waited = std::chrono::duration<double>(t0 - tw).count();
        if (copy_ok) {
            // all sign vectors in one pass over the row (up to FREIVALDS_MAX_T at a time)
            for (int v0 = 0; v0 < m.nr; v0 += FREIVALDS_MAX_T) {
                const int t = std::min(FREIVALDS_MAX_T, m.nr - v0);
                const int rc = freivalds_check_multi(t, m.s.data() + static_cast<int64_t>(v0) * m.K, m.q.data(), m.a.data(),
                                                     m.r.data() + static_cast<int64_t>(v0) * m.N, m.K, m.N, sl.x, sl.y,
                                                     c->c_f, out.data());
                if (rc < 0) copy_ok = false;
                if (rc != 1) pass = false;
                for (int v = 0; v < t; ++v)
                    if (out[4 * v + 1] > 0.0) worst = std::max(worst, out[4 * v] / out[4 * v + 1]);
            }
        }
        const double dt = std::chrono::duration<double>(Clock::now() - t0).count();
        {
            std::lock_guard<std::mutex> lk(c->mu);
            c->checked += 1;
            c->check_seconds += dt;
            c->wait_seconds += waited;
            if (!copy_ok) c->copy_error = 1;
            if (!pass || !copy_ok) {
                c->failed += 1;
                c->failures.emplace_back(sl.token, sl.matrix);
            } else if (worst > c->max_ratio) {
                c->max_ratio = worst;
            }
            c->free_slots.push_back(id);
            c->in_flight -= 1;
        }
        c->cv_free.notify_one();
        c->cv_idle.notify_all();
    }
}

// Take a free slot, waiting for a worker to return one if the ring is full.
int take_slot(ggo_cert* c) {
    std::unique_lock<std::mutex> lk(c->mu);
    if (c->free_slots.empty()) {
        const auto t0 = Clock::now();
        c->cv_free.wait(lk, [&] { return !c->free_slots.empty(); });
        c->submit_wait_seconds += std::chrono::duration<double>(Clock::now() - t0).count();
    }
    const int id = c->free_slots.front();
    c->free_slots.pop_front();
    c->in_flight += 1;
    c->submitted += 1;
    return id;
}

// n slots under one lock (the workers take the same lock after every check).
void take_slots(ggo_cert* c, int64_t n, int* ids) {
    std::unique_lock<std::mutex> lk(c->mu);
    for (int64_t i = 0; i < n; ++i) {
        if (c->free_slots.empty()) {
            const auto t0 = Clock::now();
            c->cv_free.wait(lk, [&] { return !c->free_slots.empty(); });
            c->submit_wait_seconds += std::chrono::duration<double>(Clock::now() - t0).count();
        }
        ids[i] = c->free_slots.front();
        c->free_slots.pop_front();
        c->in_flight += 1;
        c->submitted += 1;
    }
}

void enqueue(ggo_cert* c, int id) {
    {
        std::lock_guard<std::mutex> lk(c->mu);
        c->queued.push_back(id);
    }
    c->cv_work.notify_one();
}

// The rows of one submit in one step: one lock and one wake-up on the launching thread; the woken
// worker wakes the next while rows remain (a wake-up per row, or waking every worker, was a system
// call per worker on the launching thread: about 11 us per token of seven rows).
void enqueue_batch(ggo_cert* c, const int* ids, int64_t n) {
    {
        std::lock_guard<std::mutex> lk(c->mu);
        for (int64_t i = 0; i < n; ++i) c->queued.push_back(ids[i]);
    }
    c->cv_work.notify_one();
}

// One launch copies every row of a batch into its pinned slot (host memory the GPU writes through its
// mapping), instead of two runtime copies per row: 2 x rows segments, one per blockIdx.y.
constexpr int MAX_BATCH = 16;
struct GatherSeg {
    const uint16_t* src;
    uint16_t* dst;
    int64_t count;   // 16-bit elements
    int vec;         // src and dst 16-byte aligned: copy 8 elements per load and store
};
struct GatherArgs {
    GatherSeg seg[2 * MAX_BATCH];
};
constexpr int GATHER_THREADS = 256, GATHER_MAX_BLOCKS = 8;

// Each workgroup copies its share, every wave waits for its own stores, and after the barrier one
// thread makes them visible to the host with a single system-scope fence. (A fence in every thread
// cost about 60 us per launch on a decode step's seven rows: each one writes back the cache.)
__global__ __launch_bounds__(GATHER_THREADS) void k_cert_gather(GatherArgs a) {
    const GatherSeg s = a.seg[blockIdx.y];
    const int64_t stride = static_cast<int64_t>(gridDim.x) * GATHER_THREADS;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * GATHER_THREADS + threadIdx.x;
    int64_t done = 0;
    if (s.vec) {
        const int64_t n8 = s.count / 8;
        const uint4* src = reinterpret_cast<const uint4*>(s.src);
        uint4* dst = reinterpret_cast<uint4*>(s.dst);
        for (int64_t i = t0; i < n8; i += stride) dst[i] = src[i];
        done = 8 * n8;
    }
    for (int64_t i = done + t0; i < s.count; i += stride) s.dst[i] = s.src[i];
    __builtin_amdgcn_s_waitcnt(0);   // this wave's stores have completed
    __syncthreads();
    if (threadIdx.x == 0) __threadfence_system();   // ... and are visible to the host before the kernel ends
}

// Runs after the copies of a batch on the engine's stream: sets each slot's flag to its sequence
// number (a release store to host memory, read by the workers with an acquire load).
struct FlagArgs {
    uint32_t* flag[MAX_BATCH];
    uint32_t seq[MAX_BATCH];
    int n;
};

__global__ void k_cert_flags(FlagArgs a) {
    const int i = threadIdx.x;
    if (i < a.n) __hip_atomic_store(a.flag[i], a.seq[i], __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Queue the flag kernel for slots sid[0 .. n) on the engine's stream.
hipError_t mark_landed(ggo_cert* c, const int* sid, int64_t n) {
    FlagArgs fa{};
    fa.n = static_cast<int>(n);
    for (int64_t i = 0; i < n; ++i) {
        fa.flag[i] = c->slots[sid[i]].flag_dev;
        fa.seq[i] = c->slots[sid[i]].seq;
    }
    hipLaunchKernelGGL(k_cert_flags, dim3(1), dim3(64), 0, c->copy_stream, fa);
    return hipGetLastError();
}

inline double widen(uint16_t b) {
    const uint32_t u = static_cast<uint32_t>(b) << 16;
    float f;
    std::memcpy(&f, &u, sizeof f);
    return static_cast<double>(f);
}

}  // namespace

extern "C" {

static int create(int64_t max_K, int64_t max_N, int64_t nslots, int nworkers, double c_f, bool host_only,
                  ggo_cert** out) {
    if (!out || max_K < 1 || max_N < 1 || nslots < 1 || nslots > 4096 || nworkers < 1 || nworkers > 64 || !(c_f > 0.0))
        return GGO_EINVAL;
    *out = nullptr;
    ggo_cert* c = new ggo_cert;
    c->max_K = max_K;
    c->max_N = max_N;
    c->c_f = c_f;
    c->host_only = host_only;
    c->slots.resize(static_cast<size_t>(nslots));
    int rc = GGO_OK;
    uint32_t* flags_dev = nullptr;
    if (!host_only) {
        constexpr size_t LINE = 64 / sizeof(uint32_t);   // one flag per 64-byte line
        if (hipHostMalloc(reinterpret_cast<void**>(&c->flags), static_cast<size_t>(nslots) * 64) != hipSuccess ||
            hipHostGetDevicePointer(reinterpret_cast<void**>(&flags_dev), c->flags, 0) != hipSuccess) {
            rc = GGO_ELAUNCH;
        } else {
            std::memset(c->flags, 0, static_cast<size_t>(nslots) * 64);
            for (int64_t i = 0; i < nslots; ++i) {
                c->slots[i].flag = c->flags + i * LINE;
                c->slots[i].flag_dev = flags_dev + i * LINE;
            }
        }
    }
    for (int64_t i = 0; i < nslots && rc == GGO_OK; ++i) {
        Slot& s = c->slots[i];
        if (host_only) {
            s.x = new uint16_t[static_cast<size_t>(max_K)];
            s.y = new float[static_cast<size_t>(max_N)];
        } else if (hipHostMalloc(reinterpret_cast<void**>(&s.x), static_cast<size_t>(max_K) * 2) != hipSuccess ||
                   hipHostMalloc(reinterpret_cast<void**>(&s.y), static_cast<size_t>(max_N) * 4) != hipSuccess ||
                   hipHostGetDevicePointer(reinterpret_cast<void**>(&s.x_dev), s.x, 0) != hipSuccess ||
                   hipHostGetDevicePointer(reinterpret_cast<void**>(&s.y_dev), s.y, 0) != hipSuccess) {
            rc = GGO_ELAUNCH;
        }
        c->free_slots.push_back(static_cast<int>(i));
    }
    if (rc == GGO_OK && !host_only &&
        (hipStreamCreateWithFlags(&c->copy_stream, hipStreamNonBlocking) != hipSuccess ||
         hipEventCreateWithFlags(&c->ready_evt, hipEventDisableTiming) != hipSuccess))
        rc = GGO_ELAUNCH;
    if (rc == GGO_OK && !host_only) {
        // The first launch of a kernel of this source loads its code object (tens of ms); pay that here,
        // with a flag kernel that writes nothing, rather than on the first token of a decode loop.
        FlagArgs none{};
        hipLaunchKernelGGL(k_cert_flags, dim3(1), dim3(64), 0, c->copy_stream, none);
        if (hipGetLastError() != hipSuccess || hipStreamSynchronize(c->copy_stream) != hipSuccess) rc = GGO_ELAUNCH;
    }
    if (rc != GGO_OK) {
        ggo_cert_destroy(c);
        return rc;
    }
    for (int i = 0; i < nworkers; ++i) c->workers.emplace_back(worker_loop, c);
    *out = c;
    return GGO_OK;
}

int ggo_cert_create(int64_t max_K, int64_t max_N, int64_t nslots, int nworkers, double c_f, ggo_cert** out) {
    return create(max_K, max_N, nslots, nworkers, c_f, false, out);
}

int ggo_cert_create_host(int64_t max_K, int64_t max_N, int64_t nslots, int nworkers, double c_f, ggo_cert** out) {
    return create(max_K, max_N, nslots, nworkers, c_f, true, out);
}

int ggo_cert_add_matrix(ggo_cert* c, const uint16_t* W, int64_t ld, int transposed, int64_t K, int64_t N,
                        const int8_t* r, int64_t nr, int* id) {
    if (!c || !W || !r || !id || K < 1 || N < 1 || nr < 1 || nr > 64 || K > c->max_K || N > c->max_N) return GGO_EINVAL;
    if (ld < (transposed ? K : N)) return GGO_EINVAL;
    for (int64_t i = 0; i < nr * N; ++i)
        if (r[i] != 1 && r[i] != -1) return GGO_EINVAL;
    Matrix m;
    m.K = K;
    m.N = N;
    m.nr = static_cast<int>(nr);
    m.r.assign(r, r + nr * N);
    m.s.assign(static_cast<size_t>(nr * K), 0.0);
    m.q.assign(static_cast<size_t>(K), 0.0);
    m.a.assign(static_cast<size_t>(K), 0.0);
    // s_v[k] = sum_n w[k,n] r_v[n], q[k] = ||w[k,:]||_2, a[k] = sum_n |w[k,n]|, each summed over n in
    // ascending order in binary64 (the order freivalds_prepare uses)
    for (int64_t k = 0; k < K; ++k) {
        double qk = 0.0, ak = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            const double w = widen(transposed ? W[n * ld + k] : W[k * ld + n]);
            qk += w * w;
            ak += std::fabs(w);
            for (int64_t v = 0; v < nr; ++v) m.s[v * K + k] += r[v * N + n] > 0 ? w : -w;
        }
        m.q[k] = std::sqrt(qk);
        m.a[k] = ak;
    }
    std::lock_guard<std::mutex> lk(c->add_mu);
    const int n = c->nmats.load(std::memory_order_relaxed);
    if (n >= GGO_CERT_MAX_MATRICES) return GGO_EUNSUPPORTED;
    c->mats[n].reset(new Matrix(std::move(m)));
    c->nmats.store(n + 1, std::memory_order_release);
    *id = n;
    return GGO_OK;
}

static bool matrix_known(ggo_cert* c, int id) { return id >= 0 && id < c->nmats.load(std::memory_order_acquire); }

int ggo_cert_submit(ggo_cert* c, int id, const uint16_t* x_dev, const float* y_dev, int64_t token, void* stream) {
    if (!c || c->host_only || !x_dev || !y_dev || !matrix_known(c, id)) return GGO_EINVAL;
    const Matrix& m = *c->mats[id];
    std::lock_guard<std::mutex> one_submit(c->submit_mu);
    const int sid = take_slot(c);
    Slot& s = c->slots[sid];
    s.matrix = id;
    s.token = token;
    s.device = true;
    s.seq = ++c->next_seq;
    hipStream_t caller = static_cast<hipStream_t>(stream);
    hipError_t e = hipEventRecord(c->ready_evt, caller);
    if (e == hipSuccess) e = hipStreamWaitEvent(c->copy_stream, c->ready_evt, 0);
    if (e == hipSuccess) e = hipMemcpyAsync(s.x, x_dev, static_cast<size_t>(m.K) * 2, hipMemcpyDeviceToHost, c->copy_stream);
    if (e == hipSuccess) e = hipMemcpyAsync(s.y, y_dev, static_cast<size_t>(m.N) * 4, hipMemcpyDeviceToHost, c->copy_stream);
    if (e == hipSuccess) e = mark_landed(c, &sid, 1);
    if (e != hipSuccess) {
        std::lock_guard<std::mutex> lk(c->mu);
        c->free_slots.push_back(sid);
        c->in_flight -= 1;
        c->submitted -= 1;
        c->copy_error = 1;
        return GGO_ELAUNCH;
    }
    enqueue(c, sid);
    return GGO_OK;
}

int ggo_cert_submit_rows(ggo_cert* c, int64_t n, const int* ids, const uint16_t* const* x_dev,
                         const float* const* y_dev, int64_t token, void* stream) {
    // n slots are held until all are taken, so a batch larger than the ring could never be served
    if (!c || c->host_only || n < 1 || n > MAX_BATCH || n > static_cast<int64_t>(c->slots.size()) || !ids || !x_dev ||
        !y_dev)
        return GGO_EINVAL;
    for (int64_t i = 0; i < n; ++i)
        if (!matrix_known(c, ids[i]) || !x_dev[i] || !y_dev[i]) return GGO_EINVAL;
    std::lock_guard<std::mutex> one_submit(c->submit_mu);
    const auto t_submit = Clock::now();
    struct AddTime {   // on every return path
        ggo_cert* c;
        Clock::time_point t0;
        ~AddTime() {
            c->submit_ns.fetch_add(std::chrono::duration_cast<std::chrono::nanoseconds>(Clock::now() - t0).count(),
                                   std::memory_order_relaxed);
        }
    } add_time{c, t_submit};
    int sid[MAX_BATCH];
    take_slots(c, n, sid);
    GatherArgs ga;
    int64_t longest = 1;
    for (int64_t i = 0; i < n; ++i) {
        const Matrix& m = *c->mats[ids[i]];
        Slot& s = c->slots[sid[i]];
        s.matrix = ids[i];
        s.token = token;
        s.device = true;
        s.seq = ++c->next_seq;
        auto seg = [](const void* src, void* dst, int64_t count) {
            const bool vec = ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) == 0;
            return GatherSeg{static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), count, vec ? 1 : 0};
        };
        ga.seg[2 * i] = seg(x_dev[i], s.x_dev, m.K);
        ga.seg[2 * i + 1] = seg(y_dev[i], s.y_dev, 2 * m.N);
        longest = std::max(longest, 2 * m.N);
        longest = std::max(longest, m.K);
    }
    hipStream_t caller = static_cast<hipStream_t>(stream);
    hipError_t e = hipEventRecord(c->ready_evt, caller);
    if (e == hipSuccess) e = hipStreamWaitEvent(c->copy_stream, c->ready_evt, 0);
    if (e == hipSuccess) {
        // blocks per row: enough for one 16-byte copy per thread, at most GATHER_MAX_BLOCKS
        const int64_t per_block = 8 * GATHER_THREADS;
        const unsigned bx = static_cast<unsigned>(std::min<int64_t>((longest + per_block - 1) / per_block, GATHER_MAX_BLOCKS));
        hipLaunchKernelGGL(k_cert_gather, dim3(bx, static_cast<unsigned>(2 * n)), dim3(GATHER_THREADS), 0, c->copy_stream, ga);
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = mark_landed(c, sid, n);
    if (e != hipSuccess) {
        std::lock_guard<std::mutex> lk(c->mu);
        for (int64_t i = 0; i < n; ++i) {
            c->free_slots.push_back(sid[i]);
            c->in_flight -= 1;
            c->submitted -= 1;
        }
        c->copy_error = 1;
        return GGO_ELAUNCH;
    }
    enqueue_batch(c, sid, n);
    return GGO_OK;
}

int ggo_cert_submit_host(ggo_cert* c, int id, const uint16_t* x, const float* y, int64_t token) {
    if (!c || !x || !y || !matrix_known(c, id)) return GGO_EINVAL;
    const Matrix& m = *c->mats[id];
    const int sid = take_slot(c);
    Slot& s = c->slots[sid];
    s.matrix = id;
    s.token = token;
    s.device = false;
    std::memcpy(s.x, x, static_cast<size_t>(m.K) * 2);
    std::memcpy(s.y, y, static_cast<size_t>(m.N) * 4);
    enqueue(c, sid);
    return GGO_OK;
}

int ggo_cert_drain(ggo_cert* c, ggo_cert_stats* out) {
    if (!c) return GGO_EINVAL;
    std::unique_lock<std::mutex> lk(c->mu);
    c->cv_idle.wait(lk, [&] { return c->in_flight == 0; });
    if (out) {
        out->submitted = c->submitted;
        out->checked = c->checked;
        out->failed = c->failed;
        out->max_honest_ratio = c->max_ratio;
        out->check_seconds = c->check_seconds;
        out->copy_error = c->copy_error;
        out->wait_seconds = c->wait_seconds;
        out->submit_wait_seconds = c->submit_wait_seconds;
        out->submit_seconds = 1e-9 * static_cast<double>(c->submit_ns.load(std::memory_order_relaxed));
    }
    return GGO_OK;
}

int64_t ggo_cert_failures(ggo_cert* c, int64_t* tokens, int* matrices, int64_t cap) {
    if (!c || cap < 0 || (cap && (!tokens || !matrices))) return GGO_EINVAL;
    std::lock_guard<std::mutex> lk(c->mu);
    const int64_t n = std::min<int64_t>(cap, static_cast<int64_t>(c->failures.size()));
    for (int64_t i = 0; i < n; ++i) {
        tokens[i] = c->failures[i].first;
        matrices[i] = c->failures[i].second;
    }
    return static_cast<int64_t>(c->failures.size());
}

void ggo_cert_destroy(ggo_cert* c) {
    if (!c) return;
    {
        std::lock_guard<std::mutex> lk(c->mu);
        c->stop = true;
    }
    c->cv_work.notify_all();
    for (auto& t : c->workers) t.join();
    if (c->copy_stream) hipStreamSynchronize(c->copy_stream);
    for (auto& s : c->slots) {
        if (c->host_only) {
            delete[] s.x;
            delete[] s.y;
            continue;
        }
        if (s.x) hipHostFree(s.x);
        if (s.y) hipHostFree(s.y);
    }
    if (c->flags) hipHostFree(c->flags);
    if (c->ready_evt) hipEventDestroy(c->ready_evt);
    if (c->copy_stream) hipStreamDestroy(c->copy_stream);
    delete c;
}

}  // extern "C"
