// Float Freivalds certificate, host side ("Same Bits on the CPU and the GPU",
// section "The CPU as a checker: a float Freivalds certificate").
//
// For y = x W (y over the output index n) and signs r over n: precompute
// s = W r once per matrix in binary64, then for a sampled row compare
// rho = |r.y - x.s| with tau = c_f * sigma, sigma = 2^-24 sqrt(K) sum_k |x_k| q_k,
// q_k = ||W[k,:]||_2 -- the size of the rounding noise of a K-long binary32 fold
// under random signs. Also reported: a rigorous bound that no honest fold can
// exceed, gamma_{K-1} sum_k |x_k| a_k with a_k = sum_n |w_kn|, plus the host's
// own binary64 rounding allowance.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/ggo.h"
#include "kernels.hpp"

namespace {
inline double widen(uint16_t b) {
    const uint32_t u = static_cast<uint32_t>(b) << 16;
    float f;
    std::memcpy(&f, &u, sizeof f);
    return static_cast<double>(f);
}
}  // namespace

// One row against t sign vectors in one pass over x and y (s and r hold the t vectors' s = W r and
// signs back to back); the shared sums (|y|, |x| q, |x| a) are taken once. Every sum is split into
// L interleaved partial sums (element i goes to partial i mod L, each partial in ascending i), which
// are then added as ((p0 + p1) + (p2 + p3)): a fixed order, so the values and the verdict are a
// deterministic function of the inputs, and the same for a vector whether it is checked alone or
// with others. Independent partials keep the additions from waiting on one another (one running sum
// per quantity made the check about 3x slower). out gets (rho, sigma, tau, bound) per vector.
// Returns 1 when every vector accepts, 0 when one rejects, < 0 on bad arguments.
namespace {
constexpr int L = 4;

inline double fold4(const double (&p)[L]) { return (p[0] + p[1]) + (p[2] + p[3]); }

template <int T>
__attribute__((always_inline)) inline int check_body(const double* s, const double* q, const double* a, const int8_t* r, int64_t K, int64_t N, const uint16_t* x,
            const float* y, double c_f, double* out) {
    double ry[T][L] = {}, xs[T][L] = {}, xsmag[T][L] = {};
    double ymag[L] = {}, sxq[L] = {}, sxa[L] = {};
    auto y_step = [&](int64_t n, int j) {
        const double yn = static_cast<double>(y[n]);
        for (int v = 0; v < T; ++v) ry[v][j] += static_cast<double>(r[v * N + n]) * yn;   // r = +-1: exact
        ymag[j] += std::fabs(yn);
    };
    auto x_step = [&](int64_t k, int j) {
        const double xk = widen(x[k]);
        for (int v = 0; v < T; ++v) {
            const double tv = xk * s[v * K + k];
            xs[v][j] += tv;
            xsmag[v][j] += std::fabs(tv);
        }
        sxq[j] += std::fabs(xk) * q[k];
        sxa[j] += std::fabs(xk) * a[k];
    };
    const int64_t nf = N - N % L, kf = K - K % L;
    for (int64_t n0 = 0; n0 < nf; n0 += L)
#pragma unroll
        for (int j = 0; j < L; ++j) y_step(n0 + j, j);
    for (int64_t n = nf; n < N; ++n) y_step(n, static_cast<int>(n - nf));
    for (int64_t k0 = 0; k0 < kf; k0 += L)
#pragma unroll
        for (int j = 0; j < L; ++j) x_step(k0 + j, j);
    for (int64_t k = kf; k < K; ++k) x_step(k, static_cast<int>(k - kf));
    const double u = std::ldexp(1.0, -24);
    const double km1 = K > 0 ? static_cast<double>(K - 1) : 0.0;
    const double sigma = u * std::sqrt(static_cast<double>(K)) * fold4(sxq);
    const double tau = c_f * sigma;
    const double ym = fold4(ymag), xa = fold4(sxa);
    int all = 1;
    for (int v = 0; v < T; ++v) {
        const double rho = std::fabs(fold4(ry[v]) - fold4(xs[v]));
        const double host = 2.0 * static_cast<double>(N + K) * std::ldexp(1.0, -53) * (ym + fold4(xsmag[v]));
        out[4 * v + 0] = rho;
        out[4 * v + 1] = sigma;
        out[4 * v + 2] = tau;
        out[4 * v + 3] = km1 * u / (1.0 - km1 * u) * xa + host;
        if (!(rho <= tau)) all = 0;
    }
    return all;
}

// The same body compiled twice: for any x86-64 host, and with AVX2 (4 binary64 lanes per instruction)
// for hosts that have it. Contraction is off in both, so they compute the same values.
template <int T>
int check_plain(const double* s, const double* q, const double* a, const int8_t* r, int64_t K, int64_t N,
                const uint16_t* x, const float* y, double c_f, double* out) {
    return check_body<T>(s, q, a, r, K, N, x, y, c_f, out);
}

template <int T>
__attribute__((target("avx2"))) int check_avx2(const double* s, const double* q, const double* a, const int8_t* r,
                                               int64_t K, int64_t N, const uint16_t* x, const float* y, double c_f,
                                               double* out) {
    return check_body<T>(s, q, a, r, K, N, x, y, c_f, out);
}

template <int T>
int check_t(const double* s, const double* q, const double* a, const int8_t* r, int64_t K, int64_t N, const uint16_t* x,
            const float* y, double c_f, double* out) {
    static const bool avx2 = __builtin_cpu_supports("avx2");
    return avx2 ? check_avx2<T>(s, q, a, r, K, N, x, y, c_f, out) : check_plain<T>(s, q, a, r, K, N, x, y, c_f, out);
}
}  // namespace

int freivalds_check_multi(int t, const double* s, const double* q, const double* a, const int8_t* r, int64_t K,
                          int64_t N, const uint16_t* x, const float* y, double c_f, double* out) {
    if (t < 1 || t > FREIVALDS_MAX_T || K < 0 || N < 0 || !out || !(c_f >= 0.0)) return GGO_EINVAL;
    if ((K && (!s || !q || !a || !x)) || (N && (!r || !y))) return GGO_EINVAL;
    switch (t) {   // the vector count as a constant: the per-vector sums stay in registers
    case 1: return check_t<1>(s, q, a, r, K, N, x, y, c_f, out);
    case 2: return check_t<2>(s, q, a, r, K, N, x, y, c_f, out);
    case 3: return check_t<3>(s, q, a, r, K, N, x, y, c_f, out);
    case 4: return check_t<4>(s, q, a, r, K, N, x, y, c_f, out);
    case 5: return check_t<5>(s, q, a, r, K, N, x, y, c_f, out);
    case 6: return check_t<6>(s, q, a, r, K, N, x, y, c_f, out);
    case 7: return check_t<7>(s, q, a, r, K, N, x, y, c_f, out);
    default: {   // 8 or more: groups of 8, then the rest
        int all = 1;
        int v0 = 0;
        for (; v0 + 8 <= t; v0 += 8)
            all &= check_t<8>(s + v0 * K, q, a, r + v0 * N, K, N, x, y, c_f, out + 4 * v0);
        if (v0 < t) all &= freivalds_check_multi(t - v0, s + v0 * K, q, a, r + v0 * N, K, N, x, y, c_f, out + 4 * v0);
        return all;
    }
    }
}

namespace {
// Sign n of the stream `seed`: the top bit of splitmix64 (Steele, Lea and Flood, OOPSLA 2014) at counter n,
// i.e. of mix(seed + (n + 1) * 0x9E3779B97F4A7C15); a set bit gives -1.
int8_t sign_of(uint64_t seed, int64_t n) {
    uint64_t z = seed + (static_cast<uint64_t>(n) + 1u) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (z >> 63) ? int8_t(-1) : int8_t(1);
}
}  // namespace

// The per-matrix state of the certificate: the signs drawn from the seed and s = W r, q, a.
struct ggo_freivalds {
    int64_t K = 0, N = 0;
    std::vector<int8_t> r;
    std::vector<double> s, q, a;
};

extern "C" {

int freivalds_prepare_signs(const uint16_t* W, int64_t ldw, int64_t K, int64_t N, const int8_t* r, double* s,
                            double* q, double* a) {
    if (K < 0 || N < 0 || ldw < N) return GGO_EINVAL;
    if ((K && (!s || !q || !a)) || (K && N && !W) || (N && !r)) return GGO_EINVAL;
    for (int64_t n = 0; n < N; ++n)
        if (r[n] != 1 && r[n] != -1) return GGO_EINVAL;
    for (int64_t k = 0; k < K; ++k) {
        const uint16_t* row = W + k * ldw;
        double sk = 0.0, qk = 0.0, ak = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            const double w = widen(row[n]);
            sk += r[n] > 0 ? w : -w;
            qk += w * w;
            ak += std::fabs(w);
        }
        s[k] = sk;
        q[k] = std::sqrt(qk);
        a[k] = ak;
    }
    return GGO_OK;
}

int freivalds_check_signs(const double* s, const double* q, const double* a, const int8_t* r, int64_t K, int64_t N,
                          const uint16_t* x, const float* y, double c_f, double* out) {
    return freivalds_check_multi(1, s, q, a, r, K, N, x, y, c_f, out);
}

int freivalds_prepare(const uint16_t* W, int64_t ldw, int64_t K, int64_t N, uint64_t seed, ggo_freivalds** out) {
    if (!out) return GGO_EINVAL;
    *out = nullptr;
    if (K < 0 || N < 0 || ldw < N || (K && N && !W)) return GGO_EINVAL;
    ggo_freivalds* f = new (std::nothrow) ggo_freivalds;
    if (!f) return GGO_ELAUNCH;
    f->K = K;
    f->N = N;
    f->r.resize(static_cast<size_t>(N));
    for (int64_t n = 0; n < N; ++n) f->r[n] = sign_of(seed, n);
    f->s.resize(static_cast<size_t>(K));
    f->q.resize(static_cast<size_t>(K));
    f->a.resize(static_cast<size_t>(K));
    const int rc = freivalds_prepare_signs(W, ldw, K, N, f->r.data(), f->s.data(), f->q.data(), f->a.data());
    if (rc != GGO_OK) {
        delete f;
        return rc;
    }
    *out = f;
    return GGO_OK;
}

int freivalds_check(const ggo_freivalds* f, const uint16_t* x, const float* y, double c_f, double* out) {
    if (!f) return GGO_EINVAL;
    return freivalds_check_multi(1, f->s.data(), f->q.data(), f->a.data(), f->r.data(), f->K, f->N, x, y, c_f, out);
}

int freivalds_signs(const ggo_freivalds* f, int8_t* r) {
    if (!f || (f->N && !r)) return GGO_EINVAL;
    std::memcpy(r, f->r.data(), static_cast<size_t>(f->N));
    return GGO_OK;
}

void freivalds_free(ggo_freivalds* f) { delete f; }

}  // extern "C"
