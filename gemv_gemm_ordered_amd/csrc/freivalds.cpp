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
// signs back to back). For each vector the sums are those of the single-vector check, in the same
// order, so the values and the verdict are the same as t separate checks; the shared sums (|y|,
// |x| q, |x| a) are taken once. out gets (rho, sigma, tau, bound) per vector. Returns 1 when every
// vector accepts, 0 when one rejects, < 0 on bad arguments.
namespace {
template <int T>
int check_t(const double* s, const double* q, const double* a, const int8_t* r, int64_t K, int64_t N, const uint16_t* x,
            const float* y, double c_f, double* out) {
    double ry[T] = {}, xs[T] = {}, xsmag[T] = {};
    double ymag = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        const double yn = static_cast<double>(y[n]);
        for (int v = 0; v < T; ++v) ry[v] += r[v * N + n] > 0 ? yn : -yn;
        ymag += std::fabs(yn);
    }
    double sxq = 0.0, sxa = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        const double xk = widen(x[k]);
        for (int v = 0; v < T; ++v) {
            const double tv = xk * s[v * K + k];
            xs[v] += tv;
            xsmag[v] += std::fabs(tv);
        }
        sxq += std::fabs(xk) * q[k];
        sxa += std::fabs(xk) * a[k];
    }
    const double u = std::ldexp(1.0, -24);
    const double km1 = K > 0 ? static_cast<double>(K - 1) : 0.0;
    const double sigma = u * std::sqrt(static_cast<double>(K)) * sxq;
    const double tau = c_f * sigma;
    int all = 1;
    for (int v = 0; v < T; ++v) {
        const double rho = std::fabs(ry[v] - xs[v]);
        const double host = 2.0 * static_cast<double>(N + K) * std::ldexp(1.0, -53) * (ymag + xsmag[v]);
        out[4 * v + 0] = rho;
        out[4 * v + 1] = sigma;
        out[4 * v + 2] = tau;
        out[4 * v + 3] = km1 * u / (1.0 - km1 * u) * sxa + host;
        if (!(rho <= tau)) all = 0;
    }
    return all;
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

extern "C" {

int freivalds_prepare(const uint16_t* W, int64_t ldw, int64_t K, int64_t N, const int8_t* r, double* s, double* q,
                      double* a) {
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

int freivalds_check(const double* s, const double* q, const double* a, const int8_t* r, int64_t K, int64_t N,
                    const uint16_t* x, const float* y, double c_f, double* out) {
    return freivalds_check_multi(1, s, q, a, r, K, N, x, y, c_f, out);
}

}  // extern "C"
