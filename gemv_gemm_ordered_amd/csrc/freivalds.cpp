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

namespace {
inline double widen(uint16_t b) {
    const uint32_t u = static_cast<uint32_t>(b) << 16;
    float f;
    std::memcpy(&f, &u, sizeof f);
    return static_cast<double>(f);
}
}  // namespace

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
    if (K < 0 || N < 0 || !out || !(c_f >= 0.0)) return GGO_EINVAL;
    if ((K && (!s || !q || !a || !x)) || (N && (!r || !y))) return GGO_EINVAL;
    double ry = 0.0, ymag = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        const double yn = static_cast<double>(y[n]);
        ry += r[n] > 0 ? yn : -yn;
        ymag += std::fabs(yn);
    }
    double xs = 0.0, sxq = 0.0, sxa = 0.0, xsmag = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        const double xk = widen(x[k]);
        const double t = xk * s[k];
        xs += t;
        xsmag += std::fabs(t);
        sxq += std::fabs(xk) * q[k];
        sxa += std::fabs(xk) * a[k];
    }
    const double u = std::ldexp(1.0, -24);
    const double km1 = K > 0 ? static_cast<double>(K - 1) : 0.0;
    const double rho = std::fabs(ry - xs);
    const double sigma = u * std::sqrt(static_cast<double>(K)) * sxq;
    const double tau = c_f * sigma;
    const double host = 2.0 * static_cast<double>(N + K) * std::ldexp(1.0, -53) * (ymag + xsmag);
    out[0] = rho;
    out[1] = sigma;
    out[2] = tau;
    out[3] = km1 * u / (1.0 - km1 * u) * sxa + host;
    return rho <= tau ? 1 : 0;
}

}  // extern "C"
