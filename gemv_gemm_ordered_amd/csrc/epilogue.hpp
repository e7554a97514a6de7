// Fused epilogue of the matmul kernels, applied to each binary32 result y[m, n] after its fold, in
// one fixed order ("Taming Bitwise Behavior in GPU Kernels with Tensor Core", sections 1 and 7.3:
// a GEMM fused with the operation that follows it, kept bit-exact):
//
//     v = y;  v = v + bias[n];  v = act(v);  v = v + residual[m, n];  out = v, or bf16(v)
//
// (each step skipped when its operand is absent). The pages name no activation, so this library
// defines each as a fixed sequence of IEEE binary32 operations, round to nearest even, with explicit
// fused multiply-adds where an fma is meant and no other contraction:
//
//   exp(x):   n = rint(x * log2(e));  r = fma(-n, ln2_hi, x);  r = fma(-n, ln2_lo, r)
//             (Cody and Waite's two-constant reduction, 1980);  p = Horner form of the degree-7
//             Taylor polynomial of e^r, sum_{i<=7} r^i / i!, with fma;  exp = (p * 2^a) * 2^b,
//             a = floor(n / 2), b = n - a;  x > 88.75 gives +inf, x < -104 gives +0, NaN gives NaN.
//   relu(v):  v > 0 ? v : +0
//   silu(v):  v / (1 + exp(-v))
//   gelu(v):  u = c1 * (v + c2 * ((v * v) * v)),  th = 1 - 2 / (exp(2 * u) + 1),
//             out = 0.5 * (v * (1 + th)),   c1 = RN(sqrt(2 / pi)), c2 = RN(0.044715)
//   bf16(v):  round to nearest even on the upper 16 bits; NaN -> 0x7fc0
//
// Division is IEEE correctly rounded (the HIP default for binary32).
#pragma once
#include "common.hpp"

#pragma clang fp contract(off)

struct Epi {
    const float* bias;       // [N] or null
    const float* res;        // [M, N] with row stride ldr, or null
    int64_t ldr;
    int32_t act;             // GGO_ACT_*
    int32_t out_bf16;        // 0: binary32 output, 1: bfloat16 output
};

__host__ __device__ inline bool epi_identity(const Epi& e) { return !e.bias && !e.res && e.act == 0 && !e.out_bf16; }

GGO_DEV float epi_pow2(int k) { return __uint_as_float(static_cast<uint32_t>(k + 127) << 23); }   // -126 <= k <= 127

GGO_DEV float epi_exp(float x) {
    if (!(x == x)) return x;                                                  // NaN passes through
    if (x > 88.75f) return __uint_as_float(0x7f800000u);
    if (x < -104.0f) return 0.0f;
    const float n = __builtin_rintf(x * 1.44269502162933349609375f);          // RN(log2 e)
    float r = __builtin_fmaf(-n, 0.693145751953125f, x);                      // ln2_hi (15 significant bits)
    r = __builtin_fmaf(-n, 1.428606765330187045037746429443359375e-6f, r);    // RN(ln 2 - ln2_hi)
    float p = 1.98412701138295233249664306640625e-4f;                         // RN(1/5040)
    p = __builtin_fmaf(p, r, 1.388888922519981861114501953125e-3f);           // RN(1/720)
    p = __builtin_fmaf(p, r, 8.3333337679505348205566406250e-3f);             // RN(1/120)
    p = __builtin_fmaf(p, r, 4.1666667908430099487304687500e-2f);             // RN(1/24)
    p = __builtin_fmaf(p, r, 0.16666667163372039794921875f);                  // RN(1/6)
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    const int ni = static_cast<int>(n);
    const int a = ni >> 1, b = ni - a;                                        // floor(n/2), both in [-76, 64]
    return (p * epi_pow2(a)) * epi_pow2(b);
}

GGO_DEV float epi_act(float v, int act) {
    switch (act) {
    case 1:   // relu
        return v > 0.0f ? v : 0.0f;
    case 2:   // silu
        return v / (1.0f + epi_exp(-v));
    case 3: { // gelu, tanh form
        float c = v * v;
        c = c * v;
        c = 0.044714998453855514526367187500f * c;                            // RN(0.044715)
        c = v + c;
        const float u = 0.79788458347320556640625f * c;                       // RN(sqrt(2/pi))
        const float th = 1.0f - 2.0f / (epi_exp(2.0f * u) + 1.0f);
        return 0.5f * (v * (1.0f + th));
    }
    default:
        return v;
    }
}

// y + bias, the activation, + residual, with the bias b and the residual r of the output already loaded
// (each ignored when the epilogue has none)
GGO_DEV float epi_apply_loaded(const Epi& e, float y, float b, float r) {
    float v = y;
    if (e.bias) v = v + b;
    v = epi_act(v, e.act);
    if (e.res) v = v + r;
    return v;
}

GGO_DEV float epi_bias1(const Epi& e, int64_t n) { return e.bias ? e.bias[n] : 0.0f; }
GGO_DEV float epi_res1(const Epi& e, int64_t m, int64_t n) { return e.res ? e.res[m * e.ldr + n] : 0.0f; }

GGO_DEV float epi_apply(const Epi& e, float y, int64_t m, int64_t n) {
    return epi_apply_loaded(e, y, epi_bias1(e, n), epi_res1(e, m, n));
}

GGO_DEV uint16_t epi_bf16(float v) {
    const uint32_t u = __float_as_uint(v);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// Store one result of row m, column n into C (binary32 or bfloat16, row stride ldc elements), with its
// bias b and residual r already loaded.
GGO_DEV void epi_store_loaded(const Epi& e, void* C, int64_t ldc, int64_t m, int64_t n, float y, float b, float r) {
    const float v = epi_apply_loaded(e, y, b, r);
    if (e.out_bf16) static_cast<uint16_t*>(C)[m * ldc + n] = epi_bf16(v);
    else static_cast<float*>(C)[m * ldc + n] = v;
}

// Store one result of row m, column n into C (binary32 or bfloat16, row stride ldc elements).
GGO_DEV void epi_store(const Epi& e, void* C, int64_t ldc, int64_t m, int64_t n, float y) {
    epi_store_loaded(e, C, ldc, m, n, y, epi_bias1(e, n), epi_res1(e, m, n));
}

// Four consecutive results of row m, columns n .. n+3, given the bias b[n .. n+3] and the residual
// r[m, n .. n+3] already loaded (ignored when the epilogue has none), with one 16-byte (binary32) or
// 8-byte (bfloat16) store. The caller guarantees the alignment.
GGO_DEV void epi_finish4(const Epi& e, void* C, int64_t ldc, int64_t m, int64_t n, float4 y, float4 b, float4 r) {
    float v[4] = {y.x, y.y, y.z, y.w};
    if (e.bias) {
        v[0] = v[0] + b.x;
        v[1] = v[1] + b.y;
        v[2] = v[2] + b.z;
        v[3] = v[3] + b.w;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = epi_act(v[i], e.act);
    if (e.res) {
        v[0] = v[0] + r.x;
        v[1] = v[1] + r.y;
        v[2] = v[2] + r.z;
        v[3] = v[3] + r.w;
    }
    if (e.out_bf16) {
        const uint32_t lo = epi_bf16(v[0]) | (static_cast<uint32_t>(epi_bf16(v[1])) << 16);
        const uint32_t hi = epi_bf16(v[2]) | (static_cast<uint32_t>(epi_bf16(v[3])) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(C) + m * ldc + n) = make_uint2(lo, hi);
    } else {
        *reinterpret_cast<float4*>(static_cast<float*>(C) + m * ldc + n) = make_float4(v[0], v[1], v[2], v[3]);
    }
}

GGO_DEV float4 epi_bias4(const Epi& e, int64_t n) {
    return e.bias ? *reinterpret_cast<const float4*>(e.bias + n) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
}

GGO_DEV float4 epi_res4(const Epi& e, int64_t m, int64_t n) {
    return e.res ? *reinterpret_cast<const float4*>(e.res + m * e.ldr + n) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
}

// Four consecutive results with 16-byte bias / residual loads: epi_finish4 after its loads.
GGO_DEV void epi_store4(const Epi& e, void* C, int64_t ldc, int64_t m, int64_t n, float y0, float y1, float y2,
                        float y3) {
    epi_finish4(e, C, ldc, m, n, make_float4(y0, y1, y2, y3), epi_bias4(e, n), epi_res4(e, m, n));
}
