// Launch-side declarations shared by the kernel sources and the C-ABI shim.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ggo.h"
#include "epilogue.hpp"

// VEC_EP: 4-wide epilogue loads/stores. VEC_WIDE64: the 64x64 matrix-core tile may use its branch-free
// buffer loads (16-byte aligned A, 8-byte aligned W, lda, ldw and K multiples of 8, N a multiple of 4,
// A and W ranges below 2^31 bytes).
enum : uint32_t { VEC_A = 1u, VEC_W = 2u, VEC_C = 4u, VEC_EP = 8u, VEC_WIDE64 = 16u, VEC_W16 = 32u };   // VEC_W16:
// 16-byte loads of x and W^T rows (16-byte aligned, ldx, ldwt and K multiples of 8)

// One ordered problem as the kernel sees it (passed by value in the kernel arguments).
struct OrdProblem {
    const void* A;
    const uint16_t* W;
    float* C;
    int64_t lda, ldw, ldc;
    int64_t sa, sw, sc;
    int32_t M, N, K, batch;
    int32_t tiles_m, tiles_n;
    uint32_t vec;     // VEC_* bits: 16-byte loads / stores allowed
};

struct OrdGroup {
    int32_t count;
    int32_t tile_start[GGO_MAX_PROBLEMS + 1];   // prefix sums of batch * tiles_m * tiles_n
    OrdProblem p[GGO_MAX_PROBLEMS];
};

// Tile of the ordered kernel: 64 x 64 (4 x 4 per lane), 64 x 32 (4 x 2 per lane) or 16 x 16 (one output
// per lane); the caller chooses from the weight's shape and the entry point, never from M.
enum { ORD_TILE_BIG = 0, ORD_TILE_SMALL = 1, ORD_TILE_MID = 2 };
void ordered_tile_shape(int kind, int* bm, int* bn);
// wide != 0: every problem has 16-byte aligned A, W, row strides (and batch strides) of whole 16-byte
// chunks, K and N multiples of 8, and lda, ldw <= ordered_wide_max_ld(kind, a_f32)
hipError_t launch_gemm_ordered(const OrdGroup& g, int total_tiles, int a_f32, int kind, int wide, hipStream_t stream);
int64_t ordered_wide_max_ld(int kind, int a_f32);

struct GemvArgs {
    const uint16_t* x;
    const uint16_t* W;   // W [K, N]; or, with wt set, W^T [N, K] (row stride ldw)
    float* y;
    int64_t ldx, ldw, ldy;
    int32_t M, N, K;
    uint32_t vec;
    int32_t wt;
    int32_t form;     // 0: chosen from M (on W^T where allowed: 512-k stages at M = 1, the MR-row instance at
                      // M >= 2; else 64-k stages for M <= 4, else 128-k where allowed); 1: 64-k; 2: 128-k;
                      // 3: 512-k (M = 1, W^T); 4: MR rows of x per workgroup (W^T)
    int32_t rows;     // form 4: rows of x per workgroup (2, 4 or 8), or 0 for M rounded up
};
hipError_t launch_gemv_ordered(const GemvArgs& a, hipStream_t stream);
bool gemv_ordered_k128_ok(const GemvArgs& a);   // the 128-k stages can serve these operands
bool gemv_ordered_m1_ok(const GemvArgs& a);     // the 512-k stages (M = 1, W^T) can serve these operands
bool gemv_ordered_mr_ok(const GemvArgs& a);     // the MR-row instance (W^T) can serve these operands
int gemv_ordered_max_ldw();   // buffer offsets of the GEMV kernel are 32-bit
int gemv_ordered_wt_max_ldw();   // the same for W^T: a 16-row slab of W^T in one 32-bit range

struct TreeArgs {
    const uint16_t* x;
    const uint16_t* WT;
    void* y;          // binary32, or bfloat16 when ep.out_bf16
    int64_t ldx, ldwt, ldy;
    int32_t M, N, K;
    int32_t wide;     // 16-byte loads allowed (alignment, strides and K multiples of 8)
    Epi ep;
    int32_t rows;     // rows of x staged per workgroup (1, 2, 4, 8 or 16, >= M); 0: chosen from M
    int32_t form;     // 0: persistent where it can serve, else one group per workgroup; 1: persistent; 2: one group
};
hipError_t launch_gemv_tree(const TreeArgs& a, hipStream_t stream);
int gemv_tree_max_k();   // byte offsets along a row are 32-bit
int gemv_tree_persistent_max_k();   // the persistent form keeps at most this many k of x per lane in registers

// Float Freivalds check of one row against t <= FREIVALDS_MAX_T sign vectors in one pass (freivalds.cpp);
// the same values and verdicts as t calls of freivalds_check.
constexpr int FREIVALDS_MAX_T = 16;
int freivalds_check_multi(int t, const double* s, const double* q, const double* a, const int8_t* r, int64_t K,
                          int64_t N, const uint16_t* x, const float* y, double c_f, double* out);

struct MfmaArgs {
    const uint16_t* A;
    const uint16_t* W;
    void* C;          // binary32, or bfloat16 when ep.out_bf16
    int64_t lda, ldw, ldc;
    int32_t M, N, K;
    int32_t tiles_m, tiles_n;
    uint32_t vec;
    Epi ep;
};
void mfma_tile_shape(int* bm, int* bn);        // 256x128 instance (16-byte aligned operands)
void mfma_tile_shape_t256x256(int* bm, int* bn);   // 256x256 instance (the same operands)
void mfma_tile_shape_lds128(int* bm, int* bn);     // 128x128 direct-to-LDS instance (the same operands)
void mfma_tile_shape_lds64x128(int* bm, int* bn);  // 64x128 direct-to-LDS instance (the same operands)
void mfma_tile_shape_t128(int* bm, int* bn);   // 128x128 instance (any operands)
void mfma_tile_shape_t64(int* bm, int* bn);    // 64x64 instance (any operands)
hipError_t launch_gemm_mfma_invariant(const MfmaArgs& a, hipStream_t stream);
hipError_t launch_gemm_mfma_invariant_256(const MfmaArgs& a, hipStream_t stream);   // the 256x256 instance
hipError_t launch_gemm_mfma_lds128(const MfmaArgs& a, hipStream_t stream);           // 128x128, direct to LDS
hipError_t launch_gemm_mfma_lds64x128(const MfmaArgs& a, hipStream_t stream);        // 64x128, direct to LDS
hipError_t launch_gemm_mfma_t128(const MfmaArgs& a, hipStream_t stream);
hipError_t launch_gemm_mfma_t64(const MfmaArgs& a, hipStream_t stream);
// W given as W^T [N, K]: the direct-to-LDS instance of tile bm x bn (one of the four shapes above)
hipError_t launch_gemm_mfma_invariant_wt(const MfmaArgs& a, int bm, int bn, hipStream_t stream);

struct GemvMfmaArgs {
    const uint16_t* x;
    const uint16_t* WT;
    void* y;          // binary32, or bfloat16 when ep.out_bf16
    int64_t ldx, ldwt, ldy;
    int32_t M, N, K;
    Epi ep;
    int32_t rows;     // rows of x staged per stage (1, 2, 4, 8 or 16, >= M); 0: chosen from M
};
hipError_t launch_gemv_mfma(const GemvMfmaArgs& a, hipStream_t stream);   // 16-byte operands, K % 8 == 0
int gemv_mfma_max_k();   // byte offsets along a row are 32-bit
