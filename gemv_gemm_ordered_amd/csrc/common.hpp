// Shared device helpers of the batch-invariant matmul kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define GGO_DEV __device__ __forceinline__

// bfloat16 is the upper half of a binary32, so widening is exact: a 16-bit shift.
GGO_DEV float bf16_lo(uint32_t two) { return __uint_as_float(two << 16); }
GGO_DEV float bf16_hi(uint32_t two) { return __uint_as_float(two & 0xffff0000u); }
GGO_DEV float bf16_one(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// Workgroups are handed to the 8 XCDs round robin (workgroup i runs on XCD i mod 8).
// Give each XCD a contiguous range of tile indices so that neighbouring tiles, which
// share rows of A or columns of W, meet in the same XCD's L2. A bijection on [0, n).
GGO_DEV int xcd_contiguous(int bid, int n) {
    const int q = n >> 3, r = n & 7, x = bid & 7, i = bid >> 3;
    return x * q + (x < r ? x : r) + i;
}
