// gemm_epi.h -- the fused epilogue shared by every kernel.
//
// t(i, j) = acc(i, j) * row_scale[i] * col_scale[j] + bias[j], in fp32, then
// stored as fp32 or rounded to bf16 (nearest even, NaN stays NaN).  Absent
// vectors (null pointers) stand for 1, 1 and 0.  With `on` == 0 the
// accumulator is stored unchanged as fp32.

#pragma once

#include <stdint.h>

namespace epi {

struct Params {
    const float* rs;    // M row scales, or null
    const float* cs;    // N column scales, or null
    const float* bias;  // N column biases, or null
    int on;             // 0: plain fp32 store
    int out_bf16;       // 1: C holds bf16
};

__device__ __forceinline__ float apply(const Params& e, float acc, int row, int col) {
    float t = acc;
    if (e.rs) t *= e.rs[row];
    if (e.cs) t *= e.cs[col];
    if (e.bias) t += e.bias[col];
    return t;
}

// Round to bf16, nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t to_bf16(float x) {
    const __bf16 b = (__bf16)x;
    return __builtin_bit_cast(uint16_t, b);
}

// One element of C (the slow paths).
__device__ __forceinline__ void store(void* C, int64_t ldc, const Params& e, int row, int col, float acc) {
    const float t = e.on ? apply(e, acc, row, col) : acc;
    if (e.out_bf16) ((uint16_t*)C)[(int64_t)row * ldc + col] = to_bf16(t);
    else ((float*)C)[(int64_t)row * ldc + col] = t;
}

}  // namespace epi
