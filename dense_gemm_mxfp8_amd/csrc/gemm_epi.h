// gemm_epi.h -- the fused epilogue shared by every kernel.
//
// t(i, j) = acc(i, j) * row_scale[i] * col_scale[j] + bias[j], in fp32, then
// stored as fp32, rounded to bf16 (nearest even, NaN stays NaN) or rounded to
// OCP E4M3 (nearest even, saturating to +-448, NaN stays NaN).  Absent
// vectors (null pointers) stand for 1, 1 and 0.  With `on` == 0 the
// accumulator is stored unchanged as fp32.

#pragma once

#include <stdint.h>

namespace epi {

// Output element types (the values of GEMM_OUT_F32 / _BF16 / _E4M3).
enum Out { kF32 = 0, kBF16 = 1, kE4M3 = 2 };

struct Params {
    const float* rs;    // M row scales, or null
    const float* cs;    // N column scales, or null
    const float* bias;  // N column biases, or null
    int on;             // 0: plain fp32 store
    int out;            // Out: what C holds
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

// Round to OCP E4M3 ("fn": no infinities, 0x7F / 0xFF are NaN, largest
// finite +-448), nearest even.  Values beyond +-448, infinities included,
// saturate to +-448; NaN stays NaN.  The clamp runs first, so the hardware
// conversion (v_cvt_pk_fp8_f32, OCP E4M3 on gfx950) only sees values inside
// the format's range and its own overflow rule never applies.
__device__ __forceinline__ uint8_t to_e4m3(float x) {
    const float c = (x != x) ? x : __builtin_fminf(__builtin_fmaxf(x, -448.0f), 448.0f);
    return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xff);
}

// One element of C (the slow paths).
__device__ __forceinline__ void store(void* C, int64_t ldc, const Params& e, int row, int col, float acc) {
    const float t = e.on ? apply(e, acc, row, col) : acc;
    const int64_t off = (int64_t)row * ldc + col;
    if (e.out == kBF16) ((uint16_t*)C)[off] = to_bf16(t);
    else if (e.out == kE4M3) ((uint8_t*)C)[off] = to_e4m3(t);
    else ((float*)C)[off] = t;
}

}  // namespace epi
