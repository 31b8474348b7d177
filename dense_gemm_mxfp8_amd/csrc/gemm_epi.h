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

// Four consecutive elements of one row of C, columns col .. col + 3.  With
// `vec` (C's base and row pitch such that element (row, col) with col % 4 ==
// 0 is aligned to 4 elements) they go out as one 16-, 8- or 4-byte store.
__device__ __forceinline__ void store4(void* C, int64_t ldc, const Params& e, int row, int col, float a0, float a1,
                                       float a2, float a3, bool vec) {
    float t[4] = {a0, a1, a2, a3};
    if (e.on) {
#pragma unroll
        for (int c = 0; c < 4; ++c) t[c] = apply(e, t[c], row, col + c);
    }
    const int64_t off = (int64_t)row * ldc + col;
    if (!vec) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (e.out == kBF16) ((uint16_t*)C)[off + c] = to_bf16(t[c]);
            else if (e.out == kE4M3) ((uint8_t*)C)[off + c] = to_e4m3(t[c]);
            else ((float*)C)[off + c] = t[c];
        }
        return;
    }
    if (e.out == kBF16) {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 v = {(uint32_t)to_bf16(t[0]) | ((uint32_t)to_bf16(t[1]) << 16),
                         (uint32_t)to_bf16(t[2]) | ((uint32_t)to_bf16(t[3]) << 16)};
        *(u32x2*)((uint16_t*)C + off) = v;
    } else if (e.out == kE4M3) {
        *(uint32_t*)((uint8_t*)C + off) = (uint32_t)to_e4m3(t[0]) | ((uint32_t)to_e4m3(t[1]) << 8) |
                                          ((uint32_t)to_e4m3(t[2]) << 16) | ((uint32_t)to_e4m3(t[3]) << 24);
    } else {
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        *(f32x4*)((float*)C + off) = f32x4{t[0], t[1], t[2], t[3]};
    }
}

// Whether store4 may use one vector store: C's base aligned to 4 elements and
// a row pitch that is a multiple of 4 elements.
__device__ __forceinline__ bool vec4_ok(const void* C, int64_t ldc, const Params& e) {
    const int esz = e.out == kBF16 ? 2 : e.out == kE4M3 ? 1 : 4;
    return ((uintptr_t)C % (4 * esz)) == 0 && (ldc % 4) == 0;
}

}  // namespace epi
