// libgemm.hip -- hand-written gfx950 (MI355X, CDNA4) GEMM kernels and the C ABI
// declared in include/libgemm.h.
//
// C[M x N] = A[M x K] * B[K x N], fp32 accumulate and output, for bf16
// operands (B row-major "NN" or column-major "NT") and for MX block-scaled fp8
// operands (E4M3 codes, one E8M0 scale per 32 K-elements).  The problem
// statement and the tile bookkeeping follow "GPU 执行模型" (sections
// "Tile 的容量约束", "Tile 小账本", "流水与异步搬运", "正确性契约"); the
// block-scaled MMA follows "Modern GPU Programming For MLSys - 书籍总结"
// (sections 2.4 and 2.6).  The pages' kernel design targets NVIDIA Blackwell
// (TMA, TMEM, mbarriers, clusters); none of that exists on CDNA4, so the
// kernels here are built from gfx950 primitives instead:
//
//   * global->LDS tile loads: 16 bytes per lane written straight into LDS
//     (no VGPR round trip) when rows are 16-byte aligned -- `buffer_load_
//     dwordx4 ... lds` against a per-tile buffer descriptor in the 256 x 256
//     kernels (gemm_fast.h), `global_load_lds_dwordx4` in the generic kernel
//     of this file -- else 16-byte loads into VGPRs and `ds_write_b128`
//     (gemm_reg.h) or predicated element loads (the generic kernel);
//   * LDS layout: every operand row holds 128 bytes of K (64 bf16 or 128
//     fp8); its eight 16-byte chunks are XOR-swizzled with the row index so
//     that the fragment reads of 8 consecutive rows hit 8 different bank
//     groups;
//   * two LDS stages: the loads of k-tile t+1 are in flight while the matrix
//     cores work on k-tile t; one `s_waitcnt vmcnt(0)` + barrier per k-tile
//     hands a stage from the loaders to the readers (the role the pages give
//     to mbarrier phases);
//   * matrix cores: v_mfma_f32_16x16x32_bf16 (plain bf16 products, in
//     gemm_mf16.hip) or v_mfma_f32_32x32x16_bf16, and
//     v_mfma_scale_f32_32x32x64_f8f6f4, accumulating in registers;
//   * row-major B (NN): `ds_read_b64_tr_b16` transposes 4x16 blocks on the way
//     out of LDS so the B fragment arrives K-contiguous per lane;
//   * a persistent grid with a static strided tile walk, grouped raster order
//     and an XCD-aware remap of workgroup ids;
//   * tails: rows past M / columns past N lie outside the per-tile
//     descriptors and load as zero (the generic kernel re-reads the last
//     valid row or column: finite data, never stored); the partial last
//     k-tile is loaded with element predicates and zero fill;
//   * epilogue: predicated fp32 stores straight from the accumulators.
//
// Lane layouts used below.  They are not checked one instruction at a time:
// the GEMM parity tests pin them as a whole, since a map that pairs a(i, k)
// with b(k', j) for k' != k, applies a block scale to the wrong 32 elements,
// or stores a sum at the wrong (i, j) breaks the bit-exact integer-operand
// results:
//   v_mfma_f32_32x32x16_bf16: lane l supplies A[l%32][8*(l/32) + j] and
//     B[8*(l/32) + j][l%32], j = 0..7; accumulator register i of lane l is
//     D[8*(i/4) + 4*(l/32) + i%4][l%32].
//   v_mfma_f32_16x16x32_bf16: lane l supplies A[l%16][8*(l/16) + j] and
//     B[8*(l/16) + j][l%16]; accumulator register i of lane l is
//     D[4*(l/16) + i][l%16].
//   v_permlane16_swap (as __builtin_amdgcn_permlane16_swap(x, y)): result 0
//     holds x's 16-lane groups 0 and 2 in groups 0 and 2 and y's groups 0 and
//     2 in groups 1 and 3; result 1 holds x's groups 1 and 3 in groups 0 and 2
//     and y's groups 1 and 3 in groups 1 and 3 (checked on gfx950 with lane
//     indices as data).
//   v_mfma_scale_f32_32x32x64_f8f6f4 (fp8): lane l supplies row l%32; bytes
//     0..15 hold k = 16*(l/32) + j, bytes 16..31 hold k = 32 + 16*(l/32) + j;
//     the scale operand of lane q applies to row q%32, 32-block q/32.
//   ds_read_b64_tr_b16: within each 16-lane group, output element e of lane i
//     is element i%4 of the 8-byte word addressed by lane 4*e + i/4.

#include <hip/hip_runtime.h>

#include <mutex>
#include <stdio.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "libgemm.h"
#include "gemm_epi.h"
#include "gemm_fast.h"
#include "gemm_small.h"
#include "gemm_reg.h"

// Fixed device scratch of gemm_bf16_splitk_noalloc, for callers that cannot
// allocate: the split-K partial products go here instead of into a caller's
// workspace.  Every GPU the library runs on holds its own copy, at its own
// address, from the first call on it until the process ends.  In host code
// the name stands for a host-side shadow, never the device memory: the host
// uses only the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[GEMM_SCRATCH_BYTES];

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int kRowBytes = 128;   // bytes of K held per LDS operand row
constexpr int kThreads = 256;    // 4 waves: a 2 x 2 arrangement of wave tiles
constexpr int kWaves = 4;

enum Kind { kBf16NT = 0, kBf16NN = 1, kMx = 2 };

struct Args {
    const uint8_t* A;
    const uint8_t* B;
    float* C;
    const uint8_t* SA;
    const uint8_t* SB;
    int64_t lda, ldb, ldc;  // elements
    int M, N, K;
    int tiles_m, tiles_n, num_tiles, group_m;
    int kt_full;   // k-tiles lying entirely inside K
    int kt_total;  // kt_full, plus one if K leaves a partial tile
    int sld;       // scale codes per row: K / 32
    int xcd_remap; // 1: grid is a multiple of 8, spread tiles per XCD
    epi::Params epi;  // fused epilogue (C holds epi.out elements)
};

// ---------------------------------------------------------------------------
// Tile scheduler: static strided walk over tiles in grouped order.
// ---------------------------------------------------------------------------

__device__ inline int logical_block(const Args& a) {
    int bid = blockIdx.x;
    if (!a.xcd_remap) return bid;
    // Workgroups are dispatched round-robin over the 8 XCDs; renumber them so
    // that consecutive logical ids (and hence neighbouring tiles) share an XCD
    // and its L2.
    int per_xcd = gridDim.x >> 3;
    return (bid & 7) * per_xcd + (bid >> 3);
}

__device__ inline void tile_coords(const Args& a, int t, int& tm, int& tn) {
    int per_group = a.group_m * a.tiles_n;
    int g = t / per_group;
    int first = g * a.group_m;
    int gsz = min(a.tiles_m - first, a.group_m);
    int r = t - g * per_group;
    tm = first + r % gsz;
    tn = r / gsz;
}

__device__ inline void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Swizzled byte offset of 16-byte chunk `chunk` of K-contiguous LDS row `row`.
__device__ inline int kc_offset(int row, int chunk) {
    return row * kRowBytes + ((chunk ^ (row & 7)) << 4);
}

// Swizzled byte offset of element column n of k-row `k` in the N-contiguous
// LDS tile of row-major B (NN); rows hold BN bf16.
template <int BN>
__device__ inline int nn_offset(int k, int n) {
    int chunk = (n >> 3) ^ ((k & 3) << 1);
    return k * (BN * 2) + (chunk << 4) + ((n & 7) << 1);
}

// ---------------------------------------------------------------------------
// Global -> LDS loads.
// ---------------------------------------------------------------------------

// Direct (DMA-style) load of R K-contiguous rows x 128 bytes into LDS.  Each
// wave instruction fills 1 KiB = 8 rows; lane i lands at byte 16*i of it, so
// the lane fetches the logical chunk that the swizzle places there.
template <int R>
__device__ inline void load_kc_direct(uint8_t LDS_AS* dst, const uint8_t* g, int64_t ld_bytes,
                                      int row0, int nrows, int64_t kbyte, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < R / 32; ++i) {
        int q = i * kWaves + wave;
        int r = q * 8 + (lane >> 3);
        int c = (lane & 7) ^ (lane >> 3);
        int gr = min(row0 + r, nrows - 1);
        const uint8_t* src = g + (int64_t)gr * ld_bytes + kbyte + c * 16;
        __builtin_amdgcn_global_load_lds((const void*)src, (void LDS_AS*)(dst + q * 1024), 16, 0, 0);
    }
}

// Predicated load of R K-contiguous rows through VGPRs: element k of row r is
// read only if k < K (zero otherwise); rows past nrows re-read row nrows-1.
template <int R, int ESZ>
__device__ inline void load_kc_reg(uint8_t LDS_AS* dst, const uint8_t* g, int64_t ld, int row0,
                                   int nrows, int k0, int K, int tid) {
    constexpr int EPC = 16 / ESZ;  // elements per 16-byte chunk
#pragma unroll
    for (int i = 0; i < R * 8 / kThreads; ++i) {
        int idx = i * kThreads + tid;
        int r = idx >> 3, c = idx & 7;
        int gr = min(row0 + r, nrows - 1);
        int kb = k0 + c * EPC;
        const uint8_t* src = g + ((int64_t)gr * ld + kb) * ESZ;
        i32x4 v = {0, 0, 0, 0};
        if (kb + EPC <= K && (((uintptr_t)src) & 3) == 0) {
            const int* s = (const int*)src;
            v[0] = s[0]; v[1] = s[1]; v[2] = s[2]; v[3] = s[3];
        } else {
            uint8_t b[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) b[e] = 0;
            if (ESZ == 2) {
                const uint16_t* s = (const uint16_t*)src;
#pragma unroll
                for (int e = 0; e < EPC; ++e) {
                    uint16_t x = (kb + e < K) ? s[e] : (uint16_t)0;
                    b[2 * e] = (uint8_t)x;
                    b[2 * e + 1] = (uint8_t)(x >> 8);
                }
            } else {
#pragma unroll
                for (int e = 0; e < EPC; ++e) b[e] = (kb + e < K) ? src[e] : (uint8_t)0;
            }
            memcpy(&v, b, 16);
        }
        *(i32x4 LDS_AS*)(dst + kc_offset(r, c)) = v;
    }
}

// Direct load of the 64 x BN bf16 tile of row-major B (rows are k).  Requires
// N % 8 == 0; chunks past N re-read the last full chunk (never stored).
template <int BN>
__device__ inline void load_nn_direct(uint8_t LDS_AS* dst, const uint8_t* g, int64_t ldb, int k0,
                                      int n0, int N, int wave, int lane) {
    constexpr int kRowB = BN * 2;
    constexpr int kLoads = 64 * kRowB / 1024;
#pragma unroll
    for (int i = 0; i < kLoads / kWaves; ++i) {
        int q = i * kWaves + wave;
        int off = q * 1024 + lane * 16;
        int kk = off / kRowB;
        int p = (off % kRowB) >> 4;
        int c = p ^ ((kk & 3) << 1);
        int n = min(n0 + c * 8, N - 8);
        const uint8_t* src = g + ((int64_t)(k0 + kk) * ldb + n) * 2;
        __builtin_amdgcn_global_load_lds((const void*)src, (void LDS_AS*)(dst + q * 1024), 16, 0, 0);
    }
}

// Predicated load of the 64 x BN bf16 tile of row-major B through VGPRs.
template <int BN>
__device__ inline void load_nn_reg(uint8_t LDS_AS* dst, const uint8_t* g, int64_t ldb, int k0,
                                   int K, int n0, int N, int tid) {
    constexpr int kChunks = 64 * BN / 8;
#pragma unroll
    for (int i = 0; i < kChunks / kThreads; ++i) {
        int idx = i * kThreads + tid;
        int kk = idx / (BN / 8);
        int c = idx % (BN / 8);
        int k = k0 + kk;
        int nb = n0 + c * 8;
        i32x4 v = {0, 0, 0, 0};
        if (k < K) {
            const uint16_t* s = (const uint16_t*)(g + ((int64_t)k * ldb + nb) * 2);
            if (nb + 8 <= N && (((uintptr_t)s) & 3) == 0) {
                const int* s4 = (const int*)s;
                v[0] = s4[0]; v[1] = s4[1]; v[2] = s4[2]; v[3] = s4[3];
            } else {
                uint16_t h[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) h[e] = (nb + e < N) ? s[e] : (uint16_t)0;
                memcpy(&v, h, 16);
            }
        }
        *(i32x4 LDS_AS*)(dst + nn_offset<BN>(kk, c * 8)) = v;
    }
}

// ---------------------------------------------------------------------------
// The GEMM kernel.
// ---------------------------------------------------------------------------

template <int BM, int BN, int KIND, bool DIRECT>
__global__ __launch_bounds__(kThreads, (BM * BN >= 256 * 256) ? 1 : 2) void gemm_kernel(Args a) {
    constexpr int ESZ = (KIND == kMx) ? 1 : 2;        // operand element bytes
    constexpr int BK = kRowBytes / ESZ;                // K elements per k-tile
    constexpr int WTM = BM / 2, WTN = BN / 2;          // wave tile
    constexpr int MB = WTM / 32, NB = WTN / 32;        // 32x32 MFMA blocks per wave
    constexpr int A_BYTES = BM * kRowBytes;
    constexpr int B_BYTES = BN * kRowBytes;
    constexpr int STAGE = A_BYTES + B_BYTES;

    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t lda_b = a.lda * ESZ;
    const int64_t ldb_b = a.ldb * ESZ;

    const int G = gridDim.x;
    for (int t = logical_block(a); t < a.num_tiles; t += G) {
        int tm, tn;
        tile_coords(a, t, tm, tn);
        const int m0 = tm * BM, n0 = tn * BN;

        f32x16 acc[MB][NB];
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

        // MX scales of the current and the next k-tile, one dword (four
        // 32-blocks) per MFMA row block, pre-shifted per lane half.
        int sa_cur[MB], sb_cur[NB], sa_nxt[MB], sb_nxt[NB];

        auto load_scales = [&](int kt, int* sa, int* sb) {
            if constexpr (KIND == kMx) {
                const int h = lane >> 5;
#pragma unroll
                for (int i = 0; i < MB; ++i) {
                    int row = min(m0 + wm * WTM + i * 32 + (lane & 31), a.M - 1);
                    const uint8_t* p = a.SA + (int64_t)row * a.sld + kt * 4;
                    uint32_t w = 0;
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        w |= (uint32_t)((kt * 4 + b < a.sld) ? p[b] : 127) << (8 * b);
                    sa[i] = (int)(h ? (w >> 8) : w);
                }
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    int col = min(n0 + wn * WTN + j * 32 + (lane & 31), a.N - 1);
                    const uint8_t* p = a.SB + (int64_t)col * a.sld + kt * 4;
                    uint32_t w = 0;
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        w |= (uint32_t)((kt * 4 + b < a.sld) ? p[b] : 127) << (8 * b);
                    sb[j] = (int)(h ? (w >> 8) : w);
                }
            }
        };

        auto load_stage = [&](int kt, int buf) {
            uint8_t LDS_AS* As = (uint8_t LDS_AS*)smem + buf * STAGE;
            uint8_t LDS_AS* Bs = As + A_BYTES;
            const int k0 = kt * BK;
            if (DIRECT && kt < a.kt_full) {
                load_kc_direct<BM>(As, a.A, lda_b, m0, a.M, (int64_t)k0 * ESZ, wave, lane);
                if constexpr (KIND == kBf16NN)
                    load_nn_direct<BN>(Bs, a.B, a.ldb, k0, n0, a.N, wave, lane);
                else
                    load_kc_direct<BN>(Bs, a.B, ldb_b, n0, a.N, (int64_t)k0 * ESZ, wave, lane);
            } else {
                load_kc_reg<BM, ESZ>(As, a.A, a.lda, m0, a.M, k0, a.K, tid);
                if constexpr (KIND == kBf16NN)
                    load_nn_reg<BN>(Bs, a.B, a.ldb, k0, a.K, n0, a.N, tid);
                else
                    load_kc_reg<BN, ESZ>(Bs, a.B, a.ldb, n0, a.N, k0, a.K, tid);
            }
        };

        auto compute = [&](int buf) {
            const uint8_t LDS_AS* As = (const uint8_t LDS_AS*)smem + buf * STAGE;
            const uint8_t LDS_AS* Bs = As + A_BYTES;
            if constexpr (KIND == kMx) {
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    i32x8 af[MB], bfr[NB];
                    const int h = lane >> 5;
#pragma unroll
                    for (int i = 0; i < MB; ++i) {
                        int row = wm * WTM + i * 32 + (lane & 31);
                        i32x4 lo = *(const i32x4 LDS_AS*)(As + kc_offset(row, 4 * s + h));
                        i32x4 hi = *(const i32x4 LDS_AS*)(As + kc_offset(row, 4 * s + 2 + h));
                        af[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    }
#pragma unroll
                    for (int j = 0; j < NB; ++j) {
                        int row = wn * WTN + j * 32 + (lane & 31);
                        i32x4 lo = *(const i32x4 LDS_AS*)(Bs + kc_offset(row, 4 * s + h));
                        i32x4 hi = *(const i32x4 LDS_AS*)(Bs + kc_offset(row, 4 * s + 2 + h));
                        bfr[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    }
#pragma unroll
                    for (int i = 0; i < MB; ++i)
#pragma unroll
                        for (int j = 0; j < NB; ++j) {
                            if (s == 0)
                                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                    af[i], bfr[j], acc[i][j], 0, 0, 0, sa_cur[i], 0, sb_cur[j]);
                            else
                                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                    af[i], bfr[j], acc[i][j], 0, 0, 2, sa_cur[i], 2, sb_cur[j]);
                        }
                }
            } else {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    bf16x8 af[MB], bfr[NB];
                    const int chunk = 2 * ks + (lane >> 5);
#pragma unroll
                    for (int i = 0; i < MB; ++i) {
                        int row = wm * WTM + i * 32 + (lane & 31);
                        af[i] = *(const bf16x8 LDS_AS*)(As + kc_offset(row, chunk));
                    }
                    if constexpr (KIND == kBf16NN) {
                        const int g = lane >> 4, li = lane & 15;
#pragma unroll
                        for (int j = 0; j < NB; ++j) {
                            int n = wn * WTN + j * 32 + 16 * (g & 1) + 4 * (li & 3);
                            int k = ks * 16 + 8 * (g >> 1) + (li >> 2);
                            bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                (bf16x4 LDS_AS*)(Bs + nn_offset<BN>(k, n)));
                            bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                (bf16x4 LDS_AS*)(Bs + nn_offset<BN>(k + 4, n)));
                            bfr[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                        }
                    } else {
#pragma unroll
                        for (int j = 0; j < NB; ++j) {
                            int row = wn * WTN + j * 32 + (lane & 31);
                            bfr[j] = *(const bf16x8 LDS_AS*)(Bs + kc_offset(row, chunk));
                        }
                    }
#pragma unroll
                    for (int i = 0; i < MB; ++i)
#pragma unroll
                        for (int j = 0; j < NB; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j],
                                                                                acc[i][j], 0, 0, 0);
                }
            }
        };

        // Prologue: stage 0.
        load_scales(0, sa_cur, sb_cur);
        load_stage(0, 0);
        wait_vmem();
        __syncthreads();

        for (int kt = 0; kt < a.kt_total; ++kt) {
            const bool more = kt + 1 < a.kt_total;
            if (more) {
                load_stage(kt + 1, (kt + 1) & 1);
                load_scales(kt + 1, sa_nxt, sb_nxt);
            }
            compute(kt & 1);
            wait_vmem();
            __syncthreads();
            if constexpr (KIND == kMx) {
                if (more) {
#pragma unroll
                    for (int i = 0; i < MB; ++i) sa_cur[i] = sa_nxt[i];
#pragma unroll
                    for (int j = 0; j < NB; ++j) sb_cur[j] = sb_nxt[j];
                }
            }
        }

        // Epilogue: predicated fp32 stores of the accumulators.
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int col = n0 + wn * WTN + j * 32 + (lane & 31);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = m0 + wm * WTM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    if (row < a.M && col < a.N) epi::store(a.C, a.ldc, a.epi, row, col, acc[i][j][r]);
                }
            }
    }
}

// C[0:M, 0:N] := the K == 0 product (zero, through the epilogue if any).
__global__ void zero_fill_kernel(void* C, int64_t ldc, int M, int N, epi::Params e) {
    int64_t total = (int64_t)M * N;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        int64_t r = idx / N, c = idx - r * N;
        epi::store(C, ldc, e, (int)r, (int)c, 0.0f);
    }
}

// Split-K reduction: C(i, j) = epilogue(W[0](i, j) + W[1](i, j) + ... +
// W[splits-1](i, j)), the partial sums of the K ranges added in range order,
// so the result does not depend on how the ranges were scheduled.  W holds
// `splits` dense M x N fp32 planes.  With N % 4 == 0 (and W 16-byte
// aligned) each thread adds 4 consecutive elements of one row with 16-byte
// loads.  Bound by HBM: splits M N 4 bytes read, M N (4 or 2) written.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ W, int splits, int M, int N,
                                                            void* C, int64_t ldc, epi::Params e) {
    const int64_t plane = (int64_t)M * N;
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    if ((N & 3) == 0) {
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        const bool vec = epi::vec4_ok(C, ldc, e);
        for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < plane / 4; q += step) {
            f32x4 acc = *(const f32x4*)(W + 4 * q);
            for (int r = 1; r < splits; ++r) acc += *(const f32x4*)(W + r * plane + 4 * q);
            const int row = (int)(4 * q / N);
            const int col = (int)(4 * q - (int64_t)row * N);
            epi::store4(C, ldc, e, row, col, acc[0], acc[1], acc[2], acc[3], vec);
        }
        return;
    }
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < plane; q += step) {
        float acc = W[q];
        for (int r = 1; r < splits; ++r) acc += W[r * plane + q];
        const int row = (int)(q / N);
        epi::store(C, ldc, e, row, (int)(q - (int64_t)row * N), acc);
    }
}

// Zero n ints (the dynamic schedule's tile counters) with vector stores; a
// kernel rather than a memset so that the call stays capturable as kernels.
__global__ __launch_bounds__(256) void zero_words_kernel(int* p, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

// Split tiles of the stream-K style plan: the ranges' partial tiles of split
// tile i are 256 x 256 blocks r T + i of a.part (T = a.tiles_per_split), and
// C's tile a.tile0 + i = epilogue(block 0 + block T + ... + block (s-1) T),
// added in range order.  Sixteen workgroups per tile, 16 rows each; only
// elements inside M x N are read back into C (the rest of a block was never
// written).
__global__ __launch_bounds__(256) void tile_reduce_kernel(fast::Args a, int splits, void* C, int64_t ldc,
                                                          epi::Params e) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    constexpr int kT = fast::kTile;
    const int i = blockIdx.x >> 4, q = blockIdx.x & 15;
    int tm, tn;
    fast::tile_coords(a, a.tile0 + i, tm, tn);
    const int m0 = tm * kT, n0 = tn * kT;
    const int64_t plane = (int64_t)a.tiles_per_split * kT * kT;
    const float* blk = a.part + (int64_t)i * kT * kT;
    const bool vec = epi::vec4_ok(C, ldc, e);
    for (int v = threadIdx.x; v < 16 * kT / 4; v += blockDim.x) {
        const int row = 16 * q + v / (kT / 4), col = 4 * (v % (kT / 4));
        if (m0 + row >= a.M || n0 + col >= a.N) continue;
        const int64_t off = (int64_t)row * kT + col;
        f32x4 acc = *(const f32x4*)(blk + off);
        for (int r = 1; r < splits; ++r) acc += *(const f32x4*)(blk + r * plane + off);
        const float v0 = acc[0], v1 = acc[1], v2 = acc[2], v3 = acc[3];
        if (n0 + col + 3 < a.N) {
            epi::store4(C, ldc, e, m0 + row, n0 + col, v0, v1, v2, v3, vec);
            continue;
        }
        epi::store(C, ldc, e, m0 + row, n0 + col, v0);
        if (n0 + col + 1 < a.N) epi::store(C, ldc, e, m0 + row, n0 + col + 1, v1);
        if (n0 + col + 2 < a.N) epi::store(C, ldc, e, m0 + row, n0 + col + 2, v2);
    }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------

struct DeviceInfo {
    int checked;
    int supported;
    int cus;
};

constexpr int kMaxDevices = 64;
DeviceInfo g_devices[kMaxDevices];
std::mutex g_devices_mutex;

int device_info(DeviceInfo* out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return GEMM_ERR_UNSUPPORTED;
    }
    std::lock_guard<std::mutex> lock(g_devices_mutex);
    DeviceInfo& d = g_devices[dev];
    if (!d.checked) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return GEMM_ERR_UNSUPPORTED;
        }
        d.supported = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        d.cus = prop.multiProcessorCount;
        d.checked = 1;
    }
    *out = d;
    return d.supported ? GEMM_OK : GEMM_ERR_UNSUPPORTED;
}

bool aligned16(const void* p) { return (((uintptr_t)p) & 15) == 0; }

template <int BM, int BN, int KIND, bool DIRECT>
int launch(Args a, int cus, hipStream_t stream) {
    a.tiles_m = (a.M + BM - 1) / BM;
    a.tiles_n = (a.N + BN - 1) / BN;
    a.num_tiles = a.tiles_m * a.tiles_n;
    a.group_m = a.tiles_m < 8 ? a.tiles_m : 8;
    const int occupancy = (BM * BN >= 256 * 256) ? 1 : 2;
    int grid = cus * occupancy;
    if (grid > a.num_tiles) grid = a.num_tiles;
    if (grid >= 8) grid -= grid % 8;
    a.xcd_remap = (grid % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((gemm_kernel<BM, BN, KIND, DIRECT>), dim3(grid), dim3(kThreads), 0, stream, a);
    return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

int zero_fill(void* C, int64_t ldc, int64_t M, int64_t N, const epi::Params& e, hipStream_t stream) {
    int64_t total = M * N;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, C, ldc, (int)M,
                       (int)N, e);
    return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

// Common argument checks; returns GEMM_OK to proceed, 1 for "nothing to do".
int check_common(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                 int64_t ldb, int64_t ldb_min, const void* C, int64_t ldc) {
    if (M < 0 || N < 0 || K < 0) return GEMM_ERR_INVALID_ARG;
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return GEMM_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return 1;
    if (C == nullptr || ldc < N) return GEMM_ERR_INVALID_ARG;
    if (K > 0) {
        if (A == nullptr || B == nullptr) return GEMM_ERR_INVALID_ARG;
        if (lda < K || ldb < ldb_min) return GEMM_ERR_INVALID_ARG;
    }
    return GEMM_OK;
}

Args make_args(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
               int64_t ldb, void* C, int64_t ldc, int bk, const epi::Params& e) {
    Args a;
    memset(&a, 0, sizeof a);
    a.A = (const uint8_t*)A;
    a.B = (const uint8_t*)B;
    a.C = (float*)C;
    a.epi = e;
    a.lda = lda;
    a.ldb = ldb;
    a.ldc = ldc;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.kt_full = (int)(K / bk);
    a.kt_total = (int)((K + bk - 1) / bk);
    return a;
}

// Tile choice: 256 x 256 when that still gives every CU at least ~3/4 of a
// tile's worth of work, else 128 x 128 (two workgroups per CU).
bool use_big_tiles(int64_t M, int64_t N, int cus) {
    int64_t big = ((M + 255) / 256) * ((N + 255) / 256);
    return big * 4 >= (int64_t)cus * 3;
}

// The 256 x 256 kernels store C with 32-bit buffer offsets: 256 rows of C
// must span less than 2 GiB.
bool c_ok(int64_t ldc) { return ldc < ((int64_t)1 << 21); }

// Most K ranges a split-K call uses.
constexpr int kMaxSplits = 32;

// ---------------------------------------------------------------------------
// Fast path (gemm_fast.h): 256 x 256 tiles, direct-to-LDS buffer loads.
// ---------------------------------------------------------------------------

// Pipeline variant of the fast kernel: k-tile bytes per operand row, LDS
// stages and the early-DMA split.  The defaults, measured on MI355X at 4096^3
// and 8192^3, are 128-byte rows x 2 stages for bf16 NT and NN (early 6,
// spread 2) and for MX (scale ring, early 12).
struct FastVariant {
    int rb, stages, group, early, spread, waves, lookahead, mfma;
};

// Measurement builds (-DLIBGEMM_MEASURE) read switches from the environment
// that select other compiled pipelines for A/B timing:
// LIBGEMM_VARIANT=<rb>x<stages>[e<early>[d<spread>[w<waves>[l<lookahead>[m<mfma>]]]]]
// picks the pipeline (for two stages the early-DMA split, the k-steps
// between a fragment read and its MFMAs, and the MFMA shape, 32 or 16);
// LIBGEMM_GROUP=<n> the
// number of tile rows per raster band.  The library as built by default
// compiles none of those instances and reads no environment variable: every
// call runs the defaults below.
FastVariant env_variant() {
#ifndef LIBGEMM_MEASURE
    return FastVariant{0, 0, 0, -1, 0, 4, 1, 16};
#else
    static FastVariant v = [] {
        FastVariant r{0, 0, 0, -1, 0, 4, 1, 16};
        const char* e = getenv("LIBGEMM_VARIANT");
        if (e) {
            int rb = 0, st = 0, ea = -1, sp = 0, nw = 4, la = 1, mf = 16;
            const int n = sscanf(e, "%dx%de%dd%dw%dl%dm%d", &rb, &st, &ea, &sp, &nw, &la, &mf);
            if (n >= 2) {
                r.rb = rb;
                r.stages = st;
            }
            if (n >= 3) r.early = ea;
            if (n >= 4) r.spread = sp;
            if (n >= 5) r.waves = nw;
            if (n >= 6) r.lookahead = la;
            if (n == 7) r.mfma = mf;
        }
        const char* g = getenv("LIBGEMM_GROUP");
        if (g) r.group = atoi(g);
        return r;
    }();
    return v;
#endif
}

// SPLIT: split-K units (a.kslice set, `splits` K ranges): the partial sums
// go to `splits` stacked M x N planes of C.
// DYN: the dynamic tile schedule; a.tile_ctr holds 256 ints that are zeroed
// on the stream first (falls back to the static walk when the grid is not a
// multiple of 8).
template <int KIND, int RB, int S, int SG = 1, int E = 0, int D = 0, int NW = 4, bool FUSED = false,
          bool SPLIT = false, bool DYN = false, int LA = 1, int MF = 32>
int launch_fast(fast::Args a, int cus, hipStream_t stream, int group_m = 0, int splits = 1) {
    constexpr int BK = RB / (KIND == fast::kMX ? 1 : 2);
    fast::fast_tiles(a, group_m, BK);
    if (SPLIT) {
        if (a.part == nullptr) {  // every tile split, stacked dense planes
            a.dp_units = 0;
            a.tile0 = 0;
            a.tiles_per_split = a.num_tiles;
        }
        a.num_tiles = a.dp_units + a.tiles_per_split * splits;
    }
    const int grid = fast::fast_grid(a, cus);
    if constexpr (MF == 16) {
        static_assert(KIND != fast::kMX && RB == 128 && S == 2 && SG == 1 && E == 8 && D == 1 && NW == 4 && LA == 1,
                      "the 16 x 16 x 32 instances of gemm_mf16.hip");
        const bool tail = a.kt_total > a.kt_full;
        if constexpr (DYN) {
            if (a.xcd_remap) {
                hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(256), 0, stream, a.tile_ctr, 256);
                if (tail) fast::launch_mf16<KIND, true, FUSED, false, true>(grid, stream, a);
                else fast::launch_mf16<KIND, false, FUSED, false, true>(grid, stream, a);
                return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
            }
        }
        if (tail) fast::launch_mf16<KIND, true, FUSED, SPLIT, false>(grid, stream, a);
        else fast::launch_mf16<KIND, false, FUSED, SPLIT, false>(grid, stream, a);
        return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
    }
    if constexpr (DYN) {
        if (a.xcd_remap) {
            hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(256), 0, stream, a.tile_ctr, 256);
            if (a.kt_total > a.kt_full)
                hipLaunchKernelGGL((fast::gemm_fast_kernel<KIND, RB, S, true, SG, E, D, NW, FUSED, false, true, LA, MF>),
                                   dim3(grid), dim3(64 * NW), 0, stream, a);
            else
                hipLaunchKernelGGL((fast::gemm_fast_kernel<KIND, RB, S, false, SG, E, D, NW, FUSED, false, true, LA, MF>),
                                   dim3(grid), dim3(64 * NW), 0, stream, a);
            return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
        }
    }
    if (a.kt_total > a.kt_full) {
        hipLaunchKernelGGL((fast::gemm_fast_kernel<KIND, RB, S, true, SG, E, D, NW, FUSED, SPLIT, false, LA, MF>), dim3(grid),
                           dim3(64 * NW), 0, stream, a);
    } else {
        hipLaunchKernelGGL((fast::gemm_fast_kernel<KIND, RB, S, false, SG, E, D, NW, FUSED, SPLIT, false, LA, MF>), dim3(grid),
                           dim3(64 * NW), 0, stream, a);
    }
    return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

// The bf16 instances the library runs: 16 x 16 x 32 MFMAs (gemm_mf16.hip).
// Measurement builds run the 32 x 32 x 16 form instead under
// LIBGEMM_VARIANT=...m32 (the fused, split-K and dynamic entry points: 6 DMA
// instructions early, the rest over two k-steps).
template <int KIND, bool FUSED = false, bool SPLIT = false, bool DYN = false>
int launch_bf16_16(fast::Args a, int cus, hipStream_t s, int group_m, int splits = 1) {
#ifdef LIBGEMM_MEASURE
    if (env_variant().mfma == 32)
        return launch_fast<KIND, 128, 2, 1, 6, 2, 4, FUSED, SPLIT, DYN>(a, cus, s, group_m, splits);
#endif
    return launch_fast<KIND, 128, 2, 1, 8, 1, 4, FUSED, SPLIT, DYN, 1, 16>(a, cus, s, group_m, splits);
}

// The split-K units of the fast kernel.  With M or N at most 32 every tile is
// at most an eighth full in one dimension and the units mostly stream the
// other operand; there the 32 x 32 x 16 form measured faster (NT, K = 8192,
// 8 ranges, two boxes: 16 x 8192 29.8-31.8 us against 33.3-34.0 us with the
// 16 x 16 form, 8192 x 16 31.0 against 39.2 us), while from 64 rows on the
// two forms traded places between boxes and the 16 x 16 form led at
// 1024 x 1024 x 32768 (68-70 against 70-73 us).
int launch_split_bf16(bool nt, int64_t M, int64_t N, const fast::Args& a, int cus, hipStream_t s, int g,
                      int splits) {
    if (M <= 32 || N <= 32) {
        return nt ? launch_fast<fast::kNT, 128, 2, 1, 6, 2, 4, false, true>(a, cus, s, g, splits)
                  : launch_fast<fast::kNN, 128, 2, 1, 6, 2, 4, false, true>(a, cus, s, g, splits);
    }
    return nt ? launch_bf16_16<fast::kNT, false, true>(a, cus, s, g, splits)
              : launch_bf16_16<fast::kNN, false, true>(a, cus, s, g, splits);
}

#ifdef LIBGEMM_MEASURE
// The 8-wave 16 x 16 x 32 plain product (measurement builds).
template <int KIND>
int launch_w8_16(fast::Args a, int cus, hipStream_t s, int group_m) {
    fast::fast_tiles(a, group_m, 64);
    const int grid = fast::fast_grid(a, cus);
    if (a.kt_total > a.kt_full) fast::launch_mf16_w8<KIND, true>(grid, s, a);
    else fast::launch_mf16_w8<KIND, false>(grid, s, a);
    return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}
#endif

// Whether the fast kernel's preconditions hold (see gemm_fast.h).
bool fast_ok(int kind, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
             int64_t ldb, const void* SA, const void* SB) {
    const int64_t esz = kind == fast::kMX ? 1 : 2;
    const int64_t lim = (int64_t)1 << 31;
    if (!aligned16(A) || !aligned16(B)) return false;
    if ((lda * esz) % 16 || (ldb * esz) % 16) return false;
    if (256 * lda * esz >= lim) return false;
    if (kind == fast::kNN) {
        if (N % 8) return false;
        if (K * ldb * esz >= lim) return false;
    } else if (256 * ldb * esz >= lim) {
        return false;
    }
    if (kind == fast::kMX) {
        // the MX pipeline streams 64 or 128 codes per k-tile and the scale
        // codes of a k-tile as one 2- or 4-byte load per row
        if (K % 64) return false;
        if ((((uintptr_t)SA) & 1) || (((uintptr_t)SB) & 1)) return false;
    }
    (void)M;
    return true;
}

fast::Args make_fast_args(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                          const void* B, int64_t ldb, void* C, int64_t ldc, int64_t esz, const epi::Params& e) {
    fast::Args a;
    memset(&a, 0, sizeof a);
    a.A = (const uint8_t*)A;
    a.B = (const uint8_t*)B;
    a.C = (float*)C;
    a.lda_b = lda * esz;
    a.ldb_b = ldb * esz;
    a.ldc = ldc;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    // C stores bypass the caches' retention (non-temporal) only when every
    // 32-column segment a wave stores is a whole 128-byte line: then C does
    // not evict the operand panels that L2 and the Infinity Cache serve to
    // the other tiles (8192^3 on MI355X: 0.759 against 0.814 ms cached).
    // Otherwise each line is written in two parts by two stores; those go
    // with device scope, which measured best of the policies there
    // (4001 x 3003 x 2050 with ldc = 3003, same box: 61.5-62.4 us against
    // 63.7-65.2 us cached and 85 us non-temporal).
    // LIBGEMM_C_NT=0|1|2 overrides the choice (measurement builds only).
#ifdef LIBGEMM_MEASURE
    static int c_pol_env = [] {
        const char* e = getenv("LIBGEMM_C_NT");
        return e ? atoi(e) : -1;
    }();
#else
    constexpr int c_pol_env = -1;
#endif
    // bf16 or E4M3 output: a 32-column segment is 64 or 32 bytes, part of a line
    const bool lines = e.out == epi::kF32 && ((uintptr_t)C % 128 == 0) && (ldc % 32 == 0);
    a.c_pol = c_pol_env >= 0 ? c_pol_env : (lines ? fast::kCStoreStream : fast::kCStoreDevice);
    a.epi = e;
    return a;
}

int launch_fast_bf16(bool nt, const fast::Args& a, int cus, hipStream_t s) {
    const FastVariant v = env_variant();
    const int g = v.group;
    // fused epilogue: the default pipeline (in measurement builds the MF
    // switch applies; the other variants below are of the plain product)
    if (a.epi.on) {
        if (nt) return launch_bf16_16<fast::kNT, true>(a, cus, s, g);
        return launch_bf16_16<fast::kNN, true>(a, cus, s, g);
    }
    if (nt) {
#ifdef LIBGEMM_MEASURE
        if (v.rb == 64 && v.stages == 4) return launch_fast<fast::kNT, 64, 4>(a, cus, s, g);
        // 8 waves (two per SIMD, 128 x 64 wave tiles), kept for
        // measurements: at 8192^3 on MI355X the 32 x 32 form measured 1%
        // slower than its 4-wave form, the 16 x 16 form 2.7% slower (1.5x
        // the LDS fragment reads)
        if (v.waves == 8 && v.mfma == 32) return launch_fast<fast::kNT, 128, 2, 1, 4, 2, 8>(a, cus, s, g);
        if (v.waves == 8) return launch_w8_16<fast::kNT>(a, cus, s, g);
        if (v.early == 0) return launch_fast<fast::kNT, 128, 2>(a, cus, s, g);
        if (v.lookahead == 2)
            return launch_fast<fast::kNT, 128, 2, 1, 6, 2, 4, false, false, false, 2>(a, cus, s, g);
        // the 32 x 32 x 16 form: 6 DMA instructions of k-tile t+2 right
        // after the barrier of k-tile t, the other 10 over k-steps 0 and 1
        // of t+1 (MI355X, 8192^3, same box: 776.5 -> 746.5 us and 797.6 ->
        // 778.2 us); the default before the 16 x 16 form
        if (v.mfma == 32) return launch_fast<fast::kNT, 128, 2, 1, 6, 2>(a, cus, s, g);
#endif
        // default: 16 x 16 x 32 MFMAs (gemm_mf16.hip; 8192^3 on one box:
        // 718-720 us against 759-762 us for the 32 x 32 form)
        return launch_bf16_16<fast::kNT>(a, cus, s, g);
    }
#ifdef LIBGEMM_MEASURE
    if (v.waves == 8) return launch_w8_16<fast::kNN>(a, cus, s, g);
    if (v.rb == 64 && v.stages == 4) return launch_fast<fast::kNN, 64, 4>(a, cus, s, g);
    if (v.rb == 128 && v.stages == 2 && v.early == 0) return launch_fast<fast::kNN, 128, 2>(a, cus, s, g);
    if (v.lookahead == 2) return launch_fast<fast::kNN, 128, 2, 1, 6, 2, 4, false, false, false, 2>(a, cus, s, g);
    // the 32 x 32 x 16 form, as NT (MI355X, 4096^3: 108.8 -> 105.5 us
    // against 64 x 4; 8192^3: 801.5 -> 771.2 us)
    if (v.mfma == 32) return launch_fast<fast::kNN, 128, 2, 1, 6, 2>(a, cus, s, g);
#endif
    // default: 16 x 16 x 32 MFMAs, as NT (4096^3 on one box: 101.5-103.3 us
    // against 103.8-104.3 us)
    return launch_bf16_16<fast::kNN>(a, cus, s, g);
}

// ---------------------------------------------------------------------------
// Register-load path (gemm_reg.h): 256 x 256 tiles for operands whose rows
// are only 2-byte aligned.
// ---------------------------------------------------------------------------

bool reg_ok(bool nt, int64_t K, int64_t lda, int64_t ldb) {
    const int64_t lim = (int64_t)1 << 31;
    // 32-bit buffer offsets: 256 rows of A (and of B for NT), all K rows of B
    // for NN, plus the dword shift of the descriptor base
    if (256 * lda * 2 + 4 >= lim) return false;
    if (nt) return 256 * ldb * 2 + 4 < lim;
    return K * ldb * 2 + 4 < lim;
}

template <int PF, int BN, bool FUSED = false, int RB = 64>
int launch_reg_pf(bool nt, fast::Args a, int cus, hipStream_t stream) {
    constexpr int BK = regpath::bk_of(RB);
    a.tiles_m = (a.M + fast::kTile - 1) / fast::kTile;
    a.tiles_n = (a.N + BN - 1) / BN;
    a.num_tiles = a.tiles_m * a.tiles_n;
    const int g = env_variant().group;
    const int group_m = g > 0 ? g : 8;
    a.group_m = a.tiles_m < group_m ? a.tiles_m : group_m;
    a.kt_full = a.K / BK;
    a.kt_total = (a.K + BK - 1) / BK;
    // row-major B with N % 8 != 0: the last k-row ends inside a 16-byte
    // chunk, which only the tail path reads safely
    if (!nt && a.N % 8 != 0 && a.kt_full == a.kt_total) a.kt_full -= 1;
    int grid = cus < a.num_tiles ? cus : a.num_tiles;
    if (grid >= 8) grid -= grid % 8;
    a.xcd_remap = (grid % 8 == 0) ? 1 : 0;
    const bool tail = a.kt_total > a.kt_full;
    const dim3 blk(fast::kThreads);
    if (nt) {
        if (tail)
            hipLaunchKernelGGL((regpath::gemm_reg_kernel<fast::kNT, true, PF, BN, FUSED, RB>), dim3(grid), blk, 0, stream, a);
        else
            hipLaunchKernelGGL((regpath::gemm_reg_kernel<fast::kNT, false, PF, BN, FUSED, RB>), dim3(grid), blk, 0, stream, a);
    } else {
        if (tail)
            hipLaunchKernelGGL((regpath::gemm_reg_kernel<fast::kNN, true, PF, BN, FUSED, RB>), dim3(grid), blk, 0, stream, a);
        else
            hipLaunchKernelGGL((regpath::gemm_reg_kernel<fast::kNN, false, PF, BN, FUSED, RB>), dim3(grid), blk, 0, stream, a);
    }
    return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

// Tile width for the register kernel: 192 columns when that needs fewer
// rounds of tiles over the CUs, weighted by the tile's work (for example
// 4001 x 3003: 16 x 12 = 192 tiles of 256 columns leave a quarter of the CUs
// idle, 16 x 16 = 256 tiles of 192 columns fill them).
int reg_tile_n(int64_t M, int64_t N, int cus) {
    const int64_t tm = (M + 255) / 256;
    auto cost = [&](int64_t bn) {
        const int64_t tiles = tm * ((N + bn - 1) / bn);
        return ((tiles + cus - 1) / cus) * bn;
    };
    return cost(192) < cost(256) ? 192 : 256;
}

// Register sets of prefetch of the register kernel, and its k-tile row
// bytes for the plain product: 128 (k-tiles of 64, half the barriers of 64)
// measured 117 against 130 us at 4096^3 with odd leading dimensions and
// 64.0-65.0 against 64.8-67.9 us on 4001 x 3003 x 2050 (MI355X, same box).
// The fused instances keep 64-byte rows, whose epilogue fits the registers.
constexpr int kRegPF = 1;
constexpr int kRegRB = 128;

// Measurement builds: LIBGEMM_REGPF=1|2|4 (register sets of prefetch),
// LIBGEMM_REG_BN=192|256 (tile columns) and LIBGEMM_REG_RB=64 (k-tile rows)
// select other compiled instances.
int launch_reg(bool nt, const fast::Args& a, int cus, hipStream_t stream) {
    int bn = reg_tile_n(a.M, a.N, cus);
#ifdef LIBGEMM_MEASURE
    static int pf = [] {
        const char* e = getenv("LIBGEMM_REGPF");
        return e ? atoi(e) : 0;
    }();
    static int bn_env = [] {
        const char* e = getenv("LIBGEMM_REG_BN");
        return e ? atoi(e) : 0;
    }();
    if (bn_env == 192 || bn_env == 256) bn = bn_env;
    // LIBGEMM_REG_RB=64: k-tiles of 32 (plain product), with LIBGEMM_REGPF
    static int rb_env = [] {
        const char* e = getenv("LIBGEMM_REG_RB");
        return e ? atoi(e) : 0;
    }();
    if (!a.epi.on && rb_env == 64) {
        if (pf == 2) return bn == 192 ? launch_reg_pf<2, 192>(nt, a, cus, stream) : launch_reg_pf<2, 256>(nt, a, cus, stream);
        if (pf == 4) return bn == 192 ? launch_reg_pf<4, 192>(nt, a, cus, stream) : launch_reg_pf<4, 256>(nt, a, cus, stream);
        return bn == 192 ? launch_reg_pf<1, 192>(nt, a, cus, stream) : launch_reg_pf<1, 256>(nt, a, cus, stream);
    }
    if (!a.epi.on && pf == 2)
        return bn == 192 ? launch_reg_pf<2, 192, false, kRegRB>(nt, a, cus, stream)
                         : launch_reg_pf<2, 256, false, kRegRB>(nt, a, cus, stream);
#endif
    if (a.epi.on) {
        if (bn == 192) return launch_reg_pf<kRegPF, 192, true>(nt, a, cus, stream);
        return launch_reg_pf<kRegPF, 256, true>(nt, a, cus, stream);
    }
    if (bn == 192) return launch_reg_pf<kRegPF, 192, false, kRegRB>(nt, a, cus, stream);
    return launch_reg_pf<kRegPF, 256, false, kRegRB>(nt, a, cus, stream);
}

// ---------------------------------------------------------------------------
// Small-M path (gemm_small.h): row-major B streamed once, M <= 64.
// ---------------------------------------------------------------------------

bool small_ok(bool nt, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
              int64_t ldb) {
    if (nt || M > 64 || K < 1) return false;
    if (!aligned16(A) || !aligned16(B) || (lda % 8) || (ldb % 8)) return false;
    const int64_t lim = (int64_t)1 << 31;
    if (K * ldb * 2 >= lim || M * lda * 2 >= lim) return false;
    // enough column blocks to occupy the GPU; otherwise the tiled kernels
    return N >= 2048;
}

// splits > 1: K ranges of kslice rows (a multiple of small::kStepK), fp32
// partial sums to `splits` stacked M x N planes at C (ldc == N, plain e).
template <int MB, int NP, int COLS, int WAVES, int BAUX = 0>
int launch_small(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                 void* C, int64_t ldc, const epi::Params& e, hipStream_t stream, int splits = 1,
                 int64_t kslice = 0) {
    small::Args a;
    a.A = (const uint8_t*)A;
    a.B = (const uint8_t*)B;
    a.C = C;
    a.epi = e;
    a.lda_b = lda * 2;
    a.ldb_b = ldb * 2;
    a.ldc = ldc;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    if (splits <= 1) kslice = K;
    a.kslice = (int)kslice;
    a.c_split = splits > 1 ? M * N : 0;
    const int64_t per = (kslice + WAVES - 1) / WAVES;
    a.kw = (int)((per + small::kStepK - 1) / small::kStepK * small::kStepK);
    const int grid = (int)((N + COLS - 1) / COLS);
    a.pair_xcd = (COLS == 32 && grid % 16 == 0) ? 1 : 0;
#ifdef LIBGEMM_MEASURE
    static const int pair_env = [] {
        const char* e = getenv("LIBGEMM_SMALL_PAIR");
        return e ? atoi(e) : -1;
    }();
    if (pair_env == 0) a.pair_xcd = 0;  // LIBGEMM_SMALL_PAIR=0: no XCD pairing
#endif
    hipLaunchKernelGGL((small::gemm_small_m_nn<MB, NP, COLS, WAVES, BAUX>), dim3(grid, splits > 1 ? splits : 1),
                       dim3(64 * WAVES), 0, stream, a);
    return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

int launch_small_bf16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                      void* C, int64_t ldc, const epi::Params& e, hipStream_t s, int splits = 1,
                      int64_t kslice = 0, int cols = 32) {
    // wide strips (split-K partials only, M <= 16): 128 columns, 8 waves
    // (two per SIMD, so the 4 steps of B prefetch fit the registers)
    if (cols == 128 && M <= 16) {
#ifdef LIBGEMM_MEASURE
        // LIBGEMM_WIDE=<np>x<aux>: prefetch steps and B cache policy of the wide strips
        static int wv = [] {
            const char* e = getenv("LIBGEMM_WIDE");
            int np = 0, aux = 0;
            if (e && sscanf(e, "%dx%d", &np, &aux) == 2) return np * 10 + aux;
            return 0;
        }();
        if (wv == 42) return launch_small<1, 4, 128, 8, 2>(M, N, K, A, lda, B, ldb, C, ldc, e, s, splits, kslice);
        if (wv == 60) return launch_small<1, 6, 128, 8>(M, N, K, A, lda, B, ldb, C, ldc, e, s, splits, kslice);
        if (wv == 62) return launch_small<1, 6, 128, 8, 2>(M, N, K, A, lda, B, ldb, C, ldc, e, s, splits, kslice);
        if (wv == 40) return launch_small<1, 4, 128, 8>(M, N, K, A, lda, B, ldb, C, ldc, e, s, splits, kslice);
        if (wv == 22) return launch_small<1, 2, 128, 8, 2>(M, N, K, A, lda, B, ldb, C, ldc, e, s, splits, kslice);
#endif
        // 2 steps of prefetch: as fast as 4 on 16 x 8192 x 8192 (31.1 against
        // 31.3-32.1 us per call, MI355X) with half the registers
        return launch_small<1, 2, 128, 8>(M, N, K, A, lda, B, ldb, C, ldc, e, s, splits, kslice);
    }
    if (M <= 16) {
#ifdef LIBGEMM_MEASURE
        // LIBGEMM_SMALL=<np>x<cols>x<waves> selects another compiled variant
        static int sv = [] {
            const char* e = getenv("LIBGEMM_SMALL");
            int np = 0, c = 0, w = 0;
            if (e && sscanf(e, "%dx%dx%d", &np, &c, &w) == 3) return np * 10000 + c * 100 + w;
            return 0;
        }();
        if (sv == 120000 + 3208)
            return launch_small<1, 12, 32, 8>(M, N, K, A, lda, B, ldb, C, ldc, e, s, splits, kslice);
        if (sv == 80000 + 3216)
            return launch_small<1, 8, 32, 16>(M, N, K, A, lda, B, ldb, C, ldc, e, s, splits, kslice);
        if (sv == 80000 + 6416)
            return launch_small<1, 8, 64, 16>(M, N, K, A, lda, B, ldb, C, ldc, e, s, splits, kslice);
        if (sv == 80000 + 3208)
            return launch_small<1, 8, 32, 8>(M, N, K, A, lda, B, ldb, C, ldc, e, s, splits, kslice);
#endif
        return launch_small<1, 4, 32, 16>(M, N, K, A, lda, B, ldb, C, ldc, e, s, splits, kslice);
    }
    if (M <= 32) return launch_small<2, 8, 32, 8>(M, N, K, A, lda, B, ldb, C, ldc, e, s, splits, kslice);
    return launch_small<4, 4, 32, 8>(M, N, K, A, lda, B, ldb, C, ldc, e, s, splits, kslice);
}

int bf16_dispatch(bool nt, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                  const void* B, int64_t ldb, void* C, int64_t ldc, const epi::Params& e, void* stream) {
    int rc = check_common(M, N, K, A, lda, B, ldb, nt ? K : N, C, ldc);
    if (rc == 1) return GEMM_OK;
    if (rc != GEMM_OK) return rc;
    DeviceInfo dev;
    rc = device_info(&dev);
    if (rc != GEMM_OK) return rc;
    hipStream_t s = (hipStream_t)stream;
    if (K == 0) return zero_fill(C, ldc, M, N, e, s);
    Args a = make_args(M, N, K, A, lda, B, ldb, C, ldc, 64, e);
    const bool direct = aligned16(A) && aligned16(B) && (lda % 8 == 0) && (ldb % 8 == 0) &&
                        (nt || (N % 8 == 0));
    if (small_ok(nt, M, N, K, A, lda, B, ldb))
        return launch_small_bf16(M, N, K, A, lda, B, ldb, C, ldc, e, s);
    const bool big = use_big_tiles(M, N, dev.cus);
#ifdef LIBGEMM_MEASURE
    // LIBGEMM_FORCE_REG=1 runs the register-load kernel where the direct-load
    // one would
    static const bool force_reg = getenv("LIBGEMM_FORCE_REG") != nullptr;
    if (force_reg && big && c_ok(ldc) && reg_ok(nt, K, lda, ldb))
        return launch_reg(nt, make_fast_args(M, N, K, A, lda, B, ldb, C, ldc, 2, e), dev.cus, s);
#endif
    if (big && c_ok(ldc) && fast_ok(nt ? fast::kNT : fast::kNN, M, N, K, A, lda, B, ldb, nullptr, nullptr))
        return launch_fast_bf16(nt, make_fast_args(M, N, K, A, lda, B, ldb, C, ldc, 2, e), dev.cus, s);
    if (big && c_ok(ldc) && reg_ok(nt, K, lda, ldb))
        return launch_reg(nt, make_fast_args(M, N, K, A, lda, B, ldb, C, ldc, 2, e), dev.cus, s);
    if (nt) {
        if (big) return direct ? launch<256, 256, kBf16NT, true>(a, dev.cus, s)
                               : launch<256, 256, kBf16NT, false>(a, dev.cus, s);
        return direct ? launch<128, 128, kBf16NT, true>(a, dev.cus, s)
                      : launch<128, 128, kBf16NT, false>(a, dev.cus, s);
    }
    if (big) return direct ? launch<256, 256, kBf16NN, true>(a, dev.cus, s)
                           : launch<256, 256, kBf16NN, false>(a, dev.cus, s);
    return direct ? launch<128, 128, kBf16NN, true>(a, dev.cus, s)
                  : launch<128, 128, kBf16NN, false>(a, dev.cus, s);
}

const epi::Params kPlain = {nullptr, nullptr, nullptr, 0, 0};

// ---------------------------------------------------------------------------
// Split-K: the K extent cut into ranges computed by separate work units,
// whose fp32 partial sums a second pass adds in range order.
// ---------------------------------------------------------------------------

enum SplitKernel { kSplitNone = 0, kSplitFast = 1, kSplitSmall = 2 };

struct SplitPlan {
    int kernel;      // SplitKernel
    int splits;      // K ranges (1: no split)
    int64_t kslice;  // K elements per range, the last range takes the rest
    int64_t dp;      // stream-K style: whole tiles computed first (0: every tile split)
    int64_t rem;     // stream-K style: tiles split after them
    int cols;        // small-M kernel: columns per workgroup (32, or 128 for wide strips)
};

// Workspace bytes of a plan.
int64_t plan_bytes(const SplitPlan& p, int64_t M, int64_t N) {
    if (p.splits <= 1) return 0;
    if (p.rem > 0) return (int64_t)p.splits * p.rem * fast::kTile * fast::kTile * 4;
    return (int64_t)p.splits * M * N * 4;
}

// Which kernel would compute the partial sums of this problem.  `aligned`:
// the operand pointers are 16-byte aligned (the query entry point assumes
// they are).
int split_kernel(bool nt, int64_t M, int64_t N, int64_t K, bool aligned, int64_t lda, int64_t ldb) {
    const int64_t lim = (int64_t)1 << 31;
    if (!aligned || (lda % 8) || (ldb % 8)) return kSplitNone;
    // the stacked partial planes are addressed with 32-bit offsets per 256 rows
    if (!c_ok(N)) return kSplitNone;
    if (!nt && M <= 64 && N >= 2048 && K * ldb * 2 < lim && M * lda * 2 < lim) return kSplitSmall;
    if (256 * lda * 2 >= lim) return kSplitNone;
    if (nt ? 256 * ldb * 2 >= lim : (N % 8 || K * ldb * 2 >= lim)) return kSplitNone;
    return kSplitFast;
}

// The split plan.  requested > 0 asks for that many ranges (fewer when K is
// too short); 0 lets the shape decide:
//   - 256 x 256 tiles (fast kernel): when the tiles give the CUs less than
//     3/4 of a round, cut K so that tiles x ranges fills about one round,
//     each range at least 8 k-tiles (512) long;
//   - small M (small kernel): when its 32-column blocks give fewer
//     workgroups than CUs, the same with ranges of at least 1024.  With
//     M <= 16, when 128-column blocks times ranges of at least 1024 fill
//     at least 3/4 of the CUs, those wide strips are used instead, even
//     where the 32-column blocks alone would fill the CUs: each workgroup
//     then reads 256-byte row segments of B instead of 64-byte ones, which
//     streams B from HBM faster (16 x 8192 x 8192: 4 ranges of 2048);
//   - 256 x 256 tiles filling more than one round with a last round at most
//     half full (stream-K style): the full rounds run whole tiles, and only
//     the last round's tiles are split, into about CUs / (those tiles)
//     ranges of at least 512, so that the last round takes a fraction of a
//     round.  Its partial tiles go to compact 256 x 256 blocks.  A round is
//     the 256 x 256 kernel's persistent grid: the CUs rounded down to a
//     multiple of 8.
SplitPlan plan_split(bool nt, int64_t M, int64_t N, int64_t K, bool aligned, int64_t lda, int64_t ldb, int cus,
                     int requested) {
    SplitPlan p{split_kernel(nt, M, N, K, aligned, lda, ldb), 1, K, 0, 0, 32};
    if (p.kernel == kSplitNone || K <= 0) return p;
    const int64_t gran = p.kernel == kSplitFast ? 64 : small::kStepK;  // k-tile of the partial kernel
    int64_t want = requested;
    // wide strips of the small-M kernel: 128-column blocks times `s` ranges
    // of at least 1024 filling at least 3/4 of the CUs
    const int64_t wide_units = (N + 127) / 128;
    auto wide_ok = [&](int64_t s) {
        return p.kernel == kSplitSmall && M <= 16 && s >= 2 && s <= K / 1024 && wide_units * s * 4 >= (int64_t)cus * 3;
    };
    if (want <= 0 && p.kernel == kSplitSmall) {
        int64_t s = cus / wide_units;
        if (s > K / 1024) s = K / 1024;
        if (s > kMaxSplits) s = kMaxSplits;
        if (wide_ok(s)) want = s;
    }
    if (p.kernel == kSplitSmall && wide_ok(want)) p.cols = 128;
    if (want <= 0) {
        const int64_t units = p.kernel == kSplitFast ? ((M + 255) / 256) * ((N + 255) / 256) : (N + 31) / 32;
        const int64_t min_range = p.kernel == kSplitFast ? 512 : 1024;
        if (units * 4 >= (int64_t)cus * 3) {
            const int64_t grid = cus - cus % 8;
            const int64_t rem = grid > 0 ? units % grid : 0;
            if (p.kernel != kSplitFast || units <= grid || rem == 0 || rem * 2 > grid) return p;
            int64_t s = grid / rem;
            if (s > K / min_range) s = K / min_range;
            if (s > kMaxSplits) s = kMaxSplits;
            if (s < 2) return p;
            int64_t kslice = (K + s - 1) / s;
            kslice = (kslice + gran - 1) / gran * gran;
            const int64_t splits = (K + kslice - 1) / kslice;
            if (splits <= 1) return p;
            p.splits = (int)splits;
            p.kslice = kslice;
            p.dp = units - rem;
            p.rem = rem;
            return p;
        }
        want = cus / units;
        if (want > K / min_range) want = K / min_range;
        if (want > kMaxSplits) want = kMaxSplits;
    }
    if (want > kMaxSplits) want = kMaxSplits;
    if (want <= 1) return p;
    int64_t kslice = (K + want - 1) / want;
    kslice = (kslice + gran - 1) / gran * gran;
    const int64_t splits = (K + kslice - 1) / kslice;
    if (splits <= 1) return p;
    p.splits = (int)splits;
    p.kslice = kslice;
    return p;
}

// The plan a split-K call runs: plan_split on the real operands, except that
// the stream-K style plan stores whole tiles straight to C with the plain
// fp32 epilogue (the split kernel has no fused store), so any other
// epilogue, or a C too wide for 32-bit offsets, runs unsplit.
SplitPlan resolve_split(bool nt, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                        int64_t ldb, int64_t ldc, const epi::Params& e, int cus, int splits) {
    SplitPlan p = plan_split(nt, M, N, K, aligned16(A) && aligned16(B), lda, ldb, cus, splits);
    const bool plain = e.out == epi::kF32 && !e.rs && !e.cs && !e.bias;
    if (p.rem > 0 && (!plain || !c_ok(ldc))) p.splits = 1;
    return p;
}

int splitk_dispatch(bool nt, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                    int64_t ldb, void* C, int64_t ldc, const epi::Params& e, int splits, void* ws,
                    size_t ws_bytes, void* stream) {
    if (splits < 0) return GEMM_ERR_INVALID_ARG;
    int rc = check_common(M, N, K, A, lda, B, ldb, nt ? K : N, C, ldc);
    if (rc == 1) return GEMM_OK;
    if (rc != GEMM_OK) return rc;
    DeviceInfo dev;
    rc = device_info(&dev);
    if (rc != GEMM_OK) return rc;
    const SplitPlan p = resolve_split(nt, M, N, K, A, lda, B, ldb, ldc, e, dev.cus, splits);
    if (p.splits <= 1) return bf16_dispatch(nt, M, N, K, A, lda, B, ldb, C, ldc, e, stream);
    const int64_t need = plan_bytes(p, M, N);
    if (ws == nullptr || (int64_t)ws_bytes < need || ((uintptr_t)ws & 15)) return GEMM_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    if (p.rem > 0) {
        fast::Args a = make_fast_args(M, N, K, A, lda, B, ldb, C, ldc, 2, kPlain);
        a.kslice = (int)p.kslice;
        a.part = (float*)ws;
        a.dp_units = (int)p.dp;
        a.tile0 = (int)p.dp;
        a.tiles_per_split = (int)p.rem;
        const int g = env_variant().group;
        rc = launch_split_bf16(nt, M, N, a, dev.cus, s, g, p.splits);
        if (rc != GEMM_OK) return rc;
        // the same tile geometry as launch_fast's
        a.tiles_m = (a.M + fast::kTile - 1) / fast::kTile;
        a.tiles_n = (a.N + fast::kTile - 1) / fast::kTile;
        a.group_m = a.tiles_m < (g > 0 ? g : 8) ? a.tiles_m : (g > 0 ? g : 8);
        hipLaunchKernelGGL(tile_reduce_kernel, dim3((unsigned)(p.rem * 16)), dim3(256), 0, s, a, p.splits, C, ldc,
                           e);
        return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
    }
    if (p.kernel == kSplitSmall) {
        rc = launch_small_bf16(M, N, K, A, lda, B, ldb, ws, N, kPlain, s, p.splits, p.kslice, p.cols);
    } else {
        fast::Args a = make_fast_args(M, N, K, A, lda, B, ldb, ws, N, 2, kPlain);
        a.kslice = (int)p.kslice;
        a.c_pol = fast::kCStoreCached;  // the partial sums are read back at once
        const int g = env_variant().group;
        rc = launch_split_bf16(nt, M, N, a, dev.cus, s, g, p.splits);
    }
    if (rc != GEMM_OK) return rc;
    int64_t blocks = (M * N / 4 + 255) / 256;
    if (blocks > (int64_t)dev.cus * 8) blocks = (int64_t)dev.cus * 8;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const float*)ws, p.splits,
                       (int)M, (int)N, C, ldc, e);
    return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

// Device address of the current device's `scratch` array, looked up once per
// device (with that device current) and kept.
void* g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

int scratch_address(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return GEMM_ERR_UNSUPPORTED;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return GEMM_ERR_LAUNCH;
        }
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return GEMM_OK;
}

// ---------------------------------------------------------------------------
// Dynamic tile schedule (gemm_bf16_dynamic).
// ---------------------------------------------------------------------------

constexpr size_t kDynWorkspace = 1024;  // 8 counters, 128 bytes apart

int dynamic_dispatch(bool nt, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                     int64_t ldb, float* C, int64_t ldc, void* ws, size_t ws_bytes, void* stream) {
    if (ws == nullptr || ws_bytes < kDynWorkspace || ((uintptr_t)ws & 15)) return GEMM_ERR_INVALID_ARG;
    int rc = check_common(M, N, K, A, lda, B, ldb, nt ? K : N, C, ldc);
    if (rc == 1) return GEMM_OK;
    if (rc != GEMM_OK) return rc;
    DeviceInfo dev;
    rc = device_info(&dev);
    if (rc != GEMM_OK) return rc;
    if (K > 0 && use_big_tiles(M, N, dev.cus) && c_ok(ldc) &&
        fast_ok(nt ? fast::kNT : fast::kNN, M, N, K, A, lda, B, ldb, nullptr, nullptr)) {
        fast::Args a = make_fast_args(M, N, K, A, lda, B, ldb, C, ldc, 2, kPlain);
        a.tile_ctr = (int*)ws;
        hipStream_t s = (hipStream_t)stream;
        const int g = env_variant().group;
        return nt ? launch_bf16_16<fast::kNT, false, false, true>(a, dev.cus, s, g)
                  : launch_bf16_16<fast::kNN, false, false, true>(a, dev.cus, s, g);
    }
    return bf16_dispatch(nt, M, N, K, A, lda, B, ldb, C, ldc, kPlain, stream);
}

// Epilogue parameters of a fused call; GEMM_ERR_INVALID_ARG for an unknown
// output type or a C pointer not aligned to its element.  fp32 output with
// no vectors is the plain store (the lean kernel instances).
int fused_params(int out_type, const void* C, const float* rs, const float* cs, const float* bias,
                 epi::Params* e) {
    if (out_type != GEMM_OUT_F32 && out_type != GEMM_OUT_BF16 && out_type != GEMM_OUT_E4M3)
        return GEMM_ERR_INVALID_ARG;
    if (((uintptr_t)C) & (out_type == GEMM_OUT_F32 ? 3 : out_type == GEMM_OUT_BF16 ? 1 : 0))
        return GEMM_ERR_INVALID_ARG;
    e->rs = rs;
    e->cs = cs;
    e->bias = bias;
    e->out = out_type;
    e->on = (out_type != GEMM_OUT_F32 || rs || cs || bias) ? 1 : 0;
    return GEMM_OK;
}


int mx_dispatch(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                int64_t ldb, const uint8_t* scaleA, const uint8_t* scaleB, void* C, int64_t ldc,
                const epi::Params& e, void* stream) {
    int rc = check_common(M, N, K, A, lda, B, ldb, K, C, ldc);
    if (rc == 1) return GEMM_OK;
    if (rc != GEMM_OK) return rc;
    if (K % 32 != 0) return GEMM_ERR_INVALID_ARG;
    if (K > 0 && (scaleA == nullptr || scaleB == nullptr)) return GEMM_ERR_INVALID_ARG;
    DeviceInfo dev;
    rc = device_info(&dev);
    if (rc != GEMM_OK) return rc;
    hipStream_t s = (hipStream_t)stream;
    if (K == 0) return zero_fill(C, ldc, M, N, e, s);
    Args a = make_args(M, N, K, A, lda, B, ldb, C, ldc, 128, e);
    a.SA = scaleA;
    a.SB = scaleB;
    a.sld = (int)(K / 32);
    if (use_big_tiles(M, N, dev.cus) && c_ok(ldc) && fast_ok(fast::kMX, M, N, K, A, lda, B, ldb, scaleA, scaleB)) {
        fast::Args f = make_fast_args(M, N, K, A, lda, B, ldb, C, ldc, 1, e);
        f.SA = scaleA;
        f.SB = scaleB;
        f.sld = (int)(K / 32);
        const FastVariant v = env_variant();
        const uintptr_t sal = ((uintptr_t)scaleA) | ((uintptr_t)scaleB);
        // scale ring: one 16-byte load per row per 4 k-tiles of 128 codes
        const bool ring = (K % 512 == 0) && !(sal & 15);
        const bool word_scales = (K % 128 == 0) && !(sal & 3);
        if (e.on) {
            if (ring) return launch_fast<fast::kMX, 128, 2, 4, 12, 0, 4, true>(f, dev.cus, s, v.group);
            if (word_scales) return launch_fast<fast::kMX, 128, 2, 1, 0, 0, 4, true>(f, dev.cus, s, v.group);
            return launch_fast<fast::kMX, 64, 4, 1, 0, 0, 4, true>(f, dev.cus, s, v.group);
        }
#ifdef LIBGEMM_MEASURE
        if (v.rb == 64 && v.stages == 4) return launch_fast<fast::kMX, 64, 4>(f, dev.cus, s, v.group);
        if (ring && v.early == 0) return launch_fast<fast::kMX, 128, 2, 4>(f, dev.cus, s, v.group);
        if (word_scales && v.rb == 128 && v.stages == 2) return launch_fast<fast::kMX, 128, 2>(f, dev.cus, s, v.group);
#endif
        if (ring) {
            // default: 12 of the 16 DMA instructions of k-tile t+2 right
            // after the barrier of k-tile t (MI355X, 8192^3, same box:
            // 491.5 -> 427.4 us)
            return launch_fast<fast::kMX, 128, 2, 4, 12>(f, dev.cus, s, v.group);
        }
        if (word_scales) return launch_fast<fast::kMX, 128, 2>(f, dev.cus, s, v.group);
        return launch_fast<fast::kMX, 64, 4>(f, dev.cus, s, v.group);
    }
    const bool direct = aligned16(A) && aligned16(B) && (lda % 16 == 0) && (ldb % 16 == 0);
    if (use_big_tiles(M, N, dev.cus))
        return direct ? launch<256, 256, kMx, true>(a, dev.cus, s)
                      : launch<256, 256, kMx, false>(a, dev.cus, s);
    return direct ? launch<128, 128, kMx, true>(a, dev.cus, s)
                  : launch<128, 128, kMx, false>(a, dev.cus, s);
}

// ---------------------------------------------------------------------------
// MX split-K: the K ranges of the scale-ring pipeline (ranges a multiple of
// 1024, so that every range starts on a 16-byte boundary of the scale rows
// and runs whole rounds of the unrolled K loop).
// ---------------------------------------------------------------------------

// The plan of gemm_mxfp8_splitk: splits only when the 256 x 256 tiles give the
// CUs less than 3/4 of a round (as the bf16 plan), into about CUs / tiles
// ranges of at least 1024, at most kMaxSplits; the operands must suit the
// scale-ring pipeline (16-byte aligned operands and scales, rows 16-byte
// aligned, K a multiple of 512) and C's planes 32-bit offsets.  Products
// the plan leaves whole run as gemm_mxfp8_fused.
SplitPlan plan_split_mx(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                        const void* SA, const void* SB, int cus, int requested) {
    SplitPlan p{kSplitNone, 1, K, 0, 0, 32};
    const uintptr_t sal = ((uintptr_t)SA) | ((uintptr_t)SB);
    if (K <= 0 || K % 512 || (sal & 15) || !c_ok(N) || !fast_ok(fast::kMX, M, N, K, A, lda, B, ldb, SA, SB))
        return p;
    p.kernel = kSplitFast;
    // ranges of whole scale-ring rounds (8 k-tiles of 128): the pipeline runs
    // a multiple of 8 k-tiles, so a shorter remainder would be dead k-tiles
    constexpr int64_t gran = 1024;
    int64_t want = requested;
    if (want <= 0) {
        const int64_t units = ((M + 255) / 256) * ((N + 255) / 256);
        if (units * 4 >= (int64_t)cus * 3) return p;
        want = cus / units;
        if (want > K / 1024) want = K / 1024;
    }
    if (want > kMaxSplits) want = kMaxSplits;
    if (want <= 1) return p;
    int64_t kslice = (K + want - 1) / want;
    kslice = (kslice + gran - 1) / gran * gran;
    const int64_t splits = (K + kslice - 1) / kslice;
    if (splits <= 1) return p;
    p.splits = (int)splits;
    p.kslice = kslice;
    return p;
}

int mx_splitk_dispatch(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                       const uint8_t* SA, const uint8_t* SB, void* C, int64_t ldc, const epi::Params& e, int splits,
                       void* ws, size_t ws_bytes, void* stream) {
    if (splits < 0) return GEMM_ERR_INVALID_ARG;
    int rc = check_common(M, N, K, A, lda, B, ldb, K, C, ldc);
    if (rc == 1) return GEMM_OK;
    if (rc != GEMM_OK) return rc;
    if (K % 32 != 0) return GEMM_ERR_INVALID_ARG;
    if (K > 0 && (SA == nullptr || SB == nullptr)) return GEMM_ERR_INVALID_ARG;
    DeviceInfo dev;
    rc = device_info(&dev);
    if (rc != GEMM_OK) return rc;
    const SplitPlan p = plan_split_mx(M, N, K, A, lda, B, ldb, SA, SB, dev.cus, splits);
    if (p.splits <= 1) return mx_dispatch(M, N, K, A, lda, B, ldb, SA, SB, C, ldc, e, stream);
    const int64_t need = plan_bytes(p, M, N);
    if (ws == nullptr || (int64_t)ws_bytes < need || ((uintptr_t)ws & 15)) return GEMM_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    fast::Args f = make_fast_args(M, N, K, A, lda, B, ldb, ws, N, 1, kPlain);
    f.SA = SA;
    f.SB = SB;
    f.sld = (int)(K / 32);
    f.kslice = (int)p.kslice;
    f.c_pol = fast::kCStoreCached;  // the partial sums are read back at once
    rc = launch_fast<fast::kMX, 128, 2, 4, 12, 0, 4, false, true>(f, dev.cus, s, env_variant().group, p.splits);
    if (rc != GEMM_OK) return rc;
    int64_t blocks = (M * N / 4 + 255) / 256;
    if (blocks > (int64_t)dev.cus * 8) blocks = (int64_t)dev.cus * 8;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const float*)ws, p.splits,
                       (int)M, (int)N, C, ldc, e);
    return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int gemm_bf16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
              int64_t ldb, float* C, int64_t ldc, void* stream) {
    return bf16_dispatch(false, M, N, K, A, lda, B, ldb, C, ldc, kPlain, stream);
}

int gemm_bf16_nt(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                 int64_t ldb, float* C, int64_t ldc, void* stream) {
    return bf16_dispatch(true, M, N, K, A, lda, B, ldb, C, ldc, kPlain, stream);
}

int gemm_mxfp8(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
               int64_t ldb, const uint8_t* scaleA, const uint8_t* scaleB, float* C, int64_t ldc,
               void* stream) {
    return mx_dispatch(M, N, K, A, lda, B, ldb, scaleA, scaleB, C, ldc, kPlain, stream);
}

int gemm_bf16_fused(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                    int b_colmajor, void* C, int64_t ldc, int out_type, const float* row_scale,
                    const float* col_scale, const float* bias, void* stream) {
    epi::Params e;
    const int rc = fused_params(out_type, C, row_scale, col_scale, bias, &e);
    if (rc != GEMM_OK) return rc;
    return bf16_dispatch(b_colmajor != 0, M, N, K, A, lda, B, ldb, C, ldc, e, stream);
}

int gemm_mxfp8_fused(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                     const uint8_t* scaleA, const uint8_t* scaleB, void* C, int64_t ldc, int out_type,
                     const float* row_scale, const float* col_scale, const float* bias, void* stream) {
    epi::Params e;
    const int rc = fused_params(out_type, C, row_scale, col_scale, bias, &e);
    if (rc != GEMM_OK) return rc;
    return mx_dispatch(M, N, K, A, lda, B, ldb, scaleA, scaleB, C, ldc, e, stream);
}

int gemm_bf16_splitk(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                     int b_colmajor, void* C, int64_t ldc, int out_type, const float* row_scale,
                     const float* col_scale, const float* bias, int splits, void* workspace,
                     size_t workspace_bytes, void* stream) {
    epi::Params e;
    const int rc = fused_params(out_type, C, row_scale, col_scale, bias, &e);
    if (rc != GEMM_OK) return rc;
    return splitk_dispatch(b_colmajor != 0, M, N, K, A, lda, B, ldb, C, ldc, e, splits, workspace,
                           workspace_bytes, stream);
}

int gemm_bf16_dynamic(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                      int b_colmajor, float* C, int64_t ldc, void* workspace, size_t workspace_bytes,
                      void* stream) {
    return dynamic_dispatch(b_colmajor != 0, M, N, K, A, lda, B, ldb, C, ldc, workspace, workspace_bytes, stream);
}

int gemm_bf16_splitk_plan(int64_t M, int64_t N, int64_t K, int b_colmajor, int splits, int cus,
                          int* splits_used, size_t* workspace_bytes) {
    if (M < 0 || N < 0 || K < 0 || splits < 0 || cus < 0 || M > INT32_MAX || N > INT32_MAX || K > INT32_MAX)
        return GEMM_ERR_INVALID_ARG;
    if (cus == 0) {
        DeviceInfo dev;
        const int rc = device_info(&dev);
        if (rc != GEMM_OK) return rc;
        cus = dev.cus;
    }
    const bool nt = b_colmajor != 0;
    // operands assumed 16-byte aligned with dense leading dimensions
    SplitPlan p{kSplitNone, 1, K, 0, 0, 32};
    if (M > 0 && N > 0) p = plan_split(nt, M, N, K, true, K, nt ? K : N, cus, splits);
    if (splits_used) *splits_used = p.splits;
    if (workspace_bytes) *workspace_bytes = (size_t)plan_bytes(p, M, N);
    return GEMM_OK;
}

int gemm_bf16_splitk_noalloc(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                              int64_t ldb, int b_colmajor, void* C, int64_t ldc, int out_type,
                              const float* row_scale, const float* col_scale, const float* bias, int splits,
                              void* stream) {
    epi::Params e;
    int rc = fused_params(out_type, C, row_scale, col_scale, bias, &e);
    if (rc != GEMM_OK) return rc;
    if (splits < 0) return GEMM_ERR_INVALID_ARG;
    const bool nt = b_colmajor != 0;
    rc = check_common(M, N, K, A, lda, B, ldb, nt ? K : N, C, ldc);
    if (rc == 1) return GEMM_OK;
    if (rc != GEMM_OK) return rc;
    DeviceInfo dev;
    rc = device_info(&dev);
    if (rc != GEMM_OK) return rc;
    const SplitPlan p = resolve_split(nt, M, N, K, A, lda, B, ldb, ldc, e, dev.cus, splits);
    // the same plan as gemm_bf16_splitk: unsplit products need no scratch
    if (p.splits <= 1) return bf16_dispatch(nt, M, N, K, A, lda, B, ldb, C, ldc, e, stream);
    if (plan_bytes(p, M, N) > (int64_t)GEMM_SCRATCH_BYTES) return GEMM_ERR_SCRATCH;
    void* ws = nullptr;
    rc = scratch_address(&ws);
    if (rc != GEMM_OK) return rc;
    return splitk_dispatch(nt, M, N, K, A, lda, B, ldb, C, ldc, e, splits, ws, GEMM_SCRATCH_BYTES, stream);
}

int gemm_mxfp8_splitk(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                      const uint8_t* scaleA, const uint8_t* scaleB, void* C, int64_t ldc, int out_type,
                      const float* row_scale, const float* col_scale, const float* bias, int splits,
                      void* workspace, size_t workspace_bytes, void* stream) {
    epi::Params e;
    const int rc = fused_params(out_type, C, row_scale, col_scale, bias, &e);
    if (rc != GEMM_OK) return rc;
    return mx_splitk_dispatch(M, N, K, A, lda, B, ldb, scaleA, scaleB, C, ldc, e, splits, workspace,
                              workspace_bytes, stream);
}

int gemm_mxfp8_splitk_workspace(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                                int64_t ldb, const uint8_t* scaleA, const uint8_t* scaleB, const void* C,
                                int64_t ldc, int out_type, const float* row_scale, const float* col_scale,
                                const float* bias, int splits, int cus, int* splits_used, size_t* workspace_bytes) {
    epi::Params e;
    int rc = fused_params(out_type, C, row_scale, col_scale, bias, &e);
    if (rc != GEMM_OK) return rc;
    if (splits < 0 || cus < 0) return GEMM_ERR_INVALID_ARG;
    rc = check_common(M, N, K, A, lda, B, ldb, K, C, ldc);
    SplitPlan p{kSplitNone, 1, K, 0, 0, 32};
    if (rc != 1) {
        if (rc != GEMM_OK) return rc;
        if (K % 32 != 0) return GEMM_ERR_INVALID_ARG;
        if (K > 0 && (scaleA == nullptr || scaleB == nullptr)) return GEMM_ERR_INVALID_ARG;
        if (cus == 0) {
            DeviceInfo dev;
            rc = device_info(&dev);
            if (rc != GEMM_OK) return rc;
            cus = dev.cus;
        }
        p = plan_split_mx(M, N, K, A, lda, B, ldb, scaleA, scaleB, cus, splits);
    }
    if (splits_used) *splits_used = p.splits;
    if (workspace_bytes) *workspace_bytes = (size_t)plan_bytes(p, M, N);
    return GEMM_OK;
}

int gemm_bf16_splitk_workspace(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                                int64_t ldb, int b_colmajor, const void* C, int64_t ldc, int out_type,
                                const float* row_scale, const float* col_scale, const float* bias, int splits,
                                int cus, int* splits_used, size_t* workspace_bytes) {
    epi::Params e;
    int rc = fused_params(out_type, C, row_scale, col_scale, bias, &e);
    if (rc != GEMM_OK) return rc;
    if (splits < 0 || cus < 0) return GEMM_ERR_INVALID_ARG;
    const bool nt = b_colmajor != 0;
    rc = check_common(M, N, K, A, lda, B, ldb, nt ? K : N, C, ldc);
    SplitPlan p{kSplitNone, 1, K, 0, 0, 32};
    if (rc != 1) {
        if (rc != GEMM_OK) return rc;
        if (cus == 0) {
            DeviceInfo dev;
            rc = device_info(&dev);
            if (rc != GEMM_OK) return rc;
            cus = dev.cus;
        }
        p = resolve_split(nt, M, N, K, A, lda, B, ldb, ldc, e, cus, splits);
    }
    if (splits_used) *splits_used = p.splits;
    if (workspace_bytes) *workspace_bytes = (size_t)plan_bytes(p, M, N);
    return GEMM_OK;
}

const char* gemm_strerror(int code) {
    switch (code) {
        case GEMM_OK: return "success";
        case GEMM_ERR_INVALID_ARG:
            return "invalid argument (size, leading dimension or stride, pointer, alignment, output type, "
                   "head dimension or scale)";
        case GEMM_ERR_UNSUPPORTED: return "unsupported device (a gfx950 GPU is required)";
        case GEMM_ERR_LAUNCH: return "kernel launch failed";
        case GEMM_ERR_SCRATCH:
            return "the split plan needs more than the library's fixed scratch (GEMM_SCRATCH_BYTES); use "
                   "gemm_bf16_splitk with a workspace, or ask for fewer K ranges";
        default: return "unknown error code";
    }
}

int gemm_version(void) { return 301; }

}  // extern "C"
