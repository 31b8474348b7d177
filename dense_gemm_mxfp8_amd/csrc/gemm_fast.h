// gemm_fast.h -- the aligned fast path of the gfx950 GEMM kernels.
//
// One workgroup of 4 waves owns a 256 x 256 output tile at a time (a 2 x 2
// arrangement of 128 x 128 wave tiles, 256 fp32 accumulators per lane in the
// AGPR file) and walks a persistent, XCD-aware sequence of tiles.  The K loop
// streams k-tiles of RB bytes per operand row (RB = 128: 64 bf16 or 128 fp8;
// RB = 64: 32 bf16) through S LDS stages:
//
//   * global -> LDS: `buffer_load_dwordx4 ... lds` against a per-tile buffer
//     descriptor.  Every wave instruction fills 1 KiB of LDS; lane i lands at
//     byte 16 i and fetches the global 16-byte chunk that the swizzle places
//     there.  Rows past M (or N) lie beyond the descriptor's size and read as
//     zero, so the tails need no predicates on the load side.
//   * LDS layout: each operand row holds RB bytes of K; its 16-byte chunks
//     are XOR-swizzled with bits of the row index chosen for gfx950's
//     64-bank LDS (16 lanes of a 128-bit read are served per clock, so any
//     16 consecutive rows must spread one logical chunk over all 16
//     bank groups of 256 bytes).
//   * Row-major B ("NN") is staged N-contiguous (k rows of 512 bytes) and
//     read with `ds_read_b64_tr_b16`, which transposes 4 x 16 bf16 blocks on
//     the way into registers.
//   * k-tile t + S - 1 is issued while k-tile t is multiplied; one barrier
//     per k-tile hands a stage from the loaders to the readers, the role the
//     pages give to mbarrier phases.  Every stage is its own __shared__
//     object and the K loop is unrolled by S, so the compiler can tell the
//     in-flight DMA writes of later stages apart from the reads of the
//     current one and does not serialise them.
//   * matrix cores: bf16 instances run v_mfma_f32_16x16x32_bf16 over the
//     wave tile as 8 x 8 blocks in Z order (MF = 16) or
//     v_mfma_f32_32x32x16_bf16 as 4 x 4 blocks (MF = 32); MX runs
//     v_mfma_scale_f32_32x32x64_f8f6f4.  The fragments are double-buffered
//     across k-steps: the LDS reads of step s + 1 are in flight while step
//     s's MFMAs run.
//   * the last, partial k-tile (K mod BK != 0) is loaded through registers
//     with buffer loads, its bytes past K zeroed.
//   * epilogue: buffer stores straight from the accumulators (store_c,
//     store_c16), fp32 or through the fused epilogue of gemm_epi.h.
//
// Fast-path preconditions (checked on the host): 16-byte aligned A and B,
// leading dimensions that keep every row 16-byte aligned, 256 rows of either
// operand spanning less than 2 GiB, and for row-major B, N % 8 == 0.  The MX
// variant also needs K % 64 == 0 and 2-byte aligned scales.

#pragma once

#include <type_traits>
#include <utility>

#include "gemm_epi.h"

namespace fast {

constexpr int kTile = 256;      // BM = BN
constexpr int kThreads = 256;   // 4 waves in a 2 x 2 arrangement
constexpr int kWaves = 4;
constexpr int kWaveTile = 128;  // each wave: 128 x 128 outputs
constexpr int kBlocks = 4;      // 32 x 32 MFMA blocks per wave tile side
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

enum Kind { kNT = 0, kNN = 1, kMX = 2 };

// Cache policies of the C stores (Args::c_pol) and their buffer-instruction
// cache-policy bits on gfx950: non-temporal, and device scope (sc1).
constexpr int kCStoreCached = 0, kCStoreStream = 1, kCStoreDevice = 2;
constexpr int kAuxStream = 2, kAuxDevice = 16;

struct Args {
    const uint8_t* A;
    const uint8_t* B;
    float* C;
    const uint8_t* SA;
    const uint8_t* SB;
    int64_t lda_b, ldb_b;  // leading dimensions in bytes
    int64_t ldc;           // elements
    int M, N, K;
    int tiles_m, tiles_n, num_tiles, group_m;
    int kt_total;  // number of k-tiles, the last one possibly partial
    int kt_full;   // number of k-tiles lying entirely inside K
    int sld;       // MX scale bytes per row (K / 32)
    int xcd_remap;
    int c_pol;     // cache policy of the C stores: kCStoreCached, kCStoreStream or kCStoreDevice
    epi::Params epi;  // fused epilogue (C holds epi.out elements)
    // split-K instances: units 0 .. dp_units-1 are whole tiles 0 .. dp_units-1
    // (stored to C); unit dp_units + u is tile tile0 + u % tiles_per_split of
    // K range ks = u / tiles_per_split ([ks kslice, min(K, (ks + 1) kslice)),
    // kslice a multiple of the k-tile).  Its fp32 partial sums go either to
    // rows ks M .. of C (part == null: stacked dense M x N planes) or to the
    // 256 x 256 block (ks tiles_per_split + u % tiles_per_split) of `part`.
    int tiles_per_split, kslice, dp_units, tile0;
    float* part;
    // dynamic-schedule instances: 8 tile counters, one per XCD, 32 ints
    // apart (zero when the launch starts)
    int* tile_ctr;
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

#define FAST_LDS __attribute__((address_space(3)))

// s_waitcnt encodings (gfx9): vmcnt in [3:0] and [15:14], expcnt [6:4],
// lgkmcnt [11:8].
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4)); }

// Barrier that keeps the compiler from moving memory operations across it,
// without the workgroup fence of __syncthreads (whose release would wait for
// every outstanding global load, including the stages still in flight).
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Swizzle of 16-byte chunk columns for K-contiguous rows of RB bytes.
template <int RB>
__device__ __forceinline__ int swz(int row) {
    if constexpr (RB == 128) return (row >> 1) & 7;
    else return (row >> 2) & 3;
}

// Byte offset of chunk `chunk` of K-contiguous row `row`.
template <int RB>
__device__ __forceinline__ int kc_off(int row, int chunk) {
    return row * RB + ((chunk ^ swz<RB>(row)) << 4);
}

// Swizzle of the 16-byte chunks of k-row k of row-major B: bits 0..1 of k
// select chunk groups 4 apart (the four k-rows a 16-lane transposed read
// spans), bit 3 moves odd 8-row bands by 2 chunks (the 16 x 16 x 32 MFMA's
// B fragment puts k-rows 8 g .. 8 g + 3 in lane group g, so two groups of a
// 32-lane read phase read rows 8 apart at the same columns).
__device__ __forceinline__ int nn_swz(int k) { return ((k & 3) << 2) | (((k >> 3) & 1) << 1); }

// Byte offset of element column n of k-row k in the N-contiguous stage of
// row-major B (512-byte rows of 256 bf16).
__device__ __forceinline__ int nn_off(int k, int n) {
    return k * 512 + ((((n >> 3) ^ nn_swz(k))) << 4) + ((n & 7) << 1);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    int n = bytes > 0x7fffffff ? 0x7fffffff : (int)bytes;
    if (n < 0) n = 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kRsrcWord3);
}

__device__ __forceinline__ int logical_block(const Args& a) {
    int bid = blockIdx.x;
    if (!a.xcd_remap) return bid;
    // Workgroups are dispatched round-robin over the 8 XCDs; renumber them
    // so that consecutive logical ids (neighbouring tiles) share an XCD and
    // its L2.
    int per_xcd = gridDim.x >> 3;
    return (bid & 7) * per_xcd + (bid >> 3);
}

// Grouped raster: tiles are walked in column-major order inside bands of
// group_m tile rows, so concurrently running tiles share A rows and B columns.
__device__ __forceinline__ void tile_coords(const Args& a, int t, int& tm, int& tn) {
    int per_group = a.group_m * a.tiles_n;
    int g = t / per_group;
    int first = g * a.group_m;
    int gsz = min(a.tiles_m - first, a.group_m);
    int r = t - g * per_group;
    tm = first + r % gsz;
    tn = r / gsz;
}

// Dynamic schedule (the atomic tile counter): tile number of position idx in
// XCD x's queue.  The static walk gives the workgroups on XCD x (grid G,
// P = G / 8 per XCD) the tiles r G + x P + j of every round r; the dynamic
// walk keeps that split into 8 per-XCD queues, so neighbouring tiles still
// share an L2, but hands the positions out through a counter per queue.
// Round 0 (idx < P) is each workgroup's first tile, taken without a counter.
__device__ __forceinline__ int queue_tile(int x, int idx, int P, int G) {
    return (idx / P) * G + x * P + idx % P;
}

// The next tile of a workgroup on XCD x whose own queue handed it position
// idx: that tile if it exists, else one taken from the other XCDs' queues in
// turn (work stealing), else num_tiles (every queue is empty).  Positions
// grow with each grab and tile numbers grow with positions, so a tile past
// the end means the queue is exhausted.
__device__ __forceinline__ int next_tile(const Args& a, int x, int idx, int P, int G) {
    int t = queue_tile(x, idx, P, G);
    if (t < a.num_tiles) return t;
    for (int q = 1; q < 8; ++q) {
        const int xq = (x + q) & 7;
        t = queue_tile(xq, P + atomicAdd(a.tile_ctr + 32 * xq, 1), P, G);
        if (t < a.num_tiles) return t;
    }
    return a.num_tiles;
}

// Number of bytes rounded up to whole dwords (buffer range checks work on
// dwords: a range ending inside the last valid element's dword would drop it).
__device__ __forceinline__ int64_t round4(int64_t bytes) { return (bytes + 3) & ~(int64_t)3; }

// Keep the first nb bytes (0 .. 16) of a 16-byte chunk, zero the rest.
// Branch-free: dword w keeps min(max(nb - 4 w, 0), 4) bytes, through the
// mask 2^(8 b) - 1 formed in 64 bits (b = 4 gives all ones, b = 0 none).
__device__ __forceinline__ i32x4 keep_bytes(i32x4 v, int nb) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const int b = min(max(nb - 4 * w, 0), 4);
        const uint32_t m = (uint32_t)((1ull << (8 * b)) - 1ull);
        v[w] = (int)((uint32_t)v[w] & m);
    }
    return v;
}

// Partial last k-tile of a K-contiguous operand (256 rows x RB bytes) into
// a stage: buffer loads at byte soff of each row through `rs` (rows past the
// operand lie outside it and read as zero), bytes at or past kvalid_b zeroed.
// The rows are 16-byte aligned, so the loads read aligned dwords and a range
// rounded up to a dword touches nothing past the operand's last dword.  Every
// chunk is loaded, past K too (inside a row that is the row's padding or the
// next row, inside the descriptor either way; past the descriptor, zero),
// and masked afterwards: with the loads under per-lane branches the compiler
// waited for each one in turn, a full memory round trip per chunk.
template <int RB, int THREADS = kThreads>
__device__ __forceinline__ void tail_kc(uint8_t FAST_LDS* dst, __amdgpu_buffer_rsrc_t rs, int ld_b, int soff,
                                        int kvalid_b, int tid) {
    constexpr int CPR = RB / 16;
    constexpr int NI = kTile * CPR / THREADS;
    // the offsets below are invariant over the persistent tile loop; hoisted
    // out of it they would stay live through the K loop and spill
    asm volatile("" : "+v"(tid));
    i32x4 v[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int idx = i * THREADS + tid;
        const int r = idx / CPR, c = idx % CPR;
        v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, r * ld_b + c * 16, soff, 0);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int idx = i * THREADS + tid;
        const int r = idx / CPR, c = idx % CPR;
        *(i32x4 FAST_LDS*)(dst + kc_off<RB>(r, c)) = keep_bytes(v[i], kvalid_b - c * 16);
    }
}

// Partial k-tile of row-major B (k rows of 256 bf16) into a stage: k-rows at
// or past kvalid and 8-column chunks at or past ncols are zero (N % 8 == 0,
// so a chunk is either wholly inside N or wholly outside).  Loaded
// unconditionally and masked afterwards, as tail_kc (k-rows past the data
// lie outside the descriptor; chunks past N inside a row are the padding or
// the next row).
template <int BK, int THREADS = kThreads>
__device__ __forceinline__ void tail_nn(uint8_t FAST_LDS* dst, __amdgpu_buffer_rsrc_t rs, int ldb_b, int soff,
                                        int kvalid, int ncols, int tid) {
    constexpr int NI = BK * 32 / THREADS;
    asm volatile("" : "+v"(tid));  // keep the offsets inside the tile loop (as tail_kc)
    i32x4 v[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int idx = i * THREADS + tid;
        const int kk = idx >> 5, c = idx & 31;
        v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, kk * ldb_b + c * 16, soff, 0);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int idx = i * THREADS + tid;
        const int kk = idx >> 5, c = idx & 31;
        const bool keep = kk < kvalid && c * 8 < ncols;
        i32x4 z = {0, 0, 0, 0};
        *(i32x4 FAST_LDS*)(dst + nn_off(kk, c * 8)) = keep ? v[i] : z;
    }
}

// Epilogue of one wave: its 128 x 128 fp32 accumulators to C at rows
// m0w.., columns n0w..  Accumulator register r of block (i, j) holds
// C[32 i + 8 (r / 4) + 4 h + r % 4][32 j + l32].  Buffer stores against a
// descriptor that ends at the wave tile's last element inside C: rows past M
// fall outside it and are dropped by the hardware, columns past N are
// predicated (one branch per 32-column block).  Offsets are 32-bit (the
// host keeps 256 rows of C below 2 GiB), so no 64-bit address per element
// is formed.  With whole 128-byte lines per 32-column segment the stores are
// non-temporal (C is written once and never read back, so it should not
// evict operand lines from L2 and the Infinity Cache); otherwise they are
// cached so that L2 merges the two halves of each line.
// AT: cw is where output (m0w, n0w) goes and ldc its row pitch in floats
// (a split-K partial); otherwise C at (m0w, n0w) with pitch a.ldc.
template <int AUX, int NBJ, bool AT = false>
__device__ __forceinline__ void store_c_aux(const Args& a, const f32x16 (&acc)[kBlocks][NBJ], int m0w, int n0w,
                                            int h, int l32, float* cw = nullptr, int ldc = 0) {
    const int rlim = a.M - m0w;
    const int clim = a.N - n0w;
    if (rlim <= 0 || clim <= 0) return;
    const int rows = rlim < kWaveTile ? rlim : kWaveTile;
    const int cols = clim < 32 * NBJ ? clim : 32 * NBJ;
    const int ldc4 = (int)(AT ? ldc : a.ldc) * 4;
    const __amdgpu_buffer_rsrc_t rc =
        AT ? make_rsrc(cw, ((int64_t)(rows - 1) * ldc + cols) * 4)
           : make_rsrc(a.C + (int64_t)m0w * a.ldc + n0w, ((int64_t)(rows - 1) * a.ldc + cols) * 4);
    const int voff = 4 * h * ldc4 + 4 * l32;
#pragma unroll
    for (int j = 0; j < NBJ; ++j) {
        if (32 * j + l32 < cols) {
#pragma unroll
            for (int i = 0; i < kBlocks; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 32 * i + 8 * (r >> 2) + (r & 3);
                    // copy the element out first: a bit cast applied to a
                    // vector element directly is compiled as one of element 0
                    const float v = acc[i][j][r];
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rc, voff + 128 * j,
                                                          row * ldc4, AUX);
                }
        }
    }
}

// Fused epilogue (gemm_epi.h): t = acc * rs[row] * cs[col] + bias[col] in
// fp32, stored as fp32, bf16 or E4M3 (OUT), with the descriptor scheme of
// store_c_aux.
// The tile's scale and bias values were loaded into registers when the tile
// started (epi_prefetch) and staged in LDS before the epilogue (epi_stage),
// so no global load latency shows here: ev points at 3 x 256 floats (row
// scales, column scales, biases of the tile), evr / evc are this wave's
// first row / column within the tile.
template <int AUX, int NBJ, int OUT>
__device__ __forceinline__ void store_c_fused(const Args& a, const f32x16 (&acc)[kBlocks][NBJ], int m0w, int n0w,
                                              int h, int l32, const float FAST_LDS* ev, int evr, int evc) {
    const int rlim = a.M - m0w;
    const int clim = a.N - n0w;
    if (rlim <= 0 || clim <= 0) return;
    const int rows = rlim < kWaveTile ? rlim : kWaveTile;
    const int cols = clim < 32 * NBJ ? clim : 32 * NBJ;
    constexpr int ESZ = OUT == epi::kF32 ? 4 : OUT == epi::kBF16 ? 2 : 1;
    const int ldcb = (int)a.ldc * ESZ;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc((const uint8_t*)a.C + ((int64_t)m0w * a.ldc + n0w) * ESZ,
                                                ((int64_t)(rows - 1) * a.ldc + cols) * ESZ);
    const int voff = 4 * h * ldcb + ESZ * l32;
    const bool has_r = a.epi.rs != nullptr, has_c = a.epi.cs != nullptr, has_b = a.epi.bias != nullptr;
    float cf[NBJ], cb[NBJ];
#pragma unroll
    for (int j = 0; j < NBJ; ++j) {
        cf[j] = ev[256 + evc + 32 * j + l32];
        cb[j] = ev[512 + evc + 32 * j + l32];
    }
#pragma unroll
    for (int i = 0; i < kBlocks; ++i) {
        float rf[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) rf[r] = ev[evr + 32 * i + 8 * (r >> 2) + (r & 3) + 4 * h];
#pragma unroll
        for (int j = 0; j < NBJ; ++j) {
            if (32 * j + l32 < cols) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 32 * i + 8 * (r >> 2) + (r & 3);
                    float t = acc[i][j][r];
                    if (has_r) t *= rf[r];
                    if (has_c) t *= cf[j];
                    if (has_b) t += cb[j];
                    if constexpr (OUT == epi::kBF16)
                        __builtin_amdgcn_raw_buffer_store_b16(epi::to_bf16(t), rc, voff + 64 * j, row * ldcb, AUX);
                    else if constexpr (OUT == epi::kE4M3)
                        __builtin_amdgcn_raw_buffer_store_b8(epi::to_e4m3(t), rc, voff + 32 * j, row * ldcb, AUX);
                    else
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, t), rc, voff + 128 * j,
                                                              row * ldcb, AUX);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The fused epilogue's values for one tile, one row, one column and one bias
// per thread (256 threads cover 256 rows and up to 256 columns), loaded when
// the tile starts so that their latency hides under the K loop.
struct EpiRegs {
    float r, c, b;
};

__device__ __forceinline__ EpiRegs epi_prefetch(const Args& a, int m0, int n0, int bn, int tid) {
    EpiRegs v{1.0f, 1.0f, 0.0f};
    const epi::Params& e = a.epi;
    if (e.rs && m0 + tid < a.M) v.r = e.rs[m0 + tid];
    if (tid < bn && n0 + tid < a.N) {
        if (e.cs) v.c = e.cs[n0 + tid];
        if (e.bias) v.b = e.bias[n0 + tid];
    }
    return v;
}

__device__ __forceinline__ void epi_stage(float FAST_LDS* ev, const EpiRegs& v, int tid) {
    ev[tid] = v.r;
    ev[256 + tid] = v.c;
    ev[512 + tid] = v.b;
}

// FUSED: the kernel instance carries the fused epilogue (a.epi.on); plain
// instances keep the lean store path.  cw / cld (plain only): where output
// (m0w, n0w) goes and the row pitch there, for a split-K partial (null: C);
// pol: stores to C may take a.c_pol (false: cached, a partial is read back at
// once).  The policies' cache-policy bits: non-temporal (kAuxStream) for C
// whose 32-column segments are whole 128-byte lines, device scope
// (kAuxDevice) where segments share lines, cached otherwise.
template <int NBJ = kBlocks, bool FUSED = false>
__device__ __forceinline__ void store_c(const Args& a, const f32x16 (&acc)[kBlocks][NBJ], int m0w, int n0w, int h,
                                        int l32, const float FAST_LDS* ev = nullptr, int evr = 0, int evc = 0,
                                        float* cw = nullptr, int cld = 0, bool pol = true) {
    if constexpr (FUSED) {
        const bool dev = a.c_pol == kCStoreDevice;
        if (a.epi.out == epi::kBF16) {
            if (dev) store_c_fused<kAuxDevice, NBJ, epi::kBF16>(a, acc, m0w, n0w, h, l32, ev, evr, evc);
            else store_c_fused<0, NBJ, epi::kBF16>(a, acc, m0w, n0w, h, l32, ev, evr, evc);
        } else if (a.epi.out == epi::kE4M3) {
            if (dev) store_c_fused<kAuxDevice, NBJ, epi::kE4M3>(a, acc, m0w, n0w, h, l32, ev, evr, evc);
            else store_c_fused<0, NBJ, epi::kE4M3>(a, acc, m0w, n0w, h, l32, ev, evr, evc);
        } else if (a.c_pol == kCStoreStream) {
            store_c_fused<kAuxStream, NBJ, epi::kF32>(a, acc, m0w, n0w, h, l32, ev, evr, evc);
        } else if (dev) {
            store_c_fused<kAuxDevice, NBJ, epi::kF32>(a, acc, m0w, n0w, h, l32, ev, evr, evc);
        } else {
            store_c_fused<0, NBJ, epi::kF32>(a, acc, m0w, n0w, h, l32, ev, evr, evc);
        }
    } else {
        if (cw != nullptr) store_c_aux<0, NBJ, true>(a, acc, m0w, n0w, h, l32, cw, cld);
        else if (pol && a.c_pol == kCStoreStream) store_c_aux<kAuxStream, NBJ>(a, acc, m0w, n0w, h, l32);
        else if (pol && a.c_pol == kCStoreDevice) store_c_aux<kAuxDevice, NBJ>(a, acc, m0w, n0w, h, l32);
        else store_c_aux<0, NBJ>(a, acc, m0w, n0w, h, l32);
    }
}

// The plain fp32 store of a 128 x 128 wave tile held as 8 x 8 blocks of the
// 16 x 16 MFMA: lane l holds rows 4 (l / 16) + r, r = 0..3, of column l % 16
// of each block.  One v_permlane16_swap per register of two neighbouring
// column blocks leaves, in one register, rows 4 g + r (lanes 0..31, g even)
// of the 32 columns and, in the other, those of the odd g: every store
// instruction then writes two whole 128-byte row segments, as the 32 x 32
// form does, so non-temporal stores still write whole lines.
template <int AUX, bool AT = false, int BB = 8>
__device__ __forceinline__ void store_c16_aux(const Args& a, const f32x4 (&acc)[8][BB], int m0w, int n0w, int lane,
                                              float* cw = nullptr, int cld = 0) {
    const int rlim = a.M - m0w;
    const int clim = a.N - n0w;
    if (rlim <= 0 || clim <= 0) return;
    const int rows = rlim < kWaveTile ? rlim : kWaveTile;
    const int cols = clim < 16 * BB ? clim : 16 * BB;
    const int ldc4 = (int)(AT ? cld : a.ldc) * 4;
    const __amdgpu_buffer_rsrc_t rc =
        AT ? make_rsrc(cw, ((int64_t)(rows - 1) * cld + cols) * 4)
           : make_rsrc(a.C + (int64_t)m0w * a.ldc + n0w, ((int64_t)(rows - 1) * a.ldc + cols) * 4);
    // lanes 32..63 hold the rows 8 below lanes 0..31
    const int voff = ((lane >> 5) * 8) * ldc4 + 4 * (lane & 31);
    // The swap reads other lanes, so it runs with every lane active: a lane
    // whose column lies past the tile's last instead stores at an offset
    // past the descriptor's range (2^31 - 16 plus a row offset below 2^30:
    // no 32-bit wrap), which drops the store.
    constexpr int kOut = 0x7ffffff0;
#pragma unroll
    for (int jp = 0; jp < BB / 2; ++jp) {
        const int vo = (32 * jp + (lane & 31) < cols) ? voff + 128 * jp : kOut;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                // copy the elements out first (a bit cast of a vector
                // element is otherwise compiled as one of element 0)
                const float x = acc[i][2 * jp][r], y = acc[i][2 * jp + 1][r];
                const auto sw = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x),
                                                                 __builtin_bit_cast(uint32_t, y), false, false);
                __builtin_amdgcn_raw_buffer_store_b32(sw[0], rc, vo, (16 * i + r) * ldc4, AUX);
                __builtin_amdgcn_raw_buffer_store_b32(sw[1], rc, vo, (16 * i + 4 + r) * ldc4, AUX);
            }
    }
}

// The fused epilogue (gemm_epi.h) on the 16 x 16 layout: each lane applies
// t = acc * rs[row] * cs[col] + bias[col] to its own elements (rows
// 16 i + 4 (l / 16) + r of column 16 j + l % 16, with the tile's scales and
// biases from their LDS copy ev, as in store_c_fused) and converts them to
// OUT; the permlane16 swap then regroups them as in store_c16_aux, so every
// store instruction writes 32 consecutive columns of two rows.
template <int AUX, int OUT>
__device__ __forceinline__ void store_c16_fused(const Args& a, const f32x4 (&acc)[8][8], int m0w, int n0w, int lane,
                                                const float FAST_LDS* ev, int evr, int evc) {
    const int rlim = a.M - m0w;
    const int clim = a.N - n0w;
    if (rlim <= 0 || clim <= 0) return;
    const int rows = rlim < kWaveTile ? rlim : kWaveTile;
    const int cols = clim < kWaveTile ? clim : kWaveTile;
    constexpr int ESZ = OUT == epi::kF32 ? 4 : OUT == epi::kBF16 ? 2 : 1;
    const int ldcb = (int)a.ldc * ESZ;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc((const uint8_t*)a.C + ((int64_t)m0w * a.ldc + n0w) * ESZ,
                                                ((int64_t)(rows - 1) * a.ldc + cols) * ESZ);
    const int voff = ((lane >> 5) * 8) * ldcb + ESZ * (lane & 31);
    constexpr int kOut = 0x7ffffff0;  // a dropped store, as in store_c16_aux
    const bool has_r = a.epi.rs != nullptr, has_c = a.epi.cs != nullptr, has_b = a.epi.bias != nullptr;
    const int g = lane >> 4, p = lane & 15;
    float cf[8], cb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        cf[j] = ev[256 + evc + 16 * j + p];
        cb[j] = ev[512 + evc + 16 * j + p];
    }
    auto conv = [&](float t, int j, float rf) -> uint32_t {
        if (has_r) t *= rf;
        if (has_c) t *= cf[j];
        if (has_b) t += cb[j];
        if constexpr (OUT == epi::kBF16) return epi::to_bf16(t);
        else if constexpr (OUT == epi::kE4M3) return epi::to_e4m3(t);
        else return __builtin_bit_cast(uint32_t, t);
    };
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float rf[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) rf[r] = ev[evr + 16 * i + 4 * g + r];
#pragma unroll
        for (int jp = 0; jp < 4; ++jp) {
            const int vo = (32 * jp + (lane & 31) < cols) ? voff + 32 * ESZ * jp : kOut;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x = acc[i][2 * jp][r], y = acc[i][2 * jp + 1][r];
                const auto sw = __builtin_amdgcn_permlane16_swap(conv(x, 2 * jp, rf[r]), conv(y, 2 * jp + 1, rf[r]),
                                                                 false, false);
                const int r0 = (16 * i + r) * ldcb, r1 = (16 * i + 4 + r) * ldcb;
                if constexpr (OUT == epi::kBF16) {
                    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)sw[0], rc, vo, r0, AUX);
                    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)sw[1], rc, vo, r1, AUX);
                } else if constexpr (OUT == epi::kE4M3) {
                    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sw[0], rc, vo, r0, AUX);
                    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sw[1], rc, vo, r1, AUX);
                } else {
                    __builtin_amdgcn_raw_buffer_store_b32(sw[0], rc, vo, r0, AUX);
                    __builtin_amdgcn_raw_buffer_store_b32(sw[1], rc, vo, r1, AUX);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The 16 x 16 layout's epilogue.  FUSED: the fused epilogue; cw / cld (plain
// only): a split-K partial's destination and row pitch, stored cached (null:
// C under a.c_pol), as in store_c.
template <bool FUSED = false, int BB = 8>
__device__ __forceinline__ void store_c16(const Args& a, const f32x4 (&acc)[8][BB], int m0w, int n0w, int lane,
                                          const float FAST_LDS* ev = nullptr, int evr = 0, int evc = 0,
                                          float* cw = nullptr, int cld = 0) {
    if constexpr (FUSED) {
        static_assert(BB == 8, "fused epilogue: 128 x 128 wave tiles");
        const bool dev = a.c_pol == kCStoreDevice;
        if (a.epi.out == epi::kBF16) {
            if (dev) store_c16_fused<kAuxDevice, epi::kBF16>(a, acc, m0w, n0w, lane, ev, evr, evc);
            else store_c16_fused<0, epi::kBF16>(a, acc, m0w, n0w, lane, ev, evr, evc);
        } else if (a.epi.out == epi::kE4M3) {
            if (dev) store_c16_fused<kAuxDevice, epi::kE4M3>(a, acc, m0w, n0w, lane, ev, evr, evc);
            else store_c16_fused<0, epi::kE4M3>(a, acc, m0w, n0w, lane, ev, evr, evc);
        } else if (a.c_pol == kCStoreStream) {
            store_c16_fused<kAuxStream, epi::kF32>(a, acc, m0w, n0w, lane, ev, evr, evc);
        } else if (dev) {
            store_c16_fused<kAuxDevice, epi::kF32>(a, acc, m0w, n0w, lane, ev, evr, evc);
        } else {
            store_c16_fused<0, epi::kF32>(a, acc, m0w, n0w, lane, ev, evr, evc);
        }
    } else {
        if (cw != nullptr) store_c16_aux<0, true, BB>(a, acc, m0w, n0w, lane, cw, cld);
        else if (a.c_pol == kCStoreStream) store_c16_aux<kAuxStream, false, BB>(a, acc, m0w, n0w, lane);
        else if (a.c_pol == kCStoreDevice) store_c16_aux<kAuxDevice, false, BB>(a, acc, m0w, n0w, lane);
        else store_c16_aux<0, false, BB>(a, acc, m0w, n0w, lane);
    }
}

// Compile-time loop: f(integral_constant<int, B>), ..., f(integral_constant<int, E-1>).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Instruction-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSgMfma = 0x008;
constexpr int kSgVmem = 0x010;
constexpr int kSgDsRead = 0x100;
constexpr int kSgDsWrite = 0x200;

// Interleave the 16 MFMAs of one k-step with NR LDS fragment reads and ND
// DMA instructions so that memory instructions issue while the matrix core
// is busy instead of in bursts.
template <int NR, int ND, int NMF = 16>
__device__ __forceinline__ void interleave_step() {
#pragma unroll
    for (int m = 0; m < NMF; ++m) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        if (m < NR) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
        if (m < ND) __builtin_amdgcn_sched_group_barrier(kSgVmem, 1, 0);
    }
}

// The 8 x BB MFMAs of a 16 x 16 x 32 k-step visit the 8 x BB blocks of the
// wave tile (BB = 8, or 4 for 128 x 64 wave tiles) in Z order (MFMA m: A
// block z_row(m), B block z_col(m)), so the fragments a k-step needs grow as
// 2 sqrt(m): by MFMA 16 only 4 A and 4 B fragments.  The next step's
// fragments are read in the order of first use (z_frag) into the other
// register set, spread evenly over this step's MFMAs (NRD LDS reads), which
// leaves every read at least 40 MFMAs (of 64) before the one that needs it;
// a row-first order needed all 8 A fragments within the first 8 MFMAs.  The
// ND DMA instructions go after every other MFMA from the first.
template <int BB>
constexpr int z_row(int m) {
    return BB == 8 ? ((m >> 1) & 1) | ((m >> 2) & 2) | ((m >> 3) & 4) : ((m >> 1) & 1) | ((m >> 2) & 6);
}
template <int BB>
constexpr int z_col(int m) {
    return BB == 8 ? (m & 1) | ((m >> 1) & 2) | ((m >> 2) & 4) : (m & 1) | ((m >> 1) & 2);
}
// The o-th fragment in order of first use: A fragments 0..7, B fragments 8..8+BB-1.
template <int BB>
constexpr int z_frag(int o) {
    int seen = 0, n = 0;
    for (int m = 0; m < 8 * BB; ++m) {
        const int f[2] = {z_row<BB>(m), 8 + z_col<BB>(m)};
        for (int x : f) {
            if ((seen >> x) & 1) continue;
            if (n++ == o) return x;
            seen |= 1 << x;
        }
    }
    return -1;
}

// Every block once, and every fragment once in the read order.
template <int BB>
constexpr bool z_order_ok() {
    int blocks[8] = {}, frags = 0;
    for (int m = 0; m < 8 * BB; ++m) {
        const int r = z_row<BB>(m), c = z_col<BB>(m);
        if (r < 0 || r > 7 || c < 0 || c >= BB || ((blocks[r] >> c) & 1)) return false;
        blocks[r] |= 1 << c;
    }
    for (int o = 0; o < 8 + BB; ++o) {
        const int f = z_frag<BB>(o);
        if (f < 0 || f >= 8 + BB || ((frags >> f) & 1)) return false;
        frags |= 1 << f;
    }
    return true;
}
static_assert(z_order_ok<8>() && z_order_ok<4>(), "Z order of the 16 x 16 blocks");

template <int NRD, int ND, int NMF = 64>
__device__ __forceinline__ void interleave_step16() {
    static_for<0, NMF>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        constexpr int nr = ((m + 1) * NRD) / NMF - (m * NRD) / NMF;
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        if constexpr (nr > 0) __builtin_amdgcn_sched_group_barrier(kSgDsRead, nr, 0);
        if constexpr (m % 2 == 1 && m / 2 < ND) __builtin_amdgcn_sched_group_barrier(kSgVmem, 1, 0);
    });
}

// SG (MX only): k-tiles per scale group.  SG == 1 stages each k-tile's scale
// codes with the tile (one 2- or 4-byte load per row); SG > 1 keeps a
// double-buffered ring of scale groups in LDS and fetches 4 * SG bytes per
// row once per group, which cuts the scale loads' L2 requests SG-fold.
// E (two stages only): DMA instructions of k-tile kt + 2 issued in the last
// k-step of k-tile kt, right after the barrier that frees its stage, instead
// of in the first k-steps of kt + 1; an earlier start gives the loads more
// time before the wait that needs them.
// D (two stages only): k-steps over which the rest of the DMA of k-tile
// kt + 1 is spread, starting at k-step 0 of kt (0: all but the last).
// NW: waves per workgroup.  4 waves hold 128 x 128 wave tiles (one wave per
// SIMD); 8 waves hold 128 x 64 wave tiles, two per SIMD, so that one wave's
// MFMAs can run while the other waits (bf16 only).
// FUSED: the fused epilogue of gemm_epi.h instead of the plain fp32 store.
// SPLIT: split-K work units (Args::tiles_per_split, Args::kslice); each unit
// stores its fp32 partial sums, which a separate pass adds in a fixed order.
// DYN: tiles after the first are taken from per-XCD atomic counters
// (Args::tile_ctr, next_tile) instead of the static strided walk; the grid
// must be a multiple of 8.
// LA: k-steps between a fragment read and the MFMAs that use it (1 or 2;
// 2 keeps four fragment sets in registers and moves the closing wait and
// barrier of each k-tile one k-step earlier: bf16, two stages).
// MF: the bf16 MFMA shape, 32 (v_mfma_f32_32x32x16_bf16, 4 x 4 blocks per
// 128 x 128 wave tile, k-steps of 16) or 16 (v_mfma_f32_16x16x32_bf16, 8 x 8
// blocks, or 8 x 4 for 8 waves, k-steps of 32).  The same FLOPs and LDS bytes
// either way; at the board's power limit the 16 x 16 form draws less power
// per FLOP, so the clock it holds is higher.
template <int KIND, int RB, int S, bool TAIL, int SG = 1, int E = 0, int D = 0, int NW = 4, bool FUSED = false,
          bool SPLIT = false, bool DYN = false, int LA = 1, int MF = 32>
__global__ __launch_bounds__(64 * NW, 1) void gemm_fast_kernel(Args a) {
    static_assert(NW == 4 || (NW == 8 && KIND != kMX), "8 waves: bf16 only");
    static_assert(MF == 32 || (MF == 16 && KIND != kMX && LA == 1),
                  "16 x 16 MFMAs: bf16, one fragment step of lookahead");
    static_assert(!SPLIT || (!FUSED && NW == 4), "split-K: plain fp32 partial stores, 4 waves");
    static_assert(!SPLIT || KIND != kMX || SG > 1, "MX split-K: the scale-ring pipeline");
    static_assert(!DYN || (!SPLIT && NW == 4), "dynamic schedule: whole tiles, 4 waves");
    constexpr int THREADS = 64 * NW;
    constexpr int NBJ = NW == 8 ? 2 : kBlocks;  // 32-column MFMA blocks per wave tile
    constexpr int WTN = 32 * NBJ;               // wave tile columns
    constexpr int ESZ = (KIND == kMX) ? 1 : 2;  // operand element bytes
    constexpr int BK = RB / ESZ;                // K elements per k-tile
    constexpr int OPB = kTile * RB;             // bytes of one operand in one stage
    // MX: scale bytes per row per k-tile (one E8M0 code per 32 elements).
    // LDS-DMA narrower than a dword still writes one zero-extended dword per
    // lane, so every row's scales occupy 4 bytes of LDS either way.
    constexpr int SPR = (KIND == kMX) ? BK / 32 : 0;
    constexpr int SCB = (KIND == kMX && SG == 1) ? 2 * kTile * 4 : 0;  // MX scale bytes per stage
    constexpr int RING = (KIND == kMX && SG > 1) ? 2 * kTile * 4 * SG : 16;  // bytes per ring slot
    static_assert(SG == 1 || (KIND == kMX && RB == 128 && SG == 4 && S == 2), "scale ring: MX 128x2 only");
    constexpr int STAGE = 2 * OPB + SCB;
    constexpr int NI = RB * kTile / 1024 / NW;  // DMA instructions per wave per operand
    constexpr int RPK = 1024 / RB;              // K-contiguous rows per KiB
    // MFMA k-steps per k-tile: 16 bf16 or 64 fp8 elements per step
    constexpr int KS = (KIND == kMX) ? BK / 64 : BK / (MF == 16 ? 32 : 16);
    // MFMA blocks per wave tile: BA row blocks of A, BB column blocks of B
    // (32 x 32 blocks, or 16 x 16 with MF == 16), and the accumulator type
    constexpr int BA = MF == 16 ? 8 : kBlocks;
    constexpr int BB = MF == 16 ? 2 * NBJ : NBJ;
    typedef typename std::conditional<MF == 16, f32x4, f32x16>::type AccT;
    // Fragments are double-buffered over the global k-step sequence; with an
    // odd step count per k-tile the buffer parity follows the k-tile parity,
    // which the S-fold unrolled loop keeps static only for even S.
    static_assert(KS % 2 == 0 || S % 2 == 0, "odd k-steps per k-tile need an even stage count");
    static_assert(LA == 1 || (LA == 2 && KIND != kMX && S == 2 && KS >= 3), "fragment lookahead 2: bf16, 2 stages");
    // fragment sets in registers, and the k-step of each k-tile that opens
    // with the closing wait and barrier (its reads are the next stage's)
    constexpr int R = 2 * LA;
    constexpr int BS = KS - LA;
    static_assert(KIND != kMX || SPR == 2 || SPR == 4, "MX k-tile of 64 or 128 codes");
    static_assert(S >= 2 && S * STAGE <= 160 * 1024, "LDS budget");
    // DMA instructions per wave per k-tile: both operands, plus (MX) one
    // scale instruction per operand.
    constexpr int L = 2 * NI + (KIND == kMX && SG == 1 ? 2 : 0);
    // the main loop is unrolled by U k-tiles so that the stage and the scale
    // ring slot of every unrolled k-tile are compile-time constants
    constexpr int U = SG > 1 ? 2 * SG : S;
    static_assert((U * KS) % R == 0, "fragment sets: static over the unrolled loop");
    // The DMA of k-tile kt + S - 1 is issued while k-tile kt is multiplied,
    // DPS instructions per k-step.  With S >= 3 it is spread over every
    // k-step (the part issued after the closing wait is simply younger than
    // what that wait needs); with S == 2 all of it must be issued before
    // the wait, so it covers k-steps 0 .. KS-2.
    static_assert(E == 0 || (S == 2 && E <= L), "early DMA: two stages");
    static_assert(D == 0 || (S == 2 && D < KS), "DMA spread: two stages");
    constexpr int DSTEPS = (S >= 3) ? KS : (D > 0 ? D : KS - 1);
    constexpr int DPS = (L - E + DSTEPS - 1) / DSTEPS;  // DMA instructions per k-step
    // DMA instructions of the current k-tile issued before the closing wait
    constexpr int DBEFORE = (KS - 1) * DPS < L ? (KS - 1) * DPS : L;
    // Loads younger than k-tile kt+1's when the closing wait of k-tile kt
    // runs: k-tiles kt+2 .. kt+S-2 in full plus the early part of kt+S-1.
    constexpr int VM_WAIT = (S >= 3) ? (S - 3) * L + DBEFORE : 0;
    static_assert(VM_WAIT < 64, "vmcnt range");
    static_assert(KS >= 2 || S >= 3, "with one k-step per k-tile the DMA goes after the closing wait");
    typedef typename std::conditional<KIND == kMX, i32x8, bf16x8>::type Frag;

    __shared__ __attribute__((aligned(1024))) uint8_t st0[STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t st1[STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t st2[S > 2 ? STAGE : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t st3[S > 3 ? STAGE : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t st4[S > 4 ? STAGE : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t sr0[RING];
    __shared__ __attribute__((aligned(1024))) uint8_t sr1[RING];
    __shared__ float evl[FUSED ? 3 * 256 : 1];  // fused epilogue: the tile's scales and biases
    // dynamic schedule: the next tile, handed from thread 0 to the workgroup
    // through two alternating slots (a slot is rewritten only after the
    // barrier that follows every wave's read of it)
    __shared__ int tile_slot[2];
    auto stage_ptr = [&](auto sidx) -> uint8_t FAST_LDS* {
        constexpr int s = decltype(sidx)::value;
        if constexpr (s == 0) return (uint8_t FAST_LDS*)st0;
        else if constexpr (s == 1) return (uint8_t FAST_LDS*)st1;
        else if constexpr (s == 2) return (uint8_t FAST_LDS*)st2;
        else if constexpr (s == 3) return (uint8_t FAST_LDS*)st3;
        else return (uint8_t FAST_LDS*)st4;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = NW == 8 ? wave >> 2 : wave >> 1;
    const int wn = NW == 8 ? wave & 3 : wave & 1;
    const int h = lane >> 5;
    const int l32 = lane & 31;

    // ---- per-lane constants of the DMA loads ------------------------------
    // K-contiguous operand: instruction i of this wave fills KiB (NW i + wave)
    // of the operand's stage area; the swizzle of its rows does not depend
    // on i, so one lane offset plus a scalar row step covers all of them.
    const int kc_row0 = wave * RPK + lane / (RB / 16);
    const int kc_chunk = (lane % (RB / 16)) ^ swz<RB>(kc_row0);
    const int a_voff = (int)(kc_row0 * a.lda_b) + kc_chunk * 16;
    const int a_step = (int)(NW * RPK * a.lda_b);
    int b_voff, b_step, b_voff8 = 0;
    if constexpr (KIND == kNN) {
        // k rows of 512 bytes, 2 per KiB: row 2(NW i + wave) + lane / 32;
        // b_voff8 for the rows with bit 3 set (nn_swz)
        const int kk0 = 2 * wave + h;
        b_voff = (int)(kk0 * a.ldb_b) + (l32 ^ nn_swz(kk0 & 7)) * 16;
        b_voff8 = (int)(kk0 * a.ldb_b) + (l32 ^ nn_swz((kk0 & 7) | 8)) * 16;
        b_step = (int)(2 * NW * a.ldb_b);
    } else {
        b_voff = (int)(kc_row0 * a.ldb_b) + kc_chunk * 16;
        b_step = (int)(NW * RPK * a.ldb_b);
    }
    // MX scales: wave w stages the k-tile's scale dwords of rows
    // 64 w .. 64 w + 63 of both operands (one dword = four 32-blocks).
    const int sc_voff = (KIND == kMX) ? (64 * wave + lane) * a.sld : 0;

    // ---- per-lane constants of the fragment reads --------------------------
    // byte offsets in a stage of this lane's A / B chunks at step ks (block
    // 0); fp8 steps read two chunks (k 16h..16h+15 and 32+16h..32+16h+15)
    int a_rd[KS][2], b_rd[KS][2];
    int b_tr[BB];  // NN: offset of block j's transposed read at step 0
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        if constexpr (MF == 16) {
            // 16 x 16 x 32: lane l reads row l % 16 of its block, k 8 (l / 16)
            // .. +7 of the step's 32, i.e. chunk 4 ks + l / 16 (the swizzle
            // depends on row bits 1..3 only, so block i adds 16 i rows)
            a_rd[ks][0] = kc_off<RB>(wm * kWaveTile + (lane & 15), 4 * ks + (lane >> 4));
            b_rd[ks][0] = OPB + kc_off<RB>(wn * WTN + (lane & 15), 4 * ks + (lane >> 4));
            a_rd[ks][1] = b_rd[ks][1] = 0;
        } else {
            const int c0 = (KIND == kMX) ? (4 * ks + h) : (2 * ks + h);
            a_rd[ks][0] = kc_off<RB>(wm * kWaveTile + l32, c0);
            b_rd[ks][0] = OPB + kc_off<RB>(wn * WTN + l32, c0);
            a_rd[ks][1] = kc_off<RB>(wm * kWaveTile + l32, c0 + 2);
            b_rd[ks][1] = OPB + kc_off<RB>(wn * WTN + l32, c0 + 2);
        }
    }
    if constexpr (KIND == kNN && MF == 16) {
        // transposed reads for 16 x 16 x 32: lane p of each 16-lane group g
        // addresses k-row 8 g + p / 4 (and + 4 for the second half) and the
        // 4 columns from 4 (p % 4) of block j
        const int g = lane >> 4, p = lane & 15;
#pragma unroll
        for (int j = 0; j < BB; ++j) b_tr[j] = OPB + nn_off(8 * g + (p >> 2), wn * WTN + 16 * j + 4 * (p & 3));
    } else if constexpr (KIND == kNN) {
        const int g = lane >> 4, li = lane & 15;
#pragma unroll
        for (int j = 0; j < NBJ; ++j) {
            int n = wn * WTN + j * 32 + 16 * (g & 1) + 4 * (li & 3);
            int k = 8 * (g >> 1) + (li >> 2);
            b_tr[j] = OPB + nn_off(k, n);
        }
    }
    // MX: this lane's scale dwords in a stage (row block 0 of A and of B).
    const int sa_rd = 2 * OPB + 4 * (wm * kWaveTile + l32);
    const int sb_rd = 2 * OPB + 4 * kTile + 4 * (wn * kWaveTile + l32);

    const int G = gridDim.x;
    const int P = G >> 3;              // workgroups per XCD
    const int xcd = blockIdx.x & 7;    // workgroup b runs on XCD b % 8
    int slot = 0;
    for (int t = logical_block(a); t < a.num_tiles;) {
        // dynamic schedule: claim the next position of this XCD's queue now;
        // the value is needed only when the tile ends
        int claim = 0;
        if constexpr (DYN) {
            if (tid == 0) claim = P + atomicAdd(a.tile_ctr + 32 * xcd, 1);
        }
        // split-K: unit t is tile tt of K range ks; K ranges are the slow
        // index, so concurrently running units read the same k columns
        int tt = t, k0 = 0, Kl = a.K;
        float* pw = nullptr;  // split-K partial: where output (m0, n0) goes
        int pld = 0;          // and its row pitch
        if constexpr (SPLIT) {
            if (t >= a.dp_units) {
                const int u = t - a.dp_units;
                const int ks = u / a.tiles_per_split;
                const int i = u - ks * a.tiles_per_split;
                tt = a.tile0 + i;
                k0 = ks * a.kslice;
                Kl = min(a.K - k0, a.kslice);
                if (a.part != nullptr) {
                    pw = a.part + (int64_t)(ks * a.tiles_per_split + i) * (kTile * kTile);
                    pld = kTile;
                } else {
                    pw = nullptr;  // set below, once m0 and n0 are known
                    pld = -1 - ks;
                }
            }
        }
        const int KT = SPLIT ? Kl / BK : a.kt_full;  // k-tiles holding data
        const int KTM = (KT + U - 1) / U * U;        // rounded up: the rest are dead (zero) k-tiles
        int tm, tn;
        tile_coords(a, tt, tm, tn);
        const int m0 = tm * kTile, n0 = tn * kTile;
        const int rows_a = min(kTile, a.M - m0);
        const int rows_b = min(kTile, a.N - n0);
        EpiRegs epv{};
        if constexpr (FUSED) epv = epi_prefetch(a, m0, n0, kTile, tid);

        // Per-tile buffer descriptors: everything past the last valid row
        // (or, for row-major B, past the last k row) reads as zero.  The
        // dead descriptor (size 0) turns the loads of k-tiles past the end
        // into zero fill without memory traffic.
        const uint8_t* a_base = a.A + (int64_t)m0 * a.lda_b + (int64_t)k0 * ESZ;
        const __amdgpu_buffer_rsrc_t ra =
            make_rsrc(a_base, round4((int64_t)(rows_a - 1) * a.lda_b + (int64_t)Kl * ESZ));
        const uint8_t* b_base;
        __amdgpu_buffer_rsrc_t rb;
        if constexpr (KIND == kNN) {
            b_base = a.B + (int64_t)n0 * 2 + (int64_t)k0 * a.ldb_b;
            rb = make_rsrc(b_base, (int64_t)(Kl - 1) * a.ldb_b + (int64_t)(a.N - n0) * 2);
        } else {
            b_base = a.B + (int64_t)n0 * a.ldb_b + (int64_t)k0 * ESZ;
            rb = make_rsrc(b_base, round4((int64_t)(rows_b - 1) * a.ldb_b + (int64_t)Kl * ESZ));
        }
        const __amdgpu_buffer_rsrc_t rdead = make_rsrc(a.A, 0);
        __amdgpu_buffer_rsrc_t rsa = rdead, rsb = rdead;
        if constexpr (KIND == kMX) {
            // the scale codes of this unit's K range: sk0 codes of each row
            // precede it, and it holds Kl / 32 of them
            const int sk0 = k0 / 32;
            const int sl = SPLIT ? Kl / 32 : a.sld;
            rsa = make_rsrc(a.SA + (int64_t)m0 * a.sld + sk0, (int64_t)(rows_a - 1) * a.sld + sl);
            rsb = make_rsrc(a.SB + (int64_t)n0 * a.sld + sk0, (int64_t)(rows_b - 1) * a.sld + sl);
        }

        // DMA instruction d (0 .. L-1) of k-tile kt into stage s.
        auto dma = [&](auto sidx, int d, int kt, bool live) {
            uint8_t FAST_LDS* As = stage_ptr(sidx);
            if (d < NI) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(live ? ra : rdead,
                                                         (void FAST_LDS*)(As + (NW * d + wave) * 1024), 16,
                                                         a_voff, kt * RB + d * a_step, 0, 0);
            } else if (d < 2 * NI) {
                const int i = d - NI;
                const int koff = (KIND == kNN) ? kt * BK * (int)a.ldb_b : kt * RB;
                // row-major B: instruction i fills k-rows 2 (NW i + wave) and
                // + 1, whose bit 3 picks the swizzle (uniform over the wave)
                const int bv = (KIND == kNN && (((2 * (NW * i + wave)) >> 3) & 1)) ? b_voff8 : b_voff;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(live ? rb : rdead,
                                                         (void FAST_LDS*)(As + OPB + (NW * i + wave) * 1024), 16,
                                                         bv, koff + i * b_step, 0, 0);
            } else if constexpr (KIND == kMX) {
                const bool sb = d > 2 * NI;
                const __amdgpu_buffer_rsrc_t rs = live ? (sb ? rsb : rsa) : rdead;
                void FAST_LDS* dst = (void FAST_LDS*)(As + 2 * OPB + (sb ? 4 * kTile : 0) + 256 * wave);
                // one scale load per row: SPR bytes (the size operand must be a literal)
                if constexpr (SPR == 2)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 2, sc_voff, kt * SPR, 0, 0);
                else
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 4, sc_voff, kt * SPR, 0, 0);
            }
        };

        // Scale ring: group g (k-tiles SG g .. SG g + SG - 1) into slot g % 2;
        // wave w loads rows 64 w .. 64 w + 63 of both operands, 4 SG bytes each.
        auto ring_dma = [&](auto slot, int g, bool live) {
            if constexpr (KIND == kMX && SG > 1) {
                uint8_t FAST_LDS* base = decltype(slot)::value ? (uint8_t FAST_LDS*)sr1 : (uint8_t FAST_LDS*)sr0;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(live ? rsa : rdead, (void FAST_LDS*)(base + 1024 * wave),
                                                         16, sc_voff, g * 16, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(live ? rsb : rdead,
                                                         (void FAST_LDS*)(base + 4096 + 1024 * wave), 16, sc_voff,
                                                         g * 16, 0, 0);
            }
        };

        auto read_frags = [&](auto sidx, int ks, Frag* fa, Frag* fb) {
            const uint8_t FAST_LDS* base = stage_ptr(sidx);
            if constexpr (MF == 16) {
                // in the order the MFMAs first use them (z_frag)
                static_for<0, 8 + BB>([&](auto oc) {
                    constexpr int f = z_frag<BB>(decltype(oc)::value);
                    constexpr int j = f & 7;
                    if constexpr (f < 8) {
                        fa[j] = *(const bf16x8 FAST_LDS*)(base + a_rd[ks][0] + j * 16 * RB);
                    } else if constexpr (KIND == kNN) {
                        const uint8_t FAST_LDS* p = base + b_tr[j] + ks * 32 * 512;
                        bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 FAST_LDS*)p);
                        bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 FAST_LDS*)(p + 4 * 512));
                        fb[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    } else {
                        fb[j] = *(const bf16x8 FAST_LDS*)(base + b_rd[ks][0] + j * 16 * RB);
                    }
                });
                return;
            }
#pragma unroll
            for (int i = 0; i < kBlocks; ++i) {
                if constexpr (KIND == kMX) {
                    i32x4 lo = *(const i32x4 FAST_LDS*)(base + a_rd[ks][0] + i * 32 * RB);
                    i32x4 hi = *(const i32x4 FAST_LDS*)(base + a_rd[ks][1] + i * 32 * RB);
                    fa[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                } else {
                    fa[i] = *(const bf16x8 FAST_LDS*)(base + a_rd[ks][0] + i * 32 * RB);
                }
            }
#pragma unroll
            for (int j = 0; j < NBJ; ++j) {
                if constexpr (KIND == kMX) {
                    i32x4 lo = *(const i32x4 FAST_LDS*)(base + b_rd[ks][0] + j * 32 * RB);
                    i32x4 hi = *(const i32x4 FAST_LDS*)(base + b_rd[ks][1] + j * 32 * RB);
                    fb[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                } else if constexpr (KIND == kNN) {
                    const uint8_t FAST_LDS* p = base + b_tr[j] + ks * 16 * 512;
                    bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 FAST_LDS*)p);
                    bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 FAST_LDS*)(p + 4 * 512));
                    fb[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                } else {
                    fb[j] = *(const bf16x8 FAST_LDS*)(base + b_rd[ks][0] + j * 32 * RB);
                }
            }
        };
        // fragment reads per k-step (LDS instructions)
        constexpr int NR = (KIND == kMX) ? 16 : (KIND == kNN) ? BA + 2 * BB : BA + BB;
        constexpr int NMF = BA * BB;  // MFMAs per k-step

        // MX: the scale dwords of the k-tile in stage s, pre-shifted so that
        // lane half h finds its 32-block (2 ks + h) in byte 2 ks.
        int sc[2 * kBlocks];
        // scale ring (SG > 1): raw scale dwords of the next k-tile, read one
        // k-step ahead so that their LDS latency is hidden
        int scr[2 * kBlocks];
        // scales of the k-tile in stage sidx (SG == 1) or at position q of
        // the unrolled loop (SG > 1: ring slot (q / SG) % 2, dword q % SG)
        // ring: the raw dwords of k-tile position q into out (unshifted)
        auto read_ring = [&](auto qidx, int* out) {
            if constexpr (KIND == kMX && SG > 1) {
                constexpr int q = decltype(qidx)::value % U;
                const uint8_t FAST_LDS* base =
                    ((q / SG) % 2) ? (const uint8_t FAST_LDS*)sr1 : (const uint8_t FAST_LDS*)sr0;
#pragma unroll
                for (int i = 0; i < kBlocks; ++i) {
                    out[i] = *(const int FAST_LDS*)(base + 16 * (wm * kWaveTile + l32 + 32 * i) + 4 * (q % SG));
                    out[kBlocks + i] =
                        *(const int FAST_LDS*)(base + 4096 + 16 * (wn * kWaveTile + l32 + 32 * i) + 4 * (q % SG));
                }
            }
        };
        auto shift_scales = [&](const int* raw) {
#pragma unroll
            for (int i = 0; i < 2 * kBlocks; ++i) sc[i] = (int)((uint32_t)raw[i] >> (8 * h));
        };
        auto read_scales = [&](auto sidx, auto qidx) {
            if constexpr (KIND == kMX && SG > 1) {
                read_ring(qidx, scr);
                shift_scales(scr);
            } else if constexpr (KIND == kMX) {
                const uint8_t FAST_LDS* base = stage_ptr(sidx);
#pragma unroll
                for (int i = 0; i < kBlocks; ++i) {
                    // low SPR bytes: the codes of 32-blocks SPR*kt .. SPR*kt+SPR-1
                    uint32_t w = *(const uint32_t FAST_LDS*)(base + sa_rd + 128 * i);
                    uint32_t v = *(const uint32_t FAST_LDS*)(base + sb_rd + 128 * i);
                    sc[i] = (int)(w >> (8 * h));
                    sc[kBlocks + i] = (int)(v >> (8 * h));
                }
            }
        };

        AccT acc[BA][BB];
#pragma unroll
        for (int i = 0; i < BA; ++i)
#pragma unroll
            for (int j = 0; j < BB; ++j)
#pragma unroll
                for (int r = 0; r < (MF == 16 ? 4 : 16); ++r) acc[i][j][r] = 0.0f;

        auto mfma = [&](int ks, const Frag* fa, const Frag* fb, const int* scl) {
            if constexpr (MF == 16) {
                // Z order over the 8 x 8 blocks (interleave_step16)
                static_for<0, BA * BB>([&](auto mc) {
                    constexpr int r = z_row<BB>(decltype(mc)::value), c = z_col<BB>(decltype(mc)::value);
                    acc[r][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[r], fb[c], acc[r][c], 0, 0, 0);
                });
            } else {
#pragma unroll
                for (int i = 0; i < BA; ++i)
#pragma unroll
                    for (int j = 0; j < BB; ++j) {
                        if constexpr (KIND == kMX) {
                            // k-step ks covers 32-blocks 2 ks and 2 ks + 1 of the
                            // k-tile: byte 2 ks of the (pre-shifted) scale word.
                            if (ks == 0)
                                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                    fa[i], fb[j], acc[i][j], 0, 0, 0, scl[i], 0, scl[kBlocks + j]);
                            else
                                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                    fa[i], fb[j], acc[i][j], 0, 0, 2, scl[i], 2, scl[kBlocks + j]);
                        } else {
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
                        }
                    }
            }
        };

        // ---- prologue: k-tiles 0 .. S-2 into stages 0 .. S-2 --------------
        [&]<int... Is>(std::integer_sequence<int, Is...>) {
            ((
                 [&] {
#pragma unroll
                     for (int d = 0; d < L; ++d) dma(std::integral_constant<int, Is>{}, d, Is, Is < KT);
                 }()),
             ...);
        }(std::make_integer_sequence<int, S - 1>{});
        ring_dma(std::integral_constant<int, 0>{}, 0, 0 < KT);
        // early part of k-tile 1 (two stages), and with LA = 2 also the
        // part a loop iteration issues after its barrier (k-step BS + 1)
        constexpr int EP = LA == 2 ? (E + DPS < L ? E + DPS : L) : E;
#pragma unroll
        for (int d = 0; d < EP; ++d) dma(std::integral_constant<int, 1>{}, d, 1, 1 < KT);
        wait_vm<((SG > 1) ? 0 : (S - 2) * L) + EP>();
        barrier();

        // fragment set f holds the fragments of global k-step f mod R
        Frag Fa[R][BA], Fb[R][BB];
        static_for<0, LA>([&](auto tc) {
            constexpr int t = decltype(tc)::value;
            read_frags(std::integral_constant<int, 0>{}, t, Fa[t], Fb[t]);
        });
        read_scales(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
        // Let the first fragments land here, once per tile: the compiler's
        // wait analysis merges the state at the loop entry with the state at
        // the end of an iteration, and prologue reads left in flight (issued
        // in no particular order) would make it wait for all reads at the top
        // of every iteration.
        wait_lgkm0();

        // One k-tile held in stage s; meanwhile the DMA of k-tile kt + S - 1
        // fills stage s - 1 (freed by the barrier that closed k-tile kt - 1).
        auto body = [&](auto qidx, int kt) {
            constexpr int q = decltype(qidx)::value;  // position in the unrolled loop
            constexpr int s = q % S;
            auto sidx = std::integral_constant<int, s>{};
            constexpr int snext = (s + 1) % S;
            constexpr int sdma = (s + S - 1) % S;
            const int kd = kt + S - 1;
            const bool live = kd < KT;
            int scn[2 * kBlocks];
            static_for<0, KS>([&](auto ksc) {
                constexpr int ks = decltype(ksc)::value;
                constexpr int gk = q * KS + ks;  // global k-step, modulo the unrolled loop
                Frag* ca = Fa[gk % R];
                Frag* cb = Fb[gk % R];
                Frag* na = Fa[(gk + LA) % R];
                Frag* nb = Fb[(gk + LA) % R];
                // The DMA of a k-tile after its E early instructions is spread
                // over the KS - 1 k-steps that follow the barrier issuing
                // them, DPS instructions per step: slot j is the j-th of them.
                // Steps before the barrier carry k-tile kd's, steps after it
                // (LA = 2) k-tile kt + 2's into the stage just freed.
                constexpr int j = ks < BS ? KS - 1 - BS + ks : (ks == BS ? KS - 1 : ks - BS - 1);
                constexpr int d0 = E + j * DPS < L ? E + j * DPS : L;
                constexpr int d1 = E + (j + 1) * DPS < L ? E + (j + 1) * DPS : L;
                if constexpr (ks < BS) {
                    read_frags(sidx, ks + LA, na, nb);
                    if constexpr (KIND == kMX && SG > 1 && ks == 0) {
                        // scales of k-tile kt + 1: its ring slot landed before
                        // the barrier closing the k-tile that requested it
                        read_ring(std::integral_constant<int, q + 1>{}, scr);
                    }
                    static_for<d0, d1>([&](auto dc) {
                        dma(std::integral_constant<int, sdma>{}, decltype(dc)::value, kd, live);
                    });
                    if constexpr (SG > 1 && ks == 0 && q % SG == 0) {
                        // next scale group into the other ring slot (its last
                        // reader finished before the barrier closing k-tile kt-1)
                        const int g = kt / SG + 1;
                        ring_dma(std::integral_constant<int, (q / SG + 1) % 2>{}, g, g * SG < KT);
                    }
                    mfma(ks, ca, cb, sc);
                    if constexpr (MF == 16)
                        interleave_step16<NR, d1 - d0, NMF>();
                    else
                        interleave_step<NR, d1 - d0 + ((SG > 1 && ks == 0 && q % SG == 0) ? 2 : 0), NMF>();
                    // keep every MFMA of this step ahead of the closing wait
                    __builtin_amdgcn_sched_barrier(0);
                } else if constexpr (ks == BS) {
                    // Every fragment of stage s is in registers or being read,
                    // so stage s is free once the reads land; k-tile kt+1
                    // must have landed.
                    wait_lgkm0();
                    wait_vm<VM_WAIT>();
                    barrier();
                    read_frags(std::integral_constant<int, snext>{}, ks + LA - KS, na, nb);
                    static_for<d0, d1>([&](auto dc) {
                        dma(std::integral_constant<int, sdma>{}, decltype(dc)::value, kd, live);
                    });
                    // two stages: stage s is free now; start k-tile kt + 2
                    static_for<0, E>([&](auto dc) {
                        dma(sidx, decltype(dc)::value, kt + 2, kt + 2 < KT);
                    });
                    if constexpr (KIND == kMX && SG > 1) {
                        mfma(ks, ca, cb, sc);
                        shift_scales(scr);  // k-tile kt + 1's scales, read at k-step 0
                    } else if constexpr (KIND == kMX) {
#pragma unroll
                        for (int q = 0; q < 2 * kBlocks; ++q) scn[q] = sc[q];
                        read_scales(std::integral_constant<int, snext>{}, std::integral_constant<int, q + 1>{});
                        mfma(ks, ca, cb, scn);
                    } else {
                        mfma(ks, ca, cb, sc);
                    }
                    if constexpr (MF == 16)
                        interleave_step16<NR, d1 - d0 + E, NMF>();
                    else
                        interleave_step<NR, d1 - d0 + E, NMF>();
                    __builtin_amdgcn_sched_barrier(0);
                } else {
                    // after the barrier (LA = 2): the next stage's fragments,
                    // and the next part of k-tile kt + 2's DMA into stage s
                    read_frags(std::integral_constant<int, snext>{}, ks + LA - KS, na, nb);
                    static_for<d0, d1>([&](auto dc) {
                        dma(sidx, decltype(dc)::value, kt + 2, kt + 2 < KT);
                    });
                    mfma(ks, ca, cb, sc);
                    if constexpr (MF == 16)
                        interleave_step16<NR, d1 - d0, NMF>();
                    else
                        interleave_step<NR, d1 - d0, NMF>();
                    __builtin_amdgcn_sched_barrier(0);
                }
            });
        };

        for (int kt0 = 0; kt0 < KTM; kt0 += U) {
            [&]<int... Is>(std::integer_sequence<int, Is...>) {
                (body(std::integral_constant<int, Is>{}, kt0 + Is), ...);
            }(std::make_integer_sequence<int, U>{});
        }

        // The dead k-tiles still in flight carry no memory traffic; let them
        // land before the stages are reused.
        wait_vm<0>();

        // ---- partial last k-tile: predicated register loads, zero past K --
        if constexpr (TAIL && KIND != kMX) {
            barrier();  // every wave is done with the pipelined stages
            uint8_t FAST_LDS* As = stage_ptr(std::integral_constant<int, 0>{});
            const int kvalid = Kl - KT * BK;  // 0 for a split-K unit before the last
            tail_kc<RB, THREADS>(As, ra, (int)a.lda_b, KT * RB, kvalid * ESZ, tid);
            if constexpr (KIND == kNN)
                tail_nn<BK, THREADS>(As + OPB, rb, (int)a.ldb_b, KT * BK * (int)a.ldb_b, kvalid, a.N - n0, tid);
            else
                tail_kc<RB, THREADS>(As + OPB, rb, (int)a.ldb_b, KT * RB, kvalid * ESZ, tid);
            wait_lgkm0();
            barrier();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                read_frags(std::integral_constant<int, 0>{}, ks, Fa[0], Fb[0]);
                mfma(ks, Fa[0], Fb[0], sc);
            }
        }

        // ---- epilogue: fp32 stores straight from the accumulators --------
        if constexpr (FUSED) {
            static_assert(NW == 4, "fused epilogue: one row, column and bias per thread");
            epi_stage((float FAST_LDS*)evl, epv, tid);
            wait_lgkm0();
            barrier();
        }
        if constexpr (SPLIT) {
            float* cw = nullptr;
            int cld = 0;
            if (pld > 0) {
                cw = pw + wm * kWaveTile * kTile + wn * WTN;
                cld = pld;
            } else if (pld < 0) {
                // stacked dense planes: plane ks = -1 - pld, row pitch ldc
                cw = a.C + (int64_t)(m0 + wm * kWaveTile + (-1 - pld) * a.M) * a.ldc + n0 + wn * WTN;
                cld = (int)a.ldc;
            }
            if constexpr (MF == 16)
                store_c16(a, acc, m0 + wm * kWaveTile, n0 + wn * WTN, lane, nullptr, 0, 0, cw, cld);
            else
                store_c<NBJ, false>(a, acc, m0 + wm * kWaveTile, n0 + wn * WTN, h, l32, nullptr, 0, 0, cw, cld,
                                    pld == 0);
        } else {
            if constexpr (MF == 16)
                store_c16<FUSED>(a, acc, m0 + wm * kWaveTile, n0 + wn * WTN, lane, (const float FAST_LDS*)evl,
                                 wm * kWaveTile, wn * WTN);
            else
                store_c<NBJ, FUSED>(a, acc, m0 + wm * kWaveTile, n0 + wn * WTN, h, l32, (const float FAST_LDS*)evl,
                                    wm * kWaveTile, wn * WTN);
        }
        if constexpr (DYN) {
            if (tid == 0) tile_slot[slot] = next_tile(a, xcd, claim, P, G);
        }
        // The next tile's prologue overwrites stages 0 .. S-2: every wave
        // must be done reading them.
        wait_lgkm0();
        barrier();
        if constexpr (DYN) {
            t = __builtin_amdgcn_readfirstlane(tile_slot[slot]);
            slot ^= 1;
        } else {
            t += G;
        }
    }
}

// Launch geometry shared by the host launchers: the tile grid, the raster
// band height (group_m rows of tiles, 8 when group_m <= 0) and the k-tile
// counts for k-tiles of bk elements.  num_tiles may be raised afterwards
// (split-K units) before fast_grid picks the persistent grid: the CUs, or the
// work units when fewer, rounded down to a multiple of 8 (from 8 up), with
// the XCD-aware renumbering when the grid is such a multiple.
inline void fast_tiles(Args& a, int group_m, int bk) {
    a.tiles_m = (a.M + kTile - 1) / kTile;
    a.tiles_n = (a.N + kTile - 1) / kTile;
    a.num_tiles = a.tiles_m * a.tiles_n;
    if (group_m <= 0) group_m = 8;
    a.group_m = a.tiles_m < group_m ? a.tiles_m : group_m;
    a.kt_full = a.K / bk;
    a.kt_total = (a.K + bk - 1) / bk;
}

inline int fast_grid(Args& a, int cus) {
    int grid = cus < a.num_tiles ? cus : a.num_tiles;
    if (grid >= 8) grid -= grid % 8;
    a.xcd_remap = (grid % 8 == 0) ? 1 : 0;
    return grid;
}

// Launch of a bf16 instance of the 256 x 256 direct-load kernel with
// 16 x 16 x 32 MFMAs (two stages of 128-byte k-rows, 8 DMA instructions of
// k-tile t+2 after the barrier of k-tile t, the rest over one k-step) on
// `grid` workgroups; the instances are compiled in gemm_mf16.hip.
template <int KIND, bool TAIL, bool FUSED, bool SPLIT, bool DYN>
void launch_mf16(int grid, hipStream_t stream, const Args& a);
#ifdef LIBGEMM_MEASURE
template <int KIND, bool TAIL>
void launch_mf16_w8(int grid, hipStream_t stream, const Args& a);
#endif

}  // namespace fast
