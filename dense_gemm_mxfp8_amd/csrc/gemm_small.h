// gemm_small.h -- the small-M path for bf16 with row-major B ("NN").
//
// With M <= 64 the product is bound by streaming B (K x N) from HBM once; the
// arithmetic is negligible.  The kernel is laid out for that:
//
//   * one workgroup per 32-column block of B and C; wave w of W owns the
//     32-row k-steps w, w + W, w + 2W, ... of the block, so every wave
//     streams a private share of B (no barrier inside the loop) while all
//     waves of all workgroups sweep one contiguous band of B rows together;
//   * each k-step is 32 rows x 64 bytes of B: two 16-byte loads per lane,
//     issued NP steps ahead into registers (deep memory-level parallelism
//     without LDS staging of the stream), plus the 16 bytes of A each lane
//     needs for the step;
//   * the step's B rows go through a wave-private LDS buffer so that
//     `ds_read_b64_tr_b16` can hand the matrix core K-contiguous columns;
//     v_mfma_f32_16x16x32_bf16 accumulates 16 rows x 32 columns per row
//     block of A (MB blocks for M up to 16 MB);
//   * the 8 per-wave partial sums are added in LDS in wave order (a fixed
//     order, so results are deterministic) and written as fp32.
//
// Split-K: blockIdx.y selects the K range [y kslice, min(K, (y+1) kslice)),
// and the workgroup writes its fp32 partial sums to C + y c_split (plain
// store); a separate pass adds the partials in range order.  Without a
// split, gridDim.y == 1 and kslice == K.
//
// Bounds: B and A are read through buffer descriptors, so rows past K (B)
// and past M (A) read as zero; A's elements past K inside a valid row are
// masked in registers on the last step.  Columns past N only feed outputs
// that are not stored.  Preconditions (host-checked): A and B 16-byte
// aligned with 16-byte aligned rows.

#pragma once

#include "gemm_epi.h"

namespace small {

constexpr int kStepK = 32;     // k-rows per step (one 16x16x32 MFMA depth)
constexpr int kRsrcWord3 = 0x00020000;

struct Args {
    const uint8_t* A;
    const uint8_t* B;
    void* C;             // elements of type epi.out
    int64_t lda_b, ldb_b, ldc;
    int M, N, K;
    int kw;   // k-rows per wave (a multiple of kStepK)
    int pair_xcd;  // map neighbouring column blocks onto one XCD (grid % 16 == 0)
    epi::Params epi;  // fused epilogue
    int kslice;       // K range per blockIdx.y (a multiple of kStepK)
    int64_t c_split;  // fp32 elements between the partial sums of two K ranges
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

#define SMALL_LDS __attribute__((address_space(3)))

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    int n = bytes > 0x7fffffff ? 0x7fffffff : (int)bytes;
    if (n < 0) n = 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kRsrcWord3);
}

// MB: 16-row blocks of A (M <= 16 MB); NP: steps of B prefetched in
// registers; COLS: columns per workgroup (32: 64-byte row segments, 64: full
// 128-byte lines, 128: 256-byte segments); WAVES: waves per workgroup, each
// owning a K range; BAUX: cache-policy bits of the B loads (2: non-temporal,
// B is read once).
template <int MB, int NP, int COLS, int WAVES, int BAUX = 0>
__global__ __launch_bounds__(64 * WAVES, 1) void gemm_small_m_nn(Args a) {
    constexpr int kCols = COLS;
    constexpr int kWaves = WAVES;
    constexpr int kThreads = 64 * WAVES;
    constexpr int CB = COLS / 16;              // 16-column MFMA blocks
    constexpr int LPR = COLS * 2 / 16;         // lanes per B row (16 bytes each)
    constexpr int RPI = 64 / LPR;              // B rows per load instruction
    constexpr int NL = kStepK / RPI;           // B loads per lane per step
    // per wave: one 32-row B buffer; after the loop the same LDS holds the
    // partial sums: waves x MB blocks x 16 rows x (COLS + 4) fp32 (the 4
    // padding floats put the four 16-lane groups of a store on different
    // banks)
    constexpr int kBufBytes = kStepK * kCols * 2;
    constexpr int kRedLd = kCols + 4;
    constexpr int kRed = kWaves * MB * 16 * kRedLd * 4;
    constexpr int kLds = (kWaves * kBufBytes > kRed) ? kWaves * kBufBytes : kRed;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kLds];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Workgroups are dispatched round-robin over the 8 XCDs (workgroup b on
    // XCD b % 8).  With 32-column blocks two neighbouring blocks share every
    // 128-byte line of B; numbering them b = 8q + x -> block 16 (q / 2) +
    // 2x + q % 2 puts both halves of each line on XCD x, so its L2 fetches
    // the line once instead of two L2s fetching it each.
    int blk = blockIdx.x;
    if (a.pair_xcd) {
        const int q = blk >> 3, x = blk & 7;
        blk = 16 * (q >> 1) + 2 * x + (q & 1);
    }
    const int n0 = blk * kCols;
    // this workgroup's K range (the whole of K without a split)
    const int k0 = blockIdx.y * a.kslice;
    const int K = min(a.K - k0, a.kslice);
    const uint8_t* const A = a.A + (int64_t)k0 * 2;
    const uint8_t* const B = a.B + (int64_t)k0 * a.ldb_b;
    void* const C = (float*)a.C + blockIdx.y * a.c_split;
    // wave w takes the 32-row steps w, w + WAVES, w + 2 WAVES, ...: all
    // waves (and all workgroups) sweep one contiguous band of B rows together
    const int steps = a.kw / kStepK;
    auto kstep = [&](int st) { return (st * kWaves + wave) * kStepK; };

    // Buffer range checks work on whole dwords, so the ranges are rounded up
    // to 4 bytes: otherwise a last valid element sharing its dword with the
    // first invalid one would read as zero.  The (at most 2) extra bytes are
    // masked (A) or feed only columns that are not stored (B).
    // B descriptor from column n0: rows past K read as zero.
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(B + (int64_t)n0 * 2, ((int64_t)(K - 1) * a.ldb_b + (int64_t)(a.N - n0) * 2 + 3) & ~(int64_t)3);
    // A descriptor: rows past M read as zero.
    const __amdgpu_buffer_rsrc_t ra =
        make_rsrc(A, ((int64_t)(a.M - 1) * a.lda_b + (int64_t)K * 2 + 3) & ~(int64_t)3);

    // B loads: lane l covers k-row (l / LPR) (+ RPI per further load) and
    // bytes 16 (l % LPR) .. +15 of the block's row segment.
    const int b_voff = (lane / LPR) * (int)a.ldb_b + (lane % LPR) * 16;
    const int b_stepr = RPI * (int)a.ldb_b;
    // A fragment of 16x16x32: lane l holds A[m = l%16][k + 8 (l/16) .. +7].
    const int am = lane & 15, ag = lane >> 4;
    const int a_voff = am * (int)a.lda_b + 16 * ag;

    uint8_t SMALL_LDS* buf = (uint8_t SMALL_LDS*)lds + wave * kBufBytes;
    // Bank spread of the buffer: the 32-byte segment s of k-row r is stored
    // at segment s ^ seg_xor(r).  A transposed read serves 16 lanes from k-rows
    // 8 g + 0..3 (g = lane / 16) and 32 lanes from two such quartets; with
    // 256-byte rows (128 columns) all rows start on bank 0, so without the
    // XOR the eight rows of 32 lanes would hit the same eight banks.
    auto seg_xor = [](int r) {
        if constexpr (kCols == 128) return (r & 3) | ((r >> 1) & 4);
        else if constexpr (kCols == 64) return ((r >> 1) & 1) | ((r >> 2) & 2);
        else return (r >> 3) & 1;
    };
    // transposed reads: lane p of each 16-lane group addresses k-row
    // (p / 4) of its quarter (+ 4 for the second read) and 4 columns starting
    // at 4 (p % 4) of 16-column block c, i.e. byte 8 (p % 4) of segment c
    const int tp = lane & 15, tg = lane >> 4;
    const int tr_row = 8 * tg + (tp >> 2);
    const int tr_lo = tr_row * (kCols * 2) + 32 * seg_xor(tr_row) + 8 * (tp & 3);
    const int tr_hi = (tr_row + 4) * (kCols * 2) + 32 * seg_xor(tr_row + 4) + 8 * (tp & 3);

    f32x4 acc[MB][CB];
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int c = 0; c < CB; ++c) acc[b][c] = f32x4{0.f, 0.f, 0.f, 0.f};

    // zero-size descriptor: loads of steps past the wave's range are zero
    const __amdgpu_buffer_rsrc_t rdead = make_rsrc(B, 0);
    i32x4 rB[NP][NL];
    i32x4 rA[NP][MB];
    auto issue = [&](int slot, int st) {
        const bool live = st < steps;
        const int k = live ? kstep(st) : 0;
#pragma unroll
        for (int h = 0; h < NL; ++h)
            rB[slot][h] = __builtin_amdgcn_raw_buffer_load_b128(live ? rb : rdead, b_voff,
                                                                k * (int)a.ldb_b + h * b_stepr, BAUX);
#pragma unroll
        for (int b = 0; b < MB; ++b)
            rA[slot][b] = __builtin_amdgcn_raw_buffer_load_b128(live ? ra : rdead,
                                                                a_voff + b * 16 * (int)a.lda_b, k * 2, 0);
    };

    // prologue: steps 0 .. NP-2; the loop runs a multiple of NP steps, the
    // padding steps load zeros
#pragma unroll
    for (int p = 0; p < NP - 1; ++p) issue(p, p);
    const int steps_pad = (steps + NP - 1) / NP * NP;

    for (int s0 = 0; s0 < steps_pad; s0 += NP) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int st = s0 + p;
            issue((p + NP - 1) % NP, st + NP - 1);
            // this step's B rows into the wave's buffer (16-byte chunk q of
            // row r at chunk q ^ 2 seg_xor(r))
#pragma unroll
            for (int h = 0; h < NL; ++h) {
                const int r = h * RPI + lane / LPR;
                *(i32x4 SMALL_LDS*)(buf + r * (kCols * 2) + ((lane % LPR) ^ (2 * seg_xor(r))) * 16) = rB[p][h];
            }
            // A past K inside a valid row must not reach the sum
            const int kfirst = kstep(st) + 8 * ag;
            if (kfirst + 8 > K) {
#pragma unroll
                for (int b = 0; b < MB; ++b) {
                    i32x4 v = rA[p][b];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int kk = kfirst + 2 * e;
                        uint32_t w = (uint32_t)v[e];
                        if (kk >= K) w = 0;
                        else if (kk + 1 >= K) w &= 0xffffu;
                        v[e] = (int)w;
                    }
                    rA[p][b] = v;
                }
            }
            bf16x8 fb[CB];
#pragma unroll
            for (int c = 0; c < CB; ++c) {
                // segment c of the row sits at c ^ seg_xor: XOR 32 c into the
                // lane's offset (its bits 5.. hold seg_xor, bits 0..4 < 32)
                bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 SMALL_LDS*)(buf + (tr_lo ^ (32 * c))));
                bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 SMALL_LDS*)(buf + (tr_hi ^ (32 * c))));
                fb[c] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
#pragma unroll
            for (int b = 0; b < MB; ++b) {
                bf16x8 fa = __builtin_bit_cast(bf16x8, rA[p][b]);
#pragma unroll
                for (int c = 0; c < CB; ++c)
                    acc[b][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb[c], acc[b][c], 0, 0, 0);
            }
        }
    }
    __syncthreads();

    // Partial sums to LDS: block b, column block c, register r of lane l is
    // C[16 b + 4 (l/16) + r][16 c + l%16].
    float SMALL_LDS* red = (float SMALL_LDS*)lds;
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int c = 0; c < CB; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * b + 4 * (lane >> 4) + r;
                const int col = 16 * c + (lane & 15);
                red[(wave * MB * 16 + row) * kRedLd + col] = acc[b][c][r];
            }
    __syncthreads();
    // Sum over waves in wave order and store.
    for (int idx = tid; idx < MB * 16 * kCols; idx += kThreads) {
        const int row = idx / kCols, col = idx % kCols;
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s += red[(w * MB * 16 + row) * kRedLd + col];
        if (row < a.M && n0 + col < a.N) epi::store(C, a.ldc, a.epi, row, n0 + col, s);
    }
}

}  // namespace small
