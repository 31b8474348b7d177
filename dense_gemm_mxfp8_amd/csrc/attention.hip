// attention.hip -- fused attention forward for gfx950 and its C ABI
// (include/attention.h).
//
// "Modern GPU Programming For MLSys - 书籍总结", part IV (5.1-5.3): attention
// is two matrix products with a softmax between them; the running maximum of
// each row changes as key blocks arrive, so the partial output is rescaled
// before the next value product adds to it; causal masking and grouped-query
// heads are part of the kernel.  The pages build it for Blackwell (TMEM
// accumulators, warp roles); here it is one gfx950 workgroup per block of
// 128 query rows of one head, four waves of 32 rows each, streaming blocks of
// 64 keys through LDS:
//
//   * scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: K rows come from LDS as the A operand and the
//     wave's 32 query rows stay in registers as the B operand for the whole
//     kernel.  Accumulator register r of lane l then holds one query
//     (l % 32) and key row 8 (r/4) + 4 (l/32) + r % 4 of the 32-key tile.
//   * the K rows are fed to the MFMA in a permuted order (bits 2 and 3 of the
//     row index swapped), so that register r of lane l holds key
//     16 (r/8) + 8 (l/32) + r % 8: registers 8u .. 8u+7 are then exactly the
//     8 consecutive keys the B operand of a 16-key MFMA step wants from that
//     lane.  The probabilities go from the score accumulators into the value
//     product as bf16 with no data movement between lanes.
//   * the value product is computed transposed too, O^T = V^T P^T: V^T
//     fragments are read from the row-major V tile with ds_read_b64_tr_b16,
//     and the O accumulators keep the query in the lane, like the softmax
//     state (running max, running sum), so rescaling O is a multiply by a
//     per-lane scalar.  A row's reference maximum moves only when a block's
//     maximum passes it by more than 8 (log2 units), so weights stay below
//     2^8 and the rescale of O (skipped when no row of the wave moved, its
//     factor then being exactly 1) is rare after the first block.
//   * the two halves of the wave hold different keys of the same query; the
//     row maximum is combined across them with v_permlane32_swap, and the
//     row sums are kept per lane and combined once at the end.
//   * K/V tiles are double-buffered in LDS: the DMA of block t+1
//     (buffer_load ... lds, 16 bytes per lane, no VGPR round trip) is issued
//     into the other buffer before block t is multiplied; one wait and one
//     barrier per block.  Rows past seq_k lie outside the tile's buffer
//     descriptor and load as zero (and are masked).
//   * LDS rows are XOR-swizzled in 16-byte chunks so that both the K
//     fragment reads (16 rows, one chunk) and the transposing V reads
//     (4 rows x 4 chunks per 32 lanes) hit distinct banks.
//   * two workgroups per CU: while one wave runs its softmax (VALU), the
//     other wave on the SIMD keeps the matrix core busy.
//   * workgroup ids are remapped so that the query blocks of one head run on
//     one XCD and share its L2; for causal masks the blocks with the most
//     keys start first.

#include <hip/hip_runtime.h>

#include <math.h>
#include <mutex>
#include <stdint.h>
#include <type_traits>
#include <stdlib.h>
#include <string.h>

#include "attention.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

#define ALDS __attribute__((address_space(3)))

constexpr int kThreads = 256;  // 4 waves
constexpr int kQW = 32;        // query rows per wave
constexpr int kQB = 128;       // query rows per workgroup
constexpr int kKB = 64;        // keys per block
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format
constexpr float kLazy = 8.0f;  // log2 headroom of the lazily moved row maximum

struct Params {
    const uint8_t* Q;
    const uint8_t* K;
    const uint8_t* V;
    uint8_t* O;   // fp32 or bf16 elements, as o_bf16 says
    float* lse;
    int64_t q_b, q_h, k_b, k_h, v_b, v_h, o_b, o_h;  // batch / head strides, elements
    int q_s, k_s, v_s, o_s;                          // sequence strides, elements
    int Hq, group, Sq, Sk, qblocks, off;             // off = Sk - Sq
    float c;      // scale * log2(e)
    float scale;
    int xcd_remap;
    int prio;     // raise the wave's issue priority around its MFMA phases
    int o_bf16;   // store O as bf16 (nearest even) instead of fp32
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    int n = bytes > 0x7fffffff ? 0x7fffffff : (bytes < 0 ? 0 : (int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kRsrcWord3);
}

// Chunk swizzles (16-byte chunks, rows of 2 D bytes).
template <int D>
__device__ __forceinline__ int kswz(int row) {
    if constexpr (D == 128) return row & 15;
    else return (row >> 1) & 7;
}
template <int D>
__device__ __forceinline__ int vswz(int row) {
    if constexpr (D == 128) return (row & 3) << 2;
    else return ((row >> 1) & 1) << 2;
}

// s_waitcnt vmcnt(0), leaving the other counters alone.
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); }

// This wave's DMA instructions of one K or V tile: instruction n = 4 i + wave
// fills LDS bytes [1024 n, 1024 n + 1024) from the lane offsets off[i].
template <int NDMA>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t rs, uint8_t ALDS* dst, const int (&off)[NDMA],
                                         int wave) {
#pragma unroll
    for (int i = 0; i < NDMA; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (void ALDS*)(dst + (4 * i + wave) * 1024), 16, off[i], 0, 0,
                                                 0);
}

// K row fed to MFMA A-row m: bits 2 and 3 of m swapped.
__device__ __forceinline__ int perm_row(int m) {
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Own value and the value of the lane 32 away (the other half of the wave
// holds the other keys of the same query), in one v_permlane32_swap: it
// swaps lanes 32-63 of its first operand with lanes 0-31 of its second, so
// with both holding x, every lane ends with its own x in one register and its
// partner's in the other.  Written as an instruction rather than the builtin,
// whose two results the compiler treats as one value; the s_nops cover the
// VALU-write / permlane-read hazards that the compiler cannot see inside asm.
// Both halves combine the pair with a symmetric operation and end with the
// same value.
__device__ __forceinline__ void own_and_partner(float x, float& a, float& b) {
    a = x;
    b = x;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float half_max(float x) {
    float a, b;
    own_and_partner(x, a, b);
    return fmaxf(a, b);
}
__device__ __forceinline__ float half_sum(float x) {
    float a, b;
    own_and_partner(x, a, b);
    return a + b;
}

// G: query groups of 32 rows per wave.  With G = 2 every K and V fragment
// read from LDS feeds two MFMAs (half the LDS reads per FLOP) at one wave per
// SIMD; with G = 1 two waves share each SIMD.
template <int D, bool CAUSAL, int G>
__global__ __launch_bounds__(kThreads, G == 1 ? 2 : 1) void attn_fwd_kernel(Params p) {
    // the host pass only needs the launch stub; the body uses device-only
    // types (buffer descriptors, LDS address space)
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int RB = 2 * D;                  // bytes per LDS row
    constexpr int NCH = D / 8;                 // 16-byte chunks per row
    constexpr int KT = kKB * RB;               // bytes of one K or V tile
    constexpr int DS = D / 16;                 // MFMA steps over d
    constexpr int DT = D / 32;                 // 32-row d tiles of O^T
    constexpr int QB = kQB * G;                // query rows per workgroup
    // K and V tiles of the two buffers, each its own __shared__ object: the
    // compiler can then tell the in-flight DMA into one buffer apart from the
    // fragment reads of the other and does not make the reads wait for it
    __shared__ __attribute__((aligned(16))) uint8_t k_lds0[KT];
    __shared__ __attribute__((aligned(16))) uint8_t k_lds1[KT];
    __shared__ __attribute__((aligned(16))) uint8_t v_lds0[KT];
    __shared__ __attribute__((aligned(16))) uint8_t v_lds1[KT];

    // ---- (batch, head, query block) of this workgroup
    int bid = blockIdx.x;
    if (p.xcd_remap) bid = (bid & 7) * (int)(gridDim.x >> 3) + (bid >> 3);
    const int bh = bid / p.qblocks;
    const int qb = p.qblocks - 1 - (bid - bh * p.qblocks);
    const int b = bh / p.Hq;
    const int h = bh - b * p.Hq;
    const int hk = h / p.group;
    const int q0 = qb * QB;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int qw0 = q0 + wave * kQW * G;  // first query row of this wave
    int myq[G];                           // this lane's query row in group g
#pragma unroll
    for (int g = 0; g < G; ++g) myq[g] = qw0 + kQW * g + l32;

    // keys any row of the workgroup / of this wave can see
    int kend = p.Sk, wend = p.Sk;
    if constexpr (CAUSAL) {
        const int qlast = min(q0 + QB, p.Sq);
        kend = min(p.Sk, qlast + p.off);
        wend = min(p.Sk, min(qw0 + kQW * G, p.Sq) + p.off);
    }
    const int nt = kend > 0 ? (kend + kKB - 1) / kKB : 0;
    const bool wave_rows = qw0 < p.Sq;

    const uint8_t* qbase = p.Q + 2 * (b * p.q_b + h * p.q_h);
    const uint8_t* kbase = p.K + 2 * (b * p.k_b + hk * p.k_h);
    const uint8_t* vbase = p.V + 2 * (b * p.v_b + hk * p.v_h);
    const int64_t qbytes = p.Sq > 0 ? 2 * ((int64_t)(p.Sq - 1) * p.q_s + D) : 0;
    const int64_t kbytes = p.Sk > 0 ? 2 * ((int64_t)(p.Sk - 1) * p.k_s + D) : 0;
    const int64_t vbytes = p.Sk > 0 ? 2 * ((int64_t)(p.Sk - 1) * p.v_s + D) : 0;

    // ---- this wave's query rows, resident as the B operand of S^T = K Q^T
    bf16x8 qf[G][DS];
    {
        const auto rq = make_rsrc(qbase, qbytes);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int voff = myq[g] * p.q_s * 2 + 16 * hh;
#pragma unroll
            for (int s = 0; s < DS; ++s)
                qf[g][s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, voff + 32 * s, 0, 0));
        }
    }

    // ---- K/V tiles go global -> LDS by buffer_load ... lds: one wave
    // instruction fills 1 KiB of LDS (lane i at byte 16 i), i.e. RPI rows;
    // the lane fetches the global chunk that the swizzle places there.  Each
    // lane's whole offset (row and chunk) is in voffset, so rows past seq_k
    // fall outside the tile's descriptor and load as zero.
    constexpr int RPI = 1024 / RB;             // rows per DMA instruction
    constexpr int NDMA = kKB / RPI / 4;        // instructions per wave per tensor
    int k_dma[NDMA], v_dma[NDMA];
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
        const int n = 4 * i + wave;            // instruction index within the tile
        const int row = n * RPI + lane / NCH;
        const int pc = lane % NCH;             // physical chunk in LDS
        k_dma[i] = row * p.k_s * 2 + 16 * (pc ^ kswz<D>(row));
        v_dma[i] = row * p.v_s * 2 + 16 * (pc ^ vswz<D>(row));
    }

    // ---- per-lane constants of the fragment reads
    // K: A-row m = l32 reads key row perm_row(l32) (+32 for the second tile),
    // 16-byte chunk 2 s + hh at step s
    int k_rd[DS];
    {
        const int r = perm_row(l32);
#pragma unroll
        for (int s = 0; s < DS; ++s) k_rd[s] = r * RB + (((2 * s + hh) ^ kswz<D>(r)) << 4);
    }
    // V^T: ds_read_b64_tr_b16 groups of 16 lanes read 4 key rows x 16 d
    int v_rd[DT];
    {
        const int g = lane >> 4, li = lane & 15;
        const int row = 8 * (g >> 1) + (li >> 2);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int d = 32 * dt + 16 * (g & 1) + 4 * (li & 3);
            v_rd[dt] = row * RB + ((((d >> 3)) ^ vswz<D>(row)) << 4) + ((d & 7) << 1);
        }
    }

    auto k_tile = [&](auto BUF) {
        return (uint8_t ALDS*)(decltype(BUF)::value ? k_lds1 : k_lds0);
    };
    auto v_tile = [&](auto BUF) {
        return (uint8_t ALDS*)(decltype(BUF)::value ? v_lds1 : v_lds0);
    };
    auto issue_loads = [&](int t, auto BUF) {
        const int64_t kofs = (int64_t)t * kKB * p.k_s * 2;
        const int64_t vofs = (int64_t)t * kKB * p.v_s * 2;
        dma_tile<NDMA>(make_rsrc(kbase + kofs, kbytes - kofs), k_tile(BUF), k_dma, wave);
        dma_tile<NDMA>(make_rsrc(vbase + vofs, vbytes - vofs), v_tile(BUF), v_dma, wave);
    };

    f32x16 oacc[G][DT];
    float m_run[G], l_run[G];  // reference max of the raw scores q.k of the row; this lane's part of its sum
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            for (int r = 0; r < 16; ++r) oacc[g][dt][r] = 0.0f;
        m_run[g] = -INFINITY;
        l_run[g] = 0.0f;
    }

    if (nt > 0) issue_loads(0, std::integral_constant<int, 0>{});
    wait_vm0();
    __syncthreads();

    // One block; the LDS buffer is a compile-time constant (the loop is
    // unrolled by two), so buffer and tile offsets fold into the LDS
    // instructions' immediate offsets.
    auto block = [&](auto BUF, int t) {
        constexpr int buf = decltype(BUF)::value;
        const int k0 = t * kKB;
        if (t + 1 < nt) issue_loads(t + 1, std::integral_constant<int, buf ^ 1>{});

        if (wave_rows && k0 < wend) {
            const uint8_t ALDS* kt = k_tile(BUF);
            const uint8_t ALDS* vt = v_tile(BUF);
            // ---- S^T = K Q^T over the 64 keys (two 32-key tiles); each K
            // fragment feeds the G query groups
            if (p.prio) __builtin_amdgcn_s_setprio(1);
            f32x16 sacc[G][2];
#pragma unroll
            for (int g = 0; g < G; ++g)
                for (int st = 0; st < 2; ++st)
                    for (int r = 0; r < 16; ++r) sacc[g][st][r] = 0.0f;
            if constexpr (CAUSAL) {
                // Causal launches run below the power limit, where LDS
                // latency shows: their K fragments run KLA steps ahead of the
                // MFMAs (a ring of KLA + 1 steps).  Measured: +4% causal, -1%
                // unmasked (power-limited), so the unmasked form keeps reads
                // next to their MFMAs.
                constexpr int KLA = 2;
                bf16x8 kf[KLA + 1][2];
#pragma unroll
                for (int s = 0; s < KLA; ++s)
#pragma unroll
                    for (int st = 0; st < 2; ++st) kf[s][st] = *(const bf16x8 ALDS*)(kt + k_rd[s] + st * 32 * RB);
#pragma unroll
                for (int s = 0; s < DS; ++s) {
                    if (s + KLA < DS) {
#pragma unroll
                        for (int st = 0; st < 2; ++st)
                            kf[(s + KLA) % (KLA + 1)][st] = *(const bf16x8 ALDS*)(kt + k_rd[s + KLA] + st * 32 * RB);
                    }
#pragma unroll
                    for (int st = 0; st < 2; ++st) {
#pragma unroll
                        for (int g = 0; g < G; ++g)
                            sacc[g][st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s % (KLA + 1)][st], qf[g][s],
                                                                                   sacc[g][st], 0, 0, 0);
                    }
                }
                // keep that order: KLA steps of reads first, then per step two
                // reads and the step's MFMAs
                __builtin_amdgcn_sched_group_barrier(0x100, 2 * KLA, 0);
#pragma unroll
                for (int s = 0; s < DS; ++s) {
                    if (s + KLA < DS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 2 * G, 0);
                }
            } else {
#pragma unroll
                for (int s = 0; s < DS; ++s) {
#pragma unroll
                    for (int st = 0; st < 2; ++st) {
                        const bf16x8 kf = *(const bf16x8 ALDS*)(kt + k_rd[s] + st * 32 * RB);
#pragma unroll
                        for (int g = 0; g < G; ++g)
                            sacc[g][st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[g][s], sacc[g][st], 0, 0, 0);
                    }
                }
            }
            if (p.prio) __builtin_amdgcn_s_setprio(0);
            // ---- mask: keys past seq_k, and (causal) keys after the row's limit
            const bool need_mask = (k0 + kKB > p.Sk) || (CAUSAL && k0 + kKB - 1 > qw0 + p.off);
            if (need_mask) {
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const int lim = CAUSAL ? min(p.Sk - 1, myq[g] + p.off) : p.Sk - 1;
#pragma unroll
                    for (int st = 0; st < 2; ++st)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int key = k0 + 32 * st + 16 * (r >> 3) + 8 * hh + (r & 7);
                            if (key > lim) sacc[g][st][r] = -INFINITY;
                        }
                }
            }
            // ---- online softmax (reference max, rescale), per group
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float mx = sacc[g][0][0];
#pragma unroll
                for (int st = 0; st < 2; ++st)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[g][st][r]);
                mx = half_max(mx);
                // The reference maximum moves only when the block's maximum
                // passes it by more than kLazy in log2 units: weights then stay
                // below 2^kLazy, O and the row sum keep one common reference,
                // and the rescale of O is skipped for most blocks.
                const bool move = (mx - m_run[g]) * p.c > kLazy;  // true while m_run = -inf and mx finite
                const float m_new = move ? mx : m_run[g];
                const float alpha =
                    (m_run[g] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((m_run[g] - m_new) * p.c);
                const float mc = (m_new == -INFINITY) ? 0.0f : m_new * p.c;
                m_run[g] = m_new;
                float psum = 0.0f;
#pragma unroll
                for (int st = 0; st < 2; ++st)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[g][st][r], p.c, -mc));
                        sacc[g][st][r] = e;
                        psum += e;
                    }
                l_run[g] = l_run[g] * alpha + psum;
                if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                        for (int r = 0; r < 16; ++r) oacc[g][dt][r] *= alpha;
                }
            }
            // ---- O^T += V^T P^T, 16 keys per MFMA step; each V fragment
            // feeds the G query groups
            if (p.prio) __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int st = 0; st < 2; ++st) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    bf16x8 pf[G];
#pragma unroll
                    for (int g = 0; g < G; ++g)
#pragma unroll
                        for (int x = 0; x < 8; ++x) pf[g][x] = (__bf16)sacc[g][st][8 * u + x];
                    const int krow = 32 * st + 16 * u;
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) {
                        const uint8_t ALDS* pv = vt + v_rd[dt] + krow * RB;
                        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 ALDS*)pv);
                        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 ALDS*)(pv + 4 * RB));
                        const bf16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                        for (int g = 0; g < G; ++g)
                            oacc[g][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[g], oacc[g][dt], 0, 0, 0);
                    }
                }
            }
        }

        if (p.prio) __builtin_amdgcn_s_setprio(0);
        wait_vm0();  // this wave's DMA of block t + 1 has landed in LDS
        __syncthreads();
    };
    for (int t = 0; t < nt; t += 2) {
        block(std::integral_constant<int, 0>{}, t);
        if (t + 1 < nt) block(std::integral_constant<int, 1>{}, t + 1);
    }

    // ---- normalise and store
    if (!wave_rows) return;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float l_tot = half_sum(l_run[g]);
        if (myq[g] < p.Sq) {
            const int64_t orow = (b * p.o_b + h * p.o_h) + (int64_t)myq[g] * p.o_s;  // elements
            // no visible key: every weight was 0 (a visible row has one weight of exactly 1)
            const bool empty = l_tot == 0.0f;
            // a / l correctly rounded, one division per row: with the
            // correctly rounded reciprocal r, q = a r is within an ulp and one
            // fma residual step q + r (a - q l) rounds to the IEEE quotient
            // (Markstein's correction)
            const float r = empty ? 0.0f : 1.0f / l_tot;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    f32x4 v;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float a = oacc[g][dt][4 * i + j];
                        const float q = a * r;
                        v[j] = empty ? 0.0f : __builtin_fmaf(__builtin_fmaf(-q, l_tot, a), r, q);
                    }
                    const int64_t e = orow + 32 * dt + 8 * i + 4 * hh;
                    if (p.o_bf16) {
                        bf16x4 w;
#pragma unroll
                        for (int j = 0; j < 4; ++j) w[j] = (__bf16)v[j];  // nearest even
                        *(bf16x4*)(p.O + 2 * e) = w;
                    } else {
                        *(f32x4*)(p.O + 4 * e) = v;
                    }
                }
            if (p.lse && hh == 0)
                p.lse[((int64_t)b * p.Hq + h) * p.Sq + myq[g]] =
                    empty ? -INFINITY : m_run[g] * p.scale + logf(l_tot);
        }
    }
#endif
}

struct DeviceInfo {
    int checked;
    int supported;
};

constexpr int kMaxDevices = 64;
DeviceInfo g_devices[kMaxDevices];
std::mutex g_devices_mutex;

int device_supported() {
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
        d.checked = 1;
    }
    return d.supported ? GEMM_OK : GEMM_ERR_UNSUPPORTED;
}

// Query groups per wave: 1 (two waves per SIMD, the faster form measured on
// MI355X) unless the environment variable ATTN_GROUPS=2 selects two groups
// (one wave per SIMD, half the LDS reads per FLOP); read at every call.
int attn_groups() {
    const char* e = getenv("ATTN_GROUPS");
    return (e && e[0] == '2') ? 2 : 1;
}

// Wave priority around the MFMA phases.  Measurement builds
// (-DLIBGEMM_MEASURE) turn it off with ATTN_PRIO=0; the default build always
// raises it.
int attn_prio() {
#ifdef LIBGEMM_MEASURE
    const char* e = getenv("ATTN_PRIO");
    return (e && e[0] == '0') ? 0 : 1;
#else
    return 1;
#endif
}

bool aligned(const void* p, uintptr_t a) { return (((uintptr_t)p) & (a - 1)) == 0; }

// Strides (batch, head, seq) of a tensor, defaulting to dense [B][H][S][D].
void strides_of(const int64_t* given, int64_t H, int64_t S, int64_t D, int64_t out[3]) {
    if (given) {
        out[0] = given[0];
        out[1] = given[1];
        out[2] = given[2];
    } else {
        out[2] = D;
        out[1] = S * D;
        out[0] = H * S * D;
    }
}

bool strides_ok(const int64_t s[3], int64_t mult) {
    for (int i = 0; i < 3; ++i)
        if (s[i] < 0 || s[i] % mult) return false;
    return true;
}

// rows * stride elements of esize bytes (plus one row of D) fit a 31-bit offset
bool span_ok(int64_t rows, int64_t stride, int64_t D, int64_t esize) {
    return (rows * stride + D) * esize <= (int64_t)0x7fffffff;
}

template <int D, bool CAUSAL, int G>
int launch(const Params& p, int grid, hipStream_t stream) {
    hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, G>), dim3(grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

}  // namespace

extern "C" int attn_fwd_bf16_out(int64_t batch, int64_t heads_q, int64_t heads_kv,
                                 int64_t seq_q, int64_t seq_k, int64_t head_dim,
                                 const void* Q, const int64_t* q_strides,
                                 const void* K, const int64_t* k_strides,
                                 const void* V, const int64_t* v_strides,
                                 void* O, const int64_t* o_strides, int out_type,
                                 float* lse, float scale, int causal, void* stream) {
    if (out_type != GEMM_OUT_F32 && out_type != GEMM_OUT_BF16) return GEMM_ERR_INVALID_ARG;
    const int64_t o_size = out_type == GEMM_OUT_BF16 ? 2 : 4;
    if (batch < 0 || seq_q < 0 || seq_k < 0 || heads_q < 1 || heads_kv < 1) return GEMM_ERR_INVALID_ARG;
    if (heads_q % heads_kv != 0) return GEMM_ERR_INVALID_ARG;
    if (head_dim != 64 && head_dim != 128) return GEMM_ERR_INVALID_ARG;
    if (!(scale > 0.0f) || !isfinite(scale)) return GEMM_ERR_INVALID_ARG;
    if (batch > INT32_MAX || heads_q > INT32_MAX || seq_q > INT32_MAX - 256 || seq_k > INT32_MAX - 256)
        return GEMM_ERR_INVALID_ARG;
    int64_t qs[3], ks[3], vs[3], os[3];
    strides_of(q_strides, heads_q, seq_q, head_dim, qs);
    strides_of(k_strides, heads_kv, seq_k, head_dim, ks);
    strides_of(v_strides, heads_kv, seq_k, head_dim, vs);
    strides_of(o_strides, heads_q, seq_q, head_dim, os);
    if (!strides_ok(qs, 8) || !strides_ok(ks, 8) || !strides_ok(vs, 8) || !strides_ok(os, 4))
        return GEMM_ERR_INVALID_ARG;
    if (qs[2] < head_dim || ks[2] < head_dim || vs[2] < head_dim || os[2] < head_dim)
        return GEMM_ERR_INVALID_ARG;
    if (!span_ok(seq_q + 2 * kQB, qs[2], head_dim, 2) || !span_ok(seq_q + 2 * kQB, os[2], head_dim, o_size) ||
        !span_ok(seq_k + kKB, ks[2], head_dim, 2) || !span_ok(seq_k + kKB, vs[2], head_dim, 2))
        return GEMM_ERR_INVALID_ARG;
    const bool rows = batch > 0 && seq_q > 0;
    if (rows && (Q == nullptr || O == nullptr)) return GEMM_ERR_INVALID_ARG;
    if (rows && seq_k > 0 && (K == nullptr || V == nullptr)) return GEMM_ERR_INVALID_ARG;
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 4 * o_size) || !aligned(lse, 4))
        return GEMM_ERR_INVALID_ARG;
    const int rc = device_supported();
    if (rc != GEMM_OK) return rc;
    if (!rows) return GEMM_OK;

    Params p;
    p.Q = (const uint8_t*)Q;
    p.K = (const uint8_t*)K;
    p.V = (const uint8_t*)V;
    p.O = (uint8_t*)O;
    p.o_bf16 = out_type == GEMM_OUT_BF16;
    p.lse = lse;
    p.q_b = qs[0];
    p.q_h = qs[1];
    p.q_s = (int)qs[2];
    p.k_b = ks[0];
    p.k_h = ks[1];
    p.k_s = (int)ks[2];
    p.v_b = vs[0];
    p.v_h = vs[1];
    p.v_s = (int)vs[2];
    p.o_b = os[0];
    p.o_h = os[1];
    p.o_s = (int)os[2];
    p.Hq = (int)heads_q;
    p.group = (int)(heads_q / heads_kv);
    p.Sq = (int)seq_q;
    p.Sk = (int)seq_k;
    const int G = attn_groups();
    p.qblocks = (int)((seq_q + kQB * G - 1) / (kQB * G));
    p.off = (int)(seq_k - seq_q);
    p.scale = scale;
    p.c = (float)((double)scale * 1.4426950408889634);  // log2(e)
    const int64_t grid = batch * heads_q * p.qblocks;
    if (grid > INT32_MAX) return GEMM_ERR_INVALID_ARG;
    p.xcd_remap = (grid % 8 == 0) ? 1 : 0;
    p.prio = attn_prio();
    hipStream_t st = (hipStream_t)stream;
    const bool c = causal != 0;
    if (G == 2) {
        if (head_dim == 128)
            return c ? launch<128, true, 2>(p, (int)grid, st) : launch<128, false, 2>(p, (int)grid, st);
        return c ? launch<64, true, 2>(p, (int)grid, st) : launch<64, false, 2>(p, (int)grid, st);
    }
    if (head_dim == 128)
        return c ? launch<128, true, 1>(p, (int)grid, st) : launch<128, false, 1>(p, (int)grid, st);
    return c ? launch<64, true, 1>(p, (int)grid, st) : launch<64, false, 1>(p, (int)grid, st);
}

extern "C" int attn_fwd_bf16(int64_t batch, int64_t heads_q, int64_t heads_kv,
                             int64_t seq_q, int64_t seq_k, int64_t head_dim,
                             const void* Q, const int64_t* q_strides,
                             const void* K, const int64_t* k_strides,
                             const void* V, const int64_t* v_strides,
                             float* O, const int64_t* o_strides,
                             float* lse, float scale, int causal, void* stream) {
    return attn_fwd_bf16_out(batch, heads_q, heads_kv, seq_q, seq_k, head_dim, Q, q_strides, K, k_strides, V,
                             v_strides, O, o_strides, GEMM_OUT_F32, lse, scale, causal, stream);
}
