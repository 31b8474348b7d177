// gemm_reg.h -- the 256 x 256 bf16 kernel for operands whose rows are not
// 16-byte aligned (odd leading dimensions, offset base pointers).
//
// Same tile, wave arrangement, LDS layout (XOR-swizzled 64-byte k-rows for
// K-contiguous operands, 512-byte n-rows for row-major B), MFMA inner loop
// and epilogue as the direct-load kernel in gemm_fast.h; only the
// global -> LDS step differs.  LDS-DMA needs dword-aligned sources, so here
// each thread fetches its 16-byte chunks with buffer loads into registers
// (gfx950 serves 16-byte loads at any 2-byte alignment), PF k-tiles ahead of
// the stage being filled, and writes them into the swizzled stage with
// ds_write_b128:
//
//   k-step 0 of k-tile t: multiply step 0, and between its MFMAs read the
//                         fragments of step 1 (first), store the registers
//                         of k-tile t+1 into the other stage, and issue the
//                         loads of k-tile t+1+PF into the freed registers;
//   k-step 1:             wait for LDS, barrier (stage t+1 complete, stage t
//                         fully read), multiply step 1 with the reads of
//                         step 0 of t+1 between its MFMAs.
//
// The interleave is fixed with sched_group_barrier: left to itself the
// compiler issued each step's fragment reads after most of the previous
// step's MFMAs, so their LDS latency showed at every step.
//
// The partial last k-tile (K mod 32 != 0) is loaded into a register set of
// its own in the tile's prologue, with the predicated loads described below,
// and stored and multiplied after the K loop; loaded after the K loop
// instead, its latency was paid once per tile in the open.
//
// A load is thus issued PF k-tiles before its registers are stored: with
// one 256 x 192 tile per CU a k-tile is 24 MFMAs (768 matrix-core cycles) per
// wave, and the loads come from L2 or the Infinity Cache, whose latency under
// load is one to two such k-tiles, so more than one register set in flight
// is what keeps the matrix cores fed.
//
// Bounds: rows past M / N and k-rows past K (row-major B) lie outside the
// per-tile buffer descriptors and load as zero.  A descriptor starts at the
// operand's address rounded down to 4 bytes (the difference goes into the
// offsets) and ends at the data's end rounded up to 4 bytes, so every dword
// it admits shares an aligned dword with valid data: nothing past the
// operand's pages is touched.  Range checks work on the dwords a load
// actually reads, which at 2-byte alignment need not be aligned ones, so a
// 16-byte chunk that straddles the end of the data may lose its last valid
// element; such chunks are only ever loaded element by element.  They occur
// in the last k-tile of K-contiguous operands (K % 8 != 0, so the tail
// path), and in the last k-row of row-major B when N % 8 != 0, which the
// host then also routes through the tail path (one k-tile fewer in the
// main loop).

#pragma once

namespace regpath {

using namespace fast;

// k per k-tile of the register kernel with RB bytes of K per LDS row
__host__ __device__ constexpr int bk_of(int rb) { return rb / 2; }

// Descriptor over [p, p + bytes) with its base rounded down to a dword;
// `shift` receives the byte offset of p from that base.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t span_rsrc(const uint8_t* p, int64_t bytes, int& shift) {
    shift = (int)((uintptr_t)p & 3);
    return make_rsrc(p - shift, (shift + bytes + 3) & ~(int64_t)3);
}

// PF: k-tiles held in registers ahead of the stage being filled (1, 2 or 4
// register sets; k-tile j lives in set j % PF).  BN: tile columns, 256 or
// 192 (wave tiles 128 x BN/2); the narrower tile lets the host match the
// tile count to the CU count.  RB: bytes of K per LDS row, 64 (k-tiles of
// 32, 2 MFMA steps) or 128 (k-tiles of 64, 4 steps: half the barriers and
// stage hand-offs per MFMA).
// FUSED: the fused epilogue of gemm_epi.h instead of the plain fp32 store.
template <int KIND, bool TAIL, int PF = 2, int BN = kTile, bool FUSED = false, int RB = 64>
__global__ __launch_bounds__(kThreads, 1) void gemm_reg_kernel(Args a) {
    static_assert(KIND == kNT || KIND == kNN, "bf16 only");
    static_assert(RB == 64 || RB == 128, "k-tile rows of 64 or 128 bytes");
    constexpr int BK = bk_of(RB);              // k per k-tile
    constexpr int KS = BK / 16;                // 16-deep MFMA steps per k-tile
    constexpr int OPB = kTile * RB;            // bytes per operand per stage
    constexpr int STAGE = 2 * OPB;
    constexpr int CPR = RB / 16;               // 16-byte chunks per K-contiguous row
    constexpr int NC = OPB / 16 / kThreads;    // 16-byte chunks of A per thread
    static_assert(PF == 1 || PF == 2 || PF == 4, "1, 2 or 4 register sets");
    // the K loop is unrolled by U k-tiles so that the stage (k-tile parity)
    // and the register set (k-tile mod PF) of every unrolled k-tile are
    // compile-time constants
    constexpr int U = PF > 2 ? PF : 2;
    static_assert(BN == 256 || BN == 192, "tile columns");
    constexpr int NBJ = BN / 64;      // 32-column MFMA blocks per wave tile
    constexpr int WTN = BN / 2;       // wave tile columns
    constexpr int CPK = BN / 8;       // row-major B: 16-byte chunks per k-row
    constexpr int NCB = BN * RB / 16 / kThreads;  // 16-byte chunks of B per thread
    __shared__ __attribute__((aligned(1024))) uint8_t st0[STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t st1[STAGE];
    __shared__ float evl[FUSED ? 3 * 256 : 1];  // fused epilogue: the tile's scales and biases

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5;
    const int l32 = lane & 31;

    // Chunk i of this thread.  K-contiguous operand: row idx / CPR, 16-byte
    // chunk idx % CPR of the row's RB bytes.  Row-major B: k-row idx / CPK,
    // columns 8 (idx % CPK) .. +7 (LDS rows keep the 512-byte pitch).
    int a_g[NC], b_g[NCB], a_l[NC], b_l[NCB];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int idx = i * kThreads + tid;
        const int r = idx / CPR, c = idx % CPR;
        a_g[i] = r * (int)a.lda_b + c * 16;
        a_l[i] = kc_off<RB>(r, c);
    }
#pragma unroll
    for (int i = 0; i < NCB; ++i) {
        const int idx = i * kThreads + tid;
        if constexpr (KIND == kNN) {
            const int kk = idx / CPK, cn = idx % CPK;
            b_g[i] = kk * (int)a.ldb_b + cn * 16;
            b_l[i] = OPB + nn_off(kk, cn * 8);
        } else {
            const int r = idx / CPR, c = idx % CPR;
            b_g[i] = r * (int)a.ldb_b + c * 16;
            b_l[i] = OPB + kc_off<RB>(r, c);
        }
    }

    // fragment read offsets (as in gemm_fast.h)
    int a_rd[KS], b_rd[KS], b_tr[NBJ];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        a_rd[ks] = kc_off<RB>(wm * kWaveTile + l32, 2 * ks + h);
        b_rd[ks] = OPB + kc_off<RB>(wn * WTN + l32, 2 * ks + h);
    }
    if constexpr (KIND == kNN) {
        const int g = lane >> 4, li = lane & 15;
#pragma unroll
        for (int j = 0; j < NBJ; ++j) {
            int n = wn * WTN + j * 32 + 16 * (g & 1) + 4 * (li & 3);
            int k = 8 * (g >> 1) + (li >> 2);
            b_tr[j] = OPB + nn_off(k, n);
        }
    }

    const int KT = a.kt_full;
    const int KTM = (KT + U - 1) / U * U;  // the k-tiles past KT are dead (zero)

    const int G = gridDim.x;
    for (int t = logical_block(a); t < a.num_tiles; t += G) {
        int tm, tn;
        tile_coords(a, t, tm, tn);
        const int m0 = tm * kTile, n0 = tn * BN;
        const int rows_a = min(kTile, a.M - m0);
        const int rows_b = min(BN, a.N - n0);
        EpiRegs epv{};
        if constexpr (FUSED) epv = epi_prefetch(a, m0, n0, BN, tid);
        int sa, sb;
        const __amdgpu_buffer_rsrc_t ra =
            span_rsrc(a.A + (int64_t)m0 * a.lda_b, (int64_t)(rows_a - 1) * a.lda_b + (int64_t)a.K * 2, sa);
        __amdgpu_buffer_rsrc_t rb;
        if constexpr (KIND == kNN)
            rb = span_rsrc(a.B + (int64_t)n0 * 2, (int64_t)(a.K - 1) * a.ldb_b + (int64_t)(a.N - n0) * 2, sb);
        else
            rb = span_rsrc(a.B + (int64_t)n0 * a.ldb_b, (int64_t)(rows_b - 1) * a.ldb_b + (int64_t)a.K * 2, sb);
        // k-tile j lives in register set j % PF
        i32x4 ra_reg[PF][NC], rb_reg[PF][NCB];
        // k-tile kt into register set q.  A dead k-tile (kt >= KT) reads
        // zeros without traffic: its scalar offset kDead puts every lane
        // past the descriptor's range (voffset < 2^31 and the range below
        // 2^31, so the sum cannot wrap).  Selecting the offset rather than a
        // second descriptor keeps the descriptors in scalar registers.
        constexpr int kDead = 0x7fffffff;
        // chunks W0 .. W1-1 of k-tile kt into register set q (chunk w < NC:
        // A's chunk w, else B's chunk w - NC)
        auto load_range = [&](auto qidx, auto w0c, auto w1c, int kt, bool live) {
            constexpr int q = decltype(qidx)::value;
            const int ka = live ? sa + kt * RB : kDead;
            const int kb = live ? sb + ((KIND == kNN) ? kt * BK * (int)a.ldb_b : kt * RB) : kDead;
            static_for<decltype(w0c)::value, decltype(w1c)::value>([&](auto wc) {
                constexpr int w = decltype(wc)::value;
                if constexpr (w < NC) ra_reg[q][w] = __builtin_amdgcn_raw_buffer_load_b128(ra, a_g[w], ka, 0);
                else rb_reg[q][w - NC] = __builtin_amdgcn_raw_buffer_load_b128(rb, b_g[w - NC], kb, 0);
            });
        };
        using W0 = std::integral_constant<int, 0>;
        using WN = std::integral_constant<int, NC + NCB>;
        // Partial k-tile KT, holding kvalid (1 .. BK) k.  Chunks lying wholly
        // inside the data are 16-byte loads; the chunk that straddles the end
        // of a row (K-contiguous operands) or of the last columns (row-major
        // B) is read as 2-byte elements, so no load reaches past the
        // operand's last element; the rest is zero.  Rows past M / N read as
        // zero through the descriptors.
        const int kvalid = a.K - KT * BK;
        // 8 elements from byte offset voff + soff, element e kept if e < n;
        // 2-byte loads never straddle the end of the data
        auto gather = [](__amdgpu_buffer_rsrc_t rs, int voff, int soff, int n) {
            i32x4 v = {0, 0, 0, 0};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t x = __builtin_amdgcn_raw_buffer_load_b16(rs, voff + 2 * e, soff, 0);
                if (e < n) v[e >> 1] |= (int)(x << (16 * (e & 1)));
            }
            return v;
        };
        i32x4 ta_reg[NC], tb_reg[NCB];  // the partial k-tile
        auto load_tail = [&]() {
#pragma unroll
            for (int i = 0; i < NC; ++i) {
                const int idx = i * kThreads + tid;
                const int c8 = 8 * (idx % CPR);
                i32x4 va = {0, 0, 0, 0};
                if (c8 + 8 <= kvalid)
                    va = __builtin_amdgcn_raw_buffer_load_b128(ra, a_g[i], sa + KT * RB, 0);
                else if (c8 < kvalid)
                    va = gather(ra, a_g[i], sa + KT * RB, kvalid - c8);
                ta_reg[i] = va;
            }
#pragma unroll
            for (int i = 0; i < NCB; ++i) {
                const int idx = i * kThreads + tid;
                i32x4 vb = {0, 0, 0, 0};
                if constexpr (KIND == kNN) {
                    const int kk = idx / CPK, n8 = 8 * (idx % CPK);
                    const int soff = sb + KT * BK * (int)a.ldb_b;
                    if (kk < kvalid) {
                        if (n8 + 8 <= rows_b)
                            vb = __builtin_amdgcn_raw_buffer_load_b128(rb, b_g[i], soff, 0);
                        else if (n8 < rows_b)
                            vb = gather(rb, b_g[i], soff, rows_b - n8);
                    }
                } else {
                    const int c8 = 8 * (idx % CPR);
                    if (c8 + 8 <= kvalid)
                        vb = __builtin_amdgcn_raw_buffer_load_b128(rb, b_g[i], sb + KT * RB, 0);
                    else if (c8 < kvalid)
                        vb = gather(rb, b_g[i], sb + KT * RB, kvalid - c8);
                }
                tb_reg[i] = vb;
            }
        };
        // k-tile kt into register set q: zero (no traffic) past the full
        // k-tiles
        auto load = [&](auto qidx, int kt) { load_range(qidx, W0{}, WN{}, kt, kt < KT); };
        // chunks W0 .. W1-1 of register set q into stage s
        auto store_range = [&](auto qidx, auto sidx, auto w0c, auto w1c) {
            constexpr int q = decltype(qidx)::value;
            uint8_t FAST_LDS* base = decltype(sidx)::value ? (uint8_t FAST_LDS*)st1 : (uint8_t FAST_LDS*)st0;
            static_for<decltype(w0c)::value, decltype(w1c)::value>([&](auto wc) {
                constexpr int w = decltype(wc)::value;
                if constexpr (w < NC) *(i32x4 FAST_LDS*)(base + a_l[w]) = ra_reg[q][w];
                else *(i32x4 FAST_LDS*)(base + b_l[w - NC]) = rb_reg[q][w - NC];
            });
        };
        auto store = [&](auto qidx, auto sidx) { store_range(qidx, sidx, W0{}, WN{}); };
        auto read_frags = [&](auto sidx, int ks, bf16x8* fa, bf16x8* fb) {
            const uint8_t FAST_LDS* base =
                decltype(sidx)::value ? (const uint8_t FAST_LDS*)st1 : (const uint8_t FAST_LDS*)st0;
#pragma unroll
            for (int i = 0; i < kBlocks; ++i) fa[i] = *(const bf16x8 FAST_LDS*)(base + a_rd[ks] + i * 32 * RB);
#pragma unroll
            for (int j = 0; j < NBJ; ++j) {
                if constexpr (KIND == kNN) {
                    const uint8_t FAST_LDS* p = base + b_tr[j] + ks * 16 * 512;
                    bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 FAST_LDS*)p);
                    bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 FAST_LDS*)(p + 4 * 512));
                    fb[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                } else {
                    fb[j] = *(const bf16x8 FAST_LDS*)(base + b_rd[ks] + j * 32 * RB);
                }
            }
        };

        f32x16 acc[kBlocks][NBJ];
#pragma unroll
        for (int i = 0; i < kBlocks; ++i)
#pragma unroll
            for (int j = 0; j < NBJ; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
        auto mfma = [&](const bf16x8* fa, const bf16x8* fb) {
#pragma unroll
            for (int i = 0; i < kBlocks; ++i)
#pragma unroll
                for (int j = 0; j < NBJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        };
        // Instruction order of a k-step (sched_group_barrier): MFMA slot m is
        // followed by the memory instructions given it.  Steps 0 .. KS-2:
        // the NR fragment reads of the next step over the first half of the
        // MFMAs, then the step's share NWS of the stores into the next stage,
        // then as many loads of a later k-tile (they reuse the stored
        // registers).  Step KS-1: the NR reads of the next k-tile's step 0
        // over the first half of the MFMAs, so that they have landed when
        // that step's MFMAs start.
        constexpr int NMF = kBlocks * NBJ;
        constexpr int NR = (KIND == kNN) ? kBlocks + 2 * NBJ : kBlocks + NBJ;
        constexpr int NW = NC + NCB;
        auto interleave0 = [&](auto nwc) {
            constexpr int NWS = decltype(nwc)::value;
            static_for<0, NMF>([&](auto mc) {
                constexpr int m = decltype(mc)::value;
                constexpr int H = NMF / 2;
                // reads spread over slots 0 .. H-1, stores and loads over H .. NMF-1
                constexpr int r0 = m < H ? m * NR / H : NR, r1 = m < H ? (m + 1) * NR / H : NR;
                constexpr int w0 = m < H ? 0 : (m - H) * NWS / (NMF - H);
                constexpr int w1 = m < H ? 0 : (m + 1 - H) * NWS / (NMF - H);
                __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
                if constexpr (r1 > r0) __builtin_amdgcn_sched_group_barrier(kSgDsRead, r1 - r0, 0);
                if constexpr (w1 > w0) {
                    __builtin_amdgcn_sched_group_barrier(kSgDsWrite, w1 - w0, 0);
                    __builtin_amdgcn_sched_group_barrier(kSgVmem, w1 - w0, 0);
                }
            });
        };
        auto interleave1 = [&]() {
            static_for<0, NMF>([&](auto mc) {
                constexpr int m = decltype(mc)::value;
                constexpr int H = NMF / 2;
                constexpr int r0 = m < H ? m * NR / H : NR, r1 = m < H ? (m + 1) * NR / H : NR;
                __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
                if constexpr (r1 > r0) __builtin_amdgcn_sched_group_barrier(kSgDsRead, r1 - r0, 0);
            });
        };

        // prologue: k-tile 0 into stage 0, k-tiles 1 .. PF in flight to
        // registers (k-tile j in set j % PF)
        using Z = std::integral_constant<int, 0>;
        load(Z{}, 0);
        static_for<1, PF>([&](auto qc) { load(qc, decltype(qc)::value); });
        // the partial k-tile after k-tile 0: the element loads of a
        // straddling chunk wait for their data inside their branch, and that
        // wait then overlaps the wait for k-tile 0 the prologue has anyway
        if constexpr (TAIL) load_tail();
        store(Z{}, Z{});
        load(Z{}, PF);
        wait_lgkm0();
        barrier();
        bf16x8 F0a[kBlocks], F0b[NBJ], F1a[kBlocks], F1b[NBJ];
        read_frags(std::integral_constant<int, 0>{}, 0, F0a, F0b);

        auto body = [&](auto qidx, int kt) {
            constexpr int q = decltype(qidx)::value;  // kt % U
            using sidx = std::integral_constant<int, q % 2>;
            constexpr int sn = (q % 2) ^ 1;
            // k-steps 0 .. KS-2: stage of k-tile kt+1 <- registers and loads
            // of kt+1+PF, a share per step, fragments of the next step.
            // k-tile kt+1 sits in set (kt+1) % PF; kt+1+PF goes there next.
            using Q = std::integral_constant<int, (q + 1) % PF>;
            static_for<0, KS>([&](auto ksc) {
                constexpr int ks = decltype(ksc)::value;
                bf16x8* ca = (ks % 2) ? F1a : F0a;
                bf16x8* cb = (ks % 2) ? F1b : F0b;
                bf16x8* na = (ks % 2) ? F0a : F1a;
                bf16x8* nb = (ks % 2) ? F0b : F1b;
                if constexpr (ks + 1 < KS) {
                    using w0 = std::integral_constant<int, ks * NW / (KS - 1)>;
                    using w1 = std::integral_constant<int, (ks + 1) * NW / (KS - 1)>;
                    read_frags(sidx{}, ks + 1, na, nb);
                    store_range(Q{}, std::integral_constant<int, sn>{}, w0{}, w1{});
                    load_range(Q{}, w0{}, w1{}, kt + 1 + PF, kt + 1 + PF < KT);
                    mfma(ca, cb);
                    interleave0(std::integral_constant<int, w1::value - w0::value>{});
                    __builtin_amdgcn_sched_barrier(0);
                } else {
                    // last k-step: stage sn complete, stage s fully read
                    wait_lgkm0();
                    barrier();
                    read_frags(std::integral_constant<int, sn>{}, 0, na, nb);
                    mfma(ca, cb);
                    interleave1();
                    __builtin_amdgcn_sched_barrier(0);
                }
            });
        };
        for (int kt0 = 0; kt0 < KTM; kt0 += U) {
            static_for<0, U>([&](auto qc) { body(qc, kt0 + decltype(qc)::value); });
        }

        if constexpr (TAIL) {
            // the last body ended with a barrier after every wave's reads of
            // k-tile data in stage 0 (KTM is even, so stage 0 is free; the
            // reads that follow that barrier fetch the unused dead k-tile)
            uint8_t FAST_LDS* base = (uint8_t FAST_LDS*)st0;
#pragma unroll
            for (int i = 0; i < NC; ++i) *(i32x4 FAST_LDS*)(base + a_l[i]) = ta_reg[i];
#pragma unroll
            for (int i = 0; i < NCB; ++i) *(i32x4 FAST_LDS*)(base + b_l[i]) = tb_reg[i];
            wait_lgkm0();
            barrier();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                read_frags(std::integral_constant<int, 0>{}, ks, F0a, F0b);
                mfma(F0a, F0b);
            }
        }

        if constexpr (FUSED) {
            epi_stage((float FAST_LDS*)evl, epv, tid);
            wait_lgkm0();
            barrier();
        }
        store_c<NBJ, FUSED>(a, acc, m0 + wm * kWaveTile, n0 + wn * WTN, h, l32, (const float FAST_LDS*)evl,
                            wm * kWaveTile, wn * WTN);
        wait_lgkm0();
        barrier();
    }
}

}  // namespace regpath
