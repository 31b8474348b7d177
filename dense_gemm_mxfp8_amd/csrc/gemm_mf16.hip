// gemm_mf16.hip -- the bf16 instances (NT and NN: plain fp32 product, fused
// epilogue, split-K units, dynamic schedule) of the 256 x 256 direct-load
// kernel of gemm_fast.h with 16 x 16 x 32 MFMAs.
//
// It is a translation unit of its own because it is compiled without the
// machine scheduler that runs before register allocation (-mllvm
// -enable-misched=0, see build.py): with it, the 64 accumulator quads of a
// 128 x 128 wave tile were reordered into live ranges that the allocator
// could not keep in place, and it moved accumulators between registers
// around most MFMAs (hundreds of v_accvgpr moves per k-tile).  Without it the
// K loop keeps every accumulator in place; the MFMA / LDS-read / DMA
// interleave is still fixed by the kernel's sched_group_barrier groups.
//
// The 16 x 16 x 32 form does the same FLOPs with the same LDS bytes as the
// 32 x 32 x 16 one, but draws less power per FLOP, so under the board's power
// limit the clock holds higher (register-only MFMA issue on MI355X: 2045-2076
// TFLOP/s at 2.10 GHz against 1831-1836 TFLOP/s at 1.84-1.86 GHz).  Early
// DMA: 8 of the 16 instructions of k-tile t+2 right after the barrier of
// k-tile t (8192^3 NT on one box: 4 -> 746.6-749.5 us, 6 -> 726-728,
// 8 -> 718-720, 10 -> 722-725, 16 -> 750 us; the 32 x 32 form 759-762 us).
#include <hip/hip_runtime.h>

#include "libgemm.h"
#include "gemm_fast.h"

namespace fast {

template <int KIND, bool TAIL, bool FUSED, bool SPLIT, bool DYN>
void launch_mf16(int grid, hipStream_t stream, const Args& a) {
    hipLaunchKernelGGL((gemm_fast_kernel<KIND, 128, 2, TAIL, 1, 8, 1, 4, FUSED, SPLIT, DYN, 1, 16>), dim3(grid),
                       dim3(256), 0, stream, a);
}

// plain fp32 product, fused epilogue, split-K units, dynamic schedule; each
// with and without a partial last k-tile
template void launch_mf16<kNT, false, false, false, false>(int, hipStream_t, const Args&);
template void launch_mf16<kNT, true, false, false, false>(int, hipStream_t, const Args&);
template void launch_mf16<kNN, false, false, false, false>(int, hipStream_t, const Args&);
template void launch_mf16<kNN, true, false, false, false>(int, hipStream_t, const Args&);
template void launch_mf16<kNT, false, true, false, false>(int, hipStream_t, const Args&);
template void launch_mf16<kNT, true, true, false, false>(int, hipStream_t, const Args&);
template void launch_mf16<kNN, false, true, false, false>(int, hipStream_t, const Args&);
template void launch_mf16<kNN, true, true, false, false>(int, hipStream_t, const Args&);
template void launch_mf16<kNT, false, false, true, false>(int, hipStream_t, const Args&);
template void launch_mf16<kNT, true, false, true, false>(int, hipStream_t, const Args&);
template void launch_mf16<kNN, false, false, true, false>(int, hipStream_t, const Args&);
template void launch_mf16<kNN, true, false, true, false>(int, hipStream_t, const Args&);
template void launch_mf16<kNT, false, false, false, true>(int, hipStream_t, const Args&);
template void launch_mf16<kNT, true, false, false, true>(int, hipStream_t, const Args&);
template void launch_mf16<kNN, false, false, false, true>(int, hipStream_t, const Args&);
template void launch_mf16<kNN, true, false, false, true>(int, hipStream_t, const Args&);

#ifdef LIBGEMM_MEASURE
// Measurement builds: the plain product with 8 waves (two per SIMD, 128 x 64
// wave tiles as 8 x 4 blocks); 4 of each wave's 8 DMA instructions of k-tile
// t+2 after the barrier of k-tile t.
template <int KIND, bool TAIL>
void launch_mf16_w8(int grid, hipStream_t stream, const Args& a) {
    hipLaunchKernelGGL((gemm_fast_kernel<KIND, 128, 2, TAIL, 1, 4, 1, 8, false, false, false, 1, 16>), dim3(grid),
                       dim3(512), 0, stream, a);
}
template void launch_mf16_w8<kNT, false>(int, hipStream_t, const Args&);
template void launch_mf16_w8<kNT, true>(int, hipStream_t, const Args&);
template void launch_mf16_w8<kNN, false>(int, hipStream_t, const Args&);
template void launch_mf16_w8<kNN, true>(int, hipStream_t, const Args&);
#endif

}  // namespace fast
