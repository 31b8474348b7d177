/*
 * libgemm.h -- C ABI of the MI355X (gfx950) dense GEMM library.
 *
 * Operation (the matrix product of "GPU 执行模型", section "Tile 的容量约束"):
 *
 *     C[M x N] = A[M x K] * B[K x N]
 *
 * with fp32 accumulation and fp32 output, for
 *   - bf16 operands (gemm_bf16: B row-major; gemm_bf16_nt: B column-major), and
 *   - MX block-scaled fp8 operands (gemm_mxfp8): OCP E4M3 ("fn") element
 *     codes with one OCP E8M0 scale code per 32 consecutive K-elements of each
 *     row of A and each column of B.  This is the block-scaled MMA of
 *     "Modern GPU Programming For MLSys - 书籍总结", sections 2.4 and 2.6; the
 *     encodings follow the OCP Microscaling (MX) v1.0 specification.  Each
 *     output is sum over blocks b of 2^(sa-127) * 2^(sb-127) * (sum of the
 *     32 element products of block b).
 *
 * Conventions shared by every entry point (the correctness contract of
 * "GPU 执行模型", section "正确性契约"):
 *   - Sizes and leading dimensions are in ELEMENTS, as int64_t.  M, N and K
 *     may each be up to 2^31 - 1 (GEMM_ERR_INVALID_ARG beyond); operands and
 *     C may be larger than 4 GiB.  Operands whose rows or K-panels would span
 *     more than 2 GiB in one 32-bit buffer descriptor are routed to kernels
 *     with 64-bit addressing, which are slower but give the same contract.
 *   - A is row-major: element (i, k) at A[i*lda + k], lda >= K.
 *   - C is row-major fp32: element (i, j) at C[i*ldc + j], ldc >= N.  C is
 *     overwritten (no alpha/beta); elements outside the M x N block and the
 *     padding of every operand (ld > extent) are never read into a result
 *     and C outside M x N is never written.
 *   - Pointers are DEVICE pointers on the current HIP device.  The caller owns
 *     every buffer; the library never allocates, frees, copies or
 *     synchronises during a call.  Any element alignment is accepted (2 bytes
 *     for bf16, 1 byte for fp8, 4 bytes for C); 16-byte aligned operands with
 *     leading dimensions that keep rows 16-byte aligned take the fastest path.
 *   - C must not alias A, B or the scales (undefined if it does).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the legacy default
 *     stream) and the call returns without waiting; completion is observed
 *     through the stream.  Calls contain no host synchronisation and no
 *     allocation, so they may be captured into a HIP graph.
 *   - Results are deterministic: the same inputs give bitwise-identical C
 *     (no atomics, fixed reduction order for a given shape and layout).
 *   - M == 0 or N == 0: nothing is done and GEMM_OK is returned.
 *     K == 0: C[0:M, 0:N] is set to zero.
 *   - NaN and Inf propagate as in IEEE arithmetic (a NaN operand makes the
 *     outputs it feeds NaN; Inf * 0 is NaN).  fp32 subnormal results may be
 *     flushed by the matrix cores; that lies inside the accuracy contract.
 *   - Accuracy: |C - exact| <= 1e-3 * sum_k |a(i,k)| |b(k,j)| elementwise for
 *     K <= 16384; integer-valued operands whose partial sums stay below 2^24
 *     give exact results.
 *   - The library never aborts the process.  Errors are returned as the
 *     codes below and leave C untouched.
 */
#ifndef LIBGEMM_H
#define LIBGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GEMM_OK 0
/* a size is negative, a leading dimension too small, a pointer NULL with a
 * non-empty extent, (MX) K not a multiple of 32, or (fused entry points) an
 * unknown output type or a C pointer not aligned to its element */
#define GEMM_ERR_INVALID_ARG (-1)
/* the current device is not a gfx950 (MI355X-class) GPU, or no device */
#define GEMM_ERR_UNSUPPORTED (-2)
/* the HIP runtime reported an error when the kernel was enqueued */
#define GEMM_ERR_LAUNCH (-3)
/* gemm_bf16_splitk_noalloc: the split plan needs more scratch than the
 * library's fixed array holds (GEMM_SCRATCH_BYTES) */
#define GEMM_ERR_SCRATCH (-4)

/* bf16 GEMM, B row-major: A bf16 M x K (lda >= K), B bf16 K x N with
 * element (k, j) at B[k*ldb + j] (ldb >= N), C fp32 M x N (ldc >= N). */
int gemm_bf16(int64_t M, int64_t N, int64_t K,
              const void* A, int64_t lda,
              const void* B, int64_t ldb,
              float* C, int64_t ldc,
              void* stream);

/* bf16 GEMM, B column-major ("NT"): element (k, j) of B at B[j*ldb + k],
 * ldb >= K (B is stored as N rows of K).  Otherwise as gemm_bf16. */
int gemm_bf16_nt(int64_t M, int64_t N, int64_t K,
                 const void* A, int64_t lda,
                 const void* B, int64_t ldb,
                 float* C, int64_t ldc,
                 void* stream);

/* MX block-scaled fp8 GEMM.  A: E4M3 codes, M x K row-major (lda >= K).
 * B: E4M3 codes, column-major, element (k, j) at B[j*ldb + k] (ldb >= K).
 * scaleA: E8M0 codes, dense row-major M x (K/32): the scale of A's row i for
 * k in [32b, 32b+32) is scaleA[i*(K/32) + b].  scaleB: E8M0 codes, dense
 * N x (K/32): the scale of B's column j for block b is scaleB[j*(K/32) + b].
 * K must be a multiple of 32.  C fp32 M x N (ldc >= N). */
int gemm_mxfp8(int64_t M, int64_t N, int64_t K,
               const void* A, int64_t lda,
               const void* B, int64_t ldb,
               const uint8_t* scaleA, const uint8_t* scaleB,
               float* C, int64_t ldc,
               void* stream);

/* ---- fused epilogue ------------------------------------------------------
 *
 * The writeback role of "Modern GPU Programming For MLSys - 书籍总结", section
 * 4.3 (Step 7), and the fusion model of "GPU 执行模型", section "Fusion 的收益
 * 与上限": the elementwise work that would otherwise read C back is applied to
 * the fp32 accumulator before the single store:
 *
 *     t(i, j) = acc(i, j) * row_scale[i] * col_scale[j] + bias[j]
 *     C[i*ldc + j] = t rounded to the output type
 *
 * evaluated in fp32 in that order (the products may be fused into one
 * multiply-add).  row_scale (M floats), col_scale (N floats) and bias
 * (N floats) are device pointers; each may be NULL, meaning 1, 1 and 0.
 * out_type GEMM_OUT_F32 stores fp32 (C is float*); GEMM_OUT_BF16 stores bf16
 * rounded to nearest even (C is a 2-byte element array; NaN stays NaN);
 * GEMM_OUT_E4M3 stores OCP FP8 E4M3 codes (C is a byte array), t rounded to
 * nearest even with saturation: |t| beyond the largest finite E4M3 value 448,
 * infinities included, stores +-448 (0x7E / 0xFE); NaN stores a NaN code
 * (0x7F or 0xFF).  The pages name fp8 outputs without an encoding; the OCP
 * FP8 format and its saturating conversion are the reading taken here, the
 * format the MX operands already use.  ldc counts elements of the output
 * type.  K == 0 stores t with acc = 0.  Every other convention is that of the
 * entry points above; the accuracy bound applies to acc, and t adds the fp32
 * rounding of the epilogue and, for bf16 and E4M3, the final rounding. */
#define GEMM_OUT_F32 0
#define GEMM_OUT_BF16 1
#define GEMM_OUT_E4M3 2

/* bf16 operands, B row-major (b_colmajor == 0, as gemm_bf16) or column-major
 * (b_colmajor != 0, as gemm_bf16_nt). */
int gemm_bf16_fused(int64_t M, int64_t N, int64_t K,
                    const void* A, int64_t lda,
                    const void* B, int64_t ldb, int b_colmajor,
                    void* C, int64_t ldc, int out_type,
                    const float* row_scale, const float* col_scale, const float* bias,
                    void* stream);

/* MX-fp8 operands, as gemm_mxfp8. */
int gemm_mxfp8_fused(int64_t M, int64_t N, int64_t K,
                     const void* A, int64_t lda,
                     const void* B, int64_t ldb,
                     const uint8_t* scaleA, const uint8_t* scaleB,
                     void* C, int64_t ldc, int out_type,
                     const float* row_scale, const float* col_scale, const float* bias,
                     void* stream);

/* ---- split-K --------------------------------------------------------------
 *
 * "GPU 执行模型", section "编译与 autotune", lists split-K among the
 * strategies a GEMM chooses per shape, with a bounded choice for shapes not
 * seen before.  Here the K extent is cut into `splits` ranges of kslice
 * elements (a multiple of the partial kernel's k-tile; the last range takes
 * the rest).  Each range's fp32 partial product is written to its own dense
 * M x N plane of the caller's workspace, and a second kernel adds the planes
 * in range order (0, 1, 2, ...) and applies the epilogue:
 *
 *     acc(i, j) = P_0(i, j) + P_1(i, j) + ... + P_{s-1}(i, j)
 *
 * so results are deterministic for a given plan.  This fills the GPU when the
 * output has too few tiles for its compute units (a short, wide product or a
 * small M x N with a long K).
 *
 * Products whose 256 x 256 tiles fill more than one round of the compute
 * units, with a last round at most half full, get a stream-K style plan from
 * the library (splits == 0): the whole rounds compute their tiles unsplit,
 * straight into C, and only the last round's tiles are split over K, so that
 * round takes a fraction of a round's time.  Their partial products go to
 * compact 256 x 256 fp32 blocks (splits_used * left-over tiles * 256 KiB of
 * workspace) and are added per tile in range order.  This plan stores C with
 * the plain fp32 epilogue only; with another epilogue such products run
 * unsplit.
 *
 * gemm_bf16_splitk: arguments as gemm_bf16_fused, plus
 *   splits          K ranges wanted; 0 lets the library decide from the shape
 *                   (its plan is gemm_bf16_splitk_plan's).  Fewer ranges are
 *                   used when K is too short; with 1 range, or when no
 *                   split-capable kernel applies (operands not 16-byte
 *                   aligned, leading dimensions not multiples of 8 elements),
 *                   the product runs unsplit as gemm_bf16_fused and the
 *                   workspace is not touched.
 *   workspace       device memory owned by the caller, 16-byte aligned, at
 *                   least the bytes gemm_bf16_splitk_plan reports
 *                   (splits_used * M * N * 4 when every tile is split); its
 *                   contents on entry do not matter
 *                   and are overwritten.  Calls that share a workspace must
 *                   be ordered on one stream.
 *   workspace_bytes its size.
 * Errors: GEMM_ERR_INVALID_ARG as gemm_bf16_fused, or splits < 0, or a split
 * plan whose workspace is NULL, too small or not 16-byte aligned.  The
 * accuracy bound is that of the other entry points (every K range is summed
 * in fp32 and the ranges are added in fp32). */
int gemm_bf16_splitk(int64_t M, int64_t N, int64_t K,
                     const void* A, int64_t lda,
                     const void* B, int64_t ldb, int b_colmajor,
                     void* C, int64_t ldc, int out_type,
                     const float* row_scale, const float* col_scale, const float* bias,
                     int splits, void* workspace, size_t workspace_bytes,
                     void* stream);

/* The split plan of gemm_bf16_splitk for 16-byte aligned operands with dense
 * leading dimensions (lda = K; ldb = N, or K when b_colmajor): the number of
 * K ranges it uses (*splits_used, 1 = unsplit) and the workspace bytes they
 * need (*workspace_bytes, 0 when unsplit).  splits as in gemm_bf16_splitk;
 * cus: compute units to plan for, 0 = those of the current device.  Either
 * output pointer may be NULL.  Runs on the host only (no device work). */
int gemm_bf16_splitk_plan(int64_t M, int64_t N, int64_t K, int b_colmajor, int splits, int cus,
                          int* splits_used, size_t* workspace_bytes);

/* The split plan gemm_bf16_splitk runs for exactly these arguments (those of
 * gemm_bf16_splitk without the workspace and the stream): the K ranges it
 * uses (*splits_used, 1 = unsplit) and the workspace bytes they need
 * (*workspace_bytes, 0 when unsplit).  Unlike gemm_bf16_splitk_plan it takes
 * the real operand pointers and leading dimensions, whose alignment decides
 * which kernel computes the partial products, and the epilogue, which
 * decides whether a stream-K style plan applies.  The pointers are only
 * inspected (for NULL and alignment), never dereferenced.  cus: compute
 * units to plan for, 0 = those of the current device.  Errors: those
 * gemm_bf16_splitk reports for these arguments before any device work
 * (GEMM_ERR_INVALID_ARG; GEMM_ERR_UNSUPPORTED with cus == 0 and no gfx950
 * device).  Runs on the host only. */
int gemm_bf16_splitk_workspace(int64_t M, int64_t N, int64_t K,
                               const void* A, int64_t lda,
                               const void* B, int64_t ldb, int b_colmajor,
                               const void* C, int64_t ldc, int out_type,
                               const float* row_scale, const float* col_scale, const float* bias,
                               int splits, int cus, int* splits_used, size_t* workspace_bytes);

/* MX-fp8 split-K: gemm_mxfp8_fused's product with K cut into ranges, as
 * gemm_bf16_splitk (fp32 partial products in the caller's workspace, dense
 * M x N planes added in range order, then the epilogue).  Ranges are a
 * multiple of 1024 (the last takes the rest, a multiple of 512), so that each
 * starts on a 16-byte boundary of the scale rows; the plan (splits == 0)
 * splits when the 256 x 256 tiles give the
 * compute units less than 3/4 of a round, into about CUs / tiles ranges of at
 * least 1024.  Products that do not suit the split kernel (operands or
 * scales not 16-byte aligned, rows not 16-byte aligned, K not a multiple of
 * 512) or that the plan leaves whole run as gemm_mxfp8_fused and the
 * workspace is not touched.  Arguments and errors as gemm_mxfp8_fused plus
 * those of gemm_bf16_splitk for splits and the workspace. */
int gemm_mxfp8_splitk(int64_t M, int64_t N, int64_t K,
                      const void* A, int64_t lda,
                      const void* B, int64_t ldb,
                      const uint8_t* scaleA, const uint8_t* scaleB,
                      void* C, int64_t ldc, int out_type,
                      const float* row_scale, const float* col_scale, const float* bias,
                      int splits, void* workspace, size_t workspace_bytes,
                      void* stream);

/* The plan gemm_mxfp8_splitk runs for these arguments (pointers inspected,
 * never dereferenced): K ranges used and workspace bytes, as
 * gemm_bf16_splitk_workspace.  Host only. */
int gemm_mxfp8_splitk_workspace(int64_t M, int64_t N, int64_t K,
                                const void* A, int64_t lda,
                                const void* B, int64_t ldb,
                                const uint8_t* scaleA, const uint8_t* scaleB,
                                const void* C, int64_t ldc, int out_type,
                                const float* row_scale, const float* col_scale, const float* bias,
                                int splits, int cus, int* splits_used, size_t* workspace_bytes);

/* ---- split-K without a workspace -----------------------------------------
 *
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops, harnesses that forbid allocation): gemm_bf16_splitk
 * with the partial products in a fixed device array that the library itself
 * holds, GEMM_SCRATCH_BYTES per GPU, kept from the first call on that GPU
 * until the process ends.  Arguments as gemm_bf16_splitk without the
 * workspace; the split plan, the kernels and hence the results are those of
 * gemm_bf16_splitk, bit for bit.  The call allocates nothing (no hipMalloc,
 * no library routine that allocates).
 *
 * Every call on one GPU shares that GPU's array: calls that may overlap in
 * time on one GPU (different streams, different host threads without
 * ordering) race and give undefined results; order them on one stream.  The
 * array's contents between calls do not matter (every partial product is
 * written before it is read).
 * Errors: those of gemm_bf16_splitk, and GEMM_ERR_SCRATCH (C untouched) when
 * the plan needs more than GEMM_SCRATCH_BYTES, i.e. splits_used * M * N * 4
 * bytes (or the compact stream-K style blocks) as gemm_bf16_splitk_workspace
 * reports them; GEMM_ERR_LAUNCH if the runtime cannot give the array's
 * device address. */
#define GEMM_SCRATCH_BYTES ((size_t)64 << 20)

int gemm_bf16_splitk_noalloc(int64_t M, int64_t N, int64_t K,
                             const void* A, int64_t lda,
                             const void* B, int64_t ldb, int b_colmajor,
                             void* C, int64_t ldc, int out_type,
                             const float* row_scale, const float* col_scale, const float* bias,
                             int splits, void* stream);

/* ---- dynamic tile schedule -----------------------------------------------
 *
 * "Modern GPU Programming For MLSys - 书籍总结", section 2.9 (Cluster Launch
 * Control) and section 4.2 (Step 6, the persistent kernel with a tile
 * scheduler): resident workgroups ask for their next tile at run time, so a
 * workgroup that finishes early takes more work instead of idling at the
 * tail.  Here that request is an atomic increment of a tile counter in the
 * caller's workspace: 8 queues, one per XCD, each holding the tiles the
 * static walk would give that XCD's workgroups (neighbouring tiles, which
 * share the XCD's L2), and a workgroup whose queue is empty takes tiles from
 * the other queues.  Every tile is still computed by exactly one workgroup
 * with the same arithmetic, so C is bitwise identical to gemm_bf16's.
 *
 * Arguments as gemm_bf16_fused without the epilogue (fp32 C), plus
 *   workspace        device memory owned by the caller, 16-byte aligned, at
 *                    least GEMM_DYNAMIC_WORKSPACE_BYTES; the counters are
 *                    zeroed on the stream by the call itself, so its contents
 *                    on entry do not matter.  Calls that share a workspace
 *                    must be ordered on one stream.
 *   workspace_bytes  its size.
 * Products that the 256 x 256 direct-load kernel does not take run as
 * gemm_bf16 / gemm_bf16_nt, and the workspace is not touched.
 * Errors: as gemm_bf16, or a workspace that is NULL, too small or not 16-byte
 * aligned (GEMM_ERR_INVALID_ARG). */
#define GEMM_DYNAMIC_WORKSPACE_BYTES 1024

int gemm_bf16_dynamic(int64_t M, int64_t N, int64_t K,
                      const void* A, int64_t lda,
                      const void* B, int64_t ldb, int b_colmajor,
                      float* C, int64_t ldc,
                      void* workspace, size_t workspace_bytes,
                      void* stream);

/* Static text for a return code (never NULL). */
const char* gemm_strerror(int code);

/* Library version: major*10000 + minor*100 + patch. */
int gemm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBGEMM_H */
