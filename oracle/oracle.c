/*
 * oracle.c -- plain, slow, obviously-correct CPU reference for the dense GEMM
 * C[MxN] = A[MxK] * B[KxN] (bf16 operands) and its MX block-scaled fp8
 * variant (e4m3 operands, one e8m0 power-of-two scale per 32 consecutive
 * K-elements).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library's compute path may link,
 * load or call this file; only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no source, header, decoder
 * or table with the HIP library.
 *
 * Sources followed (the pages are cited by title and section):
 *  - "GPU 执行模型", section "Tile 的容量约束": the problem is the plain matrix
 *    product C = A B with A of shape MxK and B of shape KxN.
 *  - "GPU 执行模型", section "Tile 小账本": the per-K-step tile ledger
 *    (staging bytes, FLOPs counted as 2 per multiply-add, one logical HBM read
 *    of the A and B tiles, arithmetic intensity, fit against a shared-memory
 *    limit).
 *  - "Modern GPU Programming For MLSys - 书籍总结", sections 2.4 and 2.6: the
 *    block-scaled MMA (scale factors per block of the reduction axis).  The
 *    pages do not define the element or scale encodings; they are read from
 *    the public OCP Microscaling (MX) v1.0 and OCP 8-bit floating point
 *    specifications: E4M3 ("fn" variant: no infinities, S.1111.111 is NaN,
 *    largest finite 448) and E8M0 (value 2^(e-127), 0xFF is NaN), with MX
 *    blocks of 32 elements along the reduction axis.
 *
 * Arithmetic: every decoded operand value is exact in binary64; products of
 * two bf16 (8-bit significands) or two e4m3 (4-bit significands) values are
 * exact in binary64; sums are accumulated in binary64 in ascending k order.
 * The binary64 result is handed back unrounded; the caller rounds it to fp32
 * (round-to-nearest-even) when it needs the fp32 value.  Alongside each C
 * element the oracle can return sum_k |a(i,k)| |b(k,j)| (the magnitude
 * product), which scales the elementwise acceptance bound.
 *
 * Parallelism: output rows are split into contiguous chunks over POSIX
 * threads.  Each output element is still the same sequential k-ordered sum,
 * so the thread count never changes a result.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_VERSION 1

int oracle_version(void) { return ORACLE_VERSION; }

/* ------------------------------------------------------------------------ */
/* Element decoders.                                                          */
/* ------------------------------------------------------------------------ */

/* bf16 is the upper half of an IEEE binary32 word: widen and reinterpret. */
double oracle_bf16_value(uint16_t h) {
    uint32_t w = (uint32_t)h << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* OCP FP8 E4M3 ("fn"): 1 sign bit, 4 exponent bits with bias 7, 3 fraction
 * bits.  Exponent field 0 is subnormal: (m/8) * 2^-6.  Exponent 15 with
 * fraction 7 is NaN; there is no infinity, so 0x7E = +448 is the largest. */
double oracle_e4m3_value(uint8_t c) {
    int sign = (c >> 7) & 1;
    int e = (c >> 3) & 0xF;
    int m = c & 0x7;
    double mag;
    if (e == 0xF && m == 0x7) return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);             /* (m/8) * 2^(1-7) */
    else
        mag = ldexp(8.0 + (double)m, e - 10);   /* (1 + m/8) * 2^(e-7) */
    return sign ? -mag : mag;
}

/* OCP E8M0 scale: unsigned 8-bit biased exponent, value 2^(e-127);
 * 0xFF encodes NaN. */
double oracle_e8m0_value(uint8_t e) {
    if (e == 0xFF) return NAN;
    return ldexp(1.0, (int)e - 127);
}

/* ------------------------------------------------------------------------ */
/* Tile ledger ("GPU 执行模型", section "Tile 小账本").                       */
/* ------------------------------------------------------------------------ */

/* For one K-step of an m x n output tile with a k-deep reduction slice:
 *   operand elements = m*k (A slice) + k*n (B slice)
 *   hbm bytes        = element_bytes * operand elements (one logical read)
 *   staging bytes    = stages * hbm bytes (each stage holds one copy; stages
 *                      add residency, never extra HBM reads)
 *   flops            = 2*m*n*k (a multiply-add counts as two operations)
 *   intensity        = flops / hbm bytes
 *   fits             = staging bytes <= shared-memory limit
 * out[0]=staging bytes, out[1]=flops, out[2]=hbm bytes, out[3]=fits (0/1).
 * Returns -1 (and writes nothing) unless every size is positive. */
int oracle_tile_ledger(int64_t m, int64_t n, int64_t k, int64_t element_bytes,
                       int64_t stages, int64_t smem_limit, int64_t out[4],
                       double* intensity) {
    if (m <= 0 || n <= 0 || k <= 0 || element_bytes <= 0 || stages <= 0) return -1;
    int64_t operand_elements = m * k + k * n;
    int64_t hbm = element_bytes * operand_elements;
    int64_t smem = stages * hbm;
    int64_t flops = 2 * m * n * k;
    out[0] = smem;
    out[1] = flops;
    out[2] = hbm;
    out[3] = smem <= smem_limit ? 1 : 0;
    if (intensity) *intensity = (double)flops / (double)hbm;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Generic strided operand access.                                            */
/* ------------------------------------------------------------------------ */

/* Operand element (r, c) lives at base[r*rs + c*cs] (strides in elements), so
 * one loop serves row-major and column-major storage alike. */

typedef struct {
    int64_t M, N, K;
    /* bf16 problem */
    const uint16_t* A16;
    const uint16_t* B16;
    /* MX fp8 problem */
    const uint8_t* A8;
    const uint8_t* B8;
    const uint8_t* SA;
    const uint8_t* SB;
    int64_t sa_ld, sb_ld;
    /* strides (elements): A(i,k) at A[i*a_rs + k*a_cs], B(k,j) at B[k*b_rs + j*b_cs] */
    int64_t a_rs, a_cs, b_rs, b_cs;
    /* full-matrix output */
    double* C;
    double* absC;
    int64_t ldc;
    /* sampled output */
    const int64_t* rows;
    const int64_t* cols;
    int64_t nsample;
    double* out;
    double* absout;
    /* work split */
    int64_t lo, hi;
} job_t;

/* One bf16 output element: the k-ordered binary64 sum of exact products. */
static void bf16_element(const job_t* J, int64_t i, int64_t j, double* c, double* a) {
    double s = 0.0, m = 0.0;
    for (int64_t k = 0; k < J->K; ++k) {
        double x = oracle_bf16_value(J->A16[i * J->a_rs + k * J->a_cs]);
        double y = oracle_bf16_value(J->B16[k * J->b_rs + j * J->b_cs]);
        s += x * y;
        m += fabs(x) * fabs(y);
    }
    *c = s;
    *a = m;
}

/* One MX output element: for every 32-wide block b of the reduction axis,
 * the exact inner sum of decoded e4m3 products is multiplied by the two
 * block scales 2^(sa-127) * 2^(sb-127), and the block results are summed in
 * ascending b (block-scaled MMA, "Modern GPU Programming For MLSys -
 * 书籍总结" sections 2.4/2.6; block size and codes per OCP MX v1.0). */
static void mx_element(const job_t* J, int64_t i, int64_t j, double* c, double* a) {
    double s = 0.0, m = 0.0;
    int64_t nb = J->K / 32;
    for (int64_t b = 0; b < nb; ++b) {
        double sa = oracle_e8m0_value(J->SA[i * J->sa_ld + b]);
        double sb = oracle_e8m0_value(J->SB[j * J->sb_ld + b]);
        double inner = 0.0, inner_abs = 0.0;
        for (int64_t k = 32 * b; k < 32 * b + 32; ++k) {
            double x = oracle_e4m3_value(J->A8[i * J->a_rs + k * J->a_cs]);
            double y = oracle_e4m3_value(J->B8[k * J->b_rs + j * J->b_cs]);
            inner += x * y;
            inner_abs += fabs(x) * fabs(y);
        }
        s += sa * sb * inner;
        m += fabs(sa) * fabs(sb) * inner_abs;
    }
    *c = s;
    *a = m;
}

static void* run_full_bf16(void* p) {
    job_t* J = (job_t*)p;
    if (J->b_cs == 1 && J->N > 1) {
        /* Row-major B: the same ascending-k binary64 sums, formed a whole
         * output row at a time (i-k-j order) so that B is read along its
         * rows.  Every element sees exactly the additions of bf16_element in
         * the same order, so the results are bit-identical to it. */
        for (int64_t i = J->lo; i < J->hi; ++i) {
            double* crow = J->C + i * J->ldc;
            double* arow = J->absC ? J->absC + i * J->ldc : NULL;
            for (int64_t j = 0; j < J->N; ++j) {
                crow[j] = 0.0;
                if (arow) arow[j] = 0.0;
            }
            for (int64_t k = 0; k < J->K; ++k) {
                double x = oracle_bf16_value(J->A16[i * J->a_rs + k * J->a_cs]);
                const uint16_t* brow = J->B16 + k * J->b_rs;
                for (int64_t j = 0; j < J->N; ++j) {
                    double y = oracle_bf16_value(brow[j]);
                    crow[j] += x * y;
                    if (arow) arow[j] += fabs(x) * fabs(y);
                }
            }
        }
        return NULL;
    }
    for (int64_t i = J->lo; i < J->hi; ++i)
        for (int64_t j = 0; j < J->N; ++j) {
            double c, a;
            bf16_element(J, i, j, &c, &a);
            J->C[i * J->ldc + j] = c;
            if (J->absC) J->absC[i * J->ldc + j] = a;
        }
    return NULL;
}

static void* run_full_mx(void* p) {
    job_t* J = (job_t*)p;
    for (int64_t i = J->lo; i < J->hi; ++i)
        for (int64_t j = 0; j < J->N; ++j) {
            double c, a;
            mx_element(J, i, j, &c, &a);
            J->C[i * J->ldc + j] = c;
            if (J->absC) J->absC[i * J->ldc + j] = a;
        }
    return NULL;
}

static void* run_sample_bf16(void* p) {
    job_t* J = (job_t*)p;
    for (int64_t t = J->lo; t < J->hi; ++t) {
        double c, a;
        bf16_element(J, J->rows[t], J->cols[t], &c, &a);
        J->out[t] = c;
        if (J->absout) J->absout[t] = a;
    }
    return NULL;
}

static void* run_sample_mx(void* p) {
    job_t* J = (job_t*)p;
    for (int64_t t = J->lo; t < J->hi; ++t) {
        double c, a;
        mx_element(J, J->rows[t], J->cols[t], &c, &a);
        J->out[t] = c;
        if (J->absout) J->absout[t] = a;
    }
    return NULL;
}

/* Split [0, total) into nthreads contiguous chunks and run fn on each. */
static int run_split(job_t* proto, int64_t total, int nthreads, void* (*fn)(void*)) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > total) nthreads = total > 0 ? (int)total : 1;
    pthread_t th[256];
    job_t jobs[256];
    int started = 0, rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = *proto;
        jobs[t].lo = total * t / nthreads;
        jobs[t].hi = total * (t + 1) / nthreads;
        if (nthreads == 1) {
            fn(&jobs[t]);
            return 0;
        }
        if (pthread_create(&th[t], NULL, fn, &jobs[t]) != 0) {
            rc = -2;
            /* run the rest on this thread */
            for (int u = t; u < nthreads; ++u) {
                jobs[u] = *proto;
                jobs[u].lo = total * u / nthreads;
                jobs[u].hi = total * (u + 1) / nthreads;
                fn(&jobs[u]);
            }
            break;
        }
        ++started;
    }
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
    return rc == -2 ? 0 : rc;
}

/* ------------------------------------------------------------------------ */
/* Public entry points.                                                       */
/* ------------------------------------------------------------------------ */

/* bf16 GEMM, full output.  A(i,k) = A[i*a_rs + k*a_cs] (bf16 bits),
 * B(k,j) = B[k*b_rs + j*b_cs] (bf16 bits).  Writes the binary64 sum to
 * C[i*ldc + j] and, if absC is non-null, the magnitude product to
 * absC[i*ldc + j].  K == 0 gives zeros.  Returns 0, or -1 on bad sizes. */
int oracle_gemm_bf16(int64_t M, int64_t N, int64_t K,
                     const uint16_t* A, int64_t a_rs, int64_t a_cs,
                     const uint16_t* B, int64_t b_rs, int64_t b_cs,
                     double* C, double* absC, int64_t ldc, int nthreads) {
    if (M < 0 || N < 0 || K < 0 || ldc < N) return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.M = M; J.N = N; J.K = K;
    J.A16 = A; J.B16 = B;
    J.a_rs = a_rs; J.a_cs = a_cs; J.b_rs = b_rs; J.b_cs = b_cs;
    J.C = C; J.absC = absC; J.ldc = ldc;
    return run_split(&J, M, nthreads, run_full_bf16);
}

/* bf16 GEMM at nsample chosen output positions (rows[t], cols[t]); results
 * to out[t] and (optionally) absout[t]. */
int oracle_gemm_bf16_at(int64_t M, int64_t N, int64_t K,
                        const uint16_t* A, int64_t a_rs, int64_t a_cs,
                        const uint16_t* B, int64_t b_rs, int64_t b_cs,
                        const int64_t* rows, const int64_t* cols, int64_t nsample,
                        double* out, double* absout, int nthreads) {
    if (M < 0 || N < 0 || K < 0 || nsample < 0) return -1;
    for (int64_t t = 0; t < nsample; ++t)
        if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N) return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.M = M; J.N = N; J.K = K;
    J.A16 = A; J.B16 = B;
    J.a_rs = a_rs; J.a_cs = a_cs; J.b_rs = b_rs; J.b_cs = b_cs;
    J.rows = rows; J.cols = cols; J.nsample = nsample;
    J.out = out; J.absout = absout;
    return run_split(&J, nsample, nthreads, run_sample_bf16);
}

/* MX block-scaled fp8 GEMM, full output.  A(i,k) = A[i*a_rs + k*a_cs] and
 * B(k,j) = B[k*b_rs + j*b_cs] are e4m3 codes; the scale of row i of A for
 * block b (k in [32b, 32b+32)) is SA[i*sa_ld + b] and that of column j of B
 * is SB[j*sb_ld + b] (e8m0 codes).  K must be a multiple of 32. */
int oracle_gemm_mxfp8(int64_t M, int64_t N, int64_t K,
                      const uint8_t* A, int64_t a_rs, int64_t a_cs,
                      const uint8_t* B, int64_t b_rs, int64_t b_cs,
                      const uint8_t* SA, int64_t sa_ld,
                      const uint8_t* SB, int64_t sb_ld,
                      double* C, double* absC, int64_t ldc, int nthreads) {
    if (M < 0 || N < 0 || K < 0 || K % 32 != 0 || ldc < N) return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.M = M; J.N = N; J.K = K;
    J.A8 = A; J.B8 = B; J.SA = SA; J.SB = SB; J.sa_ld = sa_ld; J.sb_ld = sb_ld;
    J.a_rs = a_rs; J.a_cs = a_cs; J.b_rs = b_rs; J.b_cs = b_cs;
    J.C = C; J.absC = absC; J.ldc = ldc;
    return run_split(&J, M, nthreads, run_full_mx);
}

/* MX GEMM at nsample chosen output positions. */
int oracle_gemm_mxfp8_at(int64_t M, int64_t N, int64_t K,
                         const uint8_t* A, int64_t a_rs, int64_t a_cs,
                         const uint8_t* B, int64_t b_rs, int64_t b_cs,
                         const uint8_t* SA, int64_t sa_ld,
                         const uint8_t* SB, int64_t sb_ld,
                         const int64_t* rows, const int64_t* cols, int64_t nsample,
                         double* out, double* absout, int nthreads) {
    if (M < 0 || N < 0 || K < 0 || K % 32 != 0 || nsample < 0) return -1;
    for (int64_t t = 0; t < nsample; ++t)
        if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N) return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.M = M; J.N = N; J.K = K;
    J.A8 = A; J.B8 = B; J.SA = SA; J.SB = SB; J.sa_ld = sa_ld; J.sb_ld = sb_ld;
    J.a_rs = a_rs; J.a_cs = a_cs; J.b_rs = b_rs; J.b_cs = b_cs;
    J.rows = rows; J.cols = cols; J.nsample = nsample;
    J.out = out; J.absout = absout;
    return run_split(&J, nsample, nthreads, run_sample_mx);
}

/* ------------------------------------------------------------------------ */
/* Attention forward (the second workload of "Modern GPU Programming For     */
/* MLSys - 书籍总结", part IV, sections 5.1-5.3).                            */
/* ------------------------------------------------------------------------ */

/* What is computed, per batch b, query head h and query row i:
 *
 *   s_j   = scale * sum_d q(i,d) k(j,d)            (the score MMA, 5.1)
 *   keys  : j in [0, Sk); with the causal mask only j <= i + (Sk - Sq)
 *           (5.3 names causal masking; the pages fix no alignment, and the
 *           bottom-right one keeps the last query row seeing every key)
 *   e_j   = exp(s_j - max_j s_j),  p_j = e_j / sum_j e_j          (softmax)
 *   o(i,d)= sum_j p_j v(j,d) = (sum_j e_j v(j,d)) / sum_j e_j  (value MMA, 5.1)
 *   lse_i = max_j s_j + log(sum_j exp(s_j - max_j s_j))
 *
 * Grouped-query attention (5.3): query head h reads key/value head
 * h / (Hq / Hkv).  This is the plain definition of softmax attention; the
 * online (running-max, rescaled) form of section 5.2 reaches the same value
 * up to rounding, so the oracle does not follow it.  A row with no allowed
 * key (causal, Sq > Sk) has no softmax: its output is 0 and its lse -inf.
 *
 * Arithmetic: bf16 inputs decoded exactly, every sum in binary64 in
 * ascending index order, exp and log from the C library in binary64.
 * Alongside o(i,d) the oracle returns sum_j p_j |v(j,d)|, which scales the
 * elementwise acceptance bound. */
typedef struct {
    int64_t Hq, Hkv, Sq, Sk, D;
    const uint16_t *Q, *K, *V;
    int64_t qs[4], ks[4], vs[4];  /* element strides: batch, head, seq, dim */
    double scale;
    int causal;
    const int64_t* rows;          /* sampled rows as (b, h, i) triples, or NULL */
    double *O, *Omag, *lse;       /* outputs, dense [row][D] and [row] */
    double* work;                 /* per-thread scratch of Sk doubles */
    int64_t lo, hi;
} attn_job_t;

static void attn_row(const attn_job_t* J, int64_t b, int64_t h, int64_t i,
                     double* o, double* omag, double* lse, double* s) {
    const int64_t g = J->Hq / J->Hkv;
    const int64_t hk = h / g;
    const uint16_t* q = J->Q + b * J->qs[0] + h * J->qs[1] + i * J->qs[2];
    const uint16_t* kb = J->K + b * J->ks[0] + hk * J->ks[1];
    const uint16_t* vb = J->V + b * J->vs[0] + hk * J->vs[1];
    int64_t nkeys = J->Sk;
    if (J->causal) {
        int64_t last = i + (J->Sk - J->Sq);  /* largest allowed key */
        nkeys = last + 1 < J->Sk ? last + 1 : J->Sk;
        if (nkeys < 0) nkeys = 0;
    }
    for (int64_t d = 0; d < J->D; ++d) {
        o[d] = 0.0;
        omag[d] = 0.0;
    }
    if (nkeys == 0) {
        *lse = -INFINITY;
        return;
    }
    double mx = -INFINITY;
    for (int64_t j = 0; j < nkeys; ++j) {
        const uint16_t* k = kb + j * J->ks[2];
        double dot = 0.0;
        for (int64_t d = 0; d < J->D; ++d)
            dot += oracle_bf16_value(q[d * J->qs[3]]) * oracle_bf16_value(k[d * J->ks[3]]);
        s[j] = J->scale * dot;
        if (s[j] > mx || j == 0) mx = s[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < nkeys; ++j) {
        s[j] = exp(s[j] - mx);
        l += s[j];
    }
    /* softmax(s) V = (sum_j e_j v(j)) / (sum_j e_j): sum, then divide once */
    for (int64_t j = 0; j < nkeys; ++j) {
        const uint16_t* v = vb + j * J->vs[2];
        for (int64_t d = 0; d < J->D; ++d) {
            double x = oracle_bf16_value(v[d * J->vs[3]]);
            o[d] += s[j] * x;
            omag[d] += s[j] * fabs(x);
        }
    }
    for (int64_t d = 0; d < J->D; ++d) {
        o[d] /= l;
        omag[d] /= l;
    }
    *lse = mx + log(l);
}

static void* run_attn(void* p) {
    attn_job_t* J = (attn_job_t*)p;
    double* s = (double*)malloc(sizeof(double) * (size_t)(J->Sk > 0 ? J->Sk : 1));
    if (!s) return NULL;
    for (int64_t t = J->lo; t < J->hi; ++t) {
        int64_t b, h, i;
        if (J->rows) {
            b = J->rows[3 * t];
            h = J->rows[3 * t + 1];
            i = J->rows[3 * t + 2];
        } else {
            i = t % J->Sq;
            h = (t / J->Sq) % J->Hq;
            b = t / (J->Sq * J->Hq);
        }
        attn_row(J, b, h, i, J->O + t * J->D, J->Omag + t * J->D, J->lse + t, s);
    }
    free(s);
    return NULL;
}

static int run_attn_split(attn_job_t* proto, int64_t total, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > total) nthreads = total > 0 ? (int)total : 1;
    pthread_t th[256];
    attn_job_t jobs[256];
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = *proto;
        jobs[t].lo = total * t / nthreads;
        jobs[t].hi = total * (t + 1) / nthreads;
    }
    if (nthreads == 1) {
        run_attn(&jobs[0]);
        return 0;
    }
    for (int t = 0; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, run_attn, &jobs[t]) != 0) {
            for (int u = t; u < nthreads; ++u) run_attn(&jobs[u]);
            break;
        }
        ++started;
    }
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
    return 0;
}

static int attn_setup(attn_job_t* J, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Sk,
                      int64_t D, const uint16_t* Q, const int64_t* qs, const uint16_t* K,
                      const int64_t* ks, const uint16_t* V, const int64_t* vs, double scale,
                      int causal) {
    if (B < 0 || Hq < 1 || Hkv < 1 || Sq < 0 || Sk < 0 || D < 1 || Hq % Hkv != 0) return -1;
    memset(J, 0, sizeof *J);
    J->Hq = Hq;
    J->Hkv = Hkv;
    J->Sq = Sq;
    J->Sk = Sk;
    J->D = D;
    J->Q = Q;
    J->K = K;
    J->V = V;
    for (int t = 0; t < 4; ++t) {
        J->qs[t] = qs[t];
        J->ks[t] = ks[t];
        J->vs[t] = vs[t];
    }
    J->scale = scale;
    J->causal = causal ? 1 : 0;
    return 0;
}

/* Attention forward over every row.  Q is [B][Hq][Sq][D], K and V are
 * [B][Hkv][Sk][D] (bf16 bits), addressed through the element strides
 * qs/ks/vs = (batch, head, seq, dim).  O and Omag are dense binary64
 * [B][Hq][Sq][D]; lse is dense [B][Hq][Sq].  Returns 0, or -1 on bad sizes
 * (Hq not a multiple of Hkv included). */
int oracle_attention_fwd(int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D,
                         const uint16_t* Q, const int64_t* qs, const uint16_t* K,
                         const int64_t* ks, const uint16_t* V, const int64_t* vs,
                         double scale, int causal, double* O, double* Omag, double* lse,
                         int nthreads) {
    attn_job_t J;
    if (attn_setup(&J, B, Hq, Hkv, Sq, Sk, D, Q, qs, K, ks, V, vs, scale, causal)) return -1;
    J.O = O;
    J.Omag = Omag;
    J.lse = lse;
    return run_attn_split(&J, B * Hq * Sq, nthreads);
}

/* The same for a sample of rows: rows holds n triples (b, h, i); row t of
 * the dense outputs O/Omag [n][D] and lse [n] belongs to triple t. */
int oracle_attention_fwd_at(int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D,
                            const uint16_t* Q, const int64_t* qs, const uint16_t* K,
                            const int64_t* ks, const uint16_t* V, const int64_t* vs,
                            double scale, int causal, const int64_t* rows, int64_t n,
                            double* O, double* Omag, double* lse, int nthreads) {
    attn_job_t J;
    if (attn_setup(&J, B, Hq, Hkv, Sq, Sk, D, Q, qs, K, ks, V, vs, scale, causal)) return -1;
    for (int64_t t = 0; t < n; ++t)
        if (rows[3 * t] < 0 || rows[3 * t] >= B || rows[3 * t + 1] < 0 || rows[3 * t + 1] >= Hq ||
            rows[3 * t + 2] < 0 || rows[3 * t + 2] >= Sq)
            return -1;
    J.rows = rows;
    J.O = O;
    J.Omag = Omag;
    J.lse = lse;
    return run_attn_split(&J, n, nthreads);
}
