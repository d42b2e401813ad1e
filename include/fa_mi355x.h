/*
 * fa_mi355x.h - exact softmax attention, forward and backward, for AMD Instinct
 * MI355X (gfx950).  C ABI of libfa_mi355x.so.
 *
 * The operation (softmax attention and its gradient):
 *   S   = scale * Q_h K_g^T            (g = h / (Hq/Hkv): consecutive query heads
 *                                        share a key/value head)
 *   LSE = log sum_j exp(S_ij)           (natural log, scaled-score domain)
 *   P   = exp(S - LSE),  O = P V
 *   D   = rowsum(dO o O),  dP = dO V^T,  dS = P o (dP - D)
 *   dQ  = scale * dS K,  dK = scale * sum_{h in g} dS^T Q_h,  dV = sum_{h in g} P^T dO_h
 * The backward recomputes S and P tile by tile from Q, K and the stored LSE and
 * never writes an N_q x N_kv matrix to memory (rustytorch
 * "flash_attention_backward.cu", header comment and tiled backward kernel;
 * Triton issue "Extra transposes cause 8x speedup for sequence-parallel Flash
 * Attention backward", the key/value-block-parallel _bwd_kernel).  GQA, causal
 * masking and N_q != N_kv follow the feature list of the Liger-Kernel pull
 * request "[Kernel] Flash attention 2".
 *
 * Causal masking is bottom-right aligned: query i sees key j iff
 * j <= i + (N_kv - N_q).  A query row that sees no key gets O = 0, LSE = -inf
 * and a zero dQ row.
 *
 * Conventions shared by every call
 *   - Pointers are DEVICE pointers owned by the caller.  The library allocates
 *     nothing and keeps no state between calls; calls are safe from several host
 *     threads on different streams.
 *   - Layout: contiguous row-major, head dimension fastest.
 *       q, o, dout, dq : [B, Hq,  N_q,  d]
 *       k, v, dk, dv   : [B, Hkv, N_kv, d]
 *       lse            : [B, Hq,  N_q]  float32
 *   - dtype: FA_DTYPE_FP16 or FA_DTYPE_BF16; every 16-bit tensor of a call has
 *     that dtype.  Accumulation is float32; 16-bit results are rounded to
 *     nearest even.
 *   - Every pointer must be 16-byte aligned.  A pointer may be NULL only when its
 *     tensor has no element.
 *   - d is a multiple of 32 up to 256: 32, 64, 96, 128, 160, 192, 224 or 256 (the
 *     Liger-Kernel pull request "[Kernel] Flash attention 2", Details, claims no
 *     restriction on the head dimension; these are the widths with a kernel
 *     instance).  The fused atomic dQ path
 *     (FA_DQ_ATOMIC) is built for d = 64 and 128 only.  B, N_q, N_kv >= 0
 *     (zero-size calls are valid), Hq and Hkv >= 1 with Hq % Hkv == 0,
 *     N * d < 2^31 per head, B and Hq <= 65535.
 *   - softmax_scale must be finite and > 0.  causal: 0 = off, nonzero = on.
 *   - stream: a hipStream_t passed as void* (NULL = the null stream).  Work is
 *     enqueued asynchronously; no call synchronises.
 *   - Errors: every argument is checked on the host before anything is enqueued;
 *     on error nothing is launched and no output is written, and a negative
 *     FA_ERR_* code is returned.  FA_ERR_HIP reports a failed kernel launch.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_OK            0
#define FA_ERR_NULLPTR  -1  /* required pointer is NULL */
#define FA_ERR_SHAPE    -2  /* bad B/Hq/Hkv/N_q/N_kv, Hq % Hkv != 0, or size limits */
#define FA_ERR_HEADDIM  -3  /* d not a multiple of 32 up to 256, or FA_DQ_ATOMIC, dBias,
                               dropout or a bias that varies along heads or rows
                               with d not in {64, 128} */
#define FA_ERR_DTYPE    -4  /* dtype not FP16/BF16 */
#define FA_ERR_SCALE    -5  /* softmax_scale not finite or <= 0 */
#define FA_ERR_WORKSPACE -6 /* workspace NULL/misaligned or smaller than required */
#define FA_ERR_ALIGN    -7  /* a tensor pointer is not 16-byte aligned */
#define FA_ERR_HIP      -8  /* a kernel launch failed (hipGetLastError) */
#define FA_ERR_MODE     -9  /* unknown dq_mode, or FA_DQ_ATOMIC with a bias or dropout */
#define FA_ERR_SCRATCH  -10 /* fa_bwd_noalloc: the call needs more scratch than it holds */
#define FA_ERR_BIAS     -11 /* bias strides negative, not multiples of 8, or too large;
                               or dbias with N_kv > 2^22 */
#define FA_ERR_DROPOUT  -12 /* dropout_p not in [0, 1] */

#define FA_DTYPE_FP16 0
#define FA_DTYPE_BF16 1

/* How fa_bwd_ex produces dQ (the two dQ decompositions, compared by measurement). */
#define FA_DQ_AUTO     0  /* the faster path, as measured for this shape class */
#define FA_DQ_ATOMIC   1  /* dS K tiles added into a float32 buffer by the dK/dV
                             kernel with float atomics, then rounded to dtype */
#define FA_DQ_SEPARATE 2  /* a query-block-parallel kernel recomputes S, P, dP and
                             dS and writes dQ once; no atomics, bitwise repeatable */

/*
 * Forward: O and LSE from Q, K, V.
 * Source: the pages print no forward kernel; what the backward needs from it is
 * fixed by the two backward listings, which rebuild P = exp(S - LSE) from one
 * float per query row (rustytorch "flash_attention_backward.cu", tiled backward
 * kernel: the probabilities recomputed from the stored row statistic; Triton issue
 * "Extra transposes cause 8x speedup...", _bwd_kernel listing: p = exp(qk - m)
 * with m loaded per row).  O = softmax(S) V is the forward whose gradient the
 * backward computes.
 * Writes o [B,Hq,N_q,d] (dtype) and lse [B,Hq,N_q] (float32, natural log of the
 * row sum of exp(scale * q.k) over visible keys; -inf for a row with none).
 * Reads q, k, v.  Returns FA_OK or an FA_ERR_* code; on error nothing is written.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int Hq, int Hkv, int Nq, int Nkv, int d,
           float softmax_scale, int causal, int dtype, void* stream);

/*
 * Bytes of device workspace fa_bwd needs for these arguments (0 when the call
 * needs none).  The workspace holds the per-row D = rowsum(dO o O) (precomputed
 * per query row as the Triton issue's _bwd_kernel listing loads it), the row
 * statistic in the kernels' log2 form, the work-queue counters and, on the atomic
 * dQ path, the float32 dQ accumulator (the Triton harness's zeroed float32 dq
 * buffer).  Returns 0 for invalid arguments as well; fa_bwd then reports the
 * error.
 */
size_t fa_bwd_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nkv, int d,
                              int causal, int dtype);

/* Workspace bytes fa_bwd_ex needs with the given dq_mode. */
size_t fa_bwd_ex_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nkv, int d,
                                 int causal, int dtype, int dq_mode);

/*
 * Backward: dQ, dK, dV from Q, K, V, O, dO and LSE.
 * Source: rustytorch "flash_attention_backward.cu", tiled backward kernel (per
 * tile: S recomputed, P = exp(S - LSE), dV += P^T dO, dP = dO V^T,
 * dS = P o (dP - D), dK += dS^T Q, dQ += dS K, with D the row dot product of dO
 * and O); Triton issue "Extra transposes cause 8x speedup for sequence-parallel
 * Flash Attention backward", _bwd_kernel listing (the key-block-parallel loop over
 * query blocks with K and V resident, D precomputed, dq accumulated with float
 * atomics).  Where the two differ this library follows the definition (see the
 * operation at the top).
 * o and lse must be what fa_fwd returns for the same q, k, v and arguments (or
 * the same quantities computed elsewhere).  dq, dk, dv are fully overwritten
 * (callers need not zero them).  workspace: caller-owned device memory of at
 * least fa_bwd_workspace_bytes(...) bytes, 16-byte aligned, not shared with a
 * concurrent call; its contents on entry do not matter.  Kernels run in order
 * on `stream`, for the dQ path FA_DQ_AUTO selects: with the separate pass, the
 * query-block-parallel dQ pass (which also computes D = rowsum(dO o O) of its
 * rows) and then the key/value-block-parallel dK/dV kernel; with float atomics,
 * a row preprocess (D), the fused dK/dV/dQ kernel and a dQ conversion.  Returns
 * FA_OK or an FA_ERR_* code; a rejected call launches nothing and writes nothing.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const float* lse, const void* dout, void* dq, void* dk, void* dv,
           int B, int Hq, int Hkv, int Nq, int Nkv, int d,
           float softmax_scale, int causal, int dtype,
           void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_bwd with an explicit dQ path and optional timing events.
 * Source: the two dQ decompositions of the pages - float atomics into a float32
 * buffer from the key-block-parallel kernel (Triton issue "Extra transposes...",
 * _bwd_kernel listing, tl.atomic_add of dq; flash-attention-minimal "Implement
 * backward pass", the thread's note that atomic and plain adds time differently)
 * and a query-block-parallel pass (the grid of the rustytorch tiled backward
 * kernel, which owns a block of query rows).
 * dq_mode: FA_DQ_AUTO, FA_DQ_ATOMIC or FA_DQ_SEPARATE.
 * ev_begin / ev_end: NULL, or hipEvent_t handles (as void*) that are recorded on
 * `stream` immediately before and after the launch of the dK/dV kernel, the
 * dominant kernel of the backward, so a caller can time it alone.
 * workspace_bytes must be >= fa_bwd_ex_workspace_bytes(..., dq_mode).
 */
int fa_bwd_ex(const void* q, const void* k, const void* v, const void* o,
              const float* lse, const void* dout, void* dq, void* dk, void* dv,
              int B, int Hq, int Hkv, int Nq, int Nkv, int d,
              float softmax_scale, int causal, int dtype, int dq_mode,
              void* ev_begin, void* ev_end,
              void* workspace, size_t workspace_bytes, void* stream);

/* The dQ path FA_DQ_AUTO resolves to for these arguments (FA_DQ_ATOMIC or
 * FA_DQ_SEPARATE). */
int fa_bwd_auto_dq_mode(int B, int Hq, int Hkv, int Nq, int Nkv, int d,
                        int causal, int dtype);

/*
 * Forward with an additive score bias and dropout of the probabilities.
 * Source: the Liger-Kernel pull request "[Kernel] Flash attention 2", Details,
 * which lists an attention mask / attention bias and dropout (forward only there;
 * the backward of both is fa_bwd_bias_dropout below).  Definitions:
 *   S = scale * Q_h K_g^T + bias_h,  LSE and P from S as in fa_fwd,
 *   O = (P o Z) V  with Z_ij = 256 / T if element (i, j) is kept, else 0.
 * bias: NULL (no bias), or 16-bit values of the call's dtype, 16-byte aligned;
 *   element (b, h, i, j) of the [B, Hq, N_q, N_kv] bias sits at
 *   b * bias_stride_b + h * bias_stride_h + i * bias_stride_q + j (elements), so a
 *   zero stride broadcasts that dimension (e.g. a per-key padding mask [B,1,1,N_kv]:
 *   stride_h = stride_q = 0).  Strides are >= 0 and multiples of 8 (16-byte rows),
 *   bias_stride_q <= 2^22.  Rows are read in whole 16-byte pieces: each row must be
 *   readable for N_kv rounded up to a multiple of 8 elements (the values past N_kv
 *   are ignored).  -inf entries mask keys; a row whose every visible key is masked
 *   gets O = 0 and LSE = -inf.
 * dropout_p in [0, 1]: element (b, h, i, j) is kept iff byte j % 4 of word i % 4 of
 *   Philox4x32-10 (Salmon et al., SC 2011) with counter (j / 4, i / 4, h, b) and key
 *   (seed low word, seed high word) is below T = floor((1 - p) * 256 + 1/2); the
 *   keep probability is T / 256 (p rounded to a multiple of 1/256).  LSE is that of
 *   the undropped P, so the backward can rebuild P from it.
 * With bias NULL and dropout_p = 0 this is fa_fwd.  A bias with bias_stride_h =
 * bias_stride_q = 0 (one value per batch and key, e.g. a key-padding mask) and no
 * dropout runs at every head dim, on kernels as fast as the plain ones, as does
 * its backward when no dbias is asked for; any other bias, and dropout, need
 * d = 64 or 128 (FA_ERR_HEADDIM otherwise).  Returns FA_OK or an FA_ERR_* code;
 * on error nothing is launched or written.
 */
int fa_fwd_bias_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int Hq, int Hkv, int Nq, int Nkv, int d,
                        float softmax_scale, int causal, int dtype,
                        const void* bias, long long bias_stride_b, long long bias_stride_h,
                        long long bias_stride_q, float dropout_p, unsigned long long seed,
                        void* stream);

/*
 * Backward of fa_fwd_bias_dropout: dQ, dK, dV and, if dbias is not NULL, the bias
 * gradient dBias = dS.
 * Source: as fa_bwd; the bias is part of the score, so its gradient is the score
 * gradient; with dropout dV = (P o Z)^T dO, dP = (dO V^T) o Z, and D = rowsum(dO o O),
 * dS = P o (dP - D) keep their form (Liger-Kernel pull request "[Kernel] Flash
 * attention 2", Details: bias and dropout).
 * bias, strides, dropout_p and seed: exactly those given to the forward that made
 * o and lse.  dbias: NULL, or [B, Hq, N_q, N_kv] contiguous in the call's dtype,
 * 16-byte aligned, fully overwritten (zeros where the causal mask hides a key);
 * the gradient of a bias broadcast along some dimension is this tensor summed along
 * it (left to the caller).  The dQ path is the separate pass (FA_DQ_SEPARATE);
 * workspace as for fa_bwd_ex with FA_DQ_SEPARATE.  With bias and dbias NULL and
 * dropout_p = 0 this is fa_bwd with that path.  Returns FA_OK or an FA_ERR_* code;
 * on error nothing is launched or written.
 */
int fa_bwd_bias_dropout(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        int B, int Hq, int Hkv, int Nq, int Nkv, int d,
                        float softmax_scale, int causal, int dtype,
                        const void* bias, long long bias_stride_b, long long bias_stride_h,
                        long long bias_stride_q, void* dbias, float dropout_p,
                        unsigned long long seed, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * Allocation-free backward, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, checks, kernels and results as fa_bwd with the separate dQ
 * path (FA_DQ_SEPARATE), minus the workspace: its scratch (8 bytes per query row
 * plus 256 bytes of work-queue counters, each region 256-byte aligned) lives in a
 * static device array of FA_NOALLOC_SCRATCH_BYTES bytes that each device holds
 * from the library's first use on it until the process ends.  The call allocates
 * nothing and calls no allocating routine.  Returns FA_ERR_SCRATCH, launching
 * nothing, when the problem needs more (with 16 MiB: B*Hq*N_q up to about 2.09
 * million query rows).  Every call on a device shares that device's array: calls
 * that overlap on one device (several streams or host threads) race and must be
 * serialised by the caller.  Each call clears the counters that must start at
 * zero.
 */
#define FA_NOALLOC_SCRATCH_BYTES (16u << 20)
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dout, void* dq, void* dk, void* dv,
                   int B, int Hq, int Hkv, int Nq, int Nkv, int d,
                   float softmax_scale, int causal, int dtype, void* stream);

/* FA_NOALLOC_SCRATCH_BYTES as built into the library. */
size_t fa_bwd_noalloc_max_scratch_bytes(void);

/* Static text for a status code; never NULL. */
const char* fa_status_string(int status);

/* Library version as 10000*major + 100*minor + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
