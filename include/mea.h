/*
 * mea.h - C ABI of the memory-efficient exact attention library for AMD
 * Instinct MI355X (gfx950).
 *
 * What it computes. Exact softmax attention O = softmax(Q K^T / sqrt(d)) V
 * ("Fast and memory-efficient exact attention 分析", section 数学表达形式;
 * "当注意力成为瓶颈…", section 平方级的诅咒: the softmax normalises every row of
 * the score matrix over all keys), and its gradient. As in "Self-attention
 * Does Not Need O(n^2) Memory" (abstract; method sections), keys and values
 * are visited in tiles while every query row keeps a running maximum and a
 * running sum of exponentiated scores, and the division by that sum happens
 * once at the end, so no n x n matrix is ever stored. The backward pass
 * recomputes score tiles from the per-row statistics the forward pass saved
 * (the pages' checkpoint-and-recompute differentiation).
 *
 * Conventions shared by every entry point.
 *  - Tensors q, k, v, o, dO, dq, dk, dv are contiguous row-major
 *    [B, H, n, d] arrays in the element type `dt` (d fastest). attn_fwd and
 *    attn_bwd are self-attention: queries and keys have the same length n
 *    and every query head has its own key/value head. The *_ex and splitkv
 *    entry points generalise both (see attn_fwd_ex). No mask, no causal
 *    structure, no dropout. The score scale is fixed at 1/sqrt(d).
 *  - Every pointer is a DEVICE pointer on the current HIP device, owned by the
 *    caller, and must be 16-byte aligned. The library allocates no device
 *    memory and keeps no state between calls (attn_bwd_noalloc aside, whose
 *    scratch array is part of the loaded library); it is thread-safe.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL means
 *    the null stream). Nothing is synchronised. Inputs must stay valid and
 *    outputs untouched until the stream reaches the work.
 *  - Outputs (o, row_max, row_sum, dq, dk, dv and the part of the workspace
 *    a call uses) must not overlap one another or any input; inputs may share
 *    memory (q == k == v is allowed). Overlaps are rejected with MEA_ERR_ALIAS.
 *  - Arguments are validated on the host before any HIP call, in this order:
 *    dtype, shape, head dimension, null pointers, alignment, workspace,
 *    overlap of outputs. A
 *    call with B, H or n equal to 0 does nothing and returns MEA_OK (pointers
 *    may then be NULL). MEA_ERR_LAUNCH reports a launch failure seen by
 *    hipGetLastError right after the launch; faults during execution surface
 *    at the caller's next synchronisation, as with any HIP kernel.
 *  - Supported: dt in {MEA_DTYPE_BF16, MEA_DTYPE_F32}, d in {64, 128},
 *    n (and n_q, n_k, and (H/H_kv)*n_q) <= 2^24, B*H <= 2^24, and
 *    B*H_kv * ceil(max((H/H_kv)*n_q, n_k) / 64) <= 2^22 (B*H * ceil(n / 64)
 *    for the self-attention calls), which keeps every launch grid within 2^31
 *    work-items. Larger shapes are rejected with MEA_ERR_SHAPE.
 *  - Accuracy: bf16 inputs are multiplied exactly on bf16 MFMA with fp32
 *    accumulation; probabilities are rounded to bf16 (round-to-nearest-even)
 *    for the P V product; outputs are rounded to bf16 (RNE). fp32 inputs
 *    form scores on fp64 MFMA (exact products, fp64 sums), subtract the row
 *    maximum in fp64, then exponentiate and accumulate P V in fp32.
 */
#ifndef MEA_H
#define MEA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exported symbols of libmea.so (the library is built with hidden visibility). */
#if defined(__GNUC__) || defined(__clang__)
#define MEA_API __attribute__((visibility("default")))
#else
#define MEA_API
#endif

typedef enum {
  MEA_DTYPE_F32 = 0,  /* IEEE binary32 */
  MEA_DTYPE_BF16 = 1  /* bfloat16 */
} mea_dtype_t;

typedef enum {
  MEA_OK = 0,
  MEA_ERR_NULL = 1,        /* a required pointer is NULL */
  MEA_ERR_SHAPE = 2,       /* negative or too large B, H, n */
  MEA_ERR_UNSUPPORTED = 3, /* unsupported dtype or head dimension d */
  MEA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  MEA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required */
  MEA_ERR_LAUNCH = 6,      /* the HIP runtime rejected a kernel launch */
  MEA_ERR_ALIAS = 7        /* an output overlaps an input or another output */
} mea_status_t;

/*
 * attn_fwd - forward pass.
 *
 * o[b,h,i,:] = sum_j softmax_j(q[b,h,i,:] . k[b,h,j,:] / sqrt(d)) v[b,h,j,:]
 *
 * Keys and values are swept tile by tile with a running maximum and running
 * sum per query row, normalising once at the end ("Self-attention Does Not
 * Need O(n^2) Memory": abstract; method bullets of the English digest;
 * "当注意力成为瓶颈…", section IO感知, two-block merge).
 *
 * q, k, v : inputs [B,H,n,d] in dt.            o : output [B,H,n,d] in dt.
 * row_max : output fp32 [B,H,n] or NULL: m_i = max_j q_i.k_j / sqrt(d)
 *           (natural units of the scaled score).
 * row_sum : output fp32 [B,H,n] or NULL: l_i = sum_j exp(q_i.k_j/sqrt(d) - m_i)
 *           for the m_i stored in row_max (for fp32 inputs the maximum is
 *           found in fp64 and l_i re-based onto its fp32 rounding, so that
 *           m_i + log(l_i) is the row's log-sum-exp to fp32 rounding of l_i).
 *           The two statistics are what attn_bwd needs; pass both or neither
 *           (passing exactly one is MEA_ERR_NULL).
 * No workspace: the only memory beyond inputs and outputs is the optional
 * 8*B*H*n bytes of statistics.
 */
MEA_API mea_status_t attn_fwd(mea_dtype_t dt, int64_t B, int64_t H, int64_t n, int64_t d,
                      const void* q, const void* k, const void* v, void* o,
                      float* row_max, float* row_sum, void* stream);

/*
 * attn_bwd_workspace_bytes - bytes of device workspace attn_bwd is best given.
 *
 * The minimum is the row terms: 8 bytes per query row for bf16 (D_i =
 * sum_c dO_ic * O_ic and the base-2 log-sum-exp of the row, both fp32), 16
 * for fp32 (the log-sum-exp in fp64, D_i), times B*H*n. On a grid too small to
 * fill the GPU (at most 256 workgroups of the unsplit backward) the returned
 * size adds room for a split backward: each workgroup's sweep is cut into up
 * to 16 ranges, each writing fp32 partial gradients that a reduce pass sums
 * (at most 32 MiB in all). With only the minimum, attn_bwd runs
 * unsplit; the results agree to fp32 rounding of the partial sums.
 * Returns 0 for empty or invalid shapes.
 */
MEA_API size_t attn_bwd_workspace_bytes(mea_dtype_t dt, int64_t B, int64_t H, int64_t n, int64_t d);

/*
 * attn_bwd - backward pass of L = sum(O * dO), by recomputation.
 *
 * The pages give no gradient formulas, only that differentiation recomputes
 * chunk intermediates instead of storing them ("Self-attention Does Not Need
 * O(n^2) Memory": abstract; 方法详解; English digest method bullets). The
 * textbook Jacobian of the softmax is used:
 *   P = softmax(S), S = Q K^T / sqrt(d);  dV = P^T dO;  dP = dO V^T;
 *   D_i = sum_j P_ij dP_ij = sum_c dO_ic O_ic;  dS = P * (dP - D);
 *   dQ = dS K / sqrt(d);  dK = dS^T Q / sqrt(d).
 * P is rebuilt tile by tile from row_max and row_sum; no n x n array exists.
 * bf16 inputs take D from o (dO . O, fp32); fp32 inputs form it from the
 * rebuilt P and dP (sum_j P_ij dP_ij / sum_j P_ij, in fp64), which keeps each
 * row of dS summing to zero where one key dominates the row, and do not read o.
 *
 * q, k, v, o, dO : inputs [B,H,n,d] in dt (o from attn_fwd on the same q,k,v).
 * row_max, row_sum : the fp32 [B,H,n] statistics attn_fwd wrote for these
 *                    inputs (required).
 * dq, dk, dv : outputs [B,H,n,d] in dt; fully overwritten.
 * workspace  : device scratch, 16-byte aligned, owned by the caller: at least
 *              the row terms (8*B*H*n bytes for bf16, 16*B*H*n for fp32, else
 *              MEA_ERR_WORKSPACE), and attn_bwd_workspace_bytes(...) bytes for
 *              the split backward on small grids; its contents on entry do not
 *              matter and on return are unspecified. The part this call uses
 *              (the row terms, or the whole split layout) must not overlap the
 *              inputs or outputs.
 * Supported: dt in {MEA_DTYPE_BF16, MEA_DTYPE_F32} with d in {64, 128}. fp32
 * inputs form scores and dP on fp64 MFMA and the exponent in fp64, as the
 * forward does, and accumulate dQ, dK, dV on fp64 MFMA; P and dS are fp32.
 */
MEA_API mea_status_t attn_bwd(mea_dtype_t dt, int64_t B, int64_t H, int64_t n, int64_t d,
                      const void* q, const void* k, const void* v, const void* o,
                      const void* dO, const float* row_max, const float* row_sum,
                      void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * attn_bwd_noalloc - attn_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, arguments and errors as attn_bwd, minus
 * the workspace, which is replaced by a scratch array inside the library.
 *
 * The scratch array holds MEA_NOALLOC_SCRATCH_BYTES (32 MiB). Each GPU the
 * library runs on holds its own copy from the moment the library is loaded
 * until the process ends; its device address is looked up on the first call
 * made with that GPU current, which may itself be under HIP graph capture. The call needs the row terms of attn_bwd's
 * workspace (8*B*H*n bytes for bf16, 16*B*H*n for fp32); larger shapes are
 * rejected with MEA_ERR_WORKSPACE before anything runs. When the split layout
 * of a small grid (see attn_bwd_workspace_bytes) also fits, it is used, and
 * the results equal those of attn_bwd given that workspace, bit for bit;
 * otherwise they equal attn_bwd given the row terms only.
 * No memory is allocated and nothing needs clearing between calls: every byte
 * a call reads from the scratch array it wrote first.
 * Calls share their GPU's array: two calls that may run at the same time on
 * one GPU (different streams, or different host threads without ordering)
 * race on it and give undefined results. Calls ordered on one stream are safe.
 * MEA_ERR_LAUNCH also reports a failure to look up the array's address.
 */
#define MEA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
MEA_API mea_status_t attn_bwd_noalloc(mea_dtype_t dt, int64_t B, int64_t H, int64_t n, int64_t d,
                              const void* q, const void* k, const void* v, const void* o,
                              const void* dO, const float* row_max, const float* row_sum,
                              void* dq, void* dk, void* dv, void* stream);

/*
 * attn_fwd_ex - forward pass with separate query/key lengths and shared
 * key/value heads (grouped-query attention; multi-query when H_kv = 1).
 *
 * o[b,h,i,:] = sum_j softmax_j(q[b,h,i,:] . k[b,g(h),j,:] / sqrt(d)) v[b,g(h),j,:]
 * with g(h) = h / (H / H_kv): the H query heads form H_kv groups of
 * consecutive heads, each reading one key/value head ("当注意力成为瓶颈…",
 * section 推理优化：减少KV Cache, describes the grouping; taking consecutive
 * heads is this library's reading). n_q != n_k covers cross-attention and
 * the decoding step of the same section (a few new queries against a long
 * key/value cache).
 *
 * q, o : [B,H,n_q,d] in dt.   k, v : [B,H_kv,n_k,d] in dt.
 * row_max, row_sum : fp32 [B,H,n_q] or NULL, as for attn_fwd.
 * H must be a multiple of H_kv (else MEA_ERR_SHAPE). n_q = 0 is a no-op;
 * n_k = 0 with n_q > 0 is MEA_ERR_SHAPE (no softmax over zero keys).
 * attn_fwd(dt,B,H,n,d,...) is attn_fwd_ex(dt,B,H,H,n,n,d,...).
 */
MEA_API mea_status_t attn_fwd_ex(mea_dtype_t dt, int64_t B, int64_t H, int64_t H_kv, int64_t n_q,
                         int64_t n_k, int64_t d, const void* q, const void* k, const void* v,
                         void* o, float* row_max, float* row_sum, void* stream);

/*
 * attn_bwd_ex_workspace_bytes - workspace attn_bwd_ex is best given: the row
 * terms, 8*B*H*n_q (bf16) or 16*B*H*n_q (fp32), which are the minimum, plus
 * the split backward's partial gradients on small grids, as for
 * attn_bwd_workspace_bytes. Returns 0 for empty or invalid shapes.
 */
MEA_API size_t attn_bwd_ex_workspace_bytes(mea_dtype_t dt, int64_t B, int64_t H, int64_t H_kv,
                                   int64_t n_q, int64_t n_k, int64_t d);

/*
 * attn_bwd_ex - backward pass of attn_fwd_ex (same gradient formulas as
 * attn_bwd). A key/value head is read by every query head of its group, so
 * dk and dv are the sums over that group (chain rule).
 *
 * q, o, dO, dq : [B,H,n_q,d].   k, v, dk, dv : [B,H_kv,n_k,d].
 * row_max, row_sum : the [B,H,n_q] statistics attn_fwd_ex wrote.
 * n_q = 0 with n_k > 0 writes dk = dv = 0 (only k, v, dk, dv are then
 * checked and the workspace may be NULL); n_k = 0 with n_q > 0 is
 * MEA_ERR_SHAPE. Supported: bf16 and fp32, d in {64, 128}.
 */
MEA_API mea_status_t attn_bwd_ex(mea_dtype_t dt, int64_t B, int64_t H, int64_t H_kv, int64_t n_q,
                         int64_t n_k, int64_t d, const void* q, const void* k, const void* v,
                         const void* o, const void* dO, const float* row_max,
                         const float* row_sum, void* dq, void* dk, void* dv, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * attn_fwd_splitkv - attn_fwd_ex with the keys of every head cut into
 * consecutive ranges that separate workgroups reduce independently, for
 * grids too small to fill the GPU (few heads, few query rows, decoding).
 *
 * "Self-attention Does Not Need O(n^2) Memory" (方法详解; English digest
 * method bullets) processes key chunks independently and combines their
 * summaries; "当注意力成为瓶颈…", section IO感知, gives the two-block merge.
 * Pass 1 writes, per range and query row, the range's normalised partial
 * output (fp32) and its maximum and sum; pass 2 merges the ranges of every
 * row and writes o (and row_max / row_sum) exactly as attn_fwd_ex defines
 * them. The two passes run on `stream` in order.
 *
 * num_splits : 0 lets the library choose; k >= 1 asks for k ranges. The
 *              count used is attn_fwd_splitkv_num_splits(...): at most 256,
 *              at most one per key tile, every range non-empty. With one
 *              range this is attn_fwd_ex and needs no workspace.
 * workspace  : at least attn_fwd_splitkv_workspace_bytes(...) bytes
 *              (splits * B*H*n_q * (d + 4) * 4), 16-byte aligned, owned by
 *              the caller; may be NULL when that size is 0. Contents on entry
 *              do not matter; on return they are unspecified.
 * Other arguments and errors as attn_fwd_ex; negative num_splits is
 * MEA_ERR_SHAPE.
 */
MEA_API mea_status_t attn_fwd_splitkv(mea_dtype_t dt, int64_t B, int64_t H, int64_t H_kv, int64_t n_q,
                              int64_t n_k, int64_t d, const void* q, const void* k, const void* v,
                              void* o, float* row_max, float* row_sum, int64_t num_splits,
                              void* workspace, size_t workspace_bytes, void* stream);

/* attn_fwd_splitkv_num_splits - number of key ranges attn_fwd_splitkv uses
 * for these arguments (1 for an empty problem; 0 for invalid arguments). */
MEA_API int64_t attn_fwd_splitkv_num_splits(mea_dtype_t dt, int64_t B, int64_t H, int64_t H_kv,
                                    int64_t n_q, int64_t n_k, int64_t d, int64_t num_splits);

/* attn_fwd_splitkv_workspace_bytes - workspace attn_fwd_splitkv needs for
 * these arguments (0 when it uses one range, or for empty/invalid shapes). */
MEA_API size_t attn_fwd_splitkv_workspace_bytes(mea_dtype_t dt, int64_t B, int64_t H, int64_t H_kv,
                                        int64_t n_q, int64_t n_k, int64_t d, int64_t num_splits);

/* attn_status_str - static, NUL-terminated name of a status code
 * ("MEA_OK", "MEA_ERR_NULL", ...); "MEA_UNKNOWN_STATUS" for other values. */
MEA_API const char* attn_status_str(mea_status_t s);

/* mea_version - library version as 10000*major + 100*minor + patch. */
MEA_API int mea_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MEA_H */
