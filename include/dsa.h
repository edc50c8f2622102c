/*
 * dsa.h - C ABI of libdsa.so, the DeepSeek Sparse Attention (DSA) hot path of
 * one attention layer on an AMD Instinct MI355X (gfx950).
 *
 * The path has three stages (page "arXiv'25 | DSA ... DeepSeek-V3.2" on
 * marsggbo.github.io, section 3, its three equations; page "DeepSeekV3.2之DSA"
 * on yuyanqi.com, parts 3-5):
 *   1. lightning-indexer scores I[t,s] = sum_j w[t,j] * ReLU(q[t,j] . k[s]) with
 *      FP8 E4M3 q and k, 64 indexer heads of width 128, one key head shared by
 *      all indexer heads;
 *   2. per-query top-k (k <= 2048) over the visible history;
 *   3. MQA-mode MLA attention of 128 query heads over only the selected
 *      576-wide bf16 latent rows (512 latent dims, which are also the value, and
 *      64 rotary dims).
 *
 * Conventions shared by every call
 * --------------------------------
 * Pointers.  Every array pointer is DEVICE memory owned by the caller (for
 *   example torch allocations).  The structs themselves are read on the host
 *   during the call and may be freed when it returns.  The library never
 *   allocates or frees memory: scratch space is the caller's `ws` buffer,
 *   sized by dsa_workspace_bytes().  Arrays of 16-byte elements or rows must be
 *   16-byte aligned; `ws` must be 256-byte aligned.
 * Streams.  Each call enqueues its kernels on `stream` and returns at once;
 *   nothing synchronises.  Two calls that share a workspace must be ordered
 *   on one stream.
 * Positions.  Query i belongs to sequence q_seq[i] and sees the positions
 *   [0, q_nvis[i]) of that sequence (decode: the whole history of length L;
 *   causal prefill: n_vis = t for the token at 0-based position t).  The pages
 *   count positions from 1; the ABI counts from 0.
 * Caches.  The index-key cache (FP8 codes k_fp8[R,128] + fp32 k_scale[R]) and
 *   the latent cache (bf16 kv[R,576]) are stored per token and addressed by the
 *   same positions through one dsa_kv_layout (page "DeepSeekV3.2之DSA",
 *   part 5.2, point 3: two caches aligned by one set of indices).
 * Errors.  Each call returns DSA_OK (0) or a status below; the arguments are
 *   checked on the host before anything is launched, and nothing is launched
 *   when a check fails.  Index, block-table and length VALUES in device memory
 *   are trusted, not checked.  dsa_last_error() gives a message for the last
 *   failing call of the calling thread.
 */
#ifndef LIBDSA_DSA_H_
#define LIBDSA_DSA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Compile-time shapes (page "DeepSeekV3.2之DSA", part 3.2 table and part 5.1):
 * indexer heads and width, attention heads, latent row width, value width,
 * and the largest supported k. */
enum {
  DSA_HI = 64,
  DSA_DI = 128,
  DSA_H = 128,
  DSA_D = 576,
  DSA_DV = 512,
  DSA_KMAX = 2048
};

typedef enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1, /* null pointer, bad size, k out of [1, 2048], misalignment */
  DSA_ERR_UNSUPPORTED = 2, /* a shape or layout this library does not handle */
  DSA_ERR_WORKSPACE = 3,   /* ws is NULL or smaller than dsa_workspace_bytes() */
  DSA_ERR_HIP = 4          /* a HIP launch failed */
} dsa_status;

/* Where the tokens of each sequence live in the two caches.
 *   block_size == 0 : contiguous; position s of sequence q is row seq_row0[q] + s.
 *   block_size  > 0 : paged; block_size is a power of two and a multiple of 64;
 *                     position s of q is row
 *                     block_table[q * max_blocks + s / block_size] * block_size
 *                     + s % block_size.
 * num_rows is R, the row count of both caches (host value, used for checks). */
typedef struct dsa_kv_layout {
  int32_t num_seqs;
  int32_t block_size;
  int32_t max_blocks;
  int32_t reserved;
  int64_t num_rows;
  const int32_t *block_table; /* device int32 [num_seqs, max_blocks] if paged, else NULL */
  const int64_t *seq_row0;    /* device int64 [num_seqs] if contiguous, else NULL */
} dsa_kv_layout;

/* The queries of one call.  max_nvis is a host-side upper bound of q_nvis[]
 * (it sizes grids and workspaces; a smaller true maximum only wastes time). */
typedef struct dsa_queries {
  int32_t num_q;
  int32_t max_nvis;
  const int32_t *q_seq;  /* device int32 [num_q] */
  const int32_t *q_nvis; /* device int32 [num_q], each in [0, max_nvis] */
} dsa_queries;

/* Operation ids for dsa_workspace_bytes(). */
typedef enum dsa_op {
  DSA_OP_TOPK = 1,
  DSA_OP_MLA_DECODE = 2,
  DSA_OP_MLA_PREFILL = 3,
  DSA_OP_FORWARD = 4,
  DSA_OP_MLA_DENSE = 5     /* k is not used (any value in [1, 2048]) */
} dsa_op;

/* Per-row FP8 E4M3 quantisation, the step that writes the indexer's q and
 * key cache (page "DeepSeekV3.2之DSA", part 4.3 and part 5.2 point 3: FP8
 * index keys with a per-key dequantisation scale).
 *   x      : fp32 [rows, cols], row-major, 16-byte aligned;
 *   codes  : uint8 [rows, cols] E4M3 ("fn": max 448, no infinities);
 *   scales : fp32 [rows].
 * scale = absmax(row) / 448 (IEEE fp32 division; 1 for an all-zero row) and
 * code = E4M3(x / scale), rounded to nearest-even and saturated at +-448.
 * cols must be a multiple of 64 in [64, 512]. */
int dsa_quantize_fp8(const float *x, int64_t rows, int32_t cols, uint8_t *codes,
                     float *scales, hipStream_t stream);

/* The same quantiser with a power-of-two scale per row, the E8M0 form in which
 * the pages' indexer kernel takes its key scales (page "DeepSeekV3.2之DSA",
 * part 4.3, last step: the head sum times k_s in e8m0).  The page does not fix
 * the exponent; here e is the smallest integer with absmax(row) <= 448 * 2^e
 * (e = 0 for an all-zero row, clamped to [-127, 127]), so x / 2^e is exact and
 * never saturates:
 *   codes : uint8 [rows, cols] = E4M3(x / 2^e), rounded to nearest-even;
 *   e8m0  : uint8 [rows] = e + 127;
 *   scales: fp32 [rows] = 2^e exactly, or NULL.
 * cols must be a multiple of 64 in [64, 512]; x and codes 16-byte aligned. */
int dsa_quantize_fp8_e8m0(const float *x, int64_t rows, int32_t cols, uint8_t *codes,
                          uint8_t *e8m0, float *scales, hipStream_t stream);

/* Lightning-indexer scores (page "arXiv'25 | DSA ...", section 3, first
 * equation; page "DeepSeekV3.2之DSA", part 4.3, operation order):
 *   scores[i*ld + s] = k_scale[r(s)] * sum_j (w[i,j] * q_scale[i,j])
 *                       * ReLU(sum_d q_fp8[i,j,d] * k_fp8[r(s),d])
 * for s < q_nvis[i], where r(s) is the cache row of position s.  Entries at
 * s >= q_nvis[i] are not written.  Any constant factor (head-count or width
 * scaling) belongs in w.
 *   q_fp8   : uint8 [num_q, 64, 128] E4M3;   q_scale : fp32 [num_q, 64] or NULL (= 1);
 *   w       : fp32 [num_q, 64];
 *   k_fp8   : uint8 [R, 128] E4M3;           k_scale : fp32 [R];
 *   scores  : fp32 [num_q, ld], ld >= max_nvis, ld % 4 == 0. */
int dsa_indexer_scores(const dsa_queries *queries, const dsa_kv_layout *layout,
                       const uint8_t *q_fp8, const float *q_scale, const float *w,
                       const uint8_t *k_fp8, const float *k_scale, float *scores,
                       int64_t ld, hipStream_t stream);

/* dsa_indexer_scores with the key scales as E8M0 exponents (same page, part
 * 4.3): k_scale_e8m0 is uint8 [R], key scale 2^(b - 127) (b = 255, NaN in the
 * format, is not a valid scale), as dsa_quantize_fp8_e8m0 writes it.  One byte
 * per key instead of four; the scores equal dsa_indexer_scores' with the fp32
 * scales 2^(b - 127) bit for bit. */
int dsa_indexer_scores_e8m0(const dsa_queries *queries, const dsa_kv_layout *layout,
                            const uint8_t *q_fp8, const float *q_scale, const float *w,
                            const uint8_t *k_fp8, const uint8_t *k_scale_e8m0, float *scores,
                            int64_t ld, hipStream_t stream);

/* Top-k selection (page "arXiv'25 | DSA ...", section 3, second equation;
 * page "DeepSeekV3.2之DSA", part 4.4: indices of the min(topk, end_pos) largest
 * scores; part 4.5: a history no longer than k keeps every position).
 *   scores : fp32 [num_q, ld] (only s < q_nvis[i] is read; no NaN);
 *   idx    : int32 [num_q, k]  the count = min(k, n_vis) chosen positions in
 *            ascending order, then -1 padding;
 *   count  : int32 [num_q] or NULL.
 * Ties go to the lower position; -0 and +0 compare equal.  The result is
 * deterministic.  ws : dsa_workspace_bytes(DSA_OP_TOPK, queries, k) bytes. */
int dsa_topk(const dsa_queries *queries, const float *scores, int64_t ld, int32_t k,
             int32_t *idx, int32_t *count, void *ws, size_t ws_bytes,
             hipStream_t stream);

/* Sparse MQA-mode MLA attention (page "arXiv'25 | DSA ...", section 3, third
 * equation; page "DeepSeekV3.2之DSA", part 5.1: softmax(q . [c_kv; k_pe]^T) .
 * c_kv over the selected slots only, all 128 heads sharing one latent row).
 *   q     : bf16 [num_q, 128, 576] (absorbed query: 512 latent + 64 rotary);
 *   kv    : bf16 [R, 576] latent cache; the value is dims 0..511 of each row;
 *   idx   : int32 [num_q, k] positions; the first count[i] entries are attended
 *           (each must be in [0, q_nvis[i])); order does not matter; an entry
 *           outside that range is skipped (never read, not in the softmax);
 *   count : int32 [num_q], or NULL for min(k, q_nvis[i]);
 *   out   : fp32 [num_q, 128, 512] = sum_r softmax_r(z) * kv[r, 0:512] with
 *           z = softmax_scale * q . kv[r];
 *   lse   : fp32 [num_q, 128] natural-log sum of exp(z), or NULL.
 * An empty selection gives out = 0 and lse = -inf.
 * _decode gives a query several workgroups (for few queries), with k >= 128:
 * from 48 to 64 queries four workgroups of 32 heads each that attend over the
 * whole selection and need no workspace; up to 32 queries four such head
 * groups times several splits of the rows; otherwise several splits of the
 * rows over all heads.  Row splits write partial results that a second pass
 * merges.  _prefill gives each query one workgroup (for many queries).  All
 * compute the same function.
 * ws : dsa_workspace_bytes(DSA_OP_MLA_DECODE or _PREFILL, queries, k) bytes
 * (0 is allowed for _prefill). */
int dsa_sparse_mla_decode(const dsa_queries *queries, const dsa_kv_layout *layout,
                          const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                          const int32_t *count, int32_t k, float softmax_scale,
                          float *out, float *lse, void *ws, size_t ws_bytes,
                          hipStream_t stream);
/* dsa_sparse_mla_decode for callers that cannot allocate device memory or
 * pass a workspace (code under HIP graph capture, serving loops that forbid
 * allocation).  The split partials go to a scratch array inside the library,
 * DSA_NOALLOC_SCRATCH_BYTES on each GPU it runs on, held from module load
 * until the process ends; the call itself allocates and frees nothing.
 * Arguments and results as for dsa_sparse_mla_decode (same kernels, same
 * values), without ws.  The stream must belong to the current device.
 * Returns DSA_ERR_UNSUPPORTED, launching nothing, when this call's partials
 * (dsa_workspace_bytes(DSA_OP_MLA_DECODE, queries, k)) exceed the scratch:
 * for example 80 queries at k = 2048 fit (3 splits, 60.1 MiB), 285 queries
 * (2 splits, 142.8 MiB) do not, and 48 to 64 queries need none (head
 * groups).  Every call on one GPU shares that GPU's scratch, which keeps
 * the last call's contents: calls that overlap in time on one GPU (on
 * different streams, or unordered across threads) race and give wrong
 * results; order them on one stream. */
#define DSA_NOALLOC_SCRATCH_BYTES ((size_t)72 << 20)
int dsa_sparse_mla_decode_noalloc(const dsa_queries *queries, const dsa_kv_layout *layout,
                                  const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                                  const int32_t *count, int32_t k, float softmax_scale,
                                  float *out, float *lse, hipStream_t stream);
/* Dense mode: the same attention over every visible position [0, q_nvis[i])
 * of each query, with no indexer and no selection.  It is the pages'
 * short-context variant (page "arXiv'25 | DSA ...", section 6: short prefill
 * runs a dense masked attention that emulates DSA; page "DeepSeekV3.2之DSA",
 * part 4.5: a history no longer than k keeps every position), and the other
 * side of the sparse-versus-dense crossover.  Histories up to 2^20 positions;
 * longer ones are split over workgroups and merged, as in _decode.
 *   q, kv, out, lse : as for dsa_sparse_mla_decode;
 *   ws : dsa_workspace_bytes(DSA_OP_MLA_DENSE, queries, 1) bytes. */
int dsa_dense_mla(const dsa_queries *queries, const dsa_kv_layout *layout, const uint16_t *q,
                  const uint16_t *kv, float softmax_scale, float *out, float *lse, void *ws,
                  size_t ws_bytes, hipStream_t stream);
/* Sparse attention for many queries per call (causal prefill: query t of a
 * sequence attends to its selected positions among s < t; page "arXiv'25 |
 * DSA ...", section 3, third equation; page "DeepSeekV3.2之DSA", part 5.1).
 * The same function as dsa_sparse_mla_decode, scheduled with one workgroup
 * per query (no row splits, no partial results): the matrix-core pipeline
 * overlaps each tile's gather, QK^T, softmax and PV.  Arguments as for
 * dsa_sparse_mla_decode; ws may be NULL (dsa_workspace_bytes(
 * DSA_OP_MLA_PREFILL, ...) is 0). */
int dsa_sparse_mla_prefill(const dsa_queries *queries, const dsa_kv_layout *layout,
                           const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                           const int32_t *count, int32_t k, float softmax_scale,
                           float *out, float *lse, void *ws, size_t ws_bytes,
                           hipStream_t stream);

/* Indexer alignment loss, sparse training stage (page "arXiv'25 | DSA ...",
 * section 5.2, L_I over the selected set S_t; the mlpod.com page on
 * DeepSeek-V3.2-Exp, part 2.1.2).  For each query the target p is the
 * attention's probabilities over the set summed over the 128 heads and
 * L1-normalised over the set; the loss term is KL(p || Softmax(I)) over the
 * same set, and the gradient with respect to the indexer scores is
 * Softmax(I) - p (p is a constant: the indexer's inputs are detached).
 *   q, kv, idx, count, k : the attention's inputs, as for dsa_sparse_mla_decode
 *           (entries of idx outside [0, q_nvis[i]) are not in the set);
 *   lse    : fp32 [num_q, 128], the natural-log log-sum-exp that the attention
 *           over the same set returned (the probabilities are recomputed from
 *           q, kv and lse; a head whose lse is not finite contributes 0);
 *   scores : fp32 [num_q, ld_scores], the indexer's I by position; it must hold
 *           every position of the set (the short-history bypass of dsa_forward
 *           does not score, so training calls dsa_indexer_scores for all).  A
 *           score may be -inf (softmax weight 0: its gradient is -p, and its KL
 *           term is +inf where p > 0) but not NaN or +inf, and a non-empty set
 *           needs at least one finite score;
 *   grad   : fp32 [num_q, k] dL/dI in set order (entry j belongs to idx[i, j];
 *           0 past count and for entries not in the set);
 *   target : fp32 [num_q, k] p in the same order, or NULL;
 *   kl     : fp32 [num_q] the per-query terms; loss : fp32 [1] their sum, or NULL.
 * An empty set gives kl = 0.  No workspace; deterministic. */
int dsa_indexer_kl_sparse(const dsa_queries *queries, const dsa_kv_layout *layout,
                          const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                          const int32_t *count, int32_t k, const float *lse,
                          float softmax_scale, const float *scores, int64_t ld_scores,
                          float *grad, float *target, float *kl, float *loss,
                          hipStream_t stream);
/* Dense warm-up stage (page "arXiv'25 | DSA ...", section 5.1, L_I over every
 * visible position; the mlpod.com page, part 2.1.1): the same loss with the set
 * = [0, q_nvis[i]) and lse from dsa_dense_mla.  grad and target (or NULL) are
 * fp32 [num_q, ld_grad] by position, written for s < q_nvis[i]. */
int dsa_indexer_kl_dense(const dsa_queries *queries, const dsa_kv_layout *layout,
                         const uint16_t *q, const uint16_t *kv, const float *lse,
                         float softmax_scale, const float *scores, int64_t ld_scores,
                         float *grad, float *target, int64_t ld_grad, float *kl,
                         float *loss, hipStream_t stream);

/* Backward of the indexer score into its inputs (page "arXiv'25 | DSA ...",
 * section 3, first equation I = sum_j w_j ReLU(q_j . k); section 5: only the
 * indexer learns from its alignment loss, with its inputs detached from the
 * main model).  Given grad = dL/dI over each query's set, the gradients with
 * respect to the head weights and the dequantised FP8 query and key
 * (q_scale * q8 and k_scale * k8: the quantiser passes gradients unchanged;
 * the derivative of ReLU at exactly 0 is taken as 0):
 *   dw[i,j]     = sum_s grad[i,s] ReLU(q_j . k_s)
 *   dq[i,j,:]   = w[i,j] sum_s grad[i,s] [q_j . k_s > 0] k_s
 *   dk[r(s),:] += grad[i,s] sum_j w[i,j] [q_j . k_s > 0] q_j
 * (the sign of q_j . k_s is taken from the FP8 products summed in fp32).
 *   q_fp8, q_scale, w, k_fp8, k_scale : as for dsa_indexer_scores;
 *   idx, count, k : the set, as for dsa_indexer_kl_sparse; idx = NULL means
 *            every visible position (dense warm-up; k and count unused);
 *   grad   : fp32 dL/dI: [num_q, k] in set order when idx is given (as
 *            dsa_indexer_kl_sparse writes it), else [num_q, ld_grad] by position;
 *   dq     : fp32 [num_q, 64, 128], overwritten;
 *   dw     : fp32 [num_q, 64], overwritten;
 *   dk     : fp32 [R, 128], ADDED to (zero it first): a key row collects the
 *            terms of every query whose set holds it.
 * dk is summed with fp32 atomics, and so are dq and dw when a query's set is
 * split over workgroups (sets of more than 2048 members, or small batches):
 * there the rounding order, and so the last bits, can differ between runs.
 * With one query per key row and one workgroup per query the result is
 * deterministic.  No workspace. */
int dsa_indexer_backward(const dsa_queries *queries, const dsa_kv_layout *layout,
                         const uint8_t *q_fp8, const float *q_scale, const float *w,
                         const uint8_t *k_fp8, const float *k_scale, const int32_t *idx,
                         const int32_t *count, int32_t k, const float *grad, int64_t ld_grad,
                         float *dq, float *dw, float *dk, hipStream_t stream);

/* The whole layer hot path: indexer -> top-k -> sparse attention (page
 * "DeepSeekV3.2之DSA", part 5.1 decode data flow), with the short-history
 * bypass of part 4.5 (a query with q_nvis <= k is not scored and attends to
 * every visible position).  Arguments as in the stage calls above;
 * idx_out (int32 [num_q, k]) and lse may be NULL.
 * ws : dsa_workspace_bytes(DSA_OP_FORWARD, queries, k) bytes.  A call leaves
 * the workspace's top-k histograms zero, and a call whose workspace starts
 * zero (a zero-filled buffer, or the one the previous call used) skips their
 * clearing; any other content is detected (a histogram that does not sum to
 * its row's length) and repaired from the scores, at some cost in time, so
 * results never depend on it.  Calls that share a workspace must not overlap. */
int dsa_forward(const dsa_queries *queries, const dsa_kv_layout *layout,
                const uint8_t *q_fp8, const float *q_scale, const float *w,
                const uint8_t *k_fp8, const float *k_scale, const uint16_t *q,
                const uint16_t *kv, int32_t k, float softmax_scale, float *out,
                float *lse, int32_t *idx_out, void *ws, size_t ws_bytes,
                hipStream_t stream);

/* dsa_forward, plus stage timing: when events is non-NULL, events[0..4]
 * (created by the caller, NULL entries skipped) are recorded on `stream`
 * before the first kernel, before the indexer, after the indexer, after the
 * top-k and after the attention, so that hipEventElapsedTime gives each
 * stage's device time (the top-k's is [0, 1] + [2, 3]; [0, 1] holds no
 * kernel at present).  Same results as dsa_forward. */
int dsa_forward_profiled(const dsa_queries *queries, const dsa_kv_layout *layout,
                         const uint8_t *q_fp8, const float *q_scale, const float *w,
                         const uint8_t *k_fp8, const float *k_scale, const uint16_t *q,
                         const uint16_t *kv, int32_t k, float softmax_scale, float *out,
                         float *lse, int32_t *idx_out, void *ws, size_t ws_bytes,
                         hipStream_t stream, hipEvent_t *events);

/* Workspace size in bytes for `op` with these queries and k (0 if none is
 * needed; SIZE_MAX for invalid arguments).  Host-only, launches nothing. */
size_t dsa_workspace_bytes(int op, const dsa_queries *queries, int32_t k);

/* Static description of a status code. */
const char *dsa_status_string(int status);

/* Detail of the calling thread's last failing call ("" if none). */
const char *dsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBDSA_DSA_H_ */
