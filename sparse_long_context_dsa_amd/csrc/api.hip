// C ABI of libdsa.so: argument checks on the host, workspace carving, and the
// stream-ordered launches of the kernels in indexer.hip, indexer_bwd.hip,
// topk.hip, mla.hip, kl.hip and quant.hip.  Nothing here allocates device memory or synchronises.
#include <cstdarg>
#include <climits>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "dsa.h"
#include "dsa_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return DSA_OK;
}

int hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return ok();
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int check_queries(const dsa_queries *qr) {
  if (!qr) return fail(DSA_ERR_INVALID_ARG, "queries is NULL");
  if (qr->num_q < 0) return fail(DSA_ERR_INVALID_ARG, "num_q = %d < 0", qr->num_q);
  if (qr->max_nvis < 0) return fail(DSA_ERR_INVALID_ARG, "max_nvis = %d < 0", qr->max_nvis);
  if (qr->max_nvis > dsa::MAX_NVIS)
    return fail(DSA_ERR_UNSUPPORTED, "max_nvis = %d: histories up to %d positions", qr->max_nvis, dsa::MAX_NVIS);
  if (qr->num_q > 0 && (!qr->q_seq || !qr->q_nvis))
    return fail(DSA_ERR_INVALID_ARG, "q_seq / q_nvis must be device arrays");
  return DSA_OK;
}

int check_layout(const dsa_kv_layout *ly, dsa::KvMap &m) {
  if (!ly) return fail(DSA_ERR_INVALID_ARG, "layout is NULL");
  if (ly->num_seqs < 0 || ly->num_rows < 0) return fail(DSA_ERR_INVALID_ARG, "negative layout size");
  if (ly->num_rows > INT32_MAX) return fail(DSA_ERR_UNSUPPORTED, "more than 2^31-1 cache rows");
  if (ly->block_size == 0) {
    if (ly->num_seqs > 0 && !ly->seq_row0) return fail(DSA_ERR_INVALID_ARG, "contiguous layout needs seq_row0");
    m.block_shift = -1;
    m.max_blocks = 0;
  } else {
    const int bs = ly->block_size;
    if (bs < 64 || (bs & (bs - 1)) != 0)
      return fail(DSA_ERR_UNSUPPORTED, "block_size %d: must be a power of two >= 64", bs);
    if (ly->num_seqs > 0 && !ly->block_table) return fail(DSA_ERR_INVALID_ARG, "paged layout needs block_table");
    if (ly->max_blocks <= 0) return fail(DSA_ERR_INVALID_ARG, "paged layout needs max_blocks > 0");
    int sh = 0;
    while ((1 << sh) < bs) ++sh;
    m.block_shift = sh;
    m.max_blocks = ly->max_blocks;
  }
  m.block_table = ly->block_table;
  m.seq_row0 = ly->seq_row0;
  return DSA_OK;
}

int check_k(int32_t k) {
  if (k < 1 || k > DSA_KMAX) return fail(DSA_ERR_INVALID_ARG, "k = %d outside [1, %d]", k, (int)DSA_KMAX);
  return DSA_OK;
}

// Workspace pieces of dsa_forward.
struct FwdWs {
  float *scores;
  int64_t ld;
  int32_t *idx;
  int32_t *count;
  void *topk;
  void *mla;
};

int64_t fwd_ld(const dsa_queries *qr) { return ((int64_t)qr->max_nvis + 63) / 64 * 64; }

// The indexer selects the rows itself (scores never leave the chip) when one
// of its blocks covers each query's whole history.
bool fwd_selects_in_indexer(const dsa_queries *qr, int32_t k) {
  return qr->max_nvis > k && dsa::indexer_selects(qr->num_q, qr->max_nvis);
}

size_t fwd_bytes(const dsa_queries *qr, int32_t k, FwdWs *out, void *base) {
  const size_t nq = (size_t)qr->num_q;
  const int64_t ld = fwd_ld(qr);
  const bool sel = fwd_selects_in_indexer(qr, k);
  size_t off = 0;
  const size_t s_scores = sel ? 0 : align256(nq * (size_t)ld * 4);
  const size_t s_idx = align256(nq * (size_t)k * 4);
  const size_t s_cnt = align256(nq * 4);
  const size_t s_topk = sel ? 0 : align256(dsa::topk_ws_bytes(qr->num_q, qr->max_nvis));
  const bool decode = true;
  const size_t s_mla = align256(dsa::mla_ws_bytes(qr->num_q, k, decode));
  if (out) {
    uint8_t *p = static_cast<uint8_t *>(base);
    out->scores = reinterpret_cast<float *>(p + off);
    off += s_scores;
    out->ld = ld;
    out->idx = reinterpret_cast<int32_t *>(p + off);
    off += s_idx;
    out->count = reinterpret_cast<int32_t *>(p + off);
    off += s_cnt;
    out->topk = p + off;
    off += s_topk;
    out->mla = p + off;
    off += s_mla;
    return off;
  }
  return s_scores + s_idx + s_cnt + s_topk + s_mla;
}

int mla_common(bool decode, const dsa_queries *qr, const dsa_kv_layout *ly, const uint16_t *q, const uint16_t *kv,
               const int32_t *idx, const int32_t *count, int32_t k, float softmax_scale, float *out, float *lse,
               void *ws, size_t ws_bytes, hipStream_t stream) {
  int st;
  if ((st = check_queries(qr)) || (st = check_k(k))) return st;
  dsa::KvMap m;
  if ((st = check_layout(ly, m))) return st;
  if (qr->num_q == 0) return ok();
  if (!q || !kv || !idx || !out) return fail(DSA_ERR_INVALID_ARG, "q, kv, idx and out must be non-NULL");
  if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(out, 16))
    return fail(DSA_ERR_INVALID_ARG, "q, kv and out must be 16-byte aligned");
  const size_t need = dsa::mla_ws_bytes(qr->num_q, k, decode);
  if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, 256)))
    return fail(DSA_ERR_WORKSPACE, "workspace: need %zu bytes (256-byte aligned), got %zu", need, ws_bytes);
  dsa::MlaLaunch a{q, kv, idx, count, qr->q_seq, qr->q_nvis, m, k, qr->num_q, softmax_scale, out, lse,
                   ly->num_rows};
  return hip_status(dsa::launch_mla(a, decode, ws, stream), "sparse MLA launch");
}

// Scratch of dsa_sparse_mla_decode_noalloc: the split partials live in this
// file-scope device array instead of a caller workspace.  Each GPU holds its
// own copy (at its own address) from module load until the process ends.  In
// host code `scratch` only names the symbol: its device address comes from
// hipGetSymbolAddress, once per device with that device current, and only
// that address is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[DSA_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES];

// Device address of the current device's scratch (nullptr and a status on failure).
int scratch_of_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= MAX_DEVICES) return fail(DSA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(DSA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

}  // namespace

extern "C" {

int dsa_quantize_fp8(const float *x, int64_t rows, int32_t cols, uint8_t *codes, float *scales,
                     hipStream_t stream) {
  if (rows < 0) return fail(DSA_ERR_INVALID_ARG, "rows = %lld < 0", (long long)rows);
  if (cols < 64 || cols > 512 || cols % 64 != 0)
    return fail(DSA_ERR_UNSUPPORTED, "cols = %d: must be a multiple of 64 in [64, 512]", cols);
  if (rows == 0) return ok();
  if (!x || !codes || !scales) return fail(DSA_ERR_INVALID_ARG, "x, codes and scales must be non-NULL");
  if (!aligned(x, 16) || !aligned(codes, 16)) return fail(DSA_ERR_INVALID_ARG, "x and codes must be 16-byte aligned");
  return hip_status(dsa::launch_quantize_fp8(x, rows, cols, codes, scales, stream), "quantize launch");
}

int dsa_quantize_fp8_e8m0(const float *x, int64_t rows, int32_t cols, uint8_t *codes, uint8_t *e8m0,
                          float *scales, hipStream_t stream) {
  if (rows < 0) return fail(DSA_ERR_INVALID_ARG, "rows = %lld < 0", (long long)rows);
  if (cols < 64 || cols > 512 || cols % 64 != 0)
    return fail(DSA_ERR_UNSUPPORTED, "cols = %d: must be a multiple of 64 in [64, 512]", cols);
  if (rows == 0) return ok();
  if (!x || !codes || !e8m0) return fail(DSA_ERR_INVALID_ARG, "x, codes and e8m0 must be non-NULL");
  if (!aligned(x, 16) || !aligned(codes, 16)) return fail(DSA_ERR_INVALID_ARG, "x and codes must be 16-byte aligned");
  return hip_status(dsa::launch_quantize_fp8_e8m0(x, rows, cols, codes, e8m0, scales, stream), "quantize launch");
}

static int indexer_impl(const dsa_queries *qr, const dsa_kv_layout *ly, const uint8_t *q_fp8, const float *q_scale,
                        const float *w, const uint8_t *k_fp8, const float *k_scale, const uint8_t *k_e8m0,
                        float *scores, int64_t ld, hipStream_t stream) {
  int st;
  if ((st = check_queries(qr))) return st;
  dsa::KvMap m;
  if ((st = check_layout(ly, m))) return st;
  if (qr->num_q == 0 || qr->max_nvis == 0) return ok();
  if (!q_fp8 || !w || !k_fp8 || !(k_scale || k_e8m0) || !scores)
    return fail(DSA_ERR_INVALID_ARG, "q_fp8, w, k_fp8, the key scales and scores must be non-NULL");
  if (ld < qr->max_nvis || ld % 4 != 0) return fail(DSA_ERR_INVALID_ARG, "ld = %lld: need ld >= max_nvis and ld %% 4 == 0", (long long)ld);
  if (!aligned(q_fp8, 16) || !aligned(k_fp8, 16) || !aligned(scores, 16))
    return fail(DSA_ERR_INVALID_ARG, "q_fp8, k_fp8 and scores must be 16-byte aligned");
  dsa::IndexerLaunch a{q_fp8, q_scale, w, k_fp8, k_scale, qr->q_seq, qr->q_nvis, m, scores, ld, nullptr, -1,
                       qr->num_q, qr->max_nvis, k_e8m0};
  return hip_status(dsa::launch_indexer(a, stream), "indexer launch");
}

int dsa_indexer_scores(const dsa_queries *qr, const dsa_kv_layout *ly, const uint8_t *q_fp8, const float *q_scale,
                       const float *w, const uint8_t *k_fp8, const float *k_scale, float *scores, int64_t ld,
                       hipStream_t stream) {
  return indexer_impl(qr, ly, q_fp8, q_scale, w, k_fp8, k_scale, nullptr, scores, ld, stream);
}

int dsa_indexer_scores_e8m0(const dsa_queries *qr, const dsa_kv_layout *ly, const uint8_t *q_fp8,
                            const float *q_scale, const float *w, const uint8_t *k_fp8, const uint8_t *k_scale_e8m0,
                            float *scores, int64_t ld, hipStream_t stream) {
  return indexer_impl(qr, ly, q_fp8, q_scale, w, k_fp8, nullptr, k_scale_e8m0, scores, ld, stream);
}

int dsa_topk(const dsa_queries *qr, const float *scores, int64_t ld, int32_t k, int32_t *idx, int32_t *count,
             void *ws, size_t ws_bytes, hipStream_t stream) {
  int st;
  if ((st = check_queries(qr)) || (st = check_k(k))) return st;
  if (qr->num_q == 0) return ok();
  if (!idx) return fail(DSA_ERR_INVALID_ARG, "idx must be non-NULL");
  if (qr->max_nvis > k) {
    if (!scores) return fail(DSA_ERR_INVALID_ARG, "scores must be non-NULL");
    if (ld < qr->max_nvis || ld % 4 != 0)
      return fail(DSA_ERR_INVALID_ARG, "ld = %lld: need ld >= max_nvis and ld %% 4 == 0", (long long)ld);
    if (!aligned(scores, 16)) return fail(DSA_ERR_INVALID_ARG, "scores must be 16-byte aligned");
  }
  const size_t need = dsa::topk_ws_bytes(qr->num_q, qr->max_nvis);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(DSA_ERR_WORKSPACE, "workspace: need %zu bytes (256-byte aligned), got %zu", need, ws_bytes);
  dsa::TopkWs tw = dsa::topk_ws_carve(ws, qr->num_q, qr->max_nvis);
  hipError_t e = dsa::launch_topk_init(tw, qr->num_q, stream);
  if (e == hipSuccess) e = dsa::launch_topk_hist(scores, ld, qr->q_nvis, tw, qr->num_q, qr->max_nvis, stream);
  if (e == hipSuccess)
    e = dsa::launch_topk_select(scores, ld, qr->q_nvis, k, idx, count, tw, qr->num_q, qr->max_nvis, false, stream);
  return hip_status(e, "top-k launch");
}

int dsa_sparse_mla_decode(const dsa_queries *qr, const dsa_kv_layout *ly, const uint16_t *q, const uint16_t *kv,
                          const int32_t *idx, const int32_t *count, int32_t k, float softmax_scale, float *out,
                          float *lse, void *ws, size_t ws_bytes, hipStream_t stream) {
  return mla_common(true, qr, ly, q, kv, idx, count, k, softmax_scale, out, lse, ws, ws_bytes, stream);
}

int dsa_sparse_mla_decode_noalloc(const dsa_queries *qr, const dsa_kv_layout *ly, const uint16_t *q,
                                  const uint16_t *kv, const int32_t *idx, const int32_t *count, int32_t k,
                                  float softmax_scale, float *out, float *lse, hipStream_t stream) {
  int st;
  if ((st = check_queries(qr)) || (st = check_k(k))) return st;
  const size_t need = dsa::mla_ws_bytes(qr->num_q, k, true);
  if (need > DSA_NOALLOC_SCRATCH_BYTES)
    return fail(DSA_ERR_UNSUPPORTED,
                "dsa_sparse_mla_decode_noalloc: %d queries at k = %d need %zu bytes of split partials; the "
                "library's scratch holds %zu (use dsa_sparse_mla_decode with a workspace)",
                qr->num_q, k, need, (size_t)DSA_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  if (need > 0 && (st = scratch_of_current_device(&ws))) return st;
  return mla_common(true, qr, ly, q, kv, idx, count, k, softmax_scale, out, lse, ws,
                    need > 0 ? (size_t)DSA_NOALLOC_SCRATCH_BYTES : 0, stream);
}

int dsa_sparse_mla_prefill(const dsa_queries *qr, const dsa_kv_layout *ly, const uint16_t *q, const uint16_t *kv,
                           const int32_t *idx, const int32_t *count, int32_t k, float softmax_scale, float *out,
                           float *lse, void *ws, size_t ws_bytes, hipStream_t stream) {
  return mla_common(false, qr, ly, q, kv, idx, count, k, softmax_scale, out, lse, ws, ws_bytes, stream);
}

int dsa_dense_mla(const dsa_queries *qr, const dsa_kv_layout *ly, const uint16_t *q, const uint16_t *kv,
                  float softmax_scale, float *out, float *lse, void *ws, size_t ws_bytes, hipStream_t stream) {
  int st;
  if ((st = check_queries(qr))) return st;
  dsa::KvMap m;
  if ((st = check_layout(ly, m))) return st;
  if (qr->num_q == 0) return ok();
  if (!q || !kv || !out) return fail(DSA_ERR_INVALID_ARG, "q, kv and out must be non-NULL");
  if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(out, 16))
    return fail(DSA_ERR_INVALID_ARG, "q, kv and out must be 16-byte aligned");
  const int longest = qr->max_nvis > 0 ? qr->max_nvis : 1;
  const size_t need = dsa::mla_ws_bytes(qr->num_q, longest, true, true);
  if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, 256)))
    return fail(DSA_ERR_WORKSPACE, "workspace: need %zu bytes (256-byte aligned), got %zu", need, ws_bytes);
  dsa::MlaLaunch a{q, kv, nullptr, nullptr, qr->q_seq, qr->q_nvis, m, longest, qr->num_q, softmax_scale, out, lse,
                   ly->num_rows, true};
  return hip_status(dsa::launch_mla(a, true, ws, stream), "dense MLA launch");
}

static int kl_impl(const dsa_queries *qr, const dsa_kv_layout *ly, const uint16_t *q, const uint16_t *kv,
                   const int32_t *idx, const int32_t *count, int32_t k, const float *lse, float softmax_scale,
                   const float *scores, int64_t ld_scores, float *grad, float *target, int64_t ld_grad, float *kl,
                   float *loss, hipStream_t stream) {
  int st;
  if ((st = check_queries(qr))) return st;
  const bool sparse = idx != nullptr;
  if (sparse && (st = check_k(k))) return st;
  dsa::KvMap m;
  if ((st = check_layout(ly, m))) return st;
  if (qr->num_q > 0) {
    if (!q || !kv || !lse || !scores || !grad || !kl)
      return fail(DSA_ERR_INVALID_ARG, "q, kv, lse, scores, grad and kl must be non-NULL");
    if (!aligned(q, 16) || !aligned(kv, 16)) return fail(DSA_ERR_INVALID_ARG, "q and kv must be 16-byte aligned");
    if (ld_scores < qr->max_nvis)
      return fail(DSA_ERR_INVALID_ARG, "ld_scores = %lld < max_nvis = %d", (long long)ld_scores, qr->max_nvis);
    if (!sparse && ld_grad < qr->max_nvis)
      return fail(DSA_ERR_INVALID_ARG, "ld_grad = %lld < max_nvis = %d", (long long)ld_grad, qr->max_nvis);
  }
  if (qr->num_q == 0 && !loss) return ok();
  const int max_set = sparse ? (qr->max_nvis < k ? qr->max_nvis : k) : qr->max_nvis;
  dsa::KlLaunch a{q, kv, idx, count, qr->q_seq, qr->q_nvis, m, lse, scores, ld_scores, sparse ? k : 0, qr->num_q,
                  softmax_scale, ly->num_rows, grad, sparse ? (int64_t)k : ld_grad, target, kl, loss};
  return hip_status(dsa::launch_indexer_kl(a, max_set, stream), "indexer KL launch");
}

int dsa_indexer_kl_sparse(const dsa_queries *qr, const dsa_kv_layout *ly, const uint16_t *q, const uint16_t *kv,
                          const int32_t *idx, const int32_t *count, int32_t k, const float *lse,
                          float softmax_scale, const float *scores, int64_t ld_scores, float *grad, float *target,
                          float *kl, float *loss, hipStream_t stream) {
  if (qr && qr->num_q > 0 && !idx) return fail(DSA_ERR_INVALID_ARG, "idx must be non-NULL");
  return kl_impl(qr, ly, q, kv, idx, count, k, lse, softmax_scale, scores, ld_scores, grad, target, k, kl, loss,
                 stream);
}

int dsa_indexer_kl_dense(const dsa_queries *qr, const dsa_kv_layout *ly, const uint16_t *q, const uint16_t *kv,
                         const float *lse, float softmax_scale, const float *scores, int64_t ld_scores, float *grad,
                         float *target, int64_t ld_grad, float *kl, float *loss, hipStream_t stream) {
  return kl_impl(qr, ly, q, kv, nullptr, nullptr, 0, lse, softmax_scale, scores, ld_scores, grad, target, ld_grad,
                 kl, loss, stream);
}

int dsa_indexer_backward(const dsa_queries *qr, const dsa_kv_layout *ly, const uint8_t *q_fp8, const float *q_scale,
                         const float *w, const uint8_t *k_fp8, const float *k_scale, const int32_t *idx,
                         const int32_t *count, int32_t k, const float *grad, int64_t ld_grad, float *dq, float *dw,
                         float *dk, hipStream_t stream) {
  int st;
  if ((st = check_queries(qr))) return st;
  const bool sparse = idx != nullptr;
  if (sparse && (st = check_k(k))) return st;
  dsa::KvMap m;
  if ((st = check_layout(ly, m))) return st;
  if (qr->num_q == 0) return ok();
  if (!q_fp8 || !w || !k_fp8 || !k_scale || !grad || !dq || !dw || !dk)
    return fail(DSA_ERR_INVALID_ARG, "q_fp8, w, k_fp8, k_scale, grad, dq, dw and dk must be non-NULL");
  if (!aligned(q_fp8, 16) || !aligned(k_fp8, 16))
    return fail(DSA_ERR_INVALID_ARG, "q_fp8 and k_fp8 must be 16-byte aligned");
  if (sparse) {
    ld_grad = k;
  } else if (ld_grad < qr->max_nvis) {
    return fail(DSA_ERR_INVALID_ARG, "ld_grad = %lld < max_nvis = %d", (long long)ld_grad, qr->max_nvis);
  }
  const int max_set = sparse ? (qr->max_nvis < k ? qr->max_nvis : k) : qr->max_nvis;
  dsa::IndexerBwdLaunch a{q_fp8, q_scale, w, k_fp8, k_scale, idx, count, qr->q_seq, qr->q_nvis, m,
                          sparse ? k : 0, qr->num_q, grad, ld_grad, dq, dw, dk, ly->num_seqs};
  return hip_status(dsa::launch_indexer_bwd(a, max_set, stream), "indexer backward launch");
}

static int forward_impl(const dsa_queries *qr, const dsa_kv_layout *ly, const uint8_t *q_fp8, const float *q_scale,
                        const float *w, const uint8_t *k_fp8, const float *k_scale, const uint16_t *q,
                        const uint16_t *kv, int32_t k, float softmax_scale, float *out, float *lse, int32_t *idx_out,
                        void *ws, size_t ws_bytes, hipStream_t stream, hipEvent_t *events) {
  int st;
  if ((st = check_queries(qr)) || (st = check_k(k))) return st;
  dsa::KvMap m;
  if ((st = check_layout(ly, m))) return st;
  if (qr->num_q == 0) return ok();
  if (!q_fp8 || !w || !k_fp8 || !k_scale || !q || !kv || !out)
    return fail(DSA_ERR_INVALID_ARG, "q_fp8, w, k_fp8, k_scale, q, kv and out must be non-NULL");
  if (!aligned(q_fp8, 16) || !aligned(k_fp8, 16) || !aligned(q, 16) || !aligned(kv, 16) || !aligned(out, 16))
    return fail(DSA_ERR_INVALID_ARG, "q_fp8, k_fp8, q, kv and out must be 16-byte aligned");
  const size_t need = fwd_bytes(qr, k, nullptr, nullptr);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(DSA_ERR_WORKSPACE, "workspace: need %zu bytes (256-byte aligned), got %zu", need, ws_bytes);
  FwdWs fw;
  fwd_bytes(qr, k, &fw, ws);
  int32_t *idx = idx_out ? idx_out : fw.idx;
  dsa::TopkWs tw = dsa::topk_ws_carve(fw.topk, qr->num_q, qr->max_nvis);
  hipError_t e = hipSuccess;
  auto mark = [&](int i) {
    if (events && events[i] && e == hipSuccess) e = hipEventRecord(events[i], stream);
  };
  const bool sel = fwd_selects_in_indexer(qr, k);
  // No clear of the first-digit histograms: the top-k kernels leave them zero
  // for the next call, and a histogram that does not sum to its row's length
  // (a workspace that held other data) is rebuilt from the scores.
  mark(0);
  mark(1);
  if (sel) {
    // Every query's history fits one indexer block: the indexer writes the
    // positions (and the short histories' full lists); no scores, no top-k launch.
    dsa::IndexerLaunch ia{q_fp8, q_scale, w, k_fp8, k_scale, qr->q_seq, qr->q_nvis, m, nullptr, 0,
                          nullptr, k, qr->num_q, qr->max_nvis, nullptr, idx, fw.count, k};
    if (e == hipSuccess) e = dsa::launch_indexer(ia, stream);
    mark(2);
  } else {
    if (qr->max_nvis > k && e == hipSuccess) {
      dsa::IndexerLaunch ia{q_fp8, q_scale, w, k_fp8, k_scale, qr->q_seq, qr->q_nvis, m, fw.scores, fw.ld,
                            tw.hist, k, qr->num_q, qr->max_nvis};
      e = dsa::launch_indexer(ia, stream);
    }
    mark(2);
    if (e == hipSuccess)
      e = dsa::launch_topk_select(fw.scores, fw.ld, qr->q_nvis, k, idx, fw.count, tw, qr->num_q, qr->max_nvis,
                                  true, stream);
  }
  mark(3);
  if (e == hipSuccess) {
    dsa::MlaLaunch ma{q, kv, idx, fw.count, qr->q_seq, qr->q_nvis, m, k, qr->num_q, softmax_scale, out, lse,
                    ly->num_rows};
    const bool decode = dsa::mla_num_splits(qr->num_q, k, true) > 1;
    e = dsa::launch_mla(ma, decode, fw.mla, stream);
  }
  mark(4);
  return hip_status(e, "forward launch");
}

int dsa_forward(const dsa_queries *qr, const dsa_kv_layout *ly, const uint8_t *q_fp8, const float *q_scale,
                const float *w, const uint8_t *k_fp8, const float *k_scale, const uint16_t *q, const uint16_t *kv,
                int32_t k, float softmax_scale, float *out, float *lse, int32_t *idx_out, void *ws, size_t ws_bytes,
                hipStream_t stream) {
  return forward_impl(qr, ly, q_fp8, q_scale, w, k_fp8, k_scale, q, kv, k, softmax_scale, out, lse, idx_out, ws,
                      ws_bytes, stream, nullptr);
}

int dsa_forward_profiled(const dsa_queries *qr, const dsa_kv_layout *ly, const uint8_t *q_fp8,
                         const float *q_scale, const float *w, const uint8_t *k_fp8, const float *k_scale,
                         const uint16_t *q, const uint16_t *kv, int32_t k, float softmax_scale, float *out,
                         float *lse, int32_t *idx_out, void *ws, size_t ws_bytes, hipStream_t stream,
                         hipEvent_t *events) {
  return forward_impl(qr, ly, q_fp8, q_scale, w, k_fp8, k_scale, q, kv, k, softmax_scale, out, lse, idx_out, ws,
                      ws_bytes, stream, events);
}

size_t dsa_workspace_bytes(int op, const dsa_queries *qr, int32_t k) {
  if (!qr || qr->num_q < 0 || qr->max_nvis < 0) return SIZE_MAX;
  if (op == DSA_OP_MLA_DENSE) return dsa::mla_ws_bytes(qr->num_q, qr->max_nvis > 0 ? qr->max_nvis : 1, true, true);
  if (k < 1 || k > DSA_KMAX) return SIZE_MAX;
  switch (op) {
    case DSA_OP_TOPK:
      return dsa::topk_ws_bytes(qr->num_q, qr->max_nvis);
    case DSA_OP_MLA_DECODE:
      return dsa::mla_ws_bytes(qr->num_q, k, true);
    case DSA_OP_MLA_PREFILL:
      return dsa::mla_ws_bytes(qr->num_q, k, false);
    case DSA_OP_FORWARD:
      return fwd_bytes(qr, k, nullptr, nullptr);
    default:
      return SIZE_MAX;
  }
}

const char *dsa_status_string(int status) {
  switch (status) {
    case DSA_OK: return "ok";
    case DSA_ERR_INVALID_ARG: return "invalid argument";
    case DSA_ERR_UNSUPPORTED: return "unsupported shape or layout";
    case DSA_ERR_WORKSPACE: return "workspace missing or too small";
    case DSA_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

const char *dsa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
