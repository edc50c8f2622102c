// Per-query top-k selection over fp32 scores (gfx950).
//
// Page "arXiv'25 | DSA ... DeepSeek-V3.2", section 3 (second equation: the
// top-k of the scores over the earlier positions); page "DeepSeekV3.2之DSA",
// part 4.4 (the indices of the min(topk, end_pos) largest) and part 4.5 (a
// history no longer than k keeps everything).  Ties go to the lower position
// and -0 equals +0 (readings, the pages are silent); the output is in
// ascending position order, padded with -1.
//
// Radix select on order-preserving 32-bit keys with digits of 11 / 11 / 10
// bits.  Each digit step is a histogram and a search for the bin that holds
// the r-th largest key; three steps give the exact k-th key T and the number
// of keys equal to T to keep (the lowest positions among them).  The output
// is then one position-ordered compaction (two block scans over contiguous
// per-thread runs, so it is deterministic).
//
// Two kernels, chosen per query by its history length n:
//  * topk_row_kernel (n <= 16384, e.g. every causal-prefill row): one block
//    per query holds the whole row as keys in LDS; all passes run from LDS.
//    The first-digit histogram comes from the indexer's fused epilogue when
//    available, else from LDS atomics.
//  * topk_chunk_kernel (longer rows, e.g. 128K decode): one block per 16384
//    scores.  The scores are streamed from HBM once: each block finds the
//    threshold bin B1 from the first-digit histogram, compacts the keys with
//    digit >= B1 (the candidates, about k + |B1|) into its list in position
//    order and adds the second-digit histogram of the B1 keys into a global
//    one.  The last block of a query (atomic counter with device-scope
//    fences) gathers all lists into LDS with independent loads and finishes
//    the selection there (or from global memory if they do not fit).
#include "device_util.h"
#include "dsa_internal.h"

namespace dsa {

constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / WAVE;
constexpr int TK_PER = TOPK_ROW_MAX / TK_THREADS;  // 16 keys per thread
constexpr int LIST_CAP = 8192;                     // candidates the finalize keeps in LDS
static_assert(TOPK_CHUNK == TOPK_ROW_MAX, "one element count per thread for both kernels");

static inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

static inline int topk_nchunks(int max_nvis) {
  return max_nvis <= TOPK_ROW_MAX ? 0 : (max_nvis + TOPK_CHUNK - 1) / TOPK_CHUNK;
}

size_t topk_ws_bytes(int num_q, int max_nvis) {
  const size_t nq = (size_t)num_q;
  const size_t nc = (size_t)topk_nchunks(max_nvis);
  return align256(nq * (2 * TOPK_BINS + 1) * 4) + align256(nq * nc * 4) + nq * nc * TOPK_CHUNK * sizeof(uint2);
}

TopkWs topk_ws_carve(void *ws, int num_q, int max_nvis) {
  TopkWs w;
  const size_t nq = (size_t)num_q;
  w.nchunks = topk_nchunks(max_nvis);
  uint8_t *p = static_cast<uint8_t *>(ws);
  w.hist = reinterpret_cast<uint32_t *>(p);  // [nq, 2048] first digit
  w.hist2 = w.hist + nq * TOPK_BINS;         // [nq, 2048] second digit
  w.done = w.hist2 + nq * TOPK_BINS;         // [nq]; the three are cleared by one fill
  p += align256(nq * (2 * TOPK_BINS + 1) * 4);
  w.ccount = reinterpret_cast<uint32_t *>(p);
  p += align256(nq * w.nchunks * 4);
  w.cand = reinterpret_cast<uint2 *>(p);
  return w;
}

// ------------------------------------------------------------------ helpers
// Exclusive scan of one int per thread over the block; `total` gets the sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int *sm, int &total) {
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int inc = wave_inclusive_scan(v);
  if (lane == WAVE - 1) sm[wave] = inc;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < TK_WAVES; ++w) {
    const int s = sm[w];
    before += (w < wave) ? s : 0;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return before + inc - v;
}

// Given an LDS histogram h[NB] and a rank r >= 1 counted from the top, finds
// the bin B with above(B) < r <= above(B) + h[B] (above(B) = sum of h[b > B]).
// res[0] = B, res[1] = above(B), visible to all threads on return.
template <int NB>
__device__ void find_rank_bin(const uint32_t *h, int r, int *sm, int *res) {
  constexpr int PER = NB / TK_THREADS;
  const int hi = NB - PER * (int)threadIdx.x;  // bins [hi - PER, hi), scanned top-down
  int local = 0;
#pragma unroll
  for (int i = 1; i <= PER; ++i) local += (int)h[hi - i];
  int total;
  int acc = block_exclusive_scan(local, sm, total);
#pragma unroll
  for (int i = 1; i <= PER; ++i) {
    const int c = (int)h[hi - i];
    if (acc < r && acc + c >= r) {
      res[0] = hi - i;
      res[1] = acc;
    }
    acc += c;
  }
  __syncthreads();
}

__device__ __forceinline__ void zero_lds(uint32_t *h, int n) {
  for (int b = threadIdx.x; b < n; b += TK_THREADS) h[b] = 0u;
}

__device__ __forceinline__ void flush_hist(const uint32_t *h, uint32_t *g) {
  for (int b = threadIdx.x; b < TOPK_BINS; b += TK_THREADS) {
    const uint32_t c = h[b];
    if (c) atomicAdd(&g[b], c);
  }
}

// Loads 16 scores starting at row[i0] (i0 % 4 == 0); keys of positions >= n are 0.
__device__ __forceinline__ void load16(const float *row, int i0, int n, uint32_t *key) {
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int i = i0 + 4 * v;
    if (i + 3 < n) {
      const float4 f = *reinterpret_cast<const float4 *>(row + i);
      key[4 * v + 0] = order_key(f.x);
      key[4 * v + 1] = order_key(f.y);
      key[4 * v + 2] = order_key(f.z);
      key[4 * v + 3] = order_key(f.w);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) key[4 * v + j] = (i + j < n) ? order_key(row[i + j]) : 0u;
    }
  }
}

__device__ __forceinline__ void write_short(int32_t *out, int32_t *count, int q, int n, int k) {
  for (int i = threadIdx.x; i < k; i += TK_THREADS) out[i] = (i < n) ? i : -1;
  if (threadIdx.x == 0 && count) count[q] = n;
}

// Position-ordered emission.  The candidates are visited as contiguous runs,
// run t = [t*per, min(total, (t+1)*per)); get(i) returns (key, position).
// Keeps keys > kth and the first `ties` keys == kth.
template <typename Get>
__device__ void emit_selected(Get get, int total, uint32_t kth, int ties, int32_t *out, int k, int *sm) {
  const int per = (total + TK_THREADS - 1) / TK_THREADS;
  const int lo = min(total, per * (int)threadIdx.x), hi = min(total, lo + per);
  int my_ties = 0;
  for (int i = lo; i < hi; ++i) my_ties += (get(i).x == kth) ? 1 : 0;
  int tot;
  const int tie_rank = block_exclusive_scan(my_ties, sm, tot);
  int my_sel = 0;
  for (int i = lo, tr = tie_rank; i < hi; ++i) {
    const uint32_t key = get(i).x;
    if (key > kth || (key == kth && tr < ties)) ++my_sel;
    tr += (key == kth) ? 1 : 0;
  }
  int pos = block_exclusive_scan(my_sel, sm, tot);
  for (int i = lo, tr = tie_rank; i < hi; ++i) {
    const uint2 e = get(i);
    if (e.x > kth || (e.x == kth && tr < ties)) {
      if (pos < k) out[pos] = (int32_t)e.y;
      ++pos;
    }
    tr += (e.x == kth) ? 1 : 0;
  }
  // Exactly k are selected when the histograms and candidates agree; pad
  // defensively so a reader never sees stale entries.
  for (int i = tot + threadIdx.x; i < k; i += TK_THREADS) out[i] = -1;
}

// ------------------------------------------------------------------ kernels
__global__ __launch_bounds__(256) void topk_zero_kernel(uint32_t *p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// First-digit histogram of the rows longer than TOPK_ROW_MAX (standalone top-k).
__global__ __launch_bounds__(TK_THREADS) void topk_hist_kernel(const float *__restrict__ scores, int64_t ld,
                                                               const int32_t *__restrict__ q_nvis,
                                                               uint32_t *__restrict__ ghist, int nchunks) {
  const int q = blockIdx.x / nchunks;
  const int c = blockIdx.x - q * nchunks;
  const int n = q_nvis[q];
  const int start = c * TOPK_CHUNK;
  if (n <= TOPK_ROW_MAX || start >= n) return;
  __shared__ uint32_t h[TOPK_BINS];
  zero_lds(h, TOPK_BINS);
  __syncthreads();
  uint32_t key[TK_PER];
  const int i0 = start + TK_PER * threadIdx.x;
  load16(scores + (int64_t)q * ld, i0, n, key);
#pragma unroll
  for (int j = 0; j < TK_PER; ++j)
    if (i0 + j < n) atomicAdd(&h[key[j] >> 21], 1u);
  __syncthreads();
  flush_hist(h, ghist + (int64_t)q * TOPK_BINS);
}

struct SelectArgs {
  const float *scores;
  int64_t ld;
  const int32_t *q_nvis;
  int k;
  int hist1_valid;  // the first-digit histogram of every scored row is in ws.hist
  int32_t *idx;
  int32_t *count;
  TopkWs ws;
};

__global__ __launch_bounds__(TK_THREADS) void topk_row_kernel(SelectArgs a) {
  const int q = blockIdx.x;
  const int n = a.q_nvis[q];
  const int k = a.k;
  if (n > TOPK_ROW_MAX) return;
  int32_t *out = a.idx + (int64_t)q * k;
  if (n <= k) {
    write_short(out, a.count, q, n, k);
    return;
  }
  __shared__ uint32_t keys[TOPK_ROW_MAX];
  __shared__ uint32_t h[TOPK_BINS];
  __shared__ int sm[TK_WAVES];
  __shared__ int res[2];
  const int t = threadIdx.x;
  uint32_t key[TK_PER];
  load16(a.scores + (int64_t)q * a.ld, TK_PER * t, n, key);
#pragma unroll
  for (int j = 0; j < TK_PER; ++j) keys[TK_PER * t + j] = key[j];
  // Digit 1: key[31:21].
  if (a.hist1_valid) {
    const uint32_t *gh = a.ws.hist + (int64_t)q * TOPK_BINS;
    for (int b = t; b < TOPK_BINS; b += TK_THREADS) h[b] = gh[b];
  } else {
    zero_lds(h, TOPK_BINS);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < TK_PER; ++j)
      if (TK_PER * t + j < n) atomicAdd(&h[key[j] >> 21], 1u);
  }
  __syncthreads();
  find_rank_bin<TOPK_BINS>(h, k, sm, res);
  const uint32_t b1 = (uint32_t)res[0];
  const int r = k - res[1];
  __syncthreads();
  // Digit 2: key[20:10] of the keys in bin B1.
  zero_lds(h, TOPK_BINS);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < TK_PER; ++j)
    if (TK_PER * t + j < n && (key[j] >> 21) == b1) atomicAdd(&h[(key[j] >> 10) & 2047u], 1u);
  __syncthreads();
  find_rank_bin<TOPK_BINS>(h, r, sm, res);
  const uint32_t pre = (b1 << 11) | (uint32_t)res[0];
  const int r2 = r - res[1];
  __syncthreads();
  // Digit 3: key[9:0] of the keys with key[31:10] == pre.
  zero_lds(h, 1024);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < TK_PER; ++j)
    if (TK_PER * t + j < n && (key[j] >> 10) == pre) atomicAdd(&h[key[j] & 1023u], 1u);
  __syncthreads();
  find_rank_bin<1024>(h, r2, sm, res);
  const uint32_t kth = (pre << 10) | (uint32_t)res[0];
  const int ties = r2 - res[1];
  __syncthreads();
  emit_selected([&](int i) { return make_uint2(keys[i], (uint32_t)i); }, n, kth, ties, out, k, sm);
  if (t == 0 && a.count) a.count[q] = k;
}

// Finds the chunk holding candidate i, given the exclusive prefix off[0..nc].
__device__ __forceinline__ int locate(const int *off, int nc, int i) {
  int c = 0;
  while (c + 1 < nc && off[c + 1] <= i) ++c;
  return c;
}

__global__ __launch_bounds__(TK_THREADS) void topk_chunk_kernel(SelectArgs a) {
  const int nchunks = a.ws.nchunks;
  const int q = blockIdx.x / nchunks;
  const int c = blockIdx.x - q * nchunks;
  const int n = a.q_nvis[q];
  const int k = a.k;
  if (n <= TOPK_ROW_MAX) return;
  const int nc = (n + TOPK_CHUNK - 1) / TOPK_CHUNK;
  if (c >= nc) return;

  __shared__ uint2 lst[LIST_CAP];
  __shared__ uint32_t h[TOPK_BINS];
  __shared__ int sm[TK_WAVES];
  __shared__ int res[2];
  __shared__ int off[TOPK_MAX_CHUNKS + 1];
  __shared__ int is_last;
  const int t = threadIdx.x;

  // Threshold bin B1 from the first-digit histogram.
  const uint32_t *gh1 = a.ws.hist + (int64_t)q * TOPK_BINS;
  for (int b = t; b < TOPK_BINS; b += TK_THREADS) h[b] = gh1[b];
  __syncthreads();
  find_rank_bin<TOPK_BINS>(h, k, sm, res);
  const uint32_t b1 = (uint32_t)res[0];
  const int above1 = res[1];
  __syncthreads();
  zero_lds(h, TOPK_BINS);
  __syncthreads();

  // Candidates of this chunk (digit >= B1) in position order; second-digit
  // histogram of the keys in B1.
  const int i0 = c * TOPK_CHUNK + TK_PER * t;
  uint32_t key[TK_PER];
  load16(a.scores + (int64_t)q * a.ld, i0, n, key);
  int f = 0;
#pragma unroll
  for (int j = 0; j < TK_PER; ++j) {
    const bool in = (i0 + j < n);
    f += (in && (key[j] >> 21) >= b1) ? 1 : 0;
    if (in && (key[j] >> 21) == b1) atomicAdd(&h[(key[j] >> 10) & 2047u], 1u);
  }
  int total;
  int pos = block_exclusive_scan(f, sm, total);  // also orders the histogram updates before the flush
  uint2 *glst = a.ws.cand + ((int64_t)q * nchunks + c) * TOPK_CHUNK;
#pragma unroll
  for (int j = 0; j < TK_PER; ++j)
    if (i0 + j < n && (key[j] >> 21) >= b1) glst[pos++] = make_uint2(key[j], (uint32_t)(i0 + j));
  if (t == 0) a.ws.ccount[(int64_t)q * nchunks + c] = (uint32_t)total;
  flush_hist(h, a.ws.hist2 + (int64_t)q * TOPK_BINS);

  // The last block of this query to get here finishes the selection.  The
  // barrier orders the block's list, count and histogram writes before thread
  // 0's device-scope release (fences are cumulative), so one fence per block
  // publishes them; the last block's acquire makes the other blocks' data
  // visible to all of its threads after the second barrier.
  __syncthreads();
  if (t == 0) {
    __threadfence();
    const bool last = atomicAdd(&a.ws.done[q], 1u) == (uint32_t)(nc - 1);
    if (last) __threadfence();
    is_last = last ? 1 : 0;
  }
  __syncthreads();
  if (!is_last) return;

  const int r = k - above1;
  const uint32_t *gh2 = a.ws.hist2 + (int64_t)q * TOPK_BINS;
  for (int b = t; b < TOPK_BINS; b += TK_THREADS) h[b] = gh2[b];
  if (t == 0) {
    int s = 0;
    for (int cc = 0; cc < nc; ++cc) {
      off[cc] = s;
      s += (int)a.ws.ccount[(int64_t)q * nchunks + cc];
    }
    off[nc] = s;
  }
  __syncthreads();
  find_rank_bin<TOPK_BINS>(h, r, sm, res);
  const uint32_t pre = (b1 << 11) | (uint32_t)res[0];
  const int r2 = r - res[1];
  const int ntot = off[nc];
  const uint2 *cand_q = a.ws.cand + (int64_t)q * nchunks * TOPK_CHUNK;
  __syncthreads();
  zero_lds(h, 1024);
  const bool in_lds = ntot <= LIST_CAP;
  if (in_lds) {
    // All candidates into LDS: up to 8 independent loads per thread.
#pragma unroll
    for (int j = 0; j < LIST_CAP / TK_THREADS; ++j) {
      const int i = t + j * TK_THREADS;
      if (i < ntot) {
        const int cc = locate(off, nc, i);
        lst[i] = cand_q[(int64_t)cc * TOPK_CHUNK + (i - off[cc])];
      }
    }
  }
  __syncthreads();
  auto get_lds = [&](int i) { return lst[i]; };
  auto get_glb = [&](int i) {
    const int cc = locate(off, nc, i);
    return cand_q[(int64_t)cc * TOPK_CHUNK + (i - off[cc])];
  };
  // Digit 3 over the candidates with key[31:10] == pre.
  {
    const int per = (ntot + TK_THREADS - 1) / TK_THREADS;
    const int lo = min(ntot, per * t), hi = min(ntot, lo + per);
    for (int i = lo; i < hi; ++i) {
      const uint32_t kk = in_lds ? lst[i].x : get_glb(i).x;
      if ((kk >> 10) == pre) atomicAdd(&h[kk & 1023u], 1u);
    }
  }
  __syncthreads();
  find_rank_bin<1024>(h, r2, sm, res);
  const uint32_t kth = (pre << 10) | (uint32_t)res[0];
  const int ties = r2 - res[1];
  __syncthreads();
  int32_t *out = a.idx + (int64_t)q * k;
  if (in_lds)
    emit_selected(get_lds, ntot, kth, ties, out, k, sm);
  else
    emit_selected(get_glb, ntot, kth, ties, out, k, sm);
  if (t == 0 && a.count) a.count[q] = k;
}

hipError_t launch_topk_init(const TopkWs &ws, int num_q, hipStream_t st) {
  const int64_t n = (int64_t)num_q * (2 * TOPK_BINS + 1);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, ws.hist, n);
  return hipGetLastError();
}

hipError_t launch_topk_hist(const float *scores, int64_t ld, const int32_t *q_nvis, const TopkWs &ws, int num_q,
                            int max_nvis, hipStream_t st) {
  if (num_q == 0 || ws.nchunks == 0 || max_nvis <= TOPK_ROW_MAX) return hipSuccess;
  const int64_t blocks = (int64_t)num_q * ws.nchunks;
  hipLaunchKernelGGL(topk_hist_kernel, dim3((unsigned)blocks), dim3(TK_THREADS), 0, st, scores, ld, q_nvis,
                     ws.hist, ws.nchunks);
  return hipGetLastError();
}

hipError_t launch_topk_select(const float *scores, int64_t ld, const int32_t *q_nvis, int k, int32_t *idx,
                              int32_t *count, const TopkWs &ws, int num_q, int max_nvis, bool hist1_valid,
                              hipStream_t st) {
  if (num_q == 0) return hipSuccess;
  SelectArgs a{scores, ld, q_nvis, k, hist1_valid ? 1 : 0, idx, count, ws};
  hipLaunchKernelGGL(topk_row_kernel, dim3((unsigned)num_q), dim3(TK_THREADS), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ws.nchunks == 0 || max_nvis <= TOPK_ROW_MAX) return e;
  const int64_t blocks = (int64_t)num_q * ws.nchunks;
  hipLaunchKernelGGL(topk_chunk_kernel, dim3((unsigned)blocks), dim3(TK_THREADS), 0, st, a);
  return hipGetLastError();
}

}  // namespace dsa
