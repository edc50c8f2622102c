// Per-query top-k selection over fp32 scores (gfx950).
//
// Page "arXiv'25 | DSA ... DeepSeek-V3.2", section 3 (second equation: the
// top-k of the scores over the earlier positions); page "DeepSeekV3.2之DSA",
// part 4.4 (the indices of the min(topk, end_pos) largest) and part 4.5 (a
// history no longer than k keeps everything).  Ties go to the lower position
// and -0 equals +0 (readings, the pages are silent); the output is in
// ascending position order, padded with -1.
//
// Radix select on order-preserving 32-bit keys, digits of 11 / 11 / 10 bits:
//   1. coarse histogram of key[31:21] per query (2048 bins; LDS atomics per
//      block, then one global atomic per non-empty bin) - done either by
//      topk_hist_kernel or fused into the indexer's epilogue;
//   2. topk_select_kernel, one block per (query, 8192-score chunk): finds the
//      threshold bin B1 from the histogram (count above B1 < k <= count above
//      plus count in B1), and compacts, in position order, every score whose
//      coarse bin is >= B1 into the chunk's candidate list (ballot-free block
//      scan, so the order is deterministic);
//   3. the last block of a query to finish (atomic counter + device-scope
//      fences, so the lists of all chunks are visible) refines B1 with two
//      more digits over the candidates alone, which gives the exact k-th key
//      T and how many keys equal to T to keep, then walks the candidates in
//      position order and writes the selected positions.
// The scores are read from HBM once by step 2 (plus once by step 1 when it is
// not fused); the candidate lists hold about k + |B1| entries and stay in L2.
#include "device_util.h"
#include "dsa_internal.h"

namespace dsa {

constexpr int TK_THREADS = 256;

static inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

static inline int topk_nchunks(int max_nvis) { return max_nvis <= 0 ? 1 : (max_nvis + TOPK_CHUNK - 1) / TOPK_CHUNK; }

size_t topk_ws_bytes(int num_q, int max_nvis) {
  const size_t nq = (size_t)num_q;
  const size_t nc = (size_t)topk_nchunks(max_nvis);
  return align256(nq * (TOPK_BINS + 1) * 4) + align256(nq * nc * 4) + nq * nc * TOPK_CHUNK * sizeof(uint2);
}

TopkWs topk_ws_carve(void *ws, int num_q, int max_nvis) {
  TopkWs w;
  const size_t nq = (size_t)num_q;
  w.nchunks = topk_nchunks(max_nvis);
  uint8_t *p = static_cast<uint8_t *>(ws);
  w.hist = reinterpret_cast<uint32_t *>(p);
  w.done = w.hist + nq * TOPK_BINS;  // contiguous with hist: one zero-fill clears both
  p += align256(nq * (TOPK_BINS + 1) * 4);
  w.ccount = reinterpret_cast<uint32_t *>(p);
  p += align256(nq * w.nchunks * 4);
  w.cand = reinterpret_cast<uint2 *>(p);
  return w;
}

// ------------------------------------------------------------------ helpers
// Exclusive scan of one int per thread over the block (TK_THREADS threads).
__device__ __forceinline__ int block_exclusive_scan(int v, int *sm, int &total) {
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int inc = wave_inclusive_scan(v);
  if (lane == WAVE - 1) sm[wave] = inc;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < TK_THREADS / WAVE; ++w) {
    const int s = sm[w];
    if (w < wave) before += s;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return before + inc - v;
}

// Given an LDS histogram h[nb] and a rank r >= 1 counted from the top, finds the
// bin B with above(B) < r <= above(B) + h[B], where above(B) = sum of h[b > B].
// Result in res[0] = B, res[1] = above(B) (all threads see it on return).
template <int NB>
__device__ void find_rank_bin(const uint32_t *h, int r, int *sm, int *res) {
  constexpr int PER = NB / TK_THREADS;
  const int t = threadIdx.x;
  const int hi = NB - PER * t;  // this thread owns bins [hi - PER, hi), scanned top-down
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

// ------------------------------------------------------------------ kernels
__global__ __launch_bounds__(256) void topk_zero_kernel(uint32_t *p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

__device__ __forceinline__ float load_score(const float *row, int i) { return row[i]; }

__global__ __launch_bounds__(TK_THREADS) void topk_hist_kernel(const float *__restrict__ scores, int64_t ld,
                                                               const int32_t *__restrict__ q_nvis, int k,
                                                               uint32_t *__restrict__ ghist, int nchunks) {
  const int q = blockIdx.x / nchunks;
  const int c = blockIdx.x - q * nchunks;
  const int n = q_nvis[q];
  const int start = c * TOPK_CHUNK;
  if (n <= k || start >= n) return;
  const int end = min(start + TOPK_CHUNK, n);
  __shared__ uint32_t h[TOPK_BINS];
  for (int b = threadIdx.x; b < TOPK_BINS; b += TK_THREADS) h[b] = 0u;
  __syncthreads();
  const float *row = scores + (int64_t)q * ld;
  for (int i = start + 4 * threadIdx.x; i < end; i += 4 * TK_THREADS) {
    if (i + 3 < end) {
      const float4 v = *reinterpret_cast<const float4 *>(row + i);
      atomicAdd(&h[order_key(v.x) >> 21], 1u);
      atomicAdd(&h[order_key(v.y) >> 21], 1u);
      atomicAdd(&h[order_key(v.z) >> 21], 1u);
      atomicAdd(&h[order_key(v.w) >> 21], 1u);
    } else {
      for (int j = i; j < end; ++j) atomicAdd(&h[order_key(row[j]) >> 21], 1u);
    }
  }
  __syncthreads();
  uint32_t *gh = ghist + (int64_t)q * TOPK_BINS;
  for (int b = threadIdx.x; b < TOPK_BINS; b += TK_THREADS) {
    const uint32_t v = h[b];
    if (v) atomicAdd(&gh[b], v);
  }
}

struct SelectArgs {
  const float *scores;
  int64_t ld;
  const int32_t *q_nvis;
  int k;
  int32_t *idx;
  int32_t *count;
  TopkWs ws;
};

// Final step for one query, run by the last block to finish its chunk.
__device__ void topk_finalize(const SelectArgs &a, int q, int nc, uint32_t b1, int above1, uint32_t *h,
                              int *sm, int *res) {
  const int k = a.k;
  const int r = k - above1;  // keys to take from the threshold bin B1 (>= 1)
  const uint2 *cand_q = a.ws.cand + (int64_t)q * a.ws.nchunks * TOPK_CHUNK;
  const uint32_t *cnt_q = a.ws.ccount + (int64_t)q * a.ws.nchunks;

  // Digit 2: key[20:10] of the candidates in bin B1.
  for (int b = threadIdx.x; b < TOPK_BINS; b += TK_THREADS) h[b] = 0u;
  __syncthreads();
  for (int c = 0; c < nc; ++c) {
    const int cnt = (int)cnt_q[c];
    const uint2 *lst = cand_q + (int64_t)c * TOPK_CHUNK;
    for (int i = threadIdx.x; i < cnt; i += TK_THREADS) {
      const uint32_t key = lst[i].x;
      if ((key >> 21) == b1) atomicAdd(&h[(key >> 10) & 2047u], 1u);
    }
  }
  __syncthreads();
  find_rank_bin<TOPK_BINS>(h, r, sm, res);
  const uint32_t b2 = (uint32_t)res[0];
  const int r2 = r - res[1];
  __syncthreads();

  // Digit 3: key[9:0] of the candidates with key[31:10] == (B1, B2).
  const uint32_t pre = (b1 << 11) | b2;
  for (int b = threadIdx.x; b < 1024; b += TK_THREADS) h[b] = 0u;
  __syncthreads();
  for (int c = 0; c < nc; ++c) {
    const int cnt = (int)cnt_q[c];
    const uint2 *lst = cand_q + (int64_t)c * TOPK_CHUNK;
    for (int i = threadIdx.x; i < cnt; i += TK_THREADS) {
      const uint32_t key = lst[i].x;
      if ((key >> 10) == pre) atomicAdd(&h[key & 1023u], 1u);
    }
  }
  __syncthreads();
  find_rank_bin<1024>(h, r2, sm, res);
  const uint32_t kth = (pre << 10) | (uint32_t)res[0];  // the exact k-th largest key
  const int ties = r2 - res[1];                         // keys == kth to keep, lowest positions first
  __syncthreads();

  // Emit in position order: keys > kth, and the first `ties` keys == kth.
  int32_t *out = a.idx + (int64_t)q * k;
  int taken = 0, tie_seen = 0;
  for (int c = 0; c < nc; ++c) {
    const int cnt = (int)cnt_q[c];
    const uint2 *lst = cand_q + (int64_t)c * TOPK_CHUNK;
    for (int i0 = 0; i0 < cnt; i0 += TK_THREADS) {
      const int i = i0 + threadIdx.x;
      uint2 e = make_uint2(0u, 0u);
      if (i < cnt) e = lst[i];
      const int is_tie = (i < cnt && e.x == kth) ? 1 : 0;
      int tie_tot;
      const int tie_rank = tie_seen + block_exclusive_scan(is_tie, sm, tie_tot);
      const int sel = (i < cnt && (e.x > kth || (is_tie && tie_rank < ties))) ? 1 : 0;
      int sel_tot;
      const int pos = taken + block_exclusive_scan(sel, sm, sel_tot);
      if (sel && pos < k) out[pos] = (int32_t)e.y;
      taken += sel_tot;
      tie_seen += tie_tot;
    }
  }
  // Exactly k positions are selected when the histogram and the candidate
  // lists agree; pad defensively so a reader never sees stale entries.
  for (int i = taken + threadIdx.x; i < k; i += TK_THREADS) out[i] = -1;
  if (threadIdx.x == 0 && a.count) a.count[q] = min(taken, k);
}

__global__ __launch_bounds__(TK_THREADS) void topk_select_kernel(SelectArgs a) {
  const int nchunks = a.ws.nchunks;
  const int q = blockIdx.x / nchunks;
  const int c = blockIdx.x - q * nchunks;
  const int n = a.q_nvis[q];
  const int k = a.k;
  if (n <= k) {  // short history: every position, no scores read
    if (c == 0) {
      int32_t *out = a.idx + (int64_t)q * k;
      for (int i = threadIdx.x; i < k; i += TK_THREADS) out[i] = (i < n) ? i : -1;
      if (threadIdx.x == 0 && a.count) a.count[q] = n;
    }
    return;
  }
  const int nc = (n + TOPK_CHUNK - 1) / TOPK_CHUNK;
  if (c >= nc) return;

  __shared__ uint32_t h[TOPK_BINS];
  __shared__ int sm[TK_THREADS / WAVE];
  __shared__ int res[2];
  __shared__ int is_last;

  // Threshold bin from the coarse histogram.
  const uint32_t *gh = a.ws.hist + (int64_t)q * TOPK_BINS;
  for (int b = threadIdx.x; b < TOPK_BINS; b += TK_THREADS) h[b] = gh[b];
  __syncthreads();
  find_rank_bin<TOPK_BINS>(h, k, sm, res);
  const uint32_t b1 = (uint32_t)res[0];
  const int above1 = res[1];

  // Compact the chunk's candidates (coarse bin >= B1) in position order.
  const int start = c * TOPK_CHUNK;
  const int end = min(start + TOPK_CHUNK, n);
  const float *row = a.scores + (int64_t)q * a.ld;
  uint2 *lst = a.ws.cand + ((int64_t)q * nchunks + c) * TOPK_CHUNK;
  int written = 0;
  for (int i0 = start; i0 < end; i0 += 4 * TK_THREADS) {
    const int i = i0 + 4 * threadIdx.x;
    uint32_t key[4];
    int f = 0;
    if (i + 3 < end) {
      const float4 v = *reinterpret_cast<const float4 *>(row + i);
      key[0] = order_key(v.x); key[1] = order_key(v.y); key[2] = order_key(v.z); key[3] = order_key(v.w);
#pragma unroll
      for (int j = 0; j < 4; ++j) f += ((key[j] >> 21) >= b1) ? 1 : 0;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        key[j] = (i + j < end) ? order_key(row[i + j]) : 0u;
        f += (i + j < end && (key[j] >> 21) >= b1) ? 1 : 0;
      }
    }
    int tot;
    int pos = written + block_exclusive_scan(f, sm, tot);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (i + j < end && (key[j] >> 21) >= b1) lst[pos++] = make_uint2(key[j], (uint32_t)(i + j));
    }
    written += tot;
  }
  if (threadIdx.x == 0) a.ws.ccount[(int64_t)q * nchunks + c] = (uint32_t)written;

  // The last block of this query to get here finishes the selection.
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) is_last = (atomicAdd(&a.ws.done[q], 1u) == (uint32_t)(nc - 1)) ? 1 : 0;
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  topk_finalize(a, q, nc, b1, above1, h, sm, res);
}

hipError_t launch_topk_init(const TopkWs &ws, int num_q, hipStream_t st) {
  const int64_t n = (int64_t)num_q * (TOPK_BINS + 1);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, ws.hist, n);
  return hipGetLastError();
}

hipError_t launch_topk_hist(const float *scores, int64_t ld, const int32_t *q_nvis, int k, const TopkWs &ws,
                            int num_q, int max_nvis, hipStream_t st) {
  if (num_q == 0 || max_nvis <= k) return hipSuccess;
  const int64_t blocks = (int64_t)num_q * ws.nchunks;
  hipLaunchKernelGGL(topk_hist_kernel, dim3((unsigned)blocks), dim3(TK_THREADS), 0, st, scores, ld, q_nvis, k,
                     ws.hist, ws.nchunks);
  return hipGetLastError();
}

hipError_t launch_topk_select(const float *scores, int64_t ld, const int32_t *q_nvis, int k, int32_t *idx,
                              int32_t *count, const TopkWs &ws, int num_q, int max_nvis, hipStream_t st) {
  (void)max_nvis;
  if (num_q == 0) return hipSuccess;
  SelectArgs a{scores, ld, q_nvis, k, idx, count, ws};
  const int64_t blocks = (int64_t)num_q * ws.nchunks;
  hipLaunchKernelGGL(topk_select_kernel, dim3((unsigned)blocks), dim3(TK_THREADS), 0, st, a);
  return hipGetLastError();
}

}  // namespace dsa
