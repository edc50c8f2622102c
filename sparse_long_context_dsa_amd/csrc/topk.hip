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
// is a position-ordered compaction built from block-wide exclusive scans, so
// it is deterministic.
//
// A block of 256 threads owns 16384 consecutive scores, 64 per thread in
// registers: in each of 8 rounds every thread reads 8 consecutive scores and
// consecutive lanes read consecutive 32-byte pieces, so each load instruction
// covers whole cache lines.  Position order is (round, thread, element); the
// per-round counts of a thread are packed into two 64-bit words (12 bits per
// round) so that one pair of scans orders all 8 rounds.
//
// Kernels, chosen per query by its history length n:
//  * topk_row_kernel (n <= 16384, e.g. every causal-prefill row): one block
//    per query; only the histograms live in LDS, so many rows are selected per
//    CU at once.  The first-digit histogram comes from the indexer's fused
//    epilogue when available, else from LDS atomics.
//  * topk_chunk_kernel + topk_final_kernel (longer rows, e.g. 128K decode):
//    chunk blocks stream the scores once, find the threshold bin B1 from the
//    first-digit histogram, compact the candidates (digit >= B1, about
//    k + |B1| of them) into per-chunk lists in position order and add the
//    second-digit histogram of the B1 keys into a global one; then one block
//    per query loads the histograms and all candidate lists into LDS with
//    independent loads and finishes there (from global memory if the lists do
//    not fit).  The kernel boundary publishes the lists, so no block-level
//    device-scope fences are needed.
#include "device_util.h"
#include "dsa_internal.h"

namespace dsa {

constexpr int TK_THREADS = 256;
constexpr int TK_ROUNDS = 8;                                  // rounds per block
constexpr int TK_J = TOPK_ROW_MAX / (TK_THREADS * TK_ROUNDS);  // 8 scores per thread per round
constexpr int TK_PER = TK_ROUNDS * TK_J;                      // 64 keys per thread
constexpr int TK_ROUND_SPAN = TK_THREADS * TK_J;              // 2048 positions per round
constexpr int FIN_THREADS = 1024;
constexpr int LIST_CAP = 8192;  // candidates the finalize keeps in LDS
static_assert(TOPK_CHUNK == TOPK_ROW_MAX, "one block covers one chunk");
static_assert(TK_J == 8, "two float4 loads per round");

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
  w.done = w.hist2 + nq * TOPK_BINS;         // [nq] (unused; cleared with the histograms)
  p += align256(nq * (2 * TOPK_BINS + 1) * 4);
  w.ccount = reinterpret_cast<uint32_t *>(p);
  p += align256(nq * w.nchunks * 4);
  w.cand = reinterpret_cast<uint2 *>(p);
  return w;
}

// ------------------------------------------------------------------ helpers
// Exclusive scan over the block of one value per thread; `total` gets the sum.
template <int NT, typename T>
__device__ __forceinline__ T block_exclusive_scan(T v, T *sm, T &total) {
  constexpr int W = NT / WAVE;
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  T inc = v;
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) {
    const T o = __shfl_up(inc, d, WAVE);
    if (lane >= d) inc += o;
  }
  if (lane == WAVE - 1) sm[wave] = inc;
  __syncthreads();
  T before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const T s = sm[w];
    before += (w < wave) ? s : T(0);
    tot += s;
  }
  __syncthreads();
  total = tot;
  return before + inc - v;
}

// Given an LDS histogram h[NB] and a rank r >= 1 counted from the top, finds
// the bin B with above(B) < r <= above(B) + h[B] (above(B) = sum of h[b > B]).
// res[0] = B, res[1] = above(B), visible to all threads on return.
template <int NT, int NB>
__device__ void find_rank_bin(const uint32_t *h, int r, int *sm, int *res) {
  constexpr int PER = NB / NT;
  const int hi = NB - PER * (int)threadIdx.x;  // bins [hi - PER, hi), scanned top-down
  int local = 0;
#pragma unroll
  for (int i = 1; i <= PER; ++i) local += (int)h[hi - i];
  int total;
  int acc = block_exclusive_scan<NT>(local, sm, total);
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

template <int NT>
__device__ __forceinline__ void zero_lds(uint32_t *h, int n) {
  for (int b = threadIdx.x; b < n; b += NT) h[b] = 0u;
}

// Position of key slot (round rr, element j) of thread t relative to the block start.
__device__ __forceinline__ int slot_pos(int t, int rr, int j) { return rr * TK_ROUND_SPAN + TK_J * t + j; }

// Loads the 64 scores of this thread (positions base + slot_pos).  Positions
// >= n get key 0, below the key of any real score (even -inf maps to
// 0x007FFFFF): key 0 sits in first-digit bin 0, which no real score occupies,
// so it never reaches a threshold bin, never ties the k-th key and is never
// selected; the kernels need no separate position test.
__device__ __forceinline__ void load_keys(const float *row, int base, int n, uint32_t *key) {
  const int t = threadIdx.x;
#pragma unroll
  for (int rr = 0; rr < TK_ROUNDS; ++rr) {
    const int i = base + slot_pos(t, rr, 0);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int ii = i + 4 * h;
      if (ii + 3 < n) {
        const float4 f = *reinterpret_cast<const float4 *>(row + ii);
        key[TK_J * rr + 4 * h + 0] = order_key(f.x);
        key[TK_J * rr + 4 * h + 1] = order_key(f.y);
        key[TK_J * rr + 4 * h + 2] = order_key(f.z);
        key[TK_J * rr + 4 * h + 3] = order_key(f.w);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) key[TK_J * rr + 4 * h + j] = (ii + j < n) ? order_key(row[ii + j]) : 0u;
      }
    }
  }
}

// Per-round counts (each <= 8) packed 12 bits per round: rounds 0..4 in w0,
// 5..7 in w1.  Prefixes and totals of a field stay below 4096.
struct Packed {
  uint64_t w0, w1;
};
__device__ __forceinline__ void pack_add(Packed &p, int rr, int c) {
  if (rr < 5)
    p.w0 += (uint64_t)c << (12 * rr);
  else
    p.w1 += (uint64_t)c << (12 * (rr - 5));
}
__device__ __forceinline__ int pack_get(const Packed &p, int rr) {
  return (int)((rr < 5 ? p.w0 >> (12 * rr) : p.w1 >> (12 * (rr - 5))) & 0xFFFu);
}

// Exclusive position-order offsets of this thread's per-round counts `cnt`:
// off[rr] = (items in earlier rounds) + (items of earlier threads in round rr).
// Returns the block total.
__device__ __forceinline__ int ordered_offsets(const Packed &cnt, uint64_t *sm64, int *off) {
  uint64_t t0, t1;
  const uint64_t e0 = block_exclusive_scan<TK_THREADS>(cnt.w0, sm64, t0);
  const uint64_t e1 = block_exclusive_scan<TK_THREADS>(cnt.w1, sm64, t1);
  const Packed ex{e0, e1}, tot{t0, t1};
  int before = 0;
#pragma unroll
  for (int rr = 0; rr < TK_ROUNDS; ++rr) {
    off[rr] = before + pack_get(ex, rr);
    before += pack_get(tot, rr);
  }
  return before;
}

__device__ __forceinline__ void write_short(int32_t *out, int32_t *count, int q, int n, int k, int nt) {
  for (int i = threadIdx.x; i < k; i += nt) out[i] = (i < n) ? i : -1;
  if (threadIdx.x == 0 && count) count[q] = n;
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
  zero_lds<TK_THREADS>(h, TOPK_BINS);
  __syncthreads();
  uint32_t key[TK_PER];
  load_keys(scores + (int64_t)q * ld, start, n, key);
  const int t = threadIdx.x;
#pragma unroll
  for (int rr = 0; rr < TK_ROUNDS; ++rr)
#pragma unroll
    for (int j = 0; j < TK_J; ++j) atomicAdd(&h[key[TK_J * rr + j] >> 21], 1u);  // padding lands in bin 0
  __syncthreads();
  uint32_t *g = ghist + (int64_t)q * TOPK_BINS;
  for (int b = t; b < TOPK_BINS; b += TK_THREADS)
    if (h[b]) atomicAdd(&g[b], h[b]);
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
    write_short(out, a.count, q, n, k, TK_THREADS);
    return;
  }
  __shared__ uint32_t h[TOPK_BINS];
  __shared__ int sm[TK_THREADS / WAVE];
  __shared__ uint64_t sm64[TK_THREADS / WAVE];
  __shared__ int res[2];
  const int t = threadIdx.x;
  uint32_t key[TK_PER];
  load_keys(a.scores + (int64_t)q * a.ld, 0, n, key);
  // Digit 1: key[31:21].
  if (a.hist1_valid) {
    const uint32_t *gh = a.ws.hist + (int64_t)q * TOPK_BINS;
    for (int b = t; b < TOPK_BINS; b += TK_THREADS) h[b] = gh[b];
  } else {
    zero_lds<TK_THREADS>(h, TOPK_BINS);
    __syncthreads();
#pragma unroll
    for (int rr = 0; rr < TK_ROUNDS; ++rr)
#pragma unroll
      for (int j = 0; j < TK_J; ++j)
        atomicAdd(&h[key[TK_J * rr + j] >> 21], 1u);  // padding keys land in bin 0
  }
  __syncthreads();
  find_rank_bin<TK_THREADS, TOPK_BINS>(h, k, sm, res);
  const uint32_t b1 = (uint32_t)res[0];
  const int r = k - res[1];
  __syncthreads();
  // Digit 2: key[20:10] of the keys in bin B1.
  zero_lds<TK_THREADS>(h, TOPK_BINS);
  __syncthreads();
#pragma unroll
  for (int rr = 0; rr < TK_ROUNDS; ++rr)
#pragma unroll
    for (int j = 0; j < TK_J; ++j) {
      const uint32_t kk = key[TK_J * rr + j];
      if ((kk >> 21) == b1) atomicAdd(&h[(kk >> 10) & 2047u], 1u);
    }
  __syncthreads();
  find_rank_bin<TK_THREADS, TOPK_BINS>(h, r, sm, res);
  const uint32_t pre = (b1 << 11) | (uint32_t)res[0];
  const int r2 = r - res[1];
  __syncthreads();
  // Digit 3: key[9:0] of the keys with key[31:10] == pre.
  zero_lds<TK_THREADS>(h, 1024);
  __syncthreads();
#pragma unroll
  for (int rr = 0; rr < TK_ROUNDS; ++rr)
#pragma unroll
    for (int j = 0; j < TK_J; ++j) {
      const uint32_t kk = key[TK_J * rr + j];
      if ((kk >> 10) == pre) atomicAdd(&h[kk & 1023u], 1u);
    }
  __syncthreads();
  find_rank_bin<TK_THREADS, 1024>(h, r2, sm, res);
  const uint32_t kth = (pre << 10) | (uint32_t)res[0];
  const int ties = r2 - res[1];
  // Emit in position order: keys > kth, and the first `ties` keys == kth.
  Packed tc{0, 0};
#pragma unroll
  for (int rr = 0; rr < TK_ROUNDS; ++rr) {
    int c = 0;
#pragma unroll
    for (int j = 0; j < TK_J; ++j) c += (key[TK_J * rr + j] == kth) ? 1 : 0;
    pack_add(tc, rr, c);
  }
  int toff[TK_ROUNDS];
  ordered_offsets(tc, sm64, toff);
  Packed sc{0, 0};
  uint32_t selbits[TK_ROUNDS];
#pragma unroll
  for (int rr = 0; rr < TK_ROUNDS; ++rr) {
    int tr = toff[rr], c = 0;
    uint32_t bits = 0;
#pragma unroll
    for (int j = 0; j < TK_J; ++j) {
      const uint32_t kk = key[TK_J * rr + j];
      const bool tie = kk == kth;
      const bool sel = kk > kth || (tie && tr < ties);
      tr += tie ? 1 : 0;
      c += sel ? 1 : 0;
      bits |= (uint32_t)sel << j;
    }
    selbits[rr] = bits;
    pack_add(sc, rr, c);
  }
  int soff[TK_ROUNDS];
  const int tot = ordered_offsets(sc, sm64, soff);
#pragma unroll
  for (int rr = 0; rr < TK_ROUNDS; ++rr) {
    int pos = soff[rr];
#pragma unroll
    for (int j = 0; j < TK_J; ++j)
      if (selbits[rr] & (1u << j)) {
        if (pos < k) out[pos] = slot_pos(t, rr, j);
        ++pos;
      }
  }
  for (int i = tot + t; i < k; i += TK_THREADS) out[i] = -1;  // defensive: tot == k
  if (t == 0 && a.count) a.count[q] = min(tot, k);
}

__global__ __launch_bounds__(TK_THREADS) void topk_chunk_kernel(SelectArgs a) {
  const int nchunks = a.ws.nchunks;
  const int q = blockIdx.x / nchunks;
  const int c = blockIdx.x - q * nchunks;
  const int n = a.q_nvis[q];
  const int k = a.k;
  if (n <= TOPK_ROW_MAX) return;
  const int start = c * TOPK_CHUNK;
  if (start >= n) return;

  __shared__ uint32_t h[TOPK_BINS];
  __shared__ int sm[TK_THREADS / WAVE];
  __shared__ uint64_t sm64[TK_THREADS / WAVE];
  __shared__ int res[2];
  const int t = threadIdx.x;
  uint32_t key[TK_PER];
  load_keys(a.scores + (int64_t)q * a.ld, start, n, key);  // in flight while the histogram is read

  // Threshold bin B1 from the first-digit histogram.
  const uint32_t *gh1 = a.ws.hist + (int64_t)q * TOPK_BINS;
  for (int b = t; b < TOPK_BINS; b += TK_THREADS) h[b] = gh1[b];
  __syncthreads();
  find_rank_bin<TK_THREADS, TOPK_BINS>(h, k, sm, res);
  const uint32_t b1 = (uint32_t)res[0];
  __syncthreads();
  zero_lds<TK_THREADS>(h, TOPK_BINS);
  __syncthreads();

  // Candidates (digit >= B1) in position order; second-digit histogram of B1.
  Packed fc{0, 0};
#pragma unroll
  for (int rr = 0; rr < TK_ROUNDS; ++rr) {
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < TK_J; ++j) {
      const uint32_t kk = key[TK_J * rr + j];
      cnt += ((kk >> 21) >= b1) ? 1 : 0;
      if ((kk >> 21) == b1) atomicAdd(&h[(kk >> 10) & 2047u], 1u);
    }
    pack_add(fc, rr, cnt);
  }
  int off[TK_ROUNDS];
  const int total = ordered_offsets(fc, sm64, off);  // its barriers also complete the histogram
  uint2 *glst = a.ws.cand + ((int64_t)q * nchunks + c) * TOPK_CHUNK;
#pragma unroll
  for (int rr = 0; rr < TK_ROUNDS; ++rr) {
    int pos = off[rr];
#pragma unroll
    for (int j = 0; j < TK_J; ++j) {
      const uint32_t kk = key[TK_J * rr + j];
      if ((kk >> 21) >= b1) glst[pos++] = make_uint2(kk, (uint32_t)(start + slot_pos(t, rr, j)));
    }
  }
  if (t == 0) a.ws.ccount[(int64_t)q * nchunks + c] = (uint32_t)total;
  uint32_t *g2 = a.ws.hist2 + (int64_t)q * TOPK_BINS;
  for (int b = t; b < TOPK_BINS; b += TK_THREADS)
    if (h[b]) atomicAdd(&g2[b], h[b]);
}

// Finds the chunk holding candidate i, given the exclusive prefix off[0..nc].
__device__ __forceinline__ int locate(const int *off, int nc, int i) {
  int c = 0;
  while (c + 1 < nc && off[c + 1] <= i) ++c;
  return c;
}

__global__ __launch_bounds__(FIN_THREADS) void topk_final_kernel(SelectArgs a) {
  const int nchunks = a.ws.nchunks;
  const int q = blockIdx.x;
  const int n = a.q_nvis[q];
  const int k = a.k;
  if (n <= TOPK_ROW_MAX) return;
  const int nc = (n + TOPK_CHUNK - 1) / TOPK_CHUNK;

  __shared__ uint2 lst[LIST_CAP];
  __shared__ uint32_t h1[TOPK_BINS];
  __shared__ uint32_t h2[TOPK_BINS];
  __shared__ int sm[FIN_THREADS / WAVE];
  __shared__ int res[2];
  __shared__ int off[TOPK_MAX_CHUNKS + 1];
  const int t = threadIdx.x;

  // Everything that does not depend on anything else is requested at once.
  const uint32_t *gh1 = a.ws.hist + (int64_t)q * TOPK_BINS;
  const uint32_t *gh2 = a.ws.hist2 + (int64_t)q * TOPK_BINS;
  for (int b = t; b < TOPK_BINS; b += FIN_THREADS) {
    h1[b] = gh1[b];
    h2[b] = gh2[b];
  }
  if (t < nc) off[t + 1] = (int)a.ws.ccount[(int64_t)q * nchunks + t];
  __syncthreads();
  if (t == 0) {
    off[0] = 0;
    for (int cc = 1; cc <= nc; ++cc) off[cc] += off[cc - 1];
  }
  find_rank_bin<FIN_THREADS, TOPK_BINS>(h1, k, sm, res);  // its barriers publish off[]
  const uint32_t b1 = (uint32_t)res[0];
  const int r = k - res[1];
  __syncthreads();
  find_rank_bin<FIN_THREADS, TOPK_BINS>(h2, r, sm, res);
  const uint32_t pre = (b1 << 11) | (uint32_t)res[0];
  const int r2 = r - res[1];
  const int ntot = off[nc];
  const uint2 *cand_q = a.ws.cand + (int64_t)q * nchunks * TOPK_CHUNK;
  const bool in_lds = ntot <= LIST_CAP;
  __syncthreads();
  zero_lds<FIN_THREADS>(h1, 1024);
  if (in_lds) {
#pragma unroll
    for (int j = 0; j < LIST_CAP / FIN_THREADS; ++j) {
      const int i = t + j * FIN_THREADS;
      if (i < ntot) {
        const int cc = locate(off, nc, i);
        lst[i] = cand_q[(int64_t)cc * TOPK_CHUNK + (i - off[cc])];
      }
    }
  }
  __syncthreads();
  auto get = [&](int i) {
    if (in_lds) return lst[i];
    const int cc = locate(off, nc, i);
    return cand_q[(int64_t)cc * TOPK_CHUNK + (i - off[cc])];
  };
  // Digit 3 over the candidates with key[31:10] == pre; contiguous runs per thread.
  const int per = (ntot + FIN_THREADS - 1) / FIN_THREADS;
  const int lo = min(ntot, per * t), hi = min(ntot, lo + per);
  for (int i = lo; i < hi; ++i) {
    const uint32_t kk = get(i).x;
    if ((kk >> 10) == pre) atomicAdd(&h1[kk & 1023u], 1u);
  }
  __syncthreads();
  find_rank_bin<FIN_THREADS, 1024>(h1, r2, sm, res);
  const uint32_t kth = (pre << 10) | (uint32_t)res[0];
  const int ties = r2 - res[1];
  // Emission in position order.
  int my_ties = 0;
  for (int i = lo; i < hi; ++i) my_ties += (get(i).x == kth) ? 1 : 0;
  int tot;
  const int tie_rank = block_exclusive_scan<FIN_THREADS>(my_ties, sm, tot);
  int my_sel = 0;
  for (int i = lo, tr = tie_rank; i < hi; ++i) {
    const uint32_t kk = get(i).x;
    if (kk > kth || (kk == kth && tr < ties)) ++my_sel;
    tr += (kk == kth) ? 1 : 0;
  }
  int pos = block_exclusive_scan<FIN_THREADS>(my_sel, sm, tot);
  int32_t *out = a.idx + (int64_t)q * k;
  for (int i = lo, tr = tie_rank; i < hi; ++i) {
    const uint2 e = get(i);
    if (e.x > kth || (e.x == kth && tr < ties)) {
      if (pos < k) out[pos] = (int32_t)e.y;
      ++pos;
    }
    tr += (e.x == kth) ? 1 : 0;
  }
  for (int i = tot + t; i < k; i += FIN_THREADS) out[i] = -1;  // defensive: tot == k
  if (t == 0 && a.count) a.count[q] = min(tot, k);
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
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_final_kernel, dim3((unsigned)num_q), dim3(FIN_THREADS), 0, st, a);
  return hipGetLastError();
}

}  // namespace dsa
