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
// A row block owns up to 16384 consecutive scores in registers: 256 threads
// with 64 each (8 rounds), or 1024 threads with 16 each (2 rounds).  In each
// round every thread reads 8 consecutive scores and consecutive lanes read
// consecutive 32-byte pieces, so each load instruction covers whole cache
// lines.  Position order is (round, thread, element); the per-round counts of
// a thread are packed into two 64-bit words so that one pair of scans orders
// all rounds.
//
// Kernels, chosen per batch by its longest history:
//  * every row n <= 16384 (e.g. causal prefill): topk_row_kernel, one
//    256-thread block per query; only the histograms live in LDS, so several
//    rows are selected per CU at once.  The first-digit histogram comes from
//    the indexer's fused epilogue when available, else from LDS atomics.
//  * some row longer (e.g. 128K decode): topk_long_kernel blocks of 16
//    wavefronts, each owning 32768 consecutive positions (2048 per
//    wavefront), first find the row's threshold bin B1 of the first digit
//    (and the count above it) from the histogram built with the scores, then
//    stream the scores once and append the candidates (digit >= B1, about
//    k + |B1| per row) to per-wavefront lists in position order, ranks from
//    ballots.  A short row of such a batch is selected whole by its first
//    1024-thread block, as a row block.  topk_finish_kernel (one block per
//    long row, after the kernel boundary has published the lists) loads the
//    lists into LDS in position order and finishes there: digits 2 and 3 as
//    LDS histograms of the candidates, then the output as a position-ordered
//    compaction.  (Handing the row to its last block inside one kernel would
//    need an agent-scope fence per block, which on this part writes back and
//    invalidates the XCD's L2 and costs far more.)
#include "device_util.h"
#include "dsa_internal.h"

namespace dsa {

constexpr int TK_THREADS = 256;                               // threads of a row block
constexpr int TK_J = 8;                                       // scores per thread per round (two float4)
// A block of NT threads holding one row of up to TOPK_ROW_MAX scores in
// registers: ROUNDS rounds of TK_J consecutive scores per thread.
template <int NT>
struct RowShape {
  static constexpr int ROUNDS = TOPK_ROW_MAX / (NT * TK_J);  // 8 for 256 threads, 2 for 1024
  static constexpr int PER = ROUNDS * TK_J;                  // keys per thread
  static constexpr int ROUND_SPAN = NT * TK_J;               // positions per round
  static_assert(ROUNDS >= 1 && ROUNDS <= 8 && ROUNDS * NT * TK_J == TOPK_ROW_MAX, "whole rounds, <= 8");
};
constexpr int LONG_THREADS = TOPK_LONG_WAVES * WAVE;
constexpr int LONG_ROUNDS = TOPK_WAVE_SPAN / 512;  // rounds of 512 positions per wavefront
constexpr int TAIL_CAP = 12288;                     // candidates the finishing block keeps in LDS
static_assert(TOPK_CHUNK == TOPK_ROW_MAX, "one histogram block covers one chunk");

static inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

static inline int topk_nchunks(int max_nvis) {
  return max_nvis <= TOPK_ROW_MAX ? 0 : (max_nvis + TOPK_CHUNK - 1) / TOPK_CHUNK;
}
static inline int topk_nblk(int max_nvis) {
  return max_nvis <= TOPK_ROW_MAX ? 0 : (max_nvis + TOPK_LONG_SPAN - 1) / TOPK_LONG_SPAN;
}

size_t topk_ws_bytes(int num_q, int max_nvis) {
  const size_t nq = (size_t)num_q, nb = (size_t)topk_nblk(max_nvis);
  return align256(nq * TOPK_BINS * 4) + align256(nq * sizeof(uint2)) +
         align256(nq * nb * TOPK_LONG_WAVES * 4) + nq * nb * TOPK_LONG_SPAN * sizeof(uint2);
}

TopkWs topk_ws_carve(void *ws, int num_q, int max_nvis) {
  TopkWs w;
  const size_t nq = (size_t)num_q;
  w.nchunks = topk_nchunks(max_nvis);
  w.nblk = topk_nblk(max_nvis);
  uint8_t *p = static_cast<uint8_t *>(ws);
  w.hist = reinterpret_cast<uint32_t *>(p);  // [nq, 2048] first digit (cleared each call)
  p += align256(nq * TOPK_BINS * 4);
  w.b1info = reinterpret_cast<uint2 *>(p);   // [nq] written before it is read
  p += align256(nq * sizeof(uint2));
  w.wcnt = reinterpret_cast<uint32_t *>(p);
  p += align256(nq * w.nblk * TOPK_LONG_WAVES * 4);
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
template <int NT>
__device__ __forceinline__ int slot_pos(int t, int rr, int j) {
  return rr * RowShape<NT>::ROUND_SPAN + TK_J * t + j;
}

// Loads the scores of this thread (positions base + slot_pos).  Positions
// >= n get key 0, below the key of any real score (even -inf maps to
// 0x007FFFFF): key 0 sits in first-digit bin 0, which no real score occupies,
// so it never reaches a threshold bin, never ties the k-th key and is never
// selected; the kernels need no separate position test.
template <int NT>
__device__ __forceinline__ void load_keys(const float *row, int base, int n, uint32_t *key) {
  const int t = threadIdx.x;
#pragma unroll
  for (int rr = 0; rr < RowShape<NT>::ROUNDS; ++rr) {
    const int i = base + slot_pos<NT>(t, rr, 0);
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

// Per-round counts (each <= TK_J) packed into two 64-bit words, so that one
// pair of block scans orders every round.  A field must hold the block total
// of its round, NT * TK_J: 12-bit fields (5 per word) for 256 threads (2048),
// 32-bit fields (2 per word) for 1024 threads (8192; 2 rounds).
struct Packed {
  uint64_t w0, w1;
};
template <int NT>
struct PackShape {
  static constexpr int BITS = NT * TK_J < 4096 ? 12 : 32;
  static constexpr int PER_WORD = 64 / BITS;
  static constexpr uint64_t MASK = (1ull << BITS) - 1;
  static_assert((uint64_t)(NT * TK_J) <= MASK && RowShape<NT>::ROUNDS <= 2 * PER_WORD, "fields hold a round's total");
};
template <int NT>
__device__ __forceinline__ void pack_add(Packed &p, int rr, int c) {
  using PS = PackShape<NT>;
  if (rr < PS::PER_WORD)
    p.w0 += (uint64_t)c << (PS::BITS * rr);
  else
    p.w1 += (uint64_t)c << (PS::BITS * (rr - PS::PER_WORD));
}
template <int NT>
__device__ __forceinline__ int pack_get(const Packed &p, int rr) {
  using PS = PackShape<NT>;
  return (int)((rr < PS::PER_WORD ? p.w0 >> (PS::BITS * rr) : p.w1 >> (PS::BITS * (rr - PS::PER_WORD))) & PS::MASK);
}

// Exclusive position-order offsets of this thread's per-round counts `cnt`:
// off[rr] = (items in earlier rounds) + (items of earlier threads in round rr).
// Returns the block total.
template <int NT>
__device__ __forceinline__ int ordered_offsets(const Packed &cnt, uint64_t *sm64, int *off) {
  uint64_t t0, t1;
  const uint64_t e0 = block_exclusive_scan<NT>(cnt.w0, sm64, t0);
  const uint64_t e1 = block_exclusive_scan<NT>(cnt.w1, sm64, t1);
  const Packed ex{e0, e1}, tot{t0, t1};
  int before = 0;
#pragma unroll
  for (int rr = 0; rr < RowShape<NT>::ROUNDS; ++rr) {
    off[rr] = before + pack_get<NT>(ex, rr);
    before += pack_get<NT>(tot, rr);
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
  uint32_t key[RowShape<TK_THREADS>::PER];
  load_keys<TK_THREADS>(scores + (int64_t)q * ld, start, n, key);
  const int t = threadIdx.x;
#pragma unroll
  for (int rr = 0; rr < RowShape<TK_THREADS>::ROUNDS; ++rr)
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

// Selects row q (n <= TOPK_ROW_MAX scores) with one block of NT threads:
// digit 1 from the indexer's histogram or from LDS atomics, digits 2 and 3 as
// LDS histograms of the keys in the threshold bins, then the position-ordered
// compaction.  Every thread of the block calls it (it has block barriers).
template <int NT>
__device__ void row_select(const SelectArgs &a, const int q, const int n, uint32_t *h, int *sm, uint64_t *sm64,
                           int *res) {
  using RS = RowShape<NT>;
  const int k = a.k;
  const int t = threadIdx.x;
  int32_t *out = a.idx + (int64_t)q * k;
  if (n <= k) {
    write_short(out, a.count, q, n, k, NT);
    return;
  }
  uint32_t key[RS::PER];
  load_keys<NT>(a.scores + (int64_t)q * a.ld, 0, (int)min((int64_t)n, a.ld), key);  // never past the row's ld
  // Digit 1: key[31:21].
  if (a.hist1_valid) {
    const uint32_t *gh = a.ws.hist + (int64_t)q * TOPK_BINS;
    for (int b = t; b < TOPK_BINS; b += NT) h[b] = gh[b];
  } else {
    zero_lds<NT>(h, TOPK_BINS);
    __syncthreads();
#pragma unroll
    for (int rr = 0; rr < RS::ROUNDS; ++rr)
#pragma unroll
      for (int j = 0; j < TK_J; ++j)
        atomicAdd(&h[key[TK_J * rr + j] >> 21], 1u);  // padding keys land in bin 0
  }
  __syncthreads();
  find_rank_bin<NT, TOPK_BINS>(h, k, sm, res);
  const uint32_t b1 = (uint32_t)res[0];
  const int r = k - res[1];
  __syncthreads();
  // Digit 2: key[20:10] of the keys in bin B1.
  zero_lds<NT>(h, TOPK_BINS);
  __syncthreads();
#pragma unroll
  for (int rr = 0; rr < RS::ROUNDS; ++rr)
#pragma unroll
    for (int j = 0; j < TK_J; ++j) {
      const uint32_t kk = key[TK_J * rr + j];
      if ((kk >> 21) == b1) atomicAdd(&h[(kk >> 10) & 2047u], 1u);
    }
  __syncthreads();
  find_rank_bin<NT, TOPK_BINS>(h, r, sm, res);
  const uint32_t pre = (b1 << 11) | (uint32_t)res[0];
  const int r2 = r - res[1];
  __syncthreads();
  // Digit 3: key[9:0] of the keys with key[31:10] == pre.
  zero_lds<NT>(h, 1024);
  __syncthreads();
#pragma unroll
  for (int rr = 0; rr < RS::ROUNDS; ++rr)
#pragma unroll
    for (int j = 0; j < TK_J; ++j) {
      const uint32_t kk = key[TK_J * rr + j];
      if ((kk >> 10) == pre) atomicAdd(&h[kk & 1023u], 1u);
    }
  __syncthreads();
  find_rank_bin<NT, 1024>(h, r2, sm, res);
  const uint32_t kth = (pre << 10) | (uint32_t)res[0];
  const int ties = r2 - res[1];
  // Emit in position order: keys > kth, and the first `ties` keys == kth.
  Packed tc{0, 0};
#pragma unroll
  for (int rr = 0; rr < RS::ROUNDS; ++rr) {
    int c = 0;
#pragma unroll
    for (int j = 0; j < TK_J; ++j) c += (key[TK_J * rr + j] == kth) ? 1 : 0;
    pack_add<NT>(tc, rr, c);
  }
  int toff[RS::ROUNDS];
  ordered_offsets<NT>(tc, sm64, toff);
  Packed sc{0, 0};
  uint32_t selbits[RS::ROUNDS];
#pragma unroll
  for (int rr = 0; rr < RS::ROUNDS; ++rr) {
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
    pack_add<NT>(sc, rr, c);
  }
  int soff[RS::ROUNDS];
  const int tot = ordered_offsets<NT>(sc, sm64, soff);
#pragma unroll
  for (int rr = 0; rr < RS::ROUNDS; ++rr) {
    int pos = soff[rr];
#pragma unroll
    for (int j = 0; j < TK_J; ++j)
      if (selbits[rr] & (1u << j)) {
        if (pos < k) out[pos] = slot_pos<NT>(t, rr, j);
        ++pos;
      }
  }
  for (int i = tot + t; i < k; i += NT) out[i] = -1;  // defensive: tot == k
  if (t == 0 && a.count) a.count[q] = min(tot, k);
}

// Three wavefronts per SIMD (at most 168 VGPRs; the 64 keys per thread take
// 64): left to itself the compiler used 179 and fit two, and with only two rows
// per CU in flight the row loads, not the selection, set the pace (prefill
// top-k 0.60 -> 0.43 ms).  Four per SIMD would need spills, which measured
// slower.  Launched only when every row fits TOPK_ROW_MAX.
__global__ __launch_bounds__(TK_THREADS) __attribute__((amdgpu_waves_per_eu(3, 3))) void topk_row_kernel(
    SelectArgs a) {
  __shared__ uint32_t h[TOPK_BINS];
  __shared__ int sm[TK_THREADS / WAVE];
  __shared__ uint64_t sm64[TK_THREADS / WAVE];
  __shared__ int res[2];
  row_select<TK_THREADS>(a, blockIdx.x, a.q_nvis[blockIdx.x], h, sm, sm64, res);
}


// Lanes below this one in the wavefront (mbcnt over a ballot mask).
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}
// Exclusive prefix over the wavefront of c (0 <= c < 16) and the wave total,
// from one ballot per bit: no cross-lane data movement through LDS.
__device__ __forceinline__ int wave_excl_small(int c, int &total) {
  int ex = 0, tot = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint64_t m = __ballot((c >> b) & 1);
    ex += lanes_below(m) << b;
    tot += __popcll(m) << b;
  }
  total = tot;
  return ex;
}

__global__ __launch_bounds__(LONG_THREADS) void topk_long_kernel(SelectArgs a) {
  const int nblk = a.ws.nblk;
  const int q = blockIdx.x / nblk;
  const int c = blockIdx.x - q * nblk;
  const int n = a.q_nvis[q];
  const int k = a.k;
  __shared__ uint32_t h[TOPK_BINS];
  __shared__ int sm[LONG_THREADS / WAVE];
  __shared__ uint64_t sm64[LONG_THREADS / WAVE];
  __shared__ int res[2];
  if (n <= TOPK_ROW_MAX) {  // a short row of a batch with long rows: its first block selects it
    if (c == 0) row_select<LONG_THREADS>(a, q, n, h, sm, sm64, res);
    return;
  }
  const int nb = (n + TOPK_LONG_SPAN - 1) / TOPK_LONG_SPAN;
  if (c >= nb) return;
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & (WAVE - 1);
  const int p0 = c * TOPK_LONG_SPAN + wave * TOPK_WAVE_SPAN;
  const int p1 = min(n, p0 + TOPK_WAVE_SPAN);
  const float *row = a.scores + (int64_t)q * a.ld;

  // The row's first-digit histogram is requested before the scores: loads
  // complete in issue order, so the wait for it does not wait for them.
  const uint32_t *gh = a.ws.hist + (int64_t)q * TOPK_BINS;
  uint32_t hv[TOPK_BINS / LONG_THREADS];
#pragma unroll
  for (int i = 0; i < TOPK_BINS / LONG_THREADS; ++i) hv[i] = gh[t + i * LONG_THREADS];

  // All score loads first.  Lane l reads positions p0 + 512 u + 8 l .. +7 of
  // round u; a float4 at a position < p1 stays inside the row (ld % 4 == 0),
  // past p1 it reads position 0 and the keys become 0, below B1.
  float4 f[LONG_ROUNDS][2];
#pragma unroll
  for (int u = 0; u < LONG_ROUNDS; ++u)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int ii = p0 + 512 * u + 8 * lane + 4 * hh;
      f[u][hh] = *reinterpret_cast<const float4 *>(row + (ii < p1 ? ii : 0));
    }

  // Threshold bin B1 of the first digit and the count above it, computed by
  // every block of the row alike; the first block publishes it for the finish.
#pragma unroll
  for (int i = 0; i < TOPK_BINS / LONG_THREADS; ++i) h[t + i * LONG_THREADS] = hv[i];
  __syncthreads();
  find_rank_bin<LONG_THREADS, TOPK_BINS>(h, k, sm, res);
  const uint32_t b1 = (uint32_t)res[0];
  if (c == 0 && t == 0) a.ws.b1info[q] = make_uint2((uint32_t)res[0], (uint32_t)res[1]);

  // Candidates in position order.
  uint2 *lst = a.ws.cand + (((int64_t)q * nblk + c) * TOPK_LONG_WAVES + wave) * TOPK_WAVE_SPAN;
  int wc = 0;  // wave-uniform
#pragma unroll
  for (int u = 0; u < LONG_ROUNDS; ++u) {
    const int i0 = p0 + 512 * u + 8 * lane;
    const float v[8] = {f[u][0].x, f[u][0].y, f[u][0].z, f[u][0].w, f[u][1].x, f[u][1].y, f[u][1].z, f[u][1].w};
    uint32_t key[8];
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      key[j] = (i0 + j < p1) ? order_key(v[j]) : 0u;
      cnt += ((key[j] >> 21) >= b1) ? 1 : 0;
    }
    int tot;
    int pos = wc + wave_excl_small(cnt, tot);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if ((key[j] >> 21) >= b1) lst[pos++] = make_uint2(key[j], (uint32_t)(i0 + j));
    wc += tot;
  }
  if (lane == 0) a.ws.wcnt[((int64_t)q * nblk + c) * TOPK_LONG_WAVES + wave] = (uint32_t)wc;
}

__global__ __launch_bounds__(LONG_THREADS) void topk_finish_kernel(SelectArgs a) {
  const int nblk = a.ws.nblk;
  const int q = blockIdx.x;
  const int n = a.q_nvis[q];
  const int k = a.k;
  if (n <= TOPK_ROW_MAX) return;  // topk_row_kernel
  const int nb = (n + TOPK_LONG_SPAN - 1) / TOPK_LONG_SPAN;
  __shared__ uint32_t h[TOPK_BINS];
  __shared__ int sm[LONG_THREADS / WAVE];
  __shared__ int res[2];
  __shared__ uint2 tl[TAIL_CAP];
  __shared__ int off[TOPK_MAX_CHUNKS / 2 * TOPK_LONG_WAVES + 1];
  const int t = threadIdx.x;

  // Everything that does not depend on anything else is requested at once.
  const uint2 bi = a.ws.b1info[q];
  const uint32_t b1 = bi.x;
  const int r = k - (int)bi.y;
  const int nseg = nb * TOPK_LONG_WAVES;  // lists in position order: (block, wavefront)
  zero_lds<LONG_THREADS>(h, TOPK_BINS);
  const uint32_t *gw = a.ws.wcnt + (int64_t)q * nblk * TOPK_LONG_WAVES;
  {
    static_assert(TOPK_MAX_CHUNKS / 2 * TOPK_LONG_WAVES <= LONG_THREADS, "one list count per thread");
    int tot;
    const int ex = block_exclusive_scan<LONG_THREADS>(t < nseg ? (int)gw[t] : 0, sm, tot);
    if (t < nseg) off[t] = ex;
    if (t == 0) off[nseg] = tot;
  }
  __syncthreads();
  const int ntot = off[nseg];
  const uint2 *cq = a.ws.cand + (int64_t)q * nblk * TOPK_LONG_SPAN;
  const bool in_lds = ntot <= TAIL_CAP;
  // Candidate i lives in list s (off[s] <= i < off[s+1]) at index i - off[s].
  auto locate = [&](int i) {
    int lo = 0, hi = nseg;  // largest s with off[s] <= i
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (off[mid] <= i) lo = mid; else hi = mid;
    }
    return cq[(int64_t)lo * TOPK_WAVE_SPAN + (i - off[lo])];
  };
  if (in_lds)
    for (int i = t; i < ntot; i += LONG_THREADS) tl[i] = locate(i);
  __syncthreads();
  auto get = [&](int i) { return in_lds ? tl[i] : locate(i); };
  // Digit 2: key[20:10] of the candidates in bin B1.
  for (int i = t; i < ntot; i += LONG_THREADS) {
    const uint32_t kk = get(i).x;
    if ((kk >> 21) == b1) atomicAdd(&h[(kk >> 10) & 2047u], 1u);
  }
  __syncthreads();
  find_rank_bin<LONG_THREADS, TOPK_BINS>(h, r, sm, res);
  const uint32_t pre = (b1 << 11) | (uint32_t)res[0];
  const int r2 = r - res[1];
  const int nbound = (int)h[res[0]];  // candidates with key[31:10] == pre
  const int per = (ntot + LONG_THREADS - 1) / LONG_THREADS;
  const int lo = min(ntot, per * t), hi = min(ntot, lo + per);
  int32_t *out = a.idx + (int64_t)q * k;
  int tot;
  if (in_lds && nbound <= WAVE) {
    // Few candidates share the boundary prefix (the usual case): one
    // wavefront ranks them by (key descending, position ascending) and marks
    // the chosen r2 in place (key all ones) and the rest (key 0), so the
    // output below is a single comparison against the prefix.
    __shared__ int nb_cnt;
    __shared__ int bidx[WAVE];
    if (t == 0) nb_cnt = 0;
    __syncthreads();
    for (int i = t; i < ntot; i += LONG_THREADS)
      if ((tl[i].x >> 10) == pre) bidx[atomicAdd(&nb_cnt, 1)] = i;
    __syncthreads();
    if (t < WAVE) {
      const bool have = t < nbound;
      const uint2 me = have ? tl[bidx[t]] : make_uint2(0u, 0u);
      int rank = 0;
      for (int j = 0; j < nbound; ++j) {
        const uint2 o = tl[bidx[j]];
        rank += (o.x > me.x || (o.x == me.x && o.y < me.y)) ? 1 : 0;
      }
      // every lane has read every boundary entry before any is overwritten
      __builtin_amdgcn_wave_barrier();
      if (have) tl[bidx[t]].x = rank < r2 ? 0xFFFFFFFFu : 0u;
    }
    __syncthreads();
    // Output in position order: key[31:10] > pre (the marked boundary keys included).
    int my_sel = 0;
    for (int i = lo; i < hi; ++i) my_sel += ((tl[i].x >> 10) > pre) ? 1 : 0;
    int pos = block_exclusive_scan<LONG_THREADS>(my_sel, sm, tot);
    for (int i = lo; i < hi; ++i) {
      const uint2 e = tl[i];
      if ((e.x >> 10) > pre) {
        if (pos < k) out[pos] = (int32_t)e.y;
        ++pos;
      }
    }
  } else {
    __syncthreads();
    zero_lds<LONG_THREADS>(h, 1024);
    __syncthreads();
    // Digit 3 over the candidates with key[31:10] == pre; contiguous runs per thread.
    for (int i = lo; i < hi; ++i) {
      const uint32_t kk = get(i).x;
      if ((kk >> 10) == pre) atomicAdd(&h[kk & 1023u], 1u);
    }
    __syncthreads();
    find_rank_bin<LONG_THREADS, 1024>(h, r2, sm, res);
    const uint32_t kth = (pre << 10) | (uint32_t)res[0];
    const int ties = r2 - res[1];
    // Output in position order: keys > kth and the first `ties` keys == kth.
    int my_ties = 0;
    for (int i = lo; i < hi; ++i) my_ties += (get(i).x == kth) ? 1 : 0;
    const int tie_rank = block_exclusive_scan<LONG_THREADS>(my_ties, sm, tot);
    int my_sel = 0;
    for (int i = lo, tr = tie_rank; i < hi; ++i) {
      const uint32_t kk = get(i).x;
      if (kk > kth || (kk == kth && tr < ties)) ++my_sel;
      tr += (kk == kth) ? 1 : 0;
    }
    int pos = block_exclusive_scan<LONG_THREADS>(my_sel, sm, tot);
    for (int i = lo, tr = tie_rank; i < hi; ++i) {
      const uint2 e = get(i);
      if (e.x > kth || (e.x == kth && tr < ties)) {
        if (pos < k) out[pos] = (int32_t)e.y;
        ++pos;
      }
      tr += (e.x == kth) ? 1 : 0;
    }
  }
  for (int i = tot + t; i < k; i += LONG_THREADS) out[i] = -1;  // defensive: tot == k
  if (t == 0 && a.count) a.count[q] = min(tot, k);
}

hipError_t launch_topk_init(const TopkWs &ws, int num_q, hipStream_t st) {
  const int64_t n = (int64_t)num_q * TOPK_BINS;
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
  if (ws.nblk == 0 || max_nvis <= TOPK_ROW_MAX) {  // every row fits one row block
    hipLaunchKernelGGL(topk_row_kernel, dim3((unsigned)num_q), dim3(TK_THREADS), 0, st, a);
    return hipGetLastError();
  }
  // Some row is long: the long kernel finds each long row's threshold bin and
  // candidates, and selects each short row with its first block; the finish
  // kernel completes the long rows.
  const int64_t blocks = (int64_t)num_q * ws.nblk;
  hipLaunchKernelGGL(topk_long_kernel, dim3((unsigned)blocks), dim3(LONG_THREADS), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_finish_kernel, dim3((unsigned)num_q), dim3(LONG_THREADS), 0, st, a);
  return hipGetLastError();
}

}  // namespace dsa
