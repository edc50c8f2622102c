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
//    rows are selected per CU at once.  Batches of at most 256 rows take
//    topk_row_wide_kernel instead, the same select with 1024 threads per row.  The first-digit histogram comes from
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
#include "topk_finish.h"

namespace dsa {

constexpr int LONG_THREADS = TOPK_LONG_WAVES * WAVE;
constexpr int LONG_ROUNDS = TOPK_WAVE_SPAN / 512;  // rounds of 512 positions per wavefront
constexpr int TAIL_CAP = 12288;                     // candidates the finishing block keeps in LDS
constexpr int FINISH_THREADS = 1024;                // threads of the finishing block (512: top-k stage
                                                    // 0.5 us slower at 64 x 131072; 256: 4 us slower)
constexpr int TOPK_ROW_WIDE_MAX_Q = 256;            // up to one row per CU: 1024-thread row blocks
static_assert(TOPK_CHUNK == TOPK_ROW_MAX, "one histogram block covers one chunk");

static inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

static inline int topk_nchunks(int max_nvis) {
  return max_nvis <= TOPK_ROW_MAX ? 0 : (max_nvis + TOPK_CHUNK - 1) / TOPK_CHUNK;
}
// Blocks per row of the two-kernel path; 0 selects the streaming kernel (one
// block per row).  A row streams through one CU at only about 25 GB/s (its
// scores mostly come from HBM), against about 21 GB/s per CU but four CUs per
// row in the two-kernel path, which pays a second launch and a finishing
// pass.  Measured on this part: 16 rows of 32768 (19 us) and a ragged batch
// of 128 rows up to 131072 (33 against 48 us) favour streaming; 64 rows of
// 131072, whose four blocks per row just fill the 256 CUs, favour the two
// kernels (30 against 34 us).  Hence: streaming up to 32 rows and from 128 rows.
static inline int topk_nblk(int num_q, int max_nvis) {
  if (max_nvis <= TOPK_ROW_MAX || (max_nvis <= TOPK_STREAM_MAX && (num_q <= 32 || num_q >= 128))) return 0;
  return (max_nvis + TOPK_LONG_SPAN - 1) / TOPK_LONG_SPAN;
}

size_t topk_ws_bytes(int num_q, int max_nvis) {
  const size_t nq = (size_t)num_q, nb = (size_t)topk_nblk(num_q, max_nvis);
  return align256(nq * TOPK_BINS * 4) + align256(nq * sizeof(uint2)) +
         align256(nq * nb * TOPK_LONG_WAVES * 4) + align256(nq * nb * TOPK_BINS * 4) +
         nq * nb * TOPK_LONG_SPAN * sizeof(uint2);
}

TopkWs topk_ws_carve(void *ws, int num_q, int max_nvis) {
  TopkWs w;
  const size_t nq = (size_t)num_q;
  w.nchunks = topk_nchunks(max_nvis);
  w.nblk = topk_nblk(num_q, max_nvis);
  uint8_t *p = static_cast<uint8_t *>(ws);
  w.hist = reinterpret_cast<uint32_t *>(p);  // [nq, 2048] first digit (left zero by its readers)
  p += align256(nq * TOPK_BINS * 4);
  w.b1info = reinterpret_cast<uint2 *>(p);   // [nq] written before it is read
  p += align256(nq * sizeof(uint2));
  w.wcnt = reinterpret_cast<uint32_t *>(p);
  p += align256(nq * w.nblk * TOPK_LONG_WAVES * 4);
  w.hist2 = reinterpret_cast<uint32_t *>(p);
  p += align256(nq * w.nblk * TOPK_BINS * 4);
  w.cand = reinterpret_cast<uint2 *>(p);
  return w;
}

// ------------------------------------------------------------------ kernels
// Clears one row's first-digit histogram per block (TOPK_BINS words: 256
// threads x two 16-byte stores).
__global__ __launch_bounds__(256) void topk_zero_kernel(uint32_t *p) {
  uint4 *r = reinterpret_cast<uint4 *>(p + (int64_t)blockIdx.x * TOPK_BINS);
  static_assert(TOPK_BINS == 256 * 8, "two uint4 per thread");
  r[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
  r[threadIdx.x + 256] = make_uint4(0u, 0u, 0u, 0u);
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

// Selects row q (n <= TOPK_ROW_MAX scores) with one block of NT threads,
// digit 1 from the indexer's histogram when it built one.
template <int NT>
__device__ void row_select(const SelectArgs &a, const int q, const int n, uint32_t *h, int *sm, uint64_t *sm64,
                           int *res) {
  select_row<NT>(a.scores + (int64_t)q * a.ld, (int)min((int64_t)n, a.ld), a.k,  // never past the row's ld
                 a.hist1_valid ? HIST_GLOBAL : HIST_BUILD, a.ws.hist + (int64_t)q * TOPK_BINS, h, sm, sm64, res,
                 a.idx + (int64_t)q * a.k, a.count ? a.count + q : nullptr);
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
  __shared__ int res[TOPK_RES_WORDS];
  row_select<TK_THREADS>(a, blockIdx.x, a.q_nvis[blockIdx.x], h, sm, sm64, res);
}

// The same selection with 1024 threads per row (16 keys per thread instead of
// 64), for batches of at most as many rows as CUs, where each row has a CU to
// itself anyway and the select's chain of passes sets the time.
__global__ __launch_bounds__(LONG_THREADS) void topk_row_wide_kernel(SelectArgs a) {
  __shared__ uint32_t h[TOPK_BINS];
  __shared__ int sm[LONG_THREADS / WAVE];
  __shared__ uint64_t sm64[LONG_THREADS / WAVE];
  __shared__ int res[TOPK_RES_WORDS];
  row_select<LONG_THREADS>(a, blockIdx.x, a.q_nvis[blockIdx.x], h, sm, sm64, res);
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

// ---------------------------------------------------------------- streaming
// One 1024-thread block per row of up to TOPK_STREAM_MAX positions.  The
// row's first-digit histogram (built with the scores) gives the threshold bin
// B1 and the count above it before the block reads a score.  Wavefront w then
// streams its 1/16 of the row, ST_D rounds of 512 scores in flight, and keeps
// the candidates (digit 1 >= B1: the k largest and the rest of bin B1, about
// k + |B1| keys) as (key, position) pairs in LDS, each wavefront reserving
// its slots with one LDS atomic per round.  Digits 2 and 3 are LDS
// histograms over the candidates; the chosen positions (and, separately,
// the keys equal to the k-th) are marked in position bitmaps, the lowest
// positions among the ties are kept, and block scans over the bitmap words
// emit the positions in ascending order.  If more candidates arrive than LDS
// holds, the digit passes re-read the row instead (same result, slower).
constexpr int ST_THREADS = 1024;
constexpr int ST_WAVES = ST_THREADS / WAVE;                          // 16
constexpr int ST_ROUNDS = TOPK_STREAM_MAX / (ST_WAVES * 512);        // 16 rounds of 512 per wavefront
constexpr int ST_D = 4;                                              // rounds in flight per wavefront
constexpr int ST_CAP = 12288;                                        // candidates kept in LDS
constexpr int ST_WORDS = TOPK_STREAM_MAX / 32;                       // position bitmap words
constexpr int ST_WORDS_PER_THREAD = ST_WORDS / ST_THREADS;           // 4
static_assert(ST_WORDS_PER_THREAD * ST_THREADS == ST_WORDS && ST_ROUNDS * ST_WAVES * 512 == TOPK_STREAM_MAX,
              "whole rounds and bitmap words");

// The first-digit histogram of row[0 .. n) built in LDS with one pass over
// the scores: used when the histogram from the indexer does not sum to n (the
// workspace held other data before the call).
template <int NT>
__device__ void rebuild_first_digit(const float *row, const int n, uint32_t *h) {
  __syncthreads();
  zero_lds<NT>(h, TOPK_BINS);
  __syncthreads();
  for (int i = 4 * (int)threadIdx.x; i < n; i += 4 * NT) {  // i + 3 < ld: ld is a multiple of 4
    const float4 x = *reinterpret_cast<const float4 *>(row + i);
    const float xv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (i + e < n) atomicAdd(&h[order_key(xv[e]) >> 21], 1u);
  }
}

__global__ __launch_bounds__(ST_THREADS) void topk_stream_kernel(SelectArgs a) {
  const int q = blockIdx.x;
  const int n = a.q_nvis[q];
  const int k = a.k;
  const int t = threadIdx.x;
  __shared__ uint32_t h[TOPK_BINS];
  __shared__ int sm[ST_WAVES];
  __shared__ uint64_t sm64[ST_WAVES];
  __shared__ int res[TOPK_RES_WORDS];
  __shared__ uint32_t ck[ST_CAP];    // candidate keys
  __shared__ uint32_t cpos[ST_CAP];  // candidate positions
  __shared__ uint32_t bm[ST_WORDS];  // selected positions
  __shared__ uint32_t tbm[ST_WORDS]; // positions whose key equals the k-th
  __shared__ int ncand;
  __shared__ int bidx[WAVE];         // boundary candidates ranked directly
  __shared__ int nbnd;
  int32_t *out = a.idx + (int64_t)q * k;
  const float *row = a.scores + (int64_t)q * a.ld;
  uint32_t *gh = a.ws.hist + (int64_t)q * TOPK_BINS;
  if (n <= TOPK_ROW_MAX) {  // fits the registers of the block: one-block radix select (block-uniform)
    select_row<ST_THREADS>(row, (int)min((int64_t)n, a.ld), k, a.hist1_valid ? HIST_GLOBAL : HIST_BUILD, gh, h, sm,
                           sm64, res, out, a.count ? a.count + q : nullptr);
    return;
  }
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & (WAVE - 1);
  const int span = ((n + ST_WAVES - 1) / ST_WAVES + 511) / 512 * 512;
  const int p0 = wave * span, p1 = min(n, p0 + span);
  const int rounds = p1 > p0 ? (p1 - p0 + 511) / 512 : 0;  // wave-uniform

  // The histogram is requested before the scores: loads complete in issue
  // order, so the wait for it does not wait for them.
  uint32_t hv[TOPK_BINS / ST_THREADS];
#pragma unroll
  for (int i = 0; i < TOPK_BINS / ST_THREADS; ++i) hv[i] = gh[t + i * ST_THREADS];
  // Every lane issues the same loads for every round (positions past the
  // wavefront's end read position 0 of the row), so the waits stay exact; a
  // float4 at a position < p1 stays inside the row (ld % 4 == 0).
  float4 f[ST_D + 1][2];
  auto load_round = [&](const int u, float4 *dst) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int ii = p0 + 512 * u + 8 * lane + 4 * hh;
      dst[hh] = *reinterpret_cast<const float4 *>(row + (ii < p1 ? ii : 0));
    }
  };
#pragma unroll
  for (int u = 0; u < ST_D; ++u) load_round(u, f[u]);
#pragma unroll
  for (int i = 0; i < TOPK_BINS / ST_THREADS; ++i) h[t + i * ST_THREADS] = hv[i];
  if (t == 0) ncand = 0;
  __syncthreads();
  if (find_rank_bin<ST_THREADS, TOPK_BINS>(h, k, sm, res) != n) {  // block-uniform: not only this call's counts
    rebuild_first_digit<ST_THREADS>(row, n, h);
    __syncthreads();
    find_rank_bin<ST_THREADS, TOPK_BINS>(h, k, sm, res);
  }
  const uint32_t b1 = (uint32_t)res[0];
  const int r = k - res[1];

#pragma unroll
  for (int u = 0; u < ST_ROUNDS; ++u) {
    if (u + ST_D < ST_ROUNDS) load_round(u + ST_D, f[(u + ST_D) % (ST_D + 1)]);
    if (u < rounds) {  // wave-uniform
      const float4 *fb = f[u % (ST_D + 1)];
      const float v[8] = {fb[0].x, fb[0].y, fb[0].z, fb[0].w, fb[1].x, fb[1].y, fb[1].z, fb[1].w};
      const int i0 = p0 + 512 * u + 8 * lane;
      uint32_t key[8];
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        key[j] = (i0 + j < p1) ? order_key(v[j]) : 0u;  // 0: below any real key's bin
        cnt += ((key[j] >> 21) >= b1) ? 1 : 0;
      }
      int tot;
      const int ex = wave_excl_small(cnt, tot);
      if (tot > 0) {  // wave-uniform
        int base = 0;
        if (lane == 0) base = atomicAdd(&ncand, tot);
        base = __builtin_amdgcn_readfirstlane(base);
        int pos = base + ex;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if ((key[j] >> 21) >= b1) {
            if (pos < ST_CAP) {
              ck[pos] = key[j];
              cpos[pos] = (uint32_t)(i0 + j);
            }
            ++pos;
          }
      }
    }
  }
  __syncthreads();
  const int ntot = ncand;
  const bool over = ntot > ST_CAP;  // block-uniform

  // Applies f(key, position) to every candidate: from LDS, or, when LDS
  // overflowed, to every key of the row with digit 1 >= B1, re-read.
  auto for_each = [&](auto &&fn) {
    if (!over) {
      for (int i = t; i < ntot; i += ST_THREADS) fn(ck[i], cpos[i]);
    } else {
      for (int i = 4 * t; i < n; i += 4 * ST_THREADS) {
        const float4 x = *reinterpret_cast<const float4 *>(row + i);
        const float xv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t kk = order_key(xv[e]);
          if (i + e < n && (kk >> 21) >= b1) fn(kk, (uint32_t)(i + e));
        }
      }
    }
  };

  // Digit 2: key[20:10] of the candidates in bin B1.
  zero_lds<ST_THREADS>(h, TOPK_BINS);
  __syncthreads();
  for_each([&](uint32_t kk, uint32_t) {
    if ((kk >> 21) == b1) atomicAdd(&h[(kk >> 10) & 2047u], 1u);
  });
  __syncthreads();
  find_rank_bin<ST_THREADS, TOPK_BINS>(h, r, sm, res);
  const uint32_t pre = (b1 << 11) | (uint32_t)res[0];
  const int r2 = r - res[1];
  const int nbound = (int)h[res[0]];  // candidates with key[31:10] == pre
  // Thread t owns bitmap words [4t, 4t + 4), positions [128t, 128t + 128):
  // thread order is position order.  w: the chosen keys equal to the k-th.
  uint32_t w[ST_WORDS_PER_THREAD];
  if (!over && nbound <= WAVE) {  // block-uniform
    // Few candidates share the boundary prefix (the usual case): one
    // wavefront ranks them by (key descending, position ascending) and marks
    // the chosen r2, so neither the third digit nor a tie bitmap is needed.
#pragma unroll
    for (int i = 0; i < ST_WORDS_PER_THREAD; ++i) {
      bm[t * ST_WORDS_PER_THREAD + i] = 0u;
      w[i] = 0u;
    }
    if (t == 0) nbnd = 0;
    __syncthreads();
    for (int i = t; i < ntot; i += ST_THREADS) {
      const uint32_t kk = ck[i] >> 10, p = cpos[i];
      if (kk > pre) atomicOr(&bm[p >> 5], 1u << (p & 31));
      else if (kk == pre) bidx[atomicAdd(&nbnd, 1)] = i;
    }
    __syncthreads();
    if (t < WAVE) {
      const bool have = t < nbound;
      const uint32_t mk = have ? ck[bidx[t]] : 0u, mp = have ? cpos[bidx[t]] : 0u;
      const int rank = boundary_rank(mk, mp, nbound);
      if (have && rank < r2) atomicOr(&bm[mp >> 5], 1u << (mp & 31));
    }
    __syncthreads();
  } else {
    __syncthreads();
    // Digit 3: key[9:0] of the candidates with key[31:10] == pre.
    zero_lds<ST_THREADS>(h, 1024);
    __syncthreads();
    for_each([&](uint32_t kk, uint32_t) {
      if ((kk >> 10) == pre) atomicAdd(&h[kk & 1023u], 1u);
    });
    __syncthreads();
    find_rank_bin<ST_THREADS, 1024>(h, r2, sm, res);
    const uint32_t kth = (pre << 10) | (uint32_t)res[0];
    const int ties = r2 - res[1];
    const int tie_total = (int)h[res[0]];
    // Mark keys above the k-th, and keys equal to it, in position bitmaps.
#pragma unroll
    for (int i = 0; i < ST_WORDS_PER_THREAD; ++i) {
      bm[t * ST_WORDS_PER_THREAD + i] = 0u;
      tbm[t * ST_WORDS_PER_THREAD + i] = 0u;
    }
    __syncthreads();
    for_each([&](uint32_t kk, uint32_t p) {
      if (kk > kth) atomicOr(&bm[p >> 5], 1u << (p & 31));
      else if (kk == kth) atomicOr(&tbm[p >> 5], 1u << (p & 31));
    });
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ST_WORDS_PER_THREAD; ++i) w[i] = tbm[t * ST_WORDS_PER_THREAD + i];
    if (ties < tie_total) {  // block-uniform: only the `ties` lowest positions among the ties
      int c = 0;
#pragma unroll
      for (int i = 0; i < ST_WORDS_PER_THREAD; ++i) c += __popc(w[i]);
      int tt;
      int rank = block_exclusive_scan<ST_THREADS>(c, sm, tt);
#pragma unroll
      for (int i = 0; i < ST_WORDS_PER_THREAD; ++i) {
        uint32_t m = w[i], keep = 0u;
        while (m) {
          const uint32_t bit = m & (0u - m);
          if (rank < ties) keep |= bit;
          ++rank;
          m ^= bit;
        }
        w[i] = keep;
      }
    }
  }
  int c = 0;
#pragma unroll
  for (int i = 0; i < ST_WORDS_PER_THREAD; ++i) {
    w[i] |= bm[t * ST_WORDS_PER_THREAD + i];
    c += __popc(w[i]);
  }
  int tot;
  int pos = block_exclusive_scan<ST_THREADS>(c, sm, tot);
#pragma unroll
  for (int i = 0; i < ST_WORDS_PER_THREAD; ++i) {
    uint32_t m = w[i];
    while (m) {
      const int b = __ffs(m) - 1;
      if (pos < k) out[pos] = 32 * (t * ST_WORDS_PER_THREAD + i) + b;
      ++pos;
      m &= m - 1;
    }
  }
  for (int i = tot + t; i < k; i += ST_THREADS) out[i] = -1;  // defensive: tot == k
  if (t == 0 && a.count) a.count[q] = min(tot, k);
  // The row's first-digit histogram, cleared for the next call.  Stored last:
  // a store issued before the score loads would hold up every wait on them
  // (the memory counter counts stores and loads together, in issue order).
#pragma unroll
  for (int i = 0; i < TOPK_BINS / ST_THREADS; ++i) gh[t + i * ST_THREADS] = 0u;
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
  __shared__ int res[TOPK_RES_WORDS];
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
  // A histogram that does not sum to n (the workspace held other data) is
  // rebuilt by every block of the row from the whole row, alike.
#pragma unroll
  for (int i = 0; i < TOPK_BINS / LONG_THREADS; ++i) h[t + i * LONG_THREADS] = hv[i];
  __syncthreads();
  if (find_rank_bin<LONG_THREADS, TOPK_BINS>(h, k, sm, res) != n) {  // block-uniform
    rebuild_first_digit<LONG_THREADS>(row, n, h);
    __syncthreads();
    find_rank_bin<LONG_THREADS, TOPK_BINS>(h, k, sm, res);
  }
  const uint32_t b1 = (uint32_t)res[0];
  if (c == 0 && t == 0) a.ws.b1info[q] = make_uint2((uint32_t)res[0], (uint32_t)res[1]);
  // h turns into this span's histogram of the second digit over its keys in
  // bin B1 (find_rank_bin ends with a barrier: every thread is done with it).
  zero_lds<LONG_THREADS>(h, TOPK_BINS);
  __syncthreads();

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
      if ((key[j] >> 21) >= b1) {
        lst[pos++] = make_uint2(key[j], (uint32_t)(i0 + j));
        if ((key[j] >> 21) == b1) atomicAdd(&h[(key[j] >> 10) & 2047u], 1u);
      }
    wc += tot;
  }
  if (lane == 0) a.ws.wcnt[((int64_t)q * nblk + c) * TOPK_LONG_WAVES + wave] = (uint32_t)wc;
  __syncthreads();
  uint32_t *h2 = a.ws.hist2 + ((int64_t)q * nblk + c) * TOPK_BINS;
#pragma unroll
  for (int i = 0; i < TOPK_BINS / LONG_THREADS; ++i) h2[t + i * LONG_THREADS] = h[t + i * LONG_THREADS];
}

__global__ __launch_bounds__(FINISH_THREADS) void topk_finish_kernel(SelectArgs a) {
  const int q = blockIdx.x;
  const int n = a.q_nvis[q];
  const int k = a.k;
  if (n <= TOPK_ROW_MAX) return;  // selected whole by topk_long_kernel
  __shared__ uint32_t h[TOPK_BINS];
  __shared__ int sm[FINISH_THREADS / WAVE];
  __shared__ int res[TOPK_RES_WORDS];
  __shared__ uint32_t ck[TAIL_CAP], cpos[TAIL_CAP];
  __shared__ int off[TOPK_MAX_LISTS + 1];
  __shared__ int bidx[WAVE];
  __shared__ int nb_cnt;
  const FinishLds s{ck, cpos, TAIL_CAP, h, off, sm, res, bidx, &nb_cnt};
  int32_t *out = a.idx + (int64_t)q * k;
  const int tot = finish_row<FINISH_THREADS>(a.ws, q, n, k, s, [] {}, [&](int o, uint32_t p) {
    if (o < k) out[o] = (int32_t)p;
  });
  for (int i = tot + threadIdx.x; i < k; i += FINISH_THREADS) out[i] = -1;  // defensive: tot == k
  if (threadIdx.x == 0 && a.count) a.count[q] = min(tot, k);
  // Every block of the long kernel has read this row's first-digit histogram:
  // clear it for the next call.  Stored last, so that no wait on the finish's
  // own loads waits for these stores (the memory counter counts both, in
  // issue order).
  for (int b = threadIdx.x; b < TOPK_BINS; b += FINISH_THREADS) a.ws.hist[(int64_t)q * TOPK_BINS + b] = 0u;
}

hipError_t launch_topk_init(const TopkWs &ws, int num_q, hipStream_t st) {
  if (num_q == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_zero_kernel, dim3((unsigned)num_q), dim3(256), 0, st, ws.hist);
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
  if (max_nvis <= TOPK_ROW_MAX) {  // every row fits one row block
    if (num_q <= TOPK_ROW_WIDE_MAX_Q)
      hipLaunchKernelGGL(topk_row_wide_kernel, dim3((unsigned)num_q), dim3(LONG_THREADS), 0, st, a);
    else
      hipLaunchKernelGGL(topk_row_kernel, dim3((unsigned)num_q), dim3(TK_THREADS), 0, st, a);
    return hipGetLastError();
  }
  if (ws.nblk == 0) {  // rows up to TOPK_STREAM_MAX: one streaming block per row
    hipLaunchKernelGGL(topk_stream_kernel, dim3((unsigned)num_q), dim3(ST_THREADS), 0, st, a);
    return hipGetLastError();
  }
  // Some row is long: the long kernel finds each long row's threshold bin and
  // candidates, and selects each short row with its first block; the finish
  // kernel completes the long rows.
  const int64_t blocks = (int64_t)num_q * ws.nblk;
  hipLaunchKernelGGL(topk_long_kernel, dim3((unsigned)blocks), dim3(LONG_THREADS), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_finish_kernel, dim3((unsigned)num_q), dim3(FINISH_THREADS), 0, st, a);
  return hipGetLastError();
}

}  // namespace dsa
