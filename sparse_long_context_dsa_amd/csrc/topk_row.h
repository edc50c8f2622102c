// One-block radix selection of a row of at most TOPK_ROW_MAX fp32 scores
// (the top-k of page "arXiv'25 | DSA ... DeepSeek-V3.2", section 3, second
// equation; ties to the lower position, -0 == +0, output ascending and padded
// with -1): shared by the top-k kernels and by the indexer, which selects a
// row it has scored whole without writing its scores out.
//
// Radix select on order-preserving 32-bit keys with digits of 11 / 11 / 10
// bits: each digit is an LDS histogram and a search for the bin holding the
// r-th largest key; the output is a position-ordered compaction built from
// block-wide exclusive scans.  A block of NT threads holds the row in
// registers: ROUNDS rounds of TK_J consecutive scores per thread.
#pragma once

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
// ------------------------------------------------------------------ helpers
// Exclusive scan over the block of one value per thread; `total` gets the sum.
template <int NT, typename T>
__device__ __forceinline__ T block_exclusive_scan(T v, T *sm, T &total) {
  constexpr int W = NT / WAVE;
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const T inc = wave_inclusive_scan(v);
  if (lane == WAVE - 1) sm[wave] = inc;
  lds_barrier();
  T before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const T s = sm[w];
    before += (w < wave) ? s : T(0);
    tot += s;
  }
  lds_barrier();
  total = tot;
  return before + inc - v;
}

// Words of the block's small result slot `res` (find_rank_bin's answer and
// the boundary-key counter of select_row).
constexpr int TOPK_RES_WORDS = 4;

// Given an LDS histogram h[NB] and a rank r >= 1 counted from the top, finds
// the bin B with above(B) < r <= above(B) + h[B] (above(B) = sum of h[b > B]).
// res[0] = B, res[1] = above(B), res[2] = h[B], visible to all threads on
// return (so that h may be reused at once).  Returns
// the histogram's total (the same in every thread), which tells a caller
// whether the histogram holds what it expects.
template <int NT, int NB>
__device__ int find_rank_bin(const uint32_t *h, int r, int *sm, int *res) {
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
      res[2] = c;
    }
    acc += c;
  }
  lds_barrier();
  return total;
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
  uint64_t t0, t1 = 0, e1 = 0;
  const uint64_t e0 = block_exclusive_scan<NT>(cnt.w0, sm64, t0);
  if constexpr (RowShape<NT>::ROUNDS > PackShape<NT>::PER_WORD) e1 = block_exclusive_scan<NT>(cnt.w1, sm64, t1);
  const Packed ex{e0, e1}, tot{t0, t1};
  int before = 0;
#pragma unroll
  for (int rr = 0; rr < RowShape<NT>::ROUNDS; ++rr) {
    off[rr] = before + pack_get<NT>(ex, rr);
    before += pack_get<NT>(tot, rr);
  }
  return before;
}

// Rank of lane l's (key, position) among lanes 0 .. nb - 1 of the
// wavefront (nb <= WAVE, wave-uniform): how many have a larger key, or the
// same key at a lower position.  The other lanes' entries are read with
// v_readlane (a uniform lane index), not through LDS.
__device__ __forceinline__ int boundary_rank(uint32_t mk, uint32_t mp, int nb) {
  int rank = 0;
  for (int j = 0; j < nb; ++j) {
    const uint32_t ok = (uint32_t)__builtin_amdgcn_readlane((int)mk, j);
    const uint32_t op = (uint32_t)__builtin_amdgcn_readlane((int)mp, j);
    rank += (ok > mk || (ok == mk && op < mp)) ? 1 : 0;
  }
  return rank;
}

__device__ __forceinline__ void write_short(int32_t *out, int32_t *count, int q, int n, int k, int nt) {
  for (int i = threadIdx.x; i < k; i += nt) out[i] = (i < n) ? i : -1;
  if (threadIdx.x == 0 && count) count[q] = n;
}

// Where select_row finds the first digit's histogram.
enum HistSource { HIST_BUILD = 0, HIST_GLOBAL = 1, HIST_LDS = 2 };

// Selects one row of n <= TOPK_ROW_MAX scores (row[0 .. n), global memory or
// LDS) with one block of NT threads: digit 1 from a histogram (built here with
// LDS atomics, copied from `gh` in global memory, or already in `h`), digits 2
// and 3 as LDS histograms of the keys in the threshold bins, then the
// position-ordered compaction into out[0 .. k) and *count_out (if non-null).
// A histogram from `gh` is left cleared for the next call, and checked: if its
// bins do not sum to n (it held more than this call's counts), digit 1 is
// built from the keys instead.  Every thread of the block calls it (it has
// block barriers, for LDS only).
template <int NT>
__device__ __forceinline__ void select_row(const float *row, const int n, const int k, const int hist_src, uint32_t *gh,
                           uint32_t *h, int *sm, uint64_t *sm64, int *res, int32_t *out, int32_t *count_out) {
  using RS = RowShape<NT>;
  const int t = threadIdx.x;
  if (n <= k) {
    for (int i = t; i < k; i += NT) out[i] = (i < n) ? i : -1;
    if (t == 0 && count_out) *count_out = n;
    return;
  }
  uint32_t key[RS::PER];
  load_keys<NT>(row, 0, n, key);
  if (t == 0) res[3] = 0;  // boundary keys collected (below)
  // Digit 1: key[31:21].  Padding slots are not counted: their keys would all
  // go to bin 0, one LDS address, where a wavefront's atomics serialise (a row
  // of 4096 in 16384 slots took about 12 us more), and they rank below every
  // real key anyway.
  auto build = [&] {
    zero_lds<NT>(h, TOPK_BINS);
    lds_barrier();
#pragma unroll
    for (int rr = 0; rr < RS::ROUNDS; ++rr)
#pragma unroll
      for (int j = 0; j < TK_J; ++j)
        if (slot_pos<NT>(t, rr, j) < n) atomicAdd(&h[key[TK_J * rr + j] >> 21], 1u);
    lds_barrier();
  };
  if (hist_src == HIST_GLOBAL) {
    for (int b = t; b < TOPK_BINS; b += NT) {
      h[b] = gh[b];
      gh[b] = 0u;  // each thread clears the bins it read
    }
    lds_barrier();
  } else if (hist_src == HIST_BUILD) {
    build();
  } else {
    lds_barrier();
  }
  // A histogram from memory that does not sum to n (it held more than this
  // call's counts) is rebuilt from the keys (block-uniform).
  if (find_rank_bin<NT, TOPK_BINS>(h, k, sm, res) != n && hist_src == HIST_GLOBAL) {
    build();
    find_rank_bin<NT, TOPK_BINS>(h, k, sm, res);
  }
  const uint32_t b1 = (uint32_t)res[0];
  const int r = k - res[1];
  lds_barrier();
  // Digit 2: key[20:10] of the keys in bin B1.
  zero_lds<NT>(h, TOPK_BINS);
  lds_barrier();
#pragma unroll
  for (int rr = 0; rr < RS::ROUNDS; ++rr)
#pragma unroll
    for (int j = 0; j < TK_J; ++j) {
      const uint32_t kk = key[TK_J * rr + j];
      if ((kk >> 21) == b1) atomicAdd(&h[(kk >> 10) & 2047u], 1u);
    }
  lds_barrier();
  find_rank_bin<NT, TOPK_BINS>(h, r, sm, res);
  const uint32_t pre = (b1 << 11) | (uint32_t)res[0];
  const int r2 = r - res[1];
  const int nbound = res[2];  // keys with key[31:10] == pre
  uint32_t kth;
  int ties, tie_total;
  if (nbound <= WAVE) {  // block-uniform
    // Few keys share the boundary prefix (the usual case): they are gathered
    // into h (free: find_rank_bin has left its answer in res) and one
    // wavefront ranks them by (key descending, position ascending); the
    // r2-th is the k-th key.  No third digit.
#pragma unroll
    for (int rr = 0; rr < RS::ROUNDS; ++rr)
#pragma unroll
      for (int j = 0; j < TK_J; ++j)
        if ((key[TK_J * rr + j] >> 10) == pre) {
          const int sl = atomicAdd(&res[3], 1);
          h[sl] = key[TK_J * rr + j];
          h[WAVE + sl] = (uint32_t)slot_pos<NT>(t, rr, j);
        }
    lds_barrier();
    if (t < WAVE) {
      const bool have = t < nbound;
      const uint32_t mk = have ? h[t] : 0u, mp = have ? h[WAVE + t] : 0u;
      const int rank = boundary_rank(mk, mp, nbound);
      const uint64_t at = __ballot(have && rank == r2 - 1);
      const uint32_t kv = (uint32_t)__builtin_amdgcn_readlane((int)mk, (int)__builtin_ctzll(at));
      const int gt = (int)__popcll(__ballot(have && mk > kv));
      const int eq = (int)__popcll(__ballot(have && mk == kv));
      if (t == 0) {
        res[0] = (int)kv;
        res[1] = gt;
        res[2] = eq;
      }
    }
    lds_barrier();
    kth = (uint32_t)res[0];
    ties = r2 - res[1];
    tie_total = res[2];
  } else {
    lds_barrier();
    // Digit 3: key[9:0] of the keys with key[31:10] == pre.
    zero_lds<NT>(h, 1024);
    lds_barrier();
#pragma unroll
    for (int rr = 0; rr < RS::ROUNDS; ++rr)
#pragma unroll
      for (int j = 0; j < TK_J; ++j) {
        const uint32_t kk = key[TK_J * rr + j];
        if ((kk >> 10) == pre) atomicAdd(&h[kk & 1023u], 1u);
      }
    lds_barrier();
    find_rank_bin<NT, 1024>(h, r2, sm, res);
    kth = (pre << 10) | (uint32_t)res[0];
    ties = r2 - res[1];
    tie_total = res[2];
  }
  // Emit in position order: keys > kth, and the first `ties` keys == kth.
  // Usually every key equal to the k-th is taken (no tie is split), and the
  // tie ranks, with their block scan, are not needed.
  const bool all_ties = ties >= tie_total;  // block-uniform
  int toff[RS::ROUNDS];
#pragma unroll
  for (int rr = 0; rr < RS::ROUNDS; ++rr) toff[rr] = 0;
  if (!all_ties) {
    Packed tc{0, 0};
#pragma unroll
    for (int rr = 0; rr < RS::ROUNDS; ++rr) {
      int c = 0;
#pragma unroll
      for (int j = 0; j < TK_J; ++j) c += (key[TK_J * rr + j] == kth) ? 1 : 0;
      pack_add<NT>(tc, rr, c);
    }
    ordered_offsets<NT>(tc, sm64, toff);
  }
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
      const bool sel = kk > kth || (tie && (all_ties || tr < ties));
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
  if (t == 0 && count_out) *count_out = min(tot, k);
}


}  // namespace dsa
