// The last step of the top-k of a long row (page "arXiv'25 | DSA ...
// DeepSeek-V3.2", section 3, second equation; ties to the lower position,
// output ascending): the row's candidates -- the keys whose first digit is at
// least the threshold bin B1, left by topk_long_kernel in per-wavefront lists
// in position order -- are ranked on their second and third digits and the
// chosen positions are handed to the caller in ascending order.  (Tried and
// dropped: finishing each row in the attention kernel's prologue instead of a
// launch of its own; with 256 threads the finish took about as long as the
// separate launch it saved.)
#pragma once

#include "topk_row.h"

namespace dsa {

constexpr int TOPK_MAX_LISTS = TOPK_MAX_CHUNKS / 2 * TOPK_LONG_WAVES;  // lists of a 2^20-position row

// LDS scratch of one row's finish (the caller's arrays).
struct FinishLds {
  uint32_t *ck;    // candidate keys, `cap` entries
  uint32_t *cpos;  // candidate positions, `cap` entries
  int cap;
  uint32_t *h;     // TOPK_BINS words
  int *off;        // TOPK_MAX_LISTS + 1 list offsets
  int *sm;         // NT / WAVE words of block-scan scratch
  int *res;        // 2 words
  int *bidx;       // WAVE words
  int *nb_cnt;     // 1 word
};

// Finishes row q (n > TOPK_ROW_MAX positions, k <= n) with one block of NT
// threads.  after_issue() runs once the first loads (counts, histograms and
// the first list entries) are in flight, so that a caller's own loads
// overlap them.
// emit(o, position) receives the o-th chosen position, o ascending; returns
// the count (k).  Every thread of the block calls it (it has block barriers).
template <int NT, typename AfterIssue, typename Emit>
__device__ int finish_row(const TopkWs &ws, const int q, const int n, const int k, const FinishLds &s,
                          AfterIssue &&after_issue, Emit &&emit) {
  constexpr int SEG = (TOPK_MAX_LISTS + NT - 1) / NT;  // lists per thread in the offset scan
  constexpr int BPT = TOPK_BINS / NT;                   // histogram bins per thread
  constexpr int NW = NT / WAVE;
  constexpr int LB = 16;                                // lists per wavefront per load batch
  constexpr int LB0 = (4 * TOPK_LONG_WAVES + NW - 1) / NW;  // lists per wavefront requested with the counts:
                                                              // NW * LB0 lists cover 2^17 positions
  constexpr int E0 = 2;    // their entries per lane requested then: a 2048-position list rarely holds more than 128
  const int t = threadIdx.x;
  const int lane = t & (WAVE - 1), wave = t / WAVE;
  const int nblk = ws.nblk;
  const int nb = (n + TOPK_LONG_SPAN - 1) / TOPK_LONG_SPAN;
  const int nseg = nb * TOPK_LONG_WAVES;  // lists in position order: (block, wavefront)
  const uint2 bi = ws.b1info[q];
  const uint32_t *gw = ws.wcnt + (int64_t)q * nblk * TOPK_LONG_WAVES;
  const uint2 *cq = ws.cand + (int64_t)q * nblk * TOPK_LONG_SPAN;
  const uint32_t *h2 = ws.hist2 + (int64_t)q * nblk * TOPK_BINS;
  // Everything that depends on nothing else is requested at once, with no
  // branch around a load (a conditional load makes the compiler wait for all
  // earlier loads where its value merges): the list counts, the first
  // entries of this wavefront's first LB0 lists (wavefront w takes lists w,
  // w + NW, ...; lane j entries j and j + WAVE), before the counts say how many
  // of them are real, and every span's digit-2 histogram (summed: the row's
  // histogram of the second digit over the keys of bin B1).  Indices past the
  // row's lists or spans are clamped to its last one, so every load stays
  // inside the row's part of the workspace, and their values are dropped.
  int c[SEG];
  int local = 0;
#pragma unroll
  for (int j = 0; j < SEG; ++j) {
    const int sg = t * SEG + j;
    const int v = (int)gw[min(sg, nseg - 1)];
    c[j] = sg < nseg ? v : 0;
    local += c[j];
  }
  uint2 e0[LB0][E0];
#pragma unroll
  for (int b = 0; b < LB0; ++b) {
    const int l = min(wave + b * NW, nseg - 1);
#pragma unroll
    for (int e = 0; e < E0; ++e) e0[b][e] = cq[(int64_t)l * TOPK_WAVE_SPAN + lane + WAVE * e];
  }
  uint32_t hb[BPT];
#pragma unroll
  for (int i = 0; i < BPT; ++i) hb[i] = 0u;
  for (int c0 = 0; c0 < nb; c0 += 4) {
    uint32_t u[4][BPT];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < BPT; ++i) u[j][i] = h2[(int64_t)min(c0 + j, nb - 1) * TOPK_BINS + t + i * NT];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < BPT; ++i) hb[i] += c0 + j < nb ? u[j][i] : 0u;
  }
  int ntot;
  int ex = block_exclusive_scan<NT>(local, s.sm, ntot);
#pragma unroll
  for (int j = 0; j < SEG; ++j) {
    const int sg = t * SEG + j;
    if (sg < nseg) s.off[sg] = ex;
    ex += c[j];
  }
  if (t == 0) s.off[nseg] = ntot;
#pragma unroll
  for (int i = 0; i < BPT; ++i) s.h[t + i * NT] = hb[i];
  lds_barrier();
  const uint32_t b1 = bi.x;
  const int r = k - (int)bi.y;
  find_rank_bin<NT, TOPK_BINS>(s.h, r, s.sm, s.res);
  const uint32_t pre = (b1 << 11) | (uint32_t)s.res[0];
  const int r2 = r - s.res[1];
  const int nbound = (int)s.h[s.res[0]];  // candidates with key[31:10] == pre
  const bool in_lds = ntot <= s.cap;      // block-uniform
  // Candidate i lives in list l (off[l] <= i < off[l+1]) at index i - off[l].
  auto locate = [&](int i) {
    int lo = 0, hi = nseg;  // largest l with off[l] <= i
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s.off[mid] <= i) lo = mid; else hi = mid;
    }
    return cq[(int64_t)lo * TOPK_WAVE_SPAN + (i - s.off[lo])];
  };
  // Into LDS.  The first LB0 lists of each wavefront come from registers
  // (e0); entries past E0 * WAVE, and the lists of longer rows (LB per
  // wavefront per batch, lane j taking entry j of each), follow from memory.
  auto slots = [&](int l0, int *dst) {
#pragma unroll
    for (int b = 0; b < LB; ++b) {
      const int l = l0 + b * NW;
      const int beg = l < nseg ? s.off[l] : 0, cnt = l < nseg ? s.off[l + 1] - beg : 0;
      dst[b] = lane < cnt ? beg + lane : -1;
    }
  };
  auto batch = [&](int l0, uint2 *e, int *dst) {
    slots(l0, dst);
#pragma unroll
    for (int b = 0; b < LB; ++b) {
      const int l = l0 + b * NW;
      e[b] = dst[b] >= 0 ? cq[(int64_t)l * TOPK_WAVE_SPAN + lane] : make_uint2(0u, 0u);
    }
  };
  // Entries from `from` on of list l, one per lane and round.
  auto rest = [&](int l, int beg, int cnt, int from) {
    for (int j = lane + from; j < cnt; j += WAVE) {
      const uint2 x = cq[(int64_t)l * TOPK_WAVE_SPAN + j];
      s.ck[beg + j] = x.x;
      s.cpos[beg + j] = x.y;
    }
  };
  auto put = [&](int l0, const uint2 *e, const int *dst) {
#pragma unroll
    for (int b = 0; b < LB; ++b) {
      if (dst[b] >= 0) {
        s.ck[dst[b]] = e[b].x;
        s.cpos[dst[b]] = e[b].y;
      }
      const int l = l0 + b * NW;
      if (l < nseg) rest(l, s.off[l], s.off[l + 1] - s.off[l], WAVE);
    }
  };
  after_issue();
  if (in_lds) {
#pragma unroll
    for (int b = 0; b < LB0; ++b) {
      const int l = wave + b * NW;
      if (l < nseg) {  // wave-uniform
        const int beg = s.off[l], cnt = s.off[l + 1] - beg;
#pragma unroll
        for (int e = 0; e < E0; ++e) {
          const int j = lane + WAVE * e;
          if (j < cnt) {
            s.ck[beg + j] = e0[b][e].x;
            s.cpos[beg + j] = e0[b][e].y;
          }
        }
      }
    }
#pragma unroll
    for (int b = 0; b < LB0; ++b) {
      const int l = wave + b * NW;
      if (l < nseg) rest(l, s.off[l], s.off[l + 1] - s.off[l], E0 * WAVE);
    }
    int dst[LB];
    uint2 e[LB];
    for (int l0 = wave + NW * LB0; l0 < nseg; l0 += NW * LB) {
      batch(l0, e, dst);
      put(l0, e, dst);
    }
  }
  lds_barrier();
  auto key_of = [&](int i) { return in_lds ? s.ck[i] : locate(i).x; };
  auto entry = [&](int i) { return in_lds ? make_uint2(s.ck[i], s.cpos[i]) : locate(i); };
  const int per = (ntot + NT - 1) / NT;
  const int lo = min(ntot, per * t), hi = min(ntot, lo + per);  // contiguous run: position order
  int tot;
  if (in_lds && nbound <= WAVE) {
    // Few candidates share the boundary prefix (the usual case): one
    // wavefront ranks them by (key descending, position ascending) and marks
    // the chosen r2 in place (key all ones) and the rest (key 0), so the
    // output below is a single comparison against the prefix.
    if (t == 0) *s.nb_cnt = 0;
    lds_barrier();
    for (int i = t; i < ntot; i += NT)
      if ((s.ck[i] >> 10) == pre) s.bidx[atomicAdd(s.nb_cnt, 1)] = i;
    lds_barrier();
    if (t < WAVE) {
      const bool have = t < nbound;
      const uint32_t mk = have ? s.ck[s.bidx[t]] : 0u, mp = have ? s.cpos[s.bidx[t]] : 0u;
      const int rank = boundary_rank(mk, mp, nbound);
      if (have) s.ck[s.bidx[t]] = rank < r2 ? 0xFFFFFFFFu : 0u;
    }
    lds_barrier();
    // Output in position order: key[31:10] > pre (the marked boundary keys included).
    int my_sel = 0;
    for (int i = lo; i < hi; ++i) my_sel += ((s.ck[i] >> 10) > pre) ? 1 : 0;
    int o = block_exclusive_scan<NT>(my_sel, s.sm, tot);
    for (int i = lo; i < hi; ++i)
      if ((s.ck[i] >> 10) > pre) emit(o++, s.cpos[i]);
  } else {
    lds_barrier();
    zero_lds<NT>(s.h, 1024);
    lds_barrier();
    // Digit 3 over the candidates with key[31:10] == pre.
    for (int i = lo; i < hi; ++i) {
      const uint32_t kk = key_of(i);
      if ((kk >> 10) == pre) atomicAdd(&s.h[kk & 1023u], 1u);
    }
    lds_barrier();
    find_rank_bin<NT, 1024>(s.h, r2, s.sm, s.res);
    const uint32_t kth = (pre << 10) | (uint32_t)s.res[0];
    const int ties = r2 - s.res[1];
    // Output in position order: keys > kth and the first `ties` keys == kth.
    int my_ties = 0;
    for (int i = lo; i < hi; ++i) my_ties += (key_of(i) == kth) ? 1 : 0;
    const int tie_rank = block_exclusive_scan<NT>(my_ties, s.sm, tot);
    int my_sel = 0;
    for (int i = lo, tr = tie_rank; i < hi; ++i) {
      const uint32_t kk = key_of(i);
      if (kk > kth || (kk == kth && tr < ties)) ++my_sel;
      tr += (kk == kth) ? 1 : 0;
    }
    int o = block_exclusive_scan<NT>(my_sel, s.sm, tot);
    for (int i = lo, tr = tie_rank; i < hi; ++i) {
      const uint2 en = entry(i);
      if (en.x > kth || (en.x == kth && tr < ties)) emit(o++, en.y);
      tr += (en.x == kth) ? 1 : 0;
    }
  }
  return tot;
}

}  // namespace dsa
