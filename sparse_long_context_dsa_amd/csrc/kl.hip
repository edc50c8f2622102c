// Indexer alignment loss: the attention target and KL(target || Softmax(I)).
//
// Page "arXiv'25 | DSA ... DeepSeek-V3.2", sections 5.1 (dense warm-up: every
// visible position) and 5.2 (sparse stage: the selected set S_t), the two L_I
// equations; the mlpod.com page on DeepSeek-V3.2-Exp, parts 2.1.1 and 2.1.2.
// For query t the target p[t, :] is the main attention's probabilities summed
// over the heads and L1-normalised over the attended positions; the loss term
// is KL(p[t, :] || Softmax(I[t, :])) over the same positions, and its gradient
// with respect to the indexer scores is Softmax(I) - p (p is a constant: the
// indexer's inputs are detached from the main model).
//
// kl_target_kernel recomputes the attention logits z[h, r] = scale * q[h] .
// kv[r] on bf16 MFMA over the same gathered 32-row tiles as the sparse
// attention (the S^T = K . Q^T chain, one wavefront per 32 heads) and turns
// them into probabilities with the attention's own log-sum-exp:
// a[r] = sum_h exp(z[h, r] - lse[h]).  One block = all 128 heads of one query
// over a run of up to 1024 set members; each tile is read into LDS once and
// serves every head.  The head sum is a butterfly over the 32 head lanes of
// each half-wavefront (ds_swizzle), then a fixed-order sum of the four
// wavefronts' partials through LDS, so the result is deterministic.  Without
// an output accumulator the block needs about half the registers of the
// attention kernel, so two blocks share a CU and one's MFMAs overlap the
// other's exponentials.
//
// kl_loss_kernel (one block per query) takes the L1 norm of a, the
// log-sum-exp of the indexer scores over the set, and writes the KL term and
// the gradient in place of a.  kl_sum_kernel adds the queries' terms.
#include "mla_tile.h"

namespace dsa {

constexpr int KLT_MAX_ROWS = 1024;                         // set members per target block
constexpr int KLT_PER_THREAD = KLT_MAX_ROWS / MLA_THREADS;  // 4
constexpr int KLT_MIN_BLOCKS = 2048;                       // target blocks wanted per launch
constexpr int KL_THREADS = 256;

struct KlTargetArgs {
  KlLaunch a;
  int nsplit;
  int rows_per_split;
  float scale_log2;
};

// v from lane l ^ XOR within each group of 32 lanes (ds_swizzle, bit-mask mode:
// and-mask 0x1F, or-mask 0, xor-mask XOR).
template <int XOR>
__device__ __forceinline__ float swz_xor(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1F | (XOR << 10)));
}

// Set size of query q: the clamped count of a sparse set, or every visible position.
__device__ __forceinline__ int kl_set_size(const KlLaunch &a, int q, int nvis) {
  if (!a.idx) return nvis;
  const int c = a.count ? a.count[q] : a.k;
  return max(0, min(c, min(a.k, nvis)));
}

template <bool WIDE>
__global__ __launch_bounds__(MLA_THREADS, 2) void kl_target_kernel(KlTargetArgs p) {
  const KlLaunch &a = p.a;
  // The blocks of one query run on one XCD (block b runs on XCD b % 8), so its
  // queries are read from HBM once and then come from that XCD's L2.
  const int y = blockIdx.x >> 3;
  const int q = (y / p.nsplit) * 8 + (blockIdx.x & 7);
  const int sp = y % p.nsplit;
  if (q >= a.num_q) return;
  const int nvis = a.q_nvis[q];
  const int nset = kl_set_size(a, q, nvis);
  const int r0 = sp * p.rows_per_split;
  const int nrows = max(0, min(nset, r0 + p.rows_per_split) - r0);
  if (nrows == 0) return;  // block-uniform

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 5, c = lane & 31;
  const int head = 32 * wave + c;

  __shared__ __attribute__((aligned(16))) uint8_t tb0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t tb1[TILE_BYTES];
  // Physical row per member (bit 31: a position outside [0, n_vis)).
  __shared__ __attribute__((aligned(16))) uint32_t prow[KLT_MAX_ROWS];
  __shared__ float red[MLA_WAVES][MLA_T];  // per-wavefront head sums of one tile

  // Members -> physical rows: every lane issues the same loads (indices
  // clamped into range) before any is used.  Loads complete in issue order:
  // the sequence's first row comes first, the q fragments and the head's
  // log-sum-exp right after the positions and before those are used, so no
  // later wait (nor the row table's barrier, a bare one) holds the first
  // gathers back behind all of q.
  const int seq = a.q_seq[q];
  const uint32_t row0 = a.map.block_shift < 0 ? (uint32_t)a.map.seq_row0[seq] : 0u;
  int bad = 0;
  uint4 qb[36];
  float lse_h;
  auto load_q = [&]() {
    lse_h = a.lse[(int64_t)q * 128 + head];
    const uint16_t *qr = a.q + ((int64_t)q * 128 + head) * 576 + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) qb[ks] = *reinterpret_cast<const uint4 *>(qr + 16 * ks);
  };
  {
    int pos[KLT_PER_THREAD];
    if (a.idx) {
      const int32_t *ip = a.idx + (int64_t)q * a.k + r0;
#pragma unroll
      for (int j = 0; j < KLT_PER_THREAD; ++j) pos[j] = ip[min(tid + j * MLA_THREADS, nrows - 1)];
    } else {
#pragma unroll
      for (int j = 0; j < KLT_PER_THREAD; ++j) pos[j] = r0 + min(tid + j * MLA_THREADS, nrows - 1);
    }
    load_q();
    bool ok[KLT_PER_THREAD];
#pragma unroll
    for (int j = 0; j < KLT_PER_THREAD; ++j) {
      ok[j] = pos[j] >= 0 && pos[j] < nvis;
      pos[j] = ok[j] ? pos[j] : 0;
    }
    uint32_t row[KLT_PER_THREAD];
    if (a.map.block_shift < 0) {
#pragma unroll
      for (int j = 0; j < KLT_PER_THREAD; ++j) row[j] = row0 + (uint32_t)pos[j];
    } else {
      const int32_t *bt = a.map.block_table + (int64_t)seq * a.map.max_blocks;
      const int sh = a.map.block_shift;
      int32_t blk[KLT_PER_THREAD];
#pragma unroll
      for (int j = 0; j < KLT_PER_THREAD; ++j) blk[j] = bt[pos[j] >> sh];
#pragma unroll
      for (int j = 0; j < KLT_PER_THREAD; ++j)
        row[j] = ((uint32_t)blk[j] << sh) + (uint32_t)(pos[j] & ((1 << sh) - 1));
    }
#pragma unroll
    for (int j = 0; j < KLT_PER_THREAD; ++j) {
      const int i = tid + j * MLA_THREADS;
      if (i < nrows) {
        prow[i] = row[j] | (ok[j] ? 0u : INVALID_ROW);
        bad |= ok[j] ? 0 : 1;
      }
    }
  }
  __shared__ int bad_w[MLA_WAVES];
  {
    const int wbad = __ballot(bad) != 0ull ? 1 : 0;
    if (lane == 0) bad_w[wave] = wbad;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): prow and bad_w written
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
  static_assert(MLA_WAVES == 4, "any_bad reads four wavefront words");
  const bool any_bad = (bad_w[0] | bad_w[1] | bad_w[2] | bad_w[3]) != 0;

  const int ntiles = (nrows + MLA_T - 1) / MLA_T;
  const uint32_t brow = __builtin_amdgcn_readfirstlane((!WIDE && a.map.block_shift < 0) ? row0 : 0u);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(a.kv + (size_t)brow * 576), (short)0, 0xFFFFFFFF, 0x00020000);
  issue_tile<WIDE>(rs, a.kv, brow, prow, 0, true, nrows - 1, false, tb0, wave, lane);
  issue_tile<WIDE>(rs, a.kv, brow, prow, MLA_T, ntiles > 1, nrows - 1, false, tb1, wave, lane);

  // The head's log-sum-exp in log2 units, negated; a head with no finite
  // log-sum-exp contributes nothing.
  const float nl = (lse_h > -INFINITY && lse_h < INFINITY) ? -lse_h * LOG2E : -INFINITY;

  // QK: lane reads row c, chunk 2*ks + g of the tile.
  int qk_base[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) qk_base[j] = tile_off(c, 2 * j + g);

  float *out = a.grad + (int64_t)q * a.ld_out + r0;
  // One tile; the two buffers alternate through separate call sites, so the
  // compiler sees which buffer each LDS read and each DMA touches and does not
  // wait for the other buffer's gather before reading this one.
  auto tile_step = [&](const int t, uint8_t *buf) {
    // Tile t landed (this wavefront's part), then a bare barrier for the
    // other wavefronts' parts.
    __builtin_amdgcn_s_waitcnt(0xF70 | LOADS_PER_WAVE);  // vmcnt(9): tile t + 1 (real or not) may stay in flight
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    // S^T[row, head] for the tile's 32 rows x this wavefront's 32 heads; the
    // K fragments are read four steps ahead of their MFMA.
    v16f s;
    {
      constexpr int AHEAD = 6;
      uint4 kf[AHEAD + 1];
#pragma unroll
      for (int ks = 0; ks < AHEAD; ++ks)
        kf[ks] = *reinterpret_cast<const uint4 *>(buf + qk_base[ks & 3] + 1024 * (ks >> 2));
#pragma unroll
      for (int ks = 0; ks < 36; ++ks) {
        if (ks + AHEAD < 36)
          kf[(ks + AHEAD) % (AHEAD + 1)] =
              *reinterpret_cast<const uint4 *>(buf + qk_base[(ks + AHEAD) & 3] + 1024 * ((ks + AHEAD) >> 2));
        if (ks == 0)
          mfma_s_first(s, kf[0], qb[0]);
        else
          mfma_s(s, kf[ks % (AHEAD + 1)], qb[ks]);
        __builtin_amdgcn_sched_barrier(0);
      }
      mfma_s_drain(s);
    }

    // Head c's probability of rows 8i + 4g + j; rows past the set or outside
    // [0, n_vis) weigh 0.
    const int t0 = t * MLA_T;
    float e[16];
    if (!any_bad && t0 + MLA_T <= nrows) {
#pragma unroll
      for (int i = 0; i < 16; ++i) e[i] = __builtin_amdgcn_exp2f(fmaf(s[i], p.scale_log2, nl));
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = t0 + 8 * i + 4 * g + j;
          const bool ok = r < nrows && !(prow[min(r, nrows - 1)] & INVALID_ROW);
          e[4 * i + j] = ok ? __builtin_amdgcn_exp2f(fmaf(s[4 * i + j], p.scale_log2, nl)) : 0.0f;
        }
    }
    // Sum over the 32 heads of the half-wavefront: each butterfly step keeps
    // half of the rows and adds the partner's copy of them.  Afterwards lane
    // c holds row index ri = c >> 1 (row 8 * (ri >> 2) + 4g + (ri & 3)).
    const bool b16 = c & 16, b8 = c & 8, b4 = c & 4, b2 = c & 2;
    float v8[8], v4[4], v2[2];
#pragma unroll
    for (int k = 0; k < 8; ++k) v8[k] = (b16 ? e[k + 8] : e[k]) + swz_xor<16>(b16 ? e[k] : e[k + 8]);
#pragma unroll
    for (int k = 0; k < 4; ++k) v4[k] = (b8 ? v8[k + 4] : v8[k]) + swz_xor<8>(b8 ? v8[k] : v8[k + 4]);
#pragma unroll
    for (int k = 0; k < 2; ++k) v2[k] = (b4 ? v4[k + 2] : v4[k]) + swz_xor<4>(b4 ? v4[k] : v4[k + 2]);
    float v1 = (b2 ? v2[1] : v2[0]) + swz_xor<2>(b2 ? v2[0] : v2[1]);
    v1 += swz_xor<1>(v1);
    const int ri = c >> 1;
    if ((c & 1) == 0) red[wave][8 * (ri >> 2) + 4 * g + (ri & 3)] = v1;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // Every wavefront is past its reads of this buffer: tile t + 2 goes in.
    // Past the last tile the loads still issue (so that the compiler counts
    // the same memory operations on every path and keeps exact waits) but
    // read the set's first row again into the free buffer.
    issue_tile<WIDE>(rs, a.kv, brow, prow, t0 + 2 * MLA_T, t + 2 < ntiles, nrows - 1, false, buf, wave, lane);
    if (tid < MLA_T && t0 + tid < nrows) out[t0 + tid] = (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
  };
  int t = 0;
  for (; t + 1 < ntiles; t += 2) {  // both steps on every trip: exact waits at the loop head
    tile_step(t, tb0);
    tile_step(t + 1, tb1);
  }
  if (t < ntiles) tile_step(t, tb0);
  __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
}

// Sum over a block of KL_THREADS, in a fixed order.
__device__ __forceinline__ float kl_block_sum(float v, float *sh) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor(v, m);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  return (sh[0] + sh[1]) + (sh[2] + sh[3]);
}

// (max, sum of exp(x - max)) pairs merged.
__device__ __forceinline__ void lse_merge(float &m, float &s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  s = s * expf(m - mn) + s2 * expf(m2 - mn);
  m = mn;
}

__global__ __launch_bounds__(KL_THREADS) void kl_loss_kernel(KlLaunch a) {
  const int q = blockIdx.x;
  const int tid = threadIdx.x;
  const int nvis = a.q_nvis[q];
  const int nset = kl_set_size(a, q, nvis);
  const int nout = a.idx ? a.k : nvis;  // entries written: the whole idx row, or the history
  float *gr = a.grad + (int64_t)q * a.ld_out;
  float *tg = a.target ? a.target + (int64_t)q * a.ld_out : nullptr;
  const float *sc = a.scores + (int64_t)q * a.ld_scores;
  const int32_t *ip = a.idx ? a.idx + (int64_t)q * a.k : nullptr;
  __shared__ float sh[4];
  __shared__ float shm[4], shs[4];

  // Pass 1: the L1 norm of the head sums and the log-sum-exp of the scores.
  float sa = 0.0f, m = -INFINITY, se = 0.0f;
  for (int i = tid; i < nset; i += KL_THREADS) {
    const int pos = ip ? ip[i] : i;
    if (pos < 0 || pos >= nvis) continue;
    sa += gr[i];
    const float x = sc[pos];
    if (x == -INFINITY) continue;  // softmax weight 0 (and exp(-inf - -inf) would be NaN)
    if (x > m) {
      se = se * expf(m - x) + 1.0f;
      m = x;
    } else {
      se += expf(x - m);
    }
  }
  sa = kl_block_sum(sa, sh);
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) {
    const float m2 = shfl_xor(m, k), s2 = shfl_xor(se, k);
    lse_merge(m, se, m2, s2);
  }
  if ((tid & 63) == 0) {
    shm[tid >> 6] = m;
    shs[tid >> 6] = se;
  }
  __syncthreads();
  m = shm[0];
  se = shs[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) lse_merge(m, se, shm[w], shs[w]);
  const float lz = m + logf(se);

  // Pass 2: p = a / |a|_1, log q = I - lz, the KL term and the gradient.
  float kl = 0.0f;
  for (int i = tid; i < nout; i += KL_THREADS) {
    float gv = 0.0f, pv = 0.0f;
    if (i < nset) {
      const int pos = ip ? ip[i] : i;
      if (pos >= 0 && pos < nvis) {
        const float av = gr[i];
        pv = sa > 0.0f ? av / sa : 0.0f;
        const float lq = sc[pos] - lz;
        if (pv > 0.0f) kl += pv * (logf(pv) - lq);
        gv = expf(lq) - pv;
      }
    }
    gr[i] = gv;
    if (tg) tg[i] = pv;
  }
  kl = kl_block_sum(kl, sh);
  if (tid == 0) a.kl[q] = kl;
}

// loss = sum of the per-query terms, in a fixed order (fp64 partials).
__global__ __launch_bounds__(KL_THREADS) void kl_sum_kernel(const float *__restrict__ kl, int num_q,
                                                             float *__restrict__ loss) {
  __shared__ double sh[KL_THREADS];
  double v = 0.0;
  for (int i = threadIdx.x; i < num_q; i += KL_THREADS) v += (double)kl[i];
  sh[threadIdx.x] = v;
  __syncthreads();
  for (int w = KL_THREADS / 2; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *loss = (float)sh[0];
}

hipError_t launch_indexer_kl(const KlLaunch &a, int max_set, hipStream_t st) {
  if (a.num_q > 0 && max_set > 0) {
    KlTargetArgs p;
    p.a = a;
    int rps = KLT_MAX_ROWS;
    auto splits = [&](int r) { return (max_set + r - 1) / r; };
    while (rps > 4 * MLA_T && (int64_t)a.num_q * splits(rps) < KLT_MIN_BLOCKS) rps /= 2;
    p.nsplit = splits(rps);
    p.rows_per_split = rps;
    p.scale_log2 = a.softmax_scale * LOG2E;
    const bool wide = a.map.block_shift >= 0 && a.num_rows * (int64_t)ROW_BYTES >= 0xFFFFF000ll - ROW_BYTES;
    const int64_t nq8 = (a.num_q + 7) / 8 * 8;
    const dim3 grid((unsigned)(nq8 * p.nsplit));
    if (wide)
      hipLaunchKernelGGL((kl_target_kernel<true>), grid, dim3(MLA_THREADS), 0, st, p);
    else
      hipLaunchKernelGGL((kl_target_kernel<false>), grid, dim3(MLA_THREADS), 0, st, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.num_q > 0) {
    hipLaunchKernelGGL(kl_loss_kernel, dim3((unsigned)a.num_q), dim3(KL_THREADS), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.loss) {
    hipLaunchKernelGGL(kl_sum_kernel, dim3(1), dim3(KL_THREADS), 0, st, a.kl, a.num_q, a.loss);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace dsa
