// Sparse MQA-mode MLA attention on bf16 MFMA (gfx950).
//
// Page "arXiv'25 | DSA ... DeepSeek-V3.2", section 3 (third equation: the
// core attention reads only the latent rows of the selected positions) and
// section 4 (MQA: every head shares one latent KV, so one selection serves all
// heads); page "DeepSeekV3.2之DSA", part 5.1 (softmax(q . [c_kv; k_pe]^T) .
// c_kv over the 2048 gathered slots, num_kv_heads = 1).  The value is dims
// 0..511 of each 576-wide latent row; z = softmax_scale * q . row.
//
// One block (4 wavefronts) = one query and a run of its selected rows, all
// 128 heads, so every gathered row is read from memory once and used by every
// head.  Wavefront w owns heads [32w, 32w+32): its queries live in registers
// for the whole run (36 x 16-byte B fragments, 144 VGPRs) and so does its
// output accumulator O[32 heads, 512] in fp32 (16 x 32x32 tiles in AGPRs).
// Rows arrive in tiles of 32, gathered through the position -> row map
// straight from global memory into LDS (buffer/global loads to LDS, 16 bytes
// per lane, no staging registers), three tile buffers.  One row-major copy of each
// tile serves both products:
//   * S^T = K . Q^T (v_mfma_f32_32x32x16_bf16, M = rows, N = heads, K = 576
//     in 36 steps): A fragments are 16-byte LDS reads of a row;
//   * O = P . V (M = heads, N = dims, K = 32 rows in 2 steps): B fragments
//     (4 rows of one column per lane, twice) come from the transposing LDS
//     read ds_read_b64_tr_b16.
// 16-byte chunks of a tile row are XOR-swizzled by the row to spread banks.
// Computing S transposed puts each head in one lane column, so the online
// softmax (running max m, sum l per head) needs one cross-half exchange, and
// the S^T accumulator registers are exactly the A operand of P . V once
// rounded to bf16.  Only the per-head rescale of O needs the softmax state of
// other lanes; it goes through a 128-byte LDS slot per wavefront, is done in
// place on the AGPRs, and happens only when a running max grows by more than
// 2^8 (P stays <= 256).  exp2 with log2(e) folded into the scale.
//
// Decode splits a query's rows over several blocks that write (O/l, lse)
// partials; mla_combine_kernel merges them.  Prefill gives each query one
// block and writes the result directly.
#include <type_traits>

#include "mla_tile.h"

namespace dsa {

constexpr int NBUF = 3;                              // tiles in flight

struct MlaKernelArgs {
  MlaLaunch a;
  int nsplit;
  int rows_per_split;
  float scale_log2;
  float *part_o;    // [num_q, nsplit, 128, 512]   (nsplit > 1)
  float *part_lse;  // [num_q, nsplit, 128]
  int dense;        // prow holds the base row of each 32-row tile of positions
};

template <bool WIDE, bool PIPE>
__global__ __launch_bounds__(MLA_THREADS, 1) void mla_kernel(MlaKernelArgs p) {
  const MlaLaunch &a = p.a;
  // Decode splits: the blocks of one query run on one XCD (block b runs on
  // XCD b % 8), so the query's q and partial outputs stay in that XCD's L2.
  int q, sp;
  if (p.nsplit == 1) {
    q = blockIdx.x;
    sp = 0;
  } else {
    const int y = blockIdx.x >> 3;
    q = (y / p.nsplit) * 8 + (blockIdx.x & 7);
    sp = y % p.nsplit;
    if (q >= a.num_q) return;
  }
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;  // wave-uniform
  const int g = lane >> 5, c = lane & 31;

  // Three separately declared tile buffers: each has its own alias scope, so
  // the compiler sees that reading one tile never races with the LDS DMA that
  // fills another (one shared array would make it wait for all DMA first).
  __shared__ __attribute__((aligned(16))) uint8_t tb0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t tb1[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t tb2[TILE_BYTES];
  // Physical row per selected position (bit 31: outside [0, n_vis)); the
  // tail keeps the masked reads of a partial last tile in bounds.
  __shared__ __attribute__((aligned(16))) uint32_t prow[MLA_MAX_ROWS + MLA_T];
  // Per-head rescale factors (two slots: the pipelined schedule reads tile
  // t's at step t + 1) and 1/l for the epilogue, each wavefront's own: they
  // carry a head's value from the lane that owns its softmax state to the
  // lanes that hold its O rows.
  __shared__ __attribute__((aligned(16))) float aex[2][MLA_WAVES][32];
  __shared__ __attribute__((aligned(16))) float iex[MLA_WAVES][32];  // 1/l per head, for the epilogue

  const int nvis = a.q_nvis[q];
  int cnt = a.count ? a.count[q] : a.k;
  cnt = max(0, min(cnt, min(a.k, nvis)));
  const int r0 = sp * p.rows_per_split;
  const int nrows = max(0, min(cnt, r0 + p.rows_per_split) - r0);

  // Selected positions -> physical rows.  A position outside [0, n_vis) breaks
  // the contract; it is loaded from position 0 (in bounds, finite) and masked.
  const int seq = a.q_seq[q];
  // A contiguous cache's first row of the sequence, loaded before the q
  // fragments: loads complete in issue order, so waiting for a later one
  // would also wait for all of q.
  const uint32_t row0 = a.map.block_shift < 0 ? (uint32_t)a.map.seq_row0[seq] : 0u;
  // All of a thread's positions, and then their block-table entries, are
  // loaded before any is used, every lane issuing the same loads (indices
  // clamped into range, no branch), so they overlap instead of taking one
  // memory latency per row.
  constexpr int PER_THREAD = MLA_MAX_ROWS / MLA_THREADS;
  constexpr int PER_THREAD_T = (MLA_MAX_ROWS + MLA_T + MLA_THREADS - 1) / MLA_THREADS;
  const bool dense = p.dense != 0;
  int bad = 0;
  // Queries of this wavefront's own 32 heads: B fragments of S^T = K . Q^T.
  // Requested right after the block's first position (or block-table) loads
  // and before those values are used, so that their latency overlaps the
  // position -> row lookup and the first gathers.  A block with no rows
  // never reads them.
  uint4 qb[36];
  auto load_q = [&]() {
    const uint16_t *qr = a.q + ((int64_t)q * 128 + 32 * wave + c) * 576 + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) qb[ks] = *reinterpret_cast<const uint4 *>(qr + 16 * ks);
  };
  if (dense && nrows > 0) {  // block-uniform
    // Dense: the base row of each 32-row tile of positions r0, r0 + 32, ...
    const int nt = (nrows + MLA_T - 1) / MLA_T;  // <= MLA_MAX_ROWS + MLA_T (the launcher splits longer rows)
    uint32_t base[PER_THREAD_T];
    if (a.map.block_shift < 0) {
      const uint32_t s0 = row0 + (uint32_t)r0;
#pragma unroll
      for (int j = 0; j < PER_THREAD_T; ++j) base[j] = s0 + (uint32_t)(MLA_T * (tid + j * MLA_THREADS));
      load_q();
    } else {
      const int32_t *bt = a.map.block_table + (int64_t)seq * a.map.max_blocks;
      const int sh = a.map.block_shift;
      int32_t blk[PER_THREAD_T];
#pragma unroll
      for (int j = 0; j < PER_THREAD_T; ++j) blk[j] = bt[(r0 + MLA_T * min(tid + j * MLA_THREADS, nt - 1)) >> sh];
      load_q();
#pragma unroll
      for (int j = 0; j < PER_THREAD_T; ++j) {
        const int pos = r0 + MLA_T * min(tid + j * MLA_THREADS, nt - 1);
        base[j] = ((uint32_t)blk[j] << sh) + (uint32_t)(pos & ((1 << sh) - 1));
      }
    }
#pragma unroll
    for (int j = 0; j < PER_THREAD_T; ++j)
      if (tid + j * MLA_THREADS < nt) prow[tid + j * MLA_THREADS] = base[j];
  } else if (nrows > 0) {  // block-uniform
    const int32_t *ip = a.idx + (int64_t)q * a.k + r0;
    int pos[PER_THREAD];
#pragma unroll
    for (int j = 0; j < PER_THREAD; ++j) pos[j] = ip[min(tid + j * MLA_THREADS, nrows - 1)];
    load_q();
    bool ok[PER_THREAD];
#pragma unroll
    for (int j = 0; j < PER_THREAD; ++j) {
      ok[j] = pos[j] >= 0 && pos[j] < nvis;
      pos[j] = ok[j] ? pos[j] : 0;
    }
    uint32_t row[PER_THREAD];
    if (a.map.block_shift < 0) {  // contiguous
#pragma unroll
      for (int j = 0; j < PER_THREAD; ++j) row[j] = row0 + (uint32_t)pos[j];
    } else {  // paged
      const int32_t *bt = a.map.block_table + (int64_t)seq * a.map.max_blocks;
      const int sh = a.map.block_shift;
      int32_t blk[PER_THREAD];
#pragma unroll
      for (int j = 0; j < PER_THREAD; ++j) blk[j] = bt[pos[j] >> sh];
#pragma unroll
      for (int j = 0; j < PER_THREAD; ++j)
        row[j] = ((uint32_t)blk[j] << sh) + (uint32_t)(pos[j] & ((1 << sh) - 1));
    }
#pragma unroll
    for (int j = 0; j < PER_THREAD; ++j) {
      const int i = tid + j * MLA_THREADS;
      if (i < nrows) {
        prow[i] = row[j] | (ok[j] ? 0u : INVALID_ROW);
        bad |= ok[j] ? 0 : 1;
      }
    }
  }

  const int head = 32 * wave + c;

  // O[nt]: the 32 own heads x value dims 32*nt .. +31 (all 512 dims).
  v16f o[16];
#pragma unroll
  for (int nt = 0; nt < 16; ++nt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[nt][i] = 0.0f;
  float m_ref = -INFINITY, l_run = 0.0f;  // per own head c (both lane halves agree on m_ref)

  // Per-lane LDS address bases (everything else is an immediate offset).
  // QK: lane reads row c, chunk 2*ks + g = tile_off(c, 2*ks + g)
  // = qk_base[ks & 3] + 1024 * (ks >> 2).
  int qk_base[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) qk_base[j] = tile_off(c, 2 * j + g);
  // PV: in each 16-lane group, lane ti points at row r = ti >> 2 of its 4-row
  // set and at 4 columns (8 bytes, piece ti & 1 of chunk 4*nt + tr_x) of
  // this wavefront's value half.  The set's rows are 16*ks2 + 8*half + 4*g +
  // r: row group 2*ks2 + half, row 4*g + r inside it, so tile_off splits into
  // an immediate 9216*(2*ks2) + 1024*(nt >> 1) and one of four per-lane bases
  // tr_base[nt & 1][half] (which hold the row group of the half).
  const int ti = lane & 15, th = (lane >> 4) & 1;
  const int tr_r = ti >> 2, tr_x = 2 * th + ((ti & 3) >> 1), tr_piece = ti & 1;
  int tr_base[2][2];
#pragma unroll
  for (int odd = 0; odd < 2; ++odd)
#pragma unroll
    for (int half = 0; half < 2; ++half)
      tr_base[odd][half] = tile_off(8 * half + 4 * g + tr_r, 4 * odd + tr_x) + 8 * tr_piece;

  // prow ready; does any row need masking beyond a partial last tile?  One
  // LDS word per wavefront and a bare barrier: __syncthreads_or would also
  // wait for every outstanding load, the q fragments included, before the
  // first gathers could be issued.
  __shared__ int bad_w[MLA_WAVES];
  {
    const int wbad = __ballot(bad) != 0ull ? 1 : 0;
    if (lane == 0) bad_w[wave] = wbad;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): prow and bad_w written
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
  const bool any_bad = (bad_w[0] | bad_w[1] | bad_w[2] | bad_w[3]) != 0;
  static_assert(MLA_WAVES == 4, "any_bad reads four wavefront words");
  const int ntiles = (nrows + MLA_T - 1) / MLA_T;
  // Buffer descriptor of the latent cache from row brow on.
  const uint32_t brow = __builtin_amdgcn_readfirstlane(
      (!WIDE && a.map.block_shift < 0) ? row0 : 0u);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(a.kv + (size_t)brow * 576), (short)0, 0xFFFFFFFF, 0x00020000);
  if (ntiles > 0) issue_tile<WIDE>(rs, a.kv, brow, prow, 0, true, nrows - 1, dense, tb0, wave, lane);
  if (!PIPE && ntiles > 1) issue_tile<WIDE>(rs, a.kv, brow, prow, MLA_T, true, nrows - 1, dense, tb1, wave, lane);

  // ---- One tile, in pieces shared by the two schedules below. ----
  auto no_hook = [](int) {};

  // S^T[row, head] for the tile's 32 rows x the 32 own heads.  K fragments
  // are read QK_AHEAD steps ahead of their MFMA (ring buffer); hook(ks) runs
  // after the MFMA of step ks.
  auto qk = [&](const uint8_t *buf, v16f &s, auto &&hook) {
    constexpr int QK_AHEAD = 6;
    uint4 kf[QK_AHEAD + 1];
#pragma unroll
    for (int ks = 0; ks < QK_AHEAD; ++ks)
      kf[ks] = *reinterpret_cast<const uint4 *>(buf + qk_base[ks & 3] + 1024 * (ks >> 2));
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) {
      if (ks + QK_AHEAD < 36)
        kf[(ks + QK_AHEAD) % (QK_AHEAD + 1)] =
            *reinterpret_cast<const uint4 *>(buf + qk_base[(ks + QK_AHEAD) & 3] + 1024 * ((ks + QK_AHEAD) >> 2));
      if (ks == 0)
        mfma_s_first(s, kf[0], qb[0]);
      else
        mfma_s(s, kf[ks % (QK_AHEAD + 1)], qb[ks]);
      hook(ks);
      // Keep the written order: the scheduler would otherwise sink each read
      // next to its MFMA and undo the prefetch distance.
      __builtin_amdgcn_sched_barrier(0);
    }
    mfma_s_drain(s);
  };

  // Online softmax for own head c over the tile's rows 8i + 4g + j, in log2
  // units: z = scale_log2 * s, folded into the exp2 argument (zscale) when no
  // row is masked (scale_log2 > 0, so the max of z is scale_log2 times the
  // max of s).  Only a partial last tile, or a block whose list holds
  // positions outside [0, n_vis), masks rows to -inf.  Returns the tile max.
  auto tile_max = [&](const int t0, const v16f &s, float *z, float &zscale) -> float {
    float tmax;
    if (!any_bad && t0 + MLA_T <= nrows) {
#pragma unroll
      for (int i = 0; i < 16; ++i) z[i] = s[i];
      float m5[5];
#pragma unroll
      for (int i = 0; i < 5; ++i) m5[i] = max3f(z[3 * i], z[3 * i + 1], z[3 * i + 2]);
      const float ma = max3f(m5[0], m5[1], m5[2]), mb = max3f(m5[3], m5[4], z[15]);
      tmax = xhalf_max(max3f(ma, mb, mb)) * p.scale_log2;
      zscale = p.scale_log2;
    } else {
      tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rbase = t0 + 8 * i + 4 * g;
        // (Dense: prow holds tile bases, and every row below nrows is valid.)
        const uint4 pr = dense ? make_uint4(0u, 0u, 0u, 0u) : *reinterpret_cast<const uint4 *>(&prow[rbase]);
        const uint32_t prv[4] = {pr.x, pr.y, pr.z, pr.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool ok = (rbase + j < nrows) && (dense || !(prv[j] & INVALID_ROW));
          const float v = ok ? s[4 * i + j] * p.scale_log2 : -INFINITY;
          z[4 * i + j] = v;
          tmax = fmaxf(tmax, v);
        }
      }
      tmax = xhalf_max(tmax);
      zscale = 1.0f;
    }
    return tmax;
  };

  // The softmax update of one tile in 10 pieces, so that the pipelined
  // schedule can spread them between MFMAs.  Piece 0 moves the reference max
  // only when a head's tile max exceeds it by more than RESCALE_LOG2 (always
  // on the first tile with a valid row), so P <= 2^RESCALE_LOG2 and O is
  // rescaled rarely; an all-masked tile changes nothing.  Pieces 1-8 turn
  // two rows each into P (bf16 pairs) and the tile's sum, which piece 9 adds
  // to l_run.
  auto softmax_piece = [&](const int j, const float *z, const float zscale, const float tmax, bool &resc,
                           float &alpha, float &nmref, float &psum, uint32_t *pk) {
    if (j == 0) {
      resc = __ballot(tmax > m_ref + RESCALE_LOG2) != 0ull;
      const float m_new = resc ? fmaxf(m_ref, tmax) : m_ref;
      alpha = resc ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;  // 0 while m_ref = -inf
      l_run *= alpha;
      m_ref = m_new;
      nmref = (m_ref == -INFINITY) ? 0.0f : -m_ref;  // all rows so far masked: z = -inf, p = 0
      psum = 0.0f;
    } else if (j <= 8) {
      const int i = j - 1;
      const float e0 = __builtin_amdgcn_exp2f(fmaf(z[2 * i], zscale, nmref));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(z[2 * i + 1], zscale, nmref));
      psum += e0 + e1;
      pk[i] = pack_bf16(e0, e1);
    } else if (j == 9) {
      l_run += psum;
    }
  };

  // O += P . V over the tile's 32 rows (2 k-steps of 16) for the 32 own
  // heads and all 512 value dims (16 N-tiles).  The k-slots of lane group g
  // in step ks2 are rows 16*ks2 + 4g + {0..3} and 16*ks2 + 8 + 4g + {0..3}
  // (where the S^T accumulator put them); the transposing read gives lane l
  // the 4 rows of one of those sets at column n = l % 32: lanes 4r..4r+3 of
  // each 16-lane group point at row r of the set, 4 columns each.  32 steps
  // j = (ks2, nt); the B fragment of step j is read PV_AHEAD steps ahead of
  // its MFMA (ring buffer).  hook(j) runs after the MFMA of step j.  Each
  // wavefront reads the whole value half of the tile, so no P leaves the
  // wavefront and no barrier separates the softmax from the PV.
  auto pv = [&](const uint8_t *buf, const uint4 &a0, const uint4 &a1, auto &&hook) {
    constexpr int PV_AHEAD = PIPE ? 3 : 4;
    auto v_frag = [&](int j) {
      const int ks2 = j >> 4, nt = j & 15;
      const int off0 = tr_base[nt & 1][0] + 9216 * (2 * ks2) + 1024 * (nt >> 1);  // half 0
      const int off1 = tr_base[nt & 1][1] + 9216 * (2 * ks2) + 1024 * (nt >> 1);  // half 1
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)(buf + off0));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)(buf + off1));
      const uint2 ulo = __builtin_bit_cast(uint2, lo), uhi = __builtin_bit_cast(uint2, hi);
      return make_uint4(ulo.x, ulo.y, uhi.x, uhi.y);
    };
    uint4 vf[PV_AHEAD + 1];
#pragma unroll
    for (int j = 0; j < PV_AHEAD; ++j) vf[j] = v_frag(j);
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      if (j + PV_AHEAD < 32) vf[(j + PV_AHEAD) % (PV_AHEAD + 1)] = v_frag(j + PV_AHEAD);
      const int nt = j & 15;
      o[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf(j < 16 ? a0 : a1), as_bf(vf[j % (PV_AHEAD + 1)]), o[nt], 0,
                                                     0, 0);
      hook(j);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // O rows (own heads 8i + 4g + j) times their heads' factors, from this
  // wavefront's 32-entry slot in LDS.
  auto rescale_o = [&](const float *fac) __attribute__((always_inline)) {
    float al[16];
    read_head_values(fac, g, al);
#pragma unroll
    for (int nt = 0; nt < 16; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = o[nt][i];
        scale_acc(x, al[i]);
        o[nt][i] = x;
      }
  };

  // Tile t must have landed (every wave's part of it): wait for this wave's
  // loads of tile t, then the barrier.  In the in-order schedule tile t+1 is
  // already in flight and may stay so; the pipelined one issues it later.  A
  // bare s_barrier: __syncthreads() would add a workgroup release fence,
  // which waits for every outstanding LDS DMA, tile t+1 included.
  auto wait_tile = [&](const int t) {
    if (!PIPE && t + 1 < ntiles)
      __builtin_amdgcn_s_waitcnt(0xF70 | LOADS_PER_WAVE);  // vmcnt(9)
    else
      __builtin_amdgcn_s_waitcnt(0xF70);                   // vmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  if (!PIPE) {
    // In-order schedule (decode, where the gathers come from HBM): the
    // gather of tile t + 2 starts as tile t's compute starts, two tiles
    // ahead; then QK, softmax and PV of tile t.
    auto tile_step = [&](const int t, const uint8_t *buf, uint8_t *nbuf) {
      wait_tile(t);
      // The buffer of tile t-1 is free now (every wave is past its compute):
      // tile t + 2 goes into it.  Past the last tile the parts still issue
      // (no branch between the MFMAs, which would make the compiler drain the
      // LDS read ring), but all read one row of this block, which stays in
      // cache, into the free buffer.
      issue_tile<WIDE>(rs, a.kv, brow, prow, t * MLA_T + 2 * MLA_T, t + 2 < ntiles, nrows - 1, dense, nbuf, wave,
                       lane);
      __builtin_amdgcn_sched_barrier(0);
      v16f s;
      qk(buf, s, no_hook);
      float z[16], zscale;
      const float tmax = tile_max(t * MLA_T, s, z, zscale);
      bool resc;
      float alpha, nmref, psum;
      uint32_t pk[8];
#pragma unroll
      for (int j = 0; j < 10; ++j) softmax_piece(j, z, zscale, tmax, resc, alpha, nmref, psum, pk);
      const uint4 pa0 = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      const uint4 pa1 = make_uint4(pk[4], pk[5], pk[6], pk[7]);
      if (t > 0 && resc) {  // O is still zero on the first tile
        if (g == 0) aex[0][wave][c] = alpha;  // own slot: no other wavefront reads it
        rescale_o(aex[0][wave]);
      }
      pv(buf, pa0, pa1, no_hook);
    };
    for (int t = 0; t < ntiles; t += NBUF) {
      tile_step(t, tb0, tb2);
      if (t + 1 < ntiles) tile_step(t + 1, tb1, tb0);
      if (t + 2 < ntiles) tile_step(t + 2, tb2, tb1);
    }
  } else {
    // Pipelined schedule (prefill, where the gathers mostly hit the caches):
    // tile t's QK, with the gather of tile t + 1 issued between its MFMAs;
    // then tile t-1's PV with tile t's softmax spread between its MFMAs, so
    // the matrix cores, the vector ALUs and the memory pipeline work at once.
    // P of tile t stays in registers for one tile, and O is rescaled for
    // tile t's reference max just before that PV (the factors' LDS slots
    // alternate).
    bool resc_prev = false;
    uint4 pp0 = make_uint4(0u, 0u, 0u, 0u), pp1 = pp0;  // P of the previous tile, kept in registers
    // Tile t-1's buffer is free once every wavefront has passed the barrier of
    // tile t (its PV of tile t-2 is done); tile t + 1 goes into the buffer of
    // tile t - 2.
    auto tile_step = [&](const int t, const uint8_t *buf, uint8_t *nbuf, const uint8_t *pbuf, auto prev) {
      constexpr bool PREV = decltype(prev)::value;
      wait_tile(t);
      // Past the last tile the parts read one cached row into the free buffer.
      const uint32_t nrow = tile_row(prow, (t + 1) * MLA_T, t + 1 < ntiles, nrows - 1, dense, wave, lane);
      v16f s;
      qk(buf, s, [&](const int ks) {
        if (ks < LOADS_PER_WAVE) issue_part<WIDE>(rs, a.kv, brow, nrow, nbuf, wave, lane, ks);
      });
      float z[16], zscale;
      const float tmax = tile_max(t * MLA_T, s, z, zscale);
      bool resc;
      float alpha, nmref, psum;
      uint32_t pk[8];
      if (PREV) {
        if (resc_prev) rescale_o(aex[(t - 1) & 1][wave]);
        pv(pbuf, pp0, pp1, [&](const int j) {
          if (j < 10) softmax_piece(j, z, zscale, tmax, resc, alpha, nmref, psum, pk);
        });
      } else {
#pragma unroll
        for (int j = 0; j < 10; ++j) softmax_piece(j, z, zscale, tmax, resc, alpha, nmref, psum, pk);
      }
      if (g == 0) aex[t & 1][wave][c] = alpha;  // own slot, read at the next step
      pp0 = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      pp1 = make_uint4(pk[4], pk[5], pk[6], pk[7]);
      // O is still zero until tile 0's PV, which tile 0's factors precede.
      resc_prev = PREV && resc;
    };
    using First = std::integral_constant<bool, false>;
    using Later = std::integral_constant<bool, true>;
    if (ntiles > 0) tile_step(0, tb0, tb1, tb2, First{});
    for (int t = 1; t < ntiles; t += NBUF) {
      tile_step(t, tb1, tb2, tb0, Later{});
      if (t + 1 < ntiles) tile_step(t + 1, tb2, tb0, tb1, Later{});
      if (t + 2 < ntiles) tile_step(t + 2, tb0, tb1, tb2, Later{});
    }
    if (ntiles > 0) {
      const int lt = (ntiles - 1) % NBUF;
      if (resc_prev) rescale_o(aex[(ntiles - 1) & 1][wave]);
      pv(lt == 0 ? tb0 : lt == 1 ? tb1 : tb2, pp0, pp1, no_hook);
    }
  }
  // The last two tiles issued gathers past the end: let them land before the
  // block's LDS can be handed to another block.
  __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)

  // Normalise.  Both lane halves hold partial sums of own head c; 1/l goes
  // through the wavefront's LDS slot to the lanes that hold that head's rows.
  const float l_tot = xhalf_sum(l_run);
  const float inv = (l_tot > 0.0f) ? 1.0f / l_tot : 0.0f;
  const float lse_v = (l_tot > 0.0f) ? m_ref * LN2 + logf(l_tot) : -INFINITY;
  if (g == 0) iex[wave][c] = inv;
  __syncthreads();

  float *obase;
  float *lbase;
  if (p.nsplit == 1) {
    obase = a.out + (int64_t)q * 128 * 512;
    lbase = a.lse ? a.lse + (int64_t)q * 128 : nullptr;
  } else {
    obase = p.part_o + ((int64_t)q * p.nsplit + sp) * 128 * 512;
    lbase = p.part_lse + ((int64_t)q * p.nsplit + sp) * 128;
  }
  // Each value is scaled by its head's 1/l on its way out of the AGPRs.
  // (256 KiB of O per workgroup: the CU's store bandwidth bounds this, not
  // the instruction count; staging through LDS for 16-byte stores measured
  // slower.)
  {
    float il[16];
    read_head_values(iex[wave], g, il);
#pragma unroll
    for (int nt = 0; nt < 16; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int h = 32 * wave + 8 * i + 4 * g + j;
          {
            // Split partials (read once, by the combine) non-temporally; the
            // prefill output measured slower that way.
            const float v = read_scaled(o[nt][4 * i + j], il[4 * i + j]);
            if (p.nsplit > 1)
              __builtin_nontemporal_store(v, obase + (int64_t)h * 512 + 32 * nt + c);
            else
              obase[(int64_t)h * 512 + 32 * nt + c] = v;
          }
        }
  }
  if (lbase && g == 0) lbase[head] = lse_v;
}

// Merge split partials: out = sum_s exp(lse_s - M) O_s / sum_s exp(lse_s - M).
// NS > 0 fixes the split count at compile time, so that every partial's lse
// and value are requested before the first is used (one memory round trip
// instead of one per split); NS < 0 does the same for any count up to -NS,
// and NS = 0 takes any count, one split after the other.  A split with no row
// (lse = -inf) has weight 0 and a zero partial; all splits empty gives 0 and
// lse = -inf.
template <int NS>
__global__ __launch_bounds__(256) void mla_combine_kernel(const float *__restrict__ part_o,
                                                          const float *__restrict__ part_lse, int nsplit, int num_q,
                                                          float *__restrict__ out, float *__restrict__ lse) {
  // Same XCD as the query's split blocks (block b runs on XCD b % 8).
  const int y = blockIdx.x >> 3;
  const int q = (y >> 6) * 8 + (blockIdx.x & 7);
  if (q >= num_q) return;
  const int head = 2 * (y & 63) + (threadIdx.x >> 7);
  const int d = 4 * (threadIdx.x & 127);
  const float *pl = part_lse + (int64_t)q * nsplit * 128 + head;
  const float *po = part_o + ((int64_t)q * nsplit * 128 + head) * 512 + d;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float den = 0.0f, mx = -INFINITY;
  if (NS != 0) {
    constexpr int M = NS > 0 ? NS : (NS < 0 ? -NS : 1);
    float ls[M];
    float4 v[M];
#pragma unroll
    for (int s = 0; s < M; ++s) {
      if (NS > 0 || s < nsplit) {
        ls[s] = pl[s * 128];
        v[s] = *reinterpret_cast<const float4 *>(po + (int64_t)s * 128 * 512);
      } else {
        ls[s] = -INFINITY;
        v[s] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
#pragma unroll
    for (int s = 0; s < M; ++s) mx = fmaxf(mx, ls[s]);
#pragma unroll
    for (int s = 0; s < M; ++s) {
      const float wgt = (ls[s] == -INFINITY) ? 0.0f : expf(ls[s] - mx);
      acc.x += wgt * v[s].x; acc.y += wgt * v[s].y; acc.z += wgt * v[s].z; acc.w += wgt * v[s].w;
      den += wgt;
    }
  } else {
    for (int s = 0; s < nsplit; ++s) mx = fmaxf(mx, pl[s * 128]);
    if (mx != -INFINITY) {
      for (int s = 0; s < nsplit; ++s) {
        const float ls = pl[s * 128];
        if (ls == -INFINITY) continue;
        const float wgt = expf(ls - mx);
        const float4 v = *reinterpret_cast<const float4 *>(po + (int64_t)s * 128 * 512);
        acc.x += wgt * v.x; acc.y += wgt * v.y; acc.z += wgt * v.z; acc.w += wgt * v.w;
        den += wgt;
      }
    }
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  float4 r = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  {
    // Non-temporal: the output is not read again in the step, and its dirty
    // lines would otherwise be written back while the next indexer streams.
    typedef float ntf4 __attribute__((ext_vector_type(4)));
    const ntf4 v4 = {r.x, r.y, r.z, r.w};
    __builtin_nontemporal_store(v4, reinterpret_cast<ntf4 *>(out + ((int64_t)q * 128 + head) * 512 + d));
  }
  if (lse && (threadIdx.x & 127) == 0) lse[(int64_t)q * 128 + head] = den > 0.0f ? mx + logf(den) : -INFINITY;
}

// Row splits per query in decode.  More splits put more of the 256 CUs to
// work, but each writes a 256 KiB fp32 partial that the combine reads back.
// The count minimises a time model: the busiest CU's workgroups (about 4 us
// of prologue and epilogue, 2 us per 32-row tile), plus the partials' round
// trip at 5 TB/s.  At least 128 rows per split.
int mla_num_splits(int num_q, int k, bool decode) {
  if (!decode || num_q <= 0) return 1;
  const int max_split = k >= 128 ? (k + 127) / 128 : 1;
  int best_ns = 1;
  double best = 1e300;
  for (int ns = 1; ns <= max_split; ++ns) {
    const double tiles = (double)((k + ns * MLA_T - 1) / (ns * MLA_T));
    const double rounds = (double)(((int64_t)num_q * ns + 255) / 256);
    const double partial_us = ns > 1 ? 2.0 * num_q * ns * (128.0 * 513 * 4) / 5e6 : 0.0;
    const double t = rounds * (4.0 + 2.0 * tiles) + partial_us;
    if (t < best) {
      best = t;
      best_ns = ns;
    }
  }
  return best_ns;
}

static int rows_per_split(int k, int nsplit) {
  int r = (k + nsplit - 1) / nsplit;
  return (r + MLA_T - 1) / MLA_T * MLA_T;
}

int mla_dense_splits(int num_q, int max_nvis) {
  const int64_t max_rows = (int64_t)(MLA_MAX_ROWS + MLA_T) * MLA_T;  // tiles per workgroup x 32 rows
  const int least = (int)((max_nvis + max_rows - 1) / max_rows);
  const int ns = mla_num_splits(num_q, max_nvis, true);
  return ns > least ? ns : (least > 0 ? least : 1);
}

size_t mla_ws_bytes(int num_q, int k, bool decode, bool dense) {
  const int hs = mla_hg_splits(num_q, k, decode, dense);
  if (hs == 1) return 0;  // head groups alone: no partials
  if (hs > 1) return (size_t)num_q * hs * 128 * (512 + 1) * sizeof(float) + 256;
  const int ns = dense ? mla_dense_splits(num_q, k) : mla_num_splits(num_q, k, decode);
  if (ns <= 1) return 0;
  return (size_t)num_q * ns * 128 * (512 + 1) * sizeof(float) + 256;
}

hipError_t launch_mla(const MlaLaunch &a, bool decode, void *ws, hipStream_t st) {
  if (a.num_q == 0) return hipSuccess;
  // Offsets from the descriptor base stay below 4 GiB unless a paged pool is that large.
  const bool wide = a.map.block_shift >= 0 && a.num_rows * (int64_t)ROW_BYTES >= 0xFFFFF000ll - ROW_BYTES;
  const int hs = mla_hg_splits(a.num_q, a.k, decode, a.dense);
  MlaKernelArgs p;
  p.a = a;
  p.nsplit = hs > 0 ? hs : a.dense ? mla_dense_splits(a.num_q, a.k) : mla_num_splits(a.num_q, a.k, decode);
  p.dense = a.dense ? 1 : 0;
  p.rows_per_split = rows_per_split(a.k, p.nsplit);
  p.scale_log2 = a.softmax_scale * LOG2E;
  p.part_o = nullptr;
  p.part_lse = nullptr;
  if (p.nsplit > 1) {
    p.part_o = static_cast<float *>(ws);
    p.part_lse = p.part_o + (size_t)a.num_q * p.nsplit * 128 * 512;
  }
  const int64_t nq8 = (a.num_q + 7) / 8 * 8;  // split blocks are grouped by XCD
  const dim3 grid((unsigned)(p.nsplit == 1 ? (int64_t)a.num_q : nq8 * p.nsplit));
  // Without splits (prefill) the pipelined schedule; with them (decode) the
  // in-order one, whose gathers run two tiles ahead.
  if (hs > 0) {
    const hipError_t e = launch_mla_hg(a, p.scale_log2, wide, hs, p.part_o, p.part_lse, st);
    if (e != hipSuccess) return e;
  } else if (p.nsplit == 1) {
    if (wide)
      hipLaunchKernelGGL((mla_kernel<true, true>), grid, dim3(MLA_THREADS), 0, st, p);
    else
      hipLaunchKernelGGL((mla_kernel<false, true>), grid, dim3(MLA_THREADS), 0, st, p);
  } else {
    if (wide)
      hipLaunchKernelGGL((mla_kernel<true, false>), grid, dim3(MLA_THREADS), 0, st, p);
    else
      hipLaunchKernelGGL((mla_kernel<false, false>), grid, dim3(MLA_THREADS), 0, st, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;
  const dim3 cgrid((unsigned)(nq8 * 64));
  switch (p.nsplit) {
    case 2:
      hipLaunchKernelGGL(mla_combine_kernel<2>, cgrid, dim3(256), 0, st, p.part_o, p.part_lse, 2, a.num_q, a.out, a.lse);
      break;
    case 3:
      hipLaunchKernelGGL(mla_combine_kernel<3>, cgrid, dim3(256), 0, st, p.part_o, p.part_lse, 3, a.num_q, a.out, a.lse);
      break;
    case 4:
      hipLaunchKernelGGL(mla_combine_kernel<4>, cgrid, dim3(256), 0, st, p.part_o, p.part_lse, 4, a.num_q, a.out, a.lse);
      break;
    case 8:
      hipLaunchKernelGGL(mla_combine_kernel<8>, cgrid, dim3(256), 0, st, p.part_o, p.part_lse, 8, a.num_q, a.out, a.lse);
      break;
    default:
      if (p.nsplit <= 16)
        hipLaunchKernelGGL(mla_combine_kernel<-16>, cgrid, dim3(256), 0, st, p.part_o, p.part_lse, p.nsplit,
                           a.num_q, a.out, a.lse);
      else
        hipLaunchKernelGGL(mla_combine_kernel<0>, cgrid, dim3(256), 0, st, p.part_o, p.part_lse, p.nsplit, a.num_q,
                           a.out, a.lse);
  }
  return hipGetLastError();
}

}  // namespace dsa
