// Decode sparse MQA-mode MLA attention by head groups, on bf16 MFMA (gfx950).
//
// The same computation as mla_kernel (page "arXiv'25 | DSA ... DeepSeek-V3.2",
// section 3, third equation, and section 4: every head attends over the one
// shared latent row of each selected position; page "DeepSeekV3.2之DSA", part
// 5.1: softmax(q . [c_kv; k_pe]^T) . c_kv, value = dims 0..511 of the row),
// organised for a decode batch with too few queries to fill the chip with one
// workgroup each.  A query's 128 heads are split into four groups of 32, and
// for small batches (up to 32 queries) its selected rows into S splits as
// well: 4 S workgroups per query.  With S = 1 each workgroup attends over the
// whole selection for its 32 heads and writes final outputs, so the fp32
// partials of a row split and their round trip through memory to a combine
// pass are gone; with S > 1 the splits write (O / l, lse) partials, a quarter
// of what as many row splits over all heads would, that mla_combine_kernel
// merges.  The four head groups of a (query, split) run on one XCD at the same
// time, so a gathered row is read from HBM once and from that XCD's L2 by the
// other three.  Each CU thus takes in all the 1152-byte rows of its split; the
// gather reads every 128-byte line of a row with eight consecutive lanes, the form a CU serves at over 100 GB/s (lanes spread over
// different rows get about a third of that).
//
// Inside a workgroup the four wavefronts take the 16-row tiles in turn (tile j
// to wavefront j % 4).  Each has its own two LDS tile buffers, fills them by
// direct-to-LDS loads and reads only what it loaded itself, so the tile loop
// has no barrier.  Per tile a wavefront
//   * computes S^T = K . Q^T for its 16 rows and the 32 heads with
//     v_mfma_f32_16x16x32_bf16 (two 16-head blocks, 18 K steps of 32 dims; the
//     q fragments stay in registers, 144 VGPRs);
//   * exchanges lane rows with v_permlane16_swap, after which lane l holds
//     head l % 32 for tile rows 8 (l / 32) .. + 7: the online softmax runs on
//     those 8 values (one cross-half max), and their exponentials rounded to
//     bf16 are exactly the A operand of P . V;
//   * adds P . V over its 16 rows to its own O[32 heads, 512] with
//     v_mfma_f32_32x32x16_bf16 (K = the 16 rows, 16 tiles of 32 dims, O in
//     AGPRs), the V operand coming from the transposing read ds_read_b64_tr_b16.
// At the end the four wavefronts' (O, running max, sum) are merged through
// LDS into the workgroup's 32 output rows.
#include "mla_tile.h"

namespace dsa {

constexpr int HG_T = 16;                          // rows per tile
constexpr int HG_TILE_BYTES = HG_T * ROW_BYTES;   // 18432
constexpr int HG_PARTS = HG_TILE_BYTES / 1024;    // 18 gather instructions per tile (16 B per lane)
constexpr int HG_GROUPS = 4;                      // head groups of 32 per query
constexpr int HG_OSTRIDE = 264;                   // floats per head row in the merge area (bank spread)
constexpr int HG_OREGION = 32 * HG_OSTRIDE * 4;   // one wavefront's half of O in the merge area
static_assert(HG_PARTS * 1024 == HG_TILE_BYTES && HG_PARTS == 18, "tile = 2 row groups x 9 lines");
static_assert(2 * HG_OREGION <= MLA_WAVES * HG_TILE_BYTES, "two merge regions per tile-buffer array");

struct MlaHgArgs {
  MlaLaunch a;
  float scale_log2;
  int nsplit;          // row splits S per head group
  int rows_per_split;  // a multiple of HG_T (all k rows when S = 1)
  float *part_o;       // [num_q, S, 128, 512] (S > 1)
  float *part_lse;     // [num_q, S, 128]
};

// Tile layout in LDS: 18 blocks of 1 KiB.  Block lc + 9 rg holds the 128-byte
// line lc (16-byte chunks 8 lc .. 8 lc + 7) of tile rows 8 rg .. 8 rg + 7;
// chunk c of row r sits in slot 8 (r & 7) + ((c & 7) ^ x(r)) of its block,
// x(r) = 4 (m & 1) + (m >> 1) for m = r >> 1.  A gather instruction fills one
// block (lane i: slot i), so its eight lanes 8k .. 8k + 7 read one whole line
// of one row.  With 64 four-byte banks (16 slot positions), x keeps both read
// patterns free of conflicts:
//  * the QK read of a 16-lane group takes one chunk of all 16 rows: r & 1 and
//    the eight values of (c & 7) ^ x(r) over r >> 1 give 16 slot positions;
//  * the transposing PV read of 32 lanes takes rows 4m .. 4m + 3 of four
//    chunks 4n .. 4n + 3: rows r and r + 2 differ in bit 2 of x, which moves
//    their four chunks to the other half of the line's slot positions.
__device__ __forceinline__ int hg_xor(int r) {
  const int m = (r >> 1) & 7;
  return ((m & 1) << 2) | (m >> 1);
}
__device__ __forceinline__ int hg_off(int r, int c) {
  return 1024 * ((c >> 3) + 9 * (r >> 3)) + 16 * (8 * (r & 7) + ((c & 7) ^ hg_xor(r)));
}

// s_waitcnt vmcnt(N), other counters untouched.
template <int N>
__device__ __forceinline__ void hg_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// S^T chain on a 16x16 accumulator (VGPRs, next to the softmax that reads it;
// the AGPRs hold O).
__device__ __forceinline__ void mfma16_first(v4f &acc, const uint4 &a, const uint4 &b) {
  const v4i_t va = __builtin_bit_cast(v4i_t, a), vb = __builtin_bit_cast(v4i_t, b);
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(va), "v"(vb));
}
__device__ __forceinline__ void mfma16(v4f &acc, const uint4 &a, const uint4 &b) {
  const v4i_t va = __builtin_bit_cast(v4i_t, a), vb = __builtin_bit_cast(v4i_t, b);
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(va), "v"(vb));
}
// Covers the MFMA-write -> VALU-read distance before the lane swaps read S.
__device__ __forceinline__ void mfma16_drain(v4f &a, v4f &b) {
  asm("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(a), "+v"(b));
}

template <bool WIDE>
__global__ __launch_bounds__(MLA_THREADS, 1) void mla_hg_kernel(MlaHgArgs p) {
  const MlaLaunch &a = p.a;
  // Unit u = (query, split) runs its four head groups on XCD u % 8 (block b
  // runs on XCD b % 8), where they share the gathered rows in L2.
  const int y = blockIdx.x >> 3;
  const int u = (y / HG_GROUPS) * 8 + (blockIdx.x & 7);
  const int hg = y % HG_GROUPS;
  const int q = u / p.nsplit, sp = u % p.nsplit;
  if (q >= a.num_q) return;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;  // wave-uniform
  const int g = lane >> 5, c = lane & 31;

  // Tile buffers: parity 0 and 1 of every wavefront in two separately declared
  // arrays, so that the compiler sees a read of one never racing with the
  // direct-to-LDS fill of the other.  After the loop they hold the merge.
  __shared__ __attribute__((aligned(16))) uint8_t tb0[MLA_WAVES][HG_TILE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t tb1[MLA_WAVES][HG_TILE_BYTES];
  // Physical row per selected position (bit 31: outside [0, n_vis)); the tail
  // keeps the masked reads of a partial last tile in bounds.
  __shared__ __attribute__((aligned(16))) uint32_t prow[MLA_MAX_ROWS + HG_T];
  __shared__ __attribute__((aligned(16))) float aex[MLA_WAVES][32];  // per-head factors, own slot
  __shared__ float mw[MLA_WAVES][32], lw[MLA_WAVES][32];            // (max, sum) per head, per wavefront
  __shared__ int bad_w[MLA_WAVES];

  const int nvis = a.q_nvis[q];
  int cnt = a.count ? a.count[q] : a.k;
  cnt = max(0, min(cnt, min(a.k, nvis)));
  const int r0 = sp * p.rows_per_split;
  const int nrows = max(0, min(cnt, r0 + p.rows_per_split) - r0);
  const int seq = a.q_seq[q];
  const uint32_t row0 = a.map.block_shift < 0 ? (uint32_t)a.map.seq_row0[seq] : 0u;

  // q of the group's 32 heads, as B fragments of S^T = K . Q^T: lane l holds
  // head 32 hg + 16 hb + l % 16, dims 32 ks + 8 (l / 16) .. + 7.  Every
  // wavefront needs all of them.  The group's 36 KiB are read once, by
  // direct-to-LDS loads of whole lines (requested after the position loads,
  // so that the latencies overlap), into the second tile buffers (free until
  // the first step), and read from there by each wavefront.
  constexpr int Q_PARTS = 32 * ROW_BYTES / 1024 / MLA_WAVES;  // 9 KiB-loads per wavefront
  static_assert(Q_PARTS * 1024 * MLA_WAVES == 32 * ROW_BYTES && 32 * ROW_BYTES <= sizeof(tb1), "q stage fits");
  uint4 qb[2][18];
  // The buffer form, as for the gathers: the compiler counts these loads
  // exactly, so waits on the position loads issued before them need not wait
  // for them (the global form made that wait drain every load in flight).
  auto load_q = [&]() {
    const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.q + ((int64_t)q * 128 + 32 * hg) * 576), (short)0, 0xFFFFFFFF, 0x00020000);
#pragma unroll
    for (int j = 0; j < Q_PARTS; ++j) {
      const int part = wave * Q_PARTS + j;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qrs, (lds_void *)(&tb1[0][0] + 1024 * part), 16,
                                               1024 * part + 16 * lane, 0, 0, 0);
    }
  };

  // Selected positions -> physical rows (all of a thread's positions, then
  // all their block-table entries, every lane issuing the same loads).  A
  // position outside [0, n_vis) breaks the contract; it is read from position
  // 0 (in bounds, finite) and masked.
  constexpr int PER_THREAD = MLA_MAX_ROWS / MLA_THREADS;
  int bad = 0;
  if (nrows > 0) {  // block-uniform
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
    if (a.map.block_shift < 0) {
#pragma unroll
      for (int j = 0; j < PER_THREAD; ++j) row[j] = row0 + (uint32_t)pos[j];
    } else {
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
  // Publish the row table (a bare barrier after the LDS writes: the q loads
  // stay in flight).
  {
    const int wbad = __ballot(bad) != 0ull ? 1 : 0;
    if (lane == 0) bad_w[wave] = wbad;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
  const bool any_bad = (bad_w[0] | bad_w[1] | bad_w[2] | bad_w[3]) != 0;
  static_assert(MLA_WAVES == 4, "any_bad reads four wavefront words");
  auto bare_barrier = []() {  // LDS operations done, loads (and gathers) left in flight
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // This wavefront's tiles: j = wave + 4 i, i < ntw.
  const int nt16 = (nrows + HG_T - 1) / HG_T;
  const int ntw = nt16 > wave ? (nt16 - wave + MLA_WAVES - 1) / MLA_WAVES : 0;

  const uint32_t brow = __builtin_amdgcn_readfirstlane((!WIDE && a.map.block_shift < 0) ? row0 : 0u);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(a.kv + (size_t)brow * 576), (short)0, 0xFFFFFFFF, 0x00020000);

  // Gather of tile j into buf: instruction lc + 9 rg, lane i takes tile row
  // 8 rg + (i >> 3), bytes 128 lc + 16 ((i & 7) ^ x(row)) of it (one whole
  // line per eight lanes).  Rows past the selection repeat the last row
  // (finite, masked out of the softmax).
  const int gr0 = lane >> 3, gr1 = 8 + (lane >> 3);
  const int gb0 = 16 * ((lane & 7) ^ hg_xor(gr0)), gb1 = 16 * ((lane & 7) ^ hg_xor(gr1));
  auto issue_tile = [&](const int j, uint8_t *buf) {
    const uint32_t row_a = prow[min(HG_T * j + gr0, nrows - 1)] & ~INVALID_ROW;
    const uint32_t row_b = prow[min(HG_T * j + gr1, nrows - 1)] & ~INVALID_ROW;
#pragma unroll
    for (int i = 0; i < HG_PARTS; ++i) {
      const int rg = i / 9, lc = i % 9;
      const uint32_t row = rg ? row_b : row_a;
      const int boff = 128 * lc + (rg ? gb1 : gb0);
      if (WIDE) {
        const uint16_t *src = a.kv + (size_t)row * 576 + (boff >> 1);
        __builtin_amdgcn_global_load_lds(src, (lds_void *)(buf + 1024 * i), 16, 0, 0);
      } else {
        const uint32_t voff = (row - brow) * ROW_BYTES + (uint32_t)boff;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(buf + 1024 * i), 16, voff, 0, 0, 0);
      }
    }
  };

  // Per-lane LDS offsets.  QK step ks: lane l reads row l % 16, chunk
  // 4 ks + l / 16, at qk_base[ks & 1] + 1024 (ks >> 1).  PV tile nt (dims
  // 32 nt .. +31, chunks 4 nt .. +3), ds_read_b64_tr_b16: in each 16-lane
  // group, lane ti points at row ti / 4 of a 4-row set and 4 dims (8 bytes) of
  // the group's 16; the read hands lane l dim l % 32 of the tile for the set's
  // 4 rows.  Lane l's two sets are rows 8 (l / 32) + 0..3 and + 4..7:
  // tr_base[nt & 1][set] + 1024 (nt >> 1).
  int qk_base[2];
#pragma unroll
  for (int pp = 0; pp < 2; ++pp) qk_base[pp] = hg_off(lane & 15, 4 * pp + (lane >> 4));
  const int ti = lane & 15, th = (lane >> 4) & 1;
  int tr_base[2][2];
#pragma unroll
  for (int odd = 0; odd < 2; ++odd)
#pragma unroll
    for (int set = 0; set < 2; ++set)
      tr_base[odd][set] = hg_off(8 * g + 4 * set + (ti >> 2), 4 * odd + 2 * th + ((ti & 3) >> 1)) + 8 * (ti & 1);

  // O[nt]: the 32 heads x dims 32 nt .. +31; lane l holds dim 32 nt + l % 32
  // of heads 8 i + 4 (l / 32) + j in register 4 i + j.
  v16f o[16];
#pragma unroll
  for (int nt = 0; nt < 16; ++nt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[nt][i] = 0.0f;
  float m_ref = -INFINITY, l_run = 0.0f;  // head c (both lane halves agree on m_ref)

  auto qk = [&](const uint8_t *buf, v4f &s0, v4f &s1) {
    constexpr int AH = 4;
    uint4 kf[AH + 1];
#pragma unroll
    for (int ks = 0; ks < AH; ++ks)
      kf[ks] = *reinterpret_cast<const uint4 *>(buf + qk_base[ks & 1] + 1024 * (ks >> 1));
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      if (ks + AH < 18)
        kf[(ks + AH) % (AH + 1)] =
            *reinterpret_cast<const uint4 *>(buf + qk_base[(ks + AH) & 1] + 1024 * ((ks + AH) >> 1));
      const uint4 kk = kf[ks % (AH + 1)];
      if (ks == 0) {
        mfma16_first(s0, kk, qb[0][0]);
        mfma16_first(s1, kk, qb[1][0]);
      } else {
        mfma16(s0, kk, qb[0][ks]);
        mfma16(s1, kk, qb[1][ks]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    mfma16_drain(s0, s1);
  };

  // PV's V fragments (dims 32 nt .. +31 of the tile's 16 rows) by the
  // transposing read.  The first PV_AH are read before the softmax, which
  // hides their latency.
  constexpr int PV_AH = 4;
  auto v_frag_at = [&](const uint8_t *buf, const int nt) {
    const int o0 = tr_base[nt & 1][0] + 1024 * (nt >> 1), o1 = tr_base[nt & 1][1] + 1024 * (nt >> 1);
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)(buf + o0));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)(buf + o1));
    const uint2 ulo = __builtin_bit_cast(uint2, lo), uhi = __builtin_bit_cast(uint2, hi);
    return make_uint4(ulo.x, ulo.y, uhi.x, uhi.y);
  };
  auto pv = [&](const uint8_t *buf, const uint4 &pa, const uint4 (&v0)[PV_AH]) {
    constexpr int AH = PV_AH;
    auto v_frag = [&](const int nt) { return v_frag_at(buf, nt); };
    uint4 vf[AH + 1];
#pragma unroll
    for (int nt = 0; nt < AH; ++nt) vf[nt] = v0[nt];
#pragma unroll
    for (int nt = 0; nt < 16; ++nt) {
      if (nt + AH < 16) vf[(nt + AH) % (AH + 1)] = v_frag(nt + AH);
      o[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf(pa), as_bf(vf[nt % (AH + 1)]), o[nt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

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

  // Step i of this wavefront: tile j = wave + 4 i from buf; the next tile's
  // gather goes into nbuf (free: this wavefront finished reading it in step
  // i - 1).  Loads complete in issue order, so tile i has landed once at most
  // the next tile's 18 loads are outstanding.  Past the last tile the step
  // still issues a gather (of the last tile again, whose rows are in the
  // caches), so that the instruction stream has no branch here and the wait
  // has one count.
  auto step = [&](const int i, const uint8_t *buf, uint8_t *nbuf) {
    const int j = wave + MLA_WAVES * i;
    issue_tile(wave + MLA_WAVES * min(i + 1, ntw - 1), nbuf);
    hg_wait_vm<HG_PARTS>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    v4f s0, s1;
    qk(buf, s0, s1);
    uint4 v0[PV_AH];
#pragma unroll
    for (int nt = 0; nt < PV_AH; ++nt) v0[nt] = v_frag_at(buf, nt);
    // Lane rows: after the swap lane l holds head 32 hg + l % 32, tile rows
    // 8 (l / 32) + e in z[e] (e = 0..7).
    float z[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(s0[e]), __float_as_uint(s1[e]), false, false);
      z[e] = __uint_as_float(r[0]);
      z[4 + e] = __uint_as_float(r[1]);
    }
    // Online softmax in log2 units (z = scale_log2 * s), as in mla_kernel:
    // the reference max moves only when a head's tile max exceeds it by more
    // than RESCALE_LOG2.  Rows past the selection, or flagged outside
    // [0, n_vis), are -inf.
    float tmax, zscale;
    if (!any_bad && HG_T * j + HG_T <= nrows) {
      const float mx = max3f(max3f(z[0], z[1], z[2]), max3f(z[3], z[4], z[5]), fmaxf(z[6], z[7]));
      tmax = xhalf_max(mx) * p.scale_log2;
      zscale = p.scale_log2;
    } else {
      tmax = -INFINITY;
      const int rb = HG_T * j + 8 * g;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool ok = (rb + e < nrows) && !(prow[rb + e] & INVALID_ROW);
        z[e] = ok ? z[e] * p.scale_log2 : -INFINITY;
        tmax = fmaxf(tmax, z[e]);
      }
      tmax = xhalf_max(tmax);
      zscale = 1.0f;
    }
    const bool resc = __ballot(tmax > m_ref + RESCALE_LOG2) != 0ull;
    const float m_new = resc ? fmaxf(m_ref, tmax) : m_ref;
    const float alpha = resc ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;  // 0 while m_ref = -inf
    l_run *= alpha;
    m_ref = m_new;
    const float nmref = (m_ref == -INFINITY) ? 0.0f : -m_ref;
    float ex[8], psum = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ex[e] = __builtin_amdgcn_exp2f(fmaf(z[e], zscale, nmref));
      psum += ex[e];
    }
    l_run += psum;
    const uint4 pa = make_uint4(pack_bf16(ex[0], ex[1]), pack_bf16(ex[2], ex[3]), pack_bf16(ex[4], ex[5]),
                                pack_bf16(ex[6], ex[7]));
    if (i > 0 && resc) {  // O is still zero on the first tile
      if (g == 0) aex[wave][c] = alpha;  // own slot: no other wavefront reads it
      rescale_o(aex[wave]);
    }
    pv(buf, pa, v0);
  };

  if (ntw > 0) issue_tile(wave, tb0[wave]);
  // q through the stage: the gather of the first tile is already on its way
  // (its loads are younger than those of q, so waiting for q leaves it).
  {
    if (ntw > 0) hg_wait_vm<HG_PARTS>(); else hg_wait_vm<0>();
    bare_barrier();
    const uint8_t *sb = &tb1[0][0] + (lane & 15) * ROW_BYTES + 16 * (lane >> 4);
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int ks = 0; ks < 18; ++ks)
        qb[hb][ks] = *reinterpret_cast<const uint4 *>(sb + hb * 16 * ROW_BYTES + 64 * ks);
    bare_barrier();  // every wavefront has its q before any gather refills the stage
  }
  for (int i = 0; i < ntw; i += 2) {
    step(i, tb0[wave], tb1[wave]);
    if (i + 1 < ntw) step(i + 1, tb1[wave], tb0[wave]);
  }
  hg_wait_vm<0>();  // nothing of this wavefront's may still be landing in LDS

  // Merge the four wavefronts: per head, M = the largest running max and
  // L = the sum of l_w 2^(m_w - M); wavefront w's O scales by 2^(m_w - M) / L.
  const float l_tot = xhalf_sum(l_run);
  if (g == 0) {
    mw[wave][c] = m_ref;
    lw[wave][c] = l_tot;
  }
  __syncthreads();  // also: every wavefront is done with its tile buffers
  if (g == 0) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < MLA_WAVES; ++w) M = fmaxf(M, mw[w][c]);
    float L = 0.0f;
#pragma unroll
    for (int w = 0; w < MLA_WAVES; ++w)
      L += (mw[w][c] == -INFINITY) ? 0.0f : lw[w][c] * __builtin_amdgcn_exp2f(mw[w][c] - M);
    aex[wave][c] = (L > 0.0f) ? __builtin_amdgcn_exp2f(m_ref - M) / L : 0.0f;
    const float lse_v = (L > 0.0f) ? M * LN2 + logf(L) : -INFINITY;
    if (wave == 0 && p.nsplit > 1)
      p.part_lse[((int64_t)q * p.nsplit + sp) * 128 + 32 * hg + c] = lse_v;
    else if (wave == 0 && a.lse)
      a.lse[(int64_t)q * 128 + 32 * hg + c] = lse_v;
  }
  float fac[16];
  read_head_values(aex[wave], g, fac);  // this wavefront's own slot

  // Two rounds of 256 dims: every wavefront stores its scaled O half into its
  // region, then wavefront w sums heads 8w .. 8w+7 over the four regions and
  // writes them out (16 bytes per lane).
  auto region = [&](const int w) -> float * {
    uint8_t *base = (w < 2) ? &tb0[0][0] : &tb1[0][0];
    return reinterpret_cast<float *>(base + (w & 1) * HG_OREGION);
  };
  float *own = region(wave);
  float *out = (p.nsplit > 1 ? p.part_o + ((int64_t)q * p.nsplit + sp) * 128 * 512 : a.out + (int64_t)q * 128 * 512) +
               (int64_t)32 * hg * 512;
#pragma unroll
  for (int R = 0; R < 2; ++R) {
#pragma unroll
    for (int nt = 8 * R; nt < 8 * R + 8; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          own[(8 * i + 4 * g + jj) * HG_OSTRIDE + 32 * (nt - 8 * R) + c] =
              read_scaled(o[nt][4 * i + jj], fac[4 * i + jj]);
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < 8; ++hh) {
      const int h = 8 * wave + hh;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int w = 0; w < MLA_WAVES; ++w) {
        const float4 v = *reinterpret_cast<const float4 *>(region(w) + h * HG_OSTRIDE + 4 * lane);
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
      }
      // Non-temporal, both the final output (not read again in the step) and
      // the split partials (read once, by the combine).
      typedef float ntf4 __attribute__((ext_vector_type(4)));
      const ntf4 v4 = {acc.x, acc.y, acc.z, acc.w};
      __builtin_nontemporal_store(v4, reinterpret_cast<ntf4 *>(out + (int64_t)h * 512 + 256 * R + 4 * lane));
    }
    if (R == 0) __syncthreads();
  }
}

// Row splits S per head group for a decode batch (0: the head-group kernel is
// not used).  48 to 64 queries fill 192 to 256 CUs with S = 1 and need no
// partials.  Up to 32 queries take the largest S with 4 S workgroups per query
// still at most 256 in all and at least 128 rows per split (one round on the
// chip, a quarter of the row-split kernel's partial bytes at the same count).
// 33 to 47 queries would leave a third of the CUs idle with S = 1 and take
// two rounds with S = 2, so they stay on the row-split kernel.
int mla_hg_splits(int num_q, int k, bool decode, bool dense) {
  if (!decode || dense || num_q <= 0 || num_q > 64 || k < 128) return 0;
  if (num_q >= 48) return 1;
  if (num_q > 32) return 0;
  return std::min(256 / (HG_GROUPS * num_q), k / 128);
}

int mla_hg_rows_per_split(int k, int nsplit) {
  const int r = (k + nsplit - 1) / nsplit;
  return (r + HG_T - 1) / HG_T * HG_T;
}

hipError_t launch_mla_hg(const MlaLaunch &a, float scale_log2, bool wide, int nsplit, float *part_o,
                         float *part_lse, hipStream_t st) {
  MlaHgArgs p;
  p.a = a;
  p.scale_log2 = scale_log2;
  p.nsplit = nsplit;
  p.rows_per_split = mla_hg_rows_per_split(a.k, nsplit);
  p.part_o = part_o;
  p.part_lse = part_lse;
  const int64_t units8 = ((int64_t)a.num_q * nsplit + 7) / 8 * 8;  // (query, split) units, by XCD
  const dim3 grid((unsigned)(units8 * HG_GROUPS));
  if (wide)
    hipLaunchKernelGGL(mla_hg_kernel<true>, grid, dim3(MLA_THREADS), 0, st, p);
  else
    hipLaunchKernelGGL(mla_hg_kernel<false>, grid, dim3(MLA_THREADS), 0, st, p);
  return hipGetLastError();
}

}  // namespace dsa
