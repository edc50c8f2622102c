// Backward of the lightning-indexer score into its inputs.
//
// Page "arXiv'25 | DSA ... DeepSeek-V3.2", section 3 (first equation: the
// score I[t,s] = sum_j w[t,j] ReLU(q[t,j] . k[s])) and section 5 (only the
// indexer learns from its alignment loss; its inputs are detached from the
// main model).  Given g[t,s] = dL/dI[t,s] over each query's set, the gradients
// with respect to the head weights and the dequantised FP8 query and key
// (qh = q_scale * q8, kh = k_scale * k8; the quantiser passes gradients
// unchanged; the derivative of ReLU at 0 is taken as 0):
//   dw[t,j]     = q_scale[t,j] * sum_s c_s * max(D_js, 0)
//   dqh[t,j,:]  = w[t,j] * sum_s [D_js > 0] c_s k8_s
//   dkh[r(s),:] += g_s * sum_j [D_js > 0] e_j q8_j
// with D_js = q8_j . k8_s (exact FP8 products, summed in fp32),
// c_s = g_s * k_scale_s and e_j = w[t,j] * q_scale[t,j].
//
// One block (4 wavefronts) = one query and a run of up to 2048 members of its
// set, in tiles of 64 keys:
//   * D on FP8 MFMA (v_mfma_scale_f32_16x16x128_f8f6f4), as in the forward
//     indexer: wavefront w scores keys 16w .. 16w+15 of the tile against all 64
//     heads, the keys loaded straight into B-operand registers (the next tile's
//     one tile ahead);
//   * the gates [D > 0] go to LDS as [key][head] bf16 matrices: times c_s,
//     split into bf16 hi + lo (hi = bf16(c), lo = bf16(c - hi); hi + lo is
//     within 2^-17 |c| of c), for dq, and as plain 0/1 for dk; the keys go
//     as a [key][dim] bf16 matrix (FP8 E4M3 values are exact in bf16).  Both
//     contractions then run on bf16 MFMA (v_mfma_f32_32x32x16_bf16) with
//     products exact in fp32.  Each lane writes whole 8- and 16-byte pieces
//     of its key's rows;
//   * dkh of the tile = gates[key][head] . (e q8)[head][dim], whose B operand
//     (hi + lo) stays in registers for the whole block, then times g_s into dk
//     by fp32 atomic adds (a key row may belong to several queries);
//   * dqh += (gates c)^T[head][key] . k8[key][dim] (hi and lo) accumulates in
//     registers over the block's tiles, both operands read key-major through
//     the transposing LDS read ds_read_b64_tr_b16; dw accumulates in-lane
//     from D.
// Wavefront w owns the 32 x 64 quarter (rows 32 (w & 1), columns 64 (w >> 1))
// of both 64 x 128 products.  The 16-byte chunks of each LDS row are XOR-
// swizzled by the row so that the writes, the 16-byte reads of 16 consecutive
// rows and the transposing reads of 4 rows x 64 bytes all spread over the 64
// banks without conflicts.
#include "device_util.h"
#include "dsa_internal.h"

namespace dsa {

constexpr int IB_THREADS = 256;
constexpr int IB_TILE = 64;                 // keys per tile
constexpr int IB_MAX_MEMBERS = 2048;        // members per block
constexpr int IB_MIN_BLOCKS = 1024;
constexpr uint32_t IB_INVALID = 0x80000000u;
constexpr uint16_t BF16_ONE = 0x3F80;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));

// Byte offset of byte b of row r in the [key][head] gate matrix (128-byte
// rows) and in the [key][dim] c k8 matrices (256-byte rows): the 16-byte chunk
// index is XORed with a function of the row's low four bits.
__device__ __forceinline__ int gate_off(int r, int b) {
  const int sw = (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  return r * 128 + (((b >> 4) ^ sw) << 4) + (b & 15);
}
__device__ __forceinline__ int ck_off(int r, int b) {
  const int sw = ((r & 3) << 2) | ((r >> 2) & 3);
  return r * 256 + (((b >> 4) ^ sw) << 4) + (b & 15);
}

struct IndexerBwdArgs {
  IndexerBwdLaunch a;
  int nchunk;
  int members;  // per block, a multiple of IB_TILE
};

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);  // round to nearest even
}
__device__ __forceinline__ float bf16_value(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
// Two fp32 values as a bf16 pair (round to nearest even), the first in the low half.
__device__ __forceinline__ uint32_t pk_bf16(float2_t v) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ bf16x8_t as_bf8(const uint4 &u) { return __builtin_bit_cast(bf16x8_t, u); }
// The four FP8 E4M3 bytes of word v as fp32 (exact), lowest byte first.
__device__ __forceinline__ void fp8x4(uint32_t v, float *f) {
  f[0] = __builtin_amdgcn_cvt_f32_fp8((int)v, 0);
  f[1] = __builtin_amdgcn_cvt_f32_fp8((int)v, 1);
  f[2] = __builtin_amdgcn_cvt_f32_fp8((int)v, 2);
  f[3] = __builtin_amdgcn_cvt_f32_fp8((int)v, 3);
}

__global__ __launch_bounds__(256) void ib_zero_kernel(float *__restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// The dense instantiation is held to three workgroups per CU (its LDS allows
// three; uncapped, the compiler's register use would allow two).
template <bool DK>
__global__ __launch_bounds__(IB_THREADS, DK ? 1 : 3) void indexer_bwd_kernel(IndexerBwdArgs p) {
  const IndexerBwdLaunch &a = p.a;
  const int t = blockIdx.x / p.nchunk;
  const int chunk = blockIdx.x - t * p.nchunk;
  const int nvis = a.q_nvis[t];
  int nset = nvis;
  if (a.idx) {
    const int c = a.count ? a.count[t] : a.k;
    nset = max(0, min(c, min(a.k, nvis)));
  }
  const int m0 = chunk * p.members;
  const int nmem = min(p.members, nset - m0);
  if (nmem <= 0) return;  // block-uniform

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int l15 = lane & 15, g4 = lane >> 4;    // FP8 MFMA lane split
  const int l31 = lane & 31, g2 = lane >> 5;    // bf16 32x32 MFMA lane split
  const int half = wave & 1, dn0 = 2 * (wave >> 1);

  __shared__ __attribute__((aligned(16))) uint8_t gts[DK ? IB_TILE * 128 : 16];  // [key][head] gates (dk)
  __shared__ __attribute__((aligned(16))) uint8_t ghs[IB_TILE * 128];  // [key][head] gates x c_s, hi
  __shared__ __attribute__((aligned(16))) uint8_t gls[IB_TILE * 128];  // [key][head] gates x c_s, lo
  __shared__ __attribute__((aligned(16))) uint8_t kbs[IB_TILE * 256];  // [key][dim] k8 as bf16
  // The dense instantiation (no dk) keeps no g_s and no plain gates, so that
  // three workgroups fit a CU's LDS.
  constexpr int PER = IB_MAX_MEMBERS / IB_THREADS;
  __shared__ uint32_t mrow[IB_MAX_MEMBERS];           // physical row (IB_INVALID: not a member)
  __shared__ float mg[DK ? IB_MAX_MEMBERS : 1];       // g_s (0 for non-members)
  __shared__ float mc[IB_MAX_MEMBERS];                // c_s = g_s * k_scale_s
  __shared__ float dwred[4][64];

  // Members -> rows, g and c, all loads issued before any is used.  A
  // non-member (outside [0, n_vis), or past the run) reads position 0's row
  // with g = 0, so it adds nothing, and its dk atomics are skipped.
  const int seq = a.q_seq[t];
  const int ntile = (nmem + IB_TILE - 1) / IB_TILE;
  {
    int pos[PER];
    float gv[PER];
    const int lastm = nmem - 1;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = min(tid + j * IB_THREADS, lastm);
      pos[j] = a.idx ? a.idx[(int64_t)t * a.k + m0 + i] : m0 + i;
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = min(tid + j * IB_THREADS, lastm);
      const bool ok = pos[j] >= 0 && pos[j] < nvis;
      gv[j] = a.grad[(int64_t)t * a.ld_grad + (a.idx ? m0 + i : (ok ? pos[j] : 0))];
      pos[j] = ok ? pos[j] : -1;
    }
    uint32_t row[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) row[j] = (uint32_t)phys_row(a.map, seq, max(pos[j], 0));
    float ks[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) ks[j] = a.k_scale[row[j]];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = tid + j * IB_THREADS;
      if (i < ntile * IB_TILE) {
        const bool ok = i < nmem && pos[j] >= 0;
        mrow[i] = row[j] | (ok ? 0u : IB_INVALID);
        if (DK) mg[i] = ok ? gv[j] : 0.0f;
        mc[i] = ok ? gv[j] * ks[j] : 0.0f;
      }
    }
  }

  // Query-side operands.  A of the FP8 product: heads 16 mt + l15, bytes
  // [32 g4, +32).  e_j = w_j q_scale_j.
  const uint8_t *qp = a.q8 + (int64_t)t * (64 * 128);
  v8i qa[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) qa[mt] = load32(qp + (16 * mt + l15) * 128 + 32 * g4);
  // B of the dk product, [head][dim] = e_j q8[j][dim] as hi + lo: lane holds
  // dim 32 (dn0 + nt) + l31, heads 16 ks + 8 g2 .. + 7.
  uint4 bkh[2][4], bkl[2][4];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (!DK) break;
      const int d = 32 * (dn0 + nt) + l31;
      uint16_t hi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = 16 * ks + 8 * g2 + e;
        const float qs = a.q_scale ? a.q_scale[(int64_t)t * 64 + j] : 1.0f;
        const float x = a.w[(int64_t)t * 64 + j] * qs * __builtin_amdgcn_cvt_f32_fp8((int)qp[j * 128 + d], 0);
        hi[e] = bf16_bits(x);
        lo[e] = bf16_bits(x - bf16_value(hi[e]));
      }
      bkh[nt][ks] = make_uint4(hi[0] | (uint32_t)hi[1] << 16, hi[2] | (uint32_t)hi[3] << 16,
                               hi[4] | (uint32_t)hi[5] << 16, hi[6] | (uint32_t)hi[7] << 16);
      bkl[nt][ks] = make_uint4(lo[0] | (uint32_t)lo[1] << 16, lo[2] | (uint32_t)lo[3] << 16,
                               lo[4] | (uint32_t)lo[5] << 16, lo[6] | (uint32_t)lo[7] << 16);
    }
  __syncthreads();  // member table ready

  // Byte offsets into the tile matrices.  Writes: the gates of heads
  // 16 mt + 4 g4 .. + 3 of key kl (8 bytes), c k8 of dims 32 g4 + 8 j .. + 7
  // of key kl (16 bytes).  Transposing reads (dq's A from the gates, its B
  // from c k8): lane 32 g2 + 16 th + ti points at row ti >> 2 of the key set
  // 16 ks + 8 g2 + 4 hh .. + 3 and bytes 8 (ti & 3) of its group's 32-byte
  // column span, and receives column 16 th + ti of those 4 keys.  The
  // swizzles do not depend on ks, so ks moves the offsets by whole rows.
  const int kl = 16 * wave + l15;  // this lane's key within a tile
  const int ti = lane & 15, th = (lane >> 4) & 1;
  int gw_off[4], cw_off[4], ga_off[2], cb_off[2][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) gw_off[mt] = gate_off(kl, 32 * mt + 8 * g4);
#pragma unroll
  for (int j = 0; j < 4; ++j) cw_off[j] = ck_off(kl, 64 * g4 + 16 * j);
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int r = 8 * g2 + 4 * hh + (ti >> 2);
    ga_off[hh] = gate_off(r, 64 * half + 32 * th + 8 * (ti & 3));
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) cb_off[hh][nt] = ck_off(r, 64 * (dn0 + nt) + 32 * th + 8 * (ti & 3));
  }
  auto tr_pair = [](const uint8_t *p0, const uint8_t *p1) {
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)p0);
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)p1);
    const uint2 ulo = __builtin_bit_cast(uint2, lo), uhi = __builtin_bit_cast(uint2, hi);
    return make_uint4(ulo.x, ulo.y, uhi.x, uhi.y);
  };

  v16f dq[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[nt][r] = 0.0f;
  float dwa[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) dwa[mt][i] = 0.0f;

  // Keys of tile tt for this wavefront: member 64 tt + 16 wave + l15, bytes
  // [32 g4, +32) of its row (non-members read a valid row, see above).
  auto load_keys = [&](int tt) {
    const int mi = min(IB_TILE * tt + 16 * wave + l15, IB_TILE * ntile - 1);
    const uint32_t r = mrow[mi] & ~IB_INVALID;
    return load32(a.k8 + (int64_t)r * 128 + 32 * g4);
  };

  auto tile = [&](const int tt, const v8i &kb) {
    const int mk = IB_TILE * tt + 16 * wave + l15;  // this lane's key (member index)
    const float ck = mc[mk];
    v4f d[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) d[mt] = mfma_fp8_16x16x128(qa[mt], kb, v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) dwa[mt][i] = fmaf(fmaxf(d[mt][i], 0.0f), ck, dwa[mt][i]);

    // c_s as bf16 hi + lo (c - hi is exact in fp32); hi + lo is within
    // 2^-17 |c| of c.
    const uint32_t chb = bf16_bits(ck);
    const uint32_t clb = bf16_bits(ck - bf16_value((uint16_t)chb));
    __syncthreads();  // the previous tile's fragment reads are done
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      bool on[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) on[i] = d[mt][i] > 0.0f;
      if (DK)
        *reinterpret_cast<uint2 *>(gts + gw_off[mt]) =
            make_uint2((on[0] ? BF16_ONE : 0u) | (on[1] ? (uint32_t)BF16_ONE << 16 : 0u),
                       (on[2] ? BF16_ONE : 0u) | (on[3] ? (uint32_t)BF16_ONE << 16 : 0u));
      *reinterpret_cast<uint2 *>(ghs + gw_off[mt]) =
          make_uint2((on[0] ? chb : 0u) | (on[1] ? chb << 16 : 0u), (on[2] ? chb : 0u) | (on[3] ? chb << 16 : 0u));
      *reinterpret_cast<uint2 *>(gls + gw_off[mt]) =
          make_uint2((on[0] ? clb : 0u) | (on[1] ? clb << 16 : 0u), (on[2] ? clb : 0u) | (on[3] ? clb << 16 : 0u));
    }
    // k8 of this lane's key as bf16 (exact), dims 32 g4 + 8 j .. + 7 (key
    // words 2 j, 2 j + 1).
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t u[4];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int v = kb[2 * j + h2];
        u[2 * h2] = pk_bf16(__builtin_amdgcn_cvt_pk_f32_fp8(v, false));
        u[2 * h2 + 1] = pk_bf16(__builtin_amdgcn_cvt_pk_f32_fp8(v, true));
      }
      *reinterpret_cast<uint4 *>(kbs + cw_off[j]) = make_uint4(u[0], u[1], u[2], u[3]);
    }
    __syncthreads();  // gates and k8 visible

    // dkh of the tile's keys 32 half .. + 31, dims 32 (dn0 + nt) + l31.
    v16f dk[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) dk[nt][r] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (!DK) break;
      const uint4 ga = *reinterpret_cast<const uint4 *>(gts + gate_off(32 * half + l31, 32 * ks + 16 * g2));
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        dk[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(ga), as_bf8(bkh[nt][ks]), dk[nt], 0, 0, 0);
        dk[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(ga), as_bf8(bkl[nt][ks]), dk[nt], 0, 0, 0);
      }
    }
    // dqh of heads 32 half .. + 31, dims 32 (dn0 + nt) + l31, over the tile's 64 keys.
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint4 ah = tr_pair(ghs + ga_off[0] + 2048 * ks, ghs + ga_off[1] + 2048 * ks);
      const uint4 al = tr_pair(gls + ga_off[0] + 2048 * ks, gls + ga_off[1] + 2048 * ks);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const uint4 b = tr_pair(kbs + cb_off[0][nt] + 4096 * ks, kbs + cb_off[1][nt] + 4096 * ks);
        dq[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(ah), as_bf8(b), dq[nt], 0, 0, 0);
        dq[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(al), as_bf8(b), dq[nt], 0, 0, 0);
      }
    }
    // dk rows: accumulator register r holds key 8 (r >> 2) + 4 g2 + (r & 3).
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (!DK) break;
      const int mi = IB_TILE * tt + 32 * half + 8 * (r >> 2) + 4 * g2 + (r & 3);
      const uint32_t rw = mrow[mi];
      const float gs = mg[mi];
      if (!(rw & IB_INVALID)) {
        float *dst = a.dk + (int64_t)rw * 128 + 32 * dn0 + l31;
        unsafeAtomicAdd(dst, dk[0][r] * gs);
        unsafeAtomicAdd(dst + 32, dk[1][r] * gs);
      }
    }
  };

  v8i kb0 = load_keys(0), kb1;
  int tt = 0;
  for (; tt + 1 < ntile; tt += 2) {
    kb1 = load_keys(tt + 1);
    tile(tt, kb0);
    kb0 = load_keys(min(tt + 2, ntile - 1));
    tile(tt + 1, kb1);
  }
  if (tt < ntile) tile(tt, kb0);

  // dq: accumulator register r holds head 32 half + 8 (r >> 2) + 4 g2 + (r & 3).
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int h = 32 * half + 8 * (r >> 2) + 4 * g2 + (r & 3);
      const float wv = a.w[(int64_t)t * 64 + h];
      unsafeAtomicAdd(a.dq + ((int64_t)t * 64 + h) * 128 + 32 * (dn0 + nt) + l31, dq[nt][r] * wv);
    }
  // dw: sum over the 16 keys of the lane group, then over the wavefronts.
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = dwa[mt][i];
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) v += shfl_xor(v, m);
      if (l15 == 0) dwred[wave][16 * mt + 4 * g4 + i] = v;
    }
  __syncthreads();
  if (tid < 64) {
    const float qs = a.q_scale ? a.q_scale[(int64_t)t * 64 + tid] : 1.0f;
    const float v = (dwred[0][tid] + dwred[1][tid]) + (dwred[2][tid] + dwred[3][tid]);
    unsafeAtomicAdd(a.dw + (int64_t)t * 64 + tid, v * qs);
  }
}

// dkh for the dense mode (every visible position), key-major: one block = one
// 64-key tile of one sequence and a run of IBK_QRUN query indices; it loops
// over the queries of that run that see any key of the tile and accumulates
// dkh[key] = sum_t g_ts sum_j [D_tjs > 0] e_tj q8_tj in registers, then adds
// its sum into dk (a handful of atomic adds per block instead of 128 per
// (query, key) pair).  Per query:
//   * D^T = K . Q^T on FP8 MFMA: the tile's keys are the A operand for the
//     whole block (all 64 keys in every wavefront), wavefront w takes heads
//     16w .. 16w+15 of the query as the B operand;
//   * a[key][head] = [D > 0] e_j g_s goes to LDS head-major, as bf16 hi + lo
//     (each lane writes 4 adjacent keys of its head at once), and q8 as a
//     [head][dim] bf16 matrix (16-byte writes); dkh += a . q8 runs on bf16 MFMA
//     with the same 32 x 64 quarters per wavefront as the query-major kernel,
//     both operands read through the transposing LDS read, with the same
//     swizzles as there.
// Query order within a block is the index order (a block-wide scan), so a
// block's sum is deterministic; blocks of the same tile meet in the atomic adds.
constexpr int IBK_QRUN = 512;  // query indices per block

struct IndexerBwdDkArgs {
  IndexerBwdLaunch a;
  int tiles;   // key tiles per sequence
  int qruns;   // query runs
};

__global__ __launch_bounds__(IB_THREADS) void indexer_bwd_dk_kernel(IndexerBwdDkArgs p) {
  const IndexerBwdLaunch &a = p.a;
  const int per_seq = p.tiles * p.qruns;
  const int seq = blockIdx.x / per_seq;
  const int rem = blockIdx.x - seq * per_seq;
  const int tile = rem / p.qruns;
  const int t0 = (rem - tile * p.qruns) * IBK_QRUN;
  const int s0 = tile * IB_TILE;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int l15 = lane & 15, g4 = lane >> 4;
  const int l31 = lane & 31, g2 = lane >> 5;
  const int half = wave & 1, dn0 = 2 * (wave >> 1);

  // Two sets, alternating between queries: query i writes set i & 1 while
  // slower wavefronts may still read set (i - 1) & 1, so one barrier per
  // query suffices.
  __shared__ __attribute__((aligned(16))) uint8_t ahi[2][64 * 128];  // [head][key], gate_off
  __shared__ __attribute__((aligned(16))) uint8_t alo[2][64 * 128];
  __shared__ __attribute__((aligned(16))) uint8_t qt[2][64 * 256];   // [head][dim], ck_off
  __shared__ int qlist[IBK_QRUN];
  __shared__ int sm[IB_THREADS / WAVE];
  __shared__ int lsh[IB_THREADS / WAVE];

  // The queries of this run that see a key of the tile, in index order, and
  // the sequence's longest visible history (keys at or past it are not read).
  int n_rel = 0, lmax = 0;
  for (int base = 0; base < IBK_QRUN; base += IB_THREADS) {
    const int t = t0 + base + tid;
    bool rel = false;
    if (t < a.num_q && a.q_seq[t] == seq) {
      const int nv = a.q_nvis[t];
      lmax = max(lmax, nv);
      rel = nv > s0;
    }
    const uint64_t m = __ballot(rel);
    const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (lane == 0) sm[wave] = __popcll(m);
    __syncthreads();
    int before = n_rel;
    for (int w = 0; w < wave; ++w) before += sm[w];
    if (rel) qlist[before + below] = t;
    for (int w = 0; w < IB_THREADS / WAVE; ++w) n_rel += sm[w];
    __syncthreads();
  }
  if (n_rel == 0) return;  // block-uniform
  // Keys at or past the longest history among the run's queries of this
  // sequence are seen by none of them (and may not exist in the cache).
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) lmax = max(lmax, __shfl_xor(lmax, m, WAVE));
  if (lane == 0) lsh[wave] = lmax;
  __syncthreads();
  const int lseq = max(max(lsh[0], lsh[1]), max(lsh[2], lsh[3]));  // > s0

  // The tile's keys as the A operand (every wavefront holds all 64): key
  // 16 mt + l15, bytes [32 g4, +32).  Keys at or past lseq read key s0 (their
  // g is 0 for every query of the run, so they gather nothing).
  v8i ka[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int pos = s0 + 16 * mt + l15;
    const int64_t row = phys_row(a.map, seq, pos < lseq ? pos : s0);
    ka[mt] = load32(a.k8 + row * 128 + 32 * g4);
  }

  v16f acc[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[nt][r] = 0.0f;

  // Per-query operands, one query ahead: this wavefront's 16 heads of q8, the
  // head's e_j, and g of the 16 keys whose D values this lane holds (keys
  // 16 mt + 4 g4 + i; 0 past the query's history).
  struct QueryOps {
    v8i qb;
    float e;
    float g[16];
  };
  // Offsets from the query's (uniform) bases are 32-bit byte counts, so the
  // loads take a scalar base and a 32-bit lane offset.
  auto at = [](const auto *base, uint32_t byte_off) {
    return reinterpret_cast<decltype(base)>(reinterpret_cast<const char *>(base) + byte_off);
  };
  auto load_q = [&](int i, QueryOps &o) {
    const int t = __builtin_amdgcn_readfirstlane(qlist[min(i, n_rel - 1)]);
    const int j = 16 * wave + l15;
    o.qb = load32(at(a.q8 + (int64_t)t * (64 * 128), (uint32_t)(j * 128 + 32 * g4)));
    const float qs = a.q_scale ? *at(a.q_scale + (int64_t)t * 64, 4u * j) : 1.0f;
    o.e = *at(a.w + (int64_t)t * 64, 4u * j) * qs;
    const int nv = a.q_nvis[t];
    const float *gr = a.grad + (int64_t)t * a.ld_grad;
    if (nv >= s0 + IB_TILE) {  // uniform: the whole tile is in the history
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) o.g[4 * mt + i2] = *at(gr, 4u * (uint32_t)(s0 + 16 * mt + 4 * g4 + i2));
    } else {
      // The run holds only queries with n_vis > s0, so n_vis - 1 is a valid
      // position to read in place of those past the history.
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
          const int pos = s0 + 16 * mt + 4 * g4 + i2;
          const float gv = *at(gr, 4u * (uint32_t)min(pos, nv - 1));
          o.g[4 * mt + i2] = pos < nv ? gv : 0.0f;
        }
    }
  };

  // LDS byte offsets.  Writes: head j = 16 wave + l15, dims 32 g4 + 8 jj ..
  // + 7 of q8 (16 bytes) and keys 16 mt + 4 g4 .. + 3 of a (8 bytes).
  // Transposing reads (heads are the k index of the product): lane
  // 32 g2 + 16 th + ti points at row (head) ti >> 2 of the set
  // 16 ks + 8 g2 + 4 hh .. + 3 and bytes 8 (ti & 3) of its group's 32-byte
  // column span, and receives column 16 th + ti: key 32 half + l31 of a, or
  // dim 32 (dn0 + nt) + l31 of q8.
  const int ti = lane & 15, th = (lane >> 4) & 1;
  int qw_off[4], aw_off[4], ar_off[2], qr_off[2][2];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) qw_off[jj] = ck_off(16 * wave + l15, 64 * g4 + 16 * jj);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) aw_off[mt] = gate_off(16 * wave + l15, 32 * mt + 8 * g4);
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int r = 8 * g2 + 4 * hh + (ti >> 2);
    ar_off[hh] = gate_off(r, 64 * half + 32 * th + 8 * (ti & 3));
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) qr_off[hh][nt] = ck_off(r, 64 * (dn0 + nt) + 32 * th + 8 * (ti & 3));
  }
  auto tr_pair = [](const uint8_t *p0, const uint8_t *p1) {
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)p0);
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)p1);
    const uint2 ulo = __builtin_bit_cast(uint2, lo), uhi = __builtin_bit_cast(uint2, hi);
    return make_uint4(ulo.x, ulo.y, uhi.x, uhi.y);
  };

  auto one_query = [&](const QueryOps &o, const int set) {
    uint8_t *qts = qt[set];
    uint8_t *ah = ahi[set];
    uint8_t *al = alo[set];
    // q8 of head j as bf16: qt[head][dim], dims 32 g4 + 8 jj .. + 7 (words 2 jj, 2 jj + 1).
    const uint32_t qw[8] = {(uint32_t)o.qb[0], (uint32_t)o.qb[1], (uint32_t)o.qb[2], (uint32_t)o.qb[3],
                            (uint32_t)o.qb[4], (uint32_t)o.qb[5], (uint32_t)o.qb[6], (uint32_t)o.qb[7]};
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      uint32_t u[4];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int v = (int)qw[2 * jj + h2];
        u[2 * h2] = pk_bf16(__builtin_amdgcn_cvt_pk_f32_fp8(v, false));
        u[2 * h2 + 1] = pk_bf16(__builtin_amdgcn_cvt_pk_f32_fp8(v, true));
      }
      *reinterpret_cast<uint4 *>(qts + qw_off[jj]) = make_uint4(u[0], u[1], u[2], u[3]);
    }
    // D^T[key][head] for keys 16 mt + 4 g4 + i, head j; a = [D > 0] e_j g_s.
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const v4f d = mfma_fp8_16x16x128(ka[mt], o.qb, v4f{0.f, 0.f, 0.f, 0.f});
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = d[i] > 0.0f ? o.e * o.g[4 * mt + i] : 0.0f;
      uint32_t hi[2], lo[2];
#pragma unroll
      for (int p2 = 0; p2 < 2; ++p2) {
        hi[p2] = pk_bf16(float2_t{x[2 * p2], x[2 * p2 + 1]});
        lo[p2] = pk_bf16(float2_t{x[2 * p2] - __uint_as_float(hi[p2] << 16),
                                  x[2 * p2 + 1] - __uint_as_float(hi[p2] & 0xFFFF0000u)});
      }
      *reinterpret_cast<uint2 *>(ah + aw_off[mt]) = make_uint2(hi[0], hi[1]);
      *reinterpret_cast<uint2 *>(al + aw_off[mt]) = make_uint2(lo[0], lo[1]);
    }
    __syncthreads();  // this query's a and q8 visible
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint4 fh = tr_pair(ah + ar_off[0] + 2048 * ks, ah + ar_off[1] + 2048 * ks);
      const uint4 fl = tr_pair(al + ar_off[0] + 2048 * ks, al + ar_off[1] + 2048 * ks);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const uint4 b = tr_pair(qts + qr_off[0][nt] + 4096 * ks, qts + qr_off[1][nt] + 4096 * ks);
        acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(fh), as_bf8(b), acc[nt], 0, 0, 0);
        acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(fl), as_bf8(b), acc[nt], 0, 0, 0);
      }
    }
  };
  QueryOps o0, o1;
  load_q(0, o0);
  int i = 0;
  for (; i + 1 < n_rel; i += 2) {
    load_q(i + 1, o1);
    one_query(o0, 0);
    load_q(i + 2, o0);
    one_query(o1, 1);
  }
  if (i < n_rel) one_query(o0, 0);

  // acc register r holds key 32 half + 8 (r >> 2) + 4 g2 + (r & 3), dim 32 (dn0 + nt) + l31.
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int pos = s0 + 32 * half + 8 * (r >> 2) + 4 * g2 + (r & 3);
    if (pos < lseq) {
      float *dst = a.dk + phys_row(a.map, seq, pos) * 128 + 32 * dn0 + l31;
      unsafeAtomicAdd(dst, acc[0][r]);
      unsafeAtomicAdd(dst + 32, acc[1][r]);
    }
  }
}

hipError_t launch_indexer_bwd(const IndexerBwdLaunch &a, int max_set, hipStream_t st) {
  if (a.num_q == 0) return hipSuccess;
  const int64_t nz = (int64_t)a.num_q * 64 * 128;
  hipLaunchKernelGGL(ib_zero_kernel, dim3((unsigned)((nz + 255) / 256)), dim3(256), 0, st, a.dq, nz);
  hipLaunchKernelGGL(ib_zero_kernel, dim3((unsigned)(((int64_t)a.num_q * 64 + 255) / 256)), dim3(256), 0, st, a.dw,
                     (int64_t)a.num_q * 64);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || max_set == 0) return e;
  IndexerBwdArgs p;
  p.a = a;
  int members = IB_MAX_MEMBERS;
  auto chunks = [&](int m) { return (max_set + m - 1) / m; };
  while (members > IB_TILE && (int64_t)a.num_q * chunks(members) < IB_MIN_BLOCKS) members /= 2;
  p.members = members;
  p.nchunk = chunks(members);
  const dim3 grid((unsigned)((int64_t)a.num_q * p.nchunk));
  if (a.idx) {
    hipLaunchKernelGGL(indexer_bwd_kernel<true>, grid, dim3(IB_THREADS), 0, st, p);
    return hipGetLastError();
  }
  // Dense: dq and dw query-major, dk key-major.
  hipLaunchKernelGGL(indexer_bwd_kernel<false>, grid, dim3(IB_THREADS), 0, st, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  IndexerBwdDkArgs pk;
  pk.a = a;
  pk.tiles = (max_set + IB_TILE - 1) / IB_TILE;
  pk.qruns = (a.num_q + IBK_QRUN - 1) / IBK_QRUN;
  const int64_t blocks = (int64_t)a.num_seqs * pk.tiles * pk.qruns;
  hipLaunchKernelGGL(indexer_bwd_dk_kernel, dim3((unsigned)blocks), dim3(IB_THREADS), 0, st, pk);
  return hipGetLastError();
}

}  // namespace dsa
