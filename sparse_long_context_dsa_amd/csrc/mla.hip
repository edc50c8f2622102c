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
// output accumulator O[32 heads, 512] in fp32 (16 x 32x32 tiles, 256
// registers).  Rows arrive in tiles of 32, gathered through the position ->
// row map into LDS, double buffered:
//   * K layout: [32 rows][72 x 16 B] row-major (XOR-swizzled 16-byte chunks),
//     the A operand of S^T = K . Q^T (v_mfma_f32_32x32x16_bf16, M = rows,
//     N = heads, K = 576 in 36 steps);
//   * V^T layout: [512 dims][32 rows] (XOR-swizzled), written by an 8x8
//     register transpose while staging, the B operand of O = P . V (M = heads,
//     N = dims, K = 32 rows in 2 steps).
// Computing S transposed puts each head in one lane column, so the online
// softmax (running max m, sum l per head) needs one cross-half exchange, and
// the S^T accumulator registers are exactly the A operand of P . V once
// rounded to bf16 (the V^T rows are stored in the matching order).  Only the
// per-head rescale of O needs the softmax state of other lanes; it goes
// through a 128-byte LDS slot per wavefront and is skipped when no running max
// changed.  exp2 with log2(e) folded into the scale.
//
// Decode splits a query's rows over several blocks that write (O/l, lse)
// partials; mla_combine_kernel merges them.  Prefill gives each query one
// block and writes the result directly.
#include "device_util.h"
#include "dsa_internal.h"

namespace dsa {

constexpr int MLA_WAVES = 4;
constexpr int MLA_THREADS = MLA_WAVES * WAVE;
constexpr int MLA_T = 32;                          // rows per tile
constexpr int ROW_BYTES = 576 * 2;                 // 1152
constexpr int KL_BYTES = MLA_T * ROW_BYTES;        // 36864
constexpr int VT_BYTES = 512 * MLA_T * 2;          // 32768
constexpr int BUF_BYTES = KL_BYTES + VT_BYTES;     // 69632
constexpr int MLA_MAX_ROWS = 2048;                 // rows per block (k <= 2048)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float RESCALE_LOG2 = 8.0f;              // lazy-rescale threshold (log2 units)

struct MlaKernelArgs {
  MlaLaunch a;
  int nsplit;
  int rows_per_split;
  float scale_log2;
  float *part_o;    // [num_q, nsplit, 128, 512]   (nsplit > 1)
  float *part_lse;  // [num_q, nsplit, 128]
};

__device__ __forceinline__ v8bf as_bf(const uint4 &u) { return __builtin_bit_cast(v8bf, u); }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Byte offset of 16-byte chunk `ch` (0..71) of tile row `r` in the K layout.
__device__ __forceinline__ int kl_off(int r, int ch) { return r * ROW_BYTES + ((ch ^ ((r >> 1) & 7)) << 4); }
// Byte offset of 16-byte row-block `rb` (0..3) of value dim `d` in the V^T layout.
__device__ __forceinline__ int vt_off(int d, int rb) { return KL_BYTES + d * 64 + ((rb ^ ((d >> 2) & 3)) << 4); }

// Tile row held in slot jj (0..7) of row-block rb (0..3) of the V^T layout.
// Row-block rb = 2*ks2 + g collects the rows that lane group g contributes to
// k-step ks2 of P . V: rows 16*ks2 + 4*g + {0..3} and 16*ks2 + 8 + 4*g + {0..3}.
__device__ __forceinline__ int rb_row(int rb, int jj) {
  return 16 * (rb >> 1) + 4 * (rb & 1) + (jj & 3) + 8 * (jj >> 2);
}

// Scales one accumulator register in place.  The accumulators live in AGPRs,
// which VALU instructions cannot use as operands; the explicit read / multiply /
// write keeps them there instead of moving all of O into VGPRs.
__device__ __forceinline__ void scale_acc(float &x, float s) {
  float tmp;
  asm volatile(
      "v_accvgpr_read_b32 %1, %0\n\t"
      "s_nop 1\n\t"
      "v_mul_f32 %1, %1, %2\n\t"
      "v_accvgpr_write_b32 %0, %1\n\t"
      "s_nop 1"
      : "+a"(x), "=&v"(tmp)
      : "v"(s));
}

// Values of the 16 heads whose O rows this lane holds (heads 8i + 4g + j),
// from a 32-entry per-head array in LDS.
__device__ __forceinline__ void read_head_values(const float *x, int g, float *v) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 f = *reinterpret_cast<const float4 *>(&x[8 * i + 4 * g]);
    v[4 * i + 0] = f.x;
    v[4 * i + 1] = f.y;
    v[4 * i + 2] = f.z;
    v[4 * i + 3] = f.w;
  }
}

struct Staging {
  uint4 v[8];  // 8 rows x dims [8*dg, 8*dg+8)
  uint4 rope;  // one 16-byte chunk of the rotary part
};

__device__ __forceinline__ void stage_load(const uint16_t *__restrict__ kv, const int32_t *prow, int t0,
                                           int nrows, Staging &s) {
  const int tid = threadIdx.x;
  const int dg = tid & 63, rb = tid >> 6;
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const int r = t0 + rb_row(rb, jj);
    if (r < nrows && prow[r] >= 0) {
      s.v[jj] = *reinterpret_cast<const uint4 *>(kv + (int64_t)prow[r] * 576 + 8 * dg);
    } else {
      s.v[jj] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  const int rr = t0 + (tid >> 3);
  if (rr < nrows && prow[rr] >= 0) {
    s.rope = *reinterpret_cast<const uint4 *>(kv + (int64_t)prow[rr] * 576 + 512 + 8 * (tid & 7));
  } else {
    s.rope = make_uint4(0u, 0u, 0u, 0u);
  }
}

__device__ __forceinline__ void stage_store(uint8_t *buf, const Staging &s) {
  const int tid = threadIdx.x;
  const int dg = tid & 63, rb = tid >> 6;
  // K layout: row-major.
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) *reinterpret_cast<uint4 *>(buf + kl_off(rb_row(rb, jj), dg)) = s.v[jj];
  const int rr = tid >> 3;
  *reinterpret_cast<uint4 *>(buf + kl_off(rr, 64 + (tid & 7))) = s.rope;
  // V^T layout: transpose the 8 rows x 8 dims block in registers.
  const uint32_t *w = reinterpret_cast<const uint32_t *>(s.v);  // w[4*jj + dword]
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
    uint4 o;
    o.x = __builtin_amdgcn_perm(w[4 * 1 + (e >> 1)], w[4 * 0 + (e >> 1)], sel);
    o.y = __builtin_amdgcn_perm(w[4 * 3 + (e >> 1)], w[4 * 2 + (e >> 1)], sel);
    o.z = __builtin_amdgcn_perm(w[4 * 5 + (e >> 1)], w[4 * 4 + (e >> 1)], sel);
    o.w = __builtin_amdgcn_perm(w[4 * 7 + (e >> 1)], w[4 * 6 + (e >> 1)], sel);
    *reinterpret_cast<uint4 *>(buf + vt_off(8 * dg + e, rb)) = o;
  }
}

__global__ __launch_bounds__(MLA_THREADS, 1) void mla_kernel(MlaKernelArgs p) {
  const MlaLaunch &a = p.a;
  const int q = blockIdx.x / p.nsplit;
  const int sp = blockIdx.x - q * p.nsplit;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, c = lane & 31;

  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * BUF_BYTES];
  __shared__ __attribute__((aligned(16))) int32_t prow[MLA_MAX_ROWS + MLA_T];
  __shared__ __attribute__((aligned(16))) float xch[MLA_WAVES][32];

  const int nvis = a.q_nvis[q];
  int cnt = a.count ? a.count[q] : min(a.k, nvis);
  cnt = max(0, min(cnt, a.k));
  const int r0 = sp * p.rows_per_split;
  const int nrows = max(0, min(cnt, r0 + p.rows_per_split) - r0);

  // Selected positions -> physical rows.
  const int seq = a.q_seq[q];
  const int32_t *ip = a.idx + (int64_t)q * a.k + r0;
  // A position outside [0, n_vis) breaks the contract; it becomes a masked
  // zero row instead of an out-of-bounds read.
  for (int i = tid; i < nrows; i += MLA_THREADS) {
    const int pos = ip[i];
    prow[i] = (pos >= 0 && pos < nvis) ? (int32_t)phys_row(a.map, seq, pos) : -1;
  }

  // Queries of this wavefront's 32 heads: B fragments of S^T = K . Q^T.
  const int head = 32 * wave + c;
  uint4 qb[36];
  {
    const uint16_t *qr = a.q + ((int64_t)q * 128 + head) * 576 + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) qb[ks] = *reinterpret_cast<const uint4 *>(qr + 16 * ks);
  }

  v16f o[16];
#pragma unroll
  for (int nt = 0; nt < 16; ++nt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[nt][i] = 0.0f;
  float m_ref = -INFINITY, l_run = 0.0f;  // per head c (both lane halves agree on m_ref)

  __syncthreads();  // prow ready
  const int ntiles = (nrows + MLA_T - 1) / MLA_T;
  Staging st;
  if (ntiles > 0) {
    stage_load(a.kv, prow, 0, nrows, st);
    stage_store(smem, st);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int t0 = t * MLA_T;
    if (t + 1 < ntiles) stage_load(a.kv, prow, t0 + MLA_T, nrows, st);
    const uint8_t *buf = smem + (t & 1) * BUF_BYTES;

    // S^T[row, head] for 32 rows x 32 heads.
    v16f s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) {
      const uint4 kf = *reinterpret_cast<const uint4 *>(buf + kl_off(c, 2 * ks + g));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf(kf), as_bf(qb[ks]), s, 0, 0, 0);
      if ((ks & 3) == 3) __builtin_amdgcn_sched_barrier(0);  // bound the LDS reads in flight
    }

    // Online softmax for head c over this tile's rows 8i + 4g + j.
    float z[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rbase = t0 + 8 * i + 4 * g;
      const int4 pr = *reinterpret_cast<const int4 *>(&prow[rbase]);
      const int prv[4] = {pr.x, pr.y, pr.z, pr.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = rbase + j;
        const float v = (row < nrows && prv[j] >= 0) ? s[4 * i + j] * p.scale_log2 : -INFINITY;
        z[4 * i + j] = v;
        tmax = fmaxf(tmax, v);
      }
    }
    tmax = fmaxf(tmax, shfl_xor(tmax, 32));
    // The reference max moves only when a head's tile max exceeds it by more
    // than RESCALE_LOG2 (always on the first tile), so P <= 2^RESCALE_LOG2 and
    // O is rescaled rarely.
    // A tile whose rows are all masked leaves tmax = -inf and changes nothing.
    if (__ballot(tmax > m_ref + RESCALE_LOG2) != 0ull) {
      const float m_new = fmaxf(m_ref, tmax);
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);  // 0 on the first tile
      l_run *= alpha;
      m_ref = m_new;
      if (t > 0) {  // O is still zero on the first tile
        if (g == 0) xch[wave][c] = alpha;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        float al[16];
        read_head_values(xch[wave], g, al);
#pragma unroll
        for (int nt = 0; nt < 16; ++nt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float x = o[nt][i];
            scale_acc(x, al[i]);
            o[nt][i] = x;
          }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
      }
    }
    const float mref = (m_ref == -INFINITY) ? 0.0f : m_ref;  // all rows so far masked: z = -inf, p = 0
    float psum = 0.0f;
    uint32_t pk[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float e0 = __builtin_amdgcn_exp2f(z[2 * i] - mref);
      const float e1 = __builtin_amdgcn_exp2f(z[2 * i + 1] - mref);
      psum += e0 + e1;
      pk[i] = pack_bf16(e0, e1);
    }
    l_run += psum;

    // O += P . V over the tile's 32 rows (2 k-steps of 16).
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      const uint4 pa = make_uint4(pk[4 * ks2 + 0], pk[4 * ks2 + 1], pk[4 * ks2 + 2], pk[4 * ks2 + 3]);
#pragma unroll
      for (int nt = 0; nt < 16; ++nt) {
        const uint4 vf = *reinterpret_cast<const uint4 *>(buf + vt_off(32 * nt + c, 2 * ks2 + g));
        o[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf(pa), as_bf(vf), o[nt], 0, 0, 0);
        if ((nt & 3) == 3) __builtin_amdgcn_sched_barrier(0);
      }
    }

    if (t + 1 < ntiles) stage_store(smem + ((t + 1) & 1) * BUF_BYTES, st);
    __syncthreads();
  }

  // Normalise.  Both lane halves hold partial sums of head c.
  const float l_tot = l_run + shfl_xor(l_run, 32);
  const float inv = (l_tot > 0.0f) ? 1.0f / l_tot : 0.0f;
  const float lse_v = (l_tot > 0.0f) ? m_ref * LN2 + logf(l_tot) : -INFINITY;
  if (g == 0) xch[wave][c] = inv;
  __syncthreads();
  float il[16];
  read_head_values(xch[wave], g, il);
#pragma unroll
  for (int nt = 0; nt < 16; ++nt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float x = o[nt][i];
      scale_acc(x, il[i]);
      o[nt][i] = x;
    }

  float *obase;
  float *lbase;
  if (p.nsplit == 1) {
    obase = a.out + (int64_t)q * 128 * 512;
    lbase = a.lse ? a.lse + (int64_t)q * 128 : nullptr;
  } else {
    obase = p.part_o + ((int64_t)q * p.nsplit + sp) * 128 * 512;
    lbase = p.part_lse + ((int64_t)q * p.nsplit + sp) * 128;
  }
#pragma unroll
  for (int nt = 0; nt < 16; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int h = 32 * wave + 8 * i + 4 * g + j;
        obase[(int64_t)h * 512 + 32 * nt + c] = o[nt][4 * i + j];
      }
  if (lbase && g == 0) lbase[head] = lse_v;
}

// Merge split partials: out = sum_s exp(lse_s - M) O_s / sum_s exp(lse_s - M).
__global__ __launch_bounds__(256) void mla_combine_kernel(const float *__restrict__ part_o,
                                                          const float *__restrict__ part_lse, int nsplit,
                                                          float *__restrict__ out, float *__restrict__ lse) {
  const int q = blockIdx.x >> 6;
  const int head = 2 * (blockIdx.x & 63) + (threadIdx.x >> 7);
  const int d = 4 * (threadIdx.x & 127);
  const float *pl = part_lse + (int64_t)q * nsplit * 128 + head;
  float mx = -INFINITY;
  for (int s = 0; s < nsplit; ++s) mx = fmaxf(mx, pl[s * 128]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float den = 0.0f;
  if (mx != -INFINITY) {
    for (int s = 0; s < nsplit; ++s) {
      const float ls = pl[s * 128];
      if (ls == -INFINITY) continue;
      const float wgt = expf(ls - mx);
      const float4 v = *reinterpret_cast<const float4 *>(part_o + (((int64_t)q * nsplit + s) * 128 + head) * 512 + d);
      acc.x += wgt * v.x; acc.y += wgt * v.y; acc.z += wgt * v.z; acc.w += wgt * v.w;
      den += wgt;
    }
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  float4 r = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  *reinterpret_cast<float4 *>(out + ((int64_t)q * 128 + head) * 512 + d) = r;
  if (lse && (threadIdx.x & 127) == 0) lse[(int64_t)q * 128 + head] = den > 0.0f ? mx + logf(den) : -INFINITY;
}

int mla_num_splits(int num_q, int k, bool decode) {
  if (!decode || num_q <= 0) return 1;
  int ns = (256 + num_q - 1) / num_q;        // about one block per CU
  const int max_split = (k + 127) / 128;     // at least 128 rows per split
  ns = ns < 1 ? 1 : ns;
  ns = ns > max_split ? max_split : ns;
  return ns < 1 ? 1 : ns;
}

static int rows_per_split(int k, int nsplit) {
  int r = (k + nsplit - 1) / nsplit;
  return (r + MLA_T - 1) / MLA_T * MLA_T;
}

size_t mla_ws_bytes(int num_q, int k, bool decode) {
  const int ns = mla_num_splits(num_q, k, decode);
  if (ns <= 1) return 0;
  return (size_t)num_q * ns * 128 * (512 + 1) * sizeof(float) + 256;
}

hipError_t launch_mla(const MlaLaunch &a, bool decode, void *ws, hipStream_t st) {
  if (a.num_q == 0) return hipSuccess;
  MlaKernelArgs p;
  p.a = a;
  p.nsplit = mla_num_splits(a.num_q, a.k, decode);
  p.rows_per_split = rows_per_split(a.k, p.nsplit);
  p.scale_log2 = a.softmax_scale * LOG2E;
  p.part_o = nullptr;
  p.part_lse = nullptr;
  if (p.nsplit > 1) {
    p.part_o = static_cast<float *>(ws);
    p.part_lse = p.part_o + (size_t)a.num_q * p.nsplit * 128 * 512;
  }
  hipLaunchKernelGGL(mla_kernel, dim3((unsigned)((int64_t)a.num_q * p.nsplit)), dim3(MLA_THREADS), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;
  hipLaunchKernelGGL(mla_combine_kernel, dim3((unsigned)((int64_t)a.num_q * 64)), dim3(256), 0, st, p.part_o,
                     p.part_lse, p.nsplit, a.out, a.lse);
  return hipGetLastError();
}

}  // namespace dsa
