// Lightning-indexer scores on FP8 MFMA (gfx950).
//
//   I[i, s] = k_scale[r(s)] * sum_j (w[i,j] * q_scale[i,j]) * ReLU(q8[i,j,:] . k8[r(s),:])
//
// Page "arXiv'25 | DSA ... DeepSeek-V3.2", section 3 (first equation); page
// "DeepSeekV3.2之DSA", part 4.3 (order: FP8 q@k into fp32, ReLU times the head
// weight, sum over heads, times the key scale).  q_scale is folded into the
// head weight (same page, part 4.3: the weights carry the q scale); the key
// scale is applied after the head sum, which is exact reordering because
// k_scale > 0 and ReLU is positively homogeneous.  The key scales come either
// as fp32 or, as in that page's kernel, as E8M0 exponents (one byte per key,
// scale 2^(b - 127)): 133 instead of 136 bytes per key.
//
// Mapping: one wavefront owns one query and a run of kpw keys.  The 64
// indexer heads are the M side of v_mfma_scale_f32_16x16x128_f8f6f4 (4 M-tiles
// of 16 heads, K = 128 = the whole head width, so one MFMA per 16x16 tile);
// keys are the N side, 16 per tile, 4 tiles (64 keys) per step.  The query's
// 8 KiB of FP8 q is read once per block into LDS and from there into each
// wavefront's registers, where it stays for the whole run; keys stream from HBM
// straight into the B-operand registers (each lane reads 32 contiguous bytes
// of a key row; the two 64-byte halves of a row go to lane groups 0/1 and
// 2/3), prefetched one step ahead into the other of two register buffers.
// Every lane issues the same loads on every step (rows past the visible range
// are clamped, not skipped), and the block-table lookups are done once before
// the loop, so the waits on the prefetch count exactly the loads they need.  ReLU, the weighting and 16 of the 64 head
// terms are summed in-lane; the remaining 4-way sum across lane groups is a
// butterfly of vector-ALU lane swaps (v_permlane32_swap, v_permlane16_swap)
// that also transposes, so lane l ends with the score of key s0+l.
// Scores of four steps are staged in LDS and leave as non-temporal 16-byte
// stores (1 KiB per wavefront instruction).
//
// Optionally each block also builds a 2048-bin histogram of the top 11 bits
// of the scores' order-preserving keys (the first pass of the top-k radix
// select), so the top-k stage need not read the scores twice.
//
// When one block covers a query's whole history (up to 16384 positions: many
// queries, as in causal prefill), the block can instead select the row itself
// (page "arXiv'25 | DSA ...", section 3, second equation): the scores stay in
// LDS, the first-digit histogram is built there as they are produced, and
// the block's radix select writes the positions; no score leaves the CU.
#include "topk_row.h"

namespace dsa {

constexpr int IDX_WAVES = 4;
constexpr int IDX_KPW_MIN = 256;                 // keys per wavefront: a multiple of 64,
constexpr int IDX_KPW_MAX = 64 * WAVE;           // at most one 64-key step per lane
constexpr int64_t IDX_MIN_WAVES = 32768;         // 32 wavefronts per SIMD

typedef float nt_float4 __attribute__((ext_vector_type(4)));  // a vector type the nontemporal builtin takes

struct KeyStep {
  v8i b[4];
  float ks;
};

// E8M0 byte b -> 2^(b - 127) (b = 0 is the subnormal 2^-127; 255 is not a scale).
__device__ __forceinline__ float e8m0_value(uint32_t b) {
  return __uint_as_float(b ? b << 23 : 0x00400000u);
}

// Loads the B operands (4 tiles of 16 keys) of the 64-key step at s0, whose
// keys sit in the physical rows base .. base + 63.  Keys at or past nvis read
// the step's last visible row instead: every lane always issues the same
// loads (no branch, so the compiler's wait counts stay exact), and the scores
// of those keys are never stored.
template <bool E8M0>
__device__ __forceinline__ void load_step(const IndexerLaunch &a, int64_t base, int s0, int nvis, int lane,
                                          KeyStep &st) {
  const int sub = lane & 15, half = lane >> 4;
  const int last = nvis - 1 - s0;  // >= 0
#pragma unroll
  for (int t = 0; t < 4; ++t) st.b[t] = load32(a.k8 + (base + min(16 * t + sub, last)) * 128 + 32 * half);
  st.ks = E8M0 ? e8m0_value(a.k_e8m0[base + min(lane, last)]) : a.k_scale[base + min(lane, last)];
}

// a from this lane plus the partner value that v_permlane{16,32}_swap brings
// in: with vdst = a and src0 = b, the swap exchanges the upper half (16 or 32
// lanes) of a with the lower half of b, so each lane's two results are its
// own and its partner's (lane ^ 16 or lane ^ 32) copy of the same operand --
// a for lanes in the lower half, b for lanes in the upper half.
template <bool SWAP16>
__device__ __forceinline__ float swap_sum(float a, float b) {
  const auto r = SWAP16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false)
                        : __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float relu(float x) {
  float r;
  asm("v_max_f32 %0, 0, %1" : "=v"(r) : "v"(x));  // one instruction, no canonicalize
  return r;
}

template <bool HIST, bool E8M0, bool SEL>
// Three wavefronts per SIMD: the epilogue of key tile t overlapping tile
// t + 1's MFMAs needs 16 more registers than a serial epilogue, and left to
// itself the compiler would spend them on accumulator registers and drop to
// two wavefronts.  (SEL: the 72 KiB of LDS leave room for two blocks per CU.)
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(SEL ? 2 : 3, SEL ? 2 : 3))) void indexer_kernel(
    IndexerLaunch a, int nchunks, int kpw) {
  static_assert(!(HIST && SEL), "a selecting block keeps its histogram in LDS");
  const int q = blockIdx.x / nchunks;
  const int chunk = blockIdx.x - q * nchunks;
  const int nvis = a.q_nvis[q];
  if (SEL && nvis <= a.skip_le) {  // short history: every position is kept (block-uniform)
    for (int i = threadIdx.x; i < a.sel_k; i += blockDim.x) a.sel_idx[(int64_t)q * a.sel_k + i] = i < nvis ? i : -1;
    if (threadIdx.x == 0) a.sel_count[q] = nvis;
    return;
  }
  if (nvis <= a.skip_le || chunk * IDX_WAVES * kpw >= nvis) return;  // block-uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int seq = a.q_seq[q];

  // Physical row of each 64-key step of this wavefront's run (a step never
  // straddles a cache block), one step per lane, looked up once: the loop then
  // issues its key loads without waiting on a block-table read.  Every lane
  // looks one up (positions clamped into the history), so no branch merges
  // its value with a constant, which would make the compiler wait for all
  // loads in flight there.
  const int s_begin = (chunk * IDX_WAVES + wave) * kpw;
  const int s_end = min(s_begin + kpw, nvis);
  const int64_t lane_row = phys_row(a.map, seq, max(0, min(s_begin + 64 * lane, nvis - 1)));
  // The first step's keys are requested before q and the weights are staged,
  // so that their round trip overlaps the staging's instead of following it.
  const int nsteps = s_begin < s_end ? (s_end - s_begin + 63) >> 6 : 0;
  KeyStep kb0, kb1;
  if (nsteps > 0) load_step<E8M0>(a, readlane64(lane_row, 0), s_begin, nvis, lane, kb0);

  __shared__ uint32_t hist[(HIST || SEL) ? TOPK_BINS : 1];
  // Per-wavefront staging of 256 scores: written as 16-byte stores (1 KiB per
  // wavefront instruction), which the memory system takes much better than
  // one 256-byte store per 64 keys.
  __shared__ __attribute__((aligned(16))) float sbuf[SEL ? 1 : IDX_WAVES][256];
  // SEL: the whole row's scores, by position.
  __shared__ __attribute__((aligned(16))) float rowbuf[SEL ? TOPK_ROW_MAX : 4];
  // The query's 8 KiB of q, read once per block with contiguous 16-byte loads
  // and shared by the four wavefronts through LDS (each wavefront reading it
  // from memory in the operand layout took 4x the requests, 16 rows apart).
  __shared__ __attribute__((aligned(16))) uint8_t qlds[SEL ? 16 : 64 * 128];
  // The 64 epilogue weights w * q_scale, likewise once per block.
  __shared__ __attribute__((aligned(16))) float wq[64];
  // All of the staging's loads go out before any of their values is used:
  // every thread loads (weight and scale of head t % 64, from a valid array
  // when there are no q scales), and only the stores depend on the thread.
  static_assert(64 * 128 == 2 * 16 * IDX_WAVES * WAVE, "two 16-byte pieces per thread");
  const uint4 *qsrc = reinterpret_cast<const uint4 *>(a.q8 + (int64_t)q * (64 * 128));
  uint4 qv0, qv1;
  if (!SEL) {
    qv0 = qsrc[threadIdx.x];
    qv1 = qsrc[threadIdx.x + IDX_WAVES * WAVE];
  }
  const int hw = (int)(threadIdx.x & 63);
  const float wv = a.w[(int64_t)q * 64 + hw];
  const float qsv = (a.q_scale ? a.q_scale : a.w)[(int64_t)q * 64 + hw];
  __builtin_amdgcn_sched_barrier(0);  // the stores below wait; the loads stay above them
  if (!SEL) {
    uint4 *qdst = reinterpret_cast<uint4 *>(qlds);
    qdst[threadIdx.x] = qv0;
    qdst[threadIdx.x + IDX_WAVES * WAVE] = qv1;
  }
  if (threadIdx.x < 64) wq[threadIdx.x] = wv * (a.q_scale ? qsv : 1.0f);
  if (HIST || SEL) {
    for (int b = threadIdx.x; b < TOPK_BINS; b += blockDim.x) hist[b] = 0u;
  }
  __syncthreads();

  // A operands: 4 M-tiles of 16 heads; lane holds head 16*mt + (lane&15),
  // bytes [32*(lane>>4), +32) of the 128-byte head row.
  const uint8_t *qp = a.q8 + (int64_t)q * (64 * 128);
  v8i A[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int off = (16 * mt + (lane & 15)) * 128 + 32 * (lane >> 4);
    if (SEL) {
      A[mt] = load32(qp + off);
    } else {
      const uint4 x0 = *reinterpret_cast<const uint4 *>(qlds + off);
      const uint4 x1 = *reinterpret_cast<const uint4 *>(qlds + off + 16);
      A[mt][0] = (int)x0.x; A[mt][1] = (int)x0.y; A[mt][2] = (int)x0.z; A[mt][3] = (int)x0.w;
      A[mt][4] = (int)x1.x; A[mt][5] = (int)x1.y; A[mt][6] = (int)x1.z; A[mt][7] = (int)x1.w;
    }
  }
  // Epilogue weights for the accumulator rows this lane holds:
  // head 16*mt + 4*(lane>>4) + r.
  float coef[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const float4 c4 = *reinterpret_cast<const float4 *>(&wq[16 * mt + 4 * (lane >> 4)]);
    coef[mt][0] = c4.x;
    coef[mt][1] = c4.y;
    coef[mt][2] = c4.z;
    coef[mt][3] = c4.w;
  }

  float *srow = a.scores + (int64_t)q * a.ld;

  // A finished group of 256 scores is stored one step late, after the next
  // step's key loads are issued, so that the wait for those loads (vector
  // memory completes in order) does not also wait on the store.
  auto flush = [&](int g0) {
    const float4 v = *reinterpret_cast<const float4 *>(&sbuf[wave][4 * lane]);
    const int p0 = g0 + 4 * lane;
    if (p0 + 3 < s_end) {
      // Non-temporal: the scores are read back once, by the top-k, and should
      // not displace the key stream's lines on the way.
      const nt_float4 v4 = {v.x, v.y, v.z, v.w};
      __builtin_nontemporal_store(v4, reinterpret_cast<nt_float4 *>(srow + p0));
    } else {
      const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (p0 + e < s_end) srow[p0 + e] = vv[e];
    }
    if (HIST) {
      const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (p0 + e < s_end) atomicAdd(&hist[order_key(vv[e]) >> 21], 1u);
    }
  };

  int pending = -1;  // start of a group waiting to be stored
  // One 64-key step: prefetch the next step into `nxt`, store a finished
  // group, score the keys in `cur`.  The loop alternates two buffers, so no
  // register copy forces an early wait on the prefetch.
  auto step = [&](int s0, const KeyStep &cur, KeyStep *nxt) {
    if (nxt) load_step<E8M0>(a, readlane64(lane_row, ((s0 - s_begin) >> 6) + 1), s0 + 64, nvis, lane, *nxt);
    if (pending >= 0) {
      flush(pending);
      pending = -1;
    }
    float p[4];
    // The MFMAs of key tile t + 1 are issued before the epilogue of tile t,
    // so the matrix core works while the vector ALU weights tile t's heads.
    v4f c[2][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) c[0][mt] = mfma_fp8_16x16x128(A[mt], cur.b[0], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t + 1 < 4) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          c[(t + 1) & 1][mt] = mfma_fp8_16x16x128(A[mt], cur.b[t + 1], v4f{0.f, 0.f, 0.f, 0.f});
      }
      __builtin_amdgcn_sched_barrier(0);
      float acc_sum = 0.0f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc_sum = fmaf(coef[mt][r], relu(c[t & 1][mt][r]), acc_sum);
      p[t] = acc_sum;
    }
    // Reduce over the 4 lane groups and scatter: lane group g keeps tile g.
    // The lane swaps run on the vector ALU (no LDS round trip): swapping the
    // upper half of tile t with the lower half of tile t + 2 leaves every lane
    // with its own and its partner's (lane ^ 32) partial of the tile its half
    // keeps, in the two results; likewise for lane ^ 16 one level down.
    const float x0 = swap_sum<false>(p[0], p[2]);
    const float x1 = swap_sum<false>(p[1], p[3]);
    const float score = swap_sum<true>(x0, x1) * cur.ks;
    if (SEL) {
      if (s0 + lane < s_end) {
        rowbuf[s0 + lane] = score;
        atomicAdd(&hist[order_key(score) >> 21], 1u);
      }
      return;
    }
    const int j = ((s0 - s_begin) >> 6) & 3;  // step within the 256-key group
    sbuf[wave][64 * j + lane] = score;
    // Lane l stores keys g0 + 4l .. g0 + 4l + 3 of the group.
    if (j == 3 || s0 + 64 >= s_end) pending = s0 - 64 * j;
  };

  // Steps are taken in pairs while both have a successor to prefetch; the
  // last one or two are peeled, so the prefetch in the loop is unconditional.
  int i = 0;
  for (; i + 2 < nsteps; i += 2) {
    step(s_begin + 64 * i, kb0, &kb1);
    step(s_begin + 64 * (i + 1), kb1, &kb0);
  }
  if (nsteps - i == 2) {
    step(s_begin + 64 * i, kb0, &kb1);
    step(s_begin + 64 * (i + 1), kb1, nullptr);
  } else if (nsteps - i == 1) {
    step(s_begin + 64 * i, kb0, nullptr);
  }
  if (pending >= 0) flush(pending);

  if (SEL) {  // the row's scores and first-digit histogram are in LDS
    __shared__ int sm[IDX_WAVES];
    __shared__ uint64_t sm64[IDX_WAVES];
    __shared__ int res[TOPK_RES_WORDS];
    __syncthreads();
    select_row<IDX_WAVES * WAVE>(rowbuf, nvis, a.sel_k, HIST_LDS, nullptr, hist, sm, sm64, res,
                                 a.sel_idx + (int64_t)q * a.sel_k, a.sel_count + q);
    return;
  }

  if (HIST) {
    __syncthreads();
    uint32_t *gh = a.hist + (int64_t)q * TOPK_BINS;
    for (int b = threadIdx.x; b < TOPK_BINS; b += blockDim.x) {
      const uint32_t c = hist[b];
      if (c) atomicAdd(&gh[b], c);
    }
  }
}

// The longest run per wavefront that still gives the chip enough wavefronts:
// long runs amortise each wavefront's set-up (its query's q, weights and
// histogram), short ones keep enough loads in flight when only a few queries
// stream long histories from HBM.
static int indexer_kpw(int num_q, int max_nvis) {
  int kpw = IDX_KPW_MIN;
  while (kpw < IDX_KPW_MAX) {
    const int64_t chunks = (max_nvis + IDX_WAVES * 2 * kpw - 1) / (IDX_WAVES * 2 * kpw);
    if ((int64_t)num_q * chunks * IDX_WAVES < IDX_MIN_WAVES) break;
    kpw *= 2;
  }
  return kpw;
}

bool indexer_selects(int num_q, int max_nvis) {
  return num_q > 0 && max_nvis > 0 && max_nvis <= TOPK_ROW_MAX &&
         IDX_WAVES * indexer_kpw(num_q, max_nvis) >= max_nvis;
}

hipError_t launch_indexer(const IndexerLaunch &a, hipStream_t st) {
  if (a.num_q == 0 || a.max_nvis == 0) return hipSuccess;
  const int kpw = indexer_kpw(a.num_q, a.max_nvis);
  const int nchunks = (a.max_nvis + IDX_WAVES * kpw - 1) / (IDX_WAVES * kpw);
  const bool sel = a.sel_idx != nullptr;
  if (sel && (nchunks != 1 || a.hist || !a.sel_count || a.max_nvis > TOPK_ROW_MAX)) return hipErrorInvalidValue;
  const int64_t blocks = (int64_t)a.num_q * nchunks;
  const dim3 grid((unsigned)blocks), block(IDX_WAVES * WAVE);
  if (a.k_e8m0) {
    if (sel)
      hipLaunchKernelGGL((indexer_kernel<false, true, true>), grid, block, 0, st, a, nchunks, kpw);
    else if (a.hist)
      hipLaunchKernelGGL((indexer_kernel<true, true, false>), grid, block, 0, st, a, nchunks, kpw);
    else
      hipLaunchKernelGGL((indexer_kernel<false, true, false>), grid, block, 0, st, a, nchunks, kpw);
  } else {
    if (sel)
      hipLaunchKernelGGL((indexer_kernel<false, false, true>), grid, block, 0, st, a, nchunks, kpw);
    else if (a.hist)
      hipLaunchKernelGGL((indexer_kernel<true, false, false>), grid, block, 0, st, a, nchunks, kpw);
    else
      hipLaunchKernelGGL((indexer_kernel<false, false, false>), grid, block, 0, st, a, nchunks, kpw);
  }
  return hipGetLastError();
}

}  // namespace dsa
