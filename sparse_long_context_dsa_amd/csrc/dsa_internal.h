// Internal declarations shared by the C-ABI layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

// Device view of a cache layout (passed to kernels by value).
struct KvMap {
  const int32_t *block_table;  // paged: [num_seqs, max_blocks]
  const int64_t *seq_row0;     // contiguous: [num_seqs]
  int32_t block_shift;         // log2(block_size); -1 for contiguous
  int32_t max_blocks;
};

// Position s of sequence seq -> physical cache row.
__device__ __forceinline__ int64_t phys_row(const KvMap &m, int seq, int s) {
  if (m.block_shift < 0) return m.seq_row0[seq] + s;
  const int b = s >> m.block_shift;
  const int64_t blk = m.block_table[(int64_t)seq * m.max_blocks + b];
  return (blk << m.block_shift) + (s - (b << m.block_shift));
}

// ---------------------------------------------------------------- launchers
hipError_t launch_quantize_fp8(const float *x, int64_t rows, int cols, uint8_t *codes,
                               float *scales, hipStream_t st);

struct IndexerLaunch {
  const uint8_t *q8;
  const float *q_scale;  // may be null
  const float *w;
  const uint8_t *k8;
  const float *k_scale;
  const int32_t *q_seq;
  const int32_t *q_nvis;
  KvMap map;
  float *scores;
  int64_t ld;
  uint32_t *hist;        // optional [num_q, TOPK_BINS] coarse histogram of the scores
  int32_t skip_le;       // queries with n_vis <= skip_le are not scored (-1: none)
  int32_t num_q;
  int32_t max_nvis;
};
hipError_t launch_indexer(const IndexerLaunch &a, hipStream_t st);

// Top-k: radix digits of 11/11/10 bits; rows up to TOPK_ROW_MAX are selected
// by one block from LDS, longer rows in chunks of TOPK_CHUNK.
constexpr int TOPK_BINS = 2048;
constexpr int TOPK_ROW_MAX = 16384;
constexpr int TOPK_CHUNK = 16384;
constexpr int TOPK_MAX_CHUNKS = 64;  // histories up to 2^20 positions
constexpr int MAX_NVIS = TOPK_CHUNK * TOPK_MAX_CHUNKS;
struct TopkWs {
  uint32_t *hist;     // [num_q, TOPK_BINS] first-digit histogram
  uint32_t *hist2;    // [num_q, TOPK_BINS] second-digit histogram (long rows)
  uint32_t *done;     // [num_q] blocks finished per query (long rows)
  uint32_t *ccount;   // [num_q, nchunks]
  uint2 *cand;        // [num_q, nchunks, TOPK_CHUNK] (key, position) candidates
  int32_t nchunks;    // 0 when every row fits TOPK_ROW_MAX
};
size_t topk_ws_bytes(int num_q, int max_nvis);
TopkWs topk_ws_carve(void *ws, int num_q, int max_nvis);
hipError_t launch_topk_init(const TopkWs &ws, int num_q, hipStream_t st);
hipError_t launch_topk_hist(const float *scores, int64_t ld, const int32_t *q_nvis, const TopkWs &ws, int num_q,
                            int max_nvis, hipStream_t st);
hipError_t launch_topk_select(const float *scores, int64_t ld, const int32_t *q_nvis, int k, int32_t *idx,
                              int32_t *count, const TopkWs &ws, int num_q, int max_nvis, bool hist1_valid,
                              hipStream_t st);

// Sparse MLA.
struct MlaLaunch {
  const uint16_t *q;
  const uint16_t *kv;
  const int32_t *idx;
  const int32_t *count;  // may be null
  const int32_t *q_seq;
  const int32_t *q_nvis;
  KvMap map;
  int32_t k;
  int32_t num_q;
  float softmax_scale;
  float *out;
  float *lse;            // may be null
  int64_t num_rows;      // rows of the latent cache
};
int mla_num_splits(int num_q, int k, bool decode);
size_t mla_ws_bytes(int num_q, int k, bool decode);
hipError_t launch_mla(const MlaLaunch &a, bool decode, void *ws, hipStream_t st);

}  // namespace dsa
