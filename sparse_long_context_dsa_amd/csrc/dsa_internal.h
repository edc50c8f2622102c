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
// Power-of-two scales: e8m0[row] = e + 127, scales[row] = 2^e (scales may be null).
hipError_t launch_quantize_fp8_e8m0(const float *x, int64_t rows, int cols, uint8_t *codes,
                                    uint8_t *e8m0, float *scales, hipStream_t st);

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
  const uint8_t *k_e8m0;  // key scales as E8M0 exponents instead of k_scale (null: use k_scale)
  // Select in the indexer (only when indexer_selects(num_q, max_nvis)): the
  // scores stay on chip and each block writes its query's top-k positions
  // idx[q, 0 .. sel_k) and count[q]; hist must be null.  Queries with
  // n_vis <= skip_le keep every position.
  int32_t *sel_idx;
  int32_t *sel_count;
  int32_t sel_k;
};
// Whether one indexer block covers every query's whole history, so that the
// indexer can select the rows itself.
bool indexer_selects(int num_q, int max_nvis);
hipError_t launch_indexer(const IndexerLaunch &a, hipStream_t st);

// Top-k: radix digits of 11/11/10 bits; rows up to TOPK_ROW_MAX are selected
// by one block from registers and LDS, longer rows by blocks of TOPK_LONG_SPAN
// positions that stream the row once, the last of them finishing the row.
constexpr int TOPK_BINS = 2048;
constexpr int TOPK_ROW_MAX = 16384;
constexpr int TOPK_CHUNK = 16384;      // score chunk of the standalone first-digit histogram
constexpr int TOPK_MAX_CHUNKS = 64;    // histories up to 2^20 positions
constexpr int MAX_NVIS = TOPK_CHUNK * TOPK_MAX_CHUNKS;
constexpr int TOPK_LONG_WAVES = 16;    // wavefronts of a long-row block
constexpr int TOPK_WAVE_SPAN = 2048;   // positions per wavefront (4 rounds of 512)
constexpr int TOPK_LONG_SPAN = TOPK_LONG_WAVES * TOPK_WAVE_SPAN;  // 32768 positions per block
constexpr int TOPK_STREAM_MAX = 131072;  // rows up to this length: one streaming block per row
struct TopkWs {
  uint32_t *hist;     // [num_q, TOPK_BINS] first-digit histogram (zero between calls: readers clear it)
  uint2 *b1info;      // [num_q] long rows: (first-digit threshold bin B1, keys above B1)
  uint32_t *wcnt;     // [num_q, nblk, TOPK_LONG_WAVES] candidates per wavefront
  uint2 *cand;        // [num_q, nblk, TOPK_LONG_WAVES, TOPK_WAVE_SPAN] (key, position)
  uint32_t *hist2;    // [num_q, nblk, TOPK_BINS] per span: second-digit histogram of its keys in bin B1
  int32_t nblk;       // long-row blocks per query (0 when every row fits TOPK_ROW_MAX)
  int32_t nchunks;    // score chunks per row for the standalone histogram
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
  bool dense;            // every visible position, no idx (k = the longest history)
};
int mla_num_splits(int num_q, int k, bool decode);
// Decode batches of up to 64 queries split each query's heads over four
// workgroups, and its rows over mla_hg_splits() of them each (mla_hg_kernel;
// with one split no partials and no combine); 0 selects the row-split kernel
// (mla_kernel over all 128 heads, then the combine of the splits' partials).
int mla_hg_splits(int num_q, int k, bool decode, bool dense);
int mla_hg_rows_per_split(int k, int nsplit);
hipError_t launch_mla_hg(const MlaLaunch &a, float scale_log2, bool wide, int nsplit, float *part_o,
                         float *part_lse, hipStream_t st);
// Row splits of the dense mode: the time model, with at most 2080 tiles of 32
// rows per workgroup (its per-tile row table lives in LDS).
int mla_dense_splits(int num_q, int max_nvis);
// dense: the workspace of the dense mode, k being the longest history.
size_t mla_ws_bytes(int num_q, int k, bool decode, bool dense = false);
hipError_t launch_mla(const MlaLaunch &a, bool decode, void *ws, hipStream_t st);

// Indexer alignment loss: target a[r] = sum_h exp(z[h, r] - lse[h]) over each
// query's set (written into grad), then KL(a / |a|_1 || Softmax(I)) per query
// and its gradient (overwriting grad), and the sum over the queries.
struct KlLaunch {
  const uint16_t *q;
  const uint16_t *kv;
  const int32_t *idx;    // sparse: [num_q, k] set positions; null: every visible position
  const int32_t *count;  // may be null
  const int32_t *q_seq;
  const int32_t *q_nvis;
  KvMap map;
  const float *lse;      // [num_q, 128] the attention's log-sum-exp over the same set
  const float *scores;   // [num_q, ld_scores] indexer scores by position
  int64_t ld_scores;
  int32_t k;             // sparse: the idx row length
  int32_t num_q;
  float softmax_scale;
  int64_t num_rows;      // rows of the latent cache
  float *grad;           // [num_q, ld_out]: sparse in set order (ld_out = k), dense by position
  int64_t ld_out;
  float *target;         // may be null; same layout as grad
  float *kl;             // [num_q]
  float *loss;           // may be null
};
// max_set: the largest set (sparse: min(k, longest history); dense: the longest history).
hipError_t launch_indexer_kl(const KlLaunch &a, int max_set, hipStream_t st);

// Backward of the indexer score: dq, dw overwritten, dk accumulated (fp32 atomics).
struct IndexerBwdLaunch {
  const uint8_t *q8;     // [num_q, 64, 128]
  const float *q_scale;  // [num_q, 64] or null (1)
  const float *w;        // [num_q, 64]
  const uint8_t *k8;     // [rows, 128]
  const float *k_scale;  // [rows]
  const int32_t *idx;    // sparse: [num_q, k]; null: every visible position
  const int32_t *count;  // may be null
  const int32_t *q_seq;
  const int32_t *q_nvis;
  KvMap map;
  int32_t k;
  int32_t num_q;
  const float *grad;     // dL/dI: sparse [num_q, k] in set order, dense [num_q, ld_grad] by position
  int64_t ld_grad;
  float *dq;             // [num_q, 64, 128]
  float *dw;             // [num_q, 64]
  float *dk;             // [rows, 128], added to
  int32_t num_seqs;      // sequences of the layout (the dense mode's key tiles)
};
hipError_t launch_indexer_bwd(const IndexerBwdLaunch &a, int max_set, hipStream_t st);

}  // namespace dsa
