// Latent-row tiles for the bf16 MFMA kernels over the 576-wide MLA cache
// (sparse attention and the indexer's attention target): the LDS tile layout,
// the gather of a tile straight into LDS, and the S^T = K . Q^T chain.
//
// Rows arrive in tiles of 32 latent rows (36 KiB), gathered through a per-block
// table of physical rows; every wavefront of a 4-wavefront block loads 8 rows
// of each tile (9 x 16 bytes per lane) and reads all 32 of them back for its
// 32 heads.
#pragma once

#include "device_util.h"
#include "dsa_internal.h"

namespace dsa {

constexpr int MLA_WAVES = 4;
constexpr int MLA_THREADS = MLA_WAVES * WAVE;
constexpr int MLA_T = 32;                            // rows per tile
constexpr int ROW_BYTES = 576 * 2;                   // 1152
constexpr int TILE_BYTES = MLA_T * ROW_BYTES;        // 36864
constexpr int LOADS_PER_WAVE = TILE_BYTES / 16 / WAVE / MLA_WAVES;  // 9
constexpr uint32_t INVALID_ROW = 0x80000000u;        // marks a position outside [0, n_vis)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
static_assert(LOADS_PER_WAVE * 16 * WAVE * MLA_WAVES == TILE_BYTES, "tile = whole wave loads");

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;


__device__ __forceinline__ v8bf as_bf(const uint4 &u) { return __builtin_bit_cast(v8bf, u); }

// Tile layout in LDS.  The 32 rows x 72 chunks (16 bytes) of a tile are
// stored in four 9216-byte groups of 8 rows; inside a group, chunk block
// c >> 3 (9 blocks of 1 KiB) holds the 8 rows x 8 chunks as [row & 7][slot],
// slot = (c & 7) ^ row_xor(r).  A gather instruction then fills one
// contiguous 1 KiB block (lane l: row l >> 3, slot l & 7) and each lane reads
// a single cache row per tile.  With 64 four-byte banks, a 16-byte slot of
// row r starts in bank group 8 * (r & 1) + slot, and row_xor is chosen so
// that both read patterns hit 16 different groups:
//  * the QK read (16 lanes per cycle: 16 consecutive rows, one chunk) needs
//    row_xor to be a permutation over the 8 even and over the 8 odd rows;
//  * the transposing PV read (32 lanes per cycle: rows 4j .. 4j+3 of a
//    group, chunks 4m .. 4m+3) needs rows r and r + 2 of each such set to
//    differ in bit 2, which the chunks (bits 0-1) cannot reach.
__device__ __forceinline__ int row_xor(int r) { return (r & 7) ^ ((r >> 3) & 1) ^ (((r >> 1) & 1) << 2); }
__device__ __forceinline__ int tile_off(int r, int c) {
  return 9216 * (r >> 3) + 1024 * (c >> 3) + 128 * (r & 7) + 16 * ((c & 7) ^ row_xor(r));
}

// S^T chain of the QK product on a VGPR accumulator.  Written as asm
// statements so that S stays in VGPRs (next to the softmax that reads it)
// while all 256 AGPRs hold O; register operands only, and not volatile, so
// the LDS reads feeding them can be scheduled ahead.  Back-to-back MFMAs
// into the same accumulator need no wait states; the drain covers the
// MFMA-write -> VALU-read distance before the softmax reads S.
typedef int v4i_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void mfma_s_first(v16f &acc, const uint4 &a, const uint4 &b) {
  const v4i_t va = __builtin_bit_cast(v4i_t, a), vb = __builtin_bit_cast(v4i_t, b);
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(va), "v"(vb));
}
__device__ __forceinline__ void mfma_s(v16f &acc, const uint4 &a, const uint4 &b) {
  const v4i_t va = __builtin_bit_cast(v4i_t, a), vb = __builtin_bit_cast(v4i_t, b);
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(va), "v"(vb));
}
__device__ __forceinline__ void mfma_s_drain(v16f &acc) {
  asm("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(acc));
}

// Gathers this wavefront's share of the tile whose first row is prow entry r0:
// tile rows 8*wave .. 8*wave+7, lane l taking row l >> 3 and, in part i,
// chunk 8*i + ((l & 7) ^ row_xor(8*wave + (l >> 3))), into 1 KiB block i of
// the wavefront's 8-row group (see tile_off).  When `real` is false the parts
// read the block's first row into the (free) buffer instead, so the caller's
// instruction stream has no branch.
//
// The load is the buffer form (MUBUF) with one descriptor per block whose
// base is row `brow` of the cache, so every offset fits in 32 bits: a
// contiguous cache keeps a block's rows inside one sequence (< 2^20 rows), a
// paged pool below 4 GiB starts at row 0.  The compiler tracks this form as a
// plain memory load, so LDS reads issued while it is in flight keep exact wait
// counts.  A paged pool of 4 GiB or more (WIDE) takes the global form with
// 64-bit per-lane addresses, which the compiler treats as touching LDS and
// memory both: its LDS reads then wait for all LDS traffic.
//
// tile_row gives the lane's source row; issue_part issues part i of the
// gather (so that a caller can spread the parts between other work).
// Rows of a partial last tile past `last` repeat row `last` (finite data,
// masked out of the softmax).  In the dense mode prow holds one base row per
// 32-row tile instead (positions are consecutive, and a tile never straddles
// a cache block).
__device__ __forceinline__ uint32_t tile_row(const uint32_t *prow, int r0, bool real, int last, bool dense,
                                             int wave, int lane) {
  const int r = real ? min(r0 + 8 * wave + (lane >> 3), last) : 0;
  return dense ? prow[r >> 5] + (uint32_t)(r & (MLA_T - 1)) : prow[r] & ~INVALID_ROW;
}
template <bool WIDE>
__device__ __forceinline__ void issue_part(const __amdgpu_buffer_rsrc_t rs, const uint16_t *__restrict__ kv,
                                           uint32_t brow, uint32_t row, uint8_t *buf, int wave, int lane, int i) {
  const int cx = (lane & 7) ^ row_xor(8 * wave + (lane >> 3));
  uint8_t *dst = buf + 9216 * wave + 1024 * i;
  if (WIDE) {
    const uint16_t *src = kv + (size_t)row * 576 + 8 * cx + 64 * i;
    __builtin_amdgcn_global_load_lds(src, (lds_void *)dst, 16, 0, 0);
  } else {
    const uint32_t voff = (row - brow) * ROW_BYTES + 16 * cx + 128 * i;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)dst, 16, voff, 0, 0, 0);
  }
}
template <bool WIDE>
__device__ __forceinline__ void issue_tile(const __amdgpu_buffer_rsrc_t rs, const uint16_t *__restrict__ kv,
                                           uint32_t brow, const uint32_t *prow, int r0, bool real, int last,
                                           bool dense, uint8_t *buf, int wave, int lane) {
  const uint32_t row = tile_row(prow, r0, real, last, dense, wave, lane);
#pragma unroll
  for (int i = 0; i < LOADS_PER_WAVE; ++i) issue_part<WIDE>(rs, kv, brow, row, buf, wave, lane, i);
}

constexpr int MLA_MAX_ROWS = 2048;                   // selected rows per query (k <= 2048)
constexpr float RESCALE_LOG2 = 8.0f;                 // lazy-rescale threshold (log2 units)

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// Two floats -> two bf16 (round to nearest even) in one word, lo in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
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

// One accumulator register times s, as a VGPR value (the AGPR is unchanged).
__device__ __forceinline__ float read_scaled(const float &x, float s) {
  float r;
  asm("v_accvgpr_read_b32 %0, %1\n\t"
      "s_nop 1\n\t"
      "v_mul_f32 %0, %0, %2"
      : "=&v"(r)
      : "a"(x), "v"(s));
  return r;
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

// max(a, b, c) in one instruction.  fmaxf would add a canonicalising
// instruction per operand for values the compiler cannot see (accumulators
// written by inline asm); the scores are never signalling NaNs.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Maximum / sum of v over lanes l and l ^ 32 (one cross-half swap).
__device__ __forceinline__ float xhalf_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return max3f(a, b, b);
}
__device__ __forceinline__ float xhalf_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace dsa
