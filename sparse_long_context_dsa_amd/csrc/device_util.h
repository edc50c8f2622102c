// Small device helpers for the gfx950 (CDNA4) kernels: 64-lane wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

constexpr int WAVE = 64;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, WAVE); }
__device__ __forceinline__ int shfl_xor(int v, int mask) { return __shfl_xor(v, mask, WAVE); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor(v, m));
  return v;
}

// 16x16 FP8 (E4M3 x E4M3) product over K = 128 into fp32: lane l holds A row
// l & 15 (B column l & 15) as the 32 bytes [32 (l >> 4), +32) of its K range;
// the result's lane l holds column l & 15, rows 4 (l >> 4) .. + 3.
__device__ __forceinline__ v4f mfma_fp8_16x16x128(const v8i &a, const v8i &b, const v4f &c) {
  // Format 0 = FP8 E4M3 for both operands; E8M0 scale 127 = 2^0 (no scaling).
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0x7F7F7F7F, 0, 0x7F7F7F7F);
}

__device__ __forceinline__ v8i load32(const uint8_t *p) {
  const uint4 x0 = *reinterpret_cast<const uint4 *>(p);
  const uint4 x1 = *reinterpret_cast<const uint4 *>(p + 16);
  v8i r;
  r[0] = (int)x0.x; r[1] = (int)x0.y; r[2] = (int)x0.z; r[3] = (int)x0.w;
  r[4] = (int)x1.x; r[5] = (int)x1.y; r[6] = (int)x1.z; r[7] = (int)x1.w;
  return r;
}

// Value of v in lane l (l uniform across the wavefront).
__device__ __forceinline__ int64_t readlane64(int64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), l);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Order-preserving map fp32 -> uint32: a larger float gives a larger key.
// -0 is mapped like +0 so that the two compare equal.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Workgroup barrier for LDS traffic only: waits for this wavefront's LDS
// operations, not for its outstanding global loads (which __syncthreads'
// release fence would also wait for), so loads issued earlier keep flying.
// Use only where the threads exchange data through LDS.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Inclusive prefix sums over the 64 lanes of a wavefront from DPP moves
// (six dependent ALU steps, no trip through the LDS crossbar as a lane
// shuffle takes): row_shr 1, 2, 4, 8 make the sums within each row of 16
// lanes, then row_bcast:15 adds row 0's total to row 1 and row 2's to row 3,
// and row_bcast:31 adds the total of rows 0 and 1 to rows 2 and 3.  A lane
// with no source lane, or in a row the row mask leaves out, receives 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_or_zero(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_or_zero(uint64_t v) {
  const uint32_t lo = dpp_or_zero<CTRL, ROW_MASK>((uint32_t)v);
  const uint32_t hi = dpp_or_zero<CTRL, ROW_MASK>((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
constexpr int DPP_ROW_SHR = 0x110, DPP_ROW_BCAST15 = 0x142, DPP_ROW_BCAST31 = 0x143;
template <typename U>
__device__ __forceinline__ U wave_inclusive_scan_u(U v) {
  v += dpp_or_zero<DPP_ROW_SHR + 1, 0xF>(v);
  v += dpp_or_zero<DPP_ROW_SHR + 2, 0xF>(v);
  v += dpp_or_zero<DPP_ROW_SHR + 4, 0xF>(v);
  v += dpp_or_zero<DPP_ROW_SHR + 8, 0xF>(v);
  v += dpp_or_zero<DPP_ROW_BCAST15, 0xA>(v);
  v += dpp_or_zero<DPP_ROW_BCAST31, 0xC>(v);
  return v;
}
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  return (int)wave_inclusive_scan_u<uint32_t>((uint32_t)v);
}
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) { return wave_inclusive_scan_u<uint32_t>(v); }
__device__ __forceinline__ uint64_t wave_inclusive_scan(uint64_t v) { return wave_inclusive_scan_u<uint64_t>(v); }

}  // namespace dsa
