// Per-row FP8 E4M3 ("fn", max 448) quantiser for the indexer's q and key cache.
//
// Page "DeepSeekV3.2之DSA", part 4.3: the indexer consumes FP8 q and k with a
// dequantisation scale per key row; part 5.2 point 3: the index-key cache is
// stored per token in FP8.  Scale rule (not fixed by the pages): absmax / 448
// with an IEEE fp32 division, 1 for an all-zero row; the code is x / scale
// rounded to nearest-even on the E4M3 grid, saturated at +-448.
//
// The E8M0 variant (same page, part 4.3: the last step multiplies by the key
// scale in e8m0) takes the smallest power of two 2^e with absmax <= 448 * 2^e
// (e = 0 for an all-zero row, clamped to [-127, 127]): x / 2^e is then exact and
// never saturates, and the scale is stored as the byte e + 127.
//
// One wavefront per row; cols is a multiple of 64 (each lane owns cols/64
// elements, strided by 64 so that loads and byte stores are coalesced).
#include "device_util.h"
#include "dsa_internal.h"

namespace dsa {

// fp32 -> E4M3fn code with round-to-nearest-even, input already in [-448, 448].
__device__ __forceinline__ uint32_t e4m3_rne(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(y);
  uint32_t code;
  if (a < 0.015625f) {
    // Below the smallest normal (2^-6): multiples of 2^-9.  a * 512 is exact
    // and rintf rounds half to even.
    code = (uint32_t)rintf(a * 512.0f);  // 0..8; 8 is the smallest normal's code
  } else {
    const uint32_t au = __float_as_uint(a);
    const uint32_t e = (au >> 23) - 127u + 7u;  // biased E4M3 exponent, 1..15
    const uint32_t man = au & 0x7FFFFFu;
    code = (e << 3) | (man >> 20);
    const uint32_t rem = man & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (code & 1u))) code += 1u;  // may carry into e
  }
  return code | sign;
}

template <bool E8M0>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const float *__restrict__ x, int64_t rows,
                                                            int cols, uint8_t *__restrict__ codes,
                                                            float *__restrict__ scales,
                                                            uint8_t *__restrict__ e8m0) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int64_t row = (int64_t)blockIdx.x * (blockDim.x / WAVE) + (threadIdx.x / WAVE);
  if (row >= rows) return;
  const float *xr = x + row * cols;
  const int per = cols / WAVE;  // <= 8
  float v[8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i < per) {
      v[i] = xr[i * WAVE + lane];
      amax = fmaxf(amax, fabsf(v[i]));
    }
  }
  amax = wave_max(amax);
  uint8_t *cr = codes + row * cols;
  if (E8M0) {
    // amax = m * 2^E with m in [1, 2) (exact, subnormals included) and
    // 448 = 1.75 * 2^8, so the smallest e is E - 8 when m <= 1.75, else E - 7.
    int e = 0;
    if (amax > 0.0f) {
      const int E = ilogbf(amax);
      const float m = ldexpf(amax, -E);
      e = min(max(m <= 1.75f ? E - 8 : E - 7, -127), 127);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < per) cr[i * WAVE + lane] = (uint8_t)e4m3_rne(ldexpf(v[i], -e));  // exact scaling
    if (lane == 0) {
      e8m0[row] = (uint8_t)(e + 127);
      if (scales) scales[row] = ldexpf(1.0f, e);
    }
  } else {
    const float scale = (amax == 0.0f) ? 1.0f : amax / 448.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < per) {
        float y = v[i] / scale;
        y = fminf(fmaxf(y, -448.0f), 448.0f);
        cr[i * WAVE + lane] = (uint8_t)e4m3_rne(y);
      }
    }
    if (lane == 0) scales[row] = scale;
  }
}

hipError_t launch_quantize_fp8(const float *x, int64_t rows, int cols, uint8_t *codes,
                               float *scales, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const int waves = 4;
  const int64_t blocks = (rows + waves - 1) / waves;
  hipLaunchKernelGGL(quantize_rows_kernel<false>, dim3((unsigned)blocks), dim3(waves * WAVE), 0, st, x, rows,
                     cols, codes, scales, nullptr);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8_e8m0(const float *x, int64_t rows, int cols, uint8_t *codes, uint8_t *e8m0,
                                    float *scales, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const int waves = 4;
  const int64_t blocks = (rows + waves - 1) / waves;
  hipLaunchKernelGGL(quantize_rows_kernel<true>, dim3((unsigned)blocks), dim3(waves * WAVE), 0, st, x, rows,
                     cols, codes, scales, e8m0);
  return hipGetLastError();
}

}  // namespace dsa
