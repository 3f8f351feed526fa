// quant_row.hpp -- the per-row dynamic quantization steps as block-level
// device functions, used by the standalone quantizer and by kernels that
// quantize their activation row in place.  Every caller must be compiled
// with FP contraction off so the f32 sequence is the documented one.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace qp {

__device__ __forceinline__ float qp_min(float a, float b) { return b < a ? b : a; }
__device__ __forceinline__ float qp_max(float a, float b) { return b > a ? b : a; }

// Scale and zero point of one row, computed by the whole workgroup; every
// thread returns the same (s, z).  `red_*` are LDS scratch of one float per
// wave.  Requires blockDim.x to be a multiple of 64 and <= 64 * 16.
__device__ __forceinline__ void row_params_block(const float* __restrict__ xr, int64_t K,
                                                 float* red_min, float* red_max, float* s_out,
                                                 int32_t* z_out) {
  float lo = 0.0f, hi = 0.0f;
  for (int64_t k = threadIdx.x; k < K; k += blockDim.x) {
    float v = xr[k];
    lo = qp_min(lo, v);
    hi = qp_max(hi, v);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    lo = qp_min(lo, __shfl_xor(lo, off, 64));
    hi = qp_max(hi, __shfl_xor(hi, off, 64));
  }
  const int wave = threadIdx.x / 64, nwaves = blockDim.x / 64;
  if ((threadIdx.x & 63) == 0) {
    red_min[wave] = lo;
    red_max[wave] = hi;
  }
  __syncthreads();
  lo = red_min[0];
  hi = red_max[0];
  for (int i = 1; i < nwaves; ++i) {
    lo = qp_min(lo, red_min[i]);
    hi = qp_max(hi, red_max[i]);
  }
  float s = (hi - lo) / 255.0f;
  int32_t z = 0;
  if (s == 0.0f) {
    s = 1.0f;
  } else {
    float zf = __builtin_rintf(-128.0f - lo / s);
    zf = zf < -128.0f ? -128.0f : (zf > 127.0f ? 127.0f : zf);
    z = (int32_t)zf;
  }
  *s_out = s;
  *z_out = z;
}

__device__ __forceinline__ int8_t quantize_one(float x, float s, int32_t z) {
  float r = __builtin_rintf(x / s);
  // |x/s| <= 255 for in-row values, so the conversion is exact.
  int32_t v = (int32_t)r + z;
  v = v < -128 ? -128 : (v > 127 ? 127 : v);
  return (int8_t)v;
}

// Quantizes xr[0..K) into qr and writes zeros into qr[K..kfill).
__device__ __forceinline__ void quantize_row_block(const float* __restrict__ xr, int64_t K,
                                                   int64_t kfill, float s, int32_t z,
                                                   int8_t* __restrict__ qr) {
  for (int64_t k = threadIdx.x; k < kfill; k += blockDim.x)
    qr[k] = k < K ? quantize_one(xr[k], s, z) : (int8_t)0;
}

}  // namespace qp
