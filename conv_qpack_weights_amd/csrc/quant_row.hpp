// quant_row.hpp -- the per-row dynamic quantization steps as workgroup-level
// device functions, used by the standalone quantizer and by the A8W4 GEMV,
// which quantizes its activation row itself.  Every caller must be compiled
// with FP contraction off so the f32 sequence is the documented one:
//   rmin = min(0, min x); rmax = max(0, max x); scale = (rmax - rmin) / 255
//   (scale == 0 -> scale = 1, zp = 0); zp = clamp(rint(-128 - rmin/scale));
//   q = clamp(rint(x/scale) + zp, -128, 127)      (IEEE division, RHE rint)
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace qp {

__device__ __forceinline__ float qp_min(float a, float b) { return b < a ? b : a; }
__device__ __forceinline__ float qp_max(float a, float b) { return b > a ? b : a; }

// DPP row operations (16-lane rows): quad_perm [1,0,3,2], [2,3,0,1],
// row_half_mirror, row_mirror.  After the four steps every lane of a row
// holds the row's reduction.
template <typename Op>
__device__ __forceinline__ float row16_reduce(float v, Op op) {
  v = op(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                  0xB1, 0xF, 0xF, false)));
  v = op(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                  0x4E, 0xF, 0xF, false)));
  v = op(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                  0x141, 0xF, 0xF, false)));
  v = op(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                  0x140, 0xF, 0xF, false)));
  return v;
}

// Wave-wide reduction in a fixed order: rows reduced by DPP, then the four
// row results combined as ((r0 op r1) op r2) op r3; wave-uniform result.
template <typename Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
  v = row16_reduce(v, op);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return op(op(op(r0, r1), r2), r3);
}

struct MinOp {
  __device__ float operator()(float a, float b) const { return qp_min(a, b); }
};
struct MaxOp {
  __device__ float operator()(float a, float b) const { return qp_max(a, b); }
};
struct AddOp {
  __device__ float operator()(float a, float b) const { return a + b; }
};

// Scale and zero point from the row extremes (already widened to include 0).
__device__ __forceinline__ void params_from_range(float lo, float hi, float* s_out,
                                                  int32_t* z_out) {
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

// (symmetric rows never reach -128: |x/s| <= 127 up to one rounding)
__device__ __forceinline__ uint32_t quantize_one(float x, float s, int32_t z) {
  const float r = __builtin_rintf(x / s);
  // |x/s| <= 255 for in-row values, so the conversion is exact.
  int32_t v = (int32_t)r + z;
  v = v < -128 ? -128 : (v > 127 ? 127 : v);
  return (uint32_t)(uint8_t)(int8_t)v;
}

// Workgroup quantization of one row of K floats into `dst` (LDS or global),
// zero-filling dst[K, kfill).  Thread t owns 16 consecutive values per pass
// (16-byte loads when `vec`: x 16-byte aligned).  Codes are written 16 bytes
// at a time when `dst_vec` (dst 16-byte aligned), else byte by byte.  `red`
// is LDS scratch of 2 floats per wave.  Requires blockDim.x == NT (a
// multiple of 64).
// kChunkMajor: dst receives the codes permuted for the A8W4 GEMV -- within
// each 128-K block the 8-byte piece (t, c) holding k = 32t + 8c .. +8 goes to
// offset 32c + 8t, so the four pieces one lane needs are 32 contiguous
// bytes (requires kfill % 128 == 0 and a 16-byte aligned dst).
// The thread's first E values, loaded ahead (quantize_row_first) so that a
// caller can put the row's loads in flight before other traffic.  The loads
// are unconditional buffer loads bounded by the row (past its end they
// return zeros and touch no memory), so no branch joins their results: a
// join would make the compiler wait for them right away.  quantize_row_wg
// uses them only where a whole aligned vector lies inside the row.
struct RowFirst {
  float4 v[4];
};
template <int NT, int E = 16>
__device__ __forceinline__ RowFirst quantize_row_first(const float* __restrict__ x, int64_t K,
                                                       bool vec) {
  static_assert(E == 16 || E == 8 || E == 4, "4, 8 or 16 values per thread");
  RowFirst f;
  const int64_t k0 = (int64_t)threadIdx.x * E;
  const uint32_t bytes = (uint32_t)(K < (INT64_C(1) << 29) ? 4 * K : (INT64_C(1) << 31));
  const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(x), 0, bytes, 0x00020000);
  const uint32_t off = (uint32_t)(k0 < (INT64_C(1) << 29) ? 4 * k0 : (INT64_C(1) << 31));
#pragma unroll
  for (int q = 0; q < E / 4; ++q) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off + 16 * q, 0, 0);
    // (bit_cast of a vector element would read element 0: copy them out first)
    const uint32_t v0 = v[0], v1 = v[1], v2 = v[2], v3 = v[3];
    f.v[q] = make_float4(__builtin_bit_cast(float, v0), __builtin_bit_cast(float, v1),
                         __builtin_bit_cast(float, v2), __builtin_bit_cast(float, v3));
  }
  (void)vec;
  return f;
}

// The steps of one row's quantization, for NT threads (threadIdx.x < NT
// take part; NT a multiple of 64) and E values per thread per pass (16, or
// 8 or 4 to spread a short row over more threads).  kSym: the symmetric
// variant -- scale = max|x| / 127 (1 for an all-zero row), zero point 0,
// codes clamp(rint(x/scale), -127, 127).
//
// Step 1, row_extremes_partial: each thread's extremes over its values, a
// wave reduction, and the wave's pair written to red[wave], red[NT/64 +
// wave].  A thread's first E values stay in `first` for step 3 (rows of up
// to E*NT values are read once); `pre` optionally holds them already loaded.
// kOne: the caller guarantees K == NT*E, a 16-byte aligned x and `pre`
// (one pass of whole vectors, no fallbacks).
template <int NT, int E, bool kSym, bool kOne = false>
__device__ __forceinline__ void row_extremes_partial(const float* __restrict__ x, int64_t K,
                                                     bool vec, float* red, float4 (&first)[4],
                                                     const RowFirst* pre) {
  static_assert(E == 16 || E == 8 || E == 4, "4, 8 or 16 values per thread");
  constexpr int NW = NT / 64;
  constexpr int Q = E / 4;
  const int t = threadIdx.x;
  float lo = 0.0f, hi = 0.0f;
  if constexpr (kOne) {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const float4 v = pre->v[q];
      first[q] = v;
      if constexpr (kSym) {
        hi = qp_max(qp_max(qp_max(qp_max(hi, __builtin_fabsf(v.x)), __builtin_fabsf(v.y)),
                           __builtin_fabsf(v.z)),
                    __builtin_fabsf(v.w));
      } else {
        lo = qp_min(qp_min(qp_min(qp_min(lo, v.x), v.y), v.z), v.w);
        hi = qp_max(qp_max(qp_max(qp_max(hi, v.x), v.y), v.z), v.w);
      }
    }
  }
  for (int64_t k0 = (int64_t)t * E; !kOne && k0 < K; k0 += NT * E) {
    if (vec && k0 + E <= K) {
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const float4 v = (pre && k0 == (int64_t)t * E)
                             ? pre->v[q]
                             : *reinterpret_cast<const float4*>(x + k0 + 4 * q);
        if (k0 == (int64_t)t * E) first[q] = v;
        if constexpr (kSym) {
          hi = qp_max(qp_max(qp_max(qp_max(hi, __builtin_fabsf(v.x)), __builtin_fabsf(v.y)),
                             __builtin_fabsf(v.z)),
                      __builtin_fabsf(v.w));
        } else {
          lo = qp_min(qp_min(qp_min(qp_min(lo, v.x), v.y), v.z), v.w);
          hi = qp_max(qp_max(qp_max(qp_max(hi, v.x), v.y), v.z), v.w);
        }
      }
    } else {
      for (int j = 0; j < E; ++j)
        if (k0 + j < K) {
          const float v = x[k0 + j];
          if constexpr (kSym) {
            hi = qp_max(hi, __builtin_fabsf(v));
          } else {
            lo = qp_min(lo, v);
            hi = qp_max(hi, v);
          }
        }
    }
  }
  lo = wave_reduce(lo, MinOp{});
  hi = wave_reduce(hi, MaxOp{});
  const int wave = t >> 6;
  if ((t & 63) == 0) {
    red[wave] = lo;
    red[NW + wave] = hi;
  }
}

// Step 2 (after a barrier that makes step 1's writes visible): the row's
// scale and zero point from the waves' pairs, combined in wave order.
template <int NT, bool kSym>
__device__ __forceinline__ void row_params(const float* red, float* s_out, int32_t* z_out) {
  constexpr int NW = NT / 64;
  float lo = red[0], hi = red[NW];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    lo = qp_min(lo, red[w]);
    hi = qp_max(hi, red[NW + w]);
  }
  if constexpr (kSym) {
    float s = hi / 127.0f;
    if (s == 0.0f) s = 1.0f;
    *s_out = s;
    *z_out = 0;
  } else {
    params_from_range(lo, hi, s_out, z_out);
  }
}

// Step 3: the codes of the thread's values into dst[0, kfill) (zeros past
// K); beyond the first E values per thread, x is read again.  Codes are
// written 16 bytes at a time when `dst_vec` (dst 16-byte aligned), else
// byte by byte.
// kChunkMajor: dst receives the codes permuted for the A8W4 GEMV -- within
// each 128-K block the 8-byte piece (t, c) holding k = 32t + 8c .. +8 goes to
// offset 32c + 8t, so the four pieces one lane needs are 32 contiguous
// bytes (requires kfill % 128 == 0 and a 16-byte aligned dst).
// kOne: as for step 1, and kfill == K (the thread's E values, once).
template <int NT, int E, bool kChunkMajor, bool kSym, bool kOne = false>
__device__ __forceinline__ void row_codes(const float* __restrict__ x, int64_t K, int64_t kfill,
                                          bool vec, bool dst_vec, int8_t* __restrict__ dst,
                                          float s, int32_t z, const float4 (&first)[4]) {
  constexpr int Q = E / 4;
  const int t = threadIdx.x;
  const bool keep = kOne || (vec && (int64_t)t * E + E <= K);
  for (int64_t k0 = (int64_t)t * E; kOne || k0 < kfill; k0 += NT * E) {
    uint32_t w[Q];
    if (kOne || (vec && k0 + E <= K)) {
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const float4 v = (keep && k0 == (int64_t)t * E)
                             ? first[q]
                             : *reinterpret_cast<const float4*>(x + k0 + 4 * q);
        w[q] = quantize_one(v.x, s, z) | (quantize_one(v.y, s, z) << 8) |
               (quantize_one(v.z, s, z) << 16) | (quantize_one(v.w, s, z) << 24);
      }
    } else {
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        uint32_t acc = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t k = k0 + 4 * q + j;
          if (k < K) acc |= quantize_one(x[k], s, z) << (8 * j);
        }
        w[q] = acc;
      }
    }
    if constexpr (kChunkMajor) {
      // the 8-byte piece holding k = 128b + 32g + 8c .. +8 goes to 128b + 32c + 8g
      if constexpr (E == 4) {  // half a piece: k0 % 8 is 0 or 4
        const int64_t b = k0 >> 7, g = (k0 >> 5) & 3, cc = (k0 >> 3) & 3;
        *reinterpret_cast<uint32_t*>(dst + b * 128 + cc * 32 + g * 8 + (k0 & 4)) = w[0];
      } else {
#pragma unroll
        for (int h = 0; h < Q / 2; ++h) {
          const int64_t kk = k0 + 8 * h;
          const int64_t b = kk >> 7, g = (kk >> 5) & 3, cc = (kk >> 3) & 3;
          *reinterpret_cast<uint2*>(dst + b * 128 + cc * 32 + g * 8) =
              make_uint2(w[2 * h], w[2 * h + 1]);
        }
      }
    } else if (dst_vec && k0 + E <= kfill) {
      if constexpr (E == 16)
        *reinterpret_cast<uint4*>(dst + k0) = make_uint4(w[0], w[1], w[2], w[3]);
      else if constexpr (E == 8)
        *reinterpret_cast<uint2*>(dst + k0) = make_uint2(w[0], w[1]);
      else
        *reinterpret_cast<uint32_t*>(dst + k0) = w[0];
    } else {
      for (int j = 0; j < E && k0 + j < kfill; ++j) dst[k0 + j] = (int8_t)(w[j >> 2] >> (8 * (j & 3)));
    }
    if constexpr (kOne) break;
  }
}

// Workgroup quantization of one row of K floats into `dst` (LDS or global):
// the three steps with a barrier between the first two.  Every thread of
// the workgroup (blockDim.x == NT) takes part; `red` is LDS scratch of 2
// floats per wave.
template <int NT, bool kChunkMajor = false, int E = 16, bool kSym = false>
__device__ __forceinline__ void quantize_row_wg(const float* __restrict__ x, int64_t K,
                                                int64_t kfill, bool vec, bool dst_vec,
                                                int8_t* __restrict__ dst, float* red,
                                                float* s_out, int32_t* z_out,
                                                const RowFirst* pre = nullptr) {
  float4 first[4];
  row_extremes_partial<NT, E, kSym>(x, K, vec, red, first, pre);
  __syncthreads();
  float s;
  int32_t z;
  row_params<NT, kSym>(red, &s, &z);
  row_codes<NT, E, kChunkMajor, kSym>(x, K, kfill, vec, dst_vec, dst, s, z, first);
  *s_out = s;
  *z_out = z;
}

}  // namespace qp
