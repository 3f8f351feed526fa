// pack.hip -- one-time weight pre-pack into the library's blob.
//
// What a packed operand holds follows tract-linalg "frame/pack.rs"
// (PackedI8K4: K-contiguous int8 per output lane, zero-filled tails;
// pack_tensor_view: the padding is computed on, so it must be defined) and
// MNN "ConvInt8TiledExecutor.cpp" (reorderWeight: OIHW source with K ordered
// tap-outer / input-channel-inner; packWeightAndQuantInfo: scales stored next
// to the weights; _computeReorderQuantInfo: weight kernel sums precomputed).
// The layout itself is the GPU's: int8 weights in 32x32 (channel x K)
// sub-tiles so that each MFMA operand a GEMM wave needs is one contiguous
// kilobyte; int4 weights in 128-K blocks whose 16-byte chunks each feed four
// MFMA K-steps.
#include <cmath>
#include <cstring>
#include <vector>

#include "qp_internal.hpp"

#pragma clang fp contract(off)

namespace qp {
namespace {

// K index k -> element offset, for K built from up to three source axes
// (rank 2: one axis; OIHW: (kh, kw, ic)).
struct KMap {
  int64_t d1, d2;      // sizes of the two inner K axes
  int64_t t0, t1, t2;  // element strides of the three K axes
  __device__ __forceinline__ int64_t off(int64_t k) const {
    int64_t c = k % d2;
    int64_t ab = k / d2;
    int64_t b = ab % d1;
    int64_t a = ab / d1;
    return a * t0 + b * t1 + c * t2;
  }
};

__global__ void write_header_kernel(BlobHeader h, uint8_t* blob) {
  const uint32_t* src = reinterpret_cast<const uint32_t*>(&h);
  uint32_t* dst = reinterpret_cast<uint32_t*>(blob);
  int t = threadIdx.x;
  if (t < 64) dst[t] = src[t];
}

// One workgroup per padded row n.  Writes the row's Kpad bytes into the
// 32x32 sub-tile layout -- W[n,k] at ((n/32)*(Kpad/32) + k/32)*1024 +
// (n%32)*32 + k%32, so a GEMM wave fetches a 32-row x 32-K MFMA operand as
// one contiguous kilobyte -- plus its scale, zero point and colsum (sum over
// the real K only).
// kBlock (format 5, block-quantized int8): instead, the row's block scales
// scales[n*ldsw + b % period], stored block-major ([nblk][Npad], so a
// block's scales of consecutive channels are adjacent) (blocks of `group` K; OIHW weights repeat
// their per-input-channel-block scales over the kernel taps, period =
// IC/group) and its weight kernel sum wsum[n] = sum_b sw[n,b] * sum_{k in b}
// w[n,k] in fp64, from per-block integer sums gathered in LDS.
template <bool kBlock>
__global__ __launch_bounds__(256) void pack_s8_kernel(const int8_t* __restrict__ w, int64_t N,
                                                      int64_t K, int64_t Kpad, int64_t sn, KMap km,
                                                      const float* __restrict__ scales,
                                                      float scale, const int32_t* __restrict__ zps,
                                                      int32_t zp, uint8_t* __restrict__ blob,
                                                      int64_t data_off, int64_t scale_off,
                                                      int64_t sum_off, int64_t zp_off,
                                                      int64_t group, int64_t ldsw,
                                                      int64_t period) {
  extern __shared__ int32_t block_sum[];  // kBlock: Kpad/group entries
  const int64_t n = blockIdx.x;
  const int t = threadIdx.x;
  const bool live = n < N;
  const int64_t nblk = kBlock ? Kpad / group : 0;
  if constexpr (kBlock) {
    for (int64_t b = t; b < nblk; b += 256) block_sum[b] = 0;
    __syncthreads();
  }
  int32_t part = 0;
  uint8_t* tiles = blob + data_off + (n / 32) * (Kpad / 32) * 1024 + (n % 32) * 32;
  for (int64_t k0 = (int64_t)t * 16; k0 < Kpad; k0 += 256 * 16) {
    uint32_t words[4];
    int32_t chunk = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t v = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int64_t k = k0 + 4 * q + j;
        int32_t b = 0;
        if (live && k < K) b = w[n * sn + km.off(k)];
        chunk += b;
        v |= (uint32_t)(uint8_t)(int8_t)b << (8 * j);
      }
      words[q] = v;
    }
    part += chunk;
    if constexpr (kBlock) atomicAdd(&block_sum[k0 / group], chunk);
    *reinterpret_cast<uint4*>(tiles + (k0 / 32) * 1024 + (k0 % 32)) =
        make_uint4(words[0], words[1], words[2], words[3]);
  }
  if constexpr (kBlock) {
    __syncthreads();
    const int64_t Greal = (K + group - 1) / group;
    const int64_t Npad = gridDim.x;  // one workgroup per padded channel
    float* scol = reinterpret_cast<float*>(blob + scale_off) + n;  // [nblk][Npad]
    for (int64_t b = t; b < nblk; b += 256)
      scol[b * Npad] = (live && b < Greal) ? scales[n * ldsw + b % period] : 0.0f;
    if (t == 0) {
      double acc = 0.0;
      for (int64_t b = 0; b < nblk; ++b)
        acc = acc + (double)((live && b < Greal) ? scales[n * ldsw + b % period] : 0.0f) *
                        (double)block_sum[b];
      reinterpret_cast<float*>(blob + sum_off)[n] = live ? (float)acc : 0.0f;
    }
    return;
  }
  __shared__ int32_t red[256];
  red[t] = part;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (t < s) red[t] += red[t + s];
    __syncthreads();
  }
  if (t == 0) {
    float sc = live ? (scales ? scales[n] : scale) : 0.0f;
    int32_t z = live ? (zps ? zps[n] : zp) : 0;
    *reinterpret_cast<float*>(blob + scale_off + 4 * n) = sc;
    *reinterpret_cast<int32_t*>(blob + sum_off + 4 * n) = live ? red[0] : 0;
    *reinterpret_cast<int32_t*>(blob + zp_off + 4 * n) = z;
  }
}

// One workgroup per padded row n; thread r builds the 32-K run r (group-
// sized pieces of the row).  Within each 128-K block (64 bytes) byte
// 16c + 4t + j holds k = 32t + 8c + j (low nibble) and k = 32t + 8c + 4 + j
// (high nibble), so the 16 bytes at 16c hold the 8-K chunk c of four
// consecutive 32-K runs: one 16-byte load feeds four MFMA K-steps.  The 16
// channels of a tile store each block side by side (1 KiB per tile and
// block), and their scales likewise in quads of four groups (256 bytes), so
// one wave reads a tile's block, or its scales, as one contiguous piece.
//
// kKind selects the group-scale storage:
//  0  f32 scales (blob format 2);
//  1  bf16 scales (format 3): each scale rounded to the nearest bf16, ties
//     to even (the upper half of the f32 after adding 0x7FFF plus the lowest
//     kept bit); the channel's weight sum uses the rounded scales;
//  2  asymmetric (format 4): the source holds (offset, scale) pairs per
//     group, real weight = scale*q + offset; scales and offsets are stored
//     as two f32 arrays of the same layout, and the weight sum is that of
//     the real weights, sum_g (scale*sum q + offset*(real K in g)).
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int kKind>
__global__ __launch_bounds__(256) void pack_s4_kernel(
    const int8_t* __restrict__ w, int64_t N, int64_t K, int64_t Kpad, int64_t group, int64_t sn,
    KMap km, const float* __restrict__ sw, int64_t ldsw, uint8_t* __restrict__ blob,
    int64_t data_off, int64_t scale_off, int64_t sum_off, int64_t off_off) {
  constexpr bool kBf16 = kKind == 1, kAsym = kKind == 2;
  extern __shared__ int32_t run_sum[];  // Kpad/32 entries
  const int64_t n = blockIdx.x;
  const bool live = n < N;
  const int64_t runs = Kpad / 32;
  const int64_t G = Kpad / group;
  const int64_t Gq = (G + 3) / 4;
  const int64_t Greal = (K + group - 1) / group;
  const int64_t nblk = Kpad / 128;
  uint8_t* row = blob + data_off + (n / 16) * nblk * 1024 + (n % 16) * 64;  // + block * 1024
  int bad = 0;
  for (int64_t r = threadIdx.x; r < runs; r += blockDim.x) {
    const int64_t b = r / 4, t = r % 4;
    int32_t s = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint32_t v = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t klo = r * 32 + 8 * c + j, khi = klo + 4;
        const int32_t lo = (live && klo < K) ? w[n * sn + km.off(klo)] : 0;
        const int32_t hi = (live && khi < K) ? w[n * sn + km.off(khi)] : 0;
        bad |= (lo < -8) | (lo > 7) | (hi < -8) | (hi > 7);
        s += lo + hi;
        v |= ((uint32_t)(lo & 0xF) | ((uint32_t)(hi & 0xF) << 4)) << (8 * j);
      }
      *reinterpret_cast<uint32_t*>(row + b * 1024 + 16 * c + 4 * t) = v;
    }
    run_sum[r] = s;
  }
  if (bad) atomicOr(reinterpret_cast<int32_t*>(blob + kInvalidFlagOffset), 1);
  __syncthreads();
  // the stored values of group g's scale and offset
  auto stored = [&](int64_t g) -> float {
    const bool real = live && g < Greal;
    const float s = real ? sw[n * ldsw + (kAsym ? 2 * g + 1 : g)] : 0.0f;
    if constexpr (kBf16) return __builtin_bit_cast(float, bf16_bits(s) << 16);
    return s;
  };
  auto offset = [&](int64_t g) -> float {
    return (kAsym && live && g < Greal) ? sw[n * ldsw + 2 * g] : 0.0f;
  };
  const int64_t sidx = (n / 16) * Gq * 64 + (n % 16) * 4;
  for (int64_t g = threadIdx.x; g < 4 * Gq; g += blockDim.x) {
    const float s = stored(g);
    const int64_t e = sidx + (g / 4) * 64 + g % 4;
    if constexpr (kBf16)
      reinterpret_cast<uint16_t*>(blob + scale_off)[e] =
          (uint16_t)(__builtin_bit_cast(uint32_t, s) >> 16);
    else
      reinterpret_cast<float*>(blob + scale_off)[e] = s;
    if constexpr (kAsym) reinterpret_cast<float*>(blob + off_off)[e] = offset(g);
  }
  if (threadIdx.x == 0) {
    double acc = 0.0;
    const int64_t rpg = group / 32;
    for (int64_t g = 0; g < G; ++g) {
      int64_t gs = 0;
      for (int64_t r = g * rpg; r < (g + 1) * rpg; ++r) gs += run_sum[r];
      acc = acc + (double)stored(g) * (double)gs;
      if constexpr (kAsym) {
        int64_t cnt = K - g * group;
        cnt = cnt < 0 ? 0 : (cnt > group ? group : cnt);
        acc = acc + (double)offset(g) * (double)cnt;
      }
    }
    reinterpret_cast<float*>(blob + sum_off)[n] = live ? (float)acc : 0.0f;
  }
}

struct WeightView {
  int64_t N, K;
  int64_t sn;
  KMap km;
};

qp_status weight_view(const qp_qtensor* w, int32_t k_axis, int32_t n_axis, WeightView* v) {
  QP_REQUIRE(w, QP_EINVAL, "weights descriptor is NULL");
  if (w->rank == 2) {
    QP_REQUIRE((k_axis == 0 && n_axis == 1) || (k_axis == 1 && n_axis == 0), QP_EINVAL,
               "rank-2 weights need (k_axis, n_axis) to be a permutation of (0, 1); got (%d, %d)",
               k_axis, n_axis);
    v->N = w->shape[n_axis];
    v->K = w->shape[k_axis];
    v->sn = w->stride[n_axis];
    v->km = KMap{1, v->K, 0, 0, w->stride[k_axis]};
  } else if (w->rank == 4) {
    QP_REQUIRE(n_axis == 0 && k_axis == 1, QP_EINVAL,
               "rank-4 (OIHW) weights need n_axis = 0 and k_axis = 1; got (%d, %d)", k_axis,
               n_axis);
    int64_t IC = w->shape[1], KH = w->shape[2], KW = w->shape[3];
    v->N = w->shape[0];
    v->K = KH * KW * IC;
    v->sn = w->stride[0];
    v->km = KMap{KW, IC, w->stride[2], w->stride[3], w->stride[1]};
  } else {
    QP_FAIL(QP_EINVAL, "weights must be rank 2 or rank 4 (OIHW); got rank %d", w->rank);
  }
  for (int i = 0; i < w->rank; ++i)
    QP_REQUIRE(w->shape[i] > 0, QP_EINVAL, "weight dimension %d is %lld", i, (long long)w->shape[i]);
  QP_REQUIRE(w->rounding == QP_ROUND_HALF_EVEN, QP_EUNSUPPORTED,
             "only round-half-to-even is implemented");
  return QP_OK;
}

qp_status format_of(const qp_qtensor* w, int32_t* format) {
  if (w->dtype == QP_S8) {
    QP_REQUIRE(w->scheme == QP_PER_TENSOR || w->scheme == QP_PER_CHANNEL ||
                   w->scheme == QP_BLOCKWISE,
               QP_EUNSUPPORTED, "int8 weights support per-tensor, per-channel or blockwise "
               "scales (scheme %d)", w->scheme);
    if (w->scheme == QP_BLOCKWISE)
      QP_REQUIRE(w->zero_points == nullptr && w->zero_point == 0, QP_EUNSUPPORTED,
                 "block-quantized int8 weights are symmetric: zero points must be absent");
    *format = w->scheme == QP_BLOCKWISE ? 5 : 1;
  } else if (w->dtype == QP_S4) {
    QP_REQUIRE(w->scheme == QP_BLOCKWISE || w->scheme == QP_BLOCKWISE_BF16 ||
                   w->scheme == QP_BLOCKWISE_ASYM,
               QP_EUNSUPPORTED, "int4 weights support blockwise scales only (scheme %d)",
               w->scheme);
    QP_REQUIRE(w->zero_points == nullptr && w->zero_point == 0, QP_EUNSUPPORTED,
               "int4 blockwise weights take no integer zero points (asymmetric weights give "
               "per-group offsets through QP_BLOCKWISE_ASYM)");
    *format = w->scheme == QP_BLOCKWISE_BF16 ? 3 : (w->scheme == QP_BLOCKWISE_ASYM ? 4 : 2);
  } else {
    QP_FAIL(QP_EUNSUPPORTED, "weights must be QP_S8 or QP_S4 (dtype %d)", w->dtype);
  }
  return QP_OK;
}

}  // namespace
}  // namespace qp

extern "C" qp_status qpack_weights_size(const qp_qtensor* w, int32_t k_axis, int32_t n_axis,
                                        size_t* bytes, size_t* align) {
  using namespace qp;
  WeightView v;
  qp_status st = weight_view(w, k_axis, n_axis, &v);
  if (st) return st;
  int32_t format = 0;
  if ((st = format_of(w, &format))) return st;
  qp_packed_info g;
  if ((st = blob_geometry(format, w->scheme, v.N, v.K, format != 1 ? w->group_size : 0, &g)))
    return st;
  if (bytes) *bytes = (size_t)g.total_bytes;
  if (align) *align = (size_t)kRegionAlign;
  return QP_OK;
}

extern "C" qp_status qpack_weights(const qp_qtensor* w, const void* w_dev, int32_t k_axis,
                                   int32_t n_axis, void* packed_dev, size_t packed_bytes,
                                   qp_packed_info* info, hipStream_t stream) {
  using namespace qp;
  clear_error();
  WeightView v;
  qp_status st = weight_view(w, k_axis, n_axis, &v);
  if (st) return st;
  int32_t format = 0;
  if ((st = format_of(w, &format))) return st;
  qp_packed_info g;
  if ((st = blob_geometry(format, w->scheme, v.N, v.K, format != 1 ? w->group_size : 0, &g)))
    return st;
  QP_REQUIRE(w_dev && packed_dev && info, QP_EINVAL, "qpack_weights: null pointer argument");
  QP_REQUIRE(packed_bytes >= (size_t)g.total_bytes, QP_ESIZE,
             "packed buffer holds %zu bytes, needs %lld", packed_bytes, (long long)g.total_bytes);
  QP_REQUIRE(((uintptr_t)packed_dev % kRegionAlign) == 0, QP_EALIGN,
             "packed buffer must be %lld-byte aligned", (long long)kRegionAlign);

  BlobHeader h;
  std::memset(&h, 0, sizeof(h));
  h.magic = kMagic;
  h.version = kVersion;
  h.format = (uint32_t)format;
  h.scheme = (uint32_t)w->scheme;
  h.N = g.N;
  h.K = g.K;
  h.Npad = g.Npad;
  h.Kpad = g.Kpad;
  h.group = g.group;
  h.data_off = g.data_off;
  h.data_bytes = g.data_bytes;
  h.scale_off = g.scale_off;
  h.sum_off = g.sum_off;
  h.zp_off = g.zp_off;
  h.total_bytes = g.total_bytes;

  uint8_t* blob = static_cast<uint8_t*>(packed_dev);
  const int8_t* src = static_cast<const int8_t*>(w_dev);
  if (format == 1) {
    // Validate the scales and zero points on the host (load time only).
    const bool per_channel = w->scheme == QP_PER_CHANNEL;
    std::vector<float> sc(per_channel ? (size_t)v.N : 1);
    std::vector<int32_t> zp(w->zero_points ? (size_t)v.N : 0);
    if (per_channel) {
      QP_REQUIRE(w->scales != nullptr, QP_EINVAL, "per-channel weights need a scales array");
      if (hipMemcpyAsync(sc.data(), w->scales, sizeof(float) * sc.size(), hipMemcpyDeviceToHost,
                         stream) != hipSuccess)
        QP_FAIL(QP_EHIP, "qpack_weights: reading scales failed");
    } else {
      sc[0] = w->scale;
    }
    if (w->zero_points) {
      if (hipMemcpyAsync(zp.data(), w->zero_points, sizeof(int32_t) * zp.size(),
                         hipMemcpyDeviceToHost, stream) != hipSuccess)
        QP_FAIL(QP_EHIP, "qpack_weights: reading zero points failed");
    }
    if (hipStreamSynchronize(stream) != hipSuccess)
      QP_FAIL(QP_EHIP, "qpack_weights: stream synchronize failed");
    float smin = INFINITY, smax = 0.0f;
    for (float s : sc) {
      QP_REQUIRE(std::isfinite(s) && s > 0.0f, QP_EINVAL, "weight scales must be finite and > 0");
      smin = std::fmin(smin, s);
      smax = std::fmax(smax, s);
    }
    int32_t has_zp = w->zero_point != 0;
    for (int32_t z : zp) {
      QP_REQUIRE(z >= -128 && z <= 127, QP_EINVAL, "weight zero point %d outside int8", z);
      has_zp |= z != 0;
    }
    QP_REQUIRE(w->zero_point >= -128 && w->zero_point <= 127, QP_EINVAL,
               "weight zero point %d outside int8", w->zero_point);
    h.has_zp = has_zp;
    h.scale_min = smin;
    h.scale_max = smax;
    hipLaunchKernelGGL(write_header_kernel, dim3(1), dim3(64), 0, stream, h, blob);
    if ((st = check_launch("qpack_weights header"))) return st;
    hipLaunchKernelGGL(pack_s8_kernel<false>, dim3((unsigned)g.Npad), dim3(256), 0, stream, src,
                       v.N, v.K, g.Kpad, v.sn, v.km, per_channel ? w->scales : nullptr, w->scale,
                       w->zero_points, w->zero_point, blob, g.data_off, g.scale_off, g.sum_off,
                       g.zp_off, (int64_t)0, (int64_t)0, (int64_t)1);
    if ((st = check_launch("qpack_weights int8"))) return st;
    g.has_zero_points = has_zp;
    g.scale_min = smin;
    g.scale_max = smax;
  } else if (format == 5) {
    QP_REQUIRE(w->scales != nullptr, QP_EINVAL, "blockwise weights need a scales array");
    hipLaunchKernelGGL(write_header_kernel, dim3(1), dim3(64), 0, stream, h, blob);
    if ((st = check_launch("qpack_weights header"))) return st;
    const size_t lds = sizeof(int32_t) * (size_t)(g.Kpad / g.group);
    QP_REQUIRE(lds <= 65536, QP_EUNSUPPORTED, "block-quantized int8 packing: too many blocks");
    // rank 2: scales [N][ceil(K/group)]; OIHW: [OC][IC/group], blocks of input
    // channels, the same scale for every kernel tap
    int64_t ldsw = ceil_div(v.K, g.group), period = ldsw;
    if (w->rank == 4) {
      const int64_t IC = w->shape[1];
      QP_REQUIRE(IC % g.group == 0, QP_EINVAL,
                 "channel-blocked conv weights: the block (%lld) must divide IC (%lld)",
                 (long long)g.group, (long long)IC);
      ldsw = period = IC / g.group;
    }
    hipLaunchKernelGGL(pack_s8_kernel<true>, dim3((unsigned)g.Npad), dim3(256), lds, stream, src,
                       v.N, v.K, g.Kpad, v.sn, v.km, w->scales, 0.0f, (const int32_t*)nullptr, 0,
                       blob, g.data_off, g.scale_off, g.sum_off, g.zp_off, g.group, ldsw, period);
    if ((st = check_launch("qpack_weights int8 blockwise"))) return st;
    g.has_zero_points = 0;
  } else {
    QP_REQUIRE(w->scales != nullptr, QP_EINVAL, "blockwise weights need a scales array");
    hipLaunchKernelGGL(write_header_kernel, dim3(1), dim3(64), 0, stream, h, blob);
    if ((st = check_launch("qpack_weights header"))) return st;
    size_t lds = sizeof(int32_t) * (size_t)(g.Kpad / 32);
    const int64_t groups = ceil_div(v.K, g.group);
    if (format == 3)
      hipLaunchKernelGGL(pack_s4_kernel<1>, dim3((unsigned)g.Npad), dim3(256), lds, stream, src,
                         v.N, v.K, g.Kpad, g.group, v.sn, v.km, w->scales, groups, blob,
                         g.data_off, g.scale_off, g.sum_off, g.zp_off);
    else if (format == 4)
      hipLaunchKernelGGL(pack_s4_kernel<2>, dim3((unsigned)g.Npad), dim3(256), lds, stream, src,
                         v.N, v.K, g.Kpad, g.group, v.sn, v.km, w->scales, 2 * groups, blob,
                         g.data_off, g.scale_off, g.sum_off, g.zp_off);
    else
      hipLaunchKernelGGL(pack_s4_kernel<0>, dim3((unsigned)g.Npad), dim3(256), lds, stream, src,
                         v.N, v.K, g.Kpad, g.group, v.sn, v.km, w->scales, groups, blob,
                         g.data_off, g.scale_off, g.sum_off, g.zp_off);
    if ((st = check_launch("qpack_weights int4"))) return st;
    g.has_zero_points = 0;
  }
  *info = g;
  return QP_OK;
}

extern "C" qp_status qrepack_weights(const qp_qtensor* w, const void* w_dev, int32_t k_axis,
                                     int32_t n_axis, void* packed_dev, qp_packed_info* info,
                                     hipStream_t stream) {
  using namespace qp;
  clear_error();
  QP_REQUIRE(w && info, QP_EINVAL, "qrepack_weights: null argument");
  WeightView v;
  qp_status st = weight_view(w, k_axis, n_axis, &v);
  if (st) return st;
  int32_t format = 0;
  if ((st = format_of(w, &format))) return st;
  qp_packed_info g;
  if ((st = blob_geometry(format, w->scheme, v.N, v.K, format != 1 ? w->group_size : 0, &g)))
    return st;
  QP_REQUIRE(g.format == info->format && g.scheme == info->scheme && g.N == info->N &&
                 g.K == info->K && g.group == info->group && g.Npad == info->Npad &&
                 g.Kpad == info->Kpad && g.data_off == info->data_off &&
                 g.scale_off == info->scale_off && g.sum_off == info->sum_off &&
                 g.zp_off == info->zp_off && g.total_bytes == info->total_bytes,
             QP_EINVAL,
             "qrepack_weights: the buffer holds format %d (scheme %d) N=%lld K=%lld group=%lld; "
             "these weights need format %d (scheme %d) N=%lld K=%lld group=%lld",
             info->format, info->scheme, (long long)info->N, (long long)info->K,
             (long long)info->group, g.format, g.scheme, (long long)g.N, (long long)g.K,
             (long long)g.group);
  qp_packed_info out;
  st = qpack_weights(w, w_dev, k_axis, n_axis, packed_dev, (size_t)info->total_bytes, &out,
                     stream);
  if (st) return st;
  *info = out;
  return QP_OK;
}
