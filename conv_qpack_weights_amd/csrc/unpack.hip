// unpack.hip -- read logical weights back out of a packed blob (debugging,
// inspection, checking a restored blob).
//
// tract-linalg "frame/pack.rs" (PackedFormat::extract_at_mn_f16 /
// extract_at_mn_f32): given a packed operand and an index along M/N, copy
// that row's K values out of the panel layout, optionally as floats.  Here
// a range of output channels [n0, n0 + count) comes out as logical int8
// values ([-8, 7] for int4 blobs), their scales (and zero points for int8),
// and optionally the dequantized f32 weights: sB[n]*(q - zB[n]) for int8,
// sw[n, k/group]*q for int4 (plus the group offset for asymmetric int4).
// Only real K is written; padding is never exposed.
#include "qp_internal.hpp"

#pragma clang fp contract(off)

namespace qp {
namespace {

// Scale element e of an int4 blob: f32 (format 2) or bf16 (format 3, the
// upper half of the f32 of the same value).
__device__ __forceinline__ float scale_at(const uint8_t* blob, const qp_packed_info& b, int64_t e) {
  if (b.format == 3) {
    const uint32_t h = reinterpret_cast<const uint16_t*>(blob + b.scale_off)[e];
    return __builtin_bit_cast(float, h << 16);
  }
  return reinterpret_cast<const float*>(blob + b.scale_off)[e];
}

// One thread per (channel, k) of the requested range.
__global__ __launch_bounds__(256) void unpack_s8_kernel(const uint8_t* __restrict__ blob,
                                                        qp_packed_info b, int64_t n0,
                                                        int64_t count, int8_t* __restrict__ w,
                                                        int64_t ldw, float* __restrict__ deq,
                                                        int64_t ldd) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= count * b.K) return;
  const int64_t i = id / b.K, k = id - i * b.K;
  const int64_t n = n0 + i;
  const int64_t kblocks = b.Kpad / 32;
  const int8_t q = static_cast<const int8_t*>(static_cast<const void*>(
      blob + b.data_off))[((n / 32) * kblocks + k / 32) * 1024 + (n % 32) * 32 + k % 32];
  if (w) w[i * ldw + k] = q;
  if (deq) {
    if (b.format == 5) {  // a scale per block of `group` K, no zero point
      const float s = reinterpret_cast<const float*>(blob + b.scale_off)[(k / b.group) * b.Npad + n];
      deq[i * ldd + k] = s * (float)q;
    } else {
      const float s = reinterpret_cast<const float*>(blob + b.scale_off)[n];
      const int32_t z = reinterpret_cast<const int32_t*>(blob + b.zp_off)[n];
      deq[i * ldd + k] = s * (float)((int32_t)q - z);
    }
  }
}

__global__ __launch_bounds__(256) void unpack_s4_kernel(const uint8_t* __restrict__ blob,
                                                        qp_packed_info b, int64_t n0,
                                                        int64_t count, int8_t* __restrict__ w,
                                                        int64_t ldw, float* __restrict__ deq,
                                                        int64_t ldd) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= count * b.K) return;
  const int64_t i = id / b.K, k = id - i * b.K;
  const int64_t n = n0 + i;
  const int64_t nblk = b.Kpad / 128;
  // inside a 128-K block: k' = 32t + 8c + 4h + j sits in byte 16c + 4t + j,
  // low nibble for h = 0, high for h = 1
  const int64_t kb = k % 128;
  const int t = (int)(kb / 32), c = (int)((kb % 32) / 8), h = (int)((kb % 8) / 4), j = (int)(kb % 4);
  const uint8_t byte =
      blob[b.data_off + ((n / 16) * nblk + k / 128) * 1024 + (n % 16) * 64 + 16 * c + 4 * t + j];
  const int32_t nib = h ? (byte >> 4) : (byte & 0xF);
  const int8_t q = (int8_t)(nib >= 8 ? nib - 16 : nib);
  if (w) w[i * ldw + k] = q;
  if (deq) {
    const int64_t g = k / b.group;
    const int64_t Gq = (b.Kpad / b.group + 3) / 4;
    const int64_t e = ((n / 16) * Gq + g / 4) * 64 + (n % 16) * 4 + g % 4;
    const float s = scale_at(blob, b, e);
    if (b.format == 4)  // asymmetric: scale*q + offset
      deq[i * ldd + k] = s * (float)q + reinterpret_cast<const float*>(blob + b.zp_off)[e];
    else
      deq[i * ldd + k] = s * (float)q;
  }
}

// Scales (and zero points) of the range: int8 one per channel, int4 one per
// real group.
__global__ __launch_bounds__(256) void unpack_scales_kernel(const uint8_t* __restrict__ blob,
                                                            qp_packed_info b, int64_t n0,
                                                            int64_t count, int64_t groups,
                                                            float* __restrict__ scales,
                                                            int64_t lds,
                                                            int32_t* __restrict__ zp) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= count * groups) return;
  const int64_t i = id / groups, g = id - i * groups;
  const int64_t n = n0 + i;
  if (b.format == 1) {
    if (scales) scales[i] = reinterpret_cast<const float*>(blob + b.scale_off)[n];
    if (zp) zp[i] = reinterpret_cast<const int32_t*>(blob + b.zp_off)[n];
  } else if (b.format == 5) {
    if (scales)
      scales[i * lds + g] = reinterpret_cast<const float*>(blob + b.scale_off)[g * b.Npad + n];
  } else if (scales) {
    const int64_t Gq = (b.Kpad / b.group + 3) / 4;
    const int64_t e = ((n / 16) * Gq + g / 4) * 64 + (n % 16) * 4 + g % 4;
    if (b.format == 4) {  // (offset, scale) pairs, as given to the packer
      scales[i * lds + 2 * g] = reinterpret_cast<const float*>(blob + b.zp_off)[e];
      scales[i * lds + 2 * g + 1] = scale_at(blob, b, e);
    } else {
      scales[i * lds + g] = scale_at(blob, b, e);
    }
  }
}

}  // namespace
}  // namespace qp

extern "C" qp_status qunpack_weights(const qp_packed_info* info, const void* packed_dev,
                                     int64_t n_begin, int64_t n_count, int8_t* w_out,
                                     int64_t ldw, float* scales_out, int64_t lds,
                                     int32_t* zp_out, float* deq_out, int64_t ldd,
                                     hipStream_t stream) {
  using namespace qp;
  clear_error();
  QP_REQUIRE(info && packed_dev, QP_EINVAL, "qunpack_weights: null blob");
  QP_REQUIRE(info->format >= 1 && info->format <= 5, QP_EINVAL,
             "qunpack_weights: unknown blob format %d", info->format);
  QP_REQUIRE(n_begin >= 0 && n_count >= 0 && n_begin + n_count <= info->N, QP_EINVAL,
             "qunpack_weights: channels [%lld, %lld) outside [0, %lld)", (long long)n_begin,
             (long long)(n_begin + n_count), (long long)info->N);
  QP_REQUIRE(!w_out || ldw >= info->K, QP_EINVAL, "qunpack_weights: ldw smaller than K");
  QP_REQUIRE(!deq_out || ldd >= info->K, QP_EINVAL, "qunpack_weights: ldd smaller than K");
  QP_REQUIRE(info->format == 1 || !zp_out, QP_EINVAL,
             "qunpack_weights: only per-tensor/per-channel int8 blobs have zero points "
             "(zp_out must be NULL)");
  const int64_t groups = info->format == 1 ? 1 : ceil_div(info->K, info->group);
  const int64_t per_row = info->format == 4 ? 2 * groups : groups;
  QP_REQUIRE(!scales_out || info->format == 1 || lds >= per_row, QP_EINVAL,
             "qunpack_weights: lds smaller than %lld", (long long)per_row);
  if (n_count == 0) return QP_OK;
  const uint8_t* blob = static_cast<const uint8_t*>(packed_dev);
  const qp_packed_info b = *info;
  if (w_out || deq_out) {
    const int64_t total = n_count * info->K;
    const unsigned blocks = (unsigned)ceil_div(total, 256);
    if (info->format == 1 || info->format == 5)
      hipLaunchKernelGGL(unpack_s8_kernel, dim3(blocks), dim3(256), 0, stream, blob, b, n_begin,
                         n_count, w_out, ldw, deq_out, ldd);
    else
      hipLaunchKernelGGL(unpack_s4_kernel, dim3(blocks), dim3(256), 0, stream, blob, b, n_begin,
                         n_count, w_out, ldw, deq_out, ldd);
    qp_status st = check_launch("qunpack_weights");
    if (st) return st;
  }
  if (scales_out || zp_out) {
    const unsigned blocks = (unsigned)ceil_div(n_count * groups, 256);
    hipLaunchKernelGGL(unpack_scales_kernel, dim3(blocks), dim3(256), 0, stream, blob, b, n_begin,
                       n_count, groups, scales_out, lds, zp_out);
    return check_launch("qunpack_weights scales");
  }
  return QP_OK;
}
