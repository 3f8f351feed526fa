// quant.hip -- dynamic per-row asymmetric int8 quantization of f32 rows.
//
// MNN "ConvInt8TiledExecutor.cpp" (BatchAsyDynamicQuant) and pytorch/ao
// PR #997 (the KleidiAI "qai8dx" activations) quantize each row with its own
// scale and zero point, saturating to [-128,127]; the helpers' arithmetic is
// not printed on those pages.  The numeric contract taken is ONNX
// DynamicQuantizeLinear moved to int8, as one fixed f32 op sequence so that a
// CPU and this kernel agree bit for bit:
//   rmin = min(0, min x); rmax = max(0, max x); scale = (rmax - rmin) / 255
//   (scale == 0 -> scale = 1, zp = 0); zp = clamp(rint(-128 - rmin/scale));
//   q = clamp(rint(x/scale) + zp, -128, 127).
// Division is IEEE (correctly rounded), rint is round-half-even, and no
// multiply-add is contracted.
#include "qp_internal.hpp"
#include "quant_row.hpp"

#pragma clang fp contract(off)

namespace qp {
namespace {

// One workgroup per row.  kPerm writes the A8W4 operand order; kSym is the
// symmetric variant.
template <bool kPerm, bool kSym = false>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const float* __restrict__ x,
                                                            int64_t K, int64_t ldx,
                                                            int8_t* __restrict__ q, int64_t ldq,
                                                            int64_t kfill,
                                                            float* __restrict__ row_scale,
                                                            int32_t* __restrict__ row_zp) {
  __shared__ float red[2 * 4];
  const int64_t m = blockIdx.x;
  const float* xr = x + m * ldx;
  int8_t* qr = q + m * ldq;
  const bool vec = (((uintptr_t)xr) & 15) == 0;
  const bool dvec = (((uintptr_t)qr) & 15) == 0;
  float s;
  int32_t z;
  quantize_row_wg<256, kPerm, 16, kSym>(xr, K, kfill, vec, dvec, qr, red, &s, &z);
  if (threadIdx.x == 0) {
    row_scale[m] = s;
    if (row_zp) row_zp[m] = z;
  }
}

// Per-block variant (blocks of 32 K): each half wave owns one block of one
// row -- lane j holds element 32g + j -- and reduces the block's extremes
// with butterfly shuffles inside its 32 lanes (min and max are exact, so
// the order does not matter), then every lane applies the same f32 steps.
// Blocks are numbered row-major over [M][nb], nb = kpad / 32; elements past
// K read as 0 (the range includes 0 anyway) and are written as 0.
__global__ __launch_bounds__(256) void quantize_blocks32_kernel(
    const float* __restrict__ x, int64_t M, int64_t K, int64_t ldx, int8_t* __restrict__ q,
    int64_t ldq, int64_t nb, float* __restrict__ scale, int32_t* __restrict__ zp, int64_t ldsz) {
  const int64_t blk = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 5;
  if (blk >= M * nb) return;  // whole half waves leave together
  const int j = threadIdx.x & 31;
  const int64_t m = blk / nb, g = blk - m * nb;
  const int64_t k = g * 32 + j;
  const float v = k < K ? x[m * ldx + k] : 0.0f;
  float lo = v, hi = v;
#pragma unroll
  for (int off = 16; off > 0; off >>= 1) {
    lo = qp_min(lo, __shfl_xor(lo, off, 32));
    hi = qp_max(hi, __shfl_xor(hi, off, 32));
  }
  lo = qp_min(lo, 0.0f);
  hi = qp_max(hi, 0.0f);
  float s;
  int32_t z;
  params_from_range(lo, hi, &s, &z);
  q[m * ldq + k] = k < K ? (int8_t)quantize_one(v, s, z) : (int8_t)0;
  if (j == 0) {
    scale[m * ldsz + g] = s;
    zp[m * ldsz + g] = z;
  }
}

}  // namespace

qp_status launch_quantize_blocks32(const float* x, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                                   int64_t ldq, int64_t kpad, float* scale, int32_t* zp,
                                   int64_t ldsz, hipStream_t stream) {
  const int64_t nb = kpad / 32;
  const int64_t threads = M * nb * 32;
  if (threads == 0) return QP_OK;
  hipLaunchKernelGGL(quantize_blocks32_kernel, dim3((unsigned)ceil_div(threads, 256)), dim3(256),
                     0, stream, x, M, K, ldx, q, ldq, nb, scale, zp, ldsz);
  return check_launch("qquantize_rows_s8_blocked");
}

qp_status launch_quantize_rows(const float* x, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                               int64_t ldq, int64_t kfill, float* row_scale, int32_t* row_zp,
                               bool perm, hipStream_t stream) {
  if (M == 0) return QP_OK;
  if (perm)
    hipLaunchKernelGGL(quantize_rows_kernel<true>, dim3((unsigned)M), dim3(256), 0, stream, x, K,
                       ldx, q, ldq, kfill, row_scale, row_zp);
  else
    hipLaunchKernelGGL(quantize_rows_kernel<false>, dim3((unsigned)M), dim3(256), 0, stream, x, K,
                       ldx, q, ldq, kfill, row_scale, row_zp);
  return check_launch("qquantize_rows_s8");
}

}  // namespace qp

extern "C" qp_status qquantize_rows_s8(const float* x, int64_t M, int64_t K, int64_t ldx,
                                       int8_t* q, int64_t ldq, float* row_scale, int32_t* row_zp,
                                       hipStream_t stream) {
  using namespace qp;
  clear_error();
  QP_REQUIRE(M >= 0 && K >= 0, QP_EINVAL, "qquantize_rows_s8: negative extent");
  QP_REQUIRE(M <= 0x7fffffff, QP_EUNSUPPORTED, "qquantize_rows_s8: M too large");
  QP_REQUIRE(ldx >= K && ldq >= K, QP_EINVAL, "qquantize_rows_s8: ldx/ldq smaller than K");
  if (M == 0) return QP_OK;
  QP_REQUIRE(x && q && row_scale && row_zp, QP_EINVAL, "qquantize_rows_s8: null pointer");
  return launch_quantize_rows(x, M, K, ldx, q, ldq, K, row_scale, row_zp, false, stream);
}

extern "C" qp_status qquantize_rows_s8_sym(const float* x, int64_t M, int64_t K, int64_t ldx,
                                           int8_t* q, int64_t ldq, float* row_scale,
                                           hipStream_t stream) {
  using namespace qp;
  clear_error();
  QP_REQUIRE(M >= 0 && K >= 0, QP_EINVAL, "qquantize_rows_s8_sym: negative extent");
  QP_REQUIRE(M <= 0x7fffffff, QP_EUNSUPPORTED, "qquantize_rows_s8_sym: M too large");
  QP_REQUIRE(ldx >= K && ldq >= K, QP_EINVAL, "qquantize_rows_s8_sym: ldx/ldq smaller than K");
  if (M == 0) return QP_OK;
  QP_REQUIRE(x && q && row_scale, QP_EINVAL, "qquantize_rows_s8_sym: null pointer");
  hipLaunchKernelGGL((quantize_rows_kernel<false, true>), dim3((unsigned)M), dim3(256), 0, stream,
                     x, K, ldx, q, ldq, K, row_scale, (int32_t*)nullptr);
  return check_launch("qquantize_rows_s8_sym");
}

extern "C" qp_status qquantize_rows_s8_blocked(const float* x, int64_t M, int64_t K, int64_t ldx,
                                               int64_t block, int64_t kpad, int8_t* q,
                                               int64_t ldq, float* scale, int32_t* zp,
                                               int64_t ldsz, hipStream_t stream) {
  using namespace qp;
  clear_error();
  QP_REQUIRE(block == 32, QP_EUNSUPPORTED, "qquantize_rows_s8_blocked: block must be 32");
  QP_REQUIRE(M >= 0 && K >= 0, QP_EINVAL, "qquantize_rows_s8_blocked: negative extent");
  QP_REQUIRE(kpad >= K && kpad % 32 == 0, QP_EINVAL,
             "qquantize_rows_s8_blocked: kpad must be >= K and a multiple of 32");
  QP_REQUIRE(ldx >= K && ldq >= kpad && ldsz >= kpad / 32, QP_EINVAL,
             "qquantize_rows_s8_blocked: ldx < K, ldq < kpad or ldsz < kpad/32");
  QP_REQUIRE(M * (kpad / 32) * 32 < (INT64_C(1) << 31) * 256, QP_EUNSUPPORTED,
             "qquantize_rows_s8_blocked: too many blocks");
  if (M == 0 || kpad == 0) return QP_OK;
  QP_REQUIRE(x && q && scale && zp, QP_EINVAL, "qquantize_rows_s8_blocked: null pointer");
  return launch_quantize_blocks32(x, M, K, ldx, q, ldq, kpad, scale, zp, ldsz, stream);
}
