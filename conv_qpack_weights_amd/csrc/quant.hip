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

}  // namespace

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
