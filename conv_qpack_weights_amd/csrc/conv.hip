// conv.hip -- INT8 NHWC convolution as explicit im2col + the INT8 GEMM.
//
// MNN "ConvInt8TiledExecutor.cpp" (DenseConvInt8TiledExecutor: static int8
// convolution = im2col of the int8 input, padded with the input zero point,
// then the int8 GEMM with the requantizing post-treatment).  The weights are
// an int8 blob packed from OIHW with K ordered (kh, kw, ic).
#include <cmath>

#include "qp_internal.hpp"

namespace qp {
namespace {

struct ConvPlan {
  int64_t OH, OW, M, ldcol, ws_col, ws_gemm;
};

qp_status plan_conv(const qp_qtensor* x, const qp_packed_info* w, int32_t KH, int32_t KW,
                    int32_t sh, int32_t sw, int32_t pt, int32_t pl, int32_t pb, int32_t pr,
                    ConvPlan* p) {
  QP_REQUIRE(x && w, QP_EINVAL, "qconv2d: null descriptor");
  QP_REQUIRE(x->dtype == QP_S8 && x->rank == 4, QP_EINVAL, "qconv2d: x must be rank-4 NHWC QP_S8");
  QP_REQUIRE(w->format == 1, QP_EINVAL, "qconv2d: weights must be an int8 blob");
  const int64_t NB = x->shape[0], H = x->shape[1], W = x->shape[2], C = x->shape[3];
  QP_REQUIRE(NB > 0 && H > 0 && W > 0 && C > 0, QP_EINVAL, "qconv2d: empty input");
  QP_REQUIRE(x->stride[3] == 1 && x->stride[2] == C && x->stride[1] == W * C &&
                 x->stride[0] == H * W * C,
             QP_EUNSUPPORTED, "qconv2d: x must be contiguous NHWC");
  QP_REQUIRE(w->K == (int64_t)KH * KW * C, QP_EINVAL,
             "qconv2d: weights have K=%lld, kernel needs KH*KW*C=%lld", (long long)w->K,
             (long long)KH * KW * C);
  qp_status st = conv_out_dims(H, W, KH, KW, sh, sw, pt, pl, pb, pr, 1, 1, &p->OH, &p->OW);
  if (st) return st;
  p->M = NB * p->OH * p->OW;
  p->ldcol = w->Kpad;
  p->ws_col = round_up(p->M * p->ldcol, 256);
  p->ws_gemm = w->has_zero_points ? round_up(4 * p->M, 256) : 0;
  return QP_OK;
}

}  // namespace
}  // namespace qp

extern "C" qp_status qconv2d_s8_im2col_ws_size(const qp_qtensor* x, const qp_packed_info* w,
                                               int32_t KH, int32_t KW, int32_t stride_h,
                                               int32_t stride_w, int32_t pad_t, int32_t pad_l,
                                               int32_t pad_b, int32_t pad_r, size_t* bytes) {
  using namespace qp;
  QP_REQUIRE(bytes, QP_EINVAL, "qconv2d_s8_im2col_ws_size: null output");
  ConvPlan p;
  qp_status st = plan_conv(x, w, KH, KW, stride_h, stride_w, pad_t, pad_l, pad_b, pad_r, &p);
  if (st) return st;
  *bytes = (size_t)(p.ws_col + p.ws_gemm);
  return QP_OK;
}

extern "C" qp_status qconv2d_s8_im2col(const qp_qtensor* x, const int8_t* X,
                                       const qp_packed_info* w, const void* packedW_dev,
                                       int32_t KH, int32_t KW, int32_t stride_h, int32_t stride_w,
                                       int32_t pad_t, int32_t pad_l, int32_t pad_b, int32_t pad_r,
                                       const int32_t* bias_dev, int64_t max_abs_bias,
                                       const qp_qtensor* y, int32_t relu, void* Y, void* ws,
                                       size_t ws_bytes, hipStream_t stream) {
  using namespace qp;
  clear_error();
  ConvPlan p;
  qp_status st = plan_conv(x, w, KH, KW, stride_h, stride_w, pad_t, pad_l, pad_b, pad_r, &p);
  if (st) return st;
  QP_REQUIRE(x->scheme == QP_PER_TENSOR, QP_EUNSUPPORTED, "qconv2d: x must be per-tensor");
  QP_REQUIRE(x->rounding == QP_ROUND_HALF_EVEN, QP_EUNSUPPORTED,
             "qconv2d: only round-half-to-even is implemented");
  bool out32 = false;
  st = validate_gemm(w, w->K, x->scale, x->zero_point, bias_dev, max_abs_bias, y, &out32);
  if (st) return st;
  QP_REQUIRE(y->rank == 4 && y->shape[0] == x->shape[0] && y->shape[1] == p.OH &&
                 y->shape[2] == p.OW && y->shape[3] == w->N,
             QP_EINVAL, "qconv2d: y must be [N, OH, OW, OC] = [%lld, %lld, %lld, %lld]",
             (long long)x->shape[0], (long long)p.OH, (long long)p.OW, (long long)w->N);
  QP_REQUIRE(y->stride[3] == 1 && y->stride[2] == w->N && y->stride[1] == p.OW * w->N &&
                 y->stride[0] == p.OH * p.OW * w->N,
             QP_EUNSUPPORTED, "qconv2d: y must be contiguous NHWC");
  QP_REQUIRE(X && packedW_dev && Y && ws, QP_EINVAL, "qconv2d: null data pointer");
  QP_REQUIRE(ws_bytes >= (size_t)(p.ws_col + p.ws_gemm), QP_ESIZE,
             "qconv2d: workspace holds %zu bytes, needs %lld", ws_bytes,
             (long long)(p.ws_col + p.ws_gemm));
  QP_REQUIRE(((uintptr_t)ws % 256) == 0, QP_EALIGN, "qconv2d: workspace must be 256-byte aligned");
  int8_t* col = static_cast<int8_t*>(ws);
  st = launch_im2col(X, x->shape[0], x->shape[1], x->shape[2], x->shape[3], x->zero_point, KH, KW,
                     stride_h, stride_w, pad_t, pad_l, 1, 1, p.OH, p.OW, col, p.ldcol, stream);
  if (st) return st;
  void* gws = static_cast<uint8_t*>(ws) + p.ws_col;
  return run_gemm_s8(col, p.M, p.ldcol, x->scale, x->zero_point, w, packedW_dev, bias_dev, y->scale,
                     y->zero_point, out32, relu, Y, w->N, gws, ws_bytes - (size_t)p.ws_col, true,
                     stream);
}

// ---- qconv2d_s8: the general entry (dilation, implicit GEMM, 1x1 fastway) ----
//
// MNN DenseConvInt8TiledExecutor::onResize picks a "fastway" for a 1x1
// kernel with stride 1 and output the size of the input: the input is then
// the GEMM's activation matrix as it stands.  Otherwise the convolution is
// the im2col GEMM; here it runs as an implicit GEMM when every 16-byte
// operand piece is 16 input channels of one tap (C % 16 == 0), else through
// the explicit im2col.
namespace qp {
namespace {

enum ConvRoute { kRouteFast1x1, kRouteImplicit, kRouteExplicit };

struct ConvPlan2 {
  ConvRoute route;
  ConvShape cs;
  int64_t M, ldcol, ws_col, ws_total;
};

qp_status plan_conv2(const qp_qtensor* x, const qp_packed_info* w, int32_t KH, int32_t KW,
                     int32_t sh, int32_t sw, int32_t pt, int32_t pl, int32_t pb, int32_t pr,
                     int32_t dh, int32_t dw, ConvPlan2* p) {
  QP_REQUIRE(x && w, QP_EINVAL, "qconv2d: null descriptor");
  QP_REQUIRE(x->dtype == QP_S8 && x->rank == 4, QP_EINVAL, "qconv2d: x must be rank-4 NHWC QP_S8");
  QP_REQUIRE(w->format == 1, QP_EINVAL, "qconv2d: weights must be an int8 blob");
  const int64_t NB = x->shape[0], H = x->shape[1], W = x->shape[2], C = x->shape[3];
  QP_REQUIRE(NB > 0 && H > 0 && W > 0 && C > 0, QP_EINVAL, "qconv2d: empty input");
  QP_REQUIRE(x->stride[3] == 1 && x->stride[2] == C && x->stride[1] == W * C &&
                 x->stride[0] == H * W * C,
             QP_EUNSUPPORTED, "qconv2d: x must be contiguous NHWC");
  QP_REQUIRE(w->K == (int64_t)KH * KW * C, QP_EINVAL,
             "qconv2d: weights have K=%lld, kernel needs KH*KW*C=%lld", (long long)w->K,
             (long long)KH * KW * C);
  int64_t OH = 0, OW = 0;
  qp_status st = conv_out_dims(H, W, KH, KW, sh, sw, pt, pl, pb, pr, dh, dw, &OH, &OW);
  if (st) return st;
  p->cs = ConvShape{NB, H, W, C, OH, OW, KH, KW, sh, sw, pt, pl, dh, dw};
  p->M = NB * OH * OW;
  p->ldcol = w->Kpad;
  p->ws_col = 0;
  const int64_t ws_rowsum = w->has_zero_points ? round_up(4 * p->M, 256) : 0;
  const bool fast = KH == 1 && KW == 1 && sh == 1 && sw == 1 && pt == 0 && pl == 0 && pb == 0 &&
                    pr == 0;
  if (fast) {
    // the GEMM on X as [NB*H*W, C]; sized for its copying plan
    p->route = kRouteFast1x1;
    p->ws_total = round_up(p->M * w->Kpad, 256) + ws_rowsum;
  } else if (C % 16 == 0 && NB * H * W * C < (INT64_C(1) << 31)) {
    p->route = kRouteImplicit;
    p->ws_total = 0;
  } else {
    p->route = kRouteExplicit;
    p->ws_col = round_up(p->M * p->ldcol, 256);
    p->ws_total = p->ws_col + ws_rowsum;
  }
  return QP_OK;
}

}  // namespace
}  // namespace qp

extern "C" qp_status qconv2d_s8_ws_size(const qp_qtensor* x, const qp_packed_info* w, int32_t KH,
                                        int32_t KW, int32_t stride_h, int32_t stride_w,
                                        int32_t pad_t, int32_t pad_l, int32_t pad_b,
                                        int32_t pad_r, int32_t dil_h, int32_t dil_w,
                                        size_t* bytes) {
  using namespace qp;
  QP_REQUIRE(bytes, QP_EINVAL, "qconv2d_s8_ws_size: null output");
  ConvPlan2 p;
  qp_status st = plan_conv2(x, w, KH, KW, stride_h, stride_w, pad_t, pad_l, pad_b, pad_r, dil_h,
                            dil_w, &p);
  if (st) return st;
  *bytes = (size_t)p.ws_total;
  return QP_OK;
}

extern "C" qp_status qconv2d_s8(const qp_qtensor* x, const int8_t* X, const qp_packed_info* w,
                                const void* packedW_dev, int32_t KH, int32_t KW,
                                int32_t stride_h, int32_t stride_w, int32_t pad_t,
                                int32_t pad_l, int32_t pad_b, int32_t pad_r, int32_t dil_h,
                                int32_t dil_w, const int32_t* bias_dev, int64_t max_abs_bias,
                                const qp_qtensor* y, int32_t relu, void* Y, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  using namespace qp;
  clear_error();
  ConvPlan2 p;
  qp_status st = plan_conv2(x, w, KH, KW, stride_h, stride_w, pad_t, pad_l, pad_b, pad_r, dil_h,
                            dil_w, &p);
  if (st) return st;
  QP_REQUIRE(x->scheme == QP_PER_TENSOR, QP_EUNSUPPORTED, "qconv2d: x must be per-tensor");
  QP_REQUIRE(x->rounding == QP_ROUND_HALF_EVEN, QP_EUNSUPPORTED,
             "qconv2d: only round-half-to-even is implemented");
  bool out32 = false;
  st = validate_gemm(w, w->K, x->scale, x->zero_point, bias_dev, max_abs_bias, y, &out32);
  if (st) return st;
  QP_REQUIRE(y->rank == 4 && y->shape[0] == x->shape[0] && y->shape[1] == p.cs.OH &&
                 y->shape[2] == p.cs.OW && y->shape[3] == w->N,
             QP_EINVAL, "qconv2d: y must be [N, OH, OW, OC] = [%lld, %lld, %lld, %lld]",
             (long long)x->shape[0], (long long)p.cs.OH, (long long)p.cs.OW, (long long)w->N);
  QP_REQUIRE(y->stride[3] == 1 && y->stride[2] == w->N && y->stride[1] == p.cs.OW * w->N &&
                 y->stride[0] == p.cs.OH * p.cs.OW * w->N,
             QP_EUNSUPPORTED, "qconv2d: y must be contiguous NHWC");
  QP_REQUIRE(X && packedW_dev && Y, QP_EINVAL, "qconv2d: null data pointer");
  QP_REQUIRE(ws_bytes >= (size_t)p.ws_total, QP_ESIZE,
             "qconv2d: workspace holds %zu bytes, needs %lld", ws_bytes, (long long)p.ws_total);
  QP_REQUIRE(p.ws_total == 0 || (ws && ((uintptr_t)ws % 256) == 0), QP_EALIGN,
             "qconv2d: workspace must be non-null and 256-byte aligned");
  switch (p.route) {
    case kRouteFast1x1:
      return run_gemm_s8(X, p.M, x->shape[3], x->scale, x->zero_point, w, packedW_dev, bias_dev,
                         y->scale, y->zero_point, out32, relu, Y, w->N, ws, ws_bytes, false,
                         stream);
    case kRouteImplicit:
      QP_REQUIRE(((uintptr_t)X % 16) == 0, QP_EALIGN,
                 "qconv2d: x must be 16-byte aligned when C %% 16 == 0");
      return launch_conv_implicit(X, p.cs, x->scale, x->zero_point, w, packedW_dev, bias_dev,
                                  y->scale, y->zero_point, out32, relu, Y, stream);
    case kRouteExplicit:
    default: {
      int8_t* col = static_cast<int8_t*>(ws);
      st = launch_im2col(X, x->shape[0], x->shape[1], x->shape[2], x->shape[3], x->zero_point, KH,
                         KW, stride_h, stride_w, pad_t, pad_l, dil_h, dil_w, p.cs.OH, p.cs.OW, col,
                         p.ldcol, stream);
      if (st) return st;
      void* gws = static_cast<uint8_t*>(ws) + p.ws_col;
      return run_gemm_s8(col, p.M, p.ldcol, x->scale, x->zero_point, w, packedW_dev, bias_dev,
                         y->scale, y->zero_point, out32, relu, Y, w->N, gws,
                         ws_bytes - (size_t)p.ws_col, true, stream);
    }
  }
}

// ---- qconv2d_s8_blockwise_f32: channel-blocked int8 weights, f32 output ----
//
// MNN's dynamic-quant convolution with blockNum > 1: the weights carry one
// scale per output channel and block of input channels, the exact block sums
// are combined in float and the output is float.  The input here is int8
// with a per-tensor scale and zero point; the route is the implicit GEMM.
extern "C" qp_status qconv2d_s8_blockwise_f32(const qp_qtensor* x, const int8_t* X,
                                              const qp_packed_info* w, const void* packedW_dev,
                                              int32_t KH, int32_t KW, int32_t stride_h,
                                              int32_t stride_w, int32_t pad_t, int32_t pad_l,
                                              int32_t pad_b, int32_t pad_r, int32_t dil_h,
                                              int32_t dil_w, const float* bias_dev,
                                              float clamp_lo, float clamp_hi, float* Y,
                                              hipStream_t stream) {
  using namespace qp;
  clear_error();
  QP_REQUIRE(x && w, QP_EINVAL, "qconv2d_blockwise: null descriptor");
  QP_REQUIRE(w->format == 5, QP_EINVAL,
             "qconv2d_blockwise: weights must be a block-quantized int8 blob");
  QP_REQUIRE(x->dtype == QP_S8 && x->rank == 4, QP_EINVAL,
             "qconv2d_blockwise: x must be rank-4 NHWC QP_S8");
  const int64_t NB = x->shape[0], H = x->shape[1], W = x->shape[2], C = x->shape[3];
  QP_REQUIRE(NB > 0 && H > 0 && W > 0 && C > 0, QP_EINVAL, "qconv2d_blockwise: empty input");
  QP_REQUIRE(x->stride[3] == 1 && x->stride[2] == C && x->stride[1] == W * C &&
                 x->stride[0] == H * W * C,
             QP_EUNSUPPORTED, "qconv2d_blockwise: x must be contiguous NHWC");
  QP_REQUIRE(w->K == (int64_t)KH * KW * C, QP_EINVAL,
             "qconv2d_blockwise: weights have K=%lld, kernel needs KH*KW*C=%lld", (long long)w->K,
             (long long)KH * KW * C);
  QP_REQUIRE(C % 16 == 0 && C % w->group == 0, QP_EUNSUPPORTED,
             "qconv2d_blockwise: C must be a multiple of 16 and of the channel block (%lld)",
             (long long)w->group);
  QP_REQUIRE(x->scheme == QP_PER_TENSOR && x->rounding == QP_ROUND_HALF_EVEN, QP_EUNSUPPORTED,
             "qconv2d_blockwise: x must be per-tensor, round-half-to-even");
  QP_REQUIRE(x->zero_point >= -128 && x->zero_point <= 127, QP_EINVAL,
             "qconv2d_blockwise: input zero point outside int8");
  QP_REQUIRE(std::isfinite(x->scale) && x->scale > 0, QP_EINVAL,
             "qconv2d_blockwise: input scale must be > 0");
  QP_REQUIRE(!(clamp_lo > clamp_hi) && !std::isnan(clamp_lo) && !std::isnan(clamp_hi), QP_EINVAL,
             "qconv2d_blockwise: clamp bounds must satisfy lo <= hi");
  QP_REQUIRE(NB * H * W * C < (INT64_C(1) << 31), QP_EUNSUPPORTED,
             "qconv2d_blockwise: input of 2^31 bytes or more");
  int64_t OH = 0, OW = 0;
  qp_status st = conv_out_dims(H, W, KH, KW, stride_h, stride_w, pad_t, pad_l, pad_b, pad_r,
                               dil_h, dil_w, &OH, &OW);
  if (st) return st;
  QP_REQUIRE(X && packedW_dev && Y, QP_EINVAL, "qconv2d_blockwise: null data pointer");
  QP_REQUIRE(((uintptr_t)X % 16) == 0, QP_EALIGN, "qconv2d_blockwise: x must be 16-byte aligned");
  const ConvShape cs{NB, H, W, C, OH, OW, KH, KW, stride_h, stride_w, pad_t, pad_l, dil_h, dil_w};
  return launch_conv_implicit_blk(X, cs, x->scale, x->zero_point, w, packedW_dev, bias_dev,
                                  clamp_lo, clamp_hi, Y, stream);
}
