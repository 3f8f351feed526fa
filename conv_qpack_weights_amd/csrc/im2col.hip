// im2col.hip -- explicit int8 im2col of an NHWC tensor.
//
// MNN "ConvInt8TiledExecutor.cpp" (tileSplitFunction): the int8 im2col buffer
// is pre-filled with the INPUT zero point, so out-of-image taps stand for
// real zero, and then the in-image pixels are copied; the K order is tap
// outer, input channel inner (reorderWeight).  tract-linalg "frame/pack.rs"
// (PackedI8K4::write_with_k_outer) has the im2col patchers write straight
// into the matmul's operand layout.  Here the gather writes the GEMM's A
// operand: row m = output pixel, K contiguous, rows padded to a 16-byte
// multiple with zeros (zero, not the zero point: the packed weights are zero
// there, and the GEMM's zero-point corrections use the real K).
#include "qp_internal.hpp"

namespace qp {
namespace {

struct ConvGeom {
  int64_t NB, H, W, C, OH, OW, K;
  int32_t KH, KW, sh, sw, pt, pl, dh, dw;
};

// Each thread writes one 16-byte chunk of one im2col row.
template <bool kVec>
__global__ __launch_bounds__(256) void im2col_kernel(const int8_t* __restrict__ X, ConvGeom g,
                                                     int32_t pad_value, int8_t* __restrict__ col,
                                                     int64_t ldcol, int64_t chunks_per_row,
                                                     int64_t total_chunks) {
  int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= total_chunks) return;
  const int64_t m = id / chunks_per_row;
  const int64_t k0 = (id - m * chunks_per_row) * 16;
  const int64_t ox = m % g.OW;
  const int64_t oy = (m / g.OW) % g.OH;
  const int64_t b = m / (g.OW * g.OH);
  int8_t* dst = col + m * ldcol + k0;
  const uint32_t padw = 0x01010101u * (uint32_t)(uint8_t)(int8_t)pad_value;
  if (kVec) {
    // C % 16 == 0: the chunk lies inside one tap.
    uint4 v = make_uint4(0, 0, 0, 0);
    if (k0 < g.K) {
      const int64_t tap = k0 / g.C, ic = k0 - tap * g.C;
      const int64_t ky = tap / g.KW, kx = tap - ky * g.KW;
      const int64_t iy = oy * g.sh + ky * g.dh - g.pt, ix = ox * g.sw + kx * g.dw - g.pl;
      if (iy >= 0 && iy < g.H && ix >= 0 && ix < g.W)
        v = *reinterpret_cast<const uint4*>(X + ((b * g.H + iy) * g.W + ix) * g.C + ic);
      else
        v = make_uint4(padw, padw, padw, padw);
    }
    *reinterpret_cast<uint4*>(dst) = v;
  } else {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t acc = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t k = k0 + 4 * q + j;
        uint32_t byte = 0;
        if (k < g.K) {
          const int64_t tap = k / g.C, ic = k - tap * g.C;
          const int64_t ky = tap / g.KW, kx = tap - ky * g.KW;
          const int64_t iy = oy * g.sh + ky * g.dh - g.pt, ix = ox * g.sw + kx * g.dw - g.pl;
          int8_t val = (int8_t)pad_value;
          if (iy >= 0 && iy < g.H && ix >= 0 && ix < g.W)
            val = X[((b * g.H + iy) * g.W + ix) * g.C + ic];
          byte = (uint8_t)val;
        }
        acc |= byte << (8 * j);
      }
      w[q] = acc;
    }
    *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace

qp_status conv_out_dims(int64_t H, int64_t W, int32_t KH, int32_t KW, int32_t sh, int32_t sw,
                        int32_t pt, int32_t pl, int32_t pb, int32_t pr, int32_t dh, int32_t dw,
                        int64_t* OH, int64_t* OW) {
  QP_REQUIRE(KH > 0 && KW > 0 && sh > 0 && sw > 0, QP_EINVAL,
             "conv: kernel and stride must be positive");
  QP_REQUIRE(dh > 0 && dw > 0, QP_EINVAL, "conv: dilation must be positive");
  QP_REQUIRE(pt >= 0 && pl >= 0 && pb >= 0 && pr >= 0, QP_EINVAL, "conv: negative padding");
  // a dilated kernel spans d*(k-1)+1 input pixels
  int64_t hh = H + pt + pb - ((int64_t)dh * (KH - 1) + 1);
  int64_t ww = W + pl + pr - ((int64_t)dw * (KW - 1) + 1);
  QP_REQUIRE(hh >= 0 && ww >= 0, QP_EINVAL, "conv: kernel larger than the padded input");
  *OH = hh / sh + 1;
  *OW = ww / sw + 1;
  return QP_OK;
}

qp_status launch_im2col(const int8_t* X, int64_t NB, int64_t H, int64_t W, int64_t C,
                        int32_t pad_value, int32_t KH, int32_t KW, int32_t sh, int32_t sw,
                        int32_t pt, int32_t pl, int32_t dh, int32_t dw, int64_t OH, int64_t OW,
                        int8_t* col, int64_t ldcol, hipStream_t stream) {
  ConvGeom g{NB, H, W, C, OH, OW, (int64_t)KH * KW * C, KH, KW, sh, sw, pt, pl, dh, dw};
  const int64_t rows = NB * OH * OW;
  const int64_t chunks = ldcol / 16;
  const int64_t total = rows * chunks;
  if (total == 0) return QP_OK;
  const unsigned blocks = (unsigned)ceil_div(total, 256);
  const bool vec = (C % 16 == 0) && ((uintptr_t)X % 16 == 0);
  if (vec)
    hipLaunchKernelGGL(im2col_kernel<true>, dim3(blocks), dim3(256), 0, stream, X, g, pad_value,
                       col, ldcol, chunks, total);
  else
    hipLaunchKernelGGL(im2col_kernel<false>, dim3(blocks), dim3(256), 0, stream, X, g, pad_value,
                       col, ldcol, chunks, total);
  return check_launch("qim2col_s8");
}

}  // namespace qp

extern "C" qp_status qim2col_s8(const int8_t* X, int64_t NB, int64_t H, int64_t W, int64_t C,
                                int32_t pad_value, int32_t KH, int32_t KW, int32_t stride_h,
                                int32_t stride_w, int32_t pad_t, int32_t pad_l, int32_t pad_b,
                                int32_t pad_r, int8_t* col, int64_t ldcol, hipStream_t stream) {
  using namespace qp;
  clear_error();
  QP_REQUIRE(NB > 0 && H > 0 && W > 0 && C > 0, QP_EINVAL, "qim2col_s8: empty input");
  QP_REQUIRE(pad_value >= -128 && pad_value <= 127, QP_EINVAL, "qim2col_s8: pad value not int8");
  int64_t OH, OW;
  qp_status st = conv_out_dims(H, W, KH, KW, stride_h, stride_w, pad_t, pad_l, pad_b, pad_r, 1, 1,
                               &OH, &OW);
  if (st) return st;
  const int64_t K = (int64_t)KH * KW * C;
  QP_REQUIRE(ldcol >= K && ldcol % 16 == 0, QP_EINVAL,
             "qim2col_s8: ldcol must be >= K and a multiple of 16");
  QP_REQUIRE(X && col, QP_EINVAL, "qim2col_s8: null pointer");
  QP_REQUIRE((uintptr_t)col % 16 == 0, QP_EALIGN, "qim2col_s8: col must be 16-byte aligned");
  return launch_im2col(X, NB, H, W, C, pad_value, KH, KW, stride_h, stride_w, pad_t, pad_l, 1, 1,
                       OH, OW, col, ldcol, stream);
}
