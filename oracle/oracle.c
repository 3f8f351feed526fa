/*
 * oracle.c -- plain scalar C reference of the quantized integer matmul path.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library.  It shares no code with the GPU library
 * and reads no buffer the GPU wrote.  Each function names the passage it
 * follows; where the pages leave a step open the reading taken is stated at
 * the function.
 *
 * Pages (by title):
 *   [NPU]    "Quantized GEMM: numeric contract, SRAM, DMA and result
 *            verification", a teaching-NPU case study, sections 1-6.
 *   [MNN]    MNN "ConvInt8TiledExecutor.cpp".
 *   [TRACT]  tract-linalg 0.23.9 "frame/pack.rs".
 *   [KLEIDI] pytorch/ao PR #997 "Kleidi 4b blockwise gemv prototype".
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -shared -fPIC.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define ORC_EINVAL (-1)
#define ORC_EUNSUPPORTED (-2)
#define ORC_EOVERFLOW (-3)

static int64_t orc_ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
static int64_t orc_round_up(int64_t a, int64_t b) { return orc_ceil_div(a, b) * b; }
static int64_t orc_clamp64(int64_t v, int64_t lo, int64_t hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}
static int orc_fits_i32(int64_t v) { return v >= -2147483648LL && v <= 2147483647LL; }

/* ========================================================================
 * O1 -- integer affine GEMM.
 * [NPU] section 1: real = scale*(q - zero_point); bias lives at the
 * accumulator scale (scale_A*scale_B[n]).  [NPU] section 5: A is addressed as
 * base_A + m*lda + k and B as base_B + k*ldb + n; here both operands take an
 * explicit element stride per axis so that [K,N] and [N,K] sources are both
 * expressible.  [NPU] section 4: the accumulator is INT32 and the conservative
 * overflow check is K*65025 + |bias_int|, since a zero-point-subtracted int8
 * value has magnitude at most 255.
 * ====================================================================== */
int64_t orc_int32_bound(int64_t K, int64_t max_abs_bias) {
  return K * 65025 + max_abs_bias;
}

static int64_t orc_dot_affine(int64_t m, int64_t n, int64_t K, const int8_t* A, int64_t a_sm,
                              int64_t a_sk, int32_t zA, const int8_t* B, int64_t b_sk,
                              int64_t b_sn, int32_t zb) {
  int64_t s = 0;
  for (int64_t k = 0; k < K; ++k) {
    int64_t a = (int64_t)A[m * a_sm + k * a_sk] - zA;
    int64_t b = (int64_t)B[k * b_sk + n * b_sn] - zb;
    s += a * b;
  }
  return s;
}

int orc_gemm_affine(int64_t M, int64_t N, int64_t K, const int8_t* A, int64_t a_sm,
                    int64_t a_sk, int32_t zA, const int8_t* B, int64_t b_sk, int64_t b_sn,
                    const int32_t* zB, const int32_t* bias, int64_t* acc) {
  if (M < 0 || N < 0 || K < 0) return ORC_EINVAL;
  int rc = 0;
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t n = 0; n < N; ++n) {
      int32_t zb = zB ? zB[n] : 0;
      int64_t s = orc_dot_affine(m, n, K, A, a_sm, a_sk, zA, B, b_sk, b_sn, zb);
      if (bias) s += bias[n];
      acc[m * N + n] = s;
      if (!orc_fits_i32(s)) rc = ORC_EOVERFLOW;
    }
  }
  return rc;
}

int orc_gemm_affine_points(int64_t npts, const int64_t* ms, const int64_t* ns, int64_t K,
                           const int8_t* A, int64_t a_sm, int64_t a_sk, int32_t zA,
                           const int8_t* B, int64_t b_sk, int64_t b_sn, const int32_t* zB,
                           const int32_t* bias, int64_t* acc) {
  int rc = 0;
  for (int64_t i = 0; i < npts; ++i) {
    int64_t m = ms[i], n = ns[i];
    int32_t zb = zB ? zB[n] : 0;
    int64_t s = orc_dot_affine(m, n, K, A, a_sm, a_sk, zA, B, b_sk, b_sn, zb);
    if (bias) s += bias[n];
    acc[i] = s;
    if (!orc_fits_i32(s)) rc = ORC_EOVERFLOW;
  }
  return rc;
}

/* ========================================================================
 * O2 -- tiled model ([NPU] sections 2-4 and the "tiled model vs full integer
 * GEMM" level of the section-6 verification ladder).
 *
 * Tm x Tn x Tk tiles; every tile is executed at full size.  Out-of-range A
 * and B entries are filled with their own zero point so that they stand for
 * real zero ([NPU] section 2); out-of-range outputs are masked.  The INT32
 * accumulator of an output tile is cleared on the first K block and kept
 * across K blocks; bias is added only after the last K block ([NPU]
 * section 4).  Tile, effective-MAC and physical-slot counts are counted by
 * the loops themselves.  Budget ([NPU] section 3): double-buffered inputs,
 * one accumulator, and a reserve that is a parameter of the model.
 * ====================================================================== */
void orc_tile_budget_of(int64_t Tm, int64_t Tn, int64_t Tk, int64_t in_elem_bytes,
                        int64_t acc_elem_bytes, int64_t reserve, orc_tile_budget* out) {
  out->s_input = 2 * (Tm * Tk + Tk * Tn) * in_elem_bytes;
  out->s_acc = acc_elem_bytes * Tm * Tn;
  out->s_reserve = reserve;
  out->s_total = out->s_input + out->s_acc + out->s_reserve;
}

int orc_gemm_tiled(int64_t M, int64_t N, int64_t K, const int8_t* A, int64_t a_sm,
                   int64_t a_sk, int32_t zA, const int8_t* B, int64_t b_sk, int64_t b_sn,
                   const int32_t* zB, const int32_t* bias, int64_t Tm, int64_t Tn, int64_t Tk,
                   int64_t* acc, orc_tile_stats* st) {
  if (M < 0 || N < 0 || K < 0 || Tm <= 0 || Tn <= 0 || Tk <= 0) return ORC_EINVAL;
  orc_tile_stats s;
  memset(&s, 0, sizeof(s));
  s.tiles_m = orc_ceil_div(M, Tm);
  s.tiles_n = orc_ceil_div(N, Tn);
  s.tiles_k = orc_ceil_div(K, Tk);
  int64_t* tile = (int64_t*)malloc(sizeof(int64_t) * (size_t)(Tm * Tn));
  int8_t* ta = (int8_t*)malloc((size_t)(Tm * Tk));
  int8_t* tb = (int8_t*)malloc((size_t)(Tk * Tn));
  int32_t* tzb = (int32_t*)malloc(sizeof(int32_t) * (size_t)Tn);
  if (!tile || !ta || !tb || !tzb) {
    free(tile); free(ta); free(tb); free(tzb);
    return ORC_EINVAL;
  }
  int rc = 0;
  for (int64_t tm = 0; tm < s.tiles_m; ++tm) {
    for (int64_t tn = 0; tn < s.tiles_n; ++tn) {
      for (int64_t j = 0; j < Tn; ++j) {
        int64_t n = tn * Tn + j;
        tzb[j] = (n < N && zB) ? zB[n] : 0;
      }
      for (int64_t tk = 0; tk < s.tiles_k; ++tk) {
        /* "load" the A and B tiles, padding with each operand's zero point */
        for (int64_t i = 0; i < Tm; ++i)
          for (int64_t kk = 0; kk < Tk; ++kk) {
            int64_t m = tm * Tm + i, k = tk * Tk + kk;
            ta[i * Tk + kk] = (m < M && k < K) ? A[m * a_sm + k * a_sk] : (int8_t)zA;
          }
        for (int64_t kk = 0; kk < Tk; ++kk)
          for (int64_t j = 0; j < Tn; ++j) {
            int64_t n = tn * Tn + j, k = tk * Tk + kk;
            tb[kk * Tn + j] = (n < N && k < K) ? B[k * b_sk + n * b_sn] : (int8_t)tzb[j];
          }
        if (tk == 0)
          for (int64_t i = 0; i < Tm * Tn; ++i) tile[i] = 0;
        for (int64_t i = 0; i < Tm; ++i)
          for (int64_t j = 0; j < Tn; ++j)
            for (int64_t kk = 0; kk < Tk; ++kk) {
              int64_t m = tm * Tm + i, n = tn * Tn + j, k = tk * Tk + kk;
              tile[i * Tn + j] +=
                  ((int64_t)ta[i * Tk + kk] - zA) * ((int64_t)tb[kk * Tn + j] - tzb[j]);
              s.physical_slots += 1;
              if (m < M && n < N && k < K) s.effective_mac += 1;
            }
        s.tiles += 1;
      }
      /* post-process once, after the last K block; mask the extra M/N */
      for (int64_t i = 0; i < Tm; ++i)
        for (int64_t j = 0; j < Tn; ++j) {
          int64_t m = tm * Tm + i, n = tn * Tn + j;
          if (m >= M || n >= N) continue;
          int64_t v = tile[i * Tn + j] + (bias ? bias[n] : 0);
          acc[m * N + n] = v;
          if (!orc_fits_i32(v)) rc = ORC_EOVERFLOW;
        }
    }
  }
  s.shape_efficiency =
      s.physical_slots ? (double)s.effective_mac / (double)s.physical_slots : 0.0;
  if (st) *st = s;
  free(tile); free(ta); free(tb); free(tzb);
  return rc;
}

/* ========================================================================
 * O3 -- requantization with an integer multiplier and shift.
 * [NPU] section 1: a per-output-channel weight scale gives a per-column
 * rescale, rounding/saturation follow ONNX QuantizeLinear (round half to
 * even, saturate), and the error of the integer multiplier/shift must be
 * measured apart from the int8 error -- hence orc_ideal_rhe, the exactly
 * rounded product with the real multiplier.  [NPU] section 4: the rescale
 * happens once, after all K.  [MNN] initializeConvInt8QuantInfo and the
 * epilogue parameters of tileSplitFunction: clamp [-128,127], and with ReLU
 * the lower clamp is the output zero point.
 *
 * Reading of the multiplier/shift (the page does not fix it): the real
 * multiplier M = s_a*s_b/s_out (fp64) is written M = f*2^e with f in [0.5,1);
 * m0 = nearest-even(f*2^31) (bumped to 2^30 with e+1 when it reaches 2^31);
 * shift = 31 - e, which must be >= 0.  The contract value is the product
 * acc*m0 (exact, 64-bit) divided by 2^shift with ONE round-half-to-even.
 * ====================================================================== */
double orc_real_multiplier(float s_a, float s_b, float s_out) {
  double num = (double)s_a * (double)s_b;
  return num / (double)s_out;
}

int orc_requant_params(double real_multiplier, int32_t* m0, int32_t* shift) {
  if (!(real_multiplier > 0.0) || !isfinite(real_multiplier)) return ORC_EINVAL;
  int e = 0;
  double f = frexp(real_multiplier, &e);
  double scaled = f * 2147483648.0; /* exact: power-of-two scaling */
  int64_t q = (int64_t)nearbyint(scaled);
  if (q == (int64_t)1 << 31) {
    q = (int64_t)1 << 30;
    e += 1;
  }
  int32_t sh = 31 - e;
  if (sh < 0) return ORC_EUNSUPPORTED;
  *m0 = (int32_t)q;
  *shift = sh;
  return 0;
}

/* t / 2^shift rounded half to even, written with floor division and an
 * explicit remainder test.  Precondition |t| < 2^62. */
int64_t orc_rshift_rhe(int64_t t, int32_t shift) {
  if (shift <= 0) return t;
  if (shift >= 63) return 0; /* |t| < 2^62 gives |t/2^shift| < 1/2 */
  int64_t d = (int64_t)1 << shift;
  int64_t r = t / d;
  int64_t rem = t % d;
  if (rem < 0) {
    rem += d;
    r -= 1;
  }
  int64_t half = d / 2;
  if (rem > half || (rem == half && (r & 1))) r += 1;
  return r;
}

int32_t orc_requant_value(int64_t acc, int32_t m0, int32_t shift, int32_t zp_out, int32_t lo,
                          int32_t hi) {
  int64_t t = acc * (int64_t)m0;
  int64_t r = orc_rshift_rhe(t, shift);
  return (int32_t)orc_clamp64(r + zp_out, lo, hi);
}

/* Exact round-half-even of acc*M for the fp64 value M, in 128-bit integers:
 * M = mant * 2^(e-53) with mant < 2^53.  Result saturated to +-2^40 (only
 * ever compared after clamping to int8). */
int64_t orc_ideal_rhe(int64_t acc, double real_multiplier) {
  int e = 0;
  double f = frexp(real_multiplier, &e);
  int64_t mant = (int64_t)ldexp(f, 53);
  __int128 p = (__int128)acc * (__int128)mant;
  int sh = 53 - e;
  const __int128 cap = (__int128)1 << 40;
  if (sh <= 0) {
    if (sh < -40) return p > 0 ? (int64_t)cap : (p < 0 ? -(int64_t)cap : 0);
    __int128 v = p * ((__int128)1 << (-sh));
    if (v > cap) v = cap;
    if (v < -cap) v = -cap;
    return (int64_t)v;
  }
  if (sh >= 120) return 0;
  __int128 d = (__int128)1 << sh;
  __int128 r = p / d, rem = p % d;
  if (rem < 0) {
    rem += d;
    r -= 1;
  }
  __int128 half = d / 2;
  if (rem > half || (rem == half && (r & 1))) r += 1;
  if (r > cap) r = cap;
  if (r < -cap) r = -cap;
  return (int64_t)r;
}

int orc_requant_matrix(int64_t M, int64_t N, const int64_t* acc, float s_a, const float* s_b,
                       float s_out, int32_t zp_out, int32_t relu, int8_t* out,
                       int64_t* n_differs_from_ideal) {
  int32_t lo = relu ? zp_out : -128, hi = 127;
  int64_t differs = 0;
  for (int64_t n = 0; n < N; ++n) {
    double Mr = orc_real_multiplier(s_a, s_b[n], s_out);
    int32_t m0 = 0, sh = 0;
    int rc = orc_requant_params(Mr, &m0, &sh);
    if (rc) return rc;
    for (int64_t m = 0; m < M; ++m) {
      int64_t a = acc[m * N + n];
      if (!orc_fits_i32(a)) return ORC_EOVERFLOW;
      int32_t q = orc_requant_value(a, m0, sh, zp_out, lo, hi);
      int64_t qi = orc_clamp64(orc_ideal_rhe(a, Mr) + zp_out, lo, hi);
      if (q != qi) differs += 1;
      out[m * N + n] = (int8_t)q;
    }
  }
  if (n_differs_from_ideal) *n_differs_from_ideal = differs;
  return 0;
}

/* ========================================================================
 * O8 -- f32 output of the INT8 GEMM (dequantize, f32 bias, clamp).
 * [MNN] tileSplitFunction: when the destination is not int8 the post
 * parameters carry a float bias and f32 min/max thresholds (the Relu/Relu6
 * post parameters) instead of the integer requantization.  Reading: the
 * exact int32 accumulator of O1 (zero points corrected, no integer bias) is
 * dequantized with sA*sB[n], the f32 bias is added, then clamped:
 *   Y[m,n] = (float) clamp(sA*sB[n]*acc[m,n] + bias[n], lo, hi)
 * formed in fp64 and rounded to f32 once.
 * ====================================================================== */
int orc_dequant_matrix_f32(int64_t M, int64_t N, const int64_t* acc, float s_a,
                           const float* s_b, const float* bias, float lo, float hi, float* Y) {
  if (M < 0 || N < 0 || !(lo <= hi)) return ORC_EINVAL;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      double y = (double)s_a * (double)s_b[n] * (double)acc[m * N + n];
      if (bias) y += (double)bias[n];
      if (y < (double)lo) y = (double)lo;
      if (y > (double)hi) y = (double)hi;
      Y[m * N + n] = (float)y;
    }
  return 0;
}

/* ========================================================================
 * O4 -- convolution, written as direct loops (no im2col) so that it checks
 * the im2col route rather than repeating it.  [MNN] tileSplitFunction: the
 * int8 im2col fills out-of-image taps with the INPUT zero point, so a padded
 * tap stands for real zero.  [MNN] reorderWeight: source weights are
 * [oc, ic, kh*kw] (OIHW).  The convolution zero-point-corrects the input
 * only; the weights are symmetric (zero point 0).  Dilation (the pages show
 * none; reading: the usual definition) places tap (ky, kx) at input offset
 * (ky*dil_h, kx*dil_w); dilation 1 is the plain convolution.
 * ====================================================================== */
static int orc_conv_out_dims(int64_t H, int64_t W, int64_t KH, int64_t KW, int64_t sh,
                             int64_t sw, int64_t pt, int64_t pl, int64_t pb, int64_t pr,
                             int64_t dh, int64_t dw, int64_t* OH, int64_t* OW) {
  if (sh <= 0 || sw <= 0 || KH <= 0 || KW <= 0 || pt < 0 || pl < 0 || pb < 0 || pr < 0 ||
      dh <= 0 || dw <= 0)
    return ORC_EINVAL;
  /* a dilated kernel spans d*(k-1)+1 input pixels */
  int64_t hh = H + pt + pb - (dh * (KH - 1) + 1), ww = W + pl + pr - (dw * (KW - 1) + 1);
  if (hh < 0 || ww < 0) return ORC_EINVAL;
  *OH = hh / sh + 1;
  *OW = ww / sw + 1;
  return 0;
}

int orc_conv2d_direct(int64_t NB, int64_t H, int64_t W, int64_t C, const int8_t* X,
                      int32_t zp_in, int64_t OC, int64_t KH, int64_t KW, const int8_t* Wt,
                      int64_t stride_h, int64_t stride_w, int64_t pad_t, int64_t pad_l,
                      int64_t pad_b, int64_t pad_r, int64_t dil_h, int64_t dil_w,
                      const int32_t* bias, int64_t* acc) {
  int64_t OH, OW;
  int rc = orc_conv_out_dims(H, W, KH, KW, stride_h, stride_w, pad_t, pad_l, pad_b, pad_r, dil_h,
                             dil_w, &OH, &OW);
  if (rc) return rc;
  rc = 0;
  for (int64_t b = 0; b < NB; ++b)
    for (int64_t oy = 0; oy < OH; ++oy)
      for (int64_t ox = 0; ox < OW; ++ox)
        for (int64_t oc = 0; oc < OC; ++oc) {
          int64_t s = 0;
          for (int64_t ky = 0; ky < KH; ++ky)
            for (int64_t kx = 0; kx < KW; ++kx) {
              int64_t iy = oy * stride_h + ky * dil_h - pad_t;
              int64_t ix = ox * stride_w + kx * dil_w - pad_l;
              int inside = iy >= 0 && iy < H && ix >= 0 && ix < W;
              for (int64_t ic = 0; ic < C; ++ic) {
                int64_t xv = inside ? X[((b * H + iy) * W + ix) * C + ic] : zp_in;
                int64_t wv = Wt[((oc * C + ic) * KH + ky) * KW + kx];
                s += (xv - zp_in) * wv;
              }
            }
          if (bias) s += bias[oc];
          acc[((b * OH + oy) * OW + ox) * OC + oc] = s;
          if (!orc_fits_i32(s)) rc = ORC_EOVERFLOW;
        }
  return rc;
}

/* O4c -- convolution with channel-blocked int8 weights and f32 output.
 * [MNN] _computeReorderQuantInfo / onResize: with blockNum > 1 each output
 * channel has one scale per block of input channels (every kernel tap of
 * those channels), the block partial sums are exact integers and are
 * combined in float, and the output is float.  Reading: input per-tensor
 * (sx, zx) with out-of-image taps at zx, weights OIHW with scale
 * sw[oc][ic / icb]:
 *   Y[b,oy,ox,oc] = clamp(sx * sum_{ky,kx,ic} sw[oc][ic/icb] * (xp - zx) * w
 *                         + bias[oc], lo, hi)
 * in fp64, one rounding to f32. */
int orc_conv2d_blockwise_f32(int64_t NB, int64_t H, int64_t W, int64_t C, const int8_t* X,
                             int32_t zx, float sx, int64_t OC, int64_t KH, int64_t KW,
                             const int8_t* Wt, int64_t stride_h, int64_t stride_w, int64_t pad_t,
                             int64_t pad_l, int64_t pad_b, int64_t pad_r, int64_t dil_h,
                             int64_t dil_w, int64_t icb, const float* sw, const float* bias,
                             float lo, float hi, float* Y) {
  int64_t OH, OW;
  if (icb <= 0 || C % icb != 0) return ORC_EINVAL;
  int rc = orc_conv_out_dims(H, W, KH, KW, stride_h, stride_w, pad_t, pad_l, pad_b, pad_r, dil_h,
                             dil_w, &OH, &OW);
  if (rc) return rc;
  int64_t nblk = C / icb;
  for (int64_t b = 0; b < NB; ++b)
    for (int64_t oy = 0; oy < OH; ++oy)
      for (int64_t ox = 0; ox < OW; ++ox)
        for (int64_t oc = 0; oc < OC; ++oc) {
          double s = 0.0;
          for (int64_t blk = 0; blk < nblk; ++blk) {
            int64_t d = 0;
            for (int64_t ky = 0; ky < KH; ++ky)
              for (int64_t kx = 0; kx < KW; ++kx) {
                int64_t iy = oy * stride_h + ky * dil_h - pad_t;
                int64_t ix = ox * stride_w + kx * dil_w - pad_l;
                int inside = iy >= 0 && iy < H && ix >= 0 && ix < W;
                for (int64_t ic = blk * icb; ic < (blk + 1) * icb; ++ic) {
                  int64_t xv = inside ? X[((b * H + iy) * W + ix) * C + ic] : zx;
                  d += (xv - zx) * (int64_t)Wt[((oc * C + ic) * KH + ky) * KW + kx];
                }
              }
            s += (double)sw[oc * nblk + blk] * (double)d;
          }
          double y = (double)sx * s + (bias ? (double)bias[oc] : 0.0);
          if (y < (double)lo) y = (double)lo;
          if (y > (double)hi) y = (double)hi;
          Y[((b * OH + oy) * OW + ox) * OC + oc] = (float)y;
        }
  return 0;
}

/* Explicit im2col: row m = (b, oy, ox), column k = (ky, kx, ic) -- tap outer,
 * input channel inner, the K order of [MNN] reorderWeight. */
int orc_im2col(int64_t NB, int64_t H, int64_t W, int64_t C, const int8_t* X, int32_t pad_value,
               int64_t KH, int64_t KW, int64_t stride_h, int64_t stride_w, int64_t pad_t,
               int64_t pad_l, int64_t pad_b, int64_t pad_r, int64_t dil_h, int64_t dil_w,
               int8_t* col) {
  int64_t OH, OW;
  int rc = orc_conv_out_dims(H, W, KH, KW, stride_h, stride_w, pad_t, pad_l, pad_b, pad_r, dil_h,
                             dil_w, &OH, &OW);
  if (rc) return rc;
  int64_t Kc = KH * KW * C;
  for (int64_t b = 0; b < NB; ++b)
    for (int64_t oy = 0; oy < OH; ++oy)
      for (int64_t ox = 0; ox < OW; ++ox) {
        int64_t m = (b * OH + oy) * OW + ox;
        for (int64_t ky = 0; ky < KH; ++ky)
          for (int64_t kx = 0; kx < KW; ++kx)
            for (int64_t ic = 0; ic < C; ++ic) {
              int64_t iy = oy * stride_h + ky * dil_h - pad_t;
              int64_t ix = ox * stride_w + kx * dil_w - pad_l;
              int inside = iy >= 0 && iy < H && ix >= 0 && ix < W;
              col[m * Kc + (ky * KW + kx) * C + ic] =
                  inside ? X[((b * H + iy) * W + ix) * C + ic] : (int8_t)pad_value;
            }
      }
  return 0;
}

/* ========================================================================
 * O5 -- dynamic per-row asymmetric quantization to int8.
 * [MNN] BatchAsyDynamicQuant computes a per-row min/max, a scale and a zero
 * point, then quantizes with saturation to [-128,127]; [KLEIDI] names the
 * same "qai8dx" activation format.  Neither page prints the arithmetic, and
 * [NPU] section 1 defers rounding and saturation to ONNX.  Reading: the ONNX
 * DynamicQuantizeLinear definition (range widened to include 0, round half to
 * even, saturate), moved from uint8 to int8 (qmin = -128, qmax = 127), as
 * this fixed f32 sequence:
 *   rmin = min(0, min x); rmax = max(0, max x);
 *   scale = (rmax - rmin) / 255;     all-zero row: scale = 1, zp = 0
 *   zp = clamp(rint(-128 - rmin/scale), -128, 127)
 *   q  = clamp(rint(x/scale) + zp, -128, 127)
 * ====================================================================== */
void orc_quantize_row_s8(const float* x, int64_t K, int8_t* q, float* scale, int32_t* zp) {
  float rmin = 0.0f, rmax = 0.0f;
  for (int64_t k = 0; k < K; ++k) {
    if (x[k] < rmin) rmin = x[k];
    if (x[k] > rmax) rmax = x[k];
  }
  float s = (rmax - rmin) / 255.0f;
  int32_t z = 0;
  if (s == 0.0f) {
    s = 1.0f;
    z = 0;
  } else {
    float zf = rintf(-128.0f - rmin / s);
    z = (int32_t)orc_clamp64((int64_t)zf, -128, 127);
  }
  for (int64_t k = 0; k < K; ++k) {
    float r = rintf(x[k] / s);
    int64_t v = (int64_t)r + z;
    q[k] = (int8_t)orc_clamp64(v, -128, 127);
  }
  *scale = s;
  *zp = z;
}

void orc_quantize_rows_s8(int64_t M, int64_t K, const float* X, int64_t ldx, int8_t* Q,
                          int64_t ldq, float* scale, int32_t* zp) {
  for (int64_t m = 0; m < M; ++m) orc_quantize_row_s8(X + m * ldx, K, Q + m * ldq, &scale[m], &zp[m]);
}

/* ========================================================================
 * O5b -- dynamic quantization per row AND per block of K.  [MNN]
 * DenseConvInt8TiledExecutor::onResize: with dynamicQuantOption 2 the input
 * is cut into as many K blocks as the weights (mInputBlockNum = mBlockNum)
 * and BatchAsyDynamicQuant computes a scale and zero point per block.
 * Reading: O5's op sequence applied to each block of `block` consecutive K
 * of a row on its own (the last block may be shorter).
 * ====================================================================== */
void orc_quantize_rows_s8_blocked(int64_t M, int64_t K, int64_t block, const float* X,
                                  int64_t ldx, int8_t* Q, int64_t ldq, float* scale,
                                  int32_t* zp, int64_t ldsz) {
  int64_t G = orc_ceil_div(K, block);
  for (int64_t m = 0; m < M; ++m)
    for (int64_t g = 0; g < G; ++g) {
      int64_t k0 = g * block, len = K - k0 < block ? K - k0 : block;
      orc_quantize_row_s8(X + m * ldx + k0, len, Q + m * ldq + k0, &scale[m * ldsz + g],
                          &zp[m * ldsz + g]);
    }
}

/* ========================================================================
 * O5s -- dynamic per-row symmetric quantization to int8.
 * [MNN] BatchSymDynamicQuant: per row the largest magnitude (MNNAbsMax), a
 * scale from it (MNNQuantScale), then the codes (MNNDynamicQuant) with the
 * input zero point set to 0; the helpers' bodies are not on the page.
 * Reading, in the same f32 style as O5 (division by the dequantization
 * scale, round half to even):
 *   amax = max |x|;  scale = amax / 127;   all-zero row: scale = 1
 *   q = clamp(rint(x/scale), -127, 127)    (zero point 0)
 * ====================================================================== */
void orc_quantize_row_s8_sym(const float* x, int64_t K, int8_t* q, float* scale) {
  float amax = 0.0f;
  for (int64_t k = 0; k < K; ++k) {
    float a = fabsf(x[k]);
    if (a > amax) amax = a;
  }
  float s = amax / 127.0f;
  if (s == 0.0f) s = 1.0f;
  for (int64_t k = 0; k < K; ++k) {
    float r = rintf(x[k] / s);
    q[k] = (int8_t)orc_clamp64((int64_t)r, -127, 127);
  }
  *scale = s;
}

void orc_quantize_rows_s8_sym(int64_t M, int64_t K, const float* X, int64_t ldx, int8_t* Q,
                              int64_t ldq, float* scale) {
  for (int64_t m = 0; m < M; ++m) orc_quantize_row_s8_sym(X + m * ldx, K, Q + m * ldq, &scale[m]);
}

/* ========================================================================
 * O6b -- group scales stored as bf16.  [KLEIDI] review of the wrapper: the
 * KleidiAI kernel keeps the int4 group scales as bf16 to save space (the
 * wrapper converts the f32 scales before packing).  The conversion itself is
 * not printed; reading: round to the nearest bf16 (8 significant bits), ties
 * to even, the IEEE default.  Written from the significand: x = f*2^e with
 * f in [0.5, 1); keep rint(f*2^8)/2^8 (rint rounds half to even).  Finite,
 * normal inputs only (scales are positive and far from the denormal range).
 * ====================================================================== */
float orc_round_bf16(float x) {
  if (x == 0.0f || !isfinite(x)) return x;
  int e = 0;
  double f = frexp((double)x, &e);      /* exact: f has x's 24 bits */
  double r = rint(ldexp(f, 8));         /* 8 significant bits, ties to even */
  return (float)ldexp(r, e - 8);        /* r*2^(e-8) is a bf16 value, exact in f32 */
}

void orc_round_bf16_array(int64_t n, const float* x, float* y) {
  for (int64_t i = 0; i < n; ++i) y[i] = orc_round_bf16(x[i]);
}

/* ========================================================================
 * O6 -- int8 activations times int4 weights with one f32 scale per group of
 * `group` consecutive K ([KLEIDI]: f32 output with clamp, dynamically
 * quantized int8 activations, signed int4 weights in blocks of 32, and no
 * weight zero points).  [MNN] tileSplitFunction keeps a float accumulator
 * across quantization blocks and folds the input zero point with a weight
 * kernel sum.  Reading: the sum inside one group is exact in integers, the
 * sum across groups cannot be (each group has its own f32 scale), so it is
 * formed in fp64 and rounded to f32 once at the end; bias is added after the
 * dequantization and before the clamp.
 *   D[m,n,g] = sum_{k in g} (qa[m,k] - za[m]) * qw[n,k]
 *   Y[m,n]   = clamp(sa[m] * sum_g sw[n,g]*D[m,n,g] + bias[n], lo, hi)
 * ====================================================================== */
int orc_a8w4_blockwise(int64_t M, int64_t N, int64_t K, int64_t group, const int8_t* qa,
                       int64_t lda, const float* sa, const int32_t* za, const int8_t* qw,
                       int64_t ldw, const float* sw, int64_t ldsw, const float* bias,
                       float clamp_lo, float clamp_hi, float* Y, int64_t ldy) {
  if (M < 0 || N < 0 || K < 0 || group <= 0) return ORC_EINVAL;
  int64_t G = orc_ceil_div(K, group);
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      double sum = 0.0;
      for (int64_t g = 0; g < G; ++g) {
        int64_t d = 0;
        int64_t k1 = (g + 1) * group < K ? (g + 1) * group : K;
        for (int64_t k = g * group; k < k1; ++k)
          d += ((int64_t)qa[m * lda + k] - za[m]) * (int64_t)qw[n * ldw + k];
        sum += (double)sw[n * ldsw + g] * (double)d;
      }
      double y = (double)sa[m] * sum + (bias ? (double)bias[n] : 0.0);
      if (y < (double)clamp_lo) y = (double)clamp_lo;
      if (y > (double)clamp_hi) y = (double)clamp_hi;
      Y[m * ldy + n] = (float)y;
    }
  return 0;
}

/* ========================================================================
 * O6d -- int4 group weights times activations quantized per block (O5b),
 * the activation blocks being the weight groups: each group then has its
 * own activation scale and zero point as well as its weight scale.
 *   Y[m,n] = clamp(sum_g sa[m,g]*sw[n,g] * sum_{k in g} (qa[m,k]-za[m,g])*qw[n,k]
 *                  + bias[n], lo, hi)
 * Group sums exact in integers, the rest in fp64, one rounding to f32.
 * ====================================================================== */
int orc_a8w4_blockwise_blockq(int64_t M, int64_t N, int64_t K, int64_t group, const int8_t* qa,
                              int64_t lda, const float* sa, const int32_t* za, int64_t ldsz,
                              const int8_t* qw, int64_t ldw, const float* sw, int64_t ldsw,
                              const float* bias, float clamp_lo, float clamp_hi, float* Y,
                              int64_t ldy) {
  if (M < 0 || N < 0 || K < 0 || group <= 0) return ORC_EINVAL;
  int64_t G = orc_ceil_div(K, group);
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      double sum = 0.0;
      for (int64_t g = 0; g < G; ++g) {
        int64_t d = 0;
        int64_t k1 = (g + 1) * group < K ? (g + 1) * group : K;
        for (int64_t k = g * group; k < k1; ++k)
          d += ((int64_t)qa[m * lda + k] - za[m * ldsz + g]) * (int64_t)qw[n * ldw + k];
        sum += (double)sa[m * ldsz + g] * (double)sw[n * ldsw + g] * (double)d;
      }
      double y = sum + (bias ? (double)bias[n] : 0.0);
      if (y < (double)clamp_lo) y = (double)clamp_lo;
      if (y > (double)clamp_hi) y = (double)clamp_hi;
      Y[m * ldy + n] = (float)y;
    }
  return 0;
}

/* ========================================================================
 * O6c -- asymmetric int4 weights: a float offset per group besides the
 * scale.  [MNN] _computeReorderQuantInfo / the KleidiAI branch of the weight
 * preparation: for asymmetric weights each (channel, block) carries a pair
 * (zero, scale) with real weight = scale*q + zero (the zero shifted by the
 * int4 origin offset), and the weight kernel sum becomes the sum of the real
 * weights.  Reading: logical q in [-8, 7], w[n,k] = sw[n,g]*q[n,k] + bw[n,g]
 * (the caller gives bw already for that q), the rest as O6:
 *   Y[m,n] = clamp(sa[m] * sum_k (qa[m,k] - za[m]) * w[n,k] + bias[n], lo, hi)
 * summed per group as sw*D + bw*E, D = sum (qa-za)*q and E = sum (qa-za)
 * exact integers, the groups in fp64, one rounding to f32.
 * ====================================================================== */
int orc_a8w4_blockwise_asym(int64_t M, int64_t N, int64_t K, int64_t group, const int8_t* qa,
                            int64_t lda, const float* sa, const int32_t* za, const int8_t* qw,
                            int64_t ldw, const float* sw, const float* bw, int64_t ldsw,
                            const float* bias, float clamp_lo, float clamp_hi, float* Y,
                            int64_t ldy) {
  if (M < 0 || N < 0 || K < 0 || group <= 0) return ORC_EINVAL;
  int64_t G = orc_ceil_div(K, group);
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      double sum = 0.0;
      for (int64_t g = 0; g < G; ++g) {
        int64_t d = 0, e = 0;
        int64_t k1 = (g + 1) * group < K ? (g + 1) * group : K;
        for (int64_t k = g * group; k < k1; ++k) {
          int64_t a = (int64_t)qa[m * lda + k] - za[m];
          d += a * (int64_t)qw[n * ldw + k];
          e += a;
        }
        sum += (double)sw[n * ldsw + g] * (double)d + (double)bw[n * ldsw + g] * (double)e;
      }
      double y = (double)sa[m] * sum + (bias ? (double)bias[n] : 0.0);
      if (y < (double)clamp_lo) y = (double)clamp_lo;
      if (y > (double)clamp_hi) y = (double)clamp_hi;
      Y[m * ldy + n] = (float)y;
    }
  return 0;
}

/* ========================================================================
 * O7 -- reference writer of the library's packed-weight blob, written from
 * the format definition (not from the GPU packer).  Prior art for what a
 * packed operand holds: [TRACT] PackedI8K4 (K-inner int8 panels with
 * zero-filled tails) and pack_tensor_view (padding bytes are defined because
 * the kernel computes on them); [MNN] packWeightAndQuantInfo (scales stored
 * with the packed weights) and _computeReorderQuantInfo (weight kernel sums
 * precomputed at pack time).
 *
 * Blob = 256-byte header, then regions, each starting on a 256-byte boundary.
 * Header (little endian):
 *   u32 magic 0x4B505149, u32 version 1, u32 format (1 int8, 2 int4),
 *   u32 scheme (0 per-tensor, 1 per-channel, 2 blockwise),
 *   i64 N, K, Npad, Kpad, group, data_off, data_bytes, scale_off, sum_off,
 *   zp_off, total_bytes; i32 has_zero_points; i32 invalid-int4 flag (0);
 *   int8 format: f32 smallest and f32 largest weight scale of the real
 *   channels (bytes 112 and 116; 0 for the other formats); zero to byte 256.
 * int8 format:  Npad = roundup(N,64), Kpad = roundup(K,64);
 *   data: 32x32 sub-tiles, [Npad/32][Kpad/32][32 rows][32 bytes] -- W[n,k]
 *   at ((n/32)*(Kpad/32) + k/32)*1024 + (n%32)*32 + k%32, zero beyond N, K;
 *   scale f32[Npad], colsum i32[Npad] = sum_{k<K} W[n,k], zp i32[Npad].
 * int4 format:  Npad = roundup(N,64), Kpad = roundup(K, max(group,128))
 *   (group 32, 64, 128 or a multiple of 128).  Each channel's K is cut in
 *   blocks of 128 (64 bytes); the 16 channels of a tile n/16 store block b
 *   next to each other: channel n, block b at ((n/16)*(Kpad/128) + b)*1024
 *   + (n%16)*64.  Within a block, byte 16c+4t+j (c, t, j in 0..3) holds
 *   k = 32t+8c+j in its low nibble and k = 32t+8c+4+j in its high nibble,
 *   as 4-bit two's complement.  Scales f32 in quads of 4 groups, the 16
 *   channels of a tile side by side: sw[n,g] at float index
 *   ((n/16)*Gq + g/4)*64 + (n%16)*4 + g%4, Gq = ceil((Kpad/group)/4).
 *   wsum f32[Npad] = (float) sum_g (double)sw[n,g] * sum_{k in g} W[n,k],
 *   accumulated in fp64 in increasing g.  All padding is zero.
 * ====================================================================== */
#define ORC_HDR 256
static int64_t orc_a256(int64_t x) { return orc_round_up(x, 256); }
static void orc_put_u32(uint8_t* p, int64_t off, uint32_t v) { memcpy(p + off, &v, 4); }
static void orc_put_i32(uint8_t* p, int64_t off, int32_t v) { memcpy(p + off, &v, 4); }
static void orc_put_i64(uint8_t* p, int64_t off, int64_t v) { memcpy(p + off, &v, 8); }

static void orc_header(uint8_t* blob, uint32_t format, uint32_t scheme, int64_t N, int64_t K,
                       int64_t Npad, int64_t Kpad, int64_t group, int64_t data_bytes,
                       int64_t scale_off, int64_t sum_off, int64_t zp_off, int64_t total,
                       int32_t has_zp) {
  memset(blob, 0, ORC_HDR);
  orc_put_u32(blob, 0, 0x4B505149u);
  orc_put_u32(blob, 4, 1u);
  orc_put_u32(blob, 8, format);
  orc_put_u32(blob, 12, scheme);
  orc_put_i64(blob, 16, N);
  orc_put_i64(blob, 24, K);
  orc_put_i64(blob, 32, Npad);
  orc_put_i64(blob, 40, Kpad);
  orc_put_i64(blob, 48, group);
  orc_put_i64(blob, 56, ORC_HDR);
  orc_put_i64(blob, 64, data_bytes);
  orc_put_i64(blob, 72, scale_off);
  orc_put_i64(blob, 80, sum_off);
  orc_put_i64(blob, 88, zp_off);
  orc_put_i64(blob, 96, total);
  orc_put_i32(blob, 104, has_zp);
}

int64_t orc_packed_s8_bytes(int64_t N, int64_t K) {
  int64_t Npad = orc_round_up(N, 64), Kpad = orc_round_up(K, 64);
  return ORC_HDR + orc_a256(Npad * Kpad) + 3 * orc_a256(4 * Npad);
}

int orc_pack_s8_ref(int64_t N, int64_t K, const int8_t* Wt, int64_t w_sn, int64_t w_sk,
                    int32_t per_channel, const float* scales, const int32_t* zps,
                    uint8_t* blob) {
  if (N <= 0 || K <= 0) return ORC_EINVAL;
  int64_t Npad = orc_round_up(N, 64), Kpad = orc_round_up(K, 64);
  int64_t data_bytes = Npad * Kpad;
  int64_t scale_off = ORC_HDR + orc_a256(data_bytes);
  int64_t sum_off = scale_off + orc_a256(4 * Npad);
  int64_t zp_off = sum_off + orc_a256(4 * Npad);
  int64_t total = zp_off + orc_a256(4 * Npad);
  memset(blob, 0, (size_t)total);
  int32_t has_zp = 0;
  for (int64_t n = 0; n < N; ++n) {
    int32_t z = zps ? (per_channel ? zps[n] : zps[0]) : 0;
    if (z != 0) has_zp = 1;
  }
  orc_header(blob, 1u, per_channel ? 1u : 0u, N, K, Npad, Kpad, 0, data_bytes, scale_off,
             sum_off, zp_off, total, has_zp);
  float smin = scales[0], smax = scales[0];
  for (int64_t n = 0; per_channel && n < N; ++n) {
    if (scales[n] < smin) smin = scales[n];
    if (scales[n] > smax) smax = scales[n];
  }
  memcpy(blob + 112, &smin, 4);
  memcpy(blob + 116, &smax, 4);
  for (int64_t n = 0; n < N; ++n) {
    int64_t cs = 0;
    for (int64_t k = 0; k < K; ++k) {
      int8_t v = Wt[n * w_sn + k * w_sk];
      int64_t off = ((n / 32) * (Kpad / 32) + k / 32) * 1024 + (n % 32) * 32 + k % 32;
      blob[ORC_HDR + off] = (uint8_t)v;
      cs += v;
    }
    float sc = per_channel ? scales[n] : scales[0];
    memcpy(blob + scale_off + 4 * n, &sc, 4);
    orc_put_i32(blob, sum_off + 4 * n, (int32_t)cs);
    orc_put_i32(blob, zp_off + 4 * n, zps ? (per_channel ? zps[n] : zps[0]) : 0);
  }
  return 0;
}

static int orc_s4_group_ok(int64_t group) {
  return group > 0 && group % 32 == 0 && (128 % group == 0 || group % 128 == 0);
}

int64_t orc_packed_s4_bytes(int64_t N, int64_t K, int64_t group) {
  if (!orc_s4_group_ok(group)) return -1;
  int64_t Npad = orc_round_up(N, 64), Kpad = orc_round_up(K, group > 128 ? group : 128);
  int64_t Gq = orc_ceil_div(Kpad / group, 4);
  return ORC_HDR + orc_a256(Npad * Kpad / 2) + orc_a256(16 * Npad * Gq) + orc_a256(4 * Npad);
}

int orc_pack_s4_ref(int64_t N, int64_t K, int64_t group, const int8_t* Wt, int64_t w_sn,
                    int64_t w_sk, const float* sw, int64_t ldsw, uint8_t* blob) {
  if (N <= 0 || K <= 0 || !orc_s4_group_ok(group)) return ORC_EINVAL;
  int64_t Npad = orc_round_up(N, 64), Kpad = orc_round_up(K, group > 128 ? group : 128);
  int64_t G = Kpad / group;
  int64_t Gq = orc_ceil_div(G, 4);      /* scale quads per channel */
  int64_t nblk = Kpad / 128;            /* 128-K blocks per channel */
  int64_t data_bytes = Npad * Kpad / 2;
  int64_t scale_off = ORC_HDR + orc_a256(data_bytes);
  int64_t sum_off = scale_off + orc_a256(16 * Npad * Gq);
  int64_t total = sum_off + orc_a256(4 * Npad);
  memset(blob, 0, (size_t)total);
  orc_header(blob, 2u, 2u, N, K, Npad, Kpad, group, data_bytes, scale_off, sum_off, 0, total, 0);
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t k = 0; k < K; ++k) {
      int8_t v = Wt[n * w_sn + k * w_sk];
      if (v < -8 || v > 7) return ORC_EINVAL;
      int64_t block = k / 128, t = (k % 128) / 32, c = (k % 32) / 8, j = k % 4;
      int64_t high = (k % 8) >= 4;
      int64_t byte = ORC_HDR + ((n / 16) * nblk + block) * 1024 + (n % 16) * 64 + 16 * c + 4 * t + j;
      uint8_t nib = (uint8_t)(v & 0xF);
      blob[byte] |= high ? (uint8_t)(nib << 4) : nib;
    }
    double ws = 0.0;
    int64_t Greal = orc_ceil_div(K, group);
    for (int64_t g = 0; g < G; ++g) {
      int64_t gs = 0;
      for (int64_t k = g * group; k < (g + 1) * group && k < K; ++k) gs += Wt[n * w_sn + k * w_sk];
      float s = (g < Greal) ? sw[n * ldsw + g] : 0.0f;
      memcpy(blob + scale_off + 4 * (((n / 16) * Gq + g / 4) * 64 + (n % 16) * 4 + g % 4), &s, 4);
      ws += (double)s * (double)gs;
    }
    float wsf = (float)ws;
    memcpy(blob + sum_off + 4 * n, &wsf, 4);
  }
  return 0;
}
