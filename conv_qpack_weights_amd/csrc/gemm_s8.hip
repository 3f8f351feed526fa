// gemm_s8.hip -- INT8 x INT8 GEMM with exact INT32 accumulation, zero-point
// correction and a fused requantizing (or raw INT32) epilogue, for gfx950.
//
// Numeric contract: "Quantized GEMM: numeric contract, SRAM, DMA and result
// verification" (teaching-NPU case study) --
//   section 1: real = scale*(q - zp); bias at the accumulator scale; a
//     per-channel weight scale gives a per-column integer multiplier/shift;
//   section 2: padding must stand for real zero (here: zero bytes in both
//     operands, with the zero-point terms computed over the real K -- the
//     "equivalent mask");
//   section 4: one INT32 accumulator per output, cleared once and kept over
//     all of K; bias, activation and rescale only at the end;
//   section 5: row-major A (base + m*lda + k); the blob rows play B.
// MNN "ConvInt8TiledExecutor.cpp" (tileSplitFunction): clamp [-128,127], and
// with ReLU the lower clamp is the output zero point.
//
// Kernel design (gfx950; the pages' designs are prior art only): a workgroup
// owns a BM x BN output tile (256x256x128 for large shapes, 128x128 and
// 64x64x64 below); the activation tile goes through a 4-deep LDS ring by
// direct loads, the packed weights straight into registers one K tile ahead,
// one barrier per K tile (see gemm_s8_core.hpp).  The MFMA is issued as
// (B fragment, A fragment), so every lane ends up holding 4 consecutive
// output channels of one row; full tiles are staged through LDS and written
// as whole 16-byte row pieces.  Outputs: requantized int8, raw int32, or
// f32 (dequantize, f32 bias, clamp).
// The zero-point identity used is
//   sum (a-zA)(b-zB) = sum ab - zB*rowsum(a) - zA*colsum(b) + K*zA*zB,
// evaluated in wrapping 32-bit arithmetic, which is exact whenever the true
// result fits INT32 (checked on the host with the K*65025+|bias| bound).
#include <atomic>
#include <cmath>
#include <cstring>

#include "qp_internal.hpp"

#pragma clang fp contract(off)

#include "gemm_s8_core.hpp"

namespace qp {
namespace {

// ---- A preparation: copy to an aligned, K-padded buffer and/or row sums ---
// One wave per row.  Writes Ap[m][0..Kpad) (zeros beyond K) when `copy`, and
// rowsum[m] = sum_{k<K} A[m,k] when `rowsum` is non-null.
__global__ __launch_bounds__(256) void prep_a_kernel(const int8_t* __restrict__ A, int64_t M,
                                                     int64_t K, int64_t lda, int8_t* __restrict__ Ap,
                                                     int64_t Kpad, int32_t* __restrict__ rowsum) {
  const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (m >= M) return;
  const int8_t* src = A + m * lda;
  int32_t s = 0;
  if (Ap) {
    int8_t* dst = Ap + m * Kpad;
    for (int64_t k0 = (int64_t)lane * 16; k0 < Kpad; k0 += 64 * 16) {
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t v = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t k = k0 + 4 * q + j;
          int32_t b = k < K ? src[k] : 0;
          s += b;
          v |= (uint32_t)(uint8_t)b << (8 * j);
        }
        w[q] = v;
      }
      *reinterpret_cast<uint4*>(dst + k0) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  } else {
    for (int64_t k = lane; k < K; k += 64) s += src[k];
  }
  if (rowsum) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    if (lane == 0) rowsum[m] = s;
  }
}

// Deepest K the resident-activation kernel holds in LDS (64 rows x Kpad).
constexpr int64_t kResidentMaxKpad = 960;

template <int BM, int BN, int BK, int NW, int SA, int MF, bool kOut32, bool kRowSum, bool kHi,
          bool kF32, int WM = 1, bool kResident = false>
qp_status launch_cfg(const GemmArgs& a0, hipStream_t stream) {
  GemmArgs a = a0;
  a.tiles_m = (int32_t)ceil_div(a.M, BM);
  a.tiles_n = (int32_t)ceil_div(a.N, BN);
  a.group_m = 4;
  a.xcd_remap = 1;
  const int64_t blocks = (int64_t)a.tiles_m * a.tiles_n;
  if (blocks == 0) return QP_OK;
  QP_REQUIRE(blocks < (1LL << 31), QP_EUNSUPPORTED, "qgemm: too many tiles");
  // resident activations hold every K tile; the limit is reserved for the
  // largest depth that mode takes
  const size_t lds = kResident ? (size_t)(a.Kpad / BK) * BM * BK : (size_t)SA * BM * BK;
  const size_t lds_max = kResident ? (size_t)kResidentMaxKpad * BM : lds;
  auto kern = qgemm_s8_kernel<BM, BN, BK, NW, SA, MF, kOut32, kRowSum, kHi, kF32, WM, kResident>;
  // The LDS limit is raised once per instantiation and device (threads may
  // race to set it; repeating it is harmless).
  static std::atomic<uint64_t> lds_attr_devices{0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) QP_FAIL(QP_EHIP, "qgemm: hipGetDevice failed");
  const uint64_t bit = dev >= 0 && dev < 64 ? (UINT64_C(1) << dev) : 0;
  if (bit == 0 || (lds_attr_devices.load(std::memory_order_acquire) & bit) == 0) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_max) != hipSuccess)
      QP_FAIL(QP_EHIP, "qgemm: cannot reserve %zu bytes of LDS", lds_max);
    lds_attr_devices.fetch_or(bit, std::memory_order_release);
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(NW * 64), lds, stream, a);
  return check_launch("qgemm_s8s8 kernel");
}

// Tile configuration: 256x256 (8 waves) when that fills the chip, else
// 128x128, else 64x64 with one K-step per tile.
enum GemmCfg { kCfg256, kCfg128, kCfg64 };
GemmCfg pick_cfg(int64_t M, int64_t N, int64_t Kpad) {
  const bool k128 = (Kpad % 128) == 0;
  if (k128 && ceil_div(M, 256) * ceil_div(N, 256) >= 256) return kCfg256;
  if (k128 && ceil_div(M, 128) * ceil_div(N, 128) >= 256) return kCfg128;
  return kCfg64;
}

template <bool kOut32, bool kRowSum, bool kHi, bool kF32 = false>
qp_status launch_gemm_sel(const GemmArgs& a, bool resident, hipStream_t stream) {
  switch (pick_cfg(a.M, a.N, a.Kpad)) {
    case kCfg256:
      return launch_cfg<256, 256, 128, 8, 4, 32, kOut32, kRowSum, kHi, kF32, 2>(a, stream);
    case kCfg128:
      return launch_cfg<128, 128, 128, 4, 4, 32, kOut32, kRowSum, kHi, kF32>(a, stream);
    default:
      if (resident)
        return launch_cfg<64, 64, 64, 4, 3, 16, kOut32, kRowSum, kHi, kF32, 1, true>(a, stream);
      return launch_cfg<64, 64, 64, 4, 3, 16, kOut32, kRowSum, kHi, kF32>(a, stream);
  }
}

}  // namespace

// Host copy of the device multiplier derivation (validation only).
static bool host_mult_ok(double mr) {
  if (!(mr > 0.0) || !std::isfinite(mr)) return false;
  int e = 0;
  double f = std::frexp(mr, &e);
  int64_t q = (int64_t)std::nearbyint(f * 2147483648.0);
  if (q == ((int64_t)1 << 31)) e += 1;
  return 31 - e >= 0;
}

struct GemmPlan {
  bool copy_a;
  bool rowsum;
  bool resident;  // one launch: the GEMM reads A byte-exact and sums its rows
  int64_t ws_a, ws_rowsum, ws_total;
};

static GemmPlan plan_gemm(int64_t M, int64_t K, int64_t lda, const void* A,
                          const qp_packed_info* b) {
  GemmPlan p;
  p.rowsum = b->has_zero_points != 0;
  // The kernel addresses a 256-row A tile with 32-bit offsets from its first
  // row, so very wide strides are compacted first as well.
  p.copy_a = (K != b->Kpad) || (lda % 16 != 0) || (((uintptr_t)A) % 16 != 0) ||
             (lda > (INT64_C(1) << 22));
  p.resident = false;
  p.ws_a = p.copy_a ? round_up(M * b->Kpad, 256) : 0;
  p.ws_rowsum = p.rowsum ? round_up(4 * M, 256) : 0;
  p.ws_total = p.ws_a + p.ws_rowsum;
  return p;
}

// Small GEMMs (64x64 tiles) that would need the A copy or the row sums take
// the resident-activation kernel instead: no workspace, one launch.
static void plan_resident(GemmPlan* p, int64_t M, const qp_packed_info* b) {
  if ((p->copy_a || p->rowsum) && b->Kpad <= kResidentMaxKpad &&
      pick_cfg(M, b->N, b->Kpad) == kCfg64) {
    p->resident = true;
    p->copy_a = false;
    p->ws_a = p->ws_rowsum = p->ws_total = 0;
  }
}

qp_status run_gemm_s8(const int8_t* A, int64_t M, int64_t lda, float sA, int32_t zA,
                      const qp_packed_info* b, const void* packedB, const int32_t* bias,
                      float sOut, int32_t zp_out, bool out32, int32_t relu, void* C, int64_t ldc,
                      void* ws, size_t ws_bytes, bool a_is_padded, hipStream_t stream,
                      const GemmF32Out* f32) {
  const uint8_t* blob = static_cast<const uint8_t*>(packedB);
  GemmPlan p = plan_gemm(M, b->K, lda, A, b);
  if (a_is_padded) {
    p.copy_a = false;
    p.ws_a = 0;
    p.ws_total = p.ws_rowsum;
  }
  plan_resident(&p, M, b);
  QP_REQUIRE(ws_bytes >= (size_t)p.ws_total, QP_ESIZE, "qgemm: workspace holds %zu bytes, needs %lld",
             ws_bytes, (long long)p.ws_total);
  QP_REQUIRE(p.ws_total == 0 || (ws && ((uintptr_t)ws % 256) == 0), QP_EALIGN,
             "qgemm: workspace must be non-null and 256-byte aligned");
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  int8_t* Ap = p.copy_a ? reinterpret_cast<int8_t*>(wsb) : nullptr;
  int32_t* rs = p.rowsum && !p.resident ? reinterpret_cast<int32_t*>(wsb + p.ws_a) : nullptr;
  if (M == 0) return QP_OK;
  if (!p.resident && (p.copy_a || p.rowsum)) {
    hipLaunchKernelGGL(prep_a_kernel, dim3((unsigned)ceil_div(M, 4)), dim3(256), 0, stream, A, M,
                       b->K, lda, Ap, b->Kpad, rs);
    qp_status st = check_launch("qgemm prep A");
    if (st) return st;
  }
  GemmArgs a;
  std::memset(&a, 0, sizeof(a));
  a.A = p.copy_a ? Ap : A;
  a.lda = p.copy_a ? b->Kpad : lda;
  a.B = reinterpret_cast<const int8_t*>(blob + b->data_off);
  a.ldb = b->Kpad;
  a.M = M;
  a.N = b->N;
  a.K = b->K;
  a.Kpad = b->Kpad;
  a.Npad = b->Npad;
  a.colsum = reinterpret_cast<const int32_t*>(blob + b->sum_off);
  a.zpB = reinterpret_cast<const int32_t*>(blob + b->zp_off);
  a.sB = reinterpret_cast<const float*>(blob + b->scale_off);
  a.rowsum = rs;
  a.bias = bias;
  a.sA = sA;
  a.sOut = sOut;
  a.zA = zA;
  a.zp_out = zp_out;
  a.lo = relu ? zp_out : -128;
  a.hi = 127;
  a.C = C;
  a.ldc = ldc;
  if (f32) {
    a.bias_f = f32->bias;
    a.clo = f32->lo;
    a.chi = f32->hi;
    return p.rowsum ? launch_gemm_sel<true, true, false, true>(a, p.resident, stream)
                    : launch_gemm_sel<true, false, false, true>(a, p.resident, stream);
  }
  if (out32)
    return p.rowsum ? launch_gemm_sel<true, true, false>(a, p.resident, stream)
                    : launch_gemm_sel<true, false, false>(a, p.resident, stream);
  // All shifts >= 32 <=> every multiplier < 1/2 (with margin for the m0
  // rounding bump); known only when the scales were seen at pack time.  The
  // kernel for this case also folds the zero-point terms and the output
  // zero point into one 64-bit addend, which stays exact while every shift
  // is at most 53, i.e. every multiplier is at least 2^-23 (smaller ones
  // take the general 64-bit rounding).
  const double m_hi = (double)sA * (double)b->scale_max / (double)sOut;
  const double m_lo = (double)sA * (double)b->scale_min / (double)sOut;
  const bool hi = b->scale_max > 0.0f && m_hi * (1.0 + 1e-6) < 0.5 &&
                  m_lo * (1.0 - 1e-6) >= 0x1p-23;
  if (hi)
    return p.rowsum ? launch_gemm_sel<false, true, true>(a, p.resident, stream)
                    : launch_gemm_sel<false, false, true>(a, p.resident, stream);
  return p.rowsum ? launch_gemm_sel<false, true, false>(a, p.resident, stream)
                  : launch_gemm_sel<false, false, false>(a, p.resident, stream);
}

qp_status validate_gemm(const qp_packed_info* b, int64_t K, float sA, int32_t zA,
                        const int32_t* bias, int64_t max_abs_bias, const qp_qtensor* out,
                        bool* out32) {
  QP_REQUIRE(b && b->format == 1, QP_EINVAL, "qgemm: weights must be an int8 blob");
  QP_REQUIRE(K == b->K, QP_EINVAL, "qgemm: activation K=%lld but the weights have K=%lld",
             (long long)K, (long long)b->K);
  QP_REQUIRE(zA >= -128 && zA <= 127, QP_EINVAL, "qgemm: activation zero point %d outside int8", zA);
  QP_REQUIRE(std::isfinite(sA) && sA > 0, QP_EINVAL, "qgemm: activation scale must be > 0");
  QP_REQUIRE(out, QP_EINVAL, "qgemm: output descriptor is NULL");
  QP_REQUIRE(out->rounding == QP_ROUND_HALF_EVEN, QP_EUNSUPPORTED,
             "qgemm: only round-half-to-even is implemented");
  const int64_t bb = bias ? max_abs_bias : 0;
  QP_REQUIRE(bb >= 0, QP_EINVAL, "qgemm: max_abs_bias must be >= 0");
  QP_REQUIRE(K <= (INT64_C(2147483647) - bb) / 65025 && K * 65025 + bb <= INT64_C(2147483647),
             QP_EOVERFLOW, "qgemm: K*65025 + max|bias| = %lld exceeds INT32",
             (long long)(K * 65025 + bb));
  if (out->dtype == QP_S8) {
    *out32 = false;
    QP_REQUIRE(out->qmin == -128 && out->qmax == 127, QP_EUNSUPPORTED,
               "qgemm: int8 output saturation must be [-128,127]");
    QP_REQUIRE(out->scheme == QP_PER_TENSOR, QP_EUNSUPPORTED, "qgemm: output must be per-tensor");
    QP_REQUIRE(std::isfinite(out->scale) && out->scale > 0, QP_EINVAL,
               "qgemm: output scale must be > 0");
    QP_REQUIRE(out->zero_point >= -128 && out->zero_point <= 127, QP_EINVAL,
               "qgemm: output zero point outside int8");
    if (b->scale_max > 0.0f) {
      const double mmax = ((double)sA * (double)b->scale_max) / (double)out->scale;
      const double mmin = ((double)sA * (double)b->scale_min) / (double)out->scale;
      QP_REQUIRE(host_mult_ok(mmax) && mmin > 0.0, QP_EUNSUPPORTED,
                 "qgemm: requantization multiplier out of range (max %g)", mmax);
    }
  } else if (out->dtype == QP_S32) {
    *out32 = true;
  } else {
    QP_FAIL(QP_EUNSUPPORTED, "qgemm: output dtype must be QP_S8 or QP_S32");
  }
  return QP_OK;
}

}  // namespace qp

extern "C" qp_status qgemm_s8s8_requant_ws_size(const qp_qtensor* a, const qp_packed_info* b,
                                                size_t* bytes) {
  using namespace qp;
  QP_REQUIRE(a && b && bytes, QP_EINVAL, "qgemm_s8s8_requant_ws_size: null argument");
  QP_REQUIRE(a->rank == 2, QP_EINVAL, "qgemm: activations must be rank 2");
  // Small GEMMs need none (direct loads, or the resident-activation
  // kernel).  Otherwise the alignment of A is not known here: size for the
  // copying plan.
  if (b->Kpad <= kResidentMaxKpad && pick_cfg(a->shape[0], b->N, b->Kpad) == kCfg64) {
    *bytes = 0;
    return QP_OK;
  }
  GemmPlan p = plan_gemm(a->shape[0], a->shape[1], a->stride[0], nullptr, b);
  if (!p.copy_a) {
    p.copy_a = true;
    p.ws_a = round_up(a->shape[0] * b->Kpad, 256);
    p.ws_total = p.ws_a + p.ws_rowsum;
  }
  *bytes = (size_t)p.ws_total;
  return QP_OK;
}

extern "C" qp_status qgemm_s8s8_requant(const qp_qtensor* a, const int8_t* A,
                                        const qp_packed_info* b, const void* packedB_dev,
                                        const int32_t* bias_dev, int64_t max_abs_bias,
                                        const qp_qtensor* out, int32_t relu, void* C, void* ws,
                                        size_t ws_bytes, hipStream_t stream) {
  using namespace qp;
  clear_error();
  QP_REQUIRE(a && b && out, QP_EINVAL, "qgemm: null descriptor");
  QP_REQUIRE(a->dtype == QP_S8 && a->rank == 2, QP_EINVAL, "qgemm: A must be rank-2 QP_S8");
  QP_REQUIRE(a->scheme == QP_PER_TENSOR, QP_EUNSUPPORTED, "qgemm: A must be per-tensor");
  QP_REQUIRE(a->stride[1] == 1, QP_EUNSUPPORTED, "qgemm: A must be K-contiguous (stride[1] == 1)");
  QP_REQUIRE(a->rounding == QP_ROUND_HALF_EVEN, QP_EUNSUPPORTED,
             "qgemm: only round-half-to-even is implemented");
  const int64_t M = a->shape[0], K = a->shape[1], lda = a->stride[0];
  QP_REQUIRE(M >= 0 && K > 0 && lda >= K, QP_EINVAL, "qgemm: bad A shape/stride");
  bool out32 = false;
  qp_status st = validate_gemm(b, K, a->scale, a->zero_point, bias_dev, max_abs_bias, out, &out32);
  if (st) return st;
  QP_REQUIRE(out->rank == 2 && out->shape[0] == M && out->shape[1] == b->N, QP_EINVAL,
             "qgemm: output shape must be [M, N] = [%lld, %lld]", (long long)M, (long long)b->N);
  QP_REQUIRE(out->stride[1] == 1 && out->stride[0] >= b->N, QP_EINVAL,
             "qgemm: output must be row-major with ldc >= N");
  QP_REQUIRE(M == 0 || (A && packedB_dev && C), QP_EINVAL, "qgemm: null data pointer");
  return run_gemm_s8(A, M, lda, a->scale, a->zero_point, b, packedB_dev, bias_dev, out->scale,
                     out->zero_point, out32, relu, C, out->stride[0], ws, ws_bytes, false, stream,
                     nullptr);
}

extern "C" qp_status qgemm_s8s8_dequant_f32(const qp_qtensor* a, const int8_t* A,
                                            const qp_packed_info* b, const void* packedB_dev,
                                            const float* bias_dev, float clamp_lo,
                                            float clamp_hi, float* Y, int64_t ldy, void* ws,
                                            size_t ws_bytes, hipStream_t stream) {
  using namespace qp;
  clear_error();
  QP_REQUIRE(a && b, QP_EINVAL, "qgemm_f32: null descriptor");
  QP_REQUIRE(a->dtype == QP_S8 && a->rank == 2, QP_EINVAL, "qgemm_f32: A must be rank-2 QP_S8");
  QP_REQUIRE(a->scheme == QP_PER_TENSOR, QP_EUNSUPPORTED, "qgemm_f32: A must be per-tensor");
  QP_REQUIRE(a->stride[1] == 1, QP_EUNSUPPORTED,
             "qgemm_f32: A must be K-contiguous (stride[1] == 1)");
  QP_REQUIRE(a->rounding == QP_ROUND_HALF_EVEN, QP_EUNSUPPORTED,
             "qgemm_f32: only round-half-to-even is implemented");
  const int64_t M = a->shape[0], K = a->shape[1], lda = a->stride[0];
  QP_REQUIRE(M >= 0 && K > 0 && lda >= K, QP_EINVAL, "qgemm_f32: bad A shape/stride");
  QP_REQUIRE(b->format == 1, QP_EINVAL, "qgemm_f32: weights must be an int8 blob");
  QP_REQUIRE(K == b->K, QP_EINVAL, "qgemm_f32: activation K=%lld but the weights have K=%lld",
             (long long)K, (long long)b->K);
  QP_REQUIRE(a->zero_point >= -128 && a->zero_point <= 127, QP_EINVAL,
             "qgemm_f32: activation zero point outside int8");
  QP_REQUIRE(std::isfinite(a->scale) && a->scale > 0, QP_EINVAL,
             "qgemm_f32: activation scale must be > 0");
  QP_REQUIRE(K <= INT64_C(2147483647) / 65025, QP_EOVERFLOW,
             "qgemm_f32: K*65025 = %lld exceeds INT32", (long long)(K * 65025));
  QP_REQUIRE(!(clamp_lo > clamp_hi) && !std::isnan(clamp_lo) && !std::isnan(clamp_hi), QP_EINVAL,
             "qgemm_f32: clamp bounds must satisfy lo <= hi");
  QP_REQUIRE(ldy >= b->N, QP_EINVAL, "qgemm_f32: ldy smaller than N");
  QP_REQUIRE(M == 0 || (A && packedB_dev && Y), QP_EINVAL, "qgemm_f32: null data pointer");
  const GemmF32Out f32{bias_dev, clamp_lo, clamp_hi};
  return run_gemm_s8(A, M, lda, a->scale, a->zero_point, b, packedB_dev, nullptr, 1.0f, 0, true, 0,
                     Y, ldy, ws, ws_bytes, false, stream, &f32);
}
