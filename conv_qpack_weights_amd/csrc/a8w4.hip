// a8w4.hip -- int8 activations x int4 group-32 weights -> f32, with bias and
// clamp: the GEMV (M = 1) and GEMM (M > 1) cores.
//
// pytorch/ao PR #997 "Kleidi 4b blockwise gemv prototype" (the
// matmul_clamp_f32_qai8dxp_qsi4c32p kernels): f32 output with a clamp,
// dynamically quantized per-row int8 activations, signed int4 weights with
// one scale per group of 32 along K, no weight zero points.  MNN
// "ConvInt8TiledExecutor.cpp": the KleidiAI path quantizes the activation
// rows and then runs the matmul with a clamp; across quantization blocks the
// partial sums are accumulated in float; the activation zero point is folded
// with a precomputed weight kernel sum (BatchAsyDynamicQuant), i.e.
//   sum_g sw[n,g] sum_{k in g} (qa-za) q = sum_g sw[n,g] sum_{k in g} qa*q
//                                          - za * wsum[n].
// The sum inside one group of 32 is exact int32; across groups it is f32.
//
// Nibble unpack: the blob stores 4-bit two's complement values, byte 4w+j of
// a 32-K run holding k=8w+j (low nibble) and k=8w+4+j (high nibble).  Masking
// a word with 0xF0F0F0F0 gives the high nibbles as int8 values q*16, and
// shifting left by 4 first gives the low ones, so the signed dot4
// (v_dot4_i32_i8) and the int8 MFMA consume them with no sign fix-up; the
// factor 16 is removed exactly (a power of two) in the epilogue.
#include <cstring>

#include "qp_internal.hpp"
#include "quant_row.hpp"

#pragma clang fp contract(off)

namespace qp {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t nib_lo16(uint32_t w) { return (w << 4) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t nib_hi16(uint32_t w) { return w & 0xF0F0F0F0u; }

// 16 * sum over one 32-K run of qa*q.  a0/a1: the 32 activation bytes.
__device__ __forceinline__ int32_t run_dot16(uint4 w, uint4 a0, uint4 a1) {
  int32_t d = 0;
  d = __builtin_amdgcn_sdot4((int)a0.x, (int)nib_lo16(w.x), d, false);
  d = __builtin_amdgcn_sdot4((int)a0.y, (int)nib_hi16(w.x), d, false);
  d = __builtin_amdgcn_sdot4((int)a0.z, (int)nib_lo16(w.y), d, false);
  d = __builtin_amdgcn_sdot4((int)a0.w, (int)nib_hi16(w.y), d, false);
  d = __builtin_amdgcn_sdot4((int)a1.x, (int)nib_lo16(w.z), d, false);
  d = __builtin_amdgcn_sdot4((int)a1.y, (int)nib_hi16(w.z), d, false);
  d = __builtin_amdgcn_sdot4((int)a1.z, (int)nib_lo16(w.w), d, false);
  d = __builtin_amdgcn_sdot4((int)a1.w, (int)nib_hi16(w.w), d, false);
  return d;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ float finish(float S16, float sa, int32_t za, float wsum, float bias,
                                        float lo, float hi) {
  // y = sa * (S16/16) - (sa*za) * wsum + bias, then clamp
  float p = sa * (S16 * 0.0625f);
  float z = (sa * (float)za) * wsum;
  float y = (p - z) + bias;
  y = y < lo ? lo : y;
  y = y > hi ? hi : y;
  return y;
}

struct W4 {
  const uint8_t* data;   // [Npad][Kpad/2]
  const float* scale;    // [Npad][G]
  const float* wsum;     // [Npad]
  int64_t N, Npad, Kpad, G;
};

// ---- GEMV: one wave per RPW output channels, lanes split K by 32-K runs ----
// kFused: the workgroup quantizes the single f32 activation row itself (into
// LDS) with the same device steps as qquantize_rows_s8, after issuing its
// first weight loads.
template <int RPW, bool kFused>
__global__ __launch_bounds__(256) void a8w4_gemv_kernel(const float* __restrict__ X, int64_t K,
                                                        const int8_t* __restrict__ qa_g,
                                                        int64_t lda, const float* __restrict__ sa_g,
                                                        const int32_t* __restrict__ za_g,
                                                        int64_t M, W4 w,
                                                        const float* __restrict__ bias, float lo,
                                                        float hi, float* __restrict__ Y,
                                                        int64_t ldy) {
  extern __shared__ __attribute__((aligned(16))) int8_t qa_lds[];
  __shared__ float red_min[4], red_max[4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t nbase = ((int64_t)blockIdx.x * 4 + wave) * RPW;  // < Npad by grid sizing
  const int64_t runs = w.Kpad / 32;
  const int64_t rowbytes = w.Kpad / 2;
  constexpr int U = 2;  // runs per lane per batch

  for (int64_t m = 0; m < M; ++m) {
    float part[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) part[i] = 0.0f;
    float sa;
    int32_t za;
    const int8_t* qa;
    for (int64_t r0 = 0; r0 < runs; r0 += 64 * U) {
      uint4 wv[U][RPW];
      float sv[U][RPW];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t r = r0 + u * 64 + lane;
        const int64_t rr = r < runs ? r : runs - 1;
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
          wv[u][i] = *reinterpret_cast<const uint4*>(w.data + (nbase + i) * rowbytes + rr * 16);
          sv[u][i] = r < runs ? w.scale[(nbase + i) * w.G + rr] : 0.0f;
        }
      }
      if (r0 == 0) {
        if constexpr (kFused) {
          float s;
          int32_t z;
          row_params_block(X + m * K, K, red_min, red_max, &s, &z);
          quantize_row_block(X + m * K, K, w.Kpad, s, z, qa_lds);
          __syncthreads();
          sa = s;
          za = z;
          qa = qa_lds;
        } else {
          sa = sa_g[m];
          za = za_g[m];
          qa = qa_g + m * lda;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t r = r0 + u * 64 + lane;
        const int64_t rr = r < runs ? r : runs - 1;
        const uint4 a0 = *reinterpret_cast<const uint4*>(qa + rr * 32);
        const uint4 a1 = *reinterpret_cast<const uint4*>(qa + rr * 32 + 16);
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
          const int32_t d = run_dot16(wv[u][i], a0, a1);
          part[i] = part[i] + sv[u][i] * (float)d;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const float S = wave_sum(part[i]);
      const int64_t n = nbase + i;
      if (lane == i && n < w.N)
        Y[m * ldy + n] = finish(S, sa, za, w.wsum[n], bias ? bias[n] : 0.0f, lo, hi);
    }
    if constexpr (kFused) __syncthreads();
  }
}

// ---- GEMM: MFMA 16x16x32 per 32-K group, f32 rescale per group ----------
// Workgroup = 4 waves; wave v owns output channels n0 + 16v .. +16 and
// FM*16 rows of M.  The MFMA is issued as (weights, activations), so a lane
// holds channels 4*(lane/16)+i of row lane%16.  Per group the lane needs
// word (lane/16) of the channel's 16-byte run: 8 nibbles = k 8w..8w+7, which
// unpack to the MFMA's 8-byte operand; its activation operand is the 8 bytes
// qa[m][32g + 8w ..].
template <int FM>
__global__ __launch_bounds__(256) void a8w4_gemm_kernel(const int8_t* __restrict__ qa,
                                                        int64_t lda, const float* __restrict__ sa_g,
                                                        const int32_t* __restrict__ za_g,
                                                        int64_t M, W4 w,
                                                        const float* __restrict__ bias, float lo,
                                                        float hi, float* __restrict__ Y,
                                                        int64_t ldy) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * 64 + wave * 16;
  const int64_t mbase = (int64_t)blockIdx.y * 16 * FM;
  const int wq = lane >> 4;
  const int64_t nrow = n0 + (lane & 15);  // weight row this lane feeds
  const int64_t rowbytes = w.Kpad / 2;
  const uint32_t* wsrc = reinterpret_cast<const uint32_t*>(w.data + nrow * rowbytes) + wq;
  int64_t arow[FM];
#pragma unroll
  for (int f = 0; f < FM; ++f) {
    int64_t m = mbase + f * 16 + (lane & 15);
    arow[f] = m < M ? m : M - 1;
  }
  float acc[FM][4];
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[f][i] = 0.0f;
  const float* srow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) srow[i] = w.scale + (n0 + 4 * wq + i) * w.G;

  for (int64_t g = 0; g < w.G; ++g) {
    const uint32_t wword = wsrc[g * 4];
    const long bop = (long)(((uint64_t)nib_hi16(wword) << 32) | nib_lo16(wword));
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = srow[i][g];
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      const long aop = *reinterpret_cast<const long*>(qa + arow[f] * lda + g * 32 + wq * 8);
      v4i d = __builtin_amdgcn_mfma_i32_16x16x32_i8(bop, aop, v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[f][i] = acc[f][i] + sc[i] * (float)d[i];
    }
  }
#pragma unroll
  for (int f = 0; f < FM; ++f) {
    const int64_t m = mbase + f * 16 + (lane & 15);
    if (m >= M) continue;
    const float sa = sa_g[m];
    const int32_t za = za_g[m];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t n = n0 + 4 * wq + i;
      if (n < w.N)
        Y[m * ldy + n] = finish(acc[f][i], sa, za, w.wsum[n], bias ? bias[n] : 0.0f, lo, hi);
    }
  }
}

W4 w4_of(const qp_packed_info* b, const void* blob) {
  const uint8_t* p = static_cast<const uint8_t*>(blob);
  return W4{p + b->data_off, reinterpret_cast<const float*>(p + b->scale_off),
            reinterpret_cast<const float*>(p + b->sum_off), b->N, b->Npad, b->Kpad,
            b->Kpad / b->group};
}

qp_status validate_w4(const qp_packed_info* b, int64_t K) {
  QP_REQUIRE(b && b->format == 2, QP_EINVAL, "a8w4: weights must be an int4 blob");
  QP_REQUIRE(b->group == 32, QP_EUNSUPPORTED, "a8w4: group size %lld not implemented (32 only)",
             (long long)b->group);
  QP_REQUIRE(K == b->K, QP_EINVAL, "a8w4: activation K=%lld but the weights have K=%lld",
             (long long)K, (long long)b->K);
  return QP_OK;
}

qp_status launch_gemv(const float* X, int64_t K, const int8_t* qa, int64_t lda,
                      const float* sa, const int32_t* za, int64_t M, const W4& w,
                      const float* bias, float lo, float hi, float* Y, int64_t ldy, bool fused,
                      hipStream_t stream) {
  constexpr int RPW = 4;
  const unsigned blocks = (unsigned)ceil_div(w.N, 4 * RPW);
  const size_t lds = fused ? (size_t)w.Kpad : 0;
  if (fused)
    hipLaunchKernelGGL((a8w4_gemv_kernel<RPW, true>), dim3(blocks), dim3(256), lds, stream, X, K,
                       qa, lda, sa, za, M, w, bias, lo, hi, Y, ldy);
  else
    hipLaunchKernelGGL((a8w4_gemv_kernel<RPW, false>), dim3(blocks), dim3(256), lds, stream, X, K,
                       qa, lda, sa, za, M, w, bias, lo, hi, Y, ldy);
  return check_launch("a8w4 gemv");
}

qp_status launch_gemm(const int8_t* qa, int64_t lda, const float* sa, const int32_t* za,
                      int64_t M, const W4& w, const float* bias, float lo, float hi, float* Y,
                      int64_t ldy, hipStream_t stream) {
  const unsigned bx = (unsigned)ceil_div(w.N, 64);
  if (M <= 16) {
    hipLaunchKernelGGL(a8w4_gemm_kernel<1>, dim3(bx, 1), dim3(256), 0, stream, qa, lda, sa, za, M,
                       w, bias, lo, hi, Y, ldy);
  } else {
    const unsigned by = (unsigned)ceil_div(M, 64);
    hipLaunchKernelGGL(a8w4_gemm_kernel<4>, dim3(bx, by), dim3(256), 0, stream, qa, lda, sa, za, M,
                       w, bias, lo, hi, Y, ldy);
  }
  return check_launch("a8w4 gemm");
}

}  // namespace
}  // namespace qp

extern "C" qp_status qgemm_a8w4_blockwise_f32_ws_size(int64_t M, const qp_packed_info* w,
                                                      size_t* bytes) {
  using namespace qp;
  QP_REQUIRE(w && bytes && M >= 0, QP_EINVAL, "qgemm_a8w4_blockwise_f32_ws_size: bad argument");
  *bytes = M <= 1 ? 0 : (size_t)(round_up(M * w->Kpad, 256) + round_up(8 * M, 256));
  return QP_OK;
}

extern "C" qp_status qgemm_a8w4_blockwise_f32(const float* X, int64_t M, int64_t K, int64_t ldx,
                                              const qp_packed_info* w, const void* packedW_dev,
                                              const float* bias, float clamp_lo, float clamp_hi,
                                              float* Y, int64_t ldy, void* ws, size_t ws_bytes,
                                              hipStream_t stream) {
  using namespace qp;
  clear_error();
  qp_status st = validate_w4(w, K);
  if (st) return st;
  QP_REQUIRE(M >= 0 && ldx >= K && ldy >= w->N, QP_EINVAL, "a8w4: bad M/ldx/ldy");
  QP_REQUIRE(!(clamp_lo > clamp_hi), QP_EINVAL, "a8w4: clamp_lo > clamp_hi");
  if (M == 0) return QP_OK;
  QP_REQUIRE(X && packedW_dev && Y, QP_EINVAL, "a8w4: null data pointer");
  const W4 wv = w4_of(w, packedW_dev);
  if (M == 1)
    return launch_gemv(X, K, nullptr, 0, nullptr, nullptr, 1, wv, bias, clamp_lo, clamp_hi, Y, ldy,
                       true, stream);
  size_t need = 0;
  qgemm_a8w4_blockwise_f32_ws_size(M, w, &need);
  QP_REQUIRE(ws_bytes >= need, QP_ESIZE, "a8w4: workspace holds %zu bytes, needs %zu", ws_bytes,
             need);
  QP_REQUIRE(ws && ((uintptr_t)ws % 256) == 0, QP_EALIGN,
             "a8w4: workspace must be non-null and 256-byte aligned");
  uint8_t* p = static_cast<uint8_t*>(ws);
  int8_t* qa = reinterpret_cast<int8_t*>(p);
  float* sa = reinterpret_cast<float*>(p + round_up(M * w->Kpad, 256));
  int32_t* za = reinterpret_cast<int32_t*>(sa + M);
  st = launch_quantize_rows(X, M, K, ldx, qa, w->Kpad, w->Kpad, sa, za, stream);
  if (st) return st;
  return launch_gemm(qa, w->Kpad, sa, za, M, wv, bias, clamp_lo, clamp_hi, Y, ldy, stream);
}

extern "C" qp_status qgemm_a8w4_prequant_f32(const int8_t* qa, int64_t M, int64_t lda,
                                             const float* sa, const int32_t* za,
                                             const qp_packed_info* w, const void* packedW_dev,
                                             const float* bias, float clamp_lo, float clamp_hi,
                                             float* Y, int64_t ldy, hipStream_t stream) {
  using namespace qp;
  clear_error();
  qp_status st = validate_w4(w, w ? w->K : 0);
  if (st) return st;
  QP_REQUIRE(M >= 0 && lda >= w->Kpad && lda % 16 == 0 && ldy >= w->N, QP_EINVAL,
             "a8w4: lda must be >= Kpad and a multiple of 16; ldy >= N");
  QP_REQUIRE(!(clamp_lo > clamp_hi), QP_EINVAL, "a8w4: clamp_lo > clamp_hi");
  if (M == 0) return QP_OK;
  QP_REQUIRE(qa && sa && za && packedW_dev && Y, QP_EINVAL, "a8w4: null data pointer");
  QP_REQUIRE(((uintptr_t)qa % 16) == 0, QP_EALIGN, "a8w4: qa must be 16-byte aligned");
  const W4 wv = w4_of(w, packedW_dev);
  if (M <= 4)
    return launch_gemv(nullptr, w->K, qa, lda, sa, za, M, wv, bias, clamp_lo, clamp_hi, Y, ldy,
                       false, stream);
  return launch_gemm(qa, lda, sa, za, M, wv, bias, clamp_lo, clamp_hi, Y, ldy, stream);
}
