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
// Nibble unpack: the blob stores 4-bit two's complement values; in each
// 128-K block, the word at byte 16c + 4t holds k = 32t + 8c + j (low nibble
// of byte j) and k = 32t + 8c + 4 + j (high nibble).  Masking a word with
// 0xF0F0F0F0 gives the high nibbles as int8 values q*16, and shifting left
// by 4 first gives the low ones, so the signed dot4 (v_dot4_i32_i8) and the
// int8 MFMA consume them with no sign fix-up; the factor 16 is removed
// exactly (a power of two) in the epilogue.  One 16-byte load (chunk c of a
// block) carries the same 8 K of four consecutive groups.
#include <cstring>

#include "qp_internal.hpp"
#include "quant_row.hpp"

#pragma clang fp contract(off)

namespace qp {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t nib_lo16(uint32_t w) { return (w << 4) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t nib_hi16(uint32_t w) { return w & 0xF0F0F0F0u; }

// 16 * sum over the 8 K of one word: a0 holds qa for the word's low nibbles
// (k..k+3), a1 for its high nibbles (k+4..k+7).
__device__ __forceinline__ int32_t word_dot16(uint32_t w, uint32_t a0, uint32_t a1) {
  int32_t d = __builtin_amdgcn_sdot4((int)a0, (int)nib_lo16(w), 0, false);
  return __builtin_amdgcn_sdot4((int)a1, (int)nib_hi16(w), d, false);
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

// ---- GEMV: one wave per RPW output channels, lanes split K by 16-byte chunks ----
// Chunk h of a row is the 8-K piece c = h%4 of the four groups 4(h/4)..+3.
// All of a lane's weight chunks and scales are requested first; while they
// are in flight the workgroup quantizes the activation row (kFused, M = 1:
// the same device steps as qquantize_rows_s8) into LDS, permuted so that
// the 32 activation bytes of a chunk are contiguous; otherwise it reads the
// quantized rows from memory.  Lane partial sums are reduced with DPP in a
// fixed order.
template <int NT, int RPW, bool kFused>
__global__ __launch_bounds__(NT) void a8w4_gemv_kernel(const float* __restrict__ X, int64_t K,
                                                       const int8_t* __restrict__ qa_g,
                                                       int64_t lda, const float* __restrict__ sa_g,
                                                       const int32_t* __restrict__ za_g,
                                                       int64_t M, W4 w,
                                                       const float* __restrict__ bias, float lo,
                                                       float hi, float* __restrict__ Y,
                                                       int64_t ldy) {
  constexpr int NW = NT / 64;
  extern __shared__ __attribute__((aligned(16))) int8_t qa_lds[];
  __shared__ float red[2 * NW];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t nbase = ((int64_t)blockIdx.x * NW + wave) * RPW;  // < Npad by grid sizing
  const int64_t chunks = w.Kpad / 32;
  const int64_t rowbytes = w.Kpad / 2;
  constexpr int U = 2;  // chunks per lane per batch

  for (int64_t m = 0; m < M; ++m) {
    float part[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) part[i] = 0.0f;
    float sa = 0.0f;
    int32_t za = 0;
    for (int64_t h0 = 0; h0 < chunks; h0 += 64 * U) {
      uint4 wv[U][RPW];
      float4 sv[U][RPW];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t h = h0 + u * 64 + lane;
        const bool live = h < chunks;
        const int64_t hh = live ? h : chunks - 1;
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
          wv[u][i] = *reinterpret_cast<const uint4*>(w.data + (nbase + i) * rowbytes + hh * 16);
          const float4 s4 =
              *reinterpret_cast<const float4*>(w.scale + (nbase + i) * w.G + (hh >> 2) * 4);
          sv[u][i] = live ? s4 : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
      if (h0 == 0) {
        if constexpr (kFused) {
          const float* xr = X + m * K;
          quantize_row_wg<NT, true>(xr, K, w.Kpad, (((uintptr_t)xr) & 15) == 0, true, qa_lds,
                                    red, &sa, &za);
          __syncthreads();
        } else {
          sa = sa_g[m];
          za = za_g[m];
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t h = h0 + u * 64 + lane;
        const int64_t hh = h < chunks ? h : chunks - 1;
        uint2 a[4];
        if constexpr (kFused) {
          const int8_t* ab = qa_lds + (hh >> 2) * 128 + (hh & 3) * 32;
          const uint4 p0 = *reinterpret_cast<const uint4*>(ab);
          const uint4 p1 = *reinterpret_cast<const uint4*>(ab + 16);
          a[0] = make_uint2(p0.x, p0.y);
          a[1] = make_uint2(p0.z, p0.w);
          a[2] = make_uint2(p1.x, p1.y);
          a[3] = make_uint2(p1.z, p1.w);
        } else {
          const int8_t* ab = qa_g + m * lda + (hh >> 2) * 128 + (hh & 3) * 8;
#pragma unroll
          for (int t = 0; t < 4; ++t) a[t] = *reinterpret_cast<const uint2*>(ab + 32 * t);
        }
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
          const uint4 wq = wv[u][i];
          const float d0 = (float)word_dot16(wq.x, a[0].x, a[0].y);
          const float d1 = (float)word_dot16(wq.y, a[1].x, a[1].y);
          const float d2 = (float)word_dot16(wq.z, a[2].x, a[2].y);
          const float d3 = (float)word_dot16(wq.w, a[3].x, a[3].y);
          part[i] = part[i] + sv[u][i].x * d0;
          part[i] = part[i] + sv[u][i].y * d1;
          part[i] = part[i] + sv[u][i].z * d2;
          part[i] = part[i] + sv[u][i].w * d3;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const float S = wave_reduce(part[i], AddOp{});
      const int64_t n = nbase + i;
      if (lane == i && n < w.N)
        Y[m * ldy + n] = finish(S, sa, za, w.wsum[n], bias ? bias[n] : 0.0f, lo, hi);
    }
    if constexpr (kFused) __syncthreads();
  }
}

// ---- GEMM: MFMA 16x16x32 per 32-K group, f32 rescale per group ----------
// A workgroup owns 16 output channels and FM*16 rows of M; its 4 waves split
// the 128-K blocks of K in four contiguous ranges and their f32 partial sums
// are added in wave order through LDS.  The MFMA is issued as (weights,
// activations), so a lane holds channels 4*(lane/16)+i of row lane%16.  Lane
// (row lane%16, c = lane/16) loads chunk c of a block: the 8-K piece c of
// four groups, each unpacked to an 8-byte MFMA operand; the activation
// operand of group t is qa[m][128b + 32t + 8c ..+8].  Loads for the next
// block are issued before the current block is computed.
template <int FM>
__global__ __launch_bounds__(256) void a8w4_gemm_kernel(const int8_t* __restrict__ qa,
                                                        int64_t lda, const float* __restrict__ sa_g,
                                                        const int32_t* __restrict__ za_g,
                                                        int64_t M, W4 w,
                                                        const float* __restrict__ bias, float lo,
                                                        float hi, float* __restrict__ Y,
                                                        int64_t ldy) {
  __shared__ float red[3][FM][4][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t mbase = (int64_t)blockIdx.y * 16 * FM;
  const int c = lane >> 4;
  const int64_t rowbytes = w.Kpad / 2;
  const int8_t* wsrc = reinterpret_cast<const int8_t*>(w.data) + (n0 + (lane & 15)) * rowbytes + 16 * c;
  const int8_t* arow[FM];
#pragma unroll
  for (int f = 0; f < FM; ++f) {
    const int64_t m = mbase + f * 16 + (lane & 15);
    arow[f] = qa + (m < M ? m : M - 1) * lda + 8 * c;
  }
  const float* srow = w.scale + (n0 + 4 * c) * w.G;  // + i*G for channel 4c+i
  const int64_t nblocks = w.Kpad / 128;
  const int64_t bpw = (nblocks + 3) / 4;
  const int64_t b_begin = wave * bpw;
  const int64_t b_end = b_begin + bpw < nblocks ? b_begin + bpw : nblocks;

  float acc[FM][4];
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[f][i] = 0.0f;

  uint4 wd;
  float4 sc[4];
  uint2 av[FM][4];
  auto load = [&](int64_t b) {
    wd = *reinterpret_cast<const uint4*>(wsrc + b * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = *reinterpret_cast<const float4*>(srow + i * w.G + 4 * b);
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        av[f][t] = *reinterpret_cast<const uint2*>(arow[f] + b * 128 + 32 * t);
  };
  if (b_begin < b_end) load(b_begin);
  for (int64_t b = b_begin; b < b_end; ++b) {
    const uint4 cw = wd;
    float4 cs[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) cs[i] = sc[i];
    uint2 ca[FM][4];
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int t = 0; t < 4; ++t) ca[f][t] = av[f][t];
    if (b + 1 < b_end) load(b + 1);
    const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const long bop = (long)(((uint64_t)nib_hi16(words[t]) << 32) | nib_lo16(words[t]));
      const float s_t[4] = {t == 0 ? cs[0].x : t == 1 ? cs[0].y : t == 2 ? cs[0].z : cs[0].w,
                            t == 0 ? cs[1].x : t == 1 ? cs[1].y : t == 2 ? cs[1].z : cs[1].w,
                            t == 0 ? cs[2].x : t == 1 ? cs[2].y : t == 2 ? cs[2].z : cs[2].w,
                            t == 0 ? cs[3].x : t == 1 ? cs[3].y : t == 2 ? cs[3].z : cs[3].w};
#pragma unroll
      for (int f = 0; f < FM; ++f) {
        const long aop = (long)(((uint64_t)ca[f][t].y << 32) | ca[f][t].x);
        const v4i d = __builtin_amdgcn_mfma_i32_16x16x32_i8(bop, aop, v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[f][i] = acc[f][i] + s_t[i] * (float)d[i];
      }
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave - 1][f][i][lane] = acc[f][i];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int f = 0; f < FM; ++f) {
    const int64_t m = mbase + f * 16 + (lane & 15);
    if (m >= M) continue;
    const float sa = sa_g[m];
    const int32_t za = za_g[m];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float S = ((acc[f][i] + red[0][f][i][lane]) + red[1][f][i][lane]) + red[2][f][i][lane];
      const int64_t n = n0 + 4 * c + i;
      if (n < w.N) Y[m * ldy + n] = finish(S, sa, za, w.wsum[n], bias ? bias[n] : 0.0f, lo, hi);
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

template <int NT, int RPW>
qp_status launch_gemv_cfg(const float* X, int64_t K, const int8_t* qa, int64_t lda,
                          const float* sa, const int32_t* za, int64_t M, const W4& w,
                          const float* bias, float lo, float hi, float* Y, int64_t ldy,
                          bool fused, hipStream_t stream) {
  constexpr int rows_per_block = (NT / 64) * RPW;
  static_assert(64 % rows_per_block == 0, "blocks must tile the 64-row padding");
  const unsigned blocks = (unsigned)ceil_div(w.N, rows_per_block);
  const size_t lds = fused ? (size_t)w.Kpad : 0;
  if (fused)
    hipLaunchKernelGGL((a8w4_gemv_kernel<NT, RPW, true>), dim3(blocks), dim3(NT), lds, stream, X,
                       K, qa, lda, sa, za, M, w, bias, lo, hi, Y, ldy);
  else
    hipLaunchKernelGGL((a8w4_gemv_kernel<NT, RPW, false>), dim3(blocks), dim3(NT), lds, stream, X,
                       K, qa, lda, sa, za, M, w, bias, lo, hi, Y, ldy);
  return check_launch("a8w4 gemv");
}

qp_status launch_gemv(const float* X, int64_t K, const int8_t* qa, int64_t lda,
                      const float* sa, const int32_t* za, int64_t M, const W4& w,
                      const float* bias, float lo, float hi, float* Y, int64_t ldy, bool fused,
                      hipStream_t stream) {
  return launch_gemv_cfg<512, 2>(X, K, qa, lda, sa, za, M, w, bias, lo, hi, Y, ldy, fused, stream);
}

qp_status launch_gemm(const int8_t* qa, int64_t lda, const float* sa, const int32_t* za,
                      int64_t M, const W4& w, const float* bias, float lo, float hi, float* Y,
                      int64_t ldy, hipStream_t stream) {
  const unsigned bx = (unsigned)ceil_div(w.N, 16);
  if (M <= 16) {
    hipLaunchKernelGGL(a8w4_gemm_kernel<1>, dim3(bx, 1), dim3(256), 0, stream, qa, lda, sa, za, M,
                       w, bias, lo, hi, Y, ldy);
  } else if (M <= 64) {
    hipLaunchKernelGGL(a8w4_gemm_kernel<4>, dim3(bx, 1), dim3(256), 0, stream, qa, lda, sa, za, M,
                       w, bias, lo, hi, Y, ldy);
  } else {
    const unsigned by = (unsigned)ceil_div(M, 128);
    hipLaunchKernelGGL(a8w4_gemm_kernel<8>, dim3(bx, by), dim3(256), 0, stream, qa, lda, sa, za, M,
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
