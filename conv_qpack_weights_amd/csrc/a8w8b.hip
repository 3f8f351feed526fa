// a8w8b.hip -- int8 activations x block-quantized int8 weights -> f32, with
// bias and clamp.
//
// MNN "ConvInt8TiledExecutor.cpp" (_computeReorderQuantInfo, the dynamic
// quant path of DenseConvInt8TiledExecutor): int8 weights may carry one
// scale per output channel and K block (blockNum > 1); the partial sums of
// each block are exact integers and are accumulated across blocks in
// float, the activation zero point being folded with the weights' kernel
// sum.  Here, for a GEMM (a linear layer or a 1x1 convolution):
//   Y[m,n] = clamp(sa[m] * (sum_b sw[n,b] * sum_{k in b} qa[m,k]*q[n,k]
//                           - za[m] * wsum[n]) + bias[n], lo, hi),
//   wsum[n] = sum_b sw[n,b] * sum_{k in b} q[n,k]      (packed, fp64 -> f32)
// with blocks of 64 or 128 K.
//
// Kernel (one 128-K step at a time): the workgroup's activation rows go
// through an LDS ring filled by direct (buffer ... lds) loads of 128-byte
// row pieces, stored with 16-byte chunk p of row r at p ^ ((r >> 1) & 7);
// each wave owns one 16-channel fragment (or, for small M, one of four K
// ranges of it) and reads its weights straight from the blob's 32x32
// sub-tiles into registers, P steps ahead, with the block scales.  Each 64-K
// half of a step is one v_mfma_i32_16x16x64_i8 per 16-row fragment, issued
// as (activations, weights) so a lane holds rows 4*(l/16)+i of channel l%16
// and needs one scale per block.  An int32 block result is rescaled into an
// f32 sum as soon as its block is complete (every half for blocks of 64,
// every step for 128).  The body of every step is the same branch-free code
// (loads past the end are clamped and contribute with zero scales), so one
// constant wait count covers all steps.
#include "dev_util.hpp"
#include "qp_internal.hpp"
#include "quant_row.hpp"

#pragma clang fp contract(off)

namespace qp {
namespace {

struct W8B {
  const int8_t* data;  // 32x32 sub-tiles, [Npad/32][Kpad/32][32][32]
  const float* scale;  // [nblk][Npad]: a block's scales of all channels side by side
  const float* wsum;   // [Npad]
  int64_t N, Npad, Kpad, kblocks, nblk;
};

__device__ __forceinline__ float finish_w8(float S, float sa, int32_t za, float wsum, float bias,
                                           float lo, float hi) {
  const float p = sa * S;
  const float z = (sa * (float)za) * wsum;
  float y = (p - z) + bias;
  y = y < lo ? lo : y;
  y = y > hi ? hi : y;
  return y;
}

template <int FM, int CW, int KS, int BS, int P>
__global__ __launch_bounds__(256) void a8w8b_gemm_kernel(const int8_t* __restrict__ qa,
                                                         int64_t lda,
                                                         const float* __restrict__ sa_g,
                                                         const int32_t* __restrict__ za_g,
                                                         int64_t M, W8B w,
                                                         const float* __restrict__ bias,
                                                         float lo, float hi,
                                                         float* __restrict__ Y, int64_t ldy) {
  static_assert(CW * KS == 4, "four waves");
  static_assert(BS == 64 || BS == 128, "block of 64 or 128 K");
  // P: weight steps in flight
  constexpr int R = 4;                 // activation ring stages
  constexpr int MT = 16 * FM;          // rows per workgroup
  constexpr int SLOTS = KS * MT * 8;   // 16-byte pieces per stage
  constexpr int ND = SLOTS / 256;      // direct loads per thread per stage
  constexpr int STAGE = SLOTS * 16;
  constexpr int NSC = 128 / BS;        // block scales per step
  static_assert(SLOTS % 256 == 0, "a stage must split evenly over the workgroup");
  // One channel fragment split over the four waves' K ranges: each wave
  // loads and reads only its own rows of a stage, no barrier in the loop.
  constexpr bool kPrivA = CW == 1;
  static_assert(!kPrivA || MT * 8 == 64 * ND, "a wave's rows of a stage: ND loads per lane");
  __shared__ __attribute__((aligned(16))) int8_t ring[R * STAGE];
  __shared__ float red[KS > 1 ? (KS - 1) * CW : 1][FM][4][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ks = wave % KS;
  const int cw = wave / KS;
  const int c = lane >> 4;
  const int64_t n0 = ((int64_t)blockIdx.x * CW + cw) * 16;  // n0 + 16 <= Npad
  const int64_t mw = (int64_t)blockIdx.y * MT;
  const int64_t nsteps = w.Kpad / 128;
  const int64_t bpw = (nsteps + KS - 1) / KS;  // steps per K range
  auto range_step = [&](int r, int64_t j) {
    const int64_t b_begin = r * bpw;
    int64_t last = (b_begin + bpw < nsteps ? b_begin + bpw : nsteps) - 1;
    if (last < b_begin) last = nsteps - 1;  // empty range: park on a real step
    const int64_t b = b_begin + j;
    return b < last ? b : last;
  };
  const int64_t my_end = (ks * bpw + bpw < nsteps ? ks * bpw + bpw : nsteps);

  // ---- weights: channel n0 + l%16, 16-byte chunk c of each 64-K half ----
  const int64_t n = n0 + (lane & 15);
  const int8_t* wsrc =
      w.data + ((n >> 5) * w.kblocks + (c >> 1)) * 1024 + (n & 31) * 32 + (c & 1) * 16;
  const float* ssrc = w.scale + n;  // + block * Npad

  // ---- activation direct loads (as the A8W4 GEMM) ----
  const int8_t* const a_base = qa + mw * lda;
  uint32_t a_voff[ND];
  int a_rng[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) {
    const int s = kPrivA ? wave * (MT * 8) + 64 * i + lane : tid + 256 * i;
    const int r = (s >> 3) % MT;
    a_rng[i] = kPrivA ? wave : (32 * i + 8 * wave) / MT;
    const int p = (s & 7) ^ ((r >> 1) & 7);
    int64_t m = mw + r;
    m = m < M ? m : M - 1;
    a_voff[i] = (uint32_t)((m - mw) * lda + 16 * p);
  }
  auto issue_stage = [&](int64_t j) {
    lds_i8* st = (lds_i8*)ring + (int)(j % R) * STAGE;
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      const int64_t b = range_step(a_rng[i], j);
      const int s0 = kPrivA ? wave * (MT * 8) + 64 * i : 256 * i + 64 * wave;  // lane 0's slot
      dma16_to_lds(a_base, (lds_void_t*)(st + s0 * 16), a_voff[i],
                   (uint32_t)(b * 128));
    }
  };

  float acc[2][FM][4];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[h][f][i] = 0.0f;

  v4i wr[P][2];
  float sr[P][NSC];
  auto load_w = [&](int u, int64_t b) {
#pragma unroll
    for (int s = 0; s < 2; ++s) wr[u][s] = *reinterpret_cast<const v4i*>(wsrc + b * 4096 + s * 2048);
#pragma unroll
    for (int s = 0; s < NSC; ++s) sr[u][s] = ssrc[(b * NSC + s) * w.Npad];
  };

  auto step = [&](int u, int64_t j) {
    const lds_i8* st = (const lds_i8*)ring + (int)(j % R) * STAGE + ks * MT * 128;
    v4i af[FM][2];
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      const int r = f * 16 + (lane & 15);
      const int sw = (r >> 1) & 7;
#pragma unroll
      for (int s = 0; s < 2; ++s)
        af[f][s] = *reinterpret_cast<const __attribute__((address_space(3))) v4i*>(
            st + r * 128 + 16 * ((4 * s + c) ^ sw));
    }
    const bool live = ks * bpw + j < my_end;
    v4i cw2[2];
    float cs[NSC];
#pragma unroll
    for (int s = 0; s < 2; ++s) cw2[s] = wr[u][s];
#pragma unroll
    for (int s = 0; s < NSC; ++s) cs[s] = live ? sr[u][s] : 0.0f;
    load_w(u, range_step(ks, j + P));
    v4i d[2][FM];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int f = 0; f < FM; ++f)
        d[s][f] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[f][s], cw2[s], v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (BS == 64) {
          acc[0][f][i] = __builtin_fmaf(cs[0], (float)d[0][f][i], acc[0][f][i]);
          acc[1][f][i] = __builtin_fmaf(cs[NSC - 1], (float)d[1][f][i], acc[1][f][i]);
        } else {
          acc[0][f][i] = __builtin_fmaf(cs[0], (float)(d[0][f][i] + d[1][f][i]), acc[0][f][i]);
        }
      }
  };

  // ---- prologue: stages 0..R-2 and the weights of steps 0..P-1, drained ----
#pragma unroll
  for (int j = 0; j < R - 1; ++j) issue_stage(j);
#pragma unroll
  for (int u = 0; u < P; ++u) load_w(u, range_step(ks, u));
  // The epilogue operands of the waves that write (K range 0) come in with
  // the prologue, which is drained anyway: loaded after the last barrier
  // they would put a memory round trip (the weight sums live in the cold
  // blob) between the final sums and the stores.  Unconditional loads
  // (clamped indices, a stand-in array where there is no bias).
  float ws_e = 0.0f, bn_e = 0.0f, sa_e[FM][4];
  int32_t za_e[FM][4];
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sa_e[f][i] = 0.0f;
      za_e[f][i] = 0;
    }
  if (ks == 0) {
    const int64_t nc = n < w.N ? n : w.N - 1;
    ws_e = w.wsum[nc];
    bn_e = (bias ? bias : w.wsum)[nc];
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = mw + f * 16 + 4 * c + i;
        const int64_t mc = m < M ? m : M - 1;
        sa_e[f][i] = sa_g[mc];
        za_e[f][i] = za_g[mc];
      }
  }
  wait_vmcnt<0>();
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)

  // Loads issued after stage j+1's direct loads in the steady state: the
  // weight refill of step j+2-R and R-2 whole steps.
  constexpr int LW = 2 + NSC;
  constexpr int A_WAIT = LW + (R - 2) * (ND + LW);
  static_assert(A_WAIT < 64, "vmcnt range");
  for (int64_t j0 = 0; j0 < bpw; j0 += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const int64_t j = j0 + u;
      wait_vmcnt<A_WAIT>();
      if constexpr (!kPrivA) asm volatile("s_barrier" ::: "memory");
      issue_stage(j + R - 1);
      step(u, j);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  wait_vmcnt<0>();

  float out[FM][4];
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int i = 0; i < 4; ++i) out[f][i] = acc[0][f][i] + acc[1][f][i];
  if constexpr (KS > 1) {
    if (ks > 0) {
#pragma unroll
      for (int f = 0; f < FM; ++f)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[cw * (KS - 1) + ks - 1][f][i][lane] = out[f][i];
    }
    __syncthreads();
    if (ks != 0) return;
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < KS - 1; ++r) out[f][i] = out[f][i] + red[cw * (KS - 1) + r][f][i][lane];
  }
  if (n >= w.N) return;
  const float bn = bias ? bn_e : 0.0f;
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = mw + f * 16 + 4 * c + i;
      if (m < M) Y[m * ldy + n] = finish_w8(out[f][i], sa_e[f][i], za_e[f][i], ws_e, bn, lo, hi);
    }
}

// ---- GEMV (M = 1) with the row's dynamic quantization --------------------
// One workgroup per 16-channel fragment and two kinds of waves, as in the
// A8W4 GEMV: four quantizer waves load the f32 row (bounded, branch-free
// loads) and quantize it with the steps of qquantize_rows_s8 into LDS; four
// weight waves, one K range each, put the weight and scale loads of their
// first P steps in flight before anything waits.  Loads complete in issue
// order within a wave, so with the two jobs in different waves neither
// waits behind the other.  The steps are those of a8w8b_gemm_kernel, with
// the row's codes read from LDS as row 0 of the MFMA tile (rows 1..15 are
// zero); the four K ranges are summed in a fixed order.
template <int BS, int P>
__global__ __launch_bounds__(512) void a8w8b_gemv_fused_kernel(const float* __restrict__ X,
                                                               int64_t K, W8B w,
                                                               const float* __restrict__ bias,
                                                               float lo, float hi,
                                                               float* __restrict__ Y) {
  static_assert(BS == 64 || BS == 128, "block of 64 or 128 K");
  constexpr int NQ = 4, QT = NQ * 64, QE = 16;  // quantizer waves, threads, values a pass
  constexpr int KS = 4;                         // weight waves: K ranges
  constexpr int NSC = 128 / BS;                 // block scales per step
  extern __shared__ __attribute__((aligned(16))) int8_t qa_lds[];  // [Kpad] codes
  __shared__ float red[2 * NQ];
  __shared__ float part[KS - 1][4][64];
  __shared__ float row_param[2];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (wave < NQ) {
    const bool xvec = (((uintptr_t)X) & 15) == 0;
    const RowFirst xf = quantize_row_first<QT, QE>(X, K, xvec);
    // one pass of whole vectors (e.g. K = 4096) runs without the loops and
    // fallbacks of the general case
    const bool one = xvec && K == (int64_t)QT * QE && w.Kpad == K;
    float4 first[4];
    if (one)
      row_extremes_partial<QT, QE, false, true>(X, K, xvec, red, first, &xf);
    else
      row_extremes_partial<QT, QE, false>(X, K, xvec, red, first, &xf);
    __syncthreads();  // (1) the waves' extremes
    float s;
    int32_t z;
    row_params<QT, false>(red, &s, &z);
    if (tid == 0) {
      row_param[0] = s;
      row_param[1] = __builtin_bit_cast(float, z);
    }
    if (one)
      row_codes<QT, QE, false, false, true>(X, K, w.Kpad, xvec, true, qa_lds, s, z, first);
    else
      row_codes<QT, QE, false, false>(X, K, w.Kpad, xvec, true, qa_lds, s, z, first);
    __syncthreads();  // (2) the codes
    __syncthreads();  // (3) the K ranges' partial sums
    return;
  }
  const int ks = wave - NQ;
  const int c = lane >> 4;
  const int64_t n = (int64_t)blockIdx.x * 16 + (lane & 15);  // < Npad
  const int64_t nsteps = w.Kpad / 128;
  const int64_t bpw = (nsteps + KS - 1) / KS;  // steps per K range
  auto range_step = [&](int64_t j) {
    const int64_t b_begin = ks * bpw;
    int64_t last = (b_begin + bpw < nsteps ? b_begin + bpw : nsteps) - 1;
    if (last < b_begin) last = nsteps - 1;  // empty range: park on a real step
    const int64_t b = b_begin + j;
    return b < last ? b : last;
  };
  const int64_t my_end = (ks * bpw + bpw < nsteps ? ks * bpw + bpw : nsteps);
  const int8_t* wsrc =
      w.data + ((n >> 5) * w.kblocks + (c >> 1)) * 1024 + (n & 31) * 32 + (c & 1) * 16;
  const float* ssrc = w.scale + n;  // + block * Npad
  v4i wr[P][2];
  float sr[P][NSC];
  auto load_w = [&](int u, int64_t b) {
#pragma unroll
    for (int h = 0; h < 2; ++h) wr[u][h] = *reinterpret_cast<const v4i*>(wsrc + b * 4096 + h * 2048);
#pragma unroll
    for (int h = 0; h < NSC; ++h) sr[u][h] = ssrc[(b * NSC + h) * w.Npad];
  };
#pragma unroll
  for (int u = 0; u < P; ++u) load_w(u, range_step(u));
  const float wsum_n = ks == 0 ? w.wsum[n] : 0.0f;  // the epilogue's inputs, needed last
  const float bias_n = (ks == 0 && bias && n < w.N) ? bias[n] : 0.0f;
  __syncthreads();  // (1)
  __syncthreads();  // (2): the codes are in LDS

  const bool row0 = (lane & 15) == 0;
  float acc[2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[0][i] = acc[1][i] = 0.0f;
  auto step = [&](int u, int64_t j) {
    const int64_t b = range_step(j);
    v4i af[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const v4i v = *reinterpret_cast<const __attribute__((address_space(3))) v4i*>(
          (const lds_i8*)qa_lds + b * 128 + 64 * h + 16 * c);
      af[h] = row0 ? v : v4i{0, 0, 0, 0};
    }
    // (the first use of this step's loads stays after the barriers above)
    asm volatile("" : "+v"(wr[u][0]), "+v"(wr[u][1]));
#pragma unroll
    for (int h = 0; h < NSC; ++h) asm volatile("" : "+v"(sr[u][h]));
    const bool live = ks * bpw + j < my_end;
    v4i cw2[2];
    float cs[NSC];
#pragma unroll
    for (int h = 0; h < 2; ++h) cw2[h] = wr[u][h];
#pragma unroll
    for (int h = 0; h < NSC; ++h) cs[h] = live ? sr[u][h] : 0.0f;
    load_w(u, range_step(j + P));
    v4i d[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      d[h] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[h], cw2[h], v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (BS == 64) {
        acc[0][i] = __builtin_fmaf(cs[0], (float)d[0][i], acc[0][i]);
        acc[1][i] = __builtin_fmaf(cs[NSC - 1], (float)d[1][i], acc[1][i]);
      } else {
        acc[0][i] = __builtin_fmaf(cs[0], (float)(d[0][i] + d[1][i]), acc[0][i]);
      }
    }
  };
  for (int64_t j0 = 0; j0 < bpw; j0 += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) step(u, j0 + u);
  }
  wait_vmcnt<0>();  // the clamped refills must land before the workgroup ends

  float out[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = acc[0][i] + acc[1][i];
  if (ks > 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) part[ks - 1][i][lane] = out[i];
  }
  __syncthreads();  // (3)
  // lane l < 16 holds row 0 (register 0) of channel l
  if (ks != 0 || lane >= 16 || n >= w.N) return;
  float S = out[0];
#pragma unroll
  for (int r = 0; r < KS - 1; ++r) S = S + part[r][0][lane];
  Y[n] = finish_w8(S, row_param[0], __builtin_bit_cast(int32_t, row_param[1]), wsum_n, bias_n,
                   lo, hi);
}

W8B w8b_of(const qp_packed_info* b, const void* blob) {
  const uint8_t* p = static_cast<const uint8_t*>(blob);
  return W8B{reinterpret_cast<const int8_t*>(p + b->data_off),
             reinterpret_cast<const float*>(p + b->scale_off),
             reinterpret_cast<const float*>(p + b->sum_off), b->N, b->Npad, b->Kpad,
             b->Kpad / 32, b->Kpad / b->group};
}

qp_status validate_w8b(const qp_packed_info* b, int64_t K) {
  QP_REQUIRE(b && b->format == 5, QP_EINVAL,
             "a8w8 blockwise: weights must be a block-quantized int8 blob");
  QP_REQUIRE(b->group == 64 || b->group == 128, QP_EUNSUPPORTED,
             "a8w8 blockwise: block size %lld not implemented (64 or 128)", (long long)b->group);
  QP_REQUIRE(K == b->K, QP_EINVAL, "a8w8 blockwise: activation K=%lld but the weights have K=%lld",
             (long long)K, (long long)b->K);
  return QP_OK;
}

template <int FM, int CW, int KS, int P = 3>
qp_status launch_cfg(const int8_t* qa, int64_t lda, const float* sa, const int32_t* za, int64_t M,
                     const W8B& w, int64_t bs, const float* bias, float lo, float hi, float* Y,
                     int64_t ldy, hipStream_t stream) {
  const unsigned bx = (unsigned)ceil_div(w.N, 16 * CW);
  const int64_t by = ceil_div(M, 16 * FM);
  QP_REQUIRE(by <= 65535, QP_EUNSUPPORTED, "a8w8 blockwise: M too large");
  const dim3 grid(bx, (unsigned)by);
  if (bs == 64)
    hipLaunchKernelGGL((a8w8b_gemm_kernel<FM, CW, KS, 64, P>), grid, dim3(256), 0, stream, qa, lda,
                       sa, za, M, w, bias, lo, hi, Y, ldy);
  else
    hipLaunchKernelGGL((a8w8b_gemm_kernel<FM, CW, KS, 128, P>), grid, dim3(256), 0, stream, qa, lda,
                       sa, za, M, w, bias, lo, hi, Y, ldy);
  return check_launch("a8w8 blockwise gemm");
}

// Largest Kpad of the fused GEMV: its codes live in the workgroup's LDS.
constexpr int64_t kFusedGemvMaxKpad = 32768;

qp_status launch_gemv_fused(const float* X, int64_t K, const W8B& w, int64_t bs,
                            const float* bias, float lo, float hi, float* Y, hipStream_t stream) {
  const unsigned blocks = (unsigned)(w.Npad / 16);
  const size_t lds = (size_t)w.Kpad;
  if (bs == 64)
    hipLaunchKernelGGL((a8w8b_gemv_fused_kernel<64, 8>), dim3(blocks), dim3(512), lds, stream, X,
                       K, w, bias, lo, hi, Y);
  else
    hipLaunchKernelGGL((a8w8b_gemv_fused_kernel<128, 8>), dim3(blocks), dim3(512), lds, stream, X,
                       K, w, bias, lo, hi, Y);
  return check_launch("a8w8 blockwise gemv");
}

qp_status launch_a8w8b(const int8_t* qa, int64_t lda, const float* sa, const int32_t* za,
                       int64_t M, const W8B& w, int64_t bs, const float* bias, float lo, float hi,
                       float* Y, int64_t ldy, hipStream_t stream) {
  // small M: four K ranges per 16-channel fragment; otherwise four channel
  // fragments share the staged rows
  if (M <= 16) {
    // At most one wave per SIMD (up to 256 16-channel fragments): nothing
    // else hides the weights' latency, so each wave keeps eight steps in
    // flight; larger grids keep three (more resident waves instead).
    if (ceil_div(w.N, 16) <= 256)
      return launch_cfg<1, 1, 4, 8>(qa, lda, sa, za, M, w, bs, bias, lo, hi, Y, ldy, stream);
    return launch_cfg<1, 1, 4>(qa, lda, sa, za, M, w, bs, bias, lo, hi, Y, ldy, stream);
  }
  // (32-row workgroups up to M = 128: more of them, measured faster there)
  if (M <= 128) return launch_cfg<2, 4, 1>(qa, lda, sa, za, M, w, bs, bias, lo, hi, Y, ldy, stream);
  return launch_cfg<4, 4, 1>(qa, lda, sa, za, M, w, bs, bias, lo, hi, Y, ldy, stream);
}

}  // namespace
}  // namespace qp

extern "C" qp_status qgemm_a8w8_blockwise_f32_ws_size(int64_t M, const qp_packed_info* w,
                                                      size_t* bytes) {
  using namespace qp;
  QP_REQUIRE(w && bytes && M >= 0, QP_EINVAL, "qgemm_a8w8_blockwise_f32_ws_size: bad argument");
  // one row with its codes fitting the fused GEMV's LDS needs no workspace
  const bool fused = M <= 1 && w->Kpad <= kFusedGemvMaxKpad;
  *bytes = fused ? 0 : (size_t)(round_up(M * w->Kpad, 256) + round_up(8 * M, 256));
  return QP_OK;
}

extern "C" qp_status qgemm_a8w8_blockwise_prequant_f32(const int8_t* qa, int64_t M, int64_t lda,
                                                       const float* sa, const int32_t* za,
                                                       const qp_packed_info* w,
                                                       const void* packedW_dev, const float* bias,
                                                       float clamp_lo, float clamp_hi, float* Y,
                                                       int64_t ldy, hipStream_t stream) {
  using namespace qp;
  clear_error();
  qp_status st = validate_w8b(w, w ? w->K : 0);
  if (st) return st;
  QP_REQUIRE(M >= 0 && lda >= w->Kpad && lda % 16 == 0 && ldy >= w->N, QP_EINVAL,
             "a8w8 blockwise: lda must be >= Kpad and a multiple of 16; ldy >= N");
  QP_REQUIRE(!(clamp_lo > clamp_hi), QP_EINVAL, "a8w8 blockwise: clamp_lo > clamp_hi");
  if (M == 0) return QP_OK;
  QP_REQUIRE(qa && sa && za && packedW_dev && Y, QP_EINVAL, "a8w8 blockwise: null data pointer");
  QP_REQUIRE(((uintptr_t)qa % 16) == 0, QP_EALIGN, "a8w8 blockwise: qa must be 16-byte aligned");
  QP_REQUIRE(lda <= (INT64_C(1) << 24), QP_EUNSUPPORTED, "a8w8 blockwise: lda above 2^24 bytes");
  return launch_a8w8b(qa, lda, sa, za, M, w8b_of(w, packedW_dev), w->group, bias, clamp_lo,
                      clamp_hi, Y, ldy, stream);
}

extern "C" qp_status qgemm_a8w8_blockwise_f32(const float* X, int64_t M, int64_t K, int64_t ldx,
                                              const qp_packed_info* w, const void* packedW_dev,
                                              const float* bias, float clamp_lo, float clamp_hi,
                                              float* Y, int64_t ldy, void* ws, size_t ws_bytes,
                                              hipStream_t stream) {
  using namespace qp;
  clear_error();
  qp_status st = validate_w8b(w, K);
  if (st) return st;
  QP_REQUIRE(M >= 0 && ldx >= K && ldy >= w->N, QP_EINVAL, "a8w8 blockwise: bad M/ldx/ldy");
  QP_REQUIRE(!(clamp_lo > clamp_hi), QP_EINVAL, "a8w8 blockwise: clamp_lo > clamp_hi");
  if (M == 0) return QP_OK;
  QP_REQUIRE(X && packedW_dev && Y, QP_EINVAL, "a8w8 blockwise: null data pointer");
  if (M == 1 && w->Kpad <= kFusedGemvMaxKpad)
    return launch_gemv_fused(X, K, w8b_of(w, packedW_dev), w->group, bias, clamp_lo, clamp_hi, Y,
                             stream);
  size_t need = 0;
  qgemm_a8w8_blockwise_f32_ws_size(M, w, &need);
  QP_REQUIRE(ws_bytes >= need, QP_ESIZE, "a8w8 blockwise: workspace holds %zu bytes, needs %zu",
             ws_bytes, need);
  QP_REQUIRE(ws && ((uintptr_t)ws % 256) == 0, QP_EALIGN,
             "a8w8 blockwise: workspace must be non-null and 256-byte aligned");
  uint8_t* p = static_cast<uint8_t*>(ws);
  int8_t* qa = reinterpret_cast<int8_t*>(p);
  float* sa = reinterpret_cast<float*>(p + round_up(M * w->Kpad, 256));
  int32_t* za = reinterpret_cast<int32_t*>(sa + M);
  st = launch_quantize_rows(X, M, K, ldx, qa, w->Kpad, w->Kpad, sa, za, false, stream);
  if (st) return st;
  return launch_a8w8b(qa, w->Kpad, sa, za, M, w8b_of(w, packedW_dev), w->group, bias, clamp_lo,
                      clamp_hi, Y, ldy, stream);
}
