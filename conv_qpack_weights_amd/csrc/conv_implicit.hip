// conv_implicit.hip -- INT8 NHWC convolution as an implicit GEMM: the im2col
// gather happens in the operand loads, so no column matrix is written or
// read back.
//
// MNN "ConvInt8TiledExecutor.cpp" (DenseConvInt8TiledExecutor, its
// tileSplitFunction): the convolution is the int8 GEMM of the im2col matrix
// (K ordered tap outer, input channel inner, as reorderWeight packs the
// weights) with the packed weights, out-of-image taps standing for the INPUT
// zero point.  tract-linalg "frame/pack.rs" (PackedI8K4::write_with_k_outer)
// lets the im2col patcher write straight into the matmul's operand layout;
// here that step disappears altogether: each lane fetches its MFMA operand
// piece from the input tensor itself.
//
// Operand mapping (v_mfma_i32_16x16x64_i8, issued as (weights, activations)):
// lane l holds output pixel l%16 of a 16-pixel fragment and channels
// 4*(l/16)..+3 of a 16-channel fragment; for the K-step kt (64 K) its
// activation piece is im2col row m, K bytes kt*64 + 16*(l/16) .. +16.  With
// C % 16 == 0 those 16 bytes are 16 consecutive input channels of one tap:
// one 16-byte load from X, or the zero-point pattern when the tap falls
// outside the image, or zeros past the real K (the packed weights are zero
// there too).  The weight piece is read from the int8 blob's 32x32 sub-tiles
// exactly as in the GEMM.  The operands do not pass through LDS: a wave owns
// its rows, loads its own operands, and keeps P K-steps of loads in flight
// in registers; every step runs the same branch-free body (the loads past
// the end read clamped, in-bounds addresses and are zeroed), so one constant
// wait count covers all of them.  (LDS holds only per-column constants, the
// channel-blocked variant's scale columns, and the partial sums of the
// K-split configuration.)  The epilogue is the GEMM's: zero-point
// corrections, bias and the Q31 requantization (or the raw int32), with the
// activation row sums, needed when the weights have zero points, summed
// from the same operand pieces.
#include <cstring>

#include "gemm_s8_core.hpp"
#include "qp_internal.hpp"

#pragma clang fp contract(off)

namespace qp {
namespace {

struct ConvKArgs {
  const int8_t* X;
  int32_t H, W, C, OH, OW;
  int32_t KW, sh, sw, pt, pl, dh, dw;
  int32_t K, nk;  // K = KH*KW*C; nk = Kpad / 64
  float rcpC, rcpKW;
  int64_t M, N;
  const int8_t* B;  // blob data
  int64_t kblocks;  // Kpad / 32
  const int32_t* colsum;
  const int32_t* zpB;
  const float* sB;
  const int32_t* bias;
  float sA, sOut;
  int32_t zA, zp_out, lo, hi;
  void* Y;
  int64_t ldy;
  int32_t tiles_n;
  // channel-blocked weights (f32 output): scale of channel n and K block kb
  // at sw_blk[kb*Npad + n], blocks of 64 << blk_shift K
  int64_t Npad;
  const float* sw_blk;
  int64_t nblk;
  int32_t blk_shift;
  int32_t sw_in_lds;  // the workgroup's scale columns are staged in LDS
  const float* bias_f;
  float clo, chi;
};

// q = k / d for 0 <= k < 2^22, 0 < d: the f32 quotient is within one of
// the true one, and the remainder test fixes it.
__device__ __forceinline__ int div_small(int k, int d, float rcp) {
  int q = (int)((float)k * rcp);
  const int r = k - q * d;
  q += (int)(r >= d) - (int)(r < 0);
  return q;
}

// kBlk: channel-blocked weights with f32 output.  Each K-step's products are
// kept apart: e = MFMA(weights, the input zero point), then
// d = MFMA(weights, pieces) accumulated onto -e, so d is the step's exact
// sum of (x - zx)*w.  Its block's f32 weight scale times d (|d| < 2^22) is
// exact in f64, and the running sum over the blocks is kept in f64: with
// hundreds of blocks an f32 running sum would round by more than the output
// tolerance.  The output is f32(sx * that) + bias, clamped.  The workgroup's block
// scales ([nblk][BN]) are copied to LDS once when they fit, else each step
// reads them from memory.
// KSP == 4 (few output tiles): the four waves share one tile of pixels and
// take every fourth K-step each (wave w: steps w, w+4, ...); their sums are
// added through LDS and wave 0 writes the tile.
template <int FM, int FN, int P, bool kOut32, bool kRowSum, bool kBlk = false, int KSP = 1>
__global__ __launch_bounds__(256) void conv_implicit_kernel(ConvKArgs g) {
  static_assert(KSP == 1 || KSP == 4, "K split over 1 or 4 waves");
  constexpr int BM = (KSP == 1 ? 4 : 1) * FM * 16;  // four waves stacked along the pixels, or one tile
  constexpr int BN = FN * 16;
  constexpr int LOADS = FM + FN;  // loads per K-step and lane
  static_assert((P - 1) * LOADS < 64, "vmcnt range");
  // a lane's partial sums (f64 ones in two words) and row sums
  constexpr int NRED = FN * FM * 4 * (kBlk ? 2 : 1) + FM;
  __shared__ int32_t col_m0[BN], col_sh[BN], col_c[BN], col_zb[BN];
  __shared__ int32_t red[KSP > 1 ? KSP - 1 : 1][KSP > 1 ? NRED : 1][64];
  extern __shared__ float sw_tile[];  // kBlk with sw_in_lds: [nblk][BN]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = lane >> 4;  // 16-byte K piece of the 64-K step
  const int r16 = lane & 15;
  // channel tiles fastest, so neighbouring workgroups read the same pixels
  const int tile_n = (int)(blockIdx.x % (unsigned)g.tiles_n);
  const int64_t tile_m = blockIdx.x / (unsigned)g.tiles_n;
  const int64_t m0 = tile_m * BM + (KSP == 1 ? wave * FM * 16 : 0);
  const int64_t n0 = (int64_t)tile_n * BN;

  // ---- per-column epilogue inputs: loaded now, ahead of the main loop's
  // loads, and turned into constants after the loop.  Forming them here
  // would wait for these loads before any pixel or weight load is issued:
  // one memory round trip in front of the whole convolution.  The loads are
  // unconditional (the column clamped into range, a stand-in array where
  // there is no bias).
  float e_sb = 0.0f;
  int32_t e_zb = 0, e_bias = 0, e_cs = 0;
  if (!kBlk && tid < BN) {
    const int64_t nc = n0 + tid < g.N ? n0 + tid : g.N - 1;
    e_sb = g.sB[nc];
    e_zb = g.zpB[nc];
    e_bias = (g.bias ? g.bias : g.zpB)[nc];
    e_cs = g.colsum[nc];
  }
  auto column_constants = [&]() {
    if (!kBlk && tid < BN) {
      const int64_t n = n0 + tid;
      int32_t mm = 0, ss = 1, cc = 0, zb = 0;
      if (n < g.N) {
        derive_mult(g.sA, e_sb, g.sOut, &mm, &ss);
        zb = e_zb;
        uint32_t c = (uint32_t)(g.bias ? e_bias : 0);
        c -= (uint32_t)g.zA * (uint32_t)e_cs;
        c += (uint32_t)g.K * (uint32_t)g.zA * (uint32_t)zb;
        cc = (int32_t)c;
      }
      col_m0[tid] = mm;
      col_sh[tid] = ss;
      col_c[tid] = cc;
      col_zb[tid] = zb;
    }
  };

  // ---- this lane's pixels ----
  int32_t iy0[FM], ix0[FM];
  uint32_t pbase[FM];
  const int64_t ohw = (int64_t)g.OH * g.OW;
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    int64_t m = m0 + j * 16 + r16;
    m = m < g.M ? m : g.M - 1;
    const int64_t b = m / ohw;
    const int32_t rem = (int32_t)(m - b * ohw);
    const int32_t oy = rem / g.OW, ox = rem - oy * g.OW;
    iy0[j] = oy * g.sh - g.pt;
    ix0[j] = ox * g.sw - g.pl;
    pbase[j] = (uint32_t)(b * g.H * g.W * g.C);
  }
  // ---- weight piece sources (32x32 sub-tiles; 64 K = two K blocks) ----
  const int8_t* b_src[FN];
#pragma unroll
  for (int i = 0; i < FN; ++i) {
    const int64_t r0 = n0 + i * 16;
    b_src[i] = g.B + ((r0 >> 5) * g.kblocks + (grp >> 1)) * 1024 + ((r0 & 31) + r16) * 32 +
               (grp & 1) * 16;
  }
  const int32_t zfill = (int32_t)(0x01010101u * (uint32_t)(uint8_t)(int8_t)g.zA);
  if constexpr (kBlk) {
    if (g.sw_in_lds) {
      const float* src = g.sw_blk + n0;
      for (int t = tid; t < (int)g.nblk * BN; t += 256) {
        const int kb = t / BN;
        sw_tile[t] = src[(int64_t)kb * g.Npad + (t - kb * BN)];
      }
      __syncthreads();
    }
  }

  v4i ar[P][FM], br[P][FN];
  uint32_t vbits[P];  // bit j: fragment j's piece is an in-image load
  int32_t fill[P];    // the pattern of the other pieces: zero point, or 0 past K
  auto issue = [&](int slot, int j) {  // j: this wave's step -> K-step kt
    const int kt = KSP == 1 ? j : j * KSP + wave;
    const int k = kt * 64 + grp * 16;
    const int tap = div_small(k, g.C, g.rcpC);
    const int ic = k - tap * g.C;
    const int ky = div_small(tap, g.KW, g.rcpKW);
    const int kx = tap - ky * g.KW;
    const bool kin = k < g.K;
    uint32_t bits = 0;
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int iy = iy0[j] + ky * g.dh, ix = ix0[j] + kx * g.dw;
      const bool v = kin & ((unsigned)iy < (unsigned)g.H) & ((unsigned)ix < (unsigned)g.W);
      const uint32_t off =
          v ? pbase[j] + ((uint32_t)iy * (uint32_t)g.W + (uint32_t)ix) * (uint32_t)g.C + (uint32_t)ic
            : 0u;
      ar[slot][j] = *reinterpret_cast<const v4i*>(g.X + off);
      bits |= (uint32_t)v << j;
    }
    vbits[slot] = bits;
    fill[slot] = kin ? zfill : 0;
    const int64_t kc = kt < g.nk ? kt : g.nk - 1;
#pragma unroll
    for (int i = 0; i < FN; ++i) br[slot][i] = *reinterpret_cast<const v4i*>(b_src[i] + kc * 2048);
  };
  double accd[kBlk ? FN : 1][kBlk ? FM : 1][4];
#pragma unroll
  for (int i = 0; i < (kBlk ? FN : 1); ++i)
#pragma unroll
    for (int j = 0; j < (kBlk ? FM : 1); ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) accd[i][j][r] = 0.0;

  v4i acc[FN][FM];
  int32_t rsum[FM];
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    rsum[j] = 0;
#pragma unroll
    for (int i = 0; i < FN; ++i) acc[i][j] = v4i{0, 0, 0, 0};
  }

#pragma unroll
  for (int p = 0; p < P; ++p) issue(p, p);
  const int nloc = (g.nk + KSP - 1) / KSP;  // steps of one wave (the last may be past K)
  const int nsteps = (nloc + P - 1) / P * P;
  for (int kt0 = 0; kt0 < nsteps; kt0 += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      wait_vmcnt<(P - 1) * LOADS>();
      v4i a[FM];
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const bool v = (vbits[u] >> j) & 1u;
        const v4i f = v4i{fill[u], fill[u], fill[u], fill[u]};
        a[j] = v ? ar[u][j] : f;
        if constexpr (kRowSum) {
          int32_t s = rsum[j];
          s = __builtin_amdgcn_sdot4(a[j].x, 0x01010101, s, false);
          s = __builtin_amdgcn_sdot4(a[j].y, 0x01010101, s, false);
          s = __builtin_amdgcn_sdot4(a[j].z, 0x01010101, s, false);
          s = __builtin_amdgcn_sdot4(a[j].w, 0x01010101, s, false);
          rsum[j] = s;
        }
      }
      if constexpr (kBlk) {
        // the input zero point over this lane's real K (0 past K)
        const v4i zop = v4i{fill[u], fill[u], fill[u], fill[u]};
        const int kt = KSP == 1 ? kt0 + u : (kt0 + u) * KSP + wave;
        const int kb = (kt < g.nk ? kt : g.nk - 1) >> g.blk_shift;
        float4 sc[FN];
        if (g.sw_in_lds) {
#pragma unroll
          for (int i = 0; i < FN; ++i)
            sc[i] = *reinterpret_cast<const float4*>(sw_tile + kb * BN + i * 16 + 4 * grp);
        } else {
#pragma unroll
          for (int i = 0; i < FN; ++i)
            sc[i] = *reinterpret_cast<const float4*>(g.sw_blk + (int64_t)kb * g.Npad + n0 +
                                                     i * 16 + 4 * grp);
        }
        v4i d[FN][FM];
#pragma unroll
        for (int i = 0; i < FN; ++i) {
          v4i e = __builtin_amdgcn_mfma_i32_16x16x64_i8(br[u][i], zop, v4i{0, 0, 0, 0}, 0, 0, 0);
          e = v4i{0, 0, 0, 0} - e;
#pragma unroll
          for (int j = 0; j < FM; ++j)
            d[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(br[u][i], a[j], e, 0, 0, 0);
        }
        issue(u, kt0 + u + P);
#pragma unroll
        for (int i = 0; i < FN; ++i) {
          const double s0 = sc[i].x, s1 = sc[i].y, s2 = sc[i].z, s3 = sc[i].w;
#pragma unroll
          for (int j = 0; j < FM; ++j) {
            accd[i][j][0] = __builtin_fma(s0, (double)d[i][j][0], accd[i][j][0]);
            accd[i][j][1] = __builtin_fma(s1, (double)d[i][j][1], accd[i][j][1]);
            accd[i][j][2] = __builtin_fma(s2, (double)d[i][j][2], accd[i][j][2]);
            accd[i][j][3] = __builtin_fma(s3, (double)d[i][j][3], accd[i][j][3]);
          }
        }
        continue;
      }
#pragma unroll
      for (int j = 0; j < FM; ++j)
#pragma unroll
        for (int i = 0; i < FN; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(br[u][i], a[j], acc[i][j], 0, 0, 0);
      issue(u, kt0 + u + P);
    }
  }
  wait_vmcnt<0>();
  column_constants();
  if constexpr (KSP > 1) {  // add the waves' partial sums (this barrier also publishes
                            // the column constants)
    if (wave > 0) {
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int q = (i * FM + j) * 4 + r;
            if constexpr (kBlk) {
              const uint64_t v = __builtin_bit_cast(uint64_t, accd[i][j][r]);
              red[wave - 1][2 * q][lane] = (int32_t)(uint32_t)v;
              red[wave - 1][2 * q + 1][lane] = (int32_t)(uint32_t)(v >> 32);
            } else {
              red[wave - 1][q][lane] = acc[i][j][r];
            }
          }
#pragma unroll
      for (int j = 0; j < FM; ++j) red[wave - 1][NRED - FM + j][lane] = rsum[j];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < KSP - 1; ++w) {
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int q = (i * FM + j) * 4 + r;
            if constexpr (kBlk) {
              const uint64_t v = (uint64_t)(uint32_t)red[w][2 * q][lane] |
                                 ((uint64_t)(uint32_t)red[w][2 * q + 1][lane] << 32);
              accd[i][j][r] = accd[i][j][r] + __builtin_bit_cast(double, v);
            } else {
              acc[i][j][r] = acc[i][j][r] + red[w][q][lane];
            }
          }
#pragma unroll
      for (int j = 0; j < FM; ++j) rsum[j] += red[w][NRED - FM + j][lane];
    }
  }
  if constexpr (kBlk) {  // y = sx * sum + bias, clamped; lane: channels 4*grp+r of row r16
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const int64_t n = n0 + i * 16 + 4 * grp;
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int64_t m = m0 + j * 16 + r16;
        if (m >= g.M) continue;
        float* row = static_cast<float*>(g.Y) + m * g.ldy;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (n + r >= g.N) continue;
          float y = (float)((double)g.sA * accd[i][j][r]) + (g.bias_f ? g.bias_f[n + r] : 0.0f);
          y = y < g.clo ? g.clo : y;
          y = y > g.chi ? g.chi : y;
          row[n + r] = y;
        }
      }
    }
    return;
  }
  if constexpr (KSP == 1) __syncthreads();  // the column constants

  // Row sums: the four lanes of a pixel hold the four K pieces.
  int32_t rs[FM];
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    int32_t s = 0;
    if constexpr (kRowSum) {
      s = rsum[j];
      s += __shfl_xor(s, 16, 64);
      s += __shfl_xor(s, 32, 64);
    }
    rs[j] = s;
  }
#pragma unroll
  for (int i = 0; i < FN; ++i) {
    const int jn = i * 16 + 4 * grp;
    const v4i cc = *reinterpret_cast<const v4i*>(&col_c[jn]);
    const v4i mm = *reinterpret_cast<const v4i*>(&col_m0[jn]);
    const v4i ss = *reinterpret_cast<const v4i*>(&col_sh[jn]);
    const v4i zb = *reinterpret_cast<const v4i*>(&col_zb[jn]);
    const int64_t n = n0 + jn;
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int64_t m = m0 + j * 16 + r16;
      if (m >= g.M) continue;
      int32_t out[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint32_t a = (uint32_t)acc[i][j][r] + (uint32_t)cc[r];
        if (kRowSum) a -= (uint32_t)zb[r] * (uint32_t)rs[j];
        if constexpr (kOut32) {
          out[r] = (int32_t)a;
        } else {
          const int32_t mr = mm[r], sr = ss[r];
          out[r] = clamp_i64(rhe_shift64((int32_t)a, mr, sr) + g.zp_out, g.lo, g.hi);
        }
      }
      const bool full = n + 3 < g.N;
      if constexpr (kOut32) {
        int32_t* row = static_cast<int32_t*>(g.Y) + m * g.ldy;
        if (full && ((g.ldy & 3) == 0) && ((((uintptr_t)g.Y) & 15) == 0)) {
          *reinterpret_cast<v4i*>(row + n) = v4i{out[0], out[1], out[2], out[3]};
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < g.N) row[n + r] = out[r];
        }
      } else {
        int8_t* row = static_cast<int8_t*>(g.Y) + m * g.ldy;
        if (full && ((g.ldy & 3) == 0) && ((((uintptr_t)g.Y) & 3) == 0)) {
          *reinterpret_cast<uint32_t*>(row + n) =
              ((uint32_t)out[0] & 0xFFu) | (((uint32_t)out[1] & 0xFFu) << 8) |
              (((uint32_t)out[2] & 0xFFu) << 16) | ((uint32_t)out[3] << 24);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < g.N) row[n + r] = (int8_t)out[r];
        }
      }
    }
  }
}

// Largest LDS copy of a workgroup's block scales.
constexpr int64_t kScaleTileBytes = 32 * 1024;

template <int FM, int FN, int P, bool kOut32, bool kRowSum, bool kBlk = false, int KSP = 1>
qp_status launch_cfg(ConvKArgs a, hipStream_t stream) {
  constexpr int BM = (KSP == 1 ? 4 : 1) * FM * 16, BN = FN * 16;
  a.tiles_n = (int32_t)ceil_div(a.N, BN);
  const int64_t blocks = ceil_div(a.M, BM) * a.tiles_n;
  QP_REQUIRE(blocks < (INT64_C(1) << 31), QP_EUNSUPPORTED, "qconv2d: too many tiles");
  size_t lds = 0;
  if (kBlk && a.nblk * BN * 4 <= kScaleTileBytes) {
    a.sw_in_lds = 1;
    lds = (size_t)(a.nblk * BN * 4);
  }
  hipLaunchKernelGGL((conv_implicit_kernel<FM, FN, P, kOut32, kRowSum, kBlk, KSP>),
                     dim3((unsigned)blocks), dim3(256), lds, stream, a);
  return check_launch("qconv2d implicit kernel");
}

// The K loop runs in whole groups of P steps; P is picked so that few
// steps fall past the end of K.
template <int FM, int FN, bool kOut32, bool kRowSum, bool kBlk = false, int KSP = 1>
qp_status launch_depth(const ConvKArgs& a, hipStream_t stream) {
  if constexpr (kBlk) {  // (the per-step rescaling holds more registers: depth 2)
    return launch_cfg<FM, FN, 2, kOut32, kRowSum, kBlk, KSP>(a, stream);
  } else {
    const int64_t n = ceil_div((int64_t)a.nk, KSP);  // steps per wave
    if (n <= 2) return launch_cfg<FM, FN, 2, kOut32, kRowSum, false, KSP>(a, stream);
    if (n % 4 != 0 && n % 3 == 0) return launch_cfg<FM, FN, 3, kOut32, kRowSum, false, KSP>(a, stream);
    return launch_cfg<FM, FN, 4, kOut32, kRowSum, false, KSP>(a, stream);
  }
}

template <bool kOut32, bool kRowSum, bool kBlk = false>
qp_status launch_sel(const ConvKArgs& a, hipStream_t stream) {
  if constexpr (kBlk) {
    // The per-step rescaling holds FN*FM*4 more registers: 32-channel tiles
    // keep the occupancy (measured faster than 64-channel ones).
    if (ceil_div(a.M, 128) * ceil_div(a.N, 32) >= 512)
      return launch_depth<2, 2, kOut32, kRowSum, kBlk>(a, stream);
    if (ceil_div(a.M, 64) * ceil_div(a.N, 32) < 256 && a.nk >= 4)
      return launch_depth<1, 2, kOut32, kRowSum, kBlk, 4>(a, stream);
    return launch_depth<1, 2, kOut32, kRowSum, kBlk>(a, stream);
  } else {
    // Two 128-pixel workgroups per compute unit or more: 32 pixels per wave
    // (fewer weight loads per MFMA).  Otherwise 16 pixels per wave, for more
    // workgroups; narrow layers or too few tiles take 32-channel tiles.
    if (ceil_div(a.M, 128) * ceil_div(a.N, 64) >= 512)
      return launch_depth<2, 4, kOut32, kRowSum>(a, stream);
    if (ceil_div(a.M, 64) * ceil_div(a.N, 64) >= 256 && a.N > 32)
      return launch_depth<1, 4, kOut32, kRowSum>(a, stream);
    // Few tiles (a small image): the four waves of a workgroup split the
    // K-steps of one 16-pixel tile, four times the workgroups.
    if (ceil_div(a.M, 64) * ceil_div(a.N, 32) < 256 && a.nk >= 4)
      return launch_depth<1, 2, kOut32, kRowSum, false, 4>(a, stream);
    return launch_depth<1, 2, kOut32, kRowSum>(a, stream);
  }
}

}  // namespace

namespace {
ConvKArgs conv_args(const int8_t* X, const ConvShape& cs, float sA, int32_t zA,
                    const qp_packed_info* w, const void* packedW, void* Y) {
  const uint8_t* blob = static_cast<const uint8_t*>(packedW);
  ConvKArgs a;
  std::memset(&a, 0, sizeof(a));
  a.X = X;
  a.H = (int32_t)cs.H;
  a.W = (int32_t)cs.W;
  a.C = (int32_t)cs.C;
  a.OH = (int32_t)cs.OH;
  a.OW = (int32_t)cs.OW;
  a.KW = cs.KW;
  a.sh = cs.sh;
  a.sw = cs.sw;
  a.pt = cs.pt;
  a.pl = cs.pl;
  a.dh = cs.dh;
  a.dw = cs.dw;
  a.K = (int32_t)w->K;
  a.nk = (int32_t)(w->Kpad / 64);
  a.rcpC = 1.0f / (float)cs.C;
  a.rcpKW = 1.0f / (float)cs.KW;
  a.M = cs.NB * cs.OH * cs.OW;
  a.N = w->N;
  a.B = reinterpret_cast<const int8_t*>(blob + w->data_off);
  a.kblocks = w->Kpad / 32;
  a.colsum = reinterpret_cast<const int32_t*>(blob + w->sum_off);
  a.zpB = reinterpret_cast<const int32_t*>(blob + w->zp_off);
  a.sB = reinterpret_cast<const float*>(blob + w->scale_off);
  a.sA = sA;
  a.zA = zA;
  a.Y = Y;
  a.ldy = w->N;
  return a;
}
}  // namespace

qp_status launch_conv_implicit(const int8_t* X, const ConvShape& cs, float sA, int32_t zA,
                               const qp_packed_info* w, const void* packedW,
                               const int32_t* bias, float sOut, int32_t zp_out, bool out32,
                               int32_t relu, void* Y, hipStream_t stream) {
  ConvKArgs a = conv_args(X, cs, sA, zA, w, packedW, Y);
  a.bias = bias;
  a.sOut = sOut;
  a.zp_out = zp_out;
  a.lo = relu ? zp_out : -128;
  a.hi = 127;
  if (a.M == 0) return QP_OK;
  const bool rowsum = w->has_zero_points != 0;
  if (out32)
    return rowsum ? launch_sel<true, true>(a, stream) : launch_sel<true, false>(a, stream);
  return rowsum ? launch_sel<false, true>(a, stream) : launch_sel<false, false>(a, stream);
}

qp_status launch_conv_implicit_blk(const int8_t* X, const ConvShape& cs, float sx, int32_t zx,
                                   const qp_packed_info* w, const void* packedW,
                                   const float* bias, float lo, float hi, float* Y,
                                   hipStream_t stream) {
  ConvKArgs a = conv_args(X, cs, sx, zx, w, packedW, Y);
  a.sw_blk = a.sB;  // the block scales, [Kpad/group][Npad]
  a.Npad = w->Npad;
  a.nblk = w->Kpad / w->group;
  a.blk_shift = w->group == 128 ? 1 : 0;
  a.bias_f = bias;
  a.clo = lo;
  a.chi = hi;
  if (a.M == 0) return QP_OK;
  return launch_sel<true, false, true>(a, stream);
}

}  // namespace qp
