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
#include <type_traits>

#include "dev_util.hpp"
#include "qp_internal.hpp"
#include "quant_row.hpp"

#pragma clang fp contract(off)

namespace qp {
namespace {

__device__ __forceinline__ uint32_t nib_lo16(uint32_t w) { return (w << 4) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t nib_hi16(uint32_t w) { return w & 0xF0F0F0F0u; }

// 16 * sum over the 8 K of one word: a0 holds qa for the word's low nibbles
// (k..k+3), a1 for its high nibbles (k+4..k+7).
__device__ __forceinline__ int32_t word_dot16(uint32_t w, uint32_t a0, uint32_t a1) {
  int32_t d = __builtin_amdgcn_sdot4((int)a0, (int)nib_lo16(w), 0, false);
  return __builtin_amdgcn_sdot4((int)a1, (int)nib_hi16(w), d, false);
}

// 16 * the sum of the eight int4 values of one word
__device__ __forceinline__ int32_t word_wsum16(uint32_t w) {
  return __builtin_amdgcn_sdot4((int)nib_hi16(w), 0x01010101,
                                __builtin_amdgcn_sdot4((int)nib_lo16(w), 0x01010101, 0, false),
                                false);
}

// Per-block activation quantization: S16 already holds
// 16 * sum_g sa[g]*sw[g]*sum (qa - za[g])*q, so only the bias remains.
__device__ __forceinline__ float finish_bq(float S16, float bias, float lo, float hi) {
  float y = S16 * 0.0625f + bias;
  y = y < lo ? lo : y;
  y = y > hi ? hi : y;
  return y;
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

// The int4 blob (group 32): channel n, 128-K block b at
// ((n/16)*nblk + b)*1024 + (n%16)*64 bytes; its four group scales at scale
// element ((n/16)*nblk + b)*64 + (n%16)*4, f32 (format 2) or bf16 (format 3).
struct W4 {
  const uint8_t* data;
  const uint8_t* scale;
  const float* wsum;     // [Npad]
  int64_t N, Npad, Kpad, nblk;
  int32_t kind;          // 0: f32 scales, 1: bf16 scales, 2: f32 scales + offsets
  const uint8_t* offs;   // kind 2: f32 group offsets, laid out as the scales
};

// 16 * the sum of the 8 activation bytes of one word's K (the factor 16
// matches word_dot16).
__device__ __forceinline__ int32_t word_sum16(uint32_t a0, uint32_t a1) {
  return __builtin_amdgcn_sdot4((int)a1, 0x10101010, __builtin_amdgcn_sdot4((int)a0, 0x10101010, 0,
                                                                           false),
                                false);
}

// The four group scales of one channel and block, as f32.  A bf16 value is
// the upper half of the f32 with the same value.
template <bool kBf16>
__device__ __forceinline__ float4 load_scale4(const uint8_t* p) {
  if constexpr (kBf16) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    const uint32_t lo = u.x, hi = u.y;
    return make_float4(__builtin_bit_cast(float, lo << 16),
                       __builtin_bit_cast(float, lo & 0xFFFF0000u),
                       __builtin_bit_cast(float, hi << 16),
                       __builtin_bit_cast(float, hi & 0xFFFF0000u));
  } else {
    return *reinterpret_cast<const float4*>(p);
  }
}

// ---- GEMV: a workgroup per 16-channel tile, waves split the 128-K blocks ----
// Lane l handles channel l/4 of the tile and 16-byte chunk c = l%4 of each
// of its wave's blocks (the 8-K piece c of four groups), so one wave load
// instruction reads one tile-block: 1 KiB in one piece.  Its four group
// scales are 16 bytes shared by the four lanes of the channel.  All of a
// wave's weight and scale loads are issued first; while they are in flight
// the workgroup quantizes the activation row (kFused, M = 1: the same device
// steps as qquantize_rows_s8) into LDS, permuted so that the 32 activation
// bytes of a chunk are contiguous; otherwise it reads the quantized rows
// from memory (row-major).  Partial sums are reduced across the four lanes
// of a channel with DPP and then across the waves through LDS, in a fixed
// order.  Rows m > 0 reuse the weights held in registers.
// kBQ: the activations were quantized per block of 32 (one scale and zero
// point per row and group, [M][ldsz]); one row.  Each group piece then
// contributes sa[g]*sw[g] * (dot - za[g] * sum q), exactly in integers up to
// that product.
template <int NT, bool kFused, int kKind, bool kBQ = false>
__global__ __launch_bounds__(NT) void a8w4_gemv_kernel(const float* __restrict__ X, int64_t K,
                                                       const int8_t* __restrict__ qa_g,
                                                       int64_t lda, const float* __restrict__ sa_g,
                                                       const int32_t* __restrict__ za_g,
                                                       int64_t M, W4 w,
                                                       const float* __restrict__ bias, float lo,
                                                       float hi, float* __restrict__ Y,
                                                       int64_t ldy) {
  static_assert(!kBQ || (!kFused && kKind != 2), "per-block activations: prequantized, symmetric");
  constexpr int NW = NT / 64;
  constexpr int BB = 4;      // blocks a wave holds in registers per batch
  constexpr int MR = 4;      // rows per call (M = 1 fused, M <= 4 prequantized)
  extern __shared__ __attribute__((aligned(16))) int8_t qa_lds[];
  __shared__ float red[2 * NW];
  __shared__ float part_w[NW][16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ch = lane >> 2, c = lane & 3;
  const int64_t tile = blockIdx.x;
  const int64_t nb = w.nblk;
  const uint8_t* wbase = w.data + tile * nb * 1024 + lane * 16;
  constexpr bool kBf16 = kKind == 1, kAsym = kKind == 2;
  constexpr int ES = kBf16 ? 2 : 4;  // bytes per stored scale
  const uint8_t* sbase = w.scale + (tile * nb * 64 + ch * 4) * ES;
  const uint8_t* obase = kAsym ? w.offs + (tile * nb * 64 + ch * 4) * 4 : nullptr;
  // per-channel epilogue operands, fetched up front (off the critical path)
  const int64_t n_out = tile * 16 + (tid & 15);
  float wsum_c = 0.0f, bias_c = 0.0f;
  if (tid < 16) {
    wsum_c = w.wsum[n_out];
    bias_c = (bias && n_out < w.N) ? bias[n_out] : 0.0f;
  }

  float part[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) part[m] = 0.0f;
  float sa = 0.0f;
  int32_t za = 0;
  const bool xvec = (((uintptr_t)X) & 15) == 0;
  RowFirst xfirst;
  float sa_m[MR];
  int32_t za_m[MR];
  if constexpr (kFused) {
    xfirst = quantize_row_first<NT, 8>(X, K, xvec);  // before the weights
  } else if constexpr (!kBQ) {
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      sa_m[m] = m < M ? sa_g[m] : 0.0f;
      za_m[m] = m < M ? za_g[m] : 0;
    }
  }
  // Batches are uniform over the workgroup (every wave runs all of them);
  // block j*NW*BB + u*NW + wave, past the end clamped with zero scales.
  const int64_t nbatch = (nb + (int64_t)NW * BB - 1) / ((int64_t)NW * BB);
  for (int64_t j = 0; j < nbatch; ++j) {
    uint4 wv[BB];
    float4 sv[BB], ov[BB], saq[BB];
    int4 zaq[BB];
    int64_t blk[BB];
#pragma unroll
    for (int u = 0; u < BB; ++u) {
      const int64_t b = (j * BB + u) * NW + wave;
      blk[u] = b < nb ? b : nb - 1;
      wv[u] = *reinterpret_cast<const uint4*>(wbase + blk[u] * 1024);
      const float4 s4 = load_scale4<kBf16>(sbase + blk[u] * 64 * ES);
      sv[u] = b < nb ? s4 : make_float4(0.f, 0.f, 0.f, 0.f);
      if constexpr (kAsym) {
        const float4 o4 = load_scale4<false>(obase + blk[u] * 64 * 4);
        ov[u] = b < nb ? o4 : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      if constexpr (kBQ) {  // the row's four group parameters of this block
        saq[u] = *reinterpret_cast<const float4*>(sa_g + 4 * blk[u]);
        zaq[u] = *reinterpret_cast<const int4*>(za_g + 4 * blk[u]);
      }
    }
    if constexpr (kFused) {
      if (j == 0) {  // quantize the row while the first loads are in flight
        quantize_row_wg<NT, true, 8>(X, K, w.Kpad, xvec, true, qa_lds, red, &sa, &za, &xfirst);
        __syncthreads();
      }
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      if (m < M) {
#pragma unroll
        for (int u = 0; u < BB; ++u) {
          uint2 a[4];
          if constexpr (kFused) {
            const int8_t* ab = qa_lds + blk[u] * 128 + c * 32;
            const uint4 p0 = *reinterpret_cast<const uint4*>(ab);
            const uint4 p1 = *reinterpret_cast<const uint4*>(ab + 16);
            a[0] = make_uint2(p0.x, p0.y);
            a[1] = make_uint2(p0.z, p0.w);
            a[2] = make_uint2(p1.x, p1.y);
            a[3] = make_uint2(p1.z, p1.w);
          } else {
            const int8_t* ab = qa_g + m * lda + blk[u] * 128 + c * 8;
#pragma unroll
            for (int t = 0; t < 4; ++t) a[t] = *reinterpret_cast<const uint2*>(ab + 32 * t);
          }
          const uint4 wq = wv[u];
          if constexpr (kBQ) {
            const int32_t z0 = zaq[u].x, z1 = zaq[u].y, z2 = zaq[u].z, z3 = zaq[u].w;
            const int32_t e0 = word_dot16(wq.x, a[0].x, a[0].y) - z0 * word_wsum16(wq.x);
            const int32_t e1 = word_dot16(wq.y, a[1].x, a[1].y) - z1 * word_wsum16(wq.y);
            const int32_t e2 = word_dot16(wq.z, a[2].x, a[2].y) - z2 * word_wsum16(wq.z);
            const int32_t e3 = word_dot16(wq.w, a[3].x, a[3].y) - z3 * word_wsum16(wq.w);
            part[m] = part[m] + (saq[u].x * sv[u].x) * (float)e0;
            part[m] = part[m] + (saq[u].y * sv[u].y) * (float)e1;
            part[m] = part[m] + (saq[u].z * sv[u].z) * (float)e2;
            part[m] = part[m] + (saq[u].w * sv[u].w) * (float)e3;
            continue;
          }
          const float d0 = (float)word_dot16(wq.x, a[0].x, a[0].y);
          const float d1 = (float)word_dot16(wq.y, a[1].x, a[1].y);
          const float d2 = (float)word_dot16(wq.z, a[2].x, a[2].y);
          const float d3 = (float)word_dot16(wq.w, a[3].x, a[3].y);
          if constexpr (kAsym) {
            // a group piece's term scale*d + offset*(16 * activation sum) is
            // formed first, so the running sum takes one addition per piece
            const float e0 = (float)word_sum16(a[0].x, a[0].y);
            const float e1 = (float)word_sum16(a[1].x, a[1].y);
            const float e2 = (float)word_sum16(a[2].x, a[2].y);
            const float e3 = (float)word_sum16(a[3].x, a[3].y);
            part[m] = part[m] + __builtin_fmaf(ov[u].x, e0, sv[u].x * d0);
            part[m] = part[m] + __builtin_fmaf(ov[u].y, e1, sv[u].y * d1);
            part[m] = part[m] + __builtin_fmaf(ov[u].z, e2, sv[u].z * d2);
            part[m] = part[m] + __builtin_fmaf(ov[u].w, e3, sv[u].w * d3);
          } else {
            part[m] = part[m] + sv[u].x * d0;
            part[m] = part[m] + sv[u].y * d1;
            part[m] = part[m] + sv[u].z * d2;
            part[m] = part[m] + sv[u].w * d3;
          }
        }
      }
    }
  }
  for (int64_t m = 0; m < M && m < MR; ++m) {
    float p = part[m];
    // the four lanes of a channel: quad_perm [1,0,3,2] then [2,3,0,1]
    p = p + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, p),
                                                                  0xB1, 0xF, 0xF, false));
    p = p + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, p),
                                                                  0x4E, 0xF, 0xF, false));
    if (c == 0) part_w[wave][ch] = p;
    __syncthreads();
    if (tid < 16) {
      float S = 0.0f;
#pragma unroll
      for (int v = 0; v < NW; ++v) S = S + part_w[v][tid];
      if constexpr (!kFused) {
#pragma unroll
        for (int r = 0; r < MR; ++r)
          if (r == m) {
            sa = sa_m[r];
            za = za_m[r];
          }
      }
      if constexpr (kBQ) {
        if (n_out < w.N) Y[m * ldy + n_out] = finish_bq(S, bias_c, lo, hi);
      } else {
        if (n_out < w.N) Y[m * ldy + n_out] = finish(S, sa, za, wsum_c, bias_c, lo, hi);
      }
    }
    __syncthreads();
  }
}

// ---- GEMM: MFMA 16x16x32 per 32-K group, f32 rescale per group ----------
// A wave computes FM x FN tiles of 16 rows x 16 channels.  The MFMA is
// issued as (activations, weights), so lane l holds rows 4*(l/16)+i of
// channel l%16: one f32 scale per lane, group and channel tile.  Lane
// (channel l%16, c = l/16) loads chunk c of its tile's 128-K block (the 8-K
// piece c of four groups, each unpacked to an 8-byte operand); a tile's
// block is 1 KiB in one piece and its four group scales 256 bytes, so each
// of these loads is one contiguous, fully used span.
// The 4 waves of a workgroup are RW row groups x CW channel groups x KS
// contiguous K ranges.  The workgroup's activation rows go through an
// R-stage LDS ring filled with direct (buffer ... lds) loads of whole 128-byte
// row pieces -- shared by the CW channel groups, and not competing with the
// weight stream for L1 -- stored with chunk p of row r at chunk position
// p ^ ((r >> 1) & 7) so that the 16-byte fragment reads are conflict-free.
// With kPerm the activations were written permuted inside each 128-K block
// (piece (t, c) at 32c + 8t) and a lane's four operands are 32 contiguous
// bytes; otherwise they are four 8-byte pieces.  When a workgroup is one
// row and one channel group (its waves split K), each wave fills and reads
// only its own rows of a stage and the loop has no barrier.  Otherwise one
// barrier per block: past
// it every wave has left the previous block (its ring stage may be
// refilled) and this block's rows have landed.  Weights and scales of the
// next P blocks are in registers in flight; a block's MFMAs are issued
// before their results are rescaled, two group slots at a time, into two
// f32 chains (even and odd slots) per output.  K-range partial sums are
// added in wave order through LDS.
// kBQ (activations quantized per block of 32: sa, za are [M][ldsz]): the
// MFMA is issued the other way round, (weights, activations), so a lane
// holds channels 4*(l/16)+i of row l%16 and needs one row's group
// parameters; a second MFMA against the row's zero point replicated over K
// gives za*sum q, and each group adds sa*sw * (d - that) per output.
template <int FM, int FN, int RW, int CW, int KS, bool kPerm, int kKind, bool kBQ = false>
__global__ __launch_bounds__(256) void a8w4_gemm_kernel(const int8_t* __restrict__ qa,
                                                        int64_t lda, const float* __restrict__ sa_g,
                                                        const int32_t* __restrict__ za_g,
                                                        int64_t M, W4 w,
                                                        const float* __restrict__ bias, float lo,
                                                        float hi, float* __restrict__ Y,
                                                        int64_t ldy, int64_t ldsz) {
  static_assert(!kBQ || kKind != 2, "per-block activations take symmetric weights");
  static_assert(RW * CW * KS == 4, "four waves");
  // weight prefetch depth in blocks (kBQ holds more per block: two); a
  // deeper ring measured slower (more registers, lower occupancy)
  constexpr int P = kBQ ? 2 : 3;
  constexpr int R = 4;                      // activation ring stages
  constexpr int MT = 16 * FM * RW;          // rows per workgroup
  constexpr int SLOTS = KS * MT * 8;        // 16-byte pieces per stage
  constexpr int ND = SLOTS / 256;           // direct loads per thread per stage
  constexpr int STAGE = SLOTS * 16;         // bytes per stage
  static_assert(SLOTS % 256 == 0, "a stage must split evenly over the workgroup");
  // Each wave its own K range (one row and one channel group): a wave loads
  // and reads only its own rows of a stage, so the waves need no barrier in
  // the K loop and run decoupled (a late weight block stalls only its wave).
  constexpr bool kPrivA = RW * CW == 1;
  static_assert(!kPrivA || MT * 8 == 64 * ND, "a wave's rows of a stage: ND loads per lane");
  __shared__ __attribute__((aligned(16))) int8_t ring[R * STAGE];
  __shared__ float red[KS > 1 ? (KS - 1) * RW * CW : 1][FM][FN][4][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ks = wave % KS;
  const int cw = (wave / KS) % CW;
  const int rw = wave / (KS * CW);
  const int slot = rw * CW + cw;
  const int c = lane >> 4;
  const int64_t n0 = ((int64_t)blockIdx.x * CW + cw) * 16 * FN;  // n0 + 16*FN <= Npad
  const int64_t mw = (int64_t)blockIdx.y * MT;                    // workgroup's first row
  const int64_t nblocks = w.Kpad / 128;
  const int64_t bpw = (nblocks + KS - 1) / KS;  // blocks per K range
  // every K range runs bpw steps; steps past its end are clamped to its last
  // block and contribute with zero scales
  auto range_block = [&](int r, int64_t j) {
    const int64_t b_begin = r * bpw;
    int64_t last = (b_begin + bpw < nblocks ? b_begin + bpw : nblocks) - 1;
    if (last < b_begin) last = nblocks - 1;  // empty range: park on a real block
    const int64_t b = b_begin + j;
    return b < last ? b : last;
  };
  const int64_t my_end = (ks * bpw + bpw < nblocks ? ks * bpw + bpw : nblocks);

  // ---- weight/scale sources (tile-contiguous blob) ----
  constexpr bool kBf16 = kKind == 1, kAsym = kKind == 2;
  constexpr int ES = kBf16 ? 2 : 4;  // bytes per stored scale
  const int8_t* wsrc[FN];
  const uint8_t* ssrc[FN];
  const uint8_t* osrc[FN];
#pragma unroll
  for (int q = 0; q < FN; ++q) {
    const int64_t n = n0 + q * 16 + (lane & 15);
    wsrc[q] = reinterpret_cast<const int8_t*>(w.data) + (n >> 4) * w.nblk * 1024 +
              (lane & 15) * 64 + 16 * c;
    // kBQ: the scales of channels 4c..4c+3 (16 consecutive values) instead
    ssrc[q] = kBQ ? w.scale + ((n >> 4) * w.nblk * 64 + 16 * c) * ES
                  : w.scale + ((n >> 4) * w.nblk * 64 + (lane & 15) * 4) * ES;
    osrc[q] = kAsym ? w.offs + ((n >> 4) * w.nblk * 64 + (lane & 15) * 4) * 4 : nullptr;
  }
  // kBQ: this lane's rows' per-block activation parameters
  const float* sap[FM];
  const int32_t* zap[FM];
#pragma unroll
  for (int f = 0; f < FM; ++f) {
    int64_t m = mw + rw * 16 * FM + f * 16 + (lane & 15);
    m = m < M ? m : M - 1;
    sap[f] = kBQ ? sa_g + m * ldsz : nullptr;
    zap[f] = kBQ ? za_g + m * ldsz : nullptr;
  }

  // ---- activation direct loads: thread slot s = tid + 256*i of a stage ->
  // (K range, row, chunk position); the global chunk is position ^ swizzle.
  const int8_t* const a_base = qa + mw * lda;
  uint32_t a_voff[ND];
  int a_rng[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) {
    const int s = kPrivA ? wave * (MT * 8) + 64 * i + lane : tid + 256 * i;
    const int r = (s >> 3) % MT;
    a_rng[i] = kPrivA ? wave : (32 * i + 8 * wave) / MT;  // == (s >> 3) / MT
    const int p = (s & 7) ^ ((r >> 1) & 7);
    int64_t m = mw + r;
    m = m < M ? m : M - 1;
    a_voff[i] = (uint32_t)((m - mw) * lda + 16 * p);
  }
  auto issue_stage = [&](int64_t j) {
    lds_i8* st = (lds_i8*)ring + (int)(j % R) * STAGE;
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      const int64_t b = range_block(a_rng[i], j);
      const int s0 = kPrivA ? wave * (MT * 8) + 64 * i : 256 * i + 64 * wave;  // lane 0's slot
      dma16_to_lds(a_base, (lds_void_t*)(st + s0 * 16), a_voff[i],
                   (uint32_t)(b * 128));
    }
  };

  // ---- accumulators ----
  float acc[2][FM][FN][4];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int q = 0; q < FN; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[h][f][q][i] = 0.0f;

  uint4 wr[P][FN];
  float4 sr[P][FN], orr[P][FN];
  float4 sr4[kBQ ? P : 1][FN][4];     // kBQ: [channel 4c+i] x 4 groups
  float4 sar[kBQ ? P : 1][FM];        // kBQ: the row's 4 group scales
  int4 zar[kBQ ? P : 1][FM];          //      and zero points
  auto load_w = [&](int u, int64_t b) {
#pragma unroll
    for (int q = 0; q < FN; ++q) {
      wr[u][q] = *reinterpret_cast<const uint4*>(wsrc[q] + b * 1024);
      if constexpr (kBQ) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sr4[u][q][i] = load_scale4<kBf16>(ssrc[q] + 64 * ES * b + 4 * ES * i);
      } else {
        sr[u][q] = load_scale4<kBf16>(ssrc[q] + 64 * ES * b);
      }
      if constexpr (kAsym) orr[u][q] = load_scale4<false>(osrc[q] + 64 * 4 * b);
    }
    if constexpr (kBQ) {
#pragma unroll
      for (int f = 0; f < FM; ++f) {
        sar[u][f] = *reinterpret_cast<const float4*>(sap[f] + 4 * b);
        zar[u][f] = *reinterpret_cast<const int4*>(zap[f] + 4 * b);
      }
    }
  };

  // one block: activation operands from the stage, MFMAs, refill, rescale
  auto step = [&](int u, int64_t j) {
    const lds_i8* st = (const lds_i8*)ring + (int)(j % R) * STAGE + ks * MT * 128;
    uint2 ca[FM][4];
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      const int r = rw * 16 * FM + f * 16 + (lane & 15);
      const lds_i8* rowp = st + r * 128;
      const int sw = (r >> 1) & 7;
      if constexpr (kPerm) {
        const u32x4 p0 = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
            rowp + 16 * ((2 * c) ^ sw));
        const u32x4 p1 = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
            rowp + 16 * ((2 * c + 1) ^ sw));
        ca[f][0] = make_uint2(p0.x, p0.y);
        ca[f][1] = make_uint2(p0.z, p0.w);
        ca[f][2] = make_uint2(p1.x, p1.y);
        ca[f][3] = make_uint2(p1.z, p1.w);
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) {  // bytes 32t + 8c: chunk 2t + c/2, half c%2
          const u32x2 p = *reinterpret_cast<const __attribute__((address_space(3))) u32x2*>(
              rowp + 16 * ((2 * t + (c >> 1)) ^ sw) + 8 * (c & 1));
          ca[f][t] = make_uint2(p.x, p.y);
        }
      }
    }
    uint4 cw4[FN];
    float4 cs[FN], co[FN];
    const bool live = ks * bpw + j < my_end;
    if constexpr (kBQ) {
      // per output (channel 4c+i, row): sa[row, g] * sw[channel, g], with
      // the row scales zeroed past the end of the K range
      float4 a4[FM], s4[FN][4];
      int4 zq[FM];
#pragma unroll
      for (int f = 0; f < FM; ++f) {
        a4[f] = live ? sar[u][f] : make_float4(0.f, 0.f, 0.f, 0.f);
        zq[f] = zar[u][f];
      }
#pragma unroll
      for (int q = 0; q < FN; ++q) {
        cw4[q] = wr[u][q];
#pragma unroll
        for (int i = 0; i < 4; ++i) s4[q][i] = sr4[u][q][i];
      }
      load_w(u, range_block(ks, j + P));
#pragma unroll
      for (int t2 = 0; t2 < 4; t2 += 2) {
        v4i d[2][FM][FN], e[2][FM][FN];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int t = t2 + h;
#pragma unroll
          for (int q = 0; q < FN; ++q) {
            const uint32_t wd = h == 0 ? (t2 == 0 ? cw4[q].x : cw4[q].z)
                                       : (t2 == 0 ? cw4[q].y : cw4[q].w);
            const long bop = (long)(((uint64_t)nib_hi16(wd) << 32) | nib_lo16(wd));
#pragma unroll
            for (int f = 0; f < FM; ++f) {
              const long aop = (long)(((uint64_t)ca[f][t].y << 32) | ca[f][t].x);
              const int32_t z = t == 0 ? zq[f].x : (t == 1 ? zq[f].y : (t == 2 ? zq[f].z : zq[f].w));
              const long zop = (long)((uint64_t)(uint8_t)(int8_t)z * 0x0101010101010101ull);
              d[h][f][q] = __builtin_amdgcn_mfma_i32_16x16x32_i8(bop, aop, v4i{0, 0, 0, 0}, 0, 0, 0);
              e[h][f][q] = __builtin_amdgcn_mfma_i32_16x16x32_i8(bop, zop, v4i{0, 0, 0, 0}, 0, 0, 0);
            }
          }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int t = t2 + h;
#pragma unroll
          for (int f = 0; f < FM; ++f) {
            const float ar = t == 0 ? a4[f].x : (t == 1 ? a4[f].y : (t == 2 ? a4[f].z : a4[f].w));
#pragma unroll
            for (int q = 0; q < FN; ++q)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float4 k4 = s4[q][i];
                const float sc = t == 0 ? k4.x : (t == 1 ? k4.y : (t == 2 ? k4.z : k4.w));
                acc[h][f][q][i] = __builtin_fmaf(ar * sc, (float)(d[h][f][q][i] - e[h][f][q][i]),
                                                 acc[h][f][q][i]);
              }
          }
        }
      }
      return;
    }
#pragma unroll
    for (int q = 0; q < FN; ++q) {
      cw4[q] = wr[u][q];
      cs[q] = live ? sr[u][q] : make_float4(0.f, 0.f, 0.f, 0.f);
      if constexpr (kAsym) co[q] = live ? orr[u][q] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    load_w(u, range_block(ks, j + P));
#pragma unroll
    for (int t2 = 0; t2 < 4; t2 += 2) {
      v4i d[2][FM][FN];
      v4i e[2][FM];  // asymmetric: 16 * the rows' activation sums per group
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int q = 0; q < FN; ++q) {
          const uint32_t wd = h == 0 ? (t2 == 0 ? cw4[q].x : cw4[q].z)
                                     : (t2 == 0 ? cw4[q].y : cw4[q].w);
          const long bop = (long)(((uint64_t)nib_hi16(wd) << 32) | nib_lo16(wd));
#pragma unroll
          for (int f = 0; f < FM; ++f) {
            const long aop = (long)(((uint64_t)ca[f][t2 + h].y << 32) | ca[f][t2 + h].x);
            d[h][f][q] = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop, bop, v4i{0, 0, 0, 0}, 0, 0, 0);
          }
        }
        if constexpr (kAsym) {
#pragma unroll
          for (int f = 0; f < FM; ++f) {
            const long aop = (long)(((uint64_t)ca[f][t2 + h].y << 32) | ca[f][t2 + h].x);
            e[h][f] = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop, (long)0x1010101010101010LL,
                                                            v4i{0, 0, 0, 0}, 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int q = 0; q < FN; ++q) {
          const float sc = h == 0 ? (t2 == 0 ? cs[q].x : cs[q].z) : (t2 == 0 ? cs[q].y : cs[q].w);
          if constexpr (kAsym) {
            // the group's term scale*d + offset*e first, then one addition
            const float oc =
                h == 0 ? (t2 == 0 ? co[q].x : co[q].z) : (t2 == 0 ? co[q].y : co[q].w);
#pragma unroll
            for (int f = 0; f < FM; ++f)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                acc[h][f][q][i] = acc[h][f][q][i] + __builtin_fmaf(oc, (float)e[h][f][i],
                                                                   sc * (float)d[h][f][q][i]);
          } else {
#pragma unroll
            for (int f = 0; f < FM; ++f)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                acc[h][f][q][i] = __builtin_fmaf(sc, (float)d[h][f][q][i], acc[h][f][q][i]);
          }
        }
    }
  };

  // ---- prologue: stages 0..R-2 and weights of blocks 0..P-1, all drained ----
#pragma unroll
  for (int j = 0; j < R - 1; ++j) issue_stage(j);
#pragma unroll
  for (int u = 0; u < P; ++u) load_w(u, range_block(ks, u));
  wait_vmcnt<0>();
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): settle the scalar loads too

  // Loads issued after stage j+1's direct loads, in the steady state: the
  // weights refilled by step j+2-R, and R-2 whole steps (direct loads and a
  // weight refill each).  Earlier stages were drained in the prologue.
  // loads per weight refill: weights and scales (kBQ: four scale vectors
  // and the rows' two parameter vectors; asymmetric: the offsets too)
  constexpr int LW = kBQ ? 5 * FN + 2 * FM : (kAsym ? 3 * FN : 2 * FN);
  constexpr int A_WAIT = LW + (R - 2) * (ND + LW);
  static_assert(A_WAIT < 64, "vmcnt range");
  // The step loop is unrolled by P so the weight ring index is static.
  for (int64_t j0 = 0; j0 < bpw; j0 += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const int64_t j = j0 + u;
      // (past the last step the body still runs, with zero scales, so that
      // every iteration issues the same loads)
      wait_vmcnt<A_WAIT>();
      if constexpr (!kPrivA) asm volatile("s_barrier" ::: "memory");
      issue_stage(j + R - 1);
      step(u, j);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  wait_vmcnt<0>();  // the clamped direct loads must land before the workgroup ends

  float out[FM][FN][4];
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int q = 0; q < FN; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) out[f][q][i] = acc[0][f][q][i] + acc[1][f][q][i];
  if constexpr (KS > 1) {
    if (ks > 0) {
#pragma unroll
      for (int f = 0; f < FM; ++f)
#pragma unroll
        for (int q = 0; q < FN; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) red[slot * (KS - 1) + ks - 1][f][q][i][lane] = out[f][q][i];
    }
    __syncthreads();
    if (ks != 0) return;
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int q = 0; q < FN; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < KS - 1; ++r)
            out[f][q][i] = out[f][q][i] + red[slot * (KS - 1) + r][f][q][i][lane];
  }
  if constexpr (kBQ) {  // lane: row l%16 of fragment f, channels 4c+i
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      const int64_t m = mw + rw * 16 * FM + f * 16 + (lane & 15);
      if (m >= M) continue;
#pragma unroll
      for (int q = 0; q < FN; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t n = n0 + q * 16 + 4 * c + i;
          if (n < w.N) Y[m * ldy + n] = finish_bq(out[f][q][i], bias ? bias[n] : 0.0f, lo, hi);
        }
    }
    return;
  }
#pragma unroll
  for (int q = 0; q < FN; ++q) {
    const int64_t n = n0 + q * 16 + (lane & 15);
    if (n >= w.N) continue;
    const float ws = w.wsum[n];
    const float bn = bias ? bias[n] : 0.0f;
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = mw + rw * 16 * FM + f * 16 + 4 * c + i;
        if (m < M) Y[m * ldy + n] = finish(out[f][q][i], sa_g[m], za_g[m], ws, bn, lo, hi);
      }
  }
}

W4 w4_of(const qp_packed_info* b, const void* blob) {
  const uint8_t* p = static_cast<const uint8_t*>(blob);
  return W4{p + b->data_off, p + b->scale_off, reinterpret_cast<const float*>(p + b->sum_off),
            b->N, b->Npad, b->Kpad, b->Kpad / 128, (int32_t)(b->format - 2),
            b->format == 4 ? p + b->zp_off : nullptr};
}

qp_status validate_w4(const qp_packed_info* b, int64_t K) {
  QP_REQUIRE(b && b->format >= 2 && b->format <= 4, QP_EINVAL,
             "a8w4: weights must be an int4 blob");
  QP_REQUIRE(b->group == 32, QP_EUNSUPPORTED, "a8w4: group size %lld not implemented (32 only)",
             (long long)b->group);
  QP_REQUIRE(K == b->K, QP_EINVAL, "a8w4: activation K=%lld but the weights have K=%lld",
             (long long)K, (long long)b->K);
  return QP_OK;
}

template <int NT>
qp_status launch_gemv_cfg(const float* X, int64_t K, const int8_t* qa, int64_t lda,
                          const float* sa, const int32_t* za, int64_t M, const W4& w,
                          const float* bias, float lo, float hi, float* Y, int64_t ldy,
                          bool fused, hipStream_t stream) {
  const unsigned blocks = (unsigned)(w.Npad / 16);
  const size_t lds = fused ? (size_t)w.Kpad : 0;
#define QP_GEMV(F, KIND)                                                                      \
  hipLaunchKernelGGL((a8w4_gemv_kernel<NT, F, KIND>), dim3(blocks), dim3(NT), lds, stream, X, K, \
                     qa, lda, sa, za, M, w, bias, lo, hi, Y, ldy)
  if (fused) {
    if (w.kind == 1) QP_GEMV(true, 1);
    else if (w.kind == 2) QP_GEMV(true, 2);
    else QP_GEMV(true, 0);
  } else {
    if (w.kind == 1) QP_GEMV(false, 1);
    else if (w.kind == 2) QP_GEMV(false, 2);
    else QP_GEMV(false, 0);
  }
#undef QP_GEMV
  return check_launch("a8w4 gemv");
}

qp_status launch_gemv(const float* X, int64_t K, const int8_t* qa, int64_t lda,
                      const float* sa, const int32_t* za, int64_t M, const W4& w,
                      const float* bias, float lo, float hi, float* Y, int64_t ldy, bool fused,
                      hipStream_t stream) {
  QP_REQUIRE(M <= 4, QP_EUNSUPPORTED, "a8w4 gemv: at most 4 rows");
  return launch_gemv_cfg<512>(X, K, qa, lda, sa, za, M, w, bias, lo, hi, Y, ldy, fused, stream);
}

// One row quantized per block: sa, za hold the row's group parameters.
qp_status launch_gemv_bq(const int8_t* qa, const float* sa, const int32_t* za, const W4& w,
                         const float* bias, float lo, float hi, float* Y, hipStream_t stream) {
  constexpr int NT = 512;
  const unsigned blocks = (unsigned)(w.Npad / 16);
  if (w.kind == 1)
    hipLaunchKernelGGL((a8w4_gemv_kernel<NT, false, 1, true>), dim3(blocks), dim3(NT), 0, stream,
                       nullptr, w.Kpad, qa, w.Kpad, sa, za, 1, w, bias, lo, hi, Y, w.N);
  else
    hipLaunchKernelGGL((a8w4_gemv_kernel<NT, false, 0, true>), dim3(blocks), dim3(NT), 0, stream,
                       nullptr, w.Kpad, qa, w.Kpad, sa, za, 1, w, bias, lo, hi, Y, w.N);
  return check_launch("a8w4 gemv (per-block activations)");
}

template <int FM, int FN, int RW, int CW, int KS>
qp_status launch_gemm_cfg(const int8_t* qa, int64_t lda, bool perm, const float* sa,
                          const int32_t* za, int64_t M, const W4& w, const float* bias, float lo,
                          float hi, float* Y, int64_t ldy, int64_t ldsz, hipStream_t stream) {
  static_assert(64 % (16 * FN * CW) == 0, "channel tiles must tile the 64-channel padding");
  const unsigned bx = (unsigned)ceil_div(w.N, 16 * FN * CW);
  const int64_t by = ceil_div(M, 16 * FM * RW);
  QP_REQUIRE(by <= 65535, QP_EUNSUPPORTED, "a8w4: M too large");
  const dim3 grid(bx, (unsigned)by);
#define QP_GEMM(PERM, KIND)                                                                \
  hipLaunchKernelGGL((a8w4_gemm_kernel<FM, FN, RW, CW, KS, PERM, KIND>), grid, dim3(256), 0, \
                     stream, qa, lda, sa, za, M, w, bias, lo, hi, Y, ldy, (int64_t)0)
#define QP_GEMM_BQ(KIND)                                                                      \
  hipLaunchKernelGGL((a8w4_gemm_kernel<FM, FN, RW, CW, KS, false, KIND, true>), grid, dim3(256), \
                     0, stream, qa, lda, sa, za, M, w, bias, lo, hi, Y, ldy, ldsz)
  if (ldsz > 0) {  // per-block activation parameters
    if (w.kind == 1) QP_GEMM_BQ(1);
    else QP_GEMM_BQ(0);
  } else if (perm) {
    if (w.kind == 1) QP_GEMM(true, 1);
    else if (w.kind == 2) QP_GEMM(true, 2);
    else QP_GEMM(true, 0);
  } else {
    if (w.kind == 1) QP_GEMM(false, 1);
    else if (w.kind == 2) QP_GEMM(false, 2);
    else QP_GEMM(false, 0);
  }
#undef QP_GEMM
#undef QP_GEMM_BQ
  return check_launch("a8w4 gemm");
}

// perm: the activations are permuted inside each 128-K block (as written by
// the fused quantization); otherwise plain row-major.  ldsz > 0: sa, za are
// per-block parameters [M][ldsz] (row-major activations).
qp_status launch_gemm(const int8_t* qa, int64_t lda, bool perm, const float* sa,
                      const int32_t* za, int64_t M, const W4& w, const float* bias, float lo,
                      float hi, float* Y, int64_t ldy, hipStream_t stream, int64_t ldsz = 0) {
  // <FM, FN, RW, CW, KS>: rows per workgroup 16*FM*RW, channels 16*FN*CW.
  // Small M splits K over the waves (enough waves stream the weights); larger
  // M shares each staged activation row among several channel groups.
  if (M <= 16)
    return launch_gemm_cfg<1, 1, 1, 1, 4>(qa, lda, perm, sa, za, M, w, bias, lo, hi, Y, ldy,
                                          ldsz, stream);
  // (the per-block variant holds more per row fragment: two fragments a wave)
  if (M <= 32 || ldsz > 0)
    return launch_gemm_cfg<2, 1, 1, 4, 1>(qa, lda, perm, sa, za, M, w, bias, lo, hi, Y, ldy,
                                          ldsz, stream);
  // 64 rows x 32 channels a workgroup (two row and two channel groups):
  // measured faster than 64 x 64 with four channel groups, whose 256-VGPR
  // waves fit two a SIMD
  return launch_gemm_cfg<2, 1, 2, 2, 1>(qa, lda, perm, sa, za, M, w, bias, lo, hi, Y, ldy, ldsz,
                                        stream);
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
  st = launch_quantize_rows(X, M, K, ldx, qa, w->Kpad, w->Kpad, sa, za, true, stream);
  if (st) return st;
  return launch_gemm(qa, w->Kpad, true, sa, za, M, wv, bias, clamp_lo, clamp_hi, Y, ldy, stream);
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
  QP_REQUIRE(lda <= (INT64_C(1) << 24), QP_EUNSUPPORTED, "a8w4: lda above 2^24 bytes");
  const W4 wv = w4_of(w, packedW_dev);
  if (M <= 4)
    return launch_gemv(nullptr, w->K, qa, lda, sa, za, M, wv, bias, clamp_lo, clamp_hi, Y, ldy,
                       false, stream);
  return launch_gemm(qa, lda, false, sa, za, M, wv, bias, clamp_lo, clamp_hi, Y, ldy, stream);
}

// ---- activations quantized per block of 32 K ----------------------------
extern "C" qp_status qgemm_a8w4_blockq_f32_ws_size(int64_t M, const qp_packed_info* w,
                                                   size_t* bytes) {
  using namespace qp;
  QP_REQUIRE(w && bytes && M >= 0, QP_EINVAL, "qgemm_a8w4_blockq_f32_ws_size: bad argument");
  const int64_t nb = w->Kpad / 32;
  *bytes = (size_t)(round_up(M * w->Kpad, 256) + 2 * round_up(4 * M * nb, 256));
  return QP_OK;
}

static qp_status validate_bq(const qp_packed_info* w, int64_t K) {
  using namespace qp;
  qp_status st = validate_w4(w, K);
  if (st) return st;
  QP_REQUIRE(w->format != 4, QP_EUNSUPPORTED,
             "a8w4 per-block activations: asymmetric weights are not supported");
  return QP_OK;
}

extern "C" qp_status qgemm_a8w4_blockq_prequant_f32(const int8_t* qa, int64_t M, int64_t lda,
                                                    const float* sa, const int32_t* za,
                                                    int64_t ldsz, const qp_packed_info* w,
                                                    const void* packedW_dev, const float* bias,
                                                    float clamp_lo, float clamp_hi, float* Y,
                                                    int64_t ldy, hipStream_t stream) {
  using namespace qp;
  clear_error();
  qp_status st = validate_bq(w, w ? w->K : 0);
  if (st) return st;
  QP_REQUIRE(M >= 0 && lda >= w->Kpad && lda % 16 == 0 && ldy >= w->N, QP_EINVAL,
             "a8w4: lda must be >= Kpad and a multiple of 16; ldy >= N");
  QP_REQUIRE(ldsz >= w->Kpad / 32 && ldsz % 4 == 0, QP_EINVAL,
             "a8w4 per-block: ldsz must be >= Kpad/32 and a multiple of 4");
  QP_REQUIRE(!(clamp_lo > clamp_hi), QP_EINVAL, "a8w4: clamp_lo > clamp_hi");
  if (M == 0) return QP_OK;
  QP_REQUIRE(qa && sa && za && packedW_dev && Y, QP_EINVAL, "a8w4: null data pointer");
  QP_REQUIRE(((uintptr_t)qa % 16) == 0 && ((uintptr_t)sa % 16) == 0 && ((uintptr_t)za % 16) == 0,
             QP_EALIGN, "a8w4 per-block: qa, sa and za must be 16-byte aligned");
  QP_REQUIRE(lda <= (INT64_C(1) << 24), QP_EUNSUPPORTED, "a8w4: lda above 2^24 bytes");
  const W4 wv = w4_of(w, packedW_dev);
  if (M == 1 && lda == w->Kpad && ldy >= w->N)
    return launch_gemv_bq(qa, sa, za, wv, bias, clamp_lo, clamp_hi, Y, stream);
  return launch_gemm(qa, lda, false, sa, za, M, wv, bias, clamp_lo, clamp_hi, Y, ldy, stream, ldsz);
}

extern "C" qp_status qgemm_a8w4_blockq_f32(const float* X, int64_t M, int64_t K, int64_t ldx,
                                           const qp_packed_info* w, const void* packedW_dev,
                                           const float* bias, float clamp_lo, float clamp_hi,
                                           float* Y, int64_t ldy, void* ws, size_t ws_bytes,
                                           hipStream_t stream) {
  using namespace qp;
  clear_error();
  qp_status st = validate_bq(w, K);
  if (st) return st;
  QP_REQUIRE(M >= 0 && ldx >= K && ldy >= w->N, QP_EINVAL, "a8w4: bad M/ldx/ldy");
  QP_REQUIRE(!(clamp_lo > clamp_hi), QP_EINVAL, "a8w4: clamp_lo > clamp_hi");
  if (M == 0) return QP_OK;
  QP_REQUIRE(X && packedW_dev && Y, QP_EINVAL, "a8w4: null data pointer");
  size_t need = 0;
  qgemm_a8w4_blockq_f32_ws_size(M, w, &need);
  QP_REQUIRE(ws_bytes >= need, QP_ESIZE, "a8w4: workspace holds %zu bytes, needs %zu", ws_bytes,
             need);
  QP_REQUIRE(ws && ((uintptr_t)ws % 256) == 0, QP_EALIGN,
             "a8w4: workspace must be non-null and 256-byte aligned");
  const int64_t nb = w->Kpad / 32;
  uint8_t* p = static_cast<uint8_t*>(ws);
  int8_t* qa = reinterpret_cast<int8_t*>(p);
  float* sa = reinterpret_cast<float*>(p + round_up(M * w->Kpad, 256));
  int32_t* za = reinterpret_cast<int32_t*>(p + round_up(M * w->Kpad, 256) + round_up(4 * M * nb, 256));
  st = launch_quantize_blocks32(X, M, K, ldx, qa, w->Kpad, w->Kpad, sa, za, nb, stream);
  if (st) return st;
  const W4 wv = w4_of(w, packedW_dev);
  if (M == 1 && ldy >= w->N)
    return launch_gemv_bq(qa, sa, za, wv, bias, clamp_lo, clamp_hi, Y, stream);
  return launch_gemm(qa, w->Kpad, false, sa, za, M, wv, bias, clamp_lo, clamp_hi, Y, ldy, stream,
                     nb);
}
