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
#include <atomic>
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

// 16 bytes of LDS as a float4.  The elements are copied to scalars before
// the casts: __builtin_bit_cast applied straight to an element of a vector
// (u.y) compiles, with this compiler, to a cast of element 0.
__device__ __forceinline__ float4 lds_f4(const lds_i8* p) {
  const u32x4 u = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(p);
  const uint32_t x = u.x, y = u.y, z = u.z, w = u.w;
  return make_float4(__builtin_bit_cast(float, x), __builtin_bit_cast(float, y),
                     __builtin_bit_cast(float, z), __builtin_bit_cast(float, w));
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

// The four group scales (f32 or bf16) of one channel and 128-K block through
// a buffer resource bounded by the tile's scale region: offsets past it
// read as zeros, so blocks past the end of K contribute nothing without a
// select (which the compiler may turn into a branch around the load, whose
// join then waits for it).
template <bool kBf16>
__device__ __forceinline__ float4 load_scale4_bounded(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (kBf16) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    const uint32_t lo = v[0], hi = v[1];
    return make_float4(__builtin_bit_cast(float, lo << 16),
                       __builtin_bit_cast(float, lo & 0xFFFF0000u),
                       __builtin_bit_cast(float, hi << 16),
                       __builtin_bit_cast(float, hi & 0xFFFF0000u));
  } else {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    const uint32_t a0 = v[0], a1 = v[1], a2 = v[2], a3 = v[3];
    return make_float4(__builtin_bit_cast(float, a0), __builtin_bit_cast(float, a1),
                       __builtin_bit_cast(float, a2), __builtin_bit_cast(float, a3));
  }
}

// The dot products of one 128-K block for lane (channel l/4, chunk c = l%4):
// wq holds the chunk's 8-K piece of four groups, a[t] the activations of
// group t's piece (bytes k..k+3 in .x, k+4..k+7 in .y), sv / ov the group
// scales / offsets.  Adds the block's four group terms to `part`.
// The nibbles of the four weight words come unpacked (nibble_ops): low
// nibbles shifted up in nl[t], high ones masked in nh[t], each as int8 16*q.
struct Nibbles {
  uint32_t lo[4], hi[4];
};
__device__ __forceinline__ Nibbles nibble_ops(const uint4& wq) {
  Nibbles n;
  const uint32_t w4[4] = {wq.x, wq.y, wq.z, wq.w};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    n.lo[t] = nib_lo16(w4[t]);
    n.hi[t] = nib_hi16(w4[t]);
  }
  return n;
}
__device__ __forceinline__ int32_t nib_dot16(uint32_t lo, uint32_t hi, uint32_t a0, uint32_t a1) {
  return __builtin_amdgcn_sdot4((int)a1, (int)hi, __builtin_amdgcn_sdot4((int)a0, (int)lo, 0, false),
                                false);
}

template <int kKind>
__device__ __forceinline__ void gemv_block_terms(const Nibbles& nb, const uint2 (&a)[4],
                                                 const float4& sv, const float4& ov,
                                                 float& part) {
  const float d0 = (float)nib_dot16(nb.lo[0], nb.hi[0], a[0].x, a[0].y);
  const float d1 = (float)nib_dot16(nb.lo[1], nb.hi[1], a[1].x, a[1].y);
  const float d2 = (float)nib_dot16(nb.lo[2], nb.hi[2], a[2].x, a[2].y);
  const float d3 = (float)nib_dot16(nb.lo[3], nb.hi[3], a[3].x, a[3].y);
  if constexpr (kKind == 2) {
    // a group piece's term scale*d + offset*(16 * activation sum) is
    // formed first, so the running sum takes one addition per piece
    const float e0 = (float)word_sum16(a[0].x, a[0].y);
    const float e1 = (float)word_sum16(a[1].x, a[1].y);
    const float e2 = (float)word_sum16(a[2].x, a[2].y);
    const float e3 = (float)word_sum16(a[3].x, a[3].y);
    part = part + __builtin_fmaf(ov.x, e0, sv.x * d0);
    part = part + __builtin_fmaf(ov.y, e1, sv.y * d1);
    part = part + __builtin_fmaf(ov.z, e2, sv.z * d2);
    part = part + __builtin_fmaf(ov.w, e3, sv.w * d3);
  } else {
    part = part + sv.x * d0;
    part = part + sv.y * d1;
    part = part + sv.z * d2;
    part = part + sv.w * d3;
  }
}

// ---- GEMV with the row's dynamic quantization (M = 1) ---------------------
// (NQ quantizer waves, NWW weight waves, BB blocks per weight wave and
// batch, QE row values per quantizer thread and pass)
// One workgroup per 16-channel tile, two kinds of waves:
//  * NQ quantizer waves load the f32 row (branch-free, bounded loads) and
//    quantize it with the steps of qquantize_rows_s8 into LDS, permuted so
//    that the 32 activation bytes of a chunk are contiguous;
//  * NWW weight waves issue all their weight and scale loads at once and
//    only then wait.  Lane l handles channel l/4 of the tile and 16-byte
//    chunk c = l%4 of each of its blocks (the 8-K piece c of four groups), so
//    one load instruction reads one tile-block: 1 KiB in one piece.
// Loads complete in issue order within a wave, so a wave that both waited
// for the row and streamed weights would either hold its weight loads back
// until the row arrived or see the row arrive behind its weights; with the
// two jobs in different waves neither waits for the other.  After the codes
// are in LDS the weight waves form the exact int32 group dots and the f32
// scaled sum, reduce over the four lanes of a channel (DPP) and then over
// the weight waves through LDS in a fixed order.
// kBQ: the row is quantized per block of 32 instead (the steps of
// qquantize_rows_s8_blocked): a quantizer thread takes 16 values, the
// neighbouring lane the other 16 of the block, and one DPP lane swap gives
// the block's extremes; each block's scale and zero point go to LDS after
// the codes, and every group piece contributes sa*sw * (dot - za * sum q).
template <int NQ, int NWW, int BB, int QE, int kKind, bool kBQ = false>
__global__ __launch_bounds__((NQ + NWW) * 64) void a8w4_gemv_fused_kernel(
    const float* __restrict__ X, int64_t K, W4 w, const float* __restrict__ bias, float lo,
    float hi, float* __restrict__ Y) {
  static_assert(!kBQ || kKind != 2, "per-block activations: symmetric weights");
  constexpr int QT = NQ * 64;  // quantizer threads
  constexpr bool kBf16 = kKind == 1, kAsym = kKind == 2;
  constexpr int ES = kBf16 ? 2 : 4;  // bytes per stored scale
  // [Kpad] codes; kBQ: then [Kpad/32] f32 block scales, [Kpad/32] zero points
  extern __shared__ __attribute__((aligned(16))) int8_t qa_lds[];
  float* const bq_s = reinterpret_cast<float*>(qa_lds + w.Kpad);
  int32_t* const bq_z = reinterpret_cast<int32_t*>(qa_lds + w.Kpad) + w.Kpad / 32;
  __shared__ float red[2 * NQ];
  __shared__ float part_w[NWW][16];
  __shared__ float row_param[2];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t tile = blockIdx.x;
  const int64_t nb = w.nblk;
  const int64_t n_out = tile * 16 + (lane & 15);  // the final step's channel (weight wave 0)
  float wsum_c = 0.0f, bias_c = 0.0f;
  if (kBQ && wave < NQ) {
    const bool xvec = (((uintptr_t)X) & 15) == 0;
    for (int64_t k0 = (int64_t)tid * 16; k0 < w.Kpad; k0 += QT * 16) {
      // (both lanes of a block take the same branches: Kpad % 32 == 0)
      float v[16];
      if (xvec && k0 + 16 <= K) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 f = *reinterpret_cast<const float4*>(X + k0 + 4 * q);
          v[4 * q] = f.x;
          v[4 * q + 1] = f.y;
          v[4 * q + 2] = f.z;
          v[4 * q + 3] = f.w;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = k0 + j < K ? X[k0 + j] : 0.0f;
      }
      // the block's range, widened to include 0 (values past K read as 0)
      float lo_b = 0.0f, hi_b = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        lo_b = qp_min(lo_b, v[j]);
        hi_b = qp_max(hi_b, v[j]);
      }
      lo_b = qp_min(lo_b, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                              0, __builtin_bit_cast(int, lo_b), 0xB1, 0xF, 0xF, false)));
      hi_b = qp_max(hi_b, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                              0, __builtin_bit_cast(int, hi_b), 0xB1, 0xF, 0xF, false)));
      float s;
      int32_t z;
      params_from_range(lo_b, hi_b, &s, &z);
      uint32_t q4[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t acc = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (k0 + 4 * q + j < K) acc |= quantize_one(v[4 * q + j], s, z) << (8 * j);
        q4[q] = acc;
      }
      // the 8-byte piece holding k = 128b + 32g + 8cc .. +8 goes to 128b + 32cc + 8g
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t kk = k0 + 8 * h;
        const int64_t b = kk >> 7, g = (kk >> 5) & 3, cc = (kk >> 3) & 3;
        *reinterpret_cast<uint2*>(qa_lds + b * 128 + cc * 32 + g * 8) =
            make_uint2(q4[2 * h], q4[2 * h + 1]);
      }
      if ((tid & 1) == 0) {
        bq_s[k0 >> 5] = s;
        bq_z[k0 >> 5] = z;
      }
    }
    __syncthreads();  // (1)
    __syncthreads();  // (2) the codes and block parameters
    __syncthreads();  // (3) the partial sums
  } else if (wave < NQ) {
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
      row_codes<QT, QE, true, false, true>(X, K, w.Kpad, xvec, true, qa_lds, s, z, first);
    else
      row_codes<QT, QE, true, false>(X, K, w.Kpad, xvec, true, qa_lds, s, z, first);
    __syncthreads();  // (2) the codes
    __syncthreads();  // (3) the partial sums
  } else {
    const int ww = wave - NQ;
    const int ch = lane >> 2, c = lane & 3;
    const uint8_t* wbase = w.data + tile * nb * 1024 + lane * 16;
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(w.scale + tile * nb * 64 * ES), 0, (uint32_t)(nb * 64 * ES),
        0x00020000);
    const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(kAsym ? w.offs + tile * nb * 256 : w.scale), 0,
        (uint32_t)(kAsym ? nb * 256 : 0), 0x00020000);
    // batches of BB blocks per wave: block (j*BB + u)*NWW + ww; past the end
    // the weights are re-read from the last block (clamped) and the scales
    // read as zeros
    const int64_t nbatch = (nb + (int64_t)NWW * BB - 1) / ((int64_t)NWW * BB);
    uint4 wv[BB];
    float4 sv[BB], ov[BB];
    int64_t blk[BB];
    auto load_batch = [&](int64_t j) {
#pragma unroll
      for (int u = 0; u < BB; ++u) {
        const int64_t b = (j * BB + u) * NWW + ww;
        blk[u] = b < nb ? b : nb - 1;
        wv[u] = *reinterpret_cast<const uint4*>(wbase + blk[u] * 1024);
        sv[u] = load_scale4_bounded<kBf16>(srs, (uint32_t)((b * 64 + ch * 4) * ES));
        if constexpr (kAsym)
          ov[u] = load_scale4_bounded<false>(ors, (uint32_t)((b * 64 + ch * 4) * 4));
        else
          ov[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    };
    float part = 0.0f;
    // Nothing may wait for the weights before the barriers, where the
    // quantizer waves wait for every wave: each block's fence keeps the first
    // use of its loads (the unpack) after them, and the blocks are taken in
    // the order their loads complete.
    auto compute_batch = [&]() {
      uint4 p0[BB], p1[BB];  // the codes first: their LDS reads need no weights
#pragma unroll
      for (int u = 0; u < BB; ++u) {
        const int8_t* ab = qa_lds + blk[u] * 128 + c * 32;
        p0[u] = *reinterpret_cast<const uint4*>(ab);
        p1[u] = *reinterpret_cast<const uint4*>(ab + 16);
      }
#pragma unroll
      for (int u = 0; u < BB; ++u) {
        asm volatile("" : "+v"(wv[u].x), "+v"(wv[u].y), "+v"(wv[u].z), "+v"(wv[u].w));
        const Nibbles nb4 = nibble_ops(wv[u]);
        const uint2 a[4] = {make_uint2(p0[u].x, p0[u].y), make_uint2(p0[u].z, p0[u].w),
                            make_uint2(p1[u].x, p1[u].y), make_uint2(p1[u].z, p1[u].w)};
        if constexpr (kBQ) {  // the block's four group parameters of the row
          const float4 sq = *reinterpret_cast<const float4*>(bq_s + 4 * blk[u]);
          const int4 zq = *reinterpret_cast<const int4*>(bq_z + 4 * blk[u]);
          const uint4 wq = wv[u];
          const int32_t e0 = word_dot16(wq.x, a[0].x, a[0].y) - zq.x * word_wsum16(wq.x);
          const int32_t e1 = word_dot16(wq.y, a[1].x, a[1].y) - zq.y * word_wsum16(wq.y);
          const int32_t e2 = word_dot16(wq.z, a[2].x, a[2].y) - zq.z * word_wsum16(wq.z);
          const int32_t e3 = word_dot16(wq.w, a[3].x, a[3].y) - zq.w * word_wsum16(wq.w);
          part = part + (sq.x * sv[u].x) * (float)e0;
          part = part + (sq.y * sv[u].y) * (float)e1;
          part = part + (sq.z * sv[u].z) * (float)e2;
          part = part + (sq.w * sv[u].w) * (float)e3;
        } else {
          gemv_block_terms<kKind>(nb4, a, sv[u], ov[u], part);
        }
      }
    };
    load_batch(0);
    // weight wave 0 also fetches the epilogue operands of the tile's channels
    // (after its weights: they are needed last)
    if (ww == 0 && lane < 16) {
      wsum_c = w.wsum[n_out];
      bias_c = (bias && n_out < w.N) ? bias[n_out] : 0.0f;
    }
    __syncthreads();  // (1)
    __syncthreads();  // (2): the codes are in LDS
    compute_batch();
    for (int64_t j = 1; j < nbatch; ++j) {
      load_batch(j);
      compute_batch();
    }
    // the four lanes of a channel: quad_perm [1,0,3,2] then [2,3,0,1]
    float p = part;
    p = p + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, p),
                                                                  0xB1, 0xF, 0xF, false));
    p = p + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, p),
                                                                  0x4E, 0xF, 0xF, false));
    if (c == 0) part_w[ww][ch] = p;
    __syncthreads();  // (3)
  }
  if (wave == NQ && lane < 16) {  // weight wave 0 writes the tile
    float S = 0.0f;
#pragma unroll
    for (int v = 0; v < NWW; ++v) S = S + part_w[v][lane];
    if constexpr (kBQ) {
      if (n_out < w.N) Y[n_out] = finish_bq(S, bias_c, lo, hi);
    } else {
      const float sa = row_param[0];
      const int32_t za = __builtin_bit_cast(int32_t, row_param[1]);
      if (n_out < w.N) Y[n_out] = finish(S, sa, za, wsum_c, bias_c, lo, hi);
    }
  }
}

// ---- GEMV on quantized rows: a workgroup per 16-channel tile --------------
// Lane l handles channel l/4 of the tile and 16-byte chunk c = l%4 of each
// of its wave's blocks (the 8-K piece c of four groups), so one wave load
// instruction reads one tile-block: 1 KiB in one piece.  Its four group
// scales are 16 bytes shared by the four lanes of the channel.  The
// quantized rows (M <= 4, row-major) are read from memory.  Partial sums
// are reduced across the four lanes of a channel with DPP and then across
// the waves through LDS, in a fixed order.  Rows m > 0 reuse the weights
// held in registers.
// kBQ: the activations were quantized per block of 32 (one scale and zero
// point per row and group, [M][ldsz]); one row.  Each group piece then
// contributes sa[g]*sw[g] * (dot - za[g] * sum q), exactly in integers up to
// that product.
template <int NT, int kKind, bool kBQ = false, int BB = 4>
__global__ __launch_bounds__(NT) void a8w4_gemv_kernel(const int8_t* __restrict__ qa_g,
                                                       int64_t lda, const float* __restrict__ sa_g,
                                                       const int32_t* __restrict__ za_g,
                                                       int64_t M, W4 w,
                                                       const float* __restrict__ bias, float lo,
                                                       float hi, float* __restrict__ Y,
                                                       int64_t ldy) {
  static_assert(!kBQ || kKind != 2, "per-block activations: symmetric weights");
  constexpr int NW = NT / 64;
  // BB: blocks a wave holds in registers per batch
  constexpr int MR = 4;      // rows per call (M <= 4)
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
  float sa_m[MR];
  int32_t za_m[MR];
  if constexpr (!kBQ) {
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
      } else {
        ov[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
      if constexpr (kBQ) {  // the row's four group parameters of this block
        saq[u] = *reinterpret_cast<const float4*>(sa_g + 4 * blk[u]);
        zaq[u] = *reinterpret_cast<const int4*>(za_g + 4 * blk[u]);
      }
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      if (m < M) {
#pragma unroll
        for (int u = 0; u < BB; ++u) {
          uint2 a[4];
          const int8_t* ab = qa_g + m * lda + blk[u] * 128 + c * 8;
#pragma unroll
          for (int t = 0; t < 4; ++t) a[t] = *reinterpret_cast<const uint2*>(ab + 32 * t);
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
          } else {
            gemv_block_terms<kKind>(nibble_ops(wq), a, sv[u], ov[u], part[m]);
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
      if constexpr (kBQ) {
        if (n_out < w.N) Y[m * ldy + n_out] = finish_bq(S, bias_c, lo, hi);
      } else {
        float sa = 0.0f;
        int32_t za = 0;
#pragma unroll
        for (int r = 0; r < MR; ++r)
          if (r == m) {
            sa = sa_m[r];
            za = za_m[r];
          }
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
// f32 chains (even and odd slots) per output.  Asymmetric weights make each
// group's term (scale * dot + offset * activation sum) large next to the
// output, so there the chains hold one block's four groups only and are
// added into an f64 sum after every block: an f32 sum over all of K would
// round by more than the output tolerance.  K-range partial sums are added
// in wave order through LDS.
// kBQ (activations quantized per block of 32: sa, za are [M][ldsz]): the
// MFMA is issued the other way round, (weights, activations), so a lane
// holds channels 4*(l/16)+i of row l%16 and needs one row's group
// parameters.  The group's integer sum over (q - za) * w is one MFMA chain:
// the weights against ones (sum w, shared by the rows), then against the
// codes, then against ~za replicated over K (~za = -za - 1, which fits a
// byte where -za may not); each group then adds sa*sw times that sum per
// output.  The block's weight scales and the rows' group parameters travel
// with the codes through the LDS ring (4-byte direct loads), so only the
// weights are held in registers ahead of use.
// PW: weight prefetch depth in blocks.  kExact: every K range holds a
// multiple of 2*PW blocks (the host checks), so no step runs past its range
// and the per-step range test and zeroed scales drop out.
template <int FM, int FN, int RW, int CW, int KS, bool kPerm, int kKind, bool kBQ = false,
          int PW = 3, bool kExact = false>
__global__ __launch_bounds__(256) void a8w4_gemm_kernel(const int8_t* __restrict__ qa,
                                                        int64_t lda, const float* __restrict__ sa_g,
                                                        const int32_t* __restrict__ za_g,
                                                        int64_t M, W4 w,
                                                        const float* __restrict__ bias, float lo,
                                                        float hi, float* __restrict__ Y,
                                                        int64_t ldy, int64_t ldsz) {
  static_assert(!kBQ || kKind != 2, "per-block activations take symmetric weights");
  static_assert(RW * CW * KS == 4, "four waves");
  constexpr int P = PW;                     // weight prefetch depth in blocks
  constexpr int R = 4;                      // activation ring stages
  constexpr int MT = 16 * FM * RW;          // rows per workgroup
  constexpr int SLOTS = KS * MT * 8;        // 16-byte pieces per stage
  constexpr int ND = SLOTS / 256;           // direct loads per thread per stage
  constexpr int STAGE = SLOTS * 16;         // bytes of codes per stage
  static_assert(SLOTS % 256 == 0, "a stage must split evenly over the workgroup");
  // kBQ: after the codes, each stage holds the block's weight scales of the
  // workgroup's tiles, [K range][tile][64 values] (256 bytes a tile; bf16
  // scales fill the first half), and the rows' group parameters,
  // [K range][sa, za][row][4 groups]; both arrive as 4-byte direct loads,
  // NS and NP per thread.
  constexpr int SCB = kBQ ? KS * CW * FN * 256 : 0;
  constexpr int PAB = kBQ ? KS * MT * 32 : 0;
  constexpr int NS = SCB / 1024, NP = PAB / 1024;
  static_assert(SCB % 1024 == 0 && PAB % 1024 == 0, "kBQ: stage extras must split evenly");
  constexpr int STRIDE = STAGE + SCB + PAB;  // bytes per stage
  // Each wave its own K range (one row and one channel group): a wave loads
  // and reads only its own rows of a stage, so the waves need no barrier in
  // the K loop and run decoupled (a late weight block stalls only its wave).
  constexpr bool kPrivA = RW * CW == 1;
  static_assert(!kPrivA || MT * 8 == 64 * ND, "a wave's rows of a stage: ND loads per lane");
  // (kBQ without a barrier: a wave's scale and parameter pieces must be its
  // own K range's, which the piece mapping below gives for one tile a
  // workgroup, four K ranges and one scale piece a thread)
  static_assert(!kBQ || !kPrivA || (KS == 4 && CW * FN == 1 && NS == 1), "kBQ wave-private ring");
  // KS = 1: behind the stages, the epilogue operands of the workgroup's
  // channels and rows ([NCH] weight sums, [NCH] biases, [MT] row scales,
  // [MT] row zero points), written once after the prologue
  constexpr int NCH = CW * FN * 16;  // channels per workgroup
  constexpr bool kEpLds = KS == 1;
  constexpr int EPB = kEpLds ? (2 * NCH + 2 * MT) * 4 : 0;
  static_assert(!kEpLds || (NCH <= 256 && MT <= 256), "one epilogue operand per thread");
  __shared__ __attribute__((aligned(16))) int8_t ring[R * STRIDE + EPB];
  __shared__ float red[KS > 1 ? (KS - 1) * RW * CW : 1][FM][FN][4][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ks = wave % KS;
  const int cw = (wave / KS) % CW;
  const int rw = wave / (KS * CW);
  const int slot = rw * CW + cw;
  const int c = lane >> 4;
  // Workgroups are dispatched round-robin over the 8 XCDs in launch order
  // (x fastest).  Remapped so that each XCD takes a contiguous run of
  // (channel group, row group) pairs, row groups fastest: the row groups of
  // one channel group then share their weight tiles through one L2.
  const uint32_t gx = gridDim.x, gy = gridDim.y;
  uint32_t lin = blockIdx.y * gx + blockIdx.x;
  if (gy > 1 && ((gx * gy) & 7) == 0) lin = (lin & 7) * ((gx * gy) >> 3) + (lin >> 3);
  const uint32_t cgi = gy > 1 ? lin / gy : blockIdx.x, rgi = gy > 1 ? lin % gy : blockIdx.y;
  const int64_t n0 = ((int64_t)cgi * CW + cw) * 16 * FN;  // n0 + 16*FN <= Npad
  const int64_t mw = (int64_t)rgi * MT;                    // workgroup's first row
  // (block indices in 32 bits, wave-uniform: the clamps below are scalar
  // compares; the host keeps Kpad <= 2^24)
  const int nblocks = (int)(w.Kpad / 128);
  const int bpw = (nblocks + KS - 1) / KS;  // blocks per K range
  // every K range runs bpw steps; steps past its end are clamped to its last
  // block and contribute with zero scales
  auto range_block = [&](int r, int j) {
    const int b_begin = r * bpw;
    int last = (b_begin + bpw < nblocks ? b_begin + bpw : nblocks) - 1;
    if (last < b_begin) last = nblocks - 1;  // empty range: park on a real block
    const int b = b_begin + j;
    return (int64_t)(b < last ? b : last);
  };
  const int my_end = (ks * bpw + bpw < nblocks ? ks * bpw + bpw : nblocks);

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
    ssrc[q] = w.scale + ((n >> 4) * w.nblk * 64 + (lane & 15) * 4) * ES;
    osrc[q] = kAsym ? w.offs + ((n >> 4) * w.nblk * 64 + (lane & 15) * 4) * 4 : nullptr;
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
    // (wave-uniform: kept in a scalar register, so the range clamps of the
    // direct loads are scalar compares)
    a_rng[i] = __builtin_amdgcn_readfirstlane(kPrivA ? wave : (32 * i + 8 * wave) / MT);
    const int p = (s & 7) ^ ((r >> 1) & 7);
    int64_t m = mw + r;
    m = m < M ? m : M - 1;
    a_voff[i] = (uint32_t)((m - mw) * lda + 16 * p);
  }
  // kBQ: this thread's scale and parameter pieces.  Piece i of a wave is
  // the 64-dword chunk wave + 4i: of the scales, chunk -> (K range, tile);
  // of the parameters, chunk -> (K range, sa or za, 16 rows), lane -> (row
  // lane/4, group lane%4).  Rows past M repeat row M-1.
  constexpr int NSA = NS > 0 ? NS : 1, NPA = NP > 0 ? NP : 1;
  const uint8_t* sc_base[NSA];
  int sc_rng[NSA], sc_dst[NSA];
  const void* pa_base[NPA];
  int pa_rng[NPA], pa_dst[NPA];
  uint32_t pa_voff[NPA];
  const uint32_t sc_voff = kBf16 ? 4u * (lane & 31) : 4u * lane;  // bf16: 128 bytes a tile
  if constexpr (kBQ) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int ch = wave + 4 * i;
      sc_rng[i] = ch / (CW * FN);
      sc_base[i] = w.scale + ((int64_t)cgi * CW * FN + ch % (CW * FN)) * w.nblk * 64 * ES;
      sc_dst[i] = STAGE + ch * 256;
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int ch = wave + 4 * i;
      const int kr = ch % KS, within = ch / KS;
      const int kind = within / (MT / 16), rb = within % (MT / 16);
      pa_rng[i] = kr;
      pa_base[i] = kind ? (const void*)(za_g + mw * ldsz) : (const void*)(sa_g + mw * ldsz);
      int64_t m = mw + rb * 16 + (lane >> 2);
      m = m < M ? m : M - 1;
      pa_voff[i] = (uint32_t)(((m - mw) * ldsz + (lane & 3)) * 4);
      pa_dst[i] = STAGE + SCB + ((kr * 2 + kind) * MT + rb * 16) * 16;
    }
  }
  auto issue_stage = [&](int j) {
    lds_i8* st = (lds_i8*)ring + (int)(j % R) * STRIDE;
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      const int64_t b = range_block(a_rng[i], j);
      const int s0 = kPrivA ? wave * (MT * 8) + 64 * i : 256 * i + 64 * wave;  // lane 0's slot
      dma16_to_lds(a_base, (lds_void_t*)(st + s0 * 16), a_voff[i],
                   (uint32_t)(b * 128));
    }
    if constexpr (kBQ) {
#pragma unroll
      for (int i = 0; i < NS; ++i)
        dma4_to_lds(sc_base[i], (lds_void_t*)(st + sc_dst[i]), sc_voff,
                    (uint32_t)(range_block(sc_rng[i], j) * 64 * ES));
#pragma unroll
      for (int i = 0; i < NP; ++i)
        dma4_to_lds(pa_base[i], (lds_void_t*)(st + pa_dst[i]), pa_voff[i],
                    (uint32_t)(range_block(pa_rng[i], j) * 16));
    }
  };

  // ---- accumulators ----
  // (f64 sums: asymmetric weights after every block; per-block activations
  // after every PR blocks, so that the f32 chains stay short at deep K)
  constexpr bool kD = kAsym || kBQ;
  float acc[2][FM][FN][4];
  double accd[kD ? FM : 1][kD ? FN : 1][4];
#pragma unroll
  for (int f = 0; f < (kD ? FM : 1); ++f)
#pragma unroll
    for (int q = 0; q < (kD ? FN : 1); ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) accd[f][q][i] = 0.0;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int q = 0; q < FN; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[h][f][q][i] = 0.0f;

  // The weight ring holds PR = 2P slots when K ranges are exact: step u
  // consumes slot u and refills slot (u + P) % PR, which nothing reads any
  // more, so the refill needs no register copies at the loop's back edge.
  constexpr int PR = kExact ? 2 * P : P;
  uint4 wr[PR][FN];
  float4 sr[kBQ ? 1 : PR][FN], orr[PR][FN];
  auto load_w = [&](int u, int64_t b) {
#pragma unroll
    for (int q = 0; q < FN; ++q) {
      wr[u][q] = *reinterpret_cast<const uint4*>(wsrc[q] + b * 1024);
      if constexpr (!kBQ) sr[u][q] = load_scale4<kBf16>(ssrc[q] + 64 * ES * b);
      if constexpr (kAsym) orr[u][q] = load_scale4<false>(osrc[q] + 64 * 4 * b);
    }
  };

  // one block: activation operands from the stage, MFMAs, refill, rescale
  auto step = [&](int u, int j) {
    const lds_i8* stage = (const lds_i8*)ring + (int)(j % R) * STRIDE;
    const lds_i8* st = stage + ks * MT * 128;
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
    const bool live = kExact || ks * bpw + j < my_end;
    if constexpr (kBQ) {
      // the block's weight scales of channels 4c..4c+3 (16 consecutive
      // values of the tile's 64) and the rows' group parameters, from the
      // stage; past the end of the K range the row scales are zeroed
      float4 s4[FN][4], a4[FM];
      int4 zq[FM];
#pragma unroll
      for (int q = 0; q < FN; ++q) {
        const lds_i8* sp = stage + STAGE + ((ks * CW + cw) * FN + q) * 256;
        if constexpr (kBf16) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const u32x4 u = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
                sp + 32 * c + 16 * h);
            s4[q][2 * h] = make_float4(__builtin_bit_cast(float, u.x << 16),
                                       __builtin_bit_cast(float, u.x & 0xFFFF0000u),
                                       __builtin_bit_cast(float, u.y << 16),
                                       __builtin_bit_cast(float, u.y & 0xFFFF0000u));
            s4[q][2 * h + 1] = make_float4(__builtin_bit_cast(float, u.z << 16),
                                           __builtin_bit_cast(float, u.z & 0xFFFF0000u),
                                           __builtin_bit_cast(float, u.w << 16),
                                           __builtin_bit_cast(float, u.w & 0xFFFF0000u));
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            s4[q][i] = lds_f4(sp + 64 * c + 16 * i);
        }
      }
#pragma unroll
      for (int f = 0; f < FM; ++f) {
        const int r = rw * 16 * FM + f * 16 + (lane & 15);
        const lds_i8* pp = stage + STAGE + SCB + (ks * 2 * MT + r) * 16;
        a4[f] = lds_f4(pp);
        const u32x4 z4 = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
            pp + MT * 16);
        zq[f] = make_int4((int)z4.x, (int)z4.y, (int)z4.z, (int)z4.w);
        if (!live) a4[f] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int q = 0; q < FN; ++q) cw4[q] = wr[u][q];
      load_w((u + P) % PR, range_block(ks, j + P));
#pragma unroll
      for (int t2 = 0; t2 < 4; t2 += 2) {
        v4i d[2][FM][FN];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int t = t2 + h;
#pragma unroll
          for (int q = 0; q < FN; ++q) {
            const uint32_t wd = h == 0 ? (t2 == 0 ? cw4[q].x : cw4[q].z)
                                       : (t2 == 0 ? cw4[q].y : cw4[q].w);
            const long bop = (long)(((uint64_t)nib_hi16(wd) << 32) | nib_lo16(wd));
            // 16 * sum w of the group, the same for every row
            const v4i ws16 = __builtin_amdgcn_mfma_i32_16x16x32_i8(
                bop, (long)0x0101010101010101LL, v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
            for (int f = 0; f < FM; ++f) {
              const long aop = (long)(((uint64_t)ca[f][t].y << 32) | ca[f][t].x);
              const int32_t z = t == 0 ? zq[f].x : (t == 1 ? zq[f].y : (t == 2 ? zq[f].z : zq[f].w));
              const uint32_t nz = ~__builtin_amdgcn_perm((uint32_t)z, (uint32_t)z, 0u);
              const long zop = (long)(((uint64_t)nz << 32) | nz);
              // 16 * (sum w + sum q*w + sum (-za - 1)*w) = 16 * sum (q - za)*w
              d[h][f][q] = __builtin_amdgcn_mfma_i32_16x16x32_i8(
                  bop, zop, __builtin_amdgcn_mfma_i32_16x16x32_i8(bop, aop, ws16, 0, 0, 0), 0,
                  0, 0);
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
                acc[h][f][q][i] = __builtin_fmaf(ar * sc, (float)d[h][f][q][i], acc[h][f][q][i]);
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
    load_w((u + P) % PR, range_block(ks, j + P));
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
    if constexpr (kAsym) {  // the block's sum into the f64 one
#pragma unroll
      for (int f = 0; f < FM; ++f)
#pragma unroll
        for (int q = 0; q < FN; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            accd[f][q][i] = accd[f][q][i] + (double)(acc[0][f][q][i] + acc[1][f][q][i]);
            acc[0][f][q][i] = 0.0f;
            acc[1][f][q][i] = 0.0f;
          }
    }
  };

  // ---- prologue: stages 0..R-2 and weights of blocks 0..P-1, all drained ----
#pragma unroll
  for (int j = 0; j < R - 1; ++j) issue_stage(j);
#pragma unroll
  for (int u = 0; u < P; ++u) load_w(u, range_block(ks, u));
  // The epilogue operands come in with the prologue, which is drained
  // anyway: loaded after the main loop they put a memory round trip (the
  // weight sums live in the cold blob) between the final sums and the
  // stores.  Unconditional loads (clamped indices, a stand-in array where
  // there is no bias).  With K split over the waves (KS > 1) the writing
  // waves (K range 0) keep theirs in registers; with KS = 1 every wave
  // writes, and registers held through the loop would cost a wave a SIMD,
  // so one thread per channel and row loads them and they wait in LDS
  // behind the ring's stages (in an LDS array of their own they made the
  // compiler drain the direct loads at every step).
  constexpr bool kEpPre = KS > 1;
  constexpr int EW = kEpPre ? (kBQ ? 4 : 1) : 1;  // channel values per fragment
  float e_ws[kEpPre ? FN : 1], e_bn[kEpPre ? FN : 1][EW], e_sa[kEpPre && !kBQ ? FM : 1][4];
  int32_t e_za[kEpPre && !kBQ ? FM : 1][4];
  if constexpr (kEpPre) {
    if (ks == 0) {
#pragma unroll
      for (int q = 0; q < FN; ++q) {
#pragma unroll
        for (int i = 0; i < EW; ++i) {
          const int64_t n = n0 + q * 16 + (kBQ ? 4 * c + i : (lane & 15));
          e_bn[q][i] = (bias ? bias : w.wsum)[n < w.N ? n : w.N - 1];
          if (!kBQ) e_ws[q] = w.wsum[n];
        }
      }
      if constexpr (!kBQ) {
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t m = mw + rw * 16 * FM + f * 16 + 4 * c + i;
            e_sa[f][i] = sa_g[m < M ? m : M - 1];
            e_za[f][i] = za_g[m < M ? m : M - 1];
          }
      }
    }
  }
  const int64_t ng0 = (int64_t)cgi * NCH;  // the workgroup's first channel (ng0 + NCH <= Npad)
  float* const ep_ws = reinterpret_cast<float*>(ring + R * STRIDE);
  float* const ep_bn = ep_ws + NCH;
  float* const ep_sa = ep_bn + NCH;
  int32_t* const ep_za = reinterpret_cast<int32_t*>(ep_sa + MT);
  float l_ws = 0.0f, l_bn = 0.0f, l_sa = 0.0f;
  int32_t l_za = 0;
  if constexpr (kEpLds) {
    if (tid < NCH) {
      const int64_t n = ng0 + tid;
      if constexpr (!kBQ) l_ws = w.wsum[n];
      l_bn = (bias ? bias : w.wsum)[n < w.N ? n : w.N - 1];
    }
    if constexpr (!kBQ) {
      if (tid < MT) {
        const int64_t m = mw + tid < M ? mw + tid : M - 1;
        l_sa = sa_g[m];
        l_za = za_g[m];
      }
    }
  }
  wait_vmcnt<0>();
  if constexpr (kEpLds) {
    if (tid < NCH) {
      ep_ws[tid] = l_ws;
      ep_bn[tid] = l_bn;
    }
    if (tid < MT) {
      ep_sa[tid] = l_sa;
      ep_za[tid] = l_za;
    }
  }
  // lgkmcnt(0): settle the scalar loads (and the LDS writes above, which the
  // main loop's barriers order before the epilogue's reads)
  __builtin_amdgcn_s_waitcnt(0xC07F);

  // Loads issued after stage j+1's direct loads, in the steady state: the
  // weights refilled by step j+2-R, and R-2 whole steps (direct loads and a
  // weight refill each).  Earlier stages were drained in the prologue.
  // loads per weight refill: weights and scales (kBQ: the weights only;
  // asymmetric: the offsets too); direct loads per stage: the codes (kBQ:
  // and the scale and parameter pieces)
  constexpr int LW = kBQ ? FN : (kAsym ? 3 * FN : 2 * FN);
  constexpr int A_WAIT = LW + (R - 2) * (ND + NS + NP + LW);
  static_assert(A_WAIT < 64, "vmcnt range");
  // The step loop is unrolled by PR so the weight ring index is static.
  for (int j0 = 0; j0 < bpw; j0 += PR) {
#pragma unroll
    for (int u = 0; u < PR; ++u) {
      const int j = j0 + u;
      // (past the last step the body still runs, with zero scales, so that
      // every iteration issues the same loads)
      wait_vmcnt<A_WAIT>();
      if constexpr (!kPrivA) asm volatile("s_barrier" ::: "memory");
      issue_stage(j + R - 1);
      step(u, j);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (kBQ) {  // the f32 chains of these PR blocks into the f64 sums
#pragma unroll
      for (int f = 0; f < FM; ++f)
#pragma unroll
        for (int q = 0; q < FN; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            accd[f][q][i] = accd[f][q][i] + (double)(acc[0][f][q][i] + acc[1][f][q][i]);
            acc[0][f][q][i] = 0.0f;
            acc[1][f][q][i] = 0.0f;
          }
    }
  }
  wait_vmcnt<0>();  // the clamped direct loads must land before the workgroup ends

  float out[FM][FN][4];
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int q = 0; q < FN; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (kAsym)
          out[f][q][i] = (float)accd[f][q][i];
        else if constexpr (kBQ)
          out[f][q][i] = (float)accd[f][q][i];
        else
          out[f][q][i] = acc[0][f][q][i] + acc[1][f][q][i];
      }
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
          float bn = 0.0f;
          if (bias) {
            if constexpr (kEpPre) bn = e_bn[q][i];
            else bn = ep_bn[n - ng0];
          }
          if (n < w.N) Y[m * ldy + n] = finish_bq(out[f][q][i], bn, lo, hi);
        }
    }
    return;
  }
#pragma unroll
  for (int q = 0; q < FN; ++q) {
    const int64_t n = n0 + q * 16 + (lane & 15);
    if (n >= w.N) continue;
    float ws, bn = 0.0f;
    if constexpr (kEpPre) {
      ws = e_ws[q];
      if (bias) bn = e_bn[q][0];
    } else {
      ws = ep_ws[n - ng0];
      if (bias) bn = ep_bn[n - ng0];
    }
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = mw + rw * 16 * FM + f * 16 + 4 * c + i;
        if (m < M) {
          if constexpr (kEpPre) {
            Y[m * ldy + n] = finish(out[f][q][i], e_sa[f][i], e_za[f][i], ws, bn, lo, hi);
          } else {
            const int ml = (int)(m - mw);  // the row within the workgroup
            Y[m * ldy + n] = finish(out[f][q][i], ep_sa[ml], ep_za[ml], ws, bn, lo, hi);
          }
        }
      }
  }
}

// ---- GEMM for at most 16 rows and K <= 4096 --------------------------------
// A workgroup of 4*TPW waves covers TPW 16-channel tiles (two or three) and
// all of K: wave w takes tile w%TPW and K range w/TPW (a quarter of the
// 128-K blocks, at most BPW).  The 16 rows of activation codes go from memory
// straight into LDS once per workgroup (rows padded by 16 bytes, so that
// the 16 rows a read instruction touches fall in different banks); every
// activation read after that is an LDS read.  Reading the codes from
// memory in every wave instead (16 KiB per wave, the same lines in every
// workgroup) measured slower than the whole weight stream.  Two tiles a
// workgroup measured fastest of one, two and four (one: the codes are read
// twice as often; four: a quarter of the CUs get no workgroup); three, where
// they fit one workgroup a CU, beat two that put two workgroups on some CUs
// (11008 channels: 13.9-14.2 against 15.0 us with the row quantization).
// Each wave issues every weight and scale load of its range before it
// waits for anything; it then waits only for the codes (issued first, so
// complete first) and computes block by block as the weights arrive.  The
// four K ranges of a tile are summed in a fixed order.  The arithmetic per
// block is that of a8w4_gemm_kernel.
// kExact: K is exactly four ranges of BPW blocks, so every block of every
// range is real and the scales need no zeroing.
template <int BPW, bool kPerm, int kKind, bool kExact = false, int TPW = 2>
__global__ __launch_bounds__(TPW * 256) void a8w4_gemm_m16_kernel(
    const int8_t* __restrict__ qa, int64_t lda, const float* __restrict__ sa_g,
    const int32_t* __restrict__ za_g, int64_t M, W4 w, const float* __restrict__ bias, float lo,
    float hi, float* __restrict__ Y, int64_t ldy) {
  constexpr bool kBf16 = kKind == 1, kAsym = kKind == 2;
  constexpr int ES = kBf16 ? 2 : 4;  // bytes per stored scale
  constexpr int NW = 4 * TPW;        // waves: TPW tiles x 4 K ranges
  extern __shared__ __attribute__((aligned(16))) int8_t a_lds[];  // [16][Kpad + 16]
  __shared__ float red[3][TPW][4][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tq = wave % TPW;  // the wave's tile
  const int ks = wave / TPW;  // and K range
  const int c = lane >> 4;
  // tiles w, w + G, ... of the G-workgroup grid: neighbouring workgroups
  // read neighbouring tiles, which measured 12% faster than consecutive
  // tiles per workgroup with the weights cache-resident (the same cold).
  // A grid that covers the tiles unevenly gives its last tiles' waves the
  // final tile again: they load and compute like the others (every wave
  // takes part in the barriers) and store nothing.
  const int64_t ntile = w.Npad / 16;
  const int64_t tile_g = (int64_t)tq * gridDim.x + blockIdx.x;
  const bool tile_real = tile_g < ntile;
  const int64_t tile = tile_real ? tile_g : ntile - 1;
  const int64_t nblocks = w.Kpad / 128;
  const int64_t bpw = (nblocks + 3) / 4;
  const int64_t b0 = ks * bpw;
  const int64_t b_end = b0 + bpw < nblocks ? b0 + bpw : nblocks;
  const int64_t astr = w.Kpad + 16;  // LDS row stride

  // ---- the codes: 16 rows x Kpad bytes straight into LDS, in 1 KiB pieces
  // (a piece: 64 lanes x 16 bytes of one row); wave w takes pieces
  // w, w+NW, ...  Rows past M repeat row M-1 (their outputs are not written).
  const int ppr = (int)((w.Kpad + 1023) / 1024);  // pieces per row (<= 4)
  for (int pc = wave; pc < 16 * ppr; pc += NW) {
    const int r = pc / ppr, j = pc - r * ppr;
    const int64_t rr = r < M ? r : M - 1;
    if (j * 1024 + lane * 16 < w.Kpad)
      dma16_to_lds(qa, (lds_void_t*)((lds_i8*)a_lds + r * astr + j * 1024),
                   (uint32_t)(rr * lda + j * 1024 + lane * 16), 0);
  }
  __builtin_amdgcn_sched_barrier(0);  // the codes' loads first

  // ---- the epilogue operands of the waves that write the tile (K range 0),
  // issued before the weights: loaded after the last barrier they put a
  // memory round trip (the weight sums live in the cold blob) between the
  // final sums and the stores of every workgroup, which measured about
  // 1 us at 16 x 11008.  Issued ahead of the weights, the waits for the
  // weights stay the same in every wave.  Every load is unconditional
  // (clamped indices, a stand-in array where there is no bias).
  constexpr int NL = (kAsym ? 3 : 2) * BPW;  // weight-side loads of a wave
  const int64_t n_e = tile * 16 + (lane & 15);
  float ws_e = 0.0f, bn_e = 0.0f, sa_e[4] = {0.f, 0.f, 0.f, 0.f};
  int32_t za_e[4] = {0, 0, 0, 0};
  if (ks == 0) {
    const int64_t nb_c = n_e < w.N ? n_e : w.N - 1;
    ws_e = w.wsum[n_e];  // [Npad]
    bn_e = (bias ? bias : w.wsum)[nb_c];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = 4 * c + i < M ? 4 * c + i : M - 1;
      sa_e[i] = sa_g[m];
      za_e[i] = za_g[m];
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- every weight and scale load of the range (blocks past the range
  // read the range's last real block and get zero scales below)
  const int8_t* const wp =
      reinterpret_cast<const int8_t*>(w.data) + tile * w.nblk * 1024 + (lane & 15) * 64 + 16 * c;
  const uint8_t* const sp = w.scale + (tile * w.nblk * 64 + (lane & 15) * 4) * ES;
  const uint8_t* const op = kAsym ? w.offs + (tile * w.nblk * 64 + (lane & 15) * 4) * 4 : nullptr;
  uint4 wr[BPW];
  float4 sr[BPW], orr[kAsym ? BPW : 1];
#pragma unroll
  for (int u = 0; u < BPW; ++u) {
    const int64_t b = b0 + u < nblocks ? b0 + u : nblocks - 1;
    wr[u] = *reinterpret_cast<const uint4*>(wp + b * 1024);
    sr[u] = load_scale4<kBf16>(sp + 64 * ES * b);
    if constexpr (kAsym) orr[u] = load_scale4<false>(op + 256 * b);
  }
  // the codes (issued first, so complete first; then the epilogue
  // operands) are in LDS once no more than the weight loads are outstanding
  wait_vmcnt<NL>();
  __syncthreads();

  float acc[2][4];
  double accd[kAsym ? 4 : 1];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[0][i] = acc[1][i] = 0.0f;
    if constexpr (kAsym) accd[i] = 0.0;
  }
  const int8_t* const arow = a_lds + (lane & 15) * astr;
#pragma unroll
  for (int u = 0; u < BPW; ++u) {
    const int64_t b = b0 + u < nblocks ? b0 + u : nblocks - 1;
    uint2 ar[4];
    const int8_t* ab = arow + b * 128;
    if constexpr (kPerm) {  // the 32 bytes of chunk c's four pieces are contiguous
      const uint4 p0 = *reinterpret_cast<const uint4*>(ab + 32 * c);
      const uint4 p1 = *reinterpret_cast<const uint4*>(ab + 32 * c + 16);
      ar[0] = make_uint2(p0.x, p0.y);
      ar[1] = make_uint2(p0.z, p0.w);
      ar[2] = make_uint2(p1.x, p1.y);
      ar[3] = make_uint2(p1.z, p1.w);
    } else {  // piece t of chunk c: bytes 32t + 8c
#pragma unroll
      for (int t = 0; t < 4; ++t) ar[t] = *reinterpret_cast<const uint2*>(ab + 32 * t + 8 * c);
    }
    // a block outside the range contributes 0 * (finite dot) = 0
    float4 cs = sr[u];
    float4 co = make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (kAsym) co = orr[u];
    if constexpr (!kExact) {
      const float keep = b0 + u < b_end ? 1.0f : 0.0f;
      cs = make_float4(cs.x * keep, cs.y * keep, cs.z * keep, cs.w * keep);
      if constexpr (kAsym) co = make_float4(co.x * keep, co.y * keep, co.z * keep, co.w * keep);
    }
#pragma unroll
    for (int t2 = 0; t2 < 4; t2 += 2) {
      v4i d[2], e[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int t = t2 + h;
        const uint32_t wd = t == 0 ? wr[u].x : (t == 1 ? wr[u].y : (t == 2 ? wr[u].z : wr[u].w));
        const long bop = (long)(((uint64_t)nib_hi16(wd) << 32) | nib_lo16(wd));
        const long aop = (long)(((uint64_t)ar[t].y << 32) | ar[t].x);
        d[h] = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop, bop, v4i{0, 0, 0, 0}, 0, 0, 0);
        if constexpr (kAsym)
          e[h] = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop, (long)0x1010101010101010LL,
                                                       v4i{0, 0, 0, 0}, 0, 0, 0);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int t = t2 + h;
        const float sc = t == 0 ? cs.x : (t == 1 ? cs.y : (t == 2 ? cs.z : cs.w));
        if constexpr (kAsym) {
          const float oc = t == 0 ? co.x : (t == 1 ? co.y : (t == 2 ? co.z : co.w));
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[h][i] = acc[h][i] + __builtin_fmaf(oc, (float)e[h][i], sc * (float)d[h][i]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[h][i] = __builtin_fmaf(sc, (float)d[h][i], acc[h][i]);
        }
      }
    }
    if constexpr (kAsym) {  // the block's sum into the f64 one
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        accd[i] = accd[i] + (double)(acc[0][i] + acc[1][i]);
        acc[0][i] = acc[1][i] = 0.0f;
      }
    }
  }
  float out[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = kAsym ? (float)accd[kAsym ? i : 0] : acc[0][i] + acc[1][i];

  // ---- the four K ranges of each tile, summed in a fixed order
  if (ks > 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) red[ks - 1][tq][i][lane] = out[i];
  }
  __syncthreads();
  if (ks != 0 || !tile_real) return;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 3; ++r) out[i] = out[i] + red[r][tq][i][lane];
  if (n_e >= w.N) return;
  const float bn = bias ? bn_e : 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = 4 * c + i;
    if (m < M) Y[m * ldy + n_e] = finish(out[i], sa_e[i], za_e[i], ws_e, bn, lo, hi);
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

// Largest Kpad of the fused GEMV: its codes live in the workgroup's LDS,
// which stays within the 64 KiB a launch gets without raising its limit.
constexpr int64_t kFusedGemvMaxKpad = 32768;

// M = 1 from f32: the wave-specialized kernel.  4 quantizer waves of 16
// values a thread and 8 weight waves of four blocks a batch (768 threads)
// measured faster than 8 + 8, 4 + 12 or 8 + 4.
qp_status launch_gemv_fused(const float* X, int64_t K, const W4& w, const float* bias, float lo,
                            float hi, float* Y, hipStream_t stream) {
  const unsigned blocks = (unsigned)(w.Npad / 16);
  const size_t lds = (size_t)w.Kpad;
  constexpr int NQ = 4, NWW = 8, BB = 4, QE = 16;
  if (w.kind == 1)
    hipLaunchKernelGGL((a8w4_gemv_fused_kernel<NQ, NWW, BB, QE, 1>), dim3(blocks),
                       dim3((NQ + NWW) * 64), lds, stream, X, K, w, bias, lo, hi, Y);
  else if (w.kind == 2)
    hipLaunchKernelGGL((a8w4_gemv_fused_kernel<NQ, NWW, BB, QE, 2>), dim3(blocks),
                       dim3((NQ + NWW) * 64), lds, stream, X, K, w, bias, lo, hi, Y);
  else
    hipLaunchKernelGGL((a8w4_gemv_fused_kernel<NQ, NWW, BB, QE, 0>), dim3(blocks),
                       dim3((NQ + NWW) * 64), lds, stream, X, K, w, bias, lo, hi, Y);
  return check_launch("a8w4 gemv");
}

// M = 1 from f32 with the row quantized per block of 32 inside the GEMV
// (symmetric weights: f32 or bf16 scales); LDS holds the codes and the
// blocks' parameters.
qp_status launch_gemv_fused_bq(const float* X, int64_t K, const W4& w, const float* bias,
                               float lo, float hi, float* Y, hipStream_t stream) {
  const unsigned blocks = (unsigned)(w.Npad / 16);
  const size_t lds = (size_t)w.Kpad + 8 * (size_t)(w.Kpad / 32);
  constexpr int NQ = 4, NWW = 8, BB = 4, QE = 16;
  if (w.kind == 1)
    hipLaunchKernelGGL((a8w4_gemv_fused_kernel<NQ, NWW, BB, QE, 1, true>), dim3(blocks),
                       dim3((NQ + NWW) * 64), lds, stream, X, K, w, bias, lo, hi, Y);
  else
    hipLaunchKernelGGL((a8w4_gemv_fused_kernel<NQ, NWW, BB, QE, 0, true>), dim3(blocks),
                       dim3((NQ + NWW) * 64), lds, stream, X, K, w, bias, lo, hi, Y);
  return check_launch("a8w4 gemv (per-block activations)");
}

// M <= 4 quantized rows (row-major, lda >= Kpad).
qp_status launch_gemv(const int8_t* qa, int64_t lda, const float* sa, const int32_t* za, int64_t M,
                      const W4& w, const float* bias, float lo, float hi, float* Y, int64_t ldy,
                      hipStream_t stream) {
  QP_REQUIRE(M <= 4, QP_EUNSUPPORTED, "a8w4 gemv: at most 4 rows");
  constexpr int NT = 512;
  const unsigned blocks = (unsigned)(w.Npad / 16);
  if (w.kind == 1)
    hipLaunchKernelGGL((a8w4_gemv_kernel<NT, 1>), dim3(blocks), dim3(NT), 0, stream, qa, lda, sa,
                       za, M, w, bias, lo, hi, Y, ldy);
  else if (w.kind == 2)
    hipLaunchKernelGGL((a8w4_gemv_kernel<NT, 2>), dim3(blocks), dim3(NT), 0, stream, qa, lda, sa,
                       za, M, w, bias, lo, hi, Y, ldy);
  else
    hipLaunchKernelGGL((a8w4_gemv_kernel<NT, 0>), dim3(blocks), dim3(NT), 0, stream, qa, lda, sa,
                       za, M, w, bias, lo, hi, Y, ldy);
  return check_launch("a8w4 gemv");
}

// One row quantized per block: sa, za hold the row's group parameters.
qp_status launch_gemv_bq(const int8_t* qa, const float* sa, const int32_t* za, const W4& w,
                         const float* bias, float lo, float hi, float* Y, hipStream_t stream) {
  constexpr int NT = 512;
  const unsigned blocks = (unsigned)(w.Npad / 16);
  if (w.kind == 1)
    hipLaunchKernelGGL((a8w4_gemv_kernel<NT, 1, true>), dim3(blocks), dim3(NT), 0, stream, qa,
                       w.Kpad, sa, za, 1, w, bias, lo, hi, Y, w.N);
  else
    hipLaunchKernelGGL((a8w4_gemv_kernel<NT, 0, true>), dim3(blocks), dim3(NT), 0, stream, qa,
                       w.Kpad, sa, za, 1, w, bias, lo, hi, Y, w.N);
  return check_launch("a8w4 gemv (per-block activations)");
}

template <int FM, int FN, int RW, int CW, int KS, int PW = 3, bool kExact = false>
qp_status launch_gemm_cfg(const int8_t* qa, int64_t lda, bool perm, const float* sa,
                          const int32_t* za, int64_t M, const W4& w, const float* bias, float lo,
                          float hi, float* Y, int64_t ldy, int64_t ldsz, hipStream_t stream) {
  static_assert(64 % (16 * FN * CW) == 0, "channel tiles must tile the 64-channel padding");
  const unsigned bx = (unsigned)ceil_div(w.N, 16 * FN * CW);
  const int64_t by = ceil_div(M, 16 * FM * RW);
  QP_REQUIRE(by <= 65535, QP_EUNSUPPORTED, "a8w4: M too large");
  const dim3 grid(bx, (unsigned)by);
#define QP_GEMM(PERM, KIND)                                                                \
  hipLaunchKernelGGL((a8w4_gemm_kernel<FM, FN, RW, CW, KS, PERM, KIND, false, PW, kExact>), grid, \
                     dim3(256), 0, \
                     stream, qa, lda, sa, za, M, w, bias, lo, hi, Y, ldy, (int64_t)0)
  if (perm) {
    if (w.kind == 1) QP_GEMM(true, 1);
    else if (w.kind == 2) QP_GEMM(true, 2);
    else QP_GEMM(true, 0);
  } else {
    if (w.kind == 1) QP_GEMM(false, 1);
    else if (w.kind == 2) QP_GEMM(false, 2);
    else QP_GEMM(false, 0);
  }
#undef QP_GEMM
  return check_launch("a8w4 gemm");
}

// Per-block activation parameters (sa, za are [M][ldsz]), row-major codes.
template <int FM, int FN, int RW, int CW, int KS, int PW, bool kExact>
qp_status launch_gemm_bq_cfg(const int8_t* qa, int64_t lda, const float* sa, const int32_t* za,
                             int64_t M, const W4& w, const float* bias, float lo, float hi,
                             float* Y, int64_t ldy, int64_t ldsz, hipStream_t stream) {
  static_assert(64 % (16 * FN * CW) == 0, "channel tiles must tile the 64-channel padding");
  const unsigned bx = (unsigned)ceil_div(w.N, 16 * FN * CW);
  const int64_t by = ceil_div(M, 16 * FM * RW);
  QP_REQUIRE(by <= 65535, QP_EUNSUPPORTED, "a8w4: M too large");
  const dim3 grid(bx, (unsigned)by);
  if (w.kind == 1)
    hipLaunchKernelGGL((a8w4_gemm_kernel<FM, FN, RW, CW, KS, false, 1, true, PW, kExact>), grid,
                       dim3(256), 0, stream, qa, lda, sa, za, M, w, bias, lo, hi, Y, ldy, ldsz);
  else
    hipLaunchKernelGGL((a8w4_gemm_kernel<FM, FN, RW, CW, KS, false, 0, true, PW, kExact>), grid,
                       dim3(256), 0, stream, qa, lda, sa, za, M, w, bias, lo, hi, Y, ldy, ldsz);
  return check_launch("a8w4 gemm (per-block activations)");
}

template <int BPW, bool kPerm, int kKind, bool kExact, int TPW>
qp_status launch_gemm_m16_tpw(const int8_t* qa, int64_t lda, const float* sa, const int32_t* za,
                              int64_t M, const W4& w, const float* bias, float lo, float hi,
                              float* Y, int64_t ldy, hipStream_t stream) {
  auto kern = a8w4_gemm_m16_kernel<BPW, kPerm, kKind, kExact, TPW>;
  // The LDS limit is raised once per instantiation and device, for the
  // deepest K the instantiation takes (threads may race to set it;
  // repeating it is harmless).
  constexpr int kLdsMax = 16 * (BPW * 4 * 128 + 16);
  static std::atomic<uint64_t> lds_attr_devices{0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) QP_FAIL(QP_EHIP, "a8w4: hipGetDevice failed");
  const uint64_t bit = dev >= 0 && dev < 64 ? (UINT64_C(1) << dev) : 0;
  if (bit == 0 || (lds_attr_devices.load(std::memory_order_acquire) & bit) == 0) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsMax) != hipSuccess)
      QP_FAIL(QP_EHIP, "a8w4: cannot reserve %d bytes of LDS", kLdsMax);
    lds_attr_devices.fetch_or(bit, std::memory_order_release);
  }
  const size_t lds = (size_t)16 * (w.Kpad + 16);
  const int64_t ntile = w.Npad / 16;
  hipLaunchKernelGGL(kern, dim3((unsigned)ceil_div(ntile, TPW)), dim3(TPW * 256), lds, stream,
                     qa, lda, sa, za, M, w, bias, lo, hi, Y, ldy);
  return check_launch("a8w4 gemm (up to 16 rows)");
}

// Two or three 16-channel tiles a workgroup, whichever leaves the fewest
// tiles on the busiest CU (one workgroup of either size per CU while the
// grid fits 256 CUs; ties go to two): 11008 channels (688 tiles) take
// three, 230 workgroups of at most one a CU, against 344 workgroups of two,
// which put four tiles on 88 CUs.
inline int m16_tiles_per_workgroup(const W4& w) {
  const int64_t t = w.Npad / 16;
  const int64_t busiest2 = 2 * ceil_div(ceil_div(t, 2), 256);
  const int64_t busiest3 = 3 * ceil_div(ceil_div(t, 3), 256);
  return busiest3 < busiest2 ? 3 : 2;
}

template <int BPW, bool kPerm, int kKind, bool kExact>
qp_status launch_gemm_m16_one(const int8_t* qa, int64_t lda, const float* sa, const int32_t* za,
                              int64_t M, const W4& w, const float* bias, float lo, float hi,
                              float* Y, int64_t ldy, hipStream_t stream) {
  if (m16_tiles_per_workgroup(w) == 3)
    return launch_gemm_m16_tpw<BPW, kPerm, kKind, kExact, 3>(qa, lda, sa, za, M, w, bias, lo, hi,
                                                             Y, ldy, stream);
  return launch_gemm_m16_tpw<BPW, kPerm, kKind, kExact, 2>(qa, lda, sa, za, M, w, bias, lo, hi, Y,
                                                           ldy, stream);
}

template <int BPW>
qp_status launch_gemm_m16(const int8_t* qa, int64_t lda, bool perm, const float* sa,
                          const int32_t* za, int64_t M, const W4& w, const float* bias, float lo,
                          float hi, float* Y, int64_t ldy, hipStream_t stream) {
  const bool exact = BPW == 8 && w.nblk == 4 * BPW;
#define QP_M16(PERM, KIND)                                                                       \
  return exact ? launch_gemm_m16_one<BPW, PERM, KIND, BPW == 8>(qa, lda, sa, za, M, w, bias, lo,  \
                                                                hi, Y, ldy, stream)              \
               : launch_gemm_m16_one<BPW, PERM, KIND, false>(qa, lda, sa, za, M, w, bias, lo, hi, \
                                                             Y, ldy, stream)
  if (perm) {
    if (w.kind == 1) QP_M16(true, 1);
    if (w.kind == 2) QP_M16(true, 2);
    QP_M16(true, 0);
  }
  if (w.kind == 1) QP_M16(false, 1);
  if (w.kind == 2) QP_M16(false, 2);
  QP_M16(false, 0);
#undef QP_M16
}

// perm: the activations are permuted inside each 128-K block (as written by
// the fused quantization); otherwise plain row-major.  ldsz > 0: sa, za are
// per-block parameters [M][ldsz] (row-major activations).
qp_status launch_gemm(const int8_t* qa, int64_t lda, bool perm, const float* sa,
                      const int32_t* za, int64_t M, const W4& w, const float* bias, float lo,
                      float hi, float* Y, int64_t ldy, hipStream_t stream, int64_t ldsz = 0) {
  // Up to 16 rows and 32 blocks of K: every load of a wave at once.
  const int64_t nblocks = w.Kpad / 128;
  if (M <= 16 && ldsz == 0 && nblocks <= 32) {
    const int64_t bpw = (nblocks + 3) / 4;
    if (bpw <= 2) return launch_gemm_m16<2>(qa, lda, perm, sa, za, M, w, bias, lo, hi, Y, ldy, stream);
    if (bpw <= 4) return launch_gemm_m16<4>(qa, lda, perm, sa, za, M, w, bias, lo, hi, Y, ldy, stream);
    return launch_gemm_m16<8>(qa, lda, perm, sa, za, M, w, bias, lo, hi, Y, ldy, stream);
  }
  // <FM, FN, RW, CW, KS>: rows per workgroup 16*FM*RW, channels 16*FN*CW.
  // Small M splits K over the waves (enough waves stream the weights); larger
  // M shares each staged activation row among several channel groups.
  // Exact K ranges (a multiple of 2*PW blocks each) drop the range tests and
  // hold two weight blocks in flight in a four-slot ring.
  if (ldsz > 0) {
    if (M <= 16) {
      if (nblocks % 16 == 0)
        return launch_gemm_bq_cfg<1, 1, 1, 1, 4, 2, true>(qa, lda, sa, za, M, w, bias, lo, hi, Y,
                                                          ldy, ldsz, stream);
      return launch_gemm_bq_cfg<1, 1, 1, 1, 4, 2, false>(qa, lda, sa, za, M, w, bias, lo, hi, Y,
                                                         ldy, ldsz, stream);
    }
    if (nblocks % 4 == 0)
      return launch_gemm_bq_cfg<2, 1, 1, 4, 1, 2, true>(qa, lda, sa, za, M, w, bias, lo, hi, Y,
                                                        ldy, ldsz, stream);
    return launch_gemm_bq_cfg<2, 1, 1, 4, 1, 2, false>(qa, lda, sa, za, M, w, bias, lo, hi, Y,
                                                       ldy, ldsz, stream);
  }
  if (M <= 16)
    return launch_gemm_cfg<1, 1, 1, 1, 4>(qa, lda, perm, sa, za, M, w, bias, lo, hi, Y, ldy,
                                          ldsz, stream);
  if (M <= 32)
    return launch_gemm_cfg<2, 1, 1, 4, 1>(qa, lda, perm, sa, za, M, w, bias, lo, hi, Y, ldy,
                                          ldsz, stream);
  // 64 rows x 32 channels a workgroup (two row and two channel groups):
  // measured faster than 64 x 64 with four channel groups, whose 256-VGPR
  // waves fit two a SIMD
  // K a multiple of four blocks: no range tests, two weight blocks in flight
  // in a four-slot ring (fewer registers, more resident waves: measured
  // faster than four or eight in flight), 32 rows x 64 channels a workgroup
  // (one row group, four channel groups: half the staged activation bytes
  // of 64 x 32, measured 7% faster)
  if (nblocks % 4 == 0)
    return launch_gemm_cfg<2, 1, 1, 4, 1, 2, true>(qa, lda, perm, sa, za, M, w, bias, lo, hi, Y,
                                                   ldy, ldsz, stream);
  return launch_gemm_cfg<2, 1, 2, 2, 1>(qa, lda, perm, sa, za, M, w, bias, lo, hi, Y, ldy, ldsz,
                                        stream);
}

}  // namespace
}  // namespace qp

extern "C" qp_status qgemm_a8w4_blockwise_f32_ws_size(int64_t M, const qp_packed_info* w,
                                                      size_t* bytes) {
  using namespace qp;
  QP_REQUIRE(w && bytes && M >= 0, QP_EINVAL, "qgemm_a8w4_blockwise_f32_ws_size: bad argument");
  // one row with its codes fitting the fused GEMV's LDS needs no workspace
  const bool fused = M <= 1 && w->Kpad <= kFusedGemvMaxKpad;
  *bytes = fused ? 0 : (size_t)(round_up(M * w->Kpad, 256) + round_up(8 * M, 256));
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
  if (M == 1 && w->Kpad <= kFusedGemvMaxKpad)
    return launch_gemv_fused(X, K, wv, bias, clamp_lo, clamp_hi, Y, stream);
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
  if (M == 1) {  // codes too long for the fused GEMV's LDS: quantize, then the GEMV
    st = launch_quantize_rows(X, M, K, ldx, qa, w->Kpad, w->Kpad, sa, za, false, stream);
    if (st) return st;
    return launch_gemv(qa, w->Kpad, sa, za, 1, wv, bias, clamp_lo, clamp_hi, Y, ldy, stream);
  }
  st = launch_quantize_rows(X, M, K, ldx, qa, w->Kpad, w->Kpad, sa, za, true, stream);
  if (st) return st;
  return launch_gemm(qa, w->Kpad, true, sa, za, M, wv, bias, clamp_lo, clamp_hi, Y, ldy, stream);
}

// ---- the same product with no workspace argument -------------------------
// For callers that cannot allocate device memory.  The quantized rows live in
// a library-owned array in device memory, one per GPU, held until the process
// ends; every call on a GPU reuses that GPU's copy.  The array's host-side
// name is only a stand-in for it: its device address (one per GPU) comes
// from hipGetSymbolAddress, taken once per device with that device current,
// and only that address is ever handed to a kernel.
namespace qp {
namespace {
constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
constexpr int kNoAllocMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
std::atomic<void*> scratch_dev_ptr[kNoAllocMaxDevices];

qp_status scratch_of_current_device(uint8_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess)
    QP_FAIL(QP_EHIP, "a8w4 (no allocation): hipGetDevice failed");
  QP_REQUIRE(dev >= 0 && dev < kNoAllocMaxDevices, QP_EUNSUPPORTED,
             "a8w4 (no allocation): device %d beyond the %d supported", dev, kNoAllocMaxDevices);
  void* p = scratch_dev_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // Threads may race here; each gets the same address.
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      QP_FAIL(QP_EHIP, "a8w4 (no allocation): hipGetSymbolAddress failed: %s",
              hipGetErrorString(e));
    scratch_dev_ptr[dev].store(p, std::memory_order_release);
  }
  *out = static_cast<uint8_t*>(p);
  return QP_OK;
}
}  // namespace
}  // namespace qp

extern "C" qp_status qgemm_a8w4_blockwise_f32_noalloc(const float* X, int64_t M, int64_t K,
                                                      int64_t ldx, const qp_packed_info* w,
                                                      const void* packedW_dev, const float* bias,
                                                      float clamp_lo, float clamp_hi, float* Y,
                                                      int64_t ldy, hipStream_t stream) {
  using namespace qp;
  clear_error();
  qp_status st = validate_w4(w, K);
  if (st) return st;
  QP_REQUIRE(M >= 0 && ldx >= K && ldy >= w->N, QP_EINVAL, "a8w4: bad M/ldx/ldy");
  QP_REQUIRE(!(clamp_lo > clamp_hi), QP_EINVAL, "a8w4: clamp_lo > clamp_hi");
  if (M == 0) return QP_OK;
  QP_REQUIRE(X && packedW_dev && Y, QP_EINVAL, "a8w4: null data pointer");
  size_t need = 0;
  qgemm_a8w4_blockwise_f32_ws_size(M, w, &need);
  QP_REQUIRE(need <= kNoAllocScratchBytes, QP_ESIZE,
             "a8w4 (no allocation): M=%lld rows of Kpad=%lld need %zu bytes of scratch, "
             "more than the %zu available",
             (long long)M, (long long)w->Kpad, need, kNoAllocScratchBytes);
  if (need == 0)  // one row in the fused GEMV, which keeps its codes in LDS: no scratch
    return qgemm_a8w4_blockwise_f32(X, M, K, ldx, w, packedW_dev, bias, clamp_lo, clamp_hi, Y,
                                    ldy, nullptr, 0, stream);
  uint8_t* ws = nullptr;
  if ((st = scratch_of_current_device(&ws))) return st;
  return qgemm_a8w4_blockwise_f32(X, M, K, ldx, w, packedW_dev, bias, clamp_lo, clamp_hi, Y, ldy,
                                  ws, need, stream);
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
    return launch_gemv(qa, lda, sa, za, M, wv, bias, clamp_lo, clamp_hi, Y, ldy, stream);
  return launch_gemm(qa, lda, false, sa, za, M, wv, bias, clamp_lo, clamp_hi, Y, ldy, stream);
}

// ---- activations quantized per block of 32 K ----------------------------
extern "C" qp_status qgemm_a8w4_blockq_f32_ws_size(int64_t M, const qp_packed_info* w,
                                                   size_t* bytes) {
  using namespace qp;
  QP_REQUIRE(w && bytes && M >= 0, QP_EINVAL, "qgemm_a8w4_blockq_f32_ws_size: bad argument");
  const int64_t nb = w->Kpad / 32;
  // one row whose codes and block parameters fit the fused GEMV's LDS needs
  // no workspace
  const bool fused = M <= 1 && w->Kpad <= kFusedGemvMaxKpad;
  *bytes = fused ? 0 : (size_t)(round_up(M * w->Kpad, 256) + 2 * round_up(4 * M * nb, 256));
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
  if (M == 1 && w->Kpad <= kFusedGemvMaxKpad)
    return launch_gemv_fused_bq(X, K, w4_of(w, packedW_dev), bias, clamp_lo, clamp_hi, Y, stream);
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
