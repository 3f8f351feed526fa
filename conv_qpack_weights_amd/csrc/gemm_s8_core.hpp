// gemm_s8_core.hpp -- the INT8 MFMA GEMM kernel and its epilogue helpers.
//
// Included by gemm_s8.hip (the numeric contract is stated there) and by the
// implicit-GEMM convolution, which shares the epilogue helpers.  The kernel:
//  * workgroup tile BM x BN, K in steps of BK bytes, an SA-deep LDS ring for
//    the activations (A);
//  * A moves HBM/L2 -> LDS with direct loads (buffer_load ... lds): each lane
//    names the 16-byte chunk that lands at its slot, so the XOR swizzle is
//    applied on the global side and no VGPRs stage the data;
//  * the packed weights (B) go straight from the blob's 32x32 sub-tiles into
//    VGPRs in MFMA operand order, one K tile ahead;
//  * each wave computes all BM rows x BN/NW channels with
//    v_mfma_i32_32x32x32_i8 (large tiles) or v_mfma_i32_16x16x64_i8 (small
//    tiles), issued as (B fragment, A fragment) so a lane holds 4
//    consecutive channels of one output row;
//  * one barrier per K tile, halfway through it; the prefetch distance is
//    SA-1 tiles; every tile runs the same branch-free body;
//  * the epilogue applies the zero-point terms and bias and then the Q31
//    requantization to int8, the raw int32, or the f32 dequantization.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "dev_util.hpp"

namespace qp {

struct GemmArgs {
  const int8_t* A;
  int64_t lda;
  const int8_t* B;  // blob data, [Npad][Kpad]
  int64_t ldb;      // row stride of B in bytes (Kpad for a blob)
  int64_t M, N, K, Kpad, Npad;
  const int32_t* colsum;
  const int32_t* zpB;
  const float* sB;
  const int32_t* rowsum;  // [M] when the weights have zero points
  const int32_t* bias;    // [N] or null
  float sA, sOut;
  int32_t zA, zp_out, lo, hi;
  void* C;
  int64_t ldc;
  int32_t tiles_m, tiles_n;
  int32_t group_m;   // tile rows per raster group
  int32_t xcd_remap; // 1: give each XCD a contiguous range of the raster order
  const float* bias_f;  // f32 output: [N] or null, added after dequantization
  float clo, chi;       // f32 output: clamp bounds
};


// M_n = sA*sB/s_out in fp64; M_n = f*2^e, f in [0.5,1); m0 = rint(f*2^31),
// 2^31 -> 2^30 with e+1; shift = 31 - e.
// The kernel's rounding step needs 1 <= shift <= 62, so the two edge cases
// are mapped to equivalent pairs: shift >= 63 (|acc*M| < 1/2 for every
// acc, result 0) becomes (m0 = 0, shift = 32), which both rounding forms
// (the 64-bit one and the one in 32-bit pieces, used when every shift is
// >= 32) turn into 0; shift == 0 (M >= 2^30, every non-zero acc saturates,
// acc = 0 gives 0) becomes (2^31-1, 1), which saturates the same way and
// only occurs in launches with the 64-bit rounding.  A column whose
// multiplier is not positive and finite (the zero-scale padding columns)
// gets (0, 1).
__device__ __forceinline__ void derive_mult(float sA, float sB, float sOut, int32_t* m0,
                                            int32_t* sh) {
#pragma clang fp contract(off)
  double num = (double)sA * (double)sB;
  double mr = num / (double)sOut;
  if (!(mr > 0.0) || !(mr < __builtin_huge_val())) {
    *m0 = 0;
    *sh = 1;
    return;
  }
  int e = 0;
  double f = __builtin_frexp(mr, &e);
  int64_t q = (int64_t)__builtin_rint(f * 2147483648.0);
  if (q == ((int64_t)1 << 31)) {
    q = (int64_t)1 << 30;
    e += 1;
  }
  int s = 31 - e;
  if (s <= 0) {  // s < 0 is rejected on the host whenever the scales are known there
    s = 1;
    q = 0x7fffffff;
  } else if (s >= 63) {
    s = 32;
    q = 0;
  }
  *m0 = (int32_t)q;
  *sh = s;
}

// RHE(acc*m0 / 2^sh), 1 <= sh <= 62:
// floor((t + 2^(sh-1) - 1 + odd) / 2^sh) with odd = bit sh of t; |t| < 2^62.
__device__ __forceinline__ int64_t rhe_shift64(int32_t acc, int32_t m0, int32_t sh) {
  const int64_t t = (int64_t)acc * (int64_t)m0;
  const int64_t odd = (t >> sh) & 1;
  const int64_t half_m1 = ((int64_t)1 << (sh - 1)) - 1;
  return (t + half_m1 + odd) >> sh;
}

__device__ __forceinline__ int32_t clamp_i64(int64_t v, int32_t lo, int32_t hi) {
  v = v < lo ? lo : v;
  v = v > hi ? hi : v;
  return (int32_t)v;
}

// One v_med3_i32 (the compiler forms it from min/max only for constant
// bounds); lo <= hi, so the median of (v, lo, hi) is v clamped to [lo, hi].
__device__ __forceinline__ int32_t clamp_i32(int32_t v, int32_t lo, int32_t hi) {
  int32_t r;
  asm("v_med3_i32 %0, %1, %2, %3" : "=v"(r) : "v"(v), "v"(lo), "s"(hi));
  return r;
}

// Chunk c of LDS row r sits at chunk position c ^ swz(r): conflict-free
// 16-row fragment reads and row writes for 32 or 64 four-byte banks.
template <int BK>
__device__ __forceinline__ int swz(int row) {
  if constexpr (BK == 128)
    return (row ^ (row >> 3)) & 7;
  else
    return ((row >> 1) ^ (row >> 3)) & 3;
}


// One K tile (BK bytes of K) of the multi-step main loop for a wave:
// SUB MFMA K-steps over the FM x FN fragment grid.
//  * A fragments for the next K-step are read from LDS right after the
//    MFMAs that consume the current ones (the last K-step reads the first
//    step of the next tile, from `sa_next`);
//  * B fragments of the next tile are loaded into the register slot the
//    current K-step has just consumed;
//  * halfway through, one barrier: past it every wave has left the previous
//    tile, whose ring slot `dst` the second half refills with direct loads,
//    and the next tile's A has landed.
// Every tile runs the same branch-free body.  Near the end of K the caller
// clamps the source offsets to the last tile: the extra loads land in a
// ring slot that is no longer read (or in registers that are not used) and
// keep the number of loads issued per tile fixed, which is what makes the
// constant wait count A_WAIT exact for every tile.
template <int MF, int FM, int FN, int SUB, int BK, int IA, int NW, int SA, class AccV>
__device__ __forceinline__ void gemm_ktile(AccV (&acc)[FN][FM], v4i (&af)[FM],
                                           v4i (&breg)[SUB][FN], const lds_i8* sa,
                                           const lds_i8* sa_next, lds_i8* dst,
                                           const int8_t* a_base, const uint32_t* a_voff,
                                           uint32_t a_koff, const int8_t* const (&b_src)[FN],
                                           int64_t b_koff, int frow, int fchunk, int wave) {
  constexpr int KSTEP = MF == 16 ? 64 : 32;
  constexpr int IB = SUB * FN;
  constexpr int HALF = SUB / 2;                                      // K-steps before the barrier
  constexpr int A_PER_SUB = (IA + (SUB - HALF) - 1) / (SUB - HALF);  // direct loads per later step
  // Loads issued after the last direct load of tile kt+1: the B loads that
  // follow it, SA-3 whole tiles, and this tile's first half.  (Before the
  // first tiles everything has been drained, so the wait is then trivially
  // met.)
  constexpr int A_WAIT = FN + (SA - 3) * (IA + IB) + HALF * FN;
  static_assert(SUB >= 2 && SA >= 3, "the refill slot must differ from the two slots being read");
  static_assert(A_WAIT >= 0 && A_WAIT < 64, "vmcnt range");
#pragma unroll
  for (int sub = 0; sub < SUB; ++sub) {
    if (sub == HALF) {
      wait_vmcnt<A_WAIT>();
      asm volatile("s_barrier" ::: "memory");
    }
    if (sub >= HALF) {
      const int part = sub - HALF;
#pragma unroll
      for (int d = 0; d < A_PER_SUB; ++d) {
        const int j = part * A_PER_SUB + d;
        if (j < IA) dma16_to_lds(a_base, (lds_void_t*)(dst + (j * NW + wave) * 1024), a_voff[j], a_koff);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < FM; ++j) {
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        if constexpr (MF == 16)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(breg[sub][i], af[j], acc[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(breg[sub][i], af[j], acc[i][j], 0, 0, 0);
      }
      // af[j] is consumed: refill it with the next K-step's fragment
      const int row = j * MF + frow;
      const int c = sub + 1 < SUB ? (sub + 1) * (KSTEP / 16) + fchunk : fchunk;
      const lds_i8* src = sub + 1 < SUB ? sa : sa_next;
      af[j] = *reinterpret_cast<const __attribute__((address_space(3))) v4i*>(
          src + row * BK + ((c ^ swz<BK>(row)) * 16));
      __builtin_amdgcn_sched_barrier(0);
    }
    // breg[sub] is consumed: fetch the same K-step of the next tile
#pragma unroll
    for (int i = 0; i < FN; ++i)
      breg[sub][i] = *reinterpret_cast<const v4i*>(b_src[i] + b_koff + sub * (KSTEP / 32) * 1024);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// kShiftHi: every column's shift is in 32..53 (all multipliers in [2^-23,
// 1/2), known on the host from the weight scales), so the rounding runs in
// 32-bit pieces: u = acc*m0 + one 64-bit addend per column (the zero-point
// terms and bias times m0, 2^(sh-1), zp_out*2^sh); floor(u / 2^sh) is the
// high word shifted by sh-32 and already holds zp_out; u a multiple of 2^sh
// marks an exact tie t/2^sh = r - 1/2, whose even neighbour is r with its
// lowest bit cleared (before zp_out is added).
//
// Data movement (per workgroup tile BM x BN, K in steps of BK bytes):
//  * A (activations, row-major) goes HBM/L2 -> LDS with direct loads into an
//    SA-deep ring (prefetch distance SA-1 tiles); every wave reads all BM
//    rows from it.
//  * B (the packed weights, 32x32 sub-tiles) goes straight into VGPRs in
//    MFMA operand order, one tile ahead: each wave owns BN/NW columns, so no
//    B byte is loaded twice and LDS only carries A.
// kF32 (with kOut32): f32 output y = clamp(sA*sB[n]*acc + bias_f[n], clo, chi).
// WM: the waves form WM row groups x NW/WM column groups; a wave computes
// TM = BM/WM rows x TN = BN/(NW/WM) channels (WM = 1: every wave covers all
// rows of the tile).
// kResident (one K-step tiles only): the tile's activations for all of K are
// read once, byte-exact, into LDS -- any row stride and alignment, zeros past
// K and past M -- and the row sums the weight zero points need are formed on
// the way (LDS integer atomics); the K loop then reads only LDS.  Small
// GEMMs with an odd K or stride take this one launch instead of a padded
// copy of A plus the GEMM.
template <int BM, int BN, int BK, int NW, int SA, int MF, bool kOut32, bool kRowSum, bool kShiftHi,
          bool kF32 = false, int WM = 1, bool kResident = false>
__global__ __launch_bounds__(NW * 64) void qgemm_s8_kernel(GemmArgs g) {
  constexpr int CH = BK / 16;  // 16-byte chunks per A tile row
  constexpr int TM = BM / WM;
  constexpr int TN = BN / (NW / WM);
  constexpr int FM = TM / MF;
  constexpr int FN = TN / MF;
  constexpr int KSTEP = MF == 16 ? 64 : 32;  // K per MFMA
  constexpr int NREG = MF == 16 ? 4 : 16;    // accumulator registers per MFMA
  constexpr int SUB = BK / KSTEP;            // MFMAs along K per tile
  constexpr int IA = BM * CH / (64 * NW);    // A direct loads per wave per tile
  constexpr int IB = SUB * FN;               // B fragment loads per wave per tile
  constexpr int STAGE = BM * BK;
  typedef int accv __attribute__((ext_vector_type(NREG)));
  static_assert(BM * CH % (64 * NW) == 0, "A tile must split evenly over the waves");
  static_assert(TN % MF == 0 && TM % MF == 0 && BK % KSTEP == 0 && NW % WM == 0, "tile shape");
  static_assert(MF == 16 || MF == 32, "MFMA shape");
  static_assert(!kF32 || kOut32, "f32 output uses the 4-byte store paths");
  static_assert(SA >= 2 && (SA - 2) * IA + IB < 64, "vmcnt range");
  static_assert(!kResident || SUB == 1, "resident activations: one K-step tiles");

  extern __shared__ __attribute__((aligned(1024))) int8_t smem[];
  __shared__ int32_t col_m0[BN], col_sh[BN], col_c[BN], col_zb[BN];
  // kShiftHi: the column's whole 64-bit addend of the rounding step,
  // c*m0 + 2^(sh-1) + zp_out*2^sh (c the zero-point and bias terms, exact)
  constexpr bool kFold = kShiftHi && !kF32 && !kOut32;
  __shared__ int64_t col_ad[kFold ? BN : 1];
  __shared__ int32_t row_sum[kResident ? BM : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % (NW / WM);  // the wave's column group
  const int wm = wave / (NW / WM);  // and row group

  // ---- tile index: XCD-aware (dispatch round-robins over 8 XCDs), then
  // grouped along M so concurrent workgroups share A rows and B rows in L2.
  const int nblk = gridDim.x;
  const int lin0 = blockIdx.x;
  const int lin = g.xcd_remap && (nblk & 7) == 0 ? (lin0 & 7) * (nblk >> 3) + (lin0 >> 3) : lin0;
  const int per_group = g.group_m * g.tiles_n;
  const int grp = lin / per_group;
  const int first_m = grp * g.group_m;
  const int gsz = min(g.tiles_m - first_m, g.group_m);
  const int within = lin - grp * per_group;
  const int tile_m = first_m + within % gsz;
  const int tile_n = within / gsz;
  const int64_t m0 = (int64_t)tile_m * BM;
  const int64_t n0 = (int64_t)tile_n * BN;

  // ---- A: per-lane direct-load sources.  Instruction j fills 16-byte slots
  // [(j*NW + wave)*64, +64); lane -> slot -> (row, swizzled chunk).
  // Offsets are relative to the tile's first row (the host keeps
  // BM*lda + Kpad below 2^31).
  const int8_t* const a_base = g.A + m0 * g.lda;
  uint32_t a_voff[IA];
#pragma unroll
  for (int j = 0; j < IA; ++j) {
    const int s = (j * NW + wave) * 64 + lane;
    const int row = s / CH, c = (s % CH) ^ swz<BK>(s / CH);
    int64_t gm = m0 + row;
    gm = gm < g.M ? gm : g.M - 1;
    a_voff[j] = (uint32_t)((gm - m0) * g.lda + c * 16);
  }
  auto issue_a = [&](int kt, int stage, int j) {
    __attribute__((address_space(3))) int8_t* sbase =
        (__attribute__((address_space(3))) int8_t*)smem + stage * STAGE;
    dma16_to_lds(a_base, (lds_void_t*)(sbase + (j * NW + wave) * 1024), a_voff[j], (uint32_t)(kt * BK));
  };

  // ---- B: fragment sources in the 32x32 sub-tile layout.  MF = 32: lane
  // reads row lane%32, 16 bytes at K offset 16*(lane/32) of a 32x32 tile.
  // MF = 16: 16 rows x 64 K, lane reads row lane%16, K chunk lane/16.
  const int64_t kblocks = g.Kpad / 32;
  const int64_t nblocks = g.Npad / 32;
  const int8_t* b_src[FN];
#pragma unroll
  for (int i = 0; i < FN; ++i) {
    const int64_t r0 = n0 + wn * TN + i * MF;  // first channel of the fragment
    int64_t nb = r0 / 32;
    nb = nb < nblocks ? nb : nblocks - 1;
    if constexpr (MF == 32) {
      b_src[i] = g.B + nb * kblocks * 1024 + (lane & 31) * 32 + (lane >> 5) * 16;
    } else {
      const int c = lane >> 4;  // 16-byte chunk of the 64-K step
      b_src[i] = g.B + (nb * kblocks + (c >> 1)) * 1024 + ((r0 & 31) + (lane & 15)) * 32 +
                 (c & 1) * 16;
    }
  }
  v4i breg[SUB][FN];
  auto load_b = [&](int kt, int sub) {
    // MF=32: K block kt*BK/32 + sub; MF=16: K blocks (kt*BK + 64*sub)/32 + {0,1}
    const int64_t kb = (int64_t)kt * (BK / 32) + sub * (KSTEP / 32);
#pragma unroll
    for (int i = 0; i < FN; ++i) breg[sub][i] = *reinterpret_cast<const v4i*>(b_src[i] + kb * 1024);
  };

  // ---- per-column epilogue inputs, one column per thread.  Every load is
  // unconditional (the column clamped into range, a stand-in array where
  // there is no bias) and issued before the A tiles', so that all of them
  // are in flight at once; the constants are formed after the prologue.
  static_assert(BN <= NW * 64, "one column per thread");
  const int64_t col_nc = n0 + tid < g.N ? n0 + tid : g.N - 1;
  const float sb = g.sB[col_nc];
  const int32_t zbl = g.zpB[col_nc];
  const int32_t csl = g.colsum[col_nc];
  const int32_t bl = (g.bias ? g.bias : g.zpB)[col_nc];
  float bfl = 0.0f;
  if constexpr (kF32) bfl = (g.bias_f ? g.bias_f : g.sB)[col_nc];

  const int nk = (int)(g.Kpad / BK);
  // resident mode: B fragments of RU tiles in flight together
  constexpr int RU = 4;
  v4i bq[kResident ? RU : 1][FN];
  // Tiles past the last one load the last tile's fragments and zero them,
  // so the loads are unconditional and the extra MFMAs add nothing.
  auto load_bq = [&](int kt0) {
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      const int64_t kb = (int64_t)min(kt0 + u, nk - 1) * (BK / 32);
      const int keep = kt0 + u < nk ? -1 : 0;
#pragma unroll
      for (int i = 0; i < FN; ++i)
        bq[u][i] = *reinterpret_cast<const v4i*>(b_src[i] + kb * 1024) & keep;
    }
  };
  if constexpr (kResident) {
    // All K tiles of A into LDS stages 0..nk-1; slot s of a tile is filled
    // by lane s%64 of wave (s/64)%NW, as the direct loads would fill it.
    // A 16-byte chunk at any alignment is five aligned dwords (a dword with
    // no byte of the chunk in range is read from the chunk's first dword,
    // which holds one, so no read leaves a page the row lives in) shifted
    // into place; bytes past K are masked to zero.  No load is conditional,
    // so all of RU tiles' loads are in flight together.
    if (kRowSum && tid < BM) row_sum[tid] = 0;
    load_bq(0);
    const uintptr_t a_safe = (uintptr_t)g.A & ~(uintptr_t)3;  // A[0,0] lies in this dword
    for (int kt0 = 0; kt0 < nk; kt0 += RU) {
      uint32_t dw[RU][IA][5];
      int nv[RU][IA];
      uint32_t sh[RU][IA];
#pragma unroll
      for (int u = 0; u < RU; ++u)
#pragma unroll
        for (int j = 0; j < IA; ++j) {
          const int sl = (j * NW + wave) * 64 + lane;
          const int row = sl / CH, c = (sl % CH) ^ swz<BK>(sl / CH);
          const int64_t gm = m0 + row;
          const int64_t k0 = (int64_t)(kt0 + u) * BK + c * 16;
          const bool in = gm < g.M && k0 < g.K;
          const int64_t rem = g.K - k0;
          nv[u][j] = in ? (int)(rem < 16 ? rem : 16) : 0;
          const uintptr_t src = in ? (uintptr_t)(g.A + gm * g.lda + k0) : a_safe;
          sh[u][j] = (uint32_t)(src & 3);
          const uint32_t* base = reinterpret_cast<const uint32_t*>(src & ~(uintptr_t)3);
#pragma unroll
          for (int d = 0; d < 5; ++d)
            dw[u][j][d] = base[4 * d < nv[u][j] + (int)sh[u][j] ? d : 0];
        }
      // the zeroed row sums are visible before the first adds (this waits
      // for the loads above, which the adds need anyway)
      if (kRowSum && kt0 == 0) __syncthreads();
#pragma unroll
      for (int u = 0; u < RU; ++u) {
        if (kt0 + u >= nk) break;
#pragma unroll
        for (int j = 0; j < IA; ++j) {
          const int sl = (j * NW + wave) * 64 + lane;
          uint32_t w[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int vq = nv[u][j] - 4 * q;  // bytes of word q inside K
            const uint32_t keep = vq >= 4 ? 0xFFFFFFFFu : vq <= 0 ? 0u : (1u << (8 * vq)) - 1u;
            w[q] = __builtin_amdgcn_alignbyte(dw[u][j][q + 1], dw[u][j][q], sh[u][j]) & keep;
          }
          *reinterpret_cast<uint4*>(smem + (int64_t)(kt0 + u) * STAGE + sl * 16) =
              make_uint4(w[0], w[1], w[2], w[3]);
          if constexpr (kRowSum) {
            int32_t rsum = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) rsum = __builtin_amdgcn_sdot4((int)w[q], 0x01010101, rsum, false);
            if (rsum != 0) atomicAdd(&row_sum[sl / CH], rsum);
          }
        }
      }
    }
  } else {
    // prologue: A(0) .. A(SA-2) into the ring, B(0) into registers
#pragma unroll
    for (int p = 0; p < SA - 1; ++p)
      if (p < nk)
#pragma unroll
        for (int j = 0; j < IA; ++j) issue_a(p, p, j);
#pragma unroll
    for (int sub = 0; sub < SUB; ++sub) load_b(0, sub);
  }

  // ---- per-column epilogue constants from the inputs loaded above ----
  if (tid < BN) {
    const int j = tid;
    const int64_t n = n0 + j;
    int32_t mm = 0, ss = 63, cc = 0, zb = 0;
    if (n < g.N) {
      if constexpr (kF32) {
        // f32 output: the columns hold the dequantization scale and the bias
        mm = __builtin_bit_cast(int32_t, (float)((double)g.sA * (double)sb));
        ss = __builtin_bit_cast(int32_t, g.bias_f ? bfl : 0.0f);
      } else {
        derive_mult(g.sA, sb, g.sOut, &mm, &ss);
      }
      zb = zbl;
      uint32_t c = (uint32_t)(g.bias ? bl : 0);
      c -= (uint32_t)g.zA * (uint32_t)csl;
      c += (uint32_t)g.K * (uint32_t)g.zA * (uint32_t)zb;
      cc = (int32_t)c;
    }
    col_m0[j] = mm;
    col_sh[j] = ss;
    col_c[j] = cc;
    col_zb[j] = zb;
    if constexpr (kFold) {
      // (acc + c)*m0 + 2^(sh-1) + zp*2^sh is below 2^63 in magnitude: |acc + c|
      // < 2^31 (the host's INT32 bound), m0 < 2^31, and the host takes this
      // path only while every shift is at most 53; the addend itself is
      // formed modulo 2^64, which the multiply-add's result is too.
      uint64_t ad = 0;
      if (n < g.N) {
        const int64_t c64 = (int64_t)(g.bias ? bl : 0) - (int64_t)g.zA * (int64_t)csl +
                            (int64_t)g.K * (int64_t)g.zA * (int64_t)zb;
        ad = (uint64_t)c64 * (uint64_t)(int64_t)mm + ((uint64_t)1 << (ss - 1)) +
             ((uint64_t)(int64_t)g.zp_out << ss);
      }
      col_ad[j] = (int64_t)ad;
    }
  }

  accv acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = accv{};

  // fragment lane mapping of A: row = lane % MF, 16-byte chunk = lane / MF
  const int frow = lane % MF + wm * TM;  // the lane's A row within the tile
  const int fchunk = lane / MF;
  v4i af[FM];
  auto read_a = [&](const int8_t* sa, int sub, int j) {
    const int c = sub * (KSTEP / 16) + fchunk;
    const int row = j * MF + frow;
    af[j] = *reinterpret_cast<const v4i*>(sa + row * BK + ((c ^ swz<BK>(row)) * 16));
  };
  wait_vmcnt<0>();
  __syncthreads();  // A(0) everywhere; epilogue constants visible

  if constexpr (kResident) {
    // all of A is in LDS: no barriers; B arrives RU tiles at a time
    for (int kt0 = 0; kt0 < nk; kt0 += RU) {
      if (kt0 > 0) load_bq(kt0);
#pragma unroll
      for (int u = 0; u < RU; ++u) {
#pragma unroll
        for (int j = 0; j < FM; ++j) read_a(smem + min(kt0 + u, nk - 1) * STAGE, 0, j);
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
          for (int i = 0; i < FN; ++i) {
            if constexpr (MF == 16)
              acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bq[u][i], af[j], acc[i][j], 0, 0, 0);
            else
              acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bq[u][i], af[j], acc[i][j], 0, 0, 0);
          }
      }
    }
  } else if constexpr (SUB == 1) {
    // One K-step per tile (small tiles): barrier at the top of each tile.
    for (int kt = 0; kt < nk; ++kt) {
      if (kt > 0) {
        wait_vmcnt<0>();
        asm volatile("s_barrier" ::: "memory");
      }
      const int8_t* sa = smem + (kt % SA) * STAGE;
#pragma unroll
      for (int j = 0; j < FM; ++j) read_a(sa, 0, j);
      if (kt + SA - 1 < nk)
#pragma unroll
        for (int j = 0; j < IA; ++j) issue_a(kt + SA - 1, (kt + SA - 1) % SA, j);
#pragma unroll
      for (int j = 0; j < FM; ++j)
#pragma unroll
        for (int i = 0; i < FN; ++i) {
          if constexpr (MF == 16)
            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(breg[0][i], af[j], acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(breg[0][i], af[j], acc[i][j], 0, 0, 0);
        }
      if (kt + 1 < nk) load_b(kt + 1, 0);
    }
  } else {
    // Settle every outstanding scalar load (kernel arguments used only by
    // the epilogue): with one pending, the compiler cannot count LDS reads
    // precisely across the loop back edge and waits for all of them.
    // The first fragments are read in the loop's own order, so that the
    // counts agree on both edges into the loop.
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      read_a(smem, 0, j);
      __builtin_amdgcn_sched_barrier(0);
    }
    lds_i8* const ring = (lds_i8*)smem;
    for (int kt = 0; kt < nk; ++kt) {
      const int ka = min(kt + SA - 1, nk - 1);  // tile refilled into the free slot
      const int kb = min(kt + 1, nk - 1);       // tile whose B goes into registers
      gemm_ktile<MF, FM, FN, SUB, BK, IA, NW, SA>(
          acc, af, breg, ring + (kt % SA) * STAGE, ring + ((kt + 1) % SA) * STAGE,
          ring + ((kt + SA - 1) % SA) * STAGE, a_base, a_voff, (uint32_t)(ka * BK), b_src,
          (int64_t)kb * (BK / 32) * 1024, frow, fchunk, wave);
    }
    wait_vmcnt<0>();  // the clamped refills must land before the workgroup ends
  }

  // ---- epilogue ----
  // 16x16 MFMA: register r of a lane is channel 4*(lane/16)+r of row lane%16.
  // 32x32 MFMA: register 4q+r is channel 8q+4*(lane/32)+r of row lane%32.
  // Either way a lane owns runs of 4 consecutive channels of one row.
  constexpr int QN = NREG / 4;  // runs of 4 channels per MFMA tile
  const bool c_vec = kOut32 ? ((g.ldc & 3) == 0 && ((uintptr_t)g.C & 15) == 0)
                            : ((g.ldc & 3) == 0 && ((uintptr_t)g.C & 3) == 0);
  const bool full = c_vec && (m0 + BM <= g.M) && (n0 + BN <= g.N);
  int32_t rs[FM];
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    int64_t m = m0 + wm * TM + j * MF + (lane % MF);
    if constexpr (kResident)
      rs[j] = kRowSum ? row_sum[wm * TM + j * MF + (lane % MF)] : 0;
    else
      rs[j] = (kRowSum && m < g.M) ? g.rowsum[m] : 0;
  }
  // The clamp bounds in a VGPR let the clamp be one v_med3 (one scalar
  // operand per instruction).
  int32_t lo_v = g.lo;
  asm volatile("" : "+v"(lo_v));

  // Output values of fragment row j, channel run (i, q) of this lane.
  auto outputs = [&](int i, int q, int j, const v4i& cc, const v4i& mm, const v4i& ss,
                     const v4i& zb, const int64_t (&half)[4], const int32_t (&s2)[4],
                     const uint32_t (&mask)[4], int32_t (&out)[4]) {
    if constexpr (kFold) {
      // The rounding in 32-bit pieces, u = acc*m0 + the column's addend
      // (zero-point terms times m0, the half, the output zero point times
      // 2^sh: one multiply-add), so floor(u / 2^sh) is already the rounded-up
      // quotient plus zp_out.  The exact-tie step runs only when some lane of
      // the wave meets a tie among these four outputs (rare on real data);
      // the tie's even neighbour is taken before the zero point is added.
      int32_t rq[4];
      bool tie[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint32_t a = (uint32_t)acc[i][j][4 * q + r];
        if (kRowSum) a -= (uint32_t)zb[r] * (uint32_t)rs[j];
        const int64_t u = (int64_t)(int32_t)a * (int64_t)mm[r] + half[r];
        const int32_t hi = (int32_t)(u >> 32);
        rq[r] = hi >> s2[r];
        tie[r] = ((uint32_t)u | ((uint32_t)hi & mask[r])) == 0u;
      }
      if (__builtin_amdgcn_ballot_w64(tie[0] | tie[1] | tie[2] | tie[3]) != 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          rq[r] = tie[r] ? ((rq[r] - g.zp_out) & ~1) + g.zp_out : rq[r];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) out[r] = clamp_i32(rq[r], lo_v, g.hi);
      return;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uint32_t a = (uint32_t)acc[i][j][4 * q + r] + (uint32_t)cc[r];
      if (kRowSum) a -= (uint32_t)zb[r] * (uint32_t)rs[j];
      if constexpr (kF32) {
        // (bit_cast of a vector element would read element 0: copy it out first)
        const int32_t mr = mm[r], sr = ss[r];
        float y = __builtin_fmaf(__builtin_bit_cast(float, mr), (float)(int32_t)a,
                                 __builtin_bit_cast(float, sr));
        y = y < g.clo ? g.clo : y;
        y = y > g.chi ? g.chi : y;
        out[r] = __builtin_bit_cast(int32_t, y);
      } else if constexpr (kOut32) {
        out[r] = (int32_t)a;
      } else {
        out[r] = clamp_i64(rhe_shift64((int32_t)a, mm[r], ss[r]) + g.zp_out, lo_v, g.hi);
      }
    }
  };
  // Per-run column constants.
  auto column = [&](int i, int q, int* jn_out, v4i* cc, v4i* mm, v4i* ss, v4i* zb,
                    int64_t (&half)[4], int32_t (&s2)[4], uint32_t (&mask)[4]) {
    const int jn = wn * TN + i * MF + (MF == 16 ? 4 * (lane >> 4) : 8 * q + 4 * (lane >> 5));
    *jn_out = jn;
    *cc = *reinterpret_cast<const v4i*>(&col_c[jn]);
    *mm = *reinterpret_cast<const v4i*>(&col_m0[jn]);
    *ss = *reinterpret_cast<const v4i*>(&col_sh[jn]);
    *zb = v4i{0, 0, 0, 0};
    if (kRowSum) *zb = *reinterpret_cast<const v4i*>(&col_zb[jn]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (kF32) {  // (the shift slots hold the f32 bias)
        s2[r] = 0;
        half[r] = 0;
        mask[r] = 0;
      } else if constexpr (kFold) {  // `half` carries the column's whole addend
        s2[r] = (*ss)[r] - 32;
        half[r] = col_ad[jn + r];
        mask[r] = (1u << (s2[r] & 31)) - 1u;
      } else {
        s2[r] = (*ss)[r] - 32;
        half[r] = (int64_t)1 << ((*ss)[r] - 1);
        mask[r] = (1u << (s2[r] & 31)) - 1u;
      }
    }
  };

  // Full tiles with 16-byte aligned output rows go through LDS (the A ring
  // is free now): each wave writes its values there, then the workgroup
  // stores whole output rows with 16-byte stores, instead of each lane
  // writing 4 (int8) or 16 (int32) bytes into 32 different rows.  int32
  // tiles go 64 rows at a time.  Chunk c (16 bytes) of staged row r sits at
  // chunk position c ^ swizzle(r), which keeps the lane writes within two
  // ways of bank conflict and the row reads conflict-free.
  constexpr int ES = kOut32 ? 4 : 1;             // output element bytes
  constexpr int RB = BN * ES;                    // staged row bytes
  constexpr int CPR = RB / 16;                   // 16-byte chunks per row
  constexpr int PR = kOut32 ? 64 : BM;           // rows per pass
  constexpr bool kStaged = MF == 32 && (CPR == 8 || CPR >= 16) && PR * RB <= SA * STAGE &&
                           (PR * CPR) % (NW * 64) == 0 && PR % 64 == 0;
  const bool staged = kStaged && full && ((g.ldc * ES) % 16 == 0) && (((uintptr_t)g.C & 15) == 0);
  if (staged) {
    auto swz_row = [](int r) { return CPR >= 16 ? (r & 15) : ((r >> 1) & 7); };
    int8_t* stg = smem;
    __syncthreads();  // every wave has left the A ring
#pragma unroll
    for (int p = 0; p < BM / PR; ++p) {
#pragma unroll
      for (int i = 0; i < FN; ++i) {
#pragma unroll
        for (int q = 0; q < QN; ++q) {
          int jn;
          v4i cc, mm, ss, zb;
          int64_t half[4];
          int32_t s2[4];
          uint32_t mask[4];
          column(i, q, &jn, &cc, &mm, &ss, &zb, half, s2, mask);
#pragma unroll
          for (int j = 0; j < FM; ++j) {
            const int fr = wm * TM + j * MF;  // the fragment's first row in the tile
            if (fr < p * PR || fr >= (p + 1) * PR) continue;  // (wave-uniform)
            int32_t out[4];
            outputs(i, q, j, cc, mm, ss, zb, half, s2, mask, out);
            const int r = fr + (lane % MF) - p * PR;  // row inside the pass
            const int byte = jn * ES;                     // column byte in the row
            int8_t* dst = stg + r * RB + 16 * ((byte >> 4) ^ swz_row(r)) + (byte & 15);
            if constexpr (kOut32) {
              *reinterpret_cast<v4i*>(dst) = v4i{out[0], out[1], out[2], out[3]};
            } else {
              *reinterpret_cast<uint32_t*>(dst) =
                  ((uint32_t)out[0] & 0xFFu) | (((uint32_t)out[1] & 0xFFu) << 8) |
                  (((uint32_t)out[2] & 0xFFu) << 16) | ((uint32_t)out[3] << 24);
            }
          }
        }
      }
      __syncthreads();
      int8_t* crow0 = static_cast<int8_t*>(g.C) + ((m0 + p * PR) * g.ldc + n0) * ES;
#pragma unroll
      for (int it = 0; it < PR * CPR / (NW * 64); ++it) {
        const int id = it * NW * 64 + tid;
        const int r = id / CPR, ch = id % CPR;
        const v4i v = *reinterpret_cast<const v4i*>(stg + r * RB + 16 * (ch ^ swz_row(r)));
        *reinterpret_cast<v4i*>(crow0 + (int64_t)r * g.ldc * ES + 16 * ch) = v;
      }
      if (p + 1 < BM / PR) __syncthreads();
    }
    return;
  }

#pragma unroll
  for (int i = 0; i < FN; ++i) {
#pragma unroll
    for (int q = 0; q < QN; ++q) {
      int jn;
      v4i cc, mm, ss, zb;
      int64_t half[4];
      int32_t s2[4];
      uint32_t mask[4];
      column(i, q, &jn, &cc, &mm, &ss, &zb, half, s2, mask);
      const int64_t n = n0 + jn;
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int64_t m = m0 + wm * TM + j * MF + (lane % MF);
        int32_t out[4];
        outputs(i, q, j, cc, mm, ss, zb, half, s2, mask, out);
        if (full) {
          if constexpr (kOut32) {
            *reinterpret_cast<v4i*>(static_cast<int32_t*>(g.C) + m * g.ldc + n) =
                v4i{out[0], out[1], out[2], out[3]};
          } else {
            const uint32_t w = ((uint32_t)out[0] & 0xFFu) | (((uint32_t)out[1] & 0xFFu) << 8) |
                               (((uint32_t)out[2] & 0xFFu) << 16) | ((uint32_t)out[3] << 24);
            *reinterpret_cast<uint32_t*>(static_cast<int8_t*>(g.C) + m * g.ldc + n) = w;
          }
        } else if (m < g.M) {
          if constexpr (kOut32) {
            int32_t* crow = static_cast<int32_t*>(g.C) + m * g.ldc;
            if (c_vec && n + 3 < g.N) {
              *reinterpret_cast<v4i*>(crow + n) = v4i{out[0], out[1], out[2], out[3]};
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (n + r < g.N) crow[n + r] = out[r];
            }
          } else {
            int8_t* crow = static_cast<int8_t*>(g.C) + m * g.ldc;
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (n + r < g.N) crow[n + r] = (int8_t)out[r];
          }
        }
      }
    }
  }
}

}  // namespace qp
