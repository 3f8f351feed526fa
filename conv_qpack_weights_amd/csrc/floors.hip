// floors.hip -- machine floors measured beside the hot path: a read-only
// HBM stream and a dense int8 MFMA loop.  Built into libqpfloors.so, which
// only the benchmark loads; nothing in libqpack.so depends on it.
//
// Both kernels do no useful work: their results only feed a store that is
// taken when a value equals a constant no input produces, which keeps the
// compiler from dropping the loads and MFMAs while writing nothing.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr uint32_t kNever = 0x9E3779B9u;

// Read n16 16-byte vectors, U per thread in flight per round; the rounds
// stride over the whole grid so that each load instruction of a wave covers
// 1 KiB of contiguous memory.
template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ src,
                                                          int64_t n16, uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t x = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = src[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (x == kNever) sink[0] = x;
}

// Each wave: `iters` rounds of NACC independent v_mfma_i32_32x32x32_i8
// (65536 int8 operations each).  NACC = 16 holds 256 accumulator registers
// (one wave per SIMD); NACC = 8 leaves room for two.
// kRandom: the operands rotate through 8 register pairs of random-looking
// bytes, like the changing fragments of a GEMM on uniform int8 data; the
// MFMA's power then depends on the data, and the clock it sustains is the
// part's real dense-int8 ceiling for such data.  Otherwise the operands are
// small constant values (the clock-limited ceiling).
template <int NACC, bool kRandom>
__global__ __launch_bounds__(256) void mfma_loop_kernel(int32_t iters, uint32_t* sink) {
  constexpr int NOP = kRandom ? 8 : 1;
  const int t = threadIdx.x;
  v4i a[NOP], b[NOP];
#pragma unroll
  for (int p = 0; p < NOP; ++p) {
    if constexpr (kRandom) {
      const uint32_t s0 = 0x9E3779B9u * (uint32_t)(t + 1 + 131 * p) + blockIdx.x * 0x85EBCA6Bu;
      a[p] = v4i{(int)s0, (int)(s0 * 3u), (int)(s0 * 5u), (int)(s0 * 7u)};
      b[p] = v4i{(int)(s0 ^ 0xA5A5A5A5u), (int)(s0 * 11u), (int)(s0 * 13u), (int)(s0 * 17u)};
    } else {
      a[p] = v4i{t, t + 1, t + 2, t + 3};
      b[p] = v4i{t ^ 5, t ^ 6, t ^ 7, t ^ 9};
    }
  }
  v16i acc[NACC];
#pragma unroll
  for (int j = 0; j < NACC; ++j) acc[j] = v16i{} + j;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < NACC; ++j)
      acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[j % NOP], b[(3 * j + it) % NOP], acc[j], 0,
                                                      0, 0);
  }
  uint32_t x = 0;
#pragma unroll
  for (int j = 0; j < NACC; ++j) x ^= (uint32_t)acc[j][0] ^ (uint32_t)acc[j][15];
  if (x == kNever) sink[0] = x;
}

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 16, 16-byte aligned) with `blocks` workgroups
// of 256 threads, `unroll` (4 or 8) loads in flight per thread.
int qpf_stream_read(const void* src, int64_t bytes, int32_t blocks, int32_t unroll,
                    uint32_t* sink, hipStream_t stream) {
  if (!src || bytes <= 0 || (bytes & 15) || ((uintptr_t)src & 15) || blocks <= 0 || !sink)
    return -1;
  const int64_t n16 = bytes / 16;
  if (unroll == 8)
    hipLaunchKernelGGL(stream_read_kernel<8>, dim3(blocks), dim3(256), 0, stream,
                       static_cast<const uint4*>(src), n16, sink);
  else if (unroll == 4)
    hipLaunchKernelGGL(stream_read_kernel<4>, dim3(blocks), dim3(256), 0, stream,
                       static_cast<const uint4*>(src), n16, sink);
  else
    return -1;
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// `blocks` workgroups of four waves, each running `iters` rounds of `nacc`
// (8 or 16) MFMAs; `random` selects rotating random-looking operands.
// Operations per launch: blocks * 4 * iters * nacc * 65536.
int qpf_mfma_loop(int32_t iters, int32_t blocks, int32_t nacc, int32_t random, uint32_t* sink,
                  hipStream_t stream) {
  if (iters <= 0 || blocks <= 0 || !sink) return -1;
  if (nacc == 16 && random)
    hipLaunchKernelGGL((mfma_loop_kernel<16, true>), dim3(blocks), dim3(256), 0, stream, iters,
                       sink);
  else if (nacc == 16)
    hipLaunchKernelGGL((mfma_loop_kernel<16, false>), dim3(blocks), dim3(256), 0, stream, iters,
                       sink);
  else if (nacc == 8 && random)
    hipLaunchKernelGGL((mfma_loop_kernel<8, true>), dim3(blocks), dim3(256), 0, stream, iters,
                       sink);
  else if (nacc == 8)
    hipLaunchKernelGGL((mfma_loop_kernel<8, false>), dim3(blocks), dim3(256), 0, stream, iters,
                       sink);
  else
    return -1;
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// An empty launch: the per-kernel cost of a dispatch in the same harness.
__global__ void empty_kernel() {}
int qpf_empty(hipStream_t stream) {
  hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, stream);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
