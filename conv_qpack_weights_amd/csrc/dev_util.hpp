// dev_util.hpp -- small gfx950 device helpers shared by the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace qp {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;
typedef __attribute__((address_space(3))) int8_t lds_i8;

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] and
// [15:14], expcnt[6:4], lgkmcnt[11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (((N >> 4) & 3) << 14) | 0x70 | 0xF00);
}

// 16 bytes per lane from base + voff + soff straight into LDS (lane i lands
// at dst + 16*i; dst must be wave-uniform), through a buffer resource.  The
// buffer form is counted by the compiler as a vector-memory load only, which
// keeps its own waits for other loads exact (the global form is also counted
// against the LDS counter and makes it drain both).  The caller waits for
// these loads itself (vmcnt) before reading the LDS they fill.  The body
// exists in the device pass only.
__device__ __forceinline__ void dma16_to_lds(const void* base, lds_void_t* dst, uint32_t voff,
                                             uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000), dst,
      16, voff, soff, 0, 0);
#endif
}

// The same with 4 bytes per lane (lane i lands at dst + 4*i).
__device__ __forceinline__ void dma4_to_lds(const void* base, lds_void_t* dst, uint32_t voff,
                                            uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000), dst,
      4, voff, soff, 0, 0);
#endif
}

}  // namespace qp
