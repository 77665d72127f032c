// Small device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

// Workgroups are dispatched to the 8 XCDs round-robin (workgroup w runs on
// XCD w % 8).  Map the hardware id to a logical id so that each XCD gets one
// contiguous range of logical work items: neighbouring items (the query
// blocks of one head) then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int w, int total) {
  constexpr int kXcd = 8;
  const int xcd = w % kXcd;
  const int idx = w / kXcd;
  const int per = total / kXcd;
  const int rem = total % kXcd;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

__device__ __forceinline__ uint32_t shfl_xor_u32(uint32_t v, int mask) {
  return static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), mask, 64));
}

__device__ __forceinline__ float shfl_xor_f32(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
  const uint32_t lo = shfl_xor_u32(static_cast<uint32_t>(v), mask);
  const uint32_t hi = shfl_xor_u32(static_cast<uint32_t>(v >> 32), mask);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Make LDS writes by any lane of this wave visible to later LDS reads by
// other lanes of the same wave.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace sa
