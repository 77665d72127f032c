// Device pieces shared by the gfx950 attention kernels (attn.hip,
// attn_pair.hip): vector types, raw buffer resources, direct global-to-LDS
// copies, cross-lane reductions of the 32x32 MFMA layout and bf16 packing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace sa {
namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4s __attribute__((ext_vector_type(4)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T *)(p))

template <int N>
using Int = std::integral_constant<int, N>;
template <bool B>
using Bool = std::integral_constant<bool, B>;

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;       // log2 units
constexpr float kPMax = 4294967296.0f;      // 2^32: largest P a full tile may use before it rescales
constexpr int kBufferFlags = 0x00020000;    // raw buffer, 32-bit data format
constexpr int kVmcntZero = 0x0F70;          // s_waitcnt vmcnt(0), other counters untouched
// sched_group_barrier instruction classes
constexpr int kSchedVALU = 0x002;
constexpr int kSchedMFMA = 0x008;
constexpr int kSchedDSRead = 0x100;

// Raw buffer resource: base, no stride, num_records bytes, raw 32-bit format.
__device__ __forceinline__ i32x4s buffer_rsrc(const void *base, uint32_t num_bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4s r;
  r[0] = (int)(uint32_t)a;
  r[1] = (int)(uint32_t)(a >> 32) & 0xffff;
  r[2] = (int)num_bytes;
  r[3] = kBufferFlags;
  return r;
}

// Global -> LDS copy of 16 (or 4) bytes per lane: lane l writes LDS byte
// lds_base + 16*l (4*l).  Offsets at or past num_records read as zero.
// Issued as inline asm so the compiler does not order later LDS reads of the
// other ring slot behind it; the caller waits (vmcnt) before the barrier that
// publishes the data.
// The LDS address is lds_base + kOff (kOff folded into the M0 write, so the
// caller keeps one base register per ring slot).  A buffer load into LDS
// needs one wait state after an SALU write of M0, which the hardware does
// not check: hence the s_nop.
template <int kOff>
__device__ __forceinline__ void lds_dma_b128(const i32x4s &rsrc, uint32_t voffset, uint32_t lds_base) {
  asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "s"(lds_base), "i"(kOff)
               : "memory", "m0", "scc");
}
// The same copy with an immediate offset kImm (< 4096) on the global address:
// the immediate also moves the LDS address, so M0 takes it off again.  The
// copy lands at lds_base + kOff and reads voffset + kImm.
template <int kOff, int kImm>
__device__ __forceinline__ void lds_dma_b128_imm(const i32x4s &rsrc, uint32_t voffset, uint32_t lds_base) {
  static_assert(kImm >= 0 && kImm < 4096 && kOff >= kImm, "immediate offset out of range");
  asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen offset:%4 lds"
               :
               : "v"(voffset), "s"(rsrc), "s"(lds_base), "i"(kOff - kImm), "i"(kImm)
               : "memory", "m0", "scc");
}
// Both 128-byte halves of 8 key rows: LDS lds_base + kOff gets the bytes at
// sbase + vlane (one 16-byte piece per lane), lds_base + kOff + 1024 those
// 128 bytes further on (through the immediate offset, which moves the LDS
// address too, so M0 takes it off).  The lane address is formed inside the
// block, where it also serves as the wait state the first M0 write needs;
// the second has an s_nop.  The address register is read when each load
// issues and is free afterwards.
template <int kOff>
__device__ __forceinline__ void lds_dma_b128_x2(const i32x4s &rsrc, uint32_t sbase, uint32_t vlane,
                                                uint32_t lds_base) {
  uint32_t t;
  asm volatile(
      "s_add_u32 m0, %3, %4\n\t"
      "v_add_u32 %0, %2, %1\n\t"
      "buffer_load_dwordx4 %0, %5, 0 offen lds\n\t"
      "s_add_u32 m0, %3, %6\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %5, 0 offen offset:128 lds"
      : "=&v"(t)
      : "v"(vlane), "s"(sbase), "s"(lds_base), "i"(kOff), "s"(rsrc), "i"(kOff + 1024 - 128)
      : "memory", "m0", "scc");
}
__device__ __forceinline__ void lds_dma_b32(const i32x4s &rsrc, uint32_t voffset, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "s"(lds_base)
               : "memory", "m0");
}

// x combined with the same register of lane ^ 32 (v_permlane32_swap).
__device__ __forceinline__ float max_with_partner(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_with_partner(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

}  // namespace attn
}  // namespace sa
