// Device helpers shared by the MFMA kernels that stream blocks of bf16 rows
// through LDS with direct-to-LDS buffer loads (gfx950): vector types, buffer
// resources, the loads themselves, their waits, and MFMAs whose fp32 sums
// stay in the accumulation registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 v4bf16 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) v4bf16 lds_v4bf16;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

constexpr int kVmcnt0 = 0x0f70;          // s_waitcnt vmcnt(0) (expcnt, lgkmcnt left alone)
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer resource, gfx9 family
constexpr int kOob = 1 << 30;            // a source offset past every range

// A buffer resource over [p, p + bytes): a lane whose offset falls outside
// reads no memory and writes zeros to LDS, so a block's missing rows hold
// zeros and a padding load (bytes = 0) only writes zeros.
__device__ inline i32x4 make_rsrc(const void* p, int bytes) {
  const unsigned long long a = (unsigned long long)p;
  return i32x4{__builtin_amdgcn_readfirstlane((int)(unsigned)a),
               __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffffu)),
               __builtin_amdgcn_readfirstlane(bytes), kRsrcWord3};
}
// One direct-to-LDS load of 64 16-byte units, lane l's to dst + 16 l (inline
// asm: it writes only LDS, no register is left in flight; the callers count
// these loads by hand).
__device__ inline void dma16(const i32x4& rs, int voff, lds_char* dst) {
  const int m0 = __builtin_amdgcn_readfirstlane((int)(uintptr_t)dst);
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff),
               "s"(rs), "s"(m0)
               : "m0", "memory");
}
template <int N>
__device__ inline void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// fp32 sums that stay in the accumulation registers: inline-asm MFMAs with an
// AGPR accumulator (with the builtin the compiler may move long-lived sums
// between the register files every iteration).  Their hazards are covered by
// hand: settle_acc puts more than the 2 wait states an MFMA read needs after
// the sums are zeroed, and mfma_drain_acc waits out the last product before
// the sums are read.  The A and B operands must not come from a VALU write
// just before (LDS reads and registers loaded earlier are fine).
__device__ __forceinline__ void mfma_agpr(f32x16& acc, bf16x8 a, bf16x8 b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
template <int N>
__device__ __forceinline__ void settle_acc(f32x16 (&acc)[N]) {
#pragma unroll
  for (int k = 0; k < N; ++k) asm volatile("" : "+a"(acc[k]));
  asm volatile("s_nop 4" ::: "memory");
}
template <int N>
__device__ __forceinline__ void mfma_drain_acc(f32x16 (&acc)[N]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int k = 0; k < N; ++k) asm volatile("" : "+a"(acc[k]));
}

}  // namespace dev
}  // namespace mla
