// Vector-memory loads that a kernel issues and awaits itself, for the deep prefetch rings of
// the weight-streaming GEMM and the attention chunks.  The compiler's own waits collapse a
// deep ring (at a loop head they fall back to waiting for everything), so these loads are
// inline assembly and the kernel places each wait.
//
// The rule every user follows: the compiler takes the destination of such a load as written
// when the asm statement ends, so every loaded value must reach exactly one vm_wait that names
// it, on every path, before anything else reads it.  The registers then stay reserved until
// the data is in, and nothing copies them early.  Two alternative waits for one value would
// make the compiler merge them with copies placed before one of the waits, and a load whose
// value is never awaited leaves its registers free for reuse while the data is still landing;
// so loads are unconditional (addresses clamped in bounds instead) and every ring slot is
// awaited once more after the loop.  tests/asm_waits.py checks this on the assembly.
#pragma once
#include "common.hpp"

namespace dfl {

__device__ __forceinline__ u32x4_t vm_load16_nt(const void* p) {
  u32x4_t v;
  asm volatile("global_load_dwordx4 %0, %1, off nt" : "=v"(v) : "v"(p));
  return v;
}

__device__ __forceinline__ u32x4_t vm_load16(const void* p) {
  u32x4_t v;
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(v) : "v"(p));
  return v;
}

// The same load addressed as a wavefront-uniform base (scalar registers) plus a per-lane
// 32-bit byte offset, which saves a 64-bit address register pair per lane.
__device__ __forceinline__ u32x4_t vm_load16(const void* sbase, uint32_t voff) {
  u32x4_t v;
  asm volatile("global_load_dwordx4 %0, %1, %2" : "=v"(v) : "v"(voff), "s"(sbase));
  return v;
}

// The same, non-temporal: for streams read once (the context K/V of a draft block).
__device__ __forceinline__ u32x4_t vm_load16_nt(const void* sbase, uint32_t voff) {
  u32x4_t v;
  asm volatile("global_load_dwordx4 %0, %1, %2 nt" : "=v"(v) : "v"(voff), "s"(sbase));
  return v;
}

// s_waitcnt vmcnt(N) that also passes v through, so no use of v is scheduled before it (the
// comment names v's registers in the assembly).  Vector loads complete in issue order for
// this count, so vmcnt(N) means every load but the N most recent is in.
template <int N, class T>
__device__ __forceinline__ void vm_wait(T& v) {
  static_assert(N >= 0 && N <= 63, "vmcnt is 6 bits");
  asm volatile("s_waitcnt vmcnt(%1) ; waits for %0" : "+v"(v) : "i"(N));
}

// s_waitcnt for "at most n vector-memory operations outstanding" (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14; expcnt and lgkmcnt left at their no-wait maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  constexpr int n = N > 63 ? 63 : N;
  __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

}  // namespace dfl
