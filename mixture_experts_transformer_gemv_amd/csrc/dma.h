// Direct global -> LDS copies and the waits around them, shared by the kernels that stage tiles in LDS (gfx950).
#pragma once

#include "common.h"

// The copies are issued from inline assembly (they only set M0, no destination register).
#pragma clang diagnostic ignored "-Winline-asm"

namespace gm {

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef short i16x4_t __attribute__((ext_vector_type(4)));

// 16-byte global -> LDS copy of one wave: lane i reads base + voff (bytes; base wave-uniform) and writes LDS
// bytes [dst + 16 i, dst + 16 i + 16) (dst wave-uniform).  Inline assembly so that the compiler does not wait for
// every copy in flight before each LDS read (it cannot tell the ring stages apart); completion is awaited with
// an explicit vmcnt before the stage barrier.  No destination register; no "memory" clobber (the barrier
// sequence orders the LDS accesses).
__device__ __forceinline__ void g2lds16(const void* base, uint32_t voff, uint32_t dst) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(base), "s"(dst) : "m0");
}

// As g2lds16, with the nontemporal hint: the lines pass through the caches with low retention.  For data read
// once per launch (weights streamed by the few-token kernels), where it leaves the caches to the rest and reads
// HBM faster (measured on MI355X: 6.3 -> 6.8 TB/s for the weight streams).
__device__ __forceinline__ void g2lds16_nt(const void* base, uint32_t voff, uint32_t dst) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" : : "v"(voff), "s"(base), "s"(dst) : "m0");
}

// Descriptor of a raw (unstrided) buffer of `bytes` bytes at `base` for the copies below: a lane whose offset
// is at or past `bytes` reads zeros and touches no memory.  Word 3 selects 32-bit data (required for the range
// check of untyped loads).
__device__ __forceinline__ u32x4_t buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4_t{uint32_t(a), uint32_t(a >> 32) & 0xffffu, bytes, 0x00020000u};
}

// 16-byte buffer -> LDS copy of one wave: lane i reads buffer bytes [soff + voff, +16) (zeros if voff is out of
// range; soff wave-uniform) and writes LDS bytes [dst + 16 i, dst + 16 i + 16).  Same waiting rules as g2lds16.
__device__ __forceinline__ void b2lds16(const u32x4_t& rsrc, uint32_t soff, uint32_t voff, uint32_t dst) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               : : "v"(voff), "s"(rsrc), "s"(soff), "s"(dst) : "m0");
}

// LDS transpose read: within each 16-lane group, lane j receives element j % 4 of the 8 bytes addressed by lane
// 4 r + j / 4 (r = 0..3).
__device__ __forceinline__ u32x2_t lds_tr16(const lds_u8* p) {
  return __builtin_bit_cast(
      u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(p)));
}

// LDS 8-bit transpose read: within each 16-lane group, lane j receives byte j % 8 of the 8 bytes addressed by
// lane 2 r + j / 8 (r = 0..7), byte r of the result from lane 2 r + j / 8.
__device__ __forceinline__ u32x2_t lds_tr8(const lds_u8* p) {
  typedef int i32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2_t*)(p)));
}

// Wait until at most N vector memory operations of this wave are outstanding (copies complete in issue order).
template <int N> __device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 0..63");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N));
}

// Workgroup barrier ordering LDS accesses only (a __syncthreads would also wait for all copies in flight).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace gm
