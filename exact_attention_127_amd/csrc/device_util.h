// Device helpers shared by the matrix-core attention kernels (gfx950 only:
// LDS transposing reads, HBM -> LDS copies, vmcnt waits, half-wave
// reductions).  Included only in device compilation passes.
#pragma once
#include "common.h"

namespace attn127 {

typedef __attribute__((address_space(3))) void lds_void;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i32 lds_v2i32;

// generic pointer into a __shared__ array -> LDS address space (C-style cast:
// the address-space change is not expressible with the C++ casts)
__device__ __forceinline__ lds_void* as_lds(const char* p) { return (lds_void*)(const_cast<char*>(p)); }
__device__ __forceinline__ v4i16 ds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(const_cast<char*>(p)));
}

// Buffer descriptor for `bytes` bytes from `base`: reads past the end return 0.
__device__ __forceinline__ i32x4 buffer_desc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{static_cast<int>(static_cast<uint32_t>(a)), static_cast<int>(static_cast<uint32_t>(a >> 32)),
               static_cast<int>(bytes), 0x00020000};
}

// Buffer resource for a wave-uniform range [base, base + bytes): base and
// size go through readfirstlane, so the descriptor lives in scalar
// registers (held in vector registers, it makes the compiler wrap every
// access in a loop over the lanes' distinct descriptors).  Accesses at or
// past `bytes` read zero and drop stores.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint64_t u = (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32))) << 32) |
                     static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a)));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(u), 0, __builtin_amdgcn_readfirstlane(bytes),
                                           0x00020000);
}

// 32-bit LDS byte address of a pointer into a __shared__ array, made
// wave-uniform (an SGPR value).
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(as_lds(p))));
}

// One 16-byte-per-lane HBM -> LDS copy: lane i's 16 bytes land at LDS byte
// address lds_block + 16*i.  Issued as inline assembly so the compiler does
// not serialise it against unrelated LDS reads; completion is tracked by the
// explicit vmcnt waits of the tile loop.
__device__ __forceinline__ void dma16(const i32x4& desc, uint32_t lds_block, int voffset) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds_block);   // uniform by construction
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(m), "v"(voffset), "s"(desc) : "memory", "m0");
#pragma clang diagnostic pop
}
__device__ __forceinline__ void dma16(const i32x4& desc, const char* lds_block, int voffset) {
  dma16(desc, lds_addr(lds_block), voffset);
}

// Wait until at most n of this wave's vector-memory operations are in
// flight (s_waitcnt vmcnt(n); the expcnt and lgkmcnt fields left at maximum).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | n);
}

// v_permlane32_swap with both operands = x: lanes 0..31 get (own, partner),
// lanes 32..63 get (partner, own), partner being the lane 32 away; combining
// the pair gives the same two-lane reduction on every lane.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ v2i32 ds_read_tr8(const char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32*)(const_cast<char*>(p)));
}

}  // namespace attn127
