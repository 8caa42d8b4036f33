// Device helpers shared by the library's HIP kernels (the Huffman decoders in
// entro_decode.hip, the rANS decoder in entro_rans.hip): LDS types and
// addresses, values made visibly uniform, and the streamed output stores.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "entro_internal.h"

namespace entro {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// The workgroup's dynamic LDS.  The kernels declare no static LDS, so it
// starts at LDS address 0 (checked once per workgroup, see lds_at_zero) and
// the table placed there (Huffman two-code table, rANS slot table) is read
// at plain byte addresses.
extern __shared__ u32x4 dyn_lds[];

typedef __attribute__((address_space(3))) const uint32_t lds_u32;
typedef __attribute__((address_space(3))) const u32x2 lds_u32x2;

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p;
}

__device__ __forceinline__ bool lds_at_zero() { return lds_addr(dyn_lds) == 0u; }

typedef __attribute__((address_space(3))) void lds_void;

// Copy n16 16-byte vectors of a buffer resource (vector v at byte offset
// 16 v) to LDS (at byte address lds + 16 v) with loads that write LDS
// directly: lane l of an instruction fills the l-th 16-byte slot after the
// instruction's LDS base, 1 KiB per wavefront and instruction, so every load
// of the copy is in flight at once and no registers hold the data.  Dwords
// past the resource's range land as zero; lanes past n16 write nothing.  The
// wavefront must wait_lds_copy() before it reads the copy.  The copy's LDS
// writes do not pass through the LDS instruction queue and can land before
// an LDS read of the area that the wavefront issued earlier: its LDS reads
// are waited for first.
__device__ __forceinline__ void lds_copy16(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t n16, uint32_t lane) {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  asm volatile("" ::: "memory");
  for (uint32_t v0 = 0; v0 < n16; v0 += 64u) {
    const uint32_t v = v0 + lane;
    if (v < n16)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(uintptr_t)(lds + 16u * v0), 16, 16u * v, 0, 0, 0);
  }
}

// s_waitcnt vmcnt(0): the copies above have landed in LDS (and, the counter
// being shared, earlier stores have completed); the compiler barrier keeps
// later LDS reads below it.
__device__ __forceinline__ void wait_lds_copy() {
  __builtin_amdgcn_s_waitcnt(0x0F70);
  asm volatile("" ::: "memory");
}

// Output element of the decode kernels: the value's type and the cache
// policy of its stores (kStoreNT or kStoreCached).
template <typename T, int CP>
struct OutElem {
  T v;
  static constexpr int cp = CP;
};

// One output element per lane through a buffer resource: per-lane byte
// offset in a vector register, per-step offset in a scalar register.
// The value sits in bits [31:16] ([23:16] for codes) of the table entry and
// goes out with the d16_hi store forms, so no shift is spent on it.  (The
// outputs are never read back by the kernel, so the compiler needs no
// knowledge of these writes; they carry OutT's cache policy like every
// output store.)  The compiler does not insert hazard wait
// states around inline assembly, and a vector-memory instruction must not
// read an SGPR in the 5 cycles after a VALU wrote it (as v_readlane does when
// the resource comes back from a spill), hence the s_nop 4.
template <typename OutT>
__device__ __forceinline__ void store_out(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t e) {
  static_assert(OutT::cp == kStoreNT || OutT::cp == kStoreCached, "cache policy");
  if (sizeof(OutT) == 1 && OutT::cp == kStoreNT)
    asm volatile("s_nop 4\n\tbuffer_store_byte_d16_hi %0, %1, %2, %3 offen nt"
                 : : "v"(e), "v"(voff), "s"(r), "s"(soff));
  else if (sizeof(OutT) == 1)
    asm volatile("s_nop 4\n\tbuffer_store_byte_d16_hi %0, %1, %2, %3 offen"
                 : : "v"(e), "v"(voff), "s"(r), "s"(soff));
  else if (OutT::cp == kStoreNT)
    asm volatile("s_nop 4\n\tbuffer_store_short_d16_hi %0, %1, %2, %3 offen nt"
                 : : "v"(e), "v"(voff), "s"(r), "s"(soff));
  else
    asm volatile("s_nop 4\n\tbuffer_store_short_d16_hi %0, %1, %2, %3 offen"
                 : : "v"(e), "v"(voff), "s"(r), "s"(soff));
}

// Both outputs of a pair step with one store per lane.  ab holds the lane's
// two values packed (bf16: step t in bits [15:0], step t+1 in [31:16]; codes:
// bytes 0 and 1).  Adjacent lanes swap ab (DPP quad_perm 1,0,3,2); an even
// lane then stores its own and its odd neighbour's step-t value, an odd lane
// both step-(t+1) values, at voffp = (even lane's offset) + (lane & 1) * W
// elements.  All 64 lanes must be active; W >= 2.
template <int MODE>
__device__ __forceinline__ uint32_t pack_ab(uint32_t eA, uint32_t eB) {
  return MODE == kModeU8 ? __builtin_amdgcn_perm(eB, eA, 0x0C0C0602u) : __builtin_amdgcn_perm(eB, eA, 0x07060302u);
}

template <int MODE>
__device__ __forceinline__ uint32_t pair_sel(uint32_t lane) {
  if (MODE == kModeU8) return (lane & 1u) ? 0x0C0C0105u : 0x0C0C0400u;
  return (lane & 1u) ? 0x03020706u : 0x05040100u;
}

template <int MODE, int CP>
__device__ __forceinline__ void store_pair(__amdgpu_buffer_rsrc_t r, uint32_t voffp, uint32_t soff, uint32_t ab,
                                           uint32_t sel) {
  const uint32_t nb = (uint32_t)__builtin_amdgcn_mov_dpp((int)ab, 0xB1, 0xF, 0xF, false);
  const uint32_t v = __builtin_amdgcn_perm(nb, ab, sel);
  if (MODE == kModeU8) __builtin_amdgcn_raw_buffer_store_b16((uint16_t)v, r, (int)voffp, (int)soff, CP);
  else __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)voffp, (int)soff, CP);
}

__device__ __forceinline__ uint32_t pair_voff(uint32_t lane_off, uint32_t lane, uint32_t W, uint32_t elem) {
  return ((lane_off & ~1u) + (lane & 1u) * W) * elem;
}

// values that are equal in all lanes, made visibly uniform for the compiler
__device__ __forceinline__ uint32_t rfl(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint64_t rfl64(uint64_t v) {
  return ((uint64_t)rfl((uint32_t)(v >> 32)) << 32) | rfl((uint32_t)v);
}
}  // namespace entro
