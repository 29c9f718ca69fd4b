// Buffer-resource copies global -> LDS for the gfx950 kernels.
#pragma once
#include "common.hpp"

namespace moe {

// Buffer copies.  A raw buffer resource (stride 0) over an operand: loads at
// byte offsets (voffset + soffset) >= `bytes` are out of range and return
// zeros (what lands in LDS is then zero) without touching memory.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcWord3 = 0x00020000;   // untyped dword access
constexpr uint32_t kPadOffset = 0x7ffffff0u;  // past every operand's range

__device__ __forceinline__ uint32_t uniform(uint32_t v) {
  return __builtin_amdgcn_readfirstlane(v);
}
__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint64_t u = ((uint64_t)uniform((uint32_t)(a >> 32)) << 32) | uniform((uint32_t)a);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(u), (short)0,
                                           (int)uniform(bytes), kRsrcWord3);
}
// Cache-policy field of a buffer load: the non-temporal (streaming) hint.
constexpr int kNonTemporal = 2;

// 16 bytes per lane from r at (voff + soff) to LDS at dst + 16 * lane
template <int AUX = 0>
__device__ __forceinline__ void copy16(Rsrc r, char* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16,
                                           voff, soff, 0, AUX);
}

}  // namespace moe
