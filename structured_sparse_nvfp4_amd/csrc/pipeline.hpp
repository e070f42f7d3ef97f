// Software-pipelining helpers for gfx950 kernels that stage operands through LDS with the
// direct global->LDS loads (global_load_lds_dword[x4]). Such a load writes LDS without passing
// through registers, so the compiler does not wait for it before LDS reads: the kernels wait
// explicitly with s_waitcnt vmcnt and synchronise the workgroup with a bare s_barrier.
#pragma once
#include <hip/hip_runtime.h>

namespace ssn {

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ void lds_dma16(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)l, 16, 0, 0);
}
__device__ __forceinline__ void lds_dma4(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)l, 4, 0, 0);
}

// The same copies issued as buffer loads (MUBUF with the LDS bit) through a raw buffer resource:
// base address `base` (wave-uniform), no bounds clamp, 32-bit byte offsets (per lane `voff`,
// wave-uniform `soff`). The compiler's wait insertion treats the FLAT-encoded global form as an
// access that may complete out of order with LDS reads, so every wait for an LDS read in a
// kernel that holds one becomes lgkmcnt(0); with the buffer form it keeps exact counts.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFFF, 0x00020000);
}
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* l) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)l, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void lds_dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* l) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)l, 4, voff, soff, 0, 0);
}

// s_waitcnt vmcnt(n) with expcnt/lgkmcnt left unconstrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier without the memory fence of __syncthreads(): the fence would make the
// compiler drain every outstanding load (vmcnt(0)), including the stages still meant to be in
// flight. Visibility of a stage is established by the explicit vmcnt wait before this barrier;
// the empty asm statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace ssn
