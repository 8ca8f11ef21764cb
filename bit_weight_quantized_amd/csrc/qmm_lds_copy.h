// Global -> LDS copies (buffer loads with the LDS as destination) and the
// vmcnt waits that order them, shared by the kernels that stage operands in
// LDS without passing them through registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left at their maxima)
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// global (buffer) -> LDS copies: every lane moves 16 (4) bytes to LDS byte
// address lds + 16·lane (lds + 4·lane); lds is wave-uniform.  Written as
// inline asm so the compiler does not track them: it cannot tell the LDS
// slots apart and would wait for every copy in flight before each LDS read.
// The kernels order them with explicit vmcnt waits instead, and issue no
// other vector-memory loads while copies are in flight (or wait for all of
// them).  Each copy sets m0 itself; the compiler warns that it may not
// preserve m0 across the asm, which is sound only while no compiler-generated
// instruction in a kernel that copies keeps a value in m0 (a CPU test
// compiles the files that include this header and checks).
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(r), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void copy4_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(r), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return uint32_t(uintptr_t((lds_ptr_t)p));
}

}  // namespace qmm
