// Direct global -> LDS copies (gfx950), shared by the matrix-core kernels.
#pragma once

#include "common.hpp"

namespace msa {

typedef __attribute__((address_space(3))) void* lds_ptr;

// LDS byte address of a __shared__ object.
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(T* p) {
    return uint32_t(size_t((lds_ptr)p));
}

// One 16-byte direct global->LDS copy per lane: lane i's 16 bytes land at LDS
// byte address lds + 16 i (lds wave-uniform).  Written as asm so that the only
// waits on these copies are the explicit MSA_WAIT_VMCNT ones (the compiler
// would otherwise make every LDS read wait for every copy in flight); the copy
// has no register result.  Vector-memory operations complete in issue order,
// so any other load issued after a copy only makes a later wait stronger.
__device__ __forceinline__ void lds_copy16(const u32x4* src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(lds) : "memory", "m0");
}

// The same copy addressed as a wave-uniform base plus a per-lane 32-bit byte
// offset: lane i reads base + voff_i.  The base and the LDS address are scalar,
// so a loop of copies needs no vector address arithmetic between the
// matrix-core instructions it is interleaved with.
__device__ __forceinline__ void lds_copy16_s(const u32x4* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(base), "s"(lds)
                 : "memory", "m0");
}

}  // namespace msa

// s_waitcnt with only the vector-memory count limited (expcnt and lgkmcnt left
// at their maxima): GFX9 encoding, vmcnt in bits [3:0] and [15:14].
#define MSA_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | (7 << 4) | (15 << 8))
