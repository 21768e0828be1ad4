// lds_dma.h -- global->LDS 16-byte loads and counted waits on them, shared by
// the decode kernels that stream weights straight into LDS.
#pragma once

#include "kq_device.h"

namespace kq {

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// One global->LDS 16-byte load per lane: lane l's 16 bytes at `src` land at
// LDS byte address lds + 16*l.  Issued from asm so that the compiler does not
// treat it as an LDS store and wait for it before unrelated LDS reads; the
// kernel waits for these loads itself (vmcnt(0) and a barrier before a
// buffer is read).  The instruction has no register outputs.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(lds)
                 : "memory", "m0");
}
// The same with 4 bytes per lane: lane l's dword lands at lds + 4*l.
__device__ __forceinline__ void dma4(const void* src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(src), "s"(lds)
                 : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
    return (uint32_t)(uintptr_t)(const lds_u8*)p;
}

// Wait until at most n of this wave's vector-memory loads are outstanding
// (n is wave-uniform).  Loads complete in issue order, so waiting down to the
// number issued after a chunk's loads means that chunk has landed.  n is
// rounded down to one of a few encodable counts, which only waits longer.
#define KQ_VMCNT(N) __builtin_amdgcn_s_waitcnt(((N) & 15) | (7 << 4) | (15 << 8) | (((N) >> 4) << 14))
__device__ __forceinline__ void wait_loads_le(int n) {
    if (n >= 32) KQ_VMCNT(32);
    else if (n >= 24) KQ_VMCNT(24);
    else if (n >= 16) KQ_VMCNT(16);
    else if (n >= 12) KQ_VMCNT(12);
    else if (n >= 8) KQ_VMCNT(8);
    else if (n >= 6) KQ_VMCNT(6);
    else if (n >= 4) KQ_VMCNT(4);
    else if (n >= 3) KQ_VMCNT(3);
    else if (n >= 2) KQ_VMCNT(2);
    else if (n >= 1) KQ_VMCNT(1);
    else KQ_VMCNT(0);
}

}  // namespace kq
