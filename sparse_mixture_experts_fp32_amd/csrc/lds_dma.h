// Direct-to-LDS loads (gfx950 global_load_lds_dwordx4) and the explicit waits
// and barriers that go with them.
//
// One load copies 16 bytes per lane from global memory into LDS: lane l writes
// LDS byte lds + 16 l, where lds (wave-uniform) travels in M0. The compiler
// cannot tell which LDS bytes such a load writes, so code that keeps these
// loads in flight across barriers waits for them itself (s_waitcnt vmcnt) and
// uses the barrier below instead of __syncthreads (whose fence would drain
// every load in flight).
#pragma once

#include "device_common.h"

namespace moe {

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// sbase (wave-uniform, SGPRs) + voff (per lane) -> LDS
static __device__ __forceinline__ void dma_saddr(uint32_t lds, const void* sbase, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}
// sbase + voff -> LDS, 4 bytes per lane (lane l writes LDS byte lds + 4 l)
static __device__ __forceinline__ void dma_saddr_dword(uint32_t lds, const void* sbase, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}
// a 64-bit address per lane -> LDS
static __device__ __forceinline__ void dma_vaddr(uint32_t lds, const void* addr) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(addr)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most N of this wave's vector-memory operations are in flight and
// its LDS operations are done, then barrier.
template <int N>
static __device__ __forceinline__ void wait_barrier() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

static __device__ __forceinline__ void wait_loads_barrier(int n) {  // n wave-uniform, 0 .. 2
    switch (n) {
        case 0: wait_barrier<0>(); break;
        case 1: wait_barrier<1>(); break;
        default: wait_barrier<2>(); break;
    }
}

// A pointer the compiler can keep in scalar registers (the value must be wave-uniform).
static __device__ __forceinline__ const void* uniform_ptr(const void* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
    return reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// LDS byte address of a pointer into a __shared__ array (the low half of its
// generic address).
static __device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

}  // namespace moe
