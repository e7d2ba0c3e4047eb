// Direct memory -> LDS loads and the waits that go with them, shared by the
// kernels that stage their operands in LDS (the grouped GEMMs, the router).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {
namespace lds {

#define LOCAL __attribute__((address_space(3)))

// Workgroup barrier without a memory fence.  __syncthreads() carries a
// workgroup release fence, which makes the compiler wait for every
// outstanding vector-memory operation (vmcnt(0)) -- that would drain the
// prefetch pipeline at every K step.  Here the caller has already waited for
// the loads it needs; lgkmcnt(0) completes this wave's LDS operations, and
// the signal fences keep the compiler from moving memory accesses across.
__device__ __forceinline__ void barrier_no_fence() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt((15 << 0) | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Direct memory -> LDS loads through a buffer resource
// (buffer_load_dword[x4] ... lds): lane i reads base + soffset + voffset_i and
// its 4 or 16 bytes land at LDS byte m0 + 4i / 16i.  The per-lane offset is
// fixed for the tile and the per-step offset is a scalar, so a K step's loads
// need no vector address arithmetic.  Issued from inline assembly so that the
// compiler does not model them: its wait-count pass would otherwise make every
// later LDS read wait for all of them (vmcnt(0)), which defeats the prefetch.
// Callers wait with explicit vmcnt counts before reading a slot; the "memory"
// clobber keeps other memory accesses from moving across.
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
// Raw buffer over [p, p + 4 GiB): the offsets computed below stay inside
// the caller's buffers, as the former flat addresses did.
__device__ __forceinline__ i32x4 buffer_rsrc(const void *p) {
    const uint64_t b = (uint64_t)(uintptr_t)p;
    i32x4 r;
    r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(b >> 32) & 0xffffu));  // stride 0
    r.z = -1;                                                                       // num_records
    r.w = 0x00020000;                                                               // 32-bit raw data
    return r;
}
__device__ __forceinline__ void dma16(uint32_t lds_addr, uint32_t voff, i32x4 rsrc, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4(uint32_t lds_addr, uint32_t voff, i32x4 rsrc, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :
                 : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}

// The same loads with the non-temporal hint, for weights that one workgroup
// streams once: they then do not displace the activations, router weights
// and intermediates that the block's other kernels find in the last-level
// cache (decode-shaped chunk: block 0.170 -> 0.155 ms, every kernel of the
// block faster).  The matrix-core tiles use them only for 32-row tiles that
// are their expert's only M-tile; on taller tiles the hint made gate/up
// slower even where no other tile re-reads the weights (full chunk 234 ->
// 237.5 us, mid 46.6 -> 48.1 us).
__device__ __forceinline__ void dma16nt(uint32_t lds_addr, uint32_t voff, i32x4 rsrc, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
                 :
                 : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4nt(uint32_t lds_addr, uint32_t voff, i32x4 rsrc, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen nt lds"
                 :
                 : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}

// vmcnt(n) only (expcnt and lgkmcnt left at their no-wait maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

}  // namespace lds
}  // namespace moe
