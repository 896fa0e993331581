// Direct-to-LDS buffer loads on gfx950 and the waits that go with them.
#pragma once
#include "sa_device.hpp"

namespace sa {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource: base, no stride, `bytes` records (reads at or past them return zeros
// without a memory access), gfx9 default format word.
__device__ __forceinline__ i32x4 make_buffer_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    i32x4 r;
    r[0] = (int32_t)(uint32_t)a;
    r[1] = (int32_t)(uint32_t)(a >> 32) & 0xffff;
    r[2] = (int32_t)bytes;
    r[3] = 0x00020000;
    return r;
}

// A buffer offset past the end of every buffer a resource above may describe (the host
// keeps them under 2^31 bytes): the load returns zeros.
constexpr int kBufferPastEnd = 0x7ffffff0;

__device__ __forceinline__ uint32_t lds_byte_addr(SA_LDS const void* p) { return (uint32_t)(uintptr_t)p; }

// 16 bytes per lane from the buffer straight into LDS at m0 + 16 lane, and 4 bytes per lane
// at m0 + 4 lane (M0 holds the LDS address). Written as inline assembly on purpose: the
// compiler's memory model, seeing an LDS write whose completion it cannot order, would wait
// for every such load in flight before each LDS read and each barrier, which serialises a
// load pipeline. Completion is tracked with explicit vmcnt waits instead (vmcnt_wait), and
// the "memory" clobber keeps the compiler from moving LDS accesses across the issue. M0 is an
// operand ("{m0}"), so the compiler itself writes it and knows it is changed; the s_nop
// covers the wait state between an M0 write and an LDS-DMA load.
__device__ __forceinline__ void lds_dma16(i32x4 rsrc, uint32_t lds, int voff) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :: "v"(voff), "s"(rsrc), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void lds_dma4(i32x4 rsrc, uint32_t lds, int voff) {
    asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
                 :: "v"(voff), "s"(rsrc), "{m0}"(lds) : "memory");
}

// Wait until at most N of this wave's vector-memory operations are in flight (they complete
// in issue order for this count); also a compiler barrier for memory accesses, so LDS reads
// and writes of landed data stay behind it.
template <int N>
__device__ __forceinline__ void vmcnt_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Wait until at most n * PER loads are in flight, for a wave-uniform n in 0..MAXN
// (s_waitcnt takes an immediate).
template <int PER, int MAXN>
__device__ __forceinline__ void vmcnt_wait_groups(int n) {
    if constexpr (MAXN > 0) {
        if (n >= MAXN) {
            vmcnt_wait<PER * MAXN>();
            return;
        }
        vmcnt_wait_groups<PER, MAXN - 1>(n);
    } else {
        vmcnt_wait<0>();
    }
}

// Workgroup barrier that waits for this wave's LDS operations only, not for its loads
// (__syncthreads would also drain every direct-to-LDS load in flight).
__device__ __forceinline__ void lds_sync() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace sa
