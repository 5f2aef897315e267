// lds_dma.h -- buffer-to-LDS loads and the waits around them, for gfx950.
//
// Shared by the kernels that stream operands into LDS rings: a raw buffer
// descriptor (its range check turns loads past the end into zeros), a
// 16-byte buffer-to-LDS load per lane, a wait on this wave's vector memory
// counter, and a workgroup barrier that does not drain that counter.
//
// Counting rule for wait_vm<N>(): vector memory loads complete in the order
// they were issued, stores need not. So, to wait for a load X, N is the
// number of loads issued after X (stores issued after X only make the wait
// stricter, never unsafe).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace svdma {

// A raw buffer descriptor over n bytes from p (n <= 2^31): loads at byte
// offsets from n on read zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, unsigned n) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}

// One 16-byte buffer-to-LDS load per lane: lane l's 16 bytes at byte offset
// off of r land at lds + 16 l (lds is the same for the whole wave). Buffer
// loads rather than global ones: with a global load to LDS in flight the
// compiler must assume it may also count as an LDS access and drains every
// LDS read before the next use of one.
// kAux is the instruction's cache policy (2: non-temporal, for data read
// once, so that it leaves the L2 before data that is read again).
template <int kAux = 0>
__device__ __forceinline__ void load16(__amdgpu_buffer_rsrc_t r, unsigned off, unsigned char* lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                             (int)off, 0, 0, kAux);
}

// Wait until at most N of this wave's vector memory operations are
// outstanding, leaving the other counters.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt is six bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// A workgroup barrier that waits for this wave's LDS reads but not for its
// vector memory operations: loads into LDS are ordered by wait_vm() before
// it, and later ones stay in flight across it (a __syncthreads() fence would
// drain them). The clobber keeps the compiler from moving memory operations
// across it.
__device__ __forceinline__ void ring_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace svdma
