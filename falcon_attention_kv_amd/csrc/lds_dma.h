// Device helpers shared by the LDS-tiled kernels for gfx950: vector types, buffer
// descriptors, the buffer-to-LDS DMA and counted vector-memory waits.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace unipin {
namespace {

#define LDS_AS __attribute__((address_space(3)))

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kBufferWord3 = 0x00020000u;   // gfx9 buffer descriptor, raw 32-bit access

// Buffer descriptor as four scalar words, for the DMA issued from inline assembly.
__device__ __forceinline__ i32x4 rsrc_words(const void *base, uint32_t bytes) {
    const uint64_t addr = reinterpret_cast<uint64_t>(base);
    return i32x4{(int)(uint32_t)addr, (int)((uint32_t)(addr >> 32) & 0xffffu), (int)bytes, (int)kBufferWord3};
}

// One 16-byte-per-lane buffer-to-LDS DMA: lane l writes LDS bytes [lds + 16 l, +16) from
// buffer offset voff + soff (zeros past the record count).  It is issued from inline
// assembly so that the compiler does not treat it as a pending write to every LDS
// address (which makes it wait for all outstanding DMA before each LDS read and defeats
// the prefetch); the kernels wait for it explicitly (vmcnt, then a workgroup barrier).
// The instruction has no register results and reads its operands at issue.  It takes
// its LDS address from M0, and a scalar write of M0 needs one wait state before an LDS
// DMA reads it; the compiler cannot see that hazard inside the assembly (it sets M0 in
// the instruction just before), so the s_nop is part of the statement.
__device__ __forceinline__ void dma16(uint32_t lds, i32x4 rsrc, int voff, int soff) {
    // the descriptor, the scalar offset and M0 are wave-uniform by construction
    soff = __builtin_amdgcn_readfirstlane(soff);
    lds = __builtin_amdgcn_readfirstlane(lds);
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff),
                 "{m0}"(lds)
                 : "memory");
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

}  // namespace
}  // namespace unipin
