// gfx950 device helpers shared by the kernels that move operands straight
// from global memory into LDS (buffer_load_dwordx4 ... lds).
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

#define LDS __attribute__((address_space(3)))

namespace libgemm {
namespace dma {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// voffset beyond any buffer size the kernels accept (sizes stay below
// 2^31 bytes): a load at this offset returns zeros.
constexpr uint32_t OOB = 0x80000000u;

// Values the compiler cannot prove wave-uniform (they come out of 64-bit
// divisions done on the vector ALU) are moved to scalar registers, so that
// buffer descriptors and M0 are built once per wave instead of in a loop
// over distinct lane values.
__device__ inline int64_t uniform(int64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(uint64_t(x) >> 32));
    return static_cast<int64_t>((uint64_t(hi) << 32) | lo);
}

// Raw buffer descriptor (stride 0, 32-bit format) over `bytes` bytes from
// `addr`; reads past the end return zero.  Both arguments must be
// wave-uniform.
__device__ inline u32x4 raw_buffer(uint64_t addr, uint32_t bytes) {
    u32x4 rs;
    rs[0] = static_cast<uint32_t>(addr);
    rs[1] = static_cast<uint32_t>(addr >> 32) & 0xffffu;
    rs[2] = bytes;
    rs[3] = 0x00020000u;
    return rs;
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ inline void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// s_waitcnt lgkmcnt(0) only: every LDS read of this wave has returned.
__device__ inline void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// buffer_load_dwordx4 ... lds: 16 bytes per lane from the buffer `rs` at
// byte offset `voffset` into LDS at `lds` + 16 * lane.  Issued as inline
// assembly on purpose: the compiler does not then treat the load as a
// pending LDS write, so it does not wait for every outstanding prefetch
// before each LDS read (the prefetches target other buffers).  Visibility is
// the caller's job: s_waitcnt vmcnt for the data being consumed, then a
// workgroup barrier.  A descriptor and LDS address that are not wave-uniform
// would be wrong here, so both are taken in scalar registers.
__device__ inline void direct_load16(u32x4 rs, uint32_t lds, uint32_t voffset) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds"
        :
        : "s"(lds), "v"(voffset), "s"(rs)
        : "memory", "m0");
}

// buffer_load_dword ... lds: 4 bytes per lane from the buffer `rs` at byte
// offset `voffset` into LDS at `lds` + 4 * lane (the same contract as
// direct_load16).
__device__ inline void direct_load4(u32x4 rs, uint32_t lds, uint32_t voffset) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "buffer_load_dword %1, %2, 0 offen lds"
        :
        : "s"(lds), "v"(voffset), "s"(rs)
        : "memory", "m0");
}

}  // namespace dma
}  // namespace libgemm
