// gfx950 device primitives shared by the matrix-core kernels: fragment types, the
// bf16 matrix instruction, LDS reads (plain and transposed), the LDS-only barrier, raw
// buffer descriptors and asynchronous global->LDS copies, and wait counters.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace retn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16(u16x8_t a, u16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ u16x8_t lds16(const char* base, int byte_off) {
    return *reinterpret_cast<const u16x8_t*>(base + byte_off);
}
__device__ __forceinline__ u16x4_t lds8(const char* base, int byte_off) {
    return *reinterpret_cast<const u16x4_t*>(base + byte_off);
}
__device__ __forceinline__ u16x8_t cat(u16x4_t a, u16x4_t b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ uint16_t bf(float x) { return f32_to_bf16(x); }
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
// four floats -> four bf16 (round to nearest even), two per v_cvt_pk_bf16_f32
__device__ __forceinline__ u16x4_t bf4(f32x4_t x) {
    return __builtin_bit_cast(u16x4_t, __builtin_convertvector(x, bf16x4_t));
}

// Raw hardware 2^x (v_exp_f32).  Every argument here is <= 0 or a masked lane, and
// results below the fp32 normal range may flush to zero, which is harmless for decays.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) char lds_char_t;

// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes, result lane
// i, element j is the (i%4)-th 16-bit value at the address given by lane 4j + i/4.
// So if lane 4j+q of a group points at row t_j, columns c0+4q..c0+4q+3 of a row-major
// tile, lane i receives that tile's column c0+i at rows t_0..t_3.
__device__ __forceinline__ u16x4_t lds_tr(const char* base, int byte_off) {
    const i16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)((lds_char_t*)(base) + byte_off));
    return __builtin_bit_cast(u16x4_t, r);
}

// Reads at an absolute LDS byte address (the compiler folds constant additions into
// the instruction's offset field).
typedef __attribute__((address_space(3))) u16x8_t lds_u16x8_t;
__device__ __forceinline__ u16x8_t lds16a(uint32_t addr) { return *(const lds_u16x8_t*)(static_cast<size_t>(addr)); }
__device__ __forceinline__ u16x4_t lds_tra(uint32_t addr) {
    return __builtin_bit_cast(u16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(static_cast<size_t>(addr))));
}
// Hides how a value was computed, so the compiler keeps it in one register instead of
// re-deriving it from its parts at every use.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS operations, then
// s_barrier.  (__syncthreads() also waits for outstanding global loads, which would
// stall on the asynchronous prefetch of the next block.)  The memory clobber keeps the
// compiler from moving memory operations across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Raw buffer resource (V#) over [base, base + bytes): 48-bit base, stride 0,
// num_records = bytes, word 3 as for gfx9 raw buffers.  A lane whose offset
// (voffset + soffset) is at or past `bytes` reads zeros instead of memory; a load into
// LDS then writes those zeros.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    // every word is wave-uniform; readfirstlane keeps the descriptor in SGPRs
    return u32x4_t{static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(a))),
                   static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>((a >> 32) & 0xFFFFu))),
                   static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(bytes))), 0x00020000u};
}

// Asynchronous 16-byte-per-lane copy global -> LDS (buffer_load_dwordx4 ... lds): lane
// l reads rsrc + soffset + voffset and its 16 bytes land at LDS byte lds_addr + 16 l
// (lds_addr and soffset are wave-uniform).  The instruction writes no registers; it is
// issued from inline assembly so that the compiler does not treat it as aliasing every
// later LDS read.  The LDS address goes in through an input operand bound to m0, so the
// compiler itself sets m0 and knows it holds that value.  Completion is awaited
// explicitly (s_waitcnt vmcnt(0) followed by a workgroup barrier) before the tile is read.
__device__ __forceinline__ void buf2lds16(const u32x4_t& rsrc, uint32_t voffset, uint32_t soffset,
                                          uint32_t lds_addr) {
    // the scalar operands are wave-uniform; readfirstlane pins them to SGPRs
    const uint32_t m0v = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(lds_addr)));
    const uint32_t soff = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(soffset)));
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voffset), "s"(rsrc), "s"(soff), "{m0}"(m0v)
                 : "memory");
}
// Same for 4 bytes per lane: lane l's dword lands at LDS byte lds_addr + 4 l.
__device__ __forceinline__ void buf2lds4(const u32x4_t& rsrc, uint32_t voffset, uint32_t soffset,
                                         uint32_t lds_addr) {
    const uint32_t m0v = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(lds_addr)));
    const uint32_t soff = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(soffset)));
    asm volatile("buffer_load_dword %0, %1, %2 offen lds"
                 :
                 : "v"(voffset), "s"(rsrc), "s"(soff), "{m0}"(m0v)
                 : "memory");
}
// Wait until at most N vector memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr_of(const char* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char_t*)(p)));
}

}  // namespace
}  // namespace retn
