// Internal helpers shared by the gfx950 kernels of the retention library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace retn {

// bf16 is carried as raw 16-bit patterns in memory; conversions are explicit.
typedef uint16_t bf16_t;

// Native 4 x fp32 vector (usable with the nontemporal load/store builtins).
typedef float f32v4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// Round-to-nearest-even float -> bf16 (the hardware conversion on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float x) {
    __bf16 b = static_cast<__bf16>(x);
    return __builtin_bit_cast(bf16_t, b);
}

template <typename T> struct io;
template <> struct io<float> {
    __device__ __forceinline__ static float load(const float* p) { return *p; }
    __device__ __forceinline__ static void store(float* p, float x) { *p = x; }
};
template <> struct io<bf16_t> {
    __device__ __forceinline__ static float load(const bf16_t* p) { return bf16_to_f32(*p); }
    __device__ __forceinline__ static void store(bf16_t* p, float x) { *p = f32_to_bf16(x); }
};

// log2(e): converts a natural-log decay into the base-2 exponent used with exp2f.
constexpr float kLog2e = 1.4426950408889634f;

}  // namespace retn
