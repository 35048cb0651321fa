// Achievable-peak reference for the benchmark: a loop of independent bf16 matrix-core
// instructions (v_mfma_f32_16x16x32_bf16) with no memory traffic, so the rate it reaches
// is what the matrix cores sustain at the clock the chip runs under that load.

#include "../../include/retention.h"

#include <hip/hip_runtime.h>

#include "cdna4.h"

namespace retn {
namespace {

constexpr int kChains = 16;   // independent accumulators per wave

__global__ __launch_bounds__(512) void mfma_loop_kernel(float* out, int iters) {
    const int lane = threadIdx.x & 63;
    const u16x8_t a = u16x8_t{static_cast<uint16_t>(0x3f80 + (lane & 7)), 0x3f80, 0x3f80, 0x3f80,
                              0x3f80, 0x3f80, 0x3f80, 0x3f80};
    f32x4_t c[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) c[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kChains; ++j) c[j] = mfma16(a, a, c[j]);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kChains; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
    // one value per wave keeps the products live
    if (lane == 0) out[blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)] = s;
}

}  // namespace
}  // namespace retn

extern "C" retn_status retention_calib_mfma(float* out, int blocks, int waves, int iters, void* stream) {
    if (out == nullptr) return RETN_ERR_NULL;
    if (blocks < 1 || waves < 1 || waves > 8 || iters < 1) return RETN_ERR_SHAPE;
    hipLaunchKernelGGL(retn::mfma_loop_kernel, dim3(blocks), dim3(waves * 64), 0, static_cast<hipStream_t>(stream),
                       out, iters);
    return hipGetLastError() == hipSuccess ? RETN_OK : RETN_ERR_HIP;
}

extern "C" double retention_calib_mfma_flops(int blocks, int waves, int iters) {
    return static_cast<double>(blocks) * waves * iters * retn::kChains * (2.0 * 16 * 16 * 32);
}
