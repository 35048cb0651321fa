// Bandwidth kernels around the backward pass's forward passes: sums and conversions of
// token rows (with the gate gradient's row dot products folded in), transposed state
// copies, and the gate gradient's reversed cumulative sum per (b,h).
//
// The backward itself is the chain rule applied to the recurrence S_n = lam_n S_{n-1} +
// k_n^T v_n, o_n = q_n S_n ("RetNet retention mechanism" tutorial, section 递归推理); the
// pages name a backward recurrence for the chunked kernels ("unilm RetNet 技术指南", section
// Triton 内核与自校验测试) without printing it.  How its pieces become forward passes is
// described in backward.cpp.

#include "common.h"
#include "launch.h"

namespace retn {
namespace {

constexpr int kThreads = 256;
constexpr int kScanThreads = 1024;

unsigned grid_for(size_t work, size_t per_block) {
    const size_t g = (work + per_block - 1) / per_block;
    return static_cast<unsigned>(std::min<size_t>(std::max<size_t>(g, 1), 1u << 20));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Eight adjacent elements as fp32 (16-byte aligned addresses).
template <typename T> struct vec8;
template <> struct vec8<float> {
    __device__ __forceinline__ static void load(const float* p, float (&x)[8]) {
        const f32v4 a = *reinterpret_cast<const f32v4*>(p), b = *reinterpret_cast<const f32v4*>(p + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
    __device__ __forceinline__ static void store(float* p, const float (&x)[8]) {
        *reinterpret_cast<f32v4*>(p) = f32v4{x[0], x[1], x[2], x[3]};
        *reinterpret_cast<f32v4*>(p + 4) = f32v4{x[4], x[5], x[6], x[7]};
    }
};
template <> struct vec8<bf16_t> {
    __device__ __forceinline__ static void load(const bf16_t* p, float (&x)[8]) {
        const uint4 u = *reinterpret_cast<const uint4*>(p);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(w[i] << 16);
            x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    }
    __device__ __forceinline__ static void store(bf16_t* p, const float (&x)[8]) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = static_cast<uint32_t>(f32_to_bf16(x[2 * i])) | (static_cast<uint32_t>(f32_to_bf16(x[2 * i + 1])) << 16);
        *reinterpret_cast<uint4*>(p) = uint4{w[0], w[1], w[2], w[3]};
    }
};

// out[e] = a[e] (+ b[e]) over n elements, converted from Tin to Tout; VEC: eight per
// thread (n a multiple of 8, pointers 16-byte aligned).  out may alias a or b.
template <typename Tin, typename Tout, bool VEC>
__global__ __launch_bounds__(kThreads) void combine_kernel(const Tin* a, const Tin* b, Tout* out, size_t n) {
    const size_t stride = static_cast<size_t>(gridDim.x) * kThreads;
    if constexpr (VEC) {
        for (size_t e = (blockIdx.x * static_cast<size_t>(kThreads) + threadIdx.x) * 8; e < n; e += stride * 8) {
            float x[8];
            vec8<Tin>::load(a + e, x);
            if (b != nullptr) {
                float y[8];
                vec8<Tin>::load(b + e, y);
#pragma unroll
                for (int i = 0; i < 8; ++i) x[i] += y[i];
            }
            vec8<Tout>::store(out + e, x);
        }
    } else {
        for (size_t e = blockIdx.x * static_cast<size_t>(kThreads) + threadIdx.x; e < n; e += stride) {
            float x = io<Tin>::load(a + e);
            if (b != nullptr) x += io<Tin>::load(b + e);
            io<Tout>::store(out + e, x);
        }
    }
}

// Gate gradient rows, folded into the conversion of an fp32 gradient g (+ g2) to bf16:
// out[row] = g[row] (+ g2[row]); dG[row] = (dG[row] if accumulate) + sign * (x[row] .
// the fp32 sum).  A row of w elements (w/8 a power of two, w <= 512) is spread over w/8
// adjacent lanes, eight elements each; the lanes of a row share its loop trips.
__global__ __launch_bounds__(kThreads) void convert_dot_kernel(const float* __restrict__ g, const float* __restrict__ g2,
                                                             const bf16_t* __restrict__ x, bf16_t* __restrict__ out,
                                                             float* __restrict__ dG, size_t rows, int w, float sign,
                                                             int accumulate) {
    const int lpr = w / 8;                                // lanes per row
    const int rows_per_block = kThreads / lpr;
    const int sub = threadIdx.x % lpr;
    for (size_t row = blockIdx.x * static_cast<size_t>(rows_per_block) + threadIdx.x / lpr; row < rows;
         row += static_cast<size_t>(gridDim.x) * rows_per_block) {
        const size_t e = row * w + static_cast<size_t>(sub) * 8;
        float v[8], xv[8];
        vec8<float>::load(g + e, v);
        if (g2 != nullptr) {
            float y[8];
            vec8<float>::load(g2 + e, y);
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] += y[i];
        }
        vec8<bf16_t>::load(x + e, xv);
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) d += xv[i] * v[i];
        vec8<bf16_t>::store(out + e, v);
        for (int off = lpr / 2; off >= 1; off >>= 1) d += __shfl_xor(d, off, 64);
        if (sub == 0) dG[row] = (accumulate ? dG[row] : 0.f) + sign * d;
    }
}

// dst[p][bh][r][c] = src[bh][c][p*w + r]: the transposed state, split into `parts` row
// blocks of w = dv/parts rows, each block contiguous over (b,h).  32x32 tiles through LDS;
// blockIdx.z picks one of two (src, dst) pairs (a null src skips its half).
__global__ __launch_bounds__(kThreads) void state_transpose_kernel(const float* __restrict__ src0, float* __restrict__ dst0,
                                                                 const float* __restrict__ src1, float* __restrict__ dst1,
                                                                 int dk, int dv, int parts, size_t bh_total) {
    __shared__ float tile[32][33];
    const float* const src = blockIdx.z == 0 ? src0 : src1;
    float* const dst = blockIdx.z == 0 ? dst0 : dst1;
    if (src == nullptr) return;   // uniform over the workgroup
    const int tiles_j = (dv + 31) / 32;
    const int tj = blockIdx.x % tiles_j, tc = blockIdx.x / tiles_j;
    const int w = dv / parts;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8
    for (size_t bh = blockIdx.y; bh < bh_total; bh += gridDim.y) {   // block-uniform loop
        for (int y = ty; y < 32; y += 8) {
            const int c = tc * 32 + y, j = tj * 32 + tx;
            if (c < dk && j < dv) tile[y][tx] = src[(bh * dk + c) * dv + j];
        }
        __syncthreads();
        for (int y = ty; y < 32; y += 8) {
            const int j = tj * 32 + y, c = tc * 32 + tx;
            if (c < dk && j < dv) {
                const int p = j / w, r = j - p * w;
                dst[((static_cast<size_t>(p) * bh_total + bh) * w + r) * dk + c] = tile[tx][y];
            }
        }
        __syncthreads();
    }
}

// The same transpose in 64x64 tiles moved as 16-byte vectors (dk and dv multiples of 4,
// so that every vector stays inside one row and is aligned): thread t loads 4-float
// pieces of rows t/16 + 16i and stores 4-float pieces of output rows t/16 + 16i.  The
// LDS tile has a row stride of 65 floats, so both the row writes and the column reads
// of a wave fall in 64 distinct banks.
__global__ __launch_bounds__(kThreads) void state_transpose4_kernel(const float* __restrict__ src0,
                                                                  float* __restrict__ dst0,
                                                                  const float* __restrict__ src1,
                                                                  float* __restrict__ dst1, int dk, int dv, int parts,
                                                                  size_t bh_total) {
    __shared__ float tile[64 * 65];
    const float* const src = blockIdx.z == 0 ? src0 : src1;
    float* const dst = blockIdx.z == 0 ? dst0 : dst1;
    if (src == nullptr) return;   // uniform over the workgroup
    const int tiles_j = (dv + 63) / 64;
    const int tj = blockIdx.x % tiles_j, tc = blockIdx.x / tiles_j;
    const int w = dv / parts;
    const int u = threadIdx.x & 15, y0 = threadIdx.x >> 4;   // 16 x 16
    for (size_t bh = blockIdx.y; bh < bh_total; bh += gridDim.y) {   // block-uniform loop
        const float* const sb = src + bh * dk * dv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int y = y0 + 16 * i, c = tc * 64 + y, j = tj * 64 + 4 * u;
            float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
            if (c < dk && j < dv) x = *reinterpret_cast<const float4*>(sb + static_cast<size_t>(c) * dv + j);
            float* const t = tile + y * 65 + 4 * u;
            t[0] = x.x;
            t[1] = x.y;
            t[2] = x.z;
            t[3] = x.w;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int y = y0 + 16 * i, j = tj * 64 + y, c = tc * 64 + 4 * u;
            if (c < dk && j < dv) {
                const float* const t = tile + (4 * u) * 65 + y;
                const float4 x = make_float4(t[0], t[65], t[130], t[195]);
                const int p = j / w, r = j - p * w;
                *reinterpret_cast<float4*>(dst + ((static_cast<size_t>(p) * bh_total + bh) * w + r) * dk + c) = x;
            }
        }
        __syncthreads();
    }
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// dG[bh][n] = q_n . dq_n - k_n . dk_n: one wave per token, lanes over the row (the
// gradients in the I/O type; the matrix-core path folds this into convert_dot_kernel).
template <typename T>
__global__ __launch_bounds__(kThreads) void gate_rows_kernel(const T* __restrict__ q, const T* __restrict__ dq,
                                                           const T* __restrict__ k, const T* __restrict__ dkk,
                                                           float* __restrict__ dG, size_t rows_total, int dk) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (size_t row = blockIdx.x * static_cast<size_t>(kThreads / 64) + wave; row < rows_total;
         row += static_cast<size_t>(gridDim.x) * (kThreads / 64)) {
        const size_t base = row * dk;
        float acc = 0.f;
        for (int i = lane; i < dk; i += 64)
            acc += io<T>::load(q + base + i) * io<T>::load(dq + base + i) -
                   io<T>::load(k + base + i) * io<T>::load(dkk + base + i);
        acc = wave_sum(acc);
        if (lane == 0) dG[row] = acc;
    }
}

// dg[bh][n] = sum_{p >= n} dG[bh][p] + c[bh] with c[bh] = <A[bh], B[bh]> for two states in
// the slice layout of state_transpose (0 when A is null).  One workgroup per (b,h): the
// threads first sum the dk*dv products (contiguous within each slice block), then each
// sums a contiguous run of tokens; suffix sums of the run totals (within each wave by
// shuffles, then over the waves after it) give every run its starting value.  With few
// workgroups the kernel is bound by memory latency, so every thread issues its loads
// together: the products four 16-byte pairs at a time, and runs of up to kScanRun tokens
// held in registers.
constexpr int kScanRun = 16;

__global__ __launch_bounds__(kScanThreads) void gate_scan_kernel(const float* __restrict__ dG,
                                                               const float* __restrict__ A,
                                                               const float* __restrict__ B, int dk, int dv,
                                                               int parts, size_t bh_total,
                                                               float* __restrict__ dg, int N) {
    __shared__ float wsum[kScanThreads / 64];
    __shared__ float cval;
    const size_t bh = blockIdx.x;
    const float* src = dG + bh * N;
    float* dst = dg + bh * N;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (A != nullptr) {
        const int per_block = dv / parts * dk;
        const bool vec = per_block % 4 == 0 && ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B)) & 15u) == 0;
        float acc = 0.f;
        for (int p = 0; p < parts; ++p) {
            const size_t base = (static_cast<size_t>(p) * bh_total + bh) * per_block;
            if (vec) {
                const float4* a4 = reinterpret_cast<const float4*>(A + base);
                const float4* b4 = reinterpret_cast<const float4*>(B + base);
#pragma unroll 4
                for (int e = tid; e < per_block / 4; e += kScanThreads) {
                    const float4 x = a4[e], y = b4[e];
                    acc += x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
                }
            } else {
                for (int e = tid; e < per_block; e += kScanThreads) acc += A[base + e] * B[base + e];
            }
        }
        acc = wave_sum(acc);
        if (lane == 0) wsum[wave] = acc;
        __syncthreads();
        if (tid == 0) {
            float c = 0.f;
            for (int i = 0; i < kScanThreads / 64; ++i) c += wsum[i];
            cval = c;
        }
        __syncthreads();   // wsum is reused below
    } else if (tid == 0) {
        cval = 0.f;
    }
    const int per = (N + kScanThreads - 1) / kScanThreads;   // uniform
    const int n0 = min(N, tid * per), n1 = min(N, n0 + per);
    const bool regs = per <= kScanRun;
    float val[kScanRun];
    float s = 0.f;
    if (regs) {
#pragma unroll
        for (int i = 0; i < kScanRun; ++i) val[i] = n0 + i < n1 ? src[n0 + i] : 0.f;
#pragma unroll
        for (int i = 0; i < kScanRun; ++i) s += val[i];
    } else {
        for (int n = n0; n < n1; ++n) s += src[n];
    }
    float incl = s;   // sum over lanes lane..63 of this wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_down(incl, off, 64);
        if (lane + off < 64) incl += y;
    }
    if (lane == 0) wsum[wave] = incl;
    __syncthreads();
    float run = cval;
    for (int w2 = kScanThreads / 64 - 1; w2 > wave; --w2) run += wsum[w2];
    run += incl - s;   // the lanes after this one
    if (regs) {
#pragma unroll
        for (int i = kScanRun - 1; i >= 0; --i) {
            if (n0 + i < n1) {
                run += val[i];
                dst[n0 + i] = run;
            }
        }
    } else {
        for (int n = n1 - 1; n >= n0; --n) {
            run += src[n];
            dst[n] = run;
        }
    }
}

template <typename Tin, typename Tout>
void combine_typed(const void* a, const void* b, void* out, size_t n, hipStream_t s) {
    const Tin *pa = static_cast<const Tin*>(a), *pb = static_cast<const Tin*>(b);
    Tout* po = static_cast<Tout*>(out);
    const bool vec = n % 8 == 0 && aligned16(a) && (b == nullptr || aligned16(b)) && aligned16(out);
    if (vec)
        hipLaunchKernelGGL((combine_kernel<Tin, Tout, true>), dim3(grid_for(n / 8, kThreads)), dim3(kThreads), 0, s,
                           pa, pb, po, n);
    else
        hipLaunchKernelGGL((combine_kernel<Tin, Tout, false>), dim3(grid_for(n, kThreads)), dim3(kThreads), 0, s, pa,
                           pb, po, n);
}

}  // namespace

// in_f32 / out_f32: element types of (a, b) and of out (else the I/O type: bf16 or fp32).
hipError_t launch_rows_combine(const void* a, const void* b, void* out, size_t bh, int N, int w, bool bf16,
                               hipStream_t s, bool in_f32, bool out_f32) {
    const size_t n = bh * static_cast<size_t>(N) * w;
    if (n == 0) return hipSuccess;
    const bool fin = in_f32 || !bf16, fout = out_f32 || !bf16;
    if (fin && fout) combine_typed<float, float>(a, b, out, n, s);
    else if (fin) combine_typed<float, bf16_t>(a, b, out, n, s);
    else if (fout) combine_typed<bf16_t, float>(a, b, out, n, s);
    else combine_typed<bf16_t, bf16_t>(a, b, out, n, s);
    return hipGetLastError();
}

bool convert_dot_supported(int w, const void* g, const void* g2, const void* x, const void* out) {
    if (w % 8 != 0 || w > 512 || ((w / 8) & (w / 8 - 1)) != 0) return false;
    return aligned16(g) && (g2 == nullptr || aligned16(g2)) && aligned16(x) && aligned16(out);
}

hipError_t launch_convert_dot(const float* g, const float* g2, const void* x, void* out, float* dG, size_t bh, int N,
                              int w, float sign, bool accumulate, hipStream_t s) {
    const size_t rows = bh * static_cast<size_t>(N);
    if (rows == 0) return hipSuccess;
    const int rows_per_block = kThreads / (w / 8);
    hipLaunchKernelGGL(convert_dot_kernel, dim3(grid_for(rows, rows_per_block)), dim3(kThreads), 0, s, g, g2,
                       static_cast<const bf16_t*>(x), static_cast<bf16_t*>(out), dG, rows, w, sign,
                       accumulate ? 1 : 0);
    return hipGetLastError();
}

// Transposes src0 -> dst0 and src1 -> dst1 in one launch (either src may be null).
hipError_t launch_state_transpose(const float* src0, float* dst0, const float* src1, float* dst1, size_t bh, int dk,
                                  int dv, int parts, hipStream_t s) {
    if (bh == 0 || (src0 == nullptr && src1 == nullptr)) return hipSuccess;
    const unsigned ys = static_cast<unsigned>(std::min<size_t>(bh, 65535));
    const bool vec = dk % 4 == 0 && dv % 4 == 0 && (src0 == nullptr || (aligned16(src0) && aligned16(dst0))) &&
                     (src1 == nullptr || (aligned16(src1) && aligned16(dst1)));
    if (vec) {
        const unsigned tiles4 = static_cast<unsigned>(((dk + 63) / 64) * ((dv + 63) / 64));
        hipLaunchKernelGGL(state_transpose4_kernel, dim3(tiles4, ys, 2), dim3(kThreads), 0, s, src0, dst0, src1, dst1,
                           dk, dv, parts, bh);
        return hipGetLastError();
    }
    const unsigned tiles = static_cast<unsigned>(((dk + 31) / 32) * ((dv + 31) / 32));
    hipLaunchKernelGGL(state_transpose_kernel, dim3(tiles, ys, 2), dim3(kThreads), 0, s, src0, dst0, src1, dst1, dk, dv,
                       parts, bh);
    return hipGetLastError();
}

hipError_t launch_gate_rows(const void* q, const void* dq, const void* k, const void* dkk, float* dG, size_t bh,
                            int N, int dk, bool bf16, hipStream_t s) {
    const size_t rows = bh * static_cast<size_t>(N);
    if (rows == 0) return hipSuccess;
    const unsigned g1 = grid_for(rows, kThreads / 64);
    if (bf16)
        hipLaunchKernelGGL((gate_rows_kernel<bf16_t>), dim3(g1), dim3(kThreads), 0, s, static_cast<const bf16_t*>(q),
                           static_cast<const bf16_t*>(dq), static_cast<const bf16_t*>(k),
                           static_cast<const bf16_t*>(dkk), dG, rows, dk);
    else
        hipLaunchKernelGGL((gate_rows_kernel<float>), dim3(g1), dim3(kThreads), 0, s, static_cast<const float*>(q),
                           static_cast<const float*>(dq), static_cast<const float*>(k), static_cast<const float*>(dkk),
                           dG, rows, dk);
    return hipGetLastError();
}

// A, B: the two states of <dS, S_N> in slice layout (A null: no such term).
hipError_t launch_gate_scan(const float* dG, const float* A, const float* B, int dk, int dv, int parts, float* dg,
                            size_t bh, int N, hipStream_t s) {
    if (bh == 0 || N == 0) return hipSuccess;
    hipLaunchKernelGGL(gate_scan_kernel, dim3(static_cast<unsigned>(bh)), dim3(kScanThreads), 0, s, dG, A, B, dk, dv,
                       parts, bh, dg, N);
    return hipGetLastError();
}

}  // namespace retn
