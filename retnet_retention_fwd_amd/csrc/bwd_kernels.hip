// Bandwidth kernels around the backward pass's forward passes: time reversal and sums of
// token rows, transposed and scaled state copies, the shifted reversed gate, and the
// gate gradient (row dot products, then a reversed cumulative sum per (b,h)).
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

unsigned grid_for(size_t work, size_t per_block) {
    const size_t g = (work + per_block - 1) / per_block;
    return static_cast<unsigned>(std::min<size_t>(std::max<size_t>(g, 1), 1u << 20));
}

// out[bh, n, :] = a[bh, s(n), :] (+ b[bh, s(n), :]) with s(n) = N-1-n when flipping,
// converted from Tin to Tout.  Each thread moves V adjacent elements of one row (V
// divides the row width).
template <typename Tin, typename Tout, int V>
__global__ __launch_bounds__(kThreads) void rows_combine_kernel(const Tin* __restrict__ a, const Tin* __restrict__ b,
                                                              Tout* __restrict__ out, size_t rows_total, int N, int w,
                                                              int flip) {
    const int units = w / V;
    const size_t total = rows_total * units;
    for (size_t e = blockIdx.x * static_cast<size_t>(kThreads) + threadIdx.x; e < total;
         e += static_cast<size_t>(gridDim.x) * kThreads) {
        const size_t row = e / units;
        const int u = static_cast<int>(e - row * units);
        const size_t bh = row / N;
        const int n = static_cast<int>(row - bh * N);
        const size_t src = (bh * N + (flip ? N - 1 - n : n)) * static_cast<size_t>(w) + static_cast<size_t>(u) * V;
        const size_t dst = row * static_cast<size_t>(w) + static_cast<size_t>(u) * V;
        float x[V];
#pragma unroll
        for (int i = 0; i < V; ++i) x[i] = io<Tin>::load(a + src + i);
        if (b != nullptr) {
#pragma unroll
            for (int i = 0; i < V; ++i) x[i] += io<Tin>::load(b + src + i);
        }
#pragma unroll
        for (int i = 0; i < V; ++i) io<Tout>::store(out + dst + i, x[i]);
    }
}

// dst[p][bh][r][c] = src[bh][c][p*w + r] * f(bh): the transposed state, split into
// `parts` row blocks of w = dv/parts rows, each block contiguous over (b,h).
// f = 1/gamma[h] when inv is set and gamma given, else 1.  32x32 tiles through LDS.
__global__ __launch_bounds__(kThreads) void state_transpose_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                                 int dk, int dv, int parts, size_t bh_total,
                                                                 const float* __restrict__ gamma, int H) {
    __shared__ float tile[32][33];
    const int tiles_j = (dv + 31) / 32;
    const int tj = blockIdx.x % tiles_j, tc = blockIdx.x / tiles_j;
    const int w = dv / parts;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8
    for (size_t bh = blockIdx.y; bh < bh_total; bh += gridDim.y) {   // block-uniform loop
        const float f = gamma != nullptr ? 1.f / gamma[bh % H] : 1.f;
        for (int y = ty; y < 32; y += 8) {
            const int c = tc * 32 + y, j = tj * 32 + tx;
            if (c < dk && j < dv) tile[y][tx] = src[(bh * dk + c) * dv + j] * f;
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

// dst[bh] = src[bh] * f(bh), f = gamma[h] (mode 0), 1/gamma[h] (mode 1) or exp(g[bh, 0])
// (mode 2).  In place allowed.
__global__ __launch_bounds__(kThreads) void state_scale_kernel(const float* __restrict__ src, float* dst,
                                                             size_t per_bh, size_t bh_total,
                                                             const float* __restrict__ decay, int H, int N,
                                                             int mode) {
    const size_t total = per_bh * bh_total;
    for (size_t e = blockIdx.x * static_cast<size_t>(kThreads) + threadIdx.x; e < total;
         e += static_cast<size_t>(gridDim.x) * kThreads) {
        const size_t bh = e / per_bh;
        const float f = mode == 0 ? decay[bh % H] : mode == 1 ? 1.f / decay[bh % H] : expf(decay[bh * N]);
        dst[e] = src[e] * f;
    }
}

// gr[bh][0] = 0, gr[bh][m] = g[bh][N - m] for m >= 1: the gate of the time-reversed
// adjoint recurrence (U_n = q_n^T dO_n + exp(g_{n+1}) U_{n+1}).
__global__ __launch_bounds__(kThreads) void reverse_gate_kernel(const float* __restrict__ g, float* __restrict__ gr,
                                                              size_t bh_total, int N) {
    const size_t total = bh_total * N;
    for (size_t e = blockIdx.x * static_cast<size_t>(kThreads) + threadIdx.x; e < total;
         e += static_cast<size_t>(gridDim.x) * kThreads) {
        const size_t bh = e / N;
        const int m = static_cast<int>(e - bh * N);
        gr[e] = m == 0 ? 0.f : g[bh * N + (N - m)];
    }
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// c[bh] = <dS[bh], S_N[bh]>, S_N given transposed in part blocks (as state_transpose).
__global__ __launch_bounds__(kThreads) void state_dot_kernel(const float* __restrict__ dS,
                                                           const float* __restrict__ sfin_t, float* __restrict__ c,
                                                           int dk, int dv, int parts, size_t bh_total) {
    __shared__ float part_sums[kThreads / 64];
    const size_t bh = blockIdx.x;
    const int w = dv / parts;
    float acc = 0.f;
    for (int e = threadIdx.x; e < dk * dv; e += kThreads) {
        const int i = e / dv, j = e - i * dv;
        const int p = j / w, r = j - p * w;
        acc += dS[bh * dk * dv + e] * sfin_t[((static_cast<size_t>(p) * bh_total + bh) * w + r) * dk + i];
    }
    acc = wave_sum(acc);
    if ((threadIdx.x & 63) == 0) part_sums[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.f;
        for (int i = 0; i < kThreads / 64; ++i) t += part_sums[i];
        c[bh] = t;
    }
}

// dG[bh][n] = q_n . dq_n - k_n . dk_n: one wave per token, lanes over the row.  q, k
// are Tx; dq, dk are Tg; dk may be stored time-reversed (row N-1-n).
template <typename Tx, typename Tg>
__global__ __launch_bounds__(kThreads) void gate_rows_kernel(const Tx* __restrict__ q, const Tg* __restrict__ dq,
                                                           const Tx* __restrict__ k, const Tg* __restrict__ dkk,
                                                           float* __restrict__ dG, size_t rows_total, int N, int dk,
                                                           int flip_dk) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (size_t row = blockIdx.x * static_cast<size_t>(kThreads / 64) + wave; row < rows_total;
         row += static_cast<size_t>(gridDim.x) * (kThreads / 64)) {
        const size_t base = row * dk;
        const size_t bh = row / N;
        const int n = static_cast<int>(row - bh * N);
        const size_t kbase = flip_dk ? (bh * N + (N - 1 - n)) * dk : base;
        float acc = 0.f;
        for (int i = lane; i < dk; i += 64)
            acc += io<Tx>::load(q + base + i) * io<Tg>::load(dq + base + i) -
                   io<Tx>::load(k + base + i) * io<Tg>::load(dkk + kbase + i);
        acc = wave_sum(acc);
        if (lane == 0) dG[row] = acc;
    }
}

// dg[bh][n] = sum_{p >= n} dG[bh][p] + c[bh] (c = 0 when absent): one workgroup per
// (b,h); each thread sums a contiguous run of tokens, the run totals are scanned in
// LDS, then every thread writes its run.
__global__ __launch_bounds__(kThreads) void gate_scan_kernel(const float* __restrict__ dG, const float* __restrict__ c,
                                                           float* __restrict__ dg, int N) {
    __shared__ float tot[kThreads];
    const size_t bh = blockIdx.x;
    const float* src = dG + bh * N;
    float* dst = dg + bh * N;
    const int per = (N + kThreads - 1) / kThreads;
    const int n0 = threadIdx.x * per, n1 = min(N, n0 + per);
    float s = 0.f;
    for (int n = n0; n < n1; ++n) s += src[n];
    tot[threadIdx.x] = s;
    __syncthreads();
    if (threadIdx.x == 0) {   // exclusive suffix sums of the run totals
        float run = c != nullptr ? c[bh] : 0.f;
        for (int t = kThreads - 1; t >= 0; --t) {
            const float x = tot[t];
            tot[t] = run;
            run += x;
        }
    }
    __syncthreads();
    float run = tot[threadIdx.x];
    for (int n = n1 - 1; n >= n0; --n) {
        run += src[n];
        dst[n] = run;
    }
}

template <typename Tin, typename Tout>
void combine_typed(const void* a, const void* b, void* out, size_t rows, int N, int w, bool flip, hipStream_t s) {
    const Tin *pa = static_cast<const Tin*>(a), *pb = static_cast<const Tin*>(b);
    Tout* po = static_cast<Tout*>(out);
    if (w % 4 == 0)
        hipLaunchKernelGGL((rows_combine_kernel<Tin, Tout, 4>), dim3(grid_for(rows * (w / 4), kThreads)),
                           dim3(kThreads), 0, s, pa, pb, po, rows, N, w, flip ? 1 : 0);
    else
        hipLaunchKernelGGL((rows_combine_kernel<Tin, Tout, 1>), dim3(grid_for(rows * w, kThreads)), dim3(kThreads), 0,
                           s, pa, pb, po, rows, N, w, flip ? 1 : 0);
}

}  // namespace

// in_f32 / out_f32: element types of (a, b) and of out (else the I/O type: bf16 or fp32).
hipError_t launch_rows_combine(const void* a, const void* b, void* out, size_t bh, int N, int w, bool bf16,
                               bool flip, hipStream_t s, bool in_f32, bool out_f32) {
    const size_t rows = bh * static_cast<size_t>(N);
    if (rows == 0 || w == 0) return hipSuccess;
    const bool fin = in_f32 || !bf16, fout = out_f32 || !bf16;
    if (fin && fout) combine_typed<float, float>(a, b, out, rows, N, w, flip, s);
    else if (fin) combine_typed<float, bf16_t>(a, b, out, rows, N, w, flip, s);
    else if (fout) combine_typed<bf16_t, float>(a, b, out, rows, N, w, flip, s);
    else combine_typed<bf16_t, bf16_t>(a, b, out, rows, N, w, flip, s);
    return hipGetLastError();
}

hipError_t launch_state_transpose(const float* src, float* dst, size_t bh, int dk, int dv, int parts,
                                  const float* inv_gamma, int H, hipStream_t s) {
    if (bh == 0) return hipSuccess;
    const unsigned tiles = static_cast<unsigned>(((dk + 31) / 32) * ((dv + 31) / 32));
    const unsigned ys = static_cast<unsigned>(std::min<size_t>(bh, 65535));
    hipLaunchKernelGGL(state_transpose_kernel, dim3(tiles, ys), dim3(kThreads), 0, s, src, dst, dk, dv, parts, bh,
                       inv_gamma, H);
    return hipGetLastError();
}

hipError_t launch_state_scale(const float* src, float* dst, size_t bh, size_t per_bh, const float* decay, int H,
                              int N, int mode, hipStream_t s) {
    if (bh == 0 || per_bh == 0) return hipSuccess;
    hipLaunchKernelGGL(state_scale_kernel, dim3(grid_for(bh * per_bh, kThreads)), dim3(kThreads), 0, s, src, dst,
                       per_bh, bh, decay, H, N, mode);
    return hipGetLastError();
}

hipError_t launch_reverse_gate(const float* g, float* gr, size_t bh, int N, hipStream_t s) {
    if (bh * N == 0) return hipSuccess;
    hipLaunchKernelGGL(reverse_gate_kernel, dim3(grid_for(bh * N, kThreads)), dim3(kThreads), 0, s, g, gr, bh, N);
    return hipGetLastError();
}

hipError_t launch_state_dot(const float* dS, const float* sfin_t, float* c, size_t bh, int dk, int dv, int parts,
                            hipStream_t s) {
    if (bh == 0) return hipSuccess;
    hipLaunchKernelGGL(state_dot_kernel, dim3(static_cast<unsigned>(bh)), dim3(kThreads), 0, s, dS, sfin_t, c, dk,
                       dv, parts, bh);
    return hipGetLastError();
}

// grads_f32: dq and dk are fp32 (else the I/O type); flip_dk: dk stored time-reversed.
hipError_t launch_gate_grad(const void* q, const void* dq, const void* k, const void* dkk, const float* c,
                            float* dG, float* dg, size_t bh, int N, int dk, bool bf16, bool grads_f32, bool flip_dk,
                            hipStream_t s) {
    const size_t rows = bh * static_cast<size_t>(N);
    if (rows == 0) return hipSuccess;
    const unsigned g1 = grid_for(rows, kThreads / 64);
    const int fl = flip_dk ? 1 : 0;
    if (bf16 && grads_f32)
        hipLaunchKernelGGL((gate_rows_kernel<bf16_t, float>), dim3(g1), dim3(kThreads), 0, s,
                           static_cast<const bf16_t*>(q), static_cast<const float*>(dq),
                           static_cast<const bf16_t*>(k), static_cast<const float*>(dkk), dG, rows, N, dk, fl);
    else if (bf16)
        hipLaunchKernelGGL((gate_rows_kernel<bf16_t, bf16_t>), dim3(g1), dim3(kThreads), 0, s,
                           static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(dq),
                           static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(dkk), dG, rows, N, dk, fl);
    else
        hipLaunchKernelGGL((gate_rows_kernel<float, float>), dim3(g1), dim3(kThreads), 0, s,
                           static_cast<const float*>(q), static_cast<const float*>(dq), static_cast<const float*>(k),
                           static_cast<const float*>(dkk), dG, rows, N, dk, fl);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gate_scan_kernel, dim3(static_cast<unsigned>(bh)), dim3(kThreads), 0, s, dG, c, dg, N);
    return hipGetLastError();
}

}  // namespace retn
