// Generic chunkwise retention forward (fp32 arithmetic on the vector ALUs).
//
// Covers every in-range shape and both element types: it is the fp32 path, and the
// bf16 path for shapes the matrix-core kernel does not take.  For each chunk of L
// tokens it evaluates the chunkwise form ("RetNet retention mechanism" tutorial,
// section 块级循环, with the per-row cross-chunk decay):
//     O     = (Q K^T (.) D) V + diag(xi) (Q S_prev),  D_jl = lambda(l+1..j), xi_j = lambda(0..j)
//     S_new = lambda(0..L-1) S_prev + K^T (V (.) zeta),  zeta_l = lambda(l+1..L-1)
// where lambda(a..b) is the product of the per-token decays over chunk-local
// positions a..b: gamma^(b-a+1) per head, or exp of a sum of g when gated
// (pwwt.cn guide, section Triton 内核与自校验测试).
//
// One workgroup of 256 threads owns one (b, h) and a tile of up to 64 state columns;
// it walks the chunks in order, keeping its dk x 64 slice of S in LDS (fp32).
// rev: the walk runs over the time-reversed sequence (the backward's adjoint
// recurrence): walk position p is token N-1-p, with the decay of token N-p (gated:
// g[N-p], 0 at p = 0); per head, state_in enters divided by gamma; state_out leaves
// multiplied by the decay of token 0.

#include "common.h"
#include "launch.h"

namespace retn {

namespace {

constexpr int kThreads = 256;
constexpr int kCols = 64;      // state / output columns per workgroup
constexpr int kQRows = 16;     // query rows per sub-block
constexpr int kKeys = 32;      // keys per key block

template <typename T, bool GATED>
__global__ __launch_bounds__(kThreads) void generic_chunk_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ decay,   // gamma [H] or g [B,H,N]
    T* __restrict__ o, const float* __restrict__ state_in, float* __restrict__ state_out,
    int H, int N, int dk, int dv, int chunk, int rev) {
    extern __shared__ float smem[];
    const int kpad = dk + 1;                       // padded rows: no bank conflicts on k
    float* S = smem;                               // [dk][kCols]
    float* qb = S + dk * kCols;                    // [kQRows][dk]
    float* kb = qb + kQRows * dk;                  // [kKeys][kpad]
    float* vb = kb + kKeys * kpad;                 // [kKeys][kCols]
    float* sc = vb + kKeys * kCols;                // [kQRows][kKeys]
    float* gl = sc + kQRows * kKeys;               // [chunk] log2 cumulative decay (gated)
    float* red = gl + (GATED ? chunk : 0);         // [kThreads] scan scratch

    const int tid = threadIdx.x;
    const int bh = blockIdx.x;
    const int h = bh % H;
    const int c0 = blockIdx.y * kCols;
    const int ncol = min(kCols, dv - c0);

    const size_t qk_base = static_cast<size_t>(bh) * N * dk;
    const size_t v_base = static_cast<size_t>(bh) * N * dv;
    const size_t s_base = static_cast<size_t>(bh) * dk * dv;
    // token of walk position p
    auto tok = [&](int p) -> size_t { return static_cast<size_t>(rev ? N - 1 - p : p); };

    const float in_scale = rev && !GATED ? 1.f / decay[h] : 1.f;
    for (int e = tid; e < dk * kCols; e += kThreads) {
        const int d = e / kCols, c = e % kCols;
        float x = 0.f;
        if (state_in != nullptr && c < ncol) x = state_in[s_base + static_cast<size_t>(d) * dv + c0 + c] * in_scale;
        S[e] = x;
    }
    const float lg = GATED ? 0.f : log2f(decay[h]);   // per-head log2(gamma)
    __syncthreads();

    for (int cs = 0; cs < N; cs += chunk) {
        const int L = min(chunk, N - cs);
        if (GATED) {
            // chunk-local inclusive prefix sum of g (in log2 units): per-thread serial
            // runs, then a scan over the 256 run totals.
            const float* gb = decay + static_cast<size_t>(bh) * N;
            const int per = (L + kThreads - 1) / kThreads;
            const int a = tid * per, b = min(L, a + per);
            float run = 0.f;
            for (int j = a; j < b; ++j) {
                const int p = cs + j;
                run += (rev ? (p == 0 ? 0.f : gb[N - p]) : gb[p]) * kLog2e;
                gl[j] = run;
            }
            red[tid] = run;
            __syncthreads();
            for (int off = 1; off < kThreads; off <<= 1) {
                float add = tid >= off ? red[tid - off] : 0.f;
                __syncthreads();
                red[tid] += add;
                __syncthreads();
            }
            const float base = tid > 0 ? red[tid - 1] : 0.f;
            for (int j = a; j < b; ++j) gl[j] += base;
            __syncthreads();
        }
        // log2 of the decay from chunk start through position j (inclusive)
        auto G = [&](int j) -> float { return GATED ? gl[j] : static_cast<float>(j + 1) * lg; };
        // log2 of the decay over positions (l, j]
        auto Gd = [&](int j, int l) -> float {
            return GATED ? gl[j] - gl[l] : static_cast<float>(j - l) * lg;
        };

        // ---- outputs of the chunk, 16 query rows at a time --------------------------
        for (int r0 = 0; r0 < L; r0 += kQRows) {
            const int nr = min(kQRows, L - r0);
            for (int e = tid; e < kQRows * dk; e += kThreads) {
                const int i = e / dk, d = e % dk;
                qb[e] = i < nr ? io<T>::load(q + qk_base + tok(cs + r0 + i) * dk + d) : 0.f;
            }
            // thread -> outputs (row i = tid/64 + 4r, column c = tid % 64)
            const int c = tid % kCols;
            float acc[4] = {0.f, 0.f, 0.f, 0.f};
            const int kend = r0 + nr;                   // keys [0, kend) of the chunk
            for (int m0 = 0; m0 < kend; m0 += kKeys) {
                const int nm = min(kKeys, kend - m0);
                __syncthreads();
                for (int e = tid; e < kKeys * dk; e += kThreads) {
                    const int m = e / dk, d = e % dk;
                    kb[m * kpad + d] = m < nm ? io<T>::load(k + qk_base + tok(cs + m0 + m) * dk + d) : 0.f;
                }
                for (int e = tid; e < kKeys * kCols; e += kThreads) {
                    const int m = e / kCols, cc = e % kCols;
                    vb[e] = (m < nm && cc < ncol) ? io<T>::load(v + v_base + tok(cs + m0 + m) * dv + c0 + cc) : 0.f;
                }
                __syncthreads();
                // masked, decayed scores
                for (int e = tid; e < kQRows * kKeys; e += kThreads) {
                    const int i = e / kKeys, m = e % kKeys;
                    const int j = r0 + i, l = m0 + m;
                    float s = 0.f;
                    if (i < nr && m < nm && l <= j) {
                        for (int d = 0; d < dk; ++d) s += qb[i * dk + d] * kb[m * kpad + d];
                        s *= exp2f(Gd(j, l));
                    }
                    sc[e] = s;
                }
                __syncthreads();
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = tid / kCols + 4 * r;
                    float a = acc[r];
                    for (int m = 0; m < nm; ++m) a += sc[i * kKeys + m] * vb[m * kCols + c];
                    acc[r] = a;
                }
            }
            // cross-chunk term and store
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = tid / kCols + 4 * r;
                if (i < nr && c < ncol) {
                    float x = 0.f;
                    for (int d = 0; d < dk; ++d) x += qb[i * dk + d] * S[d * kCols + c];
                    const float out = acc[r] + exp2f(G(r0 + i)) * x;
                    io<T>::store(o + v_base + tok(cs + r0 + i) * dv + c0 + c, out);
                }
            }
            __syncthreads();
        }

        // ---- state update: S = lambda(0..L-1) S + K^T (V (.) zeta) --------------------
        const float carry = exp2f(G(L - 1));
        for (int e = tid; e < dk * kCols; e += kThreads) S[e] *= carry;
        for (int m0 = 0; m0 < L; m0 += kKeys) {
            const int nm = min(kKeys, L - m0);
            __syncthreads();
            for (int e = tid; e < kKeys * dk; e += kThreads) {
                const int m = e / dk, d = e % dk;
                kb[m * kpad + d] = m < nm ? io<T>::load(k + qk_base + tok(cs + m0 + m) * dk + d) : 0.f;
            }
            for (int e = tid; e < kKeys * kCols; e += kThreads) {
                const int m = e / kCols, cc = e % kCols;
                const float z = m < nm ? exp2f(Gd(L - 1, m0 + m)) : 0.f;
                vb[e] = (m < nm && cc < ncol) ? z * io<T>::load(v + v_base + tok(cs + m0 + m) * dv + c0 + cc) : 0.f;
            }
            __syncthreads();
            for (int e = tid; e < dk * kCols; e += kThreads) {
                const int d = e / kCols, cc = e % kCols;
                float a = S[e];
                for (int m = 0; m < nm; ++m) a += kb[m * kpad + d] * vb[m * kCols + cc];
                S[e] = a;
            }
        }
        __syncthreads();
    }

    if (state_out != nullptr) {
        const float out_scale = !rev ? 1.f : GATED ? exp2f(decay[static_cast<size_t>(bh) * N] * kLog2e) : decay[h];
        for (int e = tid; e < dk * kCols; e += kThreads) {
            const int d = e / kCols, c = e % kCols;
            if (c < ncol) state_out[s_base + static_cast<size_t>(d) * dv + c0 + c] = S[e] * out_scale;
        }
    }
}

// N = 0: the final state is the initial state (or zeros).
__global__ void copy_state_kernel(const float* __restrict__ src, float* __restrict__ dst, size_t n) {
    for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
         i += static_cast<size_t>(gridDim.x) * blockDim.x)
        dst[i] = src != nullptr ? src[i] : 0.f;
}

}  // namespace

size_t generic_chunk_lds_bytes(int dk, int chunk, bool gated) {
    size_t f = static_cast<size_t>(dk) * kCols + kQRows * dk + kKeys * (dk + 1) + kKeys * kCols +
               kQRows * kKeys + (gated ? chunk : 0) + kThreads;
    return f * sizeof(float);
}

hipError_t launch_generic_chunk(const ChunkArgs& a, hipStream_t stream) {
    const size_t lds = generic_chunk_lds_bytes(a.dk, a.chunk, a.gated);
    dim3 grid(a.B * a.H, (a.dv + kCols - 1) / kCols);
    dim3 block(kThreads);
#define RETN_LAUNCH(T, G)                                                                         \
    if (lds > 65536)                                                                              \
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&generic_chunk_kernel<T, G>),    \
                                  hipFuncAttributeMaxDynamicSharedMemorySize,                    \
                                  static_cast<int>(lds));                                        \
    hipLaunchKernelGGL((generic_chunk_kernel<T, G>), grid, block, lds, stream,                   \
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k),                   \
                       static_cast<const T*>(a.v), a.decay, static_cast<T*>(a.o), a.state_in,    \
                       a.state_out, a.H, a.N, a.dk, a.dv, a.chunk, a.reverse ? 1 : 0)
    ProfScope prof(kProfGeneric, stream);
    if (a.bf16) {
        if (a.gated) { RETN_LAUNCH(bf16_t, true); } else { RETN_LAUNCH(bf16_t, false); }
    } else {
        if (a.gated) { RETN_LAUNCH(float, true); } else { RETN_LAUNCH(float, false); }
    }
#undef RETN_LAUNCH
    return hipGetLastError();
}

hipError_t launch_copy_state(const float* src, float* dst, size_t n, hipStream_t stream) {
    if (n == 0 || dst == nullptr) return hipSuccess;
    const unsigned blocks = static_cast<unsigned>(std::min<size_t>((n + 255) / 256, 4096));
    ProfScope prof(kProfCopy, stream);
    hipLaunchKernelGGL(copy_state_kernel, dim3(blocks), dim3(256), 0, stream, src, dst, n);
    return hipGetLastError();
}

}  // namespace retn
