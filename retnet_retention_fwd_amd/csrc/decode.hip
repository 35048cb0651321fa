// Recurrent decode step ("RetNet retention mechanism" tutorial, section 递归推理):
//     S <- lambda S + k^T v   (fp32, in place),     o = q S   (with the updated S)
// lambda = gamma[h] per head, or exp(g[b,h]) for the gated variant (pwwt.cn guide,
// section 三种计算路径与增量状态).
//
// The step streams the whole fp32 state once in and once out, so it is bound by HBM
// bandwidth; the arithmetic is one FMA pair per state element.  One workgroup owns
// one (b, h) state.  In the vector kernel each thread owns a float4 column group and
// a strided set of rows (consecutive threads cover whole rows, so every load and store
// instruction moves whole 512-byte rows), issues all of its state loads before using
// them, and sums o over its rows.  The row groups that share a column are combined by
// lane exchanges inside each wave, and the waves' partial sums through LDS.

#include "common.h"
#include "launch.h"

namespace retn {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxDk = 256;

template <typename T, bool GATED, int DV, int DK>
__global__ __launch_bounds__(kThreads) void decode_vec_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ decay, float* __restrict__ S, T* __restrict__ o, int H, int dk_rt) {
    constexpr int TPR = DV / 4;            // threads per state row (one float4 each)
    constexpr int RPP = kThreads / TPR;    // rows per pass
    const int dk = DK > 0 ? DK : dk_rt;

    constexpr int RPW = 64 / TPR;          // row groups of one wave
    constexpr int NWV = kThreads / 64;     // waves
    static_assert(64 % TPR == 0 && RPP == RPW * NWV, "row groups split over the waves");
    __shared__ float qs[kMaxDk];
    __shared__ float ks[kMaxDk];
    __shared__ f32v4 red[NWV][TPR];

    const int tid = threadIdx.x;
    const int bh = blockIdx.x;
    const int cg = tid % TPR;
    const int rg = tid / TPR;

    for (int i = tid; i < dk; i += kThreads) {
        qs[i] = io<T>::load(q + static_cast<size_t>(bh) * dk + i);
        ks[i] = io<T>::load(k + static_cast<size_t>(bh) * dk + i);
    }
    const T* vp = v + static_cast<size_t>(bh) * DV + 4 * cg;
    const f32v4 vv = {io<T>::load(vp), io<T>::load(vp + 1), io<T>::load(vp + 2), io<T>::load(vp + 3)};
    const float lam = GATED ? __expf(decay[bh]) : decay[bh % H];
    __syncthreads();

    f32v4* Sp = reinterpret_cast<f32v4*>(S + static_cast<size_t>(bh) * dk * DV) + cg;
    f32v4 acc = {0.f, 0.f, 0.f, 0.f};
    if (DK > 0) {
        constexpr int NR = DK > 0 ? (DK + RPP - 1) / RPP : 1;
        f32v4 s[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const int i = rg + r * RPP;
            if (i < dk) s[r] = __builtin_nontemporal_load(Sp + static_cast<size_t>(i) * TPR);
        }
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const int i = rg + r * RPP;
            if (i < dk) {
                const float ki = ks[i], qi = qs[i];
                f32v4 x = s[r];
                x.x = fmaf(lam, x.x, ki * vv.x);
                x.y = fmaf(lam, x.y, ki * vv.y);
                x.z = fmaf(lam, x.z, ki * vv.z);
                x.w = fmaf(lam, x.w, ki * vv.w);
                __builtin_nontemporal_store(x, Sp + static_cast<size_t>(i) * TPR);
                acc.x = fmaf(qi, x.x, acc.x);
                acc.y = fmaf(qi, x.y, acc.y);
                acc.z = fmaf(qi, x.z, acc.z);
                acc.w = fmaf(qi, x.w, acc.w);
            }
        }
    } else {
#pragma unroll 4
        for (int i = rg; i < dk; i += RPP) {
            f32v4 x = __builtin_nontemporal_load(Sp + static_cast<size_t>(i) * TPR);
            const float ki = ks[i], qi = qs[i];
            x.x = fmaf(lam, x.x, ki * vv.x);
            x.y = fmaf(lam, x.y, ki * vv.y);
            x.z = fmaf(lam, x.z, ki * vv.z);
            x.w = fmaf(lam, x.w, ki * vv.w);
            __builtin_nontemporal_store(x, Sp + static_cast<size_t>(i) * TPR);
            acc.x = fmaf(qi, x.x, acc.x);
            acc.y = fmaf(qi, x.y, acc.y);
            acc.z = fmaf(qi, x.z, acc.z);
            acc.w = fmaf(qi, x.w, acc.w);
        }
    }
    // o over rows: first the RPW row groups of this wave (lanes TPR apart) by lane
    // exchanges, then the waves' partial sums through LDS
#pragma unroll
    for (int m = TPR; m < 64; m <<= 1) {
        acc.x += __shfl_xor(acc.x, m, 64);
        acc.y += __shfl_xor(acc.y, m, 64);
        acc.z += __shfl_xor(acc.z, m, 64);
        acc.w += __shfl_xor(acc.w, m, 64);
    }
    const int wave = tid >> 6;
    if ((tid & 63) < TPR) red[wave][cg] = acc;
    __syncthreads();
    // thread t < DV owns output column t
    if (tid < DV) {
        const int c4 = tid / 4, lane = tid % 4;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < NWV; ++w) {
            const f32v4 p = red[w][c4];
            sum += lane == 0 ? p.x : lane == 1 ? p.y : lane == 2 ? p.z : p.w;
        }
        io<T>::store(o + static_cast<size_t>(bh) * DV + tid, sum);
    }
}

// Any dk, dv in range: scalar accesses, columns in blocks of 64.
template <typename T, bool GATED>
__global__ __launch_bounds__(kThreads) void decode_generic_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ decay, float* __restrict__ S, T* __restrict__ o, int H, int dk,
    int dv) {
    __shared__ float qs[kMaxDk];
    __shared__ float ks[kMaxDk];
    __shared__ float red[kThreads / 64][64];
    const int tid = threadIdx.x;
    const int bh = blockIdx.x;
    for (int i = tid; i < dk; i += kThreads) {
        qs[i] = io<T>::load(q + static_cast<size_t>(bh) * dk + i);
        ks[i] = io<T>::load(k + static_cast<size_t>(bh) * dk + i);
    }
    const float lam = GATED ? __expf(decay[bh]) : decay[bh % H];
    __syncthreads();
    float* Sp = S + static_cast<size_t>(bh) * dk * dv;
    const int c_in = tid % 64, rg = tid / 64;
    for (int cb = 0; cb < dv; cb += 64) {
        const int c = cb + c_in;
        float acc = 0.f;
        if (c < dv) {
            const float vc = io<T>::load(v + static_cast<size_t>(bh) * dv + c);
            for (int i = rg; i < dk; i += kThreads / 64) {
                const float x = fmaf(lam, Sp[static_cast<size_t>(i) * dv + c], ks[i] * vc);
                Sp[static_cast<size_t>(i) * dv + c] = x;
                acc = fmaf(qs[i], x, acc);
            }
        }
        red[rg][c_in] = acc;
        __syncthreads();
        if (tid < 64 && c < dv) {
            float sum = 0.f;
#pragma unroll
            for (int r = 0; r < kThreads / 64; ++r) sum += red[r][c_in];
            io<T>::store(o + static_cast<size_t>(bh) * dv + c, sum);
        }
        __syncthreads();
    }
}

template <typename T, bool GATED>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
    const dim3 grid(a.B * a.H), block(kThreads);
    const T* q = static_cast<const T*>(a.q);
    const T* k = static_cast<const T*>(a.k);
    const T* v = static_cast<const T*>(a.v);
    T* o = static_cast<T*>(a.o);
    ProfScope prof(kProfDecode, stream);
    if (a.dv == 128 && a.dk == 128) {
        hipLaunchKernelGGL((decode_vec_kernel<T, GATED, 128, 128>), grid, block, 0, stream, q, k, v,
                           a.decay, a.state, o, a.H, a.dk);
    } else if (a.dv == 128) {
        hipLaunchKernelGGL((decode_vec_kernel<T, GATED, 128, 0>), grid, block, 0, stream, q, k, v,
                           a.decay, a.state, o, a.H, a.dk);
    } else if (a.dv == 64) {
        hipLaunchKernelGGL((decode_vec_kernel<T, GATED, 64, 0>), grid, block, 0, stream, q, k, v,
                           a.decay, a.state, o, a.H, a.dk);
    } else if (a.dv == 256) {
        hipLaunchKernelGGL((decode_vec_kernel<T, GATED, 256, 0>), grid, block, 0, stream, q, k, v,
                           a.decay, a.state, o, a.H, a.dk);
    } else {
        hipLaunchKernelGGL((decode_generic_kernel<T, GATED>), grid, block, 0, stream, q, k, v,
                           a.decay, a.state, o, a.H, a.dk, a.dv);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    if (a.bf16) return a.gated ? launch_typed<bf16_t, true>(a, stream) : launch_typed<bf16_t, false>(a, stream);
    return a.gated ? launch_typed<float, true>(a, stream) : launch_typed<float, false>(a, stream);
}

}  // namespace retn
