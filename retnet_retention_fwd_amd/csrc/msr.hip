// Gated multi-scale retention layer (the mixer around the retention operator), as the
// pwwt.cn guide describes YOCO's GateRetention (sections GateRetention 模块的内部结构 and
// 三种计算路径与增量状态):
//     q, k, v, g, gt = x Wq^T, x Wk^T, x Wv^T, x Wg^T, x Wgt^T      (no biases)
//     q, k <- interleaved rotary position rotation;  k <- k / sqrt(d_k)
//     decay  = logsigmoid(gt) / 16                                  (per token and head)
//     o      = gated retention(q, k, v, decay)                        (the chunkwise kernels)
//     z      = silu(g) * RMSNorm(o)        (per head over d_v, no affine parameters)
//     y      = z Wo^T
// Weights use the [out_features, in_features] layout, so every projection is a GEMM with
// both operands contiguous along the reduction (C = A W^T).
//
// Kernels: a bf16 matrix-core GEMM (128 x 128 tiles, two LDS stages filled by
// asynchronous global->LDS copies) whose epilogues write the operator's inputs directly
// (head layout, rotation from a per-call cos/sin table, key scaling, the log-domain gate),
// and a normalisation/gate kernel for the retention output.

#include "cdna4.h"
#include "common.h"
#include "launch.h"

#include <math.h>

#include <mutex>

namespace retn {
namespace {

constexpr int kGM = 128, kGN = 128, kGK = 64;   // GEMM tile: rows, columns, reduction step
constexpr int kGThreads = 256;                   // four waves, 2 x 2 over the tile
constexpr int kGTile = kGM * kGK * 2;            // bytes of one operand tile (16 KB)

// GEMM LDS tiles are [128 rows][64] bf16 (128-byte rows); the 16-byte unit u of row r sits
// at unit u ^ ((r >> 1) & 7), so the 16 rows of a fragment read (two rows per 256-byte
// bank cycle) cover distinct banks.
__device__ __forceinline__ int gemm_swz(int r) { return (r >> 1) & 7; }

// Epilogues: kRow stores C[M,N] row-major (bf16, or fp32 with OUTF32); kHeads stores bf16
// at [B, heads, seq, hd] (the operator's layout); kRope also turns each adjacent column
// pair (2i, 2i+1) of a head by the token's angle and multiplies by scale; kGateLog stores
// logsigmoid(C) * scale in fp32 at [B, columns, seq] (the operator's decay layout).
// kGroups: the columns are the concatenation of up to kMaxGroups projections of the same
// A, each with its own weight, output and epilogue (one launch for all of them).
enum Epi { kRow = 0, kHeads = 1, kRope = 2, kGateLog = 3, kGroups = 4 };
constexpr int kMaxGroups = 5;

// One projection of a fused launch: columns [previous group's end, end) of the launch.
// Every group but the last spans a whole number of column tiles.
struct GemmGroup {
    const bf16_t* w;   // [columns, K] weight rows, stride ldw
    void* c;           // output (layout of `kind`; kRow rows have `columns` elements)
    int end;           // exclusive end column within the launch
    int kind;          // kRow, kHeads, kRope or kGateLog
    int hd;            // head width (kHeads, kRope)
    float scale;       // kRope, kGateLog
};

struct GemmArgs {
    const bf16_t* a;   // [M, K], row stride lda
    const bf16_t* w;   // [N, K], row stride ldw
    void* c;           // output (see Epi)
    int M, N, K, lda, ldw, ldc;
    // head layouts: rows m = b * seq + n, columns = head * hd + j
    int seq, hd;
    const float2* rot;   // (cos, sin) of pair i of token n at rot[n * hd/2 + i]
    float scale;
    int ngroups;         // kGroups: the projections (N = grp[ngroups - 1].end)
    GemmGroup grp[kMaxGroups];
};

// C = A W^T with fp32 accumulation.  Requires K % 64 == 0 and N % 8 == 0 (kGroups: every
// group's width); rows past M or N read as zeros and are not stored.
template <int EPI, bool OUTF32>
__global__ __launch_bounds__(kGThreads) void gemm_tn_kernel(const GemmArgs g) {
    __shared__ __attribute__((aligned(1024))) char smem[2 * 2 * kGTile];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int tiles_n = (g.N + kGN - 1) / kGN;
    const int total = tiles_n * ((g.M + kGM - 1) / kGM);
    // XCD-aware order: consecutive launch ids rotate over the 8 XCDs; give each XCD a
    // contiguous range, so the column tiles of a row block share one L2
    int wid = blockIdx.x;
    if (total % 8 == 0) wid = (wid & 7) * (total >> 3) + (wid >> 3);
    const int m0 = (wid / tiles_n) * kGM, n0 = (wid % tiles_n) * kGN;
    const int wm = wave >> 1, wn = wave & 1;     // this wave's 64 x 64 quadrant
    // this tile's projection (workgroup-uniform): weight rows, output and epilogue
    const bf16_t* wbase = g.w;
    void* cout = g.c;
    int nstart = 0, nend = g.N, kind = EPI == kGroups ? kRow : EPI, hd = g.hd, ldc = g.ldc;
    float scale = g.scale;
    if constexpr (EPI == kGroups) {
        int gi = 0;
#pragma unroll
        for (int i = 0; i + 1 < kMaxGroups; ++i)
            if (i + 1 < g.ngroups && n0 >= g.grp[i].end) gi = i + 1;
        nstart = gi > 0 ? g.grp[gi - 1].end : 0;
        nend = g.grp[gi].end;
        wbase = g.grp[gi].w;
        cout = g.grp[gi].c;
        kind = g.grp[gi].kind;
        hd = g.grp[gi].hd;
        scale = g.grp[gi].scale;
        ldc = nend - nstart;
    }
    const int rows_a = min(kGM, g.M - m0), rows_w = min(kGN, nend - n0);
    // columns of this wave's quadrant that exist (a narrow last group computes only those)
    const int wcols = rows_w - wn * 64;
    const bf16_t* const wsrc = wbase + static_cast<size_t>(n0 - nstart) * g.ldw;
    const u32x4_t a_rs = make_rsrc(g.a + static_cast<size_t>(m0) * g.lda,
                                   static_cast<uint32_t>((rows_a - 1) * g.lda + g.K) * 2);
    const u32x4_t w_rs = make_rsrc(wsrc, static_cast<uint32_t>((rows_w - 1) * g.ldw + g.K) * 2);
    // copy i of this wave fills LDS bytes [c*1024 + 16 lane, +16), c = wave + 4 i: row
    // c*8 + lane/8 and the unit whose swizzled position is lane%8
    uint32_t aoff[4], woff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int off = (wave + 4 * i) * 1024 + lane * 16;
        const int r = off / 128, u = ((off % 128) >> 4) ^ gemm_swz(r);
        aoff[i] = static_cast<uint32_t>(r * g.lda * 2 + u * 16);
        woff[i] = static_cast<uint32_t>(r * g.ldw * 2 + u * 16);
    }
    const uint32_t lds0 = lds_addr_of(smem);
    auto issue = [&](int kt, int st) {
        const uint32_t soff = static_cast<uint32_t>(kt) * kGK * 2;
        const uint32_t base = lds0 + st * 2 * kGTile;
#pragma unroll
        for (int i = 0; i < 4; ++i) buf2lds16(a_rs, aoff[i], soff, base + (wave + 4 * i) * 1024);
#pragma unroll
        for (int i = 0; i < 4; ++i) buf2lds16(w_rs, woff[i], soff, base + kGTile + (wave + 4 * i) * 1024);
    };
    // fragment read offsets (reduction step ks adds 4 units before the swizzle)
    uint32_t ra[4], rw[4];
    int sa[4], sw[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int rowa = wm * 64 + t * 16 + l16, roww = wn * 64 + t * 16 + l16;
        ra[t] = static_cast<uint32_t>(rowa * 128);
        rw[t] = static_cast<uint32_t>(kGTile + roww * 128);
        sa[t] = gemm_swz(rowa);
        sw[t] = gemm_swz(roww);
    }
    f32x4_t acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int nk = g.K / kGK;
    issue(0, 0);
    for (int kt = 0; kt < nk; ++kt) {
        const int st = kt & 1;
        // tile kt has landed for every wave, and every wave is done with stage st ^ 1
        wait_vmcnt<0>();
        lds_barrier();
        if (kt + 1 < nk) issue(kt + 1, st ^ 1);
        const uint32_t base = lds0 + st * 2 * kGTile;
        if (wcols >= 64) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                u16x8_t af[4], wf[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int unit = ks * 4 + g4;
                    af[t] = lds16a(base + ra[t] + ((unit ^ sa[t]) << 4));
                    wf[t] = lds16a(base + rw[t] + ((unit ^ sw[t]) << 4));
                }
                // lane (g, l%16) of acc[mi][ni] gets C[row l%16 of A tile mi][columns
                // 4g..4g+3 of W tile ni]
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = mfma16(wf[ni], af[mi], acc[mi][ni]);
            }
        } else if (wcols > 0) {
            // a narrow tile: only the 16-column slices that hold columns
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int unit = ks * 4 + g4;
                u16x8_t af[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) af[t] = lds16a(base + ra[t] + ((unit ^ sa[t]) << 4));
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) {
                    if (ni * 16 >= wcols) break;
                    const u16x8_t wf = lds16a(base + rw[ni] + ((unit ^ sw[ni]) << 4));
#pragma unroll
                    for (int mi = 0; mi < 4; ++mi) acc[mi][ni] = mfma16(wf, af[mi], acc[mi][ni]);
                }
            }
        }
    }
    if (wcols <= 0) return;   // after the loop: every wave took part in its barriers
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        const int m = m0 + wm * 64 + mi * 16 + l16;
        if (m >= g.M) continue;
        const int bb = m / g.seq, tok = m % g.seq;   // head layouts
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
            const int n = n0 + wn * 64 + ni * 16 + 4 * g4;
            if (n >= nend) continue;
            const int nl = n - nstart;   // column within this projection
            f32x4_t x = acc[mi][ni];
            if (kind == kGateLog) {
                const int heads = nend - nstart;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (nl + r >= heads) break;
                    const float y = x[r];
                    static_cast<float*>(cout)[(static_cast<size_t>(bb) * heads + (nl + r)) * g.seq + tok] =
                        (fminf(y, 0.f) - log1pf(expf(-fabsf(y)))) * scale;
                }
            } else if (kind == kRow) {
                if constexpr (OUTF32)
                    *reinterpret_cast<f32x4_t*>(static_cast<float*>(cout) + static_cast<size_t>(m) * ldc + nl) = x;
                else
                    *reinterpret_cast<u16x4_t*>(static_cast<bf16_t*>(cout) + static_cast<size_t>(m) * ldc + nl) = bf4(x);
            } else {
                const int head = nl / hd, j = nl % hd;   // the four columns stay in one head
                if (kind == kRope) {
                    const float2 r0 = g.rot[static_cast<size_t>(tok) * (hd / 2) + j / 2];
                    const float2 r1 = g.rot[static_cast<size_t>(tok) * (hd / 2) + j / 2 + 1];
                    const f32x4_t y = {x[0] * r0.x - x[1] * r0.y, x[0] * r0.y + x[1] * r0.x,
                                       x[2] * r1.x - x[3] * r1.y, x[2] * r1.y + x[3] * r1.x};
                    x = y * scale;
                }
                const int heads = (nend - nstart) / hd;
                *reinterpret_cast<u16x4_t*>(static_cast<bf16_t*>(cout) +
                                            ((static_cast<size_t>(bb) * heads + head) * g.seq + tok) * hd + j) = bf4(x);
            }
        }
    }
}

// Rotation table: rot[n * half + i] = (cos, sin)(n * base^(-2i/d)) for the N tokens and
// half = d/2 pairs of a head.  The angle is formed and reduced modulo 2 pi in fp64 (it
// reaches thousands of radians), then cos and sin are taken in fp32 of the reduced angle.
__global__ __launch_bounds__(256) void rope_table_kernel(float2* __restrict__ rot, int N, int half, double log_base) {
    const size_t e = blockIdx.x * static_cast<size_t>(256) + threadIdx.x;
    if (e >= static_cast<size_t>(N) * half) return;
    const int n = static_cast<int>(e / half), i = static_cast<int>(e % half);
    const double ang = static_cast<double>(n) * exp(-log_base * (2.0 * i) / (2.0 * half));
    const double two_pi = 6.283185307179586;
    const float red = static_cast<float>(ang - two_pi * floor(ang / two_pi));
    rot[e] = make_float2(cosf(red), sinf(red));
}

// z[t, h*dv + j] = silu(gp[t, h*dv + j]) * o[b,h,n,j] / sqrt(mean_j o[b,h,n,:]^2 + eps).
// A (token, head) row is spread over gate_lanes_per_row(dv) adjacent lanes, eight
// elements per lane and pass; a wave takes 64 / that many rows.
// Lanes that share one row of d_v elements, eight elements a lane per pass: the largest
// power of two up to 64 and d_v / 8, so that a row's lanes form an aligned group that a
// butterfly of shuffles reduces.
__host__ __device__ inline int gate_lanes_per_row(int dv) {
    int l = 1;
    while (2 * l <= 64 && 2 * l <= dv / 8) l *= 2;
    return l;
}

__global__ __launch_bounds__(256) void msr_gate_kernel(const float* __restrict__ o, const bf16_t* __restrict__ gp,
                                                     bf16_t* __restrict__ z, size_t T, int N, int H, int dv,
                                                     float eps) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lpr = gate_lanes_per_row(dv), rpw = 64 / lpr, sub = lane % lpr;
    const size_t rows = T * H;
    for (size_t r0 = (blockIdx.x * static_cast<size_t>(4) + wave) * rpw; r0 < rows;
         r0 += static_cast<size_t>(gridDim.x) * 4 * rpw) {
        const size_t r = r0 + lane / lpr;   // the lanes of one row share its trip
        const bool live = r < rows;
        const size_t t = live ? r / H : 0;
        const int h = live ? static_cast<int>(r % H) : 0;
        const int b = static_cast<int>(t / N), n = static_cast<int>(t % N);
        const float* orow = o + ((static_cast<size_t>(b) * H + h) * N + n) * dv;
        const size_t zrow = t * (static_cast<size_t>(H) * dv) + static_cast<size_t>(h) * dv;
        float ss = 0.f;
        if (dv / 8 == lpr) {
            // one 8-element unit per lane: its loads (retention output and gate) go out
            // together, before the reduction, and the unit stays in registers
            f32x4_t a{}, c{};
            u16x8_t gv{};
            if (live) {
                a = *reinterpret_cast<const f32x4_t*>(orow + 8 * sub);
                c = *reinterpret_cast<const f32x4_t*>(orow + 8 * sub + 4);
                gv = *reinterpret_cast<const u16x8_t*>(gp + zrow + 8 * sub);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) ss += a[i] * a[i] + c[i] * c[i];
            for (int off = lpr / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
            const float inv = 1.f / sqrtf(ss / dv + eps);
            if (!live) continue;
            f32x4_t lo, hi;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x0 = bf16_to_f32(gv[i]), x1 = bf16_to_f32(gv[i + 4]);
                lo[i] = x0 / (1.f + expf(-x0)) * a[i] * inv;
                hi[i] = x1 / (1.f + expf(-x1)) * c[i] * inv;
            }
            *reinterpret_cast<u16x8_t*>(z + zrow + 8 * sub) = cat(bf4(lo), bf4(hi));
            continue;
        }
        for (int u = sub; live && u < dv / 8; u += lpr) {
            const f32x4_t a = *reinterpret_cast<const f32x4_t*>(orow + 8 * u);
            const f32x4_t c = *reinterpret_cast<const f32x4_t*>(orow + 8 * u + 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) ss += a[i] * a[i] + c[i] * c[i];
        }
        for (int off = lpr / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
        const float inv = 1.f / sqrtf(ss / dv + eps);
        for (int u = sub; live && u < dv / 8; u += lpr) {
            const f32x4_t a = *reinterpret_cast<const f32x4_t*>(orow + 8 * u);
            const f32x4_t c = *reinterpret_cast<const f32x4_t*>(orow + 8 * u + 4);
            const u16x8_t gv = *reinterpret_cast<const u16x8_t*>(gp + zrow + 8 * u);
            f32x4_t lo, hi;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x0 = bf16_to_f32(gv[i]), x1 = bf16_to_f32(gv[i + 4]);
                lo[i] = x0 / (1.f + expf(-x0)) * a[i] * inv;
                hi[i] = x1 / (1.f + expf(-x1)) * c[i] * inv;
            }
            *reinterpret_cast<u16x8_t*>(z + zrow + 8 * u) = cat(bf4(lo), bf4(hi));
        }
    }
}

// Log-domain decays: g[b,h,n] = logsigmoid(x[t] . wgt[h]) / 16 for the few heads of a
// token: one wave per token, lanes over D in 16-byte units (D a multiple of 8).  The
// workgroup first copies wgt into LDS when it fits (kDecayLds bytes), so the weights are
// read from memory once per workgroup instead of once per token.
constexpr int kGateHeads = 8;        // heads per pass over a token's row
constexpr int kDecayLds = 64 * 1024;
__global__ __launch_bounds__(256) void msr_decay_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ wgt,
                                                      float* __restrict__ g, size_t T, int N, int D, int H,
                                                      float inv_norm) {
    extern __shared__ __attribute__((aligned(16))) char wl[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const size_t wbytes = static_cast<size_t>(H) * D * 2;
    const bool in_lds = wbytes <= kDecayLds;
    if (in_lds) {
        for (size_t e = threadIdx.x * static_cast<size_t>(16); e < wbytes; e += 256 * 16)
            *reinterpret_cast<u16x8_t*>(wl + e) = *reinterpret_cast<const u16x8_t*>(reinterpret_cast<const char*>(wgt) + e);
        __syncthreads();
    }
    const bf16_t* w = in_lds ? reinterpret_cast<const bf16_t*>(wl) : wgt;
    for (size_t t = blockIdx.x * static_cast<size_t>(4) + wave; t < T; t += static_cast<size_t>(gridDim.x) * 4) {
        const int b = static_cast<int>(t / N), n = static_cast<int>(t % N);
        const bf16_t* xr = x + t * D;
        for (int h0 = 0; h0 < H; h0 += kGateHeads) {
            float acc[kGateHeads] = {};
            for (int u = lane; u < D / 8; u += 64) {
                const u16x8_t xv = *reinterpret_cast<const u16x8_t*>(xr + 8 * u);
                float xf[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) xf[i] = bf16_to_f32(xv[i]);
#pragma unroll
                for (int hh = 0; hh < kGateHeads; ++hh) {
                    if (h0 + hh >= H) break;
                    const u16x8_t wv = *reinterpret_cast<const u16x8_t*>(w + static_cast<size_t>(h0 + hh) * D + 8 * u);
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[hh] += xf[i] * bf16_to_f32(wv[i]);
                }
            }
#pragma unroll
            for (int hh = 0; hh < kGateHeads; ++hh) {
                float y = acc[hh];
                for (int off = 32; off >= 1; off >>= 1) y += __shfl_xor(y, off, 64);
                if (lane == 0 && h0 + hh < H)
                    g[(static_cast<size_t>(b) * H + h0 + hh) * N + n] = (fminf(y, 0.f) - log1pf(expf(-fabsf(y)))) * inv_norm;
            }
        }
    }
}

template <int EPI, bool OUTF32>
hipError_t gemm_launch(const GemmArgs& g, hipStream_t stream) {
    if (g.M == 0) return hipSuccess;
    const size_t tiles = static_cast<size_t>((g.M + kGM - 1) / kGM) * ((g.N + kGN - 1) / kGN);
    if (tiles > static_cast<size_t>(INT32_MAX)) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_tn_kernel<EPI, OUTF32>), dim3(static_cast<unsigned>(tiles)), dim3(kGThreads), 0, stream, g);
    return hipGetLastError();
}

GemmArgs gemm_args(const void* a, const void* w, void* c, int M, int N, int K) {
    GemmArgs g{};
    g.a = static_cast<const bf16_t*>(a);
    g.w = static_cast<const bf16_t*>(w);
    g.c = c;
    g.M = M;
    g.N = N;
    g.K = K;
    g.lda = K;
    g.ldw = K;
    g.ldc = N;
    g.seq = 1;
    g.hd = 1;
    g.scale = 1.f;
    return g;
}

}  // namespace

bool gemm_tn_supported(int N, int K) { return N > 0 && K > 0 && K % kGK == 0 && N % 8 == 0; }

hipError_t launch_gemm_tn(const void* a, const void* w, void* c, int M, int N, int K, bool out_f32,
                          hipStream_t stream) {
    if (!gemm_tn_supported(N, K)) return hipErrorInvalidValue;
    const GemmArgs g = gemm_args(a, w, c, M, N, K);
    return out_f32 ? gemm_launch<kRow, true>(g, stream) : gemm_launch<kRow, false>(g, stream);
}

namespace {

// Decays for shapes whose gate projection width is not a whole number of column tiles.
hipError_t launch_decay(const MsrPtrs& x, float* g, size_t T, const MsrShape& s, hipStream_t st) {
    // a few workgroups per CU, each looping over tokens (the weights are staged once each)
    const size_t wbytes = static_cast<size_t>(s.H) * s.D * 2;
    const unsigned tblocks = static_cast<unsigned>(std::min<size_t>((T + 3) / 4, 1024));
    static std::once_flag attr_once;   // thread-safe one-time init of the LDS limit
    std::call_once(attr_once, [] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&msr_decay_kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, kDecayLds);
    });
    hipLaunchKernelGGL(msr_decay_kernel, dim3(tblocks), dim3(256), wbytes <= kDecayLds ? wbytes : 0, st,
                       static_cast<const bf16_t*>(x.x), static_cast<const bf16_t*>(x.wgt), g, T, s.N, s.D, s.H,
                       1.f / 16.f);
    return hipGetLastError();
}

}  // namespace

MsrPlan msr_plan(const MsrShape& s) {
    MsrPlan p{};
    const size_t T = static_cast<size_t>(s.B) * s.N;
    const size_t qk = T * s.H * s.dk, vv = T * s.H * s.dv;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += (bytes + 255) & ~static_cast<size_t>(255);
        return o;
    };
    p.chunk = s.N > 0 ? std::min(s.chunk, s.N) : 1;
    p.ok = s.B >= 0 && s.N >= 0 && s.D > 0 && s.H > 0 && gemm_tn_supported(s.H * s.dk, s.D) &&
           gemm_tn_supported(s.H * s.dv, s.D) && gemm_tn_supported(s.D, s.H * s.dv) &&
           mfma_chunk_supported(s.dk, s.dv, p.chunk, true) && s.dk % 4 == 0 &&
           // the retention step addresses a head's rows with 32-bit byte offsets
           (static_cast<size_t>(s.N) + 64) * std::max(s.dk, s.dv) * 2 < (static_cast<size_t>(1) << 31);
    if (!p.ok || T == 0) return p;
    p.off_rot = take(static_cast<size_t>(s.N) * (s.dk / 2) * 8);
    p.off_q = take(qk * 2);
    p.off_k = take(qk * 2);
    p.off_v = take(vv * 2);
    p.off_gp = take(vv * 2);
    p.off_g = take(T * s.H * 4);
    p.off_o = take(vv * 4);
    p.off_z = take(vv * 2);
    p.ret = mfma_chunk_plan(s.B, s.H, s.N, s.dk, s.dv, p.chunk, true);
    p.off_ret = take(p.ret.workspace_bytes);
    p.total = off;
    return p;
}

hipError_t run_msr(const MsrShape& s, const MsrPtrs& x, const MsrPlan& p, void* workspace, hipStream_t st) {
    const size_t T = static_cast<size_t>(s.B) * s.N;
    if (T == 0) return hipSuccess;
    char* ws = static_cast<char*>(workspace);
    float2* rot = reinterpret_cast<float2*>(ws + p.off_rot);
    void *q = ws + p.off_q, *k = ws + p.off_k, *v = ws + p.off_v, *gp = ws + p.off_gp, *z = ws + p.off_z;
    float* g = reinterpret_cast<float*>(ws + p.off_g);
    float* o = reinterpret_cast<float*>(ws + p.off_o);
    const int M = static_cast<int>(T);
    hipError_t e;
#define RETN_TRY(call)                 \
    do {                               \
        e = (call);                    \
        if (e != hipSuccess) return e; \
    } while (0)
    const size_t pairs = static_cast<size_t>(s.N) * (s.dk / 2);
    hipLaunchKernelGGL(rope_table_kernel, dim3(static_cast<unsigned>((pairs + 255) / 256)), dim3(256), 0, st, rot, s.N,
                       s.dk / 2, log(static_cast<double>(s.rope_base)));
    RETN_TRY(hipGetLastError());
    const int nq = s.H * s.dk, nv = s.H * s.dv;
    const float kscale = 1.f / sqrtf(static_cast<float>(s.dk));
    if (nq % kGN == 0 && nv % kGN == 0) {
        // the q, k, v and gate projections and the decay logits in one launch: all five
        // read x, and one launch has one tail instead of five (the decay group's tile
        // computes only its H columns)
        GemmArgs ga = gemm_args(x.x, x.wq, q, M, 2 * nq + 2 * nv + s.H, s.D);
        ga.seq = s.N;
        ga.rot = rot;
        ga.ngroups = 5;
        ga.grp[0] = GemmGroup{static_cast<const bf16_t*>(x.wq), q, nq, kRope, s.dk, 1.f};
        ga.grp[1] = GemmGroup{static_cast<const bf16_t*>(x.wk), k, 2 * nq, kRope, s.dk, kscale};
        ga.grp[2] = GemmGroup{static_cast<const bf16_t*>(x.wv), v, 2 * nq + nv, kHeads, s.dv, 1.f};
        ga.grp[3] = GemmGroup{static_cast<const bf16_t*>(x.wg), gp, 2 * nq + 2 * nv, kRow, 1, 1.f};
        ga.grp[4] = GemmGroup{static_cast<const bf16_t*>(x.wgt), g, 2 * nq + 2 * nv + s.H, kGateLog, 1, 1.f / 16.f};
        RETN_TRY((gemm_launch<kGroups, false>(ga, st)));
    } else {
        GemmArgs gq = gemm_args(x.x, x.wq, q, M, nq, s.D);
        gq.seq = s.N;
        gq.hd = s.dk;
        gq.rot = rot;
        RETN_TRY((gemm_launch<kRope, false>(gq, st)));
        GemmArgs gk = gq;
        gk.w = static_cast<const bf16_t*>(x.wk);
        gk.c = k;
        gk.scale = kscale;
        RETN_TRY((gemm_launch<kRope, false>(gk, st)));
        GemmArgs gv = gemm_args(x.x, x.wv, v, M, nv, s.D);
        gv.seq = s.N;
        gv.hd = s.dv;
        RETN_TRY((gemm_launch<kHeads, false>(gv, st)));
        RETN_TRY((gemm_launch<kRow, false>(gemm_args(x.x, x.wg, gp, M, nv, s.D), st)));
        RETN_TRY(launch_decay(x, g, T, s, st));
    }
    ChunkArgs a{q, k, v, g, o, nullptr, nullptr, s.B, s.H, s.N, s.dk, s.dv, p.chunk, true, true,
                ws + p.off_ret, p.ret.workspace_bytes};
    if (chunk1_dot_supported(s.dk, s.dv, p.chunk)) {
        // one 128-column tile per row: the retention pass normalises and gates its own
        // fp32 rows and writes z (no fp32 round trip, no separate gate launch)
        a.ng_gate = gp;
        a.ng_out = z;
        a.ng_eps = s.norm_eps;
        RETN_TRY(launch_mfma_chunk(a, p.ret, st));
    } else {
        a.out_f32 = true;
        RETN_TRY(launch_mfma_chunk(a, p.ret, st));
        const size_t rows = T * s.H;
        const size_t rows_per_block = 4 * static_cast<size_t>(64 / gate_lanes_per_row(s.dv));
        const unsigned blocks =
            static_cast<unsigned>(std::min<size_t>((rows + rows_per_block - 1) / rows_per_block, 1u << 20));
        hipLaunchKernelGGL(msr_gate_kernel, dim3(blocks), dim3(256), 0, st, o, static_cast<const bf16_t*>(gp),
                           static_cast<bf16_t*>(z), T, s.N, s.H, s.dv, s.norm_eps);
        RETN_TRY(hipGetLastError());
    }
    RETN_TRY(launch_gemm_tn(z, x.wo, x.y, M, s.D, s.H * s.dv, false, st));
#undef RETN_TRY
    return hipSuccess;
}

}  // namespace retn
