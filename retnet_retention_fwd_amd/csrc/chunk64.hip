// bf16 chunkwise retention forward on the gfx950 matrix cores, for chunks of exactly
// 64 tokens (one LDS block per chunk).
//
// Method ("RetNet retention mechanism" tutorial, section 块级循环, with the per-row
// cross-chunk decay; gated decays from the pwwt.cn guide, section Triton 内核与自校验测试).
// For a chunk of L tokens with chunk-local log2 decays G (G_j = log2 of the product of
// the decays of positions 0..j):
//     O     = (Q K^T (.) D) V + diag(2^G) (Q S_prev),      D_jl = 2^(G_j - G_l), j >= l
//     S_new = 2^(G_{L-1}) S_prev + K^T (V (.) zeta),        zeta_l = 2^(G_{L-1} - G_l)
//
// This is the general matrix-core kernel's single-block path without its general
// machinery: every step of the walk is one whole chunk, so there is no query/key block
// bookkeeping; the walk is unrolled by two so that every LDS address is a per-lane
// pattern plus a compile-time offset; per-head decay factors of a full chunk are
// computed once (a step then needs two exponentials); the gated chunk-local prefix sums
// are formed one chunk ahead by wave 0, so no step waits on them behind a barrier.
// Fragment layouts, swizzles and the state-row permutation are those of the general
// kernel (mfma_chunk.hip), and so are its call forms: rows of q and k (and of v) with a
// stride, column slices run as extra chains, the time-reversed walk of the backward's
// adjoint recurrence (REV: walk position m reads and writes token N-1-m and takes the
// decay of token N-m, none at m = 0; per head, state_in enters divided by gamma; state_out
// leaves multiplied by the decay of token 0) and, gated, fp32 output.  For the gated
// backward's dq and dk passes (one 128-column tile per row) the output can also leave
// as bf16 together with each row's dot product against a second tensor taken from the
// fp32 accumulators (OUT = kOutDot), which the gate gradient sums.  For the gated layer
// (one 128-column tile per row) the output can leave already normalised and gated
// (OUT = kOutNormGate): z = silu(gate) * o / rms(o), bf16, in the layer's token-major
// layout, from the fp32 rows staged in LDS.
//
// Work decomposition: a workgroup owns one (b,h), one segment of the sequence and 128
// state columns; its eight waves own 16 columns each and hold their DK x 16 slice of S
// in fp32 matrix-core accumulators.  A step (one chunk) runs:
//   barrier; cross term X = diag(2^G) Q S_prev (the next chunk's K and V copies go out
//   between its matrix instructions); this wave's score tiles, decayed, bf16, into LDS;
//   barrier; (one Q stage: the next chunk's Q copies) state update; X += P V; X staged
//   in LDS as bf16 and stored in whole rows after the next barrier (fp32 output: stored
//   from the accumulators, 16 bytes per lane).
// Prefix split (two segments, no pre-pass): the second segment's workgroups first walk
// the first segment's chunks state-only for their entry state.  Per head that walk runs
// over three LDS stages of K and V (the Q and output staging areas hold the third), with
// copies two chunks ahead; gated, it stays on the walk's own two stages.

#include "cdna4.h"
#include "chunk_tiles.h"
#include "common.h"
#include "launch.h"

#include <mutex>
#include <type_traits>

namespace retn {

namespace {

constexpr int kC1Cols = 128;   // state columns per workgroup
constexpr int kC1Waves = 8;    // 16 columns per wave

// Output forms: bf16; fp32; bf16 plus the row dots of the fp32 rows with a second tensor;
// the gated layer's normalised and gated rows.
constexpr int kOutBf16 = 0, kOutF32 = 1, kOutDot = 2, kOutNormGate = 3;

// LDS layout: Q (one stage for d_k = 256, two otherwise), two stages of K and V, the P
// fragments of the current chunk, the staging area of one output block, (gated) two
// stages of the chunk-local log2 prefix sums, (row dots, norm-gate) two stages of the
// waves' partial row sums [64 rows][8 waves] and (norm-gate) one fp32 output block.
template <int DK, bool GATED, bool DOT = false, bool NG = false>
struct C1Lds {
    static constexpr int QRB = DK * 2, VRB = kC1Cols * 2;       // row bytes
    static constexpr int QS = DK == 256 ? 1 : 2;                // Q stages
    static constexpr int kQTile = kBlk * QRB, kKTile = kBlk * QRB, kVTile = kBlk * VRB;
    static constexpr int kQ = 0;
    static constexpr int kK = kQ + QS * kQTile;
    static constexpr int kV = kK + 2 * kKTile;
    static constexpr int kP = kV + 2 * kVTile;
    static constexpr int kX = kP + kPBytes;
    static constexpr int kG = kX + kBlk * kC1Cols * 2;
    static constexpr int kD = kG + (GATED ? 2 * kBlk * 4 : 0);
    static constexpr int kDStage = kBlk * kC1Waves * 4;
    static constexpr int kXF = kD + (DOT || NG ? 2 * kDStage : 0);
    static constexpr int kBytes = kXF + (NG ? kBlk * kC1Cols * 4 : 0);
    static_assert(kBytes <= kLdsBytes, "LDS layout too large");
};

template <int DK, bool GATED, bool REV, int OUT>
__global__ __launch_bounds__(kC1Waves * 64, 1) __attribute__((amdgpu_waves_per_eu(2, 2))) void chunk1_kernel(
    const KArgs ka) {
    constexpr bool OF32 = OUT == kOutF32;   // fp32 output
    constexpr bool DOT = OUT == kOutDot;    // bf16 output and row dots
    constexpr bool NG = OUT == kOutNormGate;   // normalised, gated bf16 rows
    // fp32 results for the backward (the output, or the row dots) take the state operand of
    // the cross term as two bf16 terms
    constexpr bool HILO = OUT == kOutF32 || OUT == kOutDot;
    static_assert(!DOT || (GATED && DK == 128), "row dots: gated, 128-wide scores");
    static_assert(!NG || (GATED && DK == 128 && !REV), "norm-gate: gated forward, 128-wide scores");
    using L_ = C1Lds<DK, GATED, DOT, NG>;
    constexpr int NW = kC1Waves, DVT = kC1Cols;
    constexpr int QRB = L_::QRB, VRB = L_::VRB, QS = L_::QS;
    constexpr int DT = DK / 16;    // 16-row tiles of the state
    constexpr int KS = DK / 32;    // reduction steps over DK
    constexpr int KL = KS < 4 ? KS : 4;
    constexpr int SL = KS < 4 ? KS : 4;
    using QCopy = TileCopy<QRB, false, NW, REV>;
    using VCopy = TileCopy<VRB, true, NW, REV>;
    constexpr int kNQ = QCopy::kPerWave, kNV = VCopy::kPerWave;

    const bf16_t* __restrict__ q = ka.q;
    const bf16_t* __restrict__ k = ka.k;
    const bf16_t* __restrict__ v = ka.v;
    const float* __restrict__ decay = ka.decay;
    typedef std::conditional_t<OF32, float, bf16_t> out_t;
    out_t* __restrict__ o = static_cast<out_t*>(ka.o);
    const int H = ka.H, N = ka.N, dv = ka.dv;
    const int nseg = ka.nseg, ndvt = ka.ndvt;
    extern __shared__ __attribute__((aligned(1024))) char smem[];

    // ---- work item (XCD-aware: each XCD takes a contiguous range of work ids, so a
    // (b,h)'s column tiles and segments share an L2)
    int wid = blockIdx.x;
    if (ka.total_groups % 8 == 0) wid = (wid & 7) * (ka.total_groups >> 3) + (wid >> 3);
    const int dvt = wid % ndvt;
    const int seg = (wid / ndvt) % nseg;
    const int ch = wid / (ndvt * nseg);   // chain: (b,h) and column slice
    const int nsl = ka.nsl > 1 ? ka.nsl : 1;
    const int slc = ch % nsl;
    const int bh = ch / nsl;
    const int h = bh % H;

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    const int trj = l16 >> 2, trq = l16 & 3;
    const int col0 = dvt * DVT, wcol = wave * 16;

    // prefix split (two segments): segment 1 first walks [0, pre_tokens) state-only
    const bool split = ka.pre_tokens > 0;
    const int t_begin = split ? (seg == 0 ? 0 : ka.pre_tokens) : seg * ka.seg_tokens;
    const int t_end = split ? (seg == 0 ? min(N, ka.pre_tokens) : N) : min(N, t_begin + ka.seg_tokens);
    const int nck = (t_end - t_begin + kBlk - 1) / kBlk;
    const int npre = split && seg == 1 ? ka.pre_tokens / kBlk : 0;   // prefix chunks
    const float lg = GATED ? 0.f : log2f(decay[h]);

    // rows of q and k are ldqk elements apart, rows of v ldv; o is contiguous
    const int ldqk = ka.ldqk, ldv = ka.ldv;
    const uint32_t qk_rb = static_cast<uint32_t>(ldqk) * 2, v_rb = static_cast<uint32_t>(ldv) * 2;
    const size_t qk_bh = static_cast<size_t>(bh) * N * ldqk + static_cast<size_t>(slc) * ka.sl_qk;
    const size_t v_bh = static_cast<size_t>(bh) * N * ldv;
    const size_t o_bh = static_cast<size_t>(bh) * N * dv + slc * ka.sl_o;
    const size_t s_bh = static_cast<size_t>(bh) * DK * dv + slc * ka.sl_state;
    const size_t s_stride_seg = static_cast<size_t>(DK) * dv;
    const float* g_bh = GATED ? decay + static_cast<size_t>(bh) * N : nullptr;
    // row dots: rows of the second tensor (dv elements, token order) and the dots' output
    const bf16_t* const xd_bh = DOT ? ka.xdot + static_cast<size_t>(bh) * N * dv : nullptr;
    float* const dG_bh = DOT ? ka.dG + static_cast<size_t>(bh) * N : nullptr;
    // norm-gate: token n's row of the gate and of z is ((b N + n) H + h) d_v in the layer's
    // [B, N, H, d_v] layout
    const size_t ng_b = static_cast<size_t>(bh / H) * N, ng_h = static_cast<size_t>(h) * dv;
    auto ng_off = [&](int n) -> size_t { return (ng_b + n) * static_cast<size_t>(H) * dv + ng_h; };
    // ranges end with the last row's own columns; rows past N (REV: before 0) read as zeros
    const u32x4_t q_rs = make_rsrc(q + qk_bh, static_cast<uint32_t>((N - 1) * ldqk + DK) * 2);
    const u32x4_t k_rs = make_rsrc(k + qk_bh, static_cast<uint32_t>((N - 1) * ldqk + DK) * 2);
    const u32x4_t v_rs = make_rsrc(v + v_bh + col0, static_cast<uint32_t>((N - 1) * ldv + dv - col0) * 2);
    const uint32_t lds0 = lds_addr_of(smem);
    QCopy kcp;   // Q and K tiles (same row length and swizzle)
    VCopy vcp;
    kcp.init(ldqk * 2, wave, lane, N);
    vcp.init(ldv * 2, wave, lane, N);
    const uint32_t wofs = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(wave)) * 1024u;

    // State accumulator element (dt, i) of lane (g, l%16) holds state row srow(dt, i) of
    // column col0 + wcol + l%16 (the layout of the general kernel: conflict-free K^T
    // transpose reads, and an 8-row B operand of Q S per 16-byte Q read).
    auto srow = [&](int dt, int i) -> int { return 32 * (dt >> 1) + 8 * g4 + 4 * ((dt ^ g4) & 1) + i; };

    // ---- incoming state: state_in, the scanned entry state, or (fuse_scan) composed here
    // Each stored state is fetched as one batch of loads, all issued before any is used
    // (the sched barrier keeps the scheduler from pairing every load with its use): the
    // walk's start then waits on these loads' latency once per batch.
    f32x4_t S[DT];
    {
        const int cidx = col0 + wcol + l16;
        auto fetch = [&](auto& x, const float* src) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) x[dt][i] = src[static_cast<uint32_t>(srow(dt, i) * dv + cidx)];
            __builtin_amdgcn_sched_barrier(0);
        };
        // a segment state: seg_t, one of the transposed problem (d_k and d_v exchanged),
        // whose row cidx holds this lane's four consecutive state rows in 16 bytes
        auto fetch_seg = [&](auto& x, const float* src) {
            if (ka.seg_t) {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const f32x4_t t = *reinterpret_cast<const f32x4_t*>(src + static_cast<uint32_t>(cidx * DK + srow(dt, 0)));
#pragma unroll
                    for (int i = 0; i < 4; ++i) x[dt][i] = t[i];
                }
                __builtin_amdgcn_sched_barrier(0);
            } else {
                fetch(x, src);
            }
        };
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) S[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (nseg == 1 || split || ka.fuse_scan) {
            if (ka.state_in != nullptr && ka.st_ld > 0) {
                // the incoming state in place in the caller's layout, transposed: element
                // (r, c) of slice slc is row c, column slc * DK + r of a [dv][st_ld] state
                const float* const src = ka.state_in + static_cast<size_t>(bh) * dv * ka.st_ld +
                                         static_cast<size_t>(slc) * DK;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        S[dt][i] = src[static_cast<size_t>(cidx) * ka.st_ld + srow(dt, i)];
                __builtin_amdgcn_sched_barrier(0);
            } else if (ka.state_in != nullptr) {
                fetch(S, ka.state_in + s_bh);
            }
            if (ka.state_in != nullptr) {
                if constexpr (REV && !GATED) {
                    const float inv = 1.f / decay[h];
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) S[dt] *= inv;
                }
            }
            // the local states of the segments before this one, folded in order (from no
            // incoming state, the first is taken as it is)
            const int nfold = (nseg > 1 && !split) ? seg : 0;
            const float* const ss = ka.seg_state + static_cast<size_t>(ch) * nseg * s_stride_seg;
            const float* const sl = ka.seg_log2 + static_cast<size_t>(ch) * nseg;
            int sg = 0;
            if (nfold > 0 && ka.state_in == nullptr) {
                fetch_seg(S, ss);
                sg = 1;
            }
            for (; sg < nfold; ++sg) {
                float x[DT][4];
                fetch_seg(x, ss + sg * s_stride_seg);
                const float scale = exp2f(sl[sg]);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) S[dt][i] = S[dt][i] * scale + x[dt][i];
            }
        } else {
            fetch_seg(S, ka.seg_state + (static_cast<size_t>(ch) * nseg + seg) * s_stride_seg);
        }
    }

    // ---- per-lane LDS read patterns (byte offsets within a tile)
    //   Q/K rows (row tile t, reduction step ks): pq[ks%4] + t*16*QRB + (ks/4)*256;
    //   K^T transposed reads (state tile dt, key rows r0 and r0+4, key half kh):
    //     pkt[pl][(dt/2)%4][dt%2] + kh*32*QRB + (dt/8)*256;
    //   V transposed reads: pvp + (ks*32 + 16 half)*VRB (P V), pvs[pl] + kh*32*VRB (state).
    uint32_t pq[KL], pkt[2][SL][2], pvp, pvs[2];
    {
        const int s = swz_qk<QRB / 16>(l16);
#pragma unroll
        for (int kl = 0; kl < KL; ++kl)
            pq[kl] = static_cast<uint32_t>(l16 * QRB + 16 * (4 * (kl ^ (s >> 2)) + (g4 ^ (s & 3))));
#pragma unroll
        for (int pl = 0; pl < 2; ++pl) {
            const int rb = 8 * g4 + trj + 4 * pl;
            const int w = swz_qk<QRB / 16>(rb);
#pragma unroll
            for (int sl = 0; sl < SL; ++sl)
#pragma unroll
                for (int hb = 0; hb < 2; ++hb)
                    pkt[pl][sl][hb] = static_cast<uint32_t>(rb * QRB + 16 * (4 * (sl ^ (w >> 2)) + (trq ^ (w & 3))) +
                                                            8 * (hb ^ (trq & 1)));
            const int sv = swz_v<VRB / 16>(rb);
            pvs[pl] = static_cast<uint32_t>(rb * VRB + 16 * (2 * (wave ^ (sv >> 1)) + (trq >> 1)) + 8 * (trq & 1));
        }
        const int rbp = 4 * g4 + trj;
        const int svp = swz_v<VRB / 16>(rbp);
        pvp = static_cast<uint32_t>(rbp * VRB + 16 * (2 * (wave ^ (svp >> 1)) + (trq >> 1)) + 8 * (trq & 1));
    }
    // Absolute per-lane LDS addresses of the patterns, one register each, so that every
    // stage, tile and reduction-step offset is an immediate of the read (below 64 KB).
    uint32_t aq[KL], ak[KL], akt[2][SL][2], avs[2];
#pragma unroll
    for (int kl = 0; kl < KL; ++kl) {
        aq[kl] = opaque(lds0 + L_::kQ + pq[kl]);
        ak[kl] = opaque(lds0 + L_::kK + pq[kl]);
    }
#pragma unroll
    for (int pl = 0; pl < 2; ++pl) {
#pragma unroll
        for (int sl = 0; sl < SL; ++sl)
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) akt[pl][sl][hb] = opaque(lds0 + L_::kK + pkt[pl][sl][hb]);
        avs[pl] = opaque(lds0 + L_::kV + pvs[pl]);
    }
    const uint32_t avp = opaque(lds0 + L_::kV + pvp);
    const uint32_t ap = opaque(lds0 + L_::kP + static_cast<uint32_t>(lane) * 16u);

    // ---- decays of a full chunk (per head), computed once.  Every exponent is >= 0,
    // so no factor exceeds 1.
    //   fxi[mt]:   gamma^(row + 1) for this lane's query row of row tile mt;
    //   ws[s][i]:  score weights of this wave's two tiles (gamma^(query - key), 0 above
    //              the diagonal; tiles above the diagonal are never written);
    //   fz[i]:     gamma^(31 - key) for this lane's eight keys of the second key half
    //              (the first half's are these times gamma^32).
    // The two score tiles of wave w are tile_order(w) and tile_order(w + 8).
    int tq[2], tk[2];
#pragma unroll
    for (int s16 = 0; s16 < 2; ++s16) {
        const int code = tile_order(wave + s16 * NW);
        tq[s16] = code >> 2;
        tk[s16] = code & 3;
    }
    float fxi[4], ws[2][4], fz[8];
    const float g32 = GATED ? 0.f : exp2_fast(32.f * lg);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) fxi[mt] = GATED ? 0.f : exp2_fast(static_cast<float>(mt * 16 + l16 + 1) * lg);
#pragma unroll
    for (int s16 = 0; s16 < 2; ++s16)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int dj = (tq[s16] - tk[s16]) * 16 + l16 - 4 * g4 - i;   // query - key
            ws[s16][i] = GATED || dj < 0 ? 0.f : exp2_fast(static_cast<float>(dj) * lg);
        }
#pragma unroll
    for (int i = 0; i < 8; ++i) fz[i] = GATED ? 0.f : exp2_fast(static_cast<float>(31 - 8 * g4 - i) * lg);

    // The registers hold S / 2^lk2: a chunk's decay moves the uniform lk2 instead of
    // rescaling every accumulator; contributions are multiplied by 2^-lk2 and the cross
    // term by 2^lkx (lk2 before the chunk).  Below -64 the registers are rescaled once.
    float lk2 = 0.f;
    f32x4_t X[4];

    // ---- gated: wave 0 forms the chunk-local inclusive prefix of g (times log2 e) for
    // a chunk into gl[stage][0..63] (positions past the chunk end repeat the last sum;
    // REV: walk position m takes g of token N-m, 0 at m = 0)
    float gnext = 0.f;
    auto g_load = [&](int cs) {
        if (GATED && wave == 0) {
            const int lim = t_end - cs;
            if constexpr (REV) {
                const int m = cs + lane;
                gnext = lane < lim && m > 0 ? g_bh[N - m] : 0.f;
            } else {
                gnext = lane < lim ? g_bh[cs + lane] : 0.f;
            }
        }
    };
    auto g_scan = [&](int stage) {
        if (GATED && wave == 0) {
            float incl = gnext * kLog2e;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(incl, off, 64);
                if (lane >= off) incl += y;
            }
            reinterpret_cast<float*>(smem + L_::kG)[stage * kBlk + lane] = incl;
        }
    };

    // ---- tile copies of chunk c into stage b (Q stage: b for two stages, 0 for one)
    auto k_copy = [&](int i, int b, uint32_t row0) {
        kcp.issue_one(i, lds0 + L_::kK + b * L_::kKTile + wofs, k_rs, row0 * qk_rb);
    };
    auto q_copy = [&](int i, int b, uint32_t row0) {
        kcp.issue_one(i, lds0 + L_::kQ + (QS == 2 ? b : 0) * L_::kQTile + wofs, q_rs, row0 * qk_rb);
    };
    auto v_copy = [&](int i, int b, uint32_t row0) {
        vcp.issue_one(i, lds0 + L_::kV + b * L_::kVTile + wofs, v_rs, row0 * v_rb);
    };

    // ---- per head, the state-only prefix walk of a prefix split runs over three stages
    // of K and V, so each prefix chunk's copies go out two chunks ahead (with one stage
    // ahead a state-only step waits out its copies' whole latency).  Stages 0 and 1 are
    // the walk's own; stage 2 takes the Q area (with two Q stages, the second) for K and
    // the output staging area for V, which a state-only step leaves unused.  Prefix chunk
    // p takes stage (p + 2 - npre) mod 3, so the last one is in stage 1 and its step can
    // copy the first full chunk into stage 0 and the Q area.
    constexpr bool P3 = !GATED;
    constexpr uint32_t kP2K = L_::kQ + (QS == 2 ? L_::kQTile : 0);
    static_assert(L_::kQTile == L_::kKTile && L_::kG - L_::kX == L_::kVTile, "third stage must fit the Q and staging areas");
    auto pre_copy = [&](int ps, uint32_t row0) {
        const uint32_t kb = ps == 0 ? L_::kK : ps == 1 ? L_::kK + L_::kKTile : kP2K;
        const uint32_t vb = ps == 0 ? L_::kV : ps == 1 ? L_::kV + L_::kVTile : L_::kX;
#pragma unroll
        for (int i = 0; i < kNQ; ++i) kcp.issue_one(i, lds0 + kb + wofs, k_rs, row0 * qk_rb);
#pragma unroll
        for (int i = 0; i < kNV; ++i) vcp.issue_one(i, lds0 + vb + wofs, v_rs, row0 * v_rb);
    };

    // ---- output staging: a finished block goes to LDS as bf16, row-major [64][128] with
    // the 16-byte units of row r rotated by XOR with r; after the next barrier every lane
    // stores 16-byte units, so each wave writes whole 256-byte rows.
    constexpr int kXU = DVT * 2 / 16;                 // 16-byte units per staged row
    constexpr int kXRounds = kBlk * kXU / (NW * 64);  // units per lane
    u16x8_t xv[kXRounds];
    int xs_row = -1;                                  // first token of the staged block
    auto stage_write = [&]() {
        char* const xs = smem + L_::kX;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int row = mt * 16 + l16;
            const int u = wcol / 8 + (g4 >> 1);
            *reinterpret_cast<u16x4_t*>(xs + row * (DVT * 2) + ((u ^ (row & (kXU - 1))) << 4) + (g4 & 1) * 8) =
                bf4(X[mt]);
        }
    };
    auto stage_load = [&]() {
        const char* const xs = smem + L_::kX;
#pragma unroll
        for (int r = 0; r < kXRounds; ++r) {
            const int e = r * NW * 64 + tid;
            const int row = e / kXU, u = e % kXU;
            xv[r] = *reinterpret_cast<const u16x8_t*>(xs + row * (DVT * 2) + ((u ^ (row & (kXU - 1))) << 4));
        }
    };
    auto stage_emit = [&]() {
        if constexpr (REV) {   // walk row r is token N-1-(xs_row+r)
            bf16_t* const base = reinterpret_cast<bf16_t*>(o) + o_bh + static_cast<size_t>(N - 1 - xs_row) * dv + col0;
#pragma unroll
            for (int r = 0; r < kXRounds; ++r) {
                const int e = r * NW * 64 + tid;
                const int row = e / kXU, u = e % kXU;
                *reinterpret_cast<u16x8_t*>(base + (u * 8 - row * dv)) = xv[r];
            }
        } else {
            bf16_t* const base = reinterpret_cast<bf16_t*>(o) + o_bh + static_cast<size_t>(xs_row) * dv + col0;
#pragma unroll
            for (int r = 0; r < kXRounds; ++r) {
                const int e = r * NW * 64 + tid;
                const int row = e / kXU, u = e % kXU;
                *reinterpret_cast<u16x8_t*>(base + static_cast<uint32_t>(row * dv + u * 8)) = xv[r];
            }
        }
        xs_row = -1;
    };

    // ---- prologue: P tiles above the diagonal are read by P V but never written, so
    // the P area starts zeroed; chunk 0's tiles (and decays) are copied, then the
    // incoming state's loads drain (the compiler does not count the asynchronous copies;
    // a load it still tracked inside the walk would make it wait there for them)
    {
        static_assert(kPBytes == NW * 64 * 16, "one 16-byte unit of P per thread");
        *reinterpret_cast<u16x8_t*>(smem + L_::kP + tid * 16) = u16x8_t{};
        // the first chunk walked: the first prefix chunk (no Q), or the segment's first
        const uint32_t r0 = static_cast<uint32_t>(npre > 0 ? 0 : t_begin);
        if (P3 && npre > 0) {
            // (three-stage prefix) prefix chunks 0 and 1 into their stages
            const int ph = ((2 - npre) % 3 + 3) % 3;
            pre_copy(ph, 0u);
            if (npre > 1) pre_copy((ph + 1) % 3, static_cast<uint32_t>(kBlk));
        } else {
            if (npre == 0) {
#pragma unroll
                for (int i = 0; i < kNQ; ++i) q_copy(i, 0, r0);
            }
#pragma unroll
            for (int i = 0; i < kNQ; ++i) k_copy(i, 0, r0);
#pragma unroll
            for (int i = 0; i < kNV; ++i) v_copy(i, 0, r0);
        }
        g_load(static_cast<int>(r0));
        __builtin_amdgcn_s_waitcnt(0);
        g_scan(0);
    }


    // The state update over the chunk's L keys (full: L = 64), after the caller has
    // added the chunk's decay to lk2.  K^T fragments are read one group of state tiles
    // ahead of the matrix instructions; the group size is GW (0: two tiles for d_k = 256,
    // four for d_k = 128, which leaves room for a full step's other live registers).
    auto state_update = [&](auto gw, uint32_t koff, uint32_t voff, const float* gl, int L, bool full, auto hook) {
        // rescale the registers once the state scale gets small (after the cross term,
        // which reads them at the old scale)
        if (lk2 < -64.f) {
            const float r = exp2_fast(lk2);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) S[dt] *= r;
            lk2 = 0.f;
        }

        // S += K^T (V (.) zeta) over the chunk's keys; slots are keys 32kh + 8g .. +7,
        // gathered by transpose reads of K and V.  The Kt reads of the next G state tiles
        // are issued before the matrix instructions on the current ones; hook(kh, group,
        // groups) runs between the products of each group.
        {
            const float zs = exp2_fast(-lk2);
            const float glast = GATED ? gl[L - 1] : 0.f;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                auto kt_frag = [&](int dt) -> u16x8_t {
                    const int sd = dt >> 1;
                    const uint32_t off = koff + kh * 32 * QRB + (sd / SL) * 256;
                    return cat(lds_tra(akt[0][sd % SL][dt & 1] + off), lds_tra(akt[1][sd % SL][dt & 1] + off));
                };
                constexpr int GW = decltype(gw)::value;
                constexpr int G = GW > 0 ? (GW < DT ? GW : DT) : DT < 4 ? DT : (DT >= 16 ? 2 : 4);
                u16x8_t acur[G], anext[G];
                const u16x8_t raw = cat(lds_tra(avs[0] + voff + kh * 32 * VRB), lds_tra(avs[1] + voff + kh * 32 * VRB));
#pragma unroll
                for (int jj = 0; jj < G; ++jj) acur[jj] = kt_frag(jj);
                __builtin_amdgcn_sched_barrier(0);
                float z[8];
                if constexpr (GATED) {
                    const f32x4_t ga = *reinterpret_cast<const f32x4_t*>(gl + kh * 32 + 8 * g4);
                    const f32x4_t gb = *reinterpret_cast<const f32x4_t*>(gl + kh * 32 + 8 * g4 + 4);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        z[i] = exp2_fast(glast - ga[i] - lk2);
                        z[i + 4] = exp2_fast(glast - gb[i] - lk2);
                    }
                } else if (full) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) z[i] = fz[i] * (kh == 0 ? zs * g32 : zs);
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        z[i] = exp2_fast(static_cast<float>(L - 1 - (kh * 32 + 8 * g4 + i)) * lg - lk2);
                }
                if (!full) {
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        if (kh * 32 + 8 * g4 + i >= L) z[i] = 0.f;
                }
                f32x4_t lo, hi;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    lo[i] = bf16_to_f32(raw[i]) * z[i];
                    hi[i] = bf16_to_f32(raw[i + 4]) * z[i + 4];
                }
                const u16x8_t bv = cat(bf4(lo), bf4(hi));
#pragma unroll
                for (int g0 = 0; g0 < DT; g0 += G) {
                    if (g0 + G < DT) {
#pragma unroll
                        for (int jj = 0; jj < G; ++jj) anext[jj] = kt_frag(g0 + G + jj);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int jj = 0; jj < G; ++jj) S[g0 + jj] = mfma16(acur[jj], bv, S[g0 + jj]);
                    hook(kh, g0 / G, DT / G);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int jj = 0; jj < G; ++jj) acur[jj] = anext[jj];
                }
            }
        }
    };


    // The walk: npre state-only chunks (the first segment of a prefix split, walked by
    // segment 1 for its entry state), then the segment's nck chunks.  Chunk c is staged
    // in stage c % 2; the next chunk's copies go out between the products of the cross
    // term (full steps; with one Q stage its Q copies after the P barrier) or all at once
    // before the state update (state-only steps).
    const int ntot = npre + nck;
    auto chunk_row = [&](int c) -> int { return c < npre ? c * kBlk : t_begin + (c - npre) * kBlk; };

    // ---- row dots: at a chunk's end each wave's partial dots over its 16 columns go to
    // LDS; after the next barrier wave 7 sums each row's eight partials into dG (the last
    // chunk's after the walk).  The second tensor's elements of a lane are loaded at the
    // top of the chunk.
    u16x4_t xdl[DOT ? 4 : 1];
    int dot_row = -1, dot_len = 0, dot_st = 0;   // the chunk whose partials wait in LDS
    float dg_prev = 0.f;   // wave 7, accumulating: dG of row `lane` of the chunk, loaded early
    auto dot_load = [&](int cs, int L) {
        if (wave == NW - 1 && ka.dacc && lane < L) dg_prev = dG_bh[REV ? N - 1 - (cs + lane) : cs + lane];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int row = mt * 16 + l16;
            const int tok = REV ? N - 1 - (cs + row) : cs + row;
            xdl[mt] = row < L ? *reinterpret_cast<const u16x4_t*>(xd_bh + static_cast<size_t>(tok) * dv + col0 + wcol +
                                                                    4 * g4)
                              : u16x4_t{0, 0, 0, 0};
        }
    };
    auto dot_part = [&](int st) {
        float part[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            part[mt] = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) part[mt] += X[mt][i] * bf16_to_f32(xdl[mt][i]);
            part[mt] += __shfl_xor(part[mt], 16, 64);
            part[mt] += __shfl_xor(part[mt], 32, 64);
        }
        if (g4 == 0) {
            float* const dp = reinterpret_cast<float*>(smem + L_::kD + st * L_::kDStage);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) dp[(mt * 16 + l16) * NW + wave] = part[mt];
        }
    };
    // ---- norm-gate: at a chunk's end the fp32 rows go to LDS (16-byte units XOR-rotated
    // by the row) with each wave's partial sums of squares; after the next barrier every
    // lane takes four 16-byte units, sums its row's eight partials and stores
    // silu(gate) * x / rms as bf16.  Gate values are loaded at the top of their chunk.
    constexpr int kNGU = DVT / 4;                          // 16-byte fp32 units per row
    constexpr int kNGRounds = kBlk * kNGU / (NW * 64);
    u16x4_t ngg[NG ? kNGRounds : 1];
    int ng_row = -1, ng_len = 0;
    auto ng_load = [&](int cs, int L) {
#pragma unroll
        for (int r = 0; r < kNGRounds; ++r) {
            const int e = r * NW * 64 + tid, row = e / kNGU, u = e % kNGU;
            ngg[r] = row < L ? *reinterpret_cast<const u16x4_t*>(ka.ng_gate + ng_off(cs + row) + col0 + 4 * u)
                             : u16x4_t{0, 0, 0, 0};
        }
    };
    auto ng_stage = [&]() {
        float* const xf = reinterpret_cast<float*>(smem + L_::kXF);
        float* const dp = reinterpret_cast<float*>(smem + L_::kD);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int row = mt * 16 + l16, u = wcol / 4 + g4;
            *reinterpret_cast<f32x4_t*>(xf + row * DVT + 4 * (u ^ (row & 15))) = X[mt];
            float part = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) part += X[mt][i] * X[mt][i];
            part += __shfl_xor(part, 16, 64);
            part += __shfl_xor(part, 32, 64);
            if (g4 == 0) dp[row * NW + wave] = part;
        }
    };
    auto ng_emit = [&]() {
        if (ng_row < 0) return;
        const float* const xf = reinterpret_cast<const float*>(smem + L_::kXF);
        const float* const dp = reinterpret_cast<const float*>(smem + L_::kD);
#pragma unroll
        for (int r = 0; r < kNGRounds; ++r) {
            const int e = r * NW * 64 + tid, row = e / kNGU, u = e % kNGU;
            if (row >= ng_len) continue;
            const f32x4_t x = *reinterpret_cast<const f32x4_t*>(xf + row * DVT + 4 * (u ^ (row & 15)));
            const f32x4_t a = *reinterpret_cast<const f32x4_t*>(dp + row * NW);
            const f32x4_t b = *reinterpret_cast<const f32x4_t*>(dp + row * NW + 4);
            const float ss = ((a[0] + a[1]) + (a[2] + a[3])) + ((b[0] + b[1]) + (b[2] + b[3]));
            // hardware reciprocal square root, exponential and reciprocal (about 1 ulp each,
            // far below the bf16 rounding of z)
            const float inv = __builtin_amdgcn_rsqf(ss * (1.f / static_cast<float>(DVT)) + ka.ng_eps);
            f32x4_t y;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float g = bf16_to_f32(ngg[r][i]);
                y[i] = g * __builtin_amdgcn_rcpf(1.f + exp2_fast(-g * kLog2e)) * x[i] * inv;
            }
            *reinterpret_cast<u16x4_t*>(ka.ng_out + ng_off(ng_row + row) + col0 + 4 * u) = bf4(y);
        }
        ng_row = -1;
    };
    auto dot_flush = [&]() {
        if (wave == NW - 1 && dot_row >= 0 && lane < dot_len) {
            const float* const dp = reinterpret_cast<const float*>(smem + L_::kD + dot_st * L_::kDStage) + lane * NW;
            const f32x4_t a = *reinterpret_cast<const f32x4_t*>(dp), b = *reinterpret_cast<const f32x4_t*>(dp + 4);
            const float sum = ((a[0] + a[1]) + (a[2] + a[3])) + ((b[0] + b[1]) + (b[2] + b[3]));
            float* const dst = dG_bh + (REV ? N - 1 - (dot_row + lane) : dot_row + lane);
            *dst = (ka.dacc ? dg_prev : 0.f) + ka.dsign * sum;
        }
        dot_row = -1;
    };
    constexpr int kOps = 2 * kNQ + kNV;                        // K, V, then Q copies
    constexpr int kCrossOps = QS == 2 ? kOps : kNQ + kNV;      // those issued in the cross term
    // Returns false past the last chunk.
    auto step = [&](auto stage_c, int c) -> bool {
        constexpr int ST = decltype(stage_c)::value;
        constexpr int QB = QS == 2 ? ST : 0;
        const bool sonly = !P3 && c < npre;   // the state update alone (two-stage prefix)
        const int cs = chunk_row(c);
        const int L = min(kBlk, t_end - cs);    // (prefix chunks are whole)
        const bool full = L == kBlk;
        const bool has_next = c + 1 < ntot;
        const bool next_q = c + 1 >= npre;      // the next chunk is a full step: copy its Q
        // uniform; readfirstlane keeps it (and every copy offset made from it) scalar
        const uint32_t next_row = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(chunk_row(c + 1)));
        constexpr uint32_t qoff = QB * L_::kQTile, koff = ST * L_::kKTile, voff = ST * L_::kVTile;
        const float* const gl = reinterpret_cast<const float*>(smem + L_::kG) + ST * kBlk;
        // copy op i of the next chunk (every index is tested by the callers' unrolled
        // loops, so each copy's offset register is a constant)
        auto copy_op = [&](int i) {
            if (i < kNQ) k_copy(i, 1 - ST, next_row);
            else if (i < kNQ + kNV) v_copy(i - kNQ, 1 - ST, next_row);
            else if (next_q) q_copy(i - kNQ - kNV, 1 - ST, next_row);
        };
        // ops [lo, hi) spread over nslots slots: those of slot `slot`
        auto copy_slice = [&](int lo, int hi, int slot, int nslots) {
#pragma unroll
            for (int i = 0; i < kOps; ++i)
                if (i >= lo + slot * (hi - lo) / nslots && i < lo + (slot + 1) * (hi - lo) / nslots) copy_op(i);
        };

        // this chunk's tiles (and prefix sums) have landed and are visible to every wave
        __builtin_amdgcn_s_waitcnt(0);
        lds_barrier();
        if (!OF32 && xs_row >= 0) {
            stage_load();
            stage_emit();
        }
        if constexpr (DOT) {
            dot_flush();
            if (!sonly) dot_load(cs, L);
        }
        if constexpr (NG) {
            ng_emit();
            if (!sonly) ng_load(cs, L);
        }
        if (has_next) g_load(static_cast<int>(next_row));

        // decays of this chunk
        float gj[4] = {0.f, 0.f, 0.f, 0.f};   // gated: G of this lane's query rows
        float l2chunk;
        if constexpr (GATED) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) gj[mt] = gl[mt * 16 + l16];
            l2chunk = gl[L - 1];
        } else {
            l2chunk = static_cast<float>(L) * lg;
        }
        const float lkx = lk2;
        lk2 += l2chunk;

        if (!sonly) {
            // cross term X^T = S^T Q^T over the chunk's 64 query rows
            {
                u16x8_t qa[4], qn[4];
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) qa[mt] = lds16a(aq[0] + qoff + mt * 16 * QRB);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    if (ks + 1 < KS) {
#pragma unroll
                        for (int mt = 0; mt < 4; ++mt)
                            qn[mt] = lds16a(aq[(ks + 1) % KL] + qoff + mt * 16 * QRB + ((ks + 1) / KL) * 256);
                    }
                    const u16x4_t a0 = bf4(S[2 * ks]), a1 = bf4(S[2 * ks + 1]);
                    const u16x8_t b = (g4 & 1) ? cat(a1, a0) : cat(a0, a1);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt)
                        X[mt] = mfma16(b, qa[mt], ks == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : X[mt]);
                    if constexpr (HILO) {
                        // fp32 results: the state operand also as a second bf16 term (its
                        // rounding residual), so the cross term carries ~16 mantissa bits of S
                        f32x4_t r0, r1;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            r0[i] = S[2 * ks][i] - bf16_to_f32(a0[i]);
                            r1[i] = S[2 * ks + 1][i] - bf16_to_f32(a1[i]);
                        }
                        const u16x4_t c0 = bf4(r0), c1 = bf4(r1);
                        const u16x8_t bl = (g4 & 1) ? cat(c1, c0) : cat(c0, c1);
#pragma unroll
                        for (int mt = 0; mt < 4; ++mt) X[mt] = mfma16(bl, qa[mt], X[mt]);
                    }
                    if (has_next) copy_slice(0, kCrossOps, ks, KS);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) qa[mt] = qn[mt];
                }
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const float xi = GATED ? exp2_fast(gj[mt] + lkx) : fxi[mt] * exp2_fast(lkx);
#pragma unroll
                    for (int i = 0; i < 4; ++i) X[mt][i] *= xi;
                }
            }

            // this wave's score tiles (K Q^T), decayed and rounded to bf16, into the P area
#pragma unroll
            for (int s16 = 0; s16 < 2; ++s16) {
                const int qt = tq[s16], kt = tk[s16];
                if (kt > qt) continue;   // above the diagonal: never written, stays zero
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
                u16x8_t kf[KS], qf[KS];
#pragma unroll
                for (int ks = 0; ks < KS && ks < 2; ++ks) {
                    kf[ks] = lds16a(ak[ks % KL] + koff + kt * 16 * QRB + (ks / KL) * 256);
                    qf[ks] = lds16a(aq[ks % KL] + qoff + qt * 16 * QRB + (ks / KL) * 256);
                }
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    if (ks + 2 < KS) {
                        kf[ks + 2] = lds16a(ak[(ks + 2) % KL] + koff + kt * 16 * QRB + ((ks + 2) / KL) * 256);
                        qf[ks + 2] = lds16a(aq[(ks + 2) % KL] + qoff + qt * 16 * QRB + ((ks + 2) / KL) * 256);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    acc = mfma16(kf[ks], qf[ks], acc);
                    __builtin_amdgcn_sched_barrier(0);
                }
                const int j = qt * 16 + l16;   // query row (chunk-local)
                float w[4];
                if constexpr (GATED) {
                    const f32x4_t gk = *reinterpret_cast<const f32x4_t*>(gl + kt * 16 + 4 * g4);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        w[i] = kt == qt && 4 * g4 + i > l16 ? 0.f : exp2_fast(gj[qt] - gk[i]);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) w[i] = ws[s16][i];
                }
                if (!full) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (kt * 16 + 4 * g4 + i >= L || j >= L) w[i] = 0.f;
                }
                const u16x4_t p = bf4(f32x4_t{acc[0] * w[0], acc[1] * w[1], acc[2] * w[2], acc[3] * w[3]});
                *reinterpret_cast<u16x4_t*>(smem + L_::kP + ((qt * 2 + (kt >> 1)) * 64 + lane) * 16 + (kt & 1) * 8) = p;
            }
            // every wave is past its Q reads and P is complete
            lds_barrier();

        }

        // the state update.  A state-only step is short and its next chunk's copies set
        // its pace (their latency, not its arithmetic: measured), so it issues all of them
        // before its products; a full step with one Q stage issues the Q copies between
        // the products.
        if (sonly && has_next) copy_slice(0, kOps, 0, 1);
        state_update(std::integral_constant<int, 0>{}, koff, voff, gl, L, full, [&](int kh, int gi, int ng) {
            if (!has_next) return;
            if (!sonly && QS == 1 && kh == 0) copy_slice(kCrossOps, kOps, gi, ng);
        });
        if (sonly) {
            if (has_next) g_scan(1 - ST);
            return has_next;
        }

        // X += P V over the chunk's 64 keys (as X^T += V^T P^T); V fragments by transpose
        // reads: slots {4g..4g+3} of key tile 2ks and of key tile 2ks+1
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const u16x8_t bv = cat(lds_tra(avp + voff + ks * 32 * VRB), lds_tra(avp + voff + (ks * 32 + 16) * VRB));
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                if (2 * ks > mt) continue;   // key tiles above row tile mt are zero
                const u16x8_t a = lds16a(ap + (mt * 2 + ks) * 1024);
                X[mt] = mfma16(bv, a, X[mt]);
            }
        }

        // gated: wave 0 forms the next chunk's prefix sums (its decays were loaded at the
        // top of the step; the next barrier publishes them)
        if (has_next) g_scan(1 - ST);

        if constexpr (DOT) {
            dot_part(ST);
            dot_row = cs;
            dot_len = L;
            dot_st = ST;
        }

        // the output block: bf16, staged when more chunks follow (stored after the next
        // barrier); else (and fp32) stored from the accumulators, rows past the chunk end
        // skipped (REV: walk row r of the chunk is token N-1-(cs+r))
        if (NG) {
            ng_stage();
            ng_row = cs;
            ng_len = L;
        } else if (!OF32 && full && has_next) {
            stage_write();
            xs_row = cs;
        } else {
            out_t* const base = o + o_bh + static_cast<size_t>(REV ? N - 1 - cs : cs) * dv + col0 + wcol + 4 * g4;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int row = mt * 16 + l16;
                if (row >= L) continue;
                out_t* const dst = REV ? base - static_cast<ptrdiff_t>(row) * dv : base + static_cast<uint32_t>(row * dv);
                if constexpr (OF32) *reinterpret_cast<f32x4_t*>(dst) = X[mt];
                else *reinterpret_cast<u16x4_t*>(dst) = bf4(X[mt]);
            }
        }
        return has_next;
    };

    // ---- (three-stage prefix) the state-only walk; the main walk then starts at chunk
    // npre in stage 0
    if constexpr (P3) {
        if (npre > 0) {
            // K^T read bases moved by d (stage 2 lies below them; an immediate cannot be
            // negative)
            auto kt_shift = [&](uint32_t d) {
#pragma unroll
                for (int pl = 0; pl < 2; ++pl)
#pragma unroll
                    for (int sl = 0; sl < SL; ++sl)
#pragma unroll
                        for (int hb = 0; hb < 2; ++hb) akt[pl][sl][hb] = opaque(akt[pl][sl][hb] + d);
            };
            constexpr int kPreOps = kNQ + kNV;   // one prefix chunk's copies per wave
            auto pstep = [&](auto ps_c, int p) {
                constexpr int PS = decltype(ps_c)::value;
                // chunk p has landed (chunk p+1's copies may still be in flight)
                if (p + 1 < npre) wait_vmcnt<kPreOps>();
                else wait_vmcnt<0>();
                lds_barrier();
                // every wave is past chunk p-1: its stage takes chunk p+2; the last step
                // copies the first full chunk into stage 0 and the Q area
                if (p + 2 < npre) {
                    pre_copy((PS + 2) % 3, static_cast<uint32_t>(__builtin_amdgcn_readfirstlane((p + 2) * kBlk)));
                } else if (p + 1 == npre && nck > 0) {
                    const uint32_t row = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(t_begin));
#pragma unroll
                    for (int i = 0; i < kNQ; ++i) k_copy(i, 0, row);
#pragma unroll
                    for (int i = 0; i < kNV; ++i) v_copy(i, 0, row);
#pragma unroll
                    for (int i = 0; i < kNQ; ++i) q_copy(i, 0, row);
                }
                lk2 += static_cast<float>(kBlk) * lg;
                constexpr uint32_t koff = PS == 1 ? L_::kKTile : 0;
                constexpr uint32_t voff = PS == 0 ? 0 : PS == 1 ? L_::kVTile : L_::kX - L_::kV;
                if constexpr (PS == 2) kt_shift(kP2K - L_::kK);
                // (the cross term's registers are free: K^T reads go 4 (d_k = 256) or 8 state tiles ahead)
                state_update(std::integral_constant<int, DK == 256 ? 4 : 8>{}, koff, voff, nullptr, kBlk, true, [](int, int, int) {});
                if constexpr (PS == 2) kt_shift(L_::kK - kP2K);
            };
            // the steps before the first one in stage 0 are peeled (a jump into the loop
            // would make the flow graph irreducible, which costs registers)
            int p = 0;
            const int ph = ((2 - npre) % 3 + 3) % 3;   // stage of prefix chunk 0
            if (ph == 1) {
                pstep(std::integral_constant<int, 1>{}, p++);
                if (p < npre) pstep(std::integral_constant<int, 2>{}, p++);
            } else if (ph == 2) {
                pstep(std::integral_constant<int, 2>{}, p++);
            }
            while (p < npre) {
                pstep(std::integral_constant<int, 0>{}, p);
                if (++p == npre) break;
                pstep(std::integral_constant<int, 1>{}, p);
                if (++p == npre) break;
                pstep(std::integral_constant<int, 2>{}, p);
                ++p;
            }
        }
    }
    const int c0 = P3 ? npre : 0;
    if (c0 < ntot) {
        for (int c = c0;; c += 2) {
            if (!step(std::integral_constant<int, 0>{}, c)) break;
            if (!step(std::integral_constant<int, 1>{}, c + 1)) break;
        }
    }
    if constexpr (DOT) {
        if (dot_row >= 0) {
            lds_barrier();
            dot_flush();
        }
    }
    if constexpr (NG) {
        if (ng_row >= 0) {
            lds_barrier();
            ng_emit();
        }
    }

    // ---- final state (last segment only), through LDS in whole rows of 16-byte stores
    if (seg == nseg - 1 && ka.state_out != nullptr) {
        float* const st = reinterpret_cast<float*>(smem);
        // REV: the final state leaves multiplied by the decay of token 0
        float lout = lk2;
        if constexpr (REV) lout += GATED ? g_bh[0] * kLog2e : lg;
        const float r = exp2_fast(lout);
        __builtin_amdgcn_s_waitcnt(0);
        lds_barrier();   // every wave is done with the tile buffers
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) st[srow(dt, i) * DVT + wcol + l16] = S[dt][i] * r;
        lds_barrier();
        constexpr int kU = DVT / 4;                        // 16-byte units per row
        constexpr int kRounds = DK * kU / (NW * 64);
        static_assert(kRounds * NW * 64 == DK * kU, "state rows must split evenly");
        float* const dst = ka.state_out + s_bh;
#pragma unroll
        for (int rr = 0; rr < kRounds; ++rr) {
            const int e = rr * NW * 64 + tid;
            const int row = e / kU, u = e % kU;
            *reinterpret_cast<f32x4_t*>(dst + static_cast<size_t>(row) * dv + col0 + u * 4) =
                *reinterpret_cast<const f32x4_t*>(st + row * DVT + u * 4);
        }
    }
}

template <int DK, bool GATED, bool REV, int OUT>
hipError_t launch_c1(const KArgs& ka, hipStream_t stream) {
    constexpr size_t lds = C1Lds<DK, GATED, OUT == kOutDot, OUT == kOutNormGate>::kBytes;
    static std::once_flag attr_once;   // thread-safe one-time init of the LDS limit
    std::call_once(attr_once, [] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk1_kernel<DK, GATED, REV, OUT>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    });
    ProfScope prof(kProfMain, stream);
    hipLaunchKernelGGL((chunk1_kernel<DK, GATED, REV, OUT>), dim3(ka.total_groups), dim3(kC1Waves * 64), lds,
                       stream, ka);
    return hipGetLastError();
}

template <int DK, bool GATED, int OUT>
hipError_t launch_c1_dir(const KArgs& ka, bool reverse, hipStream_t stream) {
    return reverse ? launch_c1<DK, GATED, true, OUT>(ka, stream) : launch_c1<DK, GATED, false, OUT>(ka, stream);
}

template <int DK>
hipError_t launch_c1_dk(const KArgs& ka, bool gated, bool reverse, int out, hipStream_t stream) {
    if (gated) {
        if (out == kOutF32) return launch_c1_dir<DK, true, kOutF32>(ka, reverse, stream);
        if (out == kOutDot) {
            if constexpr (DK == 128) return launch_c1_dir<DK, true, kOutDot>(ka, reverse, stream);
            return hipErrorInvalidValue;
        }
        if (out == kOutNormGate) {
            if constexpr (DK == 128) {
                if (!reverse) return launch_c1<DK, true, false, kOutNormGate>(ka, stream);
            }
            return hipErrorInvalidValue;
        }
        return launch_c1_dir<DK, true, kOutBf16>(ka, reverse, stream);
    }
    if (out != kOutBf16) return hipErrorInvalidValue;
    return launch_c1_dir<DK, false, kOutBf16>(ka, reverse, stream);
}

}  // namespace

bool chunk1_supported(int dk, int dv, int chunk, int ldqk, int ldv, int slices, bool out_f32, bool gated) {
    // copies move 16-byte units, so row strides are multiples of 8 elements
    return chunk == kBlk && (dk == 128 || dk == 256) && dv % kC1Cols == 0 && ldqk >= dk && ldv >= dv &&
           ldqk % 8 == 0 && ldv % 8 == 0 && slices >= 1 && (!out_f32 || gated);
}

bool chunk1_dot_supported(int dk, int dv, int chunk) { return chunk == kBlk && dk == 128 && dv == kC1Cols; }

hipError_t launch_chunk1(const KArgs& ka, bool gated, bool reverse, bool out_f32, bool dot, hipStream_t stream) {
    const bool ng = ka.ng_gate != nullptr;
    if ((dot || ng) && (out_f32 || (dot && ng) || !gated || !chunk1_dot_supported(ka.dk, ka.dv, kBlk) ||
                        ka.nsl > 1 || ka.ndvt != 1 || (ng && reverse)))
        return hipErrorInvalidValue;
    const int out = dot ? kOutDot : ng ? kOutNormGate : out_f32 ? kOutF32 : kOutBf16;
    if (ka.dk == 256) return launch_c1_dk<256>(ka, gated, reverse, out, stream);
    if (ka.dk == 128) return launch_c1_dk<128>(ka, gated, reverse, out, stream);
    return hipErrorInvalidValue;
}

}  // namespace retn
