// bf16 chunkwise retention forward on the gfx950 matrix cores.
//
// Method ("RetNet retention mechanism" tutorial, section 块级循环, with the per-row
// cross-chunk decay; gated decays from the pwwt.cn guide, section Triton 内核与自校验测试).
// For a chunk of L tokens with chunk-local log2 decays G (G_j = log2 of the product of
// the decays of positions 0..j):
//     O     = (Q K^T (.) D) V + diag(2^G) (Q S_prev),      D_jl = 2^(G_j - G_l), j >= l
//     S_new = 2^(G_{L-1}) S_prev + K^T (V (.) zeta),        zeta_l = 2^(G_{L-1} - G_l)
// Per head, G_j = (j+1) log2(gamma); gated, G is the inclusive prefix sum of g*log2(e).
//
// Work decomposition.  A workgroup owns one (b,h), one segment of the sequence and
// DVT state columns; it walks the segment's chunks in order, holding its DK x DVT slice
// of S in fp32 MFMA accumulators spread over its waves (NT 16-column tiles each).  A
// chunk is processed in 64-token blocks: for query block qb the scores against key
// blocks kb <= qb are formed, decayed, rounded to bf16 and multiplied with V; the
// state contribution of block qb is accumulated once the chunk's old state has been
// used by every query block.
//
// Matrix-core layout (v_mfma_f32_16x16x32_bf16): lane l supplies row l%16 of A and
// column l%16 of B, each with 8 reduction slots in group l/16; the result row
// 4*(l/16)+i, column l%16 sits in accumulator element i.  Only the pairing of slots
// between A and B matters, so each product picks the slot->index map that lets its
// operands come straight from registers:
//   * scores are computed transposed (K Q^T): a lane then holds P[query l%16][4 keys],
//     which is the A operand of P V when slots map to keys {4g..4g+3, 16+4g..16+4g+3};
//   * the state accumulators hold S[4 rows][column l%16], which is the B operand of
//     Q S when slots map to state rows the same way.
// Q, K and V blocks are copied token-major into LDS by asynchronous global->LDS loads,
// one block ahead of use.  Operands that need tokens as the reduction slots (V for
// P V, K^T and V for the state update) are gathered with LDS transpose reads.  Rows
// are XOR-swizzled in 16-byte units so that every fragment read is free of bank
// conflicts.
//
// Long sequences with few (b,h) are split into segments so that the grid fills the
// chip: a pre-pass computes each segment's local final state (the same state
// recurrence from a zero state), a scan composes them into every segment's incoming
// state, and the main pass starts each segment from that state.  This is the
// single-device form of the hierarchical chunking the pwwt.cn guide describes
// (section Triton 内核与自校验测试).

#include "cdna4.h"
#include "chunk_tiles.h"
#include "common.h"
#include "launch.h"

#include <mutex>
#include <type_traits>

namespace retn {

namespace {

constexpr int kTargetGroups = 256;
// Up to this many segments the main pass composes its entry state from the local
// segment states itself (segment s reads s of them); beyond, a scan kernel does it.
// (Measured: 8 saves the scan launch on the gated workload, 7 us of 117; with 16
// segments the longest composition costs as much as the scan.)
constexpr int kFuseScanMax = 8;
// Time of a state-only step (the state update of one 64-token chunk) relative to a full
// step of the single-block main pass, for the prefix split of two segments.
constexpr double kPrefixCost = 0.5;

// LDS layout: QS stages of Q (full pass only), NST stages of K and V blocks and of the
// decays the block's step loads (gated: the pre-pass copies its block's 64 decays once
// per wave, the full pass the chunk's decays at a chunk start), the P fragments of the
// current block pair, optionally (XST) a staging area for one 64-row output block, and
// (gated) the chunk's log2 decays.  When the buffers leave no room for P (kPInK), P is
// written into the current K buffer once every wave is done with K.
template <int DK, int DVT, bool GATED, bool HASQ, int NST, int NW, int QS = NST, bool XST = false, int XE = 2>
struct Lds {
    static constexpr int kQRow = DK * 2, kVRow = DVT * 2;
    static constexpr int kQTile = kBlk * kQRow, kKTile = kBlk * kQRow, kVTile = kBlk * kVRow;
    static constexpr int kQ = 0;                          // QS buffers (none without Q)
    static constexpr int kK = kQ + (HASQ ? QS * kQTile : 0);   // NST buffers
    static constexpr int kV = kK + NST * kKTile;          // NST buffers
    static constexpr int kGdStage = !GATED ? 0 : (HASQ ? (NST == 3 ? kMaxChunk * 4 : 0) : NW * 256);
    static constexpr int kGd = kV + NST * kVTile;         // NST stages of decays
    static constexpr int kEnd = kGd + NST * kGdStage;
    static constexpr int kGBytes = GATED ? kMaxChunk * 4 : 0;
    static constexpr int kXBytes = HASQ && XST ? kBlk * DVT * XE : 0;   // XE bytes per staged element
    static constexpr bool kPInK = HASQ && kEnd + kPBytes + kXBytes + kGBytes > kLdsBytes;
    static constexpr int kPSize = HASQ && !kPInK ? kPBytes : 0;
    static constexpr int kP = kPInK ? 0 : kEnd;           // unused when kPInK
    static constexpr int kX = kEnd + kPSize;
    static constexpr int kG = kX + kXBytes;
    static constexpr int kBytes = kG + kGBytes;
};

enum Mode { kFull = 0, kStateOnly = 1 };
// Pipeline stages: the pre-pass keeps four blocks in flight.  The full pass
// double-buffers: a third stage (which fits for d_k <= 128) measured 4-8% slower on
// every such workload -- their loads are bandwidth-, not latency-limited.
template <int DK, int DVT, bool GATED, int MODE, int NW>
constexpr int stages_for() {
    if (MODE == kFull) return 2;
    return Lds<DK, DVT, GATED, false, 4, NW>::kBytes <= kLdsBytes ? 4
         : Lds<DK, DVT, GATED, false, 3, NW>::kBytes <= kLdsBytes ? 3 : 2;
}

// Layout of the full pass with two stages: each finished output block is staged in LDS
// so that it leaves in whole 128-byte lines (one wave alone owns 32 bytes of a row).
// Q keeps two stages when that fits; otherwise single-block chunks keep one Q stage,
// refilled once every wave is past the scores.  Other shapes store from registers.
template <int DK, int DVT, bool GATED, int MODE, int NW, bool ONEBLK, bool OF32 = false>
struct Plan {
    static constexpr int NST = stages_for<DK, DVT, GATED, MODE, NW>();
    static constexpr bool kFull2 = MODE == kFull && NST == 2;
    using L2 = Lds<DK, DVT, GATED, MODE == kFull, NST, NW, NST, true, OF32 ? 4 : 2>;
    using L1 = Lds<DK, DVT, GATED, MODE == kFull, NST, NW, 1, true, OF32 ? 4 : 2>;
    static constexpr bool kQ2 = kFull2 && !L2::kPInK && L2::kBytes <= kLdsBytes;
    static constexpr bool kQ1 = kFull2 && !kQ2 && ONEBLK && !L1::kPInK && L1::kBytes <= kLdsBytes;
    static constexpr bool kStage = kQ2 || kQ1;
    static constexpr int QS = kQ1 ? 1 : NST;
    using L = std::conditional_t<kQ1, L1, std::conditional_t<kQ2, L2, Lds<DK, DVT, GATED, MODE == kFull, NST, NW>>>;
};

// Position in the walk over a segment: chunk start cs, query block qb, key block kb.
struct Step {
    int cs, qb, kb;
};

// Advance to the next (chunk, query block, key block); false past the segment end.
// The full pass visits key blocks 0..qb for each query block; the state pre-pass only
// the diagonal one.
template <int MODE>
__device__ __forceinline__ bool next_step(Step& s, int t_end, int C) {
    const int L = min(C, t_end - s.cs);
    const int nb = (L + kBlk - 1) / kBlk;
    if (MODE == kFull && s.kb < s.qb) { ++s.kb; return true; }
    if (s.qb + 1 < nb) { ++s.qb; s.kb = MODE == kFull ? 0 : s.qb; return true; }
    s.cs += C;
    s.qb = 0;
    s.kb = 0;
    return s.cs < t_end;
}

// Main kernel (MODE = kFull) and segment-state pre-pass (MODE = kStateOnly).
//   Main pass: state rows = all dk (DK == dk); a workgroup per (b,h), segment, column
//   tile.  Its incoming state is state_in (one segment), the scanned entry state in
//   seg_state, or (fuse_scan) composed here from the local states of the earlier
//   segments.
//   Pre-pass: a workgroup per (b,h), segment 0..nseg-2, DK-row tile, column tile; it
//   writes the segment's local final state (zero start) and its total log2 decay.
// ONEBLK: every chunk is a single block (chunk <= 64), so each step starts a chunk and
// the cross term can read the old state straight from the accumulators; no bf16
// snapshot of the state is kept, which frees registers for wider column tiles.
// REV: the walk runs over the time-reversed sequence (the adjoint recurrence of the
// backward pass).  Walk position m reads and writes token N-1-m; its decay is that of
// token N-m (gated: g[N-m], and 0 at m = 0); per head, state_in enters divided by gamma
// (so the first step adds to it undecayed) and state_out leaves multiplied by the
// decay of token 0.
// The LDS footprint allows one workgroup per CU, i.e. NW/4 waves per SIMD; saying so
// lets the compiler spend registers on keeping LDS reads in flight ahead of the matrix
// instructions instead of minimising registers for an occupancy that cannot happen.
// PAR (parallel form, MODE = kFull, no state): the whole sequence is one chunk and each
// workgroup owns one query block, so O = (Q K^T (.) D) V with no cross term and no state;
// the query blocks of a (b,h) run in parallel.  nseg then holds the number of query
// blocks.
template <int DK, int DVT, int NW, bool GATED, int MODE, bool ONEBLK, bool OF32, bool REV, bool PAR>
__global__ __launch_bounds__(NW * 64, 1) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void chunk_kernel(
    const KArgs ka) {
    const bf16_t* __restrict__ q = ka.q;
    const bf16_t* __restrict__ k = ka.k;
    const bf16_t* __restrict__ v = ka.v;
    const float* __restrict__ decay = ka.decay;
    // output elements: bf16, or fp32 (OF32, for callers that keep full precision)
    typedef std::conditional_t<OF32, float, bf16_t> out_t;
    out_t* __restrict__ o = static_cast<out_t*>(ka.o);
    const int H = ka.H, N = ka.N, dv = ka.dv, C = ka.C, dk = ka.dk;
    const int seg_tokens = ka.seg_tokens, nseg = ka.nseg, ndvt = ka.ndvt, ndkt = ka.ndkt;
    const int total_groups = ka.total_groups;
    using PL = Plan<DK, DVT, GATED, MODE, NW, ONEBLK, OF32>;
    constexpr int NST = PL::NST;
    using L_ = typename PL::L;
    static_assert(L_::kBytes <= kLdsBytes, "LDS layout too large");
    constexpr bool kStage = PL::kStage;   // output blocks leave through the LDS staging area
    constexpr bool kQ1 = PL::kQ1;         // one Q stage, refilled after the P barrier
    // The pre-pass splits each 64-token block between two halves of the waves (keys
    // 0..31 and 32..63): each wave then owns twice the columns, which halves the K^T
    // reads per matrix instruction; the two partial states are summed at the end.
    constexpr bool SPLITK = MODE == kStateOnly && NW >= 2;
    constexpr int NWC = SPLITK ? NW / 2 : NW;     // waves across the columns
    constexpr int NT = DVT / (16 * NWC);          // 16-column tiles per wave
    static_assert(NT >= 1 && NT * 16 * NWC == DVT && 16 % NW == 0, "bad wave split");
    constexpr int DT = DK / 16;           // 16-row tiles of the state
    constexpr int KS = DK / 32;           // reduction steps over DK
    constexpr int QRB = L_::kQRow, VRB = L_::kVRow;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    char* const Pfix = smem + L_::kP;
    float* const gl = reinterpret_cast<float*>(smem + L_::kG);

    // ---- work item: XCD-aware order (consecutive launch ids rotate over the 8 XCDs;
    // give each XCD a contiguous range of work so a (b,h)'s column tiles share an L2).
    int wid = blockIdx.x;
    if (total_groups % 8 == 0) wid = (wid & 7) * (total_groups >> 3) + (wid >> 3);
    const int nseg_grid = MODE == kFull ? nseg : nseg - 1;   // the last segment's state is not needed
    const int dvt = wid % ndvt;
    const int dkt = (wid / ndvt) % ndkt;
    // PAR: seg is the query block, the longest ones of a (b,h) first
    const int seg = PAR ? nseg - 1 - (wid / (ndvt * ndkt)) % nseg : (wid / (ndvt * ndkt)) % nseg_grid;
    const int ch = wid / (ndvt * ndkt * nseg_grid);    // chain: (b,h) and column slice
    const int nsl = ka.nsl > 1 ? ka.nsl : 1;
    const int slc = ch % nsl;
    const int bh = ch / nsl;
    const int h = bh % H;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int col0 = dvt * DVT;                         // first column of this tile
    const int cwave = SPLITK ? wave % NWC : wave;       // column position of this wave
    const int khalf = SPLITK ? wave / NWC : 0;         // pre-pass: the block half it sums
    const int wcol = cwave * 16 * NT;                   // wave's first column in the tile
    // transpose-read source coordinates of this lane within its 16-lane group
    const int trj = l16 >> 2, trq = l16 & 3;

    const int t_begin = PAR ? 0 : seg * seg_tokens;
    const int t_end = PAR ? N : min(N, t_begin + seg_tokens);
    const float lg = GATED ? 0.f : log2f(decay[h]);

    // q, k rows have dk elements; this workgroup's K tile covers dims dkt*DK .. +DK
    const int ldqk = ka.ldqk, ldv = ka.ldv;
    const size_t qk_bh = static_cast<size_t>(bh) * N * ldqk + static_cast<size_t>(slc) * ka.sl_qk;
    const size_t v_bh = static_cast<size_t>(bh) * N * ldv;
    const size_t o_bh = static_cast<size_t>(bh) * N * dv + slc * ka.sl_o;
    const size_t s_bh = static_cast<size_t>(bh) * dk * dv + slc * ka.sl_state;
    const size_t s_stride_seg = static_cast<size_t>(dk) * dv;
    const int srow0 = dkt * DK;                          // first state row of this tile
    const float* g_bh = GATED ? decay + static_cast<size_t>(bh) * N : nullptr;
    const u32x4_t g_rs = make_rsrc(GATED ? g_bh : decay, GATED ? static_cast<uint32_t>(N) * 4 : 4);
    // ranges end with the last row's own columns; rows past N read as zeros
    const u32x4_t q_rs = make_rsrc(q + qk_bh, static_cast<uint32_t>((N - 1) * ldqk + dk) * 2);
    const u32x4_t k_rs = make_rsrc(k + qk_bh + srow0, static_cast<uint32_t>((N - 1) * ldqk + dk - srow0) * 2);
    const u32x4_t v_rs = make_rsrc(v + v_bh + col0, static_cast<uint32_t>((N - 1) * ldv + dv - col0) * 2);
    const uint32_t lds0 = lds_addr_of(smem);
    TileCopy<QRB, false, NW, REV> kcp;   // Q and K tiles (same row length and swizzle)
    TileCopy<VRB, true, NW, REV> vcp;
    kcp.init(ldqk * 2, wave, lane, N);
    vcp.init(ldv * 2, wave, lane, N);

    // State accumulator element (dt, i) of lane l holds state row srow(dt, i): tiles 2s and
    // 2s+1 together cover rows 32s..32s+31, with lane group g holding rows 32s+8g..32s+8g+7
    // (even g: tile 2s +0..3, tile 2s+1 +4..7; odd g the other way round, so that the
    // transposed K reads of one tile alternate 8-byte halves).  So the B operand of Q S
    // built from tiles 2s and 2s+1 has 8 contiguous reduction rows, matching one 16-byte
    // Q read.
    auto srow = [&](int dt, int i) -> int { return 32 * (dt >> 1) + 8 * g4 + 4 * ((dt ^ g4) & 1) + i; };

    // ---- incoming state
    f32x4_t S[DT][NT];
    {
        const int cidx = col0 + wcol + l16;
        auto load = [&](const float* src, float scale, bool add) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float x = src[static_cast<uint32_t>(srow(dt, i) * dv + cidx + nt * 16)];
                        S[dt][nt][i] = add ? S[dt][nt][i] * scale + x : x;
                    }
        };
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) S[dt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (MODE == kFull && !PAR) {
            if (nseg == 1 || ka.fuse_scan) {
                // entry state of segment seg: S <- 2^(l2 of segment s) S + local state of s.
                // The first source is loaded straight into the accumulators (all loads in
                // flight together; the adding form needs temporaries and goes slower).
                int sg0 = 0;
                if (ka.state_in != nullptr) {
                    load(ka.state_in + s_bh, 0.f, false);
                    if constexpr (REV && !GATED) {
                        const float inv = 1.f / decay[h];
#pragma unroll
                        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                                for (int i = 0; i < 4; ++i) S[dt][nt][i] *= inv;
                    }
                } else if (seg > 0) {
                    load(ka.seg_state + static_cast<size_t>(ch) * nseg * s_stride_seg, 0.f, false);
                    sg0 = 1;
                }
                for (int sg = sg0; nseg > 1 && sg < seg; ++sg)
                    load(ka.seg_state + (static_cast<size_t>(ch) * nseg + sg) * s_stride_seg,
                         exp2f(ka.seg_log2[static_cast<size_t>(ch) * nseg + sg]), true);
            } else {
                load(ka.seg_state + (static_cast<size_t>(ch) * nseg + seg) * s_stride_seg, 0.f, false);
            }
        }
    }

    // bf16 B operand of Q S from tiles 2ks, 2ks+1 (reduction rows 32ks+8g .. +7 in order)
    auto state_b = [&](int ks, int nt) -> u16x8_t {
        const u16x4_t a = bf4(S[2 * ks][nt]), b = bf4(S[2 * ks + 1][nt]);
        return (g4 & 1) ? cat(b, a) : cat(a, b);
    };

    // ---- LDS read addresses.  Every fragment read of a step is one of a few per-lane
    // patterns plus the current buffer's base plus a compile-time offset (row tile,
    // reduction step, high bits of the swizzled unit):
    //   Q/K rows (row tile t, reduction step ks): pq[ks%4] + t*16*QRB + (ks/4)*256, where
    //     unit 4ks+g (+) s(l%16) = 4(ks (+) s/4) + (g (+) s%4) splits into the pattern and
    //     a multiple of 256 bytes;
    //   K^T transposed reads (state tile dt, rows r0 and r0+4, reduction half ks):
    //     pkt[plus][(dt/2)%4][dt%2] + ks*32*QRB + (dt/8)*256;
    //   V transposed reads: pvp[nt] + (ks*32 + 16 half)*VRB (P V), pvs[plus][nt] + ks*32*VRB
    //     (state update).
    constexpr int KL = KS < 4 ? KS : 4;            // distinct row-read patterns
    constexpr int SL = DK / 32 < 4 ? DK / 32 : 4;  // distinct K^T patterns per row and half
    uint32_t pq[KL], pkt[2][SL][2], pvp[NT], pvs[2][NT];
    {
        const int s = swz_qk<QRB / 16>(l16);
#pragma unroll
        for (int kl = 0; kl < KL; ++kl)
            pq[kl] = static_cast<uint32_t>(l16 * QRB + 16 * (4 * (kl ^ (s >> 2)) + (g4 ^ (s & 3))));
#pragma unroll
        for (int pl = 0; pl < 2; ++pl) {
            const int rb = 32 * khalf + 8 * g4 + trj + 4 * pl;
            const int w = swz_qk<QRB / 16>(rb);
#pragma unroll
            for (int sl = 0; sl < SL; ++sl)
#pragma unroll
                for (int hb = 0; hb < 2; ++hb)
                    pkt[pl][sl][hb] = static_cast<uint32_t>(rb * QRB + 16 * (4 * (sl ^ (w >> 2)) + (trq ^ (w & 3))) +
                                                            8 * (hb ^ (trq & 1)));
            const int sv = swz_v<VRB / 16>(rb);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                pvs[pl][nt] = static_cast<uint32_t>(rb * VRB + 16 * (2 * ((cwave * NT + nt) ^ (sv >> 1)) + (trq >> 1)) +
                                                    8 * (trq & 1));
        }
        const int rbp = 4 * g4 + trj;
        const int svp = swz_v<VRB / 16>(rbp);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            pvp[nt] = static_cast<uint32_t>(rbp * VRB + 16 * (2 * ((cwave * NT + nt) ^ (svp >> 1)) + (trq >> 1)) +
                                            8 * (trq & 1));
    }

    // The state registers hold S / 2^lk2: the chunk decay is applied by moving lk2 (a
    // uniform scalar) instead of rescaling every element; new contributions are
    // multiplied by 2^-lk2 and the query-side factor by 2^lkx.  When lk2 drops below
    // -64 the registers are rescaled once and lk2 reset, which keeps them in range.
    float lk2 = 0.f;         // log2 of the current state scale
    float lkx = 0.f;         // log2 of the scale of the chunk's incoming state
    float seg_l2 = 0.f;      // log2 of the decay accumulated over the segment (pre-pass)
    u16x8_t Sp[ONEBLK ? 1 : KS][NT];   // bf16 copy of the chunk's incoming state (B operand of Q S)
    // output accumulators of the current query block, transposed: X[mt][nt] of lane
    // (g, l%16) holds O[row mt*16 + l%16][columns wcol + nt*16 + 4g .. +3]
    f32x4_t X[4][NT];

    // log2 of the decay over chunk positions (l, j] and over [0, j] (gated form)
    auto l2d = [&](int j, int l) -> float { return gl[j] - gl[l]; };
    auto l2x = [&](int j) -> float { return GATED ? gl[j] : static_cast<float>(j + 1) * lg; };

    // Per-head form: gamma^(j-l) splits into a per-lane factor (the lane's offsets
    // inside a 16x16 tile) and a uniform factor (the tile/block offset).  Both factors
    // are kept <= 1 (non-negative exponents) so that neither overflows for small gamma:
    //   fe: diagonal tile, gamma^(q-k) for key offset k <= query offset q, else 0;
    //   fo: off-diagonal tile, gamma^(16+q-k), paired with gamma^(tile offset - 16);
    //   fq: cross term, gamma^(row offset l%16);
    //   fz: state update, gamma^(31 - key offset in a 32-key half), paired with
    //       gamma^(distance from the half's last key to the chunk end).
    float fe[4], fo[4], fz[8];
    const float fq = GATED ? 1.f : exp2_fast(static_cast<float>(l16) * lg);
    bool dmask[4];           // inside a diagonal 16x16 tile: key <= query
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        dmask[i] = 4 * g4 + i <= l16;
        fe[i] = GATED || !dmask[i] ? 0.f : exp2_fast(static_cast<float>(l16 - 4 * g4 - i) * lg);
        fo[i] = GATED ? 1.f : exp2_fast(static_cast<float>(16 + l16 - 4 * g4 - i) * lg);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) fz[i] = GATED ? 1.f : exp2_fast(static_cast<float>(31 - 8 * g4 - i) * lg);

    float gpre[8];           // two stages: wave 0's prefetch of the next chunk's decays
    int qbuf = 0, kvbuf = 0;
    constexpr int kGLoads = (kMaxChunk / 64 + NW - 1) / NW;   // full pass: decay copies per wave
    // issue the asynchronous loads of step s into buffers (qb_, kvb_)
    // Deferred copies (full pass, two stages): a step's successor tiles are issued one
    // instruction at a time between the matrix instructions of the cross term, so the
    // copies of the eight waves do not queue up at the memory pipeline all at once.
    constexpr bool kSpread = MODE == kFull && NST == 2;
    constexpr int kNQ = TileCopy<QRB, false, NW>::kPerWave, kNV = TileCopy<VRB, true, NW>::kPerWave;
    constexpr int kNOps = 2 * kNQ + kNV;       // Q, K, V copies of one step
    bool dq = false, dkv = false;              // pending: Q tile, K and V tiles
    uint32_t dq_lds = 0, dk_lds = 0, dv_lds = 0, dq_off = 0, dk_off = 0, dv_off = 0;
    auto deferred_op = [&](int i) {
        if (i < kNQ) {
            if (dq) kcp.issue_one(i, dq_lds, q_rs, dq_off);
        } else if (i < 2 * kNQ) {
            if (dkv) kcp.issue_one(i - kNQ, dk_lds, k_rs, dk_off);
        } else if (dkv) {
            vcp.issue_one(i - 2 * kNQ, dv_lds, v_rs, dv_off);
        }
    };
    // REV: byte offset of the decay of walk position m (token N-m; none at m = 0 or
    // past the sequence, which read as zeros)
    auto rev_goff = [&](int m) -> uint32_t {
        return m >= 1 && m <= N ? static_cast<uint32_t>(N - m) * 4u : kOutOfRange;
    };
    auto issue = [&](const Step& s, int qb_, int kvb_, bool defer) {
        const int k0 = s.cs + s.kb * kBlk;
        const uint32_t wofs = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(wave)) * 1024u;
        if (kSpread && defer) {
            dq = s.kb == 0;
            dkv = true;
            dq_lds = lds0 + L_::kQ + qb_ * L_::kQTile + wofs;
            dk_lds = lds0 + L_::kK + kvb_ * L_::kKTile + wofs;
            dv_lds = lds0 + L_::kV + kvb_ * L_::kVTile + wofs;
            dq_off = static_cast<uint32_t>(s.cs + s.qb * kBlk) * ldqk * 2;
            dk_off = static_cast<uint32_t>(k0) * ldqk * 2;
            dv_off = static_cast<uint32_t>(k0) * ldv * 2;
        } else {
            if (MODE == kFull && s.kb == 0) {
                const int q0 = s.cs + s.qb * kBlk;
                kcp.issue(lds0 + L_::kQ + qb_ * L_::kQTile, q_rs, static_cast<uint32_t>(q0) * ldqk * 2, wave);
            }
            kcp.issue(lds0 + L_::kK + kvb_ * L_::kKTile, k_rs, static_cast<uint32_t>(k0) * ldqk * 2, wave);
            vcp.issue(lds0 + L_::kV + kvb_ * L_::kVTile, v_rs, static_cast<uint32_t>(k0) * ldv * 2, wave);
        }
        if (GATED && MODE == kStateOnly) {
            // the pre-pass walks single blocks: every wave copies the block's 64 decays
            if constexpr (REV)
                buf2lds4(g_rs, rev_goff(s.cs + lane), 0u, lds0 + L_::kGd + kvb_ * L_::kGdStage + wave * 256);
            else
                buf2lds4(g_rs, static_cast<uint32_t>(lane) * 4u, static_cast<uint32_t>(s.cs) * 4u,
                         lds0 + L_::kGd + kvb_ * L_::kGdStage + wave * 256);
        } else if (GATED && (PAR ? s.kb == 0 : s.qb == 0 && s.kb == 0)) {
            // chunk start: the chunk's decays.  Two stages: wave 0 prefetches them into
            // registers (8 per lane).  Three stages: every wave copies 64 per instruction
            // into the stage's LDS slot, so that every wave issues the same loads.
            if (NST == 2) {
                if (wave == 0) {
                    const int lim = min(C, t_end - s.cs) - 1;
                    if constexpr (REV) {
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            const int m = s.cs + min(lane * 8 + i, lim);
                            gpre[i] = m == 0 ? 0.f : g_bh[N - m];
                        }
                    } else {
                        const float* gs = g_bh + s.cs;
#pragma unroll
                        for (int i = 0; i < 8; ++i) gpre[i] = gs[min(lane * 8 + i, lim)];
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < kGLoads; ++i) {
                    const uint32_t dst = lds0 + L_::kGd + kvb_ * L_::kGdStage + (wave + i * NW) * 256;
                    if constexpr (REV)
                        buf2lds4(g_rs, rev_goff(s.cs + 64 * (wave + i * NW) + lane), 0u, dst);
                    else
                        buf2lds4(g_rs, static_cast<uint32_t>(lane) * 4u,
                                 static_cast<uint32_t>(s.cs + 64 * (wave + i * NW)) * 4u, dst);
                }
            }
        }
    };
    // vector memory loads one step issues per wave: K and V, Q when a query block starts,
    // the decays (pre-pass: every block; full pass: chunk starts)
    constexpr int kLoadsKV = TileCopy<QRB, false, NW>::kPerWave + TileCopy<VRB, true, NW>::kPerWave;
    constexpr int kLoadsQ = TileCopy<QRB, false, NW>::kPerWave;
    constexpr int kLoadsPerStep = kLoadsKV + (GATED ? 1 : 0);   // pre-pass

    int pend_q0 = -1, pend_nq = 0;   // rows of a finished query block not yet stored
    int st_last = 0;                 // stores issued by the last step: 0 none, 1 4*NT, 2 fewer
    // lane (g, l%16) stores 4 adjacent columns of row l%16 of each 16-row tile: a
    // wave-uniform base plus a 32-bit lane offset
    // (REV: rows run backwards from token N-1-first row)
    const uint32_t st_lane = static_cast<uint32_t>(l16 * dv + 4 * g4);
    const int st_lane_rev = 4 * g4 - l16 * dv;
    auto store_pending = [&]() {
        if (MODE != kFull || pend_q0 < 0) return;
        out_t* const base = REV ? o + o_bh + static_cast<size_t>(N - 1 - pend_q0) * dv + col0 + wcol
                                : o + o_bh + static_cast<size_t>(pend_q0) * dv + col0 + wcol;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            if (pend_nq < kBlk && mt * 16 + l16 >= pend_nq) continue;   // rows past the end
            if constexpr (REV) {
                out_t* const row = base - static_cast<ptrdiff_t>(mt * 16) * dv + st_lane_rev;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    if constexpr (OF32) *reinterpret_cast<f32x4_t*>(row + nt * 16) = X[mt][nt];
                    else *reinterpret_cast<u16x4_t*>(row + nt * 16) = bf4(X[mt][nt]);
                }
            } else {
                out_t* const row = base + static_cast<size_t>(mt * 16) * dv;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    if constexpr (OF32) *reinterpret_cast<f32x4_t*>(row + st_lane + nt * 16) = X[mt][nt];
                    else *reinterpret_cast<u16x4_t*>(row + st_lane + nt * 16) = bf4(X[mt][nt]);
                }
            }
        }
        pend_q0 = -1;
    };
    // Staged output: a finished block goes to LDS in the output type, row-major [64][DVT]
    // with the 16-byte units of row r rotated by XOR with r (no bank conflicts either
    // way); after the next step's barrier the workgroup stores it in whole rows, 16
    // bytes per lane.
    constexpr int kXE = OF32 ? 4 : 2;            // bytes per output element
    constexpr int kXU = DVT * kXE / 16;          // 16-byte units per staged row
    constexpr int kXRounds = kBlk * kXU / (NW * 64);
    static_assert(!kStage || kXRounds * NW * 64 == kBlk * kXU, "staged rows must split evenly");
    int xs_q0 = -1;                              // first row of the staged block
    auto stage_write = [&]() {
        char* const xs = smem + L_::kX;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int row = mt * 16 + l16;
                if constexpr (OF32) {
                    const int u = (wcol + nt * 16) / 4 + g4;
                    *reinterpret_cast<f32x4_t*>(xs + row * (DVT * 4) + (u ^ (row & (kXU - 1))) * 16) = X[mt][nt];
                } else {
                    const int u = (wcol + nt * 16) / 8 + (g4 >> 1);
                    *reinterpret_cast<u16x4_t*>(xs + row * (DVT * 2) + (u ^ (row & (kXU - 1))) * 16 + (g4 & 1) * 8) =
                        bf4(X[mt][nt]);
                }
            }
    };
    // the reads right after the barrier, the stores a little later (between the first
    // matrix instructions of the cross term, when the step has one)
    u16x8_t xv[kStage ? kXRounds : 1];
    auto stage_load = [&]() {
        const char* const xs = smem + L_::kX;
#pragma unroll
        for (int r = 0; r < kXRounds; ++r) {
            const int e = r * NW * 64 + tid;
            const int row = e / kXU, u = e % kXU;
            xv[r] = *reinterpret_cast<const u16x8_t*>(xs + row * (DVT * kXE) + (u ^ (row & (kXU - 1))) * 16);
        }
    };
    auto stage_emit = [&]() {
        if constexpr (REV) {
            out_t* const base = o + o_bh + static_cast<size_t>(N - 1 - xs_q0) * dv + col0;
#pragma unroll
            for (int r = 0; r < kXRounds; ++r) {
                const int e = r * NW * 64 + tid;
                const int row = e / kXU, u = e % kXU;
                *reinterpret_cast<u16x8_t*>(base + (u * (16 / kXE) - row * dv)) = xv[r];
            }
        } else {
            out_t* const base = o + o_bh + static_cast<size_t>(xs_q0) * dv + col0;
#pragma unroll
            for (int r = 0; r < kXRounds; ++r) {
                const int e = r * NW * 64 + tid;
                const int row = e / kXU, u = e % kXU;
                *reinterpret_cast<u16x8_t*>(base + static_cast<uint32_t>(row * dv + u * (16 / kXE))) = xv[r];
            }
        }
        xs_q0 = -1;
    };

    // bf16 score tiles of this wave (slot s16 holds tile tile_order(wave + s16 NW)),
    // written to LDS as P fragments [qt][key pair][lane][16 B]
    u16x4_t Pr[16 / NW];
    auto write_p = [&](char* base) {
#pragma unroll
        for (int s16 = 0; s16 < 16 / NW; ++s16) {
            const int code = tile_order(wave + s16 * NW);
            const int qt = code >> 2, kt = code & 3;
            *reinterpret_cast<u16x4_t*>(base + ((qt * 2 + (kt >> 1)) * 64 + lane) * 16 + (kt & 1) * 8) = Pr[s16];
        }
    };

    // Ring bookkeeping (wave-uniform, 2 bits per K/V stage): the Q stage a step reads and
    // which optional loads (bit 0: Q, bit 1: decays) it issued.
    int qlast = PL::QS - 1;    // Q stage of the most recent Q load
    uint32_t qof = 0, ldof = 0;
    auto issue_step = [&](const Step& s, int b, bool defer) {
        const bool needq = MODE == kFull && s.kb == 0;
        const bool needg = GATED && MODE == kFull && NST == 3 && (PAR ? s.kb == 0 : s.qb == 0 && s.kb == 0);
        if (needq) qlast = qlast + 1 == PL::QS ? 0 : qlast + 1;
        issue(s, qlast, b, defer);
        qof = (qof & ~(3u << (2 * b))) | (static_cast<uint32_t>(qlast) << (2 * b));
        ldof = (ldof & ~(3u << (2 * b))) | ((needq ? 1u : 0u) | (needg ? 2u : 0u)) << (2 * b);
    };

    // Drain the loads of the incoming state before the loop: the compiler does not count
    // the asynchronous copies, so a load it still tracked inside the loop would make it
    // wait there for them.  The full pass issues its first copies before the drain, so
    // that the two latencies overlap.
    // the walk: PAR visits key blocks 0..seg of query block seg only
    auto advance = [&](Step& s) -> bool {
        if constexpr (PAR) {
            if (s.kb < s.qb) { ++s.kb; return true; }
            return false;
        } else {
            return next_step<MODE>(s, t_end, C);
        }
    };
    Step cur{t_begin, PAR ? seg : 0, 0};
    if (MODE == kFull) issue_step(cur, 0, false);
    __builtin_amdgcn_s_waitcnt(0);
    if (MODE != kFull) issue_step(cur, 0, false);
    // steps issued beyond cur (at most NST - 2 at the top of an iteration)
    Step ahead = cur;
    bool more = true;
    int inflight = 0;
    for (int i = 0; i < NST - 2 && more; ++i) {
        more = advance(ahead);
        if (more) issue_step(ahead, ++inflight, false);
    }

    while (true) {
        // this step's tiles have landed: the pre-pass lets the loads of the steps after it
        // stay in flight; the main pass (whose stores also count) waits for everything
        if (MODE == kStateOnly && NST > 2) {
            if (inflight == NST - 2) wait_vmcnt<(NST - 2) * kLoadsPerStep>();
            else wait_vmcnt<0>();
        } else if (MODE == kFull && NST == 3) {
            // The full pass issues its output stores before its loads, so the youngest
            // operations are the next step's loads; loads complete in order.
            if (inflight == 1) {
                const int nb = kvbuf + 1 == NST ? 0 : kvbuf + 1;
                switch ((ldof >> (2 * nb)) & 3u) {
                    case 0: wait_vmcnt<kLoadsKV>(); break;
                    case 1: wait_vmcnt<kLoadsKV + kLoadsQ>(); break;
                    case 2: wait_vmcnt<kLoadsKV + kGLoads>(); break;
                    default: wait_vmcnt<kLoadsKV + kLoadsQ + kGLoads>(); break;
                }
            } else {
                wait_vmcnt<0>();
            }
        } else if (kSpread && st_last == 1) {
            // the youngest operations are the previous step's output stores
            wait_vmcnt<4 * NT>();
        } else {
            __builtin_amdgcn_s_waitcnt(0);
        }
        lds_barrier();
        if (kStage && xs_q0 >= 0) stage_load();
        qbuf = static_cast<int>((qof >> (2 * kvbuf)) & 3u);
        const int L = min(C, t_end - cur.cs);
        const int qb = ONEBLK ? 0 : cur.qb, kb = ONEBLK ? 0 : cur.kb;
        const bool diag = kb == qb;
        if (PAR ? kb == 0 : qb == 0 && kb == 0) {
            // start of a chunk: decays, bf16 snapshot of the old state, S <- 2^(G_{L-1}) S
            if (GATED && MODE == kStateOnly) {
                if (wave == 0) {
                    // block-local inclusive prefix of the decays (wave 0's copy)
                    const float* gb = reinterpret_cast<const float*>(smem + L_::kGd + kvbuf * L_::kGdStage);
                    float incl = lane < L ? gb[lane] * kLog2e : 0.f;
#pragma unroll
                    for (int off = 1; off < 64; off <<= 1) {
                        const float y = __shfl_up(incl, off, 64);
                        if (lane >= off) incl += y;
                    }
                    gl[lane] = incl;
                }
                lds_barrier();
            } else if (GATED) {
                if (wave == 0) {
                    const float* gc = reinterpret_cast<const float*>(smem + L_::kGd + kvbuf * L_::kGdStage);
                    float run = 0.f, loc[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float gv = NST == 2 ? gpre[i] : gc[lane * 8 + i];
                        run += lane * 8 + i < L ? gv * kLog2e : 0.f;
                        loc[i] = run;
                    }
                    float incl = run;
#pragma unroll
                    for (int off = 1; off < 64; off <<= 1) {
                        const float y = __shfl_up(incl, off, 64);
                        if (lane >= off) incl += y;
                    }
                    const float base = incl - run;
#pragma unroll
                    for (int i = 0; i < 8; ++i) gl[lane * 8 + i] = base + loc[i];
                }
                lds_barrier();
            }
            const float l2chunk = l2x(L - 1);
            if (MODE == kFull && !ONEBLK && !PAR) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) Sp[ks][nt] = state_b(ks, nt);
            }
            lkx = lk2;
            lk2 += l2chunk;
            seg_l2 += l2chunk;
        }

        Step nxt = cur;
        const bool has_next = advance(nxt);
        // With three stages the output stores must precede the loads (see the wait
        // above); with two, the loads go first so that they start earlier.
        if (NST == 3) store_pending();
        if (more) {
            more = advance(ahead);
            if (more) {
                ++inflight;
                int b = kvbuf + inflight;
                if (b >= NST) b -= NST;
                // deferred to the cross term when this step has one
                issue_step(ahead, b, kb == 0 && !PAR);
            }
        }
        if (NST != 3) store_pending();
        // the previous block, staged before this step's barrier (steps without a cross
        // term store it here)
        if (kStage && xs_q0 >= 0 && kb != 0) stage_emit();

        const bool fullq = (qb + 1) * kBlk <= L;     // no row of the blocks is past the chunk end
        const bool fullk = (kb + 1) * kBlk <= L;
        const char* Ks = smem + L_::kK + kvbuf * L_::kKTile;
        const uint32_t qbase = lds0 + L_::kQ + qbuf * L_::kQTile;
        const uint32_t kbase = lds0 + L_::kK + kvbuf * L_::kKTile;
        const uint32_t vbase = lds0 + L_::kV + kvbuf * L_::kVTile;
        if (MODE == kFull) {
            if (kb == 0) {
                // cross-chunk term X = diag(2^G) (Q S_prev), rows of block qb (PAR: none)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) X[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
            if (kb == 0 && !PAR) {
                uint32_t cq[KL];
#pragma unroll
                for (int kl = 0; kl < KL; ++kl) cq[kl] = opaque(pq[kl] + qbase);
                // Q fragments of reduction step ks+1 are read while step ks multiplies
                // (the scheduling barriers keep the compiler from serialising them)
                u16x8_t qa[4], qn[4];
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) qa[mt] = lds16a(cq[0] + mt * 16 * QRB);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    if (ks + 1 < KS) {
#pragma unroll
                        for (int mt = 0; mt < 4; ++mt)
                            qn[mt] = lds16a(cq[(ks + 1) % KL] + mt * 16 * QRB + ((ks + 1) / KL) * 256);
                    }
                    u16x8_t b[NT];
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) b[nt] = ONEBLK ? state_b(ks, nt) : Sp[ONEBLK ? 0 : ks][nt];
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) X[mt][nt] = mfma16(b[nt], qa[mt], X[mt][nt]);   // (S^T Q^T)
                    if (kStage && ks == 0 && xs_q0 >= 0) stage_emit();
                    if (kSpread) {
                        // (one Q stage: the Q copy waits for the P barrier)
                        constexpr int first = kQ1 ? kNQ : 0, nops = kNOps - first;
#pragma unroll
                        for (int i = ks * nops / KS; i < (ks + 1) * nops / KS; ++i) deferred_op(first + i);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) qa[mt] = qn[mt];
                }
                dkv = false;
                if (!kQ1) dq = false;
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const int j = qb * kBlk + mt * 16 + l16;     // this lane's query row
                    float xi = GATED ? exp2_fast(gl[j] + lkx)
                                     : exp2_fast(static_cast<float>(qb * kBlk + mt * 16 + 1) * lg + lkx) * fq;
                    if (!fullq && j >= L) xi = 0.f;
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) X[mt][nt] *= xi;
                }
            }
            // scores of (query block qb, key block kb): the 16 tiles (qt, kt) are listed
            // causal ones first and dealt round-robin to the waves, which balances the
            // diagonal block; tiles above the diagonal are written as zeros
#pragma unroll
            for (int s16 = 0; s16 < 16 / NW; ++s16) {
                const int slot = wave + s16 * NW;
                const int code = tile_order(slot);
                const int qt = code >> 2, kt = code & 3;
                Pr[s16] = u16x4_t{};
                if (diag && kt > qt) continue;
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
                uint32_t ck[KL], cq[KL];
#pragma unroll
                for (int kl = 0; kl < KL; ++kl) {
                    ck[kl] = opaque(pq[kl] + kbase + kt * 16 * QRB);
                    cq[kl] = opaque(pq[kl] + qbase + qt * 16 * QRB);
                }
                // two reduction steps of fragments in flight ahead of the products
                u16x8_t ka[KS], qv[KS];
#pragma unroll
                for (int ks = 0; ks < KS && ks < 2; ++ks) {
                    ka[ks] = lds16a(ck[ks % KL] + (ks / KL) * 256);
                    qv[ks] = lds16a(cq[ks % KL] + (ks / KL) * 256);
                }
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    if (ks + 2 < KS) {
                        ka[ks + 2] = lds16a(ck[(ks + 2) % KL] + ((ks + 2) / KL) * 256);
                        qv[ks + 2] = lds16a(cq[(ks + 2) % KL] + ((ks + 2) / KL) * 256);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    acc = mfma16(ka[ks], qv[ks], acc);
                    __builtin_amdgcn_sched_barrier(0);
                }
                const int j = qb * kBlk + qt * 16 + l16;      // query (chunk-local)
                const bool dtile = diag && kt == qt;
                // off-diagonal tiles: gamma^(tile offset - 16), tile offset >= 16
                const float sd = GATED || dtile ? 0.f : exp2_fast(static_cast<float>((qb - kb) * kBlk + (qt - kt) * 16 - 16) * lg);
                float w[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int l = kb * kBlk + kt * 16 + 4 * g4 + i;   // key (chunk-local)
                    if (GATED) w[i] = dtile && !dmask[i] ? 0.f : exp2_fast(l2d(j, l));
                    else w[i] = dtile ? fe[i] : sd * fo[i];
                }
                if (!(fullq && fullk)) {
                    // rows or keys past the chunk end (partial blocks only)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (kb * kBlk + kt * 16 + 4 * g4 + i >= L || j >= L) w[i] = 0.f;
                }
                Pr[s16] = bf4(f32x4_t{acc[0] * w[0], acc[1] * w[1], acc[2] * w[2], acc[3] * w[3]});
            }
            if (!L_::kPInK) write_p(Pfix);
            // one Q stage: every wave is past its Q reads here, and P is complete
            if (kQ1) lds_barrier();
        }
        if (qb == 0 && kb == 0 && lk2 < -64.f) {
            // rescale the registers once the state scale gets small (after the cross
            // term, which reads them at the old scale)
            const float r = exp2_fast(lk2);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) S[dt][nt] *= r;
            lk2 = 0.f;
        }
        if (diag && !PAR) {
            // S += K^T (V (.) zeta) over the keys of block qb; slots are keys
            // 32ks + 8g .. 32ks + 8g + 7, gathered by transpose reads of K and V
#pragma unroll
            for (int kh = 0; kh < (SPLITK ? 1 : 2); ++kh) {
                // key half ks of the block (the patterns already hold the pre-pass
                // wave's half; ks only enters the decays and the key indices)
                const int ks = SPLITK ? khalf : kh;
                // zeta_l / 2^lk2: decay from key l to the chunk end, in the state's scale.
                // Full blocks: uniform gamma^(L - 32 - 32ks - 64kb) (exponent >= 0) times
                // fz; a partial block takes the power directly.
                const float sz = GATED ? 0.f : exp2_fast(static_cast<float>(L - 32 - kb * kBlk - ks * 32) * lg - lk2);
                // K^T operand of state tile dt: result lane m must receive state row
                // srow(dt, m%4 of group m/4), so source lane (j, q) reads dims
                // 32(dt/2) + 8q + 4((dt^q)&1) .. +3
                uint32_t ckt[2][SL][2];
#pragma unroll
                for (int pl = 0; pl < 2; ++pl)
#pragma unroll
                    for (int sl = 0; sl < SL; ++sl)
#pragma unroll
                        for (int hb = 0; hb < 2; ++hb) ckt[pl][sl][hb] = opaque(pkt[pl][sl][hb] + kbase + kh * 32 * QRB);
                auto kt_frag = [&](int dt) -> u16x8_t {
                    const int sd = dt >> 1;
                    return cat(lds_tra(ckt[0][sd % SL][dt & 1] + (sd / SL) * 256),
                               lds_tra(ckt[1][sd % SL][dt & 1] + (sd / SL) * 256));
                };
                // software pipeline: the reads of the next G operand tiles are issued
                // before the matrix instructions on the current ones (the scheduling
                // barriers keep the compiler from serialising reads and uses)
                constexpr int G = DT < 4 ? DT : (DT >= 16 && NW == 8 ? 2 : 4);
                u16x8_t raw[NT], acur[G], anext[G];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    raw[nt] = cat(lds_tra(vbase + pvs[0][nt] + kh * 32 * VRB), lds_tra(vbase + pvs[1][nt] + kh * 32 * VRB));
#pragma unroll
                for (int j = 0; j < G; ++j) acur[j] = kt_frag(j);
                __builtin_amdgcn_sched_barrier(0);
                float z[8];
                if (GATED) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int l = kb * kBlk + ks * 32 + 8 * g4 + i;
                        z[i] = exp2_fast(l2d(L - 1, l) - lk2);
                        if (!fullk && l >= L) z[i] = 0.f;
                    }
                } else if (fullk) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) z[i] = sz * fz[i];
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int l = kb * kBlk + ks * 32 + 8 * g4 + i;
                        z[i] = l < L ? exp2_fast(static_cast<float>(L - 1 - l) * lg - lk2) : 0.f;
                    }
                }
                u16x8_t b[NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    f32x4_t lo, hi;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        lo[i] = bf16_to_f32(raw[nt][i]) * z[i];
                        hi[i] = bf16_to_f32(raw[nt][i + 4]) * z[i + 4];
                    }
                    b[nt] = cat(bf4(lo), bf4(hi));
                }
#pragma unroll
                for (int g0 = 0; g0 < DT; g0 += G) {
                    if (g0 + G < DT) {
#pragma unroll
                        for (int j = 0; j < G; ++j) anext[j] = kt_frag(g0 + G + j);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int j = 0; j < G; ++j)
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) S[g0 + j][nt] = mfma16(acur[j], b[nt], S[g0 + j][nt]);
                    if (kQ1 && kh == 0) {
                        // one Q stage: the next block's Q copies go out here
                        constexpr int NG = DT / G;
                        const int gi = g0 / G;
#pragma unroll
                        for (int i = gi * kNQ / NG; i < (gi + 1) * kNQ / NG; ++i) deferred_op(i);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int j = 0; j < G; ++j) acur[j] = anext[j];
                }
            }
        }
        if (kQ1) dq = false;
        if (MODE == kFull) {
            // P goes to its own LDS area, or into the K buffer once no wave reads K
            const char* Pf = Pfix;
            if (L_::kPInK) {
                lds_barrier();
                write_p(const_cast<char*>(Ks));
                Pf = Ks;
            }
            if (!kQ1) lds_barrier();
            // X += P V over the 64 keys of block kb (as X^T += V^T P^T); V fragments by transpose reads:
            // slots {4g..4g+3} of key tile 2ks and of key tile 2ks+1
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                u16x8_t b[NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const uint32_t va = opaque(vbase + pvp[nt]);
                    b[nt] = cat(lds_tra(va + ks * 32 * VRB), lds_tra(va + (ks * 32 + 16) * VRB));
                }
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    if (diag && 2 * ks > mt) continue;
                    const u16x8_t a = lds16(Pf, ((mt * 2 + ks) * 64 + lane) * 16);
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) X[mt][nt] = mfma16(b[nt], a, X[mt][nt]);   // (V^T P^T)
                }
            }
        }
        if (MODE == kFull && diag) {
            pend_q0 = cur.cs + qb * kBlk;
            pend_nq = min(kBlk, L - qb * kBlk);
        }
        if (kStage && pend_q0 >= 0 && has_next && pend_nq == kBlk) {
            // full block with steps to come: staged, stored after the next barrier
            stage_write();
            xs_q0 = pend_q0;
            pend_q0 = -1;
            st_last = 0;
        } else if (kSpread) {
            // two stages: a finished block is stored at once (the next step's wait
            // skips these stores)
            st_last = pend_q0 < 0 ? 0 : pend_nq == kBlk ? 1 : 2;
            store_pending();
        }
        if (!has_next) break;
        cur = nxt;
        kvbuf = kvbuf + 1 == NST ? 0 : kvbuf + 1;
        if (inflight > 0) --inflight;
    }
    store_pending();
    if (kStage && xs_q0 >= 0) {   // (the last step stores from registers; kept for safety)
        lds_barrier();
        stage_load();
        stage_emit();
    }

    if (SPLITK) {
        // sum the two key halves: the second half's waves park their partial states in
        // LDS (the tile buffers are free once every wave is past the loop)
        float* red = reinterpret_cast<float*>(smem);
        static_assert(DK * DVT * 4 <= L_::kGd, "reduction area exceeds the tile buffers");
        const int cidx = wcol + l16;
        wait_vmcnt<0>();
        lds_barrier();
        if (khalf == 1) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) red[srow(dt, i) * DVT + cidx + nt * 16] = S[dt][nt][i];
        }
        lds_barrier();
        if (khalf == 0) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) S[dt][nt][i] += red[srow(dt, i) * DVT + cidx + nt * 16];
        }
    }

    // ---- results
    float* dst = nullptr;
    if (MODE == kFull) {
        if (!PAR && seg == nseg - 1 && ka.state_out != nullptr) dst = ka.state_out + s_bh;
    } else {
        dst = ka.seg_state + (static_cast<size_t>(ch) * nseg + seg) * s_stride_seg + static_cast<size_t>(srow0) * dv;
        if (dvt == 0 && dkt == 0 && tid == 0) ka.seg_log2[static_cast<size_t>(ch) * nseg + seg] = seg_l2;
    }
    if (dst != nullptr) {
        // the tile goes out through LDS as well, in whole rows of 16-byte stores
        float* const st = reinterpret_cast<float*>(smem);
        // REV: the final state leaves multiplied by the decay of token 0
        float lout = lk2;
        if constexpr (REV && MODE == kFull) lout += GATED ? g_bh[0] * kLog2e : lg;
        const float r = exp2_fast(lout);
        wait_vmcnt<0>();
        lds_barrier();   // every wave is done with the tile buffers
        if (!SPLITK || khalf == 0) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) st[srow(dt, i) * DVT + wcol + nt * 16 + l16] = S[dt][nt][i] * r;
        }
        lds_barrier();
        constexpr int kU = DVT / 4;                          // 16-byte units per row
        constexpr int kRounds = DK * kU / (NW * 64);
        static_assert(kRounds * NW * 64 == DK * kU, "state rows must split evenly");
#pragma unroll
        for (int rr = 0; rr < kRounds; ++rr) {
            const int e = rr * NW * 64 + tid;
            const int row = e / kU, u = e % kU;
            *reinterpret_cast<f32x4_t*>(dst + static_cast<size_t>(row) * dv + col0 + u * 4) =
                *reinterpret_cast<const f32x4_t*>(st + row * DVT + u * 4);
        }
    }
}

// Exclusive scan of segment states, in place:  buf[seg] <- state entering seg.
//   S = state_in (or 0); for seg: T = buf[seg]; buf[seg] = S; S = 2^(l2[seg]) S + T.
// in_gamma (reversed per-head walks): state_in enters divided by gamma[h].  Chains are
// (b,h) and column slice as in the main kernel (nsl slices, state_in sl_state floats apart).
// The last segment's local state is never computed (nor read).  One thread per state
// element of one (b,h); blocks_per_bh blocks per (b,h).  The local states of 8
// segments are loaded before any of them is replaced, so a batch's loads are in flight
// together (the kernel is bound by memory latency, not bandwidth).
__global__ __launch_bounds__(256) void segment_scan_kernel(float* __restrict__ buf,
                                                           const float* __restrict__ seg_log2,
                                                           const float* __restrict__ state_in,
                                                           const float* __restrict__ in_gamma, int H,
                                                           int nseg, size_t per_bh, int blocks_per_bh, int nsl,
                                                           size_t sl_state) {
    constexpr int kBatch = 8;
    const size_t bh = blockIdx.x / blocks_per_bh;   // chain
    const size_t hb = bh / nsl;                     // its (b,h)
    const int xb = blockIdx.x % blocks_per_bh;
    const float* const l2 = seg_log2 + bh * nseg;
    const float in_scale = in_gamma != nullptr ? 1.f / in_gamma[hb % H] : 1.f;
    const size_t in_off = (bh % nsl) * sl_state + hb * per_bh;
    for (size_t e = xb * static_cast<size_t>(blockDim.x) + threadIdx.x; e < per_bh;
         e += static_cast<size_t>(blocks_per_bh) * blockDim.x) {
        float s = state_in != nullptr ? state_in[in_off + e] * in_scale : 0.f;
        for (int sg0 = 0; sg0 < nseg; sg0 += kBatch) {
            float t[kBatch], f[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                t[j] = sg0 + j + 1 < nseg ? buf[(bh * nseg + sg0 + j) * per_bh + e] : 0.f;
                f[j] = sg0 + j + 1 < nseg ? l2[sg0 + j] : 0.f;
            }
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const int sg = sg0 + j;
                if (sg < nseg) {
                    buf[(bh * nseg + sg) * per_bh + e] = s;
                    s = exp2f(f[j]) * s + t[j];
                }
            }
        }
    }
}

template <int DK, int DVT, int NW, bool GATED, int MODE, bool ONEBLK, bool OF32, bool REV, bool PAR = false>
hipError_t launch_kernel(const KArgs& ka, hipStream_t stream) {
    constexpr size_t lds = Plan<DK, DVT, GATED, MODE, NW, ONEBLK, OF32>::L::kBytes;
    // the LDS limit is raised once per kernel instance (thread-safe one-time init)
    static std::once_flag attr_once;
    std::call_once(attr_once, [] {
        (void)hipFuncSetAttribute(
            reinterpret_cast<const void*>(&chunk_kernel<DK, DVT, NW, GATED, MODE, ONEBLK, OF32, REV, PAR>),
            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    });
    ProfScope prof(MODE == kFull ? kProfMain : kProfPre, stream);
    hipLaunchKernelGGL((chunk_kernel<DK, DVT, NW, GATED, MODE, ONEBLK, OF32, REV, PAR>), dim3(ka.total_groups),
                       dim3(NW * 64), lds, stream, ka);
    return hipGetLastError();
}

// Segment-state pre-pass: state-row tile DKT (<= 128) and column tile DVT, one wave
// per 16 columns.
template <bool GATED, bool REV>
hipError_t launch_pre(KArgs ka, const MfmaPlan& p, hipStream_t stream) {
    ka.ndkt = ka.dk / p.pre_dkt;
    ka.ndvt = ka.dv / p.pre_dvt;
    const int bh = ka.total_groups;   // caller passes B*H
    // the local state of a segment does not depend on how it is chunked: walk it in
    // single 64-token blocks (each block its own decay step)
    ka.C = kBlk;
    ka.total_groups = bh * (ka.nseg - 1) * ka.ndkt * ka.ndvt;
#define RETN_PRE(DKT, DVT)                                                                  \
    if (p.pre_dkt == DKT && p.pre_dvt == DVT)                                               \
        return launch_kernel<DKT, DVT, DVT / 16, GATED, kStateOnly, true, false, REV>(ka, stream);
    RETN_PRE(64, 64)
    RETN_PRE(64, 128)
    RETN_PRE(128, 64)
    RETN_PRE(128, 128)
#undef RETN_PRE
    return hipErrorInvalidValue;
}

// Kernel arguments of the main pass, after the segment-state pre-pass and (when the
// main pass does not compose the entry states itself) the scan have been launched.
template <bool GATED, bool REV>
hipError_t launch_prep(const ChunkArgs& a, const MfmaPlan& p, int dvt, hipStream_t stream, KArgs& ka) {
    ka = KArgs{};
    ka.q = static_cast<const bf16_t*>(a.q);
    ka.k = static_cast<const bf16_t*>(a.k);
    ka.v = static_cast<const bf16_t*>(a.v);
    ka.decay = a.decay;
    ka.o = a.o;
    ka.state_in = a.state_in;
    ka.state_out = a.state_out;
    ka.H = a.H;
    ka.N = a.N;
    ka.dk = a.dk;
    ka.dv = a.dv;
    ka.ldqk = a.ldqk > 0 ? a.ldqk : a.dk;
    ka.ldv = a.ldv > 0 ? a.ldv : a.dv;
    ka.C = a.chunk;
    ka.seg_tokens = p.seg_chunks * a.chunk;
    ka.nseg = p.nseg;
    ka.fuse_scan = p.fuse_scan;
    ka.nsl = a.slices > 1 ? a.slices : 1;
    ka.sl_qk = a.slice_qk;
    ka.sl_o = a.slice_o;
    ka.sl_state = a.slice_state;
    ka.pre_tokens = p.prefix_tokens;
    ka.xdot = static_cast<const bf16_t*>(a.xdot);
    ka.dG = a.dG;
    ka.dsign = a.dsign;
    ka.dacc = a.dacc ? 1 : 0;
    ka.ng_gate = static_cast<const bf16_t*>(a.ng_gate);
    ka.ng_out = static_cast<bf16_t*>(a.ng_out);
    ka.ng_eps = a.ng_eps;
    ka.st_ld = a.state_in_ld;
    ka.seg_t = a.seg_from_t ? 1 : 0;
    const int bh = a.B * a.H * ka.nsl;   // chains
    if (p.nseg > 1 && p.prefix_tokens == 0) {
        const size_t per_bh = static_cast<size_t>(a.dk) * a.dv;
        ka.seg_state = static_cast<float*>(a.workspace);
        ka.seg_log2 = ka.seg_state + static_cast<size_t>(bh) * p.nseg * per_bh;
    }
    if (p.nseg > 1 && p.prefix_tokens == 0 && !a.seg_from_t) {
        const size_t per_bh = static_cast<size_t>(a.dk) * a.dv;
        KArgs pre = ka;
        pre.total_groups = bh;
        hipError_t e = launch_pre<GATED, REV>(pre, p, stream);
        if (e != hipSuccess) return e;
        if (!p.fuse_scan) {
            const int xblocks = static_cast<int>(std::min<size_t>((per_bh + 255) / 256, 256));
            ProfScope prof(kProfScan, stream);
            hipLaunchKernelGGL(segment_scan_kernel, dim3(static_cast<unsigned>(xblocks) * bh), dim3(256), 0,
                               stream, ka.seg_state, ka.seg_log2, a.state_in, REV && !GATED ? a.decay : nullptr,
                               a.H, p.nseg, per_bh, xblocks, ka.nsl, ka.sl_state);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    ka.ndkt = 1;
    ka.ndvt = a.dv / dvt;
    ka.total_groups = bh * p.nseg * ka.ndvt;
    return hipSuccess;
}

template <int DK, int DVT, int NW, bool GATED, bool ONEBLK, bool OF32, bool REV>
hipError_t launch_shape(const ChunkArgs& a, const MfmaPlan& p, hipStream_t stream) {
    KArgs ka;
    const hipError_t e = launch_prep<GATED, REV>(a, p, DVT, stream, ka);
    if (e != hipSuccess) return e;
    return launch_kernel<DK, DVT, NW, GATED, kFull, ONEBLK, OF32, REV>(ka, stream);
}

// Chunks of exactly 64 tokens take the leaner single-block main pass (chunk64.hip).
template <bool GATED, bool REV>
hipError_t launch_chunk64(const ChunkArgs& a, const MfmaPlan& p, hipStream_t stream) {
    KArgs ka;
    const hipError_t e = launch_prep<GATED, REV>(a, p, p.dvt, stream, ka);
    if (e != hipSuccess) return e;
    return launch_chunk1(ka, GATED, REV, a.out_f32, a.xdot != nullptr, stream);
}
// Chunks of 256 or 512 tokens (d_k = 128, per-head decays) take the query-row parallel
// main pass (chunkw.hip).
template <bool REV>
hipError_t launch_chunk_rows(const ChunkArgs& a, const MfmaPlan& p, hipStream_t stream) {
    KArgs ka;
    const hipError_t e = launch_prep<false, REV>(a, p, p.dvt, stream, ka);
    if (e != hipSuccess) return e;
    return launch_chunkw(ka, stream);
}

// State columns per workgroup and waves per workgroup for a head shape.
// State columns per workgroup and waves per workgroup for a head shape.  Wider column
// tiles cut the re-reads of Q and K (from L2 and from LDS) per output column; 8 waves
// (two per SIMD) hide LDS and matrix-core latency better than 4 wider ones.  With
// dk = 256 a 128-column tile fills the LDS (P then lives in the K buffer) and needs the
// registers freed by single-block chunks.
void pick_tile(int dk, int dv, int chunk, bool gated, int& dvt, int& nw) {
    if (dk == 256 && !gated && dv % 128 == 0 && chunk <= kBlk) { dvt = 128; nw = 8; return; }
    // gated 64-token chunks run on the single-block pass, which fits 128 columns (the
    // general kernel only 64)
    if (dk == 256 && gated && dv % 128 == 0 && chunk == kBlk) { dvt = 128; nw = 8; return; }
    if (dk == 256) { dvt = 64; nw = 4; return; }
    if (dv % 128 == 0) { dvt = 128; nw = 8; return; }
    dvt = 64;
    nw = 4;
}

}  // namespace

bool seg_shareable(int B, int H, int N, int dk, int dv, int chunk, bool gated, bool out_f32) {
    const MfmaPlan p = mfma_chunk_plan(B, H, N, dk, dv, chunk, gated);
    const MfmaPlan t = mfma_chunk_plan(B, H, N, dv, dk, chunk, gated);
    return p.nseg > 1 && p.prefix_tokens == 0 && t.prefix_tokens == 0 && p.nseg == t.nseg &&
           p.seg_chunks == t.seg_chunks && p.fuse_scan == t.fuse_scan && p.workspace_bytes == t.workspace_bytes &&
           p.dvt == 128 && p.nw == 8 && chunk1_supported(dk, dv, chunk, dk, dv, 1, out_f32, gated);
}

bool chunk1_takes(const ChunkArgs& a, const MfmaPlan& p) {
    return p.dvt == 128 && p.nw == 8 &&
           chunk1_supported(a.dk, a.dv, a.chunk, a.ldqk > 0 ? a.ldqk : a.dk, a.ldv > 0 ? a.ldv : a.dv, a.slices,
                            a.out_f32, a.gated) &&
           (p.nseg == 1 || p.prefix_tokens > 0 || p.fuse_scan);
}

bool mfma_chunk_supported(int dk, int dv, int chunk, bool bf16) {
    if (!bf16) return false;
    if (dk != 64 && dk != 128 && dk != 256) return false;
    if (dv % 64 != 0 || dv > 1024) return false;
    return chunk >= 1 && chunk <= kMaxChunk;
}

MfmaPlan mfma_chunk_plan(int B, int H, int N, int dk, int dv, int chunk, bool gated) {
    MfmaPlan p{};
    pick_tile(dk, dv, chunk, gated, p.dvt, p.nw);
    const long bh = static_cast<long>(B) * H;
    const long base = bh * (dv / p.dvt);
    const int nchunks = (N + chunk - 1) / chunk;
    int want = static_cast<int>(std::max<long>(1, (kTargetGroups + base - 1) / base));
    want = std::min(want, std::max(1, nchunks));
    p.seg_chunks = (nchunks + want - 1) / want;
    p.nseg = (nchunks + p.seg_chunks - 1) / p.seg_chunks;
    p.pre_dkt = std::min(dk, 128);
    p.pre_dvt = dv % 128 == 0 ? 128 : 64;
    p.fuse_scan = p.nseg <= kFuseScanMax ? 1 : 0;
    p.prefix_tokens = 0;
    if (p.nseg == 2 && chunk == kBlk && p.dvt == 128 && nchunks >= 4 &&
        chunk1_supported(dk, dv, chunk, dk, dv, 1, false, gated)) {
        // Two segments: the second segment's workgroups compute their entry state by
        // walking the first segment state-only, which costs about kPrefixCost of a full
        // step per chunk; the first segment is made longer so both finish together.
        int sp = static_cast<int>(nchunks / (2.0 - kPrefixCost) + 0.5);
        sp = std::max(1, std::min(sp, nchunks - 1));
        p.prefix_tokens = sp * kBlk;
        p.seg_chunks = sp;
        p.fuse_scan = 0;
        p.workspace_bytes = 0;
        return p;
    }
    if (p.nseg > 1) {
        const size_t per_bh = static_cast<size_t>(dk) * dv;
        p.workspace_bytes = (static_cast<size_t>(bh) * p.nseg * per_bh + static_cast<size_t>(bh) * p.nseg) * sizeof(float);
    } else {
        p.workspace_bytes = 0;
    }
    return p;
}

namespace {

template <int DK, int DVT, int NW, bool REV>
hipError_t launch_variant(const ChunkArgs& a, const MfmaPlan& p, bool one, hipStream_t stream) {
    if (a.gated && a.out_f32)
        return one ? launch_shape<DK, DVT, NW, true, true, true, REV>(a, p, stream)
                   : launch_shape<DK, DVT, NW, true, false, true, REV>(a, p, stream);
    if (a.gated)
        return one ? launch_shape<DK, DVT, NW, true, true, false, REV>(a, p, stream)
                   : launch_shape<DK, DVT, NW, true, false, false, REV>(a, p, stream);
    return one ? launch_shape<DK, DVT, NW, false, true, false, REV>(a, p, stream)
               : launch_shape<DK, DVT, NW, false, false, false, REV>(a, p, stream);
}

template <bool REV>
hipError_t launch_dir(const ChunkArgs& a, const MfmaPlan& p, hipStream_t stream) {
    // the kernel handles any chunk in [1, 512], including chunks that are not a
    // multiple of its 64-token blocks; chunks of one block take the ONEBLK variant, and
    // chunks of exactly one block (forward, bf16 output) the single-block main pass
    const bool one = a.chunk <= kBlk;
    // the row-dot and norm-gate forms exist on the single-block pass only
    if ((a.xdot != nullptr || a.ng_gate != nullptr) &&
        !(p.dvt == 128 && p.nw == 8 && a.gated && !a.out_f32 && a.slices <= 1 && chunk1_dot_supported(a.dk, a.dv, a.chunk) &&
          !(a.ng_gate != nullptr && (a.reverse || a.xdot != nullptr))))
        return hipErrorInvalidValue;
    if (a.state_in_ld > 0 && !chunk1_takes(a, p)) return hipErrorInvalidValue;
    if (a.seg_from_t && !(a.slices <= 1 && a.ldqk <= a.dk && a.ldv <= a.dv &&
                          seg_shareable(a.B, a.H, a.N, a.dk, a.dv, a.chunk, a.gated, a.out_f32)))
        return hipErrorInvalidValue;
    if (p.dvt == 128 && p.nw == 8 &&
        chunk1_supported(a.dk, a.dv, a.chunk, a.ldqk > 0 ? a.ldqk : a.dk, a.ldv > 0 ? a.ldv : a.dv, a.slices,
                         a.out_f32, a.gated))
        return a.gated ? launch_chunk64<true, REV>(a, p, stream) : launch_chunk64<false, REV>(a, p, stream);
    if (p.prefix_tokens > 0) return hipErrorInvalidValue;   // only the single-block pass walks prefixes
    if (p.dvt == 128 && p.nw == 8 &&
        chunkw_supported(a.dk, a.dv, a.chunk, a.ldqk > 0 ? a.ldqk : a.dk, a.ldv > 0 ? a.ldv : a.dv, a.slices,
                         a.out_f32, a.reverse, a.gated))
        return launch_chunk_rows<REV>(a, p, stream);
#define RETN_SHAPE(DK, DVT, NW) \
    if (a.dk == DK && p.dvt == DVT && p.nw == NW) return launch_variant<DK, DVT, NW, REV>(a, p, one, stream);
    RETN_SHAPE(64, 64, 4)
    RETN_SHAPE(64, 128, 8)
    RETN_SHAPE(128, 64, 4)
    RETN_SHAPE(128, 128, 8)
    RETN_SHAPE(256, 64, 4)
#undef RETN_SHAPE
    // the gated form's decay array does not fit beside double-buffered 256 x 128 tiles
    if (a.dk == 256 && p.dvt == 128 && p.nw == 8 && !a.gated && !a.out_f32 && one)
        return launch_shape<256, 128, 8, false, true, false, REV>(a, p, stream);
    return hipErrorInvalidValue;
}

}  // namespace

namespace {

// Parallel form: one workgroup per (b,h), query block and column tile; no state, no
// workspace.  Chunk-length-one-block variants are not used (the query blocks differ).
template <int DK, int DVT, int NW, bool GATED>
hipError_t launch_parallel_shape(const ChunkArgs& a, hipStream_t stream) {
    KArgs ka{};
    ka.q = static_cast<const bf16_t*>(a.q);
    ka.k = static_cast<const bf16_t*>(a.k);
    ka.v = static_cast<const bf16_t*>(a.v);
    ka.decay = a.decay;
    ka.o = a.o;
    ka.H = a.H;
    ka.N = a.N;
    ka.dk = a.dk;
    ka.dv = a.dv;
    ka.ldqk = a.dk;
    ka.ldv = a.dv;
    ka.C = a.N;
    ka.seg_tokens = a.N;
    ka.nseg = (a.N + kBlk - 1) / kBlk;   // query blocks
    ka.ndkt = 1;
    ka.ndvt = a.dv / DVT;
    ka.nsl = 1;
    const size_t groups = static_cast<size_t>(a.B) * a.H * ka.nseg * ka.ndvt;
    if (groups > static_cast<size_t>(INT32_MAX)) return hipErrorInvalidValue;
    ka.total_groups = static_cast<int>(groups);
    return launch_kernel<DK, DVT, NW, GATED, kFull, false, false, false, true>(ka, stream);
}

}  // namespace

bool mfma_parallel_supported(int dk, int dv, int N, bool gated, bool bf16) {
    if (!bf16 || N < 1) return false;
    if (dk != 64 && dk != 128 && dk != 256) return false;
    if (dv % 64 != 0 || dv > 1024) return false;
    // the gated form keeps the sequence's cumulative decays in LDS
    if (gated && N > kMaxChunk) return false;
    // rows and the causal block count stay in 32-bit arithmetic
    return static_cast<size_t>(N) * std::max(dk, dv) * 2 < (static_cast<size_t>(1) << 31);
}

hipError_t launch_mfma_parallel(const ChunkArgs& a, hipStream_t stream) {
    if (!mfma_parallel_supported(a.dk, a.dv, a.N, a.gated, a.bf16)) return hipErrorInvalidValue;
    int dvt, nw;
    pick_tile(a.dk, a.dv, kBlk + 1, a.gated, dvt, nw);   // the tiles of multi-block chunks
#define RETN_PSHAPE(DK, DVT, NW)                                                                \
    if (a.dk == DK && dvt == DVT && nw == NW)                                                   \
        return a.gated ? launch_parallel_shape<DK, DVT, NW, true>(a, stream)                    \
                       : launch_parallel_shape<DK, DVT, NW, false>(a, stream);
    RETN_PSHAPE(64, 64, 4)
    RETN_PSHAPE(64, 128, 8)
    RETN_PSHAPE(128, 64, 4)
    RETN_PSHAPE(128, 128, 8)
    RETN_PSHAPE(256, 64, 4)
#undef RETN_PSHAPE
    return hipErrorInvalidValue;
}

hipError_t launch_mfma_chunk(const ChunkArgs& a, const MfmaPlan& p, hipStream_t stream) {
    // fp32 outputs: gated shapes only (the gated backward's gate gradient needs them)
    if (a.out_f32 && !a.gated) return hipErrorInvalidValue;
    // reversed walks address rows with signed 32-bit byte offsets
    if (a.reverse) {
        const size_t ld = static_cast<size_t>(std::max({a.ldqk > 0 ? a.ldqk : a.dk, a.ldv > 0 ? a.ldv : a.dv, a.dv}));
        if ((static_cast<size_t>(a.N) + kBlk) * ld * 2 >= (static_cast<size_t>(1) << 31)) return hipErrorInvalidValue;
        return launch_dir<true>(a, p, stream);
    }
    return launch_dir<false>(a, p, stream);
}

}  // namespace retn
