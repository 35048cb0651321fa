// bf16 chunkwise retention forward on the gfx950 matrix cores for chunks of 256 or 512
// tokens (d_k = 128, per-head decays).
//
// Method ("RetNet retention mechanism" tutorial, section 块级循环): for a chunk of L
// tokens with per-head decay gamma, chunk-local positions j (query) and l (key),
//     O     = (Q K^T (.) D) V + diag(xi) (Q S_prev),   D_jl = gamma^(j-l) for j >= l, xi_j = gamma^(j+1)
//     S_new = gamma^L S_prev + K^T (V (.) zeta),        zeta_l = gamma^(L-1-l)
// Every pair of tokens of one chunk goes through the scores (Q K^T (.) D, rounded to
// bf16 like every matrix operand here); only pairs in different chunks go through the
// state.
//
// Work decomposition: a workgroup owns one (b,h), one segment of the sequence (whole
// chunks) and 128 state columns, and walks the segment's chunks in order, carrying the
// state in fp32 matrix-core accumulators (each of its eight waves holds the 128 x 16
// slice of its 16 columns).  Within a chunk the waves own query rows instead: a pass
// covers 256 query rows, 32 per wave, and a chunk of 512 takes two passes.  The Q blocks
// of a pass sit in LDS from its first step (copied during the previous pass); at that
// step every wave loads its Q fragments and forms its cross term from a bf16 snapshot
// of the chunk's entry state kept in LDS.  The pass then streams the 64-token key
// blocks it needs through LDS from block 0 up; for every block up to the one holding
// its own rows (its diagonal block, its last), a wave forms its scores (K Q^T,
// decayed) in registers and accumulates P V with P taken straight from the score
// accumulators, and after the diagonal block it stores its rows of O.  The chunk's last pass also streams every block through the state
// update.  So each wave reads every K and V fragment it multiplies once per block, the
// scores never pass through LDS, and the key blocks of a chunk are read from memory
// once per pass.
//
// Query rows go to waves so that each SIMD (waves w and w + 4) holds one light and one
// heavy row group: the work of rows near the chunk start is small (few key blocks).

#include "cdna4.h"
#include "chunk_tiles.h"
#include "common.h"
#include "launch.h"

#include <mutex>
#include <type_traits>

namespace retn {

namespace {

constexpr int kWCols = 128;   // state and output columns per workgroup
constexpr int kWWaves = 8;
constexpr int kWDk = 128;

template <int C>
struct WCfg {
    static constexpr int MB = C / kBlk;                  // key blocks per chunk
    static constexpr int R = 32;                         // query rows per wave and pass
    static constexpr int NQT = R / 16;                   // query tiles per wave
    static constexpr int PROWS = kWWaves * R;            // query rows per pass
    static constexpr int PBLK = PROWS / kBlk;            // query blocks per pass
    static_assert(C % PROWS == 0, "passes must tile the chunk");
};

// LDS: two stages of one 64-token block each of K and V (128 columns), the Q blocks of
// one pass (copied a pass ahead), then the bf16 snapshot of the chunk's entry state
// [128 rows][128 columns]: 160 KB.
struct WLds {
    static constexpr int QRB = kWDk * 2, VRB = kWCols * 2;   // row bytes
    static constexpr int kKTile = kBlk * QRB, kVTile = kBlk * VRB, kQTile = kBlk * QRB;
    static constexpr int kK = 0, kV = kKTile;                 // within a K/V stage
    static constexpr int kKV = kKTile + kVTile;               // one K/V stage
    static constexpr int kQ = 2 * kKV;                        // Q block slots of a pass
    static constexpr int kS = kQ + (kWWaves * 32 / kBlk) * kQTile;
    static constexpr int kBytes = kS + kWDk * VRB;
    static_assert(kBytes <= kLdsBytes, "LDS layout too large");
    static_assert(kBytes >= kWDk * kWCols * 4, "the final state is staged through LDS");
};

// Wave w's row group in a pass: light groups 0..3 on waves 0..3, heavy groups 7..4 on
// waves 4..7 (wave w and w + 4 share a SIMD).
__device__ __forceinline__ int row_group(int wave) { return wave < 4 ? wave : 11 - wave; }

template <int C>
__global__ __launch_bounds__(kWWaves * 64, 1) __attribute__((amdgpu_waves_per_eu(2, 2))) void chunkw_kernel(
    const KArgs ka) {
    using Cf = WCfg<C>;
    using L_ = WLds;
    constexpr int NW = kWWaves, DVT = kWCols, DK = kWDk;
    constexpr int QRB = L_::QRB, VRB = L_::VRB;
    constexpr int DT = DK / 16;   // 16-row tiles of the state
    constexpr int KS = DK / 32;   // reduction steps over DK
    constexpr int R = Cf::R, NQT = Cf::NQT, PROWS = Cf::PROWS, PBLK = Cf::PBLK;
    using QCopy = TileCopy<QRB, false, NW>;
    using VCopy = TileCopy<VRB, true, NW>;
    constexpr int kNQ = QCopy::kPerWave, kNV = VCopy::kPerWave;
    constexpr int kNStore = 8 * NQT;   // output stores of a wave at the end of a pass

    const bf16_t* __restrict__ q = ka.q;
    const bf16_t* __restrict__ k = ka.k;
    const bf16_t* __restrict__ v = ka.v;
    bf16_t* __restrict__ o = static_cast<bf16_t*>(ka.o);
    const int H = ka.H, N = ka.N, dv = ka.dv;
    const int nseg = ka.nseg, ndvt = ka.ndvt;
    extern __shared__ __attribute__((aligned(1024))) char smem[];

    // ---- work item (XCD-aware: each XCD takes a contiguous range of work ids)
    int wid = blockIdx.x;
    if (ka.total_groups % 8 == 0) wid = (wid & 7) * (ka.total_groups >> 3) + (wid >> 3);
    const int dvt = wid % ndvt;
    const int seg = (wid / ndvt) % nseg;
    const int bh = wid / (ndvt * nseg);
    const int h = bh % H;

    // the wave index is uniform; readfirstlane lets the compiler keep everything derived
    // from it (row group, query block, activity) in scalar registers and branches
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    const int trj = l16 >> 2, trq = l16 & 3;
    const int col0 = dvt * DVT, wcol = wave * 16;
    const int rg = row_group(wave);

    const int t_begin = seg * ka.seg_tokens;
    const int t_end = min(N, t_begin + ka.seg_tokens);
    const float lg = log2f(ka.decay[h]);

    const size_t qk_bh = static_cast<size_t>(bh) * N * DK;
    const size_t v_bh = static_cast<size_t>(bh) * N * dv;
    const size_t s_bh = static_cast<size_t>(bh) * DK * dv;
    const size_t s_stride_seg = static_cast<size_t>(DK) * dv;
    // ranges end with the last row's own columns; rows past N read as zeros
    const u32x4_t q_rs = make_rsrc(q + qk_bh, static_cast<uint32_t>(N) * DK * 2);
    const u32x4_t k_rs = make_rsrc(k + qk_bh, static_cast<uint32_t>(N) * DK * 2);
    const u32x4_t v_rs = make_rsrc(v + v_bh + col0, static_cast<uint32_t>((N - 1) * dv + dv - col0) * 2);
    const uint32_t lds0 = lds_addr_of(smem);
    QCopy kcp;   // Q and K tiles (same row length and swizzle)
    VCopy vcp;
    kcp.init(DK * 2, wave, lane, N);
    vcp.init(dv * 2, wave, lane, N);
    const uint32_t wofs = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(wave)) * 1024u;

    // State accumulator element (dt, i) of lane (g, l%16) holds state row srow(dt, i) of
    // column col0 + wcol + l%16 (conflict-free K^T transpose reads).
    auto srow = [&](int dt, int i) -> int { return 32 * (dt >> 1) + 8 * g4 + 4 * ((dt ^ g4) & 1) + i; };

    // ---- incoming state: state_in, the scanned entry state, or (fuse_scan) composed here
    f32x4_t S[DT];
    {
        const int cidx = col0 + wcol + l16;
        auto load = [&](const float* src, float scale, bool add) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float x = src[static_cast<uint32_t>(srow(dt, i) * dv + cidx)];
                    S[dt][i] = add ? S[dt][i] * scale + x : x;
                }
        };
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) S[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (nseg == 1 || ka.fuse_scan) {
            int sg0 = 0;
            if (ka.state_in != nullptr) {
                load(ka.state_in + s_bh, 0.f, false);
            } else if (seg > 0) {
                load(ka.seg_state + static_cast<size_t>(bh) * nseg * s_stride_seg, 0.f, false);
                sg0 = 1;
            }
            for (int sg = sg0; nseg > 1 && sg < seg; ++sg)
                load(ka.seg_state + (static_cast<size_t>(bh) * nseg + sg) * s_stride_seg,
                     exp2f(ka.seg_log2[static_cast<size_t>(bh) * nseg + sg]), true);
        } else {
            load(ka.seg_state + (static_cast<size_t>(bh) * nseg + seg) * s_stride_seg, 0.f, false);
        }
    }

    // ---- per-lane LDS read addresses.  Within a 256-byte row the swizzled position of
    // a 16-byte unit is the logical one XOR a per-row pattern, and the tiles start at
    // multiples of 256 bytes, so one base per read family covers all its fragments:
    //   K/Q rows (row tile t, reduction step ks): (ak0 ^ 64 ks) + t*16*QRB (+ kQ - kK for Q);
    //   K^T transposed reads (state tile dt, rows r0 and r0+4, key half kh):
    //     (akt0[pl] ^ 64 (dt/2) ^ 8 (dt%2)) + kh*32*QRB;
    //   V^T reads of column tile c for P V: (avp0 ^ 32 c) + 32 p*VRB (+16 rows);
    //   V^T reads of this wave's column tile for the state update: avs[pl] + kh*32*VRB;
    //   snapshot reads of column tile c: (ass[pl] ^ 32 c) + 32 ks*VRB.
    uint32_t ak0, aq0, akt0[2], avs[2], avp0, ass[2];
    // base ^ x formed at its use by one v_xor (inside the asm, so the compiler neither
    // keeps every variant in a register of its own nor copies the base first)
    auto xa = [](uint32_t base, uint32_t x) -> uint32_t {
        uint32_t r;
        asm volatile("v_xor_b32 %0, %1, %2" : "=v"(r) : "s"(x), "v"(base));
        return r;
    };
    {
        const int s = swz_qk<QRB / 16>(l16);
        ak0 = opaque(lds0 + L_::kK + static_cast<uint32_t>(l16 * QRB + 16 * (4 * (s >> 2) + (g4 ^ (s & 3)))));
        // Q reads: this wave's rows sit in slot rg/2 of the pass's Q blocks, 32 (rg & 1)
        // rows in
        aq0 = opaque(lds0 + L_::kQ + static_cast<uint32_t>((rg >> 1) * L_::kQTile + (32 * (rg & 1) + l16) * QRB +
                                                            16 * (4 * (s >> 2) + (g4 ^ (s & 3)))));
#pragma unroll
        for (int pl = 0; pl < 2; ++pl) {
            const int rb = 8 * g4 + trj + 4 * pl;
            const int w = swz_qk<QRB / 16>(rb);
            akt0[pl] = opaque(lds0 + L_::kK +
                              static_cast<uint32_t>(rb * QRB + 16 * (4 * (w >> 2) + (trq ^ (w & 3))) + 8 * (trq & 1)));
            const int sv = swz_v<VRB / 16>(rb);
            avs[pl] = opaque(lds0 + L_::kV +
                             static_cast<uint32_t>(rb * VRB + 16 * (2 * (wave ^ (sv >> 1)) + (trq >> 1)) + 8 * (trq & 1)));
            ass[pl] = opaque(lds0 + L_::kS +
                             static_cast<uint32_t>(rb * VRB + 32 * (sv >> 1) + 16 * (trq >> 1) + 8 * (trq & 1)));
        }
        const int rbp = 4 * g4 + trj;
        const int gp = swz_v<VRB / 16>(rbp) >> 1;
        avp0 = opaque(lds0 + L_::kV + static_cast<uint32_t>(rbp * VRB + 32 * gp + 16 * (trq >> 1) + 8 * (trq & 1)));
    }
    static_assert(L_::kK % 256 == 0 && L_::kV % 256 == 0 && L_::kQ % 256 == 0 && L_::kS % 256 == 0 &&
                      L_::kKV % 256 == 0 && L_::kQTile % 256 == 0,
                  "tiles must start at multiples of 256 bytes");

    // ---- decays computed once (per head); every exponent is >= 0
    //   fz[i]:  gamma^(31 - 8g - i), the state-update weight of key slot i of a key half;
    //   wd[i]:  score weights of a diagonal tile (gamma^(query - key), 0 above it);
    //   wo[i]:  gamma^(16 + query - key) for a tile one below the diagonal; a tile d
    //           below it takes wo times gamma^(16 (d - 1)).
    float wd[4], wo[4], fz[8];
    const float g32 = exp2_fast(32.f * lg);
#pragma unroll
    for (int i = 0; i < 8; ++i) fz[i] = exp2_fast(static_cast<float>(31 - 8 * g4 - i) * lg);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int dj = l16 - 4 * g4 - i;
        wd[i] = dj < 0 ? 0.f : exp2_fast(static_cast<float>(dj) * lg);
        wo[i] = exp2_fast(static_cast<float>(16 + dj) * lg);
    }

    // The registers hold S / 2^lk2 (a chunk's decay moves lk2, not the accumulators).
    float lk2 = 0.f;

    // ---- the walk: steps (chunk, pass, key block kb from block 0 up to the pass's last)
    struct Pos {
        int cs;   // chunk start
        int p;    // pass
        int kb;   // key block
    };
    auto chunk_len = [&](int cs) -> int { return min(C, t_end - cs); };
    auto pass_top = [&](int cs, int p) -> int {   // the pass's last key block
        const int nb = (chunk_len(cs) + kBlk - 1) / kBlk;
        return min(nb, (p + 1) * PBLK) - 1;
    };
    auto npass = [&](int cs) -> int { return ((chunk_len(cs) + kBlk - 1) / kBlk + PBLK - 1) / PBLK; };
    // the first step of the pass after the one at s; false past the segment end
    auto next_pass = [&](Pos& s) -> bool {
        s.kb = 0;
        if (s.p + 1 < npass(s.cs)) { ++s.p; return true; }
        s.cs += C;
        s.p = 0;
        return s.cs < t_end;
    };
    auto next_pos = [&](Pos& s) -> bool {
        if (s.kb < pass_top(s.cs, s.p)) { ++s.kb; return true; }
        return next_pass(s);
    };

    // copies of the step at s (K and V into stage b), and of the Q blocks of the pass at s
    auto issue_kv = [&](const Pos& s, int b) {
        const uint32_t row0 = static_cast<uint32_t>(s.cs + s.kb * kBlk);
        const uint32_t st = lds0 + b * L_::kKV + wofs;
#pragma unroll
        for (int i = 0; i < kNQ; ++i) kcp.issue_one(i, st + L_::kK, k_rs, row0 * QRB);
#pragma unroll
        for (int i = 0; i < kNV; ++i) vcp.issue_one(i, st + L_::kV, v_rs, row0 * dv * 2);
    };
    auto issue_q = [&](const Pos& s) {
        const int nq = pass_top(s.cs, s.p) - s.p * PBLK + 1;   // query blocks of the pass
#pragma unroll
        for (int j = 0; j < PBLK; ++j) {
            if (j < nq) {
                const uint32_t row0 = static_cast<uint32_t>(s.cs + (s.p * PBLK + j) * kBlk);
                const uint32_t st = lds0 + L_::kQ + j * L_::kQTile + wofs;
#pragma unroll
                for (int i = 0; i < kNQ; ++i) kcp.issue_one(i, st, q_rs, row0 * QRB);
            }
        }
    };
    // the bf16 snapshot of the true state (S * 2^lk2) into LDS, row-major [dk][128]
    // with the V-tile swizzle
    auto write_snapshot = [&]() {
        const float r = exp2_fast(lk2);
        // element (dt, i) sits at row srow(dt, i): the row's low four bits (which fix
        // the swizzle) depend on dt's parity and i only, so eight per-lane addresses
        // (made here, not kept across the walk) plus 32 (dt/2) rows cover them
        const int col = wcol + l16;
#pragma unroll
        for (int par = 0; par < 2; ++par)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 8 * g4 + 4 * ((par ^ g4) & 1) + i;
                const uint32_t a = opaque(lds0 + L_::kS + static_cast<uint32_t>(
                                              row * VRB + (((col >> 3) ^ swz_v<VRB / 16>(row)) << 4) + (col & 7) * 2));
#pragma unroll
                for (int dt = par; dt < DT; dt += 2)
                    *reinterpret_cast<__attribute__((address_space(3))) uint16_t*>(
                        static_cast<size_t>(a + (dt >> 1) * 32 * VRB)) = bf(S[dt][i] * r);
            }
    };

    // ---- prologue: the first step's copies, the entry state's snapshot (every load
    // drains here)
    Pos cur{t_begin, 0, 0};
    Pos p1 = cur;
    bool has1 = next_pos(p1);
    issue_kv(cur, 0);
    issue_q(cur);
    __builtin_amdgcn_s_waitcnt(0);
    write_snapshot();

    f32x4_t O[8][NQT];        // O^T tiles: column tile c, query tile qt of this wave
    u16x8_t qf[NQT][KS];      // this wave's Q fragments in the current pass
    int st = 0;               // stage of the current step
    // this wave issued all kNStore output stores at the end of the last step (full
    // chunks; a partial chunk's masked stores may be skipped, and it waits for all)
    bool stored = false;
    bool q_ahead = true;      // the current pass's Q blocks have been copied
    int cs_prev = -1;

    while (true) {
        // this step's tiles have landed and every wave sees them (the youngest operations
        // may be the previous step's output stores, which need not be complete)
        if (stored) wait_vmcnt<kNStore>();
        else wait_vmcnt<0>();
        lds_barrier();
        stored = false;

        const int L = chunk_len(cur.cs);
        const bool full = L == C;
        if (cur.cs != cs_prev) {
            // start of a chunk: its decay; rescale the registers once the scale gets small
            cs_prev = cur.cs;
            lk2 += static_cast<float>(L) * lg;
            if (lk2 < -64.f) {
                const float r = exp2_fast(lk2);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) S[dt] *= r;
                lk2 = 0.f;
            }
        }
        // a pass of a single step leaves no step for the next pass's Q copies: they go
        // out here, and every wave waits for them
        if (cur.kb == 0 && !q_ahead) {
            issue_q(cur);
            __builtin_amdgcn_s_waitcnt(0);
            lds_barrier();
        }
        q_ahead = false;
        // the next step's K and V (their buffers were last read by the previous step,
        // which every wave has finished); at the pass's second step, once every wave
        // holds its Q fragments, the next pass's Q blocks
        if (has1) issue_kv(p1, st ^ 1);
        if (cur.kb == 1) {
            Pos np = cur;
            if (next_pass(np)) {
                issue_q(np);
                q_ahead = true;
            }
        }

        const int p = cur.p, kb = cur.kb;
        const int qrow0 = p * PROWS + rg * R;     // this wave's first query row (chunk-local)
        const int qb = qrow0 / kBlk;              // its query block
        const bool active = qrow0 < L && kb <= qb;
        // (a wave's rows go through every key block from 0 to its diagonal block qb)
        const bool last_pass = p + 1 == npass(cur.cs);

        if (qrow0 < L && kb == 0) {
            // this wave's Q fragments, and its cross term O^T = diag(xi) applied to S^T Q^T
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    qf[qt][ks] = lds16a(xa(aq0, 64u * ks) + static_cast<uint32_t>(qt * 16 * QRB));
            // snapshot fragments of column tile c (transposed reads, rows 8g + j + 4pl + 32ks)
            auto s_frag = [&](int c, int ks) -> u16x8_t {
                u16x4_t r[2];
#pragma unroll
                for (int pl = 0; pl < 2; ++pl)
                    r[pl] = lds_tra(xa(ass[pl], 32u * c) + static_cast<uint32_t>(32 * ks * VRB));
                return cat(r[0], r[1]);
            };
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                u16x8_t a[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) a[ks] = s_frag(c, ks);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                    for (int qt = 0; qt < NQT; ++qt)
                        O[c][qt] = mfma16(a[ks], qf[qt][ks], ks == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : O[c][qt]);
                __builtin_amdgcn_sched_barrier(0);
            }
            // times xi_j = gamma^(j+1) of each query row j
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt) {
                const float xi = exp2_fast(static_cast<float>(qrow0 + qt * 16 + l16 + 1) * lg);
#pragma unroll
                for (int c = 0; c < 8; ++c) O[c][qt] *= xi;
            }
        }

        if (active) {
            // scores of key block kb against this wave's query tiles, decayed, bf16, and
            // P V -- a pair of key tiles at a time
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
                u16x8_t pb[NQT];
                f32x4_t acc[2][NQT];
#pragma unroll
                for (int hk = 0; hk < 2; ++hk) {
                    const int kt = 2 * pr + hk;
                    // key tiles above every query tile of this wave are all zero
                    const bool any = (qrow0 + (NQT - 1) * 16) / 16 >= kb * 4 + kt;
                    u16x8_t kf[KS];
                    if (any) {
#pragma unroll
                        for (int ks = 0; ks < KS; ++ks) kf[ks] = lds16a(xa(ak0, 64u * ks) + static_cast<uint32_t>(kt * 16 * QRB));
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int qt = 0; qt < NQT; ++qt) {
                        acc[hk][qt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                        if ((qrow0 + qt * 16) / 16 >= kb * 4 + kt) {
#pragma unroll
                            for (int ks = 0; ks < KS; ++ks) acc[hk][qt] = mfma16(kf[ks], qf[qt][ks], acc[hk][qt]);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                // V^T fragments of the first four column tiles go out before the weights
                u16x8_t va[4];
                auto v_frag = [&](int c) -> u16x8_t {
                    const uint32_t b = xa(avp0, 32u * c);
                    return cat(lds_tra(b + static_cast<uint32_t>(pr * 32 * VRB)),
                               lds_tra(b + static_cast<uint32_t>((pr * 32 + 16) * VRB)));
                };
#pragma unroll
                for (int c = 0; c < 4; ++c) va[c] = v_frag(c);
#pragma unroll
                for (int qt = 0; qt < NQT; ++qt) {
                    u16x4_t half[2];
#pragma unroll
                    for (int hk = 0; hk < 2; ++hk) {
                        // tile distance (query tile - key tile) in 16-row units
                        const int d = (qrow0 + qt * 16) / 16 - (kb * 4 + 2 * pr + hk);
                        float w[4];
                        if (d > 0) {
                            const float u = exp2_fast(static_cast<float>(16 * (d - 1)) * lg);
#pragma unroll
                            for (int i = 0; i < 4; ++i) w[i] = wo[i] * u;
                        } else {
#pragma unroll
                            for (int i = 0; i < 4; ++i) w[i] = d == 0 ? wd[i] : 0.f;
                        }
                        const f32x4_t a = acc[hk][qt];
                        half[hk] = bf4(f32x4_t{a[0] * w[0], a[1] * w[1], a[2] * w[2], a[3] * w[3]});
                    }
                    pb[qt] = cat(half[0], half[1]);
                }
                // X^T += V^T P^T over this key pair: slots {4g..4g+3} of key tiles 2pr, 2pr+1
#pragma unroll
                for (int cg = 0; cg < 2; ++cg) {
                    if (cg == 1) {
#pragma unroll
                        for (int c = 0; c < 4; ++c) va[c] = v_frag(4 + c);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int c = 0; c < 4; ++c)
#pragma unroll
                        for (int qt = 0; qt < NQT; ++qt) O[cg * 4 + c][qt] = mfma16(va[c], pb[qt], O[cg * 4 + c][qt]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }

        if (last_pass) {
            // S += K^T (V (.) zeta) over key block kb; zeta_l = gamma^(L-1-l) / 2^lk2
            const float zs = exp2_fast(-lk2);
            const float ub = full ? exp2_fast(static_cast<float>(C - kBlk - kb * kBlk) * lg) * zs : 0.f;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                auto kt_frag = [&](int dt) -> u16x8_t {
                    const uint32_t off = kh * 32 * QRB;
                    const uint32_t x = 64u * (dt >> 1) + 8u * (dt & 1);
                    return cat(lds_tra(xa(akt0[0], x) + off), lds_tra(xa(akt0[1], x) + off));
                };
                constexpr int G = 4;
                u16x8_t kcur[G], knext[G];
                const u16x8_t raw = cat(lds_tra(avs[0] + kh * 32 * VRB), lds_tra(avs[1] + kh * 32 * VRB));
#pragma unroll
                for (int j = 0; j < G; ++j) kcur[j] = kt_frag(j);
                __builtin_amdgcn_sched_barrier(0);
                float z[8];
                if (full) {
                    // slot i of key half kh: gamma^(31 - 8g - i) times the half's factor
                    const float hf = kh == 0 ? ub * g32 : ub;
#pragma unroll
                    for (int i = 0; i < 8; ++i) z[i] = fz[i] * hf;
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int l = kb * kBlk + kh * 32 + 8 * g4 + i;
                        z[i] = l < L ? exp2_fast(static_cast<float>(L - 1 - l) * lg - lk2) : 0.f;
                    }
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
                        for (int j = 0; j < G; ++j) knext[j] = kt_frag(g0 + G + j);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int j = 0; j < G; ++j) S[g0 + j] = mfma16(kcur[j], bv, S[g0 + j]);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int j = 0; j < G; ++j) kcur[j] = knext[j];
                }
            }
        }

        // after its diagonal block, this wave's rows of O (rows past the chunk end skipped)
        if (kb == qb && qrow0 < L) {
            bf16_t* const base = o + v_bh + static_cast<size_t>(cur.cs + qrow0) * dv + col0;
            // per-lane element offset, made here (not kept across the walk)
            const uint32_t lo = opaque(static_cast<uint32_t>(l16 * dv + 4 * g4));
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt) {
                const int row = qt * 16 + l16;
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    if (qrow0 + row < L)
                        *reinterpret_cast<u16x4_t*>(base + (lo + static_cast<uint32_t>(qt * 16 * dv + c * 16))) =
                            bf4(O[c][qt]);
                }
            }
            stored = full;
        }

        if (!has1) break;
        if (kb == pass_top(cur.cs, p) && last_pass) {
            // end of the chunk: every wave is past its cross-term reads of the snapshot;
            // the next chunk's snapshot goes in (published by the next step's barrier)
            lds_barrier();
            write_snapshot();
        }
        cur = p1;
        has1 = next_pos(p1);
        st ^= 1;
        // the read bases move to the stage of the next step
        {
            const uint32_t dkv = st != 0 ? static_cast<uint32_t>(L_::kKV) : static_cast<uint32_t>(-L_::kKV);
            ak0 += dkv;
            akt0[0] += dkv;
            akt0[1] += dkv;
            avs[0] += dkv;
            avs[1] += dkv;
            avp0 += dkv;
        }
    }

    // ---- final state (last segment only), through LDS in whole rows of 16-byte stores
    if (seg == nseg - 1 && ka.state_out != nullptr) {
        float* const st = reinterpret_cast<float*>(smem);
        const float r = exp2_fast(lk2);
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

template <int C>
hipError_t launch_cw(const KArgs& ka, hipStream_t stream) {
    constexpr size_t lds = WLds::kBytes;
    static std::once_flag attr_once;   // thread-safe one-time init of the LDS limit
    std::call_once(attr_once, [] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&chunkw_kernel<C>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    });
    ProfScope prof(kProfMain, stream);
    hipLaunchKernelGGL((chunkw_kernel<C>), dim3(ka.total_groups), dim3(kWWaves * 64), lds, stream, ka);
    return hipGetLastError();
}

}  // namespace

// Chunks of 128 stay on the general kernel, which measured faster there (one key block
// below the diagonal leaves too little work per step for this walk's fixed costs).
bool chunkw_supported(int dk, int dv, int chunk, int ldqk, int ldv, int slices, bool out_f32, bool reverse,
                      bool gated) {
    return (chunk == 256 || chunk == 512) && dk == kWDk && dv % kWCols == 0 && ldqk == dk &&
           ldv == dv && slices <= 1 && !out_f32 && !reverse && !gated;
}

hipError_t launch_chunkw(const KArgs& ka, hipStream_t stream) {
    if (ka.dk != kWDk) return hipErrorInvalidValue;
    switch (ka.C) {
        case 256: return launch_cw<256>(ka, stream);
        case 512: return launch_cw<512>(ka, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace retn
