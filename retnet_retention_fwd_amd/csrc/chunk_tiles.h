// Shared pieces of the matrix-core chunkwise kernels: 64-token LDS blocks, the
// conflict-free row swizzles, asynchronous tile copies global -> LDS, the order of the
// 16 score tiles of a block, and the kernel argument block.
#pragma once

#include "cdna4.h"
#include "common.h"

namespace retn {

// Kernel arguments (one struct, passed by value).
struct KArgs {
    const bf16_t* q;
    const bf16_t* k;
    const bf16_t* v;
    const float* decay;      // gamma [H] or g [B,H,N]
    void* o;                 // bf16, or fp32 for the fp32-output variant
    const float* state_in;   // [B,H,dk,dv] or null (zeros)
    float* state_out;        // [B,H,dk,dv] or null
    float* seg_state;        // workspace [B*H][nseg][dk][dv]: local, then (scanned) entry states
    float* seg_log2;         // workspace [B*H][nseg]: log2 of each segment's total decay
    int H, N, dk, dv, C;
    int ldqk, ldv;           // row strides (elements) of q and k, and of v; o is contiguous
    int seg_tokens, nseg;    // sequence split: tokens per segment, segments per (b,h)
    int ndvt, ndkt;          // column tiles and (pre-pass) state-row tiles per (b,h)
    int total_groups;
    int fuse_scan;           // main pass: compose the entry state from the local states
    // column slices run as extra chains: chain c is (b,h) = c / nsl and slice c % nsl,
    // whose q/k rows start sl_qk elements further, whose output starts sl_o elements
    // further and whose state_in / state_out start sl_state floats further
    int nsl, sl_qk;
    size_t sl_o, sl_state;
    // two segments, the second of which first walks the tokens before it state-only
    // (64-token chunks only): segment 0 covers [0, pre_tokens), segment 1 the rest;
    // 0 = segments of seg_tokens each
    int pre_tokens;
    // row dots (single-block pass, gated backward): dG[token] = (dacc ? dG[token] : 0) +
    // dsign * <output row, xdot row>, taken from the fp32 accumulators; xdot rows have dv
    // elements, contiguous per (b,h)
    const bf16_t* xdot;
    float* dG;
    float dsign;
    int dacc;
    // norm-gate output (single-block pass, gated layer): instead of o, z = silu(gate) * o *
    // (mean(o^2) + eps)^(-1/2) per row, bf16, gate and z in [B, N, H, dv] layout
    const bf16_t* ng_gate;
    bf16_t* ng_out;
    float ng_eps;
    // single-block pass: > 0 means state_in is the caller's [B*H][dv][st_ld] state read
    // transposed in place (slice p's element (r, c) is row c, column p * dk + r)
    int st_ld;
    // single-block pass: 1 means seg_state holds the segment states of the transposed
    // problem (d_k and d_v exchanged), read transposed (element (r, c) at c * d_k + r)
    int seg_t;
};


namespace {

constexpr int kBlk = 64;       // tokens per LDS block
constexpr int kMaxChunk = 512;

// Row swizzles: the 16-byte unit u of row r is stored at unit u ^ swz(r).  LDS serves
// 256 bytes per clock from 64 four-byte banks: a 16-byte-per-lane read in groups of 16
// lanes, an 8-byte (or 8-byte transpose) read in groups of 32 lanes; a group is
// conflict free when its lanes cover distinct banks.
//   Q and K (row = token, units over the head dimension): score and cross-term reads
//   take one unit from 16 consecutive rows, so swz must be distinct on them; the
//   transposed K reads of the state update take 8 bytes from rows {0..3, 8..11} (or
//   {4..7, 12..15}) with the two 8-byte halves alternating over the lanes of a row, so
//   rows of such a set must land in distinct 32-byte pairs (or opposite halves).
//   With 16+ units per row, swz(r) = r with bits 1 and 2 exchanged does both; with 8
//   units per row (two rows per bank cycle), (r >> 1) & 7.
//   V (row = token, units over state columns): transposed reads take one 32-byte pair
//   from rows {0..7} (P V) or {0..3, 8..11} (state update), so swz = 2 g(r) with
//   g(r) = (r & 3) | (bit 2 ^ bit 3 of r) << 2 is distinct on both; with 8 units per
//   row, 2 (g(r) >> 1).
template <int UPR>
__device__ __forceinline__ int swz_qk(int r) {
    if (UPR >= 16) return (r & 9) | ((r & 4) >> 1) | ((r & 2) << 1);
    return (r >> 1) & 7;
}
template <int UPR>
__device__ __forceinline__ int swz_v(int r) {
    const int g = (r & 3) | ((((r >> 2) ^ (r >> 3)) & 1) << 2);
    return UPR >= 16 ? 2 * g : 2 * (g >> 1);
}

constexpr int kLdsBytes = 160 * 1024;   // LDS per workgroup on gfx950
constexpr int kPBytes = 4 * 2 * 64 * 16;   // P fragments [4 qt][2 key pairs][64 lanes][16 B]

// A buffer offset past every range this file builds (ranges stay below 2^31 bytes for
// reversed walks): loads from it return zeros.
constexpr uint32_t kOutOfRange = 0x80000000u;

// Asynchronous copy of one 64-row tile (row bytes RB) of a row-major matrix with row
// stride `sb` bytes.  Each wave issues kChunks/4 instructions of 1 KB; lane l of
// instruction i fills LDS bytes [c*1024 + 16 l, +16) with c = wave + 4 i, i.e. row
// (c*1024 + 16 l) / RB and the 16-byte unit whose swizzled position that is.
// REV: the walk runs over the time-reversed sequence, so LDS row r of the block at
// walk position t0 holds matrix row N-1-t0-r.
template <int RB, bool VSWZ, int NW, bool REV = false>
struct TileCopy {
    static constexpr int kChunks = kBlk * RB / 1024;
    static constexpr int kPerWave = kChunks / NW;
    static_assert(kChunks % NW == 0, "tile must split evenly over the waves");
    // byte offset of this lane's unit relative to the block's first row; REV: the
    // offset of row N-1-r (negative, as a two's complement, when r > N-1)
    uint32_t voff[kPerWave];

    __device__ __forceinline__ void init(int sb, int wave, int lane, int N) {
#pragma unroll
        for (int i = 0; i < kPerWave; ++i) {
            const int c = wave + i * NW;
            const int off = c * 1024 + lane * 16;
            const int r = off / RB, p = (off % RB) >> 4;
            const int u = p ^ (VSWZ ? swz_v<RB / 16>(r) : swz_qk<RB / 16>(r));
            voff[i] = static_cast<uint32_t>((REV ? N - 1 - r : r) * sb + u * 16);
        }
        (void)N;
    }
    // Offset and wave-uniform base of copy i for the block at row0 (bytes row0*sb).
    // Forward: the base carries the block; REV: the lane offset does.  A row before the
    // sequence start has a negative offset, which as a 32-bit unsigned value lies at or
    // above 2^31, past every range (ranges stay below 2^31 bytes), so it reads as zeros.
    __device__ __forceinline__ uint32_t lane_off(int i, uint32_t row0_bytes) const {
        return REV ? voff[i] - row0_bytes : voff[i];
    }
    __device__ __forceinline__ static uint32_t base_off(uint32_t row0_bytes) { return REV ? 0u : row0_bytes; }
    // Rows past the end of the tensor lie outside the buffer's range and land in LDS
    // as zeros, so every LDS row holds finite data; uses mask those rows.
    __device__ __forceinline__ void issue(uint32_t tile_lds, const u32x4_t& rsrc, uint32_t row0_bytes,
                                          int wave) const {
        const uint32_t base = tile_lds + static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(wave)) * 1024u;
#pragma unroll
        for (int i = 0; i < kPerWave; ++i)
            buf2lds16(rsrc, lane_off(i, row0_bytes), base_off(row0_bytes), base + i * NW * 1024u);
    }
    // copy i of this wave alone; wbase = tile_lds + 1024 * wave
    __device__ __forceinline__ void issue_one(int i, uint32_t wbase, const u32x4_t& rsrc, uint32_t row0_bytes) const {
        buf2lds16(rsrc, lane_off(i, row0_bytes), base_off(row0_bytes), wbase + i * NW * 1024u);
    }
};
// The 16 score tiles of a 64x64 block as qt*4+kt, causal (kt <= qt) ones first:
// 0,4,5,8,9,10,12,13,14,15, then 1,2,3,6,7,11 (one 4-bit entry per slot).
__device__ __forceinline__ int tile_order(int slot) {
    return static_cast<int>((0xB76321FEDCA98540ULL >> (4 * slot)) & 15);
}

}  // namespace
}  // namespace retn
