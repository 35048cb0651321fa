// Backward of the chunkwise retention forward, as forward passes of the same kernels.
//
// The loss is L = <dO, o> + <dS, S_N> for the recurrence S_n = lam_n S_{n-1} + k_n^T v_n,
// o_n = q_n S_n, S_{-1} = S0 ("RetNet retention mechanism" tutorial, section 递归推理; the
// gated multiplier lam_n = exp(g_n) as in "unilm RetNet 技术指南", section 三种计算路径与增量
// 状态).  The chain rule gives the adjoint U_n = dL/dS_n,
//     U_{N-1} = q_{N-1}^T dO_{N-1} + dS,   U_n = q_n^T dO_n + lam_{n+1} U_{n+1},
// and dq_n = S_n dO_n, dk_n = U_n v_n, dv_n = U_n^T k_n, dS0 = lam_0 U_0,
// dg_n = lam_n <U_n, S_{n-1}>.  Each of these is a retention forward pass:
//   * dq: the forward recurrence with (q, k, v) -> (dO, v, k) and initial state S0^T
//     (its state is S_n^T, so its outputs are dO_n S_n^T = dq_n^T, and its final state
//     is S_N^T);
//   * dv, dk: the adjoint recurrence, a forward walk over the time-reversed sequence
//     (the kernels' reversed mode: walk position m is token N-1-m and decays by lam of
//     token N-m), with (q, k, v) -> (k, q, dO) for dv and (v, dO, q) for dk, starting
//     from dS (dS^T for dk).  The dv pass ends with U_0 and writes lam_0 U_0 = dS0;
//   * dg (gated): dg_n = sum_{p >= n} (q_p . dq_p - k_p . dk_p) + <dS, S_N>, since the
//     log-decay enters only through the cumulative sums G.
// When d_v exceeds the widest score width of the kernels (256), the dq and dk passes
// (whose scores run over d_v) are split into column slices of d_v, read in place with a
// row stride, run as extra chains of one launch, and their outputs summed.

#include "launch.h"

#include <stdint.h>

namespace retn {

// bandwidth kernels (bwd_kernels.hip)
hipError_t launch_rows_combine(const void* a, const void* b, void* out, size_t bh, int N, int w, bool bf16,
                               hipStream_t s, bool in_f32 = false, bool out_f32 = false);
bool convert_dot_supported(int w, const void* g, const void* g2, const void* x, const void* out);
hipError_t launch_convert_dot(const float* g, const float* g2, const void* x, void* out, float* dG, size_t bh, int N,
                              int w, float sign, bool accumulate, hipStream_t s);
hipError_t launch_state_transpose(const float* src0, float* dst0, const float* src1, float* dst1, size_t bh, int dk,
                                  int dv, int parts, hipStream_t s);
hipError_t launch_gate_rows(const void* q, const void* dq, const void* k, const void* dkk, float* dG, size_t bh,
                            int N, int dk, bool bf16, hipStream_t s);
hipError_t launch_gate_scan(const float* dG, const float* A, const float* B, int dk, int dv, int parts, float* dg,
                            size_t bh, int N, hipStream_t s);

namespace {

constexpr int kMaxScoreWidth = 256;       // widest d_k of the forward kernels
constexpr int kGenericMaxDk = 256;
constexpr int kGenericMaxGatedChunk = 1024;

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Which kernel runs a forward pass of score width dkp and value width dvp.
enum PassKind { kNone = 0, kMfma = 1, kGeneric = 2 };

// rows_ok: a head's rows fit the matrix-core kernels' 32-bit byte offsets (signed for
// the reversed walks).
PassKind pass_kind(const BwdShape& s, int dkp, int dvp, bool strided, bool aligned, bool rows_ok) {
    if (s.bf16 && mfma_chunk_supported(dkp, dvp, s.chunk, true) && aligned && rows_ok) return kMfma;
    if (strided) return kNone;
    if (dkp > kGenericMaxDk) return kNone;
    if (s.gated && s.chunk > kGenericMaxGatedChunk) return kNone;
    return kGeneric;
}

int split_parts(int dv) {
    if (dv <= kMaxScoreWidth) return 1;
    for (int w : {256, 128, 64})
        if (dv % w == 0) return dv / w;
    return 0;
}

}  // namespace

BwdPlan bwd_plan(const BwdShape& s, const BwdPtrs* ptrs) {
    BwdPlan p{};
    p.ok = false;
    const size_t bh = static_cast<size_t>(s.B) * s.H;
    const size_t tokens = bh * s.N;
    const size_t es = s.bf16 ? 2 : 4;
    p.parts = split_parts(s.dv);
    if (p.parts == 0) return p;
    p.w = s.dv / p.parts;
    const bool strided = p.parts > 1;
    // user tensors read or written by the matrix-core passes must be 16-byte aligned
    bool aligned = true;
    if (ptrs != nullptr) {
        const void* const all[] = {ptrs->q, ptrs->k, ptrs->v, ptrs->dout, ptrs->dq, ptrs->dk, ptrs->dv};
        for (const void* x : all) aligned = aligned && al16(x);
    }
    const bool rows_ok = (static_cast<size_t>(s.N) + 64) * std::max(s.dk, s.dv) * 2 < (static_cast<size_t>(1) << 31);
    p.kind_q = pass_kind(s, p.w, s.dk, strided, aligned, rows_ok);   // dq: scores over d_v
    p.kind_v = pass_kind(s, s.dk, s.dv, false, aligned, rows_ok);    // dv: scores over d_k
    p.kind_k = pass_kind(s, p.w, s.dk, strided, aligned, rows_ok);   // dk: scores over d_v
    if (p.kind_q == kNone || p.kind_v == kNone || p.kind_k == kNone) return p;
    size_t fwd = 0;
    if (s.N > 0 && bh > 0) {
        if (p.kind_q == kMfma || p.kind_k == kMfma)
            fwd = std::max(fwd, mfma_chunk_plan(s.B, s.H * p.parts, s.N, p.w, s.dk, s.chunk, s.gated).workspace_bytes);
        if (p.kind_v == kMfma) fwd = std::max(fwd, mfma_chunk_plan(s.B, s.H, s.N, s.dk, s.dv, s.chunk, s.gated).workspace_bytes);
    }
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align256(bytes);
        return o;
    };
    const size_t sbytes = bh * s.dk * s.dv * sizeof(float);
    if (tokens == 0) {   // no passes run
        p.ok = true;
        return p;
    }
    p.off_fwd = take(fwd);
    p.fwd_bytes = fwd;
    p.off_s0t = take(s.has_s0 ? sbytes : 0);
    p.off_dst = take(s.has_ds ? sbytes : 0);
    p.off_sfin = take(s.gated && s.has_ds ? sbytes : 0);
    p.off_dG = take(s.gated ? tokens * sizeof(float) : 0);
    // gated bf16 on the matrix cores: dq and dk are accumulated in fp32, since the gate
    // gradient subtracts their dot products with q and k; the dot products are taken
    // while the fp32 values are converted to the outputs
    p.f32acc = s.gated && s.bf16 && p.kind_q == kMfma && p.kind_k == kMfma &&
               convert_dot_supported(s.dk, nullptr, nullptr, nullptr, nullptr);
    if (p.f32acc && ptrs != nullptr)
        p.f32acc = al16(ptrs->q) && al16(ptrs->k) && al16(ptrs->dq) && al16(ptrs->dk);
    // unsplit 128 x 128 heads in 64-token chunks: the single-block pass forms the dots
    // itself from its fp32 accumulators and writes dq and dk as bf16 directly
    p.rowdot = p.f32acc && p.parts == 1 && chunk1_dot_supported(p.w, s.dk, s.chunk);
    if (p.rowdot) p.f32acc = false;
    // the slices of a dq or dk pass (one slice of fp32 when unsplit for the gate gradient)
    p.off_sl = take(p.parts > 1 || p.f32acc ? p.parts * tokens * s.dk * (p.f32acc ? sizeof(float) : es) : 0);
    p.total = off;
    p.ok = true;
    return p;
}

namespace {

// One forward pass on the kernel the plan chose.
// Row dots of a pass's output (gated, see ChunkArgs::xdot).
struct RowDot {
    const void* x;
    float* dG;
    float sign;
    bool accumulate;
};

hipError_t forward_pass(const BwdShape& s, int kind, const void* q, const void* k, const void* v,
                        const float* decay, void* o, const float* state_in, float* state_out, int dkp, int dvp,
                        void* ws, size_t ws_bytes, hipStream_t st, bool rev, bool out_f32,
                        const RowDot* rd = nullptr, int st_ld = 0, bool seg_t = false) {
    ChunkArgs a{q, k, v, decay, o, state_in, state_out, s.B, s.H, s.N, dkp, dvp, s.chunk, s.bf16, s.gated, ws,
                ws_bytes};
    a.out_f32 = out_f32;
    a.reverse = rev;
    a.state_in_ld = st_ld;
    a.seg_from_t = seg_t;
    if (rd != nullptr) {
        a.xdot = rd->x;
        a.dG = rd->dG;
        a.dsign = rd->sign;
        a.dacc = rd->accumulate;
    }
    if (kind == kMfma) return launch_mfma_chunk(a, mfma_chunk_plan(s.B, s.H, s.N, dkp, dvp, s.chunk, s.gated), st);
    return launch_generic_chunk(a, st);
}

// A pass whose scores run over d_v, split into P column slices of width w run as extra
// chains of one matrix-core launch; slice p's output goes to o + p * tokens * dk.
hipError_t sliced_pass(const BwdShape& s, const BwdPlan& p, int kind, const void* q, const void* k, const void* v,
                       const float* decay, void* o, const float* state_in, float* state_out, void* ws, hipStream_t st,
                       bool rev, bool out_f32, const RowDot* rd = nullptr, int st_ld = 0, bool seg_t = false) {
    if (p.parts == 1)
        return forward_pass(s, kind, q, k, v, decay, o, state_in, state_out, p.w, s.dk, ws, p.fwd_bytes, st, rev,
                            out_f32, rd, st_ld, seg_t);
    if (rd != nullptr || seg_t) return hipErrorInvalidValue;   // row dots and shared states: whole rows
    const size_t tokens = static_cast<size_t>(s.B) * s.H * s.N;
    ChunkArgs a{q, k, v, decay, o, state_in, state_out, s.B, s.H, s.N, p.w, s.dk, s.chunk, s.bf16, s.gated, ws,
                p.fwd_bytes};
    a.ldqk = s.dv;
    a.out_f32 = out_f32;
    a.reverse = rev;
    a.slices = p.parts;
    a.slice_qk = p.w;
    a.slice_o = tokens * s.dk;
    a.slice_state = static_cast<size_t>(s.B) * s.H * p.w * s.dk;
    a.state_in_ld = st_ld;
    return launch_mfma_chunk(a, mfma_chunk_plan(s.B, s.H * p.parts, s.N, p.w, s.dk, s.chunk, s.gated), st);
}

// Per head, the dq and dk passes can read S0 and dS transposed in place (no transpose
// launch) when the single-block pass runs them with no separate scan.  Gated, the gate
// gradient pairs dS^T with the dq pass's final state in the transposed layout, so the
// transposes stay.
bool transposed_in_place(const BwdShape& s, const BwdPlan& p) {
    if (s.gated || p.kind_q != kMfma || p.kind_k != kMfma || p.f32acc || p.rowdot) return false;
    ChunkArgs a{};
    a.B = s.B;
    a.H = s.H;
    a.N = s.N;
    a.dk = p.w;
    a.dv = s.dk;
    a.chunk = s.chunk;
    a.bf16 = s.bf16;
    a.ldqk = p.parts > 1 ? s.dv : 0;
    a.slices = p.parts;
    return chunk1_takes(a, mfma_chunk_plan(s.B, s.H * p.parts, s.N, p.w, s.dk, s.chunk, s.gated));
}

}  // namespace

hipError_t run_backward(const BwdShape& s, const BwdPtrs& x, const BwdPlan& p, void* workspace, hipStream_t st) {
    const size_t bh = static_cast<size_t>(s.B) * s.H;
    if (bh == 0) return hipSuccess;
    const size_t sper = static_cast<size_t>(s.dk) * s.dv;
    if (s.N == 0) {   // no tokens: S_N = S0, so dS0 = dS
        if (x.dstate_in == nullptr) return hipSuccess;
        return launch_copy_state(x.dstate_out, x.dstate_in, bh * sper, st);
    }
    char* ws = static_cast<char*>(workspace);
    void* fws = ws + p.off_fwd;
    float* s0t = reinterpret_cast<float*>(ws + p.off_s0t);
    float* dst = reinterpret_cast<float*>(ws + p.off_dst);
    float* sfin = reinterpret_cast<float*>(ws + p.off_sfin);
    float* dG = reinterpret_cast<float*>(ws + p.off_dG);
    char* sl = ws + p.off_sl;
    const size_t tokens = bh * s.N;
    const int P = p.parts;
    const bool has_s0 = x.state_in != nullptr, has_ds = x.dstate_out != nullptr;
    const bool f32 = p.f32acc;
    // where a dq or dk pass writes: straight to the output when unsplit and not kept in fp32
    const bool direct = P == 1 && !f32;
    const size_t slice_bytes = tokens * s.dk * (f32 ? sizeof(float) : (s.bf16 ? 2 : 4));
    hipError_t e;
#define RETN_TRY(call)             \
    do {                           \
        e = (call);                \
        if (e != hipSuccess) return e; \
    } while (0)
    // the slices of a pass summed into its output (fp32 slices: with the gate gradient's
    // row dot products against xdot, added to dG with the given sign)
    auto finish = [&](void* out, const void* xdot, float sign, bool accumulate) -> hipError_t {
        if (direct) return hipSuccess;
        hipError_t r;
        if (f32) {
            for (int pi = 2; pi < P; ++pi)
                if ((r = launch_rows_combine(sl, sl + pi * slice_bytes, sl, bh, s.N, s.dk, s.bf16, st, true, true)) !=
                    hipSuccess)
                    return r;
            return launch_convert_dot(reinterpret_cast<const float*>(sl),
                                      P > 1 ? reinterpret_cast<const float*>(sl + slice_bytes) : nullptr, xdot, out, dG,
                                      bh, s.N, s.dk, sign, accumulate, st);
        }
        if ((r = launch_rows_combine(sl, sl + slice_bytes, out, bh, s.N, s.dk, s.bf16, st)) != hipSuccess) return r;
        for (int pi = 2; pi < P; ++pi)
            if ((r = launch_rows_combine(out, sl + pi * slice_bytes, out, bh, s.N, s.dk, s.bf16, st)) != hipSuccess)
                return r;
        return hipSuccess;
    };

    // transposed states in d_v slices: S0^T (dq pass), dS^T (dk pass), in one launch, unless
    // the passes read them transposed in place
    const bool tin = transposed_in_place(s, p);
    const int st_ld = tin ? s.dv : 0;
    if (!tin)
        RETN_TRY(launch_state_transpose(has_s0 ? x.state_in : nullptr, s0t, has_ds ? x.dstate_out : nullptr, dst, bh,
                                        s.dk, s.dv, P, st));
    const float* const s0_in = has_s0 ? (tin ? x.state_in : s0t) : nullptr;
    const float* const ds_in = has_ds ? (tin ? x.dstate_out : dst) : nullptr;

    // ---- dq = forward(dO, v, k) from S0^T; its final state is S_N^T (gated, with dS);
    // row dots: dG = q . dq
    const RowDot rdq{x.q, dG, 1.f, false}, rdk{x.k, dG, -1.f, true};
    RETN_TRY(sliced_pass(s, p, p.kind_q, x.dout, x.v, x.k, x.decay, direct ? x.dq : sl, s0_in,
                         s.gated && has_ds ? sfin : nullptr, fws, st, false, f32, p.rowdot ? &rdq : nullptr, st_ld));
    RETN_TRY(finish(x.dq, x.q, 1.f, false));

    // ---- dv = forward(k, q, dO) walking backwards from dS; it ends with dS0 = lam_0 U_0
    RETN_TRY(forward_pass(s, p.kind_v, x.k, x.q, x.dout, x.decay, x.dv, x.dstate_out, x.dstate_in, s.dk, s.dv, fws,
                          p.fwd_bytes, st, true, false));

    // ---- dk = forward(v, dO, q) walking backwards from dS^T.  Its state is U^T, so where
    // both passes split the sequence alike, the segment states the dv pass left in the
    // workspace serve it transposed and it runs no pre-pass of its own.
    const bool share = P == 1 && p.kind_v == kMfma && p.kind_k == kMfma &&
                       seg_shareable(s.B, s.H, s.N, s.dv, s.dk, s.chunk, s.gated, f32);
    RETN_TRY(sliced_pass(s, p, p.kind_k, x.v, x.dout, x.q, x.decay, direct ? x.dk : sl, ds_in, nullptr, fws, st, true,
                         f32, p.rowdot ? &rdk : nullptr, st_ld, share));
    RETN_TRY(finish(x.dk, x.k, -1.f, true));

    // ---- gated: dg = reversed cumulative sum of q.dq - k.dk, plus <dS, S_N> = <dS^T, S_N^T>
    if (s.gated) {
        if (!f32 && !p.rowdot) RETN_TRY(launch_gate_rows(x.q, x.dq, x.k, x.dk, dG, bh, s.N, s.dk, s.bf16, st));
        RETN_TRY(launch_gate_scan(dG, has_ds ? dst : nullptr, sfin, s.dk, s.dv, P, x.dg, bh, s.N, st));
    }
#undef RETN_TRY
    return hipSuccess;
}

}  // namespace retn
