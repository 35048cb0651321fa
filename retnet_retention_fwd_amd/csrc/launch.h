// Internal launcher interface between the C ABI (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include <algorithm>

namespace retn {

// Arguments of one chunkwise forward call, already validated.
struct ChunkArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* decay;        // gamma [H] (per head) or g [B,H,N] (gated)
    void* o;
    const float* state_in;     // may be null (zeros)
    float* state_out;          // may be null
    int B, H, N, dk, dv, chunk;
    bool bf16;
    bool gated;
    void* workspace;
    size_t workspace_bytes;
    // Row strides in elements of q and k (shared) and of v; 0 = contiguous (dk, dv).
    // Only the matrix-core path takes other strides (column slices of wider rows).
    int ldqk = 0;
    int ldv = 0;
    // Matrix-core path, gated shapes: write o as fp32 instead of bf16.
    bool out_f32 = false;
    // Walk the time-reversed sequence (the backward's adjoint recurrence): position m
    // reads and writes token N-1-m and takes the decay of token N-m (gated: g[N-m], 0 at
    // m = 0; per head: gamma, with state_in entering divided by gamma); state_out
    // leaves multiplied by the decay of token 0.
    bool reverse = false;
    // Matrix-core path: `slices` column slices of the score operands in one launch, each
    // an independent chain per (b,h) (plan with H * slices heads).  Slice p reads q and k
    // from column p * slice_qk (with the row stride ldqk), writes o from element
    // p * slice_o, and takes state_in / state_out from float p * slice_state.
    int slices = 1;
    int slice_qk = 0;
    size_t slice_o = 0, slice_state = 0;
    // Gated backward, single-block pass with one 128-column tile per row: besides the bf16
    // output, dG[token] = (dacc ? dG[token] : 0) + dsign * <fp32 output row, xdot row>,
    // xdot in the layout of o ([B,H,N,dv] bf16), dG [B,H,N].
    const void* xdot = nullptr;
    float* dG = nullptr;
    float dsign = 1.f;
    bool dacc = false;
    // Gated layer, single-block pass with one 128-column tile per row, forward: instead of
    // o, z[b, n, h, :] = silu(gate[b, n, h, :]) * o_n * (mean(o_n^2) + ng_eps)^(-1/2) as bf16
    // (gate and z in the layer's [B, N, H, dv] layout; o is not written).
    const void* ng_gate = nullptr;
    void* ng_out = nullptr;
    float ng_eps = 0.f;
    // > 0: state_in is a [B*H][dv][state_in_ld] state (the caller's layout of a pass that
    // works on the transposed state in d_k slices) read transposed in place; only where
    // chunk1_takes() says the single-block pass runs the call with no separate scan.
    int state_in_ld = 0;
    // The workspace already holds the segment states (local, or scanned entry states) that
    // an earlier call with this call's plan wrote for the transposed problem: d_k and d_v
    // exchanged, same decays, direction, segments and state_in (transposed), one slice.
    // This call skips its pre-pass and scan and reads them transposed; single-block pass
    // only (seg_shareable()).
    bool seg_from_t = false;
};

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* decay;        // gamma [H] or g [B,H]
    float* state;
    void* o;
    int B, H, dk, dv;
    bool bf16;
    bool gated;
};

// Generic kernels (any in-range shape, fp32 or bf16 elements).
size_t generic_chunk_lds_bytes(int dk, int chunk, bool gated);
hipError_t launch_generic_chunk(const ChunkArgs& a, hipStream_t stream);
hipError_t launch_copy_state(const float* src, float* dst, size_t n, hipStream_t stream);

// Matrix-core (MFMA) bf16 chunkwise path.
bool mfma_chunk_supported(int dk, int dv, int chunk, bool bf16);
// Plan of the sequence split: segments per (b,h) and the workspace it needs.
struct MfmaPlan {
    int seg_chunks;   // chunks per segment (each workgroup walks one segment)
    int nseg;         // segments per (b,h)
    int dvt;          // state columns per workgroup
    int nw;           // waves per workgroup
    int pre_dkt;      // state rows per workgroup of the segment-state pre-pass
    int pre_dvt;      // state columns per workgroup of the pre-pass
    int fuse_scan;    // 1: the main pass composes segment entry states itself
    // > 0: two segments split at this token; the second segment's workgroups walk the
    // first segment's tokens state-only before their own (no pre-pass, no workspace)
    int prefix_tokens;
    size_t workspace_bytes;
};
// A call with 64-token chunks runs on the single-block main pass (below) whenever that
// supports it, and can then take a prefix split instead of a pre-pass.
MfmaPlan mfma_chunk_plan(int B, int H, int N, int dk, int dv, int chunk, bool gated);
hipError_t launch_mfma_chunk(const ChunkArgs& a, const MfmaPlan& plan, hipStream_t stream);
// Main pass for chunks of exactly 64 tokens (chunk64.hip): d_k 128 or 256, d_v a
// multiple of 128, row strides multiples of 8 elements, any slices, either walk
// direction, fp32 output when gated.
struct KArgs;
bool chunk1_supported(int dk, int dv, int chunk, int ldqk, int ldv, int slices, bool out_f32, bool gated);
// the row-dot form (ChunkArgs::xdot): gated, d_k = d_v = 128, one slice
bool chunk1_dot_supported(int dk, int dv, int chunk);
// The call runs on the single-block pass and its entry states need no separate scan (so
// it can take ChunkArgs::state_in_ld).
bool chunk1_takes(const ChunkArgs& a, const MfmaPlan& p);
// A call of shape (B, H, N, dk, dv) can take ChunkArgs::seg_from_t from a call of the
// transposed shape (dk and dv exchanged) on the same workspace: both plans split the
// sequence into the same segments with a pre-pass, and this call runs on the
// single-block pass.
bool seg_shareable(int B, int H, int N, int dk, int dv, int chunk, bool gated, bool out_f32);
hipError_t launch_chunk1(const KArgs& ka, bool gated, bool reverse, bool out_f32, bool dot, hipStream_t stream);
// Main pass for chunks of 256 or 512 tokens (chunkw.hip): forward, per-head decays,
// bf16 output, contiguous rows, one slice, d_k 128, d_v a multiple of 128.
bool chunkw_supported(int dk, int dv, int chunk, int ldqk, int ldv, int slices, bool out_f32, bool reverse,
                      bool gated);
hipError_t launch_chunkw(const KArgs& ka, hipStream_t stream);
// Parallel form on the matrix cores (no state): O = (Q K^T (.) D) V with the query blocks
// of a (b,h) in parallel workgroups.
bool mfma_parallel_supported(int dk, int dv, int N, bool gated, bool bf16);
hipError_t launch_mfma_parallel(const ChunkArgs& a, hipStream_t stream);

// Decode step.
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// Backward of the chunkwise forward (backward.cpp): forward passes plus bandwidth kernels.
struct BwdShape {
    int B, H, N, dk, dv, chunk;   // chunk already clipped to N
    bool bf16, gated;
    bool has_s0, has_ds;          // an initial state / a final-state gradient is given
};
struct BwdPtrs {
    const void *q, *k, *v;
    const float* decay;           // gamma [H] or g [B,H,N]
    const float* state_in;        // may be null
    const void* dout;
    const float* dstate_out;      // may be null
    void *dq, *dk, *dv;
    float* dstate_in;             // may be null
    float* dg;                    // gated only
};
struct BwdPlan {
    bool ok;                      // every forward pass has a kernel
    int parts, w;                 // split of d_v for the passes whose scores run over d_v
    int kind_q, kind_v, kind_k;   // kernel of each pass (1 matrix-core, 2 generic)
    size_t fwd_bytes;             // workspace of the largest forward pass
    bool f32acc;                  // gated bf16: the dq and dk passes write fp32 (for dg)
    bool rowdot;                  // gated bf16 instead: they write bf16 and the row dots of dg
    // workspace offsets: forward-pass workspace, S0^T, dS^T, S_N^T, q.dq - k.dk, and the
    // d_v slices of a dq or dk pass
    size_t off_fwd, off_s0t, off_dst, off_sfin, off_dG, off_sl;
    size_t total;                 // workspace bytes
};
// ptrs may be null (workspace query): matrix-core passes then assume aligned tensors.
BwdPlan bwd_plan(const BwdShape& s, const BwdPtrs* ptrs);
hipError_t run_backward(const BwdShape& s, const BwdPtrs& x, const BwdPlan& p, void* workspace, hipStream_t st);

// Matrix-core GEMM C = A W^T (bf16 A [M,K], W [N,K], contiguous; fp32 accumulation;
// bf16 or fp32 C [M,N]); K % 64 == 0 and N % 8 == 0 (msr.hip).
bool gemm_tn_supported(int N, int K);
hipError_t launch_gemm_tn(const void* a, const void* w, void* c, int M, int N, int K, bool out_f32,
                          hipStream_t stream);

// Gated multi-scale retention layer (msr.hip).
struct MsrShape {
    int B, N, D, H, dk, dv, chunk;
    float rope_base, norm_eps;
};
struct MsrPtrs {
    const void *x, *wq, *wk, *wv, *wg, *wgt, *wo;
    void* y;
};
struct MsrPlan {
    bool ok;
    int chunk;
    MfmaPlan ret;   // the retention call's plan
    // workspace: cos/sin table, q, k, v, gate projection, log decays, retention output,
    // gated product, the retention call's workspace
    size_t off_rot, off_q, off_k, off_v, off_gp, off_g, off_o, off_z, off_ret;
    size_t total;   // workspace bytes
};
MsrPlan msr_plan(const MsrShape& s);
hipError_t run_msr(const MsrShape& s, const MsrPtrs& x, const MsrPlan& p, void* workspace, hipStream_t st);

// Optional per-kernel timing (HIP events around each launch, see profile.cpp).
enum ProfKind { kProfMain = 0, kProfPre = 1, kProfScan = 2, kProfGeneric = 3, kProfDecode = 4, kProfCopy = 5,
                kProfKinds = 6 };
bool prof_enabled();
hipError_t prof_enable(bool on);
hipError_t prof_read(double* ms, int* count, int nkinds, int* dropped);
// Records a begin event at construction and an end event at destruction when timing
// is on; place it around one kernel launch.
class ProfScope {
public:
    ProfScope(int kind, hipStream_t stream);
    ~ProfScope();
    ProfScope(const ProfScope&) = delete;
    ProfScope& operator=(const ProfScope&) = delete;

private:
    int slot_;
    hipStream_t stream_;
};

}  // namespace retn
