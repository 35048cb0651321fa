/*
 * retention.h -- C ABI of the MI355X (gfx950) retention operator library
 *                (libretention_fwd.so).
 *
 * The operator is RetNet's retention.  Per (batch b, head h) it carries a state
 * S in R^{dk x dv} through the sequence:
 *
 *     S_n = lambda_n * S_{n-1} + k_n^T v_n,        o_n = q_n S_n
 *
 * with lambda_n = gamma_h (one decay per head) or lambda_n = exp(g[b,h,n]) (gated,
 * per-token log-decay).  Sources, cited by page title and section:
 *   - "RetNet retention mechanism" tutorial (aiqz.cc), section 递归推理: the
 *     recurrence above; section 衰减矩阵: D_nm = gamma^(n-m) for n >= m, else 0;
 *     section 并行训练: (Q K^T (.) D) V; section 块级循环: the chunkwise form --
 *     parallel inside a chunk, the state relayed across chunks.
 *   - "Retentive Network (RetNet) 详解" (171host.com), section 3.1: the three
 *     equivalent forms (recurrent, parallel, chunkwise recurrent).
 *   - "unilm RetNet 技术指南 ... YOCO 中 Gated RetNet 的源码解析" (pwwt.cn), sections
 *     GateRetention 模块的内部结构 (log-decay gate), 三种计算路径与增量状态 (the
 *     one-token path with a constant-size state; prefill seeding the decode state)
 *     and Triton 内核与自校验测试 (chunk-end decays for the cross-chunk state).
 *
 * Conventions shared by every entry point
 *   Layout     All tensors are dense, row-major, contiguous, in DEVICE memory:
 *                q, k   [B, H, N, dk]     v, o  [B, H, N, dv]
 *                gamma  [H]  fp32         g     [B, H, N]  fp32
 *                state  [B, H, dk, dv] fp32
 *              q, k, v and o share one element type, RETN_F32 or RETN_BF16;
 *              gamma, g and states are always fp32.  Accumulation is fp32; a bf16
 *              output is rounded to nearest-even.
 *   Ownership  The caller allocates and owns every buffer.  The library keeps no
 *              pointer after a call returns and allocates no device memory.
 *   Streams    Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *              and the call returns without synchronising.
 *   Errors     Arguments are validated before anything is enqueued; on any error
 *              nothing is launched and nothing is written.  A failed launch returns
 *              RETN_ERR_HIP.  Faults inside kernels surface at the caller's next
 *              synchronisation.  Nothing is printed.
 *   Domain     gamma in (0, 1] (gamma = 1 is undecayed linear attention); g finite
 *              and <= 0.  Values are not scanned on the device.
 *   Sizes      B, H, N >= 0 (B*H*N = 0 is a valid empty call: state_out, if given,
 *              receives state_in or zeros); dk in [1, 256], dv in [1, 1024]; chunk >= 1.  The bf16 matrix-core path is used when dk is
 *              64, 128 or 256, dv is a multiple of 64 (<= 1024), chunk <= 512,
 *              q, k, v, o (and state_out, when given) are 16-byte aligned and one head's rows span less than
 *              2^31 bytes ((N + 64) * max(dk, dv) * 2 < 2^31); every other shape in
 *              range runs on the generic kernels.
 *              A ragged last chunk (N not a multiple of chunk) is computed exactly;
 *              there is no padding.
 */
#ifndef RETENTION_FWD_H
#define RETENTION_FWD_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RETN_OK = 0,
    RETN_ERR_NULL = 1,         /* a required pointer is NULL                        */
    RETN_ERR_SHAPE = 2,        /* a size is negative or out of range                */
    RETN_ERR_DTYPE = 3,        /* unknown element type                              */
    RETN_ERR_UNSUPPORTED = 4,  /* valid but not implemented (e.g. dk > 256)         */
    RETN_ERR_WORKSPACE = 5,    /* workspace missing, too small or misaligned        */
    RETN_ERR_ALIAS = 6,        /* an output overlaps an input                       */
    RETN_ERR_HIP = 7,          /* the HIP runtime reported an error at launch       */
    /* Not statuses: they widen the type's range to every int, so that any int a
       caller passes (e.g. to retention_status_string) is a valid value of it. */
    RETN_STATUS_RANGE_MIN_ = -2147483647 - 1,
    RETN_STATUS_RANGE_MAX_ = 2147483647
} retn_status;

typedef enum {
    RETN_F32 = 0,
    RETN_BF16 = 1,
    /* Not element types: every int is a valid value of the type (others are
       rejected with RETN_ERR_DTYPE). */
    RETN_DTYPE_RANGE_MIN_ = -2147483647 - 1,
    RETN_DTYPE_RANGE_MAX_ = 2147483647
} retn_dtype;

/*
 * Chunkwise-recurrent retention forward with one decay per head.
 *
 * Computes, for every (b, h), the outputs o_n = q_n S_n of the recurrence above with
 * lambda_n = gamma[h], evaluated in chunks of `chunk` tokens: inside a chunk the
 * parallel form (Q K^T (.) D) V with D_jl = gamma^(j-l) (j >= l), across chunks the
 * state, decayed by gamma^L for a chunk of L tokens, with the cross-chunk query
 * term weighted per row by gamma^(j+1) (tutorial, sections 衰减矩阵 and 块级循环).
 *
 *   q, k, v     inputs, element type `dtype`, layout above
 *   gamma       [H] fp32 per-head decays
 *   o           output [B,H,N,dv], element type `dtype`; must not overlap any input
 *   state_in    optional [B,H,dk,dv] fp32 initial state (NULL = zeros); it is decayed
 *               by the first token's lambda like any state
 *   state_out   optional [B,H,dk,dv] fp32 final state S_N (NULL = not written); may
 *               equal state_in (in-place update) but must not overlap q/k/v/o
 *   chunk       chunk size in tokens (>= 1); changes rounding only, not the result
 *   workspace   device scratch of at least retention_workspace_bytes(...) bytes,
 *               16-byte aligned (may be NULL when that is 0; RETN_ERR_WORKSPACE when
 *               it is needed and missing, smaller or misaligned); contents need not be
 *               initialised
 *   stream      hipStream_t to enqueue on
 */
retn_status retention_chunkwise_fwd(const void* q, const void* k, const void* v,
                                    const float* gamma, void* o,
                                    const float* state_in, float* state_out,
                                    int B, int H, int N, int dk, int dv, int chunk,
                                    retn_dtype dtype, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * Gated chunkwise retention forward: per-token, per-head log-decay g[B,H,N] (fp32,
 * g <= 0).  The weight of token m in output n >= m is exp(G_n - G_m) with G the
 * inclusive cumulative sum of g along the sequence, and the incoming state reaches
 * output n with weight exp(G_n) (pwwt.cn guide, sections GateRetention 模块的内部结构
 * and Triton 内核与自校验测试).  Other arguments as retention_chunkwise_fwd.
 */
retn_status gated_retention_chunkwise_fwd(const void* q, const void* k, const void* v,
                                          const float* g, void* o,
                                          const float* state_in, float* state_out,
                                          int B, int H, int N, int dk, int dv, int chunk,
                                          retn_dtype dtype, void* workspace,
                                          size_t workspace_bytes, void* stream);

/*
 * Parallel-form retention forward, the short-sequence training path (tutorial, section
 * 并行训练: O = (Q K^T (.) D) V with D[n,m] = gamma^(n-m) for n >= m, else 0; pwwt.cn
 * guide, section 三种计算路径与增量状态, names it as the first of the three paths).  No
 * state in or out and no workspace.  The result is the chunkwise forward's with a zero
 * initial state.  bf16 with dk in {64, 128, 256} and dv a multiple of 64 (<= 1024) runs
 * every 64-token query block of a (b,h) in its own workgroup; other shapes and fp32 take
 * the generic kernel.  Arguments as retention_chunkwise_fwd.
 */
retn_status retention_parallel_fwd(const void* q, const void* k, const void* v,
                                   const float* gamma, void* o,
                                   int B, int H, int N, int dk, int dv,
                                   retn_dtype dtype, void* stream);

/*
 * Gated parallel form: D[n,m] = exp(G_n - G_m) for n >= m with G the inclusive cumulative
 * sum of g (pwwt.cn guide, section 三种计算路径与增量状态, its parallel path).  The
 * matrix-core kernel keeps G of the whole sequence in LDS, so it takes N <= 512; longer
 * bf16 sequences and fp32 take the generic kernel (N <= 1024 is not required there).
 * Arguments as gated_retention_chunkwise_fwd without state and workspace.
 */
retn_status gated_retention_parallel_fwd(const void* q, const void* k, const void* v,
                                         const float* g, void* o,
                                         int B, int H, int N, int dk, int dv,
                                         retn_dtype dtype, void* stream);

/*
 * One recurrent decode step (tutorial, section 递归推理):
 *     S <- gamma[h] S + k^T v   (fp32, in place),   o = q S   (with the updated S)
 *   q, k   [B,H,dk]  v, o [B,H,dv]  element type `dtype`
 *   state  [B,H,dk,dv] fp32, read and overwritten; must not overlap q/k/v/o
 * Needs no workspace.
 */
retn_status retention_decode_step(const void* q, const void* k, const void* v,
                                  const float* gamma, float* state, void* o,
                                  int B, int H, int dk, int dv,
                                  retn_dtype dtype, void* stream);

/*
 * One gated decode step: S <- exp(g[b,h]) S + k^T v, o = q S (pwwt.cn guide, section
 * 三种计算路径与增量状态: the previous state scaled by the decay, then the new
 * k^T v added).  g is [B,H] fp32.  Other arguments as retention_decode_step.
 */
retn_status gated_retention_decode_step(const void* q, const void* k, const void* v,
                                        const float* g, float* state, void* o,
                                        int B, int H, int dk, int dv,
                                        retn_dtype dtype, void* stream);

/*
 * Backward of retention_chunkwise_fwd: the gradients of
 *     L = <grad_o, o> + <grad_state_out, state_out>
 * with respect to q, k, v and state_in, for the recurrence S_n = gamma S_{n-1} + k_n^T v_n,
 * o_n = q_n S_n (tutorial, section 递归推理; the chain rule on that recurrence, which the
 * pwwt.cn guide, section Triton 内核与自校验测试, runs as a backward recurrence).
 *   q, k, v, gamma, state_in   the forward call's inputs (state_in NULL = zeros)
 *   grad_o          [B,H,N,dv], element type `dtype`
 *   grad_state_out  optional [B,H,dk,dv] fp32 (NULL = zeros)
 *   grad_q, grad_k  [B,H,N,dk] and grad_v [B,H,N,dv], element type `dtype`
 *   grad_state_in   optional [B,H,dk,dv] fp32 (NULL = not written)
 *   chunk           chunk size of the passes (changes rounding only)
 *   workspace       16-byte aligned scratch of at least retention_bwd_workspace_bytes(...)
 *                   bytes; contents need not be initialised
 * Outputs must not overlap any input or each other (RETN_ERR_ALIAS).  Computed as
 * forward passes of the chunkwise kernels: grad_q is a forward pass over (grad_o, v, k),
 * grad_v and grad_k are forward passes that walk (k, q, grad_o) and (v, grad_o, q) from
 * the last token to the first, in place.  Shapes as the forward; for dv > 256 (bf16 only)
 * dv must be a multiple of 64, the tensors 16-byte aligned and
 * (N + 64) * max(dk, dv) * 2 < 2^31, else RETN_ERR_UNSUPPORTED.
 */
retn_status retention_chunkwise_bwd(const void* q, const void* k, const void* v,
                                    const float* gamma, const float* state_in,
                                    const void* grad_o, const float* grad_state_out,
                                    void* grad_q, void* grad_k, void* grad_v,
                                    float* grad_state_in,
                                    int B, int H, int N, int dk, int dv, int chunk,
                                    retn_dtype dtype, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * Backward of gated_retention_chunkwise_fwd; additionally writes grad_g [B,H,N] fp32,
 * the gradient with respect to the log-decays g (required).  Other arguments as
 * retention_chunkwise_bwd.
 */
retn_status gated_retention_chunkwise_bwd(const void* q, const void* k, const void* v,
                                          const float* g, const float* state_in,
                                          const void* grad_o, const float* grad_state_out,
                                          void* grad_q, void* grad_k, void* grad_v,
                                          float* grad_g, float* grad_state_in,
                                          int B, int H, int N, int dk, int dv, int chunk,
                                          retn_dtype dtype, void* workspace,
                                          size_t workspace_bytes, void* stream);

/*
 * Gated multi-scale retention layer forward (YOCO's gated RetNet mixer: pwwt.cn guide,
 * section GateRetention 模块的内部结构, with the k scaling of section 三种计算路径与增量状态):
 *     q, k, v, g, gt = x Wq^T, x Wk^T, x Wv^T, x Wg^T, x Wgt^T     (no biases)
 *     q, k <- rotation of adjacent pairs (2i, 2i+1) of token n by n * rope_base^(-2i/dk)
 *     k <- k / sqrt(dk);   decay = logsigmoid(gt) / 16   [B,H,N]
 *     o = gated_retention_chunkwise_fwd(q, k, v, decay)   (zero initial state)
 *     y = (silu(g) * RMSNorm_eps(o per head, over dv)) Wo^T
 *   x        [B,N,D] bf16;   y [B,N,D] bf16, must not overlap any input
 *   wq, wk   [H*dk, D];  wv, wg [H*dv, D];  wgt [H, D];  wo [D, H*dv]   (bf16,
 *            [out_features, in_features], contiguous, 16-byte aligned)
 *   chunk    chunk size of the retention call;  rope_base > 1;  norm_eps >= 0
 *   workspace  16-byte aligned scratch of at least gated_msr_workspace_bytes(...) bytes
 * Supported: dk in {64, 128, 256}, dv a multiple of 64 (<= 1024), D a multiple of 64,
 * chunk <= 512, (N + 64) * max(dk, dv) * 2 < 2^31; else RETN_ERR_UNSUPPORTED.  The projections run on a
 * bf16 matrix-core GEMM with fp32 accumulation; q, k, v, g enter the operator in bf16, the
 * retention output stays fp32 through the normalisation.
 */
retn_status gated_msr_fwd(const void* x, const void* wq, const void* wk, const void* wv,
                          const void* wg, const void* wgt, const void* wo, void* y,
                          int B, int N, int D, int H, int dk, int dv, int chunk,
                          float rope_base, float norm_eps, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * Bytes of workspace gated_msr_fwd needs for these sizes; 0 for unsupported sizes.
 */
size_t gated_msr_workspace_bytes(int B, int N, int D, int H, int dk, int dv, int chunk);

/*
 * Bytes of workspace the backward entry points need for these sizes (sized for an
 * initial state and a final-state gradient being given); 0 for invalid or unsupported
 * sizes, which the entry point then reports.
 */
size_t retention_bwd_workspace_bytes(int B, int H, int N, int dk, int dv, int chunk,
                                     retn_dtype dtype, int gated);

/*
 * Bytes of workspace the chunkwise entry points need for these sizes (0 when the
 * sequence is not split across workgroups).  gated: 0 = per-head gamma, 1 = gated.
 * Returns 0 for invalid sizes as well; the entry point then reports the error.
 */
size_t retention_workspace_bytes(int B, int H, int N, int dk, int dv, int chunk,
                                 retn_dtype dtype, int gated);

/* Static, human-readable name of a status code (never NULL). */
const char* retention_status_string(retn_status status);

/* Version of this ABI (incremented on any signature change). */
int retention_abi_version(void);

/*
 * Kernel timing for benchmarks (not needed for computing anything).
 * retention_profile_enable(1) starts recording: every kernel the library launches
 * afterwards is bracketed by two HIP events on its stream (up to 4096 launches
 * between read-outs; later ones are counted as dropped).  The first enable creates
 * the events on the current device; use one device and one host thread while
 * timing.  retention_profile_enable(0) stops recording.
 * retention_profile_read waits for the recorded launches, writes for each kernel kind
 * i < nkinds the summed milliseconds ms[i] and the launch count count[i], writes the
 * number of dropped launches to *dropped (if not NULL) and clears the records.
 * Kinds: 0 matrix-core chunkwise pass, 1 its segment-state pre-pass, 2 its segment
 * scan, 3 generic chunkwise kernel, 4 decode step, 5 state copy (empty sequence).
 * Errors: RETN_ERR_SHAPE (nkinds < 0), RETN_ERR_NULL, RETN_ERR_HIP.
 */
retn_status retention_profile_enable(int on);
retn_status retention_profile_read(double* ms, int* count, int nkinds, int* dropped);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, serving
 * loops and harnesses that forbid hipMalloc): retention_chunkwise_fwd without the
 * workspace arguments.  The segment-state scratch that retention_chunkwise_fwd takes
 * from the caller's workspace comes instead from a device array of the library, of
 * RETN_NOALLOC_SCRATCH_BYTES per device, which each device the library runs on holds
 * until the process ends (its address is looked up once per device; nothing is
 * allocated or freed).  Every call on a device shares that device's array and it keeps
 * the last call's contents (no call needs it zeroed: each writes what it reads):
 * calls that overlap on one device -- on different streams or threads, or inside one
 * graph without a dependency between them -- race and give wrong results.
 *   Arguments, layout, results and errors: as retention_chunkwise_fwd, plus
 *   RETN_ERR_WORKSPACE when the call would need more scratch than
 *   RETN_NOALLOC_SCRATCH_BYTES (retention_workspace_bytes(..., gated = 0) tells), and
 *   RETN_ERR_HIP when the stream's device cannot be determined.
 */
#define RETN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
retn_status retention_chunkwise_fwd_noalloc(const void* q, const void* k, const void* v,
                                            const float* gamma, void* o,
                                            const float* state_in, float* state_out,
                                            int B, int H, int N, int dk, int dv, int chunk,
                                            retn_dtype dtype, void* stream);

/*
 * Measurement helper, not part of the operator: an achievable-peak reference for the
 * bf16 matrix cores.  Launches `blocks` workgroups of `waves` waves (1..8) on `stream`;
 * each wave runs `iters` rounds of 16 independent v_mfma_f32_16x16x32_bf16 products
 * with no memory traffic and writes one float per wave to out[blocks * waves] (device
 * memory, caller-owned; the values are of no interest).  The caller times the launch;
 * retention_calib_mfma_flops returns the flops it performs.
 * Errors: RETN_ERR_NULL (out), RETN_ERR_SHAPE (sizes out of range), RETN_ERR_HIP.
 */
retn_status retention_calib_mfma(float* out, int blocks, int waves, int iters, void* stream);
double retention_calib_mfma_flops(int blocks, int waves, int iters);

#ifdef __cplusplus
}
#endif

#endif /* RETENTION_FWD_H */
