// C ABI of the retention library: argument validation and dispatch to the kernels.
//
// Every entry point validates all of its arguments before it touches the HIP runtime;
// on an error it returns a status and enqueues nothing.  See include/retention.h for
// the contract of each function.

#include "../../include/retention.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace {

constexpr int kMaxDk = 256;           // dk limit (state slice in LDS / registers)
constexpr int kMaxDv = 1024;          // dv limit
constexpr int kGenericMaxGatedChunk = 1024;  // chunk-local cumsum kept in LDS
constexpr int kParallelGenericChunk = 64;    // chunk of the generic kernel for the parallel form

struct Range {
    uintptr_t lo, hi;   // [lo, hi)
};

Range span(const void* p, size_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + bytes};
}

bool overlaps(Range a, Range b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

size_t elem_bytes(retn_dtype dt) { return dt == RETN_BF16 ? 2 : 4; }

bool valid_dtype(retn_dtype dt) { return dt == RETN_F32 || dt == RETN_BF16; }

// Shared validation of the chunkwise entry points.
retn_status validate_chunk(const void* q, const void* k, const void* v, const float* decay,
                           const void* o, const float* state_in, const float* state_out, int B,
                           int H, int N, int dk, int dv, int chunk, retn_dtype dt, bool gated) {
    if (!valid_dtype(dt)) return RETN_ERR_DTYPE;
    if (B < 0 || H < 0 || N < 0 || dk < 1 || dv < 1 || chunk < 1) return RETN_ERR_SHAPE;
    if (dk > kMaxDk || dv > kMaxDv) return RETN_ERR_UNSUPPORTED;
    const size_t bh = static_cast<size_t>(B) * H;
    if (bh > static_cast<size_t>(INT32_MAX)) return RETN_ERR_SHAPE;
    const size_t tokens = bh * N;
    if (tokens > 0 && (q == nullptr || k == nullptr || v == nullptr || o == nullptr || decay == nullptr))
        return RETN_ERR_NULL;
    const size_t es = elem_bytes(dt);
    const Range rq = span(q, tokens * dk * es), rk = span(k, tokens * dk * es),
                rv = span(v, tokens * dv * es), ro = span(o, tokens * dv * es);
    const Range rd = span(decay, (gated ? tokens : static_cast<size_t>(H)) * sizeof(float));
    const size_t sbytes = bh * dk * dv * sizeof(float);
    const Range rsi = span(state_in, state_in ? sbytes : 0), rso = span(state_out, state_out ? sbytes : 0);
    if (overlaps(ro, rq) || overlaps(ro, rk) || overlaps(ro, rv) || overlaps(ro, rd) ||
        overlaps(ro, rsi) || overlaps(ro, rso))
        return RETN_ERR_ALIAS;
    if (state_out != nullptr) {
        if (overlaps(rso, rq) || overlaps(rso, rk) || overlaps(rso, rv) || overlaps(rso, rd))
            return RETN_ERR_ALIAS;
        // in-place (state_out == state_in) is allowed; a partial overlap is not
        if (overlaps(rso, rsi) && static_cast<const void*>(state_out) != static_cast<const void*>(state_in))
            return RETN_ERR_ALIAS;
    }
    return RETN_OK;
}

// Chunks longer than the sequence are one chunk of N tokens.
int effective_chunk(int N, int chunk) { return N > 0 ? (chunk < N ? chunk : N) : 1; }

// The matrix-core kernels move 16-byte units of q, k, v and store 8-byte units of o.
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The matrix-core kernels address a head's rows with 32-bit byte offsets; longer
// heads take the generic kernel, which indexes in 64 bits.
bool use_mfma(int N, int dk, int dv, int eff_chunk, retn_dtype dt) {
    if ((static_cast<size_t>(N) + 64) * std::max(dk, dv) * 2 >= (static_cast<size_t>(1) << 31)) return false;
    return retn::mfma_chunk_supported(dk, dv, eff_chunk, dt == RETN_BF16);
}

size_t workspace_for(int B, int H, int N, int dk, int dv, int chunk, retn_dtype dt, bool gated) {
    const int c = effective_chunk(N, chunk);
    if (B <= 0 || H <= 0 || N <= 0 || !use_mfma(N, dk, dv, c, dt)) return 0;
    return retn::mfma_chunk_plan(B, H, N, dk, dv, c, gated).workspace_bytes;
}

retn_status chunk_common(const void* q, const void* k, const void* v, const float* decay, void* o,
                         const float* state_in, float* state_out, int B, int H, int N, int dk,
                         int dv, int chunk, retn_dtype dt, void* workspace, size_t workspace_bytes,
                         void* stream, bool gated) {
    retn_status st = validate_chunk(q, k, v, decay, o, state_in, state_out, B, H, N, dk, dv, chunk,
                                    dt, gated);
    if (st != RETN_OK) return st;
    const int eff_chunk = effective_chunk(N, chunk);
    // (the matrix-core kernels write state_out and the segment states in 16-byte units)
    const bool mfma = use_mfma(N, dk, dv, eff_chunk, dt) && aligned16(q) && aligned16(k) && aligned16(v) &&
                      aligned16(o) && (state_out == nullptr || aligned16(state_out));
    // The generic kernel keeps a gated chunk's cumulative decays in LDS.
    if (!mfma && gated && eff_chunk > kGenericMaxGatedChunk) return RETN_ERR_UNSUPPORTED;
    size_t need = 0;
    retn::MfmaPlan plan{};
    if (mfma && B > 0 && H > 0 && N > 0) {
        plan = retn::mfma_chunk_plan(B, H, N, dk, dv, eff_chunk, gated);
        need = plan.workspace_bytes;
    }
    if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
        return RETN_ERR_WORKSPACE;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t bh = static_cast<size_t>(B) * H;
    if (bh == 0) return RETN_OK;
    if (N == 0) {
        const hipError_t e = retn::launch_copy_state(state_in, state_out, bh * dk * dv, s);
        return e == hipSuccess ? RETN_OK : RETN_ERR_HIP;
    }
    retn::ChunkArgs a{q, k, v, decay, o, state_in, state_out, B, H, N, dk, dv, eff_chunk,
                      dt == RETN_BF16, gated, workspace, workspace_bytes};
    const hipError_t e = mfma ? retn::launch_mfma_chunk(a, plan, s) : retn::launch_generic_chunk(a, s);
    return e == hipSuccess ? RETN_OK : RETN_ERR_HIP;
}

// Parallel form: the matrix-core kernel over whole-sequence query blocks, else the
// generic kernel, which evaluates the same function chunk by chunk.
retn_status parallel_common(const void* q, const void* k, const void* v, const float* decay, void* o, int B, int H,
                            int N, int dk, int dv, retn_dtype dt, void* stream, bool gated) {
    retn_status st = validate_chunk(q, k, v, decay, o, nullptr, nullptr, B, H, N, dk, dv, 1, dt, gated);
    if (st != RETN_OK) return st;
    const size_t bh = static_cast<size_t>(B) * H;
    if (bh == 0 || N == 0) return RETN_OK;
    const bool mfma = retn::mfma_parallel_supported(dk, dv, N, gated, dt == RETN_BF16) && aligned16(q) &&
                      aligned16(k) && aligned16(v) && aligned16(o);
    const int chunk = mfma ? N : std::min(N, kParallelGenericChunk);
    retn::ChunkArgs a{q, k, v, decay, o, nullptr, nullptr, B, H, N, dk, dv, chunk, dt == RETN_BF16, gated, nullptr, 0};
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = mfma ? retn::launch_mfma_parallel(a, s) : retn::launch_generic_chunk(a, s);
    return e == hipSuccess ? RETN_OK : RETN_ERR_HIP;
}

retn_status decode_common(const void* q, const void* k, const void* v, const float* decay,
                          float* state, void* o, int B, int H, int dk, int dv, retn_dtype dt,
                          void* stream, bool gated) {
    if (!valid_dtype(dt)) return RETN_ERR_DTYPE;
    if (B < 0 || H < 0 || dk < 1 || dv < 1) return RETN_ERR_SHAPE;
    if (dk > kMaxDk || dv > kMaxDv) return RETN_ERR_UNSUPPORTED;
    const size_t bh = static_cast<size_t>(B) * H;
    if (bh > static_cast<size_t>(INT32_MAX)) return RETN_ERR_SHAPE;
    if (bh == 0) return RETN_OK;
    if (q == nullptr || k == nullptr || v == nullptr || decay == nullptr || state == nullptr ||
        o == nullptr)
        return RETN_ERR_NULL;
    const size_t es = elem_bytes(dt);
    const Range rq = span(q, bh * dk * es), rk = span(k, bh * dk * es), rv = span(v, bh * dv * es),
                ro = span(o, bh * dv * es);
    const Range rd = span(decay, (gated ? bh : static_cast<size_t>(H)) * sizeof(float));
    const Range rs = span(state, bh * dk * dv * sizeof(float));
    if (overlaps(ro, rq) || overlaps(ro, rk) || overlaps(ro, rv) || overlaps(ro, rd) || overlaps(ro, rs))
        return RETN_ERR_ALIAS;
    if (overlaps(rs, rq) || overlaps(rs, rk) || overlaps(rs, rv) || overlaps(rs, rd))
        return RETN_ERR_ALIAS;
    retn::DecodeArgs a{q, k, v, decay, state, o, B, H, dk, dv, dt == RETN_BF16, gated};
    const hipError_t e = retn::launch_decode(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? RETN_OK : RETN_ERR_HIP;
}

// Shared validation and dispatch of the backward entry points.
retn_status bwd_common(const void* q, const void* k, const void* v, const float* decay, const float* state_in,
                       const void* grad_o, const float* grad_state_out, void* grad_q, void* grad_k, void* grad_v,
                       float* grad_state_in, float* grad_g, int B, int H, int N, int dk, int dv, int chunk,
                       retn_dtype dt, void* workspace, size_t workspace_bytes, void* stream, bool gated) {
    if (!valid_dtype(dt)) return RETN_ERR_DTYPE;
    if (B < 0 || H < 0 || N < 0 || dk < 1 || dv < 1 || chunk < 1) return RETN_ERR_SHAPE;
    if (dk > kMaxDk || dv > kMaxDv) return RETN_ERR_UNSUPPORTED;
    const size_t bh = static_cast<size_t>(B) * H;
    if (bh > static_cast<size_t>(INT32_MAX)) return RETN_ERR_SHAPE;
    const size_t tokens = bh * N;
    if (tokens > 0 && (q == nullptr || k == nullptr || v == nullptr || decay == nullptr || grad_o == nullptr ||
                       grad_q == nullptr || grad_k == nullptr || grad_v == nullptr || (gated && grad_g == nullptr)))
        return RETN_ERR_NULL;
    const size_t es = elem_bytes(dt);
    const size_t sbytes = bh * dk * dv * sizeof(float);
    const Range in[] = {span(q, tokens * dk * es), span(k, tokens * dk * es), span(v, tokens * dv * es),
                        span(decay, (gated ? tokens : static_cast<size_t>(H)) * sizeof(float)),
                        span(state_in, state_in ? sbytes : 0), span(grad_o, tokens * dv * es),
                        span(grad_state_out, grad_state_out ? sbytes : 0)};
    const Range out[] = {span(grad_q, tokens * dk * es), span(grad_k, tokens * dk * es),
                         span(grad_v, tokens * dv * es), span(grad_state_in, grad_state_in ? sbytes : 0),
                         span(grad_g, gated && grad_g ? tokens * sizeof(float) : 0)};
    for (size_t i = 0; i < sizeof(out) / sizeof(out[0]); ++i) {
        for (const Range& r : in)
            if (overlaps(out[i], r)) return RETN_ERR_ALIAS;
        for (size_t j = i + 1; j < sizeof(out) / sizeof(out[0]); ++j)
            if (overlaps(out[i], out[j])) return RETN_ERR_ALIAS;
    }
    const retn::BwdShape sh{B, H, N, dk, dv, effective_chunk(N, chunk), dt == RETN_BF16, gated,
                            state_in != nullptr, grad_state_out != nullptr};
    const retn::BwdPtrs x{q, k, v, decay, state_in, grad_o, grad_state_out, grad_q, grad_k, grad_v,
                          grad_state_in, grad_g};
    const retn::BwdPlan plan = retn::bwd_plan(sh, &x);
    if (!plan.ok) return RETN_ERR_UNSUPPORTED;
    if (plan.total > 0 && (workspace == nullptr || workspace_bytes < plan.total || !aligned16(workspace)))
        return RETN_ERR_WORKSPACE;
    const hipError_t e = retn::run_backward(sh, x, plan, workspace, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? RETN_OK : RETN_ERR_HIP;
}

}  // namespace

extern "C" {

retn_status retention_chunkwise_fwd(const void* q, const void* k, const void* v,
                                    const float* gamma, void* o, const float* state_in,
                                    float* state_out, int B, int H, int N, int dk, int dv,
                                    int chunk, retn_dtype dtype, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    return chunk_common(q, k, v, gamma, o, state_in, state_out, B, H, N, dk, dv, chunk, dtype,
                        workspace, workspace_bytes, stream, false);
}

retn_status gated_retention_chunkwise_fwd(const void* q, const void* k, const void* v,
                                          const float* g, void* o, const float* state_in,
                                          float* state_out, int B, int H, int N, int dk, int dv,
                                          int chunk, retn_dtype dtype, void* workspace,
                                          size_t workspace_bytes, void* stream) {
    return chunk_common(q, k, v, g, o, state_in, state_out, B, H, N, dk, dv, chunk, dtype,
                        workspace, workspace_bytes, stream, true);
}

retn_status retention_decode_step(const void* q, const void* k, const void* v, const float* gamma,
                                  float* state, void* o, int B, int H, int dk, int dv,
                                  retn_dtype dtype, void* stream) {
    return decode_common(q, k, v, gamma, state, o, B, H, dk, dv, dtype, stream, false);
}

retn_status gated_retention_decode_step(const void* q, const void* k, const void* v,
                                        const float* g, float* state, void* o, int B, int H,
                                        int dk, int dv, retn_dtype dtype, void* stream) {
    return decode_common(q, k, v, g, state, o, B, H, dk, dv, dtype, stream, true);
}

retn_status retention_parallel_fwd(const void* q, const void* k, const void* v, const float* gamma, void* o,
                                   int B, int H, int N, int dk, int dv, retn_dtype dtype, void* stream) {
    return parallel_common(q, k, v, gamma, o, B, H, N, dk, dv, dtype, stream, false);
}

retn_status gated_retention_parallel_fwd(const void* q, const void* k, const void* v, const float* g, void* o,
                                         int B, int H, int N, int dk, int dv, retn_dtype dtype, void* stream) {
    return parallel_common(q, k, v, g, o, B, H, N, dk, dv, dtype, stream, true);
}

retn_status gated_msr_fwd(const void* x, const void* wq, const void* wk, const void* wv, const void* wg,
                          const void* wgt, const void* wo, void* y, int B, int N, int D, int H, int dk, int dv,
                          int chunk, float rope_base, float norm_eps, void* workspace, size_t workspace_bytes,
                          void* stream) {
    if (B < 0 || N < 0 || D < 1 || H < 1 || dk < 1 || dv < 1 || chunk < 1) return RETN_ERR_SHAPE;
    if (!(rope_base > 1.f) || !(norm_eps >= 0.f)) return RETN_ERR_SHAPE;
    const size_t T = static_cast<size_t>(B) * N;
    if (T > static_cast<size_t>(INT32_MAX)) return RETN_ERR_SHAPE;
    const retn::MsrShape sh{B, N, D, H, dk, dv, chunk, rope_base, norm_eps};
    const retn::MsrPlan plan = retn::msr_plan(sh);
    if (!plan.ok) return RETN_ERR_UNSUPPORTED;
    if (T == 0) return RETN_OK;
    if (x == nullptr || wq == nullptr || wk == nullptr || wv == nullptr || wg == nullptr || wgt == nullptr ||
        wo == nullptr || y == nullptr)
        return RETN_ERR_NULL;
    const size_t hk = static_cast<size_t>(H) * dk, hv = static_cast<size_t>(H) * dv;
    const Range ry = span(y, T * D * 2);
    const Range in[] = {span(x, T * D * 2), span(wq, hk * D * 2), span(wk, hk * D * 2), span(wv, hv * D * 2),
                        span(wg, hv * D * 2), span(wgt, static_cast<size_t>(H) * D * 2), span(wo, hv * D * 2)};
    for (const Range& r : in)
        if (overlaps(ry, r)) return RETN_ERR_ALIAS;
    const void* const all[] = {x, wq, wk, wv, wg, wgt, wo, y};
    for (const void* p : all)
        if (!aligned16(p)) return RETN_ERR_UNSUPPORTED;
    if (workspace == nullptr || workspace_bytes < plan.total || !aligned16(workspace)) return RETN_ERR_WORKSPACE;
    const retn::MsrPtrs ptrs{x, wq, wk, wv, wg, wgt, wo, y};
    const hipError_t e = retn::run_msr(sh, ptrs, plan, workspace, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? RETN_OK : RETN_ERR_HIP;
}

size_t gated_msr_workspace_bytes(int B, int N, int D, int H, int dk, int dv, int chunk) {
    if (B < 0 || N < 0 || D < 1 || H < 1 || dk < 1 || dv < 1 || chunk < 1) return 0;
    const retn::MsrPlan plan = retn::msr_plan(retn::MsrShape{B, N, D, H, dk, dv, chunk, 10000.f, 0.f});
    return plan.ok ? plan.total : 0;
}

size_t retention_workspace_bytes(int B, int H, int N, int dk, int dv, int chunk, retn_dtype dtype,
                                 int gated) {
    if (!valid_dtype(dtype) || B < 0 || H < 0 || N < 0 || dk < 1 || dv < 1 || chunk < 1 ||
        dk > kMaxDk || dv > kMaxDv)
        return 0;
    return workspace_for(B, H, N, dk, dv, chunk, dtype, gated != 0);
}

retn_status retention_chunkwise_bwd(const void* q, const void* k, const void* v, const float* gamma,
                                    const float* state_in, const void* grad_o, const float* grad_state_out,
                                    void* grad_q, void* grad_k, void* grad_v, float* grad_state_in, int B, int H,
                                    int N, int dk, int dv, int chunk, retn_dtype dtype, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    return bwd_common(q, k, v, gamma, state_in, grad_o, grad_state_out, grad_q, grad_k, grad_v, grad_state_in,
                      nullptr, B, H, N, dk, dv, chunk, dtype, workspace, workspace_bytes, stream, false);
}

retn_status gated_retention_chunkwise_bwd(const void* q, const void* k, const void* v, const float* g,
                                          const float* state_in, const void* grad_o, const float* grad_state_out,
                                          void* grad_q, void* grad_k, void* grad_v, float* grad_g,
                                          float* grad_state_in, int B, int H, int N, int dk, int dv, int chunk,
                                          retn_dtype dtype, void* workspace, size_t workspace_bytes,
                                          void* stream) {
    return bwd_common(q, k, v, g, state_in, grad_o, grad_state_out, grad_q, grad_k, grad_v, grad_state_in, grad_g,
                      B, H, N, dk, dv, chunk, dtype, workspace, workspace_bytes, stream, true);
}

size_t retention_bwd_workspace_bytes(int B, int H, int N, int dk, int dv, int chunk, retn_dtype dtype,
                                     int gated) {
    if (!valid_dtype(dtype) || B < 0 || H < 0 || N < 0 || dk < 1 || dv < 1 || chunk < 1 ||
        dk > kMaxDk || dv > kMaxDv)
        return 0;
    const retn::BwdShape sh{B, H, N, dk, dv, effective_chunk(N, chunk), dtype == RETN_BF16, gated != 0, true, true};
    const retn::BwdPlan plan = retn::bwd_plan(sh, nullptr);
    return plan.ok ? plan.total : 0;
}

const char* retention_status_string(retn_status status) {
    switch (status) {
        case RETN_OK: return "ok";
        case RETN_ERR_NULL: return "a required pointer is NULL";
        case RETN_ERR_SHAPE: return "a size is negative or out of range";
        case RETN_ERR_DTYPE: return "unknown element type";
        case RETN_ERR_UNSUPPORTED: return "valid arguments, but this shape is not supported";
        case RETN_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
        case RETN_ERR_ALIAS: return "an output overlaps an input";
        case RETN_ERR_HIP: return "HIP runtime error at launch";
        default: break;
    }
    return "unknown status";
}

int retention_abi_version(void) { return 1; }

retn_status retention_profile_enable(int on) {
    return retn::prof_enable(on != 0) == hipSuccess ? RETN_OK : RETN_ERR_HIP;
}

retn_status retention_profile_read(double* ms, int* count, int nkinds, int* dropped) {
    if (nkinds < 0) return RETN_ERR_SHAPE;
    if (nkinds > 0 && (ms == nullptr || count == nullptr)) return RETN_ERR_NULL;
    return retn::prof_read(ms, count, nkinds, dropped) == hipSuccess ? RETN_OK : RETN_ERR_HIP;
}

}  // extern "C"
