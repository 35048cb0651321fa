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
    size_t workspace_bytes;
};
MfmaPlan mfma_chunk_plan(int B, int H, int N, int dk, int dv, int chunk, bool gated);
hipError_t launch_mfma_chunk(const ChunkArgs& a, const MfmaPlan& plan, hipStream_t stream);

// Decode step.
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

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
