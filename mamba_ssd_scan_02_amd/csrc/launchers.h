// launchers.h -- host-side launchers of the gfx950 kernels (internal to the
// library; the public boundary is include/ssd_mi355x.h).  Each launcher
// assumes its arguments were validated by the C-ABI layer and returns the
// launch status (hipGetLastError after the launch).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

struct Dims {
    int64_t batch, seqlen, nheads, headdim, dstate, ngroups, chunk, nchunks;
};

// True when the bf16 matrix-core kernels cover these sizes.
bool mfma_path(int32_t dtype, const Dims& d);
// True when the generic kernels cover these sizes.
bool generic_path(const Dims& d);

hipError_t launch_chunk_cumsum(const Dims& d, const float* dt, const float* A, float* cs,
                               float* dtc, hipStream_t stream, bool zoh = false);

hipError_t launch_chunk_state(const Dims& d, int32_t dtype, const void* x, const void* B,
                              const float* cs, const float* dtc, float* S, hipStream_t stream);

// Chunk state that also forms the chunk cumsum (cs, dtc written for the
// later stages), where the paired-head matrix-core kernel applies.
bool chunk_state_fuses_cumsum(int32_t dtype, const Dims& d);
hipError_t launch_chunk_state_fused(const Dims& d, const void* x, const void* B, const float* dt,
                                    const float* A, bool zoh, float* cs, float* dtc, float* S,
                                    hipStream_t stream);

hipError_t launch_state_passing(const Dims& d, int32_t dtype, const float* S, const float* cs,
                                const float* init, void* Hin, float* final_state,
                                hipStream_t stream);

// Segmented (two-level associative) form of the same recurrence; the
// workspace holds the segment end states, entering states and decays.
void state_passing_segments(int64_t nc, int64_t nseg_req, int64_t* seg, int64_t* nseg);
size_t state_passing_seg_workspace_bytes(int64_t batch, int64_t H, int64_t P, int64_t N,
                                         int64_t nseg);
hipError_t launch_state_passing_seg(const Dims& d, int32_t dtype, int64_t nseg_req, const float* S,
                                    const float* cs, const float* init, void* Hin,
                                    float* final_state, void* workspace, hipStream_t stream);

hipError_t launch_chunk_scan(const Dims& d, int32_t dtype, const void* x, const void* B,
                             const void* C, const float* cs, const float* dtc, const void* Hin,
                             const float* D, void* y, hipStream_t stream);

// Chunk state and state passing in one pass (bf16 matrix-core path, chunk 256).
hipError_t launch_state_scan(const Dims& d, const void* x, const void* B, const float* cs,
                             const float* dtc, const float* init, void* Hin, float* final_state,
                             hipStream_t stream);

bool ssm_step_supported(int64_t P, int64_t N);
hipError_t launch_ssm_step(int64_t batch, int64_t H, int64_t P, int64_t N, int64_t G,
                           int32_t dtype, float* state, const void* x, const float* dt,
                           const float* A, const void* B, const void* C, const float* D,
                           void* y, hipStream_t stream, bool zoh = false);

// The steps around the scan (layer.hip).
hipError_t launch_layer_in(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
                           int K, int32_t dtype, const void* xbc, const float* w, const float* bias,
                           const float* dt_raw, const float* dt_bias, void* x, void* B, void* C,
                           float* dt, hipStream_t stream);
hipError_t launch_layer_out(int64_t n, int32_t dtype, const void* y, const void* z, void* out,
                            hipStream_t stream);

}  // namespace ssd
