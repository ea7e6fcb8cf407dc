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

// S in the storage type (bf16 for the matrix-core path).
hipError_t launch_chunk_state(const Dims& d, int32_t dtype, const void* x, const void* B,
                              const float* cs, const float* dtc, void* S, hipStream_t stream);

// Chunk state that also forms the chunk cumsum (cs, dtc written for the
// later stages), where the paired-head matrix-core kernel applies.
bool chunk_state_fuses_cumsum(int32_t dtype, const Dims& d);
hipError_t launch_chunk_state_fused(const Dims& d, const void* x, const void* B, const float* dt,
                                    const float* A, bool zoh, float* cs, float* dtc, void* S,
                                    hipStream_t stream);

hipError_t launch_state_passing(const Dims& d, int32_t dtype, const void* S, const float* cs,
                                const float* init, void* Hin, float* final_state,
                                hipStream_t stream);

// Segmented (two-level associative) form of the same recurrence; the
// workspace holds the segment end states, entering states and decays.
void state_passing_segments(int64_t nc, int64_t nseg_req, int64_t* seg, int64_t* nseg);
size_t state_passing_seg_workspace_bytes(int64_t batch, int64_t H, int64_t P, int64_t N,
                                         int64_t nseg);
hipError_t launch_state_passing_seg(const Dims& d, int32_t dtype, int64_t nseg_req, const void* S,
                                    const float* cs, const float* init, void* Hin,
                                    float* final_state, void* workspace, hipStream_t stream);

// The runs of heads the matrix-core chunk scan gives each workgroup: hg heads
// of one group per run, a group's heads in nsplit runs (mfma_path shapes).
void chunk_scan_runs(const Dims& d, int* hg, int* nsplit);

// x is read twice (chunk state, then chunk scan).  The chunk-state kernel
// reads with ordinary (cache-allocating) loads the x of the heads at run
// positions below x_keep_positions, which the chunk scan reads first, and
// non-temporally the rest, so that the chunk scan finds those heads' x in
// the 256 MB last-level cache.
constexpr double kLastLevelCacheBytes = 256.0 * 1024 * 1024;
int x_keep_positions(const Dims& d);

// With z, y receives y * silu(z) (the gate of the block around the scan):
// inside the store of the 256-token matrix-core kernel, else by the gate
// kernel in place after the chunk scan.
hipError_t launch_chunk_scan(const Dims& d, int32_t dtype, const void* x, const void* B,
                             const void* C, const float* cs, const float* dtc, const void* Hin,
                             const float* D, void* y, hipStream_t stream, const void* z = nullptr);

// Two-level recurrence between chunks (bf16 matrix-core path, chunk 256, an
// even head count per group): chunk states over runs of K chunks (T, lam,
// rdec, and the cumsum rows cs / dtc), a chain over the runs (Hr and the
// final state), and the chunk scan forming each chunk's entering state from
// T and Hr.  state_run_chunks gives the K ssd_forward uses (2 to 16), or 0
// where the per-chunk path stays (too few workgroups for runs).
bool state_runs_apply(int32_t dtype, const Dims& d);
int state_run_chunks(const Dims& d);
hipError_t launch_chunk_state_runs(const Dims& d, int K, const void* x, const void* B,
                                   const float* dt, const float* A, bool zoh, float* cs, float* dtc,
                                   void* T, float* lam, float* rdec, hipStream_t stream);
hipError_t launch_run_passing(const Dims& d, int K, const void* T, const float* rdec, const float* init,
                              void* Hr, float* final_state, hipStream_t stream);
hipError_t launch_chunk_scan_runs(const Dims& d, int K, const void* x, const void* B, const void* C,
                                  const float* cs, const float* dtc, const void* T, const void* Hr,
                                  const float* lam, const float* D, void* y, hipStream_t stream,
                                  const void* z = nullptr);

// Chunk state and state passing walked per (batch, head pair) in one pass
// (bf16 matrix-core path, chunk 128 or 256, an even head count per group).
bool state_walk_applies(int32_t dtype, const Dims& d);
hipError_t launch_state_walk(const Dims& d, const void* x, const void* B, const float* cs,
                             const float* dtc, const float* init, void* Hin, float* final_state,
                             hipStream_t stream);

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
