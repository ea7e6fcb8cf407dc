// ssd_api.cpp -- the C ABI declared in include/ssd_mi355x.h: argument
// validation, workspace carving and the launch order.  No allocation, no
// synchronisation, no global mutable state.
#include "ssd_mi355x.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "launchers.h"

namespace {

using ssd::Dims;

constexpr size_t kRegionAlign = 256;

size_t align_up(size_t v) { return (v + kRegionAlign - 1) / kRegionAlign * kRegionAlign; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Overflow-checked product of non-negative sizes; returns false on overflow.
bool mul_ok(size_t a, size_t b, size_t* out) {
    if (a != 0 && b > SIZE_MAX / a) return false;
    *out = a * b;
    return true;
}

bool elem_size(int32_t dtype, size_t* es) {
    if (dtype == SSD_DTYPE_F32) { *es = 4; return true; }
    if (dtype == SSD_DTYPE_BF16) { *es = 2; return true; }
    return false;
}

// Basic size checks shared by the forward entry points.  Sizes are bounded so
// that every index the kernels form fits the types they use.
int32_t check_dims(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                   int64_t dstate, int64_t ngroups, int64_t chunk, Dims* d) {
    if (batch < 1 || seqlen < 1 || nheads < 1 || headdim < 1 || dstate < 1 || ngroups < 1 ||
        chunk < 1)
        return SSD_ERR_SHAPE;
    if (nheads % ngroups != 0) return SSD_ERR_SHAPE;
    if (seqlen > (int64_t(1) << 30) || batch > (int64_t(1) << 24) || nheads > 65536 ||
        ngroups > 65536)
        return SSD_ERR_SHAPE;
    d->batch = batch;
    d->seqlen = seqlen;
    d->nheads = nheads;
    d->headdim = headdim;
    d->dstate = dstate;
    d->ngroups = ngroups;
    d->chunk = chunk;
    d->nchunks = (seqlen + chunk - 1) / chunk;
    // grid sizes (one workgroup per batch * chunk * head) must fit 32 bits
    if ((double)batch * (double)d->nchunks * (double)nheads > 2147483647.0) return SSD_ERR_SHAPE;
    return SSD_OK;
}

int32_t check_supported(int32_t dtype, const Dims& d) {
    size_t es;
    if (!elem_size(dtype, &es)) return SSD_ERR_UNSUPPORTED;
    if (ssd::mfma_path(dtype, d) || ssd::generic_path(d)) return SSD_OK;
    return SSD_ERR_UNSUPPORTED;
}

struct Layout {
    size_t cs, dtc, S, Hin, total;
};

bool workspace_layout(const Dims& d, int32_t dtype, Layout* lo) {
    size_t es;
    if (!elem_size(dtype, &es)) return false;
    size_t rows, states, t;
    if (!mul_ok((size_t)d.batch, (size_t)d.nheads, &t)) return false;
    if (!mul_ok(t, (size_t)d.nchunks, &t)) return false;
    if (!mul_ok(t, (size_t)d.chunk, &rows)) return false;
    size_t per_chunk_state = (size_t)d.headdim * (size_t)d.dstate;
    if (!mul_ok((size_t)d.batch * (size_t)d.nheads, (size_t)d.nchunks, &t)) return false;
    if (!mul_ok(t, per_chunk_state, &states)) return false;
    size_t b_cs, b_S, b_H;
    if (!mul_ok(rows, 4, &b_cs) || !mul_ok(states, 4, &b_S) || !mul_ok(states, es, &b_H)) return false;
    lo->cs = 0;
    lo->dtc = align_up(b_cs);
    lo->S = lo->dtc + align_up(b_cs);
    lo->Hin = lo->S + align_up(b_S);
    lo->total = lo->Hin + align_up(b_H);
    return true;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x0 = reinterpret_cast<uintptr_t>(a), x1 = x0 + na;
    const uintptr_t y0 = reinterpret_cast<uintptr_t>(b), y1 = y0 + nb;
    return x0 < y1 && y0 < x1;
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? SSD_OK : SSD_ERR_HIP; }

}  // namespace

extern "C" {

int32_t ssd_abi_version(void) { return SSD_ABI_VERSION; }

const char* ssd_status_str(int32_t status) {
    switch (status) {
        case SSD_OK: return "ok";
        case SSD_ERR_NULL: return "a required pointer is NULL";
        case SSD_ERR_SHAPE: return "invalid sizes (non-positive, nheads % ngroups != 0, or too large)";
        case SSD_ERR_UNSUPPORTED: return "unsupported dtype / headdim / dstate / chunk combination";
        case SSD_ERR_WORKSPACE: return "workspace missing or too small";
        case SSD_ERR_ALIGN: return "pointer not aligned (16 bytes for tensors, 4 for dt/A/D)";
        case SSD_ERR_HIP: return "HIP kernel launch failed";
        case SSD_ERR_ALIAS: return "an output overlaps an input";
        default: return "unknown status";
    }
}

size_t ssd_forward_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads,
                                   int64_t headdim, int64_t dstate, int64_t ngroups,
                                   int64_t chunk, int32_t dtype) {
    Dims d;
    if (check_dims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, &d) != SSD_OK) return 0;
    if (check_supported(dtype, d) != SSD_OK) return 0;
    Layout lo;
    if (!workspace_layout(d, dtype, &lo)) return 0;
    return lo.total;
}

static int32_t chunk_cumsum_impl(int64_t batch, int64_t seqlen, int64_t nheads, int64_t chunk,
                                 const float* dt, const float* A, float* cs, float* dtc,
                                 hipStream_t stream, bool zoh) {
    Dims d;
    int32_t st = check_dims(batch, seqlen, nheads, 1, 1, 1, chunk, &d);
    if (st != SSD_OK) return st;
    if (chunk > 256) return SSD_ERR_UNSUPPORTED;
    if (!dt || !A || !cs || !dtc) return SSD_ERR_NULL;
    if (!aligned(dt, 4) || !aligned(A, 4) || !aligned(cs, 4) || !aligned(dtc, 4)) return SSD_ERR_ALIGN;
    return hip_status(ssd::launch_chunk_cumsum(d, dt, A, cs, dtc, stream, zoh));
}

int32_t ssd_chunk_cumsum(int64_t batch, int64_t seqlen, int64_t nheads, int64_t chunk,
                         const float* dt, const float* A, float* cs, float* dtc,
                         hipStream_t stream) {
    return chunk_cumsum_impl(batch, seqlen, nheads, chunk, dt, A, cs, dtc, stream, false);
}

int32_t ssd_chunk_cumsum_zoh(int64_t batch, int64_t seqlen, int64_t nheads, int64_t chunk,
                             const float* dt, const float* A, float* cs, float* dtc,
                             hipStream_t stream) {
    return chunk_cumsum_impl(batch, seqlen, nheads, chunk, dt, A, cs, dtc, stream, true);
}

int32_t ssd_chunk_state(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                        int64_t dstate, int64_t ngroups, int64_t chunk, int32_t dtype,
                        const void* x, const void* B, const float* cs, const float* dtc,
                        float* S, hipStream_t stream) {
    Dims d;
    int32_t st = check_dims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, &d);
    if (st != SSD_OK) return st;
    if ((st = check_supported(dtype, d)) != SSD_OK) return st;
    if (!x || !B || !cs || !dtc || !S) return SSD_ERR_NULL;
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(S, 16) || !aligned(cs, 4) || !aligned(dtc, 4))
        return SSD_ERR_ALIGN;
    return hip_status(ssd::launch_chunk_state(d, dtype, x, B, cs, dtc, S, stream));
}

int32_t ssd_state_passing(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                          int64_t dstate, int64_t chunk, int32_t dtype, const float* S,
                          const float* cs, const float* init_state, void* Hin,
                          float* final_state, hipStream_t stream) {
    Dims d;
    int32_t st = check_dims(batch, seqlen, nheads, headdim, dstate, 1, chunk, &d);
    if (st != SSD_OK) return st;
    if ((st = check_supported(dtype, d)) != SSD_OK) return st;
    if (!S || !cs || !Hin) return SSD_ERR_NULL;
    if (!aligned(S, 16) || !aligned(Hin, 16) || !aligned(cs, 4) ||
        (init_state && !aligned(init_state, 16)) || (final_state && !aligned(final_state, 16)))
        return SSD_ERR_ALIGN;
    return hip_status(ssd::launch_state_passing(d, dtype, S, cs, init_state, Hin, final_state, stream));
}

size_t ssd_state_passing_seg_workspace_bytes(int64_t batch, int64_t nheads, int64_t headdim,
                                             int64_t dstate, int64_t nsegments) {
    if (batch < 1 || nheads < 1 || headdim < 1 || dstate < 1 || nsegments < 1) return 0;
    const double states = (double)batch * nheads * nsegments * headdim * dstate * 4.0;
    if (states > 1.0e15) return 0;
    return ssd::state_passing_seg_workspace_bytes(batch, nheads, headdim, dstate, nsegments);
}

int32_t ssd_state_passing_seg(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                              int64_t dstate, int64_t chunk, int64_t nsegments, int32_t dtype,
                              const float* S, const float* cs, const float* init_state, void* Hin,
                              float* final_state, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
    Dims d;
    int32_t st = check_dims(batch, seqlen, nheads, headdim, dstate, 1, chunk, &d);
    if (st != SSD_OK) return st;
    if ((st = check_supported(dtype, d)) != SSD_OK) return st;
    if (nsegments < 1 || nsegments > 65535) return SSD_ERR_SHAPE;
    if (!S || !cs || !Hin) return SSD_ERR_NULL;
    if (!workspace) return SSD_ERR_WORKSPACE;
    if (!aligned(S, 16) || !aligned(Hin, 16) || !aligned(cs, 4) || !aligned(workspace, 256) ||
        (init_state && !aligned(init_state, 16)) || (final_state && !aligned(final_state, 16)))
        return SSD_ERR_ALIGN;
    int64_t seg, nseg;
    ssd::state_passing_segments(d.nchunks, nsegments, &seg, &nseg);
    if (workspace_bytes < ssd::state_passing_seg_workspace_bytes(batch, nheads, headdim, dstate, nseg))
        return SSD_ERR_WORKSPACE;
    return hip_status(ssd::launch_state_passing_seg(d, dtype, nsegments, S, cs, init_state, Hin,
                                                    final_state, workspace, stream));
}

int32_t ssd_state_scan(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                       int64_t dstate, int64_t ngroups, int64_t chunk, int32_t dtype,
                       const void* x, const void* B, const float* cs, const float* dtc,
                       const float* init_state, void* Hin, float* final_state,
                       hipStream_t stream) {
    Dims d;
    int32_t st = check_dims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, &d);
    if (st != SSD_OK) return st;
    size_t es;
    if (!elem_size(dtype, &es)) return SSD_ERR_UNSUPPORTED;
    if (!ssd::mfma_path(dtype, d) || d.chunk != 256) return SSD_ERR_UNSUPPORTED;
    if (!x || !B || !cs || !dtc || !Hin) return SSD_ERR_NULL;
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(Hin, 16) || !aligned(cs, 4) ||
        !aligned(dtc, 4) || (init_state && !aligned(init_state, 16)) ||
        (final_state && !aligned(final_state, 16)))
        return SSD_ERR_ALIGN;
    return hip_status(ssd::launch_state_scan(d, x, B, cs, dtc, init_state, Hin, final_state, stream));
}

int32_t ssd_chunk_scan(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                       int64_t dstate, int64_t ngroups, int64_t chunk, int32_t dtype,
                       const void* x, const void* B, const void* C, const float* cs,
                       const float* dtc, const void* Hin, const float* D, void* y,
                       hipStream_t stream) {
    Dims d;
    int32_t st = check_dims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, &d);
    if (st != SSD_OK) return st;
    if ((st = check_supported(dtype, d)) != SSD_OK) return st;
    if (!x || !B || !C || !cs || !dtc || !Hin || !y) return SSD_ERR_NULL;
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(Hin, 16) ||
        !aligned(y, 16) || !aligned(cs, 4) || !aligned(dtc, 4) || (D && !aligned(D, 4)))
        return SSD_ERR_ALIGN;
    size_t es;
    elem_size(dtype, &es);
    const size_t ybytes = (size_t)d.batch * d.seqlen * d.nheads * d.headdim * es;
    const size_t bcbytes = (size_t)d.batch * d.seqlen * d.ngroups * d.dstate * es;
    if (overlaps(y, ybytes, x, ybytes) || overlaps(y, ybytes, B, bcbytes) ||
        overlaps(y, ybytes, C, bcbytes))
        return SSD_ERR_ALIAS;
    return hip_status(ssd::launch_chunk_scan(d, dtype, x, B, C, cs, dtc, Hin, D, y, stream));
}

static int32_t forward_impl(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                            int64_t dstate, int64_t ngroups, int64_t chunk, int32_t dtype,
                            const void* x, const float* dt, const float* A, const void* B,
                            const void* C, const float* D, const float* init_state, void* y,
                            float* final_state, void* workspace, size_t workspace_bytes,
                            hipStream_t stream, bool zoh) {
    Dims d;
    int32_t st = check_dims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, &d);
    if (st != SSD_OK) return st;
    if ((st = check_supported(dtype, d)) != SSD_OK) return st;
    if (!x || !dt || !A || !B || !C || !y) return SSD_ERR_NULL;
    Layout lo;
    if (!workspace_layout(d, dtype, &lo)) return SSD_ERR_SHAPE;
    if (!workspace || workspace_bytes < lo.total) return SSD_ERR_WORKSPACE;
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(y, 16) ||
        !aligned(workspace, 16) || !aligned(dt, 4) || !aligned(A, 4) || (D && !aligned(D, 4)) ||
        (init_state && !aligned(init_state, 16)) || (final_state && !aligned(final_state, 16)))
        return SSD_ERR_ALIGN;

    size_t es;
    elem_size(dtype, &es);
    const size_t tok = (size_t)d.batch * (size_t)d.seqlen;
    const size_t ybytes = tok * d.nheads * d.headdim * es;
    const size_t bcbytes = tok * d.ngroups * d.dstate * es;
    const size_t dtbytes = tok * d.nheads * 4;
    const size_t stbytes = (size_t)d.batch * d.nheads * d.headdim * d.dstate * 4;
    if (overlaps(y, ybytes, x, ybytes) || overlaps(y, ybytes, B, bcbytes) ||
        overlaps(y, ybytes, C, bcbytes) || overlaps(y, ybytes, dt, dtbytes) ||
        overlaps(y, ybytes, workspace, lo.total) || overlaps(y, ybytes, init_state, stbytes) ||
        overlaps(y, ybytes, final_state, stbytes) ||
        overlaps(workspace, lo.total, x, ybytes) || overlaps(workspace, lo.total, B, bcbytes) ||
        overlaps(workspace, lo.total, C, bcbytes) || overlaps(workspace, lo.total, dt, dtbytes) ||
        overlaps(workspace, lo.total, init_state, stbytes) ||
        overlaps(workspace, lo.total, final_state, stbytes))
        return SSD_ERR_ALIAS;

    char* ws = static_cast<char*>(workspace);
    float* cs = reinterpret_cast<float*>(ws + lo.cs);
    float* dtc = reinterpret_cast<float*>(ws + lo.dtc);
    float* S = reinterpret_cast<float*>(ws + lo.S);
    void* Hin = ws + lo.Hin;

    // chunk cumsum and chunk states (one launch where the paired-head kernel
    // applies), then the recurrence between chunks (the one-pass
    // ssd_state_scan measured slower than this pair at every shape tried)
    hipError_t e;
    if (ssd::chunk_state_fuses_cumsum(dtype, d)) {
        e = ssd::launch_chunk_state_fused(d, x, B, dt, A, zoh, cs, dtc, S, stream);
        if (e != hipSuccess) return SSD_ERR_HIP;
    } else {
        e = ssd::launch_chunk_cumsum(d, dt, A, cs, dtc, stream, zoh);
        if (e != hipSuccess) return SSD_ERR_HIP;
        e = ssd::launch_chunk_state(d, dtype, x, B, cs, dtc, S, stream);
        if (e != hipSuccess) return SSD_ERR_HIP;
    }
    e = ssd::launch_state_passing(d, dtype, S, cs, init_state, Hin, final_state, stream);
    if (e != hipSuccess) return SSD_ERR_HIP;
    e = ssd::launch_chunk_scan(d, dtype, x, B, C, cs, dtc, Hin, D, y, stream);
    return hip_status(e);
}

int32_t ssd_forward(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                    int64_t dstate, int64_t ngroups, int64_t chunk, int32_t dtype,
                    const void* x, const float* dt, const float* A, const void* B,
                    const void* C, const float* D, const float* init_state, void* y,
                    float* final_state, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
    return forward_impl(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype, x, dt, A,
                        B, C, D, init_state, y, final_state, workspace, workspace_bytes, stream,
                        false);
}

int32_t ssd_forward_zoh(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                        int64_t dstate, int64_t ngroups, int64_t chunk, int32_t dtype,
                        const void* x, const float* dt, const float* A, const void* B,
                        const void* C, const float* D, const float* init_state, void* y,
                        float* final_state, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
    return forward_impl(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype, x, dt, A,
                        B, C, D, init_state, y, final_state, workspace, workspace_bytes, stream,
                        true);
}

static int32_t ssm_step_impl(int64_t batch, int64_t nheads, int64_t headdim, int64_t dstate,
                             int64_t ngroups, int32_t dtype, float* state, const void* x_t,
                             const float* dt_t, const float* A, const void* B_t, const void* C_t,
                             const float* D, void* y_t, hipStream_t stream, bool zoh) {
    if (batch < 1 || nheads < 1 || headdim < 1 || dstate < 1 || ngroups < 1) return SSD_ERR_SHAPE;
    if (nheads % ngroups != 0) return SSD_ERR_SHAPE;
    if ((double)batch * (double)nheads > 2147483647.0 ||
        (double)batch * nheads * headdim > 9.0e15)
        return SSD_ERR_SHAPE;
    size_t es;
    if (!elem_size(dtype, &es)) return SSD_ERR_UNSUPPORTED;
    if (!ssd::ssm_step_supported(headdim, dstate)) return SSD_ERR_UNSUPPORTED;
    if (!state || !x_t || !dt_t || !A || !B_t || !C_t || !y_t) return SSD_ERR_NULL;
    if (!aligned(state, 16) || !aligned(x_t, 16) || !aligned(B_t, 16) || !aligned(C_t, 16) ||
        !aligned(y_t, 16) || !aligned(dt_t, 4) || !aligned(A, 4) || (D && !aligned(D, 4)))
        return SSD_ERR_ALIGN;
    const size_t ybytes = (size_t)batch * nheads * headdim * es;
    const size_t sbytes = (size_t)batch * nheads * headdim * dstate * 4;
    const size_t bcbytes = (size_t)batch * ngroups * dstate * es;
    if (overlaps(y_t, ybytes, state, sbytes) || overlaps(y_t, ybytes, x_t, ybytes) ||
        overlaps(y_t, ybytes, B_t, bcbytes) || overlaps(y_t, ybytes, C_t, bcbytes) ||
        overlaps(state, sbytes, x_t, ybytes) || overlaps(state, sbytes, B_t, bcbytes) ||
        overlaps(state, sbytes, C_t, bcbytes))
        return SSD_ERR_ALIAS;
    return hip_status(ssd::launch_ssm_step(batch, nheads, headdim, dstate, ngroups, dtype, state,
                                           x_t, dt_t, A, B_t, C_t, D, y_t, stream, zoh));
}

int32_t ssm_step(int64_t batch, int64_t nheads, int64_t headdim, int64_t dstate,
                 int64_t ngroups, int32_t dtype, float* state, const void* x_t,
                 const float* dt_t, const float* A, const void* B_t, const void* C_t,
                 const float* D, void* y_t, hipStream_t stream) {
    return ssm_step_impl(batch, nheads, headdim, dstate, ngroups, dtype, state, x_t, dt_t, A, B_t,
                         C_t, D, y_t, stream, false);
}

int32_t ssm_step_zoh(int64_t batch, int64_t nheads, int64_t headdim, int64_t dstate,
                     int64_t ngroups, int32_t dtype, float* state, const void* x_t,
                     const float* dt_t, const float* A, const void* B_t, const void* C_t,
                     const float* D, void* y_t, hipStream_t stream) {
    return ssm_step_impl(batch, nheads, headdim, dstate, ngroups, dtype, state, x_t, dt_t, A, B_t,
                         C_t, D, y_t, stream, true);
}

int32_t ssd_layer_in(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                     int64_t dstate, int64_t ngroups, int64_t kernel_width, int32_t dtype,
                     const void* xbc, const float* conv_w, const float* conv_b,
                     const float* dt_raw, const float* dt_bias, void* x, void* B, void* C,
                     float* dt, hipStream_t stream) {
    if (batch < 1 || seqlen < 1 || nheads < 1 || headdim < 1 || dstate < 1 || ngroups < 1)
        return SSD_ERR_SHAPE;
    if (nheads % ngroups != 0) return SSD_ERR_SHAPE;
    size_t es;
    if (!elem_size(dtype, &es)) return SSD_ERR_UNSUPPORTED;
    if (kernel_width < 1 || kernel_width > 8) return SSD_ERR_UNSUPPORTED;
    const double cd = (double)nheads * headdim + 2.0 * (double)ngroups * dstate;
    if (cd > 8.0 * 65535.0 * 256.0 || (double)batch > 65535.0 || (double)seqlen > 2147483647.0 ||
        (double)batch * seqlen * cd > 1.0e12)
        return SSD_ERR_SHAPE;
    if (!xbc || !conv_w || !dt_raw || !x || !B || !C || !dt) return SSD_ERR_NULL;
    if (!aligned(xbc, es) || !aligned(x, es) || !aligned(B, es) || !aligned(C, es) ||
        !aligned(conv_w, 4) || !aligned(dt_raw, 4) || !aligned(dt, 4) ||
        (conv_b && !aligned(conv_b, 4)) || (dt_bias && !aligned(dt_bias, 4)))
        return SSD_ERR_ALIGN;
    const size_t tok = (size_t)batch * (size_t)seqlen;
    const size_t inb = tok * (size_t)cd * es;
    const size_t xb = tok * (size_t)(nheads * headdim) * es, bcb = tok * (size_t)(ngroups * dstate) * es;
    const size_t dtb = tok * (size_t)nheads * 4;
    if (overlaps(x, xb, xbc, inb) || overlaps(B, bcb, xbc, inb) || overlaps(C, bcb, xbc, inb) ||
        overlaps(x, xb, B, bcb) || overlaps(x, xb, C, bcb) || overlaps(B, bcb, C, bcb) ||
        overlaps(dt, dtb, dt_raw, dtb) || overlaps(dt, dtb, xbc, inb))
        return SSD_ERR_ALIAS;
    return hip_status(ssd::launch_layer_in(batch, seqlen, nheads, headdim, ngroups, dstate,
                                           (int)kernel_width, dtype, xbc, conv_w, conv_b, dt_raw,
                                           dt_bias, x, B, C, dt, stream));
}

int32_t ssd_layer_out(int64_t n, int32_t dtype, const void* y, const void* z, void* out,
                      hipStream_t stream) {
    if (n < 1 || n > (int64_t)1000000000000LL) return SSD_ERR_SHAPE;
    size_t es;
    if (!elem_size(dtype, &es)) return SSD_ERR_UNSUPPORTED;
    if (!y || !z || !out) return SSD_ERR_NULL;
    if (!aligned(y, es) || !aligned(z, es) || !aligned(out, es)) return SSD_ERR_ALIGN;
    const size_t bytes = (size_t)n * es;
    if (overlaps(out, bytes, z, bytes) || (out != y && overlaps(out, bytes, y, bytes)))
        return SSD_ERR_ALIAS;
    return hip_status(ssd::launch_layer_out(n, dtype, y, z, out, stream));
}

}  // extern "C"
