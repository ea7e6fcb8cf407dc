// ssd_api.cpp -- the C ABI declared in include/ssd_mi355x.h: argument
// validation, workspace carving and the launch order.  No allocation and no
// synchronisation; the only global state is ssd_forward_noalloc's per-device
// array and the cache of its device addresses.
#include "ssd_mi355x.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>

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
    d->nchunks = (seqlen - 1) / chunk + 1;   // seqlen >= 1: no overflow for any chunk
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

// Workspace of ssd_forward (layout documented at ssd_forward_workspace_bytes):
// cs, dtc, S and Hin, the last two in the storage type.
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
    size_t b_cs, b_st;
    if (!mul_ok(rows, 4, &b_cs) || !mul_ok(states, es, &b_st)) return false;
    lo->cs = 0;
    lo->dtc = align_up(b_cs);
    lo->S = lo->dtc + align_up(b_cs);
    lo->Hin = lo->S + align_up(b_st);
    lo->total = lo->Hin + align_up(b_st);
    return true;
}

// The same workspace carved for the two-level recurrence (runs of K >= 2
// chunks): cs, dtc, T (one state per chunk), Hr (one per run), lam (one
// float per chunk), rdec (one per run) -- never more than the layout above.
struct RunLayout {
    size_t cs, dtc, T, Hr, lam, rdec, total;
};

bool run_layout(const Dims& d, int32_t dtype, int64_t K, RunLayout* lo) {
    size_t es;
    if (!elem_size(dtype, &es) || K < 1) return false;
    const size_t bh = (size_t)d.batch * (size_t)d.nheads;
    const size_t nruns = (size_t)((d.nchunks + K - 1) / K);
    const size_t pn = (size_t)d.headdim * (size_t)d.dstate * es;
    const size_t rows = bh * (size_t)d.nchunks * (size_t)d.chunk * 4;
    lo->cs = 0;
    lo->dtc = align_up(rows);
    lo->T = lo->dtc + align_up(rows);
    lo->Hr = lo->T + align_up(bh * (size_t)d.nchunks * pn);
    lo->lam = lo->Hr + align_up(bh * nruns * pn);
    lo->rdec = lo->lam + align_up(bh * (size_t)d.nchunks * 4);
    lo->total = lo->rdec + align_up(bh * nruns * 4);
    return true;
}

// Bytes ssd_forward needs: the larger of the two layouts where the
// two-level recurrence applies (a sequence of one or a few chunks needs more
// for Hr than the per-chunk Hin it replaces).
bool forward_workspace(const Dims& d, int32_t dtype, Layout* lo, size_t* total) {
    if (!workspace_layout(d, dtype, lo)) return false;
    *total = lo->total;
    const int K = ssd::state_runs_apply(dtype, d) ? ssd::state_run_chunks(d) : 0;
    if (K > 0) {
        RunLayout rl;
        if (!run_layout(d, dtype, K, &rl)) return false;
        if (rl.total > *total) *total = rl.total;
    }
    return true;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x0 = reinterpret_cast<uintptr_t>(a), x1 = x0 + na;
    const uintptr_t y0 = reinterpret_cast<uintptr_t>(b), y1 = y0 + nb;
    return x0 < y1 && y0 < x1;
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? SSD_OK : SSD_ERR_HIP; }

// A device array of a call: its first byte and its length (NULL: absent).
struct Span {
    const void* p;
    size_t n;
};

// SSD_ERR_ALIAS when an output overlaps an input or another output.  The
// one pair that may overlap (final_state on init_state, whose entries are
// read before they are written) is named by its indices, or -1.
template <size_t NI, size_t NO>
int32_t check_spans(const Span (&in)[NI], const Span (&out)[NO], int ok_out = -1, int ok_in = -1) {
    for (size_t o = 0; o < NO; ++o) {
        for (size_t i = 0; i < NI; ++i) {
            if ((int)o == ok_out && (int)i == ok_in) continue;
            if (overlaps(out[o].p, out[o].n, in[i].p, in[i].n)) return SSD_ERR_ALIAS;
        }
        for (size_t o2 = o + 1; o2 < NO; ++o2)
            if (overlaps(out[o].p, out[o].n, out[o2].p, out[o2].n)) return SSD_ERR_ALIAS;
    }
    return SSD_OK;
}

// Byte lengths of the arrays the stage calls share (sizes already checked,
// so no product overflows: chunk, P and N are at most 256, 128 and 128 and
// batch * chunks * heads fits 31 bits).
struct Sizes {
    size_t x, bc, dt, head, rows, states, state32;
};

Sizes sizes_of(const Dims& d, size_t es) {
    const size_t tok = (size_t)d.batch * (size_t)d.seqlen;
    const size_t bhc = (size_t)d.batch * (size_t)d.nheads * (size_t)d.nchunks;
    Sizes z;
    z.x = tok * (size_t)d.nheads * (size_t)d.headdim * es;
    z.bc = tok * (size_t)d.ngroups * (size_t)d.dstate * es;
    z.dt = tok * (size_t)d.nheads * 4;
    z.head = (size_t)d.nheads * 4;
    z.rows = bhc * (size_t)d.chunk * 4;
    z.states = bhc * (size_t)d.headdim * (size_t)d.dstate * es;
    z.state32 = (size_t)d.batch * (size_t)d.nheads * (size_t)d.headdim * (size_t)d.dstate * 4;
    return z;
}

}  // namespace

// Workspace of ssd_forward_noalloc: one array per device, resident from the
// library's load until the process ends.  Host code never uses the array's
// name as an address: its device address is looked up once per device
// (scratch_address) and that pointer is what the kernels receive.
static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the
// first call made with that device current).
int32_t scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return SSD_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return SSD_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return SSD_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SSD_OK;
}

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
    size_t total;
    if (!forward_workspace(d, dtype, &lo, &total)) return 0;
    return total;
}

int64_t ssd_forward_run_chunks(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                               int64_t dstate, int64_t ngroups, int64_t chunk, int32_t dtype) {
    Dims d;
    if (check_dims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, &d) != SSD_OK) return 0;
    if (check_supported(dtype, d) != SSD_OK || !ssd::state_runs_apply(dtype, d)) return 0;
    return ssd::state_run_chunks(d);
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
    const Sizes z = sizes_of(d, 4);
    const Span in[] = {{dt, z.dt}, {A, z.head}};
    const Span out[] = {{cs, z.rows}, {dtc, z.rows}};
    if ((st = check_spans(in, out)) != SSD_OK) return st;
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
                        void* S, hipStream_t stream) {
    Dims d;
    int32_t st = check_dims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, &d);
    if (st != SSD_OK) return st;
    if ((st = check_supported(dtype, d)) != SSD_OK) return st;
    if (!x || !B || !cs || !dtc || !S) return SSD_ERR_NULL;
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(S, 16) || !aligned(cs, 4) || !aligned(dtc, 4))
        return SSD_ERR_ALIGN;
    size_t es;
    elem_size(dtype, &es);
    const Sizes z = sizes_of(d, es);
    const Span in[] = {{x, z.x}, {B, z.bc}, {cs, z.rows}, {dtc, z.rows}};
    const Span out[] = {{S, z.states}};
    if ((st = check_spans(in, out)) != SSD_OK) return st;
    return hip_status(ssd::launch_chunk_state(d, dtype, x, B, cs, dtc, S, stream));
}

int32_t ssd_chunk_cumsum_state(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                               int64_t dstate, int64_t ngroups, int64_t chunk, int32_t dtype,
                               const void* x, const void* B, const float* dt, const float* A,
                               float* cs, float* dtc, void* S, hipStream_t stream) {
    Dims d;
    int32_t st = check_dims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, &d);
    if (st != SSD_OK) return st;
    if ((st = check_supported(dtype, d)) != SSD_OK) return st;
    if (!x || !B || !dt || !A || !cs || !dtc || !S) return SSD_ERR_NULL;
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(S, 16) || !aligned(dt, 4) || !aligned(A, 4) ||
        !aligned(cs, 4) || !aligned(dtc, 4))
        return SSD_ERR_ALIGN;
    size_t es;
    elem_size(dtype, &es);
    const Sizes z = sizes_of(d, es);
    const Span in[] = {{x, z.x}, {B, z.bc}, {dt, z.dt}, {A, z.head}};
    const Span out[] = {{cs, z.rows}, {dtc, z.rows}, {S, z.states}};
    if ((st = check_spans(in, out)) != SSD_OK) return st;
    if (ssd::chunk_state_fuses_cumsum(dtype, d))
        return hip_status(ssd::launch_chunk_state_fused(d, x, B, dt, A, 0, cs, dtc, S, stream));
    hipError_t e = ssd::launch_chunk_cumsum(d, dt, A, cs, dtc, stream, 0);
    if (e != hipSuccess) return SSD_ERR_HIP;
    return hip_status(ssd::launch_chunk_state(d, dtype, x, B, cs, dtc, S, stream));
}

int32_t ssd_state_passing(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                          int64_t dstate, int64_t chunk, int32_t dtype, const void* S,
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
    size_t es;
    elem_size(dtype, &es);
    const Sizes z = sizes_of(d, es);
    const Span in[] = {{S, z.states}, {cs, z.rows}, {init_state, z.state32}};
    const Span out[] = {{Hin, z.states}, {final_state, z.state32}};
    if ((st = check_spans(in, out, 1, 2)) != SSD_OK) return st;
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
                              const void* S, const float* cs, const float* init_state, void* Hin,
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
    size_t es;
    elem_size(dtype, &es);
    const Sizes z = sizes_of(d, es);
    const Span in[] = {{S, z.states}, {cs, z.rows}, {init_state, z.state32}};
    const Span out[] = {{Hin, z.states}, {final_state, z.state32}, {workspace, workspace_bytes}};
    if ((st = check_spans(in, out, 1, 2)) != SSD_OK) return st;
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
    const bool walk = ssd::state_walk_applies(dtype, d);
    if (!walk && (!ssd::mfma_path(dtype, d) || d.chunk != 256)) return SSD_ERR_UNSUPPORTED;
    if (!x || !B || !cs || !dtc || !Hin) return SSD_ERR_NULL;
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(Hin, 16) || !aligned(cs, 4) ||
        !aligned(dtc, 4) || (init_state && !aligned(init_state, 16)) ||
        (final_state && !aligned(final_state, 16)))
        return SSD_ERR_ALIGN;
    const Sizes z = sizes_of(d, es);
    const Span in[] = {{x, z.x}, {B, z.bc}, {cs, z.rows}, {dtc, z.rows}, {init_state, z.state32}};
    const Span out[] = {{Hin, z.states}, {final_state, z.state32}};
    if ((st = check_spans(in, out, 1, 4)) != SSD_OK) return st;
    if (walk)
        return hip_status(ssd::launch_state_walk(d, x, B, cs, dtc, init_state, Hin, final_state, stream));
    return hip_status(ssd::launch_state_scan(d, x, B, cs, dtc, init_state, Hin, final_state, stream));
}

// Shared checks of the three two-level stage calls.
static int32_t runs_check(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                          int64_t dstate, int64_t ngroups, int64_t chunk, int32_t dtype,
                          int64_t run_chunks, Dims* d) {
    int32_t st = check_dims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, d);
    if (st != SSD_OK) return st;
    size_t es;
    if (!elem_size(dtype, &es)) return SSD_ERR_UNSUPPORTED;
    if (!ssd::state_runs_apply(dtype, *d)) return SSD_ERR_UNSUPPORTED;
    if (run_chunks < 1 || run_chunks > 65536) return SSD_ERR_SHAPE;
    return SSD_OK;
}

int32_t ssd_chunk_state_runs(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                             int64_t dstate, int64_t ngroups, int64_t chunk, int32_t dtype,
                             int64_t run_chunks, const void* x, const void* B, const float* dt,
                             const float* A, float* cs, float* dtc, void* T, float* lam, float* rdec,
                             hipStream_t stream) {
    Dims d;
    int32_t st = runs_check(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype, run_chunks, &d);
    if (st != SSD_OK) return st;
    if (!x || !B || !dt || !A || !cs || !dtc || !T || !lam || !rdec) return SSD_ERR_NULL;
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(T, 16) || !aligned(dt, 4) || !aligned(A, 4) ||
        !aligned(cs, 4) || !aligned(dtc, 4) || !aligned(lam, 4) || !aligned(rdec, 4))
        return SSD_ERR_ALIGN;
    const Sizes z = sizes_of(d, 2);
    const size_t nruns = (size_t)((d.nchunks + run_chunks - 1) / run_chunks);
    const size_t bh = (size_t)d.batch * (size_t)d.nheads;
    const Span in[] = {{x, z.x}, {B, z.bc}, {dt, z.dt}, {A, z.head}};
    const Span out[] = {{cs, z.rows}, {dtc, z.rows}, {T, z.states}, {lam, bh * (size_t)d.nchunks * 4},
                        {rdec, bh * nruns * 4}};
    if ((st = check_spans(in, out)) != SSD_OK) return st;
    return hip_status(ssd::launch_chunk_state_runs(d, (int)run_chunks, x, B, dt, A, false, cs, dtc, T, lam,
                                                   rdec, stream));
}

int32_t ssd_run_passing(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                        int64_t dstate, int64_t chunk, int32_t dtype, int64_t run_chunks,
                        const void* T, const float* rdec, const float* init_state, void* Hr,
                        float* final_state, hipStream_t stream) {
    Dims d;
    int32_t st = runs_check(batch, seqlen, nheads, headdim, dstate, 1, chunk, dtype, run_chunks, &d);
    if (st != SSD_OK) return st;
    if (!T || !rdec || !Hr) return SSD_ERR_NULL;
    if (!aligned(T, 16) || !aligned(Hr, 16) || !aligned(rdec, 4) ||
        (init_state && !aligned(init_state, 16)) || (final_state && !aligned(final_state, 16)))
        return SSD_ERR_ALIGN;
    const Sizes z = sizes_of(d, 2);
    const size_t nruns = (size_t)((d.nchunks + run_chunks - 1) / run_chunks);
    const size_t bh = (size_t)d.batch * (size_t)d.nheads;
    const Span in[] = {{T, z.states}, {rdec, bh * nruns * 4}, {init_state, z.state32}};
    const Span out[] = {{Hr, bh * nruns * (size_t)(d.headdim * d.dstate) * 2}, {final_state, z.state32}};
    if ((st = check_spans(in, out, 1, 2)) != SSD_OK) return st;
    return hip_status(ssd::launch_run_passing(d, (int)run_chunks, T, rdec, init_state, Hr, final_state, stream));
}

int32_t ssd_chunk_scan_runs(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                            int64_t dstate, int64_t ngroups, int64_t chunk, int32_t dtype,
                            int64_t run_chunks, const void* x, const void* B, const void* C,
                            const float* cs, const float* dtc, const void* T, const void* Hr,
                            const float* lam, const float* D, void* y, hipStream_t stream) {
    Dims d;
    int32_t st = runs_check(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype, run_chunks, &d);
    if (st != SSD_OK) return st;
    if (!x || !B || !C || !cs || !dtc || !T || !Hr || !lam || !y) return SSD_ERR_NULL;
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(T, 16) || !aligned(Hr, 16) ||
        !aligned(y, 16) || !aligned(cs, 4) || !aligned(dtc, 4) || !aligned(lam, 4) || (D && !aligned(D, 4)))
        return SSD_ERR_ALIGN;
    const Sizes z = sizes_of(d, 2);
    const size_t nruns = (size_t)((d.nchunks + run_chunks - 1) / run_chunks);
    const size_t bh = (size_t)d.batch * (size_t)d.nheads;
    const Span in[] = {{x, z.x},      {B, z.bc},       {C, z.bc},
                       {cs, z.rows},  {dtc, z.rows},   {T, z.states},
                       {Hr, bh * nruns * (size_t)(d.headdim * d.dstate) * 2},
                       {lam, bh * (size_t)d.nchunks * 4}, {D, z.head}};
    const Span out[] = {{y, z.x}};
    if ((st = check_spans(in, out)) != SSD_OK) return st;
    return hip_status(ssd::launch_chunk_scan_runs(d, (int)run_chunks, x, B, C, cs, dtc, T, Hr, lam, D, y, stream));
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
    const Sizes z = sizes_of(d, es);
    const Span in[] = {{x, z.x},      {B, z.bc},       {C, z.bc},     {cs, z.rows},
                       {dtc, z.rows}, {Hin, z.states}, {D, z.head}};
    const Span out[] = {{y, z.x}};
    if ((st = check_spans(in, out)) != SSD_OK) return st;
    return hip_status(ssd::launch_chunk_scan(d, dtype, x, B, C, cs, dtc, Hin, D, y, stream));
}

static int32_t forward_impl(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                            int64_t dstate, int64_t ngroups, int64_t chunk, int32_t dtype,
                            const void* x, const float* dt, const float* A, const void* B,
                            const void* C, const float* D, const float* init_state, void* y,
                            float* final_state, void* workspace, size_t workspace_bytes,
                            hipStream_t stream, bool zoh, const void* z = nullptr) {
    Dims d;
    int32_t st = check_dims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, &d);
    if (st != SSD_OK) return st;
    if ((st = check_supported(dtype, d)) != SSD_OK) return st;
    if (!x || !dt || !A || !B || !C || !y) return SSD_ERR_NULL;
    Layout lo;
    size_t wtotal;
    if (!forward_workspace(d, dtype, &lo, &wtotal)) return SSD_ERR_SHAPE;
    if (!workspace || workspace_bytes < wtotal) return SSD_ERR_WORKSPACE;
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(y, 16) ||
        !aligned(workspace, 16) || !aligned(dt, 4) || !aligned(A, 4) || (D && !aligned(D, 4)) ||
        (init_state && !aligned(init_state, 16)) || (final_state && !aligned(final_state, 16)) ||
        (z && !aligned(z, 16)))
        return SSD_ERR_ALIGN;

    size_t es;
    elem_size(dtype, &es);
    const size_t tok = (size_t)d.batch * (size_t)d.seqlen;
    const size_t ybytes = tok * d.nheads * d.headdim * es;
    const size_t bcbytes = tok * d.ngroups * d.dstate * es;
    const size_t dtbytes = tok * d.nheads * 4;
    const size_t hbytes = (size_t)d.nheads * 4;
    const size_t stbytes = (size_t)d.batch * d.nheads * d.headdim * d.dstate * 4;
    // Every output (y, final_state, the workspace) must stay clear of every
    // input (the gate's z included) and of the other outputs; the one
    // permitted overlap is final_state on init_state (the state is read
    // before it is written).
    const Span inputs[] = {{x, ybytes}, {B, bcbytes}, {C, bcbytes}, {dt, dtbytes},
                           {A, hbytes}, {D, hbytes}, {init_state, stbytes}, {z, ybytes}};
    const Span outs[] = {{y, ybytes}, {workspace, wtotal}, {final_state, stbytes}};
    if ((st = check_spans(inputs, outs, 2, 6)) != SSD_OK) return st;

    char* ws = static_cast<char*>(workspace);
    float* cs = reinterpret_cast<float*>(ws + lo.cs);
    float* dtc = reinterpret_cast<float*>(ws + lo.dtc);

    hipError_t e;
    const int K = ssd::state_runs_apply(dtype, d) ? ssd::state_run_chunks(d) : 0;
    if (K > 0) {
        // the two-level recurrence between chunks: chunk states over runs of
        // K chunks, the chain over runs, and the chunk scan forming each
        // chunk's entering state itself (neither S nor Hin in memory)
        RunLayout rl;
        if (!run_layout(d, dtype, K, &rl) || rl.total > wtotal) return SSD_ERR_SHAPE;
        void* T = ws + rl.T;
        void* Hr = ws + rl.Hr;
        float* lam = reinterpret_cast<float*>(ws + rl.lam);
        float* rdec = reinterpret_cast<float*>(ws + rl.rdec);
        e = ssd::launch_chunk_state_runs(d, K, x, B, dt, A, zoh, cs, dtc, T, lam, rdec, stream);
        if (e != hipSuccess) return SSD_ERR_HIP;
        e = ssd::launch_run_passing(d, K, T, rdec, init_state, Hr, final_state, stream);
        if (e != hipSuccess) return SSD_ERR_HIP;
        return hip_status(ssd::launch_chunk_scan_runs(d, K, x, B, C, cs, dtc, T, Hr, lam, D, y, stream, z));
    }
    void* S = ws + lo.S;
    void* Hin = ws + lo.Hin;
    // chunk cumsum and chunk states (one launch where the paired-head kernel
    // applies), then the recurrence between chunks (the one-pass
    // ssd_state_scan measured slower than this pair at every shape tried)
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
    e = ssd::launch_chunk_scan(d, dtype, x, B, C, cs, dtc, Hin, D, y, stream, z);
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

int32_t ssd_forward_noalloc(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                            int64_t dstate, int64_t ngroups, int64_t chunk, int32_t dtype,
                            const void* x, const float* dt, const float* A, const void* B,
                            const void* C, const float* D, const float* init_state, void* y,
                            float* final_state, hipStream_t stream) {
    Dims d;
    int32_t st = check_dims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, &d);
    if (st != SSD_OK) return st;
    if ((st = check_supported(dtype, d)) != SSD_OK) return st;
    Layout lo;
    size_t total;
    if (!forward_workspace(d, dtype, &lo, &total)) return SSD_ERR_SHAPE;
    if (total > (size_t)SSD_NOALLOC_SCRATCH_BYTES) return SSD_ERR_WORKSPACE;
    if (!x || !dt || !A || !B || !C || !y) return SSD_ERR_NULL;
    void* ws = nullptr;
    if ((st = scratch_address(&ws)) != SSD_OK) return st;
    return forward_impl(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype, x, dt, A,
                        B, C, D, init_state, y, final_state, ws, (size_t)SSD_NOALLOC_SCRATCH_BYTES,
                        stream, false);
}

int32_t ssd_forward_gated(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                          int64_t dstate, int64_t ngroups, int64_t chunk, int32_t dtype,
                          const void* x, const float* dt, const float* A, const void* B,
                          const void* C, const float* D, const float* init_state, const void* z,
                          void* y, float* final_state, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
    if (!z) {
        Dims d;
        const int32_t st = check_dims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, &d);
        return st != SSD_OK ? st : SSD_ERR_NULL;
    }
    return forward_impl(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype, x, dt, A,
                        B, C, D, init_state, y, final_state, workspace, workspace_bytes, stream,
                        false, z);
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
