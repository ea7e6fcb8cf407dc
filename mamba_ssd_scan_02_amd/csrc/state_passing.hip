// state_passing.hip -- the linear recurrence between chunks, sequential and
// segmented.
//
// S and Hin are in the storage type (bf16 on the matrix-core path); the
// carried state itself is fp32.
//
// Only the summary state travels from one block to the next (page "Mamba-2
// (2024): SSM e attention sono la stessa cosa", section "Il trucco a blocchi"),
// and the update has the general linear form h_t = A_t h_{t-1} + b_t of page
// "State Space Model", section "Due strade, una meta", here applied once per
// chunk:  Hin_c = H_c,  H_{c+1} = exp(Acs_c[last]) H_c + S_c.
//
// Pure streaming: every state element is independent, one thread owns VW
// consecutive elements of one (batch, head) and walks the chunks in order.
// The loads of S for the next PF chunks (4 to 32, see the launcher) do not
// depend on the carried state, so they are kept in flight in a register ring
// while the chain advances.
#include "device_common.h"
#include "launchers.h"

namespace ssd {

template <int VW>
struct Vec {
    float v[VW];
};

// S is read exactly once: non-temporal loads keep it from displacing data
// that is reused.
template <int VW>
__device__ __forceinline__ Vec<VW> load_vec(const float* p, int64_t i) {
    Vec<VW> r;
    if constexpr (VW >= 4) {
#pragma unroll
        for (int q = 0; q < VW / 4; ++q) {
            const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + i * (VW / 4) + q);
            r.v[4 * q + 0] = t[0]; r.v[4 * q + 1] = t[1]; r.v[4 * q + 2] = t[2]; r.v[4 * q + 3] = t[3];
        }
    } else if constexpr (VW == 2) {
        const f32x2 t = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(p) + i);
        r.v[0] = t[0]; r.v[1] = t[1];
    } else {
        r.v[0] = __builtin_nontemporal_load(p + i);
    }
    return r;
}

// S in bf16 (the matrix-core path stores it in the storage type).
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <int VW>
__device__ __forceinline__ Vec<VW> load_vec(const bf16_t* p, int64_t i) {
    Vec<VW> r;
    if constexpr (VW == 4) {
        const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p) + i);
        r.v[0] = bf16_bits_to_f32(t[0] & 0xffffu); r.v[1] = bf16_bits_to_f32(t[0] >> 16);
        r.v[2] = bf16_bits_to_f32(t[1] & 0xffffu); r.v[3] = bf16_bits_to_f32(t[1] >> 16);
    } else {
#pragma unroll
        for (int e = 0; e < VW; ++e) r.v[e] = bf16_bits_to_f32(p[i * VW + e].bits);
    }
    return r;
}

// The ring's slots hold S as loaded (bf16 pairs stay packed) and are widened
// to fp32 only when the chain consumes them.  Widening at the load would make
// the compiler wait for each load right after issuing it, and the ring would
// hold nothing in flight.
template <typename ST, int VW>
struct RingSlot;
template <int VW>
struct RingSlot<float, VW> {
    Vec<VW> v;
    __device__ __forceinline__ void load(const float* p) { v = load_vec<VW>(p, 0); }
    __device__ __forceinline__ Vec<VW> widen() const { return v; }
};
template <int VW>
struct RingSlot<bf16_t, VW> {
    static constexpr int kWords = VW == 1 ? 1 : VW / 2;
    uint32_t w[kWords];
    __device__ __forceinline__ void load(const bf16_t* p) {
        if constexpr (VW == 4) {
            const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
            w[0] = t[0];
            w[1] = t[1];
        } else if constexpr (VW == 2) {
            w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
        } else if constexpr (VW == 1) {
            w[0] = p[0].bits;
        } else {
#pragma unroll
            for (int q = 0; q < kWords; ++q) w[q] = reinterpret_cast<const uint32_t*>(p)[q];
        }
    }
    __device__ __forceinline__ Vec<VW> widen() const {
        Vec<VW> r;
        if constexpr (VW == 1) {
            r.v[0] = bf16_bits_to_f32(w[0] & 0xffffu);
        } else {
#pragma unroll
            for (int q = 0; q < kWords; ++q) {
                r.v[2 * q] = bf16_bits_to_f32(w[q] & 0xffffu);
                r.v[2 * q + 1] = bf16_bits_to_f32(w[q] >> 16);
            }
        }
        return r;
    }
};

template <int VW, bool NT = false>
__device__ __forceinline__ void store_vec(float* p, int64_t i, const Vec<VW>& r) {
    if constexpr (VW >= 4) {
#pragma unroll
        for (int q = 0; q < VW / 4; ++q) {
            const f32x4 w = {r.v[4 * q], r.v[4 * q + 1], r.v[4 * q + 2], r.v[4 * q + 3]};
            if constexpr (NT)
                __builtin_nontemporal_store(w, reinterpret_cast<f32x4*>(p) + i * (VW / 4) + q);
            else
                reinterpret_cast<f32x4*>(p)[i * (VW / 4) + q] = w;
        }
    } else if constexpr (VW == 2) {
        reinterpret_cast<float2*>(p)[i] = make_float2(r.v[0], r.v[1]);
    } else {
        p[i] = r.v[0];
    }
}

// NT: non-temporal stores, for an Hin too large to stay in the last-level
// cache until chunk_scan reads it (see launch_sp).
template <int VW, bool NT = false>
__device__ __forceinline__ void store_vec(bf16_t* p, int64_t i, const Vec<VW>& r) {
    if constexpr (VW == 8) {
        reinterpret_cast<uint4*>(p)[i] = make_uint4(pack_bf16x2(r.v[0], r.v[1]), pack_bf16x2(r.v[2], r.v[3]),
                                                    pack_bf16x2(r.v[4], r.v[5]), pack_bf16x2(r.v[6], r.v[7]));
    } else if constexpr (VW == 4) {
        const u32x2 w = {pack_bf16x2(r.v[0], r.v[1]), pack_bf16x2(r.v[2], r.v[3])};
        if constexpr (NT)
            __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(p) + i);
        else
            reinterpret_cast<u32x2*>(p)[i] = w;
    } else if constexpr (VW == 2) {
        reinterpret_cast<uint32_t*>(p)[i] = pack_bf16x2(r.v[0], r.v[1]);
    } else {
        p[i].bits = (uint16_t)f32_to_bf16_bits(r.v[0]);
    }
}

// Walks n >= 1 chunks of one thread's VW state elements:
//     [store h at hp], h <- exp2(lg_c) h + S_c,   c = 0 .. n - 1,
// where S_c sits at src + c * sstep (elements of ST) and lg_c, the chunk's decay in
// log2 units, at dec[c * dstep].  kStore writes the entering state of every
// chunk (hp advances by hstep, sstep when hstep is 0), non-temporally with
// kNT; kSum adds the lg_c into *lsum.
//
// The ring holds the next PF chunks.  Its loads are unconditional: a load past
// the last chunk re-reads the last chunk (always in bounds) and is never used.
// Whole groups of PF chunks then run without a branch while chunks remain
// beyond the group; the last 1..PF chunks run from the ring with no further
// loads.  (A load or store under a branch makes the compiler wait for the
// ring's loads at the join, which serialises it.)
template <typename ST, typename HT, int PF, int VW, bool kStore, bool kSum, bool kNT = false>
__device__ __forceinline__ void walk_chunks(const ST* __restrict__ src, int64_t sstep,
                                            const float* __restrict__ dec, int64_t dstep, int n,
                                            HT* hp, Vec<VW>& h, float* lsum, int64_t hstep = 0) {
    if (hstep == 0) hstep = sstep;
    RingSlot<ST, VW> buf[PF];
    float lg[PF];
#pragma unroll
    for (int k = 0; k < PF; ++k) {
        const int cl = min(k, n - 1);
        buf[k].load(src + (int64_t)cl * sstep);
        lg[k] = dec[(int64_t)cl * dstep];
    }
    float ls = 0.0f;
    int c0 = 0;
    for (; c0 + PF < n; c0 += PF) {
#pragma unroll
        for (int k = 0; k < PF; ++k) {
            // slot k is consumed before its refill is issued, so the refill
            // can land in the same registers (no copy, hence no wait, at the
            // loop's back edge); the barrier keeps that order
            const float a = fast_exp2(lg[k]);
            if (kSum) ls += lg[k];
            if (kStore) {
                store_vec<VW, kNT>(hp, 0, h);
                hp += hstep;
            }
            const Vec<VW> sv = buf[k].widen();
#pragma unroll
            for (int e = 0; e < VW; ++e) h.v[e] = a * h.v[e] + sv.v[e];
            __builtin_amdgcn_sched_barrier(0);
            const int cn = min(c0 + k + PF, n - 1);
            buf[k].load(src + (int64_t)cn * sstep);
            lg[k] = dec[(int64_t)cn * dstep];
        }
    }
#pragma unroll
    for (int k = 0; k < PF; ++k) {
        if (c0 + k < n) {
            const float a = fast_exp2(lg[k]);
            if (kSum) ls += lg[k];
            if (kStore) {
                store_vec<VW, kNT>(hp, 0, h);
                hp += hstep;
            }
            const Vec<VW> sv = buf[k].widen();
#pragma unroll
            for (int e = 0; e < VW; ++e) h.v[e] = a * h.v[e] + sv.v[e];
        }
    }
    if (kSum) *lsum = ls;
}

template <int VW>
__device__ __forceinline__ Vec<VW> start_state(const float* init, int64_t idx) {
    Vec<VW> h;
    if (init) {
        h = load_vec<VW>(init, idx);
    } else {
#pragma unroll
        for (int e = 0; e < VW; ++e) h.v[e] = 0.0f;
    }
    return h;
}

// Element indices below are in units of VW floats; pnv = P N / VW.  Grids put
// (batch, head) on x, so the decays are uniform across a workgroup and come
// from scalar loads, off the vector memory counter that paces the S ring.
template <typename HT, int PF, int VW, bool NT>
__global__ __launch_bounds__(256) void state_passing_kernel(const HT* __restrict__ S,
                                                            const float* __restrict__ cs,
                                                            const float* init, HT* __restrict__ Hin,
                                                            float* fin, int pnv, int nc, int Q) {
    const int64_t bh = blockIdx.x;
    const int off = blockIdx.y * 256 + threadIdx.x;
    if (off >= pnv) return;
    const int64_t idx = bh * pnv + off;
    Vec<VW> h = start_state<VW>(init, idx);
    const int64_t base = (bh * nc * (int64_t)pnv + off) * VW;
    walk_chunks<HT, HT, PF, VW, true, false, NT>(S + base, (int64_t)pnv * VW,
                                                 cs + bh * nc * (int64_t)Q + (Q - 1), Q, nc, Hin + base, h,
                                                 nullptr);
    if (fin) store_vec<VW>(fin, idx, h);
}

// ---------------------------------------------------------------------------
// Segmented form: two consecutive steps of a linear recurrence merge into one
// step of the same kind (the parallel scan of page "State Space Model",
// section "Dai sistemi dinamici a Mamba"): (a1, s1) then (a2, s2) is
// (a2 a1, a2 s1 + s2).  So the chunks are cut into segments of `seg` chunks
// and scanned in two levels:
//   1. seg_reduce: each segment's end state from zero, E_s, and its summed
//      log2 decay D_s (all segments in parallel);
//   2. seg_carry:  the state entering each segment, Hs_{s+1} = exp2(D_s) Hs_s
//      + E_s from the initial state, and the final state (a chain of nseg);
//   3. seg_down:   each segment again from Hs_s, writing Hin (all in parallel).
// Depth nc / nseg + nseg instead of nc, for 1.5x the S reads.

template <typename ST, int PF, int VW>
__global__ __launch_bounds__(256) void sp_seg_reduce_kernel(const ST* __restrict__ S,
                                                            const float* __restrict__ cs,
                                                            float* __restrict__ E,
                                                            float* __restrict__ Dseg, int pnv,
                                                            int nc, int Q, int seg, int nseg) {
    const int64_t bh = blockIdx.x;
    const int s = blockIdx.y;
    const int off = blockIdx.z * 256 + threadIdx.x;
    if (off >= pnv) return;
    const int c0 = s * seg, n = min(seg, nc - c0);
    Vec<VW> h;
#pragma unroll
    for (int e = 0; e < VW; ++e) h.v[e] = 0.0f;
    float ls = 0.0f;
    walk_chunks<ST, float, PF, VW, false, true>(S + ((bh * nc + c0) * (int64_t)pnv + off) * VW,
                                            (int64_t)pnv * VW,
                                            cs + (bh * nc + c0) * (int64_t)Q + (Q - 1), Q, n,
                                            (float*)nullptr, h, &ls);
    store_vec<VW>(E, (bh * nseg + s) * (int64_t)pnv + off, h);
    if (off == 0) Dseg[bh * nseg + s] = ls;
}

template <int PF, int VW>
__global__ __launch_bounds__(256) void sp_seg_carry_kernel(const float* __restrict__ E,
                                                           const float* __restrict__ Dseg,
                                                           const float* init,
                                                           float* __restrict__ Hs, float* fin,
                                                           int pnv, int nseg) {
    const int64_t bh = blockIdx.x;
    const int off = blockIdx.y * 256 + threadIdx.x;
    if (off >= pnv) return;
    const int64_t idx = bh * pnv + off;
    Vec<VW> h = start_state<VW>(init, idx);
    const int64_t base = (bh * nseg * (int64_t)pnv + off) * VW;
    walk_chunks<float, float, PF, VW, true, false>(E + base, (int64_t)pnv * VW, Dseg + bh * nseg, 1, nseg,
                                                   Hs + base, h, nullptr);
    if (fin) store_vec<VW>(fin, idx, h);
}

template <typename HT, int PF, int VW>
__global__ __launch_bounds__(256) void sp_seg_down_kernel(const HT* __restrict__ S,
                                                          const float* __restrict__ cs,
                                                          const float* __restrict__ Hs,
                                                          HT* __restrict__ Hin, int pnv, int nc,
                                                          int Q, int seg, int nseg) {
    const int64_t bh = blockIdx.x;
    const int s = blockIdx.y;
    const int off = blockIdx.z * 256 + threadIdx.x;
    if (off >= pnv) return;
    const int c0 = s * seg, n = min(seg, nc - c0);
    Vec<VW> h = load_vec<VW>(Hs, (bh * nseg + s) * (int64_t)pnv + off);
    const int64_t base = ((bh * nc + c0) * (int64_t)pnv + off) * VW;
    walk_chunks<HT, HT, PF, VW, true, false>(S + base, (int64_t)pnv * VW,
                                             cs + (bh * nc + c0) * (int64_t)Q + (Q - 1), Q, n, Hin + base,
                                             h, nullptr);
}

// ---------------------------------------------------------------------------
// The second level of the two-level recurrence whose first level is the
// chunk state over runs of K chunks (chunk_state_runs_kernel): a chain over
// the runs,
//     Hr_0 = init,   Hr_{r+1} = exp2(rdec_r) Hr_r + T_{last chunk of run r},
// writing every run's entering state Hr_r (storage type) and the final state
// exp2(rdec_last) Hr_last + T_{nc-1} (fp32).  Full runs end at chunk
// rK + K - 1, so their T are K chunks apart; the last run may be shorter and
// ends at chunk nc - 1.
template <typename HT, int PF, int VW>
__global__ __launch_bounds__(256) void run_passing_kernel(const HT* __restrict__ T,
                                                          const float* __restrict__ rdec,
                                                          const float* init, HT* __restrict__ Hr,
                                                          float* fin, int pnv, int nc, int K,
                                                          int nruns) {
    const int64_t bh = blockIdx.x;
    const int off = blockIdx.y * 256 + threadIdx.x;
    if (off >= pnv) return;
    const int64_t idx = bh * pnv + off;
    Vec<VW> h = start_state<VW>(init, idx);
    const int64_t pn = (int64_t)pnv * VW;
    const HT* tb = T + (bh * nc * (int64_t)pnv + off) * VW;
    HT* hb = Hr + (bh * nruns * (int64_t)pnv + off) * VW;
    if (nruns > 1)
        walk_chunks<HT, HT, PF, VW, true, false>(tb + (int64_t)(K - 1) * pn, (int64_t)K * pn,
                                                 rdec + bh * nruns, 1, nruns - 1, hb, h, nullptr, pn);
    store_vec<VW>(hb, (int64_t)(nruns - 1) * pnv, h);
    if (fin) {
        const float a = fast_exp2(rdec[bh * nruns + nruns - 1]);
        RingSlot<HT, VW> last;
        last.load(tb + (int64_t)(nc - 1) * pn);
        const Vec<VW> tv = last.widen();
#pragma unroll
        for (int e = 0; e < VW; ++e) h.v[e] = a * h.v[e] + tv.v[e];
        store_vec<VW>(fin, idx, h);
    }
}

hipError_t launch_run_passing(const Dims& d, int K, const void* T, const float* rdec, const float* init,
                              void* Hr, float* final_state, hipStream_t stream) {
    const int nc = (int)d.nchunks, nruns = (nc + K - 1) / K;
    constexpr int VW = 4;
    const int pnv = (int)(d.headdim * d.dstate / VW);
    const dim3 grid((unsigned)(d.batch * d.nheads), (unsigned)((pnv + 255) / 256));
    const bf16_t* t = static_cast<const bf16_t*>(T);
    bf16_t* hr = static_cast<bf16_t*>(Hr);
    if (nruns > 64)
        run_passing_kernel<bf16_t, 16, VW><<<grid, 256, 0, stream>>>(t, rdec, init, hr, final_state, pnv, nc, K, nruns);
    else
        run_passing_kernel<bf16_t, 4, VW><<<grid, 256, 0, stream>>>(t, rdec, init, hr, final_state, pnv, nc, K, nruns);
    return hipGetLastError();
}

constexpr double kHinTemporalMaxBytes = 64.0 * 1024 * 1024;

template <typename HT, int PF, int VW>
static void launch_sp_vw(const Dims& d, const void* S, const float* cs, const float* init,
                         void* Hin, float* fin, hipStream_t stream) {
    const int pnv = (int)(d.headdim * d.dstate / VW);
    const dim3 grid((unsigned)(d.batch * d.nheads), (unsigned)((pnv + 255) / 256));
    // Hin is read once, by chunk_scan.  Where it fits well inside the 256 MB
    // last-level cache, ordinary stores leave it there for that read (the
    // 130M-shaped forward, 25 MB: 65.9 us against 67.1 with non-temporal
    // stores on one box, equal on another); beyond, non-temporal stores
    // write it back during state passing instead of during chunk_scan (2.7B
    // shape, 168 MB: state passing 61 -> 70 us, chunk_scan 205 -> 197 us,
    // the forward within 1% either way).
    const double hin_bytes = (double)d.batch * (double)d.nheads * (double)d.nchunks *
                             (double)(d.headdim * d.dstate) * (double)sizeof(HT);
    const HT* s = static_cast<const HT*>(S);
    HT* h = reinterpret_cast<HT*>(Hin);
    if (hin_bytes > kHinTemporalMaxBytes)
        state_passing_kernel<HT, PF, VW, true><<<grid, 256, 0, stream>>>(s, cs, init, h, fin, pnv,
                                                                         (int)d.nchunks, (int)d.chunk);
    else
        state_passing_kernel<HT, PF, VW, false><<<grid, 256, 0, stream>>>(s, cs, init, h, fin, pnv,
                                                                          (int)d.nchunks, (int)d.chunk);
}

// Four elements per thread where P * N allows (measured best at the
// 2.7B shape: 2, 8 or a one-round grid were slower).  Ring depth: 4 chunks
// for short chains, where many waves per SIMD hide the latency; 16 for long
// chains, and 32 when the whole grid is at most two waves per SIMD (32
// chains of 4,096 chunks: 2.32 ms with the old branchy ring, 1.28 ms now, the
// same at depths 16 to 48).
template <typename HT>
static void launch_sp(const Dims& d, const void* S, const float* cs, const float* init,
                      void* Hin, float* fin, hipStream_t stream) {
    const bool longseq = d.nchunks >= 64;
    if ((d.headdim * d.dstate) % 4 == 0) {
        int dev = 0, cus = 256;
        if (hipGetDevice(&dev) == hipSuccess) {
            int v = 0;
            if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
        }
        const double waves = (double)d.batch * (double)d.nheads * (double)(d.headdim * d.dstate / 4) / 64.0;
        if (longseq && waves <= 8.0 * cus) launch_sp_vw<HT, 32, 4>(d, S, cs, init, Hin, fin, stream);
        else if (longseq) launch_sp_vw<HT, 16, 4>(d, S, cs, init, Hin, fin, stream);
        else launch_sp_vw<HT, 4, 4>(d, S, cs, init, Hin, fin, stream);
    } else {
        if (longseq) launch_sp_vw<HT, 32, 1>(d, S, cs, init, Hin, fin, stream);
        else launch_sp_vw<HT, 8, 1>(d, S, cs, init, Hin, fin, stream);
    }
}

// Segment length and count actually used for a requested count.
void state_passing_segments(int64_t nc, int64_t nseg_req, int64_t* seg, int64_t* nseg) {
    const int64_t want = nseg_req < 1 ? 1 : (nseg_req > nc ? nc : nseg_req);
    *seg = (nc + want - 1) / want;
    *nseg = (nc + *seg - 1) / *seg;
}

static int64_t up256(int64_t v) { return (v + 255) / 256 * 256; }

size_t state_passing_seg_workspace_bytes(int64_t batch, int64_t H, int64_t P, int64_t N,
                                         int64_t nseg) {
    const int64_t states = batch * H * nseg * P * N * 4;
    return (size_t)(2 * up256(states) + up256(batch * H * nseg * 4));
}

template <typename HT, int VW>
static void launch_seg_vw(const Dims& d, int64_t seg, int64_t nseg, const void* Sv, const float* cs,
                          const float* init, void* Hin, float* fin, char* ws, hipStream_t stream) {
    const HT* S = static_cast<const HT*>(Sv);
    const int pnv = (int)(d.headdim * d.dstate / VW);
    const int64_t states = d.batch * d.nheads * nseg * d.headdim * d.dstate * 4;
    float* E = reinterpret_cast<float*>(ws);
    float* Hs = reinterpret_cast<float*>(ws + up256(states));
    float* Dseg = reinterpret_cast<float*>(ws + 2 * up256(states));
    const unsigned bh = (unsigned)(d.batch * d.nheads), eb = (unsigned)((pnv + 255) / 256);
    const dim3 g3(bh, (unsigned)nseg, eb), g2(bh, eb);
    constexpr int PFS = VW == 4 ? 8 : 16;   // segment walks: many waves hide the latency
    sp_seg_reduce_kernel<HT, PFS, VW><<<g3, 256, 0, stream>>>(S, cs, E, Dseg, pnv, (int)d.nchunks,
                                                          (int)d.chunk, (int)seg, (int)nseg);
    sp_seg_carry_kernel<16, VW><<<g2, 256, 0, stream>>>(E, Dseg, init, Hs, fin, pnv, (int)nseg);
    sp_seg_down_kernel<HT, PFS, VW><<<g3, 256, 0, stream>>>(S, cs, Hs, reinterpret_cast<HT*>(Hin), pnv,
                                                            (int)d.nchunks, (int)d.chunk, (int)seg,
                                                            (int)nseg);
}

hipError_t launch_state_passing_seg(const Dims& d, int32_t dtype, int64_t nseg_req, const void* S,
                                    const float* cs, const float* init, void* Hin,
                                    float* final_state, void* workspace, hipStream_t stream) {
    int64_t seg, nseg;
    state_passing_segments(d.nchunks, nseg_req, &seg, &nseg);
    char* ws = static_cast<char*>(workspace);
    const bool v4 = (d.headdim * d.dstate) % 4 == 0;
    if (dtype == 1) {
        if (v4) launch_seg_vw<bf16_t, 4>(d, seg, nseg, S, cs, init, Hin, final_state, ws, stream);
        else launch_seg_vw<bf16_t, 1>(d, seg, nseg, S, cs, init, Hin, final_state, ws, stream);
    } else {
        if (v4) launch_seg_vw<float, 4>(d, seg, nseg, S, cs, init, Hin, final_state, ws, stream);
        else launch_seg_vw<float, 1>(d, seg, nseg, S, cs, init, Hin, final_state, ws, stream);
    }
    return hipGetLastError();
}

hipError_t launch_state_passing(const Dims& d, int32_t dtype, const void* S, const float* cs,
                                const float* init, void* Hin, float* final_state,
                                hipStream_t stream) {
    if (dtype == 1)
        launch_sp<bf16_t>(d, S, cs, init, Hin, final_state, stream);
    else
        launch_sp<float>(d, S, cs, init, Hin, final_state, stream);
    return hipGetLastError();
}

}  // namespace ssd
