// state_passing.hip -- the linear recurrence between chunks.
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

template <int VW>
__device__ __forceinline__ void store_vec(float* p, int64_t i, const Vec<VW>& r) {
    if constexpr (VW >= 4) {
#pragma unroll
        for (int q = 0; q < VW / 4; ++q)
            reinterpret_cast<float4*>(p)[i * (VW / 4) + q] =
                make_float4(r.v[4 * q], r.v[4 * q + 1], r.v[4 * q + 2], r.v[4 * q + 3]);
    } else if constexpr (VW == 2) {
        reinterpret_cast<float2*>(p)[i] = make_float2(r.v[0], r.v[1]);
    } else {
        p[i] = r.v[0];
    }
}

template <int VW>
__device__ __forceinline__ void store_vec(bf16_t* p, int64_t i, const Vec<VW>& r) {
    if constexpr (VW == 8) {
        reinterpret_cast<uint4*>(p)[i] = make_uint4(pack_bf16x2(r.v[0], r.v[1]), pack_bf16x2(r.v[2], r.v[3]),
                                                    pack_bf16x2(r.v[4], r.v[5]), pack_bf16x2(r.v[6], r.v[7]));
    } else if constexpr (VW == 4) {
        reinterpret_cast<uint2*>(p)[i] = make_uint2(pack_bf16x2(r.v[0], r.v[1]), pack_bf16x2(r.v[2], r.v[3]));
    } else if constexpr (VW == 2) {
        reinterpret_cast<uint32_t*>(p)[i] = pack_bf16x2(r.v[0], r.v[1]);
    } else {
        p[i].bits = (uint16_t)f32_to_bf16_bits(r.v[0]);
    }
}

// Element indices below are in units of VW floats.
template <typename HT, int PF, int VW>
__global__ __launch_bounds__(256) void state_passing_kernel(const float* __restrict__ S,
                                                            const float* __restrict__ cs,
                                                            const float* init, HT* __restrict__ Hin,
                                                            float* fin, int pnv, int nc, int Q) {
    // grid: (batch * heads, element blocks): bh is uniform across the
    // workgroup, so the per-chunk decays are scalar loads, off the vector
    // memory counter that paces the S ring.
    const int64_t bh = blockIdx.x;
    const int off = blockIdx.y * 256 + threadIdx.x;
    if (off >= pnv) return;
    const int64_t idx = bh * pnv + off;

    Vec<VW> h;
    if (init) {
        h = load_vec<VW>(init, idx);
    } else {
#pragma unroll
        for (int e = 0; e < VW; ++e) h.v[e] = 0.0f;
    }
    const int64_t base = bh * nc * (int64_t)pnv + off;
    const float* dec = cs + bh * nc * (int64_t)Q + (Q - 1);

    // The ring holds the next PF chunks.  Its loads are unconditional: a load
    // past the last chunk re-reads the last chunk (always in bounds) and is
    // never used.  Whole groups of PF chunks then run without a branch while
    // chunks remain beyond the group; the last 1..PF chunks run from the ring
    // with no further loads.  (A load
    // or store under a branch makes the compiler wait for the ring's loads at
    // the join, which serialises it.)
    Vec<VW> buf[PF];
    float lg[PF];
#pragma unroll
    for (int k = 0; k < PF; ++k) {
        const int cl = min(k, nc - 1);
        buf[k] = load_vec<VW>(S + (base + (int64_t)cl * pnv) * VW, 0);
        lg[k] = dec[(int64_t)cl * Q];
    }
    HT* hp = Hin + base * VW;
    const int64_t step = (int64_t)pnv * VW;   // floats of one chunk's states
    int c0 = 0;
    for (; c0 + PF < nc; c0 += PF) {
#pragma unroll
        for (int k = 0; k < PF; ++k) {
            // slot k is consumed before its refill is issued, so the refill
            // can land in the same registers (no copy, hence no wait, at the
            // loop's back edge); the barrier keeps that order
            const float a = fast_exp2(lg[k]);
            store_vec<VW>(hp, 0, h);
            hp += step;
#pragma unroll
            for (int e = 0; e < VW; ++e) h.v[e] = a * h.v[e] + buf[k].v[e];
            __builtin_amdgcn_sched_barrier(0);
            const int cn = min(c0 + k + PF, nc - 1);
            buf[k] = load_vec<VW>(S + (base + (int64_t)cn * pnv) * VW, 0);
            lg[k] = dec[(int64_t)cn * Q];
        }
    }
#pragma unroll
    for (int k = 0; k < PF; ++k) {
        if (c0 + k < nc) {
            const float a = fast_exp2(lg[k]);
            store_vec<VW>(hp, 0, h);
            hp += step;
#pragma unroll
            for (int e = 0; e < VW; ++e) h.v[e] = a * h.v[e] + buf[k].v[e];
        }
    }
    if (fin) store_vec<VW>(fin, idx, h);
}

template <typename HT, int PF, int VW>
static void launch_sp_vw(const Dims& d, const float* S, const float* cs, const float* init,
                         void* Hin, float* fin, hipStream_t stream) {
    const int pnv = (int)(d.headdim * d.dstate / VW);
    const dim3 grid((unsigned)(d.batch * d.nheads), (unsigned)((pnv + 255) / 256));
    state_passing_kernel<HT, PF, VW><<<grid, 256, 0, stream>>>(
        S, cs, init, reinterpret_cast<HT*>(Hin), fin, pnv, (int)d.nchunks, (int)d.chunk);
}

// Four elements per thread where P * N allows (measured best at the
// 2.7B shape: 2, 8 or a one-round grid were slower).  Ring depth: 4 chunks
// for short chains, where many waves per SIMD hide the latency; 16 for long
// chains, and 32 when the whole grid is at most two waves per SIMD (32
// chains of 4,096 chunks: 2.32 ms with the old branchy ring, 1.28 ms now, the
// same at depths 16 to 48).
template <typename HT>
static void launch_sp(const Dims& d, const float* S, const float* cs, const float* init,
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

hipError_t launch_state_passing(const Dims& d, int32_t dtype, const float* S, const float* cs,
                                const float* init, void* Hin, float* final_state,
                                hipStream_t stream) {
    if (dtype == 1)
        launch_sp<bf16_t>(d, S, cs, init, Hin, final_state, stream);
    else
        launch_sp<float>(d, S, cs, init, Hin, final_state, stream);
    return hipGetLastError();
}

}  // namespace ssd
