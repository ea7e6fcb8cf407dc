// chunk_state.hip -- each chunk's end state, starting from a zero state:
//
//     S_c[p][n] = sum_j w_j x_j[p] B_j[n],   w_j = exp(Acs[last] - Acs[j]) dt_j
//
// The summary state that leaves a block (page "Mamba-2 (2024): SSM e
// attention sono la stessa cosa", section "Il trucco a blocchi"), written as
// one matrix product per (batch, chunk, head) -- the block matmuls that page
// tech.tersel.eu ("Rewolucja Mamba-2 i teoria State Space Duality SSD") puts on
// the matrix units.
//
// Matrix-core kernel (bf16 storage, P = 64, N = 128): M = P, N = N, K = the
// chunk's tokens, with v_mfma_f32_32x32x16_bf16 and fp32 accumulation.  Both
// operands are token-major in memory while the instruction wants the K index
// (tokens) contiguous per lane: 32-token blocks of B and x are copied
// straight into LDS (lds_pipe.h) and read back transposed with
// ds_read_b64_tr_b16, which hands each lane 4 consecutive tokens of one
// column.  w_j is applied to the B fragment in fp32 and the product rounded
// once to bf16.
//
// Generic kernel (fp32 or bf16, any P, N within limits): tiles of 32 tokens in
// LDS, fp32 FMA on the vector units.
#include "device_common.h"
#include "launchers.h"
#include "lds_pipe.h"

namespace ssd {

// Multiply the 8 bf16 of a fragment by 8 fp32 weights and round back to bf16.
__device__ __forceinline__ uint4 scale_bf16x8(uint4 v, const float (&w)[8]) {
    const uint32_t in[4] = {v.x, v.y, v.z, v.w};
    uint32_t out[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const float lo = bf16_bits_to_f32(in[m] & 0xffffu) * w[2 * m];
        const float hi = bf16_bits_to_f32(in[m] >> 16) * w[2 * m + 1];
        out[m] = pack_bf16x2(lo, hi);
    }
    return make_uint4(out[0], out[1], out[2], out[3]);
}

// Store the two 32-row tiles acc[0..1] (MFMA result layout: register r of
// lane (hf, l32) of wave w is row p = 32 mt + 8 (r / 4) + 4 hf + r % 4,
// column n = 32 w + l32) of a P x N = 64 x 128 state into row-major bf16 at
// dst.  Neighbouring lanes swap one value so that each holds two adjacent
// columns of one row (registers r and r + 1 are rows p and p + 1) and writes
// them as one word: even lanes row p at columns n, n + 1, odd lanes row p + 1
// at columns n - 1, n.  Non-temporal: the state is read once, later.
__device__ __forceinline__ void store_state_bf16(const f32x16 (&acc)[2], bf16_t* dst, int lane, int n) {
    constexpr int N = 128;
    const bool odd = (lane & 1) != 0;
    const int hf = lane >> 5;
    uint32_t* row = reinterpret_cast<uint32_t*>(dst);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const float h0v = acc[mt][r], h1v = acc[mt][r + 1];
            const float got = __shfl_xor(odd ? h0v : h1v, 1, 64);
            const float keep = odd ? h1v : h0v;
            const int rr = odd ? r + 1 : r;
            const int p = 32 * mt + 8 * (rr >> 2) + 4 * hf + (rr & 3);
            const uint32_t w = odd ? pack_bf16x2(got, keep) : pack_bf16x2(keep, got);
            __builtin_nontemporal_store(w, &row[(p * N + (n & ~1)) >> 1]);
        }
}

constexpr int kStateRing = 3;
// Stages issued after stage jt when step jt waits for it (R - 1 are issued
// ahead, none past the last of NT).
__host__ __device__ constexpr int state_ring_ahead(int NT, int R, int jt) {
    return (NT - 1 - jt) < (R - 2) ? (NT - 1 - jt) : (R - 2);
}
// The ring's issue order (stages of DPS copies) replayed against those
// waits: stage jt must have landed at step jt.
constexpr bool state_ring_waits_hold(int NT, int R, int DPS) {
    VmemLog o;
    for (int k = 0; k < R - 1 && k < NT; ++k) o.push(k, DPS);
    for (int jt = 0; jt < NT; ++jt) {
        if (!o.wait(DPS * state_ring_ahead(NT, R, jt)) || !o.landed(jt)) return false;
        if (jt + R - 1 < NT) o.push(jt + R - 1, DPS);
    }
    return true;
}
// Heads per workgroup where a group's head count allows it, else one.  At the
// 2.7B shape: 1 head 151 us, 2 heads 134-138 us, 4 heads 139-141 us.
constexpr int kStateHeads = 2;

// One workgroup (4 waves) per (batch, chunk, head).  Wave w owns state
// columns n in [32w, 32w+32) for both 32-row tiles of p.  The chunk's tokens
// stream through a 3-buffer ring of 32-token blocks of B and x copied
// straight into LDS; both operands are read token-contiguous with tr16, and
// the decay-and-step weight w_j is applied to the B fragment in fp32 before
// the single rounding to bf16.
template <int Q>
__global__ __launch_bounds__(256, 2) void chunk_state_mfma_kernel(const bf16_t* __restrict__ x,
                                                                  const bf16_t* __restrict__ Bm,
                                                                  const float* __restrict__ cs,
                                                                  const float* __restrict__ dtc,
                                                                  bf16_t* __restrict__ S, int L, int H,
                                                                  int G, int nc) {
    constexpr int P = 64, N = 128, W = 4, NT = Q / 32;
    constexpr int DPS = 12 / W;          // copies per wave per 32-token stage
    constexpr int R = kStateRing;        // ring stages (R - 1 issued ahead)
    static_assert(state_ring_waits_hold(NT, R, DPS), "chunk_state wait counts do not cover its copies");
    __shared__ uint4 bsr[R][512];
    __shared__ uint4 xsr[R][256];
    __shared__ float wv[Q];

    const uint32_t wg = xcd_logical_id(blockIdx.x, gridDim.x);
    const int h = (int)(wg % (uint32_t)H);
    const int bc = (int)(wg / (uint32_t)H);
    const int c = bc % nc, b = bc / nc;
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hf = lane >> 5, l32 = lane & 31;
    const int64_t row = (((int64_t)b * H + h) * nc + c) * Q;
    const int tok0 = c * Q;
    const int64_t xstride = (int64_t)H * P, bstride = (int64_t)G * N;
    const bf16_t* xbase = x + ((int64_t)b * L * H + h) * P;
    const bf16_t* bbase = Bm + ((int64_t)b * L * G + g) * N;

    // ordinary loads first, so that the compiler's wait for them does not
    // also wait for the LDS copies issued after: w_j = exp2(cs_last - cs_j) dt_j
    float w_v = 0.0f;
    if (tid < Q) w_v = fast_exp2(cs[row + Q - 1] - cs[row + tid]) * dtc[row + tid];
    asm volatile("" ::: "memory");
    const BxOffsets<W> bxo = bx_offsets<W>(wave, lane, xstride, bstride);
#pragma unroll
    for (int k = 0; k < R - 1; ++k)
        if (k < NT) issue_bx_stage<W>(wave, lane, tok0 + 32 * k, L, xbase, xstride, bbase, bstride, bxo, bsr[k], xsr[k]);
    if (tid < Q) wv[tid] = w_v;

    // tr16 addressing: lane r of group grp supplies token row 8*(grp/2) + r/4
    // (+ 16u + 4*half) and column quad 16*(grp%2) + 4*(r%4) (identity order).
    const int grp = lane >> 4, rr = lane & 15;
    const int trow0 = 8 * (grp >> 1) + (rr >> 2);
    const int qcol = 16 * (grp & 1) + 4 * (rr & 3);

    f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) {
        uint4* bst = bsr[jt % R];
        uint4* xst = xsr[jt % R];
        wait_vmcnt_n(DPS * state_ring_ahead(NT, R, jt));   // a constant once the loop is unrolled
        barrier_lds();
        if (jt + R - 1 < NT)
            issue_bx_stage<W>(wave, lane, tok0 + 32 * (jt + R - 1), L, xbase, xstride, bbase, bstride, bxo,
                              bsr[(jt + R - 1) % R], xsr[(jt + R - 1) % R]);
        const SSD_LDS char* xb = (const SSD_LDS char*)lds(xst);
        const SSD_LDS char* bb = (const SSD_LDS char*)lds(bst);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int r0 = 16 * u + trow0, r1 = r0 + 4;
            // B^T fragment: columns n = 32*wave + 16*(grp%2) + i, 8 tokens
            uint4 bq;
            {
                const int nc4 = 32 * wave + qcol;
                const int chk = nc4 >> 3, sub = (nc4 & 7) * 2;
                const uint2 lo = tr16(bb + r0 * 256 + ((chk ^ swz_b(r0)) << 4) + sub);
                const uint2 hi = tr16(bb + r1 * 256 + ((chk ^ swz_b(r1)) << 4) + sub);
                bq = make_uint4(lo.x, lo.y, hi.x, hi.y);
            }
            float wj[8];
#pragma unroll
            for (int sidx = 0; sidx < 8; ++sidx) wj[sidx] = wv[32 * jt + 16 * u + 8 * hf + sidx];
            const bf16x8 bw = __builtin_bit_cast(bf16x8, scale_bf16x8(bq, wj));
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const int pc = 32 * mt + qcol;
                const int chk = pc >> 3, sub = (pc & 7) * 2;
                const uint2 lo = tr16(xb + r0 * 128 + ((chk ^ swz_x(r0)) << 4) + sub);
                const uint2 hi = tr16(xb + r1 * 128 + ((chk ^ swz_x(r1)) << 4) + sub);
                const bf16x8 xq = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
                acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xq, bw, acc[mt], 0, 0, 0);
            }
        }
    }

    store_state_bf16(acc, S + (((int64_t)b * H + h) * nc + c) * (int64_t)(P * N), lane, 32 * wave + l32);
}

// HG (2 or 4) heads per workgroup: one workgroup per (batch, chunk, HG
// consecutive heads of one group).  Their x rows are HG * 128 contiguous
// bytes per token, copied with the same swizzle as B's rows (the LDS banks
// repeat every 256 bytes, so rows of 256 or 512 bytes see the same pattern),
// and each B fragment read from LDS serves all HG heads (scaled by each
// head's weights).  Wave w owns state columns n in [32w, 32w+32) of every
// head.  Wider rows read faster from HBM than one head's 128-byte rows, and B
// crosses L2 -> LDS once per HG heads.  x is copied non-temporally (138 ->
// 132 us at the 2.7B shape), except for the heads whose x the chunk scan
// reads first (x_keep_positions), which stay in the last-level cache.
template <int W, int HG>
struct BxhOffsets {
    static constexpr int XC = 4 * HG / W;   // x copies per wave per stage
    uint32_t b[8 / W];
    uint32_t x[XC];
};

template <int W, int HG>
__device__ __forceinline__ BxhOffsets<W, HG> bxh_offsets(int wave, int lane, int64_t xstride,
                                                         int64_t bstride) {
    constexpr int PPR = 8 * HG, RPC = 64 / PPR;   // x: 16-byte pieces per row, rows per copy
    BxhOffsets<W, HG> o;
#pragma unroll
    for (int i = 0; i < 8 / W; ++i) {
        const int r = 4 * (wave + i * W) + (lane >> 4);
        o.b[i] = (uint32_t)r * (uint32_t)bstride * 2u + 16u * (uint32_t)((lane & 15) ^ swz_b(r));
    }
#pragma unroll
    for (int i = 0; i < BxhOffsets<W, HG>::XC; ++i) {
        const int r = RPC * (wave + i * W) + lane / PPR;
        o.x[i] = (uint32_t)r * (uint32_t)xstride * 2u + 16u * (uint32_t)((lane % PPR) ^ swz_b(r));
    }
    return o;
}

// 32 tokens of B (32 x 256 B) and of the heads' x (32 x HG * 128 B) into one
// pipeline buffer; rows past the end re-read the last token (their weights
// are zero).
template <int W, int HG>
__device__ __forceinline__ void issue_bxh_stage(int wave, int lane, int tokbase, int L,
                                                const bf16_t* xbase, int64_t xstride,
                                                const bf16_t* bbase, int64_t bstride,
                                                const BxhOffsets<W, HG>& off, uint4* bst, uint4* xst,
                                                bool keep) {
    constexpr int PPR = 8 * HG, RPC = 64 / PPR, XC = BxhOffsets<W, HG>::XC;
    asm volatile("" : "+s"(tokbase));
    if (tokbase + 31 < L) {
        const char* bb = reinterpret_cast<const char*>(bbase + (int64_t)tokbase * bstride);
        const char* xb = reinterpret_cast<const char*>(xbase + (int64_t)tokbase * xstride);
#pragma unroll
        for (int i = 0; i < 8 / W; ++i) dma16(bb, off.b[i], lds(bst) + (wave + i * W) * 64);
        if (keep) {
#pragma unroll
            for (int i = 0; i < XC; ++i) dma16(xb, off.x[i], lds(xst) + (wave + i * W) * 64);
        } else {
#pragma unroll
            for (int i = 0; i < XC; ++i) dma16_nt(xb, off.x[i], lds(xst) + (wave + i * W) * 64);
        }
        return;
    }
    const int tb = min(tokbase, L - 1);
    const char* bb = reinterpret_cast<const char*>(bbase + (int64_t)tb * bstride);
    const char* xb = reinterpret_cast<const char*>(xbase + (int64_t)tb * xstride);
    const uint32_t bs2 = (uint32_t)bstride * 2u, xs2 = (uint32_t)xstride * 2u;
#pragma unroll
    for (int i = 0; i < 8 / W; ++i) {
        const int k = wave + i * W;
        const int r = 4 * k + (lane >> 4);
        const uint32_t dr = (uint32_t)(min(tokbase + r, L - 1) - tb);
        dma16(bb, dr * bs2 + 16u * (uint32_t)((lane & 15) ^ swz_b(r)), lds(bst) + k * 64);
    }
#pragma unroll
    for (int i = 0; i < XC; ++i) {
        const int k = wave + i * W;
        const int r = RPC * k + lane / PPR;
        const uint32_t dr = (uint32_t)(min(tokbase + r, L - 1) - tb);
        dma16_nt(xb, dr * xs2 + 16u * (uint32_t)((lane % PPR) ^ swz_b(r)), lds(xst) + k * 64);
    }
}

// LDS of the paired-head body below.  Once the last stage has been read,
// the ring holds the heads' S tiles on their way out (stage_store_states):
// head 0 in bsr, the others in xsr.
template <int Q, int HG, int RING = kStateRing>
struct StateSmem {
    uint4 bsr[RING][512];
    uint4 xsr[RING][32 * 128 * HG / 16];
    float wv[HG][Q];
    double wsum[HG][4];
    float cslast[HG];
};

// Write the HG heads' S tiles (acc[e], the MFMA result layout of
// chunk_state_pair) as bf16 rows into LDS at st[e] (row p at 256 p, 16-byte
// chunk k at (k ^ swz_b(p)) 16: lane pairs swap one value as in
// store_state_bf16, so each writes a word of two adjacent columns), then
// store them as whole 256-byte rows, 16 lanes a row: 1 KB of S per store
// instruction instead of four 64-byte pieces, and full lines reach memory.
// Non-temporal: S is read once, later.  Every wave must be past its last read
// of st before the call.
template <int HG>
__device__ __forceinline__ void stage_store_states(const f32x16 (&acc)[HG][2], SSD_LDS char* const (&st)[HG],
                                                   bf16_t* const (&dst)[HG], int wave, int lane) {
    const bool odd = (lane & 1) != 0;
    const int hf = lane >> 5;
    const int n = 32 * wave + (lane & 31);
    const int nb = 2 * (n & ~1);   // byte of the column pair in its row
#pragma unroll
    for (int e = 0; e < HG; ++e)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float h0v = acc[e][mt][r], h1v = acc[e][mt][r + 1];
                const float got = __shfl_xor(odd ? h0v : h1v, 1, 64);
                const float keep = odd ? h1v : h0v;
                const int rr = odd ? r + 1 : r;
                const int p = 32 * mt + 8 * (rr >> 2) + 4 * hf + (rr & 3);
                const uint32_t w = odd ? pack_bf16x2(got, keep) : pack_bf16x2(keep, got);
                *reinterpret_cast<SSD_LDS uint32_t*>(st[e] + p * 256 + (((nb >> 4) ^ swz_b(p)) << 4) +
                                                     (nb & 15)) = w;
            }
    barrier_lds();
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const int k = lane & 15;
#pragma unroll
    for (int m = 0; m < 4 * HG; ++m) {
        const int row = 4 * (wave + 4 * m) + (lane >> 4);   // 0 .. 64 HG - 1
        const int e = row >> 6, p = row & 63;
        const u32x4 v = *reinterpret_cast<const SSD_LDS u32x4*>(st[e] + p * 256 + ((k ^ swz_b(p)) << 4));
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst[e] + p * 128 + 8 * k));
    }
}

// The chunk states of HG heads of one group for one (batch, chunk): acc[e][mt]
// = S_c of head h0 + e, p tile mt, in the MFMA result layout (lane (hf, l32)
// of wave w, register r: p = 32 mt + 8 (r / 4) + 4 hf + r % 4, n = 32 w + l32);
// cl[e] = the chunk's summed decay (cs of its last token, log2 units).
//
// FUSE: the workgroup also forms its heads' chunk cumsum (what
// chunk_cumsum_kernel computes) from dt and A instead of reading cs and dtc:
// an fp64 inclusive prefix of dt A log2(e) over the chunk's tokens (a wave
// scan, then the wave totals), rounded once to fp32, and dt (or its
// zero-order-hold weight) as dtc.  Both rows are written out at the end for
// the later stages.
template <int Q, int HG, bool FUSE, bool CARRY = false, int RING = kStateRing>
__device__ __forceinline__ void chunk_state_pair(StateSmem<Q, HG, RING>& sm, int b, int c, int h0,
                                                 const bf16_t* __restrict__ x,
                                                 const bf16_t* __restrict__ Bm, const float* cs,
                                                 const float* dtc, int L, int H, int G, int nc,
                                                 const float* __restrict__ dtin,
                                                 const float* __restrict__ A, float* csw,
                                                 float* dtcw, int zoh, bool keepx, f32x16 (&acc)[HG][2],
                                                 float (&cl)[HG]) {
    constexpr int W = 4, NT = Q / 32;
    constexpr int XR = 128 * HG;                         // bytes of a token's x row
    constexpr int DPS = 8 / W + BxhOffsets<W, HG>::XC;   // copies per wave per stage
    constexpr int R = RING;
    static_assert(state_ring_waits_hold(NT, R, DPS), "chunk_state wait counts do not cover its copies");
    auto& bsr = sm.bsr;
    auto& xsr = sm.xsr;
    auto& wv = sm.wv;

    const int g = h0 / (H / G);
    int tid = threadIdx.x;
    // inside a run's loop over chunks: the thread index is opaque to the
    // compiler, so the body's many lane addresses are formed per chunk
    // instead of hoisted out of the loop and held in registers across it
    if constexpr (CARRY) asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hf = lane >> 5;
    const int64_t row0 = (((int64_t)b * H + h0) * nc + c) * Q;   // head h0 + e: + e * nc * Q
    const int tok0 = c * Q;
    const int64_t xstride = (int64_t)H * 64, bstride = (int64_t)G * 128;
    const bf16_t* xbase = x + ((int64_t)b * L * H + h0) * 64;
    const bf16_t* bbase = Bm + ((int64_t)b * L * G + g) * 128;

    // ordinary loads first (their values are used, so waited for, before the
    // copies are issued): w_j = exp2(cs_last - cs_j) dt_j for each head
    float wreg[HG];
    float csv[HG], dcv[HG];    // FUSE: this thread's token's cs and dtc
    double v[HG];              // FUSE: dt A log2(e) of this thread's token, then its prefix
    if constexpr (FUSE) {
        float dl[HG];
        const int t = tok0 + tid;
        const bool in = tid < Q && t < L;
        const float* dsrc = dtin + ((int64_t)b * L + min(t, L - 1)) * H + h0;
#pragma unroll
        for (int e = 0; e < HG; ++e) dl[e] = dsrc[e];   // both loads in flight together
#pragma unroll
        for (int e = 0; e < HG; ++e) {
            const float d = in ? dl[e] : 0.0f;
            const float ah = A[h0 + e];
            dcv[e] = zoh ? zoh_weight(d, ah) : d;
            v[e] = (double)d * ((double)ah * 1.4426950408889634074);
            asm volatile("" : "+v"(v[e]), "+v"(dcv[e]));   // formed (loads waited for) here
        }
    } else {
#pragma unroll
        for (int e = 0; e < HG; ++e) {
            const int64_t row = row0 + (int64_t)e * nc * Q;
            wreg[e] = tid < Q ? fast_exp2(cs[row + Q - 1] - cs[row + tid]) * dtc[row + tid] : 0.0f;
            cl[e] = cs[row + Q - 1];
        }
    }
    asm volatile("" ::: "memory");
    const BxhOffsets<W, HG> off = bxh_offsets<W, HG>(wave, lane, xstride, bstride);
#pragma unroll
    for (int k = 0; k < R - 1; ++k)
        if (k < NT) issue_bxh_stage<W, HG>(wave, lane, tok0 + 32 * k, L, xbase, xstride, bbase, bstride, off, bsr[k], xsr[k], keepx);
    if constexpr (FUSE) {
        // the prefix while the first copies are in flight (LDS-only barriers:
        // a full barrier would wait for the copies)
#pragma unroll
        for (int e = 0; e < HG; ++e) {
#pragma unroll
            for (int off2 = 1; off2 < 64; off2 <<= 1) {
                const double o = __shfl_up(v[e], off2, 64);
                if (lane >= off2) v[e] += o;
            }
            if (lane == 63) sm.wsum[e][wave] = v[e];
        }
        barrier_lds();
#pragma unroll
        for (int e = 0; e < HG; ++e) {
            double base = 0.0;
            for (int w2 = 0; w2 < wave; ++w2) base += sm.wsum[e][w2];
            csv[e] = (float)(base + v[e]);
            if (tid == Q - 1) sm.cslast[e] = csv[e];
        }
        barrier_lds();
#pragma unroll
        for (int e = 0; e < HG; ++e) {
            cl[e] = sm.cslast[e];
            wreg[e] = tid < Q ? fast_exp2(cl[e] - csv[e]) * dcv[e] : 0.0f;
        }
    }
    if (tid < Q) {
#pragma unroll
        for (int e = 0; e < HG; ++e) wv[e][tid] = wreg[e];
    }

    const int grp = lane >> 4, rr = lane & 15;
    const int trow0 = 8 * (grp >> 1) + (rr >> 2);
    const int qcol = 16 * (grp & 1) + 4 * (rr & 3);

    // from zero, or (CARRY: acc holds the state entering the chunk) from that
    // state decayed through the chunk, exp2(cs_last) H, so that the products
    // below leave the state after the chunk
#pragma unroll
    for (int e = 0; e < HG; ++e) {
        if constexpr (CARRY) {
            const float a = fast_exp2(cl[e]);
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[e][mt][r] *= a;
        } else {
            acc[e][0] = acc[e][1] = f32x16{};
        }
    }
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) {
        uint4* bst = bsr[jt % R];
        uint4* xst = xsr[jt % R];
        wait_vmcnt_n(DPS * state_ring_ahead(NT, R, jt));   // a constant once the loop is unrolled
        barrier_lds();
        if (jt + R - 1 < NT)
            issue_bxh_stage<W, HG>(wave, lane, tok0 + 32 * (jt + R - 1), L, xbase, xstride, bbase, bstride,
                                   off, bsr[(jt + R - 1) % R], xsr[(jt + R - 1) % R], keepx);
        const SSD_LDS char* xb = (const SSD_LDS char*)lds(xst);
        const SSD_LDS char* bb = (const SSD_LDS char*)lds(bst);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int r0 = 16 * u + trow0, r1 = r0 + 4;
            uint4 bq;
            {
                const int nc4 = 32 * wave + qcol;
                const int chk = nc4 >> 3, sub = (nc4 & 7) * 2;
                const uint2 lo = tr16(bb + r0 * 256 + ((chk ^ swz_b(r0)) << 4) + sub);
                const uint2 hi = tr16(bb + r1 * 256 + ((chk ^ swz_b(r1)) << 4) + sub);
                bq = make_uint4(lo.x, lo.y, hi.x, hi.y);
            }
#pragma unroll
            for (int e = 0; e < HG; ++e) {
                float wj[8];
#pragma unroll
                for (int sidx = 0; sidx < 8; ++sidx) wj[sidx] = wv[e][32 * jt + 16 * u + 8 * hf + sidx];
                const bf16x8 bw = __builtin_bit_cast(bf16x8, scale_bf16x8(bq, wj));
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    const int pc = 64 * e + 32 * mt + qcol;
                    const int chk = pc >> 3, sub = (pc & 7) * 2;
                    const uint2 lo = tr16(xb + r0 * XR + ((chk ^ swz_b(r0)) << 4) + sub);
                    const uint2 hi = tr16(xb + r1 * XR + ((chk ^ swz_b(r1)) << 4) + sub);
                    const bf16x8 xq = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
                    acc[e][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xq, bw, acc[e][mt], 0, 0, 0);
                }
            }
        }
    }

    if constexpr (FUSE) {   // the cumsum rows, after every copy (they would skew the wait counts)
#pragma unroll
        for (int e = 0; e < HG; ++e) {
            const int64_t row = row0 + (int64_t)e * nc * Q;
            if (tid < Q) {
                csw[row + tid] = csv[e];
                dtcw[row + tid] = dcv[e];
            }
        }
    }
}

// One workgroup (4 waves) per (batch, chunk, HG heads of one group); each
// writes its heads' S_c (and, with FUSE, their cumsum rows).
template <int Q, int HG, bool FUSE>
__global__ __launch_bounds__(256, 2) void chunk_state_mfmah_kernel(const bf16_t* __restrict__ x,
                                                                   const bf16_t* __restrict__ Bm,
                                                                   const float* cs, const float* dtc,
                                                                   bf16_t* __restrict__ S, int L,
                                                                   int H, int G, int nc,
                                                                   const float* __restrict__ dtin,
                                                                   const float* __restrict__ A,
                                                                   float* csw, float* dtcw, int zoh,
                                                                   int keep_run, int keep_k) {
    constexpr int P = 64, N = 128;
    __shared__ StateSmem<Q, HG> sm;
    const int HP = H / HG;
    const uint32_t wg = xcd_logical_id(blockIdx.x, gridDim.x);
    const int h0 = HG * (int)(wg % (uint32_t)HP);
    const int bc = (int)(wg / (uint32_t)HP);
    const int c = bc % nc, b = bc / nc;
    // x of the heads at the chunk scan's first run positions stays cached
    const bool keepx = (h0 % (H / G)) % keep_run < keep_k;
    f32x16 acc[HG][2];
    float cl[HG];
    chunk_state_pair<Q, HG, FUSE>(sm, b, c, h0, x, Bm, cs, dtc, L, H, G, nc, dtin, A, csw, dtcw, zoh,
                                  keepx, acc, cl);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    static_assert(sizeof(sm.bsr) >= P * N * 2 && sizeof(sm.xsr) >= (HG - 1) * P * N * 2,
                  "the ring holds the S tiles");
    bf16_t* dst[HG];
    SSD_LDS char* st[HG];
#pragma unroll
    for (int e = 0; e < HG; ++e) {
        dst[e] = S + (((int64_t)b * H + h0 + e) * nc + c) * (int64_t)(P * N);
        st[e] = e == 0 ? (SSD_LDS char*)lds(&sm.bsr[0][0]) : (SSD_LDS char*)lds(&sm.xsr[0][0]) + (e - 1) * P * N * 2;
    }
    barrier_lds();   // every wave is past its last read of the ring
    stage_store_states<HG>(acc, st, dst, wave, lane);
}

// ---------------------------------------------------------------------------
// Chunk states over runs of K consecutive chunks (the first level of a
// two-level recurrence between chunks).  Two steps of the linear recurrence
// H_{c+1} = exp2(cs_last,c) H_c + S_c merge into one step of the same kind
// (the parallel scan of page "State Space Model", section "Dai sistemi
// dinamici a Mamba"), so the state entering chunk c of run r splits into the
// part formed inside the run from a zero start and the run's entering state
// decayed to chunk c:  Hin_c = T_{c-1} + exp2(lam_c) Hr_r  (c past the run's
// first chunk; Hin = Hr_r at the first), where
//     T_c   = the state after chunk c from zero at the run's start,
//     lam_c = the summed log2 decay of the run's chunks before c,
//     rdec_r = the summed log2 decay of the whole run.
// One workgroup (4 waves) per (batch, run, head pair of one group) walks the
// run's chunks with the paired-head chunk state above (the cumsum in its
// prologue), carrying the state in the MFMA accumulators, decayed by each
// chunk's own decay before the chunk's products add onto it; after every
// chunk it stores T_c (bf16, staged through the idle ring as whole rows) and
// lam_c, after the run rdec_r.  The run's entering states Hr then come from a
// chain over runs (state_passing.hip), and chunk_scan forms Hin_c from T_{c-1}
// and Hr_r itself, so neither the per-chunk S nor the per-chunk Hin reaches
// memory.
// Three workgroups per CU, as the one-chunk kernel: the lane addresses of
// the chunk body and of the T store are formed inside the loop over chunks
// (opaque thread index), so only the carried state and a few scalars live
// across it (151 VGPRs, no spills).
template <int Q, int HG>
__global__ __launch_bounds__(256, 3) void chunk_state_runs_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ Bm, bf16_t* __restrict__ T,
    float* __restrict__ lam, float* __restrict__ rdec, int L, int H, int G, int nc, int K, int nruns,
    const float* __restrict__ dtin, const float* __restrict__ A, float* csw, float* dtcw, int zoh,
    int keep_run, int keep_k) {
    constexpr int P = 64, N = 128;
    __shared__ StateSmem<Q, HG> sm;
    const int HP = H / HG;
    const uint32_t wg = xcd_logical_id(blockIdx.x, gridDim.x);
    const int h0 = HG * (int)(wg % (uint32_t)HP);
    const int br = (int)(wg / (uint32_t)HP);
    const int r = br % nruns, b = br / nruns;
    const int c0 = r * K, c1 = min(c0 + K, nc);
    const bool keepx = (h0 % (H / G)) % keep_run < keep_k;
    const int tid = threadIdx.x;
    static_assert(sizeof(sm.bsr) >= P * N * 2 && sizeof(sm.xsr) >= (HG - 1) * P * N * 2,
                  "the ring holds the T tiles");
    SSD_LDS char* st[HG];
#pragma unroll
    for (int e = 0; e < HG; ++e)
        st[e] = e == 0 ? (SSD_LDS char*)lds(&sm.bsr[0][0]) : (SSD_LDS char*)lds(&sm.xsr[0][0]) + (e - 1) * P * N * 2;
    f32x16 acc[HG][2];
    float cl[HG], lsum[HG];
#pragma unroll
    for (int e = 0; e < HG; ++e) lsum[e] = 0.0f;
    // the run starts from zero; every chunk decays the carried state (a zero
    // state stays exactly zero: the decay factors lie in [0, 1]) and adds its
    // products
#pragma unroll
    for (int e = 0; e < HG; ++e) acc[e][0] = acc[e][1] = f32x16{};
    for (int c = c0; c < c1; ++c) {
        chunk_state_pair<Q, HG, true, true>(sm, b, c, h0, x, Bm, nullptr, nullptr, L, H, G, nc, dtin, A, csw,
                                            dtcw, zoh, keepx, acc, cl);
        bf16_t* dst[HG];
#pragma unroll
        for (int e = 0; e < HG; ++e) {
            const int64_t bhc = ((int64_t)b * H + h0 + e) * nc + c;
            dst[e] = T + bhc * (int64_t)(P * N);
            if (tid == 0) lam[bhc] = lsum[e];
            // wave-uniform: kept in scalar registers across the run
            lsum[e] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                                    __builtin_bit_cast(int, lsum[e] + cl[e])));
        }
        barrier_lds();   // every wave is past its last read of the ring
        {
            // the store's lane addresses formed per chunk (an opaque index,
            // as in chunk_state_pair), not held across the loop
            int t = threadIdx.x;
            asm volatile("" : "+v"(t));
            stage_store_states<HG>(acc, st, dst, __builtin_amdgcn_readfirstlane(t >> 6), t & 63);
        }
        barrier_lds();   // every wave has read its staged rows back before the ring refills
    }
    if (tid == 0) {
#pragma unroll
        for (int e = 0; e < HG; ++e) rdec[((int64_t)b * H + h0 + e) * nruns + r] = lsum[e];
    }
}

// ---------------------------------------------------------------------------
// Walked chunk state: chunk state and the recurrence between chunks in one
// pass per (batch, head pair), so that no chunk's S reaches memory.  Only
// the summary state crosses from one block to the next (page "Mamba-2
// (2024): SSM e attention sono la stessa cosa", section "Il trucco a
// blocchi"): one workgroup (4 waves, one per CU) walks the whole sequence of
// its two heads in 32-token blocks, keeping the running state in the MFMA
// accumulators (the layout of the paired-head chunk state above: wave w owns
// state columns n in [32w, 32w + 32) of both heads).  At each chunk's start
// it writes the state entering the chunk (Hin, bf16) and scales the state by
// the chunk's decay, H <- exp2(cs_last) H; the chunk's products, weighted
// w_j = exp2(cs_last - cs_j) dt_j as in S_c, then accumulate onto it, which
// leaves exp2(cs_last) H_c + S_c = H_{c+1}.  After the last chunk the state
// is the final state.
//
// B and the two heads' x rows stream through an 8-stage LDS ring (16 KB a
// stage, seven stages ahead: the walk of one chain is paced by how much is
// in flight, not by the CU's throughput), and each chunk's cs/dt rows arrive
// one chunk ahead.  Blocks past the end re-read the last token (their
// weights are zero) and rows past the last chunk read as zeros, so every
// wave issues the same operations at every step and every wait is a
// constant (checked at compile time below).
constexpr int kWalkRing = 8;                           // ring stages (7 ahead)
constexpr int kWalkDps = 4;                            // copies per wave per stage (B 2, x 2)
constexpr int kWalkRows = 4;                           // row copies per wave per chunk
constexpr int kWalkHin = 32;                           // Hin stores per wave per chunk

// Operations issued after stage k = c NT + jt when step jt of chunk c waits
// for it: the stages issued ahead of it, plus chunk c's Hin stores and the
// next chunk's row copies when they came after stage k's copies (which does
// not depend on NT while the ring is shallower than a chunk is long).
__host__ __device__ constexpr int walk_ops_after(int /*NT*/, int jt) {
    return (kWalkRing - 2) * kWalkDps + (jt < kWalkRing - 1 ? kWalkHin + kWalkRows : 0);
}
// The issue order replayed against those waits over a few chunks (labels:
// stage k, rows of chunk c, Hin stores of chunk c): at each step its stage,
// and at each chunk's start (after a wait that leaves only the previous
// chunk's NT stages pending) its rows, must have landed.
constexpr bool walk_waits_hold(int NT, int nc) {
    auto stl = [](int k) { return 1000 + k; };
    auto rwl = [](int c) { return 5000 + c; };
    VmemLog o;
    o.push(rwl(0), kWalkRows);
    for (int k = 0; k < kWalkRing - 1; ++k) o.push(stl(k), kWalkDps);
    if (!o.wait((kWalkRing - 1) * kWalkDps) || !o.landed(rwl(0))) return false;
    for (int c = 0; c < nc; ++c) {
        if (c > 0 && (!o.wait(NT * kWalkDps) || !o.landed(rwl(c)))) return false;
        o.push(6000 + c, kWalkHin);
        o.push(rwl(c + 1), kWalkRows);
        for (int jt = 0; jt < NT; ++jt) {
            const int k = c * NT + jt;
            if (!o.wait(walk_ops_after(NT, jt)) || !o.landed(stl(k))) return false;
            o.push(stl(k + kWalkRing - 1), kWalkDps);
        }
    }
    return true;
}
static_assert(walk_waits_hold(8, 1) && walk_waits_hold(8, 3) && walk_waits_hold(4, 1) &&
              walk_waits_hold(4, 4), "state walk wait counts do not cover its copies");

template <int NT>
__global__ __launch_bounds__(256, 1) void state_walk_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ Bm, const float* __restrict__ cs,
    const float* __restrict__ dtc, const float* init, bf16_t* __restrict__ Hin, float* fin, int L,
    int H, int G, int nc) {
    constexpr int Q = 32 * NT, HG = 2, W = 4, P = 64, N = 128, R = kWalkRing;
    constexpr int XR = 128 * HG;
    static_assert(BxhOffsets<W, HG>::XC + 8 / W == kWalkDps, "copies per stage");
    __shared__ uint4 bsr[R][512];            // B blocks: 32 x 256 B
    __shared__ uint4 xsr[R][32 * XR / 16];   // x blocks: 32 x (2 heads x 128 B)
    __shared__ float rows[2][HG][2][Q];      // cs and dt rows by chunk parity
    __shared__ float wv[HG][Q];

    const int HP = H / HG;
    const int b = (int)blockIdx.x / HP, h0 = HG * ((int)blockIdx.x % HP);
    const int g = h0 / (H / G);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hf = lane >> 5, l32 = lane & 31;
    const int n = 32 * wave + l32;
    const int64_t xstride = (int64_t)H * P, bstride = (int64_t)G * N;
    const bf16_t* xbase = x + ((int64_t)b * L * H + h0) * P;
    const bf16_t* bbase = Bm + ((int64_t)b * L * G + g) * N;
    const int64_t rowbase = ((int64_t)b * H + h0) * nc;   // (b, h0, chunk 0) row; head h0 + e at + e nc
    const BxhOffsets<W, HG> off = bxh_offsets<W, HG>(wave, lane, xstride, bstride);

    // cs / dt rows of chunk c (records empty past the last chunk): wave w
    // copies row e = w / 2, array w % 2, 256 floats in 4 copies
    const int re = wave >> 1, ra = wave & 1;
    const float* rsrc = (ra == 0 ? cs : dtc) + (rowbase + (int64_t)re * nc) * Q;
    auto issue_rows = [&](int c) {
        const __amdgpu_buffer_rsrc_t rr = make_rs(rsrc + (int64_t)c * Q, c < nc ? Q * 4 : 0);
#pragma unroll
        for (int i = 0; i < kWalkRows; ++i)
            dma4_rs(rr, 4u * (uint32_t)(64 * i + lane) % (4u * Q), lds(&rows[c & 1][re][ra][0]) + (64 * i) % Q);
    };
    auto issue_stage = [&](int k) {
        issue_bxh_stage<W, HG>(wave, lane, 32 * k, L, xbase, xstride, bbase, bstride, off, bsr[k % R],
                               xsr[k % R], false);
    };

    // running state, from init or zero
    f32x16 acc[HG][2];
#pragma unroll
    for (int e = 0; e < HG; ++e)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int p = 32 * mt + 8 * (r >> 2) + 4 * hf + (r & 3);
                acc[e][mt][r] = init ? init[(((int64_t)b * H + h0 + e) * P + p) * N + n] : 0.0f;
            }
    asm volatile("" ::: "memory");
    issue_rows(0);
#pragma unroll
    for (int k = 0; k < R - 1; ++k) issue_stage(k);
    wait_vmcnt<(R - 1) * kWalkDps>();   // rows of chunk 0

    const int grp = lane >> 4, rr4 = lane & 15;
    const int trow0 = 8 * (grp >> 1) + (rr4 >> 2);
    const int qcol = 16 * (grp & 1) + 4 * (rr4 & 3);

    for (int c = 0; c < nc; ++c) {
        // chunk c's rows were copied at chunk c - 1's start, before its NT stages
        if (c > 0) wait_vmcnt<NT * kWalkDps>();
        barrier_lds();   // chunk c's rows are visible; every wave is done with chunk c - 1's weights
        float cl[HG];
#pragma unroll
        for (int e = 0; e < HG; ++e) {
            const float* rc = rows[c & 1][e][0];
            cl[e] = rc[Q - 1];
            if (tid < Q) wv[e][tid] = fast_exp2(cl[e] - rc[tid]) * rows[c & 1][e][1][tid];
        }
        // the state entering chunk c (bf16), then its decay
#pragma unroll
        for (int e = 0; e < HG; ++e) {
            store_state_bf16(acc[e], Hin + (rowbase + (int64_t)e * nc + c) * (int64_t)(P * N), lane, n);
            const float a = fast_exp2(cl[e]);
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[e][mt][r] *= a;
        }
        issue_rows(c + 1);
#pragma unroll
        for (int jt = 0; jt < NT; ++jt) {
            const int k = c * NT + jt;
            wait_vmcnt_n(walk_ops_after(NT, jt));   // a constant once the loop is unrolled
            barrier_lds();                          // stage k (and, at jt = 0, the weights) visible
            issue_stage(k + R - 1);
            const SSD_LDS char* xb = (const SSD_LDS char*)lds(xsr[k % R]);
            const SSD_LDS char* bb = (const SSD_LDS char*)lds(bsr[k % R]);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int r0 = 16 * u + trow0, r1 = r0 + 4;
                uint4 bq;
                {
                    const int nc4 = 32 * wave + qcol;
                    const int chk = nc4 >> 3, sub = (nc4 & 7) * 2;
                    const uint2 lo = tr16(bb + r0 * 256 + ((chk ^ swz_b(r0)) << 4) + sub);
                    const uint2 hi = tr16(bb + r1 * 256 + ((chk ^ swz_b(r1)) << 4) + sub);
                    bq = make_uint4(lo.x, lo.y, hi.x, hi.y);
                }
#pragma unroll
                for (int e = 0; e < HG; ++e) {
                    float wj[8];
#pragma unroll
                    for (int sidx = 0; sidx < 8; ++sidx) wj[sidx] = wv[e][32 * jt + 16 * u + 8 * hf + sidx];
                    const bf16x8 bw = __builtin_bit_cast(bf16x8, scale_bf16x8(bq, wj));
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt) {
                        const int pc = 64 * e + 32 * mt + qcol;
                        const int chk = pc >> 3, sub = (pc & 7) * 2;
                        const uint2 lo = tr16(xb + r0 * XR + ((chk ^ swz_b(r0)) << 4) + sub);
                        const uint2 hi = tr16(xb + r1 * XR + ((chk ^ swz_b(r1)) << 4) + sub);
                        const bf16x8 xq = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
                        acc[e][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xq, bw, acc[e][mt], 0, 0, 0);
                    }
                }
            }
        }
    }
    wait_vmcnt<0>();   // prefetches past the end land before the workgroup's LDS goes away
    if (fin) {
#pragma unroll
        for (int e = 0; e < HG; ++e)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int p = 32 * mt + 8 * (r >> 2) + 4 * hf + (r & 3);
                    fin[(((int64_t)b * H + h0 + e) * P + p) * N + n] = acc[e][mt][r];
                }
    }
}

// ---------------------------------------------------------------------------
// Generic kernel: one workgroup per (batch, chunk, head); each thread owns
// up to MAXO outputs (p, n) of the P x N state.
template <typename T, int MAXO>
__global__ __launch_bounds__(256) void chunk_state_generic_kernel(
    const T* __restrict__ x, const T* __restrict__ Bm, const float* __restrict__ cs,
    const float* __restrict__ dtc, T* __restrict__ S, int L, int H, int P, int N, int G,
    int Q, int nc) {
    extern __shared__ float smem[];
    float* xs = smem;              // [32][P]
    float* bs = smem + 32 * P;     // [32][N]
    float* wv = bs + 32 * N;       // [32]
    const int w = blockIdx.x;
    const int h = w % H;
    const int bc = w / H;
    const int c = bc % nc, b = bc / nc;
    const int g = h / (H / G);
    const int tid = threadIdx.x;
    const int64_t row = (((int64_t)b * H + h) * nc + c) * Q;
    const float cl = cs[row + Q - 1];
    const int PN = P * N;

    float acc[MAXO];
#pragma unroll
    for (int k = 0; k < MAXO; ++k) acc[k] = 0.0f;

    for (int j0 = 0; j0 < Q; j0 += 32) {
        if (tid < 32) {
            const int j = j0 + tid;
            wv[tid] = (j < Q) ? fast_exp2(cl - cs[row + j]) * dtc[row + j] : 0.0f;
        }
        __syncthreads();
        for (int e = tid; e < 32 * P; e += 256) {
            const int jj = e / P, p = e - jj * P;
            const int t = c * Q + j0 + jj;
            xs[e] = (j0 + jj < Q && t < L) ? Elem<T>::load(x, (((int64_t)b * L + t) * H + h) * P + p) * wv[jj] : 0.0f;
        }
        for (int e = tid; e < 32 * N; e += 256) {
            const int jj = e / N, n = e - jj * N;
            const int t = c * Q + j0 + jj;
            bs[e] = (j0 + jj < Q && t < L) ? Elem<T>::load(Bm, (((int64_t)b * L + t) * G + g) * N + n) : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < MAXO; ++k) {
            const int o = tid + 256 * k;
            if (o < PN) {
                const int p = o / N, n = o - p * N;
                float s = acc[k];
                for (int jj = 0; jj < 32; ++jj) s += xs[jj * P + p] * bs[jj * N + n];
                acc[k] = s;
            }
        }
        __syncthreads();
    }
    T* Sp = S + (((int64_t)b * H + h) * nc + c) * (int64_t)PN;
#pragma unroll
    for (int k = 0; k < MAXO; ++k) {
        const int o = tid + 256 * k;
        if (o < PN) Elem<T>::store(Sp, o, acc[k]);
    }
}

template <typename T, int MAXO>
static void launch_generic(const Dims& d, const void* x, const void* B, const float* cs,
                           const float* dtc, void* S, hipStream_t stream) {
    const size_t shmem = sizeof(float) * (32 * (d.headdim + d.dstate) + 32);
    const unsigned blocks = (unsigned)(d.batch * d.nchunks * d.nheads);
    chunk_state_generic_kernel<T, MAXO><<<blocks, 256, shmem, stream>>>(
        static_cast<const T*>(x), static_cast<const T*>(B), cs, dtc, static_cast<T*>(S), (int)d.seqlen,
        (int)d.nheads, (int)d.headdim, (int)d.dstate, (int)d.ngroups, (int)d.chunk,
        (int)d.nchunks);
}

template <typename T>
static void launch_generic_t(const Dims& d, const void* x, const void* B, const float* cs,
                             const float* dtc, void* S, hipStream_t stream) {
    const int64_t per = (d.headdim * d.dstate + 255) / 256;
    if (per <= 1) launch_generic<T, 1>(d, x, B, cs, dtc, S, stream);
    else if (per <= 2) launch_generic<T, 2>(d, x, B, cs, dtc, S, stream);
    else if (per <= 4) launch_generic<T, 4>(d, x, B, cs, dtc, S, stream);
    else if (per <= 8) launch_generic<T, 8>(d, x, B, cs, dtc, S, stream);
    else if (per <= 16) launch_generic<T, 16>(d, x, B, cs, dtc, S, stream);
    else if (per <= 32) launch_generic<T, 32>(d, x, B, cs, dtc, S, stream);
    else launch_generic<T, 64>(d, x, B, cs, dtc, S, stream);
}

bool mfma_path(int32_t dtype, const Dims& d) {
    // chunk-relative y offsets of the scan kernel's buffer stores fit 31 bits
    return dtype == 1 && d.headdim == 64 && d.dstate == 128 &&
           (d.chunk == 64 || d.chunk == 128 || d.chunk == 256) &&
           (double)d.chunk * (double)d.nheads * (double)d.headdim * 2.0 < 2147483647.0;
}

bool generic_path(const Dims& d) {
    return d.headdim >= 1 && d.headdim <= 128 && d.dstate >= 1 && d.dstate <= 128 &&
           d.chunk >= 1 && d.chunk <= 256;
}

bool chunk_state_fuses_cumsum(int32_t dtype, const Dims& d) {
    return mfma_path(dtype, d) && (d.nheads / d.ngroups) % kStateHeads == 0;
}

hipError_t launch_chunk_state_fused(const Dims& d, const void* x, const void* B, const float* dt,
                                    const float* A, bool zoh, float* cs, float* dtc, void* Sv,
                                    hipStream_t stream) {
    bf16_t* S = static_cast<bf16_t*>(Sv);
    const unsigned hblocks = (unsigned)(d.batch * d.nchunks * d.nheads / kStateHeads);
    const bf16_t* xb = static_cast<const bf16_t*>(x);
    const bf16_t* bb = static_cast<const bf16_t*>(B);
    const int L = (int)d.seqlen, H = (int)d.nheads, G = (int)d.ngroups, nc = (int)d.nchunks;
    const int z = zoh ? 1 : 0;
    int krun = 1, nsplit = 1;
    chunk_scan_runs(d, &krun, &nsplit);
    const int kk = x_keep_positions(d);
    switch (d.chunk) {
        case 64: chunk_state_mfmah_kernel<64, kStateHeads, true><<<hblocks, 256, 0, stream>>>(xb, bb, nullptr, nullptr, S, L, H, G, nc, dt, A, cs, dtc, z, krun, kk); break;
        case 128: chunk_state_mfmah_kernel<128, kStateHeads, true><<<hblocks, 256, 0, stream>>>(xb, bb, nullptr, nullptr, S, L, H, G, nc, dt, A, cs, dtc, z, krun, kk); break;
        default: chunk_state_mfmah_kernel<256, kStateHeads, true><<<hblocks, 256, 0, stream>>>(xb, bb, nullptr, nullptr, S, L, H, G, nc, dt, A, cs, dtc, z, krun, kk); break;
    }
    return hipGetLastError();
}

bool state_runs_apply(int32_t dtype, const Dims& d) {
    return chunk_state_fuses_cumsum(dtype, d) && d.chunk == 256;
}

// Run length for ssd_forward, or 0 to keep the per-chunk path.  Longer runs
// shorten the chain over runs and keep more states out of memory, but leave
// fewer workgroups for the run walks, whose chunks are sequential: take the
// longest K in {16, 8, 4, 2} whose grid still gives every CU four workgroups
// (three run at a time on a CU).  Measured (chunk-state runs + run chain
// + chunk scan in the forward's order, one box): 2.7B shape K = 4 / 8: 337.8 /
// 336.3 us against 365.0 us for the per-chunk path (K = 4 taken); 1M-token
// sequence K = 8 / 16 / 32 / 64: 5,644 / 5,581 / 5,617 / 5,641 us against
// 6,097 (K = 16); the 130M shape has 96 head-pair sequences of 8 chunks, too
// few workgroups at any K (K = 2 / 4 / 8: 71.6 / 77.7 / 103.4 us against
// 66.8), and keeps the per-chunk path.
int state_run_chunks(const Dims& d) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    }
    const double chains = (double)d.batch * (double)(d.nheads / kStateHeads);
    for (int K = 16; K >= 2; K /= 2) {
        const double wgs = chains * (double)((d.nchunks + K - 1) / K);
        if (wgs >= 2.0 * 2.0 * cus) return K;
    }
    return 0;
}

hipError_t launch_chunk_state_runs(const Dims& d, int K, const void* x, const void* B,
                                   const float* dt, const float* A, bool zoh, float* cs, float* dtc,
                                   void* T, float* lam, float* rdec, hipStream_t stream) {
    const int nc = (int)d.nchunks, nruns = (nc + K - 1) / K;
    const unsigned blocks = (unsigned)(d.batch * nruns * (d.nheads / kStateHeads));
    int krun = 1, nsplit = 1;
    chunk_scan_runs(d, &krun, &nsplit);
    chunk_state_runs_kernel<256, kStateHeads><<<blocks, 256, 0, stream>>>(
        static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(B), static_cast<bf16_t*>(T), lam,
        rdec, (int)d.seqlen, (int)d.nheads, (int)d.ngroups, nc, K, nruns, dt, A, cs, dtc, zoh ? 1 : 0,
        krun, x_keep_positions(d));
    return hipGetLastError();
}

bool state_walk_applies(int32_t dtype, const Dims& d) {
    return mfma_path(dtype, d) && d.chunk >= 128 && (d.nheads / d.ngroups) % 2 == 0;
}

hipError_t launch_state_walk(const Dims& d, const void* x, const void* B, const float* cs,
                             const float* dtc, const float* init, void* Hin, float* final_state,
                             hipStream_t stream) {
    const unsigned blocks = (unsigned)(d.batch * (d.nheads / 2));
    const bf16_t* xb = static_cast<const bf16_t*>(x);
    const bf16_t* bb = static_cast<const bf16_t*>(B);
    bf16_t* hb = static_cast<bf16_t*>(Hin);
    const int L = (int)d.seqlen, H = (int)d.nheads, G = (int)d.ngroups, nc = (int)d.nchunks;
    if (d.chunk == 128)
        state_walk_kernel<4><<<blocks, 256, 0, stream>>>(xb, bb, cs, dtc, init, hb, final_state, L, H, G, nc);
    else
        state_walk_kernel<8><<<blocks, 256, 0, stream>>>(xb, bb, cs, dtc, init, hb, final_state, L, H, G, nc);
    return hipGetLastError();
}

hipError_t launch_chunk_state(const Dims& d, int32_t dtype, const void* x, const void* B,
                              const float* cs, const float* dtc, void* Sv, hipStream_t stream) {
    if (mfma_path(dtype, d)) {
        bf16_t* S = static_cast<bf16_t*>(Sv);
        const unsigned blocks = (unsigned)(d.batch * d.nchunks * d.nheads);
        const bf16_t* xb = static_cast<const bf16_t*>(x);
        const bf16_t* bb = static_cast<const bf16_t*>(B);
        const int L = (int)d.seqlen, H = (int)d.nheads, G = (int)d.ngroups, nc = (int)d.nchunks;
        if ((d.nheads / d.ngroups) % kStateHeads == 0) {
            const unsigned hblocks = blocks / (unsigned)kStateHeads;
            int krun = 1, nsplit = 1;
            chunk_scan_runs(d, &krun, &nsplit);
            const int kk = x_keep_positions(d);
            switch (d.chunk) {
                case 64: chunk_state_mfmah_kernel<64, kStateHeads, false><<<hblocks, 256, 0, stream>>>(xb, bb, cs, dtc, S, L, H, G, nc, nullptr, nullptr, nullptr, nullptr, 0, krun, kk); break;
                case 128: chunk_state_mfmah_kernel<128, kStateHeads, false><<<hblocks, 256, 0, stream>>>(xb, bb, cs, dtc, S, L, H, G, nc, nullptr, nullptr, nullptr, nullptr, 0, krun, kk); break;
                default: chunk_state_mfmah_kernel<256, kStateHeads, false><<<hblocks, 256, 0, stream>>>(xb, bb, cs, dtc, S, L, H, G, nc, nullptr, nullptr, nullptr, nullptr, 0, krun, kk); break;
            }
            return hipGetLastError();
        }
        switch (d.chunk) {
            case 64: chunk_state_mfma_kernel<64><<<blocks, 256, 0, stream>>>(xb, bb, cs, dtc, S, L, H, G, nc); break;
            case 128: chunk_state_mfma_kernel<128><<<blocks, 256, 0, stream>>>(xb, bb, cs, dtc, S, L, H, G, nc); break;
            default: chunk_state_mfma_kernel<256><<<blocks, 256, 0, stream>>>(xb, bb, cs, dtc, S, L, H, G, nc); break;
        }
    } else if (dtype == 1) {
        launch_generic_t<bf16_t>(d, x, B, cs, dtc, Sv, stream);
    } else {
        launch_generic_t<float>(d, x, B, cs, dtc, Sv, stream);
    }
    return hipGetLastError();
}

}  // namespace ssd
