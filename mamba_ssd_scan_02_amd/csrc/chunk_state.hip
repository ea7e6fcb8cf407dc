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
                                                                  float* __restrict__ S, int L, int H,
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

    // ordinary loads first (see chunk_scan): w_j = exp2(cs_last - cs_j) dt_j
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

    float* Sp = S + (((int64_t)b * H + h) * nc + c) * (int64_t)(P * N);
    const int n = 32 * wave + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int p = 8 * (r >> 2) + 4 * hf + (r & 3);
        __builtin_nontemporal_store(acc[0][r], &Sp[p * N + n]);
        __builtin_nontemporal_store(acc[1][r], &Sp[(32 + p) * N + n]);
    }
}

// HG (2 or 4) heads per workgroup: one workgroup per (batch, chunk, HG
// consecutive heads of one group).  Their x rows are HG * 128 contiguous
// bytes per token, copied with the same swizzle as B's rows (the LDS banks
// repeat every 256 bytes, so rows of 256 or 512 bytes see the same pattern),
// and each B fragment read from LDS serves all HG heads (scaled by each
// head's weights).  Wave w owns state columns n in [32w, 32w+32) of every
// head.  Wider rows read faster from HBM than one head's 128-byte rows, and B
// crosses L2 -> LDS once per HG heads.  x is read once, with non-temporal
// copies (138 -> 132 us at the 2.7B shape).
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
                                                const BxhOffsets<W, HG>& off, uint4* bst, uint4* xst) {
    constexpr int PPR = 8 * HG, RPC = 64 / PPR, XC = BxhOffsets<W, HG>::XC;
    asm volatile("" : "+s"(tokbase));
    if (tokbase + 31 < L) {
        const char* bb = reinterpret_cast<const char*>(bbase + (int64_t)tokbase * bstride);
        const char* xb = reinterpret_cast<const char*>(xbase + (int64_t)tokbase * xstride);
#pragma unroll
        for (int i = 0; i < 8 / W; ++i) dma16(bb, off.b[i], lds(bst) + (wave + i * W) * 64);
#pragma unroll
        for (int i = 0; i < XC; ++i) dma16_nt(xb, off.x[i], lds(xst) + (wave + i * W) * 64);
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

// FUSE: the workgroup also forms its heads' chunk cumsum (what
// chunk_cumsum_kernel computes) from dt and A instead of reading cs and dtc:
// an fp64 inclusive prefix of dt A log2(e) over the chunk's tokens (a wave
// scan, then the wave totals), rounded once to fp32, and dt (or its
// zero-order-hold weight) as dtc.  Both rows are written out at the end for
// the later stages.
template <int Q, int HG, bool FUSE>
__global__ __launch_bounds__(256, 2) void chunk_state_mfmah_kernel(const bf16_t* __restrict__ x,
                                                                   const bf16_t* __restrict__ Bm,
                                                                   const float* cs, const float* dtc,
                                                                   float* __restrict__ S, int L,
                                                                   int H, int G, int nc,
                                                                   const float* __restrict__ dtin,
                                                                   const float* __restrict__ A,
                                                                   float* csw, float* dtcw, int zoh) {
    constexpr int P = 64, N = 128, W = 4, NT = Q / 32;
    constexpr int XR = 128 * HG;                         // bytes of a token's x row
    constexpr int DPS = 8 / W + BxhOffsets<W, HG>::XC;   // copies per wave per stage
    constexpr int R = kStateRing;
    static_assert(state_ring_waits_hold(NT, R, DPS), "chunk_state wait counts do not cover its copies");
    __shared__ uint4 bsr[R][512];
    __shared__ uint4 xsr[R][32 * XR / 16];
    __shared__ float wv[HG][Q];

    const int HP = H / HG;
    const uint32_t wg = xcd_logical_id(blockIdx.x, gridDim.x);
    const int h0 = HG * (int)(wg % (uint32_t)HP);
    const int bc = (int)(wg / (uint32_t)HP);
    const int c = bc % nc, b = bc / nc;
    const int g = h0 / (H / G);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hf = lane >> 5, l32 = lane & 31;
    const int64_t row0 = (((int64_t)b * H + h0) * nc + c) * Q;   // head h0 + e: + e * nc * Q
    const int tok0 = c * Q;
    const int64_t xstride = (int64_t)H * P, bstride = (int64_t)G * N;
    const bf16_t* xbase = x + ((int64_t)b * L * H + h0) * P;
    const bf16_t* bbase = Bm + ((int64_t)b * L * G + g) * N;

    // ordinary loads first (their values are used, so waited for, before the
    // copies are issued): w_j = exp2(cs_last - cs_j) dt_j for each head
    float wreg[HG];
    float csv[HG], dcv[HG];    // FUSE: this thread's token's cs and dtc
    __shared__ double wsum[HG][4];
    __shared__ float cslast[HG];
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
        }
    }
    asm volatile("" ::: "memory");
    const BxhOffsets<W, HG> off = bxh_offsets<W, HG>(wave, lane, xstride, bstride);
#pragma unroll
    for (int k = 0; k < R - 1; ++k)
        if (k < NT) issue_bxh_stage<W, HG>(wave, lane, tok0 + 32 * k, L, xbase, xstride, bbase, bstride, off, bsr[k], xsr[k]);
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
            if (lane == 63) wsum[e][wave] = v[e];
        }
        barrier_lds();
#pragma unroll
        for (int e = 0; e < HG; ++e) {
            double base = 0.0;
            for (int w2 = 0; w2 < wave; ++w2) base += wsum[e][w2];
            csv[e] = (float)(base + v[e]);
            if (tid == Q - 1) cslast[e] = csv[e];
        }
        barrier_lds();
#pragma unroll
        for (int e = 0; e < HG; ++e) wreg[e] = tid < Q ? fast_exp2(cslast[e] - csv[e]) * dcv[e] : 0.0f;
    }
    if (tid < Q) {
#pragma unroll
        for (int e = 0; e < HG; ++e) wv[e][tid] = wreg[e];
    }

    const int grp = lane >> 4, rr = lane & 15;
    const int trow0 = 8 * (grp >> 1) + (rr >> 2);
    const int qcol = 16 * (grp & 1) + 4 * (rr & 3);

    f32x16 acc[HG][2];   // [head][p tile]
#pragma unroll
    for (int e = 0; e < HG; ++e) acc[e][0] = acc[e][1] = f32x16{};
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) {
        uint4* bst = bsr[jt % R];
        uint4* xst = xsr[jt % R];
        wait_vmcnt_n(DPS * state_ring_ahead(NT, R, jt));   // a constant once the loop is unrolled
        barrier_lds();
        if (jt + R - 1 < NT)
            issue_bxh_stage<W, HG>(wave, lane, tok0 + 32 * (jt + R - 1), L, xbase, xstride, bbase, bstride,
                                   off, bsr[(jt + R - 1) % R], xsr[(jt + R - 1) % R]);
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
    const int n = 32 * wave + l32;
#pragma unroll
    for (int e = 0; e < HG; ++e) {
        float* Sp = S + (((int64_t)b * H + h0 + e) * nc + c) * (int64_t)(P * N);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int p = 8 * (r >> 2) + 4 * hf + (r & 3);
            __builtin_nontemporal_store(acc[e][0][r], &Sp[p * N + n]);
            __builtin_nontemporal_store(acc[e][1][r], &Sp[(32 + p) * N + n]);
        }
    }
}

// ---------------------------------------------------------------------------
// Generic kernel: one workgroup per (batch, chunk, head); each thread owns
// up to MAXO outputs (p, n) of the P x N state.
template <typename T, int MAXO>
__global__ __launch_bounds__(256) void chunk_state_generic_kernel(
    const T* __restrict__ x, const T* __restrict__ Bm, const float* __restrict__ cs,
    const float* __restrict__ dtc, float* __restrict__ S, int L, int H, int P, int N, int G,
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
    float* Sp = S + (((int64_t)b * H + h) * nc + c) * (int64_t)PN;
#pragma unroll
    for (int k = 0; k < MAXO; ++k) {
        const int o = tid + 256 * k;
        if (o < PN) Sp[o] = acc[k];
    }
}

template <typename T, int MAXO>
static void launch_generic(const Dims& d, const void* x, const void* B, const float* cs,
                           const float* dtc, float* S, hipStream_t stream) {
    const size_t shmem = sizeof(float) * (32 * (d.headdim + d.dstate) + 32);
    const unsigned blocks = (unsigned)(d.batch * d.nchunks * d.nheads);
    chunk_state_generic_kernel<T, MAXO><<<blocks, 256, shmem, stream>>>(
        static_cast<const T*>(x), static_cast<const T*>(B), cs, dtc, S, (int)d.seqlen,
        (int)d.nheads, (int)d.headdim, (int)d.dstate, (int)d.ngroups, (int)d.chunk,
        (int)d.nchunks);
}

template <typename T>
static void launch_generic_t(const Dims& d, const void* x, const void* B, const float* cs,
                             const float* dtc, float* S, hipStream_t stream) {
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
           (d.chunk == 128 || d.chunk == 256) &&
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
                                    const float* A, bool zoh, float* cs, float* dtc, float* S,
                                    hipStream_t stream) {
    const unsigned hblocks = (unsigned)(d.batch * d.nchunks * d.nheads / kStateHeads);
    const bf16_t* xb = static_cast<const bf16_t*>(x);
    const bf16_t* bb = static_cast<const bf16_t*>(B);
    const int L = (int)d.seqlen, H = (int)d.nheads, G = (int)d.ngroups, nc = (int)d.nchunks;
    const int z = zoh ? 1 : 0;
    switch (d.chunk) {
        case 64: chunk_state_mfmah_kernel<64, kStateHeads, true><<<hblocks, 256, 0, stream>>>(xb, bb, nullptr, nullptr, S, L, H, G, nc, dt, A, cs, dtc, z); break;
        case 128: chunk_state_mfmah_kernel<128, kStateHeads, true><<<hblocks, 256, 0, stream>>>(xb, bb, nullptr, nullptr, S, L, H, G, nc, dt, A, cs, dtc, z); break;
        default: chunk_state_mfmah_kernel<256, kStateHeads, true><<<hblocks, 256, 0, stream>>>(xb, bb, nullptr, nullptr, S, L, H, G, nc, dt, A, cs, dtc, z); break;
    }
    return hipGetLastError();
}

hipError_t launch_chunk_state(const Dims& d, int32_t dtype, const void* x, const void* B,
                              const float* cs, const float* dtc, float* S, hipStream_t stream) {
    if (mfma_path(dtype, d)) {
        const unsigned blocks = (unsigned)(d.batch * d.nchunks * d.nheads);
        const bf16_t* xb = static_cast<const bf16_t*>(x);
        const bf16_t* bb = static_cast<const bf16_t*>(B);
        const int L = (int)d.seqlen, H = (int)d.nheads, G = (int)d.ngroups, nc = (int)d.nchunks;
        if ((d.nheads / d.ngroups) % kStateHeads == 0) {
            const unsigned hblocks = blocks / (unsigned)kStateHeads;
            switch (d.chunk) {
                case 64: chunk_state_mfmah_kernel<64, kStateHeads, false><<<hblocks, 256, 0, stream>>>(xb, bb, cs, dtc, S, L, H, G, nc, nullptr, nullptr, nullptr, nullptr, 0); break;
                case 128: chunk_state_mfmah_kernel<128, kStateHeads, false><<<hblocks, 256, 0, stream>>>(xb, bb, cs, dtc, S, L, H, G, nc, nullptr, nullptr, nullptr, nullptr, 0); break;
                default: chunk_state_mfmah_kernel<256, kStateHeads, false><<<hblocks, 256, 0, stream>>>(xb, bb, cs, dtc, S, L, H, G, nc, nullptr, nullptr, nullptr, nullptr, 0); break;
            }
            return hipGetLastError();
        }
        switch (d.chunk) {
            case 64: chunk_state_mfma_kernel<64><<<blocks, 256, 0, stream>>>(xb, bb, cs, dtc, S, L, H, G, nc); break;
            case 128: chunk_state_mfma_kernel<128><<<blocks, 256, 0, stream>>>(xb, bb, cs, dtc, S, L, H, G, nc); break;
            default: chunk_state_mfma_kernel<256><<<blocks, 256, 0, stream>>>(xb, bb, cs, dtc, S, L, H, G, nc); break;
        }
    } else if (dtype == 1) {
        launch_generic_t<bf16_t>(d, x, B, cs, dtc, S, stream);
    } else {
        launch_generic_t<float>(d, x, B, cs, dtc, S, stream);
    }
    return hipGetLastError();
}

}  // namespace ssd
