// chunk_scan.hip -- the output of each chunk:
//
//     y_i = sum_{j<=i} (C_i . B_j) exp(Acs_i - Acs_j) dt_j x_j      (i)
//           + exp(Acs_i) Hin_c C_i                                  (ii)
//           + D_h x_i                                               (iii)
//
// (i) is the quadratic, attention-like form used inside a block: masked
// attention without softmax whose weights say how much of token j survived
// until token i (page "State Space Model", section "Due strade, una meta";
// page "Mamba-2 (2024): SSM e attention sono la stessa cosa", sections "Due
// modi di guardare la stessa matrice" and "Il trucco a blocchi").  (ii) is the
// summary state carried in from earlier blocks, read out by C after decaying
// through the chunk; (iii) is the D x term of y = C h + D x (page "Puntata 205",
// section "Cos'e' un SSM, in 30 secondi").
//
// Matrix-core kernel (bf16, P = 64, N = 128, Q in {64, 128, 256}); one
// workgroup of Q/64 waves per (batch, chunk, head); v_mfma_f32_32x32x16_bf16.
// Everything is computed transposed, Y^T[p][i], so that each lane owns one
// output token i (the MFMA result column) -- that makes the masked weights
// G~^T[j][i] of a 32 x 32 tile come out of the C.B^T product in exactly the
// register layout the next product needs as its B operand: no LDS round trip.
//   * G^T = B_j C_i^T  (M = 32 tokens j, N = 32 tokens i, K = N = 128).  The
//     A-operand row m of the tile reads token pi(m) of the j block; pi is the
//     permutation that makes accumulator register r of lane half hf hold token
//     16*(r/8) + 8*hf + r%8, i.e. the 8 K-slots of each following product
//     are 8 consecutive tokens.
//   * G~ = G * exp2(cs_i - cs_j) * dt_j below the diagonal (factorised as
//     exp2(cs_i - c0) * [exp2(c0 - cs_j) dt_j] with c0 the block's first
//     token, the bracket precomputed once per token), masked on the diagonal
//     block with D added on its diagonal (term iii); rounded to bf16.
//   * Y^T += X^T G~^T (M = P rows in two 32-row tiles, K = 32 tokens).  A-row m
//     reads channel sigma(m) so that a lane ends with 16 consecutive channels
//     of its token: two 16-byte stores per tile.
//   * Term (ii) first: Y^T = Hin C^T (K = N), then each column scaled by
//     exp2(cs_i).
// Wave w owns i tiles {w, 2W-1-w} so that every wave has the same number of
// causal (j <= i) tiles.  C fragments of the wave's own tokens stay in
// registers for the whole kernel; the carried state and the j blocks of B
// (32 rows) and x (32 rows) are copied straight into LDS (lds_pipe.h) through
// a 3-buffer ring, two blocks ahead, and x is read back transposed with tr16.
//
// Generic kernel (fp32 or bf16, any P, N within limits): the same three terms
// in fp32 on the vector units, 32 x 32 tiles in LDS.
#include <cmath>

#include "device_common.h"
#include "launchers.h"
#include "lds_pipe.h"

namespace ssd {

// Row m = 8a + 4hf + b of a 32-row MFMA tile.
__device__ __forceinline__ int perm_pi(int m) {
    const int a = m >> 3, hf = (m >> 2) & 1, b = m & 3;
    return 16 * (a >> 1) + 8 * hf + 4 * (a & 1) + b;
}
__device__ __forceinline__ int perm_sigma(int m) {
    const int a = m >> 3, hf = (m >> 2) & 1, b = m & 3;
    return 16 * hf + 4 * a + b;
}

// ---------------------------------------------------------------------------
// Pieces shared by the two matrix-core kernels.  A workgroup has 4 waves (or
// Q/64 for short chunks); wave w owns i tiles it_[0] = w and it_[1] = 2W-1-w.

// Per-lane tr16 addressing of the X^T operand (see lds_pipe.h): lane r of
// 16-lane group grp supplies token row 8*(grp/2) + r/4 and channel quad qb,
// so lane i receives channel 32*mt + sigma(16*(grp%2) + i).
struct XtAddr {
    int qb, trow0;
};
__device__ __forceinline__ XtAddr xt_addr(int lane) {
    const int grp = lane >> 4, rr = lane & 15;
    XtAddr a;
    a.qb = ((rr & 1) ? 16 : 0) + ((rr & 2) ? 4 : 0) + ((grp & 1) ? 8 : 0);
    a.trow0 = 8 * (grp >> 1) + (rr >> 2);
    return a;
}

// Largest decay across one 32-token output tile (log2 units) for which the
// factorised weights are used; beyond it the per-token factors could
// overflow, and the tile takes the direct form.
constexpr float kMaxTileDecayLog2 = 64.0f;

__device__ __forceinline__ float uniform_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

// Accumulator register r of lane (l32, hf) of a G^T tile holds block token
// j = 16*(r/8) + 8*hf + r%8 and column (output token) i = l32.
__host__ __device__ constexpr int gt_row(int r, int hf) { return 16 * (r >> 3) + 8 * hf + (r & 7); }

// Causal keep bits of the diagonal block for this lane (direct form).
__device__ __forceinline__ uint32_t diag_keep_bits(int l32, int hf) {
    const int t = l32 - 8 * hf;
    const int n0 = min(max(t + 1, 0), 8), n1 = min(max(t - 15, 0), 8);
    return ((1u << n0) - 1u) | (((1u << n1) - 1u) << 8);
}

// Bit r set iff accumulator register r of this lane is the diagonal entry
// j == i of the diagonal block (at most one per lane; direct form).
__device__ __forceinline__ uint32_t diag_eq_bits(int l32, int hf) {
    const int t = l32 - 8 * hf;
    if (t >= 0 && t < 8) return 1u << t;
    if (t >= 16 && t < 24) return 1u << (t - 8);
    return 0u;
}

// The same two sets as lane masks of one register r of a diagonal block,
// constant for every wave (register r holds j - 8 hf = 16 (r / 8) + r % 8
// of column i = l32): j <= i holds in lanes l32 >= jr of the first half
// and l32 >= jr + 8 of the second; j == i in lanes r and 40 + r (r < 8) or
// r + 8 and 48 + r (r >= 8).
__host__ __device__ constexpr uint64_t diag_keep_lanes(int r) {
    return ((0xffffffffull << (16 * (r >> 3) + (r & 7))) & 0xffffffffull) |
           (((0xffffffffull << (16 * (r >> 3) + (r & 7) + 8)) & 0xffffffffull) << 32);
}
__host__ __device__ constexpr uint64_t diag_eq_lanes(int r) {
    return r < 8 ? (1ull << r) | (1ull << (40 + r)) : (1ull << (r + 8)) | (1ull << (48 + r));
}
constexpr bool diag_lanes_match() {
    for (int r = 0; r < 16; ++r)
        for (int lane = 0; lane < 64; ++lane) {
            const int t = (lane & 31) - 8 * (lane >> 5), jr = 16 * (r >> 3) + (r & 7);
            if ((((diag_keep_lanes(r) >> lane) & 1u) != 0) != (t >= jr)) return false;
            if ((((diag_eq_lanes(r) >> lane) & 1u) != 0) != (t == jr)) return false;
        }
    return true;
}
static_assert(diag_lanes_match(), "diagonal lane masks disagree with the register layout");

// b in the lanes of mask m, a elsewhere: one select, no compare.
__device__ __forceinline__ float lane_select(float a, float b, uint64_t m) {
    float d;
    asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "s"(m));
    return d;
}

// C fragments of the wave's own tokens (B operand of both C products).
// Tokens past the end of the sequence re-read the last token: C_i only
// reaches output column i, which is not stored for those tokens.
__device__ __forceinline__ void load_c_frags(uint4 (&cf)[2][8], const bf16_t* Cm, int64_t b, int L,
                                             int G, int g, int tok0, const int (&it_)[2], int hf,
                                             int l32) {
    constexpr int N = 128;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int tok = min(tok0 + 32 * it_[t] + l32, L - 1);
        const bf16_t* crow = Cm + ((b * L + tok) * G + g) * N + 8 * hf;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) cf[t][kk] = *reinterpret_cast<const uint4*>(crow + 16 * kk);
    }
}

// Per-tile factors.  With the factorised form (fact), tile t's weights are
// exp2(cs_i - cs_j) dt_j = colf_i * rf_j, colf_i = exp2(cs_i - cref) and
// rf_j = exp2(cref - cs_j) dt_j with cref = cs of the tile's first token:
// the accumulator gathers sum_j x_j G_ji rf_j (+ D x_i / colf_i on the
// diagonal), starts from exp2(cref) * (Hin C_i) and is scaled by colf_i at
// the end.  Otherwise (direct form) the weights are formed per element and
// the state term is scaled by exp2(cs_i).
struct TileF {
    bool fact;
    float colf;     // final column scale (1 for the direct form)
    float sstate;   // scale of the state term
    float dprime;   // D / colf_i, the diagonal addend of the factorised form
};

// (ii) carried state: acc[t][mt] = sstate_t * sum_n Hin[p][n] C[i][n].
__device__ __forceinline__ void scan_state_term(f32x16 (&acc)[2][2], const uint4* hs,
                                                const uint4 (&cf)[2][8], const TileF (&tf)[2],
                                                int hf, int l32) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) acc[t][mt] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int pr = 32 * mt + perm_sigma(l32);
            const int ch = 2 * kk + hf;
            const bf16x8 a = __builtin_bit_cast(bf16x8, hs[pr * 16 + (ch ^ swz_h(pr))]);
#pragma unroll
            for (int t = 0; t < 2; ++t)
                acc[t][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, cf[t][kk]), acc[t][mt], 0, 0, 0);
        }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[t][mt][r] *= tf[t].sstate;
}

// (i) + (iii) for j block jt: G^T tiles from the B block, decay weights
// (+ D on the diagonal), then Y^T += X^T G~^T.
template <int Q>
__device__ __forceinline__ void scan_block(f32x16 (&acc)[2][2], int jt, const uint4* bst,
                                           const uint4* xst, const float* cs_s, const float* dt_s,
                                           const float* rfT, const uint4 (&cf)[2][8],
                                           const float (&csi)[2], const int (&it_)[2],
                                           const TileF (&tf)[2], float Dh, XtAddr xa, int hf,
                                           int l32, uint32_t diag_keep, uint32_t diag_eq) {
    if (it_[1] < jt) return;   // it_[1] >= it_[0]: nothing left for this wave
    const bool act0 = it_[0] >= jt;
    // G^T tiles.  The branch sits outside the K loop, and the B-row reads
    // run two steps ahead of the products (the scheduler, short of
    // registers, would otherwise wait out each read's latency in turn).
    f32x16 gacc[2];
    {
        const int jr = perm_pi(l32);
        const uint4* brow = bst + jr * 16;
        const int sw = swz_b(jr);
        bf16x8 bq[2];
        bq[0] = __builtin_bit_cast(bf16x8, brow[hf ^ sw]);
        bq[1] = __builtin_bit_cast(bf16x8, brow[(2 + hf) ^ sw]);
        if (act0) {
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const bf16x8 cur = bq[kk & 1];
                if (kk + 2 < 8) bq[kk & 1] = __builtin_bit_cast(bf16x8, brow[(2 * (kk + 2) + hf) ^ sw]);
                gacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, __builtin_bit_cast(bf16x8, cf[0][kk]), kk ? gacc[0] : f32x16{}, 0, 0, 0);
                gacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, __builtin_bit_cast(bf16x8, cf[1][kk]), kk ? gacc[1] : f32x16{}, 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const bf16x8 cur = bq[kk & 1];
                if (kk + 2 < 8) bq[kk & 1] = __builtin_bit_cast(bf16x8, brow[(2 * (kk + 2) + hf) ^ sw]);
                gacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, __builtin_bit_cast(bf16x8, cf[1][kk]), kk ? gacc[1] : f32x16{}, 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    const SSD_LDS char* xb = (const SSD_LDS char*)lds(xst);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        if (t == 0 && !act0) continue;
        uint32_t pk[8];
        const bool dgb = it_[t] == jt;
        if (tf[t].fact) {
            // rf_j of this tile's reference for the lane's 16 block tokens
            const float* rfb = rfT + it_[t] * Q + 32 * jt + 8 * hf;
            const float4 f0 = *reinterpret_cast<const float4*>(rfb);
            const float4 f1 = *reinterpret_cast<const float4*>(rfb + 4);
            const float4 f2 = *reinterpret_cast<const float4*>(rfb + 16);
            const float4 f3 = *reinterpret_cast<const float4*>(rfb + 20);
            const float rf[16] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w,
                                  f2.x, f2.y, f2.z, f2.w, f3.x, f3.y, f3.z, f3.w};
            if (!dgb) {
#pragma unroll
                for (int r2 = 0; r2 < 8; ++r2)
                    pk[r2] = pack_bf16x2(gacc[t][2 * r2] * rf[2 * r2], gacc[t][2 * r2 + 1] * rf[2 * r2 + 1]);
            } else {
                // causal mask j <= i and D on j == i, selects on constant
                // lane masks
                float v[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float w = lane_select(0.0f, gacc[t][r] * rf[r], diag_keep_lanes(r));
                    v[r] = lane_select(w, w + tf[t].dprime, diag_eq_lanes(r));
                }
#pragma unroll
                for (int r2 = 0; r2 < 8; ++r2) pk[r2] = pack_bf16x2(v[2 * r2], v[2 * r2 + 1]);
            }
        } else {
            // direct weights for a tile with too much decay to factorise
            const float* csb = cs_s + 32 * jt + 8 * hf;
            const float* dtb = dt_s + 32 * jt + 8 * hf;
            const uint32_t keep = dgb ? diag_keep : 0xffffu;
            const uint32_t deq = dgb ? diag_eq : 0u;
#pragma unroll
            for (int r2 = 0; r2 < 8; ++r2) {
                float v2[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int r = 2 * r2 + e;
                    const int jl = 16 * (r >> 3) + (r & 7);
                    const float kf = (float)((keep >> r) & 1u);
                    const float df = (float)((deq >> r) & 1u);
                    v2[e] = gacc[t][r] * (fast_exp2(fminf(csi[t] - csb[jl], 0.0f)) * dtb[jl] * kf) + Dh * df;
                }
                pk[r2] = pack_bf16x2(v2[0], v2[1]);
            }
        }
        const bf16x8 gq[2] = {__builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3])),
                              __builtin_bit_cast(bf16x8, make_uint4(pk[4], pk[5], pk[6], pk[7]))};
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int pc = 32 * mt + xa.qb;          // multiple of 4
            const int chk = pc >> 3, sub = (pc & 7) * 2;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int r0 = 16 * u + xa.trow0, r1 = r0 + 4;
                const uint2 lo = tr16(xb + r0 * 128 + ((chk ^ swz_x(r0)) << 4) + sub);
                const uint2 hi = tr16(xb + r1 * 128 + ((chk ^ swz_x(r1)) << 4) + sub);
                const bf16x8 xq = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
                acc[t][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xq, gq[u], acc[t][mt], 0, 0, 0);
            }
        }
    }
}

// y rows of the wave's own tokens: lane owns token i, channels
// 32*mt + 16*hf + 0..15 (two 16-byte stores per tile), after the final
// column scale.  Buffer stores against a record bounded by the sequence end:
// every wave always issues its 8 stores (fixed memory-counter arithmetic),
// and the hardware drops those of tokens past the end.
__device__ __forceinline__ void scan_store_y(const f32x16 (&acc)[2][2], const TileF (&tf)[2],
                                             __amdgpu_buffer_rsrc_t yrs, int rowbytes,
                                             const int (&it_)[2], int hf, int l32) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int off = (32 * it_[t] + l32) * rowbytes + 32 * hf;
        const float s = tf[t].colf;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            uint32_t w8[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) w8[k] = pack_bf16x2(acc[t][mt][2 * k] * s, acc[t][mt][2 * k + 1] * s);
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
            const u32x4 v0 = {w8[0], w8[1], w8[2], w8[3]};
            const u32x4 v1 = {w8[4], w8[5], w8[6], w8[7]};
            __builtin_amdgcn_raw_buffer_store_b128(v0, yrs, off + 64 * mt, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b128(v1, yrs, off + 64 * mt + 16, 0, 0);
        }
    }
}

// Pipeline buffer k of a 4-deep ring (compile-time k after unrolling).
template <typename T>
__device__ __forceinline__ T* ring4(int k, T* a0, T* a1, T* a2, T* a3) {
    const int m = k & 3;
    return m == 0 ? a0 : (m == 1 ? a1 : (m == 2 ? a2 : a3));
}

// Memory operations a wave issues at loop step k of a head (stage k + 3 of
// this head or of the next, and at k = 0 the next head's carried state and
// cs/dt rows).
__host__ __device__ constexpr int scan_issue_ops(int NT, int k, bool more, int DPS, int DH, int DC) {
    return (k + 3 < NT ? DPS : (more ? DPS : 0)) + (k == 0 && more ? DH + DC : 0);
}
// Operations issued after stage jt of the current head and before the wait
// at step jt: stages 0..2 came at the end of the previous head, followed by
// its NY y stores.
__host__ __device__ constexpr int scan_ops_after(int NT, int jt, bool more, int DPS, int DH, int DC,
                                                 int NY) {
    int n = 0;
    if (jt <= 2) {
        n = (2 - jt) * DPS + NY;
        for (int k = 0; k < jt; ++k) n += scan_issue_ops(NT, k, more, DPS, DH, DC);
    } else {
        n = (jt == 3 && more) ? DH + DC : 0;   // issued right after stage 3
        for (int k = jt - 2; k < jt; ++k) n += scan_issue_ops(NT, k, more, DPS, DH, DC);
    }
    return n;
}

// The streaming kernel's issue order for a run of hg heads (labels: stage s
// of head h, carried state, cs/dt rows, y stores), replayed against the
// counts above: each step's stage, and before the next head its carried
// state and rows, must have landed.
constexpr bool scan_waits_hold(int NT, int W, int hg) {
    const int DPS = 12 / W, DH = 16 / W, DC = 2, NY = 8;
    auto stage = [](int h, int s) { return 1000 + 16 * h + s; };
    auto hin = [](int h) { return 2000 + h; };
    auto rows = [](int h) { return 3000 + h; };
    VmemLog o;
    o.push(rows(0), DC);
    o.push(hin(0), DH);
    for (int s = 0; s < 3; ++s) o.push(stage(0, s), DPS);
    if (!o.wait(0)) return false;
    for (int hi = 0; hi < hg; ++hi) {
        const bool more = hi + 1 < hg;
        for (int jt = 0; jt < NT; ++jt) {
            if (!o.wait(scan_ops_after(NT, jt, more, DPS, DH, DC, NY)) || !o.landed(stage(hi, jt))) return false;
            if (jt + 3 < NT) o.push(stage(hi, jt + 3), DPS);
            else if (more) o.push(stage(hi + 1, jt + 3 - NT), DPS);
            if (jt == 0 && more) {
                o.push(hin(hi + 1), DH);
                o.push(rows(hi + 1), DC);
            }
        }
        o.push(4000 + hi, NY);
        if (more && (!o.wait((NT - 1) * DPS + NY) || !o.landed(hin(hi + 1)) || !o.landed(rows(hi + 1))))
            return false;
    }
    return true;
}
static_assert(scan_waits_hold(8, 4, 1) && scan_waits_hold(8, 4, 2) && scan_waits_hold(8, 4, 5) &&
              scan_waits_hold(4, 2, 1) && scan_waits_hold(4, 2, 2) && scan_waits_hold(4, 2, 5),
              "chunk_scan wait counts do not cover its copies");

// ---------------------------------------------------------------------------
// One workgroup per (batch, chunk, run of hg heads of one group).  The heads
// share C, so the C fragments are loaded once; everything a head needs
// besides (its carried state, cs/dt rows, x) streams in while the previous
// head computes:
//   per wave and head, in issue order (Q = 256: 4 waves, 3 copies a stage):
//     jt = 0: stage 3, Hin(next) x4, cs/dt(next) x2
//     jt = 1..4: stages 4..7;  jt = 5..7: stages 0..2 of the next head
//     end: 8 y stores
// and the wait before block jt leaves exactly the operations issued after
// stage jt outstanding (fewer on the last head, which prefetches nothing).
template <int Q>
__global__ __launch_bounds__(Q, 2) void chunk_scan_mfma_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ Bm, const bf16_t* __restrict__ Cm,
    const float* __restrict__ cs, const float* __restrict__ dtc, const bf16_t* __restrict__ Hin,
    const float* __restrict__ D, bf16_t* __restrict__ y, int L, int H, int G, int nc, int hg) {
    constexpr int P = 64, N = 128, W = Q / 64, NT = Q / 32;
    static_assert(NT % 4 == 0, "the ring index must repeat every head");
    constexpr int DPS = 12 / W;      // LDS-copy instructions per wave per stage
    constexpr int DH = 16 / W;       // ... for the carried state
    constexpr int DC = 2;            // ... for the cs and dt rows
    constexpr int NY = 8;            // y stores per wave
    // One array per copy target in flight (the compiler tracks a few LDS
    // copy targets separately and waits for all copies beyond that).
    __shared__ uint4 hs[1024];                              // Hin, 64 rows x 256 B
    __shared__ uint4 st0[768], st1[768], st2[768], st3[768];   // stages: B 32 x 256 B, x 32 x 128 B
    __shared__ float csdt_n[2 * Q];                         // next head's cs and dt rows
    __shared__ float cs_s[Q];                               // current head's
    __shared__ float dt_s[Q];
    __shared__ __align__(16) float rfT[NT * Q];             // rf_j per output tile

    const int ngr = H / hg;
    const uint32_t wg = xcd_logical_id(blockIdx.x, gridDim.x);
    const int hgi = (int)(wg % (uint32_t)ngr);
    const int bc = (int)(wg / (uint32_t)ngr);
    const int c = bc % nc, b = bc / nc;
    const int h0 = hgi * hg;
    const int g = h0 / (H / G);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hf = lane >> 5, l32 = lane & 31;
    const int tok0 = c * Q;
    const int64_t xstride = (int64_t)H * P, bstride = (int64_t)G * N;
    const bf16_t* bbase = Bm + ((int64_t)b * L * G + g) * N;
    const int rowbytes = H * P * 2;
    // end of the chunk's last valid row (within the chunk: Q rows of a
    // token row's bytes fit 31 bits)
    const int yrecord = (min(L - tok0, Q) - 1) * rowbytes + P * 2;

    // Copies for head h0: cs/dt rows, the carried state, stages 0..2.
    auto issue_csdt = [&](int h) {
        const int64_t row = (((int64_t)b * H + h) * nc + c) * Q;
        dma4(cs + row, 4u * (uint32_t)tid, lds(csdt_n) + 64 * wave);
        dma4(dtc + row, 4u * (uint32_t)tid, lds(csdt_n) + Q + 64 * wave);
    };
    // per-lane copy offsets, fixed for the whole workgroup
    const BxOffsets<W> bxo = bx_offsets<W>(wave, lane, xstride, bstride);
    uint32_t hoff[DH];
#pragma unroll
    for (int i = 0; i < DH; ++i) {
        const int r = 4 * (wave + i * W) + (lane >> 4);
        hoff[i] = (uint32_t)(r * N + 8 * ((lane & 15) ^ swz_h(r))) * 2u;
    }
    auto issue_hin = [&](int h) {
        const bf16_t* hsrc = Hin + ((((int64_t)b * H + h) * nc + c) * (int64_t)(P * N));
#pragma unroll
        for (int i = 0; i < DH; ++i) dma16(hsrc, hoff[i], lds(hs) + (wave + i * W) * 64);
    };
    auto issue_stage = [&](int h, int s, uint4* bst, uint4* xst) {
        const bf16_t* xbase = x + ((int64_t)b * L * H + h) * P;
        issue_bx_stage<W>(wave, lane, tok0 + 32 * s, L, xbase, xstride, bbase, bstride, bxo, bst, xst);
    };
    // rf table and current cs/dt rows from the copied next-head rows.
    auto make_tables = [&]() {
        const float cv = csdt_n[tid], dv = csdt_n[Q + tid];
        cs_s[tid] = cv;
        dt_s[tid] = dv;
#pragma unroll
        for (int k = 0; k < NT; ++k)
            if (k >= (tid >> 5)) rfT[k * Q + tid] = fast_exp2(fminf(csdt_n[32 * k] - cv, kMaxTileDecayLog2)) * dv;
    };

    issue_csdt(h0);
    issue_hin(h0);
    issue_stage(h0, 0, st0, st0 + 512);
    issue_stage(h0, 1, st1, st1 + 512);
    issue_stage(h0, 2, st2, st2 + 512);
    const int it_[2] = {wave, 2 * W - 1 - wave};
    uint4 cf[2][8];
    load_c_frags(cf, Cm, b, L, G, g, tok0, it_, hf, l32);
    wait_vmcnt<0>();
    barrier_lds();
    make_tables();
    barrier_lds();

    for (int hi = 0; hi < hg; ++hi) {
        const int h = h0 + hi;
        // Lane-dependent values are re-derived every head: laundering the
        // lane index keeps the compiler from hoisting every LDS address of
        // the unrolled block loop out of the head loop (which costs far more
        // registers than recomputing them).
        int lane_o = lane;
        asm volatile("" : "+v"(lane_o));
        const int hf_o = lane_o >> 5, l32_o = lane_o & 31;
        const XtAddr xa = xt_addr(lane_o);
        const uint32_t dkeep = diag_keep_bits(l32_o, hf_o);
        const uint32_t deq = diag_eq_bits(l32_o, hf_o);
        const bool more = hi + 1 < hg;
        const float Dh = D ? D[h] : 0.0f;
        float csi[2];
        TileF tf[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int i0 = 32 * it_[t];
            const float cref = cs_s[i0];
            csi[t] = cs_s[i0 + l32_o];
            tf[t].fact = uniform_f(cref - cs_s[i0 + 31]) <= kMaxTileDecayLog2;
            if (tf[t].fact) {
                tf[t].colf = fast_exp2(csi[t] - cref);
                tf[t].sstate = fast_exp2(cref);
                tf[t].dprime = Dh * fast_exp2(cref - csi[t]);
            } else {
                tf[t].colf = 1.0f;
                tf[t].sstate = fast_exp2(csi[t]);
                tf[t].dprime = 0.0f;
            }
        }
        f32x16 acc[2][2];
        scan_state_term(acc, hs, cf, tf, hf_o, l32_o);

#pragma unroll
        for (int jt = 0; jt < NT; ++jt) {
            // stage jt has landed once only the operations issued after it
            // are outstanding (the first head's stages 0..2 were waited for
            // in full before the loop)
            if (more) wait_vmcnt_n(scan_ops_after(NT, jt, true, DPS, DH, DC, NY));
            else wait_vmcnt_n(scan_ops_after(NT, jt, false, DPS, DH, DC, NY));
            barrier_lds();
            uint4* nst = ring4(jt + 3, st0, st1, st2, st3);
            if (jt + 3 < NT) {
                issue_stage(h, jt + 3, nst, nst + 512);
            } else if (more) {
                issue_stage(h + 1, jt + 3 - NT, nst, nst + 512);
            }
            if (jt == 0 && more) {
                issue_hin(h + 1);
                issue_csdt(h + 1);
            }
            uint4* cst = ring4(jt, st0, st1, st2, st3);
            scan_block<Q>(acc, jt, cst, cst + 512, cs_s,
                          dt_s, rfT, cf, csi, it_, tf, Dh, xa, hf_o, l32_o, dkeep, deq);
        }
        const __amdgpu_buffer_rsrc_t yrs = __builtin_amdgcn_make_buffer_rsrc(
            y + (((int64_t)b * L + tok0) * H + h) * P, (short)0, yrecord, 0x00020000);
        scan_store_y(acc, tf, yrs, rowbytes, it_, hf_o, l32_o);
        if (more) {
            // the next head's carried state and cs/dt rows (issued at step 0)
            wait_vmcnt_n((NT - 1) * DPS + NY);
            barrier_lds();
            make_tables();
            barrier_lds();
        }
    }
}

// ---------------------------------------------------------------------------
// Resident kernel (Q = 256): one workgroup of 4 waves per CU and per (batch,
// chunk, group, run of heads).  G^T = B_j C_i^T does not depend on the head,
// so each wave forms its 9 causal G^T tiles once (8 products each, operands
// loaded straight into registers) and keeps them in registers for all of the
// run's heads; per head only the decay weights, the Y^T products and the
// carried-state product remain.  A head's x rows, carried state and cs/dt
// rows (50 KB) are copied into one of three LDS slots two heads ahead, so
// the workgroup meets once per head.
//   per wave and head, in issue order: copies for head k + 2 (x 8, Hin 4,
//   cs 1, dt 1), then the y stores of its two tiles (4 each).
// Wave w owns i tiles t1 = 7 - w (blocks 0..7-w, processed first) and
// t0 = w (blocks 0..w): slot s < 8 - w is (t1, s), slot s >= 8 - w is
// (t0, s - 8 + w).
namespace rsl {
constexpr int kX = 0;          // x: 256 rows x 128 B
constexpr int kH = 32768;      // Hin: 64 rows x 256 B
constexpr int kCs = 49152;     // cs: 256 floats
constexpr int kDt = 50176;     // dt: 256 floats
constexpr int kSlot = 51200;
constexpr int kCopies = 14;    // LDS-copy instructions per wave per head
constexpr int kStores = 8;     // y stores per wave per head
constexpr int kPartCopies[4] = {4, 4, 4, 2};   // x rows 0..127, x rows 128..255, Hin, cs + dt
static_assert(kPartCopies[0] + kPartCopies[1] + kPartCopies[2] + kPartCopies[3] == kCopies, "copy count");

// The resident kernel's issue order (labels: copies of head k, y stores of
// head k) replayed against its waits at the top of each head: head k's
// copies must have landed.  Its tile-(7 - w) stores follow slot 3 for every
// wave, so both store groups come after the head's copies.
constexpr bool waits_hold(int heads) {
    VmemLog o;
    o.push(100, kCopies);
    o.push(101, kCopies);
    for (int k = 0; k < heads; ++k) {
        const int cnt = k == 0 ? 0 : (k == 1 ? kCopies + kStores : kCopies + 2 * kStores);
        if (!o.wait(cnt) || !o.landed(100 + k)) return false;
        for (int part = 0; part < 4; ++part) o.push(100 + k + 2, kPartCopies[part]);
        o.push(200 + k, kStores);
    }
    return true;
}
static_assert(waits_hold(1) && waits_hold(2) && waits_hold(3) && waits_hold(12) && waits_hold(40),
              "resident chunk_scan wait counts do not cover its copies");
}  // namespace rsl

// Carried-state term of both of the wave's tiles, acc[q][mt] = sstate_q *
// Hin C_q^T (q = 0: t0, 1: t1).  The 16 Hin fragments are read at the top
// of the head (rs_hin_read), ahead of the head's other LDS work: with one
// wave per SIMD nothing else would cover their latency.
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void rs_hin_read(u32x4v (&a)[8][2], const SSD_LDS uint4* hs, int hf, int l32) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int pr = 32 * mt + perm_sigma(l32);
            const int ch = 2 * kk + hf;
            a[kk][mt] = *reinterpret_cast<const SSD_LDS u32x4v*>(hs + pr * 16 + (ch ^ swz_h(pr)));
        }
}
__device__ __forceinline__ void rs_state_terms(f32x16 (&acc)[2][2], const u32x4v (&a)[8][2],
                                               const uint4 (&cf)[2][8], const TileF (&tf)[2]) {
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) acc[q][mt] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int q = 0; q < 2; ++q)
                acc[q][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[kk][mt]), __builtin_bit_cast(bf16x8, cf[q][kk]), acc[q][mt], 0, 0, 0);
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[q][mt][r] *= tf[q].sstate;
}

// LDS operands of one slot: the rf values of the lane's 16 block tokens
// (rs_fetch_rf) and the X^T fragments of the block (rs_fetch_x, xq[mt][u]).
struct SlotRf {
    f32x4 f[4];
};
struct SlotX {
    u32x4v xq[2][2];
};
__device__ __forceinline__ void rs_fetch_rf(SlotRf& o, const SSD_LDS float* rfs, int hf) {
    const SSD_LDS float* rfb = rfs + 8 * hf;
    o.f[0] = *reinterpret_cast<const SSD_LDS f32x4*>(rfb);
    o.f[1] = *reinterpret_cast<const SSD_LDS f32x4*>(rfb + 4);
    o.f[2] = *reinterpret_cast<const SSD_LDS f32x4*>(rfb + 16);
    o.f[3] = *reinterpret_cast<const SSD_LDS f32x4*>(rfb + 20);
}
__device__ __forceinline__ void rs_fetch_x(SlotX& o, const SSD_LDS char* xb, XtAddr xa) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        const int pc = 32 * mt + xa.qb;
        const int chk = pc >> 3, sub = (pc & 7) * 2;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int r0 = 16 * u + xa.trow0, r1 = r0 + 4;
            const u32x2v lo = __builtin_bit_cast(u32x2v, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (SSD_LDS v4s*)(xb + r0 * 128 + ((chk ^ swz_x(r0)) << 4) + sub)));
            const u32x2v hi = __builtin_bit_cast(u32x2v, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (SSD_LDS v4s*)(xb + r1 * 128 + ((chk ^ swz_x(r1)) << 4) + sub)));
            o.xq[mt][u] = u32x4v{lo.x, lo.y, hi.x, hi.y};
        }
    }
}

// Weights of one slot as the B operand of its products (bf16 pairs): the
// resident G^T tile gt times rf_j, plus D' on the entry j == i of a
// diagonal block (rs_weights_fact; the causal mask of the diagonal blocks is
// already in gt), or, for a tile with too much decay to factorise, the
// direct form (rs_weights_direct).  Register r of a lane holds the entry
// j - 8 hf = 16 (r / 8) + r % 8 of column i = l32 of the block.
__device__ __forceinline__ void rs_weights_fact(u32x4v (&gq)[2], const f32x16& gt, const SlotRf& in,
                                                bool dgb, float dprime) {
    auto rf = [&](int r) {
        const f32x4 q = r < 4 ? in.f[0] : (r < 8 ? in.f[1] : (r < 12 ? in.f[2] : in.f[3]));
        return q[r & 3];
    };
    float v[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = gt[r] * rf(r);
    if (dgb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = lane_select(v[r], v[r] + dprime, diag_eq_lanes(r));
    }
    uint32_t pk[8];
#pragma unroll
    for (int r2 = 0; r2 < 8; ++r2) pk[r2] = pack_bf16x2(v[2 * r2], v[2 * r2 + 1]);
    gq[0] = u32x4v{pk[0], pk[1], pk[2], pk[3]};
    gq[1] = u32x4v{pk[4], pk[5], pk[6], pk[7]};
}
__device__ __forceinline__ void rs_weights_direct(u32x4v (&gq)[2], const f32x16& gt,
                                                  const SSD_LDS float* csb, const SSD_LDS float* dtb,
                                                  float csi, float Dh, bool dgb, int hf, int l32) {
    // gt is zero above the diagonal of a diagonal block
    const SSD_LDS float* cb = csb + 8 * hf;
    const SSD_LDS float* db = dtb + 8 * hf;
    const uint32_t deq = dgb ? diag_eq_bits(l32, hf) : 0u;
    uint32_t pk[8];
#pragma unroll
    for (int r2 = 0; r2 < 8; ++r2) {
        float v2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int r = 2 * r2 + e;
            const int jl = 16 * (r >> 3) + (r & 7);
            const float df = (float)((deq >> r) & 1u);
            v2[e] = gt[r] * (fast_exp2(fminf(csi - cb[jl], 0.0f)) * db[jl]) + Dh * df;
        }
        pk[r2] = pack_bf16x2(v2[0], v2[1]);
    }
    gq[0] = u32x4v{pk[0], pk[1], pk[2], pk[3]};
    gq[1] = u32x4v{pk[4], pk[5], pk[6], pk[7]};
}

// acc += X^T G~^T for one slot (M = P rows in two 32-row tiles, K = the
// block's 32 tokens).
__device__ __forceinline__ void rs_products(f32x16 (&acc)[2], const SlotX& x, const u32x4v (&gq)[2]) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int u = 0; u < 2; ++u)
            acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x.xq[mt][u]),
                                                              __builtin_bit_cast(bf16x8, gq[u]), acc[mt], 0, 0, 0);
}

// y rows of tile t (lane owns token 32 t + l32, channels 32 mt + 16 hf +
// 0..15) after the final column scale; 4 buffer stores, dropped past the end.
__device__ __forceinline__ void rs_store(const f32x16 (&acc)[2], float colf, __amdgpu_buffer_rsrc_t yrs,
                                         int rowbytes, int t, int hf, int l32) {
    const int off = (32 * t + l32) * rowbytes + 32 * hf;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        uint32_t w8[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) w8[k] = pack_bf16x2(acc[mt][2 * k] * colf, acc[mt][2 * k + 1] * colf);
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 v0 = {w8[0], w8[1], w8[2], w8[3]};
        const u32x4 v1 = {w8[4], w8[5], w8[6], w8[7]};
        __builtin_amdgcn_raw_buffer_store_b128(v0, yrs, off + 64 * mt, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(v1, yrs, off + 64 * mt + 16, 0, 0);
    }
}

__global__ __launch_bounds__(256, 1) void chunk_scan_resident_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ Bm, const bf16_t* __restrict__ Cm,
    const float* __restrict__ cs, const float* __restrict__ dtc, const bf16_t* __restrict__ Hin,
    const float* __restrict__ D, bf16_t* __restrict__ y, int L, int H, int G, int nc, int hg,
    int nsplit) {
    constexpr int Q = 256, P = 64, N = 128;
    __shared__ __align__(16) char slots[3 * rsl::kSlot];
    __shared__ __align__(16) float rfw[4][288];

    const uint32_t wg = xcd_logical_id(blockIdx.x, gridDim.x);
    const int split = (int)(wg % (uint32_t)nsplit);
    const uint32_t bcg = wg / (uint32_t)nsplit;
    const int g = (int)(bcg % (uint32_t)G);
    const int bc = (int)(bcg / (uint32_t)G);
    const int c = bc % nc, b = bc / nc;
    const int hpg = H / G;
    const int h0 = g * hpg + split * hg;
    const int cnt = min(hg, hpg - split * hg);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    __builtin_assume(wave >= 0 && wave < 4);
    const int hf = lane >> 5, l32 = lane & 31;
    const int tok0 = c * Q;
    const int rowbytes = H * P * 2;
    // end of the chunk's last valid row, for x and y (within the chunk: Q
    // rows of a token row's bytes fit 31 bits)
    const int xrecord = (min(L - tok0, Q) - 1) * rowbytes + P * 2;
    const int t0 = wave, t1 = 7 - wave;
    SSD_LDS char* const sl0 = (SSD_LDS char*)lds(slots);

    // Per-lane copy offsets.  x copy i covers rows 32 i + 8 w .. + 7; Hin
    // copy i rows 16 i + 4 w .. + 3.
    const uint32_t xo0 = (uint32_t)(8 * wave + (lane >> 3)) * (uint32_t)rowbytes +
                         16u * (uint32_t)((lane & 7) ^ swz_x(lane >> 3));
    const uint32_t xstep = 32u * (uint32_t)rowbytes;
    uint32_t ho[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 16 * i + 4 * wave + (lane >> 4);
        ho[i] = (uint32_t)(r * 256 + 16 * ((lane & 15) ^ swz_h(r)));
    }
    // Copies of head k into the slot at byte offset so, in four parts (x
    // rows 0..127, x rows 128..255, Hin, cs/dt); past the run's last head
    // they read empty records (zeros, no memory traffic), which keeps every
    // wait count fixed.  (Non-temporal x copies were 1% faster alone and made
    // the whole forward 1-2% slower.)
    auto issue_part = [&](int k, uint32_t so, int part) {
        const bool real = k < cnt;
        const int h = h0 + (real ? k : 0);
        SSD_LDS char* s = sl0 + so;
        if (part < 2) {
            const __amdgpu_buffer_rsrc_t rx =
                make_rs(x + (((int64_t)b * L + tok0) * H + h) * P, real ? xrecord : 0);
#pragma unroll
            for (int i = 4 * part; i < 4 * part + 4; ++i)
                dma16_rs(rx, xo0 + (uint32_t)i * xstep, s + rsl::kX + (4 * i + wave) * 1024);
        } else if (part == 2) {
            const __amdgpu_buffer_rsrc_t rh =
                make_rs(Hin + (((int64_t)b * H + h) * nc + c) * (int64_t)(P * N), real ? P * N * 2 : 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) dma16_rs(rh, ho[i], s + rsl::kH + (4 * i + wave) * 1024);
        } else {
            const int64_t row = (((int64_t)b * H + h) * nc + c) * Q;
            dma4_rs(make_rs(cs + row, real ? Q * 4 : 0), 4u * (uint32_t)tid, s + rsl::kCs + 256 * wave);
            dma4_rs(make_rs(dtc + row, real ? Q * 4 : 0), 4u * (uint32_t)tid, s + rsl::kDt + 256 * wave);
        }
    };
    auto issue_head = [&](int k, uint32_t so) {
#pragma unroll
        for (int part = 0; part < 4; ++part) issue_part(k, so, part);
    };

    issue_head(0, 0);
    issue_head(1, rsl::kSlot);

    // C fragments of the wave's tiles (cf[0]: t0, cf[1]: t1) and the
    // resident G^T tiles.
    const int it_[2] = {t0, t1};
    uint4 cf[2][8];
    load_c_frags(cf, Cm, b, L, G, g, tok0, it_, hf, l32);
    f32x16 gt[9];
    {
        // B rows of slot s's block in registers, two slots ahead of the
        // products (the scheduler would otherwise pull each load down to its
        // use and wait out the latency slot by slot)
        const int jr = perm_pi(l32);
        uint4 bq[3][8];
        auto load_b = [&](int s, uint4 (&dst)[8]) {
            const int jt = s < 8 - wave ? s : s - (8 - wave);
            const int tok = min(tok0 + 32 * jt + jr, L - 1);
            const bf16_t* brow = Bm + (((int64_t)b * L + tok) * G + g) * N + 8 * hf;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) dst[kk] = *reinterpret_cast<const uint4*>(brow + 16 * kk);
        };
        load_b(0, bq[0]);
        load_b(1, bq[1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < 9; ++s) {
            if (s + 2 < 9) load_b(s + 2, bq[(s + 2) % 3]);
            __builtin_amdgcn_sched_barrier(0);
            const uint4 (&bs)[8] = bq[s % 3];
            f32x16 a = {};
            if (s < 8 - wave) {
#pragma unroll
                for (int kk = 0; kk < 8; ++kk)
                    a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, bs[kk]), __builtin_bit_cast(bf16x8, cf[1][kk]), a, 0, 0, 0);
            } else {
#pragma unroll
                for (int kk = 0; kk < 8; ++kk)
                    a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, bs[kk]), __builtin_bit_cast(bf16x8, cf[0][kk]), a, 0, 0, 0);
            }
            if (s == 8 || s == 7 - wave) {
                // a diagonal block: its causal mask j <= i does not depend
                // on the head, so it is applied here once
#pragma unroll
                for (int r = 0; r < 16; ++r) a[r] = lane_select(0.0f, a[r], diag_keep_lanes(r));
            }
            gt[s] = a;
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    uint32_t so = 0;   // slot of head k
    for (int k = 0; k < cnt; ++k) {
        // head k's copies have landed once only those issued after them are
        // outstanding: (k >= 2) y stores of k - 2, copies of k + 1, y
        // stores of k - 1
        if (k == 0) wait_vmcnt<0>();
        else if (k == 1) wait_vmcnt<rsl::kCopies + rsl::kStores>();
        else wait_vmcnt<rsl::kCopies + 2 * rsl::kStores>();
        barrier_lds();
        // every wave is past head k - 1: its slot takes head k + 2, copied in
        // parts during slots 0..3 (all before this head's first y stores:
        // the wait counts above hold)
        const uint32_t so2 = so >= (uint32_t)rsl::kSlot ? so - rsl::kSlot : so + 2 * rsl::kSlot;

        const int h = h0 + k;
        const SSD_LDS char* S = sl0 + so;
        const SSD_LDS float* css = (const SSD_LDS float*)(S + rsl::kCs);
        const SSD_LDS float* dts = (const SSD_LDS float*)(S + rsl::kDt);
        const float Dh = D ? D[h] : 0.0f;
        int lane_o = lane;
        asm volatile("" : "+v"(lane_o));
        const int hf_o = lane_o >> 5, l32_o = lane_o & 31;
        const XtAddr xa = xt_addr(lane_o);
        u32x4v ha[8][2];
        rs_hin_read(ha, (const SSD_LDS uint4*)(S + rsl::kH), hf_o, l32_o);

        // the head's cs/dt reads all at once: the tile factors' (tf[0]: t0,
        // tf[1]: t1) and those of the rf rows of the wave's 9 slots,
        // rfw[s][j] = exp2(cref_t - cs_j) dt_j (row entries e = lane + 64 q)
        float cref[2], ctail[2], csi[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int i0 = 32 * it_[q];
            cref[q] = css[i0];
            ctail[q] = css[i0 + 31];
            csi[q] = css[i0 + l32_o];
        }
        float rft[5], rfc[5], rfd[5];
#pragma unroll
        for (int q = 0; q < 5; ++q) {
            const int e = min(lane_o + 64 * q, 287);
            const int s = e >> 5, j = e & 31;
            const bool first = s < 8 - wave;
            const int t = first ? t1 : t0;
            const int jt = first ? s : s - (8 - wave);
            rft[q] = css[32 * t];
            rfc[q] = css[32 * jt + j];
            rfd[q] = dts[32 * jt + j];
        }
        TileF tf[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            tf[q].fact = uniform_f(cref[q] - ctail[q]) <= kMaxTileDecayLog2;
            if (tf[q].fact) {
                tf[q].colf = fast_exp2(csi[q] - cref[q]);
                tf[q].sstate = fast_exp2(cref[q]);
                tf[q].dprime = Dh * fast_exp2(cref[q] - csi[q]);
            } else {
                tf[q].colf = 1.0f;
                tf[q].sstate = fast_exp2(csi[q]);
                tf[q].dprime = 0.0f;
            }
        }
        SSD_LDS float* rfo = lds(&rfw[wave][0]);
#pragma unroll
        for (int q = 0; q < 5; ++q) {
            const int e = lane_o + 64 * q;
            if (q < 4 || e < 288) rfo[e] = fast_exp2(fminf(rft[q] - rfc[q], kMaxTileDecayLog2)) * rfd[q];
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

        const __amdgpu_buffer_rsrc_t yrs = __builtin_amdgcn_make_buffer_rsrc(
            y + (((int64_t)b * L + tok0) * H + h) * P, (short)0, xrecord, 0x00020000);
        f32x16 acc[2][2];
        rs_state_terms(acc, ha, cf, tf);
        // slot s's LDS operands are read while slot s - 1 computes
        auto slot_jt = [&](int s) { return s < 8 - wave ? s : s - (8 - wave); };
        SlotRf rc, rn;
        SlotX xc, xn;
        rs_fetch_rf(rc, rfo, hf_o);
        rs_fetch_x(xc, S + rsl::kX + slot_jt(0) * 4096, xa);
#pragma unroll
        for (int s = 0; s < 9; ++s) {
            if (s + 1 < 9) {
                rs_fetch_rf(rn, rfo + 32 * (s + 1), hf_o);
                rs_fetch_x(xn, S + rsl::kX + slot_jt(s + 1) * 4096, xa);
            }
            __builtin_amdgcn_sched_barrier(0);
            const int jt = slot_jt(s);
            const bool first = s < 8 - wave;
            const bool dgb = first ? (s == 7 - wave) : (s == 8);
            u32x4v gq[2];
            rs_weights_fact(gq, gt[s], rc, dgb, first ? tf[1].dprime : tf[0].dprime);
            if (!(first ? tf[1].fact : tf[0].fact))
                rs_weights_direct(gq, gt[s], css + 32 * jt, dts + 32 * jt, first ? csi[1] : csi[0], Dh,
                                  dgb, hf_o, l32_o);
            if (first) {
                rs_products(acc[1], xc, gq);
                if (s == 7 - wave) rs_store(acc[1], tf[1].colf, yrs, rowbytes, t1, hf_o, l32_o);
            } else {
                rs_products(acc[0], xc, gq);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (s < 4) {
                issue_part(k + 2, so2, s);
                __builtin_amdgcn_sched_barrier(0);
            }
            rc = rn;
            xc = xn;
        }
        rs_store(acc[0], tf[0].colf, yrs, rowbytes, t0, hf_o, l32_o);
        so = so + rsl::kSlot == 3 * rsl::kSlot ? 0 : so + rsl::kSlot;
    }
    // the copies of the two heads past the end read empty records; nothing
    // in flight may outlive the workgroup's LDS
    wait_vmcnt<0>();
}

// ---------------------------------------------------------------------------
// Generic kernel: workgroup per (batch, chunk, head, 32-token i tile).
template <typename T, int MAXO>
__global__ __launch_bounds__(256) void chunk_scan_generic_kernel(
    const T* __restrict__ x, const T* __restrict__ Bm, const T* __restrict__ Cm,
    const float* __restrict__ cs, const float* __restrict__ dtc, const T* __restrict__ Hin,
    const float* __restrict__ D, T* __restrict__ y, int L, int H, int P, int N, int G, int Q,
    int nc) {
    extern __shared__ float smem[];
    float* ci = smem;              // [32][N]
    float* bj = ci + 32 * N;       // [32][N]
    float* xj = bj + 32 * N;       // [32][P]
    float* wm = xj + 32 * P;       // [32][33]
    float* csv = wm + 32 * 33;     // [Q]
    float* dtv = csv + Q;          // [Q]
    const int w = blockIdx.x;
    const int h = w % H;
    const int bc = w / H;
    const int c = bc % nc, b = bc / nc;
    const int g = h / (H / G);
    const int i0 = blockIdx.y * 32;
    const int tid = threadIdx.x;
    const int64_t row = (((int64_t)b * H + h) * nc + c) * Q;
    const int tok0 = c * Q;
    const float Dh = D ? D[h] : 0.0f;

    for (int e = tid; e < Q; e += 256) {
        csv[e] = cs[row + e];
        dtv[e] = dtc[row + e];
    }
    for (int e = tid; e < 32 * N; e += 256) {
        const int ii = e / N, n = e - ii * N;
        const int tok = tok0 + i0 + ii;
        ci[e] = (i0 + ii < Q && tok < L) ? Elem<T>::load(Cm, (((int64_t)b * L + tok) * G + g) * N + n) : 0.0f;
    }
    __syncthreads();

    // (ii) carried state
    const T* hrow = Hin + (((int64_t)b * H + h) * nc + c) * (int64_t)(P * N);
    float acc[MAXO];
#pragma unroll
    for (int k = 0; k < MAXO; ++k) {
        const int o = tid + 256 * k;   // o = ii * P + p
        acc[k] = 0.0f;
        if (o < 32 * P) {
            const int ii = o / P, p = o - ii * P;
            if (i0 + ii < Q) {
                float s = 0.0f;
                for (int n = 0; n < N; ++n) s += ci[ii * N + n] * Elem<T>::load(hrow, (int64_t)p * N + n);
                acc[k] = s * fast_exp2(csv[i0 + ii]);
            }
        }
    }

    // (i) + (iii)
    for (int j0 = 0; j0 <= i0; j0 += 32) {
        __syncthreads();
        for (int e = tid; e < 32 * N; e += 256) {
            const int jj = e / N, n = e - jj * N;
            const int tok = tok0 + j0 + jj;
            bj[e] = (j0 + jj < Q && tok < L) ? Elem<T>::load(Bm, (((int64_t)b * L + tok) * G + g) * N + n) : 0.0f;
        }
        for (int e = tid; e < 32 * P; e += 256) {
            const int jj = e / P, p = e - jj * P;
            const int tok = tok0 + j0 + jj;
            xj[e] = (j0 + jj < Q && tok < L) ? Elem<T>::load(x, (((int64_t)b * L + tok) * H + h) * P + p) : 0.0f;
        }
        __syncthreads();
        for (int e = tid; e < 32 * 32; e += 256) {
            const int ii = e >> 5, jj = e & 31;
            const int i = i0 + ii, j = j0 + jj;
            float v = 0.0f;
            if (j <= i && i < Q) {
                float s = 0.0f;
                for (int n = 0; n < N; ++n) s += ci[ii * N + n] * bj[jj * N + n];
                v = s * fast_exp2(csv[i] - csv[j]) * dtv[j];
                if (i == j) v += Dh;
            }
            wm[ii * 33 + jj] = v;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < MAXO; ++k) {
            const int o = tid + 256 * k;
            if (o < 32 * P) {
                const int ii = o / P, p = o - ii * P;
                float s = acc[k];
                for (int jj = 0; jj < 32; ++jj) s += wm[ii * 33 + jj] * xj[jj * P + p];
                acc[k] = s;
            }
        }
    }
#pragma unroll
    for (int k = 0; k < MAXO; ++k) {
        const int o = tid + 256 * k;
        if (o < 32 * P) {
            const int ii = o / P, p = o - ii * P;
            const int tok = tok0 + i0 + ii;
            if (i0 + ii < Q && tok < L) Elem<T>::store(y, (((int64_t)b * L + tok) * H + h) * P + p, acc[k]);
        }
    }
}

template <typename T, int MAXO>
static void launch_generic(const Dims& d, const void* x, const void* B, const void* C,
                           const float* cs, const float* dtc, const void* Hin, const float* D,
                           void* y, hipStream_t stream) {
    const size_t shmem = sizeof(float) * (64 * d.dstate + 32 * d.headdim + 32 * 33 + 2 * d.chunk);
    dim3 grid((unsigned)(d.batch * d.nchunks * d.nheads), (unsigned)((d.chunk + 31) / 32));
    chunk_scan_generic_kernel<T, MAXO><<<grid, 256, shmem, stream>>>(
        static_cast<const T*>(x), static_cast<const T*>(B), static_cast<const T*>(C), cs, dtc,
        static_cast<const T*>(Hin), D, static_cast<T*>(y), (int)d.seqlen, (int)d.nheads,
        (int)d.headdim, (int)d.dstate, (int)d.ngroups, (int)d.chunk, (int)d.nchunks);
}

template <typename T>
static void launch_generic_t(const Dims& d, const void* x, const void* B, const void* C,
                             const float* cs, const float* dtc, const void* Hin, const float* D,
                             void* y, hipStream_t stream) {
    const int64_t per = (32 * d.headdim + 255) / 256;
    if (per <= 1) launch_generic<T, 1>(d, x, B, C, cs, dtc, Hin, D, y, stream);
    else if (per <= 2) launch_generic<T, 2>(d, x, B, C, cs, dtc, Hin, D, y, stream);
    else if (per <= 4) launch_generic<T, 4>(d, x, B, C, cs, dtc, Hin, D, y, stream);
    else if (per <= 8) launch_generic<T, 8>(d, x, B, C, cs, dtc, Hin, D, y, stream);
    else if (per <= 16) launch_generic<T, 16>(d, x, B, C, cs, dtc, Hin, D, y, stream);
    else launch_generic<T, 32>(d, x, B, C, cs, dtc, Hin, D, y, stream);
}

// Heads per workgroup of the matrix-core kernel: a divisor of the heads per
// group (they share C) chosen so that the grid fills whole rounds of the
// machine (two workgroups per CU), with a small charge per workgroup for
// its start-up copies.
static int scan_heads_per_workgroup(const Dims& d) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    }
    const double slots = 2.0 * cus;
    const int64_t hpg = d.nheads / d.ngroups;
    const double items = (double)d.batch * (double)d.nchunks * (double)d.nheads;
    int best = 1;
    double best_cost = 1e300;
    for (int64_t hg = 1; hg <= hpg && hg <= 64; ++hg) {
        if (hpg % hg) continue;
        const double rounds = std::ceil(items / (double)hg / slots);
        const double cost = rounds * ((double)hg + 0.5);
        if (cost < best_cost - 1e-9) { best_cost = cost; best = (int)hg; }
    }
    return best;
}

// Shortest run of heads for which the resident kernel beats the streaming
// one (measured on the MI355X: 40-head runs gain, 4- and 6-head runs lose).
constexpr int kResidentMinHeads = 12;

// Heads per workgroup of the resident kernel (one workgroup per CU): a run
// of hg heads of one group, the group's heads split into nsplit runs, with
// a start-up charge (the resident tiles, the first copies) of 1.5 heads.
static void scan_resident_split(const Dims& d, int* hg_out, int* nsplit_out) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    }
    const int64_t hpg = d.nheads / d.ngroups;
    const double units = (double)d.batch * (double)d.nchunks * (double)d.ngroups;
    int best = (int)hpg;
    double best_cost = 1e300;
    for (int64_t hg = 1; hg <= hpg; ++hg) {
        const int64_t ns = (hpg + hg - 1) / hg;
        const double rounds = std::ceil(units * (double)ns / (double)cus);
        const double cost = rounds * ((double)hg + 1.5);
        if (cost < best_cost - 1e-9) { best_cost = cost; best = (int)hg; }
    }
    *hg_out = best;
    *nsplit_out = (int)((hpg + best - 1) / best);
}

hipError_t launch_chunk_scan(const Dims& d, int32_t dtype, const void* x, const void* B,
                             const void* C, const float* cs, const float* dtc, const void* Hin,
                             const float* D, void* y, hipStream_t stream) {
    if (mfma_path(dtype, d)) {
        const bf16_t* xb = static_cast<const bf16_t*>(x);
        const bf16_t* bb = static_cast<const bf16_t*>(B);
        const bf16_t* cb = static_cast<const bf16_t*>(C);
        const bf16_t* hb = static_cast<const bf16_t*>(Hin);
        bf16_t* yb = static_cast<bf16_t*>(y);
        const int L = (int)d.seqlen, H = (int)d.nheads, G = (int)d.ngroups, nc = (int)d.nchunks;
        if (d.chunk == 256) {
            // the resident kernel pays for its start-up (9 tiles' products
            // and a pipeline fill) once per run of heads: worth it for long
            // runs only
            int hg = 0, nsplit = 0;
            scan_resident_split(d, &hg, &nsplit);
            if (hg >= kResidentMinHeads) {
                const unsigned blocks = (unsigned)(d.batch * nc * G * nsplit);
                chunk_scan_resident_kernel<<<blocks, 256, 0, stream>>>(xb, bb, cb, cs, dtc, hb, D, yb, L, H, G, nc, hg, nsplit);
                return hipGetLastError();
            }
        }
        const int hg = scan_heads_per_workgroup(d);
        const unsigned blocks = (unsigned)(d.batch * nc * (d.nheads / hg));
        switch (d.chunk) {
            case 128: chunk_scan_mfma_kernel<128><<<blocks, 128, 0, stream>>>(xb, bb, cb, cs, dtc, hb, D, yb, L, H, G, nc, hg); break;
            default: chunk_scan_mfma_kernel<256><<<blocks, 256, 0, stream>>>(xb, bb, cb, cs, dtc, hb, D, yb, L, H, G, nc, hg); break;
        }
    } else if (dtype == 1) {
        launch_generic_t<bf16_t>(d, x, B, C, cs, dtc, Hin, D, y, stream);
    } else {
        launch_generic_t<float>(d, x, B, C, cs, dtc, Hin, D, y, stream);
    }
    return hipGetLastError();
}

}  // namespace ssd
