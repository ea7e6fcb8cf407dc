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

// Largest decay inside one 32-token block (log2 units) for which the
// factorised weights are used; beyond it the row factor exp2(c0 - cs_j)
// could overflow, and the direct form is taken.
constexpr float kMaxBlockDecayLog2 = 64.0f;

__device__ __forceinline__ float uniform_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

// Causal keep bits of the diagonal block for this lane.  Accumulator
// register r of lane (l32, hf) holds token j = 16*(r/8) + 8*hf + r%8 of the
// block and column i = l32: with t = l32 - 8*hf, registers r < 8 are kept
// iff r <= t and registers r >= 8 iff r - 8 <= t - 16.
__device__ __forceinline__ uint32_t diag_keep_bits(int l32, int hf) {
    const int t = l32 - 8 * hf;
    const int n0 = min(max(t + 1, 0), 8), n1 = min(max(t - 15, 0), 8);
    return ((1u << n0) - 1u) | (((1u << n1) - 1u) << 8);
}

// Bit r set iff accumulator register r of this lane is the diagonal entry
// j == i of the diagonal block (at most one per lane).
__device__ __forceinline__ uint32_t diag_eq_bits(int l32, int hf) {
    const int t = l32 - 8 * hf;
    if (t >= 0 && t < 8) return 1u << t;
    if (t >= 16 && t < 24) return 1u << (t - 8);
    return 0u;
}

// C fragments of the wave's own tokens (B operand of both C products).
__device__ __forceinline__ void load_c_frags(uint4 (&cf)[2][8], const bf16_t* Cm, int64_t b, int L,
                                             int G, int g, int tok0, const int (&it_)[2], int hf,
                                             int l32) {
    constexpr int N = 128;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int tok = tok0 + 32 * it_[t] + l32;
        const bf16_t* crow = Cm + ((b * L + tok) * G + g) * N + 8 * hf;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
            cf[t][kk] = (tok < L) ? *reinterpret_cast<const uint4*>(crow + 16 * kk) : make_uint4(0, 0, 0, 0);
    }
}

// (ii) carried state: acc[t][mt] = exp2(cs_i) * sum_n Hin[p][n] C[i][n].
__device__ __forceinline__ void scan_state_term(f32x16 (&acc)[2][2], const uint4* hs,
                                                const uint4 (&cf)[2][8], const float (&csi)[2],
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
    for (int t = 0; t < 2; ++t) {
        const float s = fast_exp2(csi[t]);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[t][mt][r] *= s;
    }
}

// (i) + (iii) for j block jt: G^T tiles from the B block, masked decay
// weights (+ D on the diagonal), then Y^T += X^T G~^T.
__device__ __forceinline__ void scan_block(f32x16 (&acc)[2][2], int jt, const uint4* bst,
                                           const uint4* xst, const float* cs_s, const float* dt_s,
                                           const float* rf_s, const uint4 (&cf)[2][8],
                                           const float (&csi)[2], const int (&it_)[2], float Dh,
                                           XtAddr xa, int hf, int l32, uint32_t diag_keep,
                                           uint32_t diag_eq) {
    if (it_[1] < jt) return;   // it_[1] >= it_[0]: nothing left for this wave
    const bool act0 = it_[0] >= jt;
    f32x16 gacc[2] = {f32x16{}, f32x16{}};
    {
        const int jr = perm_pi(l32);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const int ch = 2 * kk + hf;
            const bf16x8 bq = __builtin_bit_cast(bf16x8, bst[jr * 16 + (ch ^ swz_b(jr))]);
            if (act0)
                gacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bq, __builtin_bit_cast(bf16x8, cf[0][kk]), gacc[0], 0, 0, 0);
            gacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bq, __builtin_bit_cast(bf16x8, cf[1][kk]), gacc[1], 0, 0, 0);
        }
    }
    const SSD_LDS char* xb = (const SSD_LDS char*)lds(xst);
    const float* csb = cs_s + 32 * jt + 8 * hf;
    const float* dtb = dt_s + 32 * jt + 8 * hf;
    const float* rfb = rf_s + 32 * jt + 8 * hf;
    // factorised weights exp2(cs_i - c0) * [exp2(c0 - cs_j) dt_j] for blocks
    // below the diagonal whose own decay stays under 2^64 (c0 = cs of the
    // block's first token; the row factors rf_s are precomputed per block)
    const float c0 = cs_s[32 * jt];
    const bool fact = uniform_f(c0 - cs_s[32 * jt + 31]) <= kMaxBlockDecayLog2;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        if (t == 0 && !act0) continue;
        uint32_t pk[8];
        const bool dgb = it_[t] == jt;
        if (!dgb && fact) {
            const float colf = fast_exp2(csi[t] - c0);
#pragma unroll
            for (int r2 = 0; r2 < 8; ++r2) {
                const int r = 2 * r2;
                const int jl = 16 * (r >> 3) + (r & 7);
                pk[r2] = pack_bf16x2(gacc[t][r] * (rfb[jl] * colf), gacc[t][r + 1] * (rfb[jl + 1] * colf));
            }
        } else {
            // diagonal block (causal keep bits, D on the diagonal) or a block
            // with too much decay for the factorisation: direct weights
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
// 32*mt + 16*hf + 0..15 (two 16-byte stores per tile).
__device__ __forceinline__ void scan_store_y(const f32x16 (&acc)[2][2], bf16_t* y, int64_t b, int L,
                                             int H, int h, int tok0, const int (&it_)[2], int hf,
                                             int l32, bool guard) {
    constexpr int P = 64;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int tok = tok0 + 32 * it_[t] + l32;
        if (guard && tok >= L) continue;
        bf16_t* yrow = y + ((b * L + tok) * H + h) * P;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            uint32_t w8[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) w8[k] = pack_bf16x2(acc[t][mt][2 * k], acc[t][mt][2 * k + 1]);
            uint4* dst = reinterpret_cast<uint4*>(yrow + 32 * mt + 16 * hf);
            dst[0] = make_uint4(w8[0], w8[1], w8[2], w8[3]);
            dst[1] = make_uint4(w8[4], w8[5], w8[6], w8[7]);
        }
    }
}

// ---------------------------------------------------------------------------
// One workgroup per (batch, chunk, head).
template <int Q>
__global__ __launch_bounds__(Q, 2) void chunk_scan_mfma_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ Bm, const bf16_t* __restrict__ Cm,
    const float* __restrict__ cs, const float* __restrict__ dtc, const bf16_t* __restrict__ Hin,
    const float* __restrict__ D, bf16_t* __restrict__ y, int L, int H, int G, int nc) {
    constexpr int P = 64, N = 128, W = Q / 64, NT = Q / 32;
    constexpr int DPS = 12 / W;   // LDS-copy instructions per wave per stage
    __shared__ uint4 hs[1024];                         // Hin, 64 rows x 256 B
    __shared__ uint4 bs0[512], bs1[512], bs2[512];     // B stages, 32 rows x 256 B
    __shared__ uint4 xs0[256], xs1[256], xs2[256];     // x stages, 32 rows x 128 B
    __shared__ float cs_s[Q];
    __shared__ float dt_s[Q];
    __shared__ float rf_s[Q];

    const uint32_t wg = xcd_logical_id(blockIdx.x, gridDim.x);
    const int h = (int)(wg % (uint32_t)H);
    const int bc = (int)(wg / (uint32_t)H);
    const int c = bc % nc, b = bc / nc;
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hf = lane >> 5, l32 = lane & 31;
    const int64_t bh = (int64_t)b * H + h;
    const int64_t row = (bh * nc + c) * Q;
    const int tok0 = c * Q;
    const float Dh = D ? D[h] : 0.0f;
    const int64_t xstride = (int64_t)H * P, bstride = (int64_t)G * N;
    const bf16_t* xbase = x + ((int64_t)b * L * H + h) * P;
    const bf16_t* bbase = Bm + ((int64_t)b * L * G + g) * N;

    // Ordinary loads are written to LDS / consumed before any LDS copy is
    // issued: the compiler waits for vmcnt(0) on such uses once a copy is in
    // flight.
    {
        const float cv = cs[row + tid], dv = dtc[row + tid];
        cs_s[tid] = cv;
        dt_s[tid] = dv;
        // row factor of token tid within its 32-token block (see scan_block)
        rf_s[tid] = fast_exp2(fminf(cs[row + (tid & ~31)] - cv, kMaxBlockDecayLog2)) * dv;
    }
    const int it_[2] = {wave, 2 * W - 1 - wave};
    uint4 cf[2][8];
    load_c_frags(cf, Cm, b, L, G, g, tok0, it_, hf, l32);
    float csi[2];
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    {
        const bf16_t* hsrc = Hin + (bh * nc + c) * (int64_t)(P * N);
#pragma unroll
        for (int i = 0; i < 16 / W; ++i) {
            const int k = wave + i * W;
            const int r = 4 * k + (lane >> 4);
            const int cc = (lane & 15) ^ swz_h(r);
            dma16(hsrc + r * N + 8 * cc, lds(hs) + k * 64);
        }
    }
    issue_bx_stage<W>(wave, lane, tok0, L, xbase, xstride, bbase, bstride, bs0, xs0);
    if (NT > 1) issue_bx_stage<W>(wave, lane, tok0 + 32, L, xbase, xstride, bbase, bstride, bs1, xs1);

    if (NT > 1) wait_vmcnt<2 * DPS>(); else wait_vmcnt<DPS>();
    barrier_lds();
    csi[0] = cs_s[32 * it_[0] + l32];
    csi[1] = cs_s[32 * it_[1] + l32];
    f32x16 acc[2][2];
    scan_state_term(acc, hs, cf, csi, hf, l32);
    const XtAddr xa = xt_addr(lane);
    const uint32_t dkeep = diag_keep_bits(l32, hf);
    const uint32_t deq = diag_eq_bits(l32, hf);

#pragma unroll
    for (int jt = 0; jt < NT; ++jt) {
        uint4* bst = (jt % 3 == 0) ? bs0 : ((jt % 3 == 1) ? bs1 : bs2);
        uint4* xst = (jt % 3 == 0) ? xs0 : ((jt % 3 == 1) ? xs1 : xs2);
        if (jt + 1 < NT) wait_vmcnt<DPS>(); else wait_vmcnt<0>();
        barrier_lds();
        if (jt + 2 < NT) {
            uint4* nb = ((jt + 2) % 3 == 0) ? bs0 : (((jt + 2) % 3 == 1) ? bs1 : bs2);
            uint4* nx = ((jt + 2) % 3 == 0) ? xs0 : (((jt + 2) % 3 == 1) ? xs1 : xs2);
            issue_bx_stage<W>(wave, lane, tok0 + 32 * (jt + 2), L, xbase, xstride, bbase, bstride, nb, nx);
        }
        scan_block(acc, jt, bst, xst, cs_s, dt_s, rf_s, cf, csi, it_, Dh, xa, hf, l32, dkeep, deq);
    }
    scan_store_y(acc, y, b, L, H, h, tok0, it_, hf, l32, true);
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
        {
            const unsigned blocks = (unsigned)(d.batch * nc * d.nheads);
            switch (d.chunk) {
                case 64: chunk_scan_mfma_kernel<64><<<blocks, 64, 0, stream>>>(xb, bb, cb, cs, dtc, hb, D, yb, L, H, G, nc); break;
                case 128: chunk_scan_mfma_kernel<128><<<blocks, 128, 0, stream>>>(xb, bb, cb, cs, dtc, hb, D, yb, L, H, G, nc); break;
                default: chunk_scan_mfma_kernel<256><<<blocks, 256, 0, stream>>>(xb, bb, cb, cs, dtc, hb, D, yb, L, H, G, nc); break;
            }
        }
    } else if (dtype == 1) {
        launch_generic_t<bf16_t>(d, x, B, C, cs, dtc, Hin, D, y, stream);
    } else {
        launch_generic_t<float>(d, x, B, C, cs, dtc, Hin, D, y, stream);
    }
    return hipGetLastError();
}

}  // namespace ssd
