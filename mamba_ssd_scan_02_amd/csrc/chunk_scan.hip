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
//   * G~ = G * exp2(cs_i - cs_j) * dt_j for j <= i, 0 above the diagonal, + D
//     on the diagonal (term iii), rounded to bf16.
//   * Y^T += X^T G~^T (M = P rows in two 32-row tiles, K = 32 tokens).  A-row m
//     reads channel sigma(m) so that a lane ends with 16 consecutive channels
//     of its token: two 16-byte stores per tile.
//   * Term (ii) first: Y^T = Hin C^T (K = N), then each column scaled by
//     exp2(cs_i).
// Wave w owns i tiles {w, 2W-1-w} so that every wave has the same number of
// causal (j <= i) tiles.  C fragments of the wave's own tokens stay in
// registers for the whole kernel; the j blocks of B (32 rows) and X^T (64 x 32)
// stream through a 12 KB LDS window.
//
// Generic kernel (fp32 or bf16, any P, N within limits): the same three terms
// in fp32 on the vector units, 32 x 32 tiles in LDS.
#include "device_common.h"
#include "launchers.h"

namespace ssd {

__device__ __forceinline__ void transpose8x8_bf16_scan(const uint4 (&in)[8], uint4 (&out)[8]) {
    uint32_t w[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        w[i][0] = in[i].x; w[i][1] = in[i].y; w[i][2] = in[i].z; w[i][3] = in[i].w;
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int m = q >> 1;
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t lo = w[2 * k][m], hi = w[2 * k + 1][m];
            o[k] = (q & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        out[q] = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

// Row m = 8a + 4hf + b of a 32-row MFMA tile.
__device__ __forceinline__ int perm_pi(int m) {
    const int a = m >> 3, hf = (m >> 2) & 1, b = m & 3;
    return 16 * (a >> 1) + 8 * hf + 4 * (a & 1) + b;
}
__device__ __forceinline__ int perm_sigma(int m) {
    const int a = m >> 3, hf = (m >> 2) & 1, b = m & 3;
    return 16 * hf + 4 * a + b;
}

template <int Q>
__global__ __launch_bounds__(Q) void chunk_scan_mfma_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ Bm, const bf16_t* __restrict__ Cm,
    const float* __restrict__ cs, const float* __restrict__ dtc, const bf16_t* __restrict__ Hin,
    const float* __restrict__ D, bf16_t* __restrict__ y, int L, int H, int G, int nc) {
    constexpr int P = 64, N = 128, W = Q / 64, NT = Q / 32;
    __shared__ float cs_s[Q];
    __shared__ float dt_s[Q];
    __shared__ uint4 win[1024];          // 16 KB: Hin [64][16] or B block [32][16] + X^T [64][4]
    uint4* hs = win;
    uint4* bsm = win;
    uint4* xsm = win + 512;

    const uint32_t wg = xcd_logical_id(blockIdx.x, gridDim.x);
    const int h = (int)(wg % (uint32_t)H);
    const int bc = (int)(wg / (uint32_t)H);
    const int c = bc % nc, b = bc / nc;
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hf = lane >> 5, l32 = lane & 31;
    const int64_t row = (((int64_t)b * H + h) * nc + c) * Q;
    const int tok0 = c * Q;
    const float Dh = D ? D[h] : 0.0f;

    for (int e = tid; e < Q; e += Q) {
        cs_s[e] = cs[row + e];
        dt_s[e] = dtc[row + e];
    }
    const uint4* hsrc = reinterpret_cast<const uint4*>(Hin + (((int64_t)b * H + h) * nc + c) * (int64_t)(P * N));
    for (int e = tid; e < 1024; e += Q) {
        const int r = e >> 4, ch = e & 15;
        hs[r * 16 + (ch ^ (r & 7))] = hsrc[e];
    }

    const int it_[2] = {wave, 2 * W - 1 - wave};
    uint4 cf[2][8];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int tok = tok0 + 32 * it_[t] + l32;
        const bf16_t* crow = Cm + (((int64_t)b * L + tok) * G + g) * N + 8 * hf;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
            cf[t][kk] = (tok < L) ? *reinterpret_cast<const uint4*>(crow + 16 * kk) : make_uint4(0, 0, 0, 0);
    }
    __syncthreads();

    // (ii) carried state: Y^T[p][i] = sum_n Hin[p][n] C[i][n], scaled by exp2(cs_i)
    f32x16 acc[2][2];
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
            const bf16x8 a = __builtin_bit_cast(bf16x8, hs[pr * 16 + (ch ^ (pr & 7))]);
#pragma unroll
            for (int t = 0; t < 2; ++t)
                acc[t][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, cf[t][kk]), acc[t][mt], 0, 0, 0);
        }
    }
    float csi[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        csi[t] = cs_s[32 * it_[t] + l32];
        const float s = fast_exp2(csi[t]);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[t][mt][r] *= s;
    }

    // (i) + (iii): stream the j blocks
    for (int jt = 0; jt < NT; ++jt) {
        __syncthreads();
        for (int e = tid; e < 512; e += Q) {
            const int r = e >> 4, ch = e & 15;
            const int tok = tok0 + 32 * jt + r;
            bsm[r * 16 + (ch ^ (r & 7))] =
                (tok < L) ? *reinterpret_cast<const uint4*>(Bm + (((int64_t)b * L + tok) * G + g) * N + 8 * ch)
                          : make_uint4(0, 0, 0, 0);
        }
        if (tid < 32) {
            const int tg = tid >> 3, pb = tid & 7;
            uint4 rr[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int tok = tok0 + 32 * jt + 8 * tg + i;
                rr[i] = (tok < L) ? *reinterpret_cast<const uint4*>(x + (((int64_t)b * L + tok) * H + h) * P + 8 * pb)
                                  : make_uint4(0, 0, 0, 0);
            }
            uint4 o[8];
            transpose8x8_bf16_scan(rr, o);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int p = 8 * pb + q;
                xsm[p * 4 + (tg ^ ((p >> 1) & 3))] = o[q];
            }
        }
        __syncthreads();

        // B operand rows of this j block, shared by the wave's two i tiles
        bf16x8 bfr[8];
        {
            const int jr = perm_pi(l32);
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const int ch = 2 * kk + hf;
                bfr[kk] = __builtin_bit_cast(bf16x8, bsm[jr * 16 + (ch ^ (jr & 7))]);
            }
        }
        bf16x8 xfr[2][2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int pr = 32 * mt + perm_sigma(l32);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int blk = 2 * u + hf;
                xfr[mt][u] = __builtin_bit_cast(bf16x8, xsm[pr * 4 + (blk ^ ((pr >> 1) & 3))]);
            }
        }

#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int it = it_[t];
            if (it < jt) continue;
            f32x16 gacc = {};
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
                gacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[kk], __builtin_bit_cast(bf16x8, cf[t][kk]), gacc, 0, 0, 0);
            const int i = 32 * it + l32;
            uint32_t pk[8];
#pragma unroll
            for (int r2 = 0; r2 < 8; ++r2) {
                float v2[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int r = 2 * r2 + e;
                    const int j = 32 * jt + 16 * (r >> 3) + 8 * hf + (r & 7);
                    float v = 0.0f;
                    if (j <= i) v = gacc[r] * fast_exp2(csi[t] - cs_s[j]) * dt_s[j];
                    if (j == i) v += Dh;
                    v2[e] = v;
                }
                pk[r2] = pack_bf16x2(v2[0], v2[1]);
            }
            const bf16x8 g0 = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
            const bf16x8 g1 = __builtin_bit_cast(bf16x8, make_uint4(pk[4], pk[5], pk[6], pk[7]));
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                acc[t][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xfr[mt][0], g0, acc[t][mt], 0, 0, 0);
                acc[t][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xfr[mt][1], g1, acc[t][mt], 0, 0, 0);
            }
        }
    }

    // write y: lane owns token i, channels 32*mt + 16*hf + 0..15
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int tok = tok0 + 32 * it_[t] + l32;
        if (tok >= L) continue;
        bf16_t* yrow = y + (((int64_t)b * L + tok) * H + h) * P;
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
        const unsigned blocks = (unsigned)(d.batch * d.nchunks * d.nheads);
        const bf16_t* xb = static_cast<const bf16_t*>(x);
        const bf16_t* bb = static_cast<const bf16_t*>(B);
        const bf16_t* cb = static_cast<const bf16_t*>(C);
        const bf16_t* hb = static_cast<const bf16_t*>(Hin);
        bf16_t* yb = static_cast<bf16_t*>(y);
        const int L = (int)d.seqlen, H = (int)d.nheads, G = (int)d.ngroups, nc = (int)d.nchunks;
        switch (d.chunk) {
            case 64: chunk_scan_mfma_kernel<64><<<blocks, 64, 0, stream>>>(xb, bb, cb, cs, dtc, hb, D, yb, L, H, G, nc); break;
            case 128: chunk_scan_mfma_kernel<128><<<blocks, 128, 0, stream>>>(xb, bb, cb, cs, dtc, hb, D, yb, L, H, G, nc); break;
            default: chunk_scan_mfma_kernel<256><<<blocks, 256, 0, stream>>>(xb, bb, cb, cs, dtc, hb, D, yb, L, H, G, nc); break;
        }
    } else if (dtype == 1) {
        launch_generic_t<bf16_t>(d, x, B, C, cs, dtc, Hin, D, y, stream);
    } else {
        launch_generic_t<float>(d, x, B, C, cs, dtc, Hin, D, y, stream);
    }
    return hipGetLastError();
}

}  // namespace ssd
