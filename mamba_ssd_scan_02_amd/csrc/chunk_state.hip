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
// (tokens) contiguous per lane, so every 8 x 8 block of (tokens x columns) is
// loaded as eight 16-byte rows, transposed in registers and written to LDS
// with one 16-byte store per column.  LDS rows are 64 tokens (128 B); the
// 16-byte block index is XOR-swizzled with (row ^ row/8) & 7 so that both
// the transposing stores and the operand loads touch 8 distinct block
// columns.  w_j x_j is formed in fp32 and rounded once to bf16.
//
// Generic kernel (fp32 or bf16, any P, N within limits): tiles of 32 tokens in
// LDS, fp32 FMA on the vector units.
#include "device_common.h"
#include "launchers.h"

namespace ssd {

// ---------------------------------------------------------------------------
// Register transpose of an 8 x 8 block of bf16.
// in[i]  : 8 values of row i (token i), word m holds columns 2m (lo), 2m+1 (hi)
// out[q] : 8 values of column q, word k holds tokens 2k (lo), 2k+1 (hi)
__device__ __forceinline__ void transpose8x8_bf16(const uint4 (&in)[8], uint4 (&out)[8]) {
    uint32_t w[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        w[i][0] = in[i].x; w[i][1] = in[i].y; w[i][2] = in[i].z; w[i][3] = in[i].w;
    }
    uint32_t o[8][4];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int m = q >> 1;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t lo = w[2 * k][m], hi = w[2 * k + 1][m];
            o[q][k] = (q & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) out[q] = make_uint4(o[q][0], o[q][1], o[q][2], o[q][3]);
}

__device__ __forceinline__ int swz8(int row) { return (row ^ (row >> 3)) & 7; }

// Scale the 8 bf16 of one word-quad by w in fp32 and round back to bf16.
__device__ __forceinline__ uint4 scale_bf16x8(uint4 v, float w) {
    uint32_t in[4] = {v.x, v.y, v.z, v.w};
    uint32_t out[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const float lo = bf16_bits_to_f32(in[m] & 0xffffu) * w;
        const float hi = bf16_bits_to_f32(in[m] >> 16) * w;
        out[m] = pack_bf16x2(lo, hi);
    }
    return make_uint4(out[0], out[1], out[2], out[3]);
}

template <int Q>
__global__ __launch_bounds__(256) void chunk_state_mfma_kernel(const bf16_t* __restrict__ x,
                                                               const bf16_t* __restrict__ Bm,
                                                               const float* __restrict__ cs,
                                                               const float* __restrict__ dtc,
                                                               float* __restrict__ S, int L, int H,
                                                               int G, int nc) {
    constexpr int P = 64, N = 128, KB = 64;
    __shared__ uint4 xs[P * (KB / 8)];   // [p][token block], 8 KB
    __shared__ uint4 bs[N * (KB / 8)];   // [n][token block], 16 KB
    __shared__ float wv[KB];

    const uint32_t wg = xcd_logical_id(blockIdx.x, gridDim.x);
    const int h = (int)(wg % (uint32_t)H);
    const int bc = (int)(wg / (uint32_t)H);
    const int c = bc % nc, b = bc / nc;
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t row = (((int64_t)b * H + h) * nc + c) * Q;
    const float cl = cs[row + Q - 1];

    f32x16 acc0 = {}, acc1 = {};

    for (int kb = 0; kb < Q / KB; ++kb) {
        const int tb = c * Q + kb * KB;
        if (tid < KB) {
            const int j = kb * KB + tid;
            wv[tid] = fast_exp2(cl - cs[row + j]) * dtc[row + j];
        }
        __syncthreads();
        if (tid < 64) {
            // x task: tokens 8*tg .. +7, columns 8*pb .. +7
            const int tg = tid >> 3, pb = tid & 7;
            uint4 r[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int t = tb + 8 * tg + i;
                r[i] = (t < L) ? *reinterpret_cast<const uint4*>(x + (((int64_t)b * L + t) * H + h) * P + 8 * pb)
                               : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) r[i] = scale_bf16x8(r[i], wv[8 * tg + i]);
            uint4 o[8];
            transpose8x8_bf16(r, o);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int p = 8 * pb + q;
                xs[p * 8 + (tg ^ swz8(p))] = o[q];
            }
        } else if (tid < 192) {
            // B task: tokens 8*tg .. +7, columns 8*nb .. +7
            const int u = tid - 64;
            const int nb = u & 15, tg = u >> 4;
            uint4 r[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int t = tb + 8 * tg + i;
                r[i] = (t < L) ? *reinterpret_cast<const uint4*>(Bm + (((int64_t)b * L + t) * G + g) * N + 8 * nb)
                               : make_uint4(0, 0, 0, 0);
            }
            uint4 o[8];
            transpose8x8_bf16(r, o);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int n = 8 * nb + q;
                bs[n * 8 + (tg ^ swz8(n))] = o[q];
            }
        }
        __syncthreads();
        const int pr0 = lane & 31, pr1 = 32 + (lane & 31), nr = 32 * wave + (lane & 31);
#pragma unroll
        for (int kk = 0; kk < KB / 16; ++kk) {
            const int blk = 2 * kk + (lane >> 5);
            const bf16x8 a0 = __builtin_bit_cast(bf16x8, xs[pr0 * 8 + (blk ^ swz8(pr0))]);
            const bf16x8 a1 = __builtin_bit_cast(bf16x8, xs[pr1 * 8 + (blk ^ swz8(pr1))]);
            const bf16x8 bb = __builtin_bit_cast(bf16x8, bs[nr * 8 + (blk ^ swz8(nr))]);
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bb, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bb, acc1, 0, 0, 0);
        }
    }

    float* Sp = S + (((int64_t)b * H + h) * nc + c) * (int64_t)(P * N);
    const int n = 32 * wave + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int p = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        Sp[p * N + n] = acc0[r];
        Sp[(32 + p) * N + n] = acc1[r];
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
    return dtype == 1 && d.headdim == 64 && d.dstate == 128 &&
           (d.chunk == 64 || d.chunk == 128 || d.chunk == 256);
}

bool generic_path(const Dims& d) {
    return d.headdim >= 1 && d.headdim <= 128 && d.dstate >= 1 && d.dstate <= 128 &&
           d.chunk >= 1 && d.chunk <= 256;
}

hipError_t launch_chunk_state(const Dims& d, int32_t dtype, const void* x, const void* B,
                              const float* cs, const float* dtc, float* S, hipStream_t stream) {
    if (mfma_path(dtype, d)) {
        const unsigned blocks = (unsigned)(d.batch * d.nchunks * d.nheads);
        const bf16_t* xb = static_cast<const bf16_t*>(x);
        const bf16_t* bb = static_cast<const bf16_t*>(B);
        const int L = (int)d.seqlen, H = (int)d.nheads, G = (int)d.ngroups, nc = (int)d.nchunks;
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
