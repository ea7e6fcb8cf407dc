// chunk_cumsum.hip -- per-chunk inclusive prefix of dt * A_h (scaled by
// log2 e), plus dt rearranged head-major.
//
// The decay between two tokens is the product of the per-token factors
// exp(dt_t A_h) (the fading weights 1, 1/2, 1/4 ... of the water-tank example,
// page "State Space Model", section "Un sistema che riassume il passato"), so
// inside a chunk every such product is exp of a difference of this prefix.
// Storing log2(e) * prefix lets consumers use the hardware exp2 directly.
//
// One workgroup (4 waves) per (batch, chunk, 32-head slice).  The [Q x 32]
// slab of dt is read coalesced along heads into LDS; each wave then scans
// one head's Q values (up to 4 per lane, wave-level prefix by shuffles) with
// fp64 accumulation, rounding once to fp32 on the store.
#include "device_common.h"
#include "launchers.h"

namespace ssd {

constexpr int kCsHeads = 32;

__global__ __launch_bounds__(256) void chunk_cumsum_kernel(const float* __restrict__ dt,
                                                           const float* __restrict__ A,
                                                           float* __restrict__ cs,
                                                           float* __restrict__ dtc, int L,
                                                           int H, int Q, int nc) {
    __shared__ float tile[256][kCsHeads + 1];
    const int b = blockIdx.x / nc;
    const int c = blockIdx.x % nc;
    const int h0 = blockIdx.y * kCsHeads;
    const int nh = min(kCsHeads, H - h0);
    const int t0 = c * Q;
    const int nt = min(Q, L - t0);

    for (int e = threadIdx.x; e < Q * nh; e += blockDim.x) {
        const int j = e / nh, hh = e % nh;
        tile[j][hh] = (j < nt) ? dt[((int64_t)b * L + t0 + j) * H + h0 + hh] : 0.0f;
    }
    __syncthreads();

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int epl = (Q + 63) >> 6;  // values per lane, <= 4
    for (int hh = wave; hh < nh; hh += 4) {
        const int h = h0 + hh;
        const double a = (double)A[h] * 1.4426950408889634074;
        double pre[4];
        double run = 0.0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int j = lane * epl + k;
            const double v = (k < epl && j < Q) ? (double)tile[j][hh] * a : 0.0;
            run += v;
            pre[k] = run;
        }
        double incl = run;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const double o = __shfl_up(incl, off, 64);
            if (lane >= off) incl += o;
        }
        const double excl = incl - run;
        float* csr = cs + (((int64_t)b * H + h) * nc + c) * Q;
        float* dtr = dtc + (((int64_t)b * H + h) * nc + c) * Q;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int j = lane * epl + k;
            if (k < epl && j < Q) {
                csr[j] = (float)(excl + pre[k]);
                dtr[j] = tile[j][hh];
            }
        }
    }
}

hipError_t launch_chunk_cumsum(const Dims& d, const float* dt, const float* A, float* cs,
                               float* dtc, hipStream_t stream) {
    dim3 grid((unsigned)(d.batch * d.nchunks), (unsigned)((d.nheads + kCsHeads - 1) / kCsHeads));
    chunk_cumsum_kernel<<<grid, 256, 0, stream>>>(dt, A, cs, dtc, (int)d.seqlen, (int)d.nheads,
                                                  (int)d.chunk, (int)d.nchunks);
    return hipGetLastError();
}

}  // namespace ssd
