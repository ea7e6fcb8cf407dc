// chunk_cumsum.hip -- per-chunk inclusive prefix of dt * A_h (scaled by
// log2 e), plus dt rearranged head-major.
//
// The decay between two tokens is the product of the per-token factors
// exp(dt_t A_h) (the fading weights 1, 1/2, 1/4 ... of the water-tank example,
// page "State Space Model", section "Un sistema che riassume il passato"), so
// inside a chunk every such product is exp of a difference of this prefix.
// Storing log2(e) * prefix lets consumers use the hardware exp2 directly.
//
// One workgroup (256 threads) per (batch, chunk, 8-head slice).  The [Q x 8]
// slab of dt is read into LDS (32 bytes per token row).  Thread (segment s,
// head hh) then sums its Q/32 consecutive tokens in fp64, the 32 segment
// totals of a head are combined through LDS, and each thread writes its
// segment's prefix (rounded once to fp32) back into LDS.  Both outputs leave
// as whole head rows of Q contiguous floats.  (8-head slices: 9.5 us at the
// 2.7B shape, against 14.2 us with 32-head slices, 11.7 with 4 and 24 with
// 64; the results are bitwise the same.)
#include "device_common.h"
#include "launchers.h"

namespace ssd {

constexpr int kCsHeads = 8;                // heads per workgroup
constexpr int kCsSegs = 256 / kCsHeads;    // token segments per head (one thread each)

__global__ __launch_bounds__(256) void chunk_cumsum_kernel(const float* __restrict__ dt,
                                                           const float* __restrict__ A,
                                                           float* __restrict__ cs,
                                                           float* __restrict__ dtc, int L,
                                                           int H, int Q, int nc, int zoh) {
    __shared__ float dts[256][kCsHeads + 1];
    __shared__ float css[256][kCsHeads + 1];
    __shared__ double segsum[kCsSegs][kCsHeads];
    const int b = blockIdx.x / nc;
    const int c = blockIdx.x - b * nc;
    const int h0 = blockIdx.y * kCsHeads;
    const int nh = min(kCsHeads, H - h0);
    const int t0 = c * Q;
    const int nt = min(Q, L - t0);
    const int tid = threadIdx.x;
    const int hh = tid % kCsHeads, seg = tid / kCsHeads;

    {
        // all of a thread's loads in flight before the first LDS write
        const float* src = dt + ((int64_t)b * L + t0) * H + h0 + hh;
        float v[256 / kCsSegs];
#pragma unroll
        for (int k = 0; k < 256 / kCsSegs; ++k) {
            const int j = seg + kCsSegs * k;
            v[k] = (j < nt && hh < nh) ? src[(int64_t)j * H] : 0.0f;
        }
#pragma unroll
        for (int k = 0; k < 256 / kCsSegs; ++k) {
            const int j = seg + kCsSegs * k;
            if (j < Q) dts[j][hh] = v[k];
        }
    }
    __syncthreads();

    const int sl = (Q + kCsSegs - 1) / kCsSegs;
    const int j0 = min(seg * sl, Q), j1 = min(j0 + sl, Q);
    const double a = (hh < nh) ? (double)A[h0 + hh] * 1.4426950408889634074 : 0.0;
    double run = 0.0;
    for (int j = j0; j < j1; ++j) run += (double)dts[j][hh] * a;
    segsum[seg][hh] = run;
    __syncthreads();
    run = 0.0;
    for (int s = 0; s < seg; ++s) run += segsum[s][hh];
    for (int j = j0; j < j1; ++j) {
        run += (double)dts[j][hh] * a;
        css[j][hh] = (float)run;
    }
    __syncthreads();

    for (int k = 0; k < nh; ++k) {
        const int64_t off = (((int64_t)b * H + h0 + k) * nc + c) * Q;
        const float ak = A[h0 + k];
        for (int j = tid; j < Q; j += 256) {
            cs[off + j] = css[j][k];
            const float d = dts[j][k];
            dtc[off + j] = zoh ? zoh_weight(d, ak) : d;
        }
    }
}

hipError_t launch_chunk_cumsum(const Dims& d, const float* dt, const float* A, float* cs,
                               float* dtc, hipStream_t stream, bool zoh) {
    dim3 grid((unsigned)(d.batch * d.nchunks), (unsigned)((d.nheads + kCsHeads - 1) / kCsHeads));
    chunk_cumsum_kernel<<<grid, 256, 0, stream>>>(dt, A, cs, dtc, (int)d.seqlen, (int)d.nheads,
                                                  (int)d.chunk, (int)d.nchunks, zoh ? 1 : 0);
    return hipGetLastError();
}

}  // namespace ssd
