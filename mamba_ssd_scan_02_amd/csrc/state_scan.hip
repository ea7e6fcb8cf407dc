// state_scan.hip -- each chunk's entering state and the final state in one
// pass over the sequence:
//
//     H_0 = init,   H_{c+1} = exp(Acs_c[last]) H_c + S_c,
//     S_c[p][n] = sum_j w_j x_j[p] B_j[n],   w_j = exp(Acs_c[last] - Acs_c[j]) dt_j
//
// This is the block recurrence that carries only a summary state from one
// block to the next (page "Mamba-2 (2024): SSM e attention sono la stessa
// cosa", section "Il trucco a blocchi"): the same recursion the token-level
// scan runs, with a block's decay product in place of one token's factor
// (page "State Space Model", section "Un sistema che riassume il passato").
// It computes what the chunk-state and state-passing stages compute
// together, without writing the per-chunk states S_c to memory: the running
// state lives in the matrix-core accumulators, is scaled by the chunk's
// decay before the chunk's products are added onto it, and only the state
// entering each chunk (Hin, the storage dtype) and the final state (fp32)
// leave the chip.
//
// Matrix-core kernel (bf16 storage, P = 64, N = 128, chunk 256).
// One workgroup (4 waves) per (batch, head, half of P); the workgroup walks
// the sequence in 32-token blocks.  Wave w owns state columns
// n in [32w, 32w + 32): C[n][p] += sum_j B_j[n] (w_j x_j[p]) with
// v_mfma_f32_32x32x16_bf16, M = n (B rows), N = p (x rows), K = tokens, both
// operands read token-contiguous with tr16.  Blocks of B (32 x 256 B, from
// L2: all heads of a group share them) are copied straight into a 4-buffer
// LDS ring three blocks ahead, and blocks of the workgroup's half of x
// (32 x 64 B, from HBM) into an 8-buffer ring seven blocks ahead, through
// bounds-checked buffer records (tokens
// past the end read as zeros, so every wave issues the same copies at every
// step and the waits are constants).  Each block's x rows are scaled by w_j
// in LDS one step before they are used (4 multiplies per thread, shared by
// the four waves) and rounded to bf16 once.
#include <cmath>

#include "device_common.h"
#include "launchers.h"
#include "lds_pipe.h"

namespace ssd {

namespace {

// Operations each wave issues: at every step 2 copies of B (block k + 3)
// then 1 of x (block k + 7), at a chunk's step 0 then 2 row copies (cs, dt),
// and 4 Hin stores at a chunk's start.  Before the scale at step jt block
// k + 1 must have landed: its x copy is older than its B copy (issued at
// step k - 2), so waiting for the B copy suffices; counted after it: that
// step's x copy, step k - 1's copies, and the row copies and stores that
// fall in between.
constexpr int kSsDps = 3, kSsDc = 2, kSsNh = 4;
__host__ __device__ constexpr int sscan_ops_after(int jt) {
    return jt == 0 ? 1 + kSsDps + kSsNh
         : jt == 1 ? 1 + kSsNh + kSsDps + kSsDc
         : jt == 2 ? 1 + kSsDc + kSsDps
                   : 1 + kSsDps;
}
// The issue order replayed against those counts over a few chunks (labels:
// B block k, x block k, rows of chunk c, Hin stores of chunk c): at step k
// the block scaled (x k + 1) and the block multiplied (B k) must have landed,
// and at a chunk's last step the next chunk's rows.
constexpr bool sscan_waits_hold(int nc) {
    auto bl = [](int k) { return 1000 + k; };
    auto xl = [](int k) { return 2000 + k; };
    auto rl = [](int c) { return 3000 + c; };
    VmemLog o;
    o.push(rl(0), kSsDc);
    for (int k = 0; k < 7; ++k) o.push(xl(k), 1);
    for (int k = 0; k < 3; ++k) o.push(bl(k), 2);
    if (!o.wait(0)) return false;
    for (int c = 0; c < nc; ++c) {
        o.push(4000 + c, kSsNh);
        for (int jt = 0; jt < 8; ++jt) {
            const int k = 8 * c + jt;
            if (!o.wait(sscan_ops_after(jt < 3 ? jt : 3)) || !o.landed(xl(k + 1)) || !o.landed(bl(k)))
                return false;
            if (jt == 7 && !o.landed(rl(c + 1))) return false;
            o.push(bl(k + 3), 2);
            o.push(xl(k + 7), 1);
            if (jt == 0) o.push(rl(c + 1), kSsDc);
        }
    }
    return true;
}
static_assert(kSsDps == 2 + 1, "two B copies and one x copy per step");
static_assert(sscan_waits_hold(1) && sscan_waits_hold(2) && sscan_waits_hold(4),
              "state_scan wait counts do not cover its copies");

}  // namespace

template <int Q>
__global__ __launch_bounds__(256, 3) void state_scan_mfma_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ Bm, const float* __restrict__ cs,
    const float* __restrict__ dtc, const float* init, bf16_t* __restrict__ Hin, float* fin, int L,
    int H, int G, int nc) {
    constexpr int P = 64, N = 128, NT = Q / 32;
    static_assert(NT == 8, "the ring index repeats every chunk and the next chunk's rows land by step 4");
    __shared__ uint4 st0[512], st1[512], st2[512], st3[512];   // B blocks, 32 x 256 B
    __shared__ uint4 xr[NT][128];                              // x blocks, 32 x 64 B (one chunk)
    __shared__ float csdt[2][2 * Q];                           // cs and dt rows, by chunk parity
    __shared__ uint4 sink[64];                                 // target of the waves' dummy x copies

    const uint32_t wg = xcd_logical_id(blockIdx.x, gridDim.x);
    const int ph = (int)(wg & 1u);
    const int bh = (int)(wg >> 1);
    const int h = bh % H, b = bh / H;
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hf = lane >> 5, l32 = lane & 31;
    const int64_t xstride = (int64_t)H * P, bstride = (int64_t)G * N;
    const bf16_t* xbase = x + ((int64_t)b * L * H + h) * P + 32 * ph;
    const bf16_t* bbase = Bm + ((int64_t)b * L * G + g) * N;
    const int64_t rowbase = ((int64_t)b * H + h) * nc;   // (b, h, chunk 0) row of cs/dt/Hin
    // cs and dt rows of this (batch, head): nc chunks of Q floats
    const __amdgpu_buffer_rsrc_t rcs = make_rs(cs + rowbase * Q, (int64_t)nc * Q * 4);
    const __amdgpu_buffer_rsrc_t rdt = make_rs(dtc + rowbase * Q, (int64_t)nc * Q * 4);

    // per-lane copy offsets (block-relative); the x rows (32 x 64 B, two
    // copies of 64 lanes) are copied by waves 0 and 1, and waves 2 and 3
    // issue an empty copy (offset past every record: zeros into `sink`) so
    // that every wave issues the same number of copies
    uint32_t boff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = 4 * (wave + 4 * i) + (lane >> 4);
        boff[i] = (uint32_t)r * (uint32_t)bstride * 2u + 16u * (uint32_t)((lane & 15) ^ swz_b(r));
    }
    const uint32_t xoff = (uint32_t)(16 * (wave & 1) + (lane >> 2)) * (uint32_t)xstride * 2u + 16u * (uint32_t)(lane & 3);
    const uint32_t bblk = 32u * (uint32_t)bstride * 2u, xblk = 32u * (uint32_t)xstride * 2u;

    // records of chunk c's B and x rows (empty past the last chunk)
    auto rec_b = [&](int c) {
        return make_rs(bbase + (int64_t)c * Q * bstride, ((int64_t)L - (int64_t)c * Q) * bstride * 2);
    };
    auto rec_x = [&](int c) {
        return make_rs(xbase + (int64_t)c * Q * xstride, ((int64_t)L - (int64_t)c * Q) * xstride * 2);
    };
    auto issue_b = [&](__amdgpu_buffer_rsrc_t rb, int jb, uint4* st) {
        dma16_rs(rb, boff[0] + (uint32_t)jb * bblk, lds(st) + wave * 64);
        dma16_rs(rb, boff[1] + (uint32_t)jb * bblk, lds(st) + (wave + 4) * 64);
    };
    auto issue_x = [&](__amdgpu_buffer_rsrc_t rx, int jb, uint4* xs) {
        if (wave < 2) dma16_rs(rx, xoff + (uint32_t)jb * xblk, lds(xs) + wave * 64);
        else dma16_rs(rx, 0x80000000u, lds(sink));
    };
    auto issue_rows = [&](int c) {   // cs and dt rows of chunk c (zeros past the last)
        const uint32_t o = 4u * (uint32_t)(c * Q + 64 * wave + lane);
        dma4_rs(rcs, o, lds(csdt[c & 1]) + 64 * wave);
        dma4_rs(rdt, o, lds(csdt[c & 1]) + Q + 64 * wave);
    };
    // w_j x_j in place for block jb of chunk c: thread t owns 4 channels
    // (8 bytes) of token row t / 8
    auto scale_block = [&](int c, int jb, uint4* xs) {
        const float* rows = csdt[c & 1];
        const int j = 32 * jb + (tid >> 3);
        const float w = fast_exp2(rows[Q - 1] - rows[j]) * rows[Q + j];
        uint2* p = reinterpret_cast<uint2*>(xs) + tid;
        const uint2 v = *p;
        *p = make_uint2(pack_bf16x2(bf16_bits_to_f32(v.x & 0xffffu) * w, bf16_bits_to_f32(v.x >> 16) * w),
                        pack_bf16x2(bf16_bits_to_f32(v.y & 0xffffu) * w, bf16_bits_to_f32(v.y >> 16) * w));
    };

    // running state C[n][p]: lane owns p = 32 ph + l32, register r holds
    // n = 32 w + 8 (r / 4) + 4 hf + r % 4
    f32x16 acc;
    const int p = 32 * ph + l32;
    const int n0 = 32 * wave + 4 * hf;
    if (init) {
        const float* ip = init + ((int64_t)b * H + h) * (int64_t)(P * N) + (int64_t)p * N + n0;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const float4 v = *reinterpret_cast<const float4*>(ip + 8 * a);
            acc[4 * a + 0] = v.x;
            acc[4 * a + 1] = v.y;
            acc[4 * a + 2] = v.z;
            acc[4 * a + 3] = v.w;
        }
    } else {
        acc = f32x16{};
    }
    {
        const __amdgpu_buffer_rsrc_t rb = rec_b(0), rx = rec_x(0);
        issue_rows(0);
#pragma unroll
        for (int k = 0; k < NT - 1; ++k) issue_x(rx, k, xr[k]);
        issue_b(rb, 0, st0);
        issue_b(rb, 1, st1);
        issue_b(rb, 2, st2);
    }
    wait_vmcnt<0>();
    barrier_lds();
    scale_block(0, 0, xr[0]);

    // tr16 addressing (lds_pipe.h): lane r of 16-lane group grp supplies
    // token row 8 (grp / 2) + r / 4 (+ 16 u, + 4 for the second half) and
    // column quad 16 (grp % 2) + 4 (r % 4); lane l of the result holds
    // column l % 32 of the operand.
    const int grp = lane >> 4, rr = lane & 15;
    const int trow0 = 8 * (grp >> 1) + (rr >> 2);
    const int qcol = 16 * (grp & 1) + 4 * (rr & 3);

    for (int c = 0; c < nc; ++c) {
        // state entering chunk c, then its decay: H <- exp(Acs_c[last]) H
        {
            bf16_t* hp = Hin + (rowbase + c) * (int64_t)(P * N) + (int64_t)p * N + n0;
#pragma unroll
            for (int a = 0; a < 4; ++a)
                *reinterpret_cast<uint2*>(hp + 8 * a) =
                    make_uint2(pack_bf16x2(acc[4 * a], acc[4 * a + 1]), pack_bf16x2(acc[4 * a + 2], acc[4 * a + 3]));
            const float decay = fast_exp2(csdt[c & 1][Q - 1]);
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] *= decay;
        }
        const __amdgpu_buffer_rsrc_t rb0 = rec_b(c), rx0 = rec_x(c);
        const __amdgpu_buffer_rsrc_t rb1 = rec_b(c + 1), rx1 = rec_x(c + 1);
#pragma unroll
        for (int jt = 0; jt < NT; ++jt) {
            // block k + 1 has landed once only later operations are pending
            if (jt == 0) wait_vmcnt<sscan_ops_after(0)>();
            else if (jt == 1) wait_vmcnt<sscan_ops_after(1)>();
            else if (jt == 2) wait_vmcnt<sscan_ops_after(2)>();
            else wait_vmcnt<sscan_ops_after(3)>();
            barrier_lds();
            uint4* cur = (jt % 4 == 0) ? st0 : (jt % 4 == 1) ? st1 : (jt % 4 == 2) ? st2 : st3;
            uint4* fut = ((jt + 3) % 4 == 0) ? st0 : ((jt + 3) % 4 == 1) ? st1 : ((jt + 3) % 4 == 2) ? st2 : st3;
            // block k + 1 (the next chunk's first at the last step; past the
            // last chunk its rows and weights are zeros)
            if (jt + 1 < NT) scale_block(c, jt + 1, xr[jt + 1]);
            else scale_block(c + 1, 0, xr[0]);
            if (jt + 3 < NT) issue_b(rb0, jt + 3, fut);
            else issue_b(rb1, jt + 3 - NT, fut);
            // x of block k + 7 into the slot block k - 1 used
            if (jt == 0) issue_x(rx0, NT - 1, xr[NT - 1]);
            else issue_x(rx1, jt - 1, xr[jt - 1]);
            if (jt == 0) issue_rows(c + 1);
            // C[n][p] += sum_j (B_j[n]) (w_j x_j[p]) over the block's 32 tokens
            const SSD_LDS char* bb = (const SSD_LDS char*)lds(cur);
            const SSD_LDS char* xb = (const SSD_LDS char*)lds(xr[jt]);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int r0 = 16 * u + trow0, r1 = r0 + 4;
                const int nc4 = 32 * wave + qcol;
                const int chk = nc4 >> 3, sub = (nc4 & 7) * 2;
                const uint2 blo = tr16(bb + r0 * 256 + ((chk ^ swz_b(r0)) << 4) + sub);
                const uint2 bhi = tr16(bb + r1 * 256 + ((chk ^ swz_b(r1)) << 4) + sub);
                const uint2 xlo = tr16(xb + r0 * 64 + 2 * qcol);
                const uint2 xhi = tr16(xb + r1 * 64 + 2 * qcol);
                const bf16x8 aq = __builtin_bit_cast(bf16x8, make_uint4(blo.x, blo.y, bhi.x, bhi.y));
                const bf16x8 bq = __builtin_bit_cast(bf16x8, make_uint4(xlo.x, xlo.y, xhi.x, xhi.y));
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, bq, acc, 0, 0, 0);
            }
        }
    }
    wait_vmcnt<0>();   // prefetches past the end (zeros) land before the workgroup leaves
    if (fin) {
        float* fp = fin + ((int64_t)b * H + h) * (int64_t)(P * N) + (int64_t)p * N + n0;
#pragma unroll
        for (int a = 0; a < 4; ++a)
            *reinterpret_cast<float4*>(fp + 8 * a) = make_float4(acc[4 * a], acc[4 * a + 1], acc[4 * a + 2], acc[4 * a + 3]);
    }
}

hipError_t launch_state_scan(const Dims& d, const void* x, const void* B, const float* cs,
                             const float* dtc, const float* init, void* Hin, float* final_state,
                             hipStream_t stream) {
    const unsigned blocks = (unsigned)(d.batch * d.nheads * 2);
    const bf16_t* xb = static_cast<const bf16_t*>(x);
    const bf16_t* bb = static_cast<const bf16_t*>(B);
    bf16_t* hb = static_cast<bf16_t*>(Hin);
    const int L = (int)d.seqlen, H = (int)d.nheads, G = (int)d.ngroups, nc = (int)d.nchunks;
    state_scan_mfma_kernel<256><<<blocks, 256, 0, stream>>>(xb, bb, cs, dtc, init, hb, final_state, L, H, G, nc);
    return hipGetLastError();
}

}  // namespace ssd
