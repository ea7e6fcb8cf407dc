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
// Matrix-core kernels (bf16, P = 64, N = 128, Q in {64, 128, 256}),
// v_mfma_f32_32x32x16_bf16.
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
//   * Term (ii): Y^T += Hin C^T (K = N), scaled per column by exp2(cs_i)
//     (or exp2 of the tile's reference, in the factorised form).
// Two kernels take these steps, both for runs of heads sharing one B/C group
// and both copying each head's x rows, carried state and cs/dt rows straight
// into LDS (lds_pipe.h) one head ahead: G^T does not depend on the head, so
// it is formed once per chunk and kept in registers across the run.
//   * the paired kernel (Q = 256): 8 waves, two per SIMD, the chunk's 36
//     blocks split over pairs of waves (see its own description below);
//   * the short-chunk kernel (Q = 64 or 128): Q / 16 waves, one output tile
//     and half the channels each, direct weights.
//
// Generic kernel (fp32 or bf16, any P, N within limits): the same three terms
// in fp32 on the vector units, 32 x 32 tiles in LDS.
#include <algorithm>
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
// Pieces shared by the two matrix-core kernels.

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

// The causal set j <= i and the diagonal j == i of a diagonal block as lane
// masks of one register r, constant for every wave (register r holds
// j - 8 hf = 16 (r / 8) + r % 8 of column i = l32): j <= i holds in lanes
// l32 >= jr of the first half and l32 >= jr + 8 of the second; j == i in
// lanes r and 40 + r (r < 8) or r + 8 and 48 + r (r >= 8).
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

// b in the lanes of mask m, a elsewhere: one select, no compare.  Its
// operands must not come straight from a matrix-core product: the compiler
// does not see inside the asm, so it would not insert the wait states that
// reading an MFMA result needs (mask_causal below is the form for those).
__device__ __forceinline__ float lane_select(float a, float b, uint64_t m) {
    float d;
    asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "s"(m));
    return d;
}

// The causal mask j <= i of a diagonal block's G^T tile, applied to the
// MFMA result itself with plain selects (the compiler then waits for the
// product before reading it): lane (l32, hf) keeps register r iff
// l32 >= gt_row(r, hf).
__device__ __forceinline__ void mask_causal(f32x16& a, int l32, int hf) {
#pragma unroll
    for (int r = 0; r < 16; ++r) a[r] = l32 >= gt_row(r, hf) ? a[r] : 0.0f;
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

// ---------------------------------------------------------------------------
// Pieces of the paired kernel below (Q = 256): per-slot LDS operands, the
// slot's weights and its products (the direct weights also serve the
// short-chunk kernel).
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

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
// Direct weights, exp2(cs_i - cs_j) dt_j per element, with D added on the
// diagonal by constant lane masks (no per-lane flag values that the
// compiler would keep live across the head loop).
__device__ __forceinline__ void rs_weights_direct(u32x4v (&gq)[2], const f32x16& gt,
                                                  const SSD_LDS float* csb, const SSD_LDS float* dtb,
                                                  float csi, float Dh, bool dgb, int hf) {
    // gt is zero above the diagonal of a diagonal block
    const SSD_LDS float* cb = csb + 8 * hf;
    const SSD_LDS float* db = dtb + 8 * hf;
    float v[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int jl = 16 * (r >> 3) + (r & 7);
        v[r] = gt[r] * (fast_exp2(fminf(csi - cb[jl], 0.0f)) * db[jl]);
    }
    if (dgb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = lane_select(v[r], v[r] + Dh, diag_eq_lanes(r));
    }
    uint32_t pk[8];
#pragma unroll
    for (int r2 = 0; r2 < 8; ++r2) pk[r2] = pack_bf16x2(v[2 * r2], v[2 * r2 + 1]);
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

// ---------------------------------------------------------------------------
// Paired resident kernel (Q = 256): one workgroup of 8 waves per CU and per
// (batch, chunk, group, run of heads), two waves per SIMD, so that one
// wave's vector work (the decay weights) overlaps the other's matrix-core
// products and LDS reads.  The chunk's 36 causal 32 x 32 blocks and 8
// carried-state terms are split over 4 pairs of waves: pair p owns output
// tiles 7 - p and p (9 blocks).  Its lead wave (waves 0..3) takes blocks
// 0..4 of tile 7 - p and that tile's state term; its helper wave (waves
// 4..7) takes blocks 5..7 - p of tile 7 - p, all of tile p and tile p's
// state term.  The helper's partial sums of tile 7 - p reach the lead through
// LDS.  Each wave keeps the G^T tiles of its own 5 or 4 blocks in registers
// for the whole run of heads.  A head's x rows, carried state and cs/dt rows
// are copied into one of two LDS slots one head ahead, spread over the
// previous head's blocks.  Every wave stores its tile of head k after the
// barrier that opens head k + 1 (the lead of pairs 0..2 once it has added
// the helper's partial sums), so the workgroup still meets once per head:
// it writes the tile as bf16 rows into the four 1 KB pieces of head k's
// slot that it will itself fill with head k + 2's x rows, and stores them
// back as whole 128-byte token rows (8 lanes per row) -- the y traffic
// then leaves the CU as full-line writes rather than 16-byte pieces.
namespace rpl {
constexpr int kX = 0;          // x: 256 rows x 128 B
constexpr int kH = 32768;      // Hin: 64 rows x 256 B
constexpr int kCs = 49152;     // cs: 256 floats
constexpr int kDt = 50176;     // dt: 256 floats
constexpr int kSlot = 51200;
constexpr int kRedTile = 8192;                 // one tile's partial sums: 32 tokens x 64 channels fp32
constexpr int kRed = 2 * kSlot;                // [head parity][pair 0..2] partial tiles
constexpr int kRf = kRed + 2 * 3 * kRedTile;   // [wave][160] rf rows of the wave's blocks
constexpr int kBytes = kRf + 8 * 160 * 4;
static_assert(kBytes <= 160 * 1024, "paired chunk_scan LDS");
constexpr int kCopies = 7;     // LDS-copy instructions per wave per head: x 4, Hin 2, cs or dt 1
constexpr int kStores = 4;     // y stores of one tile (8 token rows each)

// The issue order of one wave (labels: copies of head k, y stores of head
// k) replayed against its wait at the top of each head, vmcnt(0): head k's
// copies must have landed (trivially: nothing may be outstanding).
constexpr bool waits_hold(int heads) {
    VmemLog o;
    o.push(100, kCopies);
    for (int k = 0; k < heads; ++k) {
        if (!o.wait(0) || !o.landed(100 + k)) return false;
        if (k > 0) o.push(1000 + k - 1, kStores);
        if (k + 1 < heads) o.push(100 + k + 1, kCopies);
    }
    return true;
}
static_assert(waits_hold(1) && waits_hold(2) && waits_hold(40), "paired chunk_scan waits");

// Byte offset of 16-byte chunk c of token row r (0..31) of a staged y tile
// within its 1 KB piece (rows 8 m .. 8 m + 7 in piece m).  The chunk index
// is XORed with f(r) = ((r / 2) % 8) ^ ((r / 16) % 2): the lanes that share
// an LDS cycle then reach distinct 16-byte bank groups whether the LDS
// serves 16 or 32 lanes of a 16-byte access per cycle -- one chunk of 16 or
// 32 rows when the tile is written (f is one-to-one on the rows of equal
// r % 2 among 16 and of equal r % 4 among 32), 8 chunks of 2 or 4 rows
// when it is read back.
__device__ __forceinline__ int stage_off(int r, int c) {
    return (r & 7) * 128 + ((c ^ ((r >> 1) & 7) ^ ((r >> 4) & 1)) << 4);
}
// Order in which a wave issues its 7 copy instructions of the next head,
// two per block from the first block on: cs or dt (needed first), x, Hin.
constexpr int kIssueOrder[kCopies] = {6, 0, 1, 2, 3, 4, 5};
}  // namespace rpl

// The state entering a chunk from the two-level recurrence between chunks
// (runs of K chunks; chunk_state_runs_kernel): Hin_c = T_{c-1} + exp2(lam_c)
// Hr_r past a run's first chunk, Hr_r at it.  The slot's state rows then
// come from T_{c-1} (or Hr_r) by the same copies that bring Hin, and the wave
// that copied a piece of them adds exp2(lam_c) times the same piece of Hr_r
// (loaded into registers with the copies, a head ahead) once its copies have
// landed, rounding once to bf16, before the barrier that opens the head.
struct RunState {
    const bf16_t* Hr;    // [B][H][nruns][P][N], storage type
    const float* lam;    // [B][H][nc]
    int K, nruns;
};

// One wave of the paired kernel; ROLE 0 = lead, 1 = helper.  RUNS: the
// carried state is formed from the two-level recurrence's T (passed as Hin)
// and Hr (RunState) instead of read whole.  GATED: z is given and the store
// writes y silu(z) (a template parameter, so that neither form carries the
// other's branches through its loop over heads).
template <int ROLE, bool RUNS, bool GATED>
__device__ __forceinline__ void paired_run(const bf16_t* __restrict__ x, const bf16_t* __restrict__ Bm,
                                           const bf16_t* __restrict__ Cm, const float* __restrict__ cs,
                                           const float* __restrict__ dtc, const bf16_t* __restrict__ Hin,
                                           const float* __restrict__ D, const bf16_t* __restrict__ z,
                                           bf16_t* __restrict__ y, int L, int H, int G, int nc, int b,
                                           int c, int g, int h0, int cnt, int wave, int lane,
                                           SSD_LDS char* sm, const RunState& rs) {
    using namespace rpl;
    constexpr int Q = 256, P = 64, N = 128;
    constexpr int NB = ROLE == 0 ? 5 : 4;       // blocks of this wave
    const int p = wave & 3;
    const int thi = 7 - p, tlo = p;
    const int nh = ROLE == 0 ? NB : 3 - p;      // its blocks 0..nh-1 belong to tile thi
    const int own = ROLE == 0 ? thi : tlo;      // the tile whose state term and store it makes
    const int hf = lane >> 5, l32 = lane & 31;
    const int tok0 = c * Q;
    const int rowbytes = H * P * 2;
    // end of the chunk's last valid row, for x and y (Q rows fit 31 bits)
    const int xrecord = (min(L - tok0, Q) - 1) * rowbytes + P * 2;
    // block i: output tile bt(i), j block bs(i)
    auto bt = [&](int i) { return i < nh ? thi : tlo; };
    auto bs = [&](int i) { return ROLE == 0 ? i : (i < nh ? 5 + i : i - nh); };

    // Copy offsets.  x copy m covers rows 8 q .. 8 q + 7 and Hin copy m rows
    // 4 q .. 4 q + 3, q = wave + 8 m; cs (waves 0..3) or dt (4..7) a quarter
    // row each.
    const uint32_t xo0 = (uint32_t)(8 * wave + (lane >> 3)) * (uint32_t)rowbytes +
                         16u * (uint32_t)((lane & 7) ^ swz_x(lane >> 3));
    const uint32_t xstep = 64u * (uint32_t)rowbytes;
    uint32_t ho[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int r = 4 * (wave + 8 * m) + (lane >> 4);
        ho[m] = (uint32_t)(r * 256 + 16 * ((lane & 15) ^ swz_h(r)));
    }
    // copy instruction m (0..6) of head k into the slot at s: x parts 0..3,
    // Hin parts 4 and 5, the cs or dt quarter 6.  The seven are spread over
    // the first four blocks of the previous head (kIssueOrder), so that a
    // wave held at issue by a full memory pipeline leaves its SIMD to the
    // other wave and the last copy still has most of a head to land.
    // RUNS: the run of chunk c, whether c is past the run's first chunk (then
    // the slot takes T_{c-1} and Hr is added), and the next head's Hr pieces
    // and lam_c, loaded with its copies
    const int run = RUNS ? c / rs.K : 0;
    const bool comb = RUNS && c % rs.K != 0;
    uint4 hrp[2] = {};
    float lamp = 0.0f;
    auto state_tile = [&](int h) {
        if (RUNS) {
            const int64_t bh = (int64_t)b * H + h;
            return comb ? Hin + (bh * nc + c - 1) * (int64_t)(P * N)
                        : rs.Hr + (bh * rs.nruns + run) * (int64_t)(P * N);
        }
        return Hin + (((int64_t)b * H + h) * nc + c) * (int64_t)(P * N);
    };
    auto issue_part = [&](int k, SSD_LDS char* s, int m) {
        const int h = h0 + k;
        if (m < 4) {
            const __amdgpu_buffer_rsrc_t rx = make_rs(x + (((int64_t)b * L + tok0) * H + h) * P, xrecord);
            dma16_rs(rx, xo0 + (uint32_t)m * xstep, s + kX + (wave + 8 * m) * 1024);
        } else if (m < 6) {
            const __amdgpu_buffer_rsrc_t rh = make_rs(state_tile(h), P * N * 2);
            dma16_rs(rh, ho[m - 4], s + kH + (wave + 8 * (m - 4)) * 1024);
        } else {
            // with the head's first copy: its Hr pieces and lam, which the
            // combine at the head's top waits for
            if (comb) {
                const int64_t bh = (int64_t)b * H + h;
                const char* hr = reinterpret_cast<const char*>(rs.Hr + (bh * rs.nruns + run) * (int64_t)(P * N));
                hrp[0] = *reinterpret_cast<const uint4*>(hr + ho[0]);
                hrp[1] = *reinterpret_cast<const uint4*>(hr + ho[1]);
                lamp = rs.lam[bh * nc + c];
            }
            const int64_t row = (((int64_t)b * H + h) * nc + c) * Q;
            const int part = wave & 3;
            dma4_rs(make_rs((wave < 4 ? cs : dtc) + row, Q * 4), 4u * (uint32_t)(64 * part + lane),
                    s + (wave < 4 ? kCs : kDt) + 256 * part);
        }
    };
    auto issue = [&](int k, SSD_LDS char* s) {
#pragma unroll
        for (int m = 0; m < kCopies; ++m) issue_part(k, s, m);
    };
    auto yrs_of = [&](int k) {
        return __builtin_amdgcn_make_buffer_rsrc(y + (((int64_t)b * L + tok0) * H + h0 + k) * P, (short)0,
                                                 xrecord, 0x00020000);
    };

    issue(0, sm);

    // C fragments of the tile(s) of this wave's blocks and the resident G^T
    // tiles of its blocks (the diagonal block's causal mask applied once).
    uint4 cfo[8];   // tile own
    uint4 cfh[8];   // tile thi (helper, prologue only)
    auto load_cf = [&](uint4 (&cf)[8], int t) {
        const int tok = min(tok0 + 32 * t + l32, L - 1);
        const bf16_t* crow = Cm + (((int64_t)b * L + tok) * G + g) * N + 8 * hf;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) cf[kk] = *reinterpret_cast<const uint4*>(crow + 16 * kk);
    };
    load_cf(cfo, own);
    if (ROLE == 1 && nh > 0) load_cf(cfh, thi);
    f32x16 gt[NB];
    {
        const int jr = perm_pi(l32);
        uint4 bq[3][8];
        auto load_b = [&](int i, uint4 (&dst)[8]) {
            const int tok = min(tok0 + 32 * bs(i) + jr, L - 1);
            const bf16_t* brow = Bm + (((int64_t)b * L + tok) * G + g) * N + 8 * hf;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) dst[kk] = *reinterpret_cast<const uint4*>(brow + 16 * kk);
        };
        load_b(0, bq[0]);
        load_b(1, bq[1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            if (i + 2 < NB) load_b(i + 2, bq[(i + 2) % 3]);
            __builtin_amdgcn_sched_barrier(0);
            const uint4 (&bv)[8] = bq[i % 3];
            f32x16 a = {};
            if (ROLE == 1 && i < nh) {
#pragma unroll
                for (int kk = 0; kk < 8; ++kk)
                    a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, bv[kk]), __builtin_bit_cast(bf16x8, cfh[kk]), a, 0, 0, 0);
            } else {
#pragma unroll
                for (int kk = 0; kk < 8; ++kk)
                    a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, bv[kk]), __builtin_bit_cast(bf16x8, cfo[kk]), a, 0, 0, 0);
            }
            if (bs(i) == bt(i)) {
                mask_causal(a, l32, hf);
            }
            gt[i] = a;
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // The wave's tile of head k - 1 (before its column scale), stored at the
    // top of head k: the lead of pairs 0..2 first adds the helper's partial
    // sums; then the tile goes as bf16 rows into this wave's pieces of head
    // k - 1's slot (the pieces its own copies of head k + 1's x rows will
    // fill next) and out as whole token rows.
    f32x16 keep[2];
    float keep_colf = 1.0f;
    auto store_kept = [&](int k) {
        // the gate's z rows (same layout and record as y), loaded first so
        // that the staging below covers their latency
        const int tr = lane >> 3, tc = lane & 7;
        u32x4v zr[4];
        if constexpr (GATED) {
            const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<bf16_t*>(z) + (((int64_t)b * L + tok0) * H + h0 + k) * P, (short)0, xrecord, 0x00020000);
#pragma unroll
            for (int m = 0; m < 4; ++m)
                zr[m] = __builtin_bit_cast(u32x4v, __builtin_amdgcn_raw_buffer_load_b128(
                                                       zrs, (32 * own + 8 * m + tr) * rowbytes + 16 * tc, 0, 0));
        }
        if (ROLE == 0 && p < 3) {
            const SSD_LDS f32x4* red = (const SSD_LDS f32x4*)(sm + kRed + ((k & 1) * 3 + p) * kRedTile);
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 v = red[(4 * mt + q) * 64 + lane];
#pragma unroll
                    for (int e = 0; e < 4; ++e) keep[mt][4 * q + e] += v[e];
                }
        }
        SSD_LDS char* const sb = sm + (k & 1) * kSlot + kX;
        // lane (l32, hf) holds token row l32, channels 32 mt + 16 hf + 8 q
        // + 0..7 in keep[mt][8 q ..]: chunk 4 mt + 2 hf + q of the row
        SSD_LDS char* const wrow = sb + (wave + 8 * (l32 >> 3)) * 1024;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                u32x4v w;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    w[e] = pack_bf16x2(keep[mt][8 * q + 2 * e] * keep_colf, keep[mt][8 * q + 2 * e + 1] * keep_colf);
                *reinterpret_cast<SSD_LDS u32x4v*>(wrow + stage_off(l32, 4 * mt + 2 * hf + q)) = w;
            }
        // lane l: row 8 m + l / 8 of the tile, chunk l % 8; rows past the
        // sequence end fall outside the record and are dropped.  With the
        // gate, out = y silu(z) on the bf16 y, rounded once more: what the
        // separate gate kernel computes from the stored y.
        const __amdgpu_buffer_rsrc_t yrs = yrs_of(k);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int r = 8 * m + tr;
            u32x4v v = *reinterpret_cast<const SSD_LDS u32x4v*>(sb + (wave + 8 * m) * 1024 + stage_off(r, tc));
            if constexpr (GATED) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float y0 = bf16_bits_to_f32(v[e] & 0xffffu), y1 = bf16_bits_to_f32(v[e] >> 16);
                    const float z0 = bf16_bits_to_f32(zr[m][e] & 0xffffu), z1 = bf16_bits_to_f32(zr[m][e] >> 16);
                    v[e] = pack_bf16x2(y0 * silu_f(z0), y1 * silu_f(z1));
                }
            }
            __builtin_amdgcn_raw_buffer_store_b128(v, yrs, (32 * own + r) * rowbytes + 16 * tc, 0, 0);
        }
    };

    const XtAddr xa = xt_addr(lane);
    SSD_LDS float* const rfo = (SSD_LDS float*)(sm + kRf) + 160 * wave;
    for (int k = 0; k < cnt; ++k) {
        wait_vmcnt<0>();
        if (comb) {
            // this wave's two landed pieces of T_{c-1}: + exp2(lam_c) Hr_r
            const float lf = fast_exp2(lamp);
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                SSD_LDS u32x4v* q = (SSD_LDS u32x4v*)(sm + (k & 1) * kSlot + kH + (wave + 8 * m) * 1024) + lane;
                const u32x4v t = *q;
                const u32x4v hv = __builtin_bit_cast(u32x4v, hrp[m]);
                u32x4v o;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    o[e] = pack_bf16x2(fmaf(lf, bf16_bits_to_f32(hv[e] & 0xffffu), bf16_bits_to_f32(t[e] & 0xffffu)),
                                       fmaf(lf, bf16_bits_to_f32(hv[e] >> 16), bf16_bits_to_f32(t[e] >> 16)));
                *q = o;
            }
        }
        barrier_lds();
        // every wave is past head k - 1: its slot takes this wave's tile of
        // head k - 1 on its way out, then head k + 1, copied during this
        // head's first four blocks (the staged rows have been read back by
        // then: the stores consume them before the first copy is issued)
        if (k > 0) store_kept(k - 1);
        const bool next = k + 1 < cnt;
        SSD_LDS char* const snext = sm + ((k + 1) & 1) * kSlot;

        const SSD_LDS char* S = sm + (k & 1) * kSlot;
        const SSD_LDS float* css = (const SSD_LDS float*)(S + kCs);
        const SSD_LDS float* dts = (const SSD_LDS float*)(S + kDt);
        const float Dh = D ? D[h0 + k] : 0.0f;
        auto tile_f = [&](int t, float& csi) {
            const float cref = css[32 * t], ctail = css[32 * t + 31];
            csi = css[32 * t + l32];
            TileF f;
            f.fact = uniform_f(cref - ctail) <= kMaxTileDecayLog2;
            if (f.fact) {
                f.colf = fast_exp2(csi - cref);
                f.sstate = fast_exp2(cref);
                f.dprime = Dh * fast_exp2(cref - csi);
            } else {
                f.colf = 1.0f;
                f.sstate = fast_exp2(csi);
                f.dprime = 0.0f;
            }
            return f;
        };
        float csi_h = 0.0f, csi_l = 0.0f;
        const TileF tfh = tile_f(thi, csi_h);
        TileF tfl = tfh;
        if (ROLE == 1) tfl = tile_f(tlo, csi_l);
        // rf rows of the wave's blocks: rfo[32 i + j] = exp2(cref - cs_j) dt_j
        // for token j of block i against its tile's first token
#pragma unroll
        for (int q = 0; q < (32 * NB + 63) / 64; ++q) {
            const int e = lane + 64 * q;
            if (e < 32 * NB) {
                const int i = e >> 5, j = e & 31;
                const int jj = 32 * bs(i) + j;
                rfo[e] = fast_exp2(fminf(css[32 * bt(i)] - css[jj], kMaxTileDecayLog2)) * dts[jj];
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

        f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            if (ROLE == 1 && i == nh && nh > 0) {
                // the helper's blocks of tile thi are done: hand them over
                SSD_LDS f32x4* red = (SSD_LDS f32x4*)(sm + kRed + ((k & 1) * 3 + p) * kRedTile);
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        red[(4 * mt + q) * 64 + lane] =
                            f32x4{acc[mt][4 * q], acc[mt][4 * q + 1], acc[mt][4 * q + 2], acc[mt][4 * q + 3]};
                    }
                acc[0] = f32x16{};
                acc[1] = f32x16{};
            }
            if (next && i < 4) {
                issue_part(k + 1, snext, kIssueOrder[2 * i]);
                if (2 * i + 1 < kCopies) issue_part(k + 1, snext, kIssueOrder[2 * i + 1]);
            }
            const bool hi = i < nh;
            const int s = bs(i);
            SlotRf rf;
            rs_fetch_rf(rf, rfo + 32 * i, hf);
            SlotX xs;
            rs_fetch_x(xs, S + kX + s * 4096, xa);
            const bool dg = s == bt(i);
            u32x4v gq[2];
            if (hi ? tfh.fact : tfl.fact)
                rs_weights_fact(gq, gt[i], rf, dg, hi ? tfh.dprime : tfl.dprime);
            else
                rs_weights_direct(gq, gt[i], css + 32 * s, dts + 32 * s, hi ? csi_h : csi_l, Dh, dg, hf);
            rs_products(acc, xs, gq);
        }

        // (ii) for tile own: accS = Hin C_own^T, added as sstate * accS
        {
            const SSD_LDS uint4* hs = (const SSD_LDS uint4*)(S + kH);
            f32x16 accS[2] = {f32x16{}, f32x16{}};
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                u32x4v ha[4][2];
#pragma unroll
                for (int kq = 0; kq < 4; ++kq)
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt) {
                        const int pr = 32 * mt + perm_sigma(l32);
                        const int ch = 2 * (4 * kh + kq) + hf;
                        ha[kq][mt] = *reinterpret_cast<const SSD_LDS u32x4v*>(hs + pr * 16 + (ch ^ swz_h(pr)));
                    }
#pragma unroll
                for (int kq = 0; kq < 4; ++kq)
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt)
                        accS[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ha[kq][mt]), __builtin_bit_cast(bf16x8, cfo[4 * kh + kq]), accS[mt], 0, 0, 0);
            }
            const TileF& tfo = ROLE == 0 ? tfh : tfl;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[mt][r] = fmaf(tfo.sstate, accS[mt][r], acc[mt][r]);
            keep[0] = acc[0];
            keep[1] = acc[1];
            keep_colf = tfo.colf;
        }
    }
    // the last head's tiles (and the helpers' last partial sums)
    barrier_lds();
    store_kept(cnt - 1);
    wait_vmcnt<0>();
}

template <bool RUNS, bool GATED>
__global__ __launch_bounds__(512, 1) void chunk_scan_paired_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ Bm, const bf16_t* __restrict__ Cm,
    const float* __restrict__ cs, const float* __restrict__ dtc, const bf16_t* __restrict__ Hin,
    const float* __restrict__ D, const bf16_t* __restrict__ z, bf16_t* __restrict__ y, int L, int H,
    int G, int nc, int hg, int nsplit, RunState rs) {
    __shared__ __align__(16) char smem[rpl::kBytes];
    const uint32_t wg = xcd_logical_id(blockIdx.x, gridDim.x);
    const int split = (int)(wg % (uint32_t)nsplit);
    const uint32_t bcg = wg / (uint32_t)nsplit;
    const int g = (int)(bcg % (uint32_t)G);
    const int bc = (int)(bcg / (uint32_t)G);
    const int c = bc % nc, b = bc / nc;
    const int hpg = H / G;
    const int h0 = g * hpg + split * hg;
    const int cnt = min(hg, hpg - split * hg);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    __builtin_assume(wave >= 0 && wave < 8);
    SSD_LDS char* const sm = (SSD_LDS char*)lds(smem);
    if (wave < 4)
        paired_run<0, RUNS, GATED>(x, Bm, Cm, cs, dtc, Hin, D, z, y, L, H, G, nc, b, c, g, h0, cnt, wave, lane,
                                   sm, rs);
    else
        paired_run<1, RUNS, GATED>(x, Bm, Cm, cs, dtc, Hin, D, z, y, L, H, G, nc, b, c, g, h0, cnt, wave, lane,
                                   sm, rs);
}

// ---------------------------------------------------------------------------
// Short chunks (Q = 64 or 128): one workgroup of W = Q / 16 waves per (batch,
// chunk, group, run of heads).  The chunk's causal 32 x 32 blocks of G^T =
// B C^T (3 or 10) do not depend on the head: they are formed once per run and
// stay in registers.  Wave w owns output tile t = w / 2 (tokens 32 t ..
// 32 t + 31) for channels 32 (w % 2) .. + 31, so the two waves of a tile both
// form its t + 1 blocks.  A head's x rows (Q x 128 B), carried state (16 KB)
// and cs/dt rows are copied into one of two LDS slots one head ahead.  Every
// weight is formed directly, exp2(cs_i - cs_j) dt_j per element (over so few
// tokens the factorised form saves little), and the state term is scaled by
// exp2(cs_i).  Each lane stores 16 consecutive channels of its token (two
// 16-byte stores); tokens past the end fall outside the y record and are
// dropped.  SLOTS LDS slots keep SLOTS - 1 heads' copies in flight.
template <int Q, int SLOTS>
struct ShortScan {
    static constexpr int NT = Q / 32;          // output tiles
    static constexpr int W = 2 * NT;           // waves
    static constexpr int kX = 0;               // x: Q rows x 128 B
    static constexpr int kH = Q * 128;         // Hin: 64 rows x 256 B
    static constexpr int kCs = kH + 16384;     // cs: Q floats
    static constexpr int kDt = kCs + 4 * Q;    // dt: Q floats
    static constexpr int kSlot = kDt + 4 * Q;
    static constexpr int kBytes = SLOTS * kSlot;
    static constexpr int kHinCopies = 16 / W;  // 1 KB Hin pieces per wave
    static constexpr int kRowCopies = Q / 32;  // 256-byte cs/dt pieces, one per wave
    static constexpr int kStores = 2;          // y stores per wave and head
    static_assert(kSlot % 16 == 0 && kBytes <= 160 * 1024 && kRowCopies <= W, "short-chunk chunk_scan LDS");
};

// Operations a wave issued after head k's copies when it waits for them at
// the top of head k (copies: per head, c of them; the issue order is the
// copies of heads 0 .. SLOTS - 2, then per head j: the copies of head
// j + SLOTS - 1, head j's y stores): the copies of the heads after k already
// issued and the y stores of the heads since head k's copies.
__host__ __device__ constexpr int short_ops_after(int slots, int c, int cnt, int k) {
    int n = 0;
    for (int i = k + 1; i <= k + slots - 2 && i < cnt; ++i) n += c;
    for (int j = (k - slots + 1 > 0 ? k - slots + 1 : 0); j < k; ++j) n += 2;
    return n;
}
constexpr bool short_waits_hold(int slots, int c, int cnt) {
    VmemLog o;
    for (int i = 0; i < slots - 1 && i < cnt; ++i) o.push(100 + i, c);
    for (int k = 0; k < cnt; ++k) {
        if (!o.wait(short_ops_after(slots, c, cnt, k)) || !o.landed(100 + k)) return false;
        if (k + slots - 1 < cnt) o.push(100 + k + slots - 1, c);
        o.push(500 + k, 2);
    }
    return true;
}
constexpr bool short_waits_hold_all() {
    for (int slots = 2; slots <= 4; ++slots)
        for (int c = 4; c <= 7; ++c)
            for (int cnt = 1; cnt <= 9; ++cnt)
                if (!short_waits_hold(slots, c, cnt)) return false;
    return true;
}
static_assert(short_waits_hold_all(), "short-chunk chunk_scan wait counts do not cover its copies");

template <int Q, int SLOTS>
__global__ __launch_bounds__(Q * 4, Q == 64 ? 2 : 1) void chunk_scan_short_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ Bm, const bf16_t* __restrict__ Cm,
    const float* __restrict__ cs, const float* __restrict__ dtc, const bf16_t* __restrict__ Hin,
    const float* __restrict__ D, bf16_t* __restrict__ y, int L, int H, int G, int nc, int hg,
    int nsplit) {
    using K = ShortScan<Q, SLOTS>;
    constexpr int P = 64, N = 128, NT = K::NT, W = K::W;
    __shared__ __align__(16) char smem[K::kBytes];
    const uint32_t wg = xcd_logical_id(blockIdx.x, gridDim.x);
    const int split = (int)(wg % (uint32_t)nsplit);
    const uint32_t bcg = wg / (uint32_t)nsplit;
    const int g = (int)(bcg % (uint32_t)G);
    const int bc = (int)(bcg / (uint32_t)G);
    const int c = bc % nc, b = bc / nc;
    const int hpg = H / G;
    const int h0 = g * hpg + split * hg;
    const int cnt = min(hg, hpg - split * hg);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    __builtin_assume(wave >= 0 && wave < W);
    const int t = wave >> 1, mt = wave & 1;
    const int hf = lane >> 5, l32 = lane & 31;
    const int tok0 = c * Q;
    const int rowbytes = H * P * 2;
    // end of the chunk's last valid row, for x and y
    const int xrecord = (min(L - tok0, Q) - 1) * rowbytes + P * 2;
    SSD_LDS char* const sm = (SSD_LDS char*)lds(smem);

    // Copies of head k into the slot at s: x rows 8 q .. 8 q + 7 for the
    // pieces q = wave + W m (m = 0, 1), Hin rows 4 q .. 4 q + 3 for q = wave +
    // W m (m < 16 / W), and 256-byte piece `wave` of the cs row then the dt
    // row.
    const uint32_t xo = (uint32_t)(8 * wave + (lane >> 3)) * (uint32_t)rowbytes +
                        16u * (uint32_t)((lane & 7) ^ swz_x(lane >> 3));
    const uint32_t xstep = (uint32_t)(8 * W) * (uint32_t)rowbytes;
    uint32_t ho[K::kHinCopies];
#pragma unroll
    for (int m = 0; m < K::kHinCopies; ++m) {
        const int r = 4 * (wave + W * m) + (lane >> 4);
        ho[m] = (uint32_t)(r * 256 + 16 * ((lane & 15) ^ swz_h(r)));
    }
    const int rarr = wave / (Q / 64), rpart = wave % (Q / 64);   // cs/dt piece of this wave
    auto issue = [&](int k, SSD_LDS char* s) {
        const int h = h0 + k;
        const __amdgpu_buffer_rsrc_t rx = make_rs(x + (((int64_t)b * L + tok0) * H + h) * P, xrecord);
#pragma unroll
        for (int m = 0; m < 2; ++m) dma16_rs(rx, xo + (uint32_t)m * xstep, s + K::kX + (wave + W * m) * 1024);
        const __amdgpu_buffer_rsrc_t rh =
            make_rs(Hin + (((int64_t)b * H + h) * nc + c) * (int64_t)(P * N), P * N * 2);
#pragma unroll
        for (int m = 0; m < K::kHinCopies; ++m) dma16_rs(rh, ho[m], s + K::kH + (wave + W * m) * 1024);
        if (wave < K::kRowCopies) {
            const int64_t row = (((int64_t)b * H + h) * nc + c) * Q;
            dma4_rs(make_rs((rarr == 0 ? cs : dtc) + row, Q * 4), 4u * (uint32_t)(64 * rpart + lane),
                    s + (rarr == 0 ? K::kCs : K::kDt) + 256 * rpart);
        }
    };

    const int ncopy = 2 + K::kHinCopies + (wave < K::kRowCopies ? 1 : 0);
#pragma unroll
    for (int i = 0; i < SLOTS - 1; ++i)
        if (i < cnt) issue(i, sm + i * K::kSlot);

    // C fragments of tile t (B operand of both C products) and the G^T
    // blocks (t, s), s <= t, the diagonal one masked to j <= i.  Tokens past
    // the end re-read the last token (their weights or outputs are dropped).
    uint4 cf[8];
    {
        const int tok = min(tok0 + 32 * t + l32, L - 1);
        const bf16_t* crow = Cm + (((int64_t)b * L + tok) * G + g) * N + 8 * hf;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) cf[kk] = *reinterpret_cast<const uint4*>(crow + 16 * kk);
    }
    f32x16 gt[NT];
    {
        const int jr = perm_pi(l32);
#pragma unroll
        for (int sb = 0; sb < NT; ++sb) {
            gt[sb] = f32x16{};
            if (sb > t) continue;
            const int tok = min(tok0 + 32 * sb + jr, L - 1);
            const bf16_t* brow = Bm + (((int64_t)b * L + tok) * G + g) * N + 8 * hf;
            uint4 bq[8];
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) bq[kk] = *reinterpret_cast<const uint4*>(brow + 16 * kk);
            f32x16 a = {};
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
                a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, bq[kk]),
                                                            __builtin_bit_cast(bf16x8, cf[kk]), a, 0, 0, 0);
            if (sb == t) mask_causal(a, l32, hf);
            gt[sb] = a;
        }
    }

    const XtAddr xa = xt_addr(lane);
    const int pc = 32 * mt + xa.qb;
    const int xchk = pc >> 3, xsub = (pc & 7) * 2;
    const int pr = 32 * mt + perm_sigma(l32);
    for (int k = 0; k < cnt; ++k) {
        // head k's copies have landed, and every wave is past head k - 1,
        // whose slot now takes head k + SLOTS - 1
        wait_vmcnt_n(short_ops_after(SLOTS, ncopy, cnt, k));
        barrier_lds();
        if (k + SLOTS - 1 < cnt) issue(k + SLOTS - 1, sm + ((k + SLOTS - 1) % SLOTS) * K::kSlot);
        const SSD_LDS char* S = sm + (k % SLOTS) * K::kSlot;
        const SSD_LDS float* css = (const SSD_LDS float*)(S + K::kCs);
        const SSD_LDS float* dts = (const SSD_LDS float*)(S + K::kDt);
        const float Dh = D ? D[h0 + k] : 0.0f;
        const float csi = css[32 * t + l32];

        // (i) + (iii): Y^T += X^T G~^T over the tile's blocks
        f32x16 acc = {};
#pragma unroll
        for (int sb = 0; sb < NT; ++sb) {
            if (sb > t) continue;
            u32x4v gq[2];
            rs_weights_direct(gq, gt[sb], css + 32 * sb, dts + 32 * sb, csi, Dh, sb == t, hf);
            const SSD_LDS char* xb = S + K::kX + sb * 4096;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int r0 = 16 * u + xa.trow0, r1 = r0 + 4;
                const u32x2v lo = __builtin_bit_cast(u32x2v, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (SSD_LDS v4s*)(xb + r0 * 128 + ((xchk ^ swz_x(r0)) << 4) + xsub)));
                const u32x2v hi = __builtin_bit_cast(u32x2v, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (SSD_LDS v4s*)(xb + r1 * 128 + ((xchk ^ swz_x(r1)) << 4) + xsub)));
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, u32x4v{lo.x, lo.y, hi.x, hi.y}),
                    __builtin_bit_cast(bf16x8, gq[u]), acc, 0, 0, 0);
            }
        }
        // (ii): accS = Hin C_t^T, added as exp2(cs_i) accS
        {
            const SSD_LDS uint4* hs = (const SSD_LDS uint4*)(S + K::kH);
            f32x16 accS = {};
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const int ch = 2 * kk + hf;
                const u32x4v ha = *reinterpret_cast<const SSD_LDS u32x4v*>(hs + pr * 16 + (ch ^ swz_h(pr)));
                accS = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ha),
                                                               __builtin_bit_cast(bf16x8, cf[kk]), accS, 0, 0, 0);
            }
            const float ss = fast_exp2(csi);
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = fmaf(ss, accS[r], acc[r]);
        }
        // y: token 32 t + l32, channels 32 mt + 16 hf + 0..15
        const __amdgpu_buffer_rsrc_t yrs = __builtin_amdgcn_make_buffer_rsrc(
            y + (((int64_t)b * L + tok0) * H + h0 + k) * P, (short)0, xrecord, 0x00020000);
        const int off = (32 * t + l32) * rowbytes + 64 * mt + 32 * hf;
        uint32_t w8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) w8[e] = pack_bf16x2(acc[2 * e], acc[2 * e + 1]);
        __builtin_amdgcn_raw_buffer_store_b128(u32x4v{w8[0], w8[1], w8[2], w8[3]}, yrs, off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(u32x4v{w8[4], w8[5], w8[6], w8[7]}, yrs, off + 16, 0, 0);
    }
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

// Heads per workgroup of the resident kernels: a run of hg heads of one
// group, the group's heads split into nsplit runs, with per_cu workgroups
// resident on a CU and a start-up charge (the resident tiles, the first
// copies) of `startup` heads.
static void scan_run_split(const Dims& d, int per_cu, double startup, int* hg_out, int* nsplit_out) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    }
    const int64_t hpg = d.nheads / d.ngroups;
    const double units = (double)d.batch * (double)d.nchunks * (double)d.ngroups;
    const double slots = (double)per_cu * (double)cus;
    int best = (int)hpg;
    double best_cost = 1e300;
    for (int64_t hg = 1; hg <= hpg; ++hg) {
        const int64_t ns = (hpg + hg - 1) / hg;
        const double rounds = std::ceil(units * (double)ns / slots);
        const double cost = rounds * ((double)hg + startup);
        if (cost < best_cost - 1e-9) { best_cost = cost; best = (int)hg; }
    }
    *hg_out = best;
    *nsplit_out = (int)((hpg + best - 1) / best);
}

void chunk_scan_runs(const Dims& d, int* hg, int* nsplit) {
    // the paired kernel pays for its start-up (each wave's 5 or 4 G^T tiles
    // and the first head's copies) once per run of heads, one workgroup per
    // CU; the short-chunk kernels take three (Q = 64: 4 waves, 49 KB of LDS)
    // or one (Q = 128: 8 waves, 66 KB) per CU
    if (d.chunk == 256) scan_run_split(d, 1, 1.5, hg, nsplit);
    else if (d.chunk == 64) scan_run_split(d, 3, 1.0, hg, nsplit);
    else scan_run_split(d, 1, 1.0, hg, nsplit);
}

int x_keep_positions(const Dims& d) {
    // the chunk scan takes run position k of every run at about the same
    // time, so ordinary (cache-allocating) x reads for the first positions
    // give its first heads' x from the last-level cache; budget: ~5/8 of the
    // cache, leaving room for what the kernels between allocate
    int hg = 0, nsplit = 0;
    chunk_scan_runs(d, &hg, &nsplit);
    const double per_position = (double)d.batch * (double)d.seqlen * (double)d.headdim * 2.0 *
                                (double)d.ngroups * (double)nsplit;
    const double k = std::floor(0.625 * kLastLevelCacheBytes / per_position);
    return (int)std::min<double>(k, (double)hg);
}

hipError_t launch_chunk_scan(const Dims& d, int32_t dtype, const void* x, const void* B,
                             const void* C, const float* cs, const float* dtc, const void* Hin,
                             const float* D, void* y, hipStream_t stream, const void* z) {
    if (mfma_path(dtype, d)) {
        const bf16_t* xb = static_cast<const bf16_t*>(x);
        const bf16_t* bb = static_cast<const bf16_t*>(B);
        const bf16_t* cb = static_cast<const bf16_t*>(C);
        const bf16_t* hb = static_cast<const bf16_t*>(Hin);
        bf16_t* yb = static_cast<bf16_t*>(y);
        const int L = (int)d.seqlen, H = (int)d.nheads, G = (int)d.ngroups, nc = (int)d.nchunks;
        int hg = 0, nsplit = 0;
        chunk_scan_runs(d, &hg, &nsplit);
        const unsigned blocks = (unsigned)(d.batch * nc * G * nsplit);
        if (d.chunk == 256) {
            const bf16_t* zb = static_cast<const bf16_t*>(z);
            if (zb)
                chunk_scan_paired_kernel<false, true><<<blocks, 512, 0, stream>>>(
                    xb, bb, cb, cs, dtc, hb, D, zb, yb, L, H, G, nc, hg, nsplit, RunState{});
            else
                chunk_scan_paired_kernel<false, false><<<blocks, 512, 0, stream>>>(
                    xb, bb, cb, cs, dtc, hb, D, nullptr, yb, L, H, G, nc, hg, nsplit, RunState{});
            return hipGetLastError();   // the gate, if any, is inside
        }
        if (d.chunk == 64) {
            chunk_scan_short_kernel<64, 2><<<blocks, 256, 0, stream>>>(xb, bb, cb, cs, dtc, hb, D, yb, L, H, G,
                                                                    nc, hg, nsplit);
        } else {
            // two slots: three and four (one and two more heads in flight)
            // measured 1-5% slower at the 2.7B, 130M and long-context shapes
            chunk_scan_short_kernel<128, 2><<<blocks, 512, 0, stream>>>(xb, bb, cb, cs, dtc, hb, D, yb, L, H, G,
                                                                     nc, hg, nsplit);
        }
    } else if (dtype == 1) {
        launch_generic_t<bf16_t>(d, x, B, C, cs, dtc, Hin, D, y, stream);
    } else {
        launch_generic_t<float>(d, x, B, C, cs, dtc, Hin, D, y, stream);
    }
    hipError_t e = hipGetLastError();
    // the other kernels store y first; the gate then runs in place
    if (e == hipSuccess && z)
        e = launch_layer_out(d.batch * d.seqlen * d.nheads * d.headdim, dtype, y, z, y, stream);
    return e;
}

hipError_t launch_chunk_scan_runs(const Dims& d, int K, const void* x, const void* B, const void* C,
                                  const float* cs, const float* dtc, const void* T, const void* Hr,
                                  const float* lam, const float* D, void* y, hipStream_t stream,
                                  const void* z) {
    const int L = (int)d.seqlen, H = (int)d.nheads, G = (int)d.ngroups, nc = (int)d.nchunks;
    int hg = 0, nsplit = 0;
    chunk_scan_runs(d, &hg, &nsplit);
    const unsigned blocks = (unsigned)(d.batch * nc * G * nsplit);
    const RunState rs{static_cast<const bf16_t*>(Hr), lam, K, (nc + K - 1) / K};
    const bf16_t* xb = static_cast<const bf16_t*>(x);
    const bf16_t* bb = static_cast<const bf16_t*>(B);
    const bf16_t* cb = static_cast<const bf16_t*>(C);
    const bf16_t* tb = static_cast<const bf16_t*>(T);
    const bf16_t* zb = static_cast<const bf16_t*>(z);
    bf16_t* yb = static_cast<bf16_t*>(y);
    if (zb)
        chunk_scan_paired_kernel<true, true><<<blocks, 512, 0, stream>>>(xb, bb, cb, cs, dtc, tb, D, zb, yb, L, H,
                                                                         G, nc, hg, nsplit, rs);
    else
        chunk_scan_paired_kernel<true, false><<<blocks, 512, 0, stream>>>(xb, bb, cb, cs, dtc, tb, D, nullptr, yb,
                                                                          L, H, G, nc, hg, nsplit, rs);
    return hipGetLastError();
}

}  // namespace ssd
