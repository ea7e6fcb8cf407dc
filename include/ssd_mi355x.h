/*
 * ssd_mi355x.h -- C ABI of the MI355X (gfx950) selective-scan library.
 *
 * The library evaluates the selective state space model with one scalar decay
 * per head (the Mamba-2 "state space duality" layer):
 *
 *     a_t        = exp(dt[b,t,h] * A[h])
 *     h_t[p][n]  = a_t * h_{t-1}[p][n] + dt[b,t,h] * x[b,t,h,p] * B[b,t,g,n]
 *     y[b,t,h,p] = sum_n C[b,t,g,n] * h_t[p][n] + D[h] * x[b,t,h,p]
 *
 * with g = h / (H / G) the B/C group of head h and h_{-1} the initial state.
 *
 * Sources (page title, section):
 *  - discrete recurrence with zero-order-hold decay exp(Delta A) and input
 *    scaled by Delta B: "State Space Model" (book.paithon.it), "Un sistema che
 *    riassume il passato"; "State Space Models (SSM)" (ultralytics.com),
 *    "Come funzionano gli SSM";
 *  - scalar transition a_t I, equal to masked linear attention without
 *    softmax: "State Space Model", "Due strade, una meta" and "Da ricordare";
 *  - y = C h + D x: "Puntata 205 -- State Space Models e Mamba"
 *    (aiperbabbani.it), "Cos'e' un SSM, in 30 secondi";
 *  - per-token Delta, B, C (selectivity): same page, "Mamba (Gu & Dao,
 *    dicembre 2023): selective scan";
 *  - the block algorithm evaluated by ssd_forward -- quadratic masked form
 *    inside each chunk, only the summary state carried between chunks --
 *    "Mamba-2 (2024): SSM e attention sono la stessa cosa" (paithon.it),
 *    "Il trucco a blocchi"; "Architektury Mamba-2, State Space Models i
 *    liniowa atencja..." (tech.tersel.eu), "Rewolucja Mamba-2 i teoria State
 *    Space Duality SSD";
 *  - two ways to run one model: all tokens at once to train / prefill, one
 *    token at a time with a fixed-size state to generate: "State Space
 *    Model", "Un sistema che riassume il passato" (end of the water-tank
 *    passage); tech.tersel.eu, "Porownanie zlozonosci obliczeniowej i
 *    zachowania pamieci" (constant memory while generating).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer to a contiguous row-major
 *    array; the caller allocates and owns all memory, including the
 *    workspace.  The library allocates nothing and keeps no pointer after a
 *    call returns; apart from ssd_forward_noalloc's per-device array (see
 *    there) it has no mutable global state, so calls are reentrant.
 *  - Work is enqueued on `stream` (NULL = the null stream) and the call
 *    returns at once.  SSD_OK means every kernel was launched; results are
 *    valid once the stream has completed.  No call synchronises.
 *  - All arguments are checked before any launch.  An error is reported as a
 *    status code; no exception crosses the ABI and nothing is written.
 *  - Alignment: x, B, C, y, states and workspace must be 16-byte aligned;
 *    dt, A and D 4-byte aligned (SSD_ERR_ALIGN otherwise).
 *  - dtype (ssd_dtype) is the storage type of x, B, C and y.  dt, A, D and
 *    every state are fp32.  Arithmetic is fp32 (bf16 operands of the matrix
 *    instructions, fp32 accumulation and fp32 states).
 *  - Preconditions that are documented, not checked on the device:
 *    dt >= 0, A <= 0, finite inputs.  NaN/Inf propagate.
 *  - Layouts (B = batch, L = seqlen, H = nheads, P = headdim, N = dstate,
 *    G = ngroups, Q = chunk, nc = ceil(L / Q)):
 *        x, y      [B][L][H][P]        dt        [B][L][H]
 *        Bm, Cm    [B][L][G][N]        A, D      [H]
 *        init, final, state            [B][H][P][N]
 *  - H must be a multiple of G.  L may be any length >= 1; the last chunk may
 *    be partial.
 *  - Supported shapes (ssd_forward and the stage calls): either dtype with
 *    1 <= P <= 128, 1 <= N <= 128, 1 <= Q <= 256; bf16 with P = 64, N = 128
 *    and Q in {64, 128, 256} runs on the matrix cores, everything else on
 *    the vector units.  Anything else returns SSD_ERR_UNSUPPORTED.
 */
#ifndef SSD_MI355X_H
#define SSD_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_ABI_VERSION 8

typedef enum { SSD_DTYPE_F32 = 0, SSD_DTYPE_BF16 = 1 } ssd_dtype;

typedef enum {
    SSD_OK = 0,
    SSD_ERR_NULL = 1,        /* a required pointer is NULL                         */
    SSD_ERR_SHAPE = 2,       /* a size is < 1, H % G != 0, or sizes overflow         */
    SSD_ERR_UNSUPPORTED = 3, /* (dtype, P, N, chunk) not compiled in                 */
    SSD_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than required              */
    SSD_ERR_ALIGN = 5,       /* a pointer is not aligned as stated above             */
    SSD_ERR_HIP = 6,         /* a kernel launch failed (hipGetLastError)             */
    SSD_ERR_ALIAS = 7        /* an output overlaps an input it must not overlap      */
} ssd_status;

/* Version of this ABI (SSD_ABI_VERSION). */
int32_t ssd_abi_version(void);

/* Static, NUL-terminated description of a status code.  Never NULL. */
const char* ssd_status_str(int32_t status);

/*
 * Bytes of device workspace ssd_forward needs for these sizes, or 0 if the
 * sizes are invalid or unsupported.  The workspace holds, each region
 * 256-byte aligned and in this order:
 *     cs   fp32 [B][H][nc][Q]  log2(e) * inclusive prefix of dt*A in the chunk
 *     dtc  fp32 [B][H][nc][Q]  dt rearranged head-major (0 past the end)
 *     S    [B][H][nc][P][N]    each chunk's end state, starting from zero
 *     Hin  [B][H][nc][P][N]    state entering each chunk
 * S and Hin are in the storage type (bf16 for bf16, fp32 for fp32): each is
 * written once and read once, as a summand of the fp32 carried state (S) or
 * a matrix operand (Hin); the carried state itself stays fp32.  Where the
 * two-level recurrence between chunks applies (see ssd_chunk_state_runs) the
 * forward carves the same workspace as cs, dtc, T [B][H][nc][P][N],
 * Hr [B][H][nruns][P][N], lam [B][H][nc], rdec [B][H][nruns] instead, and the
 * size returned is the larger of the two layouts.  The run length (and so
 * the size) is chosen for the device current at the call: a workspace sized
 * on a device with fewer CUs than the one the forward runs on can be too
 * small there (SSD_ERR_WORKSPACE, nothing launched).
 */
size_t ssd_forward_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads,
                                   int64_t headdim, int64_t dstate, int64_t ngroups,
                                   int64_t chunk, int32_t dtype);

/*
 * Whole-sequence forward (training / prefill): y and the final state from x,
 * dt, A, B, C, D and an optional initial state, by the block algorithm with
 * chunk length `chunk` (see the block-algorithm sources above).  Runs, in
 * order on `stream`: ssd_chunk_cumsum, ssd_chunk_state, ssd_state_passing,
 * ssd_chunk_scan (the cumsum inside the chunk-state launch where the
 * paired-head matrix-core kernel applies); where the two-level recurrence
 * applies (bf16, P = 64, N = 128, chunk 256, an even head count per group)
 * ssd_chunk_state_runs, ssd_run_passing and ssd_chunk_scan_runs instead.
 *   D           may be NULL: no skip term.
 *   init_state  may be NULL: zero initial state.  When given it is decayed by
 *               exp(dt_0 A) at the first token, like any carried state.
 *   final_state may be NULL: not written.  It may alias init_state (the
 *               state is read before it is overwritten); it must not overlap
 *               any other input, y or the workspace (SSD_ERR_ALIAS).
 *   y           must not overlap any input (x, dt, A, B, C, D, init_state),
 *               final_state or the workspace (SSD_ERR_ALIAS).
 *   workspace   at least ssd_forward_workspace_bytes(...) bytes; it must not
 *               overlap any input or output (SSD_ERR_ALIAS).
 */
int32_t ssd_forward(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                    int64_t dstate, int64_t ngroups, int64_t chunk, int32_t dtype,
                    const void* x, const float* dt, const float* A, const void* B,
                    const void* C, const float* D, const float* init_state, void* y,
                    float* final_state, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/*
 * ssd_forward followed by the gate of the block around the scan: y receives
 * (C h + D x) * silu(z), z [B][L][H][P] in the storage type -- the output
 * gate of a Mamba block (page "State Space Models (SSM)", section "Da S4 a
 * Mamba"; ssd_layer_out computes the same).  Where the 256-token matrix-core
 * chunk scan runs, the gate is applied inside its store (y is never stored
 * ungated; z is read there instead of a separate pass over y, z and out),
 * elsewhere by the gate kernel in place after the scan.  Either way the
 * result is what ssd_forward then ssd_layer_out(y, z, out = y) give, bit for
 * bit.  z must not overlap y, final_state or the workspace (SSD_ERR_ALIAS);
 * z NULL is SSD_ERR_NULL.  Everything else as ssd_forward.
 */
int32_t ssd_forward_gated(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                          int64_t dstate, int64_t ngroups, int64_t chunk, int32_t dtype,
                          const void* x, const float* dt, const float* A, const void* B,
                          const void* C, const float* D, const float* init_state, const void* z,
                          void* y, float* final_state, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * ssd_forward for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * computation, arguments and errors without the workspace arguments.  The
 * workspace is a device array of SSD_NOALLOC_SCRATCH_BYTES that the library
 * holds on every device it runs on until the process ends; the call itself
 * allocates nothing.  Sizes whose workspace (ssd_forward_workspace_bytes)
 * exceeds it return SSD_ERR_WORKSPACE before any launch: 64 MiB holds, for
 * example, the Mamba-2-130M-shaped layer (batch 8, 2,048 tokens, 24 heads of
 * 64, N = 128, chunk 256).  Every call on one device shares that device's
 * array: calls whose executions overlap on one device (other streams, other
 * threads) race and must be serialised by the caller.  Nothing in the array
 * has to start at zero; it keeps whatever the last call left there.
 */
#define SSD_NOALLOC_SCRATCH_BYTES (64u << 20)
int32_t ssd_forward_noalloc(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                            int64_t dstate, int64_t ngroups, int64_t chunk, int32_t dtype,
                            const void* x, const float* dt, const float* A, const void* B,
                            const void* C, const float* D, const float* init_state, void* y,
                            float* final_state, hipStream_t stream);

/*
 * ssd_forward with the exact zero-order hold for the input term: the step
 * adds expm1(dt A) / A * x (outer) B instead of dt * x (outer) B (dt itself
 * where A = 0), i.e. Bbar = (Abar - 1) / A B, the discretisation of the
 * recurrent-versus-convolutional demonstration on page "State Space Models
 * (SSM)" (ultralytics.com glossary), section "Come funzionano gli SSM".  The
 * decay exp(dt A) is unchanged.  Same arguments, layouts, ownership and
 * errors as ssd_forward; the workspace's dtc region holds the weights.
 */
int32_t ssd_forward_zoh(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                        int64_t dstate, int64_t ngroups, int64_t chunk, int32_t dtype,
                        const void* x, const float* dt, const float* A, const void* B,
                        const void* C, const float* D, const float* init_state, void* y,
                        float* final_state, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * One decode step for every (batch, head) -- one token of generation with a
 * fixed-size state ("State Space Model", "Un sistema che riassume il
 * passato"; tech.tersel.eu, constant memory while generating):
 *     a = exp(dt_t[b,h] A[h]);  state = a state + dt_t x_t (outer) B_t;
 *     y_t = C_t . state + D x_t
 *   state  fp32 [B][H][P][N], read and written in place.
 *   x_t, y_t [B][H][P] (dtype)   dt_t fp32 [B][H]   B_t, C_t [B][G][N] (dtype)
 *   A, D   fp32 [H]; D may be NULL.
 * The signature adds A, D and y_t to (state, x_t, dt_t, B_t, C_t): the
 * recurrence needs the decay and the skip term, and the step's output.
 * Supported: any P <= 1024, N <= 1024 (fast path when N is a multiple of 4
 * and N / 4 divides 64).
 */
int32_t ssm_step(int64_t batch, int64_t nheads, int64_t headdim, int64_t dstate,
                 int64_t ngroups, int32_t dtype, float* state, const void* x_t,
                 const float* dt_t, const float* A, const void* B_t, const void* C_t,
                 const float* D, void* y_t, hipStream_t stream);

/*
 * ssm_step with the exact zero-order hold: state = a state + w x_t (outer)
 * B_t with w = expm1(dt_t A) / A (dt_t where A = 0), as in ssd_forward_zoh.
 * Same arguments, layouts and errors as ssm_step.
 */
int32_t ssm_step_zoh(int64_t batch, int64_t nheads, int64_t headdim, int64_t dstate,
                     int64_t ngroups, int32_t dtype, float* state, const void* x_t,
                     const float* dt_t, const float* A, const void* B_t, const void* C_t,
                     const float* D, void* y_t, hipStream_t stream);

/*
 * The four stages of ssd_forward, callable one by one (per-stage checks and
 * timing).  Arrays named after the workspace regions have the layouts given
 * at ssd_forward_workspace_bytes.  Every stage call returns SSD_ERR_ALIAS,
 * before any launch, when one of its outputs overlaps one of its inputs or
 * another of its outputs; the one permitted overlap is final_state on
 * init_state (each entry is read before it is written).
 */

/* cs, dtc from dt and A: the per-chunk inclusive prefix of dt * A, scaled by
 * log2(e), and dt rearranged head-major.  Past the end of the sequence cs
 * repeats its last value and dtc is 0.  (Decay weights multiply along the
 * sequence -- the fading weights 1, 1/2, 1/4 ... of the water-tank example,
 * "State Space Model", "Un sistema che riassume il passato" -- so their
 * logarithms add up.) */
int32_t ssd_chunk_cumsum(int64_t batch, int64_t seqlen, int64_t nheads, int64_t chunk,
                         const float* dt, const float* A, float* cs, float* dtc,
                         hipStream_t stream);

/* ssd_chunk_cumsum for the zero-order hold: cs as above; dtc holds the
 * input weight expm1(dt A) / A (dt where A = 0), evaluated in fp64 and
 * rounded once (see ssd_forward_zoh). */
int32_t ssd_chunk_cumsum_zoh(int64_t batch, int64_t seqlen, int64_t nheads, int64_t chunk,
                             const float* dt, const float* A, float* cs, float* dtc,
                             hipStream_t stream);

/* S [B][H][nc][P][N] in the storage type: each chunk's end state from a
 * zero start, S_c[p][n] = sum_j exp(Acs_last - Acs_j) dt_j x_j[p] B_j[n]
 * ("Il trucco a blocchi": only a summary state leaves a block), accumulated
 * in fp32 and rounded once. */
int32_t ssd_chunk_state(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                        int64_t dstate, int64_t ngroups, int64_t chunk, int32_t dtype,
                        const void* x, const void* B, const float* cs, const float* dtc,
                        void* S, hipStream_t stream);

/* cs, dtc and S from dt, A, x and B: ssd_chunk_cumsum followed by
 * ssd_chunk_state, as ssd_forward runs them -- one launch where the bf16
 * matrix-core chunk-state kernel takes two heads per workgroup (the cumsum
 * then runs in its prologue and writes the same cs and dtc), two launches
 * otherwise.  Same layouts and checks as the two calls. */
int32_t ssd_chunk_cumsum_state(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                               int64_t dstate, int64_t ngroups, int64_t chunk, int32_t dtype,
                               const void* x, const void* B, const float* dt, const float* A,
                               float* cs, float* dtc, void* S, hipStream_t stream);

/* Hin and final_state from S (both in the storage type of `dtype`): the
 * linear recurrence between chunks in fp32, H_0 = init (or 0), Hin_c = H_c,
 * H_{c+1} = exp(Acs_last) H_c + S_c, final = H_nc.  init_state /
 * final_state may be NULL and may alias. */
int32_t ssd_state_passing(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                          int64_t dstate, int64_t chunk, int32_t dtype, const void* S,
                          const float* cs, const float* init_state, void* Hin,
                          float* final_state, hipStream_t stream);

/* The same outputs as ssd_state_passing, by a two-level associative scan:
 * two steps of a linear recurrence merge into one step of the same kind
 * (page "State Space Model", book.paithon.it, section "Dai sistemi dinamici a
 * Mamba", the parallel scan), so the nc chunks are cut into segments of
 * ceil(nc / nsegments) chunks (fewer segments if that leaves some empty);
 * each segment's end state from zero and its summed decay are formed in
 * parallel, a short chain over the segments gives the state entering each
 * one, and every segment is walked again from that state to write Hin.  The
 * depth is about nc / nsegments + nsegments steps instead of nc, for 1.5x the
 * reads of S.  Results equal ssd_state_passing's up to rounding order.
 * nsegments: 1 .. 65535 (values above nc act as nc).  workspace: device
 * memory of at least ssd_state_passing_seg_workspace_bytes(batch, nheads,
 * headdim, dstate, nsegments) bytes, 256-byte aligned, owned by the caller
 * and free for the call's duration (SSD_ERR_WORKSPACE otherwise).  Other
 * arguments, layouts and errors as ssd_state_passing. */
size_t ssd_state_passing_seg_workspace_bytes(int64_t batch, int64_t nheads, int64_t headdim,
                                             int64_t dstate, int64_t nsegments);
int32_t ssd_state_passing_seg(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                              int64_t dstate, int64_t chunk, int64_t nsegments, int32_t dtype,
                              const void* S, const float* cs, const float* init_state, void* Hin,
                              float* final_state, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * The two-level recurrence between chunks that ssd_forward runs where it
 * applies (bf16, P = 64, N = 128, chunk 256, an even number of heads per
 * group; SSD_ERR_UNSUPPORTED elsewhere).  Two steps of the linear recurrence
 * H_{c+1} = exp(Acs_last,c) H_c + S_c merge into one step of the same kind
 * (page "State Space Model", book.paithon.it, section "Dai sistemi dinamici a
 * Mamba", the parallel scan), so with the chunks cut into runs of
 * run_chunks = K consecutive chunks (run r: chunks rK .. min(rK + K, nc) - 1,
 * nruns = ceil(nc / K); K in 1 .. 65536):
 *     T_c    = the state after chunk c from a zero state at its run's start,
 *     lam_c  = the summed decay (log2 units, as cs) of the run's chunks before c,
 *     rdec_r = the summed decay (log2 units) of run r's chunks,
 *     Hr_0   = init (or 0),  Hr_{r+1} = exp2(rdec_r) Hr_r + T_{last chunk of r},
 *     Hin_c  = Hr_r at a run's first chunk, else T_{c-1} + exp2(lam_c) Hr_r,
 *     final  = exp2(rdec_last) Hr_last + T_{nc-1}.
 * Only every K-th state crosses memory twice; the per-chunk S and Hin never do.
 */

/* The run length K ssd_forward uses at these sizes (2 to 16: the longest
 * whose run walks still fill two rounds of the device's CUs), or 0 where it
 * keeps the per-chunk stages (unsupported sizes included).  The stage calls
 * below with this K run exactly the forward's kernels. */
int64_t ssd_forward_run_chunks(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                               int64_t dstate, int64_t ngroups, int64_t chunk, int32_t dtype);

/* cs and dtc as ssd_chunk_cumsum; T [B][H][nc][P][N] (dtype, accumulated in
 * fp32 and rounded once), lam [B][H][nc] and rdec [B][H][nruns] (fp32). */
int32_t ssd_chunk_state_runs(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                             int64_t dstate, int64_t ngroups, int64_t chunk, int32_t dtype,
                             int64_t run_chunks, const void* x, const void* B, const float* dt,
                             const float* A, float* cs, float* dtc, void* T, float* lam, float* rdec,
                             hipStream_t stream);

/* Hr [B][H][nruns][P][N] (dtype; the chain runs in fp32) and final_state
 * (fp32, may be NULL) from T and rdec; init_state may be NULL and may alias
 * final_state. */
int32_t ssd_run_passing(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                        int64_t dstate, int64_t chunk, int32_t dtype, int64_t run_chunks,
                        const void* T, const float* rdec, const float* init_state, void* Hr,
                        float* final_state, hipStream_t stream);

/* y as ssd_chunk_scan, with each chunk's entering state formed from T, Hr
 * and lam as above (T_{c-1} + exp2(lam_c) Hr_r evaluated in fp32 and rounded
 * once to dtype). */
int32_t ssd_chunk_scan_runs(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                            int64_t dstate, int64_t ngroups, int64_t chunk, int32_t dtype,
                            int64_t run_chunks, const void* x, const void* B, const void* C,
                            const float* cs, const float* dtc, const void* T, const void* Hr,
                            const float* lam, const float* D, void* y, hipStream_t stream);

/* Hin and final_state straight from x, B, cs and dtc: what ssd_chunk_state
 * followed by ssd_state_passing compute, in one pass that keeps the running
 * state on chip and never writes S (the block recurrence of "Il trucco a
 * blocchi" run as the token recurrence of "Un sistema che riassume il
 * passato" with one factor per block).  Same arguments, layouts, aliasing
 * rules (init_state / final_state may be NULL and may alias) and outputs as
 * that pair.  One workgroup walks the whole sequence of each (batch, head
 * pair) where the heads of a group pair up (chunk 128 or 256), of each
 * (batch, head, half of P) otherwise (chunk 256).  Matrix-core path only:
 * dtype bf16, headdim 64, dstate 128; anything else returns
 * SSD_ERR_UNSUPPORTED.  (ssd_forward runs ssd_chunk_state and
 * ssd_state_passing instead: one walk per CU cannot use the whole device's
 * bandwidth, and that pair measured faster.) */
int32_t ssd_state_scan(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                       int64_t dstate, int64_t ngroups, int64_t chunk, int32_t dtype,
                       const void* x, const void* B, const float* cs, const float* dtc,
                       const float* init_state, void* Hin, float* final_state,
                       hipStream_t stream);

/* y from the chunk's own tokens (masked C.B^T weighted by exp(Acs_i - Acs_j)
 * dt_j, the attention-like quadratic form), the carried state
 * (exp(Acs_i) Hin_c C_i) and D x. */
int32_t ssd_chunk_scan(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                       int64_t dstate, int64_t ngroups, int64_t chunk, int32_t dtype,
                       const void* x, const void* B, const void* C, const float* cs,
                       const float* dtc, const void* Hin, const float* D, void* y,
                       hipStream_t stream);

/*
 * The steps a Mamba block puts around the scan: each block wraps the selective
 * SSM with a short convolution and a SiLU gate, and Delta, B, C depend on the
 * current token (page "State Space Models (SSM)", ultralytics.com glossary,
 * section "Da S4 a Mamba").  silu(v) = v / (1 + exp(-v)),
 * softplus(v) = log(1 + exp(v)).
 *
 * ssd_layer_in: the scan's inputs from the block's pre-activations.
 *   xbc     [B][L][Cd] (dtype), Cd = H P + 2 G N: the channels of x (head
 *           major, then p), then of B (group major, then n), then of C.
 *   conv_w  fp32 [Cd][K], 1 <= K <= 8: a depthwise causal filter per channel;
 *           tap k weighs the input K - 1 - k tokens back (tap K - 1 is the
 *           current token); inputs before the first token are zero.
 *   conv_b  fp32 [Cd] or NULL (no bias).
 *   dt_raw  fp32 [B][L][H];  dt_bias fp32 [H] or NULL.
 *   outputs x [B][L][H][P], B and C [B][L][G][N] (dtype):
 *           silu(conv_b + filter * xbc) split by channel;
 *           dt fp32 [B][L][H] = softplus(dt_raw + dt_bias).
 *   The outputs must not overlap the inputs or each other (SSD_ERR_ALIAS).
 *   Errors: SSD_ERR_SHAPE (non-positive sizes, H % G, batch > 65535,
 *   Cd > 134215680, batch L Cd > 1e12),
 *   SSD_ERR_UNSUPPORTED (dtype, K), SSD_ERR_NULL, SSD_ERR_ALIGN (element
 *   alignment).  8-channel vector accesses are used when H P and G N are
 *   multiples of 8 and the arrays are 16-byte aligned.
 */
int32_t ssd_layer_in(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                     int64_t dstate, int64_t ngroups, int64_t kernel_width, int32_t dtype,
                     const void* xbc, const float* conv_w, const float* conv_b,
                     const float* dt_raw, const float* dt_bias, void* x, void* B, void* C,
                     float* dt, hipStream_t stream);

/*
 * ssd_layer_out: the gate behind the scan, out = y * silu(z), over n
 * elements of dtype (any layout, the same for all three), 1 <= n <= 1e12.
 * out may be y (in place) but must not overlap z or partly overlap y.
 * Errors: SSD_ERR_SHAPE, SSD_ERR_UNSUPPORTED (dtype), SSD_ERR_NULL,
 * SSD_ERR_ALIGN (element alignment), SSD_ERR_ALIAS.
 */
int32_t ssd_layer_out(int64_t n, int32_t dtype, const void* y, const void* z, void* out,
                      hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SSD_MI355X_H */
