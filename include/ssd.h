/*
 * ssd.h - C ABI of the MI355X (gfx950) Mamba-2 SSD chunked-scan forward.
 *
 * The operation (per batch row r and head h):
 *
 *     H_t = a_t * H_{t-1} + x_t B_t^T,    y_t = H_t C_t + D_h x_t,
 *     a_t = exp(dt_t * A_h),  A_h = -exp(A_log_h)
 *
 * with the P x N state H carried across tokens.  The recurrence and its
 * matrix (dual) form Y = [L o (C B^T)] X are defined on "088 Mamba-2: writing
 * the recurrent state as a structured matrix" (wq-win.github.io), sections 2.1
 * and 2.2; the chunked evaluation (quadratic diagonal blocks, states passed
 * between chunks) is its section 2.3 and section 3, and key design 2 of
 * "Mamba-2 - Transformer and SSM share one algebra" (awesome.papernotes.org).
 * The decay a = exp(Delta A) is from the selective-SSM section of the "Mamba"
 * paper story (ai.tomabc.com); the skip term D x from section 2 of "Mamba and
 * state space models" (wang-x-xia.github.io); B and C shared by groups of heads
 * from key design 3 of the papernotes page.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers to dense, contiguous, row-major
 *    arrays in the layouts given below.  The caller allocates and frees every
 *    buffer, including the workspace; the library allocates no memory.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream).
 *    No entry point synchronises the stream; errors raised by the kernels
 *    themselves surface at the caller's next synchronisation.
 *  - Every function returns SSD_OK (0) or a positive SSD_ERR_* code; nothing
 *    aborts and no C++ exception crosses the ABI.  Argument checks run on the
 *    host before any HIP call, so a rejected call has enqueued nothing.
 *  - The library keeps no per-call state; concurrent calls on different
 *    streams with disjoint outputs and workspaces are safe (except
 *    ssd_forward_noalloc, whose calls on one GPU share a static scratch array).
 *  - A call only launches kernels on `stream` (no allocation, memset, copy or
 *    synchronisation), so it may be recorded into a HIP graph by stream capture
 *    and replayed; the captured pointers must stay valid for every replay.
 */
#ifndef SSD_MI355X_H
#define SSD_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_ABI_VERSION 5

/* Element type of x, B and C.  dt, A_log, D, init_state, y and final_state are
 * always fp32.  BF16: bf16 operands, fp32 accumulation; F32: fp32 throughout. */
typedef enum { SSD_DTYPE_F32 = 0, SSD_DTYPE_BF16 = 1 } ssd_dtype_t;

/* flags */
enum {
    /* Euler input scaling: the state is written with dt_t * x_t instead of x_t
     * (B-bar = Delta B).  D still multiplies the unscaled x_t.  Off by default:
     * the recurrence above has no Delta on x. */
    SSD_FLAG_DT_SCALES_X = 1u << 0,
    /* Step size Delta = softplus(dt + dt_bias[h]) instead of dt + dt_bias[h]
     * (the Mamba block maps its step-size projection plus a learned per-head
     * bias through softplus: the simplified Mamba block pseudocode of the
     * "Mamba" paper story).  softplus(v) = log(1 + e^v), evaluated in fp32. */
    SSD_FLAG_DT_SOFTPLUS = 1u << 1,
    /* Exact zero-order-hold input scaling: the state is written with
     * (exp(Delta A) - 1) / A * x_t, the solution over one step of
     * h' = A h + B x with x and B held constant (the pages name the
     * zero-order hold in section 2 of "Mamba and state space models" without
     * giving B-bar).  D multiplies the unscaled x_t.  Exclusive with
     * SSD_FLAG_DT_SCALES_X (both set: SSD_ERR_UNSUPPORTED). */
    SSD_FLAG_ZOH = 1u << 2
};

enum {
    SSD_OK = 0,
    SSD_ERR_NULL_POINTER = 1,   /* a required pointer is NULL                        */
    SSD_ERR_BAD_SHAPE = 2,      /* negative size, H % G != 0, nseqs inconsistent ... */
    SSD_ERR_UNSUPPORTED = 3,    /* (dtype, headdim, dstate, chunk_len) not built      */
    SSD_ERR_ALIGNMENT = 4,      /* a tensor pointer is not 16-byte aligned            */
    SSD_ERR_WORKSPACE = 5,      /* workspace NULL or smaller than ssd_workspace_size  */
    SSD_ERR_ALIAS = 6,          /* an output overlaps an input or the other output    */
    SSD_ERR_HIP = 7,            /* a HIP runtime call or kernel launch failed         */
    SSD_ERR_NO_DEVICE = 8,      /* no HIP device is available                         */
    SSD_ERR_SCRATCH = 9         /* ssd_forward_noalloc: the problem needs more scratch
                                   than SSD_NOALLOC_SCRATCH_BYTES                      */
};

/* Size of the static device scratch array of ssd_forward_noalloc (32 MiB). */
#define SSD_NOALLOC_SCRATCH_BYTES (32u << 20)

typedef struct {
    int64_t batch;      /* b: rows                                                  */
    int64_t seqlen;     /* T: tokens per row (may be 0)                             */
    int64_t nheads;     /* H                                                        */
    int64_t headdim;    /* P: channels per head (x and y)                           */
    int64_t dstate;     /* N: state size (B and C)                                  */
    int64_t ngroups;    /* G: B/C groups; head h reads group h / (H / G)            */
    int64_t chunk_len;  /* Q: chunk length of the block algorithm (see below)      */
    int64_t nseqs;      /* number of sequences: == batch without seq_idx            */
    int32_t dtype;      /* ssd_dtype_t                                              */
    uint32_t flags;     /* SSD_FLAG_*                                               */
    int32_t segments;   /* segments per row for the split-row path of ssd_forward and
                           ssd_backward: 0 lets the library choose (the default);
                           n > 0 forces n (clamped to the row's blocks), 1 no split.
                           A scheduling choice only: every value gives the same
                           function.  Must be >= 0                                  */
    int32_t reserved;   /* must be 0                                                */
} ssd_problem_t;

/* Host-only check of a problem description (no HIP call).  Supported builds:
 *   BF16: headdim in {32, 64}, dstate in {64, 128, 256}
 *   F32 : headdim in {16, 32, 64}, dstate in {16, 32, 64, 128}
 * chunk_len: 16, 32, or any positive multiple of 64.  The chunk length does
 * not change the function computed (every chunking of the sequence gives the
 * same y and final state up to rounding, section 1 of "088 Mamba-2"); the
 * kernel evaluates the sequence in blocks of 32 rows (chunk_len 16 or 32) or 64
 * rows (multiples of 64), passing the state between blocks (the past-to-future
 * parts of a diagonal block are low rank, exactly as between chunks).
 * A negative `segments` gives SSD_ERR_BAD_SHAPE, a nonzero `reserved`
 * SSD_ERR_UNSUPPORTED. */
int ssd_validate(const ssd_problem_t* p);

/* Bytes of device workspace ssd_forward needs for this problem; 0 when it needs
 * none (then workspace may be NULL) or when the problem is invalid.  A row is
 * scanned in one pass with every intermediate (C.B^T tiles, decays, the
 * carried state) on chip, unless there are at most 128 (row, head) items and
 * rows of at least 16 blocks (block: 64 tokens, or 32 for chunk_len < 64):
 * then rows are cut into segments that run in parallel, and the workspace holds
 * each segment's state (fp32 P x N) and carried decay, (batch, nheads,
 * segments - 1) of each.  The chunked algorithm's inter-chunk state passing at
 * segment granularity (section 3 of "088 Mamba-2"; key design 2 on the
 * papernotes page).  Depends on the problem only (its `segments` field forces
 * the number of segments per row); the contents need no initialisation. */
size_t ssd_workspace_size(const ssd_problem_t* p);

/* Full forward on `stream`: one kernel launch, or three when rows are split
 * into segments (see ssd_workspace_size).
 *   x          (batch, seqlen, nheads, headdim)   dtype
 *   dt         (batch, seqlen, nheads)            fp32: the step sizes, or with SSD_FLAG_DT_SOFTPLUS
 *                                                 their pre-activation (any real value)
 *   dt_bias    (nheads)                           fp32 added to dt before the step-size map, or NULL (= 0)
 *   A_log      (nheads)                           fp32; A_h = -exp(A_log[h])
 *   B, C       (batch, seqlen, ngroups, dstate)   dtype
 *   D          (nheads)                           fp32, or NULL for no skip term
 *   init_state (nseqs, nheads, headdim, dstate)   fp32, or NULL for zero initial states
 *   seq_idx    (batch, seqlen)                    int32 or NULL
 *   y          (batch, seqlen, nheads, headdim)   fp32 output
 *   final_state(nseqs, nheads, headdim, dstate)   fp32 output, or NULL
 *   workspace / workspace_bytes                   >= ssd_workspace_size(p) bytes, 256-byte aligned
 *                                                 (NULL / 0 when that size is 0)
 *
 * seq_idx packs independent sequences into rows: seq_idx[r][t] is the id of
 * the sequence token t of row r belongs to.  Ids are nondecreasing along each
 * row, global over the batch (0 .. nseqs-1), and no id appears in two rows.
 * At the first token of sequence k the state is replaced by init_state[k] (or
 * zero) and then updated by that token; final_state[k] is the state after the
 * last token of k.  No state crosses a sequence boundary.  Without seq_idx,
 * row r is sequence r (nseqs must equal batch).  Ids outside 0..nseqs-1 are
 * clamped (memory-safe, values undefined).  final_state rows of ids that never
 * occur are not written.  final_state may be the same buffer as init_state
 * (in-place state carry) only without seq_idx and when ssd_workspace_size(p)
 * is 0 (each row scanned in one piece): then every state element is read and
 * later written by the same wave.  With seq_idx, or with rows split into
 * segments that run concurrently, an in-place call is rejected with
 * SSD_ERR_ALIAS, as is any other overlap between an output and an input.
 * A row of seqlen 0 leaves its final state equal to its initial state. */
int ssd_forward(const ssd_problem_t* p,
                const void* x, const float* dt, const float* dt_bias, const float* A_log,
                const void* B, const void* C, const float* D,
                const float* init_state, const int32_t* seq_idx,
                float* y, float* final_state,
                void* workspace, size_t workspace_bytes, void* stream);

/* ssd_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, semantics, kernels and results as
 * ssd_forward, minus workspace / workspace_bytes: when the problem needs a
 * workspace (ssd_workspace_size(p) > 0: rows split into segments), the
 * library's own file-scope device array of SSD_NOALLOC_SCRATCH_BYTES stands in
 * for it.  A problem that needs more (ssd_workspace_size(p) >
 * ssd_noalloc_scratch_bytes()) is rejected with SSD_ERR_SCRATCH before any HIP
 * call.  The call itself allocates nothing: no hipMalloc, no hipFree, no
 * allocating library routine.  Each GPU the library runs on holds its own copy
 * of the array until the process ends; its device address is looked up once
 * per device, on the first call that needs it.  Every call on one GPU shares
 * that GPU's array, and the contents of the previous call are left in it (the
 * kernels write every scratch element they read, so nothing needs clearing):
 * calls that overlap in time on one GPU (on different streams, or from
 * different threads without ordering) race on the scratch and must not be
 * issued. */
int ssd_forward_noalloc(const ssd_problem_t* p,
                        const void* x, const float* dt, const float* dt_bias, const float* A_log,
                        const void* B, const void* C, const float* D,
                        const float* init_state, const int32_t* seq_idx,
                        float* y, float* final_state, void* stream);

/* SSD_NOALLOC_SCRATCH_BYTES, as built into the loaded library. */
size_t ssd_noalloc_scratch_bytes(void);

/* One token of the recurrence (decoding), for every row and head, on the
 * fp32 state in place:
 *     state <- a * state + x B^T,   y = state C + D x,   a = exp(dt * A_h)
 * exactly ssd_forward with seqlen 1, init_state = final_state = state (the
 * recurrence of "088 Mamba-2", section 2.1, one step at a time; a chunked
 * prefill followed by steps continues the same sequence).
 *   p          problem with seqlen == 1 and nseqs == batch (chunk_len any valid value)
 *   x          (batch, 1, nheads, headdim)   dtype
 *   dt         (batch, 1, nheads)            fp32
 *   dt_bias    (nheads) fp32, or NULL
 *   A_log      (nheads)                      fp32
 *   B, C       (batch, 1, ngroups, dstate)   dtype
 *   D          (nheads) fp32, or NULL
 *   state      (batch, nheads, headdim, dstate) fp32, read and written (required)
 *   y          (batch, 1, nheads, headdim)   fp32 output
 * The flags (Euler or zero-order-hold input scaling, softplus step size) and
 * dt_bias apply as in ssd_forward.  One kernel launch; bound by
 * reading and writing the state once.  y and state must not overlap each other
 * or any input (SSD_ERR_ALIAS). */
int ssd_step(const ssd_problem_t* p,
             const void* x, const float* dt, const float* dt_bias, const float* A_log,
             const void* B, const void* C, const float* D,
             float* state, float* y, void* stream);

/* Bytes of device workspace ssd_backward needs (0 if the problem is invalid):
 * per-token scalars and dt transposed to (batch, nheads, seqlen), per-(sequence,
 * head) scalars, a table of the packed sequences, and, when a group holds more than one
 * head, each head's dB and dC contribution, (batch, seqlen, nheads, dstate)
 * each in the input type (bf16 or fp32), before the fp32 sum over the group;
 * and each 64-token (bf16) or 32-token (fp32) block's incoming state,
 * (batch, nheads, blocks, headdim, dstate) in the input type.  The contents need no
 * initialisation. */
size_t ssd_backward_workspace_size(const ssd_problem_t* p);

/* Gradients of the forward map (training).  For a scalar loss L with
 * dL/dy = dy and dL/dfinal_state = dfinal (NULL: L does not depend on the
 * final states), writes dL/d(every input).  The pages give no backward
 * algorithm: this is the chain rule applied to the recurrence of "088
 * Mamba-2" (section 2.1), G_t = dL/dS_t = dy_t C_t^T + a_{t+1} G_{t+1},
 * evaluated with the same block (dual) form as the forward (sections 2.2-3).
 *   inputs     as ssd_forward (same problem, flags and tensors), plus
 *   dy         (batch, seqlen, nheads, headdim)   fp32
 *   dfinal     (nseqs, nheads, headdim, dstate)   fp32, or NULL
 *   outputs (fp32):
 *   dx         (batch, seqlen, nheads, headdim)
 *   ddt        (batch, seqlen, nheads)     with respect to the dt input (through softplus if flagged)
 *   dA_log     (nheads)
 *   dB, dC     (batch, seqlen, ngroups, dstate)   summed over the heads of each group
 *   dD         (nheads), or NULL
 *   dinit      (nseqs, nheads, headdim, dstate), or NULL (the gradient with respect to
 *              init_state, also when init_state is NULL, i.e. at a zero initial state)
 *   ddt_bias   (nheads), or NULL
 *   workspace  >= ssd_backward_workspace_size(p) bytes, 256-byte aligned
 * With seq_idx (packed sequences, as in ssd_forward) dfinal and dinit are per
 * sequence; a sequence id that does not occur gets dinit = 0.  Each (sequence,
 * head) is walked on its own, in blocks aligned to the sequence's first token;
 * a device-side table of the sequences is built from seq_idx first (the host
 * never reads it).  Supported shapes: BF16 headdim 32 or 64 with dstate 64,
 * 128 or 256; F32 headdim 16, 32 or 64 with dstate 16 .. 128.  Outputs must not
 * overlap any input, the workspace or each other (SSD_ERR_ALIAS).  x, B, C, dy,
 * dx, dB, dC, init_state, dfinal and dinit need 16-byte alignment, the rest 4.
 * Two kernel launches walk each (row, head) once forwards and once backwards
 * with the state on chip; then, with more than one head per group, a sum of the
 * heads' dB and dC; then the per-head sums over rows.  Per-head sums are taken in
 * a fixed order, so results are deterministic. */
int ssd_backward(const ssd_problem_t* p,
                 const void* x, const float* dt, const float* dt_bias, const float* A_log,
                 const void* B, const void* C, const float* D,
                 const float* init_state, const int32_t* seq_idx,
                 const float* dy, const float* dfinal,
                 float* dx, float* ddt, float* dA_log, float* dB, float* dC,
                 float* dD, float* dinit, float* ddt_bias,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Static description of an error code. */
const char* ssd_strerror(int status);

/* SSD_ABI_VERSION of the loaded library. */
int ssd_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SSD_MI355X_H */
