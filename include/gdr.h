/*
 * gdr.h — C ABI of libgdr, the MI355X (gfx950) gated delta rule operator.
 *
 * The operator is the Gated Delta Network chunked prefill that the FlashQLA
 * pages centre on ("Main functions" on the aiboss88 page; "Introduction" and
 * "Usage" in the PyPI README).  Per (sequence, v-head) it evaluates
 *
 *     S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = scale * S_t q_t,
 *
 * with the state stored as h = S^T (K x V, the README's state shape
 * [.., H_v, K, V]).  q/k head hq serves v heads hv with hv / (H_v/H_q) == hq.
 * Evaluation is chunked (64 tokens): an in-chunk cumulative log-gate, the
 * strictly lower decayed beta*K K^T matrix A, T = (I + A)^{-1}, and a serial
 * scan over chunks that produces the chunk-start states and the output.
 *
 * The argument lists follow the low-level API of the README ("Usage", "Low-level
 * API"): the forward takes the five input tensors, the output scale, an optional
 * initial state and optional sequence offsets, and hands back five results in
 * the order gate cumsum, A, o, chunk-start states, final state; the backward
 * takes the same inputs plus the forward's gate cumsum and A, the gradients of
 * o and of the final state, and hands back the gradients of q, k, v, beta, g
 * and the initial state, in that order.  Here the forward's gate result is the
 * in-chunk cumulative log-gate and its A is T, one 64-wide row per token.
 *
 * Conventions (all entry points):
 *  - Every pointer in an args struct is a DEVICE pointer unless stated; all
 *    tensors are contiguous row-major in the layouts given, 16-byte aligned.
 *  - The caller allocates and owns every buffer, including the workspace.
 *    The library allocates nothing, holds no state between calls (but for
 *    the static scratch buffer of gdr_fwd_noalloc), never synchronises the
 *    stream and never reads device memory on the host.
 *    Calls on different streams may run concurrently if their buffers do
 *    not overlap.
 *  - Validation happens on the host before any launch.  A non-zero return
 *    means nothing was launched (GDR_ELAUNCH: a launch failed part way).
 *  - NaN/Inf inputs are not checked; they propagate.
 */
#ifndef GDR_H
#define GDR_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDR_ABI_VERSION 7
#define GDR_CHUNK 64
#define GDR_FWD_STAGES 3
#define GDR_BWD_STAGES 4

/* return codes */
#define GDR_OK 0
#define GDR_EINVAL -1     /* null required pointer, bad size, misalignment, H_v % H_q != 0, B != 1 with cu_seqlens,
                             a shape past the launch grids: B T >= 2^31 tokens, or (N + 7) H_q >= 2^24 for
                             the chunk-count bound N of gdr_tblocks_bytes */
#define GDR_ENOTSUP -2    /* K or V not in {64, 128}; unsupported dtype */
#define GDR_EWORKSPACE -3 /* workspace_bytes below what gdr_*_workspace reports */
#define GDR_ELAUNCH -4    /* a HIP launch failed */
#define GDR_ESCRATCH -5   /* gdr_fwd_noalloc: the problem needs more scratch than GDR_SCRATCH_BYTES */

/* size of the static per-device scratch buffer of gdr_fwd_noalloc */
#define GDR_SCRATCH_BYTES ((size_t)256 << 20)

/* element types */
#define GDR_BF16 0
#define GDR_F32 1

/* sequence-split ("AutoCP") modes of the forward.  The pages' AutoCP splits a
   long sequence into segments that run in parallel, each warmed up from a zero
   state over a few chunks before its own (aiboss88 "Core advantages"; efeozkan
   blog "1. Gate-Driven Automatic Intra-Card Context Parallelism (AutoCP)"). */
#define GDR_CP_AUTO 0   /* split where the device model of gdr_fwd predicts a gain (the
                           window priced at one chunk); each segment warms up over a
                           window chosen from its gates: the latest chunk from which the
                           log-gates up to the segment's start sum to -24 ln 2 or less
                           (the zero start is then within 2^-24 of the true state), or
                           the sequence start (exact) when none does.  Safe for gates
                           that do not decay; costs about one chunk of warm-up per
                           segment on gates that decay as the configs' do */
#define GDR_CP_OFF 1    /* exact scan, one segment per sequence */
#define GDR_CP_WARMUP 2 /* always split; each segment warms up from a zero state over
                           cp_warmup_chunks chunks (the pages use 6 to 8): approximate
                           where the gates do not decay within that window */
#define GDR_CP_EXACT 3  /* always split, exactly: each segment's transition matrix and
                           zero-start end state are scanned in parallel, a serial carry
                           over the segments gives their true start states, then the
                           segments run again with output */
#define GDR_CP_AUTO_EXACT 4 /* the exact split where the device model predicts a gain */
#define GDR_CP_AUTO_PAGES 5 /* the pages' trigger and window: split when B*H_v <= 40, or
                               B*H_v <= 56 and T >= 8192 (constants tuned for a 132-SM
                               GPU), warming up over cp_warmup_chunks as GDR_CP_WARMUP */

typedef struct {
    /* sizes.  With cu_seqlens, B must be 1, T is the packed token count and
       n_seq the number of sequences; otherwise n_seq is ignored (= B). */
    int64_t B, T, H_q, H_v, K, V, n_seq;
    int32_t dtype;     /* element type of q, k, v: GDR_BF16 or GDR_F32 */
    int32_t out_dtype; /* element type of o: GDR_F32 or GDR_BF16 */
    float scale;       /* output scale, usually K^-1/2 */
    int32_t cp_mode;           /* GDR_CP_* */
    int32_t cp_segment_chunks; /* split mode: chunks per segment; 0 = chosen for the device
                                  (see gdr_fwd) */
    int32_t cp_warmup_chunks;  /* split mode: warm-up window in chunks, 0 = 8 */
    /* inputs */
    const void *q;              /* [B,T,H_q,K] dtype */
    const void *k;              /* [B,T,H_q,K] dtype; each row should have unit L2 norm */
    const void *v;              /* [B,T,H_v,V] dtype */
    const float *g;             /* [B,T,H_v] per-token log-decay (<= 0 for decay) */
    const float *beta;          /* [B,T,H_v] */
    const float *initial_state; /* [N,H_v,K,V], N = B or n_seq; NULL = zeros */
    const int32_t *cu_seqlens;  /* [n_seq+1] token offsets: 0, non-decreasing, T last; or NULL.
                                   The library reads them on the device only and clamps
                                   each entry to [previous entry, T] (the first to [0, T])
                                   before any kernel uses them, so offsets outside that
                                   range cannot make a kernel touch memory past the
                                   tensors; the results are then those of the clamped
                                   offsets.  Callers validate them where they are on the
                                   host (the Python binding does) */
    /* outputs */
    void *o;                    /* [B,T,H_v,V] out_dtype */
    float *final_state;         /* [N,H_v,K,V]; NULL = not wanted */
    float *g_cum;               /* [B,T,H_v] in-chunk cumulative log-gate; NULL = kept in workspace */
    float *A;                   /* [B,T,H_v,64] row r of the token's chunk of T = (I+A)^{-1},
                                   zero past the chunk end; NULL = kept in workspace */
    float *h;                   /* [NT,H_v,K,V] chunk-start states (NT = sum of ceil(len/64));
                                   NULL = not written */
    void *h_bwd;                /* [NT,H_v] chunk-start states in the backward's layout, 4 K V
                                   bytes each: fp32 [K][V] for fp32 inputs, for bf16 inputs
                                   bf16 hi then lo planes of h^T [V][K]; passed on as
                                   gdr_bwd_args.h_bwd, it saves the backward's recompute of
                                   the states.  NULL = not written.  The states must be
                                   exact: with h_bwd, GDR_CP_AUTO splits as
                                   GDR_CP_AUTO_EXACT, and h, GDR_CP_WARMUP or
                                   GDR_CP_AUTO_PAGES is GDR_EINVAL */
    void *tblk_bwd;             /* gdr_tblocks_bytes() bytes, or NULL: the per-(chunk, v head)
                                   T blocks (T = (I+A)^{-1} and the chunk's gate scalars) in
                                   the backward's layout; for bf16 inputs the forward's own
                                   blocks (the backward reads the same layout, and they then
                                   take no workspace), for fp32 inputs a second copy; passed
                                   on as gdr_bwd_args.tblk_bwd, they save the backward's
                                   rebuild of them from A and g_cum */
    float *w_out;               /* [B,T,H_v,K] W = T diag(beta e^g_cum) K, NULL = not computed */
    float *u_out;               /* [B,T,H_v,V] U = T diag(beta) V, NULL = not computed */
    /* timing hook: NULL, or a HOST array of 2*GDR_FWD_STAGES events, a start
       and a stop per stage (chunk prep, scan with output, W/U).  They are bound
       to the stage's kernel launches (hipExtLaunchKernel): the start event
       takes the start of the stage's first kernel, the stop event the end of
       its last, with no marker packets between kernels.  A stage that launches
       nothing records both on the stream at once.  A NULL entry is skipped.
       Not for concurrent calls from one host thread (the binding is per
       thread) */
    hipEvent_t *events;
    /* scratch */
    void *workspace;
    size_t workspace_bytes;
} gdr_fwd_args;

typedef struct {
    int64_t B, T, H_q, H_v, K, V, n_seq;
    int32_t dtype;      /* element type of q, k, v, do */
    int32_t grad_dtype; /* element type of dq, dk, dv: GDR_BF16 or GDR_F32 */
    int32_t cp_mode;    /* sequence split of the recurrences: GDR_CP_AUTO or
                           GDR_CP_AUTO_EXACT (split where the device model of gdr_fwd
                           predicts a gain), GDR_CP_OFF or GDR_CP_EXACT; the split is
                           always exact here (GDR_CP_WARMUP is an invalid argument) */
    int32_t cp_segment_chunks; /* chunks per segment; 0 = chosen for the device as in gdr_fwd */
    float scale;
    const void *q, *k, *v;      /* as in gdr_fwd_args */
    const float *g_cum;         /* [B,T,H_v] the forward's g_cum */
    const float *beta;          /* [B,T,H_v] */
    const float *A;             /* [B,T,H_v,64] the forward's A */
    const void *dout;           /* [B,T,H_v,V] gradient of o, dtype */
    const float *dht;           /* [N,H_v,K,V] gradient of final_state; NULL = zeros */
    const float *initial_state; /* [N,H_v,K,V] or NULL */
    const int32_t *cu_seqlens;  /* [n_seq+1] or NULL */
    const void *h_bwd;          /* the forward's h_bwd for the same inputs, or NULL (the states
                                   are then recomputed) */
    const void *tblk_bwd;       /* the forward's tblk_bwd for the same inputs, or NULL (the T
                                   blocks are then rebuilt from A and g_cum).  With it and bf16
                                   inputs, g_cum and A are not read and may be NULL */
    void *dq, *dk;              /* [B,T,H_q,K] grad_dtype, summed over the v heads of each q/k head */
    void *dv;                   /* [B,T,H_v,V] grad_dtype */
    float *dbeta;               /* [B,T,H_v] gradient w.r.t. beta */
    float *dg;                  /* [B,T,H_v] gradient w.r.t. the raw per-token g */
    float *dh0;                 /* [N,H_v,K,V] gradient of initial_state (NULL initial_state
                                   means zeros); NULL = not wanted */
    /* timing hook: NULL, or a HOST array of 2*GDR_BWD_STAGES events, a start
       and a stop per stage (T-block rebuild, chunk-start state recompute,
       reverse scan, chunk-local gradients), bound to the stages' kernel
       launches as in gdr_fwd_args; NULL entries are skipped */
    hipEvent_t *events;
    void *workspace;
    size_t workspace_bytes;
} gdr_bwd_args;

/* GDR_ABI_VERSION of the loaded library. */
int gdr_abi_version(void);

/* Static description of a return code ("ok", "invalid argument", ...). */
const char *gdr_strerror(int code);

/* Workspace bytes gdr_fwd needs for these sizes and options (pointers are
   not read).  The workspace is this library's own (the pages define no such
   argument): the caller allocates it, so the library itself never does.  With a sequence split and cp_segment_chunks = 0 the segment
   length, and with it the workspace of GDR_CP_EXACT, follows the compute
   units of the current device (256 if none can be queried): query with the
   device current that will run the call.  Returns GDR_OK or a validation
   error (GDR_EINVAL also when a split would give more than 2^30 (segment,
   sequence, v head) triples, which would overflow the launch grid). */
int gdr_fwd_workspace(const gdr_fwd_args *args, size_t *bytes);

/* Forward chunked prefill on `stream`: the low-level forward of the README
   ("Usage", "Low-level API"), which returns the in-chunk cumulative gate, A,
   o, the chunk-start states and the final state, evaluated by the chunked
   steps of the efeozkan blog ("2. Hardware-Friendly Algebraic
   Reformulation").  Computes o (and the optional outputs).  Chunks never
   cross a sequence boundary; the last chunk of a sequence may be partial; an
   empty sequence copies initial_state to final_state.  With GDR_CP_WARMUP and
   GDR_CP_AUTO_PAGES the chunk-start states and the output of segments after
   the first are the warm-up approximation (exact when the window reaches the
   start of the sequence); GDR_CP_AUTO chooses each segment's window on the
   device from the gates, so that its result differs from the exact one by at
   most 2^-24 of the state (the window reaches back to the sequence start
   where the gates do not decay).  With cp_segment_chunks = 0 the
   segment length L is chosen from the compute-unit count of the stream's
   device (one scan workgroup per unit): the segment count S that minimises
   rounds x (L + warm-up window) for the warm-up split and
   rounds x 3 L + (S - 1) for the exact one, rounds = ceil(S x workgroups per
   segment index / units), L = ceil(chunks / S); the pages' sliding-window
   method leaves L to a runtime model (they suggest sqrt(chunks) for theirs).
   GDR_CP_AUTO_EXACT splits only where that model predicts a gain over one
   segment.  Returns GDR_ELAUNCH if the device cannot be queried. */
int gdr_fwd(const gdr_fwd_args *args, hipStream_t stream);

/* The forward of gdr_fwd for callers that cannot allocate device memory (code
   under HIP graph capture, serving loops that must not allocate, harnesses that
   forbid it): the same arguments, outputs and kernels, but the scratch that
   gdr_fwd takes in args->workspace (T blocks, packed-sequence tables, the exact
   split's states) comes from a buffer the library owns: a static device array of
   GDR_SCRATCH_BYTES (256 MiB) per GPU, which each GPU the library runs this
   entry point on holds until the process ends.  args->workspace and
   workspace_bytes are ignored.  No hipMalloc, hipFree or other allocating call is
   made.  Returns GDR_ESCRATCH, launching nothing, when the problem needs more
   scratch than that (gdr_fwd_workspace gives the need: the prefill shard of
   B=4, T=4096, H_v=32, K=V=128 takes 109 MB; about 20,000 (chunk, v head) pairs
   of bf16 inputs fit); GDR_ELAUNCH if the buffer's device address cannot be had.  Every call on
   one GPU uses that GPU's one buffer: calls that overlap in time on one GPU
   (other streams, other host threads) race and must be serialised by the
   caller; consecutive calls on one stream are ordered.  Nothing in the buffer
   needs to start at zero: each call writes what it reads.  The first call on a
   device takes the buffer's address and must not be captured; later calls
   (with args->events NULL) may be captured into a HIP graph and replayed. */
int gdr_fwd_noalloc(const gdr_fwd_args *args, hipStream_t stream);

/* Bytes of the T blocks of gdr_fwd_args.tblk_bwd for these sizes: one block
   per (chunk, v head) for an upper bound on the chunk count (B ceil(T/64), or
   ceil(T/64) + n_seq with cu_seqlens), 13,312 bytes each for bf16 inputs
   (rows 0-31 of T stored at half width: the other half is zero) and 17,408
   for fp32 inputs.
   Returns GDR_OK or a validation error. */
int gdr_tblocks_bytes(const gdr_fwd_args *args, size_t *bytes);

/* Workspace bytes gdr_bwd needs for these sizes (pointers are not read; the
   workspace is this library's own, as for gdr_fwd_workspace):
   T blocks (unless tblk_bwd is given), the chunk-start states (unless h_bwd
   is given) and the chunk-end state gradients, 4 K V bytes each per
   (chunk, v head); with a sequence split also, per
   (sequence, v head, segment), the K x K transition and four K x V states
   (fp32) and a 512-byte zero row.  The split follows the compute units of
   the current device, as for gdr_fwd_workspace.  Returns GDR_OK or a
   validation error. */
int gdr_bwd_workspace(const gdr_bwd_args *args, size_t *bytes);

/* Backward of the exact forward (GDR_CP_OFF) on `stream`: the low-level
   backward of the README ("Usage", "Low-level API"), which takes the forward's
   g and A with the output gradient and returns dq, dk, dv, dbeta, dg and dh0.
   Gradients of <dout, o> + <dht, final_state> for an fp32 o, with respect to
   q, k, v, beta, the raw per-token g and initial_state.  g_cum and A must be what
   gdr_fwd returned for the same inputs.  The chunk-start states are
   recomputed unless the forward's h_bwd is given, the T blocks rebuilt
   unless its tblk_bwd is given.  dq and dk are written in full (rows of every
   token); every output is overwritten, none accumulated into.  With a
   sequence split (cp_mode) the chunk-start states and the reverse scan are
   split exactly (gdr_fwd's GDR_CP_EXACT applied to both recurrences; the
   reverse one carries the end-state gradients with the transposed segment
   transitions).  Returns GDR_ELAUNCH if the stream's device cannot be
   queried. */
int gdr_bwd(const gdr_bwd_args *args, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */
