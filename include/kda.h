/*
 * kda.h -- C ABI of the MI355X (gfx950) KDA prefill library, libkda.so.
 *
 * Kimi Delta Attention (KDA) is a gated delta-rule linear-attention
 * recurrence with one decay per key channel.  For each sequence and head,
 * with a dk x dv state S,
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t,          alpha_t = exp(g_t)   (g_t <= 0, per key channel)
 *
 * where q_t, k_t are L2-normalised inside the library (x / sqrt(|x|^2 + 1e-6),
 * q then multiplied by `scale`) when cfg->qk_l2norm is 1.  The pages this
 * library follows name KDA and its serving machinery but do not write the
 * recurrence out; the statement above is the standard KDA definition.
 *
 * Two paths compute it:
 *
 *  - Chunked prefill (kda_prefill): sequences packed by cu_seqlens, one
 *    state block per sequence (kern PR #44 "Prefill-only pipeline
 *    parallelism", commit "k3: flash-kda builds a varlen variant": cu_seqlens
 *    splits the rows into sequences, each with its own state block, and a
 *    tile-prefix step lays out the tiles), with optional state checkpoints
 *    (ROCm/ATOM PR #2709 "PP8 prefill for P/D serving", Changes: KDA state
 *    checkpoints on the chunk grid).
 *
 *  - Segment path for one long sequence (pegainfer PR #970 "cross-process CP
 *    whale gang", whale-lane commit text: each segment exports a KDA (M,D)
 *    package, packages are combined all-prefix or by a Blelloch prefix scan):
 *        kda_segment_package -> kda_segment_scan -> kda_output_fixup
 *        -> kda_checkpoint_write
 *    Segment j maps its incoming state to S_out = M_j S_in + D_j.  Its outputs
 *    are first computed from a zero state (o_local) and then corrected from
 *    its incoming state S_in^j.  All segments run as parallel work on one GPU.
 *
 *  - Resume (kda_prefill_resume): chunked prefill that continues sequences
 *    from states held in a slot pool, e.g. a checkpoint rung restored from a
 *    prefix cache, with rungs kept on the original sequence's grid (ROCm/ATOM
 *    PR #2709, Changes: prefix caching of KDA state; demand checkpoints and
 *    the prompt-end anchor floored onto the chunk grid).
 *
 *  - Short convolution (kda_short_conv, kda_conv_halo): the causal
 *    depthwise convolution KDA applies to q, k, v along tokens, with a
 *    per-sequence window state and the halo between segments.
 *
 *  - Decode (kda_decode): one new token per sequence against a pool of
 *    states addressed by read and write slots (ROCm/ATOM PR #2709, review
 *    notes: the fused sigmoid-gated delta-rule update takes a read-side state
 *    index beside the write table, so a forked request resumes a shared
 *    prefix state), with the gate activations optionally fused.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Layouts (row-major, contiguous): q, k, g [T,H,dk]; v, o [T,H,dv];
 *    beta [T,H]; states [., H, dk, dv] (key-major); M [., H, dk, dk].
 *  - q, k, v, o are float32 (io_dtype KDA_DTYPE_F32) or bfloat16
 *    (KDA_DTYPE_BF16, raw 16-bit storage).  g, beta and all states are
 *    float32 (the short convolution's windows are in the I/O dtype).
 *    Arithmetic: fp32 accumulation; matrix products on MFMA with bf16
 *    operands for bf16 I/O and fp32 operands for fp32 I/O.
 *  - Supported shapes: dk, dv in {64, 128} (dk == dv or not) for both I/O
 *    dtypes; chunk == 64 (the short convolution: see there).  Other shapes
 *    return KDA_ERR_UNSUPPORTED.  fp32 I/O with dk = 128 runs a
 *    token-recurrent kernel (one token at a time, the state in registers):
 *    its fp32 hand-off tiles would not fit in the 160 KiB of LDS the chunked
 *    engine's workgroup has.  It computes the same results (fp32) far slower
 *    than the chunked engine.
 *  - Every pointer is a device pointer unless stated.  Tensors (q, k, v, g,
 *    o, states, M, D, workspace) must be 16-byte aligned, beta 4-byte and the
 *    int64 index arrays 8-byte aligned (KDA_ERR_ALIGN otherwise).
 *  - Ownership: the caller owns every buffer.  The library allocates no
 *    device memory; scratch comes from the caller's workspace, sized by the
 *    matching *_workspace query (kda_prefill_noalloc: a fixed array inside
 *    the library, the only device memory it holds between calls).
 *  - Asynchrony: all work is enqueued on `stream` (a hipStream_t; NULL = the
 *    null stream) without synchronising.  Argument errors are detected on
 *    the host and returned before anything is launched.  A failed launch
 *    returns KDA_ERR_DEVICE.  Device-side data (cu_seqlens monotone, segment
 *    starts chunk-aligned, g <= 0) is not validated by the calls: that would
 *    need a sync.  kda_validate_inputs checks it on the device for debug runs.
 *  - Numerical domain: the per-channel log-decay summed over any aligned
 *    16-token block must stay above about -80 (a mean alpha above ~0.007
 *    per token); beyond it intermediate exponentials leave fp32 range.
 *  - Threading: reentrant; the only process state is a per-thread error
 *    string and, for kda_prefill_noalloc, its fixed per-device scratch.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define KDA_OK              0
#define KDA_ERR_ARG         1  /* null pointer, negative size, bad enum          */
#define KDA_ERR_UNSUPPORTED 2  /* shape / dtype / chunk the library does not build */
#define KDA_ERR_ALIGN       3  /* a device pointer is not 16-byte aligned        */
#define KDA_ERR_WORKSPACE   4  /* workspace missing or smaller than the query    */
#define KDA_ERR_DEVICE      5  /* a kernel launch failed                          */

#define KDA_DTYPE_F32  0
#define KDA_DTYPE_BF16 1

#define KDA_SCAN_SEQUENTIAL 0
#define KDA_SCAN_BLELLOCH   1

/* Problem description, read on the host during the call only. */
typedef struct {
    int32_t num_heads;   /* H                                              */
    int32_t dk, dv;      /* key / value head dims                          */
    int32_t chunk;       /* must be 64                                     */
    int32_t io_dtype;    /* KDA_DTYPE_F32 or KDA_DTYPE_BF16 (q, k, v, o)   */
    float scale;         /* query scale applied after normalisation        */
    int32_t qk_l2norm;   /* 1: L2-normalise q and k in-kernel; 0: use as is */
} kda_config;

/*
 * State checkpoints.  Rungs sit at sequence-relative positions p = m*interval
 * (m >= 1, p <= sequence length): the state after the first p tokens.
 * interval is a positive multiple of the chunk (0 = no checkpoints).  The
 * rung of sequence n at p is row offsets[n] + p/interval - 1 of `states`
 * [rows, H, dk, dv].  offsets (device int64 [N+1]) may be NULL for a single
 * sequence (rows then start at 0).
 */
typedef struct {
    int32_t interval;
    const int64_t *offsets;
    float *states;
} kda_ckpt;

/*
 * A pool of fp32 states [n_slots, H, dk, dv] addressed per sequence by slot.
 * read_idx[n] is the slot holding sequence n's state before its new tokens
 * (an index < 0 or >= n_slots means a zero state); write_idx[n] is the slot
 * that receives its state after them (< 0 or >= n_slots: not written).
 * read_idx[n] == write_idx[n] updates the slot in place; two different slots
 * fork the state and leave the read slot as it was.  A call's write slots must
 * differ from one another and from every other sequence's read slot, and
 * calls that overlap on one pool race.  Both index arrays are device int32
 * [N]; out-of-range indices are treated as above, never dereferenced.
 */
typedef struct {
    float *states;
    int64_t n_slots;
    const int32_t *read_idx;
    const int32_t *write_idx;
} kda_state_pool;

/* ------------------------------------------------------------------------ */
/* Chunked prefill                                                           */
/* ------------------------------------------------------------------------ */

/* Workspace bytes kda_prefill needs for N packed sequences (never 0): the
 * longest-first schedule, or for one long sequence the buffers of its
 * segmented processing (see kda_prefill). */
size_t kda_prefill_workspace(const kda_config *cfg, int64_t T, int32_t N);

/*
 * Chunked KDA prefill of N sequences packed along T.
 *   q, k [T,H,dk], v [T,H,dv] (io_dtype); g [T,H,dk], beta [T,H] (fp32);
 *   cu_seqlens: device int64 [N+1], cu_seqlens[0] = 0, cu_seqlens[N] = T,
 *       non-decreasing; a zero-length sequence keeps its S0;
 *   S0 [N,H,dk,dv] initial states, NULL = zeros;
 *   S_final [N,H,dk,dv] final states, NULL = not written;
 *   o [T,H,dv] outputs (io_dtype);
 *   ckpt: NULL or checkpoints as described at kda_ckpt;
 *   ws / ws_bytes: scratch of at least kda_prefill_workspace() bytes.
 * Work is scheduled longest sequence first.  N = 0 or T = 0 is a no-op.
 *
 * A single sequence (N = 1) whose heads would occupy fewer workgroups than
 * the device has compute units is processed as segments of at least 512
 * tokens on the chunk grid (the segment path below, run inside ws: packages,
 * a sequential scan, the output fix-up and checkpoint rungs), when ws_bytes
 * holds its buffers; otherwise in one pass.  kda_prefill_workspace returns
 * that size for calls without checkpoints.  With checkpoints (and
 * ckpt->offsets NULL) the segmented path also needs
 * round256(T/interval * H * dk * dv * 4) bytes more for the rungs' own
 * parts (the fix-up writes the rungs).  Both paths give the same result up
 * to fp32 rounding.
 */
int kda_prefill(const kda_config *cfg, const void *q, const void *k, const void *v,
                const float *g, const float *beta, const int64_t *cu_seqlens, int32_t N,
                int64_t T, const float *S0, float *S_final, void *o, const kda_ckpt *ckpt,
                void *ws, size_t ws_bytes, void *stream);

/*
 * kda_prefill for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and arguments, with no workspace argument.  Its
 * scratch is a fixed array of KDA_NOALLOC_SCRATCH_BYTES inside the library,
 * one per device, held until the process ends; the call makes no hipMalloc
 * or hipFree and calls no allocating routine.  The result is the one
 * kda_prefill gives with a workspace of that size: a single sequence runs as
 * segments when their buffers fit (64 MiB holds them for 8,192 tokens at
 * H = 32, d = 128 without checkpoints), otherwise in one pass.
 * KDA_ERR_WORKSPACE when N * 4 bytes of schedule exceed the scratch.  Every
 * call on one device shares that device's scratch: calls that overlap on a
 * device (other streams, other threads) race and must be serialised by the
 * caller.  No byte of the scratch needs to start at zero: a call reads only
 * what it wrote earlier in the same call.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (64u << 20)
int kda_prefill_noalloc(const kda_config *cfg, const void *q, const void *k, const void *v,
                        const float *g, const float *beta, const int64_t *cu_seqlens, int32_t N,
                        int64_t T, const float *S0, float *S_final, void *o, const kda_ckpt *ckpt,
                        void *stream);

/*
 * Chunked prefill that continues N sequences from states in a pool.
 * Arguments as kda_prefill, except:
 *   pool: sequence n starts from slot pool->read_idx[n] and its final state
 *       is stored in slot pool->write_idx[n] (see kda_state_pool; a slot may
 *       be read and written by the same sequence: it is then updated in
 *       place);
 *   pos0: device int64 [N], the absolute position in its original sequence
 *       of each sequence's first token, a multiple of the chunk (NULL = all
 *       0).  The tokens are positions pos0[n] .. pos0[n] + len - 1;
 *   ckpt: rungs at absolute positions P = m*interval with
 *       pos0[n] < P <= pos0[n] + len, at row
 *       offsets[n] + P/interval - pos0[n]/interval - 1.
 * Resuming from the rung at P with pos0 = P reproduces the continuous run's
 * outputs, later rungs and final state (up to rounding).  Workspace as
 * kda_prefill_workspace(cfg, T, N).
 */
int kda_prefill_resume(const kda_config *cfg, const void *q, const void *k, const void *v,
                       const float *g, const float *beta, const int64_t *cu_seqlens, int32_t N,
                       int64_t T, const int64_t *pos0, const kda_state_pool *pool, void *o,
                       const kda_ckpt *ckpt, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------ */
/* Segment path (one sequence of T tokens split into nseg segments)         */
/* ------------------------------------------------------------------------ */

/*
 * Per-segment packages.  seg_start: device int64 [nseg+1], seg_start[0] = 0,
 * seg_start[nseg] = T, every interior start a multiple of the chunk.
 * Writes, for every segment j and head h:
 *   o_local [T,H,dv]  outputs of the segment computed from a zero state;
 *   M [nseg,H,dk,dk]  the segment's linear part (product of its token maps);
 *                     M = NULL skips it (a caller whose incoming states are
 *                     all zero, or that only needs o_local and D);
 *   D [nseg,H,dk,dv]  the segment's state when started from zero;
 *   with ckpt != NULL (states unused here) and sub_M / sub_D non-NULL, the
 *   sub-package (Pi_p, S0_p) of every rung p inside (seg_start[j],
 *   seg_start[j+1]]: the map from S_in^j to the state at p, at rung row
 *   p/interval - 1 of sub_M [rows,H,dk,dk] and sub_D [rows,H,dk,dv]
 *   (sub_M = NULL skips Pi_p: kda_output_fixup_ckpt needs only sub_D;
 *   sub_M needs M).
 * One kernel launch: the value blocks (o_local, D, sub_D) and, with M, the M
 * blocks after them in the same grid.  No workspace is needed (ws may be
 * NULL).  When nseg * H would leave compute units idle, a workspace of at
 * least kda_segment_package_workspace(cfg, T, nseg) bytes (a nonzero query)
 * lets the call split every segment into f chunk-aligned sub-segments, run
 * their packages in one launch, and merge them left to right (sub-segment k
 * fixed up from the accumulated state of 0..k-1, its rungs included, then
 * (M, D) composed); the results equal the unsplit call's up to fp32
 * rounding.  With the bf16 or fp32 chunked shapes the queried size also holds
 * the fix-up operators (as kda_fixop describes) of sub-segments 1..f-1, kept
 * by their M blocks, so that a merge step corrects those sub-segments as a
 * product; a workspace large enough only for the split without them merges
 * by the recurrence alone.
 */
/* Workspace bytes that let kda_segment_package split its segments (0 when it
 * would not split them: enough units already, or segments too short). */
size_t kda_segment_package_workspace(const kda_config *cfg, int64_t T, int32_t nseg);

int kda_segment_package(const kda_config *cfg, const void *q, const void *k, const void *v,
                        const float *g, const float *beta, int64_t T, const int64_t *seg_start,
                        int32_t nseg, void *o_local, float *M, float *D, const kda_ckpt *ckpt,
                        float *sub_M, float *sub_D, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes for kda_segment_scan.  Blelloch scan: required; the padded
 * packages, flags per package and two counters per head.  Sequential scan:
 * optional; one flag per package (a first launch tests each M once for zero,
 * instead of every workgroup of a head testing every M), and with ws = NULL or
 * fewer bytes the scan runs without it, with the same results.  Concurrent
 * scans need separate workspaces. */
size_t kda_segment_scan_workspace(const kda_config *cfg, int32_t nseg, int32_t algo);

/*
 * Prefix scan of the packages: S_in^0 = S0 (NULL = zeros),
 * S_in^{j+1} = M_j S_in^j + D_j.  Writes S_in [nseg,H,dk,dv] and
 * S_final [H,dk,dv].  algo KDA_SCAN_SEQUENTIAL walks the segments in order;
 * KDA_SCAN_BLELLOCH runs a work-efficient up-sweep / down-sweep exclusive
 * scan over the composition (Mb,Db) o (Ma,Da) = (Mb Ma, Mb Da + Db), padded
 * with identity packages to a power of two, in the workspace (at most 4096
 * segments; more return KDA_ERR_UNSUPPORTED).  Products with an exactly
 * zero or identity factor are not formed unless the other factor holds an
 * infinity or a NaN.  The products of one tree level are shared out over up
 * to 8 workgroups per head, which wait for each other inside the launch
 * (bounded waits; the launch uses at most half of the workgroups the device
 * holds at once).  The results do not depend on that split.  M and D are
 * not modified.
 */
int kda_segment_scan(const kda_config *cfg, int32_t nseg, const float *M, const float *D,
                     const float *S0, float *S_in, float *S_final, int32_t algo,
                     void *ws, size_t ws_bytes, void *stream);

/*
 * Output fix-up: o holds o_local on entry and the final outputs on return,
 * o_t += contribution of S_in^j propagated through segment j.  The
 * correction stops exactly once the propagated state is all zeros in fp32.
 * No workspace is needed.
 */
int kda_output_fixup(const kda_config *cfg, const void *q, const void *k, const float *g,
                     const float *beta, int64_t T, const int64_t *seg_start, int32_t nseg,
                     const float *S_in, void *o, void *ws, size_t ws_bytes, void *stream);

/*
 * The output fix-up and the segment path's checkpoint rungs in one launch
 * (the fused form of kda_output_fixup followed by kda_checkpoint_write, for
 * callers that skip the rung sub-packages sub_M): while the fix-up
 * propagates S_in^j through segment j it has Pi_p S_in^j at every rung p
 * inside (seg_start[j], seg_start[j+1]], and writes
 *     ckpt->states[p/interval - 1] = Pi_p S_in^j + sub_D[p/interval - 1];
 * once the propagated state is exactly zero the remaining rungs of the
 * segment are copies of their sub_D rows.  ckpt->offsets is unused (one
 * sequence, rows from 0); sub_D [rows, H, dk, dv] as written by
 * kda_segment_package.  ckpt = NULL is kda_output_fixup.  The rung states
 * equal kda_checkpoint_write's up to fp32 rounding (the same map applied by
 * the chunk recurrence instead of one product with sub_M).  ckpt->states may
 * be sub_D itself: the rungs are then formed in place, and the rows after
 * the propagated state has reached zero are left as they are (already their
 * values), which saves copying them; otherwise the two must not overlap.
 */
int kda_output_fixup_ckpt(const kda_config *cfg, const void *q, const void *k, const float *g,
                          const float *beta, int64_t T, const int64_t *seg_start, int32_t nseg,
                          const float *S_in, void *o, const kda_ckpt *ckpt, const float *sub_D,
                          void *ws, size_t ws_bytes, void *stream);

/*
 * Fix-up operator of the segment packages (the chunked engine's shapes: not
 * fp32 I/O with dk = 128).  The M blocks of the package launch propagate the
 * identity through each segment until it is exactly zero; with the configs'
 * gates that takes a few chunks.  With an operator they also keep, for the
 * first `chunks` chunks of segment j, what that identity gives output row t:
 *     X[j][t - seg_start[j]][h][:] = Pi_t^T qhat_t
 * Pi_t maps segment j's incoming state to its state after token t, and qhat_t
 * is the query as the outputs use it (normalised and scaled).  They also write
 *     len[j][h][b] = the chunks after which columns 64b..64b+63 of the
 *                    propagated identity are exactly zero,
 * or the segment's chunk count when the segment ends within `chunks` chunks
 * first (all its rows are kept), or -1 otherwise.  Since every row past len
 * chunks has a correction of exactly zero, the fix-up corrects a segment whose
 * len are all >= 0 as o_t += (S_in^j)^T X_t over those rows, with no
 * recurrence.  An operator whose `chunks` covers the longest segment therefore
 * makes the fix-up a product whatever the gates (with long memory, rungs then
 * come from kda_checkpoint_write and sub_M: Pi covers one rung).  A segment walks the recurrence as kda_output_fixup_ckpt does
 * when one of its len is -1, when its incoming state holds an infinity or a
 * NaN, or when a checkpoint rung falls among the corrected rows and Pi does
 * not cover it.  Pi covers the first rung after the segment start when the
 * fix-up's checkpoint interval is fx->interval, as Pi S_in + sub_D; a second
 * rung among the rows needs the recurrence.  The results equal the
 * recurrence's up to rounding (X is rounded once to the I/O dtype).
 * This recasts the pages' fix-up step; it is not a step the pages name.
 */
typedef struct kda_fixop {
    int32_t chunks;    /* chunks of rows kept per segment, >= 1 */
    int32_t interval;  /* checkpoint interval of Pi (a multiple of chunk), 0: no Pi */
    void *X;           /* [nseg, chunks * chunk, H, dk] in io_dtype, 16-byte aligned;
                          rows past a segment's end are not written */
    int32_t *len;      /* [nseg, H, dk / 64], 4-byte aligned */
    int32_t *route;    /* [nseg, H], 4-byte aligned: written and read by the
                          fix-up (1 where a segment walks the recurrence) */
    float *Pi;         /* [nseg, H, dk, dk], 16-byte aligned, or NULL: the
                          propagated identity at the segment's first multiple
                          of `interval` when it falls within the kept chunks */
} kda_fixop;

/* kda_segment_package that also writes the fix-up operator *fx.  M is
 * required (the M blocks form the operator).  With the workspace that
 * kda_segment_package_workspace asks for, the segments are split into
 * sub-segments as kda_segment_package splits them; the operator then comes
 * from each segment's first sub-segment (a segment whose identity has not
 * vanished by the end of its first sub-segment gets len -1).
 * KDA_ERR_UNSUPPORTED for fp32 I/O with dk = 128. */
int kda_segment_package_fx(const kda_config *cfg, const void *q, const void *k, const void *v,
                           const float *g, const float *beta, int64_t T,
                           const int64_t *seg_start, int32_t nseg, void *o_local, float *M,
                           float *D, const kda_ckpt *ckpt, float *sub_M, float *sub_D,
                           const kda_fixop *fx, void *ws, size_t ws_bytes, void *stream);

/* kda_output_fixup_ckpt (ckpt may be NULL) with the operator that
 * kda_segment_package_fx wrote for the same inputs, segments and chunks
 * (fx = NULL: kda_output_fixup_ckpt).  Two launches: the segments the
 * operator covers, one light workgroup each, then the recurrence for the
 * others (its workgroups for covered segments end at once).  No workspace;
 * calls sharing one fx must not overlap (route). */
int kda_output_fixup_fx(const kda_config *cfg, const void *q, const void *k, const float *g,
                        const float *beta, int64_t T, const int64_t *seg_start, int32_t nseg,
                        const float *S_in, void *o, const kda_ckpt *ckpt, const float *sub_D,
                        const kda_fixop *fx, void *stream);

/*
 * Checkpoint states of the segment path: for every rung p (see kda_ckpt;
 * one sequence, so rows start at 0) inside segment j,
 *     states[p/interval - 1] = sub_M[row] S_in^j + sub_D[row]
 * from the sub-packages written by kda_segment_package.
 */
int kda_checkpoint_write(const kda_config *cfg, const kda_ckpt *ckpt, int64_t T,
                         const int64_t *seg_start, int32_t nseg, const float *S_in,
                         const float *sub_M, const float *sub_D, void *stream);

/* ------------------------------------------------------------------------ */
/* Decode                                                                    */
/* ------------------------------------------------------------------------ */

/*
 * One decode step: sequence n takes one new token, row n of
 *   q, k [N,H,dk], v [N,H,dv] (io_dtype); g [N,H,dk], beta [N,H] (fp32);
 * gate_logits 0: g is log alpha and beta is beta, as in prefill;
 *             1: both are logits, activated in the kernel as
 *                log alpha = -softplus(g) and beta = sigmoid(beta);
 * pool: the states read and written as described at kda_state_pool;
 * o [N,H,dv] (io_dtype): o_n = S_n^T q_n with the updated state.
 * Shapes: dk, dv in {64, 128}, for either io_dtype.  N = 0 is a no-op.
 * No workspace.  One kernel launch.
 */
int kda_decode(const kda_config *cfg, int32_t N, const void *q, const void *k, const void *v,
               const float *g, const float *beta, int32_t gate_logits,
               const kda_state_pool *pool, void *o, void *stream);

/* ------------------------------------------------------------------------ */
/* Short causal convolution over tokens                                      */
/* ------------------------------------------------------------------------ */

#define KDA_ACT_NONE 0
#define KDA_ACT_SILU 1

/*
 * Window slots of the short convolution: states [n_slots, width-1, channels]
 * in the I/O dtype hold the last width-1 inputs of a sequence (oldest row
 * first).  read_idx[n] is the slot read as sequence n's window (NULL, or an
 * index outside [0, n_slots): zeros); write_idx[n] the slot that receives its
 * new window (NULL or outside: not stored).  Windows are read before any is
 * written, so a sequence may update its own slot in place; a call's write
 * slots must differ from one another and from every other sequence's read
 * slot.
 */
typedef struct {
    void *states;
    int64_t n_slots;
    const int32_t *read_idx;
    const int32_t *write_idx;
} kda_conv_state;

/*
 * Depthwise causal convolution along tokens (kern PR #44: the varlen stage
 * kernels gather the KDA short-conv inputs per sequence and update its
 * window; ROCm/ATOM PR #2709: the conv state follows a fork through a read
 * index).  For sequence n (rows cu_seqlens[n] .. cu_seqlens[n+1]-1 of
 * x [T, channels]) and x~ = (its window, its rows):
 *     y_t[c] = act(bias[c] + sum_{j<width} weight[c][j] * x~_{t-width+1+j}[c])
 * (the last tap multiplies the current token); its new window is the last
 * width-1 rows of x~.  act: KDA_ACT_NONE or KDA_ACT_SILU (z / (1 + e^-z)).
 *   x, y [T, channels] in io_dtype, 16-byte aligned, y not aliasing x;
 *   weight [channels, width] fp32, bias [channels] fp32 or NULL;
 *   cu_seqlens device int64 [N+1]; state NULL (zero windows, none stored).
 * channels a multiple of 8; width in [2, 8].  Decode is the case of one
 * token per sequence.  Two launches: outputs, then the new windows.
 */
int kda_short_conv(int32_t io_dtype, int32_t channels, int32_t width, int32_t activation,
                   const void *x, int64_t T, const int64_t *cu_seqlens, int32_t N,
                   const float *weight, const float *bias, const kda_conv_state *state, void *y,
                   void *stream);

/*
 * Conv halo of a split sequence (pegainfer PR #970: a context-parallel rank
 * publishes its conv halo tail with its KDA packages): for every segment j of
 * x [T, channels] (bounds device int64 [nseg+1]), the width-1 input rows
 * before bounds[j+1] (zeros before row 0) are copied into slot
 * dst->write_idx[j] of dst->states.  Reading segment j+1 with that slot as its
 * window makes a per-segment kda_short_conv equal to the whole-sequence one.
 */
int kda_conv_halo(int32_t io_dtype, int32_t channels, int32_t width, const void *x, int64_t T,
                  const int64_t *bounds, int32_t nseg, const kda_conv_state *dst, void *stream);

/* ------------------------------------------------------------------------ */
/* Diagnostics                                                               */
/* ------------------------------------------------------------------------ */
const char *kda_status_string(int status);

/*
 * Debug check of device-side inputs the calls take on trust.  Counts, into
 * report[0 .. KDA_CHECK_FIELDS) (device int32, 4-byte aligned, zeroed by the
 * call; read it after the stream's work), for a tensor of T tokens with
 * cfg->num_heads heads and cfg->dk key channels:
 *   [KDA_CHECK_BOUNDS]         entries of bounds[0..n] at fault: bounds[0] != 0,
 *                              bounds[n] != T, a decrease, or (chunk_aligned = 1,
 *                              for segment starts) an interior entry off the
 *                              chunk grid.  bounds = cu_seqlens (n sequences) or
 *                              seg_start (n segments); NULL: one unit [0, T).
 *   [KDA_CHECK_G_POSITIVE]     elements of g above 0 (a decay alpha = e^g above 1);
 *   [KDA_CHECK_G_NONFINITE]    elements of g that are infinite or NaN;
 *   [KDA_CHECK_G_BLOCK_FLOOR]  (16-token block, head, channel) triples whose
 *                              summed g is below -80, the blocks counted from
 *                              each unit's first token: the numerical domain
 *                              stated above;
 *   [KDA_CHECK_BETA_NONFINITE] elements of beta that are infinite or NaN.
 * g [T, H, dk] and beta [T, H] may each be NULL (not checked).  All zeros:
 * the inputs are inside what the kernels assume.  Enqueued on `stream`; it
 * reads g once (about T * H * dk * 4 bytes) and is meant for debug runs.
 */
#define KDA_CHECK_BOUNDS         0
#define KDA_CHECK_G_POSITIVE     1
#define KDA_CHECK_G_NONFINITE    2
#define KDA_CHECK_G_BLOCK_FLOOR  3
#define KDA_CHECK_BETA_NONFINITE 4
#define KDA_CHECK_FIELDS         8
int kda_validate_inputs(const kda_config *cfg, int64_t T, const int64_t *bounds, int32_t n,
                        int32_t chunk_aligned, const float *g, const float *beta,
                        int32_t *report, void *stream);
/* Detail of the last error returned on the calling thread ("" if none). */
const char *kda_last_error(void);
/* Library version, "major.minor.patch". */
const char *kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
