/*
 * gdn2.h -- C ABI of libgdn2: the Gated DeltaNet-2 forward sequence-mixing
 * hot path on AMD MI355X (gfx950).
 *
 * The method (Gated DeltaNet-2 post on tilnote.io, section on the GDN-2
 * design; news.hamidun.com item, section on the architecture) keeps one
 * fixed-size state S (d_k x d_v, rows = key channels, columns = value
 * channels) per sequence and value head. For each token t, in this order:
 *
 *   S~  = diag(a_t) S                       decay, channel-wise on the key axis
 *   r_t = S~^T k_t                          key read of the decayed state
 *   S   = S~ - (b_t * k_t) r_t^T + k_t (w_t * v_t)^T
 *                                           erase (gate b on the key axis),
 *                                           write (gate w on the value axis)
 *   o_t = S^T q_t                           the query reads the updated state
 *
 * The read/update/read order and the state orientation follow the delta-rule
 * tutorial on ai-systems-engineering.com ("write with KV, read with Q" and
 * "record the difference" sections). The pages describe the decoupled erase
 * and write only in prose; the placement above is the plainest reading, and
 * it reduces to the delta rule S + beta k (v - S^T k)^T when a = 1 and
 * b = w = beta (tutorial, beta section).
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller. The library
 *    never allocates, frees or retains device memory and keeps no state
 *    between calls; calls are thread-safe.
 *  - Tensors are contiguous, row-major, in these layouts:
 *      q, k : [B, T, H_qk, d_k]      dtype of desc (fp32 or bf16)
 *      v    : [B, T, H_v,  d_v]      dtype of desc
 *      a, b : [B, T, H_v,  d_k]      fp32 (decay in (0,1], erase gate)
 *      w    : [B, T, H_v,  d_v]      fp32 (write gate)
 *      o    : [B, T, H_v,  d_v]      dtype of desc (fp32 -> bf16 rounds to nearest even)
 *      S0, S_T, S : [B, H_v, d_k, d_v]  fp32
 *    Value head h uses query/key head h / (H_v / H_qk) (contiguous groups,
 *    as in the grouped 16 QK / 32 V head layout of the aiki wiki entry on
 *    Gated DeltaNet, "how it works").
 *  - Preconditions that are documented, not checked (checking would cost
 *    bandwidth): a in (0, 1]; finite inputs (NaN/Inf propagate). Keys and
 *    queries are used as given: the library never normalises them.
 *  - `stream` is a hipStream_t (NULL = the default stream). Every call only
 *    enqueues work and returns; device faults surface on the stream.
 *  - Argument errors return a status before anything is enqueued.
 */
#ifndef GDN2_H_
#define GDN2_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN2_OK = 0,
  GDN2_ERR_NULL_POINTER = 1, /* a required pointer is NULL */
  GDN2_ERR_BAD_SHAPE = 2,    /* negative size, H_v % H_qk != 0, decode with T != 1,
                                a tensor pointer not 16-byte aligned (4-byte for the
                                tensors of one fp32 per token and value head:
                                beta, alpha and their gradients) */
  GDN2_ERR_UNSUPPORTED = 3,  /* valid but not built: d_k, d_v not in {16,32,64,128}, chunk not in {16,32,64},
                                or (prefill and backward) max(H_qk, H_v) * max(d_k, d_v) * 4 * 64 > 2^31 - 1
                                (one chunk of the widest token rows must fit a buffer range:
                                H <= 65535 at d = 128) */
  GDN2_ERR_BAD_DTYPE = 4,    /* dtype is neither GDN2_F32 nor GDN2_BF16 */
  GDN2_ERR_WORKSPACE = 5,    /* workspace smaller than gdn2_chunk_forward_workspace_bytes() */
  GDN2_ERR_HIP = 6,          /* the HIP runtime reported an error at launch */
  GDN2_ERR_ALIAS = 7,        /* o or the workspace overlaps an input, the state or each other */
  GDN2_ERR_SCRATCH = 8       /* gdn2_chunk_forward_noalloc: the problem needs more scratch than
                                GDN2_NOALLOC_SCRATCH_BYTES */
} gdn2_status;

typedef enum { GDN2_F32 = 0, GDN2_BF16 = 1 } gdn2_dtype;

/* Problem description. B: sequences; T: tokens per sequence; H_qk / H_v:
 * query-key heads / value heads (H_v % H_qk == 0); d_k, d_v: head dims;
 * chunk: the LONGEST chunk of the prefill the caller allows (a performance
 * knob only: results agree at every supported chunk). The prefill runs the
 * longest supported chunk not above it whose working set fits one compute
 * unit: at d_k = 128 in bf16 that is 32 when 64 is asked for (64 does not fit
 * the 160 KiB of LDS); gdn2_chunk_forward_plan() reports the chunk that runs.
 * dtype: a gdn2_dtype for q, k, v, o. */
typedef struct {
  int32_t B, T, H_qk, H_v, d_k, d_v, chunk;
  int32_t dtype;
} gdn2_desc;

/* Bytes of device workspace gdn2_chunk_forward needs for `desc` (0 if none).
 * Nonzero when the prefill splits long sequences into segments processed in
 * parallel: that happens when the unsplit call would occupy few workgroups
 * (few sequences x value heads) and T spans many chunks; the environment
 * variable GDN2_PREFILL_SPLIT=<n>, read at each call, forces n segments
 * (1: never split). The split computes the same recurrence: every segment
 * runs from a zero state while identity columns give its transition matrix;
 * the exact entering states (up to rounding) follow from those in order, and
 * each segment's outputs are then corrected by its entering state's
 * contribution (d_k == d_v; otherwise the segments run again from their
 * entering states). The workspace holds the segments' states and transitions
 * (fp32) and, for the correction, d_k values of the input dtype per token
 * and value head. Returns 0 for an invalid description as well; the forward
 * call reports the error. */
size_t gdn2_chunk_forward_workspace_bytes(const gdn2_desc *desc);

/* How gdn2_chunk_forward (and its gate forms) would run `desc`: the chunk
 * length actually used (the longest supported one not above desc->chunk that
 * fits, see gdn2_desc) into *chunk_run, and the number of segments each
 * sequence is split into (1: unsplit) into *segments. Either output pointer
 * may be NULL. Host-only: enqueues nothing, needs no device. Returns the
 * status gdn2_chunk_forward would return for the description's checks. */
gdn2_status gdn2_chunk_forward_plan(const gdn2_desc *desc, int32_t *chunk_run, int32_t *segments);

/* Prefill: run T tokens of every (sequence, value head) through the
 * recurrence above, starting from S0, writing every output o_t and the final
 * state S_T. Computed chunk-parallel: within each chunk of `chunk` tokens
 * the key reads come from one triangular solve and the outputs from dense
 * products, with the state carried across chunks in fp32. The result equals
 * the token-by-token recurrence up to rounding.
 *   S0  : may be NULL (zero state).
 *   S_T : may be NULL (not written); may alias S0 exactly (in-place update).
 *   o   : must not overlap any input or S_T (GDN2_ERR_ALIAS).
 *   workspace / workspace_bytes: device scratch of at least
 *         gdn2_chunk_forward_workspace_bytes(desc) bytes, 16-byte aligned,
 *         not overlapping any tensor (may be NULL if that is 0). Smaller:
 *         GDN2_ERR_WORKSPACE; overlapping: GDN2_ERR_ALIAS. Its contents are
 *         scratch on entry and exit, owned by the caller.
 * T == 0 is valid: S_T = S0 (or zeros). Any T >= 0 is accepted; a last
 * partial chunk is stepped token by token. */
gdn2_status gdn2_chunk_forward(const gdn2_desc *desc, const void *q, const void *k, const void *v,
                               const float *a, const float *b, const float *w, const float *S0,
                               void *o, float *S_T, void *workspace, size_t workspace_bytes,
                               void *stream);

/* Bytes of the static device scratch of gdn2_chunk_forward_noalloc (64 MiB).
 * Each device that runs the library holds one such array until the process
 * ends. */
#define GDN2_NOALLOC_SCRATCH_BYTES (64u << 20)

/* gdn2_chunk_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): it allocates nothing and calls no
 * allocating routine. Same arguments, results and errors as
 * gdn2_chunk_forward; the scratch that a split of long sequences needs is
 * taken from a static device array of GDN2_NOALLOC_SCRATCH_BYTES per device,
 * whose address is looked up on the first call on each device. The split is
 * planned within that array: where the output correction's scratch
 * (gdn2_chunk_forward_workspace_bytes(desc)) fits, the results are bit for
 * bit those of gdn2_chunk_forward (the same kernels and plan); where only
 * the segment states and transitions fit, the segments run a second time
 * instead of being corrected (equal up to rounding). Problems whose states
 * and transitions alone do not fit (e.g. very many segments forced with
 * GDN2_PREFILL_SPLIT) return GDN2_ERR_SCRATCH before anything is enqueued;
 * problems that need no scratch never touch the array. The array is shared by every call on a device
 * and keeps the last call's contents: calls of this entry point that overlap
 * in time on one device (other streams, other host threads) race on it and
 * must be serialised by the caller. Nothing in it needs to start cleared. */
gdn2_status gdn2_chunk_forward_noalloc(const gdn2_desc *desc, const void *q, const void *k, const void *v,
                                       const float *a, const float *b, const float *w, const float *S0,
                                       void *o, float *S_T, void *stream);

/* Prefill with coupled gates: the erase gate and the write gate are one
 * scalar per token and value head, b_t = w_t = beta_t (all channels): the
 * form of the earlier Gated DeltaNet and Kimi Delta Attention, whose erase
 * and write share one scalar gate (GDN-2 note, section on the delta rule's
 * basic idea and its limits), with GDN-2's channel-wise decay kept. The
 * update is then S = S~ + beta_t k_t (v_t - r_t)^T. Same arguments as
 * gdn2_chunk_forward with b, w replaced by
 *   beta: [B, T, H_v] fp32 (4-byte alignment suffices: a view starting at
 *         any token of a larger tensor is accepted).
 * The result equals gdn2_chunk_forward with b = beta * ones(d_k) and
 * w = beta * ones(d_v) up to rounding: with b = beta the erase-side Gram
 * matrices are the key-side ones with column s scaled by beta_s, so only two
 * of the four are formed as products (scaled in fp32). The two per-channel
 * gate arrays are not read, which removes about 40% of the prefill's memory
 * traffic at d = 128. The same workspace rules apply
 * (gdn2_chunk_forward_workspace_bytes). */
gdn2_status gdn2_chunk_forward_coupled(const gdn2_desc *desc, const void *q, const void *k, const void *v,
                                       const float *a, const float *beta, const float *S0, void *o,
                                       float *S_T, void *workspace, size_t workspace_bytes, void *stream);

/* Prefill with scalar gates: the decay is also one scalar per token and
 * value head (all key channels), a_t = alpha_t, with coupled erase/write
 * gates b_t = w_t = beta_t: the form of the earlier Gated DeltaNet (GDN-2
 * note, section on the delta rule's basic idea and its limits; wiki, how it
 * works). Same arguments as gdn2_chunk_forward_coupled with
 *   a: [B, T, H_v] fp32 (one decay per token and value head).
 * The result equals gdn2_chunk_forward with a = alpha * ones(d_k),
 * b = beta * ones(d_k), w = beta * ones(d_v) up to rounding (two Gram
 * matrices formed, as for gdn2_chunk_forward_coupled); no per-channel gate
 * array is read. */
gdn2_status gdn2_chunk_forward_scalar(const gdn2_desc *desc, const void *q, const void *k, const void *v,
                                      const float *a, const float *beta, const float *S0, void *o,
                                      float *S_T, void *workspace, size_t workspace_bytes, void *stream);

/* Prefill of a batch of sequences of different lengths packed along the
 * token axis (the serving layout; GDN-2 note and wiki describe the layer's
 * use in serving long and short requests alike). desc->B is the number of
 * sequences and desc->T the total number of tokens; q, k are
 * [T, H_qk, d_k], v, w, o [T, H_v, d_v], a, b [T, H_v, d_k] (a leading batch
 * dimension of 1 is the same memory); sequence n is tokens
 * cu_seqlens[n] .. cu_seqlens[n+1]-1.
 *   cu_seqlens: device pointer to B+1 int32 offsets, cu_seqlens[0] = 0,
 *         non-decreasing, cu_seqlens[B] = T (a precondition: device memory
 *         is not read by the host; offsets outside [0, T] are clamped to it).
 *         Required when B > 0 (GDN2_ERR_NULL_POINTER).
 *   S0, S_T: [B, H_v, d_k, d_v] fp32, one state per sequence, as for
 *         gdn2_chunk_forward (S0 may be NULL, S_T may be NULL or alias S0).
 * Each sequence is computed exactly as gdn2_chunk_forward computes it alone
 * (the same chunk boundaries from its first token, a ragged last chunk
 * stepped token by token); an empty sequence gives S_T = S0. Sequences are
 * never split into segments: no workspace is used. Errors as for
 * gdn2_chunk_forward. */
gdn2_status gdn2_chunk_forward_varlen(const gdn2_desc *desc, const int32_t *cu_seqlens, const void *q,
                                      const void *k, const void *v, const float *a, const float *b,
                                      const float *w, const float *S0, void *o, float *S_T, void *stream);

/* Gate forms of the packed-sequence calls below (each as the unpacked entry
 * point of the same form describes it):
 *   GDN2_GATES_CHANNEL: a, b [T, H_v, d_k], w [T, H_v, d_v] fp32 (gdn2_chunk_forward);
 *   GDN2_GATES_PREACT : the same shapes, pre-activations in the input dtype
 *                       (gdn2_chunk_forward_preact);
 *   GDN2_GATES_COUPLED: a [T, H_v, d_k] fp32, b = beta [T, H_v] fp32, w unused
 *                       (may be NULL) (gdn2_chunk_forward_coupled);
 *   GDN2_GATES_SCALAR : a = alpha [T, H_v], b = beta [T, H_v] fp32, w unused
 *                       (gdn2_chunk_forward_scalar).
 * Any other value is GDN2_ERR_UNSUPPORTED. */
typedef enum {
  GDN2_GATES_CHANNEL = 0,
  GDN2_GATES_PREACT = 1,
  GDN2_GATES_COUPLED = 2,
  GDN2_GATES_SCALAR = 3
} gdn2_gates;

/* gdn2_chunk_forward_varlen for any gate form: packed sequences exactly as
 * there (cu_seqlens, one state per sequence, no workspace, each sequence
 * computed as the unpacked call of the same gate form computes it alone),
 * with the gates of `gates` (token axis of T tokens in all). Serving a model
 * of the Gated DeltaNet form over a packed batch is GDN2_GATES_SCALAR.
 * Errors as for gdn2_chunk_forward_varlen, the gate tensors checked for
 * overlap with the output at their own sizes. */
gdn2_status gdn2_chunk_forward_varlen_gates(const gdn2_desc *desc, const int32_t *cu_seqlens, gdn2_gates gates,
                                            const void *q, const void *k, const void *v, const void *a,
                                            const void *b, const void *w, const float *S0, void *o, float *S_T,
                                            void *stream);

/* Prefill with the per-channel gates given as pre-activations: a_pre, b_pre
 * ([B, T, H_v, d_k]) and w_pre ([B, T, H_v, d_v]) in the input dtype
 * (desc->dtype, bf16 or fp32) instead of fp32 activated values. The kernel
 * activates them in fp32: decay a = exp(-softplus(a_pre)) = 1 / (1 + e^a_pre),
 * erase gate b = sigmoid(b_pre), write gate w = sigmoid(w_pre) (values in
 * (0, 1) as the step above needs; the pages describe the gates only as
 * channel-wise values, and this is the usual parameterisation of such
 * gates). With bf16 inputs the gates cross HBM at half the bytes. Everything
 * else (layouts, S0/S_T, workspace, splitting, errors) is as for
 * gdn2_chunk_forward; the gate tensors are checked for overlap with the
 * output at their input-dtype size. */
gdn2_status gdn2_chunk_forward_preact(const gdn2_desc *desc, const void *q, const void *k, const void *v,
                                      const void *a_pre, const void *b_pre, const void *w_pre, const float *S0,
                                      void *o, float *S_T, void *workspace, size_t workspace_bytes,
                                      void *stream);

/* Decode: one token per sequence (desc->T must be 1). Reads the state S,
 * applies the step above and writes S back in place, and writes o.
 * Inputs are shaped as for the prefill with T = 1 (B = number of sequences).
 * S streams through HBM once: read once, written once. */
gdn2_status gdn2_decode_step(const gdn2_desc *desc, const void *q, const void *k, const void *v,
                             const float *a, const float *b, const float *w, float *S, void *o,
                             void *stream);

/* gdn2_decode_step in any gate form (gdn2_gates): a, b, w shaped as for
 * gdn2_chunk_forward_varlen_gates with one token per sequence ([B, 1, H_v, d_k]
 * per-channel gates or their pre-activations in the input dtype; beta and
 * alpha [B, 1, H_v] fp32, 4-byte alignment; w unused, may be NULL, for the
 * coupled and scalar forms), i.e. the decode of gdn2_chunk_forward_preact,
 * _coupled and _scalar. The gates are staged once per head before the state
 * streams through, so every form moves the same state bytes. Errors as for
 * gdn2_decode_step; an unknown form is GDN2_ERR_UNSUPPORTED. */
gdn2_status gdn2_decode_step_gates(const gdn2_desc *desc, gdn2_gates gates, const void *q, const void *k,
                                   const void *v, const void *a, const void *b, const void *w, float *S, void *o,
                                   void *stream);

/* Backward pass of gdn2_chunk_forward: the gradients of a loss with respect
 * to every input, given its gradients dO = dLoss/do and dS_T = dLoss/dS_T.
 * The pages define no backward pass; training the layer (the Gated
 * DeltaNet-2 post on tilnote.io reports a 1.3B-parameter model trained on
 * 100B tokens) needs the exact derivative of the forward map above, which
 * is what this computes (in chunk form or through the per-token recurrence:
 * see "How it runs" below).
 *
 * Arguments (all device pointers, caller-owned, contiguous row-major):
 *   desc : as for gdn2_chunk_forward. The chunk length is checked as there
 *          but does not change the method or the result.
 *   q, k, v, a, b, w, S0 : the forward call's inputs (S0 may be NULL: zero).
 *   dO   : [B, T, H_v, d_v] in the input dtype.
 *   dS_T : [B, H_v, d_k, d_v] fp32, or NULL (zero: S_T unused by the loss).
 *   dq, dk : [B, T, H_qk, d_k] in the input dtype; a query/key head shared by
 *          several value heads gets the sum of their gradients.
 *   dv   : [B, T, H_v, d_v] in the input dtype.
 *   da, db : [B, T, H_v, d_k] fp32.   dw : [B, T, H_v, d_v] fp32.
 *   dS0  : [B, H_v, d_k, d_v] fp32, or NULL (not written). It may be the
 *          same pointer as dS_T (in place), but not a partial overlap.
 *   workspace : gdn2_chunk_backward_workspace_bytes(desc) bytes, 256-byte
 *          aligned; NULL only when that size is 0. Contents on return are
 *          unspecified. Its size:
 *          - bf16 inputs with d_k = d_v = 128 (the chunk form below): per
 *            32-token chunk and value head the state entering it and the
 *            adjoint of the state leaving it (bf16, d_k * d_v each), the
 *            chunk's adjoint operands (3 * 32 * d_k bf16) and its decay
 *            (d_k fp32), plus one more state per sequence and value head:
 *            about 2.8 KB per token and value head, 1.49 GB at B8 T4096 H16;
 *            with few long sequences (segments below) also three fp32
 *            d_k * d_v states per segment and value head (2.97 GB at B1
 *            T65536 H16, 8 segments); and at least what the per-token
 *            backward needs in rounds;
 *          - otherwise (the per-token backward): fp32 state checkpoints
 *            every 4 tokens, per 64-column block key-side partial sums and
 *            every token's k-read, about
 *            (d_k * d_v / 4 + (4 * d_k + 1) * ceil(d_v / 64) + d_v) * 4 bytes
 *            per token and value head, plus d_k * d_v * 4 per sequence and
 *            value head (more with the segment split below).
 * How it runs. bf16 inputs with d_k = d_v = 128, every gate form: in chunk
 * form on the matrix cores (the prefill run again storing the state at every
 * 32-token chunk boundary; per chunk the operands of the state adjoint's
 * chunk step; the adjoint swept from the last chunk to the first; every
 * gradient of a chunk from its entering state and exiting adjoint). Few long
 * sequences (where the prefill's split plan, allowed up to two rounds of
 * first-pass workgroups, would cut them into segments of equal length;
 * GDN2_PREFILL_SPLIT included) run both sequential parts over the segments at
 * once: the chunk states from every segment's exact entering state (the
 * prefill's split passes), and the adjoint sweep as the prefill's split in
 * reverse (each segment from a zero exiting adjoint and on the identity's
 * columns, the exact exiting adjoints handed from segment to segment, then
 * every segment again from its own). Its
 * products take bf16 operands with fp32 accumulation, the states and
 * adjoints at chunk boundaries rounded to bf16 (the prefill's own rounding
 * of its chunk products), within the bf16 tolerance. A chunk in which some
 * key channel decays by less than e^-60 over each half (the prefill steps
 * such chunks token by token) is beyond its operands' range: then (the
 * stream is synchronised once to find out) the per-token backward runs
 * instead, in rounds of 512-token segments that fit this workspace.
 * Otherwise the per-token backward: reverse mode through the recurrence,
 * fp32 arithmetic; with few sequences x value heads and long sequences as
 * segments in parallel (entering states from the prefill's split passes,
 * exiting adjoints from one adjoint-only sweep, then each segment as a
 * packed sequence), which the workspace query accounts for; gradients that
 * depend on the forward states then carry the prefill's rounding. The
 * environment variables GDN2_BACKWARD_CHUNKED (0: never the chunk form,
 * and the query returns the per-token size; 2: only the chunk form, failing
 * with GDN2_ERR_HIP where it cannot run) and GDN2_BACKWARD_SPLIT=<n> (n
 * segments for the per-token backward; 1: never split) are read at each
 * call. Gradients of bf16 inputs are rounded to bf16 (RNE) from fp32 sums.
 * The result is deterministic (no atomics).
 * Errors: as for gdn2_chunk_forward; a missing required pointer is
 * GDN2_ERR_NULL_POINTER, a small or misaligned workspace GDN2_ERR_WORKSPACE /
 * GDN2_ERR_BAD_SHAPE, and an output or the workspace overlapping an input,
 * another output or each other GDN2_ERR_ALIAS. */
size_t gdn2_chunk_backward_workspace_bytes(const gdn2_desc *desc);
gdn2_status gdn2_chunk_backward(const gdn2_desc *desc, const void *q, const void *k, const void *v,
                                const float *a, const float *b, const float *w, const float *S0,
                                const void *dO, const float *dS_T, void *dq, void *dk, void *dv, float *da,
                                float *db, float *dw, float *dS0, void *workspace, size_t workspace_bytes,
                                void *stream);

/* Backward pass of gdn2_chunk_forward_preact: arguments as for
 * gdn2_chunk_backward with a_pre, b_pre, w_pre the forward call's gate
 * pre-activations (input dtype), and da_pre, db_pre, dw_pre the gradients
 * with respect to them, in the input dtype (through the activations:
 * d exp(-softplus(x))/dx = -a (1 - a), d sigmoid(x)/dx = s (1 - s)). The
 * workspace is gdn2_chunk_backward_workspace_bytes(desc) bytes. */
gdn2_status gdn2_chunk_backward_preact(const gdn2_desc *desc, const void *q, const void *k, const void *v,
                                       const void *a_pre, const void *b_pre, const void *w_pre, const float *S0,
                                       const void *dO, const float *dS_T, void *dq, void *dk, void *dv,
                                       void *da_pre, void *db_pre, void *dw_pre, float *dS0, void *workspace,
                                       size_t workspace_bytes, void *stream);

/* Backward pass of gdn2_chunk_forward_coupled (erase and write gate one
 * scalar beta per token and value head, b = beta * ones(d_k),
 * w = beta * ones(d_v)). Arguments as for gdn2_chunk_backward, with
 *   a     : [B, T, H_v, d_k] fp32 per-channel decay, da its gradient (same shape);
 *   beta  : [B, T, H_v] fp32; dbeta : [B, T, H_v] fp32, the gradient of beta
 *           through both of its uses: the sum over the key channels of the
 *           erase gate's gradient plus the sum over the value columns of the
 *           write gate's gradient (chain rule through the broadcasts).
 * No write-gate gradient is written. The workspace is
 * gdn2_chunk_backward_workspace_bytes(desc) bytes; errors as there. */
gdn2_status gdn2_chunk_backward_coupled(const gdn2_desc *desc, const void *q, const void *k, const void *v,
                                        const float *a, const float *beta, const float *S0, const void *dO,
                                        const float *dS_T, void *dq, void *dk, void *dv, float *da, float *dbeta,
                                        float *dS0, void *workspace, size_t workspace_bytes, void *stream);

/* Backward pass of gdn2_chunk_forward_scalar (a = alpha * ones(d_k) as well):
 * as gdn2_chunk_backward_coupled with alpha : [B, T, H_v] fp32 and
 * dalpha : [B, T, H_v] fp32, the sum over the key channels of the decay's
 * gradient. */
gdn2_status gdn2_chunk_backward_scalar(const gdn2_desc *desc, const void *q, const void *k, const void *v,
                                       const float *alpha, const float *beta, const float *S0, const void *dO,
                                       const float *dS_T, void *dq, void *dk, void *dv, float *dalpha, float *dbeta,
                                       float *dS0, void *workspace, size_t workspace_bytes, void *stream);

/* Backward pass of gdn2_chunk_forward_varlen: desc->B sequences packed along
 * desc->T tokens, sequence n = tokens cu_seqlens[n] .. cu_seqlens[n+1]-1
 * (cu_seqlens: B + 1 non-decreasing int32 device offsets; offsets outside
 * [0, T] are clamped). The token tensors (q, k, v, a, b, w, dO and the token
 * gradients) hold desc->T tokens; S0, dS_T and dS0 hold one state per
 * sequence. Packed sequences run the per-token backward: each sequence's
 * gradients are those of gdn2_chunk_backward's per-token backward on that
 * sequence alone, bit for bit (equal to its chunk form up to rounding). The
 * workspace is gdn2_chunk_backward_varlen_workspace_bytes(desc) bytes (the
 * per-token backward's regions over T tokens in all). Errors as for
 * gdn2_chunk_backward, plus GDN2_ERR_NULL_POINTER for a null cu_seqlens when
 * B > 0. */
size_t gdn2_chunk_backward_varlen_workspace_bytes(const gdn2_desc *desc);
gdn2_status gdn2_chunk_backward_varlen(const gdn2_desc *desc, const int32_t *cu_seqlens, const void *q,
                                       const void *k, const void *v, const float *a, const float *b, const float *w,
                                       const float *S0, const void *dO, const float *dS_T, void *dq, void *dk,
                                       void *dv, float *da, float *db, float *dw, float *dS0, void *workspace,
                                       size_t workspace_bytes, void *stream);

/* gdn2_chunk_backward_varlen for any gate form (gdn2_gates): the gradients of
 * gdn2_chunk_forward_varlen_gates. Gate gradients take the shapes and types
 * of the gates, as in the unpacked backward of the same form: da, db, dw
 * (CHANNEL, fp32; PREACT, input dtype, gradients of the pre-activations);
 * da and db = dbeta (COUPLED; SCALAR: da = dalpha [T, H_v]), dw unused (may
 * be NULL). Workspace: gdn2_chunk_backward_varlen_workspace_bytes(desc);
 * each sequence's gradients are those of the unpacked call's per-token
 * backward on it alone.
 * Errors as for gdn2_chunk_backward_varlen. */
gdn2_status gdn2_chunk_backward_varlen_gates(const gdn2_desc *desc, const int32_t *cu_seqlens, gdn2_gates gates,
                                             const void *q, const void *k, const void *v, const void *a,
                                             const void *b, const void *w, const float *S0, const void *dO,
                                             const float *dS_T, void *dq, void *dk, void *dv, void *da, void *db,
                                             void *dw, float *dS0, void *workspace, size_t workspace_bytes,
                                             void *stream);

/* Static, human-readable text for a status code. */
const char *gdn2_status_string(gdn2_status status);

/* Library version: major * 10000 + minor * 100 + patch. */
int gdn2_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN2_H_ */
