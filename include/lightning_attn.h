/*
 * lightning_attn.h -- C ABI of the MI355X (gfx950) lightning attention library.
 *
 * What is computed: causal linear attention with a per-head scalar decay, in
 * the blockwise ("lightning") form.  For every (sequence, head) with decay
 * lambda in (0, 1], rows q_t, k_t, v_t in R^d and a d x d state S:
 *
 *     S_t = lambda * S_{t-1} + k_t^T v_t,      o_t = q_t S_t,
 *
 * i.e. o_t = sum_{s<=t} lambda^(t-s) (q_t . k_s) v_s + lambda^(t+1) q_t S_init.
 * Sources: MiniMax-01 technical report (full Chinese translation on
 * blog.csdn.net), section 2.2.1 "Lightning Attention" (causal left product,
 * eq. 4, with the diagonal included; right-product recurrence, eq. 5; block
 * split into a left product inside blocks and a right product between
 * blocks, with the block state carried forward and kv_0 = 0), section 2.2.4
 * (recurrent form, eq. 12, used for decoding), section 3.2.2 and Fig. 12
 * (diagonal decay matrix; LASP+ local prefix states combined into global
 * ones), section 3.3.1-3.3.2 (fused prefill front end; fused decode state
 * update; prefill and decode as separate kernels); K3 reading notes
 * (cutenote.app), "position decay term" and "CP for linear attention" (any
 * chunking gives the same result).  The report leaves normalisation, SiLU
 * and the output gate out of the derivation; the plain entry points compute
 * the recurrence alone, and lightning_attn_fwd_gated adds one stated reading
 * of those steps around it.
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates device memory, never synchronises and is re-entrant; the
 *     only state it keeps between calls is the per-thread diagnostic string of
 *     lightning_attn_last_hip_error.  Every kernel is launched asynchronously
 *     on `hip_stream` (a hipStream_t; NULL = the null stream).  The prefill
 *     schedule may be chosen with the environment variable
 *     LIGHTNING_ATTN_PREFILL=phased|fused (read at each call, the workspace
 *     size queries included, so keep it fixed between a query and the call
 *     it sizes; default phased); both give the same results up to rounding.
 *     The fused schedule hands states between workgroups through flags in
 *     the workspace; a wait that exceeds its bound (a stalled GPU, never a
 *     normal run) gives up rather than hang and makes the outputs and final
 *     states of the affected head NaN from that segment on, so such a failure
 *     is never a silently wrong result.
 *   - Arrays are dense and row-major with d fastest.  Outputs must not alias
 *     inputs (decode's `state` is read-modify-write by design).  Every
 *     tensor, state, snapshot and workspace pointer must be 16-byte aligned
 *     (the kernels move 16 bytes per access); a misaligned one is
 *     LA_ERR_INVALID_ARG.
 *   - q, k, v and out share one element type: LA_BF16 (bfloat16) or LA_FP32.
 *     States (init, final, decode state) are always float32, laid out
 *     S[i][j] with i the key feature (row) and j the value feature.
 *   - decay[h] is head h's lambda as float32; 0 < lambda <= 1 is a
 *     precondition the library does not check (it would need a device read).
 *   - Arithmetic: bf16 inputs run on bf16 MFMA with float32 accumulation and
 *     a float32 state (the state and the masked scores are rounded to bf16 as
 *     MFMA operands); float32 inputs run in float32 throughout.
 *   - Errors: arguments are validated before anything is launched; a failed
 *     validation launches nothing and leaves every buffer untouched.  Sizes
 *     beyond what one launch can hold are LA_ERR_UNSUPPORTED: more than 2^40
 *     tokens, a plan with more than 2^23 - 1 (segment, head) pairs (a HIP
 *     launch holds at most 2^32 - 1 work-items; the output pass runs 512
 *     threads per pair), or a decode step over more than 2^24 - 1
 *     (sequence, head) pairs.  After the launches, a HIP launch error maps to
 *     LA_ERR_HIP.  Faults inside a kernel surface at the caller's next
 *     synchronisation, as usual for HIP.  No C++ exception crosses this
 *     interface.
 */
#ifndef LIGHTNING_ATTN_H
#define LIGHTNING_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Each enum ends with a *_FORCE_INT32 value that is never used: it makes
 * every int a valid value of the type, so an out-of-range code a C caller
 * passes is rejected as documented (LA_ERR_UNSUPPORTED, "unknown status")
 * rather than being undefined in the C++ implementation. */
typedef enum {
  LA_OK = 0,
  LA_ERR_INVALID_ARG = 1,  /* NULL pointer where data is needed, negative size */
  LA_ERR_UNSUPPORTED = 2,  /* d not in {64, 128}, block not LA_BLOCK_AUTO or one of
                              16, 32, 64, 128, 256, dtype */
  LA_ERR_WORKSPACE = 3,    /* workspace NULL or smaller than *_workspace_size */
  LA_ERR_HIP = 4,          /* a HIP launch reported an error */
  LA_STATUS_FORCE_INT32 = 0x7fffffff
} la_status;

typedef enum { LA_FP32 = 0, LA_BF16 = 1, LA_DTYPE_FORCE_INT32 = 0x7fffffff } la_dtype;

/* segment_tokens value of the prefill entry points: every sequence is one
 * segment, walked by one workgroup per head.  No state crosses a segment,
 * so the output pass is the only launch and no workspace is needed (the
 * workspace size queries return 0).  The choice for batches of many short
 * sequences (serving), whose cost is the launch chain, not the arithmetic;
 * a long sequence is then walked by a single workgroup per head. */
enum { LA_SEGMENT_PER_SEQUENCE = -1 };

/* block value of every entry point that takes one: the library picks the
 * level from the mean input length of the call, as the MiniMax-01 report's
 * multi-level padding (section 3.3.3) picks 32, 64, 128 or 256 by length.
 * The mean is N for fixed-length calls and ceil(total_N / num_seqs) for
 * packed ones (both known on the host): at most 32 tokens -> block 32, at
 * most 64 -> 64, longer -> 128.  Deterministic for given sizes, and the
 * workspace size queries resolve it the same way. */
enum { LA_BLOCK_AUTO = 0 };

/* Memory layout of q, k, v and out for the *_layout entry points (the other
 * prefill entry points take LA_HEAD_MAJOR).  LA_TOKEN_MAJOR is the layout a
 * projection produces ([B][N][H*d], heads side by side in each token row),
 * read and written as it is: the kernels address every token row through a
 * row stride, so no layout pass runs in front of or behind the attention
 * (MiniMax-01 report, section 3.3.1: the prefill front-end's layout
 * adjustment is folded into the kernels that read Q, K and V). */
typedef enum {
  LA_HEAD_MAJOR = 0,  /* fixed: [B][H][N][d];  packed: [H][total_N][d] */
  LA_TOKEN_MAJOR = 1, /* fixed: [B][N][H][d];  packed: [total_N][H][d] */
  LA_LAYOUT_FORCE_INT32 = 0x7fffffff
} la_layout;

/* Human-readable name of a status code (static storage; never NULL). */
const char *lightning_attn_status_string(la_status s);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int lightning_attn_version(void);

/* Diagnostic: the HIP error string behind the most recent LA_ERR_HIP
 * returned on the calling thread ("no HIP error" if none).  Static storage. */
const char *lightning_attn_last_hip_error(void);

/*
 * Prefill over fixed-length sequences (MiniMax-01 report, section 2.2.1,
 * block expansion; section 3.2.2 for the sequence-parallel state scan).
 *
 *   q, k, v, out : [B][H][N][d] of `dt`.
 *   decay        : [H] float32.
 *   block        : block (chunk) length of the blockwise form, one of
 *                  16, 32, 64, 128, 256, or LA_BLOCK_AUTO (the level from
 *                  the mean input length).  Any block length gives the same
 *                  result up to rounding (K3 notes, CP for linear
 *                  attention).  It chooses the kernel the way the MiniMax-01
 *                  report's multi-level padding (section 3.3.3) chooses a
 *                  block by input length: for bf16 with d = 128, 128 and 256
 *                  run 128-token chunks (one workgroup per CU), 64 runs
 *                  64-token and 16 or 32 run 32-token chunks (two workgroups
 *                  per CU, the choice for short inputs: decode-like and
 *                  prefix-continuation batches).  float32 inputs and d = 64
 *                  run 32-token chunks for every block.  The workspace size
 *                  query takes the same block.
 *   init_state   : [B][H][d][d] float32, or NULL for a zero initial state.
 *   final_state  : [B][H][d][d] float32 state after token N-1 (equal to the
 *                  initial state when N == 0), or NULL if not wanted.
 *   segment_tokens: 0 = automatic.  LA_SEGMENT_PER_SEQUENCE: every
 *                  sequence is one segment (for fixed lengths the same as N).
 *                  Otherwise the length, in tokens, of the independent
 *                  segments the token axis is cut into (results are
 *                  identical up to rounding for every value).  A value equal
 *                  to N keeps every sequence in one segment and needs no
 *                  workspace.
 *   workspace    : device scratch of at least
 *                  lightning_attn_fwd_workspace_size(...) bytes (may be NULL
 *                  when that size is 0).  Its contents on entry do not matter.
 *
 * B, H >= 0, N >= 0, d in {64, 128}.  B*H == 0 is a no-op.  q, k, v, out may
 * be NULL only when N == 0.  Returns LA_ERR_INVALID_ARG for a negative
 * segment_tokens other than LA_SEGMENT_PER_SEQUENCE.
 */
size_t lightning_attn_fwd_workspace_size(int B, int H, int64_t N, int d, int block, la_dtype dt,
                                         int64_t segment_tokens);

la_status lightning_attn_fwd(const void *q, const void *k, const void *v, const float *decay,
                             int B, int H, int64_t N, int d, int block, la_dtype dt,
                             const float *init_state, void *out, float *final_state,
                             int64_t segment_tokens, void *workspace, size_t workspace_bytes,
                             void *hip_stream);

/*
 * lightning_attn_fwd for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  The same computation, arguments and results as
 * lightning_attn_fwd, without the workspace: the prefill's scratch (the
 * segment states) lives in a device array inside the library,
 * lightning_attn_noalloc_scratch_bytes() bytes (256 MiB) on every GPU the
 * library runs on, held from its first use until the process ends.  The
 * call allocates nothing; the device address of that array is looked up on
 * the first call on a device, which must be the current device (the one
 * hip_stream belongs to).
 *
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind (nothing in it needs to start at zero; the single-pass schedule
 * clears its flags with a kernel).  Calls that overlap on one GPU (other
 * streams, other host threads) race on it and give wrong results: order
 * them on one stream, or use lightning_attn_fwd with a workspace each.
 *
 * Returns LA_ERR_WORKSPACE, launching nothing, when the call needs more
 * scratch than the array holds, i.e. when lightning_attn_fwd_workspace_size
 * for the same arguments exceeds lightning_attn_noalloc_scratch_bytes()
 * (e.g. many short segments over many heads); LA_ERR_HIP if the array's
 * address cannot be obtained; otherwise as lightning_attn_fwd.
 */
size_t lightning_attn_noalloc_scratch_bytes(void);

la_status lightning_attn_fwd_noalloc(const void *q, const void *k, const void *v,
                                     const float *decay, int B, int H, int64_t N, int d,
                                     int block, la_dtype dt, const float *init_state, void *out,
                                     float *final_state, int64_t segment_tokens,
                                     void *hip_stream);

/*
 * lightning_attn_fwd with per-kernel timing (a measurement aid; the same
 * computation as lightning_attn_fwd, for which phase_events == NULL).
 *
 *   phase_events : NULL, or an array of 4 hipEvent_t handles owned by the
 *                  caller (created on the stream's device; timing-enabled if
 *                  durations are wanted).  They are recorded on hip_stream:
 *                  [0] before the first launch of the call, [1] after the
 *                  segment local-state pass, [2] after the segment scan,
 *                  [3] after the output pass.  A phase the plan does not run
 *                  (no scan for single-segment sequences; the single-pass
 *                  kernel does all three) records its event at the same point
 *                  as the one before it.
 *
 * A call that launches nothing (B*H == 0, or N == 0 without final_state)
 * records no event.  Returns LA_ERR_HIP if recording an event fails (after
 * launching the work); otherwise as lightning_attn_fwd.
 */
la_status lightning_attn_fwd_timed(const void *q, const void *k, const void *v,
                                   const float *decay, int B, int H, int64_t N, int d, int block,
                                   la_dtype dt, const float *init_state, void *out,
                                   float *final_state, int64_t segment_tokens, void *workspace,
                                   size_t workspace_bytes, void *hip_stream,
                                   void *const *phase_events);

/*
 * lightning_attn_fwd for either memory layout (la_layout): q, k, v and out
 * are [B][H][N][d] for LA_HEAD_MAJOR (exactly lightning_attn_fwd) or
 * [B][N][H][d] for LA_TOKEN_MAJOR, each row of d elements contiguous.
 * init_state / final_state keep the [B][H][d][d] layout.  The workspace size
 * does not depend on the layout.
 *
 * Returns LA_ERR_UNSUPPORTED for an unknown layout, or for LA_TOKEN_MAJOR
 * when 128 token rows span 2^31 bytes or more (H * d >= 4194304); otherwise
 * as lightning_attn_fwd.
 */
la_status lightning_attn_fwd_layout(const void *q, const void *k, const void *v,
                                    const float *decay, int B, int H, int64_t N, int d, int block,
                                    la_dtype dt, la_layout layout, const float *init_state,
                                    void *out, float *final_state, int64_t segment_tokens,
                                    void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * Prefill over packed variable-length sequences ("data packing", MiniMax-01
 * report section 3.2; varlen support for LASP+, section 3.2.2).  Sequence j
 * occupies tokens cu_seqlens[j] .. cu_seqlens[j+1]-1 of every head; the state
 * starts afresh at every sequence (from init_states[j], or zero), and no
 * padding is needed or applied.
 *
 *   q, k, v, out : [H][total_N][d] of `dt`.
 *   cu_seqlens   : [num_seqs + 1] int32 DEVICE array, non-decreasing, with
 *                  cu_seqlens[0] == 0 and cu_seqlens[num_seqs] == total_N
 *                  (a precondition; not checked, it lives on the device).
 *                  Zero-length sequences are allowed.
 *   init_states  : [num_seqs][H][d][d] float32 or NULL (zero).
 *   final_states : [num_seqs][H][d][d] float32 or NULL.
 *   segment_tokens: as for lightning_attn_fwd; segments are cut on the
 *                  concatenated token axis (they may start inside a
 *                  sequence), except with LA_SEGMENT_PER_SEQUENCE.
 *   Other arguments as for lightning_attn_fwd.
 */
size_t lightning_attn_fwd_varlen_workspace_size(int num_seqs, int H, int64_t total_N, int d,
                                                int block, la_dtype dt, int64_t segment_tokens);

la_status lightning_attn_fwd_varlen(const void *q, const void *k, const void *v,
                                    const float *decay, const int32_t *cu_seqlens, int num_seqs,
                                    int H, int64_t total_N, int d, int block, la_dtype dt,
                                    const float *init_states, void *out, float *final_states,
                                    int64_t segment_tokens, void *workspace,
                                    size_t workspace_bytes, void *hip_stream);

/*
 * lightning_attn_fwd_varlen for either memory layout: q, k, v and out are
 * [H][total_N][d] for LA_HEAD_MAJOR (exactly lightning_attn_fwd_varlen) or
 * [total_N][H][d] for LA_TOKEN_MAJOR.  Errors as lightning_attn_fwd_layout.
 */
la_status lightning_attn_fwd_varlen_layout(const void *q, const void *k, const void *v,
                                           const float *decay, const int32_t *cu_seqlens,
                                           int num_seqs, int H, int64_t total_N, int d, int block,
                                           la_dtype dt, la_layout layout,
                                           const float *init_states, void *out,
                                           float *final_states, int64_t segment_tokens,
                                           void *workspace, size_t workspace_bytes,
                                           void *hip_stream);

/*
 * lightning_attn_fwd_varlen_layout that also stores prefix-state snapshots:
 * the state of every sequence after each multiple of snapshot_interval of
 * its tokens, a prefix cache for linear attention (K3 reading notes,
 * "inference engine" part: a linear-attention state is rewritten at every
 * token, so keeping all of them defeats the method and keeping none loses
 * prefix caching; the cache keeps one prefix state per block).  A request
 * that shares the first m * snapshot_interval tokens of a cached sequence
 * continues from snapshot m as its init_states row and prefills only the
 * rest (MiniMax-01 report, sections 3.3.2-3.3.3: batches whose inputs carry
 * a prefix cache).
 *
 *   snapshot_interval: tokens between snapshots, >= 1.  Snapshot m (m = 1 ..
 *                  floor(n_j / snapshot_interval)) of sequence j, of length
 *                  n_j, is the state after its token m * snapshot_interval - 1
 *                  (counted from the sequence start, and including the
 *                  sequence's init_states row); when snapshot_interval
 *                  divides n_j the last snapshot equals the final state.
 *                  Chunks are cut at snapshot points, so an interval that is
 *                  a multiple of 128 tokens (bf16, d = 128) or 32 tokens
 *                  (otherwise) keeps the kernels' chunks whole.
 *   snapshot_offsets: [num_seqs + 1] int32 DEVICE array: snapshot m of
 *                  sequence j goes to row snapshot_offsets[j] + m - 1.  A
 *                  precondition (not checked, it lives on the device): the
 *                  rows of different snapshots are distinct and lie inside
 *                  `snapshots`, e.g. snapshot_offsets = the exclusive prefix
 *                  sum of floor(n_j / snapshot_interval).
 *   snapshots    : [rows][H][d][d] float32, written only at the rows above
 *                  (one row is a whole [H][d][d] state set, usable directly
 *                  as an init_states row).  Must not alias any other buffer.
 *                  snapshots and snapshot_offsets may be NULL when
 *                  snapshot_interval > total_N (no sequence reaches a
 *                  snapshot point); then nothing is stored.
 *   Other arguments and the workspace as for lightning_attn_fwd_varlen_layout
 *   (the workspace size does not depend on the snapshots).
 *
 * Returns LA_ERR_INVALID_ARG if snapshot_interval < 1, or if snapshots or
 * snapshot_offsets is NULL while snapshot_interval <= total_N; otherwise as
 * lightning_attn_fwd_varlen_layout.
 */
la_status lightning_attn_fwd_varlen_snapshots(
    const void *q, const void *k, const void *v, const float *decay, const int32_t *cu_seqlens,
    int num_seqs, int H, int64_t total_N, int d, int block, la_dtype dt, la_layout layout,
    const float *init_states, void *out, float *final_states, int64_t snapshot_interval,
    const int32_t *snapshot_offsets, float *snapshots, int64_t segment_tokens, void *workspace,
    size_t workspace_bytes, void *hip_stream);

/*
 * Prefill with the normalisation, SiLU activation and gate that the
 * MiniMax-01 report places around the attention of its TransNormer blocks
 * and leaves out of its derivation (section 2.2.1; it gives no formula).
 * The reading computed here, each part selected by a bit of `flags`:
 *
 *   LA_SILU_Q, LA_SILU_K, LA_SILU_V : q, k, v replaced by SiLU(x) =
 *        x / (1 + e^-x), elementwise, as they are read (the recurrence and
 *        the final state use the activated values);
 *   LA_NORM : every output row divided by its RMS over the head's d
 *        channels, sqrt(mean_j o[j]^2 + eps), then multiplied by
 *        norm_weight[h][j] (NULL: ones);
 *   LA_GATE : every output element multiplied by sigmoid(gate) =
 *        1 / (1 + e^-gate), gate laid out like out (an output gate computed
 *        by the caller, e.g. a projection of the layer input).
 *
 * Fused into the prefill: the activations are applied to the tiles as they
 * are loaded, the normalisation to the float32 accumulators of each output
 * row, weight and gate to the row as it is stored; nothing else reads or
 * writes out.  With flags == 0 this is lightning_attn_fwd_layout with
 * block 128 (bit for bit), always in the three-phase schedule.
 *
 *   flags        : any combination of LA_SILU_Q, LA_SILU_K, LA_SILU_V,
 *                  LA_NORM, LA_GATE (other bits: LA_ERR_INVALID_ARG).
 *   gate         : like out (q's layout and dtype); needed with LA_GATE,
 *                  else may be NULL.
 *   norm_weight  : [H][d] float32 or NULL; used with LA_NORM.
 *   eps          : >= 0 and finite; used with LA_NORM.
 *   Other arguments as for lightning_attn_fwd_layout, without `block`: the
 *   path runs 128-token chunks (a row's d channels sit in four lanes of one
 *   wave); workspace from lightning_attn_fwd_gated_workspace_size (the
 *   three-phase plan at block 128, whatever LIGHTNING_ATTN_PREFILL says).
 *   bf16 with d = 128 only (otherwise LA_ERR_UNSUPPORTED).
 */
enum { LA_SILU_Q = 1, LA_SILU_K = 2, LA_SILU_V = 4, LA_NORM = 8, LA_GATE = 16 };

size_t lightning_attn_fwd_gated_workspace_size(int B, int H, int64_t N, int d, la_dtype dt,
                                               int64_t segment_tokens);

la_status lightning_attn_fwd_gated(const void *q, const void *k, const void *v,
                                   const float *decay, int B, int H, int64_t N, int d,
                                   la_dtype dt, la_layout layout, int flags, const void *gate,
                                   const float *norm_weight, float eps,
                                   const float *init_state, void *out, float *final_state,
                                   int64_t segment_tokens, void *workspace,
                                   size_t workspace_bytes, void *hip_stream);

/*
 * lightning_attn_fwd_gated over packed variable-length sequences: the
 * arguments of lightning_attn_fwd_varlen_layout (without `block`) and the
 * gated ones above; gate laid out like out ([H][total_N][d] or
 * [total_N][H][d]); workspace from
 * lightning_attn_fwd_varlen_gated_workspace_size.
 */
size_t lightning_attn_fwd_varlen_gated_workspace_size(int num_seqs, int H, int64_t total_N, int d,
                                                      la_dtype dt, int64_t segment_tokens);

la_status lightning_attn_fwd_varlen_gated(const void *q, const void *k, const void *v,
                                          const float *decay, const int32_t *cu_seqlens,
                                          int num_seqs, int H, int64_t total_N, int d,
                                          la_dtype dt, la_layout layout, int flags,
                                          const void *gate, const float *norm_weight, float eps,
                                          const float *init_states, void *out,
                                          float *final_states, int64_t segment_tokens,
                                          void *workspace, size_t workspace_bytes,
                                          void *hip_stream);

/*
 * One recurrent decode step (MiniMax-01 report, section 2.2.4, eq. 12;
 * section 3.3.1, fused decode state update):
 *     state <- lambda_h * state + k^T v,   out = q state   (updated state).
 *
 *   q, k, v, out : [B][H][d] of `dt`.
 *   state        : [B][H][d][d] float32, read and rewritten in place.
 *   B, H >= 0 (B*H == 0 is a no-op), d in {64, 128}.
 */
la_status lightning_attn_decode(const void *q, const void *k, const void *v, const float *decay,
                                float *state, void *out, int B, int H, int d, la_dtype dt,
                                void *hip_stream);

/*
 * Prefill with channel-wise decay (K3 reading notes, "gated DeltaNet": the
 * scalar decay replaced by one decay per channel, strictly more general,
 * here without the delta rule): head h has a decay alpha[h][i] for every key
 * channel i,
 *     S_t[i][j] = alpha_i S_{t-1}[i][j] + k_t[i] v_t[j],   o_t = q_t S_t.
 * With all channels equal it is lightning_attn_fwd_layout.
 *
 *   alpha        : [H][d] float32 DEVICE array, 0 < alpha <= 1 (a
 *                  precondition, not checked: it lives on the device).
 *   Other arguments as for lightning_attn_fwd_layout (workspace from
 *   lightning_attn_fwd_chdecay_workspace_size).  bf16 with d = 128 runs on
 *   MFMA in 64-token chunks, the decay inside a chunk written as an absolute
 *   position around the chunk's middle row (Q scaled by alpha^(q-32), K by
 *   alpha^(32-c); the K3 notes bound the decay over such a window so that
 *   the factors stay inside the BF16 range).  A head whose smallest alpha is
 *   below 1/8 (where those factors would pass 2^96) runs its output pass on
 *   the vector-ALU kernel instead, in float32 with tabulated powers and no
 *   range limit (slower); so does every head for other inputs.  Always the
 *   three-phase segment schedule (LIGHTNING_ATTN_PREFILL is ignored).
 */
size_t lightning_attn_fwd_chdecay_workspace_size(int B, int H, int64_t N, int d, int block,
                                                 la_dtype dt, int64_t segment_tokens);

la_status lightning_attn_fwd_chdecay(const void *q, const void *k, const void *v,
                                     const float *alpha, int B, int H, int64_t N, int d, int block,
                                     la_dtype dt, la_layout layout, const float *init_state,
                                     void *out, float *final_state, int64_t segment_tokens,
                                     void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * Channel-wise decay over packed variable-length sequences: the arguments
 * of lightning_attn_fwd_varlen_layout with alpha [H][d] (as above) in place
 * of the per-head decay; workspace from
 * lightning_attn_fwd_chdecay_varlen_workspace_size.  LA_SEGMENT_PER_SEQUENCE
 * is not offered here (LA_ERR_UNSUPPORTED).
 */
size_t lightning_attn_fwd_chdecay_varlen_workspace_size(int num_seqs, int H, int64_t total_N,
                                                        int d, int block, la_dtype dt,
                                                        int64_t segment_tokens);

la_status lightning_attn_fwd_chdecay_varlen(const void *q, const void *k, const void *v,
                                            const float *alpha, const int32_t *cu_seqlens,
                                            int num_seqs, int H, int64_t total_N, int d,
                                            int block, la_dtype dt, la_layout layout,
                                            const float *init_states, void *out,
                                            float *final_states, int64_t segment_tokens,
                                            void *workspace, size_t workspace_bytes,
                                            void *hip_stream);

/*
 * One recurrent decode step with channel-wise decay (the decode counterpart
 * of lightning_attn_fwd_chdecay):
 *     state[i][j] <- alpha[h][i] state[i][j] + k[i] v[j],   out = q state.
 *   alpha : [H][d] float32 DEVICE array.  Other arguments, layouts and errors
 *           as for lightning_attn_decode.
 */
la_status lightning_attn_decode_chdecay(const void *q, const void *k, const void *v,
                                        const float *alpha, float *state, void *out, int B, int H,
                                        int d, la_dtype dt, void *hip_stream);

/*
 * Backward pass of the fixed-length prefill (training): the gradients of a
 * scalar loss L with respect to q, k, v and the initial state, given
 * dout = dL/dout and dfinal = dL/dfinal_state.  The pages train with
 * lightning attention (MiniMax-01 report, section 2.2.2.4 and Fig. 8:
 * training speed in tokens per GPU per second) but print no backward pass;
 * this one is the derivative of the recurrence above.  With G_t = dL/dS_t
 * (G_t = q_t^T do_t + lambda G_{t+1}, starting from dfinal):
 *     dq_t = do_t S_t^T,   dk_t = v_t G_t^T,   dv_t = k_t G_t,
 *     dinit = lambda G_0   (dfinal when N == 0).
 * Each of dq, dk, dv is itself a decayed linear attention (dq causal over
 * (do, v, k) from init^T; dv and dk anti-causal over (k, q, do) and
 * (v, do, q) from dfinal), computed by the prefill kernels, the anti-causal
 * ones over a time-reversed view of the same buffers.
 *
 *   q, k, v, dout        : as for lightning_attn_fwd_layout (layout selects
 *                          [B][H][N][d] or [B][N][H][d]), of `dt`.
 *   dfinal, init_state   : [B][H][d][d] float32, or NULL (zero).
 *   dq, dk, dv           : outputs, q's layout and dtype.
 *   dinit                : [B][H][d][d] float32 output, or NULL if not wanted.
 *   workspace            : device scratch of at least
 *                          lightning_attn_bwd_workspace_size(...) bytes (always
 *                          nonzero: the backward keeps four state sets there).
 *   Other arguments as for lightning_attn_fwd_layout.  The prefill schedule is
 *   always the three-phase one (LIGHTNING_ATTN_PREFILL is ignored here).
 *
 * Preconditions (not checked): lambda > 0 with |dfinal| / lambda finite in
 * float32 (the anti-causal passes start from dfinal / lambda).  Returns as
 * lightning_attn_fwd_layout; LA_ERR_WORKSPACE if the workspace is NULL or
 * smaller than the size above.
 */
size_t lightning_attn_bwd_workspace_size(int B, int H, int64_t N, int d, int block, la_dtype dt,
                                         int64_t segment_tokens);

la_status lightning_attn_bwd(const void *q, const void *k, const void *v, const float *decay,
                             const void *dout, const float *dfinal, const float *init_state,
                             void *dq, void *dk, void *dv, float *dinit, int B, int H, int64_t N,
                             int d, int block, la_dtype dt, la_layout layout,
                             int64_t segment_tokens, void *workspace, size_t workspace_bytes,
                             void *hip_stream);

/*
 * A forward / backward pair for training (MiniMax-01 report, section
 * 2.2.2.4, the trained lightning attention).  The backward's dq pass is
 * itself a causal decayed linear attention whose state is S_t^T, so its
 * segment entering states are the forward's, transposed: a forward that
 * keeps them lets the backward skip that pass's local-state pass and scan.
 *
 * lightning_attn_saved_states_size: bytes of `saved` for these arguments
 * ([nseg][H][d][d] float32 for the backward's segment plan), 0 when the plan
 * cuts no sequence (nothing to keep; `saved` may then be NULL).
 *
 * lightning_attn_fwd_save: lightning_attn_fwd_layout on the backward's
 * segment plan (always the three-phase schedule; LIGHTNING_ATTN_PREFILL is
 * ignored), which also writes the transposed entering state of every
 * segment into `saved` (device, caller-owned, saved_bytes at least the size
 * above).  The workspace must hold lightning_attn_bwd_workspace_size(...)
 * bytes for the same arguments (the pair can share one workspace).  Returns
 * LA_ERR_INVALID_ARG for a missing or short `saved`, otherwise as
 * lightning_attn_fwd_layout.
 *
 * lightning_attn_bwd_saved: lightning_attn_bwd, taking the dq pass's
 * segment entering states from `saved`, which must come from a
 * lightning_attn_fwd_save call with the same q, k, v, decay, init_state and
 * shape arguments (segment_tokens included) and be unchanged since;
 * anything else gives wrong dq without an error.  dk, dv and dinit do not
 * use it.  Results equal lightning_attn_bwd's to float32 rounding.
 */
size_t lightning_attn_saved_states_size(int B, int H, int64_t N, int d, int block, la_dtype dt,
                                        int64_t segment_tokens);

la_status lightning_attn_fwd_save(const void *q, const void *k, const void *v, const float *decay,
                                  int B, int H, int64_t N, int d, int block, la_dtype dt,
                                  la_layout layout, const float *init_state, void *out,
                                  float *final_state, int64_t segment_tokens, float *saved,
                                  size_t saved_bytes, void *workspace, size_t workspace_bytes,
                                  void *hip_stream);

la_status lightning_attn_bwd_saved(const void *q, const void *k, const void *v, const float *decay,
                                   const void *dout, const float *dfinal, const float *init_state,
                                   void *dq, void *dk, void *dv, float *dinit, int B, int H,
                                   int64_t N, int d, int block, la_dtype dt, la_layout layout,
                                   int64_t segment_tokens, const float *saved, size_t saved_bytes,
                                   void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * The training pair for packed variable-length sequences: as above, with the
 * arguments of lightning_attn_fwd_varlen_layout and lightning_attn_bwd_varlen
 * (workspace from lightning_attn_bwd_varlen_workspace_size; `saved` sized by
 * lightning_attn_varlen_saved_states_size, 0 when no segment cuts a
 * sequence, as with LA_SEGMENT_PER_SEQUENCE).  cu_seqlens must be the same
 * in both calls.
 */
size_t lightning_attn_varlen_saved_states_size(int num_seqs, int H, int64_t total_N, int d,
                                               int block, la_dtype dt, int64_t segment_tokens);

la_status lightning_attn_fwd_varlen_save(const void *q, const void *k, const void *v,
                                         const float *decay, const int32_t *cu_seqlens,
                                         int num_seqs, int H, int64_t total_N, int d, int block,
                                         la_dtype dt, la_layout layout, const float *init_states,
                                         void *out, float *final_states, int64_t segment_tokens,
                                         float *saved, size_t saved_bytes, void *workspace,
                                         size_t workspace_bytes, void *hip_stream);

la_status lightning_attn_bwd_varlen_saved(const void *q, const void *k, const void *v,
                                          const float *decay, const void *dout,
                                          const int32_t *cu_seqlens, int num_seqs, int H,
                                          int64_t total_N, int d, int block, la_dtype dt,
                                          la_layout layout, const float *dfinals,
                                          const float *init_states, void *dq, void *dk, void *dv,
                                          float *dinits, int64_t segment_tokens,
                                          const float *saved, size_t saved_bytes,
                                          void *workspace, size_t workspace_bytes,
                                          void *hip_stream);

/*
 * lightning_attn_bwd for packed variable-length sequences (training on
 * packed data, MiniMax-01 report section 3.2): q, k, v, dout, dq, dk, dv as
 * for lightning_attn_fwd_varlen_layout; dfinals, init_states and dinits are
 * [num_seqs][H][d][d] float32 (dfinals and init_states may be NULL, dinits
 * NULL when not wanted).  Every sequence is independent; a zero-length
 * sequence gets dinits = dfinals.  The anti-causal passes run over a
 * time-reversed view of each sequence in place.  Workspace from
 * lightning_attn_bwd_varlen_workspace_size; other arguments, preconditions
 * and errors as for lightning_attn_bwd and lightning_attn_fwd_varlen_layout.
 */
size_t lightning_attn_bwd_varlen_workspace_size(int num_seqs, int H, int64_t total_N, int d,
                                                int block, la_dtype dt, int64_t segment_tokens);

la_status lightning_attn_bwd_varlen(const void *q, const void *k, const void *v,
                                    const float *decay, const void *dout,
                                    const int32_t *cu_seqlens, int num_seqs, int H,
                                    int64_t total_N, int d, int block, la_dtype dt,
                                    la_layout layout, const float *dfinals,
                                    const float *init_states, void *dq, void *dk, void *dv,
                                    float *dinits, int64_t segment_tokens, void *workspace,
                                    size_t workspace_bytes, void *hip_stream);

/*
 * One step of a mixed serving batch (MiniMax-01 report, section 3.3.2:
 * inputs of one token are memory-bound and need few compute units, so they
 * go to a kernel of their own, separate from the inputs of more than one
 * token, and the two kernels run in parallel on two streams; section 3.3.1
 * for the fused decode state update).  The caller splits its batch:
 *
 *   prefill part : sequences with more than one new token (or with a prefix
 *                  to continue), as for lightning_attn_fwd_varlen_layout:
 *                  prefill_q/k/v/out, cu_seqlens, num_seqs, total_N, layout,
 *                  init_states (e.g. prefix-cache snapshots), final_states,
 *                  segment_tokens and the workspace.  Launched on
 *                  prefill_stream.
 *   decode part  : decode_B sequences with one new token each, as for
 *                  lightning_attn_decode: decode_q/k/v/out [decode_B][H][d],
 *                  decode_state [decode_B][H][d][d] updated in place.
 *                  Launched on decode_stream.
 *   decay, H, d, block, dt are shared by both parts.
 *
 * The two parts must not share any output buffer; either may be empty
 * (num_seqs == 0 and total_N == 0, or decode_B == 0).  The streams may be
 * the same (the parts then run one after the other) or different (they run
 * concurrently); the call returns once both parts are launched, and the
 * caller synchronises each stream it passed.  Both parts are validated
 * before anything is launched: any invalid argument launches nothing.
 * Returns the first failing part's status, as the two entry points above
 * define them.
 */
la_status lightning_attn_mixed_step(
    const void *prefill_q, const void *prefill_k, const void *prefill_v,
    const int32_t *cu_seqlens, int num_seqs, int64_t total_N, la_layout layout,
    const float *init_states, void *prefill_out, float *final_states, int64_t segment_tokens,
    void *workspace, size_t workspace_bytes, void *prefill_stream, const void *decode_q,
    const void *decode_k, const void *decode_v, float *decode_state, void *decode_out,
    int decode_B, void *decode_stream, const float *decay, int H, int d, int block,
    la_dtype dt);

#ifdef __cplusplus
}
#endif

#endif /* LIGHTNING_ATTN_H */
