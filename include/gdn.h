/*
 * gdn.h -- C ABI of libgdn: the chunked gated-delta-rule prefill (GDN and KDA) on MI355X,
 * its single-token decode step, and the gated RMSNorm of the output.
 *
 * The operation (pages "split_prefill.rs" -- prefill_gdn_full, prefill_gdn_full_batched,
 * prefill_gdn_full_batched_fla_varlen -- and "metrale_model_arch/glm5next_kda/prefill.rs"
 * -- Glm5NextKdaLayer::prefill, prefill_with_pad_fill and its launch sequence conv_prefill,
 * l2, split_widen, chunk_prepare, chunk_scan):
 *
 *   1. optional front end: causal depthwise conv1d over every channel of the packed
 *      [q | k | v] rows (conv_k taps, no bias) followed by SiLU, starting from and
 *      advancing a carried window of the last conv_k-1 raw inputs per channel;
 *   2. optional L2 normalisation of q and k per token and head, q <- q / sqrt(|q|^2+eps),
 *      k <- k / sqrt(|k|^2+eps), then q <- scale * q;
 *   3. the gated delta rule, with S = h^T (dv x dk) per head and alpha_t = exp(g_t):
 *        S_t = S_{t-1} diag(alpha_t) - beta_t (S_{t-1} diag(alpha_t) k_t - v_t) k_t^T,
 *        o_t = S_t q_t,
 *      evaluated chunk by chunk (cumulative log-gates, the beta-weighted WY/UT transform,
 *      then the inter-chunk scan that carries h). alpha_t is one scalar per head (GDN) or
 *      one value per key channel (KDA);
 *   4. optional output gate (gdn_params.z): o <- o / sqrt(mean(o^2) + eps) * w * silu(z)
 *      per token and head (page "split_prefill.rs", prefill_phase3).
 *   gdn_decode / kda_decode run steps 1-4 for one new token per stream.
 *
 * Conventions shared by every entry point
 *   - Every pointer argument except `p` is a DEVICE pointer; `p` is a host pointer.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream) and never
 *     synchronise. The library never allocates caller-visible memory and keeps no state
 *     between calls except lazily created per-device kernel handles.
 *   - The caller owns every buffer. h and conv_state are read and then overwritten in
 *     place. o is written only at real token rows: rows at or past a stream's end keep
 *     their previous bytes.
 *   - Positions at or past a stream's end (padding, or the tail of an allocation) are
 *     never read; NaN or huge values there have no effect.
 *   - Element types: q/k/v, the raw rows and conv_state are `p->dtype` (GDN_F32 or
 *     GDN_BF16); o, g, beta, h and conv_w are float32. (o is float32 for bf16 inputs too:
 *     rounding o itself to bf16 already costs about 2e-2 of max|error|/RMS on these
 *     heavy-tailed outputs.) The dense products run on MFMA with fp32 accumulation, with
 *     fp16 operands for bf16 inputs (hi + lo pairs where a single fp16 rounding would
 *     show in o or h) and fp32 operands for float32 inputs.
 *   - Front end: with bf16 rows, 2 to 4 taps and ld_qkv < 2^24, on the shapes with a fused
 *     instance (dk = dv = 128 or 64, and dk = 128 with dv = 256; either gate, shared q/k
 *     heads included), the conv + SiLU + L2 run inside the scan's load stage in fp32
 *     straight from the raw rows (no activation buffer; k, and with the scalar gate q,
 *     enter the products as fp16 hi + lo pairs, v in fp32); at dk = dv the scalar gate's
 *     output gate then rides in the same kernel's o flush. A bf16 front-end call outside
 *     those is refused with GDN_E_UNSUPPORTED; with float32 rows the front end runs as a
 *     kernel of its own that hands the scan fp32 activations through the workspace.
 *   - Errors: every check below runs on the host before anything is enqueued; on error
 *     nothing is launched and no buffer changes (the pages refuse a bad token count before
 *     any launch). GDN_E_HIP reports a failed launch.
 *   - Not thread-safe per device for concurrent calls sharing one workspace.
 *   - Graph capture: a call enqueues kernel launches only (no memset, copy, allocation or
 *     host wait), so after one eager call of the same shape on the device (which does the
 *     one-time kernel setup) it can be captured in a HIP graph and replayed; each replay
 *     reads and advances the states as the captured call did. Profiling must be off while
 *     capturing.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define GDN_OK 0
#define GDN_E_ARG (-1)         /* bad count, null pointer, bad stride, bad B            */
#define GDN_E_UNSUPPORTED (-2) /* (dk, dv, chunk, dtype, conv_k) not compiled in        */
#define GDN_E_WORKSPACE (-3)   /* ws_bytes smaller than gdn_workspace_bytes() requires  */
#define GDN_E_HIP (-4)         /* a HIP launch or query failed                          */

/* element types of q/k/v, raw rows and conv_state */
#define GDN_F32 0
#define GDN_BF16 1

/* call kinds for gdn_workspace_bytes */
#define GDN_KIND_SINGLE 0
#define GDN_KIND_BATCHED 1
#define GDN_KIND_VARLEN 2
/* OR-ed into the kind of gdn_segments / gdn_segment_plan / gdn_workspace_bytes: the plan
 * and workspace of a KDA call (per-key-channel gate) instead of a GDN call (scalar gate);
 * the two differ */
#define GDN_PLAN_KDA 0x100

typedef struct gdn_params {
    int32_t H;      /* value heads: g, beta, o and the states have H heads (see Hqk)      */
    int32_t dk;     /* key head dim                                                       */
    int32_t dv;     /* value head dim. Compiled (dk, dv): bf16 (64, 64), (128, 128),
                       (128, 256); f32 (64, 64), (64, 128). dv != dk runs unsegmented and
                       gates o (if asked) in a separate pass                              */
    int32_t chunk;  /* tokens per chunk: 64                                               */
    float eps;      /* L2 eps for q and k; eps < 0: q and k are used as given (no L2)     */
    float scale;    /* multiplies q after the optional L2 (normally 1/sqrt(dk))           */
    int32_t dtype;  /* GDN_F32 or GDN_BF16                                                */
    int32_t conv_k; /* 0: no front end; 2..4: causal depthwise conv taps + SiLU           */
    int64_t ld_qkv; /* row stride, in elements, of the q, k and v rows                    */
    /* Optional output gate, the gated RMSNorm that opens the next phase (page
     * "split_prefill.rs", prefill_phase3: gated RMSNorm of the GDN output with Z). With z
     * non-NULL, every o row of every head leaves as
     *     y = o / sqrt(mean(o^2) + norm_eps) * norm_w * silu(z),   silu(z) = z / (1+e^-z),
     * the mean over that head's dv values, instead of o itself. Zero-initialise the struct
     * (or set z = NULL) to leave o ungated.                                               */
    const void *z;        /* DEVICE, rows like o: row r, head h at z + r*ld_z + h*dv, in
                             dtype; 16-byte aligned. NULL = no gate.                       */
    const float *norm_w;  /* DEVICE [dv] float weights shared by the heads, 16-byte aligned */
    int64_t ld_z;         /* row stride of z in elements (>= H*dv, 16-byte multiple)       */
    float norm_eps;       /* >= 0, finite                                                   */
    /* q/k heads (0 = H). With 0 < Hqk < H, H must be a multiple of Hqk and each q/k head
     * serves H/Hqk consecutive value heads: value head h reads q/k head h / (H/Hqk). The
     * packed rows are then [q (Hqk*dk) | k (Hqk*dk) | v (H*dv)], cd = 2*Hqk*dk + H*dv,
     * and the conv channels of q/k head j are j*dk + c and Hqk*dk + j*dk + c.            */
    int32_t Hqk;
} gdn_params;

/*
 * Single stream of t tokens (pages: "split_prefill.rs" prefill_gdn_full;
 * "metrale_model_arch/glm5next_kda/prefill.rs" Glm5NextKdaLayer::prefill, which refuses
 * t == 0 or t above the workspace's token capacity before any launch).
 *
 *   q, k, v   row i of q is q + i*ld_qkv, head h at offset h*dk (k likewise, v at h*dv).
 *             With the front end on, these are the raw conv inputs of the packed row
 *             [q | k | v]: the conv channel of q element (h, c) is h*dk + c, of k element
 *             H*dk + h*dk + c, of v element 2*H*dk + h*dv + c (cd = 2*H*dk + H*dv), with
 *             Hqk in place of H for q and k when p->Hqk is set.
 *   g         [t][H] float log-gates (kda_prefill: [t][H][dk], one per key channel).
 *   beta      [t][H] float, used as given.
 *   h         [H][dk][dv] float state, in/out.
 *   conv_state [cd][conv_k-1] in dtype, oldest first, in/out (NULL iff conv_k == 0).
 *   conv_w    [cd][conv_k] float taps; tap conv_k-1 multiplies the current token (NULL
 *             iff conv_k == 0).
 *   o         [t][H][dv] float32, out (16-byte aligned).
 *   t         1 <= t <= the max_tokens the workspace was sized for.
 *   ws        device workspace of ws_bytes >= gdn_workspace_bytes(p, 1, t, GDN_KIND_SINGLE)
 *             (may be NULL when that size is 0).
 */
int gdn_prefill(const gdn_params *p, const void *q, const void *k, const void *v,
                const float *g, const float *beta, float *h, void *conv_state,
                const float *conv_w, void *o, int64_t t, void *ws, size_t ws_bytes,
                void *stream);

/* Same as gdn_prefill with the per-key-channel gate: g is [t][H][dk], 16-byte aligned, and
 * must be a decay (g <= 0; see kda_prefill_batched) (page
 * "metrale_model_arch/glm5next_kda/prefill.rs", the KDA chunked prefill). */
int kda_prefill(const gdn_params *p, const void *q, const void *k, const void *v,
                const float *g, const float *beta, float *h, void *conv_state,
                const float *conv_w, void *o, int64_t t, void *ws, size_t ws_bytes,
                void *stream);

/*
 * gdn_prefill without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. The call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine): its workspace is a device array of gdn_noalloc_scratch_bytes() (64 MiB) that
 * the library holds on every GPU it runs on until the process ends. Its device address is
 * looked up on the first call on each device, which must be the current device and the
 * device of `stream`.
 *   - Arguments, layouts and results are those of gdn_prefill.
 *   - GDN_E_WORKSPACE when the workspace the call cannot run without (float32 rows with
 *     the front end: t * cd floats of activations) exceeds the array; segment states
 *     that do not fit make the scan run unsegmented, with the same results up to rounding.
 *   - GDN_E_HIP if the array's address cannot be looked up.
 *   - Every call on a GPU uses that GPU's one array: calls that overlap on one GPU (two
 *     streams, or host threads) race and give undefined results. Nothing in the array has
 *     to start at zero; every call writes what it later reads.
 */
int gdn_prefill_noalloc(const gdn_params *p, const void *q, const void *k, const void *v,
                        const float *g, const float *beta, float *h, void *conv_state,
                        const float *conv_w, void *o, int64_t t, void *stream);
/* Size in bytes of the device array behind gdn_prefill_noalloc. */
size_t gdn_noalloc_scratch_bytes(void);

/*
 * B streams of equal length t_per_stream lying back to back: stream b owns rows
 * [b*t_per_stream, (b+1)*t_per_stream) of q/k/v/g/beta/o (page "split_prefill.rs",
 * prefill_gdn_full_batched: one h-state pointer per stream, streams of equal length).
 *   h_ptrs          device array of B device pointers, each to a [H][dk][dv] float state.
 *   conv_state_ptrs device array of B device pointers to [cd][conv_k-1] windows (NULL iff
 *                   conv_k == 0).
 *   ws              >= gdn_workspace_bytes(p, B, B*t_per_stream, GDN_KIND_BATCHED).
 * B >= 1 and t_per_stream >= 1, else GDN_E_ARG.
 */
int gdn_prefill_batched(const gdn_params *p, const void *q, const void *k, const void *v,
                        const float *g, const float *beta, float *const *h_ptrs,
                        void *const *conv_state_ptrs, const float *conv_w, void *o,
                        int32_t B, int64_t t_per_stream, void *ws, size_t ws_bytes,
                        void *stream);

/*
 * B streams of different lengths described by cu_seqlens (page "split_prefill.rs",
 * prefill_gdn_full_batched_fla_varlen): stream b owns rows [cu_seqlens[b],
 * cu_seqlens[b+1]). Chunks restart at every stream start.
 *   cu_seqlens   device int32 [B+1], cu_seqlens[0] == 0, non-decreasing,
 *                cu_seqlens[B] == total_tokens. A zero-length stream is a no-op (its state
 *                is left as it was). The host does not read device memory, so violations
 *                give undefined results unless gdn_debug_validate is on (it then detects
 *                them on the device and the call touches nothing).
 *   total_tokens host copy of cu_seqlens[B] (>= 1).
 *   max_seqlen   host upper bound of the longest stream (1 <= max_seqlen <= total_tokens).
 *   ws           >= gdn_workspace_bytes(p, B, total_tokens, GDN_KIND_VARLEN).
 */
int gdn_prefill_varlen(const gdn_params *p, const void *q, const void *k, const void *v,
                       const float *g, const float *beta, float *const *h_ptrs,
                       void *const *conv_state_ptrs, const float *conv_w, void *o,
                       const int32_t *cu_seqlens, int32_t B, int64_t total_tokens,
                       int32_t max_seqlen, void *ws, size_t ws_bytes, void *stream);

/*
 * The per-key-channel gate for equal-length and varlen streams: as gdn_prefill_batched and
 * gdn_prefill_varlen with g [rows][H][dk] (one log-gate per key channel, 16-byte aligned).
 * The gate must be a decay, g <= 0: chunk products are factored at 16-token block
 * boundaries with factors e^(G_r - G_ref) <= 1 held in fp16, and the diagonal 16x16 blocks
 * in fp32 with a mid-block reference whose exponents are clamped at 80 (a decay stronger
 * than e^-80 over 8 tokens of one channel is flushed).
 */
int kda_prefill_batched(const gdn_params *p, const void *q, const void *k, const void *v,
                        const float *g, const float *beta, float *const *h_ptrs,
                        void *const *conv_state_ptrs, const float *conv_w, void *o,
                        int32_t B, int64_t t_per_stream, void *ws, size_t ws_bytes,
                        void *stream);
int kda_prefill_varlen(const gdn_params *p, const void *q, const void *k, const void *v,
                       const float *g, const float *beta, float *const *h_ptrs,
                       void *const *conv_state_ptrs, const float *conv_w, void *o,
                       const int32_t *cu_seqlens, int32_t B, int64_t total_tokens,
                       int32_t max_seqlen, void *ws, size_t ws_bytes, void *stream);

/*
 * One decode step: a single new token for each of B streams (page
 * "metrale_model_arch/glm5next_kda/prefill.rs" names decode_k, the single-token step, beside
 * the prefill's profile buckets). The token goes through the same steps as a prefill row:
 * the optional front end (advancing each stream's window by one raw input), the optional
 * L2 and q scale, then one step of the recurrence on the stream's state, and o_t = S_t q_t.
 * The result equals a varlen prefill with cu_seqlens = {0, 1, ..., B}.
 *   q, k, v   row b (stream b's token) at q + b*ld_qkv; head and channel layout as for
 *             gdn_prefill.
 *   g         [B][H] float log-gates (kda_decode: [B][H][dk]); beta [B][H] float.
 *   h_ptrs    device array of B device pointers, each to a [H][dk][dv] float state,
 *             16-byte aligned, in/out. The B states must not overlap.
 *   conv_state_ptrs, conv_w  as for gdn_prefill_batched (NULL iff conv_k == 0).
 *   o         [B][H][dv] float32, out (16-byte aligned).
 * (dk, dv) = (64, 64), (128, 128), (64, 128) or (128, 256), either dtype (else
 * GDN_E_UNSUPPORTED); B >= 1. No workspace. The step is one kernel (plus a small pass that
 * advances the q/k windows when Hqk < H); with profiling enabled it is recorded in
 * GDN_PROF_RECUR.
 */
int gdn_decode(const gdn_params *p, const void *q, const void *k, const void *v,
               const float *g, const float *beta, float *const *h_ptrs,
               void *const *conv_state_ptrs, const float *conv_w, void *o, int32_t B,
               void *stream);
int kda_decode(const gdn_params *p, const void *q, const void *k, const void *v,
               const float *g, const float *beta, float *const *h_ptrs,
               void *const *conv_state_ptrs, const float *conv_w, void *o, int32_t B,
               void *stream);

/*
 * Per-chunk work table of a varlen call (the bookkeeping of
 * prefill_gdn_full_batched_fla_varlen: total_nt = sum_b ceil(len_b/chunk) chunks,
 * max_num_chunks = max_b ceil(len_b/chunk)). Writes, on `stream`, table[4*i .. 4*i+3] =
 * {stream b, first row of the chunk, rows in the chunk, chunk index within b} for chunk
 * i in stream-major order, and *count = total_nt. table holds max_entries rows; chunks
 * beyond it are counted but not written. cu_seqlens as for gdn_prefill_varlen.
 */
int gdn_chunk_table(const int32_t *cu_seqlens, int32_t B, int32_t chunk, int32_t *table,
                    int64_t max_entries, int32_t *count, void *stream);

/*
 * Stage timing, the counterpart of the pages' profile buckets around the KDA prefill's
 * front end and recurrence (page "metrale_model_arch/glm5next_kda/prefill.rs",
 * profile::start / profile::end with KDA_FRONT, KDA_RECUR, KDA_BACK). While enabled, every
 * call records a hipEvent pair around each of its kernels on the call's stream:
 *   GDN_PROF_FRONT  the front kernel (conv + SiLU + L2) of float32 front-end calls; for
 *                   segmented calls with the scalar gate it also holds the warm-start plan.
 *                   bf16 front-end calls run the front end inside the chunk kernel.
 *   GDN_PROF_RECUR  the fused chunk kernel (front end for bf16 rows, WY/UT preparation,
 *                   inter-chunk scan), the warm-start plan when it has no front kernel to
 *                   ride in, the chain of segment maps and the window copies
 *   GDN_PROF_STATE  unused by prefill calls (the windows go out with the scan); kept so
 *                   that bucket numbers stay fixed
 *   GDN_PROF_GATE   the output gate when it runs as its own pass (the per-key-channel gate
 *                   at dk = dv = 128 or with float32 inputs; elsewhere it is fused into the
 *                   o flush of the chunk kernel or the decode kernel and nothing is
 *                   recorded here)
 * gdn_profile_read waits for every recorded pair, writes the summed milliseconds and the
 * launch count of buckets 0..nbuckets-1, and forgets the records. Host pointers; events
 * are created once and reused. Enabling costs two event records per kernel.
 */
#define GDN_PROF_FRONT 0
#define GDN_PROF_RECUR 1
#define GDN_PROF_STATE 2
#define GDN_PROF_GATE 3
#define GDN_PROF_BUCKETS 4
int gdn_profile_enable(int on);
int gdn_profile_read(double *ms_total, int64_t *launches, int32_t nbuckets);

/* Bytes of device workspace a call of `kind` with B streams and up to max_tokens rows in
 * total needs (0 if none). Returns 0 for invalid parameters. The size is that of a GDN
 * call (scalar gate); or GDN_PLAN_KDA into kind for a KDA call, whose front end (when
 * conv_k > 0) always needs room for its activations.
 *
 * For varlen calls (B <= 1024) it also holds B int32: the streams ranked by length, so that
 * when a call has more (stream, head) workgroups than the device has CUs the longest
 * streams are dispatched first (written by a small kernel on the call's stream; a
 * workspace without room for it keeps the index order).
 *
 * The workspace holds the front end's activations and, for single and batched calls with
 * fewer (stream, head) work units than the device has compute units, the states of the
 * segmented scan: each stream is cut into S segments of whole chunks; one launch runs
 * segment 0 and gives, for every inner segment, its end state from a zero state and its
 * dk x dk transition (the end state from the identity with v = 0); a chain over the
 * segments turns these into each segment's start state; a second launch runs segments
 * 1..S-1 from their start states. (The pages' chunked scan carries h serially across a
 * stream's chunks; the recurrence is affine in h, so the segment maps compose exactly up
 * to rounding.) A call whose ws_bytes covers the front end but not the segment states runs
 * unsegmented.
 *
 * Two shortcuts of the segmented scan depend on the gates, decided on the device: with keys
 * of unit length or less (eps >= 0), every token multiplies a segment's transition by a
 * factor of norm at most exp(g_t) (KDA: exp of the token's largest channel log-gate) while
 * beta_t lies in [0, 1.9]. Once a running sum of these log-gates is below -110 the
 * transition is zero in fp32: with the scalar gate a transition job then stops and writes
 * zeros, and the chain copies that step's end state. And when every segment boundary of a
 * (stream, head) has a window of chunks inside the previous segment whose sum is below -16,
 * each segment starts from a zero state that many chunks early ("warm start"), all in the
 * first launch, with no chain. The state a warm start drops is at most e^-16 (< 2^-23) of
 * the state's norm at the start of that window: the fp32 rounding of that state, and below
 * the precision of the hi + lo operand pairs that carry the state through every chunk,
 * unless the state shrank by orders of magnitude across the window. Segments of calls that
 * can start warm are of equal length. Slowly decaying heads take the chain; one call may
 * hold both. */
size_t gdn_workspace_bytes(const gdn_params *p, int32_t B, int64_t max_tokens, int32_t kind);

/* Segments per stream (S >= 3, or 0 for an unsegmented scan) that a single (kind
 * GDN_KIND_SINGLE, B = 1) or batched (GDN_KIND_BATCHED) GDN call (KDA call with
 * GDN_PLAN_KDA or-ed into kind) with these parameters, t_per_stream tokens per stream and
 * ws_bytes of workspace would use on the current device; always 0 for GDN_KIND_VARLEN.
 * Negative status for invalid arguments, or GDN_E_UNSUPPORTED when that call is not
 * compiled for these parameters. Host only; enqueues nothing. */
int gdn_segments(const gdn_params *p, int32_t kind, int32_t B, int64_t t_per_stream,
                 size_t ws_bytes);

/* The same plan with its segment lengths: returns what gdn_segments returns and, for a
 * segmented plan, writes the tokens of segment 0 to *seg0_tokens and of each of segments
 * 1..S-2 to *seg_tokens (multiples of the chunk; segment S-1 takes the rest of each
 * stream); both are set to 0 otherwise. Either pointer may be NULL. Segment 0 may be longer
 * than the inner segments: the plan is the cheapest one under a list-schedule estimate of
 * the two launches on the device's compute units, and segment 0 runs beside the inner
 * segments' map jobs, which cost less per chunk than a chunk that writes o. */
int gdn_segment_plan(const gdn_params *p, int32_t kind, int32_t B, int64_t t_per_stream,
                     size_t ws_bytes, int64_t *seg0_tokens, int64_t *seg_tokens);

/*
 * Debug validation of what the host cannot see without a synchronisation: the device-side
 * cu_seqlens of varlen calls and the log-gates of per-key-channel calls (which must be a
 * decay). Off by default. With `status` a DEVICE pointer to an int32, every later prefill
 * call (any entry point, any stream) first launches a check on its stream; each violation
 * ORs one of the bits below into *status, and then every other kernel of that call returns
 * without reading or writing anything, so a malformed cu_seqlens cannot make the call
 * access memory outside its buffers (h, o and the windows keep their bytes). The caller
 * clears *status, makes its calls, and reads *status after synchronising the stream. NULL
 * turns the checks off. The setting is process-wide; it costs one small launch per call
 * (plus one read of the log-gates for per-key-channel calls). Returns GDN_OK.
 */
#define GDN_BAD_CU_START 1   /* cu_seqlens[0] != 0                                   */
#define GDN_BAD_CU_ORDER 2   /* cu_seqlens decreases somewhere                         */
#define GDN_BAD_CU_TOTAL 4   /* cu_seqlens[B] != total_tokens                          */
#define GDN_BAD_CU_MAXLEN 8  /* a stream longer than max_seqlen                        */
#define GDN_BAD_KDA_GATE 16  /* a per-key-channel log-gate above 0 or NaN, in a real row */
int gdn_debug_validate(int32_t *status);

/*
 * Debug bound of the segmented scan's flag waits. Inside one launch some workgroups wait
 * for flags that earlier workgroups of the grid set (the last warm-started segment waits
 * until the job that reads the stream's initial state and windows has read them; jobs of
 * the second launch wait for the chain of segment maps). Each wait polls a bounded number of
 * times, by default about a second's worth plus room for the longest job, and the last
 * warm-started segment falls back to a copy by the second launch when its wait gives up.
 * polls >= 0 replaces the bound for every later call (0: the last warm-started segment
 * takes the fallback at once; a chained segment would proceed without its start state, so
 * this is for tests of warm-started calls); -1 restores the default. The setting is
 * process-wide. Returns GDN_OK, or GDN_E_ARG for polls < -1.
 */
int gdn_debug_flag_polls(int32_t polls);

/* Static description of a status code. */
const char *gdn_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* GDN_H */
