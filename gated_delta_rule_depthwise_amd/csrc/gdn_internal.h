// gdn_internal.h -- argument blocks shared by the C-ABI layer and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Where a call's streams lie in the packed rows: stream b owns rows [start_b, end_b).
//   cu != nullptr : start_b = cu[b], end_b = cu[b+1]           (varlen)
//   cu == nullptr : start_b = b * tps, end_b = start_b + tps    (single stream or batched)
struct Streams {
    const int32_t *cu;
    int64_t tps;
    int32_t B;
};


// The output gate as a separate pass over rows [0, N) of o, all heads.
struct GateArgs {
    const int32_t *dbg;     // debug validation status (device), or nullptr
    float *o;               // [N][H][dv], in/out
    const void *z;
    int64_t ld_z;
    const float *w;         // [dv]
    int64_t N;
    int32_t H, dv;
    float eps;
};

// Slots of the segmented scan, each one [H][dk][dv] fp32 (dk == dv): H(b, s), s = 1..S-1;
// B(b, s) and A(b, s), s = 1..S-2; then one flag per (b, s, head), 1.0 when the transition
// job of (b, s, head) found A(b, s) to be zero (it then wrote zeros), else 0.0; then the
// warm-start plan: per (b, s, head) the chunks of warm-up before segment s (0: none found;
// a (stream, head) runs warm when every s = 1..S-1 found one); then 16 int flags per (b,
// head) that order workgroups of one launch (see the kFlag offsets below).
struct SegLayout {
    int64_t slot;  // floats per slot
    int32_t B, S, H;
    __host__ __device__ int64_t h(int b, int s) const
    {
        return ((int64_t)b * (S - 1) + s - 1) * slot;
    }
    __host__ __device__ int64_t bs(int b, int s) const
    {
        return ((int64_t)B * (S - 1) + (int64_t)b * (S - 2) + s - 1) * slot;
    }
    __host__ __device__ int64_t as(int b, int s) const
    {
        return ((int64_t)B * (2 * S - 3) + (int64_t)b * (S - 2) + s - 1) * slot;
    }
    __host__ __device__ int64_t zero_flag(int b, int s, int head) const
    {
        return (int64_t)B * (3 * S - 5) * slot + ((int64_t)b * S + s) * H + head;
    }
    __host__ __device__ int64_t warm_chunks(int b, int s, int head) const
    {
        return (int64_t)B * (3 * S - 5) * slot + (int64_t)B * S * H +
               ((int64_t)b * S + s) * H + head;
    }
    __host__ __device__ int64_t flags(int b, int head) const
    {
        return (int64_t)B * (3 * S - 5) * slot + (int64_t)B * 2 * S * H +
               ((int64_t)b * H + head) * 16;
    }
    __host__ __device__ int64_t chain_done(int b, int head, int cbk) const
    {
        return flags(b, head) + kFlagChain + cbk;
    }
    __host__ __device__ int64_t total() const
    {
        return (int64_t)B * (3 * S - 5) * slot + (int64_t)B * 2 * S * H + (int64_t)B * H * 16;
    }
    // Flag offsets within a (stream, head)'s 16 (dv slices <= 2):
    //   kFlagChain + c   the chain of state columns 16c..16c+15 is done (c < 8; second launch)
    //   kFlagRead + sl   job 0 has read the initial state and windows of slice sl (first
    //                    launch, calls with a warm-start plan)
    //   kFlagFallback + sl   the last warm job gave up waiting for that and left the final
    //                    state (and windows) in slot H(b, S-1) for the second launch to copy
    static constexpr int kFlagChain = 0, kFlagRead = 8, kFlagFallback = 10;
};

// The plan's warm-up chunk count of boundary s = lane + 1 (1 past the last boundary): whole
// waves read all S - 1 <= 64 counts with one load each, so they arrive after one memory
// latency, not S - 1 dependent ones.
__device__ __forceinline__ float warm_lane_count(const float *seg_ws, const SegLayout &lay,
                                                 int b, int head)
{
    const int s = (int)(threadIdx.x & 63) + 1;
    return s < lay.S ? seg_ws[lay.warm_chunks(b, s, head)] : 1.f;
}

// Warm mode of a (stream, head), from warm_lane_count of every lane: each boundary found its
// window (the plan leaves a positive chunk count, 0 where it found none).
__device__ __forceinline__ bool warm_head(float lane_count)
{
    return __ballot(!(lane_count > 0.f)) == 0;
}

// The staged windows [B][cd][W] (bf16) of a fused front-end call copied to the caller's;
// a zero-length stream wrote none and keeps its window.
struct WindowCopyArgs {
    const int32_t *dbg;     // debug validation status (device), or nullptr
    const void *win_ws;
    void *conv_state;
    void *const *conv_state_ptrs;
    Streams st;
    int32_t cd, W;
};


// Warm-start plan of a segmented call: per (stream, head), each chunk's total log-gate and
// whether its betas lie in [0, 1.9]; per segment boundary the fewest chunks before it whose
// log-gates sum below -16; warm mode when every boundary has such a window inside the
// previous segment. With the per-key-channel gate a token's bound is its largest channel
// log-gate (the norm of a token's transition is at most its largest channel decay).
struct WarmArgs {
    const int32_t *dbg;     // debug validation status (device), or nullptr
    const float *g;         // [N][H]
    const float *beta;      // [N][H]
    Streams st;
    int32_t H;
    int32_t nseg;
    int64_t seg0_len, seg_len;
    float *seg_ws;
    SegLayout lay;
};

// Front end: conv + SiLU (+ L2 and scale of q, k) over every channel of the packed rows.
struct FrontArgs {
    const int32_t *dbg;     // debug validation status (device), or nullptr
    const void *q, *k, *v;  // raw rows, as in ChunkArgs
    int64_t ld;
    const float *conv_w;    // [cd][K]
    void *conv_state;       // [cd][K-1] (single stream) when conv_state_ptrs == nullptr
    void *const *conv_state_ptrs;
    void *y;                // out: [N][cd] packed activations (fp16 for bf16 rows), stride cd
    Streams st;
    int64_t N;
    int32_t H, Hqk, dk, dv, K;  // cd = 2*Hqk*dk + H*dv
    int32_t do_l2;
    float eps, scale;
    int32_t tile_rows;      // tokens per workgroup tile: a multiple of 4, >= 32
    // warm-start plan run by extra workgroups of the same launch (it reads only gates and
    // betas), when warm_groups > 0: one per (stream, head)
    WarmArgs warm;
    int32_t warm_groups;
};

// Fused chunk kernel: per (stream, head, dv slice), every chunk of the stream in order.
struct ChunkArgs {
    const int32_t *dbg;     // debug validation status (device), or nullptr
    const void *q, *k, *v;  // row r, value head h: q + r*ld + (h/qk_group)*dk (k likewise),
    int64_t ld;             // v + r*ld + h*dv
    const float *g;         // [N][H] or [N][H][dk]
    const float *beta;      // [N][H]
    float *h;               // single state [H][dk][dv] (when h_ptrs == nullptr)
    float *const *h_ptrs;   // per-stream states
    float *o;               // [N][H][dv]
    Streams st;
    int32_t H;              // value heads (the grid and the states)
    int32_t qk_group;       // value heads per q/k head (H / Hqk)
    int32_t do_l2;          // normalise q and k rows on load
    int32_t unit_keys;      // keys arrive normalised or are normalised on load (|k| <= 1)
    float eps;
    float scale;            // multiplies q on load
    // Segmented scan of long streams (see SegLayout). pass 0: each workgroup walks a whole
    // stream. pass 1: job 0 runs segment 0 from the stream's state (o written, end state to
    // slot H(b, 1)); jobs 1..S-2 run segment j from h = 0 (end state to slot B(b, j)); jobs
    // S-1..2S-4 run segment j-(S-2) from h = I with v = 0 (end state, the segment's
    // transition, to slot A(b, j-(S-2))). pass 2: chain_groups workgroups first, which
    // chain h(b, s+1) = A(b, s) h(b, s) + B(b, s) into slots H(b, 2..S-1), then job j runs
    // segment j+1 from slot H(b, j+1) (o written; the last segment's end state to the
    // stream's state), for j >= 1 once the chain of its columns is done. Segment 0 holds
    // seg0_len tokens, segments 1..S-2 seg_len each, segment S-1 the rest of the stream.
    int32_t pass;
    int32_t nseg;           // S
    int32_t chain_groups;   // pass 2: B * H * dv / 16
    // calls with a warm-start plan (which clears the read flags first): the last warm job
    // writes the final state and windows to the caller's buffers itself, once job 0 of the
    // same launch has read the initial ones (a bounded wait of at most wait_polls polls)
    int32_t direct_final;
    int32_t wait_polls;
    // warm starts (scalar gate, unit keys): pass 1 also holds S-1 warm jobs (segments
    // 1..S-1 from h = 0 a few chunks early), run when the (stream, head) is in warm mode;
    // the map jobs and the jobs of pass 2 then return at once, and the chain's workgroups
    // only copy the final state (and windows) over where the last warm job left them in the
    // workspace (without direct_final, or when its wait gave up)
    int32_t warm;
    // set by the launch: workgroups [0, job_groups) are jobs; the rest update the front
    // end's carried windows (window_items = streams x channels, 0 when there is none)
    int32_t job_groups;
    int64_t window_items;
    int32_t window_dtype;   // 1: bf16 rows, 0: fp32
    FrontArgs window;
    int64_t seg0_len;       // tokens of segment 0, a multiple of the chunk
    int64_t seg_len;        // tokens of each inner segment, a multiple of the chunk
    float *seg_ws;
    // varlen: the stream of workgroup slot i (streams ranked longest first), or nullptr
    const int32_t *order;
    // output gate (fused instances): o <- o / sqrt(mean(o^2) + norm_eps) * norm_w * silu(z)
    const void *z;          // row r of head h: z + r*ld_z + h*dv (bf16, or float for f32)
    int64_t ld_z;
    const float *norm_w;    // [dv]
    float norm_eps;
    // Front end fused into the load stage (q, k, v are the raw bf16 conv inputs, conv_k
    // taps): the conv taps, the carried windows (read by the job holding a stream's first
    // chunk) and where the job that ends a stream puts the new windows: the caller's
    // windows, or win_ws when a later kernel must copy them there -- in warm mode without
    // direct_final or when its wait gave up (the chain's workgroups, after the launch that
    // read the old windows) and when several
    // workgroups read one window (win_shared: q/k heads shared by value heads, or dv
    // slices; window_copy_kernel at the end of the call).
    const float *conv_w;            // [cd][conv_k]
    void *conv_state;               // [cd][conv_k-1] of the single stream (conv_state_ptrs == nullptr)
    void *const *conv_state_ptrs;   // per stream
    void *win_ws;                   // [B][cd][conv_k-1] bf16
    int32_t cd;                     // channels of a packed row
    int32_t conv_k;
    int32_t win_shared;
};

// One decode step: a single token per stream through the front end (optional), L2 and the
// recurrence, h updated in place.
struct DecodeArgs {
    const void *q, *k, *v;           // row b (stream b's token): q + b*ld + h*dk, ...
    int64_t ld;
    const float *g;                  // [B][H] or [B][H][dk]
    const float *beta;               // [B][H]
    float *const *h_ptrs;            // per-stream [H][dk][dv]
    void *const *conv_state_ptrs;    // per-stream [cd][K-1] (K > 0)
    const float *conv_w;             // [cd][K] (K > 0)
    float *o;                        // [B][H][dv]
    int32_t B, H, Hqk, dk, dv, K;    // value head h reads q/k head h / (H / Hqk)
    int32_t do_l2;
    float eps, scale;
    const void *z;                   // output gate (nullptr: off): row b at z + b*ld_z
    int64_t ld_z;
    const float *norm_w;             // [dv]
    float norm_eps;
};

// Debug validation of a call's device-side inputs: cu_seqlens (when cu is set) and the
// per-key-channel log-gates (when g is set, ng values of the real rows); violations OR
// GDN_BAD_* bits into *status, and every kernel of the call then returns at once.
struct ValidateArgs {
    const int32_t *cu;
    int32_t B;
    int64_t total;
    int32_t max_seqlen;
    const float *g;
    int64_t ng;
    int32_t *status;
};

// A kernel of a call checked by the debug validation returns at once when a violation was
// found (the check ran before it on the call's stream).
__device__ __forceinline__ bool debug_stop(const int32_t *dbg)
{
    return dbg && *(volatile const int32_t *)dbg != 0;
}

// Launchers (defined in gdn_kernels.hip and gdn_decode.hip). Return hipSuccess or the
// launch error.
hipError_t launch_validate(const ValidateArgs &a, hipStream_t s);
hipError_t launch_front(int dtype, const FrontArgs &a, hipStream_t s);
// in_kind: 0 = f32 rows, 1 = bf16 rows, 3 = bf16 raw rows with the front end fused;
// nv: dv columns per workgroup (the grid is B * H * dv / nv workgroups); waves: waves per
// workgroup, 0 = the first compiled instance of that width; gate: the instance with the
// output gate fused into its o flush (ChunkArgs z, ld_z, norm_w, norm_eps); chunk: rows
// per chunk (64, or 32 where an instance has it)
hipError_t launch_chunk(int in_kind, int dk, int dv, int kda, int nv, int waves, int gate,
                        int chunk, const ChunkArgs &a, int grid, hipStream_t s);
// the output gate as its own pass (dtype: element type of z, GDN_F32 or GDN_BF16)
hipError_t launch_gate(int dtype, const GateArgs &a, hipStream_t s);
hipError_t launch_window_copy(const WindowCopyArgs &a, hipStream_t s);
// The same plan with one workgroup per (stream, head, boundary), reading only the gates of
// each boundary's window; with the per-key-channel gate (kda) a token's bound is its
// largest channel log-gate (g is then [N][H][dk]).
hipError_t launch_warm_boundaries(const WarmArgs &a, int kda, int dk, hipStream_t s);
hipError_t launch_decode(int dtype, int kda, const DecodeArgs &a, hipStream_t s);
// q/k windows of a decode step with Hqk < H (several workgroups read them): shifted after
// the step by a pass of its own
hipError_t launch_decode_qk_window(int dtype, const DecodeArgs &a, hipStream_t s);
// order[i] = the stream of rank i by length, longest first (ties by index), B <= 1024
hipError_t launch_stream_order(const int32_t *cu, int32_t B, int32_t *order, hipStream_t s);
hipError_t launch_chunk_table(const int32_t *cu, int32_t B, int32_t chunk, int32_t *table,
                              int64_t max_entries, int32_t *count, hipStream_t s);
// 1 if the (in_kind, dk, dv, kda, nv, waves, gate, chunk) instance exists.
int chunk_instance_exists(int in_kind, int dk, int dv, int kda, int nv, int waves, int gate,
                          int chunk);

}  // namespace gdn
