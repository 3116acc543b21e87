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

// Fused chunk kernel: per (stream, head, dv slice), every chunk of the stream in order.
struct ChunkArgs {
    const void *q, *k, *v;  // row r of head h: q + r*ld + h*dk (k likewise, v + h*dv)
    int64_t ld;
    const float *g;         // [N][H] or [N][H][dk]
    const float *beta;      // [N][H]
    float *h;               // single state [H][dk][dv] (when h_ptrs == nullptr)
    float *const *h_ptrs;   // per-stream states
    float *o;               // [N][H][dv]
    Streams st;
    int32_t H;
    int32_t do_l2;          // normalise q and k rows on load
    float eps;
    float scale;            // multiplies q on load
};

// Front end: conv + SiLU (+ L2 and scale of q, k) over every channel of the packed rows.
struct FrontArgs {
    const void *q, *k, *v;  // raw rows, as in ChunkArgs
    int64_t ld;
    const float *conv_w;    // [cd][K]
    void *conv_state;       // [cd][K-1] (single stream) when conv_state_ptrs == nullptr
    void *const *conv_state_ptrs;
    void *y;                // out: [N][cd] packed activations (fp16 for bf16 rows), stride cd
    Streams st;
    int64_t N;
    int32_t H, dk, dv, K;
    int32_t do_l2;
    float eps, scale;
};

// Launchers (defined in gdn_kernels.hip). Return hipSuccess or the launch error.
hipError_t launch_front(int dtype, const FrontArgs &a, hipStream_t s);
// new carried conv windows; must run after every kernel that reads the old ones
hipError_t launch_conv_state(int dtype, const FrontArgs &a, hipStream_t s);
// in_kind: 0 = f32 rows, 1 = bf16 rows, 2 = fp16 activations written by the front end;
// nv: dv columns per workgroup (the grid is B * H * dv / nv workgroups); waves: waves per
// workgroup, 0 = the first compiled instance of that width
hipError_t launch_chunk(int in_kind, int dk, int dv, int kda, int nv, int waves,
                        const ChunkArgs &a, int grid, hipStream_t s);
hipError_t launch_chunk_table(const int32_t *cu, int32_t B, int32_t chunk, int32_t *table,
                              int64_t max_entries, int32_t *count, hipStream_t s);
// 1 if the (in_kind, dk, dv, kda, nv, waves) instance exists.
int chunk_instance_exists(int in_kind, int dk, int dv, int kda, int nv, int waves);

}  // namespace gdn
