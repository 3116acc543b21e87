// gdn_decode.hip -- one decode step of the gated delta rule on gfx950: a single token per
// stream (the pages' decode_k, named beside the prefill's profile buckets in
// "metrale_model_arch/glm5next_kda/prefill.rs").
//
// The token goes through the same front end as a prefill row (causal depthwise conv over
// the carried window + SiLU, the window advanced by one raw input), the L2 of q and k and
// the q scale, then one step of the recurrence on the state h = S^T [dk][dv]:
//   h' = diag(alpha) h,   d = beta (v - h'^T k),   h <- h' + k d^T,   o = h^T q.
// The step reads and writes the whole state once, so it is bound by HBM on h. One
// workgroup per (stream, head) holds its head's state in registers: each lane owns 4
// adjacent columns of every P-th row, so one wave instruction moves whole rows of h as
// 16-byte lanes. All arithmetic is fp32. With the output gate on, o leaves as
// o / sqrt(mean(o^2) + eps) * w * silu(z) over the head's dv values.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_internal.h"

namespace gdn {

namespace {

typedef __bf16 bf16;

constexpr int DEC_THREADS = 256;

__device__ __forceinline__ float to_float(float x) { return x; }
__device__ __forceinline__ float to_float(bf16 x) { return (float)x; }

// The state is read once and written once per step: nontemporal accesses keep it from
// displacing cached data (measured on the 64-stream batch: 63 us -> 51 us per launch).
typedef float nt4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 load_nt(const float *p)
{
    const nt4 v = __builtin_nontemporal_load((const nt4 *)p);
    return float4{v.x, v.y, v.z, v.w};
}

__device__ __forceinline__ void store_nt(float *p, float4 v)
{
    const nt4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, (nt4 *)p);
}

// 4 adjacent values of the output gate's z as floats
__device__ __forceinline__ float4 load4(const float *p) { return *(const float4 *)p; }
__device__ __forceinline__ float4 load4(const bf16 *p)
{
    const uint2 u = *(const uint2 *)p;
    return float4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                  __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
}

__device__ __forceinline__ float silu(float x)
{
    return x * __builtin_amdgcn_rcpf(1.f + __expf(-x));
}

// Sum over the 64 lanes of a wave, every lane gets the result.
__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int m = 1; m < 64; m <<= 1)
        x += __shfl_xor(x, m);
    return x;
}

template <typename T, int DK, int DV, bool KDA, int K>
__global__ void __launch_bounds__(DEC_THREADS) decode_kernel(const DecodeArgs a)
{
    constexpr int W = K > 0 ? K - 1 : 0;
    constexpr int CPR = DV / 4;              // lanes per row of h, 4 columns each
    constexpr int P = DEC_THREADS / CPR;     // row groups
    constexpr int RP = DK / P;               // rows per thread: p, p + P, p + 2P, ...
    static_assert(DEC_THREADS % CPR == 0 && DK % P == 0, "thread map");
    __shared__ __align__(16) float sq[DK], sk[DK], sv[DV], sa[DK];
    __shared__ float4 red[P][CPR];

    const int H = a.H, Hqk = a.Hqk;
    const int b = blockIdx.x / H, head = blockIdx.x - b * H;
    const int head_qk = head / (H / Hqk);  // the q/k head this value head reads
    // q/k windows are advanced here only when no other workgroup reads them (Hqk == H);
    // otherwise by decode_qk_window_kernel after the step
    const bool own_qk = Hqk == H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int jc = tid % CPR, p = tid / CPR;
    float *hp = a.h_ptrs[b] + (int64_t)head * DK * DV + 4 * jc;

    // the state loads go first: they are the bulk of the step and do not depend on the
    // front end
    float4 hr[RP];
#pragma unroll
    for (int r = 0; r < RP; ++r)
        hr[r] = load_nt(hp + (int64_t)(p + r * P) * DV);

    // output gate operands of this lane's 4 columns (the lanes that finish o)
    float4 zv = {0.f, 0.f, 0.f, 0.f}, wv = {0.f, 0.f, 0.f, 0.f};
    if (a.z && p == 0) {
        zv = load4((const T *)a.z + (int64_t)b * a.ld_z + (int64_t)head * DV + 4 * jc);
        wv = *(const float4 *)(a.norm_w + 4 * jc);
    }

    // front end (or the given activations) for this head's q, k and v channels
    for (int c = tid; c < 2 * DK + DV; c += DEC_THREADS) {
        const int sec = c < DK ? 0 : c < 2 * DK ? 1 : 2;
        const int e = sec == 0 ? c : sec == 1 ? c - DK : c - 2 * DK;
        const T *src = (const T *)(sec == 0 ? a.q : sec == 1 ? a.k : a.v);
        const int64_t col = sec == 2 ? (int64_t)head * DV + e : (int64_t)head_qk * DK + e;
        const T raw = src[(int64_t)b * a.ld + col];
        float x = to_float(raw);
        if constexpr (K > 0) {
            const int64_t ch =
                (sec == 0 ? 0 : sec == 1 ? (int64_t)Hqk * DK : 2 * (int64_t)Hqk * DK) + col;
            T *win = (T *)a.conv_state_ptrs[b] + ch * W;
            const float *w = a.conv_w + ch * K;
            float acc = w[K - 1] * x;
            T old[W > 0 ? W : 1];
#pragma unroll
            for (int i = 0; i < W; ++i) {
                old[i] = win[i];
                acc += w[i] * to_float(old[i]);
            }
            // the window keeps the last K-1 raw inputs, oldest first
            if (sec == 2 || own_qk) {
#pragma unroll
                for (int i = 0; i + 1 < W; ++i)
                    win[i] = old[i + 1];
                win[W - 1] = raw;
            }
            x = silu(acc);
        }
        (sec == 0 ? sq : sec == 1 ? sk : sv)[e] = x;
    }
    __syncthreads();

    // L2 of q (wave 0) and k (wave 1), q scale
    if (wave < 2) {
        float *x = wave == 0 ? sq : sk;
        float ss = 0.f;
        for (int i = lane; i < DK; i += 64)
            ss += x[i] * x[i];
        ss = wave_sum(ss);
        float mul = a.do_l2 ? rsqrtf(ss + a.eps) : 1.f;
        if (wave == 0)
            mul *= a.scale;
        for (int i = lane; i < DK; i += 64)
            x[i] *= mul;
    }
    if constexpr (KDA) {
        for (int i = tid; i < DK; i += DEC_THREADS)
            sa[i] = __expf(a.g[((int64_t)b * H + head) * DK + i]);
    }
    __syncthreads();

    const float alpha = KDA ? 1.f : __expf(a.g[(int64_t)b * H + head]);
    const float beta = a.beta[(int64_t)b * H + head];

    // h' = diag(alpha) h and this thread's part of (h'^T k) for its 4 columns
    float4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < RP; ++r) {
        const int row = p + r * P;
        const float al = KDA ? sa[row] : alpha, kr = sk[row];
        hr[r].x *= al, hr[r].y *= al, hr[r].z *= al, hr[r].w *= al;
        s.x += kr * hr[r].x, s.y += kr * hr[r].y, s.z += kr * hr[r].z, s.w += kr * hr[r].w;
    }
    red[p][jc] = s;
    __syncthreads();
    s = red[0][jc];
#pragma unroll
    for (int pp = 1; pp < P; ++pp) {
        const float4 t = red[pp][jc];
        s.x += t.x, s.y += t.y, s.z += t.z, s.w += t.w;
    }
    const float4 vv = *(const float4 *)(sv + 4 * jc);
    const float4 d = {beta * (vv.x - s.x), beta * (vv.y - s.y), beta * (vv.z - s.z),
                      beta * (vv.w - s.w)};
    __syncthreads();  // red is reused below

    // h <- h' + k d^T and this thread's part of (h^T q)
    float4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < RP; ++r) {
        const int row = p + r * P;
        const float kr = sk[row], qr = sq[row];
        hr[r].x += kr * d.x, hr[r].y += kr * d.y, hr[r].z += kr * d.z, hr[r].w += kr * d.w;
        o.x += qr * hr[r].x, o.y += qr * hr[r].y, o.z += qr * hr[r].z, o.w += qr * hr[r].w;
        store_nt(hp + (int64_t)row * DV, hr[r]);
    }
    red[p][jc] = o;
    __syncthreads();
    if (p == 0) {
        o = red[0][jc];
#pragma unroll
        for (int pp = 1; pp < P; ++pp) {
            const float4 t = red[pp][jc];
            o.x += t.x, o.y += t.y, o.z += t.z, o.w += t.w;
        }
        if (a.z) {  // o <- o / sqrt(mean(o^2) + eps) * w * silu(z); the row is lanes 0..CPR-1
            float ss = o.x * o.x + o.y * o.y + o.z * o.z + o.w * o.w;
#pragma unroll
            for (int m = 1; m < CPR; m <<= 1)
                ss += __shfl_xor(ss, m);
            const float inv = rsqrtf(ss * (1.f / DV) + a.norm_eps);
            o.x *= inv * wv.x * silu(zv.x), o.y *= inv * wv.y * silu(zv.y);
            o.z *= inv * wv.z * silu(zv.z), o.w *= inv * wv.w * silu(zv.w);
        }
        *(float4 *)(a.o + ((int64_t)b * H + head) * DV + 4 * jc) = o;
    }
}

template <typename T, int DK, int DV, bool KDA>
hipError_t launch_dk(const DecodeArgs &a, hipStream_t s)
{
    const dim3 grid((unsigned)((int64_t)a.B * a.H));
    const dim3 block(DEC_THREADS);
    switch (a.K) {
    case 0: hipLaunchKernelGGL((decode_kernel<T, DK, DV, KDA, 0>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_kernel<T, DK, DV, KDA, 2>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((decode_kernel<T, DK, DV, KDA, 3>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_kernel<T, DK, DV, KDA, 4>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, bool KDA>
hipError_t launch_t(const DecodeArgs &a, hipStream_t s)
{
    if (a.dk == 128 && a.dv == 128)
        return launch_dk<T, 128, 128, KDA>(a, s);
    if (a.dk == 64 && a.dv == 64)
        return launch_dk<T, 64, 64, KDA>(a, s);
    if (a.dk == 128 && a.dv == 256)
        return launch_dk<T, 128, 256, KDA>(a, s);
    if (a.dk == 64 && a.dv == 128)
        return launch_dk<T, 64, 128, KDA>(a, s);
    return hipErrorInvalidValue;
}

// The q/k windows of a step whose q/k heads serve several value heads: every reader has
// finished (the decode kernel ran before on the same stream). One thread per (stream,
// q/k channel).
template <typename T, int K>
__global__ void __launch_bounds__(256) decode_qk_window_kernel(const DecodeArgs a)
{
    constexpr int W = K - 1;
    const int nqk = 2 * a.Hqk * a.dk;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)a.B * nqk)
        return;
    const int b = (int)(idx / nqk), c = (int)(idx - (int64_t)b * nqk);
    const int qk = a.Hqk * a.dk;
    const T *src = c < qk ? (const T *)a.q + c : (const T *)a.k + (c - qk);
    T *win = (T *)a.conv_state_ptrs[b] + (int64_t)c * W;
    T old[W];
#pragma unroll
    for (int i = 0; i < W; ++i)
        old[i] = win[i];
#pragma unroll
    for (int i = 0; i + 1 < W; ++i)
        win[i] = old[i + 1];
    win[W - 1] = src[(int64_t)b * a.ld];
}

template <typename T>
hipError_t launch_qk_window_t(const DecodeArgs &a, hipStream_t s)
{
    const unsigned g = (unsigned)(((int64_t)a.B * 2 * a.Hqk * a.dk + 255) / 256);
    switch (a.K) {
    case 2: hipLaunchKernelGGL((decode_qk_window_kernel<T, 2>), dim3(g), dim3(256), 0, s, a); break;
    case 3: hipLaunchKernelGGL((decode_qk_window_kernel<T, 3>), dim3(g), dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_qk_window_kernel<T, 4>), dim3(g), dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_qk_window(int dtype, const DecodeArgs &a, hipStream_t s)
{
    return dtype ? launch_qk_window_t<bf16>(a, s) : launch_qk_window_t<float>(a, s);
}

hipError_t launch_decode(int dtype, int kda, const DecodeArgs &a, hipStream_t s)
{
    if (dtype)
        return kda ? launch_t<bf16, true>(a, s) : launch_t<bf16, false>(a, s);
    return kda ? launch_t<float, true>(a, s) : launch_t<float, false>(a, s);
}

}  // namespace gdn
