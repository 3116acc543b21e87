// gdn_kernels.hip -- gfx950 (CDNA4) kernels of the chunked gated-delta-rule prefill.
//
// Two kernels carry the path (pages "metrale_model_arch/glm5next_kda/prefill.rs" --
// the launch sequence conv_prefill, l2, fill, split_widen, chunk_prepare, chunk_scan of
// prefill_with_pad_fill -- and "split_prefill.rs" -- the batched and varlen entry points):
//
//  * front_kernel: causal depthwise conv1d + SiLU over every channel of the packed
//    [q | k | v] rows, then L2 of each q and k head vector and the q scale, written once as
//    packed activations. Parallel over (channel group, token tile). A small follow-up
//    kernel advances the carried conv windows once every tile has read the old ones.
//    Replaces conv_prefill + l2 + split_widen.
//  * chunk_kernel: one workgroup per (stream, head, dv slice) walks the stream's chunks in
//    order. Per chunk it builds the cumulative log-gates, K K^T and Q K^T on MFMA, the
//    unit-lower-triangular inverse T = (I + M)^-1 by 16x16 block substitution, the WY/UT
//    factors W = T diag(beta) (K . a) and U~ = T diag(beta) V, and then the state
//    products U = U~ - W h, O = (Q . a) h + P U, h <- a_C h + (K . a_C/a)^T U with h held
//    in MFMA accumulator registers across chunks. Replaces chunk_prepare + chunk_scan and
//    the separate q/k/v widen buffers; tail rows of a partial chunk are zeroed by select on
//    load, never read.
//
// MFMA fragment convention (v_mfma_f32_16x16x32_f16, and 8 x v_mfma_f32_16x16x4_f32 for
// float inputs): lane l = 16*g + c holds, for a 32-wide contraction block starting at k0,
// the k indices k0 + 4g + {0..3} and k0 + 16 + 4g + {0..3}. With this order, the 16x16
// fp32 accumulators of two m-blocks (rows 4g+i of each) are directly the B operand of the
// next product, so h, U and intermediate results never leave registers.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_internal.h"

namespace gdn {

typedef __bf16 bf16;
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef _Float16 f16x4 __attribute__((__vector_size__(4 * sizeof(_Float16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef float f32x8 __attribute__((__vector_size__(8 * sizeof(float))));

// MFMA operand type of a tile element type: fp16 operands (bf16 inputs convert to fp16
// exactly; fp16 keeps 3 more mantissa bits at the same MFMA rate) or fp32 operands.
template <typename T>
struct Tr;
template <>
struct Tr<f16> {
    typedef f16x8 frag;
    static constexpr int VEC = 8;  // elements per 16-byte access
};
template <>
struct Tr<float> {
    typedef f32x8 frag;
    static constexpr int VEC = 4;
};

// ------------------------------------------------------------------------------------
// small helpers

__device__ __forceinline__ void mma(f32x4 &d, const f16x8 &a, const f16x8 &b)
{
    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, d, 0, 0, 0);
}

__device__ __forceinline__ void mma(f32x4 &d, const f32x8 &a, const f32x8 &b)
{
#pragma unroll
    for (int j = 0; j < 8; ++j)
        d = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], d, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// 16 bytes of global memory -> floats (8 for 2-byte types, 4 for float)
__device__ __forceinline__ void load_vec(const bf16 *p, float (&x)[8])
{
    const uint4 u = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void load_vec(const f16 *p, float (&x)[8])
{
    const f16x8 v = *reinterpret_cast<const f16x8 *>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i)
        x[i] = (float)v[i];
}
__device__ __forceinline__ void load_vec(const float *p, float (&x)[4])
{
    const float4 f = *reinterpret_cast<const float4 *>(p);
    x[0] = f.x, x[1] = f.y, x[2] = f.z, x[3] = f.w;
}

// floats -> 16 bytes (global or LDS)
__device__ __forceinline__ void store_vec(f16 *p, const float (&x)[8])
{
    f16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        v[i] = (f16)x[i];
    *reinterpret_cast<f16x8 *>(p) = v;
}
__device__ __forceinline__ void store_vec(float *p, const float (&x)[4])
{
    *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
}

// Operand fragment from a row-major LDS tile X[row][k] (row stride ld elements):
// row = row0 + (lane & 15), k = k0 + 4g + {0..3} and k0 + 16 + 4g + {0..3}.
__device__ __forceinline__ f16x8 ld_frag(const f16 *X, int ld, int row0, int k0, int lane)
{
    const f16 *p = X + (row0 + (lane & 15)) * ld + k0 + 4 * (lane >> 4);
    const f16x4 lo = *reinterpret_cast<const f16x4 *>(p);
    const f16x4 hi = *reinterpret_cast<const f16x4 *>(p + 16);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f32x8 ld_frag(const float *X, int ld, int row0, int k0, int lane)
{
    const float *p = X + (row0 + (lane & 15)) * ld + k0 + 4 * (lane >> 4);
    const f32x4 lo = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 hi = *reinterpret_cast<const f32x4 *>(p + 16);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// B operand of a 32-deep block from the accumulators of its two 16-row halves.
template <typename T>
__device__ __forceinline__ typename Tr<T>::frag pack(const f32x4 &d0, const f32x4 &d1);
template <>
__device__ __forceinline__ f16x8 pack<f16>(const f32x4 &d0, const f32x4 &d1)
{
    f16x8 f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[i] = (f16)d0[i];
        f[4 + i] = (f16)d1[i];
    }
    return f;
}
template <>
__device__ __forceinline__ f32x8 pack<float>(const f32x4 &d0, const f32x4 &d1)
{
    return __builtin_shufflevector(d0, d1, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ void stream_bounds(const Streams &s, int b, int64_t &start,
                                              int64_t &end)
{
    if (s.cu) {
        start = s.cu[b];
        end = s.cu[b + 1];
    } else {
        start = (int64_t)b * s.tps;
        end = start + s.tps;
    }
}

// ------------------------------------------------------------------------------------
// front end: conv + SiLU (+ L2, scale)

constexpr int FRONT_THREADS = 256;
constexpr int FRONT_ROWS = 32;  // tokens per tile
constexpr int FRONT_CPT = 8;    // channels per thread

template <typename T>
__device__ __forceinline__ void load8(const T *p, float (&x)[8])
{
    load_vec(p, x);  // 2-byte element types: one 16-byte access
}
template <>
__device__ __forceinline__ void load8<float>(const float *p, float (&x)[8])
{
    float a[4], b[4];
    load_vec(p, a);
    load_vec(p + 4, b);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        x[i] = a[i], x[4 + i] = b[i];
}
template <typename T>
__device__ __forceinline__ void store8(T *p, const float (&x)[8])
{
    store_vec(p, x);
}
template <>
__device__ __forceinline__ void store8<float>(float *p, const float (&x)[8])
{
    const float a[4] = {x[0], x[1], x[2], x[3]}, b[4] = {x[4], x[5], x[6], x[7]};
    store_vec(p, a);
    store_vec(p + 4, b);
}

// stream containing row t (largest b with start_b <= t < end_b); rows of zero-length
// streams are skipped because their start equals the next start.
__device__ __forceinline__ int find_stream(const Streams &s, int64_t t)
{
    if (!s.cu)
        return (int)(t / s.tps);
    int lo = 0, hi = s.B - 1;  // invariant: cu[lo] <= t
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s.cu[mid] <= t)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

template <typename T, typename TOUT, int K>
__global__ void __launch_bounds__(FRONT_THREADS) front_kernel(const FrontArgs a)
{
    constexpr int W = K - 1;
    const int cd = 2 * a.H * a.dk + a.H * a.dv;
    const int cg = blockIdx.x * FRONT_THREADS + threadIdx.x;  // channel group
    const int c0 = cg * FRONT_CPT;                              // first packed channel
    const bool active = c0 < cd;
    const int qk = a.H * a.dk;
    const int sec = !active ? 2 : (c0 < qk ? 0 : (c0 < 2 * qk ? 1 : 2));
    const T *src = sec == 0 ? (const T *)a.q + c0
                 : sec == 1 ? (const T *)a.k + (c0 - qk)
                            : (const T *)a.v + (c0 - 2 * qk);
    const int lanes_per_head = a.dk / FRONT_CPT;  // power of two, <= 64

    float w[K][FRONT_CPT];
#pragma unroll
    for (int j = 0; j < K; ++j)
#pragma unroll
        for (int i = 0; i < FRONT_CPT; ++i)
            w[j][i] = active ? a.conv_w[(int64_t)(c0 + i) * K + j] : 0.f;

    const int64_t t0 = (int64_t)blockIdx.y * FRONT_ROWS;
    const int64_t t1 = min(t0 + FRONT_ROWS, a.N);
    if (t0 >= t1)
        return;  // uniform over the block

    // win[j] = extended position (p_t - W + j) of the next token t, where the extended
    // sequence of stream b is [carried window (W) | rows start_b .. end_b-1].
    float win[W > 0 ? W : 1][FRONT_CPT];
    int b = find_stream(a.st, t0);
    int64_t sb, eb;
    stream_bounds(a.st, b, sb, eb);
    auto init_window = [&](int64_t t) {
        const T *cs = a.conv_state_ptrs ? (const T *)a.conv_state_ptrs[b]
                                        : (const T *)a.conv_state;
#pragma unroll
        for (int j = 0; j < W; ++j) {
            const int64_t e = (t - sb) + j;
            float x[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            if (active) {
                if (e < W) {
#pragma unroll
                    for (int i = 0; i < FRONT_CPT; ++i)
                        x[i] = (float)cs[(int64_t)(c0 + i) * W + e];
                } else {
                    load8<T>(src + (sb + e - W) * a.ld, x);
                }
            }
#pragma unroll
            for (int i = 0; i < FRONT_CPT; ++i)
                win[j][i] = x[i];
        }
    };
    init_window(t0);

    TOUT *y = (TOUT *)a.y;
    for (int64_t t = t0; t < t1; ++t) {
        if (t >= eb) {  // the next non-empty stream starts at t
            do {
                ++b;
                stream_bounds(a.st, b, sb, eb);
            } while (eb <= t);
            init_window(t);
        }
        float x[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (active)
            load8<T>(src + t * a.ld, x);
        float z[FRONT_CPT];
#pragma unroll
        for (int i = 0; i < FRONT_CPT; ++i) {
            float acc = w[K - 1][i] * x[i];
#pragma unroll
            for (int j = 0; j < W; ++j)
                acc += w[j][i] * win[j][i];
            z[i] = acc / (1.f + __expf(-acc));
        }
#pragma unroll
        for (int j = 0; j + 1 < W; ++j)
#pragma unroll
            for (int i = 0; i < FRONT_CPT; ++i)
                win[j][i] = win[j + 1][i];
        if (W > 0) {
#pragma unroll
            for (int i = 0; i < FRONT_CPT; ++i)
                win[W > 0 ? W - 1 : 0][i] = x[i];
        }
        if (a.do_l2) {  // uniform; q and k heads are whole aligned lane groups
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < FRONT_CPT; ++i)
                ss += z[i] * z[i];
            for (int m = 1; m < lanes_per_head; m <<= 1)
                ss += __shfl_xor(ss, m);
            if (sec < 2) {
                const float inv = rsqrtf(ss + a.eps) * (sec == 0 ? a.scale : 1.f);
#pragma unroll
                for (int i = 0; i < FRONT_CPT; ++i)
                    z[i] *= inv;
            }
        } else if (sec == 0) {
#pragma unroll
            for (int i = 0; i < FRONT_CPT; ++i)
                z[i] *= a.scale;
        }
        if (active)
            store8<TOUT>(y + t * (int64_t)cd + c0, z);
    }
}

// New carried window of every stream: the last K-1 entries of [old window | rows].
// Runs after front_kernel (which reads the old windows), one thread per (stream, channel).
template <typename T, int K>
__global__ void __launch_bounds__(256) conv_state_kernel(const FrontArgs a)
{
    constexpr int W = K - 1;
    const int cd = 2 * a.H * a.dk + a.H * a.dv;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)a.st.B * cd)
        return;
    const int b = (int)(idx / cd), c = (int)(idx - (int64_t)b * cd);
    int64_t sb, eb;
    stream_bounds(a.st, b, sb, eb);
    const int64_t len = eb - sb;
    if (len <= 0)
        return;
    T *cs = a.conv_state_ptrs ? (T *)a.conv_state_ptrs[b] : (T *)a.conv_state;
    const int qk = a.H * a.dk;
    const T *src = c < qk ? (const T *)a.q + c
                 : c < 2 * qk ? (const T *)a.k + (c - qk)
                              : (const T *)a.v + (c - 2 * qk);
    T old[W > 0 ? W : 1], nw[W > 0 ? W : 1];
#pragma unroll
    for (int j = 0; j < W; ++j)
        old[j] = cs[(int64_t)c * W + j];
#pragma unroll
    for (int j = 0; j < W; ++j) {
        const int64_t e = len + j;
        T v = old[0];
#pragma unroll
        for (int jj = 0; jj < W; ++jj)
            if (e == jj)
                v = old[jj];
        nw[j] = e < W ? v : src[(sb + e - W) * a.ld];
    }
#pragma unroll
    for (int j = 0; j < W; ++j)
        cs[(int64_t)c * W + j] = nw[j];
}

template <typename T, typename TOUT, int K>
hipError_t launch_front_tk(const FrontArgs &a, hipStream_t s)
{
    const int cd = 2 * a.H * a.dk + a.H * a.dv;
    const int groups = cd / FRONT_CPT;
    dim3 grid((groups + FRONT_THREADS - 1) / FRONT_THREADS,
              (unsigned)((a.N + FRONT_ROWS - 1) / FRONT_ROWS));
    hipLaunchKernelGGL((front_kernel<T, TOUT, K>), grid, dim3(FRONT_THREADS), 0, s, a);
    return hipGetLastError();
}

template <typename T, int K>
hipError_t launch_state_tk(const FrontArgs &a, hipStream_t s)
{
    const int cd = 2 * a.H * a.dk + a.H * a.dv;
    const int64_t n = (int64_t)a.st.B * cd;
    hipLaunchKernelGGL((conv_state_kernel<T, K>), dim3((unsigned)((n + 255) / 256)), dim3(256),
                       0, s, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_state_t(const FrontArgs &a, hipStream_t s)
{
    switch (a.K) {
    case 2: return launch_state_tk<T, 2>(a, s);
    case 3: return launch_state_tk<T, 3>(a, s);
    case 4: return launch_state_tk<T, 4>(a, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_conv_state(int dtype, const FrontArgs &a, hipStream_t s)
{
    return dtype ? launch_state_t<bf16>(a, s) : launch_state_t<float>(a, s);
}

template <typename T, typename TOUT>
hipError_t launch_front_t(const FrontArgs &a, hipStream_t s)
{
    switch (a.K) {
    case 2: return launch_front_tk<T, TOUT, 2>(a, s);
    case 3: return launch_front_tk<T, TOUT, 3>(a, s);
    case 4: return launch_front_tk<T, TOUT, 4>(a, s);
    default: return hipErrorInvalidValue;
    }
}

// bf16 raw rows give fp16 activations (the chunk kernel's operand type); f32 gives f32
hipError_t launch_front(int dtype, const FrontArgs &a, hipStream_t s)
{
    return dtype ? launch_front_t<bf16, f16>(a, s) : launch_front_t<float, float>(a, s);
}

// ------------------------------------------------------------------------------------
// fused chunk kernel

constexpr int CH = 64;  // chunk length

template <typename T, int DK, int DV, int NW, bool KDA>
struct ChunkCfg {
    static constexpr int NV = 16 * NW;  // dv columns per workgroup
    static constexpr int PAD = 16 / (int)sizeof(T);
    static constexpr int LDQ = DK + PAD;  // Qs, Ks, Ws: [64][LDQ]
    static constexpr int LDT = CH + PAD;  // KTs [DK][LDT], VTs [NV][LDT], Ps/Tb/Tba [64][LDT]
    static constexpr int LDF = CH + 4;    // Ms, Tf: [64][LDF] float
    static constexpr int SZ_Q = CH * LDQ * (int)sizeof(T);
    static constexpr int SZ_KT = DK * LDT * (int)sizeof(T);
    static constexpr int SZ_VT = NV * LDT * (int)sizeof(T);
    static constexpr int SZ_P = CH * LDT * (int)sizeof(T);
    static constexpr int SZ_F = CH * LDF * 4;
    static constexpr int OFF_Q = 0;
    static constexpr int OFF_K = OFF_Q + SZ_Q;
    static constexpr int OFF_W = OFF_K + SZ_Q;  // Ms aliases Ws (dead before Ws is built)
    static constexpr int OFF_KT = OFF_W + (SZ_Q > SZ_F ? SZ_Q : SZ_F);
    static constexpr int OFF_VT = OFF_KT + SZ_KT;
    static constexpr int OFF_P = OFF_VT + SZ_VT;
    static constexpr int OFF_TB = OFF_P + SZ_P;
    static constexpr int OFF_TBA = OFF_TB + SZ_P;
    // fp16 operands: T is applied as an fp16 hi + lo pair (two MFMAs), which keeps the
    // WY factors at about fp32 accuracy; fp32 operands need no split
    static constexpr bool SPLIT = sizeof(T) == 2;
    static constexpr int OFF_TBL = OFF_TBA + SZ_P;
    static constexpr int OFF_TBAL = OFF_TBL + (SPLIT ? SZ_P : 0);
    static constexpr int OFF_TF = OFF_TBAL + (SPLIT ? SZ_P : 0);
    static constexpr int OFF_G = OFF_TF + SZ_F;  // gam[64], bet[64]
    static constexpr int BYTES = OFF_G + 2 * CH * 4;
};

// T_IJ = -T_II * sum_{K=J}^{I-1} M_IK T_KJ for one 16x16 block (one wave, fp32 MFMA).
template <int LDF>
__device__ __forceinline__ void solve_block(const float *Ms, float *Tf, int I, int J, int lane)
{
    const int g = lane >> 4, c = lane & 15;
    f32x4 y = zero4();
    for (int Kb = J; Kb < I; ++Kb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float av = Ms[(16 * I + c) * LDF + 16 * Kb + 4 * g + i];
            const float bv = Tf[(16 * Kb + 4 * g + i) * LDF + 16 * J + c];
            y = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, y, 0, 0, 0);
        }
    }
    f32x4 t = zero4();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float av = Tf[(16 * I + c) * LDF + 16 * I + 4 * g + i];
        t = __builtin_amdgcn_mfma_f32_16x16x4f32(av, y[i], t, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        Tf[(16 * I + 4 * g + i) * LDF + 16 * J + c] = -t[i];
}

template <typename TIN, typename T, int DK, int DV, int NW, bool KDA>
__global__ void __launch_bounds__(NW * 64) chunk_kernel(const ChunkArgs a)
{
    static_assert(sizeof(TIN) == sizeof(T), "16-byte loads fill whole operand vectors");
    using C = ChunkCfg<T, DK, DV, NW, KDA>;
    constexpr int NV = C::NV, LDQ = C::LDQ, LDT = C::LDT, LDF = C::LDF;
    constexpr int VEC = Tr<T>::VEC;
    constexpr int NT = NW * 64;
    typedef typename Tr<T>::frag frag;

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    T *Qs = (T *)(smem + C::OFF_Q);
    T *Ks = (T *)(smem + C::OFF_K);
    T *Ws = (T *)(smem + C::OFF_W);
    float *Ms = (float *)(smem + C::OFF_W);
    T *KTs = (T *)(smem + C::OFF_KT);
    T *VTs = (T *)(smem + C::OFF_VT);
    T *Ps = (T *)(smem + C::OFF_P);
    T *Tb = (T *)(smem + C::OFF_TB);
    T *Tba = (T *)(smem + C::OFF_TBA);
    T *Tbl = (T *)(smem + C::OFF_TBL);    // lo parts (fp16 operands only)
    T *Tbal = (T *)(smem + C::OFF_TBAL);
    float *Tf = (float *)(smem + C::OFF_TF);
    float *gam = (float *)(smem + C::OFF_G);
    float *bet = gam + CH;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g4 = lane >> 4, c16 = lane & 15;

    const int H = a.H;
    const int BH = a.st.B * H;
    const int slice = blockIdx.x / BH, bh = blockIdx.x - slice * BH;
    const int b = bh / H, head = bh - b * H;
    int64_t start, end;
    stream_bounds(a.st, b, start, end);
    float *hp = (a.h_ptrs ? a.h_ptrs[b] : a.h) + (int64_t)head * DK * DV;
    const int colw = slice * NV + wave * 16;  // this wave's first dv column

    const TIN *qg = (const TIN *)a.q + head * DK;
    const TIN *kg = (const TIN *)a.k + head * DK;
    const TIN *vg = (const TIN *)a.v + head * DV + slice * NV;
    float *og = (float *)a.o + head * DV + colw + c16;
    const int64_t ld = a.ld;

    // P's blocks above the diagonal that the 32-deep steps touch stay zero
    for (int idx = tid; idx < 2 * 256; idx += NT) {
        const int blk = idx >> 8, e = idx & 255;
        const int r = 32 * blk + (e >> 4), s = 32 * blk + 16 + (e & 15);
        Ps[r * LDT + s] = (T)0.f;
    }

    // state, D layout: hs[mb][i] = h[16 mb + 4 g + i][colw + c]
    f32x4 hs[DK / 16];
#pragma unroll
    for (int mb = 0; mb < DK / 16; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            hs[mb][i] = hp[(int64_t)(16 * mb + 4 * g4 + i) * DV + colw + c16];

    for (int64_t cs = start; cs < end; cs += CH) {
        const int L = (int)min((int64_t)CH, end - cs);

        // ---- A: load q, k (L2, scale), v^T, g, beta; rows >= L read as 0 -------------
        {
            constexpr int LPR = DK / VEC, RPW = 64 / LPR;
            for (int rr = wave * RPW + lane / LPR; rr < 2 * CH; rr += NW * RPW) {
                const bool isk = rr >= CH;
                const int r = rr & (CH - 1);
                const int c0 = (lane % LPR) * VEC;
                float x[VEC];
#pragma unroll
                for (int i = 0; i < VEC; ++i)
                    x[i] = 0.f;
                if (r < L)
                    load_vec((isk ? kg : qg) + (cs + r) * ld + c0, x);
                float mul = isk ? 1.f : a.scale;
                if (a.do_l2) {
                    float ss = 0.f;
#pragma unroll
                    for (int i = 0; i < VEC; ++i)
                        ss += x[i] * x[i];
#pragma unroll
                    for (int m = 1; m < LPR; m <<= 1)
                        ss += __shfl_xor(ss, m);
                    mul = r < L ? mul * rsqrtf(ss + a.eps) : 0.f;
                }
#pragma unroll
                for (int i = 0; i < VEC; ++i)
                    x[i] *= mul;
                store_vec((isk ? Ks : Qs) + r * LDQ + c0, x);
                if (isk) {
#pragma unroll
                    for (int i = 0; i < VEC; ++i)
                        KTs[(c0 + i) * LDT + r] = (T)x[i];
                }
            }
            constexpr int LPV = NV / VEC, RPV = 64 / LPV;
            for (int r = wave * RPV + lane / LPV; r < CH; r += NW * RPV) {
                const int c0 = (lane % LPV) * VEC;
                float x[VEC];
#pragma unroll
                for (int i = 0; i < VEC; ++i)
                    x[i] = 0.f;
                if (r < L)
                    load_vec(vg + (cs + r) * ld + c0, x);
#pragma unroll
                for (int i = 0; i < VEC; ++i)
                    VTs[(c0 + i) * LDT + r] = (T)x[i];
            }
            if (tid < CH) {
                const bool ok = tid < L;
                gam[tid] = ok ? a.g[(cs + tid) * H + head] : 0.f;
                bet[tid] = ok ? a.beta[(cs + tid) * H + head] : 0.f;
            }
        }
        __syncthreads();

        // ---- B: cumulative log-gate (inclusive scan over the chunk) --------------------
        if (wave == 0) {
            float x = gam[lane];
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off);
                if (lane >= off)
                    x += y;
            }
            gam[lane] = x;
        }
        __syncthreads();

        // ---- C: M = strict_tril(diag(beta) K K^T . decay), P = tril(Q K^T . decay) ------
        {
            for (int task = wave; task < 20; task += NW) {
                const bool isq = task >= 10;
                const int p = isq ? task - 10 : task;
                const int I = p < 1 ? 0 : p < 3 ? 1 : p < 6 ? 2 : 3;
                const int J = p - I * (I + 1) / 2;
                const T *As = isq ? Qs : Ks;
                f32x4 acc = zero4();
#pragma unroll
                for (int kb = 0; kb < DK / 32; ++kb)
                    mma(acc, ld_frag(As, LDQ, 16 * I, 32 * kb, lane),
                        ld_frag(Ks, LDQ, 16 * J, 32 * kb, lane));
                const int s = 16 * J + c16;
                const float gs = gam[s];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * I + 4 * g4 + i;
                    const float dec = __expf(fminf(gam[r] - gs, 0.f));
                    if (isq)
                        Ps[r * LDT + s] = (T)(s <= r ? dec * acc[i] : 0.f);
                    else
                        Ms[r * LDF + s] = s < r ? bet[r] * dec * acc[i] : 0.f;
                }
            }
        }
        __syncthreads();

        // ---- D: T = (I + M)^-1 by 16x16 block substitution -----------------------------
        if (wave == 0) {  // diagonal blocks: lane -> (block lane/16, column lane%16)
            const int base = 16 * g4, j = c16;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float s = r == j ? 1.f : 0.f;
#pragma unroll
                for (int t = 0; t < r; ++t)
                    s -= Ms[(base + r) * LDF + base + t] * x[t];
                x[r] = s;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r)
                Tf[(base + r) * LDF + base + j] = x[r];
        }
        __syncthreads();
        for (int I = 1 + wave; I <= 3; I += NW)
            solve_block<LDF>(Ms, Tf, I, I - 1, lane);
        __syncthreads();
        for (int I = 2 + wave; I <= 3; I += NW)
            solve_block<LDF>(Ms, Tf, I, I - 2, lane);
        __syncthreads();
        if (wave == 0)
            solve_block<LDF>(Ms, Tf, 3, 0, lane);
        __syncthreads();
        // Tb = T diag(beta), Tba = T diag(beta . a), zero above the diagonal
        for (int idx = tid; idx < CH * CH; idx += NT) {
            const int r = idx >> 6, s = idx & 63;
            const float t = s <= r ? Tf[r * LDF + s] : 0.f;
            const float tb = t * bet[s];
            const float tba = tb * __expf(gam[s]);
            const T tb_hi = (T)tb, tba_hi = (T)tba;
            Tb[r * LDT + s] = tb_hi;
            Tba[r * LDT + s] = tba_hi;
            if constexpr (C::SPLIT) {
                Tbl[r * LDT + s] = (T)(tb - (float)tb_hi);
                Tbal[r * LDT + s] = (T)(tba - (float)tba_hi);
            }
        }
        __syncthreads();

        // ---- E: W = Tba K (shared), U~ = Tb V (per wave) -------------------------------
        for (int task = wave; task < 4 * (DK / 16); task += NW) {
            const int I = task & 3, nb = task >> 2;
            f32x4 acc = zero4();
            for (int kb = 0; kb <= (I >> 1); ++kb) {
                const frag kt = ld_frag(KTs, LDT, 16 * nb, 32 * kb, lane);
                mma(acc, ld_frag(Tba, LDT, 16 * I, 32 * kb, lane), kt);
                if constexpr (C::SPLIT)
                    mma(acc, ld_frag(Tbal, LDT, 16 * I, 32 * kb, lane), kt);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                Ws[(16 * I + 4 * g4 + i) * LDQ + 16 * nb + c16] = (T)acc[i];
        }
        f32x4 ut[4];
        {
            const frag vt0 = ld_frag(VTs, LDT, 16 * wave, 0, lane);
            const frag vt1 = ld_frag(VTs, LDT, 16 * wave, 32, lane);
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                ut[I] = zero4();
                mma(ut[I], ld_frag(Tb, LDT, 16 * I, 0, lane), vt0);
                if constexpr (C::SPLIT)
                    mma(ut[I], ld_frag(Tbl, LDT, 16 * I, 0, lane), vt0);
                if (I >= 2) {
                    mma(ut[I], ld_frag(Tb, LDT, 16 * I, 32, lane), vt1);
                    if constexpr (C::SPLIT)
                        mma(ut[I], ld_frag(Tbl, LDT, 16 * I, 32, lane), vt1);
                }
            }
        }
        __syncthreads();

        // ---- F: state products for this wave's 16 columns ------------------------------
        {
            frag hf[DK / 32];
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb)
                hf[kb] = pack<T>(hs[2 * kb], hs[2 * kb + 1]);
            f32x4 u[4], o[4];
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                f32x4 wh = zero4(), qh = zero4();
#pragma unroll
                for (int kb = 0; kb < DK / 32; ++kb) {
                    mma(wh, ld_frag(Ws, LDQ, 16 * I, 32 * kb, lane), hf[kb]);
                    mma(qh, ld_frag(Qs, LDQ, 16 * I, 32 * kb, lane), hf[kb]);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * I + 4 * g4 + i;
                    u[I][i] = ut[I][i] - wh[i];
                    o[I][i] = qh[i] * __expf(gam[r]);
                }
            }
            const frag uf0 = pack<T>(u[0], u[1]), uf1 = pack<T>(u[2], u[3]);
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                mma(o[I], ld_frag(Ps, LDT, 16 * I, 0, lane), uf0);
                if (I >= 2)
                    mma(o[I], ld_frag(Ps, LDT, 16 * I, 32, lane), uf1);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * I + 4 * g4 + i;
                    if (r < L)
                        og[(cs + r) * (int64_t)H * DV] = o[I][i];
                }
            }
            const float gC = gam[CH - 1];
            const float aC = __expf(gC);
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    u[I][i] *= __expf(gC - gam[16 * I + 4 * g4 + i]);
            const frag vf0 = pack<T>(u[0], u[1]), vf1 = pack<T>(u[2], u[3]);
#pragma unroll
            for (int mb = 0; mb < DK / 16; ++mb) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    hs[mb][i] *= aC;
                mma(hs[mb], ld_frag(KTs, LDT, 16 * mb, 0, lane), vf0);
                mma(hs[mb], ld_frag(KTs, LDT, 16 * mb, 32, lane), vf1);
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int mb = 0; mb < DK / 16; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            hp[(int64_t)(16 * mb + 4 * g4 + i) * DV + colw + c16] = hs[mb][i];
}

template <typename TIN, typename T, int DK, int DV, int NW, bool KDA>
hipError_t launch_chunk_t(const ChunkArgs &a, int grid, hipStream_t s)
{
    using C = ChunkCfg<T, DK, DV, NW, KDA>;
    static_assert(C::BYTES <= 160 * 1024, "LDS budget");
    static_assert(DV % C::NV == 0, "slices");
    auto kern = chunk_kernel<TIN, T, DK, DV, NW, KDA>;
    static bool attr_set = false;  // per instance; same value on every device
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, C::BYTES);
        if (e != hipSuccess)
            return e;
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(NW * 64), C::BYTES, s, a);
    return hipGetLastError();
}

// Instances: (input element, operand type, input kind, dk, dv, waves per workgroup).
// Input kind: 0 = f32 rows, 1 = bf16 rows, 2 = fp16 activations of the front end.
#define GDN_CHUNK_INSTANCES(X)          \
    X(bf16, f16, 1, 128, 128, 8)        \
    X(bf16, f16, 1, 128, 128, 4)        \
    X(bf16, f16, 1, 128, 128, 2)        \
    X(bf16, f16, 1, 128, 128, 1)        \
    X(f16, f16, 2, 128, 128, 8)         \
    X(f16, f16, 2, 128, 128, 4)         \
    X(f16, f16, 2, 128, 128, 2)         \
    X(f16, f16, 2, 128, 128, 1)         \
    X(bf16, f16, 1, 64, 64, 4)          \
    X(bf16, f16, 1, 64, 64, 1)          \
    X(f16, f16, 2, 64, 64, 4)           \
    X(f16, f16, 2, 64, 64, 1)           \
    X(float, float, 0, 64, 64, 4)       \
    X(float, float, 0, 64, 64, 1)

hipError_t launch_chunk(int in_kind, int dk, int dv, int kda, int nw, const ChunkArgs &a,
                        int grid, hipStream_t s)
{
#define X(TIN, T, IK, DK, DV, NW)                                    \
    if (in_kind == IK && dk == DK && dv == DV && nw == NW && !kda)   \
        return launch_chunk_t<TIN, T, DK, DV, NW, false>(a, grid, s);
    GDN_CHUNK_INSTANCES(X)
#undef X
    return hipErrorInvalidValue;
}

int chunk_instance_exists(int in_kind, int dk, int dv, int kda, int nw)
{
#define X(TIN, T, IK, DK, DV, NW)                                   \
    if (in_kind == IK && dk == DK && dv == DV && nw == NW && !kda)  \
        return 1;
    GDN_CHUNK_INSTANCES(X)
#undef X
    return 0;
}

// ------------------------------------------------------------------------------------
// varlen chunk table: one block, streams handled CT_THREADS at a time

constexpr int CT_THREADS = 256;

__global__ void __launch_bounds__(CT_THREADS)
chunk_table_kernel(const int32_t *cu, int32_t B, int32_t chunk, int32_t *table,
                   int64_t max_entries, int32_t *count)
{
    __shared__ int64_t part[CT_THREADS];
    int64_t base = 0;
    for (int32_t b0 = 0; b0 < B; b0 += CT_THREADS) {
        const int32_t b = b0 + threadIdx.x;
        int64_t n = 0, start = 0, len = 0;
        if (b < B) {
            start = cu[b];
            len = (int64_t)cu[b + 1] - start;
            n = len > 0 ? (len + chunk - 1) / chunk : 0;
        }
        part[threadIdx.x] = n;
        __syncthreads();
        for (int off = 1; off < CT_THREADS; off <<= 1) {  // inclusive scan
            const int64_t v = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
            __syncthreads();
            part[threadIdx.x] += v;
            __syncthreads();
        }
        const int64_t first = base + part[threadIdx.x] - n;
        for (int64_t c = 0; c < n; ++c) {
            const int64_t e = first + c;
            if (e < max_entries) {
                table[4 * e + 0] = b;
                table[4 * e + 1] = (int32_t)(start + c * chunk);
                table[4 * e + 2] = (int32_t)min((int64_t)chunk, len - c * chunk);
                table[4 * e + 3] = (int32_t)c;
            }
        }
        base += part[CT_THREADS - 1];
        __syncthreads();
    }
    if (threadIdx.x == 0)
        *count = (int32_t)base;
}

hipError_t launch_chunk_table(const int32_t *cu, int32_t B, int32_t chunk, int32_t *table,
                              int64_t max_entries, int32_t *count, hipStream_t s)
{
    hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(CT_THREADS), 0, s, cu, B, chunk,
                       table, max_entries, count);
    return hipGetLastError();
}

}  // namespace gdn
