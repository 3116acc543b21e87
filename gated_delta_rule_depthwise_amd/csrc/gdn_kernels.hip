// gdn_kernels.hip -- gfx950 (CDNA4) kernels of the chunked gated-delta-rule prefill.
//
// Pages "metrale_model_arch/glm5next_kda/prefill.rs" (the launch sequence conv_prefill, l2,
// fill, split_widen, chunk_prepare, chunk_scan of prefill_with_pad_fill) and
// "split_prefill.rs" (the batched and varlen entry points):
//
//  * chunk_kernel: one workgroup per (stream, head, dv slice) walks the stream's chunks in
//    order (or, for few long streams, one segment of them; see chain_block). Per chunk:
//    the load stage brings the chunk's rows into LDS tiles -- with the front end fused
//    (bf16 raw rows), the causal depthwise conv + SiLU, the L2 of q and k and the q scale
//    run here in fp32 on raw rows that arrived by LDS-DMA one chunk ahead; otherwise the
//    rows (or the front kernel's activations) are L2-normalised on load. Then the
//    cumulative log-gates, M = strict_tril(diag(beta) K K^T . decay) and P = tril(Q K^T .
//    decay) on MFMA, the inverse of each 16x16 diagonal block of (I + M), and the state
//    products U = T diag(beta)(V - diag(a) K h) by block forward substitution, O =
//    diag(a) Q h + P U and h <- a_C h + K^T diag(a_C / a) U, with h held in MFMA
//    accumulators across chunks. Tail rows of a partial chunk are zeroed by select, never
//    read. Replaces chunk_prepare + chunk_scan and the q/k/v widen buffers.
//  * front_kernel: the front end as a kernel of its own, for the calls the chunk kernel
//    does not fuse it into (float32 rows, the per-key-channel gate, shared q/k heads,
//    dv != dk, 2 or 3 taps, the output gate): conv + SiLU, L2 and q scale written once as
//    packed activations (fp32 for float32 rows, fp16 for bf16 rows). The carried windows
//    are then advanced by extra workgroups of the first chunk-kernel launch.
//  * chain_block: the chain of segment maps of the segmented scan, and the hand-over of
//    warm-started streams' final states and windows, run by workgroups at the front of the
//    chunk kernel's second launch of a segmented call.
//  * decode lives in gdn_decode.hip.
//
// MFMA fragment convention (v_mfma_f32_16x16x32_f16, and 8 x v_mfma_f32_16x16x4_f32 for
// float inputs): lane l = 16*g + c holds, for a 32-wide contraction block starting at k0,
// the k indices k0 + 4g + {0..3} and k0 + 16 + 4g + {0..3}. With this order, the 16x16
// fp32 accumulators of two m-blocks (rows 4g+i of each) are directly the B operand of the
// next product, so h, U and intermediate results never leave registers.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gdn.h"
#include "gdn_internal.h"

namespace gdn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
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

// Cross-lane moves on DPP: a VALU operand modifier, so a reduction or scan step costs a few
// cycles instead of an LDS round trip per step. A lane whose source falls outside its row
// reads 0.
namespace dpp {
constexpr int QUAD_XOR1 = 0xB1, QUAD_XOR2 = 0x4E;  // quad_perm [1,0,3,2] and [2,3,0,1]
constexpr int ROW_SHR = 0x110, ROW_MIRROR = 0x140, ROW_HALF_MIRROR = 0x141;
constexpr int ROW_BCAST15 = 0x142, ROW_BCAST31 = 0x143;
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float mov(float x)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xf,
                                           true));
}
}  // namespace dpp

// Streaming accesses: 16-byte loads of rows that are read once and stores of o, which is
// written once, as nontemporal accesses so they do not displace cached data (measured:
// front kernel -10% on T=16384, chunk kernel -2..5%).
typedef unsigned int nt_u4 __attribute__((ext_vector_type(4)));
typedef float nt_f4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream16(const void *p)
{
    const nt_u4 v = __builtin_nontemporal_load((const nt_u4 *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_stream16(void *p, float4 v)
{
    const nt_f4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, (nt_f4 *)p);
}

// LDS-DMA of 16 bytes per lane: global p -> LDS byte address lds + 16 * lane (lds uniform
// over the wave). Issued as inline asm: for the builtin the compiler assumes that every
// later LDS read may read the transfer's destination and waits for all loads in flight
// before each one, which stalls a whole stage on a prefetch meant for the next chunk. The
// callers wait for their transfers themselves (vmcnt(0), then a barrier) before reading
// the destination, and do not touch it while transfers are in flight.
// The global address is a uniform base (an SGPR pair) plus a 32-bit byte offset per lane,
// so a transfer costs the wave no vector address arithmetic.
__device__ __forceinline__ void dma16(const void *base, uint32_t off, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(base), "s"(lds)
                 : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// Sum over aligned groups of N lanes, N in {4, 8, 16}; every lane of a group gets the same
// bits (each step adds the same two partial sums in both lanes).
template <int N>
__device__ __forceinline__ float group_sum(float x)
{
    static_assert(N == 4 || N == 8 || N == 16, "DPP groups are quads, half rows or rows");
    x += dpp::mov<dpp::QUAD_XOR1>(x);
    x += dpp::mov<dpp::QUAD_XOR2>(x);
    if constexpr (N >= 8)
        x += dpp::mov<dpp::ROW_HALF_MIRROR>(x);
    if constexpr (N >= 16)
        x += dpp::mov<dpp::ROW_MIRROR>(x);
    return x;
}

// Inclusive prefix sum over the 64 lanes of a wave: a scan within each row of 16 lanes,
// then the totals of rows 0 and 2 into rows 1 and 3, then that of rows 0-1 into rows 2-3.
__device__ __forceinline__ float wave_scan(float x)
{
    x += dpp::mov<dpp::ROW_SHR + 1>(x);
    x += dpp::mov<dpp::ROW_SHR + 2>(x);
    x += dpp::mov<dpp::ROW_SHR + 4>(x);
    x += dpp::mov<dpp::ROW_SHR + 8>(x);
    x += dpp::mov<dpp::ROW_BCAST15, 0xa>(x);
    x += dpp::mov<dpp::ROW_BCAST31, 0xc>(x);
    return x;
}

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
// raw 16-byte vector -> floats
__device__ __forceinline__ void unpack(const bf16 *, const uint4 &u, float (&x)[8])
{
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void unpack(const f16 *, const uint4 &u, float (&x)[8])
{
    const f16x8 v = __builtin_bit_cast(f16x8, u);
#pragma unroll
    for (int i = 0; i < 8; ++i)
        x[i] = (float)v[i];
}
__device__ __forceinline__ void unpack(const float *, const uint4 &u, float (&x)[4])
{
    x[0] = __uint_as_float(u.x), x[1] = __uint_as_float(u.y);
    x[2] = __uint_as_float(u.z), x[3] = __uint_as_float(u.w);
}

// 4 floats -> 4 elements (8 or 16 bytes)
__device__ __forceinline__ void store_vec4(f16 *p, const float (&x)[4])
{
    *reinterpret_cast<f16x4 *>(p) = f16x4{(f16)x[0], (f16)x[1], (f16)x[2], (f16)x[3]};
}
__device__ __forceinline__ void store_vec4(float *p, const float (&x)[4])
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

// Q/K operand tiles [64][DK]. Rows are padded to 8 dwords past a multiple of 32 banks,
// which suits the transposed reads (4 rows x 4 chunks of 4 elements per 16 lanes). For the
// row-wise fragment reads (16 consecutive rows at one chunk) the chunks of row r are
// permuted as ch ^ ((r / 4) mod 4): rows r and r + 4 then land 2 dwords apart instead of on
// the same banks. The permutation touches the low 2 bits of the chunk index only, so the
// offsets between the chunks a lane reads stay compile-time constants.
template <typename T, int DK>
struct QK {
    static constexpr bool SWZ = sizeof(T) == 2;
    static constexpr int LD = DK + 32 / (int)sizeof(T);
    // element offset of the chunk holding elements (r, 4 ch .. 4 ch + 3)
    __device__ static __forceinline__ int at(int r, int ch)
    {
        return r * LD + (SWZ ? (ch ^ ((r >> 2) & 3)) : ch) * 4;
    }
};

// ld_frag for a Q/K tile. row0 is a multiple of 16 and k0 of 32, so the permutation of a
// lane's chunks depends on the lane alone: the offset is row0 * LD + k0 plus a lane part
// (the same in every call, so the compiler keeps one address per tile and folds the rest
// into the instruction's offset), and chunk ch + 4 sits 16 elements after chunk ch.
template <int DK>
__device__ __forceinline__ int qk_lane_part(int lane)
{
    using L = QK<f16, DK>;
    return (lane & 15) * L::LD + ((lane >> 4) ^ ((lane >> 2) & 3)) * 4;
}
template <int DK>
__device__ __forceinline__ f16x8 ld_frag_qk(const f16 *X, int row0, int k0, int lane)
{
    using L = QK<f16, DK>;
    const f16 *p = X + row0 * L::LD + k0 + qk_lane_part<DK>(lane);
    const f16x4 lo = *reinterpret_cast<const f16x4 *>(p);
    const f16x4 hi = *reinterpret_cast<const f16x4 *>(p + 16);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
template <int DK>
__device__ __forceinline__ f32x8 ld_frag_qk(const float *X, int row0, int k0, int lane)
{
    return ld_frag(X, QK<float, DK>::LD, row0, k0, lane);
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
constexpr int FRONT_ROWS = 32;  // fewest tokens per tile
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

constexpr int CH = 64;  // chunk length

// Warm starts: a segment starts from h = 0 once the chunks before it bound the norm of
// their transition by e^kWarmLogBound. The state it drops is then at most e^-16 (< 2^-23)
// of the state's norm at the start of that window: the fp32 rounding of that state, and
// below the precision of the hi + lo operand pairs (about 2^-22) through which every chunk
// already passes the state, unless the state shrank by orders of magnitude across the
// window. (A transition job's early stop, which substitutes an exact zero, waits for e^-110:
// below half the smallest fp32 subnormal.)
constexpr float kWarmLogBound = -16.f;

// The plan of one (stream, head) in one workgroup (extra workgroups of the float32 front
// kernel); see WarmArgs. Wave w takes boundaries w + 1, w + 5, ...:
// it walks back from the boundary over the previous segment's chunks, four at a time (lane l
// reading row l of each), until their log-gates sum below kWarmLogBound.
__device__ __forceinline__ void warm_plan_block(const WarmArgs &a, int bh)
{
    const int b = bh / a.H, head = bh - b * a.H;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    if (tid < 16)  // the read flags the scan's first launch orders two of its jobs by
        reinterpret_cast<int *>(a.seg_ws + a.lay.flags(b, head))[tid] = 0;
    int64_t start, end;
    stream_bounds(a.st, b, start, end);
    const int S = a.nseg;
    for (int s = wv + 1; s <= S - 1; s += 4) {  // uniform per wave
        const int64_t cs = (a.seg0_len + (int64_t)(s - 1) * a.seg_len) / CH;
        const int64_t cp = s == 1 ? 0 : (a.seg0_len + (int64_t)(s - 2) * a.seg_len) / CH;
        float acc = 0.f;
        int w = 0, done = 0;  // done: 1 found, -1 not possible
        for (int64_t c0 = cs - 1; c0 >= cp && !done; c0 -= 4) {
            float gv[4], bv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t r = start + (c0 - u) * CH + lane;
                const bool in = c0 - u >= cp && r < end;
                gv[u] = in ? a.g[r * a.H + head] : 0.f;
                bv[u] = in ? a.beta[r * a.H + head] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float sum = __builtin_bit_cast(
                    float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wave_scan(gv[u])),
                                                     63));
                const bool bad = __ballot(!(bv[u] >= 0.f && bv[u] <= 1.9f)) != 0;
                if (!done && c0 - u >= cp) {
                    if (bad) {
                        done = -1;
                    } else {
                        acc += sum;
                        ++w;
                        if (acc < kWarmLogBound)
                            done = 1;
                    }
                }
            }
        }
        if (lane == 0)
            a.seg_ws[a.lay.warm_chunks(b, s, head)] = done == 1 ? (float)w : 0.f;
    }
}

// One workgroup per (stream, head, boundary s = 1..S-1): it walks back from the boundary over
// the previous segment's chunks, RC chunks per round (all their gates requested at once),
// and records the fewest chunks whose
// bounds sum below kWarmLogBound (0: none inside the previous segment, or a beta outside
// [0, 1.9] first). A token's bound is its log-gate, or with the per-key-channel gate its
// largest channel log-gate: lanes take a share of a row's channels, a maximum over them,
// then a sum over the chunk's rows. Only the gates of the window are read.
template <bool KDA, int DK>
__global__ void __launch_bounds__(KDA ? 1024 : 256) warm_boundary_kernel(const WarmArgs a)
{
    if (debug_stop(a.dbg))
        return;
    // per round: GDN 4 chunks on 4 waves (one per wave, a row per lane); KDA 8 chunks on 16
    // waves, two per chunk, 32 rows per wave read 8 rows per instruction with 8 lanes per
    // row (whole 128-byte lines), 4 row groups of 8
    constexpr int NWV = KDA ? 16 : 4, RC = KDA ? 8 : 4;
    constexpr int PPL = KDA ? DK / 32 : 1;  // 16-byte pieces of a row per lane (KDA)
    __shared__ float part[NWV];
    __shared__ int bad_beta[NWV];
    const int S = a.nseg;
    const int bh = blockIdx.x / (S - 1), s = blockIdx.x - bh * (S - 1) + 1;
    const int b = bh / a.H, head = bh - b * a.H;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    if (s == 1 && tid < 16)  // the read flags the scan's first launch orders two jobs by
        reinterpret_cast<int *>(a.seg_ws + a.lay.flags(b, head))[tid] = 0;
    int64_t start, end;
    stream_bounds(a.st, b, start, end);
    const int64_t cs = (a.seg0_len + (int64_t)(s - 1) * a.seg_len) / CH;
    const int64_t cp = s == 1 ? 0 : (a.seg0_len + (int64_t)(s - 2) * a.seg_len) / CH;
    float acc = 0.f;
    int w = 0, done = 0;  // done: 1 found, -1 not possible (uniform over the workgroup)
    for (int64_t ctop = cs - 1; ctop >= cp && !done; ctop -= RC) {
        float gv = 0.f;
        bool bad_row = false;
        if constexpr (KDA) {
            const int64_t c = ctop - (wv >> 1);
            const int r0 = (wv & 1) * 32 + (lane >> 3);  // + 8 rg
            uint4 u[4][PPL];
            bool in[4];
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int64_t r = start + c * CH + r0 + 8 * rg;
                in[rg] = c >= cp && r < end;
                const float *row = a.g + (r * a.H + head) * DK + 4 * (lane & 7);
#pragma unroll
                for (int q = 0; q < PPL; ++q)
                    u[rg][q] = in[rg] ? load_stream16(row + 32 * q) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                float m = -__builtin_inff();
#pragma unroll
                for (int q = 0; q < PPL; ++q)
                    m = fmaxf(m, fmaxf(fmaxf(__uint_as_float(u[rg][q].x),
                                             __uint_as_float(u[rg][q].y)),
                                       fmaxf(__uint_as_float(u[rg][q].z),
                                             __uint_as_float(u[rg][q].w))));
                m = fmaxf(m, __shfl_xor(m, 1));
                m = fmaxf(m, __shfl_xor(m, 2));
                m = fmaxf(m, __shfl_xor(m, 4));  // the row's largest channel log-gate
                if ((lane & 7) == 0 && in[rg]) {
                    gv += m;
                    const float bv = a.beta[(start + c * CH + r0 + 8 * rg) * a.H + head];
                    bad_row = bad_row || !(bv >= 0.f && bv <= 1.9f);
                }
            }
        } else {
            const int64_t c = ctop - wv;
            const int64_t r = start + c * CH + lane;
            if (c >= cp && r < end) {
                gv = a.g[r * a.H + head];
                const float bv = a.beta[r * a.H + head];
                bad_row = !(bv >= 0.f && bv <= 1.9f);
            }
        }
        const float sum = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wave_scan(gv)), 63));
        const bool bad = __ballot(bad_row) != 0;
        if (lane == 0) {
            part[wv] = sum;
            bad_beta[wv] = bad;
        }
        __syncthreads();
        if (tid == 0) {
#pragma unroll
            for (int jj = 0; jj < RC; ++jj) {
                const int64_t cc = ctop - jj;
                const float csum = KDA ? part[2 * jj] + part[2 * jj + 1] : part[jj];
                const int cbad = KDA ? bad_beta[2 * jj] | bad_beta[2 * jj + 1] : bad_beta[jj];
                if (!done && cc >= cp) {
                    if (cbad) {
                        done = -1;
                    } else {
                        acc += csum;
                        ++w;
                        if (acc < kWarmLogBound)
                            done = 1;
                    }
                }
            }
            bad_beta[0] = done;  // broadcast
        }
        __syncthreads();
        done = bad_beta[0];
        __syncthreads();
    }
    if (tid == 0)
        a.seg_ws[a.lay.warm_chunks(b, s, head)] = done == 1 ? (float)w : 0.f;
}

template <typename T, typename TOUT, int K>
__global__ void __launch_bounds__(FRONT_THREADS) front_kernel(const FrontArgs a)
{
    if (debug_stop(a.dbg))
        return;
    static_assert(FRONT_THREADS == 256, "the warm-start plan runs on 256 threads");
    if (blockIdx.y >= (a.N + a.tile_rows - 1) / a.tile_rows) {  // extra rows: warm plan
        const int64_t i = (int64_t)(blockIdx.y - (a.N + a.tile_rows - 1) / a.tile_rows) *
                              gridDim.x + blockIdx.x;
        if (i < a.warm_groups)
            warm_plan_block(a.warm, (int)i);
        return;
    }
    constexpr int W = K - 1;
    const int cd = 2 * a.Hqk * a.dk + a.H * a.dv;
    const int cg = blockIdx.x * FRONT_THREADS + threadIdx.x;  // channel group
    const int c0 = cg * FRONT_CPT;                              // first packed channel
    const bool active = c0 < cd;
    const int qk = a.Hqk * a.dk;
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

    const int64_t t0 = (int64_t)blockIdx.y * a.tile_rows;
    const int64_t t1 = min(t0 + a.tile_rows, a.N);
    if (t0 >= t1)
        return;  // uniform over the block

    // win[j] = extended position (p_t - W + j) of the next token t, where the extended
    // sequence of stream b is [carried window (W) | rows start_b .. end_b-1].
    float win[W > 0 ? W : 1][FRONT_CPT];
    auto init_window = [&](int64_t t, int b, int64_t sb) {
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

    TOUT *y = (TOUT *)a.y;
    constexpr int RB = 4;  // rows per batch; the next batch is in flight while one is used
    // Branch-free raw loads, so that a batch's loads are in flight together and nothing
    // waits on them until the batch is used: rows past the range repeat its last row and
    // channels past cd read channel group 0; neither is used.
    constexpr int NU = 8 * (int)sizeof(T) / 16;  // 16-byte pieces per 8 channels
    uint4 xn[RB][NU];
    const T *lsrc = active ? src : (const T *)a.q;
    auto load_batch = [&](int64_t tb, int64_t r1) {
#pragma unroll
        for (int u = 0; u < RB; ++u)
#pragma unroll
            for (int h = 0; h < NU; ++h)
                xn[u][h] = load_stream16(lsrc + min(tb + u, r1 - 1) * a.ld +
                                         h * (16 / (int)sizeof(T)));
    };
    // The tile's rows, one stream at a time (a tile lies in one stream unless streams are
    // shorter than a tile).
    int b = find_stream(a.st, t0);
    for (int64_t r0 = t0; r0 < t1;) {
        int64_t sb, eb;
        stream_bounds(a.st, b, sb, eb);
        if (eb <= r0) {  // an empty stream, or the end of the previous one
            ++b;
            continue;
        }
        const int64_t r1 = min(t1, eb);
        init_window(r0, b, sb);
        load_batch(r0, r1);
        for (int64_t tb = r0; tb < r1; tb += RB) {
            float xs[RB][8];
#pragma unroll
            for (int u = 0; u < RB; ++u)
#pragma unroll
                for (int h = 0; h < NU; ++h) {
                    float v[8 / NU];
                    unpack((const T *)nullptr, xn[u][h], v);
#pragma unroll
                    for (int i = 0; i < 8 / NU; ++i)
                        xs[u][h * (8 / NU) + i] = v[i];
                }
            if (tb + RB < r1)
                load_batch(tb + RB, r1);
#pragma unroll
            for (int u = 0; u < RB; ++u) {
                const int64_t t = tb + u;
                if (t >= r1)
                    break;  // uniform over the block
                float z[FRONT_CPT];
#pragma unroll
                for (int i = 0; i < FRONT_CPT; ++i) {
                    float acc = w[K - 1][i] * xs[u][i];
#pragma unroll
                    for (int j = 0; j < W; ++j)
                        acc += w[j][i] * win[j][i];
                    z[i] = acc * __builtin_amdgcn_rcpf(1.f + __expf(-acc));  // SiLU
                }
#pragma unroll
                for (int j = 0; j + 1 < W; ++j)
#pragma unroll
                    for (int i = 0; i < FRONT_CPT; ++i)
                        win[j][i] = win[j + 1][i];
                if (W > 0) {
#pragma unroll
                    for (int i = 0; i < FRONT_CPT; ++i)
                        win[W > 0 ? W - 1 : 0][i] = xs[u][i];
                }
                if (a.do_l2) {  // uniform; q and k heads are whole aligned lane groups
                    float ss = 0.f;
#pragma unroll
                    for (int i = 0; i < FRONT_CPT; ++i)
                        ss += z[i] * z[i];
                    if (lanes_per_head == 16)
                        ss = group_sum<16>(ss);
                    else if (lanes_per_head == 8)
                        ss = group_sum<8>(ss);
                    else
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
        r0 = r1;
        ++b;
    }
}

// New carried window of every stream: the last K-1 entries of [old window | rows], one
// item per (stream, channel); after every reader of the old window.
template <typename T, int K>
__device__ __forceinline__ void conv_window_update(const FrontArgs &a, int64_t idx)
{
    constexpr int W = K - 1;
    const int cd = 2 * a.Hqk * a.dk + a.H * a.dv;
    if (idx >= (int64_t)a.st.B * cd)
        return;
    const int b = (int)(idx / cd), c = (int)(idx - (int64_t)b * cd);
    int64_t sb, eb;
    stream_bounds(a.st, b, sb, eb);
    const int64_t len = eb - sb;
    if (len <= 0)
        return;
    T *cs = a.conv_state_ptrs ? (T *)a.conv_state_ptrs[b] : (T *)a.conv_state;
    const int qk = a.Hqk * a.dk;
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

// The window update for item idx (stream-major channels) of a call of element type dtype
// (1: bf16, 0: fp32) and a.K taps, for launches that carry it in extra workgroups.
__device__ __forceinline__ void conv_window_item(const FrontArgs &a, int dtype, int64_t idx)
{
    if (dtype) {
        switch (a.K) {
        case 2: conv_window_update<bf16, 2>(a, idx); break;
        case 3: conv_window_update<bf16, 3>(a, idx); break;
        case 4: conv_window_update<bf16, 4>(a, idx); break;
        }
    } else {
        switch (a.K) {
        case 2: conv_window_update<float, 2>(a, idx); break;
        case 3: conv_window_update<float, 3>(a, idx); break;
        case 4: conv_window_update<float, 4>(a, idx); break;
        }
    }
}

template <typename T, typename TOUT, int K>
hipError_t launch_front_tk(const FrontArgs &a, hipStream_t s)
{
    const int cd = 2 * a.Hqk * a.dk + a.H * a.dv;
    const int groups = cd / FRONT_CPT;
    if (a.tile_rows < FRONT_ROWS || a.tile_rows % 4)
        return hipErrorInvalidValue;
    const unsigned gx = (unsigned)((groups + FRONT_THREADS - 1) / FRONT_THREADS);
    dim3 grid(gx, (unsigned)((a.N + a.tile_rows - 1) / a.tile_rows +
                             (a.warm_groups + gx - 1) / gx));
    hipLaunchKernelGGL((front_kernel<T, TOUT, K>), grid, dim3(FRONT_THREADS), 0, s, a);
    return hipGetLastError();
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

// float32 rows (bf16 rows run the front end inside the chunk kernel)
hipError_t launch_front(int dtype, const FrontArgs &a, hipStream_t s)
{
    return dtype ? hipErrorInvalidValue : launch_front_t<float, float>(a, s);
}

// ------------------------------------------------------------------------------------
// output gate: y = o / sqrt(mean(o^2) + eps) * w * silu(z) over the dv values of a row

// 4 adjacent z values: one 8-byte load (bf16) or one 16-byte load (float)
template <typename TZ>
struct Z4;
template <>
struct Z4<bf16> {
    typedef uint2 raw;
    __device__ static raw load(const bf16 *p) { return *reinterpret_cast<const uint2 *>(p); }
    __device__ static raw zero() { return make_uint2(0, 0); }
    __device__ static float4 get(const raw &u)
    {
        return float4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                      __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
    }
};
template <>
struct Z4<float> {
    typedef float4 raw;
    __device__ static raw load(const float *p) { return *reinterpret_cast<const float4 *>(p); }
    __device__ static raw zero() { return float4{0.f, 0.f, 0.f, 0.f}; }
    __device__ static float4 get(const raw &u) { return u; }
};

constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;
constexpr float kExpCap = 80.f * kLog2e;  // largest exponent of a decay factor, log2 units

__device__ __forceinline__ float silu(float z)
{
    return z * __builtin_amdgcn_rcpf(1.f + __expf(-z));
}

// o (4 values of a row) times inv_rms * w * silu(z)
__device__ __forceinline__ float4 gate4(float4 o, float inv_rms, float4 w, float4 z)
{
    return float4{o.x * inv_rms * w.x * silu(z.x), o.y * inv_rms * w.y * silu(z.y),
                  o.z * inv_rms * w.z * silu(z.z), o.w * inv_rms * w.w * silu(z.w)};
}

// Sum over aligned groups of N lanes (N a power of two <= 64).
template <int N>
__device__ __forceinline__ float lane_group_sum(float x)
{
#pragma unroll
    for (int m = 1; m < N; m <<= 1)
        x += __shfl_xor(x, m);
    return x;
}

// Separate pass for instances that cannot stage whole o rows: rows [0, N) x H heads of o
// gated in place. One group of dv/4 lanes (16, 32 or a wave) per (row, head), 4 values
// per lane.
template <typename TZ, int DV>
__global__ void __launch_bounds__(256) gate_kernel(const GateArgs a)
{
    if (debug_stop(a.dbg))
        return;
    constexpr int LPI = DV / 4, IPB = 256 / LPI;  // lanes per item, items per block
    const int64_t item = (int64_t)blockIdx.x * IPB + threadIdx.x / LPI;
    const int j = threadIdx.x % LPI;
    const bool live = item < a.N * a.H;
    const int64_t row = live ? item / a.H : 0, head = live ? item - row * a.H : 0;
    float *op = a.o + (row * a.H + head) * DV + 4 * j;
    float4 o = live ? *reinterpret_cast<const float4 *>(op) : float4{0.f, 0.f, 0.f, 0.f};
    const typename Z4<TZ>::raw z =
        live ? Z4<TZ>::load((const TZ *)a.z + row * a.ld_z + head * DV + 4 * j) : Z4<TZ>::zero();
    const float4 w = *reinterpret_cast<const float4 *>(a.w + 4 * j);
    const float ss = lane_group_sum<LPI>(o.x * o.x + o.y * o.y + o.z * o.z + o.w * o.w);
    o = gate4(o, rsqrtf(ss * (1.f / DV) + a.eps), w, Z4<TZ>::get(z));
    if (live)
        *reinterpret_cast<float4 *>(op) = o;
}

hipError_t launch_gate(int dtype, const GateArgs &a, hipStream_t s)
{
    const int64_t items = a.N * a.H;
    if (a.dv == 128) {
        const unsigned g = (unsigned)((items + 7) / 8);
        if (dtype)
            hipLaunchKernelGGL((gate_kernel<bf16, 128>), dim3(g), dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((gate_kernel<float, 128>), dim3(g), dim3(256), 0, s, a);
    } else if (a.dv == 64) {
        const unsigned g = (unsigned)((items + 15) / 16);
        if (dtype)
            hipLaunchKernelGGL((gate_kernel<bf16, 64>), dim3(g), dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((gate_kernel<float, 64>), dim3(g), dim3(256), 0, s, a);
    } else if (a.dv == 256) {
        const unsigned g = (unsigned)((items + 3) / 4);
        if (dtype)
            hipLaunchKernelGGL((gate_kernel<bf16, 256>), dim3(g), dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((gate_kernel<float, 256>), dim3(g), dim3(256), 0, s, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------
// fused chunk kernel


template <typename T, int DK, int DV, int NW, int NCB, bool KDA, bool GATE = false,
          bool FRONT = false, int CHK = 64>
struct ChunkCfg {
    static constexpr int CH = CHK;  // rows per chunk (64, or 32 without the fused front end)
    static constexpr int NV = 16 * NW * NCB;  // dv columns per workgroup (16*NCB per wave)
    // fp16 operands: T = (I+M)^-1 and P are applied as fp16 hi + lo pairs, and the
    // right-hand operands of T X and P U too, which keeps those products at about fp32
    // accuracy; fp32 operands need no split
    static constexpr bool SPLIT = sizeof(T) == 2;
    // Row strides. 16-bit tiles: P and M operand tiles 2 dwords past a multiple of 32, so
    // a fragment read (16 rows at one 8-byte piece) and a D-layout store (4 rows 4 apart,
    // 8 dwords each) touch distinct banks; V 4 dwords past, so the D-layout element reads
    // of rows 4 apart fall in separate halves of the banks. Q and K are permuted instead
    // of padded (see QK). fp32 tiles: 8 dwords past.
    static constexpr int PAD = 32 / (int)sizeof(T);
    static constexpr int LDQ = QK<T, DK>::LD;                  // Qs, Ks: [64][LDQ]
    static constexpr int LDV = NV + (SPLIT ? 8 : PAD);         // Vs: [64][LDV]
    static constexpr int LDT = CH + (SPLIT ? 4 : PAD);         // P and M operand tiles
    static constexpr int LDF = CH + 4;    // Ms, Tf: [64][LDF] float
    static constexpr int LDG = DK + 4;    // per-channel gate: Gk [64][LDG] float
    static constexpr int SZ_Q = CH * LDQ * (int)sizeof(T);
    static constexpr int SZ_V = CH * LDV * (int)sizeof(T);
    static constexpr int SZ_P = CH * LDT * (int)sizeof(T);
    static constexpr int SZ_F = CH * LDF * 4;
    static constexpr int SZ_MS = SZ_F > SZ_Q ? SZ_F : SZ_Q;  // the KDA gated K^T tile reuses it
    // Front end fused into the load stage (bf16 raw rows; conv + SiLU + L2 per chunk):
    // k is stored as fp16 hi + lo tiles and, with the scalar gate, q too; v is never a
    // tile: the raw v rows of the chunk, with the KC - 1 rows before it, sit in a raw
    // region from which each lane convolves the values of its own D-layout rows in fp32.
    // The raw q|k rows of the next chunk land by LDS-DMA on tiles that are dead from the
    // end of the chunk's last read of q and k until the next load stage (scalar gate: the
    // two Q tiles and the inversion scratch, read up to the preparation; per-key-channel
    // gate: the Q and K tiles, whose products with h are taken right after the gates'
    // rescale), and the raw v rows on their own region.
    // The per-key-channel gate keeps k as an fp16 hi + lo pair in every fp16 instance: the
    // rescaled operands (the gate factors of M and P, K e^G, K e^(G_C - G)) are formed from
    // k in about fp32, and K e^(G_C - G), which builds the state, is itself a hi + lo pair
    // (the lo half over the K lo tile once the rescale has read it).
    static constexpr bool KLO = FRONT || (KDA && SPLIT);  // K lo tile
    static constexpr bool QLO = FRONT && !KDA;            // Q lo tile
    static constexpr bool XSCR = FRONT && !KDA;           // separate inversion scratch
    static constexpr int KC = 4;                 // conv taps of the fused front end
    static constexpr int RR = CH + KC - 1;       // raw rows per chunk
    static constexpr int SZ_QF = QLO ? 2 * SZ_Q : SZ_Q;  // Q (hi, lo)
    static constexpr int LDX = 20;               // row stride of the 16x16 inversion scratch
    static constexpr int SZ_X = 4 * 16 * LDX * 4;
    static constexpr int RQ = DK * 2;            // bytes per raw q (or k) row
    static constexpr int RQK = 2 * RQ;           // bytes per raw q and k row
    // raw q rows [RR][DK], then raw k rows [RR][DK] (bf16), from OFF_Q
    __host__ __device__ static constexpr int raw_qk(int tensor, int row)
    {
        return (tensor * RR + row) * RQ;
    }
    // raw v rows in blocks of 4 (one LDS-DMA instruction each), 32 bytes of padding after
    // each block: the u16 reads of D-layout rows 4 apart (one block apart) then fall 8
    // banks apart
    static constexpr int RVR = NV * 2;            // bytes per raw v row
    static constexpr int RVBLK = 4 * RVR + 32;    // bytes per block of 4 rows
    __host__ __device__ static constexpr int raw_v(int row)
    {
        return (row >> 2) * RVBLK + (row & 3) * RVR;
    }
    static constexpr int SZ_RV = (RR + 3) / 4 * RVBLK;
    static constexpr int OFF_Q = 0;
    static constexpr int OFF_QL = SZ_Q;               // Q lo
    static constexpr int OFF_X = SZ_QF;               // inversion scratch (scalar-gate fusion)
    static constexpr int OFF_K = SZ_QF + (XSCR ? SZ_X : 0);
    static constexpr int OFF_KL = OFF_K + SZ_Q;      // K lo
    static constexpr int OFF_V = OFF_KL + (KLO ? SZ_Q : 0);      // V tile, or the raw v rows
    static constexpr int OFF_P = OFF_V + (FRONT ? SZ_RV : SZ_V);  // P (hi)
    static constexpr int OFF_PL = OFF_P + SZ_P;                   // P (lo)
    static constexpr int OFF_MT = OFF_PL + (SPLIT ? SZ_P : 0);    // M_IJ (J<I), T_II
    // diagonal blocks of M, fp32; per-key-channel gate: K e^(G_C - G) (hi) after the rescale
    static constexpr int OFF_M = OFF_MT + SZ_P;
    static constexpr int OFF_GK = OFF_M + (XSCR ? 0 : SZ_MS);  // per-channel cumulative log-gates
    // Gamma[64], beta[64], a = e^Gamma [64], a_C / a [64]
    static constexpr int OFF_G = OFF_GK + (KDA ? CH * LDG * 4 : 0);
    // o rows (fp32). Fused front end: rows 4 apart (the lane groups of a D-layout write)
    // 16 banks apart
    static constexpr int LDO = NV + (FRONT ? 4 : 16);
    // + the running log decay bound of a transition job (one float, padded to 16 bytes;
    // scalar gate without the fused output gate only); per-key-channel gate: + e^(G_C) per
    // channel
    static constexpr bool STOP = !KDA && !GATE;
    static constexpr int OFF_O = OFF_G + 4 * CH * 4 + (STOP ? 16 : 0) + (KDA ? DK * 4 : 0);
    // o is staged in LDS when it fits (not with the per-channel gate tile at 128 columns)
    static constexpr bool STAGE_O = OFF_O + CH * LDO * 4 <= 160 * 1024;
    // fused front end: the q and k conv taps of this head, [2][KC][DK] float
    static constexpr int OFF_CW = OFF_O + (STAGE_O ? CH * LDO * 4 : 0);
    // output gate: the z rows of a chunk (the caller's element type, as wide as T) and the
    // norm weights of the NV columns
    static constexpr int OFF_Z = OFF_CW + (FRONT ? 2 * KC * DK * 4 : 0);
    static constexpr int ZROW = NV * (int)sizeof(T);
    // fused front end with the output gate: no LDS left for a z tile; each thread holds
    // the z values of its o flush in registers instead
    static constexpr bool ZREG = GATE && FRONT;
    static constexpr int OFF_W = OFF_Z + (GATE && !ZREG ? CH * ZROW : 0);
    static constexpr int BYTES = OFF_W + (GATE ? NV * 4 : 0);
    // the raw q|k rows land on the dead tiles at the start of the layout
    static_assert(!FRONT || RR * RQK <= (KDA ? OFF_KL : OFF_K), "raw q|k rows fit");
    static_assert(!FRONT || (SPLIT && !(GATE && KDA) && NCB == 1 && (STAGE_O || KDA)),
                  "fused front end: fp16 operands, one column block per wave, the output "
                  "gate with the scalar gate only");
};

// Operand fragment that runs down the columns of a row-major LDS tile X[k][n]:
// lane (g, c) gets X[k0 + kappa(g, i)][n0 + c], i = 0..7, with kappa as in ld_frag.
// fp16 tiles use the gfx950 LDS transpose read: within each 16-lane group, output lane j,
// element i comes from source lane 4i + j/4, element j%4; so source lane s of group g
// addresses row k0 + 4g + s/4, columns n0 + 4(s%4) .. +3, and the second read adds 16 rows.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f16x8 ld_frag_t(const f16 *X, int ld, int k0, int n0, int lane)
{
    const int g = lane >> 4, s = lane & 15;
    const f16 *p0 = X + (k0 + 4 * g + (s >> 2)) * ld + n0 + 4 * (s & 3);
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p0);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p0 + 16 * ld));
    const f16x4 flo = __builtin_bit_cast(f16x4, lo), fhi = __builtin_bit_cast(f16x4, hi);
    return __builtin_shufflevector(flo, fhi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f32x8 ld_frag_t(const float *X, int ld, int k0, int n0, int lane)
{
    const int g = lane >> 4, c = lane & 15;
    const float *p = X + (k0 + 4 * g) * ld + n0 + c;
    f32x8 f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[i] = p[i * ld];
        f[4 + i] = p[(16 + i) * ld];
    }
    return f;
}

// ld_frag_t for a Q/K tile
template <int DK>
__device__ __forceinline__ f16x8 ld_frag_t_qk(const f16 *X, int k0, int n0, int lane)
{
    // k0 is a multiple of 16 and n0 of 16: the chunk permutation of row k0 + 4g + s/4 is g,
    // so the offset is k0 * LD + n0 plus a lane part, and the second read is 16 rows on
    using L = QK<f16, DK>;
    const int g = lane >> 4, s = lane & 15;
    const f16 *p = X + k0 * L::LD + n0 + (4 * g + (s >> 2)) * L::LD + ((s & 3) ^ g) * 4;
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + 16 * L::LD));
    const f16x4 flo = __builtin_bit_cast(f16x4, lo), fhi = __builtin_bit_cast(f16x4, hi);
    return __builtin_shufflevector(flo, fhi, 0, 1, 2, 3, 4, 5, 6, 7);
}
template <int DK>
__device__ __forceinline__ f32x8 ld_frag_t_qk(const float *X, int k0, int n0, int lane)
{
    return ld_frag_t(X, QK<float, DK>::LD, k0, n0, lane);
}


// fp32 -> fp16 hi + lo: hi = x rounded to fp16, lo = (x - hi) rounded to fp16. hi is one
// packed conversion per pair; x - hi comes from v_fma_mix_f32, which reads x as fp32 and hi
// straight from its fp16 half (the difference is exact in fp32), and the lo pair is one more
// packed conversion: the same bits as converting hi back, subtracting and converting again,
// in 2 instructions per element instead of 4. (Full-register results only: an instruction
// that writes half a register leaves a forwarding hazard the compiler cannot see in asm.)
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split2(float x0, float x1, uint32_t &hi, uint32_t &lo)
{
    hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){x0, x1}, f16x2));
    float d0, d1;
    asm("v_fma_mix_f32 %0, %2, 1.0, -%4 op_sel_hi:[0,0,1]\n\t"
        "v_fma_mix_f32 %1, %3, 1.0, -%4 op_sel:[0,0,1] op_sel_hi:[0,0,1]"
        : "=&v"(d0), "=&v"(d1)
        : "v"(x0), "v"(x1), "v"(hi));
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){d0, d1}, f16x2));
}
__device__ __forceinline__ void split4(const f32x4 &x, f16x4 &hi, f16x4 &lo)
{
    uint32_t h0, l0, h1, l1;
    split2(x[0], x[1], h0, l0);
    split2(x[2], x[3], h1, l1);
    hi = __builtin_bit_cast(f16x4, (u32x2){h0, h1});
    lo = __builtin_bit_cast(f16x4, (u32x2){l0, l1});
}

// Widening with v_fma_mix_f32 (fp16 sources read straight from their half of a register,
// one rounding to fp32, full-register results): the two fp32 values hi + lo of a packed
// pair of fp16 hi halves and lo halves (exact: hi + lo needs at most 24 bits), and a
// packed fp16 element times an fp32 factor. Each is one instruction per element where the
// separate conversions and the add or multiply take three or two, with the same bits.
__device__ __forceinline__ void widen_hl2(uint32_t hi, uint32_t lo, float &x0, float &x1)
{
    asm("v_fma_mix_f32 %0, %2, 1.0, %3 op_sel_hi:[1,0,1]\n\t"
        "v_fma_mix_f32 %1, %2, 1.0, %3 op_sel:[1,0,1] op_sel_hi:[1,0,1]"
        : "=&v"(x0), "=&v"(x1)
        : "v"(hi), "v"(lo));
}
__device__ __forceinline__ void widen_mul2(uint32_t h2, float f0, float f1, float &x0, float &x1)
{
    asm("v_fma_mix_f32 %0, %2, %3, 0 op_sel_hi:[1,0,0]\n\t"
        "v_fma_mix_f32 %1, %2, %4, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
        : "=&v"(x0), "=&v"(x1)
        : "v"(h2), "v"(f0), "v"(f1));
}
// the same over 4 elements (8-byte vectors of fp16)
__device__ __forceinline__ f32x4 widen_hl4(const f16x4 &hi, const f16x4 &lo)
{
    const u32x2 h = __builtin_bit_cast(u32x2, hi), l = __builtin_bit_cast(u32x2, lo);
    float x0, x1, x2, x3;
    widen_hl2(h[0], l[0], x0, x1);
    widen_hl2(h[1], l[1], x2, x3);
    return f32x4{x0, x1, x2, x3};
}
__device__ __forceinline__ f32x4 widen_mul4(const f16x4 &v, const f32x4 &f)
{
    const u32x2 h = __builtin_bit_cast(u32x2, v);
    float x0, x1, x2, x3;
    widen_mul2(h[0], f[0], f[1], x0, x1);
    widen_mul2(h[1], f[2], f[3], x2, x3);
    return f32x4{x0, x1, x2, x3};
}

// d += A B for 16x16 blocks with a 16-deep contraction in about fp32 accuracy:
// a[i] = A[c][4g+i], b[i] = B[4g+i][c] (lane = 16g + c); d in the same D layout.
template <bool SPLIT>
__device__ __forceinline__ void mm16(f32x4 &d, const f32x4 &a, const f32x4 &b)
{
    if constexpr (SPLIT) {
        f16x4 ah, al, bh, bl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ah[i] = (f16)a[i];
            al[i] = (f16)(a[i] - (float)ah[i]);
            bh[i] = (f16)b[i];
            bl[i] = (f16)(b[i] - (float)bh[i]);
        }
        d = __builtin_amdgcn_mfma_f32_16x16x16f16(ah, bh, d, 0, 0, 0);
        d = __builtin_amdgcn_mfma_f32_16x16x16f16(ah, bl, d, 0, 0, 0);
        d = __builtin_amdgcn_mfma_f32_16x16x16f16(al, bh, d, 0, 0, 0);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            d = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], d, 0, 0, 0);
    }
}

// A-operand fragment of 16x16 block (I, K) of a row-major fp32 tile: a[i] = X[16I+c][16K+4g+i]
__device__ __forceinline__ f32x4 blk_a(const float *X, int ld, int I, int K, int lane)
{
    return *reinterpret_cast<const f32x4 *>(X + (16 * I + (lane & 15)) * ld + 16 * K +
                                            4 * (lane >> 4));
}
// B-operand fragment of block (K, J): b[i] = X[16K+4g+i][16J+c]
__device__ __forceinline__ f32x4 blk_b(const float *X, int ld, int K, int J, int lane)
{
    const float *p = X + (16 * K + 4 * (lane >> 4)) * ld + 16 * J + (lane & 15);
    return f32x4{p[0], p[ld], p[2 * ld], p[3 * ld]};
}

// A-operand fragment of 16x16 block (I, J) of a row-major operand tile (16-deep products):
// a[i] = X[16I+c][16J+4g+i], returned as fp32 values
__device__ __forceinline__ f32x4 blk_a16(const f16 *X, int ld, int I, int J, int lane)
{
    const f16x4 v = *reinterpret_cast<const f16x4 *>(X + (16 * I + (lane & 15)) * ld + 16 * J +
                                                     4 * (lane >> 4));
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ f32x4 blk_a16(const float *X, int ld, int I, int J, int lane)
{
    return blk_a(X, ld, I, J, lane);
}

// d += A B for 16x16 blocks (16-deep): A block (I, J) of a stored operand tile, B an fp32
// D-layout value given as an fp16 hi + lo pair (or split here). A is a single fp16 operand:
// its rounding adds no measurable error to o or h (the M blocks below the diagonal and the
// inverted diagonal blocks enter U only through products with the split right-hand side),
// while rounding B does. fp32 tiles use fp32 MFMA directly.
// d += A (B_hi + B_lo) for a 16x16 A fragment already in registers (a[i] = A[c][4g+i]), as
// one 32-deep product of [A A] and [B_hi; B_lo] (the 16-deep product takes as long as the
// 32-deep one on gfx950)
__device__ __forceinline__ void mm16_frag(f32x4 &d, const f16x4 &a, const f16x4 &bh,
                                          const f16x4 &bl)
{
    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_shufflevector(a, a, 0, 1, 2, 3, 0, 1, 2, 3),
                                               __builtin_shufflevector(bh, bl, 0, 1, 2, 3, 4, 5, 6, 7),
                                               d, 0, 0, 0);
}
__device__ __forceinline__ void mm16_pre(f32x4 &d, const f16 *X, int ld, int I, int J,
                                         const f16x4 &bh, const f16x4 &bl, int lane)
{
    const f16x4 a = *reinterpret_cast<const f16x4 *>(X + (16 * I + (lane & 15)) * ld + 16 * J +
                                                    4 * (lane >> 4));
    // A B_hi + A B_lo as one 32-deep product of [A A] and [B_hi; B_lo] (the 16-deep product
    // takes as long as the 32-deep one on gfx950)
    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_shufflevector(a, a, 0, 1, 2, 3, 0, 1, 2, 3),
                                               __builtin_shufflevector(bh, bl, 0, 1, 2, 3, 4, 5, 6, 7),
                                               d, 0, 0, 0);
}
__device__ __forceinline__ void mm16_pre(f32x4 &d, const f16 *X, int ld, int I, int J,
                                         const f32x4 &b, int lane)
{
    f16x4 bh, bl;
    split4(b, bh, bl);
    mm16_pre(d, X, ld, I, J, bh, bl, lane);
}
__device__ __forceinline__ void mm16_pre(f32x4 &d, const float *X, int ld, int I, int J,
                                         const f32x4 &b, int lane)
{
    const f32x4 a = blk_a(X, ld, I, J, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        d = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], d, 0, 0, 0);
}

// fp32 D-layout value -> fp16 hi + lo

// hi + lo operand pair of the B operand built from two D-layout accumulators
template <typename T>
__device__ __forceinline__ void pack_split(const f32x4 &d0, const f32x4 &d1,
                                           typename Tr<T>::frag &hi, typename Tr<T>::frag &lo)
{
    if constexpr (sizeof(T) == 2) {
        f16x4 h0, l0, h1, l1;
        split4(d0, h0, l0);
        split4(d1, h1, l1);
        hi = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
        lo = __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7);
    } else {
        hi = pack<T>(d0, d1);
    }
}

// Task j of a wave in the preparation stage, or -1: block b (numbered row by row over the
// 10 lower 16x16 blocks of a chunk) + 16 * part, part 0 = both products of the block,
// 1 = M only, 2 = P only. Diagonal blocks (0, 2, 5, 9) come first on waves 0-3, which
// also invert them; two blocks below the diagonal are split between two waves so that
// the waves without an inversion carry about as much as the ones with.
template <int NW, int NB = 4>
__device__ __forceinline__ int block_task(int wave, int j)
{
    if constexpr (NB == 2) {  // 32-row chunks: blocks 0 (0, 0), 1 (1, 0), 2 (1, 1)
        constexpr int tab[8] = {0, 2, 1, -1, -1, -1, -1, -1};
        return j == 0 ? tab[wave] : -1;
    } else if constexpr (NW == 8) {
        constexpr int tab[8][2] = {{0, -1}, {2, -1}, {5, -1},      {9, -1},
                                   {1, 22}, {3, 23}, {4, 38}, {8, 39}};
        return tab[wave][j];
    } else {
        constexpr int tab[4][3] = {{0, 1, 19}, {2, 4, 22}, {5, 7, 35}, {9, 8, 38}};
        return tab[wave][j];
    }
}

// ------------------------------------------------------------------------------------
// segmented scan: chain the segment maps, h(b, s+1) = A(b, s) h(b, s) + B(b, s)

// Waits until the n <= 64 flags f[0..n) are nonzero (lane l polls f[l], at most polls
// times, ChunkArgs::wait_polls); loads after it see what the workgroups that set them wrote
// before setting them. Called by whole waves. Every flag is set by a workgroup that
// precedes its waiters in the grid, and workgroups dispatch in grid order, so the flags are
// set while a waiter polls; the bound keeps every wave finite regardless. Returns whether
// every flag was seen set.
__device__ __forceinline__ bool wait_flags(const int *f, int n, int polls)
{
    const int lane = (int)(threadIdx.x & 63);
    bool ok = lane >= n;
    for (int it = 0; it < polls; ++it) {
        if (!ok)
            ok = __hip_atomic_load(f + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
        if (__ballot(!ok) == 0)
            break;
        __builtin_amdgcn_s_sleep(8);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return __ballot(!ok) == 0;
}

// The chain of one (stream, head, 16 state columns), blk = column block * B*H + (stream,
// head), by a workgroup of NWV waves at the front of the second launch. The 16 columns of
// h(b, s) sit in LDS; wave w computes row blocks w, w + NWV, ... of the next state with fp32
// MFMA (one block per wave at dk = 128 with 8 waves: the chain is latency-bound). The A and
// B blocks a wave needs for step s+1 are loaded into registers while step s computes, so
// each step waits on memory once at most. When the last step is stored, the column block's
// flag (reset by job 0 of the first launch) releases the second launch's jobs of segments
// 2..S-1, which wait for it before they read their start states.
// A (stream, head) in warm mode has no chain: its last segment ran in the first launch,
// beside the job that read the stream's initial state, so it left its end state in slot
// H(b, S-1) (and, with the front end fused and windows not shared, the new windows in
// win_ws); the workgroup copies its share to the caller's buffers (with direct_final that
// job waited for the read and wrote them itself, unless its wait gave up: then it took the
// slot and set the fallback flag of its dv slice, and the copy happens here).
template <int DK, int NWV, int NV>
__device__ __forceinline__ void chain_block(const ChunkArgs &a, const SegLayout &lay, int blk,
                                            unsigned char *lds)
{
    constexpr int NRB = DK / 16, RBW = (NRB + NWV - 1) / NWV;  // row blocks, per wave
    float(*hsm)[20] = reinterpret_cast<float(*)[20]>(lds);     // rows 4 apart 16 banks apart
    float *zf = reinterpret_cast<float *>(lds + DK * 20 * sizeof(float));
    // Workgroups go to the 8 XCDs round-robin by index: with the column block as the slow
    // index, the column blocks of one (stream, head) share an XCD (B*H a multiple of 8),
    // so that XCD's L2 serves that head's A to all of them.
    const int BH = lay.B * a.H;
    const int cbk = blk / BH, bh = blk - cbk * BH;
    const int b = bh / a.H, head = bh - b * a.H;
    const int64_t hoff = (int64_t)head * DK * DK;
    float *state = a.h_ptrs ? a.h_ptrs[b] : a.h;
    if (a.warm && warm_head(warm_lane_count(a.seg_ws, lay, b, head))) {
        if (a.direct_final &&
            reinterpret_cast<const int *>(a.seg_ws + lay.flags(b, head))
                    [SegLayout::kFlagFallback + 16 * cbk / NV] == 0)
            return;
        const float *src = a.seg_ws + lay.h(b, lay.S - 1) + hoff;
        for (int idx = threadIdx.x; idx < DK * 16; idx += NWV * 64) {
            const int64_t e = (int64_t)(idx >> 4) * DK + 16 * cbk + (idx & 15);
            state[hoff + e] = src[e];
        }
        if (a.win_ws && !a.win_shared) {  // bf16 windows [cd][W]; this head's q, k, v channels
            const int W = a.conv_k - 1, hq = head / a.qk_group, Hqk = a.H / a.qk_group;
            const int nch = 2 * DK + DK, per = (nch * W + DK / 16 - 1) / (DK / 16);
            const uint16_t *ws = (const uint16_t *)a.win_ws + (int64_t)b * a.cd * W;
            uint16_t *cw = (uint16_t *)(a.conv_state_ptrs ? a.conv_state_ptrs[b] : a.conv_state);
            for (int e = cbk * per + (int)threadIdx.x; e < min((cbk + 1) * per, nch * W);
                 e += NWV * 64) {
                const int ch = e / W, j = e - W * ch;
                const int gc = ch < 2 * DK ? (ch >= DK ? Hqk * DK : 0) + hq * DK + ch % DK
                                           : 2 * Hqk * DK + head * DK + ch - 2 * DK;
                cw[(int64_t)gc * W + j] = ws[(int64_t)gc * W + j];
            }
        }
        return;  // the second launch's jobs of a warm (stream, head) return without waiting
    }
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = lane >> 4, c16 = lane & 15;
    const int col0 = 16 * cbk;
    const int S = lay.S;
    const float *h1 = a.seg_ws + lay.h(b, 1) + hoff;
    for (int idx = tid; idx < DK * 16; idx += NWV * 64)
        hsm[idx >> 4][idx & 15] = h1[(int64_t)(idx >> 4) * DK + col0 + (idx & 15)];
    // the zero-transition flags of every step, read once (visible after the first barrier)
    if (tid < S - 2)
        zf[tid] = a.seg_ws[lay.zero_flag(b, tid + 1, head)];

    // A step whose transition job found A(b, s) zero is h(b, s+1) = B(b, s): no A to load, no
    // product, and no wait for h(b, s) (the flag is the same for the whole workgroup).
    auto zero_at = [&](int s) { return zf[s - 1] != 0.f; };
    // A blocks and B rows of the next two steps (ring of 2), so a step's loads have two
    // steps' time to arrive
    f32x4 av[2][RBW][NRB], bv[2][RBW];
    auto load = [&](int s, int slot, bool flags_known) {
        const float *A = a.seg_ws + lay.as(b, s) + hoff;  // [dk][dk]
        const float *Bm = a.seg_ws + lay.bs(b, s) + hoff;
        const bool za = flags_known && zero_at(s);
#pragma unroll
        for (int j = 0; j < RBW; ++j) {
            const int rb = wave + NWV * j;
            if (rb < NRB) {
                if (!za) {
#pragma unroll
                    for (int kb = 0; kb < NRB; ++kb)
                        av[slot][j][kb] = blk_a(A, DK, rb, kb, lane);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    bv[slot][j][i] = Bm[(int64_t)(16 * rb + 4 * g4 + i) * DK + col0 + c16];
            }
        }
    };
    auto step = [&](int s, int slot) {
        const bool zs = zero_at(s);
        f32x4 acc[RBW];
#pragma unroll
        for (int j = 0; j < RBW; ++j) {
            const int rb = wave + NWV * j;
            acc[j] = bv[slot][j];
            if (rb < NRB && !zs) {
#pragma unroll
                for (int kb = 0; kb < NRB; ++kb) {
                    const float *hc = &hsm[16 * kb + 4 * g4][c16];
                    mm16<false>(acc[j], av[slot][j][kb], f32x4{hc[0], hc[20], hc[40], hc[60]});
                }
            }
        }
        if (s + 2 <= S - 2)
            load(s + 2, slot, true);
        if (!zs)
            __syncthreads();  // every wave has read h(b, s)
        float *Hn = a.seg_ws + lay.h(b, s + 1) + hoff;
#pragma unroll
        for (int j = 0; j < RBW; ++j) {
            const int rb = wave + NWV * j;
            if (rb < NRB) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * rb + 4 * g4 + i;
                    hsm[r][c16] = acc[j][i];
                    Hn[(int64_t)r * DK + col0 + c16] = acc[j][i];
                }
            }
        }
        // the next step reads h(b, s+1) from every wave's rows unless its transition is zero
        // (each wave writes the same rows in every step, so a zero step needs no wait)
        if (s + 1 <= S - 2 && !zero_at(s + 1))
            __syncthreads();
    };
    // the first two steps' blocks are requested before the flags are visible (A included)
    load(1, 0, false);
    if (S - 2 >= 2)
        load(2, 1, false);
    __syncthreads();  // h(b, 1) and the flags
    // the ring slot is a compile-time index: steps go in pairs
    for (int s = 1; s <= S - 2; s += 2) {
        step(s, 0);
        if (s + 1 <= S - 2)
            step(s + 1, 1);
    }
    // every wave's stores of the chain reach the agent-coherent level, then one flag
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (tid == 0)
        __hip_atomic_store(reinterpret_cast<int *>(a.seg_ws + lay.chain_done(b, head, cbk)), 1,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename TIN, typename T, int DK, int DV, int NW, int NCB, bool KDA, bool GATE,
          bool FRONT, int CHK = 64>
__global__ void __launch_bounds__(NW * 64)
    __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) chunk_kernel(const ChunkArgs a)
{
    static_assert(sizeof(TIN) == sizeof(T), "16-byte loads fill whole operand vectors");
    static_assert(NW == 4 || NW == 8, "one or two waves per SIMD");
    static_assert(!FRONT || std::is_same<TIN, bf16>::value, "fused front end: bf16 raw rows");
    // rows per chunk and 16-row blocks per chunk: 64 (4 blocks), or 32 (2 blocks) on the
    // register path without the output gate
    constexpr int CH = CHK, NB = CH / 16;
    static_assert(CH == 64 || (CH == 32 && !FRONT && !GATE), "chunk rows");
    using C = ChunkCfg<T, DK, DV, NW, NCB, KDA, GATE, FRONT, CHK>;
    // the output gate normalises whole o rows, which the staged o holds
    static_assert(!GATE || (C::STAGE_O && C::NV == DV), "output gate needs staged o rows");
    // z comes in the caller's element type (bf16 also when the operands are fp16)
    typedef typename std::conditional<sizeof(TIN) == 4, float, bf16>::type TZ;
    constexpr int NV = C::NV, LDQ = C::LDQ, LDV = C::LDV, LDT = C::LDT, LDF = C::LDF;
    constexpr int LDG = C::LDG, LDO = C::LDO;
    constexpr bool SPLIT = C::SPLIT;
    constexpr int VEC = Tr<T>::VEC;
    constexpr int NT = NW * 64;
    typedef typename Tr<T>::frag frag;
    // row -> lane maps of the 16-byte loads
    constexpr int LPR = DK / VEC, RPW = 64 / LPR, NQK = 2 * CH / (NW * RPW);
    constexpr int LPV = NV / VEC, RPV = 64 / LPV, NVV = CH / (NW * RPV);
    static_assert(NQK * NW * RPW == 2 * CH && NVV * NW * RPV == CH, "load map");
    // per-channel gate rows (fp32): 16-byte pieces per row and rows per wave pass
    constexpr int GPR = DK * 4 / 16, GRW = 64 / GPR, NGK = KDA ? CH / (NW * GRW) : 1;
    static_assert(!KDA || NGK * NW * GRW == CH, "gate load map");

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    if (debug_stop(a.dbg))
        return;

    const int tid0 = threadIdx.x, lane0 = tid0 & 63;
    const int wave0 = __builtin_amdgcn_readfirstlane(tid0 >> 6);

    if (blockIdx.x >= a.job_groups) {  // extra workgroups: the front end's new windows
        conv_window_item(a.window, a.window_dtype,
                         (int64_t)(blockIdx.x - a.job_groups) * NT + tid0);
        return;
    }
    int gid = blockIdx.x;
    if (a.chain_groups) {  // second launch of a segmented call: the chain's workgroups first
        if (gid < a.chain_groups) {
            if constexpr (DK == DV && (DK == 64 || DK == 128))
                chain_block<DK, NW, NV>(
                    a, SegLayout{(int64_t)a.H * DK * DV, a.st.B, a.nseg, a.H}, gid, smem);
            return;
        }
        gid -= a.chain_groups;
    }
    const int H = a.H;
    const int BH = a.st.B * H;
    constexpr int NS = DV / NV;  // dv slices
    const int jp = gid / (BH * NS), jr = gid - jp * (BH * NS);
    const int slice = jr / BH, bh = jr - slice * BH;
    const int bi = bh / H, head = bh - bi * H;
    const int b = a.order ? a.order[bi] : bi;  // varlen: longest streams dispatch first
    int64_t start, end;
    stream_bounds(a.st, b, start, end);
    const int64_t sbeg = start;  // the stream's first row
    float *state = (a.h_ptrs ? a.h_ptrs[b] : a.h);
    bool last_seg = true;    // this job's rows end the stream (fused front end: it writes the
    bool win_staged = false; // new windows, to the warm-mode staging area if win_staged)
    // segmented scan: this job's rows, where its state comes from and goes to
    const float *hin = state;  // nullptr: start from 0
    float *hout = state;       // nullptr: the end state is not needed
    bool h_ident = false, v_zero = false, write_o = true;
    float *zflag = nullptr;  // transition jobs: whether their transition was found zero
    int64_t warm_rows = 0;   // warm jobs: rows run from h = 0 before the segment, without o
    const int *chain_flags = nullptr;  // second-launch jobs: the chain flags of their columns
    // direct_final: job 0 sets, and the last warm job waits for, this slice's read flag
    int read_role = 0;  // 1: set it, 2: wait for it
    if (a.pass != 0) {
        const SegLayout lay{(int64_t)H * DK * DV, a.st.B, a.nseg, H};
        const int S = a.nseg;
        // warm mode of this (stream, head): uniform over the workgroup; the jobs it makes
        // redundant return before touching LDS or a barrier
        const float wcount = a.warm ? warm_lane_count(a.seg_ws, lay, b, head) : 0.f;
        const bool warm = a.warm && warm_head(wcount);
        int seg;
        if (a.pass == 1) {
            // Job order: 0 segment 0, 1..S-2 end states, S-1..2S-4 transitions, 2S-3..3S-5
            // warm jobs of segments 1..S-1. With warm starts possible the grid puts the warm
            // jobs right after segment 0 and the map jobs last: workgroups dispatch in grid
            // order, and in warm mode the map jobs return at once, so they then neither sit
            // in front of the warm jobs nor delay their start.
            const int job = !a.warm || jp == 0 ? jp : jp < S ? 2 * S - 4 + jp : jp - S + 1;
            if (job >= 2 * S - 3) {  // warm job of segment job - (2S - 4)
                if (!warm)
                    return;
                seg = job - (2 * S - 4);
                hin = nullptr;
                // The last segment's end state is the stream's final state. Job 0 of this
                // launch reads the stream's initial state from the same buffer, so it goes to
                // slot H(b, S-1) (unused in warm mode), and the chain's workgroups of the
                // next launch copy it over; with direct_final the job waits for job 0's read
                // flag and writes the caller's state and windows itself.
                hout = seg < S - 1 ? nullptr : a.seg_ws + lay.h(b, S - 1);
                warm_rows = (int64_t)__builtin_bit_cast(
                                float, __builtin_amdgcn_readlane(
                                           __builtin_bit_cast(int, wcount), seg - 1)) *
                            CH;
                win_staged = true;
                if (a.direct_final && seg == S - 1) {
                    hout = state;
                    win_staged = false;
                    read_role = 2;
                }
            } else {
                if (warm && job > 0)
                    return;
                if (job == 0 && tid0 < NV / 16)  // this job's columns: chain not done yet
                    reinterpret_cast<int *>(
                        a.seg_ws + lay.chain_done(b, head, slice * (NV / 16)))[tid0] = 0;
                seg = job <= S - 2 ? job : job - (S - 2);
                if (job == 0 && a.direct_final)
                    read_role = 1;
                if (job > 0) {
                    hin = nullptr;
                    write_o = false;
                    h_ident = v_zero = job > S - 2;
                }
                hout = a.seg_ws + (job == 0 ? lay.h(b, 1) : job <= S - 2 ? lay.bs(b, seg)
                                                                           : lay.as(b, seg));
                if (h_ident)
                    zflag = a.seg_ws + lay.zero_flag(b, seg, head);
            }
        } else {
            if (warm)
                return;
            seg = jp + 1;
            hin = a.seg_ws + lay.h(b, seg);
            if (seg >= 2)  // slot H(b, seg) comes from the chain of this launch
                chain_flags = reinterpret_cast<const int *>(
                    a.seg_ws + lay.chain_done(b, head, slice * (NV / 16)));
            if (seg < S - 1)
                hout = nullptr;
        }
        const int64_t s0 = start;
        start = min(s0 + (seg == 0 ? 0 : a.seg0_len + (seg - 1) * a.seg_len), end);
        if (seg < S - 1)  // the last segment runs to the stream's end
            end = min(start + (seg == 0 ? a.seg0_len : a.seg_len), end);
        last_seg = seg == S - 1;
    }
    // o is written from row o_start on (never by map jobs); a warm job starts warm_rows
    // earlier, from h = 0, with chunks that compute no o
    const int64_t o_start = write_o ? start : INT64_MAX;
    start -= warm_rows;
    const int64_t hoff = (int64_t)head * DK * DV;
    const int colw = slice * NV + wave0 * 16 * NCB;  // this wave's first dv column

    const int head_qk = head / a.qk_group;  // the q/k head this value head reads
    const TIN *qg = (const TIN *)a.q + head_qk * DK;
    const TIN *kg = (const TIN *)a.k + head_qk * DK;
    const TIN *vg = (const TIN *)a.v + head * DV + slice * NV;
    float *ob = a.o + head * DV + slice * NV;  // this workgroup's o columns
    const int64_t ld = a.ld;

    // blocks above the diagonal that the 32-deep steps over P touch stay 0
    for (int idx = tid0; idx < 2 * 256; idx += NT) {
        const int blk = idx >> 8, e = idx & 255;
        const int off = (32 * blk + (e >> 4)) * LDT + 32 * blk + 16 + (e & 15);
        ((T *)(smem + C::OFF_P))[off] = (T)0.f;
        if constexpr (SPLIT)
            ((T *)(smem + C::OFF_PL))[off] = (T)0.f;
    }

    // state, D layout: hs[cb][mb][i] = h[16 mb + 4 g + i][colw + 16 cb + c]
    f32x4 hs[NCB][DK / 16];

    // Raw 16-byte vectors of the next chunk, loaded one chunk ahead so that the HBM latency
    // hides behind a whole chunk of work. Rows at or past the stream's end are never read.
    uint4 pq[NQK], pv[NVV], pgk[NGK];
    float pg = 0.f, pb = 0.f;
    // Per-thread row pointers at chunk offset 0 (held across the loop; a chunk adds one
    // uniform offset) and the chunk row each 16-byte piece belongs to.
    const TIN *qk_src[NQK];
    const TIN *v_src[NVV];
    int gk_off[NGK];
    int qk_row[NQK], v_row[NVV], gk_row[NGK];
    bool qk_isk[NQK];
#pragma unroll
    for (int it = 0; it < NQK; ++it) {
        const int rr = wave0 * RPW + lane0 / LPR + it * NW * RPW;
        qk_row[it] = rr & (CH - 1);
        qk_isk[it] = rr >= CH;
        qk_src[it] = (rr >= CH ? kg : qg) + (int64_t)qk_row[it] * ld + (lane0 % LPR) * VEC;
    }
#pragma unroll
    for (int it = 0; it < NVV; ++it) {
        v_row[it] = wave0 * RPV + lane0 / LPV + it * NW * RPV;
        v_src[it] = vg + (int64_t)v_row[it] * ld + (lane0 % LPV) * VEC;
    }
#pragma unroll
    for (int it = 0; it < NGK; ++it) {
        gk_row[it] = wave0 * GRW + lane0 / GPR + it * NW * GRW;
        gk_off[it] = (gk_row[it] * H + head) * DK + (lane0 % GPR) * 4;
    }
    // Fused front end: the raw rows of the chunk at c0 (Lc rows) and the KC - 1 rows before
    // it go straight into LDS by LDS-DMA, one 16-byte piece per lane (a wave instruction
    // fills up to 1 KiB): raw row rho of a region holds stream row c0 - (KC - 1) + rho: the
    // q rows, then the k rows (RQ bytes each), and the v rows in padded blocks of 4 (raw_v).
    // Rows before the
    // stream's first row (the carried window, at the first chunk) are stored before the
    // loop; rows at or past the chunk's end are never read and never used.
    constexpr int KC = C::KC;
    const int qk_heads = H / a.qk_group;
    // The raw rows used are [max(stream start, c0 - (KC - 1)), c0 + Lc): raw row indices
    // [rlo, rhi) of the chunk. Addresses are a uniform row base plus a 32-bit lane offset
    // (the host keeps RR row strides within 32 bits for these calls).
    // part 0: the v rows; part 1: the q|k rows
    // A q|k instruction covers RPQ whole raw rows (1 KiB), a v instruction 4 rows (RVR
    // bytes each: 1 KiB at 128 columns, the upper half of the lanes idle at 64). Each lane's
    // byte offset from the instruction's first row is the same in every instruction.
    constexpr int LPQ = DK / 8, RPQ = 64 / LPQ, NQI = (C::RR + RPQ - 1) / RPQ;
    constexpr int LPVR = NV / 8, NVI = (C::RR + 3) / 4;
    const int64_t ldb = ld * (int64_t)sizeof(TIN);
    // this wave's instruction slots [i0, i1) of a part (the whole part by default)
    auto prefetch_raw = [&](int64_t c0, int Lc, bool with_q, int lane, int wave, int part,
                            int i0 = 0, int i1 = 1 << 20) {
        const int rlo = (int)max((int64_t)0, sbeg - (c0 - (KC - 1)));
        const int rhi = Lc + KC - 1;
        const bool full = rlo == 0 && rhi == C::RR;  // every raw row of the region
        const int64_t r0 = c0 - (KC - 1);
        if (part == 1) {
            const int lr = lane / LPQ;
            const uint32_t off = (uint32_t)(lr * ldb) + (uint32_t)(lane % LPQ) * 16u;
            // instructions [0, NQI) fill the q rows, [NQI, 2 NQI) the k rows
#pragma unroll
            for (int i = 0; i < (2 * NQI + NW - 1) / NW; ++i) {
                const int n = wave + NW * i;
                const int t = n >= NQI, m = n - t * NQI;
                const int row = RPQ * m + lr;
                const bool ok = full ? row < C::RR : row >= rlo && row < rhi;
                if (i >= i0 && i < i1 && n < 2 * NQI && (t || with_q) && ok)
                    dma16((const char *)(t ? kg : qg) + (r0 + RPQ * m) * ldb, off,
                          lds_addr(smem + C::OFF_Q + C::raw_qk(t, 0) + 1024 * m));
            }
        } else if (!v_zero) {
            const int lr = lane / LPVR;
            const uint32_t off = (uint32_t)(lr * ldb) + (uint32_t)(lane % LPVR) * 16u;
#pragma unroll
            for (int i = 0; i < (NVI + NW - 1) / NW; ++i) {
                const int n = wave + NW * i;
                const int row = 4 * n + lr;
                const bool ok = full ? row < C::RR : row >= rlo && row < rhi;
                if (i >= i0 && i < i1 && n < NVI && lane < 4 * LPVR && ok)
                    dma16((const char *)vg + (r0 + 4 * n) * ldb, off,
                          lds_addr(smem + C::OFF_V + C::RVBLK * n));
            }
        }
    };
    // conv channel of q/k element c (tensor 0: q, 1: k) and of v column c of this workgroup
    auto qk_channel = [&](int tensor, int c) {
        return (tensor ? qk_heads * DK : 0) + head_qk * DK + c;
    };
    auto v_channel = [&](int c) { return 2 * qk_heads * DK + head * DV + slice * NV + c; };
    // With K = conv_k < KC taps the conv runs as KC taps, the first KC - K of them zero,
    // and the window keeps the last K - 1 raw inputs.
    const int Kt = FRONT ? a.conv_k : KC, Wn = Kt - 1, tap0 = KC - Kt;
    float wv[FRONT ? KC : 1];  // this lane's v column taps (fused front end)
    // The raw rows of the next chunk go out in three groups spread over the state stage
    // (group 0 at its start, 1 before P U, 2 before the state update): every workgroup
    // runs the same steps at about the same time, and the rows of a whole chunk requested
    // at once by every CU exceed what HBM delivers in that time, which would stall each
    // wave on its own requests.
    constexpr int SQ = (2 * NQI + NW - 1) / NW, SV = (NVI + NW - 1) / NW;
    auto prefetch_group = [&](int64_t c0, int Lc, int grp) {
        const bool with_q = c0 >= o_start;
        const int lane = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        if (grp == 0)
            prefetch_raw(c0, Lc, with_q, lane, wave, 1, 0, (SQ + 1) / 2);
        if (grp == 1) {
            prefetch_raw(c0, Lc, with_q, lane, wave, 1, (SQ + 1) / 2, SQ);
            prefetch_raw(c0, Lc, with_q, lane, wave, 0, 0, (SV + 1) / 2);
        }
        if (grp == 2)
            prefetch_raw(c0, Lc, with_q, lane, wave, 0, (SV + 1) / 2, SV);
    };
    // rows = false: the gates only (the fused front end's rows then go by prefetch_group)
    auto prefetch = [&](int64_t c0, int Lc, bool rows = true) {
        const int64_t roff = c0 * ld;
        const bool with_q = c0 >= o_start;  // q rows only feed o
        if constexpr (FRONT) {
            if (rows) {
                const int lane = threadIdx.x & 63;
                const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
                prefetch_raw(c0, Lc, with_q, lane, wave, 1);
                prefetch_raw(c0, Lc, with_q, lane, wave, 0);
            }
        } else if (Lc == CH) {  // a whole chunk: only wave-uniform conditions
#pragma unroll
            for (int it = 0; it < NQK; ++it)
                pq[it] = qk_isk[it] || with_q ? load_stream16(qk_src[it] + roff)
                                              : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int it = 0; it < NVV; ++it)
                pv[it] = !v_zero ? load_stream16(v_src[it] + roff) : make_uint4(0, 0, 0, 0);
        } else {
#pragma unroll
            for (int it = 0; it < NQK; ++it)
                pq[it] = qk_row[it] < Lc && (qk_isk[it] || with_q)
                             ? load_stream16(qk_src[it] + roff)
                             : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int it = 0; it < NVV; ++it)
                pv[it] = v_row[it] < Lc && !v_zero
                             ? load_stream16(v_src[it] + roff)
                             : make_uint4(0, 0, 0, 0);
        }
        if constexpr (KDA) {
            const float *gbase = a.g + c0 * H * DK;
#pragma unroll
            for (int it = 0; it < NGK; ++it) {
                int go = gk_off[it];  // opaque per call, as for the scalar gates below
                asm volatile("" : "+v"(go));
                pgk[it] = gk_row[it] < Lc ? load_stream16(gbase + go) : make_uint4(0, 0, 0, 0);
            }
        }
        if (threadIdx.x < CH) {
            // this lane's row of the gates and betas, derived from the thread index in each
            // call: a per-lane offset held across the chunk loop is spilled, and its reload
            // waits for every load and store in flight
            int tx = threadIdx.x;
            asm volatile("" : "+v"(tx));
            const int go = (tx & (CH - 1)) * H;
            if constexpr (!KDA)
                pg = (int)threadIdx.x < Lc ? (a.g + (c0 * H + head))[go] : 0.f;
            pb = (int)threadIdx.x < Lc ? (a.beta + (c0 * H + head))[go] : 0.f;
        }
    };
    // the first chunk's rows are requested before the state, the taps and the carried
    // window, whose loads the workgroup then waits for while the rows are in flight
    if (start < end)
        prefetch(start, (int)min((int64_t)CH, end - start));
    if (chain_flags)  // (uniform) every wave, before it reads its share of the start state
        wait_flags(chain_flags, NV / 16, a.wait_polls);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int mb = 0; mb < DK / 16; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * mb + 4 * (lane0 >> 4) + i;
                const int col = colw + 16 * cb + (lane0 & 15);
                hs[cb][mb][i] = hin ? hin[hoff + (int64_t)row * DV + col]
                                    : (h_ident && row == col ? 1.f : 0.f);
            }
    if constexpr (FRONT) {
        // q and k taps of this head into LDS, [tensor][tap][channel], times -log2(e): the
        // conv then gives -z log2(e), the argument of the exp2 in the SiLU (see stage A)
        for (int idx = tid0; idx < 2 * KC * DK; idx += NT) {
            const int t = idx / (KC * DK), rem = idx - t * KC * DK, j = rem / DK;
            ((float *)(smem + C::OFF_CW))[idx] =
                j < tap0 ? 0.f
                         : a.conv_w[(int64_t)qk_channel(t, rem - j * DK) * Kt + j - tap0] *
                               -kLog2e;
        }
#pragma unroll
        for (int j = 0; j < KC; ++j)
            wv[j] = j < tap0 ? 0.f
                             : a.conv_w[(int64_t)v_channel(16 * wave0 + (lane0 & 15)) * Kt +
                                        j - tap0];
        // the stream's first chunk: raw rows 0 .. KC-2 are the carried window, after zeros
        // in the rows a shorter window does not reach (multiplied by zero taps; never read
        // from stale LDS)
        if (start == sbeg && start < end) {
            const TIN *cw = (const TIN *)(a.conv_state_ptrs ? a.conv_state_ptrs[b]
                                                            : a.conv_state);
            constexpr int W = KC - 1;
            for (int idx = tid0; idx < (2 * DK + NV) * W; idx += NT) {
                const int ch = idx / W, j = idx - ch * W, e = j - (W - Wn);
                if (ch < 2 * DK)
                    *(TIN *)(smem + C::OFF_Q + C::raw_qk(ch >= DK, j) + (ch % DK) * 2) =
                        e < 0 ? (TIN)0.f : cw[(int64_t)qk_channel(ch >= DK, ch % DK) * Wn + e];
                else
                    *(TIN *)(smem + C::OFF_V + C::raw_v(j) + (ch - 2 * DK) * 2) =
                        e < 0 ? (TIN)0.f : cw[(int64_t)v_channel(ch - 2 * DK) * Wn + e];
            }
        }
    }

    // o of a chunk is staged in LDS and written out during the next chunk's preparation
    // stage: vector loads and stores share one completion counter, so stores issued at the
    // end of a chunk would hold up the wait for the next chunk's rows. Full rows go out as
    // 16-byte stores.
    // Output gate: the z rows of a chunk go straight from HBM into the z tile with LDS-DMA
    // loads issued beside the next chunk's prefetch (no registers held; the chunk start's
    // wait for the prefetch covers them); the flush of that chunk's o reads them from LDS.
    // One 16-byte load per lane, LZ lanes per row: a wave's load k covers tile rows
    // RL k .. RL k + RL - 1 (RL = 64 / LZ), lane l writing row RL k + l / LZ, bytes
    // 16 (l % LZ) .. +15 of it.
    constexpr int V4 = NV / 4, RPP = NT / V4, NR = CH / RPP;
    static_assert(NT % V4 == 0 && CH % RPP == 0 && (V4 == 16 || V4 == 32), "o row map");
    constexpr int LZ = C::ZROW / 16, RL = 64 / LZ;
    static_assert(!GATE || C::ZREG || ((LZ == 8 || LZ == 16) && (CH / RL) % NW == 0),
                  "z tile map");
    // z in registers (fused front end): thread tid holds z of rows it * RPP + tid / V4,
    // columns 4 (tid % V4) .. +3 -- the values its flush of that chunk's o gates
    typename Z4<TZ>::raw zr[C::ZREG ? NR : 1];
    const TZ *zg = GATE ? (const TZ *)a.z + head * DV : nullptr;
    auto load_z = [&](int64_t c0, int Lc, int lane, int wave) {
        if constexpr (C::ZREG) {
            const int tid = threadIdx.x, j = tid % V4;
#pragma unroll
            for (int it = 0; it < NR; ++it) {
                const int r = it * RPP + tid / V4;
                zr[it] = r < Lc ? Z4<TZ>::load(zg + (c0 + r) * a.ld_z + 4 * j) : Z4<TZ>::zero();
            }
            return;
        }
        typedef __attribute__((address_space(1))) void gptr;
        typedef __attribute__((address_space(3))) void lptr;
        constexpr int NZI = CH / RL / NW;  // loads per wave
#pragma unroll
        for (int i = 0; i < NZI; ++i) {
            const int grp = wave * NZI + i, r = RL * grp + lane / LZ;
            if (r < Lc)
                __builtin_amdgcn_global_load_lds(
                    (gptr *)(zg + (c0 + r) * a.ld_z + (lane % LZ) * (16 / (int)sizeof(TZ))),
                    (lptr *)(smem + C::OFF_Z + grp * RL * C::ZROW), 16, 0, 0);
        }
    };
    if constexpr (GATE) {
        for (int i = tid0; i < NV; i += NT)
            ((float *)(smem + C::OFF_W))[i] = a.norm_w[i];
    }
    auto flush_o = [&](const float *Os, int64_t c0, int Lc, int tid) {
        const int j = tid % V4;
        float4 ov[NR];
#pragma unroll
        for (int it = 0; it < NR; ++it)
            ov[it] = *reinterpret_cast<const float4 *>(Os + (it * RPP + tid / V4) * LDO + 4 * j);
        if constexpr (GATE) {
            // row sums of squares over the V4 lanes of each row (every lane takes part), the
            // NR rows' reductions independent of each other
            float ss[NR];
#pragma unroll
            for (int it = 0; it < NR; ++it) {
                const float4 o = ov[it];
                ss[it] = group_sum<16>(o.x * o.x + o.y * o.y + o.z * o.z + o.w * o.w);
                if constexpr (V4 == 32)  // rows of 32 lanes: add the other 16 (swizzle xor 16)
                    ss[it] += __int_as_float(
                        __builtin_amdgcn_ds_swizzle(__float_as_int(ss[it]), 0x401F));
            }
            const float4 w = *reinterpret_cast<const float4 *>(smem + C::OFF_W + 16 * j);
#pragma unroll
            for (int it = 0; it < NR; ++it) {
                const int r = it * RPP + tid / V4;
                const typename Z4<TZ>::raw z =
                    C::ZREG ? zr[it]
                            : *reinterpret_cast<const typename Z4<TZ>::raw *>(
                                  smem + C::OFF_Z + r * C::ZROW + 4 * j * (int)sizeof(TZ));
                ov[it] = gate4(ov[it], rsqrtf(ss[it] * (1.f / DV) + a.norm_eps), w,
                               Z4<TZ>::get(z));
            }
        }
        if (Lc == CH) {  // a whole chunk: no per-row test
#pragma unroll
            for (int it = 0; it < NR; ++it)
                store_stream16(ob + (c0 + it * RPP + tid / V4) * (int64_t)H * DV + 4 * j,
                               ov[it]);
        } else {
#pragma unroll
            for (int it = 0; it < NR; ++it) {
                const int r = it * RPP + tid / V4;
                if (r < Lc)
                    store_stream16(ob + (c0 + r) * (int64_t)H * DV + 4 * j, ov[it]);
            }
        }
    };

    // X = V - diag(a) K h and O = diag(a) Q h for column block cb of this wave (the
    // per-channel gate's tiles carry e^G already)
    // Fused front end: V is the conv + SiLU of the raw v rows (Vs is then the raw region),
    // computed here in fp32 for this lane's D-layout rows 16 I + 4 g + i and column; rows
    // at or past the chunk's end (Lc rows) are 0. Q h takes q's fp16 hi part.
    // Fused front end: WO (this chunk computes o, i.e. Q h) is a compile-time copy of each
    // case, and a row block's fragment reads are all issued before its products with no
    // branch between. (The register-path instances, which hold the next chunk's rows in
    // registers, interleave reads and products: batching them would spill.)
    auto kh_qh_wo = [&](auto wo, int cb, f32x4 (&x)[NB], f32x4 (&o)[NB],
                        const float (&ar)[NB][4], const T *Ks, const void *Qs, const void *Vs,
                        int wave, int lane, int g4, int c16, int Lc) {
        constexpr bool WO = decltype(wo)::value;
        const int vc = 16 * (wave * NCB + cb);  // this block's columns within Vs
        frag hf[DK / 32];
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb)
            hf[kb] = pack<T>(hs[cb][2 * kb], hs[cb][2 * kb + 1]);
#pragma unroll
        for (int I = 0; I < NB; ++I) {
            f32x4 kh = zero4(), qh = zero4();
            if constexpr (FRONT) {
                frag kf[DK / 32], qf[WO ? DK / 32 : 1];
#pragma unroll
                for (int kb = 0; kb < DK / 32; ++kb) {
                    kf[kb] = ld_frag_qk<DK>(Ks, 16 * I, 32 * kb, lane);
                    if constexpr (WO)
                        qf[kb] = ld_frag_qk<DK>((const T *)Qs, 16 * I, 32 * kb, lane);
                }
#pragma unroll
                for (int kb = 0; kb < DK / 32; ++kb) {
                    mma(kh, kf[kb], hf[kb]);
                    if constexpr (WO)
                        mma(qh, qf[kb], hf[kb]);
                }
            } else {
#pragma unroll
                for (int kb = 0; kb < DK / 32; ++kb) {
                    mma(kh, ld_frag_qk<DK>(Ks, 16 * I, 32 * kb, lane), hf[kb]);
                    if (write_o)
                        mma(qh, ld_frag_qk<DK>((const T *)Qs, 16 * I, 32 * kb, lane), hf[kb]);
                }
            }
            float v[4];
            if constexpr (FRONT) {
                // raw rows 16 I + 4 g .. + KC + 2 of this column (raw row = chunk row + KC - 1):
                // block 4 I + g of the raw region and the next one
                const unsigned char *rv = (const unsigned char *)Vs + (vc + c16) * 2 +
                                          (4 * I + g4) * C::RVBLK;
                float xr[KC + 3];
#pragma unroll
                for (int u = 0; u < KC + 3; ++u)
                    xr[u] = __uint_as_float(
                        (uint32_t)*(const unsigned short *)(rv + C::raw_v(u)) << 16);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float acc = 0.f;
#pragma unroll
                    for (int j = 0; j < KC; ++j)
                        acc += wv[j] * xr[i + j];
                    // computed on every lane and then selected: a branch around it per
                    // element would cost more than the SiLU (stale rows never reach v)
                    float sv = silu(acc);
                    asm volatile("" : "+v"(sv));
                    v[i] = 16 * I + 4 * g4 + i < Lc && !v_zero ? sv : 0.f;
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    v[i] = (float)((const T *)Vs)[(16 * I + 4 * g4 + i) * LDV + vc + c16];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float arr = KDA ? 1.f : ar[I][i];
                x[I][i] = v[i] - arr * kh[i];
                o[I][i] = arr * qh[i];
            }
        }
    };
    auto kh_qh = [&](int cb, f32x4 (&x)[NB], f32x4 (&o)[NB], const float (&ar)[NB][4],
                     const T *Ks, const void *Qs, const void *Vs, int wave, int lane, int g4,
                     int c16, int Lc) {
        if (!FRONT || write_o)
            kh_qh_wo(std::true_type{}, cb, x, o, ar, Ks, Qs, Vs, wave, lane, g4, c16, Lc);
        else
            kh_qh_wo(std::false_type{}, cb, x, o, ar, Ks, Qs, Vs, wave, lane, g4, c16, Lc);
    };

    // A transition job stops once its transition has underflowed. Token t multiplies it by
    // (I - beta_t k_t k_t^T) alpha_t, of norm <= alpha_t when beta_t |k_t|^2 lies in [0, 2];
    // a chunk by a factor of norm <= e^(Gamma_C). Once the running bound is below e^-110
    // (under half the smallest fp32 subnormal) every entry is 0 in fp32 and stays 0 through
    // the remaining chunks, so the job writes zeros and ends. The bound is read only after
    // a chunk's barriers (never before the first chunk), by every wave alike.
    // (not in the instances with the output gate fused, which have no registers to spare)
    if (C::STOP && tid0 == 0)
        ((float *)(smem + C::OFF_G))[4 * CH] = 0.f;
    const bool may_stop = C::STOP && h_ident && a.unit_keys;
    auto underflowed = [&]() {
        return may_stop && __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                                         __builtin_bit_cast(int, ((const float *)(
                                                             smem + C::OFF_G))[4 * CH]))) < -110.f;
    };
    if (read_role) {  // (uniform) direct_final
        const SegLayout lay{(int64_t)H * DK * DV, a.st.B, a.nseg, H};
        int *rf = reinterpret_cast<int *>(a.seg_ws + lay.flags(b, head)) + SegLayout::kFlagRead +
                  slice;
        if (read_role == 1) {
            // job 0: every wave's loads of the initial state and windows are done
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (tid0 == 0)
                __hip_atomic_store(rf, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            // the last warm job, which writes the caller's state and windows: job 0 has read
            // them. Both start in the first round of workgroups, so this waits for little
            // more than job 0's first loads, and nothing inside the chunk loop has to check.
            // Should the wait give up, the job takes the slot and the staging area instead
            // and flags it, and the second launch copies them over.
            if (!wait_flags(rf, 1, a.wait_polls)) {
                hout = a.seg_ws + lay.h(b, lay.S - 1);
                win_staged = true;
                if (tid0 == 0)
                    rf[SegLayout::kFlagFallback - SegLayout::kFlagRead] = 1;
            }
        }
    }
    for (int64_t cs = start; cs < end && !(cs > start && underflowed()); cs += CH) {
        const int L = (int)min((int64_t)CH, end - cs);
        write_o = cs >= o_start;  // this chunk computes o
        // Thread coordinates and tile addresses are re-derived from opaque copies in every
        // chunk: otherwise the compiler hoists each per-lane LDS address out of the loop
        // and holds a register for every one of them across all stages.
        int zo = 0, tz = threadIdx.x;
        asm volatile("" : "+s"(zo));
        asm volatile("" : "+v"(tz));
        const int tid = tz, lane = tz & 63, g4 = lane >> 4, c16 = lane & 15;
        const int wave = __builtin_amdgcn_readfirstlane(tz >> 6);
        T *Qs = (T *)(smem + zo + C::OFF_Q);
        T *Ks = (T *)(smem + zo + C::OFF_K);
        T *Vs = (T *)(smem + zo + C::OFF_V);
        T *Ps = (T *)(smem + zo + C::OFF_P);
        T *Psl = (T *)(smem + zo + C::OFF_PL);
        T *MTh = (T *)(smem + zo + C::OFF_MT);
        float *Ms = (float *)(smem + zo + C::OFF_M);
        float *Gk = (float *)(smem + zo + C::OFF_GK);
        float *graw = (float *)(smem + zo + C::OFF_G);
        float *bet = graw + CH;
        float *ea = graw + 2 * CH;  // a_r = e^Gamma_r
        float *ed = graw + 3 * CH;  // a_C / a_r
        float *Os = (float *)(smem + zo + C::OFF_O);
        T *Kl = (T *)(smem + zo + C::OFF_KL);      // fused front end: K lo
        T *Ql = (T *)(smem + zo + C::OFF_QL);      // fused front end: Q lo
        float *Xs = (float *)(smem + zo + C::OFF_X);  // fused front end: inversion scratch

        // the previous chunk's z tile (LDS-DMA, counted like the prefetch loads) lands
        // before the barrier that precedes its flush
        if constexpr (GATE)
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

        if constexpr (FRONT) {
            // ---- A (fused front end): raw rows -> conv + SiLU -> L2, scale -> tiles -------
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's LDS-DMA rows
            __syncthreads();  // every wave's rows, and the window rows of a first chunk
            // Lane group gi of LQ lanes takes 8 channels each of one tensor (q or k) for rows
            // 4 rg .. 4 rg + 3, so a row's L2 sum is a sum over the group (DPP).
            constexpr int LQ = DK / 8, GPW = 64 / LQ;
            static_assert(NW * GPW / 2 * 4 == CH, "conv row map");
            const int gi = lane / LQ, cg = lane % LQ, tsr = gi & 1;
            const int rg = wave * (GPW / 2) + (gi >> 1);
            const unsigned char *rq = smem + zo + C::OFF_Q + C::raw_qk(tsr, 0) + cg * 16;
            const float *wt = (const float *)(smem + zo + C::OFF_CW) + tsr * KC * DK + 8 * cg;
            float y[4][8];
            {
                float w[KC][8];
#pragma unroll
                for (int j = 0; j < KC; ++j)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const f32x4 t4 = *reinterpret_cast<const f32x4 *>(wt + j * DK + 4 * h);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            w[j][4 * h + e] = t4[e];
                    }
                uint4 raw[KC + 3];
#pragma unroll
                for (int u = 0; u < KC + 3; ++u)
                    raw[u] = *reinterpret_cast<const uint4 *>(rq + (4 * rg + u) * C::RQ);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
                    for (int j = 0; j < KC; ++j) {
                        float xv[8];
                        unpack((const bf16 *)nullptr, raw[i + j], xv);
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            acc[e] += w[j][e] * xv[e];
                    }
                    // acc = -z log2(e): e^-z = exp2(acc), and acc / (1 + e^-z) is
                    // -log2(e) SiLU(z); the factor is taken out below
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        y[i][e] = acc[e] *
                                  __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(acc[e]));
                }
            }
            // L2 of each row over the head, the q scale; rows at or past the end are 0. The
            // rows hold -log2(e) SiLU(z): y / sqrt(|y|^2 + eps) of the SiLU rows is
            // -y' / sqrt(|y'|^2 + eps log2(e)^2) of these, and without L2 they are rescaled
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float m = tsr ? -1.f : -a.scale;
                if (a.do_l2) {
                    float ss = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        ss += y[i][e] * y[i][e];
                    m *= rsqrtf(group_sum<LQ>(ss) + a.eps * (kLog2e * kLog2e));
                } else {
                    m *= kLn2;
                }
                const bool live = 4 * rg + i < L;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    y[i][e] = live ? y[i][e] * m : 0.f;
            }
            // the stream's last chunk: the new windows are its raw rows L + KC - 1 - Wn ..
            // L + KC - 2 (the last Wn entries of [old window | rows]), read before the tiles
            // cover them
            if (last_seg && cs + CH >= end) {
                TIN *wo = win_staged || a.win_shared
                              ? (TIN *)a.win_ws + (int64_t)b * a.cd * Wn
                              : (TIN *)(a.conv_state_ptrs ? a.conv_state_ptrs[b]
                                                          : a.conv_state);
                const int r0 = L + KC - 1 - Wn;
                for (int idx = tid; idx < (2 * DK + NV) * Wn; idx += NT) {
                    const int ch = idx / Wn, j = idx - ch * Wn;
                    if (ch < 2 * DK)
                        wo[(int64_t)qk_channel(ch >= DK, ch % DK) * Wn + j] =
                            *(const TIN *)(smem + zo + C::OFF_Q + C::raw_qk(ch >= DK, r0 + j) +
                                           (ch % DK) * 2);
                    else
                        wo[(int64_t)v_channel(ch - 2 * DK) * Wn + j] = *(const TIN *)(
                            smem + zo + C::OFF_V + C::raw_v(r0 + j) + (ch - 2 * DK) * 2);
                }
            }
            __syncthreads();  // the raw q|k rows are read before the Q tile covers them
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * rg + i;
                if (tsr == 1 || write_o) {  // q only feeds o
                    T *dh = tsr ? Ks : Qs, *dl = tsr ? Kl : Ql;
                    // the 4-element chunks 2 cg and 2 cg + 1 of row r sit side by side in
                    // the permuted layout (the permutation flips the low 2 bits of the chunk
                    // index), in swapped order when it flips bit 0: one 16-byte store each
                    f16x4 hi4[2], lo4[2];
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        split4(f32x4{y[i][4 * h], y[i][4 * h + 1], y[i][4 * h + 2],
                                     y[i][4 * h + 3]},
                               hi4[h], lo4[h]);
                    const int sw = (r >> 2) & 1;
                    const int off = QK<T, DK>::at(r, 2 * cg) - 4 * sw;
                    const f16x8 hv = sw ? __builtin_shufflevector(hi4[1], hi4[0], 0, 1, 2, 3,
                                                                  4, 5, 6, 7)
                                        : __builtin_shufflevector(hi4[0], hi4[1], 0, 1, 2, 3,
                                                                  4, 5, 6, 7);
                    *reinterpret_cast<f16x8 *>(dh + off) = hv;
                    if (tsr == 1 || C::QLO) {
                        const f16x8 lv = sw ? __builtin_shufflevector(lo4[1], lo4[0], 0, 1, 2,
                                                                      3, 4, 5, 6, 7)
                                            : __builtin_shufflevector(lo4[0], lo4[1], 0, 1, 2,
                                                                      3, 4, 5, 6, 7);
                        *reinterpret_cast<f16x8 *>(dl + off) = lv;
                    }
                }
            }
        } else {
        // ---- A: registers -> LDS: q, k (L2, scale), v, raw gates, beta -----------------
#pragma unroll
        for (int it = 0; it < NQK; ++it) {
            const int rr = wave * RPW + lane / LPR + it * NW * RPW;
            const bool isk = rr >= CH;
            const int r = rr & (CH - 1);
            const int c0 = (lane % LPR) * VEC;
            float x[VEC];
            unpack((const TIN *)nullptr, pq[it], x);
            float mul = isk ? 1.f : a.scale;
            if (a.do_l2) {
                float ss = 0.f;
#pragma unroll
                for (int i = 0; i < VEC; ++i)
                    ss += x[i] * x[i];
                if constexpr (LPR == 4 || LPR == 8 || LPR == 16) {
                    ss = group_sum<LPR>(ss);
                } else {
#pragma unroll
                    for (int m = 1; m < LPR; m <<= 1)
                        ss += __shfl_xor(ss, m);
                }
                float rs = rsqrtf(ss + a.eps);  // on every lane, then selected
                asm volatile("" : "+v"(rs));
                mul = r < L ? mul * rs : 0.f;
            }
#pragma unroll
            for (int i = 0; i < VEC; ++i)
                x[i] *= mul;
            T *dst = isk ? Ks : Qs;
#pragma unroll
            for (int h = 0; h < VEC / 4; ++h) {  // 4-element chunks of the Q/K layout
                const float y[4] = {x[4 * h], x[4 * h + 1], x[4 * h + 2], x[4 * h + 3]};
                if constexpr (C::KLO && SPLIT) {
                    f16x4 hi4, lo4;
                    split4(f32x4{y[0], y[1], y[2], y[3]}, hi4, lo4);
                    *reinterpret_cast<f16x4 *>(dst + QK<T, DK>::at(r, c0 / 4 + h)) = hi4;
                    if (isk)
                        *reinterpret_cast<f16x4 *>(Kl + QK<T, DK>::at(r, c0 / 4 + h)) = lo4;
                } else {
                    store_vec4(dst + QK<T, DK>::at(r, c0 / 4 + h), y);
                }
            }
        }
#pragma unroll
        for (int it = 0; it < NVV; ++it) {
            const int r = wave * RPV + lane / LPV + it * NW * RPV;
            float x[VEC];
            unpack((const TIN *)nullptr, pv[it], x);
            store_vec(Vs + r * LDV + (lane % LPV) * VEC, x);
        }
        }
        if constexpr (KDA) {
#pragma unroll
            for (int it = 0; it < NGK; ++it) {
                const int r = wave * GRW + lane / GPR + it * NW * GRW;
                *reinterpret_cast<uint4 *>(Gk + r * LDG + (lane % GPR) * 4) = pgk[it];
            }
        }
        if (tid < CH) {  // wave 0: Gamma = inclusive prefix sum of the log-gates, and decays
            const float gam = wave_scan(pg);
            const float gl = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gam), CH - 1));
            graw[tid] = gam;
            bet[tid] = pb;
            ea[tid] = __expf(gam);
            ed[tid] = __expf(gl - gam);
            if constexpr (C::STOP) {
                // running log of a bound on the norm of the job's transition: each chunk
                // adds Gamma_C, valid while every beta lies in [0, 1.9] (else +inf; 1.9
                // leaves room for keys a rounding above unit length: beta |k|^2 < 2)
                const bool bad = __ballot(!(pb >= 0.f && pb <= 1.9f)) != 0;
                if (tid == 0)
                    graw[4 * CH] += bad ? __builtin_inff() : gl;
            }
        }
        __syncthreads();

        // ---- B: cumulative log-gate; lane r of every wave holds Gamma_r -----------------
        if constexpr (KDA) {
            // per channel, in place in Gk, in log2 units (Gamma log2(e), for the exp2 of every
            // decay factor): each thread scans CH/PARTS rows of one channel, then adds the
            // totals of the parts above it
            // The parts' totals go through the Ms tile, unused until the preparation.
            constexpr int PARTS = NT / DK, RP = CH / PARTS;
            static_assert(PARTS * DK * 4 <= C::SZ_MS, "part totals");
            const int c = tid % DK, part = tid / DK;
            float *tot = (float *)(smem + zo + C::OFF_M);
            float xs[RP];
            float run = 0.f;
#pragma unroll
            for (int j = 0; j < RP; ++j) {
                run += Gk[(part * RP + j) * LDG + c] * kLog2e;
                xs[j] = run;
            }
            tot[part * DK + c] = run;
            __syncthreads();
            float add = 0.f;
#pragma unroll
            for (int pp = 0; pp < PARTS - 1; ++pp) {
                float t = tot[pp * DK + c];  // read by every lane, then selected
                asm volatile("" : "+v"(t));
                add += pp < part ? t : 0.f;
            }
#pragma unroll
            for (int j = 0; j < RP; ++j)
                Gk[(part * RP + j) * LDG + c] = xs[j] + add;
            __syncthreads();
        }
        const float gC = graw[CH - 1];  // graw holds Gamma (written in stage A)
        float gr[NB][4];  // Gamma at the D-layout rows 16I + 4g + i of this lane
#pragma unroll
        for (int I = 0; I < NB; ++I) {
            const f32x4 v = *reinterpret_cast<const f32x4 *>(graw + 16 * I + 4 * g4);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                gr[I][i] = v[i];
        }
        float gcol[NB];  // Gamma at the D-layout columns 16J + c of this lane
#pragma unroll
        for (int J = 0; J < NB; ++J)
            gcol[J] = graw[16 * J + c16];

        // The previous chunk's o goes out now, behind this stage's arithmetic; the next
        // chunk's rows are requested at the start of the state stage. (Issued together
        // right after the loads above, they would hold every wave while the CU's
        // vector-memory path drains.)
        if (C::STAGE_O && cs - CH >= o_start && cs > start)
            flush_o(Os, cs - CH, CH, tid);  // only the last chunk of a stream is partial

        // Two waves share a SIMD and the older one wins every issue slot: without help the
        // second wave of each SIMD (waves 4-7) reaches each barrier last. They get the
        // higher priority from here to the end of the K h / Q h products.
        if (NW == 8 && wave >= 4)
            __builtin_amdgcn_s_setprio(1);

        // K h and Q h need only this chunk's tiles and the state: with one column block per
        // wave they run here, before the preparation's barrier, where they fill the time
        // the waves without a diagonal inversion would otherwise wait (not with the
        // per-channel gate, whose tiles are rescaled after the preparation; measured -2%
        // per chunk on the segmented 4096-token stream)
        constexpr bool EARLY = NCB == 1 && !KDA;
        float ar[NB][4], dr[NB][4];  // a_r = e^Gamma_r and a_C / a_r at this lane's rows
#pragma unroll
        for (int I = 0; I < NB; ++I) {
            const f32x4 va = *reinterpret_cast<const f32x4 *>(ea + 16 * I + 4 * g4);
            const f32x4 vd = *reinterpret_cast<const f32x4 *>(ed + 16 * I + 4 * g4);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ar[I][i] = va[i], dr[I][i] = vd[i];
        }
        f32x4 xe[EARLY ? NB : 1], oe[EARLY ? NB : 1];
        if constexpr (EARLY)
            kh_qh(0, xe, oe, ar, Ks, Qs, Vs, wave, lane, g4, c16, L);

        // ---- C: M = strict_tril(diag(beta) K K^T . decay), P = tril(Q K^T . decay) ------
        // The 10 lower 16x16 blocks (I, J), numbered row by row. Waves 0-3 each take one
        // diagonal block and invert it right away, T_II = (I + M_II)^-1; the 6 blocks below
        // the diagonal are spread over the other waves (8 waves) or the same ones (4 waves).
        // Both products of a block share the K_J operand. T_II and the off-diagonal M_IJ go
        // to the MT tile (fp16), P to Ps/Psl as an fp16 hi + lo pair.
        constexpr int NJ = NB == 2 ? 1 : NW == 8 ? 2 : 3;
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb) {
            const int code = block_task<NW, NB>(wave, jb);
            if (code < 0)
                break;
            const int p = code & 15, part = code >> 4;
            const bool do_m = part != 2, do_p = part != 1 && write_o;  // P only feeds o
            const int I = p < 1 ? 0 : p < 3 ? 1 : p < 6 ? 2 : 3;
            const int J = p - I * (I + 1) / 2;
            f32x4 am = zero4(), ap = zero4();
            // D layout -> A layout through LDS, in this diagonal block's own corner of Ms or
            // (fused front end) its own scratch block (no other wave touches it)
            float *scr = C::XSCR ? Xs + 16 * I * C::LDX : Ms + 16 * I * LDF + 16 * I;
            constexpr int lds = C::XSCR ? C::LDX : LDF;
            auto to_a = [&](const f32x4 &d) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    scr[(4 * g4 + i) * lds + c16] = d[i];
                return blk_a(scr, lds, 0, 0, lane);
            };
            // T_II = (I - N)^-1 with N = -M_II strictly lower (N^16 = 0):
            // (I + N)(I + N^2)(I + N^4)(I + N^8), the products on fp32 MFMA; step(k) is
            // called between the inverse's dependent steps (k = 0..3) to issue independent
            // work into their latency
            // After a step, which may branch around its work, the inverse reads the fp32
            // MFMA result issued before it: the wait states that read needs are kept here,
            // at the join, since the compiler counted them only along the path through the
            // step's work (on the other path the d = 64 instance read the result too early
            // and got wrong transitions and end states whenever a chunk computed no o).
            auto settle = [] {
                __builtin_amdgcn_sched_barrier(0);
                asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
            };
            auto invert = [&](const f32x4 &m, auto step) {
                f32x4 nb;  // N, D layout
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    nb[i] = -m[i];
                const f32x4 na = to_a(nb);
                step(0);
                f32x4 n2 = zero4(), n3 = zero4(), n4 = zero4(), n8 = zero4();
                mm16<false>(n2, na, nb);  // N^2
                step(1);
                settle();
                mm16<false>(n3, na, n2);  // N^3
                const f32x4 n2a = to_a(n2);
                step(2);
                settle();
                mm16<false>(n4, n2a, n2);  // N^4
                const f32x4 n4a = to_a(n4);
                step(3);
                settle();
                mm16<false>(n8, n4a, n4);  // N^8
                const f32x4 n8a = to_a(n8);
                f32x4 x;  // (I + N)(I + N^2) = I + N + N^2 + N^3
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    x[i] = ((4 * g4 + i) == c16 ? 1.f : 0.f) + nb[i] + n2[i] + n3[i];
                f32x4 y = x;
                mm16<false>(y, n4a, x);  // (I + N^4) X
                f32x4 z = y;
                mm16<false>(z, n8a, y);  // (I + N^8) Y
                return z;
            };
            if (!KDA && FRONT && I == J) {
                // Diagonal block, scalar gate (fused front end; the register-path instances
                // have no registers to hold K_I across the inverse): M_II first, then its
                // inverse with P_II's products issued between the inverse's dependent steps,
                // then P_II's stores.
                const int base = 16 * I, s = base + c16;
                frag kf[DK / 32];
#pragma unroll
                for (int kb = 0; kb < DK / 32; ++kb) {
                    kf[kb] = ld_frag_qk<DK>(Ks, base, 32 * kb, lane);
                    mma(am, kf[kb], kf[kb]);
                }
                const f32x4 bet4 = *reinterpret_cast<const f32x4 *>(bet + base + 4 * g4);
                float gs = gcol[0];
#pragma unroll
                for (int jj = 1; jj < NB; ++jj)
                    gs = I == jj ? gcol[jj] : gs;
                float dec[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = base + 4 * g4 + i;
                    float grr = gr[0][i];
#pragma unroll
                    for (int ii = 1; ii < NB; ++ii)
                        grr = I == ii ? gr[ii][i] : grr;
                    dec[i] = __expf(grr - gs);  // e^(G_r - G_s); the upper part is masked
                    am[i] = s < r ? bet4[i] * dec[i] * am[i] : 0.f;
                }
                auto p_step = [&](int kb) {  // the inverse has 4 steps, DK / 32 <= 4
                    static_assert(DK / 32 <= 4, "P steps");
                    if (!do_p || kb >= DK / 32)
                        return;
                    if constexpr (FRONT) {
                        // Q K^T with q and k as fp16 hi + lo pairs (the lo x lo term is below
                        // fp32 rounding)
                        const frag qh8 = ld_frag_qk<DK>(Qs, base, 32 * kb, lane);
                        mma(ap, qh8, kf[kb]);
                        mma(ap, qh8, ld_frag_qk<DK>(Kl, base, 32 * kb, lane));
                        mma(ap, ld_frag_qk<DK>(Ql, base, 32 * kb, lane), kf[kb]);
                    } else {
                        mma(ap, ld_frag_qk<DK>(Qs, base, 32 * kb, lane), kf[kb]);
                    }
                };
                const f32x4 z = invert(am, p_step);
                if (do_p) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = base + 4 * g4 + i;
                        const float pv_ = s <= r ? dec[i] * ap[i] : 0.f;
                        const T phi = (T)pv_;
                        Ps[r * LDT + s] = phi;
                        if constexpr (SPLIT)
                            Psl[r * LDT + s] = (T)(pv_ - (float)phi);
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    MTh[(base + 4 * g4 + i) * LDT + base + c16] = (T)z[i];
                continue;
            }
            if constexpr (!KDA) {
#pragma unroll
                for (int kb = 0; kb < DK / 32; ++kb) {
                    const frag fb = ld_frag_qk<DK>(Ks, 16 * J, 32 * kb, lane);
                    if (do_m)
                        mma(am, ld_frag_qk<DK>(Ks, 16 * I, 32 * kb, lane), fb);
                    if (do_p) {
                        if constexpr (FRONT) {
                            // Q K^T with q and k as fp16 hi + lo pairs (the lo x lo term is
                            // below fp32 rounding)
                            const frag qh8 = ld_frag_qk<DK>(Qs, 16 * I, 32 * kb, lane);
                            mma(ap, qh8, fb);
                            mma(ap, qh8, ld_frag_qk<DK>(Kl, 16 * J, 32 * kb, lane));
                            mma(ap, ld_frag_qk<DK>(Ql, 16 * I, 32 * kb, lane), fb);
                        } else {
                            mma(ap, ld_frag_qk<DK>(Qs, 16 * I, 32 * kb, lane), fb);
                        }
                    }
                }
            } else if (I != J) {
                // off-diagonal block: reference row b = 16I (first row of block I), so
                // both factors e^(G_r - G_b) (r >= b) and e^(G_b - G_s) (s < b) are <= 1
                const float *gb = Gk + 16 * I * LDG;
                const float *gr_ = Gk + (16 * I + c16) * LDG;
                const float *gs_ = Gk + (16 * J + c16) * LDG;
#pragma unroll
                for (int kb = 0; kb < DK / 32; ++kb) {
                    const int c0 = 32 * kb + 4 * g4;
                    const f32x4 b0 = *reinterpret_cast<const f32x4 *>(gb + c0);
                    const f32x4 b1 = *reinterpret_cast<const f32x4 *>(gb + c0 + 16);
                    const f32x4 r0 = *reinterpret_cast<const f32x4 *>(gr_ + c0);
                    const f32x4 r1 = *reinterpret_cast<const f32x4 *>(gr_ + c0 + 16);
                    const f32x4 s0 = *reinterpret_cast<const f32x4 *>(gs_ + c0);
                    const f32x4 s1 = *reinterpret_cast<const f32x4 *>(gs_ + c0 + 16);
                    f32x4 ea0, ea1, eb0, eb1;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        ea0[i] = __builtin_amdgcn_exp2f(r0[i] - b0[i]);
                        ea1[i] = __builtin_amdgcn_exp2f(r1[i] - b1[i]);
                        eb0[i] = __builtin_amdgcn_exp2f(b0[i] - s0[i]);
                        eb1[i] = __builtin_amdgcn_exp2f(b1[i] - s1[i]);
                    }
                    const frag fb = ld_frag_qk<DK>(Ks, 16 * J, 32 * kb, lane);
                    if constexpr (SPLIT) {
                        // k in about fp32 (hi + lo) before the factors are applied; the
                        // fragment's elements 0-3 and 4-7 are channels c0 + 0..3, c0 + 16..19
                        auto lo4 = [](const frag &f) {
                            return __builtin_shufflevector(f, f, 0, 1, 2, 3);
                        };
                        auto hi4 = [](const frag &f) {
                            return __builtin_shufflevector(f, f, 4, 5, 6, 7);
                        };
                        auto wid = [&](const frag &h, const frag *l, bool upper) {
                            if constexpr (C::KLO)
                                return upper ? widen_hl4(hi4(h), hi4(*l))
                                             : widen_hl4(lo4(h), lo4(*l));
                            else
                                return __builtin_convertvector(upper ? hi4(h) : lo4(h), f32x4);
                        };
                        auto pack = [](const f32x4 &x0, const f32x4 &x1) {
                            const f16x4 h0 = __builtin_convertvector(x0, f16x4);
                            const f16x4 h1 = __builtin_convertvector(x1, f16x4);
                            return __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
                        };
                        frag fbl{};
                        if constexpr (C::KLO)
                            fbl = ld_frag_qk<DK>(Kl, 16 * J, 32 * kb, lane);
                        const frag gbf = pack(wid(fb, &fbl, false) * eb0,
                                              wid(fb, &fbl, true) * eb1);
                        if (do_m) {
                            const frag fk = ld_frag_qk<DK>(Ks, 16 * I, 32 * kb, lane);
                            frag fkl{};
                            if constexpr (C::KLO)
                                fkl = ld_frag_qk<DK>(Kl, 16 * I, 32 * kb, lane);
                            mma(am, pack(wid(fk, &fkl, false) * ea0, wid(fk, &fkl, true) * ea1),
                                gbf);
                        }
                        if (do_p) {
                            const frag fq = ld_frag_qk<DK>(Qs, 16 * I, 32 * kb, lane);
                            mma(ap, pack(widen_mul4(lo4(fq), ea0), widen_mul4(hi4(fq), ea1)),
                                gbf);
                        }
                    } else {
                        frag fk = ld_frag_qk<DK>(Ks, 16 * I, 32 * kb, lane);
                        frag fq = ld_frag_qk<DK>(Qs, 16 * I, 32 * kb, lane);
                        frag fbs = fb;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            fk[i] *= ea0[i];
                            fk[4 + i] *= ea1[i];
                            fq[i] *= ea0[i];
                            fq[4 + i] *= ea1[i];
                            fbs[i] *= eb0[i];
                            fbs[4 + i] *= eb1[i];
                        }
                        if (do_m)
                            mma(am, fk, fbs);
                        if (do_p)
                            mma(ap, fq, fbs);
                    }
                }
            } else {
                // diagonal block: mid-block reference m = 16I + 8, so each factor spans at
                // most 8 tokens of decay (exponents clamped at 80, 80 log2(e) in the log2
                // units of Gk). The gated operands can exceed the fp16 range, so the block's
                // products run on fp32 MFMA, whose A and B elements of a lane come from one
                // row and one channel: lane (g, c) takes row 16I + c and, over the 32 steps,
                // channels 32g .. 32g + 31 (the contraction order is free), read as 4-element
                // chunks of the tiles (k as its hi + lo pair).
                const float *gm = Gk + (16 * I + 8) * LDG;
                const float *grs = Gk + (16 * I + c16) * LDG;
                if constexpr (SPLIT) {
                    typedef T T4 __attribute__((ext_vector_type(4)));
                    const int r = 16 * I + c16;
#pragma unroll
                    for (int jj = 0; jj < DK / 16; ++jj) {
                        const int q4 = (DK / 16) * g4 + jj;  // 4-channel chunk
                        const int off = QK<T, DK>::at(r, q4);
                        const T4 kh4 = *reinterpret_cast<const T4 *>(Ks + off);
                        const T4 qh4 = *reinterpret_cast<const T4 *>(Qs + off);
                        T4 kl4{};
                        if constexpr (C::KLO)
                            kl4 = *reinterpret_cast<const T4 *>(Kl + off);
                        const f32x4 gr4 = *reinterpret_cast<const f32x4 *>(grs + 4 * q4);
                        const f32x4 gm4 = *reinterpret_cast<const f32x4 *>(gm + 4 * q4);
                        f32x4 ea4, eb4;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float d = gr4[e] - gm4[e];
                            ea4[e] = __builtin_amdgcn_exp2f(fminf(d, kExpCap));
                            eb4[e] = __builtin_amdgcn_exp2f(fminf(-d, kExpCap));
                        }
                        f32x4 kx4;
                        if constexpr (C::KLO)
                            kx4 = widen_hl4(__builtin_bit_cast(f16x4, kh4),
                                            __builtin_bit_cast(f16x4, kl4));
                        else
                            kx4 = __builtin_convertvector(__builtin_bit_cast(f16x4, kh4), f32x4);
                        const f32x4 ka4 = kx4 * ea4, kb4 = kx4 * eb4;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            am = __builtin_amdgcn_mfma_f32_16x16x4f32(ka4[e], kb4[e], am, 0, 0, 0);
                        if (do_p) {
                            const f32x4 qa4 = widen_mul4(__builtin_bit_cast(f16x4, qh4), ea4);
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                ap = __builtin_amdgcn_mfma_f32_16x16x4f32(qa4[e], kb4[e], ap, 0,
                                                                          0, 0);
                        }
                    }
                } else {
                    const T *kr = Ks + (16 * I + c16) * LDQ;
                    const T *qr = Qs + (16 * I + c16) * LDQ;
#pragma unroll 8
                    for (int j4 = 0; j4 < DK / 4; ++j4) {
                        const int ch = 4 * j4 + g4;
                        const float d = grs[ch] - gm[ch];
                        const float ea = __builtin_amdgcn_exp2f(fminf(d, kExpCap));
                        const float bv = (float)kr[ch] * __builtin_amdgcn_exp2f(fminf(-d, kExpCap));
                        am = __builtin_amdgcn_mfma_f32_16x16x4f32((float)kr[ch] * ea, bv, am, 0,
                                                                  0, 0);
                        ap = __builtin_amdgcn_mfma_f32_16x16x4f32((float)qr[ch] * ea, bv, ap, 0,
                                                                  0, 0);
                    }
                }
            }
            const int s = 16 * J + c16;
            // this lane's betas (rows 16 I + 4 g + i), read whether or not a row is used, so
            // that the selects below stay selects
            const f32x4 bet4 = *reinterpret_cast<const f32x4 *>(bet + 16 * I + 4 * g4);
            float gs = gcol[0];
#pragma unroll
            for (int jj = 1; jj < NB; ++jj)
                gs = J == jj ? gcol[jj] : gs;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * I + 4 * g4 + i;
                float grr = gr[0][i];
#pragma unroll
                for (int ii = 1; ii < NB; ++ii)
                    grr = I == ii ? gr[ii][i] : grr;
                // decay e^(G_r - G_s) for s <= r (the per-channel gate has it inside the
                // products); the masked upper part is discarded by the selects below
                const float dec = KDA ? 1.f : __expf(grr - gs);
                if (do_p) {
                    const float pv_ = s <= r ? dec * ap[i] : 0.f;
                    const T phi = (T)pv_;
                    Ps[r * LDT + s] = phi;
                    if constexpr (SPLIT)
                        Psl[r * LDT + s] = (T)(pv_ - (float)phi);
                }
                const float mv = s < r ? bet4[i] * dec * am[i] : 0.f;
                am[i] = mv;
                if (I != J && do_m)
                    MTh[r * LDT + s] = (T)mv;
            }
            if (I == J) {
                const f32x4 z = invert(am, [](int) {});
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    MTh[(16 * I + 4 * g4 + i) * LDT + 16 * I + c16] = (T)z[i];
            }
        }
        __syncthreads();
        T *Kd = (T *)(smem + zo + C::OFF_M);  // per-channel gate: (K . e^(G_C - G)), over Ms
        if constexpr (KDA) {
            // Ks <- K . e^G, Qs <- Q . e^G, Kd <- K . e^(G_C - G): every factor is <= 1.
            // A thread owns 4 channels of NI rows (the same channels in each, so G_C is read
            // once); all its tile reads are issued before the exponentials, as 4-element
            // vectors.
            typedef T T4 __attribute__((ext_vector_type(4)));
            constexpr int NI = CH * (DK / 4) / NT;
            static_assert(NI * NT == CH * (DK / 4) && NT % (DK / 4) == 0, "rescale map");

            const int c0 = (tid % (DK / 4)) * 4, r0 = tid / (DK / 4);
            // (k = hi + lo; the K lo tile then takes the lo half of K e^(G_C - G))
            const f32x4 gcv = *reinterpret_cast<const f32x4 *>(Gk + (CH - 1) * LDG + c0);
            // e^(G_C) per channel, for the state update
            if (r0 == 0) {
                f32x4 e;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    e[i] = __builtin_amdgcn_exp2f(gcv[i]);
                *reinterpret_cast<f32x4 *>(graw + 4 * CH + c0) = e;
            }
            T4 kv[NI], klv[NI], qv[NI];
            f32x4 gv[NI];
#pragma unroll
            for (int it = 0; it < NI; ++it) {
                const int r = r0 + it * (NT / (DK / 4));
                const int off = QK<T, DK>::at(r, c0 / 4);
                kv[it] = *reinterpret_cast<const T4 *>(Ks + off);
                if constexpr (C::KLO)
                    klv[it] = *reinterpret_cast<const T4 *>(Kl + off);
                qv[it] = *reinterpret_cast<const T4 *>(Qs + off);
                gv[it] = *reinterpret_cast<const f32x4 *>(Gk + r * LDG + c0);
            }
#pragma unroll
            for (int it = 0; it < NI; ++it) {
                const int r = r0 + it * (NT / (DK / 4));
                const int off = QK<T, DK>::at(r, c0 / 4);
                T4 kd, kdl, ke, qe;
                f32x4 e4, d4;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    e4[i] = __builtin_amdgcn_exp2f(gv[it][i]);
                    d4[i] = __builtin_amdgcn_exp2f(gcv[i] - gv[it][i]);
                }
                if constexpr (SPLIT) {
                    const f16x4 k16 = __builtin_bit_cast(f16x4, kv[it]);
                    f32x4 kx4;
                    if constexpr (C::KLO)
                        kx4 = widen_hl4(k16, __builtin_bit_cast(f16x4, klv[it]));
                    else
                        kx4 = __builtin_convertvector(k16, f32x4);
                    f16x4 h4, l4;
                    split4(kx4 * d4, h4, l4);
                    kd = __builtin_bit_cast(T4, h4);
                    kdl = __builtin_bit_cast(T4, l4);
                    ke = __builtin_bit_cast(T4, __builtin_convertvector(kx4 * e4, f16x4));
                    qe = __builtin_bit_cast(
                        T4, __builtin_convertvector(
                                widen_mul4(__builtin_bit_cast(f16x4, qv[it]), e4), f16x4));
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float kx = kv[it][i];
                        kd[i] = kx * d4[i];
                        ke[i] = kx * e4[i];
                        qe[i] = qv[it][i] * e4[i];
                    }
                }
                *reinterpret_cast<T4 *>(Kd + off) = kd;
                if constexpr (C::KLO)
                    *reinterpret_cast<T4 *>(Kl + off) = kdl;
                *reinterpret_cast<T4 *>(Ks + off) = ke;
                *reinterpret_cast<T4 *>(Qs + off) = qe;
            }
            __syncthreads();
        }

        // Per-key-channel gate with the front end fused: K h, Q h and the v conv run here,
        // on the rescaled tiles, so that Q, K and the raw v rows are dead before the next
        // chunk's raw rows land on them
        constexpr bool LATE = FRONT && KDA;
        f32x4 xl[LATE ? NB : 1], ol[LATE ? NB : 1];
        if constexpr (LATE) {
            kh_qh(0, xl, ol, ar, Ks, Qs, Vs, wave, lane, g4, c16, L);
            __syncthreads();
        }
        const bool pf = cs + CH < end;  // the next chunk's rows and gates
        const int pfL = (int)min((int64_t)CH, end - cs - CH);
        if (pf)
            prefetch(cs + CH, pfL, false);
        if (FRONT && pf)
            prefetch_group(cs + CH, pfL, 0);
        if constexpr (GATE) {
            if (write_o)
                load_z(cs, L, lane, wave);
        }

        // ---- F: state products for this wave's 16*NCB columns -------------------------
        //   X = V - diag(a) K h,  U = T diag(beta) X,  O = diag(a) Q h + P U,
        //   h <- a_C h + K^T diag(a_C / a) U
        const float aC = ea[CH - 1];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            f32x4 x[NB], o[NB];
            if constexpr (EARLY) {
#pragma unroll
                for (int I = 0; I < NB; ++I)
                    x[I] = xe[I], o[I] = oe[I];
            } else if constexpr (LATE) {
#pragma unroll
                for (int I = 0; I < NB; ++I)
                    x[I] = xl[I], o[I] = ol[I];
            } else {
                kh_qh(cb, x, o, ar, Ks, Qs, Vs, wave, lane, g4, c16, L);
            }
            if (NW == 8 && wave >= 4 && cb == NCB - 1)
                __builtin_amdgcn_s_setprio(0);
            // U = T diag(beta) X by block forward substitution on (I + M) U = diag(beta) X:
            // U_I = T_II (beta X_I - sum_{J<I} M_IJ U_J), right-hand sides as hi + lo pairs
            // (fp16 operands: each U block is split into hi + lo once, for the later blocks
            // and for P U)
            f32x4 u[NB];
            f16x4 uhs[NB], uls[NB];
            // fp16 operands: the blocks of MT (T_II and M_IJ, J < I) and this lane's betas are
            // all read before the substitution starts, so that its chain of dependent
            // products waits on LDS once
            f16x4 mt[SPLIT ? NB * (NB + 1) / 2 : 1];
            f32x4 bt[NB];
#pragma unroll
            for (int I = 0; I < NB; ++I) {
                bt[I] = *reinterpret_cast<const f32x4 *>(bet + 16 * I + 4 * g4);
                if constexpr (SPLIT) {
#pragma unroll
                    for (int J = 0; J <= I; ++J)
                        mt[I * (I + 1) / 2 + J] = *reinterpret_cast<const f16x4 *>(
                            (const T *)MTh + (16 * I + c16) * LDT + 16 * J + 4 * g4);
                }
            }
#pragma unroll
            for (int I = 0; I < NB; ++I) {
                f32x4 acc = zero4();
#pragma unroll
                for (int J = 0; J < I; ++J) {
                    if constexpr (SPLIT)
                        mm16_frag(acc, mt[I * (I + 1) / 2 + J], uhs[J], uls[J]);
                    else
                        mm16_pre(acc, MTh, LDT, I, J, u[J], lane);
                }
                f32x4 z;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    z[i] = bt[I][i] * x[I][i] - acc[i];
                u[I] = zero4();
                if constexpr (SPLIT) {
                    f16x4 zh, zl;
                    split4(z, zh, zl);
                    mm16_frag(u[I], mt[I * (I + 1) / 2 + I], zh, zl);
                    split4(u[I], uhs[I], uls[I]);
                } else {
                    mm16_pre(u[I], MTh, LDT, I, I, z, lane);
                }
            }
            if (FRONT && pf)
                prefetch_group(cs + CH, pfL, 1);
            // O += P U with P and U as hi + lo pairs
            if (write_o) {
                // 32-deep column blocks of P (16-row pairs of U)
                constexpr int NKB = NB / 2;
                frag uh[NKB], ul[NKB];
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    if constexpr (SPLIT) {
                        uh[kb] = __builtin_shufflevector(uhs[2 * kb], uhs[2 * kb + 1], 0, 1, 2,
                                                         3, 4, 5, 6, 7);
                        ul[kb] = __builtin_shufflevector(uls[2 * kb], uls[2 * kb + 1], 0, 1, 2,
                                                         3, 4, 5, 6, 7);
                    } else {
                        pack_split<T>(u[2 * kb], u[2 * kb + 1], uh[kb], ul[kb]);
                    }
                }
#pragma unroll
                for (int I = 0; I < NB; ++I) {
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb) {
                        if (kb > (I >> 1))
                            continue;
                        const frag ph = ld_frag(Ps, LDT, 16 * I, 32 * kb, lane);
                        mma(o[I], ph, uh[kb]);
                        if constexpr (SPLIT) {
                            mma(o[I], ph, ul[kb]);
                            mma(o[I], ld_frag(Psl, LDT, 16 * I, 32 * kb, lane), uh[kb]);
                        }
                    }
                    const int col = 16 * (wave * NCB + cb) + c16;
                    if constexpr (!C::STAGE_O) {
                        // The stores below sit behind a branch on the chunk's length. The wait
                        // states an MFMA result needs before it is read are kept here, ahead
                        // of that branch: the compiler counted them only along one path.
                        __builtin_amdgcn_sched_barrier(0);
                        asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    if constexpr (C::STAGE_O) {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            Os[(16 * I + 4 * g4 + i) * LDO + col] = o[I][i];
                    } else if (L == CH) {  // a whole chunk: no per-row test
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            ob[(cs + 16 * I + 4 * g4 + i) * (int64_t)H * DV + col] = o[I][i];
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int r = 16 * I + 4 * g4 + i;
                            if (r < L)
                                ob[(cs + r) * (int64_t)H * DV + col] = o[I][i];
                        }
                    }
                }
            }
            if (FRONT && pf)
                prefetch_group(cs + CH, pfL, 2);
            // h <- a_C h + K^T (diag(a_C / a) U); per-channel gate:
            // h <- diag(e^G_C) h + (K . e^(G_C - G))^T U
            if constexpr (!KDA) {
#pragma unroll
                for (int I = 0; I < NB; ++I)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        u[I][i] *= dr[I][i];
            }
            // U as an fp16 hi + lo pair here too: the state accumulates these products over
            // the whole stream, and heavy-tailed states (max/RMS ~ 50) need U beyond fp16
            // (a single fp16 U left err(h) at 3.3% on such a state; the pair: 1.8%, for
            // 2-4% more time per chunk)
            // (the 32-row halves of the chunk: two at 64 rows, one at 32)
            frag vf0, vf1, vl0, vl1;
            pack_split<T>(u[0], u[1], vf0, vl0);
            if constexpr (NB == 4)
                pack_split<T>(u[2], u[3], vf1, vl1);
#pragma unroll
            for (int mb = 0; mb < DK / 16; ++mb) {
                if constexpr (KDA) {
                    const f32x4 ec =
                        *reinterpret_cast<const f32x4 *>(graw + 4 * CH + 16 * mb + 4 * g4);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        hs[cb][mb][i] *= ec[i];
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        hs[cb][mb][i] *= aC;
                }
                const T *Kt = KDA ? Kd : Ks;
                const frag k0 = ld_frag_t_qk<DK>(Kt, 0, 16 * mb, lane);
                mma(hs[cb][mb], k0, vf0);
                if constexpr (SPLIT)
                    mma(hs[cb][mb], k0, vl0);
                if constexpr (NB == 4) {
                    const frag k1 = ld_frag_t_qk<DK>(Kt, 32, 16 * mb, lane);
                    mma(hs[cb][mb], k1, vf1);
                    if constexpr (SPLIT)
                        mma(hs[cb][mb], k1, vl1);
                }
                if constexpr (C::KLO) {  // the k operand as an fp16 hi + lo pair as well
                    mma(hs[cb][mb], ld_frag_t_qk<DK>(Kl, 0, 16 * mb, lane), vf0);
                    if constexpr (NB == 4)
                        mma(hs[cb][mb], ld_frag_t_qk<DK>(Kl, 32, 16 * mb, lane), vf1);
                }
            }
        }
        __syncthreads();
    }
    const bool zero_transition = underflowed();
    if (zero_transition) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int mb = 0; mb < DK / 16; ++mb)
                hs[cb][mb] = zero4();
    }
    if (zflag && tid0 == 0)  // every transition job writes its flag (the workspace is reused)
        *zflag = zero_transition ? 1.f : 0.f;
    if constexpr (GATE) {  // the last chunk's z tile: every wave's LDS-DMA loads landed
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }
    if (C::STAGE_O && end > o_start && start < end) {  // the last chunk's o (the loop ends
                                                          // on a barrier)
        const int64_t last = start + (end - start - 1) / CH * CH;
        flush_o((const float *)(smem + C::OFF_O), last, (int)(end - last), tid0);
    }

    if (hout) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int mb = 0; mb < DK / 16; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    hout[hoff + (int64_t)(16 * mb + 4 * (lane0 >> 4) + i) * DV + colw + 16 * cb +
                         (lane0 & 15)] = hs[cb][mb][i];
    }
}

template <typename TIN, typename T, int DK, int DV, int NW, int NCB, bool KDA, bool GATE,
          bool FRONT, int CHK>
hipError_t launch_chunk_t(const ChunkArgs &a, int grid, hipStream_t s)
{
    using C = ChunkCfg<T, DK, DV, NW, NCB, KDA, GATE, FRONT, CHK>;
    static_assert(C::BYTES <= 160 * 1024, "LDS budget");
    static_assert(DV % C::NV == 0, "slices");
    auto kern = chunk_kernel<TIN, T, DK, DV, NW, NCB, KDA, GATE, FRONT, CHK>;
    static bool attr_set = false;  // per instance; same value on every device
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, C::BYTES);
        if (e != hipSuccess)
            return e;
        attr_set = true;
    }
    ChunkArgs ar = a;
    ar.job_groups = grid;
    const int64_t extra = (a.window_items + NW * 64 - 1) / (NW * 64);
    if ((int64_t)grid + extra > (int64_t)INT32_MAX)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(kern, dim3((unsigned)(grid + extra)), dim3(NW * 64), C::BYTES, s, ar);
    return hipGetLastError();
}

// Instances: (input element, operand type, input kind, dk, dv, waves, column blocks of 16
// per wave, per-channel gate, output gate fused, front end fused, rows per chunk). The
// 32-row instances (register path, no output gate) exist for the chunk-size invariance of
// the results; 64 rows is the default. Input kind: 0 = f32
// rows, 1 = bf16 rows, 2 = fp16 activations of the front kernel, 3 = bf16 raw rows with the
// conv front end fused into the load stage. A workgroup covers NW * NCB * 16 dv columns of one
// (stream, head). The default (widest) shapes that stage o also come with the output gate
// fused into the o flush, where o and the z tile fit in LDS; the per-channel-gate instances
// at 128 columns (o not staged) and fp32 at 64 columns (no room for the z tile) gate o in
// a separate pass (gate_kernel), and so do the dk != dv shapes, whose value rows span two
// workgroups (dv = 2 dk: two column slices of one (stream, head)).
#define GDN_CHUNK_INSTANCES(X)                          \
    X(bf16, f16, 1, 128, 128, 8, 1, false, false, false, 64) \
    X(bf16, f16, 1, 128, 128, 4, 2, false, false, false, 64) \
    X(bf16, f16, 1, 128, 128, 4, 1, false, false, false, 64) \
    X(bf16, f16, 1, 64, 64, 4, 1, false, false, false, 64) \
    X(float, float, 0, 64, 64, 4, 1, false, false, false, 64) \
    X(bf16, f16, 1, 128, 128, 8, 1, true, false, false, 64) \
    X(bf16, f16, 1, 128, 128, 4, 1, true, false, false, 64) \
    X(bf16, f16, 1, 64, 64, 4, 1, true, false, false, 64) \
    X(float, float, 0, 64, 64, 4, 1, true, false, false, 64) \
    X(bf16, f16, 1, 128, 128, 8, 1, false, true, false, 64) \
    X(bf16, f16, 1, 64, 64, 4, 1, false, true, false, 64) \
    X(float, float, 0, 64, 64, 4, 1, false, true, false, 64) \
    X(bf16, f16, 1, 64, 64, 4, 1, true, true, false, 64) \
    X(bf16, f16, 1, 128, 256, 8, 1, false, false, false, 64) \
    X(bf16, f16, 1, 128, 256, 8, 1, true, false, false, 64) \
    X(float, float, 0, 64, 128, 4, 1, false, false, false, 64) \
    X(float, float, 0, 64, 128, 4, 1, true, false, false, 64) \
    X(bf16, f16, 3, 128, 128, 8, 1, false, false, true, 64) \
    X(bf16, f16, 3, 128, 128, 8, 1, false, true, true, 64) \
    X(bf16, f16, 3, 64, 64, 4, 1, false, false, true, 64) \
    X(bf16, f16, 3, 64, 64, 4, 1, false, true, true, 64) \
    X(bf16, f16, 3, 128, 128, 8, 1, true, false, true, 64) \
    X(bf16, f16, 3, 64, 64, 4, 1, true, false, true, 64) \
    X(bf16, f16, 3, 128, 256, 8, 1, false, false, true, 64) \
    X(bf16, f16, 3, 128, 256, 8, 1, true, false, true, 64) \
    X(bf16, f16, 1, 128, 128, 8, 1, false, false, false, 32) \
    X(bf16, f16, 1, 128, 128, 8, 1, true, false, false, 32) \
    X(float, float, 0, 64, 64, 4, 1, false, false, false, 32) \
    X(float, float, 0, 64, 64, 4, 1, true, false, false, 32)

// nv: dv columns per workgroup; waves: 0 = the default for that width; gate: the instance
// with the output gate fused; chunk: rows per chunk
hipError_t launch_chunk(int in_kind, int dk, int dv, int kda, int nv, int waves, int gate,
                        int chunk, const ChunkArgs &a, int grid, hipStream_t s)
{
#define X(TIN, T, IK, DK, DV, NW, NCB, KD, G, F, CK)                                   \
    if (in_kind == IK && dk == DK && dv == DV && nv == 16 * NW * NCB && !kda == !KD && \
        (waves == 0 || waves == NW) && !gate == !G && chunk == CK)                     \
        return launch_chunk_t<TIN, T, DK, DV, NW, NCB, KD, G, F, CK>(a, grid, s);
    GDN_CHUNK_INSTANCES(X)
#undef X
    return hipErrorInvalidValue;
}

int chunk_instance_exists(int in_kind, int dk, int dv, int kda, int nv, int waves, int gate,
                          int chunk)
{
#define X(TIN, T, IK, DK, DV, NW, NCB, KD, G, F, CK)                                   \
    if (in_kind == IK && dk == DK && dv == DV && nv == 16 * NW * NCB && !kda == !KD && \
        (waves == 0 || waves == NW) && !gate == !G && chunk == CK)                     \
        return 1;
    GDN_CHUNK_INSTANCES(X)
#undef X
    return 0;
}

hipError_t launch_warm_boundaries(const WarmArgs &a, int kda, int dk, hipStream_t s)
{
    const int64_t grid = (int64_t)a.st.B * a.H * (a.nseg - 1);
    if (a.nseg < 3 || a.seg0_len % CH || a.seg_len % CH || grid > (int64_t)INT32_MAX)
        return hipErrorInvalidValue;
    if (!kda)
        hipLaunchKernelGGL((warm_boundary_kernel<false, 0>), dim3((unsigned)grid), dim3(256), 0,
                           s, a);
    else if (dk == 128)
        hipLaunchKernelGGL((warm_boundary_kernel<true, 128>), dim3((unsigned)grid), dim3(1024),
                           0, s, a);
    else if (dk == 64)
        hipLaunchKernelGGL((warm_boundary_kernel<true, 64>), dim3((unsigned)grid), dim3(1024),
                           0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

// Debug validation (see ValidateArgs): grid-stride over the B + 1 entries of cu_seqlens
// and the ng log-gates; one atomic OR per wave that found something.
__global__ void __launch_bounds__(256) validate_kernel(const ValidateArgs a)
{
    uint32_t bad = 0;
    const int64_t stride = (int64_t)gridDim.x * 256;
    const int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (a.cu) {
        for (int64_t b = i0; b <= a.B; b += stride) {
            const int32_t c = a.cu[b];
            if (b == 0 && c != 0)
                bad |= GDN_BAD_CU_START;
            if (b == a.B && (int64_t)c != a.total)
                bad |= GDN_BAD_CU_TOTAL;
            if (b < a.B) {
                const int32_t d = a.cu[b + 1];
                if (d < c)
                    bad |= GDN_BAD_CU_ORDER;
                else if (d - c > a.max_seqlen)
                    bad |= GDN_BAD_CU_MAXLEN;
            }
        }
    }
    if (a.g) {
        for (int64_t e = i0; e < a.ng; e += stride)
            if (!(a.g[e] <= 0.f))  // a NaN is no decay either
                bad |= GDN_BAD_KDA_GATE;
    }
    for (int m = 32; m >= 1; m >>= 1)
        bad |= (uint32_t)__shfl_xor((int)bad, m);
    if ((threadIdx.x & 63) == 0 && bad)
        atomicOr(a.status, (int32_t)bad);
}

hipError_t launch_validate(const ValidateArgs &a, hipStream_t s)
{
    const int64_t n = max((int64_t)a.B + 1, a.ng);
    const int64_t blocks = min((n + 255) / 256, (int64_t)4096);
    hipLaunchKernelGGL(validate_kernel, dim3((unsigned)max(blocks, (int64_t)1)), dim3(256), 0,
                       s, a);
    return hipGetLastError();
}

// One thread per (stream, window entry): the staged windows to the caller's.
__global__ void __launch_bounds__(256) window_copy_kernel(const WindowCopyArgs a)
{
    if (debug_stop(a.dbg))
        return;
    const int64_t per = (int64_t)a.cd * a.W;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)a.st.B * per)
        return;
    const int b = (int)(i / per);
    const int64_t e = i - (int64_t)b * per;
    int64_t sb, eb;
    stream_bounds(a.st, b, sb, eb);
    if (eb <= sb)
        return;
    uint16_t *cw = (uint16_t *)(a.conv_state_ptrs ? a.conv_state_ptrs[b] : a.conv_state);
    cw[e] = ((const uint16_t *)a.win_ws)[i];
}

hipError_t launch_window_copy(const WindowCopyArgs &a, hipStream_t s)
{
    const int64_t n = (int64_t)a.st.B * a.cd * a.W;
    if (n < 1 || (n + 255) / 256 > (int64_t)INT32_MAX)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(window_copy_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       a);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------
// varlen chunk table: one block, streams handled CT_THREADS at a time

constexpr int CT_THREADS = 256;

// Streams ranked by length, longest first: with more workgroups than CUs, the longest
// streams then start in the first round instead of waiting behind short ones (list
// scheduling, longest first). One thread per stream counts the streams ahead of it.
__global__ void __launch_bounds__(256) stream_order_kernel(const int32_t *cu, int32_t B,
                                                           int32_t *order)
{
    __shared__ int32_t len[1024];
    for (int i = threadIdx.x; i < B; i += 256)
        len[i] = cu[i + 1] - cu[i];
    __syncthreads();
    for (int b = threadIdx.x; b < B; b += 256) {
        const int32_t lb = len[b];
        int rank = 0;
        for (int j = 0; j < B; ++j)
            rank += len[j] > lb || (len[j] == lb && j < b);
        order[rank] = b;
    }
}

hipError_t launch_stream_order(const int32_t *cu, int32_t B, int32_t *order, hipStream_t s)
{
    if (B < 1 || B > 1024)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_order_kernel, dim3(1), dim3(256), 0, s, cu, B, order);
    return hipGetLastError();
}

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
