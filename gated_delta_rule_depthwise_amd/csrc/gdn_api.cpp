// gdn_api.cpp -- the C ABI of libgdn: host-side validation, workspace carving and launches.
//
// Every check runs before anything is enqueued, so a refused call changes no buffer (page
// "metrale_model_arch/glm5next_kda/prefill.rs": a call outside 1..=max_tokens tokens is
// refused before a launch). Device memory is never read on the host.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <utility>
#include <vector>

#include "gdn.h"
#include "gdn_internal.h"

using gdn::ChunkArgs;
using gdn::FrontArgs;
using gdn::Streams;

namespace {

// ---- stage timing: hipEvents around each kernel of a call, on the call's stream ------
namespace prof {
std::atomic<bool> enabled{false};
std::mutex mu;
struct Rec {
    int bucket;
    hipEvent_t a, b;
};
std::vector<Rec> pending;
std::vector<hipEvent_t> pool;

hipEvent_t take()
{
    std::lock_guard<std::mutex> g(mu);
    if (!pool.empty()) {
        hipEvent_t e = pool.back();
        pool.pop_back();
        return e;
    }
    // timing only: no system-scope fence (cache write-back) when the event is recorded,
    // which would add its own cost to the bracketed kernel
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess)
        return nullptr;
    return e;
}
}  // namespace prof

// Records the start of a bucket at construction and its end at done(), when enabled.
struct Stage {
    int bucket;
    hipStream_t s;
    hipEvent_t a = nullptr;
    Stage(int bucket_, hipStream_t s_) : bucket(bucket_), s(s_)
    {
        if (prof::enabled.load(std::memory_order_relaxed)) {
            a = prof::take();
            if (a && hipEventRecord(a, s) != hipSuccess)
                a = nullptr;
        }
    }
    void done()
    {
        if (!a)
            return;
        hipEvent_t b = prof::take();
        if (b && hipEventRecord(b, s) == hipSuccess) {
            std::lock_guard<std::mutex> g(prof::mu);
            prof::pending.push_back({bucket, a, b});
        }
        a = nullptr;
    }
};

// flag-wait bound of the segmented scan (-1: computed per call): see gdn_debug_flag_polls
std::atomic<int32_t> flag_polls{-1};

// debug validation status word (device), or nullptr: see gdn_debug_validate
std::atomic<int32_t *> debug_status{nullptr};

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int elem_bytes(int dtype) { return dtype == GDN_BF16 ? 2 : 4; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int32_t qk_heads(const gdn_params *p) { return p->Hqk ? p->Hqk : p->H; }

int64_t conv_dim(const gdn_params *p)
{
    return 2 * (int64_t)qk_heads(p) * p->dk + (int64_t)p->H * p->dv;
}

// With bf16 rows the front end runs inside the chunk kernel's load stage (conv + SiLU +
// L2 in fp32 on the raw rows, no activation buffer); the kernel forms a chunk's row
// offsets in 32 bits, so it needs row strides below 2^24 elements. With float32 rows it
// runs as a kernel of its own that hands the chunk kernel fp32 activations.
bool fused_front(const gdn_params *p, int kda)
{
    if (p->conv_k < 2 || p->conv_k > 4 || p->dtype != GDN_BF16 || p->ld_qkv >= (1 << 24))
        return false;
    for (int nv : {128, 64})
        if (p->dv % nv == 0 &&
            gdn::chunk_instance_exists(3, p->dk, p->dv, kda, nv, 0, 0, p->chunk))
            return true;
    return false;
}

// input kind of the chunk kernel: 0 = f32 rows (or the front kernel's fp32 activations),
// 1 = bf16 rows, 3 = bf16 raw rows with the front end fused
int in_kind(const gdn_params *p, int kda)
{
    if (p->dtype != GDN_BF16)
        return 0;
    return p->conv_k == 0 ? 1 : 3;
}

// Workgroup shape: dv columns per workgroup and waves per workgroup: the widest compiled
// instance, so that one workgroup per (stream, head) computes the chunk preparation once
// for all its columns and 8-wave instances hide latency with two waves per SIMD.
struct Shape {
    int nv, waves;
};

Shape pick_shape(const gdn_params *p, int kda)
{
    const int ik = in_kind(p, kda);
    for (int nv : {128, 64}) {
        if (p->dv % nv == 0 &&
            gdn::chunk_instance_exists(ik, p->dk, p->dv, kda, nv, 0, 0, p->chunk))
            return Shape{nv, 0};
    }
    return Shape{0, 0};
}

int check_params(const gdn_params *p, int kda)
{
    if (!p)
        return GDN_E_ARG;
    if (p->H < 1 || p->dk < 1 || p->dv < 1 || p->H > 4096)
        return GDN_E_ARG;
    if (p->Hqk < 0 || p->Hqk > p->H || (p->Hqk && p->H % p->Hqk))
        return GDN_E_ARG;
    if (!(p->eps == p->eps) || !(p->scale == p->scale))
        return GDN_E_ARG;
    if (p->dtype != GDN_F32 && p->dtype != GDN_BF16)
        return GDN_E_UNSUPPORTED;
    if (p->chunk != 64 && p->chunk != 32)  // 32: the instances that have it (pick_shape)
        return GDN_E_UNSUPPORTED;
    if (p->conv_k != 0 && (p->conv_k < 2 || p->conv_k > 4))
        return GDN_E_UNSUPPORTED;
    if (p->conv_k != 0 && p->dtype == GDN_BF16 && !fused_front(p, kda))
        return GDN_E_UNSUPPORTED;
    const Shape sh = pick_shape(p, kda);
    if (sh.nv == 0)
        return GDN_E_UNSUPPORTED;
    const int64_t vec = 16 / elem_bytes(p->dtype);
    if (p->ld_qkv < (int64_t)qk_heads(p) * p->dk || p->ld_qkv < (int64_t)p->H * p->dv ||
        p->ld_qkv % vec != 0)
        return GDN_E_ARG;
    if (p->z) {  // output gate (fused, or a separate pass over o rows of dv 64/128/256)
        if (p->dv != 64 && p->dv != 128 && p->dv != 256)
            return GDN_E_UNSUPPORTED;
        if (!p->norm_w || !aligned16(p->z) || !aligned16(p->norm_w) ||
            p->ld_z < (int64_t)p->H * p->dv || p->ld_z % vec != 0 ||
            !(p->norm_eps >= 0.f) || !(p->norm_eps < INFINITY))
            return GDN_E_ARG;
    }
    return GDN_OK;
}

// streams of a varlen call ranked by length (workspace, after the activations)
constexpr int32_t kMaxOrderB = 1024;
size_t order_bytes(int32_t B) { return B <= kMaxOrderB ? align_up((size_t)B * 4) : 0; }

// A fused front end whose windows are read by several workgroups (q/k heads shared by
// value heads, or value heads split into column slices) stages the new windows and copies
// them once every reader is done.
bool win_shared(const gdn_params *p, int kda)
{
    return qk_heads(p) < p->H || pick_shape(p, kda).nv < p->dv;
}

// staged windows of a fused front end: [B][cd][conv_k-1] bf16
size_t win_bytes(const gdn_params *p, int kda, int32_t B)
{
    if (p->conv_k == 0 || !fused_front(p, kda))
        return 0;
    return align_up((size_t)B * (size_t)conv_dim(p) * (p->conv_k - 1) * 2);
}

// at the start of the workspace: the front kernel's activations (float32 rows), or the
// staged windows of a fused front end with shared windows
size_t front_bytes(const gdn_params *p, int kda, int64_t max_tokens, int32_t B)
{
    if (p->conv_k == 0)
        return 0;
    if (fused_front(p, kda))
        return win_shared(p, kda) ? win_bytes(p, kda, B) : 0;
    return align_up((size_t)max_tokens * (size_t)conv_dim(p) * elem_bytes(p->dtype));
}

// ---- segmented scan of long streams -----------------------------------------------------
// With few (stream, head) pairs most CUs would idle while each workgroup walks its stream
// chunk by chunk. Streams of equal length are then cut into S segments: one launch runs
// segment 0 and, for every inner segment, its end state from h = 0 and its dk x dk
// transition (the same recurrence from h = I with v = 0); a second launch chains
// h_{s+1} = A_s h_s + b_s in workgroups at the front of its grid and runs segments 1..S-1
// from their start states.
constexpr int kMaxSeg = 12;
// the kernels read a (stream, head)'s S - 1 warm-start counts one per lane of a wave
static_assert(kMaxSeg - 1 <= 64, "segment boundaries per wave");

int cu_count()
{
    static std::atomic<int> cached{0};
    int n = cached.load();
    if (n > 0)
        return n;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n < 1)
        n = 256;
    cached.store(n);
    return n;
}

struct SegPlan {
    int S;             // 0: no segmentation
    int64_t seg0_len;  // tokens of segment 0
    int64_t seg_len;   // tokens of each inner segment (the last segment takes the rest)
};

// Finishing time of `n` equal jobs of duration `d` dispatched in order onto the CUs, whose
// free times are kept as (time, count) groups sorted by time (a launch's workgroups go to
// the CUs as they free up, one per CU).
struct CuPool {
    std::vector<std::pair<double, int64_t>> free;  // (time, CUs), ascending
    double end = 0.0;
    explicit CuPool(int ncu) : free{{0.0, (int64_t)ncu}} {}
    void run(int64_t n, double d)
    {
        while (n > 0) {
            std::pair<double, int64_t> f = free.front();
            free.erase(free.begin());
            const int64_t m = n < f.second ? n : f.second;
            n -= m;
            if (m < f.second)
                free.insert(free.begin(), {f.first, f.second - m});
            const double t = f.first + d;
            end = t > end ? t : end;
            auto it = free.begin();
            while (it != free.end() && it->first < t)
                ++it;
            if (it != free.end() && it->first == t)
                it->second += m;
            else
                free.insert(it, {t, m});
        }
    }
};

// Relative cost of one chunk step by job kind, measured on the 4096-token front-end
// stream (32 heads, d = 128, all CUs busy): a step that writes o 8.5 us, an end-state job
// from h = 0 (no q rows, no o) 7.0 us, a transition job (from h = I, v = 0) 6.2 us; one
// step of the chain of segment maps about 3 us, plus 3 us to start it.
constexpr double kStepB = 0.82, kStepA = 0.73, kChainStep = 0.35, kChainBase = 0.35;

// Estimated time, in chunk steps that write o, of the segmented scan of U work units per
// job with segment lengths (in chunks) l0, l1 (segments 1..S-2) and the rest.
double seg_cost(int S, int64_t l0, int64_t l1, int64_t last, int64_t U, int ncu)
{
    CuPool p1(ncu);  // pass 1 in dispatch order: segment 0, end states, transitions
    p1.run(U, (double)l0);
    p1.run((int64_t)(S - 2) * U, kStepB * (double)l1);
    p1.run((int64_t)(S - 2) * U, kStepA * (double)l1);
    CuPool p2(ncu);  // pass 2: segments 1..S-2, then the last one
    p2.run((int64_t)(S - 2) * U, (double)l1);
    p2.run(U, (double)last);
    return p1.end + p2.end + kChainBase + kChainStep * (S - 2);
}

// The plan of one call: cached for the last shape asked (every call of a model layer asks
// the same).
// With warm starts possible (max_s > 0), S is at most max_s: a call in warm mode runs segment
// 0 and S - 1 warm jobs per (stream, head) in one launch, which then fits one round.
SegPlan seg_search(int64_t nc, int64_t U, int ncu, int max_s)
{
    static std::mutex mu;
    static int64_t k_nc = -1, k_u = -1;
    static int k_ncu = -1, k_max = -1;
    static SegPlan k_plan{0, 0, 0};
    std::lock_guard<std::mutex> g(mu);
    if (nc == k_nc && U == k_u && ncu == k_ncu && max_s == k_max)
        return k_plan;
    CuPool serial(ncu);
    serial.run(U, (double)nc);
    double best = 0.8 * serial.end;  // segment only for a clear gain
    SegPlan plan{0, 0, 0};
    for (int S = 3; S <= kMaxSeg && S <= nc && (max_s == 0 || S <= max_s); ++S) {
        // inner segments from about nc / S to nc / (S - 2) chunks, segment 0 up to about
        // twice as long; long streams are searched on a coarser grid (at most ~32 x 64
        // candidates per S)
        const int64_t lo = nc / S > 2 ? nc / S - 1 : 1;
        const int64_t hi = (nc + S - 3) / (S - 2);
        const int64_t st1 = (hi - lo) / 32 + 1;
        for (int64_t l1 = lo; l1 <= hi; l1 += st1) {
            const int64_t st0 = (2 * l1 + 2) / 64 + 1;
            for (int64_t l0 = 1; l0 <= 2 * l1 + 2; l0 += st0) {
                const int64_t last = nc - l0 - (S - 2) * l1;
                if (last < 1)
                    break;
                const double c = seg_cost(S, l0, l1, last, U, ncu);
                if (c < best)
                    best = c, plan = SegPlan{S, l0 * 64, l1 * 64};
            }
        }
    }
    k_nc = nc, k_u = U, k_ncu = ncu, k_max = max_s, k_plan = plan;
    return plan;
}

// Warm starts apply to calls whose keys have unit length or less (L2 in the call or in the
// front end); the scalar gate is checked at launch.
bool warm_capable(const gdn_params *p) { return p->eps >= 0.f; }

SegPlan seg_plan(const gdn_params *p, int kda, int32_t B, int64_t tps, int nslices, int ncu)
{
    SegPlan none{0, 0, 0};
    if (p->dk != p->dv || p->chunk != 64 || tps < 1)
        return none;
    const int64_t nc = (tps + 63) / 64;
    const int64_t U = (int64_t)B * p->H * nslices;
    const int max_s = warm_capable(p) && ncu / U >= 3 ? (int)(ncu / U) : 0;
    (void)kda;
    SegPlan sp = seg_search(nc, U, ncu, max_s);
    if (max_s > 0 && sp.S > 0) {
        // A call that can start warm runs segment 0 and the S - 1 warm jobs side by side,
        // each warm job w chunks longer than its segment: equal segments give the shortest
        // critical path, L + w, for every w up to the segment length L (a longer segment 0
        // only pays off when the segments chain). The last segment takes what is left.
        const int64_t S = sp.S;
        int64_t l = (nc + S - 1) / S;
        if (nc - (S - 1) * l < 1)
            l = nc / S;
        sp.seg0_len = sp.seg_len = l * 64;
    }
    return sp;
}

// the segment states, and for a fused front end without shared windows the windows that a
// warm-started stream stages when its last job falls back to the second launch's copy
size_t seg_bytes(const gdn_params *p, int kda, int32_t B, int S)
{
    if (S < 3)
        return 0;
    const gdn::SegLayout lay{(int64_t)p->H * p->dk * p->dv, B, S, p->H};
    return align_up((size_t)lay.total() * sizeof(float)) +
           (win_shared(p, kda) ? 0 : win_bytes(p, kda, B));
}

struct Call {
    const gdn_params *p;
    int kda;
    const void *q, *k, *v;
    const float *g, *beta;
    float *h;
    float *const *h_ptrs;
    void *conv_state;
    void *const *conv_state_ptrs;
    const float *conv_w;
    void *o;
    Streams st;
    int64_t N;
    int32_t max_seqlen;  // varlen: the caller's bound on a stream's length
    void *ws;
    size_t ws_bytes;
    hipStream_t stream;
};

int run(const Call &c)
{
    const gdn_params *p = c.p;
    int rc = check_params(p, c.kda);
    if (rc != GDN_OK)
        return rc;
    if (!c.q || !c.k || !c.v || !c.g || !c.beta || !c.o || (!c.h && !c.h_ptrs))
        return GDN_E_ARG;
    if (!aligned16(c.q) || !aligned16(c.k) || !aligned16(c.v) || !aligned16(c.o) ||
        (c.kda && !aligned16(c.g)))
        return GDN_E_ARG;
    const bool front = p->conv_k > 0;
    if (front != (c.conv_w != nullptr) ||
        front != (c.conv_state != nullptr || c.conv_state_ptrs != nullptr))
        return GDN_E_ARG;
    if (c.N < 1 || c.N > (int64_t)INT32_MAX)
        return GDN_E_ARG;
    const bool fused_fe = front && fused_front(p, c.kda);
    const bool shared = fused_fe && win_shared(p, c.kda);
    const size_t need = front_bytes(p, c.kda, c.N, c.st.B);
    if (c.ws_bytes < need || (need && !c.ws))
        return GDN_E_WORKSPACE;
    if (need && !aligned16(c.ws))
        return GDN_E_ARG;

    const int64_t BH = (int64_t)c.st.B * p->H;
    const Shape sh = pick_shape(p, c.kda);
    const int ik = in_kind(p, c.kda);
    // the output gate rides in the o flush where the instance stages o, else its own pass
    const int fused = p->z && gdn::chunk_instance_exists(ik, p->dk, p->dv, c.kda, sh.nv,
                                                         sh.waves, 1, p->chunk);
    const int64_t grid = BH * (p->dv / sh.nv);
    if (grid > (int64_t)INT32_MAX)
        return GDN_E_ARG;
    // segmented scan when it pays, the workspace has room for its states and the job
    // counts of its launches fit a grid
    SegPlan sp{0, 0, 0};
    bool warm = false;
    if (!c.st.cu) {
        sp = seg_plan(p, c.kda, c.st.B, c.st.tps, p->dv / sh.nv, cu_count());
        warm = sp.S && warm_capable(p);
        const int64_t jobs1 = warm ? 3 * sp.S - 4 : 2 * sp.S - 3;
        if (sp.S && (c.ws_bytes < need + seg_bytes(p, c.kda, c.st.B, sp.S) ||
                     grid * jobs1 > (int64_t)INT32_MAX ||
                     BH * (p->dv / 16) + grid * (sp.S - 1) > (int64_t)INT32_MAX))
            sp = SegPlan{0, 0, 0}, warm = false;
    }

    // varlen calls with more workgroups than CUs: streams dispatch longest first, from a
    // ranking kept in the workspace after the front end's activations
    int32_t *order = nullptr;
    if (c.st.cu && c.ws && c.st.B <= kMaxOrderB && grid > cu_count() &&
        c.ws_bytes >= need + order_bytes(c.st.B))
        order = (int32_t *)((char *)c.ws + need);

    // debug validation of the device-side inputs, before every other kernel of the call
    int32_t *dbg = debug_status.load();
    if (dbg) {
        gdn::ValidateArgs va{};
        va.cu = c.st.cu;
        va.B = c.st.B;
        va.total = c.N;
        va.max_seqlen = c.max_seqlen;
        va.status = dbg;
        if (c.kda) {
            va.g = c.g;
            va.ng = c.N * p->H * p->dk;
        }
        if (gdn::launch_validate(va, c.stream) != hipSuccess)
            return GDN_E_HIP;
    }

    ChunkArgs ca{};
    ca.dbg = dbg;
    ca.order = order;
    ca.g = c.g;
    ca.beta = c.beta;
    ca.h = c.h;
    ca.h_ptrs = c.h_ptrs;
    ca.o = (float *)c.o;
    ca.st = c.st;
    ca.H = p->H;
    ca.qk_group = p->H / qk_heads(p);
    ca.eps = p->eps;
    if (fused) {
        ca.z = p->z;
        ca.ld_z = p->ld_z;
        ca.norm_w = p->norm_w;
        ca.norm_eps = p->norm_eps;
    }
    // warm starts (segmented calls): the plan of each (stream, head) from its gates, run by
    // extra workgroups of the front launch when there is one, else by a launch of its own
    // at the start of the scan
    const gdn::SegLayout lay{(int64_t)p->H * p->dk * p->dv, c.st.B, sp.S, p->H};
    float *seg_ws = sp.S ? (float *)((char *)c.ws + need) : nullptr;
    void *win_ws = shared ? c.ws
                   : sp.S && fused_fe
                       ? (char *)seg_ws + align_up((size_t)lay.total() * sizeof(float))
                       : nullptr;
    gdn::WarmArgs wa{};
    wa.dbg = dbg;
    ca.warm = warm;
    if (ca.warm) {
        wa.g = c.g, wa.beta = c.beta, wa.st = c.st, wa.H = p->H;
        wa.nseg = sp.S, wa.seg0_len = sp.seg0_len, wa.seg_len = sp.seg_len;
        wa.seg_ws = seg_ws, wa.lay = lay;
    }
    FrontArgs fa{};
    fa.dbg = dbg;
    if (fused_fe) {
        // conv + SiLU + L2 in the chunk kernel's load stage, straight from the raw rows
        ca.q = c.q, ca.k = c.k, ca.v = c.v, ca.ld = p->ld_qkv;
        ca.do_l2 = p->eps >= 0.f;
        ca.unit_keys = ca.do_l2;
        ca.scale = p->scale;
        ca.conv_w = c.conv_w;
        ca.conv_state = c.conv_state;
        ca.conv_state_ptrs = c.conv_state_ptrs;
        ca.win_ws = win_ws;
        ca.cd = (int32_t)conv_dim(p);
        ca.conv_k = p->conv_k;
        ca.win_shared = shared;
    } else if (front) {
        if (ca.warm && !c.kda) {
            fa.warm = wa;
            fa.warm_groups = c.st.B * p->H;
        }
        fa.q = c.q, fa.k = c.k, fa.v = c.v, fa.ld = p->ld_qkv;
        fa.conv_w = c.conv_w;
        fa.conv_state = c.conv_state;
        fa.conv_state_ptrs = c.conv_state_ptrs;
        fa.y = c.ws;
        fa.st = c.st;
        fa.N = c.N;
        fa.H = p->H, fa.Hqk = qk_heads(p), fa.dk = p->dk, fa.dv = p->dv, fa.K = p->conv_k;
        fa.do_l2 = p->eps >= 0.f;
        fa.eps = p->eps;
        fa.scale = p->scale;
        // Tiles long enough that the grid is about one round of workgroups (3 per CU at
        // the front kernel's occupancy), at least 32 tokens: a tile's window set-up and
        // its first loads are paid once per tile.
        {
            const int64_t groups = (conv_dim(p) / 8 + 255) / 256;
            const int64_t target = 3 * (int64_t)cu_count();
            int64_t rows = (c.N * groups + target - 1) / target;
            rows = (rows + 3) / 4 * 4;
            fa.tile_rows = (int32_t)(rows < 32 ? 32 : rows > 4096 ? 4096 : rows);
        }
        Stage st(GDN_PROF_FRONT, c.stream);
        if (gdn::launch_front(p->dtype, fa, c.stream) != hipSuccess)
            return GDN_E_HIP;
        st.done();
        const size_t es = elem_bytes(p->dtype);
        char *y = (char *)c.ws;
        ca.q = y;
        ca.k = y + (size_t)qk_heads(p) * p->dk * es;
        ca.v = y + (size_t)2 * qk_heads(p) * p->dk * es;
        ca.ld = conv_dim(p);
        ca.do_l2 = 0;
        ca.unit_keys = p->eps >= 0.f;  // the front end normalised q and k
        ca.scale = 1.f;
        // the new carried windows: extra workgroups of the scan's first launch (after the
        // front end, the only reader of the old windows)
        ca.window = fa;
        ca.window_dtype = p->dtype == GDN_BF16;
        ca.window_items = (int64_t)c.st.B * conv_dim(p);
    } else {
        ca.q = c.q, ca.k = c.k, ca.v = c.v, ca.ld = p->ld_qkv;
        ca.do_l2 = p->eps >= 0.f;
        ca.unit_keys = ca.do_l2;
        ca.scale = p->scale;
    }
    {
        Stage st(GDN_PROF_RECUR, c.stream);
        if (order && gdn::launch_stream_order(c.st.cu, c.st.B, order, c.stream) != hipSuccess)
            return GDN_E_HIP;
        if (!sp.S) {
            if (gdn::launch_chunk(ik, p->dk, p->dv, c.kda, sh.nv, sh.waves, fused, p->chunk,
                                  ca, (int)grid, c.stream) != hipSuccess)
                return GDN_E_HIP;
        } else {
            ca.nseg = sp.S;
            ca.seg0_len = sp.seg0_len;
            ca.seg_len = sp.seg_len;
            ca.seg_ws = seg_ws;
            if (ca.warm && (c.kda || !(front && !fused_fe))) {
                if (gdn::launch_warm_boundaries(wa, c.kda, p->dk, c.stream) != hipSuccess)
                    return GDN_E_HIP;
            }
            ca.pass = 1;
            const int64_t jobs1 = ca.warm ? 3 * sp.S - 4 : 2 * sp.S - 3;
            // the warm-start plan above cleared the read flags: the last warm job writes the
            // final state and windows itself
            ca.direct_final = ca.warm;
            // a flag wait outlasts any job it waits for: 2^20 polls plus 256 per chunk of the
            // stream (a chunk step outlasts 256 poll sleeps)
            ca.wait_polls = (int32_t)std::min<int64_t>(
                INT32_MAX, (int64_t)(1 << 20) + 256 * ((c.st.tps + 63) / 64));
            if (flag_polls.load() >= 0)
                ca.wait_polls = flag_polls.load();
            if (gdn::launch_chunk(ik, p->dk, p->dv, c.kda, sh.nv, sh.waves, fused, p->chunk,
                                  ca, (int)(grid * jobs1), c.stream) != hipSuccess)
                return GDN_E_HIP;
            // the chain's workgroups (one per stream, head and 16 state columns) ahead of
            // the jobs of segments 1..S-1
            ca.pass = 2;
            ca.window_items = 0;  // the windows went out with pass 1
            ca.chain_groups = (int32_t)(BH * (p->dv / 16));
            if (gdn::launch_chunk(ik, p->dk, p->dv, c.kda, sh.nv, sh.waves, fused, p->chunk,
                                  ca, (int)(ca.chain_groups + grid * (sp.S - 1)),
                                  c.stream) != hipSuccess)
                return GDN_E_HIP;
        }
        if (shared) {  // every workgroup that read the old windows is done
            gdn::WindowCopyArgs wc{};
            wc.dbg = dbg;
            wc.win_ws = win_ws;
            wc.conv_state = c.conv_state, wc.conv_state_ptrs = c.conv_state_ptrs;
            wc.st = c.st, wc.cd = (int32_t)conv_dim(p), wc.W = p->conv_k - 1;
            if (gdn::launch_window_copy(wc, c.stream) != hipSuccess)
                return GDN_E_HIP;
        }
        st.done();
    }
    if (p->z && !fused) {
        gdn::GateArgs ga{};
        ga.dbg = dbg;
        ga.o = (float *)c.o;
        ga.z = p->z;
        ga.ld_z = p->ld_z;
        ga.w = p->norm_w;
        ga.N = c.N;
        ga.H = p->H, ga.dv = p->dv;
        ga.eps = p->norm_eps;
        Stage st(GDN_PROF_GATE, c.stream);
        if (gdn::launch_gate(p->dtype, ga, c.stream) != hipSuccess)
            return GDN_E_HIP;
        st.done();
    }
    return GDN_OK;
}

int single(const gdn_params *p, int kda, const void *q, const void *k, const void *v,
           const float *g, const float *beta, float *h, void *conv_state,
           const float *conv_w, void *o, int64_t t, void *ws, size_t ws_bytes,
           void *stream)
{
    if (!h || t < 1)
        return GDN_E_ARG;
    Call c{};
    c.p = p, c.kda = kda, c.q = q, c.k = k, c.v = v, c.g = g, c.beta = beta;
    c.h = h, c.conv_state = conv_state, c.conv_w = conv_w, c.o = o;
    c.st = Streams{nullptr, t, 1};
    c.N = t, c.ws = ws, c.ws_bytes = ws_bytes, c.stream = (hipStream_t)stream;
    return run(c);
}

}  // namespace

// ---- the allocation-free single-stream call: its workspace is a file-scope device array,
// one per device, whose device address is looked up once per device --------------------
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices];  // device address of `scratch` on each device

// The address of `scratch` on the current device. In host code the array's name stands in
// for it but is not a device address, so only this pointer is ever handed to a kernel.
int scratch_on_current_device(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return GDN_E_HIP;
    std::lock_guard<std::mutex> g(scratch_mu);
    if (!scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
            return GDN_E_HIP;
        scratch_ptr[dev] = ptr;
    }
    *out = scratch_ptr[dev];
    return GDN_OK;
}
}  // namespace

extern "C" {

int gdn_prefill_noalloc(const gdn_params *p, const void *q, const void *k, const void *v,
                        const float *g, const float *beta, float *h, void *conv_state,
                        const float *conv_w, void *o, int64_t t, void *stream)
{
    int rc = check_params(p, 0);
    if (rc != GDN_OK)
        return rc;
    if (t < 1)
        return GDN_E_ARG;
    // the part of the workspace a call cannot run without must fit the array; segment
    // states that do not fit make the scan run unsegmented
    if (front_bytes(p, 0, t, 1) > GDN_NOALLOC_SCRATCH_BYTES)
        return GDN_E_WORKSPACE;
    void *ws = nullptr;
    rc = scratch_on_current_device(&ws);
    if (rc != GDN_OK)
        return rc;
    return single(p, 0, q, k, v, g, beta, h, conv_state, conv_w, o, t, ws,
                  GDN_NOALLOC_SCRATCH_BYTES, stream);
}

size_t gdn_noalloc_scratch_bytes(void) { return GDN_NOALLOC_SCRATCH_BYTES; }

int gdn_prefill(const gdn_params *p, const void *q, const void *k, const void *v,
                const float *g, const float *beta, float *h, void *conv_state,
                const float *conv_w, void *o, int64_t t, void *ws, size_t ws_bytes,
                void *stream)
{
    return single(p, 0, q, k, v, g, beta, h, conv_state, conv_w, o, t, ws, ws_bytes, stream);
}

int kda_prefill(const gdn_params *p, const void *q, const void *k, const void *v,
                const float *g, const float *beta, float *h, void *conv_state,
                const float *conv_w, void *o, int64_t t, void *ws, size_t ws_bytes,
                void *stream)
{
    return single(p, 1, q, k, v, g, beta, h, conv_state, conv_w, o, t, ws, ws_bytes, stream);
}

namespace {
int batched(const gdn_params *p, int kda, const void *q, const void *k, const void *v,
            const float *g, const float *beta, float *const *h_ptrs,
            void *const *conv_state_ptrs, const float *conv_w, void *o, int32_t B,
            int64_t t_per_stream, void *ws, size_t ws_bytes, void *stream)
{
    if (B < 1 || t_per_stream < 1 || !h_ptrs)
        return GDN_E_ARG;
    if (t_per_stream > (int64_t)INT32_MAX / B)
        return GDN_E_ARG;
    Call c{};
    c.p = p, c.kda = kda, c.q = q, c.k = k, c.v = v, c.g = g, c.beta = beta;
    c.h_ptrs = h_ptrs, c.conv_state_ptrs = conv_state_ptrs, c.conv_w = conv_w, c.o = o;
    c.st = Streams{nullptr, t_per_stream, B};
    c.N = (int64_t)B * t_per_stream, c.ws = ws, c.ws_bytes = ws_bytes;
    c.stream = (hipStream_t)stream;
    return run(c);
}

int varlen(const gdn_params *p, int kda, const void *q, const void *k, const void *v,
           const float *g, const float *beta, float *const *h_ptrs,
           void *const *conv_state_ptrs, const float *conv_w, void *o,
           const int32_t *cu_seqlens, int32_t B, int64_t total_tokens, int32_t max_seqlen,
           void *ws, size_t ws_bytes, void *stream)
{
    if (B < 1 || !h_ptrs || !cu_seqlens || total_tokens < 1 || max_seqlen < 1 ||
        max_seqlen > total_tokens)
        return GDN_E_ARG;
    Call c{};
    c.p = p, c.kda = kda, c.q = q, c.k = k, c.v = v, c.g = g, c.beta = beta;
    c.h_ptrs = h_ptrs, c.conv_state_ptrs = conv_state_ptrs, c.conv_w = conv_w, c.o = o;
    c.st = Streams{cu_seqlens, 0, B};
    c.N = total_tokens, c.ws = ws, c.ws_bytes = ws_bytes, c.stream = (hipStream_t)stream;
    c.max_seqlen = max_seqlen;
    return run(c);
}
}  // namespace

int gdn_prefill_batched(const gdn_params *p, const void *q, const void *k, const void *v,
                        const float *g, const float *beta, float *const *h_ptrs,
                        void *const *conv_state_ptrs, const float *conv_w, void *o,
                        int32_t B, int64_t t_per_stream, void *ws, size_t ws_bytes,
                        void *stream)
{
    return batched(p, 0, q, k, v, g, beta, h_ptrs, conv_state_ptrs, conv_w, o, B,
                   t_per_stream, ws, ws_bytes, stream);
}

int kda_prefill_batched(const gdn_params *p, const void *q, const void *k, const void *v,
                        const float *g, const float *beta, float *const *h_ptrs,
                        void *const *conv_state_ptrs, const float *conv_w, void *o,
                        int32_t B, int64_t t_per_stream, void *ws, size_t ws_bytes,
                        void *stream)
{
    return batched(p, 1, q, k, v, g, beta, h_ptrs, conv_state_ptrs, conv_w, o, B,
                   t_per_stream, ws, ws_bytes, stream);
}

int gdn_prefill_varlen(const gdn_params *p, const void *q, const void *k, const void *v,
                       const float *g, const float *beta, float *const *h_ptrs,
                       void *const *conv_state_ptrs, const float *conv_w, void *o,
                       const int32_t *cu_seqlens, int32_t B, int64_t total_tokens,
                       int32_t max_seqlen, void *ws, size_t ws_bytes, void *stream)
{
    return varlen(p, 0, q, k, v, g, beta, h_ptrs, conv_state_ptrs, conv_w, o, cu_seqlens, B,
                  total_tokens, max_seqlen, ws, ws_bytes, stream);
}

int kda_prefill_varlen(const gdn_params *p, const void *q, const void *k, const void *v,
                       const float *g, const float *beta, float *const *h_ptrs,
                       void *const *conv_state_ptrs, const float *conv_w, void *o,
                       const int32_t *cu_seqlens, int32_t B, int64_t total_tokens,
                       int32_t max_seqlen, void *ws, size_t ws_bytes, void *stream)
{
    return varlen(p, 1, q, k, v, g, beta, h_ptrs, conv_state_ptrs, conv_w, o, cu_seqlens, B,
                  total_tokens, max_seqlen, ws, ws_bytes, stream);
}

namespace {
int decode(const gdn_params *p, int kda, const void *q, const void *k, const void *v,
           const float *g, const float *beta, float *const *h_ptrs,
           void *const *conv_state_ptrs, const float *conv_w, void *o, int32_t B,
           void *stream)
{
    int rc = check_params(p, kda);
    if (rc != GDN_OK)
        return rc;
    if (!((p->dk == 64 || p->dk == 128) && (p->dv == p->dk || p->dv == 2 * p->dk)))
        return GDN_E_UNSUPPORTED;
    if (B < 1 || (int64_t)B * p->H > (int64_t)INT32_MAX)
        return GDN_E_ARG;
    if (!q || !k || !v || !g || !beta || !h_ptrs || !o)
        return GDN_E_ARG;
    if (!aligned16(o))
        return GDN_E_ARG;
    const bool front = p->conv_k > 0;
    if (front != (conv_w != nullptr) || front != (conv_state_ptrs != nullptr))
        return GDN_E_ARG;
    gdn::DecodeArgs a{};
    a.q = q, a.k = k, a.v = v, a.ld = p->ld_qkv;
    a.g = g, a.beta = beta, a.h_ptrs = h_ptrs;
    a.conv_state_ptrs = conv_state_ptrs, a.conv_w = conv_w;
    a.o = (float *)o;
    a.B = B, a.H = p->H, a.Hqk = qk_heads(p), a.dk = p->dk, a.dv = p->dv, a.K = p->conv_k;
    a.do_l2 = p->eps >= 0.f;
    a.eps = p->eps;
    a.scale = p->scale;
    a.z = p->z;
    a.ld_z = p->ld_z;
    a.norm_w = p->norm_w;
    a.norm_eps = p->norm_eps;
    // one fused launch: front end, recurrence step and window update (plus a pass for the
    // q/k windows when q/k heads are shared)
    Stage st(GDN_PROF_RECUR, (hipStream_t)stream);
    if (gdn::launch_decode(p->dtype, kda, a, (hipStream_t)stream) != hipSuccess)
        return GDN_E_HIP;
    if (front && a.Hqk != a.H &&
        gdn::launch_decode_qk_window(p->dtype, a, (hipStream_t)stream) != hipSuccess)
        return GDN_E_HIP;
    st.done();
    return GDN_OK;
}
}  // namespace

int gdn_decode(const gdn_params *p, const void *q, const void *k, const void *v,
               const float *g, const float *beta, float *const *h_ptrs,
               void *const *conv_state_ptrs, const float *conv_w, void *o, int32_t B,
               void *stream)
{
    return decode(p, 0, q, k, v, g, beta, h_ptrs, conv_state_ptrs, conv_w, o, B, stream);
}

int kda_decode(const gdn_params *p, const void *q, const void *k, const void *v,
               const float *g, const float *beta, float *const *h_ptrs,
               void *const *conv_state_ptrs, const float *conv_w, void *o, int32_t B,
               void *stream)
{
    return decode(p, 1, q, k, v, g, beta, h_ptrs, conv_state_ptrs, conv_w, o, B, stream);
}

int gdn_chunk_table(const int32_t *cu_seqlens, int32_t B, int32_t chunk, int32_t *table,
                    int64_t max_entries, int32_t *count, void *stream)
{
    if (!cu_seqlens || B < 1 || chunk < 1 || !count || max_entries < 0 ||
        (max_entries > 0 && !table))
        return GDN_E_ARG;
    if (gdn::launch_chunk_table(cu_seqlens, B, chunk, table, max_entries, count,
                                (hipStream_t)stream) != hipSuccess)
        return GDN_E_HIP;
    return GDN_OK;
}

size_t gdn_workspace_bytes(const gdn_params *p, int32_t B, int64_t max_tokens, int32_t kind)
{
    const int kda = (kind & GDN_PLAN_KDA) ? 1 : 0;
    kind &= ~GDN_PLAN_KDA;
    if (check_params(p, kda) != GDN_OK)
        return 0;
    if (B < 1 || max_tokens < 1 || kind < GDN_KIND_SINGLE || kind > GDN_KIND_VARLEN)
        return 0;
    // room for any segment plan a call of up to max_tokens can make: only calls with fewer
    // (stream, head, slice) workgroups than CUs ever segment
    size_t seg = 0;
    const Shape sh = pick_shape(p, kda);
    if (kind != GDN_KIND_VARLEN && p->dk == p->dv && sh.nv > 0 &&
        (int64_t)B * p->H * (p->dv / sh.nv) < cu_count() && max_tokens / B >= 3 * 64)
        seg = seg_bytes(p, kda, B, kMaxSeg);
    if (kind == GDN_KIND_VARLEN)
        seg = order_bytes(B);
    return front_bytes(p, kda, max_tokens, B) + seg;
}

int gdn_segment_plan(const gdn_params *p, int32_t kind, int32_t B, int64_t t_per_stream,
                     size_t ws_bytes, int64_t *seg0_tokens, int64_t *seg_tokens)
{
    if (seg0_tokens)
        *seg0_tokens = 0;
    if (seg_tokens)
        *seg_tokens = 0;
    const int kda = (kind & GDN_PLAN_KDA) ? 1 : 0;
    kind &= ~GDN_PLAN_KDA;
    const int rc = check_params(p, kda);
    if (rc != GDN_OK)
        return rc;
    if (B < 1 || t_per_stream < 1 || kind < GDN_KIND_SINGLE || kind > GDN_KIND_VARLEN ||
        (kind == GDN_KIND_SINGLE && B != 1))
        return GDN_E_ARG;
    if (kind == GDN_KIND_VARLEN)
        return 0;
    const Shape sh = pick_shape(p, kda);
    const SegPlan sp = seg_plan(p, kda, B, t_per_stream, p->dv / sh.nv, cu_count());
    const size_t need = front_bytes(p, kda, (int64_t)B * t_per_stream, B);
    if (!sp.S || ws_bytes < need + seg_bytes(p, kda, B, sp.S))
        return 0;
    if (seg0_tokens)
        *seg0_tokens = sp.seg0_len;
    if (seg_tokens)
        *seg_tokens = sp.seg_len;
    return sp.S;
}

int gdn_segments(const gdn_params *p, int32_t kind, int32_t B, int64_t t_per_stream,
                 size_t ws_bytes)
{
    return gdn_segment_plan(p, kind, B, t_per_stream, ws_bytes, nullptr, nullptr);
}

int gdn_debug_validate(int32_t *status)
{
    debug_status.store(status);
    return GDN_OK;
}

int gdn_debug_flag_polls(int32_t polls)
{
    if (polls < -1)
        return GDN_E_ARG;
    flag_polls.store(polls);
    return GDN_OK;
}

int gdn_profile_enable(int on)
{
    prof::enabled.store(on != 0);
    return GDN_OK;
}

int gdn_profile_read(double *ms_total, int64_t *launches, int32_t nbuckets)
{
    if (nbuckets < 0 || (nbuckets > 0 && (!ms_total || !launches)))
        return GDN_E_ARG;
    for (int32_t i = 0; i < nbuckets; ++i)
        ms_total[i] = 0.0, launches[i] = 0;
    std::vector<prof::Rec> recs;
    {
        std::lock_guard<std::mutex> g(prof::mu);
        recs.swap(prof::pending);
    }
    int rc = GDN_OK;
    for (const prof::Rec &r : recs) {
        float ms = 0.f;
        if (hipEventSynchronize(r.b) != hipSuccess ||
            hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
            rc = GDN_E_HIP;
        else if (r.bucket < nbuckets)
            ms_total[r.bucket] += ms, launches[r.bucket] += 1;
    }
    std::lock_guard<std::mutex> g(prof::mu);
    for (const prof::Rec &r : recs)
        prof::pool.push_back(r.a), prof::pool.push_back(r.b);
    return rc;
}

const char *gdn_status_string(int status)
{
    switch (status) {
    case GDN_OK: return "ok";
    case GDN_E_ARG: return "invalid argument";
    case GDN_E_UNSUPPORTED: return "unsupported configuration";
    case GDN_E_WORKSPACE: return "workspace too small";
    case GDN_E_HIP: return "HIP launch failed";
    default: return "unknown status";
    }
}

}  // extern "C"
