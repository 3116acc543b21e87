// Host-side checks of libgdn's C ABI, built with AddressSanitizer on the host code (device
// code is built normally) and run without a GPU: every path that runs before a launch --
// argument validation of every entry point, workspace sizing, segment plans, status
// strings, the profiling buckets, the debug-validation switch -- over a grid of shapes,
// valid and invalid. Device pointers are fake, 16-byte aligned addresses: no call that
// gets them may enqueue anything, so none is ever dereferenced. Exit status 0 when every
// check holds.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gdn.h"

static int fails = 0, checks = 0;
#define CHECK(c)                                                                \
    do {                                                                        \
        ++checks;                                                               \
        if (!(c)) {                                                             \
            fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #c);        \
            ++fails;                                                            \
        }                                                                       \
    } while (0)

static gdn_params make(int H, int dk, int dv, int dtype, int conv_k, int Hqk)
{
    gdn_params p;
    memset(&p, 0, sizeof p);
    p.H = H, p.dk = dk, p.dv = dv, p.chunk = 64, p.eps = 1e-6f, p.scale = 0.125f;
    p.dtype = dtype, p.conv_k = conv_k, p.Hqk = Hqk;
    p.ld_qkv = 2LL * (Hqk ? Hqk : H) * dk + (int64_t)H * dv;
    return p;
}

int main()
{
    void *const D = (void *)(uintptr_t)0x100000;  // fake device addresses
    void *const D2 = (void *)(uintptr_t)0x200000;
    float *const Df = (float *)D;
    void *const *const Dp = (void *const *)D;
    float *const *const Dfp = (float *const *)D;
    const int32_t *const Dc = (const int32_t *)D2;

    // ---- workspace sizes and segment plans over a grid of shapes --------------------
    const int Hs[] = {1, 2, 3, 4, 32, 64};
    const int dims[][2] = {{64, 64}, {128, 128}, {128, 256}, {64, 128}, {96, 96}, {128, 64}};
    const int64_t Ts[] = {1, 63, 64, 65, 200, 4096, 16384, 1 << 20};
    for (int H : Hs)
        for (auto &d : dims)
            for (int dtype : {GDN_F32, GDN_BF16, 7})
                for (int conv_k : {0, 2, 3, 4, 5})
                    for (int Hqk : {0, 1, H / 2})
                        for (int kda : {0, GDN_PLAN_KDA}) {
                            gdn_params p = make(H, d[0], d[1], dtype, conv_k, Hqk);
                            for (int kind : {GDN_KIND_SINGLE, GDN_KIND_BATCHED, GDN_KIND_VARLEN})
                                for (int32_t B : {1, 3, 8})
                                    for (int64_t T : Ts) {
                                        const size_t ws =
                                            gdn_workspace_bytes(&p, B, T * B, kind | kda);
                                        CHECK(ws % 256 == 0);
                                        int64_t l0 = -1, l1 = -1;
                                        const int S = gdn_segment_plan(
                                            &p, kind | kda, B, T, ws, &l0, &l1);
                                        if (kind == GDN_KIND_SINGLE && B != 1) {
                                            CHECK(S < 0);
                                            continue;
                                        }
                                        CHECK(S == gdn_segments(&p, kind | kda, B, T, ws));
                                        if (S <= 0) {
                                            CHECK(l0 == 0 && l1 == 0);
                                        } else {
                                            CHECK(S >= 3 && S <= 12 && kind != GDN_KIND_VARLEN);
                                            CHECK(l0 > 0 && l1 > 0 && l0 % 64 == 0 &&
                                                  l1 % 64 == 0 && l0 + (S - 2) * l1 < T);
                                        }
                                    }
                            CHECK(gdn_workspace_bytes(&p, 0, 10, GDN_KIND_SINGLE) == 0);
                            CHECK(gdn_workspace_bytes(&p, 1, 0, GDN_KIND_SINGLE) == 0);
                            CHECK(gdn_workspace_bytes(&p, 1, 10, 9) == 0);
                        }
    CHECK(gdn_workspace_bytes(nullptr, 1, 10, GDN_KIND_SINGLE) == 0);

    // ---- refusals before any launch --------------------------------------------------
    gdn_params f = make(2, 64, 64, GDN_F32, 0, 0);
    CHECK(gdn_prefill(&f, D, D, D, Df, Df, Df, nullptr, nullptr, D, 0, nullptr, 0, nullptr) ==
          GDN_E_ARG);
    CHECK(gdn_prefill(&f, D, D, D, Df, Df, nullptr, nullptr, nullptr, D, 10, nullptr, 0,
                      nullptr) == GDN_E_ARG);
    CHECK(gdn_prefill(&f, (char *)D + 4, D, D, Df, Df, Df, nullptr, nullptr, D, 10, nullptr, 0,
                      nullptr) == GDN_E_ARG);
    CHECK(gdn_prefill(nullptr, D, D, D, Df, Df, Df, nullptr, nullptr, D, 10, nullptr, 0,
                      nullptr) == GDN_E_ARG);
    gdn_params bad = f;
    bad.chunk = 16;
    CHECK(kda_prefill(&bad, D, D, D, Df, Df, Df, nullptr, nullptr, D, 10, nullptr, 0,
                      nullptr) == GDN_E_UNSUPPORTED);
    bad = f;
    bad.ld_qkv = 100;
    CHECK(gdn_prefill(&bad, D, D, D, Df, Df, Df, nullptr, nullptr, D, 10, nullptr, 0,
                      nullptr) == GDN_E_ARG);
    bad = f;
    bad.scale = __builtin_nanf("");
    CHECK(gdn_prefill(&bad, D, D, D, Df, Df, Df, nullptr, nullptr, D, 10, nullptr, 0,
                      nullptr) == GDN_E_ARG);
    gdn_params ff = make(2, 64, 64, GDN_F32, 4, 0);  // float32 front end: activations
    const size_t need = gdn_workspace_bytes(&ff, 1, 10, GDN_KIND_SINGLE);
    CHECK(need >= 10 * 384 * 4);
    CHECK(gdn_prefill(&ff, D, D, D, Df, Df, Df, D, Df, D, 10, D2, need - 1, nullptr) ==
          GDN_E_WORKSPACE);
    CHECK(gdn_prefill(&ff, D, D, D, Df, Df, Df, D, nullptr, D, 10, D2, need, nullptr) ==
          GDN_E_ARG);
    gdn_params bw = make(4, 128, 128, GDN_BF16, 4, 0);
    bw.ld_qkv = 1 << 24;  // the fused front end needs 32-bit row offsets
    CHECK(gdn_prefill(&bw, D, D, D, Df, Df, Df, D, Df, D, 10, nullptr, 0, nullptr) ==
          GDN_E_UNSUPPORTED);
    CHECK(gdn_prefill_batched(&f, D, D, D, Df, Df, Dfp, nullptr, nullptr, D, 0, 10, nullptr, 0,
                              nullptr) == GDN_E_ARG);
    CHECK(kda_prefill_batched(&f, D, D, D, Df, Df, Dfp, nullptr, nullptr, D, 2, 0, nullptr, 0,
                              nullptr) == GDN_E_ARG);
    CHECK(gdn_prefill_batched(&f, D, D, D, Df, Df, Dfp, nullptr, nullptr, D, 1 << 20, 1 << 12,
                              nullptr, 0, nullptr) == GDN_E_ARG);
    CHECK(gdn_prefill_varlen(&f, D, D, D, Df, Df, Dfp, nullptr, nullptr, D, nullptr, 2, 10, 5,
                             nullptr, 0, nullptr) == GDN_E_ARG);
    CHECK(kda_prefill_varlen(&f, D, D, D, Df, Df, Dfp, nullptr, nullptr, D, Dc, 2, 10, 11,
                             nullptr, 0, nullptr) == GDN_E_ARG);
    CHECK(gdn_prefill_varlen(&f, D, D, D, Df, Df, Dfp, nullptr, nullptr, D, Dc, 0, 10, 5,
                             nullptr, 0, nullptr) == GDN_E_ARG);
    CHECK(gdn_decode(&f, D, D, D, Df, Df, Dfp, nullptr, nullptr, D, 0, nullptr) == GDN_E_ARG);
    CHECK(kda_decode(&f, D, D, D, Df, Df, nullptr, nullptr, nullptr, D, 2, nullptr) ==
          GDN_E_ARG);
    gdn_params d96 = make(2, 96, 96, GDN_F32, 0, 0);
    CHECK(gdn_decode(&d96, D, D, D, Df, Df, Dfp, nullptr, nullptr, D, 2, nullptr) ==
          GDN_E_UNSUPPORTED);
    CHECK(gdn_chunk_table(nullptr, 2, 64, (int32_t *)D, 10, (int32_t *)D, nullptr) ==
          GDN_E_ARG);
    CHECK(gdn_chunk_table(Dc, 2, 0, (int32_t *)D, 10, (int32_t *)D, nullptr) == GDN_E_ARG);
    (void)Dp;

    // the allocation-free call refuses before it looks up its array
    CHECK(gdn_noalloc_scratch_bytes() == ((size_t)64 << 20));
    CHECK(gdn_prefill_noalloc(&f, D, D, D, Df, Df, Df, nullptr, nullptr, D, 0, nullptr) ==
          GDN_E_ARG);
    gdn_params big = make(32, 64, 64, GDN_F32, 4, 0);
    CHECK(gdn_prefill_noalloc(&big, D, D, D, Df, Df, Df, D, Df, D, 1 << 20, nullptr) ==
          GDN_E_WORKSPACE);

    // output gate and shared q/k head arguments
    gdn_params g = make(2, 64, 64, GDN_F32, 0, 0);
    g.z = D;
    CHECK(gdn_prefill(&g, D, D, D, Df, Df, Df, nullptr, nullptr, D, 10, nullptr, 0, nullptr) ==
          GDN_E_ARG);  // no norm weights
    g.norm_w = Df, g.ld_z = 128, g.norm_eps = -1.f;
    CHECK(gdn_prefill(&g, D, D, D, Df, Df, Df, nullptr, nullptr, D, 10, nullptr, 0, nullptr) ==
          GDN_E_ARG);
    gdn_params q = make(6, 64, 64, GDN_F32, 0, 4);
    CHECK(gdn_prefill(&q, D, D, D, Df, Df, Df, nullptr, nullptr, D, 10, nullptr, 0, nullptr) ==
          GDN_E_ARG);

    // ---- status strings, profiling buckets, debug switch -------------------------------
    for (int s = -10; s <= 10; ++s)
        CHECK(gdn_status_string(s) != nullptr && strlen(gdn_status_string(s)) > 0);
    double ms[GDN_PROF_BUCKETS];
    int64_t n[GDN_PROF_BUCKETS];
    CHECK(gdn_profile_read(ms, n, GDN_PROF_BUCKETS) == GDN_OK);
    for (int i = 0; i < GDN_PROF_BUCKETS; ++i)
        CHECK(ms[i] == 0.0 && n[i] == 0);
    CHECK(gdn_profile_read(nullptr, nullptr, 2) == GDN_E_ARG);
    CHECK(gdn_profile_enable(1) == GDN_OK && gdn_profile_enable(0) == GDN_OK);
    CHECK(gdn_debug_validate((int32_t *)D) == GDN_OK && gdn_debug_validate(nullptr) == GDN_OK);

    printf("asan driver: %d of %d checks failed\n", fails, checks);
    return fails != 0;
}
