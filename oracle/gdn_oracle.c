/*
 * gdn_oracle.c -- plain fp64 CPU oracle for the chunked gated-delta-rule prefill.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library. The product path never
 * calls it and shares no code, header or table with it.
 *
 * What it computes is the plain definition, token by token, in double precision:
 *
 *   front end (pages: "metrale_model_arch/glm5next_kda/prefill.rs", the conv_prefill
 *   launch and its "conv + SiLU only" comment; "split_prefill.rs",
 *   prefill_phase1_conv1d_one): a causal depthwise conv1d over each channel of the packed
 *   [q | k | v] rows, no bias (the launch passes a null bias), followed by SiLU. The conv
 *   starts from a carried window of the last K-1 raw inputs and leaves the last K-1 raw
 *   inputs of the extended sequence behind as the new window.
 *
 *   L2 + scale (same page, the l2 launch with l2_eps, and the 1/sqrt(hd) argument of the
 *   chunk_scan launch): q <- scale * q / sqrt(sum q^2 + eps), k <- k / sqrt(sum k^2 + eps),
 *   per token and head.
 *
 *   recurrence (the gated delta rule of Gated DeltaNet, Yang, Kautz & Hatamizadeh 2024;
 *   the per-key-channel gate of Kimi Delta Attention; "split_prefill.rs", prefill_gdn_full:
 *   "the GDN recurrence"): with S = h^T (dv x dk) and alpha_t = exp(g_t),
 *       S <- S diag(alpha_t)
 *       S <- S - beta_t (S k_t - v_t) k_t^T
 *       o_t = S q_t
 *   alpha_t is one scalar per head (GDN) or one value per key channel (KDA).
 *
 *   output gate (page "split_prefill.rs", prefill_phase3: the gated RMSNorm of the GDN
 *   output with Z comes first in phase 3): per token and head, over the dv values of o,
 *       y_j = o_j / sqrt(mean_j o_j^2 + eps) * w_j * silu(z_j),   silu(z) = z / (1 + e^-z)
 *   with one weight per value channel shared by every head.
 *
 * Readings where the pages are silent:
 *   - conv taps follow the cross-correlation convention: tap K-1 multiplies the current
 *     token, tap 0 the token K-1 steps back;
 *   - the conv window holds raw (pre-conv) inputs, oldest first, [C][K-1];
 *   - g is the log of the decay; the decay is applied before the delta update;
 *   - beta is used as given (already through its sigmoid);
 *   - the gated RMSNorm normalises before gating (the norm sees o alone), over one head's
 *     dv values, with eps inside the square root and a [dv] weight.
 *
 * Parity of the conv tap orientation is unpinned by the pages (only the library
 * convention of torch.nn.functional.conv1d pins it).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EARG (-1)
#define ORACLE_ENOMEM (-2)

/*
 * Causal depthwise conv1d + SiLU over one stream.
 *   x      [T][C]   raw inputs (fp64 copies of the caller's values)
 *   w      [C][K]   taps; w[c][K-1] multiplies the current token
 *   st     [C][K-1] carried window, oldest first (may be NULL: zeros)
 *   y      [T][C]   out: silu(conv)
 *   st_out [C][K-1] out: the last K-1 entries of [st | x] per channel
 */
int gdn_oracle_conv_silu(int64_t T, int32_t C, int32_t K, const double *x,
                         const double *w, const double *st, double *y,
                         double *st_out)
{
    if (T < 0 || C <= 0 || K < 1 || !x || !w || !y)
        return ORACLE_EARG;
    const int32_t W = K - 1;
    int failed = 0; /* set (never cleared) by any thread whose buffer could not be had */
#pragma omp parallel for schedule(static)
    for (int32_t c = 0; c < C; ++c) {
        /* extended sequence for this channel: xe[0..W-1] = window, xe[W+t] = x[t] */
        double *xe = (double *)malloc(sizeof(double) * (size_t)(T + W + 1));
        if (!xe) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        for (int32_t j = 0; j < W; ++j)
            xe[j] = st ? st[(int64_t)c * W + j] : 0.0;
        for (int64_t t = 0; t < T; ++t)
            xe[W + t] = x[t * C + c];
        for (int64_t t = 0; t < T; ++t) {
            double z = 0.0;
            for (int32_t j = 0; j < K; ++j)
                z += w[(int64_t)c * K + j] * xe[t + j];
            y[t * C + c] = z / (1.0 + exp(-z));
        }
        if (st_out)
            for (int32_t j = 0; j < W; ++j)
                st_out[(int64_t)c * W + j] = xe[T + j];
        free(xe);
    }
    return failed ? ORACLE_ENOMEM : ORACLE_OK;
}

/* q <- scale * q / sqrt(|q|^2 + eps) over n entries */
static void l2_scale(double *dst, const double *src, int32_t n, double eps,
                     double scale)
{
    double ss = 0.0;
    for (int32_t i = 0; i < n; ++i)
        ss += src[i] * src[i];
    const double inv = 1.0 / sqrt(ss + eps);
    for (int32_t i = 0; i < n; ++i)
        dst[i] = src[i] * inv * scale;
}

/*
 * Token-by-token recurrence for B streams lying back to back.
 *   cu    [B+1]        stream b owns rows [cu[b], cu[b+1])
 *   q, k  [N][H][dk]   v [N][H][dv]
 *   g     [N][H] (gate_per_channel == 0) or [N][H][dk] (== 1), log decay
 *   beta  [N][H]
 *   l2    nonzero: normalise q and k (eps); zero: use them as given
 *   scale multiplies q in both cases (after the L2 when there is one)
 *   h     [B][H][dk][dv]  in: initial state of each stream, out: final state
 *   o     [N][H][dv]      out
 * Rows outside [cu[0], cu[B]) are never read or written.
 */
int gdn_oracle_recurrence(int32_t B, const int64_t *cu, int32_t H, int32_t dk,
                          int32_t dv, const double *q, const double *k,
                          const double *v, const double *g,
                          int32_t gate_per_channel, const double *beta,
                          int32_t l2, double eps, double scale, double *h,
                          double *o)
{
    if (B < 1 || H < 1 || dk < 1 || dv < 1 || !cu || !q || !k || !v || !g ||
        !beta || !h || !o)
        return ORACLE_EARG;
    for (int32_t b = 0; b < B; ++b)
        if (cu[b + 1] < cu[b])
            return ORACLE_EARG;
    int failed = 0; /* set (never cleared) by any thread whose buffers could not be had */
    const int64_t units = (int64_t)B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < units; ++u) {
        const int32_t b = (int32_t)(u / H), hd = (int32_t)(u % H);
        double *S = h + ((int64_t)b * H + hd) * dk * dv; /* S^T, [dk][dv] */
        double *qn = (double *)malloc(sizeof(double) * dk);
        double *kn = (double *)malloc(sizeof(double) * dk);
        double *e = (double *)malloc(sizeof(double) * dv);
        if (!qn || !kn || !e) {
#pragma omp atomic write
            failed = 1;
            free(qn), free(kn), free(e);
            continue;
        }
        for (int64_t t = cu[b]; t < cu[b + 1]; ++t) {
            const double *qt = q + (t * H + hd) * dk;
            const double *kt = k + (t * H + hd) * dk;
            const double *vt = v + (t * H + hd) * dv;
            const double bt = beta[t * H + hd];
            if (l2) {
                l2_scale(qn, qt, dk, eps, scale);
                l2_scale(kn, kt, dk, eps, 1.0);
            } else {
                for (int32_t i = 0; i < dk; ++i)
                    qn[i] = qt[i] * scale;
                memcpy(kn, kt, sizeof(double) * dk);
            }
            /* S <- S diag(alpha): column i of S is row i of the stored h */
            for (int32_t i = 0; i < dk; ++i) {
                const double gi = gate_per_channel ? g[(t * H + hd) * dk + i]
                                                   : g[t * H + hd];
                const double a = exp(gi);
                for (int32_t j = 0; j < dv; ++j)
                    S[(int64_t)i * dv + j] *= a;
            }
            /* e = S k - v */
            for (int32_t j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int32_t i = 0; i < dk; ++i)
                    acc += S[(int64_t)i * dv + j] * kn[i];
                e[j] = acc - vt[j];
            }
            /* S <- S - beta e k^T */
            for (int32_t i = 0; i < dk; ++i)
                for (int32_t j = 0; j < dv; ++j)
                    S[(int64_t)i * dv + j] -= bt * e[j] * kn[i];
            /* o = S q */
            double *ot = o + (t * H + hd) * dv;
            for (int32_t j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int32_t i = 0; i < dk; ++i)
                    acc += S[(int64_t)i * dv + j] * qn[i];
                ot[j] = acc;
            }
        }
        free(qn), free(kn), free(e);
    }
    return failed ? ORACLE_ENOMEM : ORACLE_OK;
}

/* Threads the OpenMP runtime will use for the loops above (for reporting). */
/* Gated RMSNorm of rows of dv values: y = o / sqrt(mean(o^2) + eps) * w * silu(z). */
int gdn_oracle_gated_rmsnorm(int64_t rows, int32_t dv, const double *o, const double *z,
                             const double *w, double eps, double *y)
{
    if (rows < 0 || dv < 1 || !o || !z || !w || !y || !(eps >= 0.0))
        return ORACLE_EARG;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const double *orow = o + r * dv, *zrow = z + r * dv;
        double ss = 0.0;
        for (int32_t j = 0; j < dv; ++j)
            ss += orow[j] * orow[j];
        const double inv = 1.0 / sqrt(ss / dv + eps);
        for (int32_t j = 0; j < dv; ++j) {
            const double zj = zrow[j];
            y[r * dv + j] = orow[j] * inv * w[j] * (zj / (1.0 + exp(-zj)));
        }
    }
    return ORACLE_OK;
}

int gdn_oracle_num_threads(void)
{
    int n = 1;
#ifdef _OPENMP
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
#endif
    return n;
}
