/*
 * moe_oracle.c -- plain, slow, obviously-correct CPU reference for one
 * decode-time Mixture-of-Experts layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no
 * code, header, table or helper with the GPU library and never calls it.
 *
 * What it computes (all arithmetic in IEEE double, one token at a time):
 *
 *   Sources.  The pages (the Kimi K3 decode article, spke.com/es/ai/article/3589
 *   and its Korean text spke.com/ko/ai/article/3589, Part 1 section 3 "MoE
 *   scheduling and overlap"; the Hungarian summary "A vLLM ugynoki kodolassal
 *   gyorsitotta a Kimi K3-at", section "Kevesebb kernel, osszehangoltabb
 *   vegrehajtas") name the parts of the layer: router scores, the routed
 *   experts, the shared expert on its own stream, and a memory-bound weight
 *   stream at small batch.  They give no formulas.  The formulas below are
 *   the plainest reading of a gated-SwiGLU MoE decode layer; every reading
 *   taken where the pages are silent is listed in the design notes.
 *
 *   1. router logits      z[e] = sum_h x[h] * Wr[e][h] + b[e]
 *   2. selection          S = the k experts with the largest z,
 *                         ordered by (z descending, expert index ascending)
 *   3. routing weights    softmax: w_j = exp(z_j - m) / sum_{i in S} exp(z_i - m)
 *                         sigmoid: w_j = sig(z_j) / sum_{i in S} sig(z_i)
 *                         (without renormalisation: softmax over all E, or the
 *                         plain sigmoid), then times routed_scale
 *   4. routed experts     y_j = W2_j ( silu(W1_j x) * (W3_j x) ),
 *                         silu(v) = v / (1 + exp(-v))
 *   5. shared expert      s = S2 ( silu(S1 x) * (S3 x) )
 *   6. output             out = add_residual * x + s + sum_{j in S} w_j y_j
 *
 * Data layout (row-major, bf16 bit patterns as uint16):
 *   x   [B][H]       Wr  [E][H]       bias fp32 [E] or NULL
 *   per expert e: W13_e [2I][H] (rows 0..I-1 gate W1, rows I..2I-1 up W3),
 *                 W2_e  [H][I]
 *   shared: S13 [2Is][H] (gate rows then up rows), S2 [H][Is]
 * Expert weights are passed as per-expert pointer tables so a caller can
 * hand over only the experts the step touches; a NULL entry for an expert
 * that is selected is an error (return -3).
 *
 * Pins (tests that tie this code to something other than itself):
 * brute-force subset selection, a hand-computed closed-form example, the
 * dense SwiGLU special case (E=1, k=1) against a library FFN, a dense
 * all-experts NumPy formulation, and the invariants listed in the tests.
 * Parity unpinned: only whether this layer matches a real trained Kimi K3
 * layer (score function, shared-expert combine): no model definition or
 * weights exist to check it against.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t hidden;        /* H  */
    int32_t n_experts;     /* E  */
    int32_t top_k;         /* k  */
    int32_t inter;         /* I  */
    int32_t shared_inter;  /* Is, 0 = no shared expert */
    int32_t batch;         /* B  */
    int32_t score_fn;      /* 0 softmax, 1 sigmoid */
    int32_t renormalize;   /* 1: normalise the selected weights to sum 1 */
    double  routed_scale;
    int32_t add_residual;
} oracle_cfg;

/* bf16 is the upper half of an IEEE binary32; every bf16 is exact in double. */
static double bf(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double silu(double v) { return v / (1.0 + exp(-v)); }
static double sigm(double v) { return 1.0 / (1.0 + exp(-v)); }

static int check_cfg(const oracle_cfg* c)
{
    if (!c) return -1;
    if (c->hidden < 1 || c->n_experts < 1 || c->top_k < 1 || c->top_k > c->n_experts ||
        c->inter < 1 || c->shared_inter < 0 || c->batch < 0)
        return -1;
    if (c->score_fn != 0 && c->score_fn != 1) return -1;
    return 0;
}

/* Step 1 for one token: z[e] = <x, Wr[e]> + b[e]. */
static void router_row(const oracle_cfg* c, const uint16_t* xt, const uint16_t* wr,
                       const float* bias, double* z)
{
    const int H = c->hidden;
    for (int e = 0; e < c->n_experts; ++e) {
        double acc = 0.0;
        const uint16_t* w = wr + (size_t)e * H;
        for (int h = 0; h < H; ++h) acc += bf(xt[h]) * bf(w[h]);
        z[e] = acc + (bias ? (double)bias[e] : 0.0);
    }
}

/* true when expert a ranks before expert b */
static int ranks_before(const double* z, int a, int b)
{
    return z[a] > z[b] || (z[a] == z[b] && a < b);
}

/* Steps 2 and 3 for one token.  Selection is a plain repeated scan for the
 * best not-yet-taken expert, which yields the ranking order directly. */
static void select_and_weigh(const oracle_cfg* c, const double* z, int32_t* idx, double* w)
{
    const int E = c->n_experts, k = c->top_k;
    char* taken = (char*)calloc((size_t)E, 1);
    for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int e = 0; e < E; ++e)
            if (!taken[e] && (best < 0 || ranks_before(z, e, best))) best = e;
        taken[best] = 1;
        idx[j] = best;
    }
    free(taken);

    if (c->score_fn == 0) {               /* softmax */
        double m = z[idx[0]];             /* largest selected logit */
        if (c->renormalize) {
            double den = 0.0;
            for (int j = 0; j < k; ++j) den += exp(z[idx[j]] - m);
            for (int j = 0; j < k; ++j) w[j] = exp(z[idx[j]] - m) / den;
        } else {                          /* probability under softmax over all E */
            double mm = z[0];
            for (int e = 1; e < E; ++e) if (z[e] > mm) mm = z[e];
            double den = 0.0;
            for (int e = 0; e < E; ++e) den += exp(z[e] - mm);
            for (int j = 0; j < k; ++j) w[j] = exp(z[idx[j]] - mm) / den;
        }
    } else {                              /* sigmoid */
        double den = 0.0;
        for (int j = 0; j < k; ++j) den += sigm(z[idx[j]]);
        for (int j = 0; j < k; ++j)
            w[j] = c->renormalize ? sigm(z[idx[j]]) / den : sigm(z[idx[j]]);
    }
    for (int j = 0; j < k; ++j) w[j] *= c->routed_scale;
}

/* Step 4/5 for one token: y = W2 ( silu(W1 x) * (W3 x) ), with W13 = [W1; W3]
 * of shape [2n][H] and W2 of shape [H][n].  y has H entries, overwritten. */
static void swiglu_ffn(int H, int n, const uint16_t* w13, const uint16_t* w2,
                       const uint16_t* xt, double* hbuf, double* y)
{
    for (int i = 0; i < n; ++i) {
        const uint16_t* g = w13 + (size_t)i * H;
        const uint16_t* u = w13 + (size_t)(n + i) * H;
        double gs = 0.0, us = 0.0;
        for (int h = 0; h < H; ++h) {
            double xv = bf(xt[h]);
            gs += bf(g[h]) * xv;
            us += bf(u[h]) * xv;
        }
        hbuf[i] = silu(gs) * us;
    }
    for (int r = 0; r < H; ++r) {
        const uint16_t* row = w2 + (size_t)r * n;
        double acc = 0.0;
        for (int i = 0; i < n; ++i) acc += bf(row[i]) * hbuf[i];
        y[r] = acc;
    }
}

/* ---------------------------------------------------------------- exports */

int oracle_router_logits(const oracle_cfg* c, const uint16_t* x, const uint16_t* wr,
                         const float* bias, double* z)
{
    if (check_cfg(c) || !x || !wr || !z) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < c->batch; ++t)
        router_row(c, x + (size_t)t * c->hidden, wr, bias, z + (size_t)t * c->n_experts);
    return 0;
}

int oracle_select(const oracle_cfg* c, const double* z, int32_t* idx, double* w)
{
    if (check_cfg(c) || !z || !idx || !w) return -1;
    for (int t = 0; t < c->batch; ++t)
        select_and_weigh(c, z + (size_t)t * c->n_experts, idx + (size_t)t * c->top_k,
                         w + (size_t)t * c->top_k);
    return 0;
}

/* One dense SwiGLU FFN per token (no routing): y[t] = W2 (silu(W1 x_t) * (W3 x_t)). */
int oracle_swiglu(int32_t H, int32_t n, int32_t B, const uint16_t* w13, const uint16_t* w2,
                  const uint16_t* x, double* y)
{
    if (H < 1 || n < 1 || B < 0 || !w13 || !w2 || !x || !y) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < B; ++t) {
        double* hbuf = (double*)malloc(sizeof(double) * (size_t)n);
        swiglu_ffn(H, n, w13, w2, x + (size_t)t * H, hbuf, y + (size_t)t * H);
        free(hbuf);
    }
    return 0;
}

/* Whole layer.  out64 [B][H], idx [B][k], w [B][k]. */
int oracle_forward(const oracle_cfg* c, const uint16_t* x, const uint16_t* wr, const float* bias,
                   const uint16_t* const* w13_e, const uint16_t* const* w2_e,
                   const uint16_t* s13, const uint16_t* s2,
                   double* out64, int32_t* idx, double* w)
{
    if (check_cfg(c) || !x || !wr || !w13_e || !w2_e || !out64 || !idx || !w) return -1;
    if (c->shared_inter > 0 && (!s13 || !s2)) return -1;
    const int H = c->hidden, E = c->n_experts, k = c->top_k, I = c->inter, Is = c->shared_inter;
    int status = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < c->batch; ++t) {
        const uint16_t* xt = x + (size_t)t * H;
        double* z = (double*)malloc(sizeof(double) * (size_t)E);
        double* y = (double*)malloc(sizeof(double) * (size_t)H);
        double* hb = (double*)malloc(sizeof(double) * (size_t)(I > Is ? I : Is));
        double* o = out64 + (size_t)t * H;
        int32_t* it = idx + (size_t)t * k;
        double* wt = w + (size_t)t * k;

        router_row(c, xt, wr, bias, z);
        select_and_weigh(c, z, it, wt);

        for (int r = 0; r < H; ++r) o[r] = c->add_residual ? bf(xt[r]) : 0.0;
        for (int j = 0; j < k; ++j) {
            const int e = it[j];
            if (!w13_e[e] || !w2_e[e]) {
#pragma omp atomic write
                status = -3;
                continue;
            }
            swiglu_ffn(H, I, w13_e[e], w2_e[e], xt, hb, y);
            for (int r = 0; r < H; ++r) o[r] += wt[j] * y[r];
        }
        if (Is > 0) {
            swiglu_ffn(H, Is, s13, s2, xt, hb, y);
            for (int r = 0; r < H; ++r) o[r] += y[r];
        }
        free(z);
        free(y);
        free(hb);
    }
    return status;
}

/* Lets a caller check that it loaded a library built with OpenMP. */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
