/*
 * ORACLE -- test infrastructure only.  Nothing in the product path links or
 * calls this file; only tests/, the smoke check and the benchmark's CPU
 * baseline do.
 *
 * fp32 router logits with a fixed summation order.
 *
 * The pages state that the router runs in fp32 ("fp32 router logits" in the
 * EP forward path of "Halo's 2.8x over TRL is not a kernel, and its own
 * benchmark proves it", section "Where the gap actually is"; and
 * `fp32_router: true` in the LFM2 recipe of section "The small-hardware end").
 * They do not fix an accumulation order.  Because top-k decisions on near-ties
 * depend on the last bit of a logit, the order is fixed here as part of the
 * definition:
 *
 *   L[t,e] = ((fma-chain over c = 0..d-1 of x[t,c]*w_r[e,c], starting at +0)
 *             + bias[e]) + noise[t,e]
 *
 * each step a single-rounding fp32 fused multiply-add, then one fp32 add for
 * the bias and one for the additive noise (both optional).
 *
 * The loop nest walks c in the outer position and e in the inner one so that
 * the independent chains of different experts advance together; every chain
 * still sees its terms in the order c = 0, 1, ..., d-1, so each output is
 * exactly the chain above.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static void chain_generic(const float *x, const float *wt, int d, int E, float *acc)
{
    for (int c = 0; c < d; ++c) {
        const float xc = x[c];
        const float *wc = wt + (size_t)c * E;
        for (int e = 0; e < E; ++e)
            acc[e] = fmaf(xc, wc[e], acc[e]);
    }
}

__attribute__((target("fma")))
static void chain_fma(const float *x, const float *wt, int d, int E, float *acc)
{
    for (int c = 0; c < d; ++c) {
        const float xc = x[c];
        const float *wc = wt + (size_t)c * E;
        for (int e = 0; e < E; ++e)
            acc[e] = __builtin_fmaf(xc, wc[e], acc[e]);
    }
}

/* x[T,d], w_r[E,d], bias[E] or NULL, noise[T,E] or NULL  ->  logits[T,E].
 * Returns 0, or -1 if a scratch allocation fails. */
int oracle_router_logits(const float *x, const float *w_r, const float *bias,
                         const float *noise, int64_t T, int d, int E, float *logits)
{
    float *wt = (float *)malloc(sizeof(float) * (size_t)d * (size_t)E);
    if (!wt) return -1;
    for (int e = 0; e < E; ++e)
        for (int c = 0; c < d; ++c)
            wt[(size_t)c * E + e] = w_r[(size_t)e * d + c];
    const int have_fma = __builtin_cpu_supports("fma");
    int fail = 0;
#pragma omp parallel
    {
        float *acc = (float *)malloc(sizeof(float) * (size_t)E);
        if (!acc) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t t = 0; t < T; ++t) {
                for (int e = 0; e < E; ++e) acc[e] = 0.0f;
                if (have_fma) chain_fma(x + (size_t)t * d, wt, d, E, acc);
                else          chain_generic(x + (size_t)t * d, wt, d, E, acc);
                for (int e = 0; e < E; ++e) {
                    float v = acc[e];
                    if (bias)  v = v + bias[e];
                    if (noise) v = v + noise[(size_t)t * E + e];
                    logits[(size_t)t * E + e] = v;
                }
            }
            free(acc);
        }
    }
    free(wt);
    return fail ? -1 : 0;
}
