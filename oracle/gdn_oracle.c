/*
 * Oracle for the gated delta rule: a plain, slow, token-by-token float64 recurrence on the CPU.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load this library.  It shares no code, header or constant with the HIP library.
 *
 * What it computes (math orientation S in R^{dv x dk}, o_t = S_t q_t):
 *   S_t = S_{t-1} ( alpha_t (I - beta_t k_t k_t^T) ) + beta_t v_t k_t^T
 * -- "Architecture Thread I: Gated Attention, DeltaNet, and Hybrid Models", section "Gated
 *    DeltaNet", state-update equation; the same equation appears in "Gated Attention
 *    Architectures", section 3 (Gated DeltaNet), Mathematical Formulation.
 * The readout o_t = S_t q_t is the one used for linear attention in "Gated Attention
 * Architectures", section 1 (GLA), recurrent form.
 *
 * Expanding the product gives the erase/write form used below, exactly (up to rounding order):
 *   u_t     = S_{t-1} k_t                    (old memory's prediction for k_t)
 *   delta_t = beta_t (v_t - alpha_t u_t)
 *   S_t     = alpha_t S_{t-1} + delta_t k_t^T
 * -- "Architecture Thread I", section on DeltaNet, erase/write decomposition, with the decay
 *    alpha_t applied to the whole old state as the Gated DeltaNet equation requires.
 *
 * Storage: the state is stored transposed, h = S^T, as [B, Hv, dk, dv] with dv contiguous, which
 * is the [d_k, d_v] memory layout of the delta loop in "Decoding Next-Generation LLM
 * Architectures", section 3.2.  With h = S^T:  u = h^T k,  h <- alpha h + k delta^T,  o = h^T q.
 *
 * Heads: value head j reads query/key head floor(j / (Hv / Hqk)) (grouped heads, contiguous
 * groups).  Inputs are float64 copies of exactly the values handed to the GPU.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* q, k: [B,T,Hqk,dk]; v: [B,T,Hv,dv]; g (= log alpha), beta: [B,T,Hv];
 * s0: [B,Hv,dk,dv] or NULL (zeros); o: [B,T,Hv,dv]; s_final: [B,Hv,dk,dv] or NULL.
 * q is multiplied by `scale` before the readout.  Returns 0, or -1 on bad sizes / no memory. */
int gdn_oracle_recurrent(const double* q, const double* k, const double* v, const double* g,
                         const double* beta, const double* s0, double* o, double* s_final,
                         int B, int T, int Hqk, int Hv, int dk, int dv, double scale, int nthreads)
{
    if (B <= 0 || T < 0 || Hqk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || Hv % Hqk != 0) return -1;
    const int grp = Hv / Hqk;
    const long long nchains = (long long)B * Hv;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(|: bad)
#endif
    for (long long c = 0; c < nchains; ++c) {
        const int b = (int)(c / Hv), j = (int)(c % Hv), i = j / grp;
        double* h = (double*)malloc(sizeof(double) * (size_t)dk * dv);
        double* u = (double*)malloc(sizeof(double) * (size_t)dv);
        if (!h || !u) { free(h); free(u); bad |= 1; continue; }
        if (s0) memcpy(h, s0 + (size_t)c * dk * dv, sizeof(double) * (size_t)dk * dv);
        else memset(h, 0, sizeof(double) * (size_t)dk * dv);
        for (int t = 0; t < T; ++t) {
            const size_t tqk = (((size_t)b * T + t) * Hqk + i);
            const size_t tv = (((size_t)b * T + t) * Hv + j);
            const double* kt = k + tqk * dk;
            const double* qt = q + tqk * dk;
            const double* vt = v + tv * dv;
            const double alpha = exp(g[tv]);
            const double bt = beta[tv];
            /* u = h^T k  (= S_{t-1} k_t) */
            for (int cc = 0; cc < dv; ++cc) u[cc] = 0.0;
            for (int r = 0; r < dk; ++r)
                for (int cc = 0; cc < dv; ++cc) u[cc] += h[(size_t)r * dv + cc] * kt[r];
            /* delta = beta (v - alpha u);  h <- alpha h + k delta^T */
            for (int cc = 0; cc < dv; ++cc) u[cc] = bt * (vt[cc] - alpha * u[cc]);
            for (int r = 0; r < dk; ++r)
                for (int cc = 0; cc < dv; ++cc)
                    h[(size_t)r * dv + cc] = alpha * h[(size_t)r * dv + cc] + kt[r] * u[cc];
            /* o_t = h^T (scale q)  (= S_t q_t, read after the update) */
            double* ot = o + tv * dv;
            for (int cc = 0; cc < dv; ++cc) ot[cc] = 0.0;
            for (int r = 0; r < dk; ++r) {
                const double qr = scale * qt[r];
                for (int cc = 0; cc < dv; ++cc) ot[cc] += h[(size_t)r * dv + cc] * qr;
            }
        }
        if (s_final) memcpy(s_final + (size_t)c * dk * dv, h, sizeof(double) * (size_t)dk * dv);
        free(h);
        free(u);
    }
    return bad ? -1 : 0;
}

/* Number of threads an OpenMP parallel region of this library would use. */
int gdn_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

