/*
 * Oracle for Kimi Delta Attention (KDA): the delta rule with a per-key-channel decay, plain
 * token-by-token float64 recurrence on the CPU.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load this library.  It shares no code, header or constant with the HIP library.
 *
 * What it computes ("Gated Attention Architectures", section 8 (KDA), Mathematical Formulation):
 *   S_t = (I - beta_t k_t k_t^T) D_t S_{t-1} + beta_t v_t k_t^T,   o_t = S_t^T q_t,
 *   D_t = diag(alpha_t), alpha_t in (0, 1]^{dk}, one decay per key channel,
 * with S in R^{dk x dv} (the key axis first, as in that section's formula and its decay along the
 * key axis), stored as [B, Hv, dk, dv] with dv contiguous.  Expanded, exactly (up to rounding):
 *   h' = D_t h                (each key row m scaled by alpha_t[m])
 *   u  = h'^T k_t,  delta = beta_t (v_t - u),  h = h' + k_t delta^T,  o_t = h^T (scale q_t)
 * g = log alpha is given per (token, value head, key channel); beta one per (token, value head).
 * Value head j reads query/key head floor(j / (Hv / Hqk)).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* q, k: [B,T,Hqk,dk]; v: [B,T,Hv,dv]; g: [B,T,Hv,dk]; beta: [B,T,Hv];
 * s0: [B,Hv,dk,dv] or NULL (zeros); o: [B,T,Hv,dv]; s_final: [B,Hv,dk,dv] or NULL. */
int gdn_oracle_kda_recurrent(const double* q, const double* k, const double* v, const double* g,
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
            const double* gt = g + tv * dk;
            const double bt = beta[tv];
            /* h <- D_t h: key row m decays by alpha_t[m] */
            for (int r = 0; r < dk; ++r) {
                const double a = exp(gt[r]);
                for (int cc = 0; cc < dv; ++cc) h[(size_t)r * dv + cc] *= a;
            }
            /* u = h^T k;  delta = beta (v - u);  h <- h + k delta^T */
            for (int cc = 0; cc < dv; ++cc) u[cc] = 0.0;
            for (int r = 0; r < dk; ++r)
                for (int cc = 0; cc < dv; ++cc) u[cc] += h[(size_t)r * dv + cc] * kt[r];
            for (int cc = 0; cc < dv; ++cc) u[cc] = bt * (vt[cc] - u[cc]);
            for (int r = 0; r < dk; ++r)
                for (int cc = 0; cc < dv; ++cc) h[(size_t)r * dv + cc] += kt[r] * u[cc];
            /* o_t = h^T (scale q) */
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
