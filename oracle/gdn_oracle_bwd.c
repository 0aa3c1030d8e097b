/*
 * Oracle for the backward pass of the gated delta rule: reverse-mode adjoint of the plain
 * float64 recurrence in gdn_oracle.c, token by token, on the CPU.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load this library.  It shares no code, header or constant with the HIP library.
 *
 * The recurrence differentiated is the Gated DeltaNet state update ("Architecture Thread I:
 * Gated Attention, DeltaNet, and Hybrid Models", section "Gated DeltaNet"; "Gated Attention
 * Architectures", section 3) in its erase/write form, state stored as h = S^T [B, Hv, dk, dv],
 * readout o_t = h_t^T (scale q_t); value head j reads query/key head floor(j / (Hv / Hqk)).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/*
 * Backward of the same recurrence (reverse-mode adjoint, token by token, float64).
 *
 * Given dL/do_t (dout) and dL/dh_T (dsf, or NULL for zero), where h_T is the final state,
 * returns dL/dq, dL/dk (per value head: [B,T,Hv,dk]; a query/key head's gradient is the sum over
 * the value heads of its group), dL/dv [B,T,Hv,dv], dL/dg and dL/dbeta [B,T,Hv] and dL/dS0
 * [B,Hv,dk,dv].  Every step of the forward above is differentiated in turn, latest token first:
 *   o = h_t^T (scale q)          dh += scale q do^T,        dq  = scale h_t do
 *   h_t = a h_{t-1} + k d^T      dd  = dh^T k,  dk += dh d,   da  = <dh, h_{t-1}>,   dh_{t-1} = a dh
 *   d = beta (v - a u)           dbeta = <dd, v - a u>,  dv = beta dd,  du = -beta a dd,
 *                                da += -beta <dd, u>
 *   u = h_{t-1}^T k              dh_{t-1} += k du^T,  dk += h_{t-1} du
 *   a = exp(g)                   dg = a da
 * The states h_{t-1} are recomputed from checkpoints taken every 64 tokens.
 */
int gdn_oracle_recurrent_bwd(const double* q, const double* k, const double* v, const double* g,
                             const double* beta, const double* s0, const double* dout, const double* dsf,
                             double* dq_v, double* dk_v, double* dvv, double* dg, double* dbeta,
                             double* ds0, int B, int T, int Hqk, int Hv, int dk, int dv, double scale,
                             int nthreads)
{
    if (B <= 0 || T < 0 || Hqk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || Hv % Hqk != 0) return -1;
    const int grp = Hv / Hqk;
    const int SEG = 64;
    const int nseg = (T + SEG - 1) / SEG;
    const size_t hsz = (size_t)dk * dv;
    const long long nchains = (long long)B * Hv;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(|: bad)
#endif
    for (long long c = 0; c < nchains; ++c) {
        const int b = (int)(c / Hv), j = (int)(c % Hv), i = j / grp;
        double* ck = (double*)malloc(sizeof(double) * hsz * (size_t)(nseg > 0 ? nseg : 1));
        double* hs = (double*)malloc(sizeof(double) * hsz * (size_t)(SEG + 1));
        double* dh = (double*)malloc(sizeof(double) * hsz);
        double* u = (double*)malloc(sizeof(double) * (size_t)dv);
        double* dd = (double*)malloc(sizeof(double) * (size_t)dv);
        double* du = (double*)malloc(sizeof(double) * (size_t)dv);
        double* d = (double*)malloc(sizeof(double) * (size_t)dv);
        if (!ck || !hs || !dh || !u || !dd || !du || !d) {
            free(ck); free(hs); free(dh); free(u); free(dd); free(du); free(d);
            bad |= 1;
            continue;
        }
        /* forward, keeping the state at the start of every segment */
        double* h = hs;
        if (s0) memcpy(h, s0 + (size_t)c * hsz, sizeof(double) * hsz);
        else memset(h, 0, sizeof(double) * hsz);
        for (int t = 0; t < T; ++t) {
            if (t % SEG == 0) memcpy(ck + (size_t)(t / SEG) * hsz, h, sizeof(double) * hsz);
            const size_t tqk = (((size_t)b * T + t) * Hqk + i), tv = (((size_t)b * T + t) * Hv + j);
            const double* kt = k + tqk * dk;
            const double* vt = v + tv * dv;
            const double a = exp(g[tv]), bt = beta[tv];
            for (int cc = 0; cc < dv; ++cc) u[cc] = 0.0;
            for (int r = 0; r < dk; ++r)
                for (int cc = 0; cc < dv; ++cc) u[cc] += h[(size_t)r * dv + cc] * kt[r];
            for (int cc = 0; cc < dv; ++cc) u[cc] = bt * (vt[cc] - a * u[cc]);
            for (int r = 0; r < dk; ++r)
                for (int cc = 0; cc < dv; ++cc) h[(size_t)r * dv + cc] = a * h[(size_t)r * dv + cc] + kt[r] * u[cc];
        }
        /* backward */
        if (dsf) memcpy(dh, dsf + (size_t)c * hsz, sizeof(double) * hsz);
        else memset(dh, 0, sizeof(double) * hsz);
        for (int sg = nseg - 1; sg >= 0; --sg) {
            const int t0 = sg * SEG, t1 = (t0 + SEG < T) ? t0 + SEG : T;
            /* states of the segment: hs[s] is the state before token t0 + s */
            memcpy(hs, ck + (size_t)sg * hsz, sizeof(double) * hsz);
            for (int t = t0; t < t1; ++t) {
                const size_t tqk = (((size_t)b * T + t) * Hqk + i), tv = (((size_t)b * T + t) * Hv + j);
                const double* kt = k + tqk * dk;
                const double* vt = v + tv * dv;
                const double a = exp(g[tv]), bt = beta[tv];
                const double* hp = hs + (size_t)(t - t0) * hsz;
                double* hn = hs + (size_t)(t - t0 + 1) * hsz;
                for (int cc = 0; cc < dv; ++cc) u[cc] = 0.0;
                for (int r = 0; r < dk; ++r)
                    for (int cc = 0; cc < dv; ++cc) u[cc] += hp[(size_t)r * dv + cc] * kt[r];
                for (int cc = 0; cc < dv; ++cc) d[cc] = bt * (vt[cc] - a * u[cc]);
                for (int r = 0; r < dk; ++r)
                    for (int cc = 0; cc < dv; ++cc) hn[(size_t)r * dv + cc] = a * hp[(size_t)r * dv + cc] + kt[r] * d[cc];
            }
            for (int t = t1 - 1; t >= t0; --t) {
                const size_t tqk = (((size_t)b * T + t) * Hqk + i), tv = (((size_t)b * T + t) * Hv + j);
                const double* kt = k + tqk * dk;
                const double* qt = q + tqk * dk;
                const double* vt = v + tv * dv;
                const double* dot = dout + tv * dv;
                const double a = exp(g[tv]), bt = beta[tv];
                const double* hp = hs + (size_t)(t - t0) * hsz;
                const double* hn = hs + (size_t)(t - t0 + 1) * hsz;
                double* dqt = dq_v + tv * dk;
                double* dkt = dk_v + tv * dk;
                /* o = h_t^T (scale q) */
                for (int r = 0; r < dk; ++r) {
                    double acc = 0.0;
                    for (int cc = 0; cc < dv; ++cc) {
                        dh[(size_t)r * dv + cc] += scale * qt[r] * dot[cc];
                        acc += hn[(size_t)r * dv + cc] * dot[cc];
                    }
                    dqt[r] = scale * acc;
                }
                /* recompute u and d of this token */
                for (int cc = 0; cc < dv; ++cc) u[cc] = 0.0;
                for (int r = 0; r < dk; ++r)
                    for (int cc = 0; cc < dv; ++cc) u[cc] += hp[(size_t)r * dv + cc] * kt[r];
                for (int cc = 0; cc < dv; ++cc) d[cc] = bt * (vt[cc] - a * u[cc]);
                /* h_t = a h_{t-1} + k d^T */
                double da = 0.0;
                for (int cc = 0; cc < dv; ++cc) dd[cc] = 0.0;
                for (int r = 0; r < dk; ++r) {
                    double acc = 0.0;
                    for (int cc = 0; cc < dv; ++cc) {
                        const double x = dh[(size_t)r * dv + cc];
                        dd[cc] += x * kt[r];
                        acc += x * d[cc];
                        da += x * hp[(size_t)r * dv + cc];
                    }
                    dkt[r] = acc;
                }
                /* d = beta (v - a u) */
                double db = 0.0, du_u = 0.0;
                for (int cc = 0; cc < dv; ++cc) {
                    db += dd[cc] * (vt[cc] - a * u[cc]);
                    dvv[tv * dv + cc] = bt * dd[cc];
                    du[cc] = -bt * a * dd[cc];
                    du_u += dd[cc] * u[cc];
                }
                da += -bt * du_u;
                dbeta[tv] = db;
                /* u = h_{t-1}^T k;  dh_{t-1} = a dh + k du^T */
                for (int r = 0; r < dk; ++r) {
                    double acc = 0.0;
                    for (int cc = 0; cc < dv; ++cc) {
                        acc += hp[(size_t)r * dv + cc] * du[cc];
                        dh[(size_t)r * dv + cc] = a * dh[(size_t)r * dv + cc] + kt[r] * du[cc];
                    }
                    dkt[r] += acc;
                }
                dg[tv] = a * da;
            }
        }
        memcpy(ds0 + (size_t)c * hsz, dh, sizeof(double) * hsz);
        free(ck); free(hs); free(dh); free(u); free(dd); free(du); free(d);
    }
    return bad ? -1 : 0;
}
