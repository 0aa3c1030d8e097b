/* Runs the float64 oracle (oracle/gdn_oracle*.c, compiled into this program with AddressSanitizer
 * and UndefinedBehaviorSanitizer) over small inputs: ragged and empty sequences, grouped heads,
 * with and without initial and final states, alpha = 0 and beta at its limits, and sizes it must
 * reject.  Test infrastructure: built and run by tests/test_sanitizers.py.  Exit status 0 means
 * every call returned what it should and produced finite values; a sanitizer report aborts. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int gdn_oracle_recurrent(const double*, const double*, const double*, const double*, const double*,
                         const double*, double*, double*, int, int, int, int, int, int, double, int);
int gdn_oracle_recurrent_bwd(const double*, const double*, const double*, const double*, const double*,
                             const double*, const double*, const double*, double*, double*, double*,
                             double*, double*, double*, int, int, int, int, int, int, double, int);
int gdn_oracle_kda_recurrent(const double*, const double*, const double*, const double*, const double*,
                             const double*, double*, double*, int, int, int, int, int, int, double, int);

static unsigned long long rng = 88172645463325252ULL;
static double uni(void)
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (double)(rng >> 11) / 9007199254740992.0;
}

static double* arr(size_t n, double lo, double hi)
{
    double* p = (double*)malloc(sizeof(double) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * uni();
    return p;
}

static int finite_all(const double* p, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(p[i])) return 0;
    return 1;
}

static int fails = 0;
#define CHECK(c)                                                         \
    do {                                                                 \
        if (!(c)) {                                                      \
            fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
            ++fails;                                                     \
        }                                                                \
    } while (0)

static void one(int B, int T, int Hqk, int Hv, int dk, int dv, int with_s0, int with_sf, int gate_case)
{
    const size_t nqk = (size_t)B * T * Hqk * dk, nv = (size_t)B * T * Hv * dv, ng = (size_t)B * T * Hv;
    const size_t ns = (size_t)B * Hv * dk * dv;
    double *q = arr(nqk, -0.5, 0.5), *k = arr(nqk, -0.5, 0.5), *v = arr(nv, -1, 1);
    double *g = arr(ng, -0.3, 0.0), *beta = arr(ng, 0.0, 1.0), *s0 = with_s0 ? arr(ns, -0.1, 0.1) : NULL;
    for (size_t i = 0; i < ng; ++i) {
        if (gate_case == 1 && i % 3 == 0) g[i] = -INFINITY; /* alpha = 0 */
        if (gate_case == 2) beta[i] = i % 2 ? 0.0 : 1.0;
    }
    double *o = arr(nv, 0, 0), *sf = with_sf ? arr(ns, 0, 0) : NULL;
    CHECK(gdn_oracle_recurrent(q, k, v, g, beta, s0, o, sf, B, T, Hqk, Hv, dk, dv, 0.75, 2) == 0);
    CHECK(finite_all(o, nv));
    if (sf) CHECK(finite_all(sf, ns));
    /* backward: gradients of <dO, O> + <dS, S_T>; dq and dk per value head [B,T,Hv,dk] */
    const size_t nqv = (size_t)B * T * Hv * dk;
    double *dout = arr(nv, -1, 1), *dsf = arr(ns, -1, 1);
    double *dq = arr(nqv, 0, 0), *dkk = arr(nqv, 0, 0), *dvv = arr(nv, 0, 0), *dg = arr(ng, 0, 0);
    double *db = arr(ng, 0, 0), *ds0 = arr(ns, 0, 0);
    if (gate_case != 1) { /* the adjoint's exp(g) = 0 path is covered by the forward */
        CHECK(gdn_oracle_recurrent_bwd(q, k, v, g, beta, s0, dout, dsf, dq, dkk, dvv, dg, db, ds0, B, T, Hqk, Hv, dk,
                                       dv, 0.75, 2) == 0);
        CHECK(finite_all(dq, nqv) && finite_all(dkk, nqv) && finite_all(dvv, nv) && finite_all(dg, ng) &&
              finite_all(db, ng) && finite_all(ds0, ns));
    }
    /* KDA: one log decay per key channel */
    double* gk = arr(ng * dk, -0.3, 0.0);
    CHECK(gdn_oracle_kda_recurrent(q, k, v, gk, beta, s0, o, sf, B, T, Hqk, Hv, dk, dv, 1.0, 2) == 0);
    CHECK(finite_all(o, nv));
    free(q); free(k); free(v); free(g); free(beta); free(s0); free(o); free(sf);
    free(dout); free(dsf); free(dq); free(dkk); free(dvv); free(dg); free(db); free(ds0); free(gk);
}

int main(void)
{
    one(2, 37, 1, 2, 8, 4, 1, 1, 0);
    one(1, 1, 2, 4, 4, 8, 0, 1, 0);
    one(3, 0, 1, 1, 4, 4, 1, 1, 0);   /* empty sequence: the final state is the initial one */
    one(1, 70, 1, 3, 6, 5, 1, 0, 0);  /* 70 tokens cross the adjoint's 64-token checkpoints */
    one(2, 20, 1, 2, 4, 4, 1, 1, 1);  /* alpha = 0 on a third of the tokens */
    one(1, 25, 1, 1, 4, 4, 1, 1, 2);  /* beta in {0, 1} */
    /* sizes the oracle must reject */
    double x = 0.0, y = 0.0;
    CHECK(gdn_oracle_recurrent(&x, &x, &x, &x, &x, NULL, &y, NULL, 1, 1, 2, 3, 1, 1, 1.0, 1) == -1); /* Hv % Hqk */
    CHECK(gdn_oracle_recurrent(&x, &x, &x, &x, &x, NULL, &y, NULL, 0, 1, 1, 1, 1, 1, 1.0, 1) == -1);
    CHECK(gdn_oracle_kda_recurrent(&x, &x, &x, &x, &x, NULL, &y, NULL, 1, -1, 1, 1, 1, 1, 1.0, 1) == -1);
    if (fails) return 1;
    printf("oracle driver: ok\n");
    return 0;
}
