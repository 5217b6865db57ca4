/* The fp64 oracle (oracle/gdn_oracle.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer: small random problems through every entry
 * point (forward with chunk states, a head selection, the input transforms
 * and v_new, summaries, merge, backward),
 * ragged and empty units, and the invalid arguments it must reject. Every
 * output array is exactly as large as its declared shape. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int gdn_oracle_fwd(int64_t n_units, const int64_t* offsets, int64_t H, int64_t K, int64_t V, const float* q,
                   const float* k, const float* v, const float* g, const float* beta, int gate_per_key,
                   int use_exp2, double scale, const double* S0, int64_t n_sel, const int64_t* heads_sel,
                   double* o, double* S_final, int64_t chunk, double* chunk_states, int qk_l2norm,
                   int beta_sigmoid, double eps, double* v_new, int n_threads);
int gdn_oracle_summary(int64_t n_units, const int64_t* offsets, int64_t H, int64_t K, int64_t V, const float* k,
                       const float* v, const float* g, const float* beta, int gate_per_key, int use_exp2,
                       int64_t n_sel, const int64_t* heads_sel, double* S_ext, double* M, int qk_l2norm,
                       int beta_sigmoid, double eps, int n_threads);
int gdn_oracle_merge(int64_t n_seg, int64_t n, int64_t K, int64_t V, const double* S_ext, const double* M,
                     const double* S0, double* S_init);
int gdn_oracle_bwd(int64_t n_units, const int64_t* offsets, int64_t H, int64_t K, int64_t V, const float* q,
                   const float* k, const float* v, const float* g, const float* beta, int gate_per_key, int use_exp2,
                   double scale, const double* S0, const double* dout, const double* dht, double* dq, double* dk,
                   double* dv, double* dg, double* dbeta, double* dS0, int n_threads);

static uint64_t state = 88172645463325252ull;
static double urand(void) {
    state ^= state << 13; state ^= state >> 7; state ^= state << 17;
    return (double)(state >> 11) / 9007199254740992.0;
}
static float* rnd(size_t n, double lo, double hi) {
    float* p = malloc(sizeof(float) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) p[i] = (float)(lo + (hi - lo) * urand());
    return p;
}

int main(void) {
    int bad = 0;
    for (int it = 0; it < 60; ++it) {
        const int64_t H = 1 + it % 3, K = 4 + it % 5, V = 3 + it % 4, n_units = 1 + it % 4;
        int64_t offs[8];
        offs[0] = 0;
        for (int64_t u = 1; u <= n_units; ++u) offs[u] = offs[u - 1] + (int64_t)(urand() * 70);   /* empty units allowed */
        const int64_t N = offs[n_units], chunk = 16;
        const int pk = it & 1;
        float *q = rnd((size_t)(N * H * K), -1, 1), *k = rnd((size_t)(N * H * K), -1, 1);
        float *v = rnd((size_t)(N * H * V), -1, 1), *beta = rnd((size_t)(N * H), 0, 1);
        float* g = rnd((size_t)(N * H * (pk ? K : 1)), -0.5, 0);
        int64_t n_chunks = 0;
        for (int64_t u = 0; u < n_units; ++u) n_chunks += (offs[u + 1] - offs[u] + chunk - 1) / chunk;
        const int64_t sel[2] = {H - 1, 0};
        const int64_t n_sel = H > 1 ? 2 : 1;
        double* o = malloc(sizeof(double) * (size_t)(N * n_sel * V + 1));
        double* fin = malloc(sizeof(double) * (size_t)(n_units * n_sel * K * V));
        double* cs = malloc(sizeof(double) * (size_t)(n_chunks * n_sel * K * V + 1));
        double* S0 = malloc(sizeof(double) * (size_t)(n_units * H * K * V));
        for (int64_t i = 0; i < n_units * H * K * V; ++i) S0[i] = urand() - 0.5;
        double* vn = malloc(sizeof(double) * (size_t)(N * n_sel * V + 1));
        bad |= gdn_oracle_fwd(n_units, offs, H, K, V, q, k, v, g, beta, pk, it & 2, 0.5, S0, n_sel, sel, o, fin,
                              chunk, cs, it & 4, it & 8, 1e-6, (it & 16) ? NULL : vn, 2) != 0;
        free(vn);
        double* ext = malloc(sizeof(double) * (size_t)(n_units * H * K * V));
        double* M = malloc(sizeof(double) * (size_t)(n_units * H * K * K));
        bad |= gdn_oracle_summary(n_units, offs, H, K, V, k, v, g, beta, pk, it & 2, H, NULL, ext, M, it & 4, it & 8,
                                  1e-6, 2) != 0;
        double* si = malloc(sizeof(double) * (size_t)((n_units + 1) * H * K * V));
        if (K == V) bad |= gdn_oracle_merge(n_units, H, K, V, ext, M, S0, si) != 0;
        /* backward, with dL/dh_final on even iterations */
        double* dout = malloc(sizeof(double) * (size_t)(N * H * V + 1));
        for (int64_t i = 0; i < N * H * V; ++i) dout[i] = urand() - 0.5;
        double* dq = malloc(sizeof(double) * (size_t)(N * H * K + 1));
        double* dk = malloc(sizeof(double) * (size_t)(N * H * K + 1));
        double* dv = malloc(sizeof(double) * (size_t)(N * H * V + 1));
        double* dgr = malloc(sizeof(double) * (size_t)(N * H * (pk ? K : 1) + 1));
        double* dbt = malloc(sizeof(double) * (size_t)(N * H + 1));
        double* dS0 = malloc(sizeof(double) * (size_t)(n_units * H * K * V));
        bad |= gdn_oracle_bwd(n_units, offs, H, K, V, q, k, v, g, beta, pk, it & 2, 0.5, S0, dout,
                              (it & 4) ? NULL : S0, dq, dk, dv, dgr, dbt, (it & 8) ? NULL : dS0, 2) != 0;
        bad |= gdn_oracle_bwd(n_units, offs, H, K, V, q, k, v, g, beta, pk, 0, 0.5, NULL, NULL, NULL, dq, dk, dv,
                              dgr, dbt, NULL, 1) == 0;
        free(dout); free(dq); free(dk); free(dv); free(dgr); free(dbt); free(dS0);
        /* rejected arguments */
        int64_t broken[3] = {0, 5, 3};
        bad |= gdn_oracle_fwd(2, broken, H, K, V, q, k, v, g, beta, pk, 0, 1.0, NULL, H, NULL, NULL, NULL, 0, NULL,
                              0, 0, 0.0, NULL, 1) == 0;
        const int64_t wrong_head[1] = {H};
        bad |= gdn_oracle_fwd(n_units, offs, H, K, V, q, k, v, g, beta, pk, 0, 1.0, NULL, 1, wrong_head, o, NULL,
                              0, NULL, 0, 0, 0.0, NULL, 1) == 0;
        bad |= gdn_oracle_summary(n_units, offs, H, K, V, k, v, g, beta, pk, 0, H + 1, NULL, ext, M, 0, 0, 0.0,
                                  1) == 0;
        bad |= gdn_oracle_merge(-1, H, K, V, ext, M, NULL, si) == 0;
        free(q); free(k); free(v); free(beta); free(g); free(o); free(fin); free(cs); free(S0);
        free(ext); free(M); free(si);
    }
    printf("oracle driver: %s\n", bad ? "FAILED" : "ok");
    return bad;
}
