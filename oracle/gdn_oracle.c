/*
 * Plain fp64 CPU oracle for the gated delta rule forward.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link,
 * load or call this file: only the tests, the smoke check and the CPU
 * baseline leg of the benchmark use it. It shares no code, header, table or
 * helper with the HIP library.
 *
 * What it computes (one (unit, head) pair at a time, token by token, in the
 * order the tokens appear; a "unit" is a document of a packed batch, a batch
 * row, or a segment of a row):
 *
 *   d      = b^{g_t}                (b = e, or 2 when use_exp2; g_t is a
 *                                    scalar per (token, head) or a K-vector)
 *   h     <- Diag(d) h              (decay first)
 *   p      = h^T k_t                (V-vector)
 *   h     <- h + beta_t k_t (v_t - p)^T
 *   o_t    = scale * h^T q_t
 *
 * h is the K x V state.  For a scalar gate the decay-then-update order is the
 * recurrence h_t = exp(g_t) (I - beta_t k_t k_t^T) h_{t-1} + beta_t k_t v_t^T
 * of the gated delta rule problem statement.  For a per-key gate the state is
 * decayed before the delta update; that is the order of the chunk recurrence
 * on the hyper-parallel state_summary.py coverage page
 * (kda_split_state_summary_kernel: the residual u - w*state is taken before
 * the state is scaled by 2^{g_last} and the gated-key update added).
 *
 * Segment summaries (same page, kda_split_state_summary_kernel, and the
 * apply_kda_state_summary helper on the hyper-parallel Diff Coverage page):
 * running a segment from an entry state S gives M*S + S_ext, where
 *   S_ext = the state reached from S = 0, and
 *   M     = the product of the per-token maps (I - beta k k^T) Diag(d),
 *           i.e. the same update with v = 0 applied to X = I (K x K).
 *
 * Backward (reverse mode of the same token recurrence; the backward slots of
 * the native GDN op on the hyper-parallel Diff Coverage page,
 * _AscendCGDN.backward: dq, dk, dv, dbeta and the raw-gate gradient dg),
 * given do_t = dL/do_t and dL/dh_final, with h~ = Diag(d) h_{t-1} the
 * decayed state and u = v_t - h~^T k_t, token by token from the last:
 *
 *   dh    += scale q_t do_t^T          dq_t = scale h_t do_t
 *   dv_t   = beta_t dh^T k_t           dbeta_t = k_t^T dh u
 *   dk_t   = beta_t dh u - h~ dv_t     dh~ = dh - k_t dv_t^T
 *   dg_t   = ln(b) sum_j dh~[i][j] h~[i][j]   (summed over i for a scalar gate)
 *   dh     = Diag(d) dh~
 *
 * and dL/dS0 is dh after the unit's first token. The states h_{t-1}, h_t
 * are recomputed chunk by chunk (64 tokens) from the state stored at each
 * chunk start, with the forward's own operations, so they are the forward's
 * values.
 *
 * Input transforms (the in-kernel options of the native prepare on the Diff
 * Coverage page, use_qk_l2norm_in_kernel and use_beta_sigmoid_in_kernel,
 * whose slots q_hat, k_hat, q_rstd, k_rstd and beta_eff the ten-slot result
 * names): with qk_l2norm, q_t and k_t are replaced by x * r with
 * r = 1 / sqrt(sum_i x_i^2 + eps) before anything else; with beta_sigmoid,
 * beta_t by 1 / (1 + e^{-beta_t}).  The forward can also return
 * v_new_t = beta_t (v_t - p) (p as above), the value the token writes: the
 * chunk form's v_new = u - w h (chunk_fwd_h on the same page returns it),
 * which unrolled over a chunk is exactly this per-token quantity.
 *
 * All arithmetic is fp64.  Inputs are fp32 arrays (exact copies of the
 * rounded bf16 or fp32 inputs).  Layout: the token axis is flat (a
 * [B,T,H,D] tensor is viewed as [B*T, H, D]); units are given by token
 * offsets into that axis.
 *
 * Return value: 0 on success, -1 on an invalid argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double decay_of(double x, int use_exp2) { return use_exp2 ? exp2(x) : exp(x); }

static int check_offsets(int64_t n_units, const int64_t* offsets) {
    if (n_units < 0 || offsets == NULL) return -1;
    if (offsets[0] < 0) return -1;
    for (int64_t u = 0; u < n_units; ++u)
        if (offsets[u + 1] < offsets[u]) return -1;
    return 0;
}

/* x as fp64, L2-normalised when l2norm is set; returns the reciprocal norm
 * used (1 without normalisation). */
static double load_vec(double* dst, const float* src, int64_t K, int l2norm, double eps) {
    double ss = 0.0;
    for (int64_t i = 0; i < K; ++i) {
        dst[i] = (double)src[i];
        ss += dst[i] * dst[i];
    }
    const double r = l2norm ? 1.0 / sqrt(ss + eps) : 1.0;
    if (l2norm)
        for (int64_t i = 0; i < K; ++i) dst[i] *= r;
    return r;
}

static double beta_of(float b, int sigmoid) { return sigmoid ? 1.0 / (1.0 + exp(-(double)b)) : (double)b; }

/* One token of the recurrence applied to the K x V state h (row i = key i). */
static void token_step(double* h, int64_t K, int64_t V, const double* kt, const float* vt,
                       double beta, const double* d /* [K] decay per key row */, double* p) {
    for (int64_t i = 0; i < K; ++i) {
        double di = d[i];
        double* hi = h + i * V;
        for (int64_t j = 0; j < V; ++j) hi[j] *= di;
    }
    for (int64_t j = 0; j < V; ++j) p[j] = 0.0;
    for (int64_t i = 0; i < K; ++i) {
        double ki = kt[i];
        const double* hi = h + i * V;
        for (int64_t j = 0; j < V; ++j) p[j] += hi[j] * ki;
    }
    for (int64_t i = 0; i < K; ++i) {
        double bk = beta * kt[i];
        double* hi = h + i * V;
        for (int64_t j = 0; j < V; ++j) hi[j] += bk * ((double)vt[j] - p[j]);
    }
}

static void gate_vector(double* d, const float* g, int64_t t, int64_t H, int64_t hd, int64_t K,
                        int gate_per_key, int use_exp2) {
    if (gate_per_key) {
        const float* gt = g + (t * H + hd) * K;
        for (int64_t i = 0; i < K; ++i) d[i] = decay_of((double)gt[i], use_exp2);
    } else {
        double s = decay_of((double)g[t * H + hd], use_exp2);
        for (int64_t i = 0; i < K; ++i) d[i] = s;
    }
}

int gdn_oracle_fwd(int64_t n_units, const int64_t* offsets, int64_t H, int64_t K, int64_t V,
                   const float* q, const float* k, const float* v, const float* g, const float* beta,
                   int gate_per_key, int use_exp2, double scale, const double* S0, int64_t n_sel,
                   const int64_t* heads_sel, double* o, double* S_final, int64_t chunk,
                   double* chunk_states, int qk_l2norm, int beta_sigmoid, double eps, double* v_new,
                   int n_threads) {
    if (check_offsets(n_units, offsets) != 0 || H <= 0 || K <= 0 || V <= 0) return -1;
    if (n_sel <= 0 || n_sel > H) return -1;
    if (chunk_states != NULL && chunk <= 0) return -1;
    /* first chunk index of every unit, for the chunk-boundary state output */
    int64_t* chunk_base = (int64_t*)calloc((size_t)n_units + 1, sizeof(int64_t));
    if (!chunk_base) return -1;
    if (chunk_states != NULL)
        for (int64_t u = 0; u < n_units; ++u) {
            int64_t len = offsets[u + 1] - offsets[u];
            chunk_base[u + 1] = chunk_base[u] + (len + chunk - 1) / chunk;
        }
    int64_t n_tasks = n_units * n_sel;
    int bad = 0;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
#endif
    for (int64_t task = 0; task < n_tasks; ++task) {
        int64_t u = task / n_sel, s = task % n_sel;
        int64_t hd = heads_sel ? heads_sel[s] : s;
        if (hd < 0 || hd >= H) { bad |= 1; continue; }
        double* h = (double*)malloc(sizeof(double) * (size_t)(K * V));
        double* p = (double*)malloc(sizeof(double) * (size_t)V);
        double* d = (double*)malloc(sizeof(double) * (size_t)K);
        double* kx = (double*)malloc(sizeof(double) * (size_t)K);
        double* qx = (double*)malloc(sizeof(double) * (size_t)K);
        if (!h || !p || !d || !kx || !qx) { free(h); free(p); free(d); free(kx); free(qx); bad |= 1; continue; }
        if (S0) memcpy(h, S0 + (u * H + hd) * K * V, sizeof(double) * (size_t)(K * V));
        else memset(h, 0, sizeof(double) * (size_t)(K * V));
        int64_t t0 = offsets[u], t1 = offsets[u + 1];
        for (int64_t t = t0; t < t1; ++t) {
            int64_t local = t - t0;
            if (chunk_states && local % chunk == 0)
                memcpy(chunk_states + ((chunk_base[u] + local / chunk) * n_sel + s) * K * V, h,
                       sizeof(double) * (size_t)(K * V));
            gate_vector(d, g, t, H, hd, K, gate_per_key, use_exp2);
            load_vec(kx, k + (t * H + hd) * K, K, qk_l2norm, eps);
            const double bt = beta_of(beta[t * H + hd], beta_sigmoid);
            const float* vt = v + (t * H + hd) * V;
            token_step(h, K, V, kx, vt, bt, d, p);
            if (v_new) {
                double* nt = v_new + (t * n_sel + s) * V;
                for (int64_t j = 0; j < V; ++j) nt[j] = bt * ((double)vt[j] - p[j]);
            }
            if (o) {
                load_vec(qx, q + (t * H + hd) * K, K, qk_l2norm, eps);
                double* ot = o + (t * n_sel + s) * V;
                for (int64_t j = 0; j < V; ++j) ot[j] = 0.0;
                for (int64_t i = 0; i < K; ++i) {
                    double qi = qx[i];
                    const double* hi = h + i * V;
                    for (int64_t j = 0; j < V; ++j) ot[j] += hi[j] * qi;
                }
                for (int64_t j = 0; j < V; ++j) ot[j] *= scale;
            }
        }
        if (S_final) memcpy(S_final + (u * n_sel + s) * K * V, h, sizeof(double) * (size_t)(K * V));
        free(h); free(p); free(d); free(kx); free(qx);
    }
    free(chunk_base);
    return bad ? -1 : 0;
}

/*
 * Per-unit summaries: S_ext[u] (K x V, the state reached from zero) and
 * M[u] (K x K, the state map with v = 0 applied to the identity).  Either
 * output may be NULL.
 */
int gdn_oracle_summary(int64_t n_units, const int64_t* offsets, int64_t H, int64_t K, int64_t V,
                       const float* k, const float* v, const float* g, const float* beta,
                       int gate_per_key, int use_exp2, int64_t n_sel, const int64_t* heads_sel,
                       double* S_ext, double* M, int qk_l2norm, int beta_sigmoid, double eps,
                       int n_threads) {
    if (check_offsets(n_units, offsets) != 0 || H <= 0 || K <= 0 || V <= 0) return -1;
    if (n_sel <= 0 || n_sel > H) return -1;
    int64_t n_tasks = n_units * n_sel;
    int bad = 0;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
#endif
    for (int64_t task = 0; task < n_tasks; ++task) {
        int64_t u = task / n_sel, s = task % n_sel;
        int64_t hd = heads_sel ? heads_sel[s] : s;
        if (hd < 0 || hd >= H) { bad |= 1; continue; }
        double* h = (double*)calloc((size_t)(K * V), sizeof(double));
        double* x = (double*)calloc((size_t)(K * K), sizeof(double));
        double* p = (double*)malloc(sizeof(double) * (size_t)(V > K ? V : K));
        double* d = (double*)malloc(sizeof(double) * (size_t)K);
        float* zero_v = (float*)calloc((size_t)K, sizeof(float));
        double* kx = (double*)malloc(sizeof(double) * (size_t)K);
        if (!h || !x || !p || !d || !zero_v || !kx) {
            free(h); free(x); free(p); free(d); free(zero_v); free(kx); bad |= 1; continue;
        }
        for (int64_t i = 0; i < K; ++i) x[i * K + i] = 1.0;
        for (int64_t t = offsets[u]; t < offsets[u + 1]; ++t) {
            gate_vector(d, g, t, H, hd, K, gate_per_key, use_exp2);
            double b = beta_of(beta[t * H + hd], beta_sigmoid);
            load_vec(kx, k + (t * H + hd) * K, K, qk_l2norm, eps);
            if (S_ext) token_step(h, K, V, kx, v + (t * H + hd) * V, b, d, p);
            if (M) token_step(x, K, K, kx, zero_v, b, d, p);
        }
        if (S_ext) memcpy(S_ext + (u * n_sel + s) * K * V, h, sizeof(double) * (size_t)(K * V));
        if (M) memcpy(M + (u * n_sel + s) * K * K, x, sizeof(double) * (size_t)(K * K));
        free(h); free(x); free(p); free(d); free(zero_v); free(kx);
    }
    return bad ? -1 : 0;
}

/*
 * Merge of segment summaries in order: S_init[0] = S0 (zero when NULL),
 * S_init[s+1] = M_s S_init[s] + S_ext[s] (apply_kda_state_summary on the
 * hyper-parallel Diff Coverage page: matmul(transition, initial_state) +
 * state_ext).  Arrays: S_ext [n_seg][n][K][V], M [n_seg][n][K][K],
 * S0 [n][K][V], S_init [n_seg + 1][n][K][V] (the last entry is the state at
 * the end of the last segment).  n counts independent states (rows x heads).
 */
int gdn_oracle_merge(int64_t n_seg, int64_t n, int64_t K, int64_t V, const double* S_ext,
                     const double* M, const double* S0, double* S_init) {
    if (n_seg < 0 || n <= 0 || K <= 0 || V <= 0) return -1;
    for (int64_t r = 0; r < n; ++r) {
        double* first = S_init + r * K * V;
        if (S0) memcpy(first, S0 + r * K * V, sizeof(double) * (size_t)(K * V));
        else memset(first, 0, sizeof(double) * (size_t)(K * V));
    }
    for (int64_t s = 0; s < n_seg; ++s)
        for (int64_t r = 0; r < n; ++r) {
            const double* prev = S_init + (s * n + r) * K * V;
            double* next = S_init + ((s + 1) * n + r) * K * V;
            const double* m = M + (s * n + r) * K * K;
            const double* e = S_ext + (s * n + r) * K * V;
            for (int64_t i = 0; i < K; ++i)
                for (int64_t j = 0; j < V; ++j) {
                    double acc = e[i * V + j];
                    for (int64_t c = 0; c < K; ++c) acc += m[i * K + c] * prev[c * V + j];
                    next[i * V + j] = acc;
                }
        }
    return 0;
}

/*
 * Backward of gdn_oracle_fwd (see the header). dout [N][H][V] and dht
 * [n_units][H][K][V] (NULL: zero) are fp64; outputs dq, dk [N][H][K], dv
 * [N][H][V], dbeta [N][H], dg [N][H] (scalar gate) or [N][H][K] (per key)
 * and dS0 [n_units][H][K][V] (may be NULL) are fp64, for every head.
 */
int gdn_oracle_bwd(int64_t n_units, const int64_t* offsets, int64_t H, int64_t K, int64_t V,
                   const float* q, const float* k, const float* v, const float* g, const float* beta,
                   int gate_per_key, int use_exp2, double scale, const double* S0, const double* dout,
                   const double* dht, double* dq, double* dk, double* dv, double* dg, double* dbeta,
                   double* dS0, int n_threads) {
    if (check_offsets(n_units, offsets) != 0 || H <= 0 || K <= 0 || V <= 0) return -1;
    if (!dout || !dq || !dk || !dv || !dg || !dbeta) return -1;
    const int64_t C = 64;                       /* tokens per recomputed chunk */
    const double lnb = use_exp2 ? log(2.0) : 1.0;
    const int64_t KV = K * V;
    int64_t n_tasks = n_units * H;
    int bad = 0;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
#endif
    for (int64_t task = 0; task < n_tasks; ++task) {
        const int64_t u = task / H, hd = task % H;
        const int64_t t0 = offsets[u], t1 = offsets[u + 1], n = t1 - t0;
        const int64_t nc = (n + C - 1) / C;
        double* ck = (double*)malloc(sizeof(double) * (size_t)((nc > 0 ? nc : 1) * KV));   /* chunk-start states */
        double* st = (double*)malloc(sizeof(double) * (size_t)((C + 1) * KV));            /* states in a chunk */
        double* dh = (double*)malloc(sizeof(double) * (size_t)KV);
        double* ht = (double*)malloc(sizeof(double) * (size_t)KV);                        /* h~ */
        double* d = (double*)malloc(sizeof(double) * (size_t)K);
        double* p = (double*)malloc(sizeof(double) * (size_t)V);
        double* uu = (double*)malloc(sizeof(double) * (size_t)V);
        double* dvt = (double*)malloc(sizeof(double) * (size_t)V);
        double* tmp = (double*)malloc(sizeof(double) * (size_t)K);
        double* kx = (double*)malloc(sizeof(double) * (size_t)K);
        if (!ck || !st || !dh || !ht || !d || !p || !uu || !dvt || !tmp || !kx) {
            free(ck); free(st); free(dh); free(ht); free(d); free(p); free(uu); free(dvt); free(tmp); free(kx);
            bad |= 1;
            continue;
        }
        /* forward, keeping the state at every chunk start */
        double* h = st;
        if (S0) memcpy(h, S0 + (u * H + hd) * KV, sizeof(double) * (size_t)KV);
        else memset(h, 0, sizeof(double) * (size_t)KV);
        for (int64_t t = t0; t < t1; ++t) {
            if ((t - t0) % C == 0) memcpy(ck + ((t - t0) / C) * KV, h, sizeof(double) * (size_t)KV);
            gate_vector(d, g, t, H, hd, K, gate_per_key, use_exp2);
            load_vec(kx, k + (t * H + hd) * K, K, 0, 0.0);
            token_step(h, K, V, kx, v + (t * H + hd) * V, (double)beta[t * H + hd], d, p);
        }
        /* reverse */
        if (dht) memcpy(dh, dht + (u * H + hd) * KV, sizeof(double) * (size_t)KV);
        else memset(dh, 0, sizeof(double) * (size_t)KV);
        for (int64_t c = nc - 1; c >= 0; --c) {
            const int64_t a = t0 + c * C, b = (a + C < t1) ? a + C : t1;
            /* st[i] = state after token a + i - 1 (st[0] = chunk-start state) */
            memcpy(st, ck + c * KV, sizeof(double) * (size_t)KV);
            for (int64_t t = a; t < b; ++t) {
                double* nx = st + (t - a + 1) * KV;
                memcpy(nx, st + (t - a) * KV, sizeof(double) * (size_t)KV);
                gate_vector(d, g, t, H, hd, K, gate_per_key, use_exp2);
                load_vec(kx, k + (t * H + hd) * K, K, 0, 0.0);
                token_step(nx, K, V, kx, v + (t * H + hd) * V, (double)beta[t * H + hd], d, p);
            }
            for (int64_t t = b - 1; t >= a; --t) {
                const double* hprev = st + (t - a) * KV;
                const double* hcur = st + (t - a + 1) * KV;
                const float* qt = q + (t * H + hd) * K;
                const float* kt = k + (t * H + hd) * K;
                const float* vt = v + (t * H + hd) * V;
                const double* dot = dout + (t * H + hd) * V;
                const double bt = (double)beta[t * H + hd];
                /* output: dh += scale q do^T, dq = scale h_t do */
                for (int64_t i = 0; i < K; ++i) {
                    double acc = 0.0;
                    for (int64_t j = 0; j < V; ++j) {
                        dh[i * V + j] += scale * (double)qt[i] * dot[j];
                        acc += hcur[i * V + j] * dot[j];
                    }
                    dq[(t * H + hd) * K + i] = scale * acc;
                }
                /* the decayed state and the residual */
                gate_vector(d, g, t, H, hd, K, gate_per_key, use_exp2);
                for (int64_t i = 0; i < K; ++i)
                    for (int64_t j = 0; j < V; ++j) ht[i * V + j] = d[i] * hprev[i * V + j];
                for (int64_t j = 0; j < V; ++j) {
                    double acc = 0.0;
                    for (int64_t i = 0; i < K; ++i) acc += ht[i * V + j] * (double)kt[i];
                    uu[j] = (double)vt[j] - acc;
                }
                /* dv = beta dh^T k; dbeta = k^T dh u; dk = beta dh u - h~ dv */
                double db = 0.0;
                for (int64_t j = 0; j < V; ++j) {
                    double acc = 0.0;
                    for (int64_t i = 0; i < K; ++i) acc += dh[i * V + j] * (double)kt[i];
                    dvt[j] = bt * acc;
                    db += acc * uu[j];
                }
                dbeta[t * H + hd] = db;
                for (int64_t j = 0; j < V; ++j) dv[(t * H + hd) * V + j] = dvt[j];
                for (int64_t i = 0; i < K; ++i) {
                    double a1 = 0.0, a2 = 0.0;
                    for (int64_t j = 0; j < V; ++j) {
                        a1 += dh[i * V + j] * uu[j];
                        a2 += ht[i * V + j] * dvt[j];
                    }
                    dk[(t * H + hd) * K + i] = bt * a1 - a2;
                }
                /* dh~ = dh - k dv^T, the gate gradient, then dh = Diag(d) dh~ */
                for (int64_t i = 0; i < K; ++i) {
                    double acc = 0.0;
                    for (int64_t j = 0; j < V; ++j) {
                        const double x = dh[i * V + j] - (double)kt[i] * dvt[j];
                        acc += x * ht[i * V + j];
                        dh[i * V + j] = d[i] * x;
                    }
                    tmp[i] = lnb * acc;
                }
                if (gate_per_key) {
                    for (int64_t i = 0; i < K; ++i) dg[(t * H + hd) * K + i] = tmp[i];
                } else {
                    double s = 0.0;
                    for (int64_t i = 0; i < K; ++i) s += tmp[i];
                    dg[t * H + hd] = s;
                }
            }
        }
        if (dS0) memcpy(dS0 + (u * H + hd) * KV, dh, sizeof(double) * (size_t)KV);
        free(ck); free(st); free(dh); free(ht); free(d); free(p); free(uu); free(dvt); free(tmp); free(kx);
    }
    return bad ? -1 : 0;
}

int gdn_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
