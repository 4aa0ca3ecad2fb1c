/*
 * Body of the sequential reference recurrences.  Included twice by
 * lrs_oracle.c, once with REAL=double (suffix _f64) and once with REAL=float
 * (suffix _f32).  Every loop below is the plain definition of the recurrence,
 * one time step after another, with no blocking, fusion or reordering.
 *
 * TEST INFRASTRUCTURE: see the header comment of lrs_oracle.c.
 */

#define ORC_CAT2(a, b) a##b
#define ORC_CAT(a, b) ORC_CAT2(a, b)
#define ORC_FN(name) ORC_CAT(name, SFX)

/*
 * First-order FMA recurrence, per channel (b, n):
 *     s_t = a_t * s_{t-1} + b_t,   t = 1..T,   s_0 = s0[b,n] (0 when s0 is NULL)
 * [SunnyNet log §2.1, the "FMA" form of the unified update].
 * Layout: a, bb, s are [B,T,N] row-major; s0, s_final are [B,N].
 * Memory row t-1 of s holds s_t; s_final = s_T.
 * The channels of one batch row are advanced together (loop over n inside the
 * loop over t) only so that memory is read in order; each channel's own
 * arithmetic is the definition, step by step.
 */
void ORC_FN(orc_scan_fma)(const REAL* a, const REAL* bb, const REAL* s0, REAL* s,
                          REAL* s_final, int64_t B, int64_t T, int64_t N, int nthreads) {
    int64_t nblk = (N + ORC_NBLK - 1) / ORC_NBLK;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (int64_t w = 0; w < B * nblk; ++w) {
        int64_t b = w / nblk, n_lo = (w % nblk) * ORC_NBLK;
        int64_t n_hi = n_lo + ORC_NBLK < N ? n_lo + ORC_NBLK : N;
        REAL st[ORC_NBLK];
        for (int64_t n = n_lo; n < n_hi; ++n) st[n - n_lo] = s0 ? s0[b * N + n] : (REAL)0;
        for (int64_t t = 0; t < T; ++t) {
            int64_t row = (b * T + t) * N;
            for (int64_t n = n_lo; n < n_hi; ++n) {
                REAL prod = a[row + n] * st[n - n_lo];
                REAL next = prod + bb[row + n];
                st[n - n_lo] = next;
                s[row + n] = next;
            }
        }
        for (int64_t n = n_lo; n < n_hi; ++n) s_final[b * N + n] = st[n - n_lo];
    }
}

/*
 * Gated (convex) first-order recurrence, per channel (b, n):
 *     s_t = a_t * s_{t-1} + (1 - a_t) * u_t
 * [SunnyNet log §2.1, the gated form of the unified update], evaluated in the
 * literal order written there.  Layout and s0 / s_final as orc_scan_fma.
 */
void ORC_FN(orc_scan_gated)(const REAL* a, const REAL* u, const REAL* s0, REAL* s,
                            REAL* s_final, int64_t B, int64_t T, int64_t N, int nthreads) {
    int64_t nblk = (N + ORC_NBLK - 1) / ORC_NBLK;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (int64_t w = 0; w < B * nblk; ++w) {
        int64_t b = w / nblk, n_lo = (w % nblk) * ORC_NBLK;
        int64_t n_hi = n_lo + ORC_NBLK < N ? n_lo + ORC_NBLK : N;
        REAL st[ORC_NBLK];
        for (int64_t n = n_lo; n < n_hi; ++n) st[n - n_lo] = s0 ? s0[b * N + n] : (REAL)0;
        for (int64_t t = 0; t < T; ++t) {
            int64_t row = (b * T + t) * N;
            for (int64_t n = n_lo; n < n_hi; ++n) {
                REAL at = a[row + n];
                REAL keep = at * st[n - n_lo];
                REAL inject = ((REAL)1 - at) * u[row + n];
                REAL next = keep + inject;
                st[n - n_lo] = next;
                s[row + n] = next;
            }
        }
        for (int64_t n = n_lo; n < n_hi; ++n) s_final[b * N + n] = st[n - n_lo];
    }
}

/*
 * Reverse (adjoint) pass of the two elementwise recurrences, per channel (b, n):
 * the back-ends' reverse-scan entry [SunnyNet log §8], read as the gradient
 * pass used in training.  Given the forward states s_t and the gradient ds_t
 * of a loss with respect to each output s_t (plus ds_final with respect to
 * the returned final state), the total derivative with respect to s_t is
 *     gs_T = ds_T + ds_final,     gs_t = ds_t + a_{t+1} * gs_{t+1}   (t < T)
 * because s_t enters the loss directly and through s_{t+1} = a_{t+1} s_t + ...
 * The input gradients follow from one step's partial derivatives:
 *     FMA   s_t = a_t s_{t-1} + b_t:           da_t = gs_t * s_{t-1},  db_t = gs_t
 *     gated s_t = a_t s_{t-1} + (1-a_t) u_t:   da_t = gs_t * (s_{t-1} - u_t),
 *                                               du_t = gs_t * (1 - a_t)
 *     both: ds0 = a_1 * gs_1
 * with s_0 = s0 (0 when s0 is NULL).  Layout: a, u, s, ds, da, dx are
 * [B,T,N] (memory row t-1 holds step t); s0, ds_final, ds0 are [B,N];
 * ds_final NULL means zero, ds0 NULL means not wanted.  `u` is read only by
 * the gated form (pass NULL for the FMA form, whose dx is db).
 */
static void ORC_FN(orc_elem_bwd)(int gated, const REAL* a, const REAL* u, const REAL* s0,
                                 const REAL* s, const REAL* ds, const REAL* ds_final, REAL* da,
                                 REAL* dx, REAL* ds0, int64_t B, int64_t T, int64_t N,
                                 int nthreads) {
    int64_t nblk = (N + ORC_NBLK - 1) / ORC_NBLK;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (int64_t w = 0; w < B * nblk; ++w) {
        int64_t b = w / nblk, n_lo = (w % nblk) * ORC_NBLK;
        int64_t n_hi = n_lo + ORC_NBLK < N ? n_lo + ORC_NBLK : N;
        REAL gs[ORC_NBLK];
        for (int64_t t = T - 1; t >= 0; --t) {
            int64_t row = (b * T + t) * N;
            for (int64_t n = n_lo; n < n_hi; ++n) {
                REAL later;
                if (t == T - 1) later = ds_final ? ds_final[b * N + n] : (REAL)0;
                else later = a[row + N + n] * gs[n - n_lo];
                REAL g = ds[row + n] + later;
                gs[n - n_lo] = g;
                REAL prev = t > 0 ? s[row - N + n] : (s0 ? s0[b * N + n] : (REAL)0);
                if (gated) {
                    da[row + n] = g * (prev - u[row + n]);
                    dx[row + n] = g * ((REAL)1 - a[row + n]);
                } else {
                    da[row + n] = g * prev;
                    dx[row + n] = g;
                }
            }
        }
        if (ds0)
            for (int64_t n = n_lo; n < n_hi; ++n) ds0[b * N + n] = a[b * T * N + n] * gs[n - n_lo];
    }
}

void ORC_FN(orc_scan_fma_bwd)(const REAL* a, const REAL* s0, const REAL* s, const REAL* ds,
                              const REAL* ds_final, REAL* da, REAL* db, REAL* ds0, int64_t B,
                              int64_t T, int64_t N, int nthreads) {
    ORC_FN(orc_elem_bwd)(0, a, NULL, s0, s, ds, ds_final, da, db, ds0, B, T, N, nthreads);
}

void ORC_FN(orc_scan_gated_bwd)(const REAL* a, const REAL* u, const REAL* s0, const REAL* s,
                                const REAL* ds, const REAL* ds_final, REAL* da, REAL* du,
                                REAL* ds0, int64_t B, int64_t T, int64_t N, int nthreads) {
    ORC_FN(orc_elem_bwd)(1, a, u, s0, s, ds, ds_final, da, du, ds0, B, T, N, nthreads);
}

/*
 * Decay-separable outer-product state recurrence with readout, per (b, h):
 *     alpha_t[i] = exp(g[b,t,h])        (decay_mode 0: one decay per head and step)
 *     alpha_t[i] = exp(g[b,t,h,i])      (decay_mode 1: one decay per key row)
 *     S_t[i][j]  = alpha_t[i] * S_{t-1}[i][j] + (kappa_t * k_t[i]) * v_t[j]
 *     o_t[j]     = scale * sum_i S_t[i][j] * q_t[i]      (read after the update)
 * Mamba-2: decay exp(dt*A) shared by the whole state, injection (dt*B) outer x
 * [SunnyNet log §4.1]; GLA: decay diag(exp(gk)) on the key axis, readout
 * scale * S^T q [SunnyNet log §4.3]; both restated in [vs llama.cpp §3].
 * kappa_t = k_scale[b,t,h] (1 when k_scale is NULL), or, with a per-key
 * scale, kappa_t[i] = k_scale_key[b,t,h,i]: the matrix associative memory
 * S_t = p (.) S_{t-1} + (1 - p) (.) (v_t (x) k_t) [vs llama.cpp §8] is this
 * recurrence with a per-key p: g = log p, kappa = 1 - p.
 * Layouts: q, k [B,T,Hg,K]; v, o [B,T,H,V]; g [B,T,H] or [B,T,H,K];
 * k_scale [B,T,H]; k_scale_key [B,T,H,K]; s0, s_final [B,H,K,V].  Head h
 * reads q/k group h/(H/Hg).  At most one of k_scale, k_scale_key is given.
 */
void ORC_FN(orc_scan_diag_outer)(const REAL* q, const REAL* k, const REAL* v, const REAL* g,
                                 int decay_mode, const REAL* k_scale, const REAL* k_scale_key,
                                 REAL scale, const REAL* s0, REAL* o, REAL* s_final, int64_t B,
                                 int64_t T, int64_t H, int64_t Hg, int64_t K, int64_t V,
                                 int nthreads) {
    int64_t heads_per_group = H / Hg;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t bh = 0; bh < B * H; ++bh) {
        int64_t b = bh / H, h = bh % H, grp = h / heads_per_group;
        REAL* S = (REAL*)malloc(sizeof(REAL) * (size_t)(K * V));
        REAL* alpha = (REAL*)malloc(sizeof(REAL) * (size_t)K);
        for (int64_t e = 0; e < K * V; ++e) S[e] = s0 ? s0[bh * K * V + e] : (REAL)0;
        for (int64_t t = 0; t < T; ++t) {
            const REAL* qt = q + ((b * T + t) * Hg + grp) * K;
            const REAL* kt = k + ((b * T + t) * Hg + grp) * K;
            const REAL* vt = v + ((b * T + t) * H + h) * V;
            REAL kap = k_scale ? k_scale[(b * T + t) * H + h] : (REAL)1;
            for (int64_t i = 0; i < K; ++i) {
                REAL gi = decay_mode == 0 ? g[(b * T + t) * H + h] : g[((b * T + t) * H + h) * K + i];
                alpha[i] = ORC_EXP(gi);
            }
            for (int64_t i = 0; i < K; ++i) {
                REAL kap_i = k_scale_key ? k_scale_key[((b * T + t) * H + h) * K + i] : kap;
                REAL kk = kap_i * kt[i];
                for (int64_t j = 0; j < V; ++j) {
                    REAL keep = alpha[i] * S[i * V + j];
                    REAL inject = kk * vt[j];
                    S[i * V + j] = keep + inject;
                }
            }
            REAL* ot = o + ((b * T + t) * H + h) * V;
            for (int64_t j = 0; j < V; ++j) {
                REAL acc = 0;
                for (int64_t i = 0; i < K; ++i) acc += S[i * V + j] * qt[i];
                ot[j] = scale * acc;
            }
        }
        for (int64_t e = 0; e < K * V; ++e) s_final[bh * K * V + e] = S[e];
        free(S);
        free(alpha);
    }
}

/*
 * Delta rule with readout, rank-1 form, per (b, h):
 *     p_j      = sum_i S_{t-1}[i][j] * k_t[i]          (p = S^T k)
 *     delta_j  = beta_t * (v_t[j] - p_j)
 *     S_t[i][j]= S_{t-1}[i][j] + k_t[i] * delta_j       (S += k outer delta)
 *     o_t[j]   = scale * sum_i S_t[i][j] * q_t[i]       (o = scale * S^T q)
 * [SunnyNet log §4.2]; restated in [vs llama.cpp §3].  The pages read out
 * with no scale, i.e. scale = 1.
 * Layouts: q, k [B,T,H,K]; v, o [B,T,H,V]; beta [B,T,H]; s0, s_final [B,H,K,V].
 */
void ORC_FN(orc_scan_delta)(const REAL* q, const REAL* k, const REAL* v, const REAL* beta,
                            REAL scale, const REAL* s0, REAL* o, REAL* s_final, int64_t B,
                            int64_t T, int64_t H, int64_t K, int64_t V, int nthreads) {
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t bh = 0; bh < B * H; ++bh) {
        int64_t b = bh / H, h = bh % H;
        REAL* S = (REAL*)malloc(sizeof(REAL) * (size_t)(K * V));
        REAL* dl = (REAL*)malloc(sizeof(REAL) * (size_t)V);
        for (int64_t e = 0; e < K * V; ++e) S[e] = s0 ? s0[bh * K * V + e] : (REAL)0;
        for (int64_t t = 0; t < T; ++t) {
            const REAL* qt = q + ((b * T + t) * H + h) * K;
            const REAL* kt = k + ((b * T + t) * H + h) * K;
            const REAL* vt = v + ((b * T + t) * H + h) * V;
            REAL bt = beta[(b * T + t) * H + h];
            for (int64_t j = 0; j < V; ++j) {
                REAL p = 0;
                for (int64_t i = 0; i < K; ++i) p += S[i * V + j] * kt[i];
                dl[j] = bt * (vt[j] - p);
            }
            for (int64_t i = 0; i < K; ++i)
                for (int64_t j = 0; j < V; ++j) S[i * V + j] += kt[i] * dl[j];
            REAL* ot = o + ((b * T + t) * H + h) * V;
            for (int64_t j = 0; j < V; ++j) {
                REAL acc = 0;
                for (int64_t i = 0; i < K; ++i) acc += S[i * V + j] * qt[i];
                ot[j] = scale * acc;
            }
        }
        for (int64_t e = 0; e < K * V; ++e) s_final[bh * K * V + e] = S[e];
        free(S);
        free(dl);
    }
}

/*
 * Delta rule, explicit form, per (b, h): a second, independent implementation
 * of the same update, written as a dense K x K transition
 *     M_t = I - beta_t * k_t k_t^T,      S_t = M_t S_{t-1} + beta_t * k_t v_t^T
 * [SunnyNet log §4.2, the explicit (I - beta k k^T) S + beta k v^T form that
 * the page says must be implemented and checked separately from the rank-1
 * form].  Readout and layouts as orc_scan_delta.
 */
void ORC_FN(orc_scan_delta_explicit)(const REAL* q, const REAL* k, const REAL* v,
                                     const REAL* beta, REAL scale, const REAL* s0, REAL* o,
                                     REAL* s_final, int64_t B, int64_t T, int64_t H, int64_t K,
                                     int64_t V, int nthreads) {
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t bh = 0; bh < B * H; ++bh) {
        int64_t b = bh / H, h = bh % H;
        REAL* S = (REAL*)malloc(sizeof(REAL) * (size_t)(K * V));
        REAL* Sn = (REAL*)malloc(sizeof(REAL) * (size_t)(K * V));
        REAL* M = (REAL*)malloc(sizeof(REAL) * (size_t)(K * K));
        for (int64_t e = 0; e < K * V; ++e) S[e] = s0 ? s0[bh * K * V + e] : (REAL)0;
        for (int64_t t = 0; t < T; ++t) {
            const REAL* qt = q + ((b * T + t) * H + h) * K;
            const REAL* kt = k + ((b * T + t) * H + h) * K;
            const REAL* vt = v + ((b * T + t) * H + h) * V;
            REAL bt = beta[(b * T + t) * H + h];
            for (int64_t r = 0; r < K; ++r)
                for (int64_t c = 0; c < K; ++c)
                    M[r * K + c] = (r == c ? (REAL)1 : (REAL)0) - bt * kt[r] * kt[c];
            for (int64_t r = 0; r < K; ++r)
                for (int64_t j = 0; j < V; ++j) {
                    REAL acc = 0;
                    for (int64_t c = 0; c < K; ++c) acc += M[r * K + c] * S[c * V + j];
                    Sn[r * V + j] = acc + bt * kt[r] * vt[j];
                }
            REAL* tmp = S;
            S = Sn;
            Sn = tmp;
            REAL* ot = o + ((b * T + t) * H + h) * V;
            for (int64_t j = 0; j < V; ++j) {
                REAL acc = 0;
                for (int64_t i = 0; i < K; ++i) acc += S[i * V + j] * qt[i];
                ot[j] = scale * acc;
            }
        }
        for (int64_t e = 0; e < K * V; ++e) s_final[bh * K * V + e] = S[e];
        free(S);
        free(Sn);
        free(M);
    }
}

/*
 * Delta rule with a per-key decay (RWKV-7's state update), rank-1 form, per
 * (b, h):
 *     w_t[i]   = exp(g[b,t,h,i])                         (decay on the key axis)
 *     p_j      = sum_i S_{t-1}[i][j] * k_t[i]             (read-back of the OLD state)
 *     delta_j  = beta_t * (v_t[j] - p_j)
 *     S_t[i][j]= w_t[i] * S_{t-1}[i][j] + k_t[i] * delta_j
 *     o_t[j]   = scale * sum_i S_t[i][j] * q_t[i]
 * [SunnyNet log §5.1]: the page writes S_t = S_{t-1} (.) w_t - (S_{t-1} k_t) k_t^T
 * + v_t k_t^T for a state stored value-major; stored key-major ([K,V]) as
 * here, with the in-context rate beta_t that the page's formula leaves out
 * (beta = 1 gives the page's form), that is
 * S_t = (diag(w_t) - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T: the removal
 * reads the state before the decay.  With w = 1 it is orc_scan_delta.
 * Layouts: q, k, g [B,T,H,K]; v, o [B,T,H,V]; beta [B,T,H]; s0, s_final [B,H,K,V].
 */
void ORC_FN(orc_scan_delta_decay)(const REAL* q, const REAL* k, const REAL* v, const REAL* g,
                                  const REAL* beta, REAL scale, const REAL* s0, REAL* o,
                                  REAL* s_final, int64_t B, int64_t T, int64_t H, int64_t K,
                                  int64_t V, int nthreads) {
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t bh = 0; bh < B * H; ++bh) {
        int64_t b = bh / H, h = bh % H;
        REAL* S = (REAL*)malloc(sizeof(REAL) * (size_t)(K * V));
        REAL* dl = (REAL*)malloc(sizeof(REAL) * (size_t)V);
        for (int64_t e = 0; e < K * V; ++e) S[e] = s0 ? s0[bh * K * V + e] : (REAL)0;
        for (int64_t t = 0; t < T; ++t) {
            const REAL* qt = q + ((b * T + t) * H + h) * K;
            const REAL* kt = k + ((b * T + t) * H + h) * K;
            const REAL* gt = g + ((b * T + t) * H + h) * K;
            const REAL* vt = v + ((b * T + t) * H + h) * V;
            REAL bt = beta[(b * T + t) * H + h];
            for (int64_t j = 0; j < V; ++j) {
                REAL p = 0;
                for (int64_t i = 0; i < K; ++i) p += S[i * V + j] * kt[i];
                dl[j] = bt * (vt[j] - p);
            }
            for (int64_t i = 0; i < K; ++i) {
                REAL wi = ORC_EXP(gt[i]);
                for (int64_t j = 0; j < V; ++j) S[i * V + j] = wi * S[i * V + j] + kt[i] * dl[j];
            }
            REAL* ot = o + ((b * T + t) * H + h) * V;
            for (int64_t j = 0; j < V; ++j) {
                REAL acc = 0;
                for (int64_t i = 0; i < K; ++i) acc += S[i * V + j] * qt[i];
                ot[j] = scale * acc;
            }
        }
        for (int64_t e = 0; e < K * V; ++e) s_final[bh * K * V + e] = S[e];
        free(S);
        free(dl);
    }
}

/*
 * The same update as orc_scan_delta_decay, written as a dense K x K
 * transition [SunnyNet log §5.1, in the key-major reading above]:
 *     M_t = diag(w_t) - beta_t * k_t k_t^T,   S_t = M_t S_{t-1} + beta_t * k_t v_t^T
 * implemented separately from the rank-1 form.  Readout and layouts as there.
 */
void ORC_FN(orc_scan_delta_decay_explicit)(const REAL* q, const REAL* k, const REAL* v,
                                           const REAL* g, const REAL* beta, REAL scale,
                                           const REAL* s0, REAL* o, REAL* s_final, int64_t B,
                                           int64_t T, int64_t H, int64_t K, int64_t V,
                                           int nthreads) {
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t bh = 0; bh < B * H; ++bh) {
        int64_t b = bh / H, h = bh % H;
        REAL* S = (REAL*)malloc(sizeof(REAL) * (size_t)(K * V));
        REAL* Sn = (REAL*)malloc(sizeof(REAL) * (size_t)(K * V));
        REAL* M = (REAL*)malloc(sizeof(REAL) * (size_t)(K * K));
        for (int64_t e = 0; e < K * V; ++e) S[e] = s0 ? s0[bh * K * V + e] : (REAL)0;
        for (int64_t t = 0; t < T; ++t) {
            const REAL* qt = q + ((b * T + t) * H + h) * K;
            const REAL* kt = k + ((b * T + t) * H + h) * K;
            const REAL* gt = g + ((b * T + t) * H + h) * K;
            const REAL* vt = v + ((b * T + t) * H + h) * V;
            REAL bt = beta[(b * T + t) * H + h];
            for (int64_t r = 0; r < K; ++r)
                for (int64_t c = 0; c < K; ++c)
                    M[r * K + c] = (r == c ? ORC_EXP(gt[r]) : (REAL)0) - bt * kt[r] * kt[c];
            for (int64_t r = 0; r < K; ++r)
                for (int64_t j = 0; j < V; ++j) {
                    REAL acc = 0;
                    for (int64_t c = 0; c < K; ++c) acc += M[r * K + c] * S[c * V + j];
                    Sn[r * V + j] = acc + bt * kt[r] * vt[j];
                }
            REAL* tmp = S;
            S = Sn;
            Sn = tmp;
            REAL* ot = o + ((b * T + t) * H + h) * V;
            for (int64_t j = 0; j < V; ++j) {
                REAL acc = 0;
                for (int64_t i = 0; i < K; ++i) acc += S[i * V + j] * qt[i];
                ot[j] = scale * acc;
            }
        }
        for (int64_t e = 0; e < K * V; ++e) s_final[bh * K * V + e] = S[e];
        free(S);
        free(Sn);
        free(M);
    }
}

#undef ORC_FN
#undef ORC_CAT
#undef ORC_CAT2
