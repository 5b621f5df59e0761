/*
 * Plain fp64 CPU oracle for the gated delta rule forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The product path
 * (the HIP library and its Python binding) never calls, links or imports it,
 * and it shares no code, header, table or helper with that path.
 *
 * Every routine is a slow, literal statement of what the method computes:
 * scalar loops in double precision, no blocking, no SIMD intrinsics, no
 * fast-math.  Inputs arrive as float32 arrays (a bf16 input is passed as the
 * float32 that holds the same value exactly) and are widened to double on
 * read.  Outputs are double.  The only parallelism is an OpenMP loop over
 * independent (batch, head) pairs, or over independent tokens for the prep.
 *
 * Sources (web pages, cited by title and section):
 *   [cam]  Sana "fused_cam_gdn.py" - camera-branch prep and scan.
 *   [dp]   msj19 "gated_deltaproduct" test.py - chunkwise gated DeltaProduct.
 *   [cp]   Sana "fused_gdn_cp.py" - context-parallel wrappers (state
 *          conventions in the module docstring).
 *
 * State convention throughout: S has shape (Dk, Dv), rows indexed by the key
 * dimension and columns by the value dimension, as in [cam] _cam_scan_kernel
 * (comment on the state layout) and [dp] gated_chunk_delta_rule_fwd_kernel_h.
 * The read-out is o = scale * S^T q.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static int thread_num(void) {
#ifdef _OPENMP
    return omp_get_thread_num();
#else
    return 0;
#endif
}

/* ------------------------------------------------------------------------ */
/* O1: gated delta rule, token by token.                                    */
/*                                                                          */
/* For one (b, h), starting from S = h0 (or 0), for t = 0 .. T-1:           */
/*   S <- exp(g_t) S                       (gate the carried state)         */
/*   p <- S^T k_t                          (what the gated state predicts)  */
/*   S <- S + beta_t k_t (v_t - p)^T       (delta-rule correction)          */
/*   o_t <- scale * S^T q_t                (read-out after the update)      */
/* and finally hT = S.  This is the recurrence                              */
/*   S_t = exp(g_t) (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T       */
/* written in the (Dk, Dv) state convention.  Cites: [cam] _cam_scan_kernel */
/* with one token per frame (decay, predict, correct, read out); [dp] the   */
/* chunk kernels, whose token-level meaning this is for r = 1.              */
/* Layouts: q,k (B,T,H,Dk); v (B,T,H,Dv); beta, g (B,T,H);                  */
/* h0, hT (B,H,Dk,Dv); o (B,T,H,Dv).                                        */
/* ------------------------------------------------------------------------ */
int oracle_gdn_recurrent(int B, int T, int H, int Dk, int Dv,
                         const float *q, const float *k, const float *v,
                         const float *beta, const float *g, double scale,
                         const float *h0, double *o, double *hT, int nthreads) {
    if (B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0) return -1;
    set_threads(nthreads);
    int npairs = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < npairs; ++bh) {
        int b = bh / H, h = bh % H;
        double *S = (double *)calloc((size_t)Dk * Dv, sizeof(double));
        double *p = (double *)malloc(sizeof(double) * (size_t)Dv);
        if (h0)
            for (int i = 0; i < Dk * Dv; ++i) S[i] = (double)h0[(size_t)bh * Dk * Dv + i];
        for (int t = 0; t < T; ++t) {
            size_t row = ((size_t)b * T + t) * H + h;
            const float *qt = q + row * Dk, *kt = k + row * Dk, *vt = v + row * Dv;
            double decay = exp((double)g[row]);
            double bt = (double)beta[row];
            for (int i = 0; i < Dk * Dv; ++i) S[i] *= decay;
            for (int j = 0; j < Dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < Dk; ++i) acc += S[(size_t)i * Dv + j] * (double)kt[i];
                p[j] = acc;
            }
            for (int i = 0; i < Dk; ++i) {
                double ki = bt * (double)kt[i];
                for (int j = 0; j < Dv; ++j) S[(size_t)i * Dv + j] += ki * ((double)vt[j] - p[j]);
            }
            for (int j = 0; j < Dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < Dk; ++i) acc += S[(size_t)i * Dv + j] * (double)qt[i];
                o[row * Dv + j] = scale * acc;
            }
        }
        if (hT)
            for (int i = 0; i < Dk * Dv; ++i) hT[(size_t)bh * Dk * Dv + i] = S[i];
        free(S);
        free(p);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* O2: gated DeltaProduct, token by token ([dp]).                           */
/*                                                                          */
/* The key of width K = r*dk is split into r sub-keys k_{t,a} (columns      */
/* a*dk .. (a+1)*dk-1).  Step a of token t writes with the sub-key k_{t,a}  */
/* into row block a of the state, and erases along the key                  */
/*   e_{t,a} = sum_b M[a][b] E_b k_{t,b}                                    */
/* (E_b places a dk-vector into row block b; M is the r x r step mask read  */
/* as in gated_chunk_scaled_dot_kkt_fwd_kernel, where column b of the mask  */
/* weights sub-key b for every step a).  Per token:                         */
/*   P   <- exp(g_t) S                                                      */
/*   p_a <- P^T e_{t,a}            for every a, all from the same P         */
/*   S   <- P + sum_a beta_{t,a} E_a k_{t,a} (v_t - p_a)^T                  */
/*   o_t <- scale * S^T q_t                                                 */
/* Steps of one token do not see each other's writes: the intra-chunk      */
/* matrix of [dp] is strictly lower triangular over tokens, so entries      */
/* between two steps of one token are zero.                                 */
/* Layouts: q,k (B,T,H,r*dk); v (B,T,H,Dv); beta (B,T,H,r); g (B,T,H);      */
/* mask (r,r) row-major double; h0,hT (B,H,r*dk,Dv); o (B,T,H,Dv).          */
/* ------------------------------------------------------------------------ */
int oracle_deltaproduct_recurrent(int B, int T, int H, int r, int dk, int Dv,
                                  const float *q, const float *k, const float *v,
                                  const float *beta, const float *g,
                                  const double *mask, double scale,
                                  const float *h0, double *o, double *hT,
                                  int nthreads) {
    if (B < 0 || T < 0 || H < 0 || r <= 0 || dk <= 0 || Dv <= 0) return -1;
    set_threads(nthreads);
    int K = r * dk;
    int npairs = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < npairs; ++bh) {
        int b = bh / H, h = bh % H;
        double *S = (double *)calloc((size_t)K * Dv, sizeof(double));
        double *pa = (double *)malloc(sizeof(double) * (size_t)r * Dv);
        double *e = (double *)malloc(sizeof(double) * (size_t)K);
        if (h0)
            for (int i = 0; i < K * Dv; ++i) S[i] = (double)h0[(size_t)bh * K * Dv + i];
        for (int t = 0; t < T; ++t) {
            size_t row = ((size_t)b * T + t) * H + h;
            const float *qt = q + row * K, *kt = k + row * K, *vt = v + row * Dv;
            const float *bt = beta + row * r;
            double decay = exp((double)g[row]);
            for (int i = 0; i < K * Dv; ++i) S[i] *= decay;
            for (int a = 0; a < r; ++a) {
                for (int bb = 0; bb < r; ++bb)
                    for (int c = 0; c < dk; ++c)
                        e[bb * dk + c] = mask[a * r + bb] * (double)kt[bb * dk + c];
                for (int j = 0; j < Dv; ++j) {
                    double acc = 0.0;
                    for (int i = 0; i < K; ++i) acc += S[(size_t)i * Dv + j] * e[i];
                    pa[(size_t)a * Dv + j] = acc;
                }
            }
            for (int a = 0; a < r; ++a) {
                double ba = (double)bt[a];
                for (int c = 0; c < dk; ++c) {
                    int i = a * dk + c;
                    double ki = ba * (double)kt[i];
                    for (int j = 0; j < Dv; ++j)
                        S[(size_t)i * Dv + j] += ki * ((double)vt[j] - pa[(size_t)a * Dv + j]);
                }
            }
            for (int j = 0; j < Dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < K; ++i) acc += S[(size_t)i * Dv + j] * (double)qt[i];
                o[row * Dv + j] = scale * acc;
            }
        }
        if (hT)
            for (int i = 0; i < K * Dv; ++i) hT[(size_t)bh * K * Dv + i] = S[i];
        free(S);
        free(pa);
        free(e);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* O3: camera-branch prep, per token ([cam] _precompute_cam_inv_rms,        */
/* _cam_prep_kernel, cam_prep_func).                                        */
/*                                                                          */
/* For token (b, n), with C = H*D channels:                                 */
/*   inv_rms_x = 1 / sqrt(sum_c x_c^2 / C + eps)    for x in {q, k}         */
/* and for every head h, on the D values of that head:                      */
/*   q~ = relu(q * inv_rms_q * w_q)          (relu(x) = x if x > 0 else 0)  */
/*   k~ = relu(k * inv_rms_k * w_k) * k_scale                               */
/*   v~ = v                                  (no norm, relu or scale)       */
/*   k_pre_sq = ||k~||^2 over all D                                         */
/*   first D/2 values, in D/8 groups of 4:  y_g = P x_g  (4x4 times 4-vec), */
/*      P = proj_q for q and proj_kv for k and v (per token)                */
/*   second D/2 values (index r within that half):                          */
/*      y[r] = x[r] * cos[n][r] + x[r ^ 1] * sin[n][r]                      */
/*      (interleaved-pair RoPE tables, [cam] _prepare_ucpe_rope_tables)     */
/*   k_post_sq = ||k_out||^2 over all D                                     */
/*   inflation_sq = max(k_post_sq, 1e-12) / max(k_pre_sq, 1e-12)            */
/* Layouts: qkv (B,N,3,H,D) (slot 0 = q, 1 = k, 2 = v); w (H*D) or NULL for */
/* all-ones; proj (B,N,4,4) row-major; rope tables (N, D/2);                */
/* outputs q,k,v (B,H,N,D); k_pre_sq, k_post_sq, inflation_sq (B,H,N).      */
/* ------------------------------------------------------------------------ */
static void prep_head(int D, const float *x, double inv_rms, const float *w,
                      int relu, double post_scale, const float *P, const float *cs,
                      const float *sn, double *xin, double *out) {
    int half = D / 2;
    for (int d = 0; d < D; ++d) {
        double val = (double)x[d];
        if (relu) {
            val = val * inv_rms * (w ? (double)w[d] : 1.0);
            val = val > 0.0 ? val : 0.0;
            val *= post_scale;
        }
        xin[d] = val;
    }
    for (int grp = 0; grp < half / 4; ++grp)
        for (int i = 0; i < 4; ++i) {
            double acc = 0.0;
            for (int j = 0; j < 4; ++j) acc += (double)P[i * 4 + j] * xin[grp * 4 + j];
            out[grp * 4 + i] = acc;
        }
    for (int rr = 0; rr < half; ++rr)
        out[half + rr] = xin[half + rr] * (double)cs[rr] + xin[half + (rr ^ 1)] * (double)sn[rr];
}

int oracle_cam_prep(int B, int N, int H, int D, const float *qkv,
                    const float *q_norm_w, const float *k_norm_w,
                    const float *proj_q, const float *proj_kv,
                    const float *rope_cos, const float *rope_sin,
                    double k_scale, double eps,
                    double *q_out, double *k_out, double *v_out,
                    double *k_pre_sq, double *k_post_sq, double *inflation_sq,
                    int nthreads) {
    if (B < 0 || N < 0 || H <= 0 || D <= 0 || D > 512 || (D % 8) != 0) return -1;
    set_threads(nthreads);
    int C = H * D, half = D / 2;
    long ntok = (long)B * N;
#pragma omp parallel for schedule(static)
    for (long bn = 0; bn < ntok; ++bn) {
        int b = (int)(bn / N), n = (int)(bn % N);
        const float *tok = qkv + (size_t)bn * 3 * C;
        const float *xq = tok, *xk = tok + C, *xv = tok + 2 * C;
        double sq = 0.0, sk = 0.0;
        for (int c = 0; c < C; ++c) {
            sq += (double)xq[c] * (double)xq[c];
            sk += (double)xk[c] * (double)xk[c];
        }
        double inv_q = 1.0 / sqrt(sq / C + eps);
        double inv_k = 1.0 / sqrt(sk / C + eps);
        const float *Pq = proj_q + (size_t)bn * 16, *Pkv = proj_kv + (size_t)bn * 16;
        const float *cs = rope_cos + (size_t)n * half, *sn = rope_sin + (size_t)n * half;
        double xin[512], out[512];
        for (int h = 0; h < H; ++h) {
            size_t obase = (((size_t)b * H + h) * N + n) * D;
            size_t sbase = ((size_t)b * H + h) * N + n;
            prep_head(D, xq + h * D, inv_q, q_norm_w ? q_norm_w + h * D : NULL, 1, 1.0, Pq, cs, sn, xin, out);
            for (int d = 0; d < D; ++d) q_out[obase + d] = out[d];
            prep_head(D, xk + h * D, inv_k, k_norm_w ? k_norm_w + h * D : NULL, 1, k_scale, Pkv, cs, sn, xin, out);
            double pre = 0.0, post = 0.0;
            for (int d = 0; d < D; ++d) {
                pre += xin[d] * xin[d];
                post += out[d] * out[d];
                k_out[obase + d] = out[d];
            }
            k_pre_sq[sbase] = pre;
            k_post_sq[sbase] = post;
            if (inflation_sq)
                inflation_sq[sbase] = (post > 1e-12 ? post : 1e-12) / (pre > 1e-12 ? pre : 1e-12);
            prep_head(D, xv + h * D, 0.0, NULL, 0, 1.0, Pkv, cs, sn, xin, out);
            for (int d = 0; d < D; ++d) v_out[obase + d] = out[d];
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* O8: backward of O3 ([cam] _cam_prep_bwd_kernel and                      */
/* _cam_prep_bwd_dispatch): reverse mode through the prep steps of one      */
/* token, last step first.  Upstream gradients: gq, gk, gv of the outputs   */
/* q, k, v (B,H,N,D) and, each nullable, gpre, gpost, ginfl of k_pre_sq,    */
/* k_post_sq and inflation_sq (B,H,N).  Per head:                           */
/*   inflation = max(post, 1e-12) / max(pre, 1e-12) sends                   */
/*     ginfl / max(pre, 1e-12) to post (if post > 1e-12) and                */
/*     -ginfl max(post, 1e-12) / pre^2 to pre (if pre > 1e-12);             */
/*   post = ||k_out||^2 sends 2 k_out gpost to k_out; pre = ||k~||^2 sends  */
/*     2 k~ gpre to k~;                                                     */
/*   RoPE half: y[r] = x[r] c[r] + x[r^1] s[r] gives                        */
/*     gx[r] = gy[r] c[r] + gy[r^1] s[r^1];                                 */
/*   UCPE half: y_g = P x_g gives gx_g = P^T gy_g and dP += gy_g x_g^T       */
/*     (summed over groups and heads; proj_q from q, proj_kv from k and v); */
/*   k~ = relu(a) k_scale, q~ = relu(a), a = x inv_rms w: ga = gx k_scale   */
/*     (or gx) where a > 0, else 0;                                         */
/*   RMSNorm over the token's C channels: dw_c += ga_c x_c inv_rms (summed  */
/*     over tokens) and gx_c = inv_rms w_c ga_c                             */
/*       - inv_rms^3 / C x_c sum_c' ga_c' w_c' x_c';                        */
/*   v skips norm, relu and scale: gv_raw = gx.                             */
/* Outputs: dqkv (B,N,3,H,D); dq_w, dk_w (H*D); dproj_q, dproj_kv (B,N,4,4).*/
/* ------------------------------------------------------------------------ */
static void prep_head_bwd(int D, const double *gy, const double *xin, const float *P, const float *cs,
                          const float *sn, double *gx, double *dP) {
    int half = D / 2;
    for (int grp = 0; grp < half / 4; ++grp)
        for (int j = 0; j < 4; ++j) {
            double acc = 0.0;
            for (int i = 0; i < 4; ++i) {
                acc += (double)P[i * 4 + j] * gy[grp * 4 + i];
                dP[i * 4 + j] += gy[grp * 4 + i] * xin[grp * 4 + j];
            }
            gx[grp * 4 + j] = acc;
        }
    for (int rr = 0; rr < half; ++rr)
        gx[half + rr] = gy[half + rr] * (double)cs[rr] + gy[half + (rr ^ 1)] * (double)sn[rr ^ 1];
}

int oracle_cam_prep_bwd(int B, int N, int H, int D, const float *qkv,
                        const float *q_norm_w, const float *k_norm_w,
                        const float *proj_q, const float *proj_kv,
                        const float *rope_cos, const float *rope_sin,
                        double k_scale, double eps,
                        const float *gq, const float *gk, const float *gv,
                        const float *gpre, const float *gpost, const float *ginfl,
                        double *dqkv, double *dq_w, double *dk_w,
                        double *dproj_q, double *dproj_kv, int nthreads) {
    if (B < 0 || N < 0 || H <= 0 || D <= 0 || D > 512 || (D % 8) != 0) return -1;
    set_threads(nthreads);
    int C = H * D, half = D / 2;
    long ntok = (long)B * N;
    int nt = oracle_max_threads();
    double *wpart = (double *)calloc((size_t)nt * 2 * C, sizeof(double));   /* per-thread dq_w, dk_w */
#pragma omp parallel
    {
        double *myw = wpart + (size_t)thread_num() * 2 * C;
        double *gaq = (double *)malloc(sizeof(double) * C), *gak = (double *)malloc(sizeof(double) * C);
#pragma omp for schedule(static)
        for (long bn = 0; bn < ntok; ++bn) {
            int b = (int)(bn / N), n = (int)(bn % N);
            const float *tok = qkv + (size_t)bn * 3 * C;
            const float *xq = tok, *xk = tok + C, *xv = tok + 2 * C;
            double sq = 0.0, sk = 0.0;
            for (int c = 0; c < C; ++c) {
                sq += (double)xq[c] * (double)xq[c];
                sk += (double)xk[c] * (double)xk[c];
            }
            double inv_q = 1.0 / sqrt(sq / C + eps);
            double inv_k = 1.0 / sqrt(sk / C + eps);
            const float *Pq = proj_q + (size_t)bn * 16, *Pkv = proj_kv + (size_t)bn * 16;
            const float *cs = rope_cos + (size_t)n * half, *sn = rope_sin + (size_t)n * half;
            double *dPq = dproj_q + (size_t)bn * 16, *dPkv = dproj_kv + (size_t)bn * 16;
            for (int i = 0; i < 16; ++i) dPq[i] = dPkv[i] = 0.0;
            double *out_q = dqkv + (size_t)bn * 3 * C, *out_k = out_q + C, *out_v = out_k + C;
            double xin[512], yo[512], gy[512], gx[512];
            for (int h = 0; h < H; ++h) {
                size_t obase = (((size_t)b * H + h) * N + n) * D;
                size_t sbase = ((size_t)b * H + h) * N + n;
                const float *wq = q_norm_w ? q_norm_w + h * D : NULL, *wk = k_norm_w ? k_norm_w + h * D : NULL;
                /* q */
                prep_head(D, xq + h * D, inv_q, wq, 1, 1.0, Pq, cs, sn, xin, yo);
                for (int d = 0; d < D; ++d) gy[d] = (double)gq[obase + d];
                prep_head_bwd(D, gy, xin, Pq, cs, sn, gx, dPq);
                for (int d = 0; d < D; ++d) {
                    double a = (double)xq[h * D + d] * inv_q * (wq ? (double)wq[d] : 1.0);
                    gaq[h * D + d] = a > 0.0 ? gx[d] : 0.0;
                }
                /* k, with the norm outputs */
                prep_head(D, xk + h * D, inv_k, wk, 1, k_scale, Pkv, cs, sn, xin, yo);
                double pre = 0.0, post = 0.0;
                for (int d = 0; d < D; ++d) {
                    pre += xin[d] * xin[d];
                    post += yo[d] * yo[d];
                }
                double gpo = gpost ? (double)gpost[sbase] : 0.0, gpr = gpre ? (double)gpre[sbase] : 0.0;
                if (ginfl) {
                    double gi = (double)ginfl[sbase];
                    if (post > 1e-12) gpo += gi / (pre > 1e-12 ? pre : 1e-12);
                    if (pre > 1e-12) gpr -= gi * (post > 1e-12 ? post : 1e-12) / (pre * pre);
                }
                for (int d = 0; d < D; ++d) gy[d] = (double)gk[obase + d] + 2.0 * yo[d] * gpo;
                prep_head_bwd(D, gy, xin, Pkv, cs, sn, gx, dPkv);
                for (int d = 0; d < D; ++d) {
                    gx[d] += 2.0 * xin[d] * gpr;
                    double a = (double)xk[h * D + d] * inv_k * (wk ? (double)wk[d] : 1.0);
                    gak[h * D + d] = a > 0.0 ? gx[d] * k_scale : 0.0;
                }
                /* v */
                prep_head(D, xv + h * D, 0.0, NULL, 0, 1.0, Pkv, cs, sn, xin, yo);
                for (int d = 0; d < D; ++d) gy[d] = (double)gv[obase + d];
                prep_head_bwd(D, gy, xin, Pkv, cs, sn, gx, dPkv);
                for (int d = 0; d < D; ++d) out_v[h * D + d] = gx[d];
            }
            /* RMSNorm backward over all C channels, and the weight gradients */
            double s_q = 0.0, s_k = 0.0;
            for (int c = 0; c < C; ++c) {
                s_q += gaq[c] * (q_norm_w ? (double)q_norm_w[c] : 1.0) * (double)xq[c];
                s_k += gak[c] * (k_norm_w ? (double)k_norm_w[c] : 1.0) * (double)xk[c];
            }
            for (int c = 0; c < C; ++c) {
                double w_q = q_norm_w ? (double)q_norm_w[c] : 1.0, w_k = k_norm_w ? (double)k_norm_w[c] : 1.0;
                out_q[c] = inv_q * w_q * gaq[c] - inv_q * inv_q * inv_q / C * (double)xq[c] * s_q;
                out_k[c] = inv_k * w_k * gak[c] - inv_k * inv_k * inv_k / C * (double)xk[c] * s_k;
                myw[c] += gaq[c] * (double)xq[c] * inv_q;
                myw[C + c] += gak[c] * (double)xk[c] * inv_k;
            }
        }
        free(gaq);
        free(gak);
    }
    for (int c = 0; c < C; ++c) {
        double a = 0.0, b2 = 0.0;
        for (int t = 0; t < nt; ++t) {
            a += wpart[(size_t)t * 2 * C + c];
            b2 += wpart[(size_t)t * 2 * C + C + c];
        }
        dq_w[c] = a;
        dk_w[c] = b2;
    }
    free(wpart);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* O4: camera-branch numerator-only scan, frame-synchronous ([cam]          */
/* _cam_scan_kernel, forward direction).                                    */
/*                                                                          */
/* Tokens come in F frames of S tokens.  For one (b, h), S = h0 (or 0), for */
/* frame f = 0 .. F-1:                                                      */
/*   P <- exp(g_f) S                       (one gate per frame)             */
/*   S <- P + sum_{s in f} beta_s k_s (v_s - P^T k_s)^T                     */
/*        (every token of the frame predicts from the same gated state P)   */
/*   o_s <- scale * S^T q_s   for s in f   (read-out after the frame update)*/
/* and hT = S after the last frame.  A loaded h0 is the state at the end of */
/* a prefix; the first frame's gate applies to it ([cam] _cam_scan_kernel   */
/* docstring on resuming from a saved state).                               */
/* Layouts: q,k,v (B,H,F*S,D); beta (B,H,F*S); g (B,H,F); h0,hT (B,H,D,D);  */
/* out (B,H,F*S,D).                                                         */
/* ------------------------------------------------------------------------ */
int oracle_frame_scan(int B, int H, int F, int S, int D,
                      const float *q, const float *k, const float *v,
                      const float *beta, const float *g, double scale,
                      const float *h0, double *out, double *hT, int nthreads) {
    if (B < 0 || H < 0 || F < 0 || S <= 0 || D <= 0) return -1;
    set_threads(nthreads);
    int npairs = B * H;
    size_t N = (size_t)F * S;
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < npairs; ++bh) {
        double *St = (double *)calloc((size_t)D * D, sizeof(double));
        double *P = (double *)malloc(sizeof(double) * (size_t)D * D);
        double *p = (double *)malloc(sizeof(double) * (size_t)D);
        if (h0)
            for (int i = 0; i < D * D; ++i) St[i] = (double)h0[(size_t)bh * D * D + i];
        for (int f = 0; f < F; ++f) {
            double decay = exp((double)g[(size_t)bh * F + f]);
            for (int i = 0; i < D * D; ++i) {
                P[i] = decay * St[i];
                St[i] = P[i];
            }
            for (int s = 0; s < S; ++s) {
                size_t n = (size_t)f * S + s;
                const float *ks = k + ((size_t)bh * N + n) * D, *vs = v + ((size_t)bh * N + n) * D;
                double bs = (double)beta[(size_t)bh * N + n];
                for (int j = 0; j < D; ++j) {
                    double acc = 0.0;
                    for (int i = 0; i < D; ++i) acc += P[(size_t)i * D + j] * (double)ks[i];
                    p[j] = acc;
                }
                for (int i = 0; i < D; ++i) {
                    double ki = bs * (double)ks[i];
                    for (int j = 0; j < D; ++j) St[(size_t)i * D + j] += ki * ((double)vs[j] - p[j]);
                }
            }
            for (int s = 0; s < S; ++s) {
                size_t n = (size_t)f * S + s;
                const float *qs = q + ((size_t)bh * N + n) * D;
                for (int j = 0; j < D; ++j) {
                    double acc = 0.0;
                    for (int i = 0; i < D; ++i) acc += St[(size_t)i * D + j] * (double)qs[i];
                    out[((size_t)bh * N + n) * D + j] = scale * acc;
                }
            }
        }
        if (hT)
            for (int i = 0; i < D * D; ++i) hT[(size_t)bh * D * D + i] = St[i];
        free(St);
        free(P);
        free(p);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Closed-form inverse of a rigid transform ([cam] _invert_SE3):            */
/*   [R t; 0 1]^-1 = [R^T  -R^T t; 0 1].                                    */
/* in, out: n row-major 4x4 matrices.                                       */
/* ------------------------------------------------------------------------ */
void oracle_invert_se3(long n, const double *in, double *out) {
    for (long m = 0; m < n; ++m) {
        const double *A = in + m * 16;
        double *Y = out + m * 16;
        for (int i = 0; i < 16; ++i) Y[i] = 0.0;
        for (int i = 0; i < 3; ++i)
            for (int j = 0; j < 3; ++j) Y[i * 4 + j] = A[j * 4 + i];
        for (int i = 0; i < 3; ++i) {
            double acc = 0.0;
            for (int j = 0; j < 3; ++j) acc += Y[i * 4 + j] * A[j * 4 + 3];
            Y[i * 4 + 3] = -acc;
        }
        Y[15] = 1.0;
    }
}

/* ------------------------------------------------------------------------ */
/* O6: gradients of O1 (reverse mode through its steps).                   */
/*                                                                          */
/* Given dL/do_t (dout) and dL/dS_T (dhT, or 0), the steps of O1 are        */
/* walked from the last token back, each one's adjoint taken in turn:       */
/*   read-out  o = scale S^T q     : dS += scale q do^T, dq = scale S do    */
/*   correct   S = P + beta k r^T, r = v - p                                */
/*                                 : dP = dS, dk = beta dS r,               */
/*                                   dbeta = k^T dS r, dv = beta dS^T k,    */
/*                                   dp = -dv                               */
/*   predict   p = P^T k           : dP += k dp^T, dk += P dp               */
/*   gate      P = exp(g) S_prev   : dS_prev = exp(g) dP, dg = <dP, P>      */
/* and dh0 = dS_0.  S_prev of every token is recomputed forward from a     */
/* state kept every 64 tokens (same steps as O1).  [dp] lists the chunk    */
/* backward kernels of this rule; this is the gradient they compute,       */
/* taken on the token recurrence.                                           */
/* Layouts as O1; dout (B,T,H,Dv); dhT, dh0 (B,H,Dk,Dv); dq, dk (B,T,H,Dk); */
/* dv (B,T,H,Dv); dbeta, dg (B,T,H).  dhT and h0 may be NULL; dh0 may be   */
/* NULL (not stored).                                                       */
/* ------------------------------------------------------------------------ */
static void o1_step(int Dk, int Dv, double *S, double *p, const float *kt, const float *vt,
                    double decay, double bt) {
    for (int i = 0; i < Dk * Dv; ++i) S[i] *= decay;
    for (int j = 0; j < Dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < Dk; ++i) acc += S[(size_t)i * Dv + j] * (double)kt[i];
        p[j] = acc;
    }
    for (int i = 0; i < Dk; ++i) {
        double ki = bt * (double)kt[i];
        for (int j = 0; j < Dv; ++j) S[(size_t)i * Dv + j] += ki * ((double)vt[j] - p[j]);
    }
}

int oracle_gdn_recurrent_bwd(int B, int T, int H, int Dk, int Dv,
                             const float *q, const float *k, const float *v,
                             const float *beta, const float *g, double scale,
                             const float *h0, const float *dout, const float *dhT,
                             double *dq, double *dk, double *dv, double *dbeta,
                             double *dg, double *dh0, int nthreads) {
    if (B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0) return -1;
    set_threads(nthreads);
    const int SEG = 64;
    int nseg = (T + SEG - 1) / SEG;
    int npairs = B * H;
    size_t sz = (size_t)Dk * Dv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < npairs; ++bh) {
        int b = bh / H, h = bh % H;
        double *ck = (double *)malloc(sizeof(double) * sz * (size_t)(nseg > 0 ? nseg : 1));
        double *st = (double *)malloc(sizeof(double) * sz * (SEG + 1));
        double *S = (double *)calloc(sz, sizeof(double));
        double *dS = (double *)calloc(sz, sizeof(double));
        double *p = (double *)malloc(sizeof(double) * (size_t)Dv);
        double *r = (double *)malloc(sizeof(double) * (size_t)Dv);
        double *u = (double *)malloc(sizeof(double) * (size_t)Dv);
        double *dp = (double *)malloc(sizeof(double) * (size_t)Dv);
        if (h0)
            for (size_t i = 0; i < sz; ++i) S[i] = (double)h0[(size_t)bh * sz + i];
        /* forward: the state entering every segment */
        for (int t = 0; t < T; ++t) {
            size_t row = ((size_t)b * T + t) * H + h;
            if (t % SEG == 0) memcpy(ck + (size_t)(t / SEG) * sz, S, sizeof(double) * sz);
            o1_step(Dk, Dv, S, p, k + row * Dk, v + row * Dv, exp((double)g[row]), (double)beta[row]);
        }
        if (dhT)
            for (size_t i = 0; i < sz; ++i) dS[i] = (double)dhT[(size_t)bh * sz + i];
        for (int s = nseg - 1; s >= 0; --s) {
            int t0 = s * SEG, t1 = t0 + SEG < T ? t0 + SEG : T;
            /* st[i] = state before token t0 + i, st[t1 - t0] = after the last */
            memcpy(st, ck + (size_t)s * sz, sizeof(double) * sz);
            for (int t = t0; t < t1; ++t) {
                size_t row = ((size_t)b * T + t) * H + h;
                double *nx = st + (size_t)(t - t0 + 1) * sz;
                memcpy(nx, st + (size_t)(t - t0) * sz, sizeof(double) * sz);
                o1_step(Dk, Dv, nx, p, k + row * Dk, v + row * Dv, exp((double)g[row]), (double)beta[row]);
            }
            for (int t = t1 - 1; t >= t0; --t) {
                size_t row = ((size_t)b * T + t) * H + h;
                const float *qt = q + row * Dk, *kt = k + row * Dk, *vt = v + row * Dv;
                const float *dot = dout + row * Dv;
                const double *Sp = st + (size_t)(t - t0) * sz;       /* S_{t-1} */
                const double *Sc = st + (size_t)(t - t0 + 1) * sz;   /* S_t */
                double a = exp((double)g[row]), bt = (double)beta[row];
                /* read-out */
                for (int i = 0; i < Dk; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < Dv; ++j) {
                        dS[(size_t)i * Dv + j] += scale * (double)qt[i] * (double)dot[j];
                        acc += Sc[(size_t)i * Dv + j] * (double)dot[j];
                    }
                    dq[row * Dk + i] = scale * acc;
                }
                /* correct: p = (a S_prev)^T k, r = v - p, u = dS^T k */
                double db = 0.0;
                for (int j = 0; j < Dv; ++j) {
                    double pa = 0.0, ua = 0.0;
                    for (int i = 0; i < Dk; ++i) {
                        pa += a * Sp[(size_t)i * Dv + j] * (double)kt[i];
                        ua += dS[(size_t)i * Dv + j] * (double)kt[i];
                    }
                    p[j] = pa;
                    r[j] = (double)vt[j] - pa;
                    u[j] = ua;
                    dv[row * Dv + j] = bt * ua;
                    dp[j] = -bt * ua;
                    db += ua * r[j];
                }
                dbeta[row] = db;
                /* dk from the correction and the prediction; dP and dg */
                double dgs = 0.0;
                for (int i = 0; i < Dk; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < Dv; ++j) {
                        double P = a * Sp[(size_t)i * Dv + j];
                        double dP = dS[(size_t)i * Dv + j] + (double)kt[i] * dp[j];
                        acc += bt * dS[(size_t)i * Dv + j] * r[j] + P * dp[j];
                        dgs += dP * P;
                        dS[(size_t)i * Dv + j] = a * dP;   /* gate: dS_prev */
                    }
                    dk[row * Dk + i] = acc;
                }
                dg[row] = dgs;
            }
        }
        if (dh0)
            for (size_t i = 0; i < sz; ++i) dh0[(size_t)bh * sz + i] = dS[i];
        free(ck); free(st); free(S); free(dS); free(p); free(r); free(u); free(dp);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* O7: gradients of O4 (reverse mode through its frame steps).             */
/*                                                                          */
/* With the steps of frame f of O4, P = exp(g_f) S_{f-1},                   */
/* S_f = P + sum_s beta_s k_s (v_s - P^T k_s)^T, o_s = scale S_f^T q_s, and  */
/* dS = dL/dS_f (dhT, or 0, after the last frame), the frames are walked    */
/* from the last back, each step's adjoint taken in turn:                   */
/*   read-out  for s in f: dS += scale q_s do_s^T, dq_s = scale S_f do_s    */
/*   correct   for s in f: r_s = v_s - P^T k_s, u_s = dS^T k_s,             */
/*             dv_s = beta_s u_s, dbeta_s = u_s . r_s, dp_s = -beta_s u_s,  */
/*             dk_s = beta_s dS r_s;  dP = dS                               */
/*   predict   for s in f: dP += k_s dp_s^T, dk_s += P dp_s                 */
/*   gate      dS_{f-1} = exp(g_f) dP, dg_f = <dP, P>                       */
/* and dh0 = dS after frame 0.  Every state S_0 .. S_F is kept.  [cam]      */
/* names the backward of this scan (_cam_scan_bwd_kernel); this is the      */
/* gradient it computes.                                                    */
/* Layouts as O4; dout (B,H,F*S,D); dhT, dh0 (B,H,D,D); dq, dk, dv          */
/* (B,H,F*S,D); dbeta (B,H,F*S); dg (B,H,F).  h0, dhT, dh0 may be NULL.     */
/* ------------------------------------------------------------------------ */
int oracle_frame_scan_bwd(int B, int H, int F, int S, int D,
                          const float *q, const float *k, const float *v,
                          const float *beta, const float *g, double scale,
                          const float *h0, const float *dout, const float *dhT,
                          double *dq, double *dk, double *dv, double *dbeta,
                          double *dg, double *dh0, int nthreads) {
    if (B < 0 || H < 0 || F < 0 || S <= 0 || D <= 0) return -1;
    set_threads(nthreads);
    int npairs = B * H;
    size_t N = (size_t)F * S, sz = (size_t)D * D;
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < npairs; ++bh) {
        double *st = (double *)calloc(sz * (size_t)(F + 1), sizeof(double));   /* S_0 .. S_F */
        double *dS = (double *)calloc(sz, sizeof(double));
        double *P = (double *)malloc(sizeof(double) * sz);
        double *dP = (double *)malloc(sizeof(double) * sz);
        double *r = (double *)malloc(sizeof(double) * (size_t)D);
        double *u = (double *)malloc(sizeof(double) * (size_t)D);
        if (h0)
            for (size_t i = 0; i < sz; ++i) st[i] = (double)h0[(size_t)bh * sz + i];
        /* forward: every frame's state */
        for (int f = 0; f < F; ++f) {
            const double *Sp = st + (size_t)f * sz;
            double *Sn = st + (size_t)(f + 1) * sz;
            double decay = exp((double)g[(size_t)bh * F + f]);
            for (size_t i = 0; i < sz; ++i) Sn[i] = P[i] = decay * Sp[i];
            for (int s = 0; s < S; ++s) {
                size_t n = (size_t)bh * N + (size_t)f * S + s;
                const float *ks = k + n * D, *vs = v + n * D;
                double bs = (double)beta[n];
                for (int j = 0; j < D; ++j) {
                    double acc = 0.0;
                    for (int i = 0; i < D; ++i) acc += P[(size_t)i * D + j] * (double)ks[i];
                    r[j] = (double)vs[j] - acc;
                }
                for (int i = 0; i < D; ++i)
                    for (int j = 0; j < D; ++j) Sn[(size_t)i * D + j] += bs * (double)ks[i] * r[j];
            }
        }
        if (dhT)
            for (size_t i = 0; i < sz; ++i) dS[i] = (double)dhT[(size_t)bh * sz + i];
        for (int f = F - 1; f >= 0; --f) {
            const double *Sp = st + (size_t)f * sz, *Sc = st + (size_t)(f + 1) * sz;
            double decay = exp((double)g[(size_t)bh * F + f]);
            for (size_t i = 0; i < sz; ++i) P[i] = decay * Sp[i];
            /* read-out */
            for (int s = 0; s < S; ++s) {
                size_t n = (size_t)bh * N + (size_t)f * S + s;
                const float *qs = q + n * D, *dos = dout + n * D;
                for (int i = 0; i < D; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < D; ++j) {
                        dS[(size_t)i * D + j] += scale * (double)qs[i] * (double)dos[j];
                        acc += Sc[(size_t)i * D + j] * (double)dos[j];
                    }
                    dq[n * D + i] = scale * acc;
                }
            }
            /* correct and predict, token by token (all read dS = dL/dS_f) */
            for (size_t i = 0; i < sz; ++i) dP[i] = dS[i];
            for (int s = 0; s < S; ++s) {
                size_t n = (size_t)bh * N + (size_t)f * S + s;
                const float *ks = k + n * D, *vs = v + n * D;
                double bs = (double)beta[n], db = 0.0;
                for (int j = 0; j < D; ++j) {
                    double pa = 0.0, ua = 0.0;
                    for (int i = 0; i < D; ++i) {
                        pa += P[(size_t)i * D + j] * (double)ks[i];
                        ua += dS[(size_t)i * D + j] * (double)ks[i];
                    }
                    r[j] = (double)vs[j] - pa;
                    u[j] = ua;
                    dv[n * D + j] = bs * ua;
                    db += ua * r[j];
                }
                dbeta[n] = db;
                for (int i = 0; i < D; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < D; ++j) {
                        double dp = -bs * u[j];
                        acc += bs * dS[(size_t)i * D + j] * r[j] + P[(size_t)i * D + j] * dp;
                        dP[(size_t)i * D + j] += (double)ks[i] * dp;
                    }
                    dk[n * D + i] = acc;
                }
            }
            /* gate */
            double dgs = 0.0;
            for (size_t i = 0; i < sz; ++i) {
                dgs += dP[i] * P[i];
                dS[i] = decay * dP[i];
            }
            dg[(size_t)bh * F + f] = dgs;
        }
        if (dh0)
            for (size_t i = 0; i < sz; ++i) dh0[(size_t)bh * sz + i] = dS[i];
        free(st); free(dS); free(P); free(dP); free(r); free(u);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* O9: backward of O2 (gated DeltaProduct), reverse mode through the token  */
/* steps of O2, last token first.  With w_a = E_a k_{t,a} (write key),      */
/* e_a = sum_b M[a][b] E_b k_{t,b} (erase key), P = exp(g_t) S_{t-1},       */
/* p_a = P^T e_a, r_a = v_t - p_a, S_t = P + sum_a beta_a w_a r_a^T and     */
/* o_t = scale S_t^T q_t, each token's adjoint, given dS = dL/dS_t:          */
/*   read-out : dS += scale q do^T,  dq = scale S_t do                      */
/*   correct  : u_a = dS^T w_a,  dbeta_a = u_a . r_a,  dv += beta_a u_a,    */
/*              dp_a = -beta_a u_a,  dw_a = beta_a dS r_a,  dP = dS         */
/*   predict  : dP += sum_a e_a dp_a^T,  de_a = P dp_a                      */
/*   keys     : dk_{t,a} = E_a^T dw_a + sum_c M[c][a] E_a^T de_c            */
/*   gate     : dg = <dP, P>,  dS_{t-1} = exp(g_t) dP                        */
/* and dh0 = dS_0.  States are recomputed from one kept every 64 tokens.    */
/* Layouts as O2; dout (B,T,H,Dv); dhT, dh0 (B,H,r*dk,Dv); dq, dk           */
/* (B,T,H,r*dk); dv (B,T,H,Dv); dbeta (B,T,H,r); dg (B,T,H).                */
/* ------------------------------------------------------------------------ */
static void o2_step(int r, int dk, int Dv, double *S, double *pa, double *e, const float *kt, const float *vt,
                    const float *bt, const double *mask, double decay) {
    int K = r * dk;
    for (int i = 0; i < K * Dv; ++i) S[i] *= decay;
    for (int a = 0; a < r; ++a) {
        for (int bb = 0; bb < r; ++bb)
            for (int c = 0; c < dk; ++c) e[bb * dk + c] = mask[a * r + bb] * (double)kt[bb * dk + c];
        for (int j = 0; j < Dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < K; ++i) acc += S[(size_t)i * Dv + j] * e[i];
            pa[(size_t)a * Dv + j] = acc;
        }
    }
    for (int a = 0; a < r; ++a)
        for (int c = 0; c < dk; ++c) {
            int i = a * dk + c;
            double ki = (double)bt[a] * (double)kt[i];
            for (int j = 0; j < Dv; ++j) S[(size_t)i * Dv + j] += ki * ((double)vt[j] - pa[(size_t)a * Dv + j]);
        }
}

int oracle_deltaproduct_bwd(int B, int T, int H, int r, int dk, int Dv,
                            const float *q, const float *k, const float *v,
                            const float *beta, const float *g, const double *mask, double scale,
                            const float *h0, const float *dout, const float *dhT,
                            double *dq, double *dkk, double *dv, double *dbeta,
                            double *dg, double *dh0, int nthreads) {
    if (B < 0 || T < 0 || H < 0 || r <= 0 || r > 8 || dk <= 0 || Dv <= 0) return -1;
    set_threads(nthreads);
    const int SEG = 64;
    int K = r * dk;
    int nseg = (T + SEG - 1) / SEG;
    int npairs = B * H;
    size_t sz = (size_t)K * Dv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < npairs; ++bh) {
        int b = bh / H, h = bh % H;
        double *ck = (double *)malloc(sizeof(double) * sz * (size_t)(nseg > 0 ? nseg : 1));
        double *st = (double *)malloc(sizeof(double) * sz * (SEG + 1));
        double *S = (double *)calloc(sz, sizeof(double));
        double *dS = (double *)calloc(sz, sizeof(double));
        double *dP = (double *)malloc(sizeof(double) * sz);
        double *pa = (double *)malloc(sizeof(double) * (size_t)r * Dv);
        double *ra = (double *)malloc(sizeof(double) * (size_t)r * Dv);
        double *ua = (double *)malloc(sizeof(double) * (size_t)r * Dv);
        double *e = (double *)malloc(sizeof(double) * (size_t)r * K);   /* erase key of each step */
        double *de = (double *)malloc(sizeof(double) * (size_t)K);
        if (h0)
            for (size_t i = 0; i < sz; ++i) S[i] = (double)h0[(size_t)bh * sz + i];
        for (int t = 0; t < T; ++t) {
            size_t row = ((size_t)b * T + t) * H + h;
            if (t % SEG == 0) memcpy(ck + (size_t)(t / SEG) * sz, S, sizeof(double) * sz);
            o2_step(r, dk, Dv, S, pa, e, k + row * K, v + row * Dv, beta + row * r, mask, exp((double)g[row]));
        }
        if (dhT)
            for (size_t i = 0; i < sz; ++i) dS[i] = (double)dhT[(size_t)bh * sz + i];
        for (int s = nseg - 1; s >= 0; --s) {
            int t0 = s * SEG, t1 = t0 + SEG < T ? t0 + SEG : T;
            memcpy(st, ck + (size_t)s * sz, sizeof(double) * sz);
            for (int t = t0; t < t1; ++t) {
                size_t row = ((size_t)b * T + t) * H + h;
                double *nx = st + (size_t)(t - t0 + 1) * sz;
                memcpy(nx, st + (size_t)(t - t0) * sz, sizeof(double) * sz);
                o2_step(r, dk, Dv, nx, pa, e, k + row * K, v + row * Dv, beta + row * r, mask, exp((double)g[row]));
            }
            for (int t = t1 - 1; t >= t0; --t) {
                size_t row = ((size_t)b * T + t) * H + h;
                const float *qt = q + row * K, *kt = k + row * K, *vt = v + row * Dv, *bt = beta + row * r;
                const float *dot = dout + row * Dv;
                const double *Sp = st + (size_t)(t - t0) * sz;       /* S_{t-1} */
                const double *Sc = st + (size_t)(t - t0 + 1) * sz;   /* S_t */
                double a = exp((double)g[row]);
                /* read-out */
                for (int i = 0; i < K; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < Dv; ++j) {
                        dS[(size_t)i * Dv + j] += scale * (double)qt[i] * (double)dot[j];
                        acc += Sc[(size_t)i * Dv + j] * (double)dot[j];
                    }
                    dq[row * K + i] = scale * acc;
                }
                /* erase keys, predictions p_a = (a S_prev)^T e_a, residuals, u_a = dS^T w_a */
                for (int st_ = 0; st_ < r; ++st_)
                    for (int bb = 0; bb < r; ++bb)
                        for (int c = 0; c < dk; ++c)
                            e[(size_t)st_ * K + bb * dk + c] = mask[st_ * r + bb] * (double)kt[bb * dk + c];
                for (int j = 0; j < Dv; ++j) dv[row * Dv + j] = 0.0;
                for (int st_ = 0; st_ < r; ++st_) {
                    double db = 0.0, bs = (double)bt[st_];
                    for (int j = 0; j < Dv; ++j) {
                        double p = 0.0, u = 0.0;
                        for (int i = 0; i < K; ++i) p += a * Sp[(size_t)i * Dv + j] * e[(size_t)st_ * K + i];
                        for (int c = 0; c < dk; ++c)
                            u += dS[(size_t)(st_ * dk + c) * Dv + j] * (double)kt[st_ * dk + c];
                        pa[(size_t)st_ * Dv + j] = p;
                        ra[(size_t)st_ * Dv + j] = (double)vt[j] - p;
                        ua[(size_t)st_ * Dv + j] = u;
                        dv[row * Dv + j] += bs * u;
                        db += u * ((double)vt[j] - p);
                    }
                    dbeta[row * r + st_] = db;
                }
                /* dP = dS + sum_a e_a dp_a^T (dp_a = -beta_a u_a); dg; write-key and erase-key gradients */
                double dgs = 0.0;
                for (size_t i = 0; i < sz; ++i) dP[i] = dS[i];
                for (int st_ = 0; st_ < r; ++st_) {
                    double bs = (double)bt[st_];
                    for (int i = 0; i < K; ++i) {
                        double ei = e[(size_t)st_ * K + i];
                        if (ei == 0.0) continue;
                        for (int j = 0; j < Dv; ++j) dP[(size_t)i * Dv + j] += ei * (-bs * ua[(size_t)st_ * Dv + j]);
                    }
                }
                for (int i = 0; i < K; ++i) dkk[row * K + i] = 0.0;
                for (int st_ = 0; st_ < r; ++st_) {
                    double bs = (double)bt[st_];
                    /* dw_a = beta_a dS r_a on row block a */
                    for (int c = 0; c < dk; ++c) {
                        int i = st_ * dk + c;
                        double acc = 0.0;
                        for (int j = 0; j < Dv; ++j) acc += dS[(size_t)i * Dv + j] * ra[(size_t)st_ * Dv + j];
                        dkk[row * K + i] += bs * acc;
                    }
                    /* de_a = P dp_a, sent to the sub-keys through the mask */
                    for (int i = 0; i < K; ++i) {
                        double acc = 0.0;
                        for (int j = 0; j < Dv; ++j) acc += a * Sp[(size_t)i * Dv + j] * (-bs * ua[(size_t)st_ * Dv + j]);
                        de[i] = acc;
                    }
                    for (int bb = 0; bb < r; ++bb)
                        for (int c = 0; c < dk; ++c) dkk[row * K + bb * dk + c] += mask[st_ * r + bb] * de[bb * dk + c];
                }
                for (size_t i = 0; i < sz; ++i) {
                    dgs += dP[i] * a * Sp[i];
                    dS[i] = a * dP[i];
                }
                dg[row] = dgs;
            }
        }
        if (dh0)
            for (size_t i = 0; i < sz; ++i) dh0[(size_t)bh * sz + i] = dS[i];
        free(ck); free(st); free(S); free(dS); free(dP); free(pa); free(ra); free(ua); free(e); free(de);
    }
    return 0;
}

