/*
 * Driver for the sanitizer build of the oracle (AddressSanitizer and
 * UndefinedBehaviorSanitizer, host code): every exported oracle routine once
 * on small inputs, each buffer allocated at exactly the size its layout
 * needs, so that any read or write past a tensor, any use of uninitialised
 * heap memory through an index error, or any signed overflow in the index
 * arithmetic stops the run with a report.  Shapes include a ragged last
 * segment (T not a multiple of the oracle's 64-token backward segment) and
 * a non-power-of-two width.
 *
 * TEST INFRASTRUCTURE ONLY, like the oracle it drives; built and run by the
 * test suite (a CPU test), never by the product path.
 *
 * Exit status 0 when every call returns 0 and every output is finite.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_gdn_recurrent(int B, int T, int H, int Dk, int Dv, const float *q, const float *k, const float *v,
                         const float *beta, const float *g, double scale, const float *h0, double *o, double *hT,
                         int nthreads);
int oracle_deltaproduct_recurrent(int B, int T, int H, int r, int dk, int Dv, const float *q, const float *k,
                                  const float *v, const float *beta, const float *g, const double *mask,
                                  double scale, const float *h0, double *o, double *hT, int nthreads);
int oracle_cam_prep(int B, int N, int H, int D, const float *qkv, const float *q_norm_w, const float *k_norm_w,
                    const float *proj_q, const float *proj_kv, const float *rope_cos, const float *rope_sin,
                    double k_scale, double eps, double *q_out, double *k_out, double *v_out, double *k_pre_sq,
                    double *k_post_sq, double *inflation_sq, int nthreads);
int oracle_cam_prep_bwd(int B, int N, int H, int D, const float *qkv, const float *q_norm_w, const float *k_norm_w,
                        const float *proj_q, const float *proj_kv, const float *rope_cos, const float *rope_sin,
                        double k_scale, double eps, const float *gq, const float *gk, const float *gv,
                        const float *gpre, const float *gpost, const float *ginfl, double *dqkv, double *dq_w,
                        double *dk_w, double *dproj_q, double *dproj_kv, int nthreads);
int oracle_frame_scan(int B, int H, int F, int S, int D, const float *q, const float *k, const float *v,
                      const float *beta, const float *g, double scale, const float *h0, double *out, double *hT,
                      int nthreads);
int oracle_gdn_recurrent_bwd(int B, int T, int H, int Dk, int Dv, const float *q, const float *k, const float *v,
                             const float *beta, const float *g, double scale, const float *h0, const float *dout,
                             const float *dhT, double *dq, double *dk, double *dv, double *dbeta, double *dg,
                             double *dh0, int nthreads);
int oracle_frame_scan_bwd(int B, int H, int F, int S, int D, const float *q, const float *k, const float *v,
                          const float *beta, const float *g, double scale, const float *h0, const float *dout,
                          const float *dhT, double *dq, double *dk, double *dv, double *dbeta, double *dg,
                          double *dh0, int nthreads);
int oracle_deltaproduct_bwd(int B, int T, int H, int r, int dk, int Dv, const float *q, const float *k,
                            const float *v, const float *beta, const float *g, const double *mask, double scale,
                            const float *h0, const float *dout, const float *dhT, double *dq, double *dkk,
                            double *dv, double *dbeta, double *dg, double *dh0, int nthreads);
void oracle_invert_se3(long n, const double *in, double *out);

static unsigned long long rng = 0x9e3779b97f4a7c15ull;

/* uniform in [lo, hi) from a 64-bit linear congruential generator */
static float uni(float lo, float hi) {
    rng = rng * 6364136223846793005ull + 1442695040888963407ull;
    return lo + (hi - lo) * (float)((rng >> 40) * (1.0 / 16777216.0));
}

static float *fbuf(size_t n, float lo, float hi) {
    float *p = malloc(n * sizeof(float) + 1);
    for (size_t i = 0; i < n; ++i) p[i] = uni(lo, hi);
    return p;
}

static double *dbuf(size_t n) { return malloc(n * sizeof(double) + 1); }

static int failures = 0;

static void check(const char *what, int rc, const double *x, size_t n) {
    if (rc != 0) {
        fprintf(stderr, "%s: returned %d\n", what, rc);
        ++failures;
        return;
    }
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) {
            fprintf(stderr, "%s: non-finite output at %zu\n", what, i);
            ++failures;
            return;
        }
}

static void gdn_case(int B, int T, int H, int Dk, int Dv) {
    size_t nk = (size_t)B * T * H * Dk, nv = (size_t)B * T * H * Dv, ns = (size_t)B * T * H;
    size_t nh = (size_t)B * H * Dk * Dv;
    float *q = fbuf(nk, -0.3f, 0.3f), *k = fbuf(nk, -0.3f, 0.3f), *v = fbuf(nv, -1.f, 1.f);
    float *beta = fbuf(ns, 0.1f, 0.9f), *g = fbuf(ns, -0.5f, -0.01f), *h0 = fbuf(nh, -0.2f, 0.2f);
    float *dout = fbuf(nv, -1.f, 1.f), *dhT = fbuf(nh, -0.2f, 0.2f);
    double *o = dbuf(nv), *hT = dbuf(nh);
    check("oracle_gdn_recurrent", oracle_gdn_recurrent(B, T, H, Dk, Dv, q, k, v, beta, g, 0.5, h0, o, hT, 1), o, nv);
    check("oracle_gdn_recurrent hT", 0, hT, nh);
    double *dq = dbuf(nk), *dk = dbuf(nk), *dv = dbuf(nv), *db = dbuf(ns), *dg = dbuf(ns), *dh0 = dbuf(nh);
    check("oracle_gdn_recurrent_bwd",
          oracle_gdn_recurrent_bwd(B, T, H, Dk, Dv, q, k, v, beta, g, 0.5, h0, dout, dhT, dq, dk, dv, db, dg, dh0, 1),
          dq, nk);
    check("oracle_gdn_recurrent_bwd dh0", 0, dh0, nh);
    free(q), free(k), free(v), free(beta), free(g), free(h0), free(dout), free(dhT);
    free(o), free(hT), free(dq), free(dk), free(dv), free(db), free(dg), free(dh0);
}

static void dp_case(int B, int T, int H, int dk, int Dv) {
    const int r = 2, K = r * dk;
    size_t nk = (size_t)B * T * H * K, nv = (size_t)B * T * H * Dv, ns = (size_t)B * T * H;
    size_t nh = (size_t)B * H * K * Dv;
    const double mask[4] = {1.0, 0.0, 0.7, 1.0};
    float *q = fbuf(nk, -0.3f, 0.3f), *k = fbuf(nk, -0.3f, 0.3f), *v = fbuf(nv, -1.f, 1.f);
    float *beta = fbuf(ns * r, 0.1f, 0.9f), *g = fbuf(ns, -0.5f, -0.01f), *h0 = fbuf(nh, -0.2f, 0.2f);
    float *dout = fbuf(nv, -1.f, 1.f), *dhT = fbuf(nh, -0.2f, 0.2f);
    double *o = dbuf(nv), *hT = dbuf(nh);
    check("oracle_deltaproduct_recurrent",
          oracle_deltaproduct_recurrent(B, T, H, r, dk, Dv, q, k, v, beta, g, mask, 0.5, h0, o, hT, 1), o, nv);
    double *dq = dbuf(nk), *dkk = dbuf(nk), *dv = dbuf(nv), *db = dbuf(ns * r), *dg = dbuf(ns), *dh0 = dbuf(nh);
    check("oracle_deltaproduct_bwd",
          oracle_deltaproduct_bwd(B, T, H, r, dk, Dv, q, k, v, beta, g, mask, 0.5, h0, dout, dhT, dq, dkk, dv, db, dg,
                                  dh0, 1),
          dkk, nk);
    free(q), free(k), free(v), free(beta), free(g), free(h0), free(dout), free(dhT);
    free(o), free(hT), free(dq), free(dkk), free(dv), free(db), free(dg), free(dh0);
}

static void scan_case(int B, int H, int F, int S, int D) {
    size_t N = (size_t)F * S, nx = (size_t)B * H * N * D, ns = (size_t)B * H * N, nh = (size_t)B * H * D * D;
    float *q = fbuf(nx, -0.3f, 0.3f), *k = fbuf(nx, -0.3f, 0.3f), *v = fbuf(nx, -1.f, 1.f);
    float *beta = fbuf(ns, 0.1f, 0.9f), *g = fbuf((size_t)B * H * F, -0.5f, -0.01f), *h0 = fbuf(nh, -0.2f, 0.2f);
    float *dout = fbuf(nx, -1.f, 1.f), *dhT = fbuf(nh, -0.2f, 0.2f);
    double *out = dbuf(nx), *hT = dbuf(nh);
    check("oracle_frame_scan", oracle_frame_scan(B, H, F, S, D, q, k, v, beta, g, 0.5, h0, out, hT, 1), out, nx);
    double *dq = dbuf(nx), *dk = dbuf(nx), *dv = dbuf(nx), *db = dbuf(ns), *dg = dbuf((size_t)B * H * F);
    double *dh0 = dbuf(nh);
    check("oracle_frame_scan_bwd",
          oracle_frame_scan_bwd(B, H, F, S, D, q, k, v, beta, g, 0.5, h0, dout, dhT, dq, dk, dv, db, dg, dh0, 1), dq,
          nx);
    free(q), free(k), free(v), free(beta), free(g), free(h0), free(dout), free(dhT);
    free(out), free(hT), free(dq), free(dk), free(dv), free(db), free(dg), free(dh0);
}

static void prep_case(int B, int N, int H, int D) {
    size_t C = (size_t)H * D, ntok = (size_t)B * N, nx = ntok * 3 * C, no = (size_t)B * H * N * D;
    size_t ns = (size_t)B * H * N, np = ntok * 16, nr = (size_t)N * (D / 2);
    float *qkv = fbuf(nx, -1.f, 1.f), *wq = fbuf(C, 0.5f, 1.5f), *wk = fbuf(C, 0.5f, 1.5f);
    float *pq = fbuf(np, -1.f, 1.f), *pkv = fbuf(np, -1.f, 1.f), *cs = fbuf(nr, -1.f, 1.f), *sn = fbuf(nr, -1.f, 1.f);
    double *qo = dbuf(no), *ko = dbuf(no), *vo = dbuf(no), *pre = dbuf(ns), *post = dbuf(ns), *infl = dbuf(ns);
    check("oracle_cam_prep",
          oracle_cam_prep(B, N, H, D, qkv, wq, wk, pq, pkv, cs, sn, 0.8, 1e-6, qo, ko, vo, pre, post, infl, 1), ko, no);
    float *gq = fbuf(no, -1.f, 1.f), *gk = fbuf(no, -1.f, 1.f), *gv = fbuf(no, -1.f, 1.f);
    float *gpre = fbuf(ns, -1.f, 1.f), *gpost = fbuf(ns, -1.f, 1.f), *ginfl = fbuf(ns, -1.f, 1.f);
    double *dqkv = dbuf(nx), *dqw = dbuf(C), *dkw = dbuf(C), *dpq = dbuf(np), *dpkv = dbuf(np);
    check("oracle_cam_prep_bwd",
          oracle_cam_prep_bwd(B, N, H, D, qkv, wq, wk, pq, pkv, cs, sn, 0.8, 1e-6, gq, gk, gv, gpre, gpost, ginfl,
                              dqkv, dqw, dkw, dpq, dpkv, 1),
          dqkv, nx);
    check("oracle_cam_prep_bwd weights", 0, dqw, C);
    free(qkv), free(wq), free(wk), free(pq), free(pkv), free(cs), free(sn);
    free(qo), free(ko), free(vo), free(pre), free(post), free(infl);
    free(gq), free(gk), free(gv), free(gpre), free(gpost), free(ginfl);
    free(dqkv), free(dqw), free(dkw), free(dpq), free(dpkv);
}

static void se3_case(void) {
    /* two rigid transforms (row-major 4x4): a rotation about z with a
       translation, and the identity */
    double in[32] = {0}, out[32];
    const double c = cos(0.3), s = sin(0.3);
    double a[16] = {c, -s, 0, 1, s, c, 0, 2, 0, 0, 1, 3, 0, 0, 0, 1};
    for (int i = 0; i < 16; ++i) in[i] = a[i];
    for (int i = 0; i < 4; ++i) in[16 + 5 * i] = 1.0;
    oracle_invert_se3(2, in, out);
    check("oracle_invert_se3", 0, out, 32);
}

int main(void) {
    gdn_case(2, 70, 2, 16, 32);    /* T ragged against 64-token segments */
    gdn_case(1, 1, 1, 48, 16);     /* one token, width not a power of two */
    gdn_case(1, 0, 1, 16, 16);     /* no tokens */
    dp_case(1, 67, 2, 16, 16);
    scan_case(1, 2, 3, 5, 16);
    scan_case(1, 1, 0, 4, 16);     /* no frames */
    prep_case(2, 3, 2, 16);
    prep_case(1, 2, 3, 48);
    se3_case();
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("oracle sanitizer run: all routines clean\n");
    return 0;
}
