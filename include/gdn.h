/*
 * gdn.h - C ABI of the MI355X (gfx950) gated delta rule forward library.
 *
 * Four operations (and the scan's normaliser stream), each a forward pass
 * over device-resident tensors:
 *
 *   gdn_chunk_fwd           chunkwise gated delta rule (r = 1)
 *   deltaproduct_chunk_fwd  chunkwise gated DeltaProduct (r sub-keys per token)
 *   gdn_recurrent_fwd       camera-branch numerator-only scan, frame-synchronous
 *   gdn_recurrent_den_fwd   its normaliser (denominator) stream
 *   gdn_prep                camera-branch per-token prep (RMSNorm over all
 *                           channels, ReLU, K-scale, UCPE 4x4, RoPE, ||k||^2)
 *   gdn_prep_bwd            gradients of gdn_prep (qkv, norm weights, projections)
 *   gdn_bwd                 gradients of gdn_chunk_fwd (q, k, v, beta, g, h0)
 *   deltaproduct_bwd        gradients of deltaproduct_chunk_fwd (r = 2, lower
 *                           unitriangular step mask)
 *   gdn_recurrent_bwd       gradients of gdn_recurrent_fwd (forward direction)
 *
 * Sources (web pages, cited by title and section):
 *   [dp]  msj19 "gated_deltaproduct" test.py: gated_chunk_scaled_dot_kkt_fwd,
 *         solve_tril, gated_fwd_recompute_w_u, gated_chunk_fwd_h_fn,
 *         gated_chunk_fwd_o_fn.
 *   [cam] Sana "fused_cam_gdn.py": cam_prep_func, _cam_prep_kernel,
 *         cam_scan_func, _cam_scan_kernel.
 *   [cp]  Sana "fused_gdn_cp.py": module docstring (KV and Z recurrences).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named as tensors are DEVICE pointers to dense row-major arrays
 *   with the shapes given below (last index fastest).  The only host pointer
 *   is `step_mask` of deltaproduct_chunk_fwd and deltaproduct_bwd.
 * - `dtype` selects the element type of the q/k/v (and qkv) inputs:
 *   GDN_DTYPE_F32 or GDN_DTYPE_BF16.  Gates (beta, log_decay), states
 *   (h0, hT) and the prep's projection and RoPE tables are always float32.
 * - `out_dtype` selects the element type of the chunk outputs o.
 * - The state S of one (batch, head) has shape (Dk, Dv): rows follow the key
 *   dimension, columns the value dimension.  The read-out is o = scale*S^T q.
 * - h0 (initial state) may be NULL (zero state); hT (final state) may be
 *   NULL (not stored).  h0 is the state at the end of a prefix: the first
 *   token's (or frame's) gate applies to it, so running [0,T1) then [T1,T)
 *   with h0 = hT of the first call equals one call over [0,T).
 * - Ownership: all buffers belong to the caller.  The library keeps no
 *   pointer after the call returns, allocates no memory, and enqueues all
 *   work on `stream` (a hipStream_t passed as void*, NULL = default stream);
 *   the caller keeps buffers alive until that stream has finished.  Its only
 *   process-wide state is a per-device cache of the compute-unit count
 *   (atomic, set on first use) besides the thread-local error text.
 * - Work space: entry points that need scratch device memory take
 *   (workspace, workspace_bytes); the matching *_workspace_bytes() query
 *   returns the size needed (0 means workspace may be NULL).
 * - Errors: every entry point validates all arguments before launching
 *   anything and returns GDN_OK (0) or a negative GDN_E* code; nothing is
 *   launched on error.  gdn_last_error() returns a message for the last
 *   failing call on the calling thread.  No exception or abort crosses the
 *   ABI.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    GDN_OK = 0,
    GDN_EINVAL = -1,        /* null pointer, bad size, misaligned pointer      */
    GDN_EUNSUPPORTED = -2,  /* a size or option outside the supported set      */
    GDN_EWORKSPACE = -3,    /* workspace smaller than *_workspace_bytes()      */
    GDN_EHIP = -4           /* HIP launch or runtime failure                   */
};

enum { GDN_DTYPE_F32 = 0, GDN_DTYPE_BF16 = 1 };

/* Message for the last non-zero return on this thread ("" if none). */
const char *gdn_last_error(void);

/* ABI version; bumped on any incompatible change. */
int gdn_abi_version(void);

/*
 * gdn_chunk_fwd - chunkwise gated delta rule forward.
 *
 * Per (b, h) and token t, with S = h0 (or 0):
 *   S_t = exp(g_t) (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
 *   o_t = scale * S_t^T q_t,          hT = S_T.
 * Computed chunk by chunk ([dp] the chunk kernels with r = 1): chunk-local
 * cumsum of g, the strictly-lower intra-chunk matrix
 * A[t,s] = beta_t (k_t . k_s) exp(G_t - G_s), T = (I + A)^-1 from 16x16
 * diagonal blocks and exact block merges, the WY form, the sequential
 * inter-chunk state pass and the output product.  For long sequences over
 * few heads (bf16, chunk 64, Dk <= 128) the state pass runs segment-parallel:
 * per-segment transitions and states from zero, composed, then each segment
 * from its true start ([cp] module docstring); the work space then also
 * holds one Dk x (Dk + Dv) fp32 pair per segment.
 *
 *   q, k      (B, T, H, Dk)  dtype
 *   v         (B, T, H, Dv)  dtype
 *   beta      (B, T, H)      float32
 *   log_decay (B, T, H)      float32, g_t (gate exp(g_t); normally <= 0)
 *   h0, hT    (B, H, Dk, Dv) float32, nullable
 *   o         (B, T, H, Dv)  out_dtype
 * Supported: Dk and Dv multiples of 16 with Dv <= 256 and
 *   bf16 inputs:  Dk <= 256 at chunk 16 or 32, Dk <= 128 at chunk 64;
 *   fp32 inputs:  Dk <= 256 at chunk 16 or 32, Dk <= 64 at chunk 64;
 * any T >= 0 (a last chunk shorter than `chunk` is handled); token rows of
 * H*Dk and H*Dv elements below 2^24.  A Dk that is not a power of two runs
 * the next power of two's kernels with the extra features read as zero
 * (e.g. Dk = 112 as 128).  16-byte aligned tensor pointers.  Other
 * combinations return GDN_EUNSUPPORTED (the work-space query returns 0).
 */
int gdn_chunk_fwd(const void *q, const void *k, const void *v,
                  const float *beta, const float *log_decay, float scale,
                  const float *h0, float *hT, void *o,
                  int B, int T, int H, int Dk, int Dv, int chunk,
                  int dtype, int out_dtype,
                  void *workspace, size_t workspace_bytes, void *stream);

size_t gdn_chunk_fwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, int chunk,
                                     int dtype);

/*
 * gdn_chunk_fwd_noalloc - gdn_chunk_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, meaning, kernels and
 * results as gdn_chunk_fwd, without (workspace, workspace_bytes): the work
 * space is a static device array of GDN_NOALLOC_SCRATCH_BYTES inside the
 * library, one copy per device, looked up on the first call on a device and
 * held until the process ends.  This entry point calls no hipMalloc,
 * hipFree or allocating library routine.
 * Limit: shapes whose gdn_chunk_fwd_workspace_bytes exceeds
 * GDN_NOALLOC_SCRATCH_BYTES are rejected with GDN_EWORKSPACE (B=2 H=16
 * T=4096 Dk=Dv=128 chunk 64 bf16 needs 73 MB and runs; B=1 H=16 T=65536
 * needs over 300 MB and is rejected).
 * Every call on one device shares that device's array: calls that overlap
 * on one device (on different streams, or from several threads without
 * ordering) race and give wrong results; serialise them.  Nothing in the
 * array needs to start at zero (each call writes every entry it reads).
 */
#define GDN_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)
int gdn_chunk_fwd_noalloc(const void *q, const void *k, const void *v,
                          const float *beta, const float *log_decay, float scale,
                          const float *h0, float *hT, void *o,
                          int B, int T, int H, int Dk, int Dv, int chunk,
                          int dtype, int out_dtype, void *stream);

/*
 * deltaproduct_chunk_fwd - chunkwise gated DeltaProduct forward ([dp]).
 *
 * The key of width K = r*dk is split into r sub-keys k_{t,a}.  Step a of
 * token t writes with k_{t,a} into row block a of the (K, Dv) state and
 * erases along e_{t,a} = sum_b M[a][b] k_{t,b} (placed in row block b).
 * Per token: P = exp(g_t) S; p_a = P^T e_{t,a} for all a from the same P;
 * S = P + sum_a beta_{t,a} E_a k_{t,a} (v_t - p_a)^T; o_t = scale S^T q_t.
 * With r = 1 and M = [[1]] this is gdn_chunk_fwd.  For r = 2 with a lower
 * unitriangular mask [[1, 0], [m, 1]] and bf16 inputs the row blocks are two
 * chained gated delta rules (block 1's values are v - m times block 0's
 * prediction) and run as two passes of 64-token chunks, whatever `chunk`.
 *
 *   q, k       (B, T, H, r*dk) dtype
 *   v          (B, T, H, Dv)   dtype
 *   beta       (B, T, H, r)    float32, one per step
 *   log_decay  (B, T, H)       float32
 *   step_mask  (r, r)          float32 HOST array, row-major M[a][b]
 *   h0, hT     (B, H, r*dk, Dv) float32, nullable
 *   o          (B, T, H, Dv)   out_dtype
 * Supported: r = 1 as gdn_chunk_fwd; r = 2 with dk in {16, 32, 64, 128}
 * and chunk in {16, 32} (bf16 and fp32 inputs); Dv a multiple of 16 up to
 * 256; H*r*dk and H*Dv below 2^24.  Other combinations return
 * GDN_EUNSUPPORTED.
 */
int deltaproduct_chunk_fwd(const void *q, const void *k, const void *v,
                           const float *beta, const float *log_decay,
                           const float *step_mask, int r, float scale,
                           const float *h0, float *hT, void *o,
                           int B, int T, int H, int dk, int Dv, int chunk,
                           int dtype, int out_dtype,
                           void *workspace, size_t workspace_bytes, void *stream);

size_t deltaproduct_chunk_fwd_workspace_bytes(int B, int T, int H, int r, int dk, int Dv,
                                              int chunk, int dtype);

/*
 * gdn_recurrent_fwd - camera-branch numerator-only scan ([cam]
 * _cam_scan_kernel, both directions; cam_scan_func), frame-synchronous.
 *
 * Tokens come in F frames of S tokens (N = F*S).  Forward (reverse = 0),
 * per (b, h), with S = h0:
 *   P = exp(g_f) S_{f-1};
 *   S_f = P + sum_{s in f} beta_s k_s (v_s - P^T k_s)^T
 *       (every token of the frame predicts from the same gated state P);
 *   out_s = scale * S_f^T q_s for s in f;    hT = S_F.
 * With S = 1 this is the token-level gated delta rule.
 *
 * Reverse (reverse = 1; [cam] REVERSE branch of _cam_scan_kernel and the
 * flip-and-shift reference of cam_scan_func): the forward scan run over
 * frames F-1 .. 0 with k, v, beta shifted by one frame, so frame f reads the
 * state R_f built from frames f+1 .. F-1 only:
 *   R_{F-1} = 0;   R_f = (I - G_{f+1}) exp(g_{f+1}) R_{f+1} + H_{f+1},
 *   G_j = sum_{s in j} beta_s k_s k_s^T,  H_j = sum_{s in j} beta_s k_s v_s^T;
 *   out_s = scale * R_f^T q_s for s in f.
 * The reverse scan takes no h0 and returns no hT (both must be NULL,
 * GDN_EUNSUPPORTED otherwise), as on the page.
 *
 *   q, k, v    (B, H, N, D)  dtype   (the layout gdn_prep writes)
 *   beta       (B, H, N)     float32
 *   log_decay  (B, H, F)     float32, one gate per frame
 *   h0, hT     (B, H, D, D)  float32, nullable
 *   out        (B, H, N, D)  float32
 *   reverse    0 or 1
 * Supported: D a multiple of 16 up to 128 (a D that is not a power of two
 * runs the next power of two's kernels with the extra features read as
 * zero); F >= 0; S >= 1.
 */
int gdn_recurrent_fwd(const void *q, const void *k, const void *v,
                      const float *beta, const float *log_decay, float scale,
                      const float *h0, float *hT, float *out,
                      int B, int H, int F, int S, int D, int dtype, int reverse,
                      void *workspace, size_t workspace_bytes, void *stream);

size_t gdn_recurrent_fwd_workspace_bytes(int B, int H, int F, int S, int D, int dtype);

/*
 * gdn_recurrent_bwd - gradients of gdn_recurrent_fwd's outputs (out, hT) in
 * the forward direction ([cam] _cam_scan_bwd_kernel, the backward of
 * cam_scan_func), frame-synchronous like the forward.
 *
 * With P_f = exp(g_f) S_{f-1}, G_f = sum_{s in f} beta_s k_s k_s^T and
 * X_f = dL/dS_f including frame f's read-out (A_f = scale Q_f^T dO_f),
 * walked from the last frame back (X_{F-1} = dhT + A_{F-1}):
 *   X_{f-1} = exp(g_f) (I - G_f) X_f + A_{f-1},  dh0 = exp(g_0)(I - G_0) X_0,
 *   dlog_decay_f = <(I - G_f) X_f, P_f>,
 * and per token s of frame f, u_s = X_f^T k_s, r_s = v_s - P_f^T k_s:
 *   dq_s = scale S_f dout_s,  dv_s = beta_s u_s,  dbeta_s = u_s . r_s,
 *   dk_s = beta_s (X_f r_s - P_f u_s).
 *
 *   q, k, v, dout   (B, H, N, D)  dtype (dout = dL/dout)
 *   beta            (B, H, N)     float32
 *   log_decay       (B, H, F)     float32
 *   h0, dhT         (B, H, D, D)  float32, nullable (zero)
 *   dq, dk, dv      (B, H, N, D)  float32
 *   dbeta           (B, H, N)     float32
 *   dlog_decay      (B, H, F)     float32
 *   dh0             (B, H, D, D)  float32, nullable (not stored)
 * Supported: bf16 inputs; D in {32, 64, 128}; F >= 0; S >= 1.  q, k, v,
 * dout, dq, dk, dv 16-byte aligned, the other tensors 4-byte.  The work
 * space (gdn_recurrent_bwd_workspace_bytes) holds the forward's per-frame
 * G_f, H_f and S_f, the partial A_f and every X_f.
 */
int gdn_recurrent_bwd(const void *q, const void *k, const void *v,
                      const float *beta, const float *log_decay, float scale,
                      const float *h0, const void *dout, const float *dhT,
                      float *dq, float *dk, float *dv, float *dbeta, float *dlog_decay,
                      float *dh0, int B, int H, int F, int S, int D, int dtype,
                      void *workspace, size_t workspace_bytes, void *stream);

size_t gdn_recurrent_bwd_workspace_bytes(int B, int H, int F, int S, int D, int dtype);

/*
 * gdn_recurrent_den_fwd - normaliser (denominator) stream of the camera
 * branch ([cp] module docstring: the Z recurrence next to the KV state, its
 * per-frame transition decay_f (I - P_z) and input B_z = sum of k beta).
 * Per (b, h), frame-synchronous like gdn_recurrent_fwd, with a vector state
 * z in R^D (z = z0 or 0):
 *   z_f = exp(g_f) (I - P_f) z_{f-1} + b_f,
 *   P_f = sum_{s in f} beta_s kz_s kz_s^T,   b_f = sum_{s in f} beta_s kz_s;
 *   den_s = scale * qd_s . z_f   for s in f;   zT = z_F.
 * This is gdn_recurrent_fwd with every value equal to 1, so z is any column
 * of that scan's state.  reverse = 1 runs the anti-causal direction exactly
 * as gdn_recurrent_fwd does (no z0, no zT).  The caller forms
 * num / (den + eps) itself, as on the page.
 *
 *   q_den, k_z  (B, H, N, D)  dtype   (the read-out and key rows of the
 *                                      stream; the page's Z keys carry no RoPE)
 *   beta        (B, H, N)     float32
 *   log_decay   (B, H, F)     float32, one gate per frame
 *   z0, zT      (B, H, D)     float32, nullable
 *   den         (B, H, N)     float32
 * Supported: D a multiple of 16 up to 128; F >= 0; S >= 1.  Work space:
 * gdn_recurrent_den_fwd_workspace_bytes.
 */
int gdn_recurrent_den_fwd(const void *q_den, const void *k_z,
                          const float *beta, const float *log_decay, float scale,
                          const float *z0, float *zT, float *den,
                          int B, int H, int F, int S, int D, int dtype, int reverse,
                          void *workspace, size_t workspace_bytes, void *stream);

size_t gdn_recurrent_den_fwd_workspace_bytes(int B, int H, int F, int S, int D, int dtype);

/*
 * gdn_prep - camera-branch prep ([cam] cam_prep_func, _cam_prep_kernel),
 * one pass over the packed projection.
 *
 * For token (b, n) with C = H*D channels: inv_rms_x = 1/sqrt(mean_c x_c^2
 * + norm_eps) for x in {q, k}; per head: q~ = relu(q inv_rms_q w_q),
 * k~ = relu(k inv_rms_k w_k) * k_scale, v~ = v; k_pre_sq = ||k~||^2; first
 * D/2 values in groups of 4: y = P x (P = proj_q for q, proj_kv for k, v);
 * second D/2 values: y[d] = x[d] rope_cos[n][d] + x[d^1] rope_sin[n][d];
 * k_post_sq = ||k_out||^2; inflation_sq = max(post,1e-12)/max(pre,1e-12).
 *
 *   qkv              (B, N, 3, H, D) dtype (slot 0 q, 1 k, 2 v)
 *   q_norm_w, k_norm_w (H*D)         float32, nullable (= all ones)
 *   proj_q, proj_kv  (B, N, 4, 4)    float32, row-major per token
 *   rope_cos, rope_sin (N, D/2)      float32, interleaved-pair tables
 *   q_out, k_out, v_out (B, H, N, D) out_dtype (the page writes the input
 *                    dtype; GDN_DTYPE_F32 keeps the full fp32 result)
 *   k_pre_sq, k_post_sq (B, H, N)    float32
 *   inflation_sq     (B, H, N)       float32, nullable (not stored)
 * Supported: D a multiple of 16 up to 128; H * D' <= 4096 with D' the
 * smallest power of two >= D (e.g. H <= 32 at D = 112).  qkv, the q/k/v outputs,
 * the norm weights and the RoPE tables must be 16-byte aligned (they are
 * read and written as 16-byte vectors); the other float tensors 4-byte.
 */
int gdn_prep(const void *qkv, const float *q_norm_w, const float *k_norm_w,
             const float *proj_q, const float *proj_kv,
             const float *rope_cos, const float *rope_sin,
             float k_scale, float norm_eps,
             void *q_out, void *k_out, void *v_out,
             float *k_pre_sq, float *k_post_sq, float *inflation_sq,
             int B, int N, int H, int D, int dtype, int out_dtype, void *stream);

/*
 * gdn_prep_bwd - gradients of gdn_prep ([cam] _cam_prep_bwd_kernel and
 * _cam_prep_bwd_dispatch, including the RMSNorm backward the page leaves
 * to torch).  Reverse mode through the prep's steps, with the forward's
 * values recomputed per token: the norm outputs send
 * 2 k_out (dk_post_sq + [post > 1e-12] dinflation_sq / max(pre, 1e-12)) to
 * k_out and 2 k~ (dk_pre_sq - [pre > 1e-12] dinflation_sq max(post, 1e-12)
 * / pre^2) to k~; RoPE^T on the second half (gx[d] = gy[d] cos[d] +
 * gy[d^1] sin[d^1]); UCPE^T on the first (gx_g = P^T gy_g, dP += gy_g x_g^T
 * over groups and heads); the ReLU mask and K-scale; the RMSNorm backward
 * over all C channels (gx_c = inv w_c ga_c - inv^3/C x_c sum ga w x, and
 * dw_c = sum over tokens of ga_c x_c inv).
 *
 *   qkv, weights, proj, tables, k_scale, norm_eps: as gdn_prep (dtype)
 *   dq_out, dk_out, dv_out  (B, H, N, D)  grad_dtype (dL/d of the outputs)
 *   dk_pre_sq, dk_post_sq, dinflation_sq  (B, H, N) float32, nullable (zero)
 *   dqkv                    (B, N, 3, H, D) float32
 *   dq_norm_w, dk_norm_w    (H*D) float32, nullable (not formed)
 *   dproj_q, dproj_kv       (B, N, 4, 4) float32, both or neither nullable
 * Supported: as gdn_prep.  The work space (gdn_prep_bwd_workspace_bytes,
 * needed only for the weight gradients) holds one partial sum of the
 * weight gradients per wave; they are added in a fixed order.
 */
int gdn_prep_bwd(const void *qkv, const float *q_norm_w, const float *k_norm_w,
                 const float *proj_q, const float *proj_kv,
                 const float *rope_cos, const float *rope_sin, float k_scale, float norm_eps,
                 const void *dq_out, const void *dk_out, const void *dv_out,
                 const float *dk_pre_sq, const float *dk_post_sq, const float *dinflation_sq,
                 float *dqkv, float *dq_norm_w, float *dk_norm_w, float *dproj_q, float *dproj_kv,
                 int B, int N, int H, int D, int dtype, int grad_dtype,
                 void *workspace, size_t workspace_bytes, void *stream);

size_t gdn_prep_bwd_workspace_bytes(int B, int N, int H, int D);

/*
 * gdn_bwd - gradients of gdn_chunk_fwd's outputs (o, hT) ([dp] lists the
 * chunk backward kernels of this rule: prepare_dv, dhu, dqkw, WY backward).
 *
 * bf16 inputs with Dk in {32, 64, 128} and Dv a multiple of 32 up to 128
 * (and T > 0, H Dk and H Dv below 2^24) take the chunkwise path, 64-token chunks on MFMA: the chunk
 * prep (T = (I + A)^-1, its transpose, the transposed causal scores), the
 * forward state pass keeping every chunk's start state S and residual
 * R = V - e^G K S, the reverse pass over the chunks,
 *   dVn = scale Pm^T dO + diag(e^{G_L - G}) K dS',  dX = T^T dVn,
 *   dS = e^{G_L} dS' + scale Q^T diag(e^G) dO - K^T diag(e^G beta) dX,
 * (dS' = dhT, or 0, after the last chunk; dh0 = dS before the first), and
 * the per-chunk gradients of q, k, v, beta and g from S, dS', R and dX.
 * Every other shape walks the token recurrence backwards: with
 * P = exp(g_t) S_{t-1}, p = P^T k_t, S_t = P + beta_t k_t (v_t - p)^T,
 * o_t = scale S_t^T q_t and dS = dL/dS_t,
 *   dS += scale q_t do_t^T,  dq_t = scale S_t do_t,  r = v_t - p,
 *   u = dS^T k_t,  dv_t = beta_t u,  dbeta_t = u . r,  dp = -beta_t u,
 *   dk_t = beta_t dS r + P dp,  dP = dS + k_t dp^T,  dg_t = <dP, P>,
 *   dS = exp(g_t) dP;   dh0 = dS after token 0,
 * with states recomputed from copies kept every 12 tokens.
 *
 *   q, k            (B, T, H, Dk)  dtype
 *   v, dout         (B, T, H, Dv)  dtype (dout = dL/do)
 *   beta, log_decay (B, T, H)      float32
 *   h0, dhT         (B, H, Dk, Dv) float32, nullable (zero)
 *   dq, dk          (B, T, H, Dk)  float32
 *   dv              (B, T, H, Dv)  float32
 *   dbeta, dlog_decay (B, T, H)    float32 (dlog_decay = dL/dg)
 *   dh0             (B, H, Dk, Dv) float32, nullable (not stored)
 * Supported: Dk in {16, 32, 64, 128}; Dv a multiple of 16 up to 4096; any
 * T >= 0.  q, k, v, dout, dq and dk 16-byte aligned, the other tensors
 * 4-byte.  The
 * work space depends on the path, hence on dtype; gdn_bwd_workspace_bytes
 * is the only authority on its size.  Chunkwise path: per 64-token chunk
 * and head, T and T^T (16 KiB), the scores (10 KiB), the gate table, S and
 * dS' (2 Dk Dv * 4 bytes), R and dX (2 * 64 Dv * 4 bytes).  Token path:
 * the states kept every 12 tokens and per-16-column partial sums, about
 * (Dk Dv / 12 + (2 Dk + 2) Dv / 16) * 4 bytes per token and head.
 */
size_t gdn_bwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, int dtype);
int gdn_bwd(const void *q, const void *k, const void *v,
            const float *beta, const float *log_decay, float scale,
            const float *h0, const void *dout, const float *dhT,
            float *dq, float *dk, float *dv, float *dbeta, float *dlog_decay,
            float *dh0, int B, int T, int H, int Dk, int Dv, int dtype,
            void *workspace, size_t workspace_bytes, void *stream);

/*
 * deltaproduct_bwd - gradients of deltaproduct_chunk_fwd's outputs (o, hT)
 * for r = 2 with a lower unitriangular step mask M = [[1, 0], [m, 1]] ([dp]:
 * the forward's chunk kernels with two steps per token; the backward is
 * that forward's reverse mode).
 *
 * With that mask the state's row block 0 is a gated delta rule on
 * (q_0, k_0, v, beta_0) and row block 1 one on (q_1, k_1, v', beta_1), with
 * v'_t = (1 - m) v_t + m e_t and e_t = v_t minus block 0's prediction at
 * token t (its per-token error, the same for every chunk size), both under
 * the one gate g.  The gradients come from two chunkwise backward passes
 * (64-token chunks, MFMA) as in gdn_bwd: block 1's, whose v gradient is
 * that of v' (dv'), then block 0's with the error gradient dE = m dv'
 * (through e = R - A~ Vn: dVn gains -A~^T dE, the state recurrence
 * -K^T diag(e^G) dE, the gram gradient -(beta dX + dE) Vn^T), giving
 *   dv = beta_0 dX_0 + dv',  dg = dg_0 + dg_1,
 * dq, dk, dbeta and dh0 per sub-key block.
 *
 *   q, k            (B, T, H, 2*dk) dtype (sub-key a in columns a*dk ..)
 *   v, dout         (B, T, H, Dv)   dtype (dout = dL/do)
 *   beta            (B, T, H, 2)    float32
 *   log_decay       (B, T, H)       float32
 *   step_mask       (2, 2)          float32 HOST array, row-major
 *   h0, dhT         (B, H, 2*dk, Dv) float32, nullable (zero)
 *   dq, dk          (B, T, H, 2*dk) float32
 *   dv              (B, T, H, Dv)   float32
 *   dbeta           (B, T, H, 2)    float32
 *   dlog_decay      (B, T, H)       float32
 *   dh0             (B, H, 2*dk, Dv) float32, nullable (not stored)
 * Supported: bf16 inputs, r = 2, M[0][0] = M[1][1] = 1 and M[0][1] = 0,
 * dk in {32, 64, 128}, Dv a multiple of 32 from 32 to 128, H 2 dk and
 * H Dv below 2^24, any T >= 0 (T = 0 gives dh0 = dhT).  Other masks,
 * types and widths return GDN_EUNSUPPORTED.  q, k, v, dout, dq, dk, dv 16-byte aligned; h0, dhT,
 * dh0 16-byte; the other tensors 4-byte; workspace 256-byte aligned.  The
 * work space (deltaproduct_bwd_workspace_bytes, 0 for an unsupported
 * shape) holds gdn_bwd's chunkwise regions for each sub-key, A~ in two
 * fragment layouts and v' (B*H*ceil(T/64)*64*Dv floats).
 */
size_t deltaproduct_bwd_workspace_bytes(int B, int T, int H, int r, int dk, int Dv, int dtype);
int deltaproduct_bwd(const void *q, const void *k, const void *v,
                     const float *beta, const float *log_decay,
                     const float *step_mask, int r, float scale,
                     const float *h0, const void *dout, const float *dhT,
                     float *dq, float *dk, float *dv, float *dbeta, float *dlog_decay,
                     float *dh0, int B, int T, int H, int sub_dk, int Dv, int dtype,
                     void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
