"""fp64 CPU oracle for the gated delta rule forward pass (test infrastructure).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library or its binding, and the product path never imports
it.

The arithmetic lives in ``gdn_oracle.c`` (plain scalar double-precision loops,
built with gcc by :func:`build`); this module only marshals numpy arrays into
it.  ``chunkwise_ref`` holds the fp64 chunkwise (WY) form, used by the tests
to pin the token recurrences by brute force.

Functions (inputs are float32 numpy arrays holding the exact values the GPU
receives; outputs are float64):

* :func:`gdn_recurrent`            - O1, gated delta rule token by token.
* :func:`deltaproduct_recurrent`   - O2, gated DeltaProduct token by token.
* :func:`cam_prep`                 - O3, camera-branch prep per token.
* :func:`frame_scan`               - O4, frame-synchronous numerator-only scan.
* :func:`frame_scan_reverse`       - O4 in the anti-causal direction.
* :func:`frame_den`                - the normaliser (Z) stream of O4.
* :func:`gdn_recurrent_bwd`        - O6, gradients of O1 (reverse mode).
* :func:`frame_scan_bwd`           - O7, gradients of O4 (reverse mode).
* :func:`cam_prep_bwd`             - O8, gradients of O3 (reverse mode).
* :func:`deltaproduct_bwd`         - O9, gradients of O2 (reverse mode).
* :func:`invert_se3`               - closed-form rigid-transform inverse.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile ``gdn_oracle.c`` with gcc (-O2, OpenMP, no fast-math)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           "-Wall", "-Wextra", "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if (not os.path.exists(_LIB_PATH)
            or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    D = ctypes.c_double
    lib.oracle_gdn_recurrent.argtypes = [I, I, I, I, I, P, P, P, P, P, D, P, P, P, I]
    lib.oracle_deltaproduct_recurrent.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, D, P, P, P, I]
    lib.oracle_cam_prep.argtypes = [I, I, I, I, P, P, P, P, P, P, P, D, D, P, P, P, P, P, P, I]
    lib.oracle_frame_scan.argtypes = [I, I, I, I, I, P, P, P, P, P, D, P, P, P, I]
    lib.oracle_gdn_recurrent_bwd.argtypes = [I, I, I, I, I, P, P, P, P, P, D, P, P, P,
                                             P, P, P, P, P, P, I]
    lib.oracle_frame_scan_bwd.argtypes = [I, I, I, I, I, P, P, P, P, P, D, P, P, P,
                                          P, P, P, P, P, P, I]
    lib.oracle_cam_prep_bwd.argtypes = [I, I, I, I, P, P, P, P, P, P, P, D, D, P, P, P, P, P, P, P, P, P,
                                        P, P, I]
    lib.oracle_deltaproduct_bwd.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, D, P, P, P, P, P, P, P, P, P, I]
    lib.oracle_invert_se3.argtypes = [ctypes.c_long, P, P]
    lib.oracle_invert_se3.restype = None
    lib.oracle_max_threads.argtypes = []
    for fn in (lib.oracle_gdn_recurrent, lib.oracle_gdn_recurrent_bwd, lib.oracle_frame_scan_bwd,
               lib.oracle_deltaproduct_recurrent,
               lib.oracle_cam_prep, lib.oracle_cam_prep_bwd, lib.oracle_deltaproduct_bwd, lib.oracle_frame_scan,
               lib.oracle_max_threads):
        fn.restype = ctypes.c_int
    _lib = lib
    return lib


def max_threads() -> int:
    return _load().oracle_max_threads()


def _f32(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name}: invalid arguments (rc={rc})")


def gdn_recurrent(q, k, v, beta, g, scale=1.0, h0=None, nthreads=0):
    """O1.  q,k (B,T,H,Dk); v (B,T,H,Dv); beta,g (B,T,H); h0 (B,H,Dk,Dv).

    Returns (o (B,T,H,Dv), hT (B,H,Dk,Dv)) in float64.
    """
    q, k, v, beta, g, h0 = map(_f32, (q, k, v, beta, g, h0))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == q.shape and v.shape[:3] == (B, T, H)
    assert beta.shape == (B, T, H) and g.shape == (B, T, H)
    assert h0 is None or h0.shape == (B, H, Dk, Dv)
    o = np.zeros((B, T, H, Dv), np.float64)
    hT = np.zeros((B, H, Dk, Dv), np.float64)
    rc = _load().oracle_gdn_recurrent(B, T, H, Dk, Dv, _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                      _ptr(g), float(scale), _ptr(h0), _ptr(o), _ptr(hT),
                                      int(nthreads))
    _check(rc, "gdn_recurrent")
    return o, hT


def gdn_recurrent_bwd(q, k, v, beta, g, dout, scale=1.0, h0=None, dhT=None, nthreads=0):
    """O6.  Gradients of :func:`gdn_recurrent`'s (o, hT) under the upstream
    gradients dout (B,T,H,Dv) and dhT (B,H,Dk,Dv, or None = 0).  Returns
    (dq, dk, dv, dbeta, dg, dh0) in float64 (dg is the gradient of the
    log-decay g)."""
    q, k, v, beta, g, dout, h0, dhT = map(_f32, (q, k, v, beta, g, dout, h0, dhT))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == q.shape and v.shape[:3] == (B, T, H) and dout.shape == v.shape
    assert beta.shape == (B, T, H) and g.shape == (B, T, H)
    for st in (h0, dhT):
        assert st is None or st.shape == (B, H, Dk, Dv)
    dq = np.zeros((B, T, H, Dk), np.float64)
    dk = np.zeros((B, T, H, Dk), np.float64)
    dv = np.zeros((B, T, H, Dv), np.float64)
    dbeta = np.zeros((B, T, H), np.float64)
    dg = np.zeros((B, T, H), np.float64)
    dh0 = np.zeros((B, H, Dk, Dv), np.float64)
    rc = _load().oracle_gdn_recurrent_bwd(B, T, H, Dk, Dv, _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                          _ptr(g), float(scale), _ptr(h0), _ptr(dout), _ptr(dhT),
                                          _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbeta), _ptr(dg),
                                          _ptr(dh0), int(nthreads))
    _check(rc, "gdn_recurrent_bwd")
    return dq, dk, dv, dbeta, dg, dh0


def deltaproduct_recurrent(q, k, v, beta, g, mask, scale=1.0, h0=None, nthreads=0):
    """O2.  q,k (B,T,H,r*dk); v (B,T,H,Dv); beta (B,T,H,r); g (B,T,H);
    mask (r,r); h0 (B,H,r*dk,Dv).  Returns (o, hT) in float64."""
    q, k, v, beta, g, h0 = map(_f32, (q, k, v, beta, g, h0))
    mask = np.ascontiguousarray(mask, dtype=np.float64)
    B, T, H, K = q.shape
    r = mask.shape[0]
    assert mask.shape == (r, r) and K % r == 0
    dk = K // r
    Dv = v.shape[-1]
    assert k.shape == q.shape and beta.shape == (B, T, H, r) and g.shape == (B, T, H)
    assert h0 is None or h0.shape == (B, H, K, Dv)
    o = np.zeros((B, T, H, Dv), np.float64)
    hT = np.zeros((B, H, K, Dv), np.float64)
    rc = _load().oracle_deltaproduct_recurrent(B, T, H, r, dk, Dv, _ptr(q), _ptr(k), _ptr(v),
                                               _ptr(beta), _ptr(g), _ptr(mask), float(scale),
                                               _ptr(h0), _ptr(o), _ptr(hT), int(nthreads))
    _check(rc, "deltaproduct_recurrent")
    return o, hT


def deltaproduct_bwd(q, k, v, beta, g, mask, dout, scale=1.0, h0=None, dhT=None, nthreads=0):
    """O9.  Gradients of :func:`deltaproduct_recurrent`'s (o, hT) under dout
    (B,T,H,Dv) and dhT (B,H,r*dk,Dv, or None).  Returns (dq, dk, dv, dbeta
    (B,T,H,r), dg (B,T,H), dh0) in float64."""
    q, k, v, beta, g, dout, h0, dhT = map(_f32, (q, k, v, beta, g, dout, h0, dhT))
    mask = np.ascontiguousarray(mask, np.float64)
    B, T, H, K = q.shape
    r = mask.shape[0]
    assert mask.shape == (r, r) and K % r == 0 and beta.shape == (B, T, H, r)
    Dv = v.shape[-1]
    dq = np.zeros((B, T, H, K), np.float64)
    dk = np.zeros((B, T, H, K), np.float64)
    dv = np.zeros((B, T, H, Dv), np.float64)
    dbeta = np.zeros((B, T, H, r), np.float64)
    dg = np.zeros((B, T, H), np.float64)
    dh0 = np.zeros((B, H, K, Dv), np.float64)
    rc = _load().oracle_deltaproduct_bwd(B, T, H, r, K // r, Dv, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
                                         _ptr(mask), float(scale), _ptr(h0), _ptr(dout), _ptr(dhT), _ptr(dq),
                                         _ptr(dk), _ptr(dv), _ptr(dbeta), _ptr(dg), _ptr(dh0), int(nthreads))
    _check(rc, "deltaproduct_bwd")
    return dq, dk, dv, dbeta, dg, dh0


def cam_prep(qkv, q_norm_w, k_norm_w, proj_q, proj_kv, rope_cos, rope_sin,
             k_scale, eps, nthreads=0):
    """O3.  qkv (B,N,3,H,D); weights (H*D,) or None; proj (B,N,4,4);
    rope tables (N, D/2).  Returns dict of float64 arrays: q, k, v (B,H,N,D)
    and k_pre_sq, k_post_sq, inflation_sq (B,H,N)."""
    qkv, q_norm_w, k_norm_w, proj_q, proj_kv, rope_cos, rope_sin = map(
        _f32, (qkv, q_norm_w, k_norm_w, proj_q, proj_kv, rope_cos, rope_sin))
    B, N, three, H, D = qkv.shape
    assert three == 3
    assert proj_q.shape == (B, N, 4, 4) and proj_kv.shape == (B, N, 4, 4)
    assert rope_cos.shape == (N, D // 2) and rope_sin.shape == (N, D // 2)
    out = {name: np.zeros((B, H, N, D), np.float64) for name in ("q", "k", "v")}
    for name in ("k_pre_sq", "k_post_sq", "inflation_sq"):
        out[name] = np.zeros((B, H, N), np.float64)
    rc = _load().oracle_cam_prep(B, N, H, D, _ptr(qkv), _ptr(q_norm_w), _ptr(k_norm_w),
                                 _ptr(proj_q), _ptr(proj_kv), _ptr(rope_cos), _ptr(rope_sin),
                                 float(k_scale), float(eps), _ptr(out["q"]), _ptr(out["k"]),
                                 _ptr(out["v"]), _ptr(out["k_pre_sq"]), _ptr(out["k_post_sq"]),
                                 _ptr(out["inflation_sq"]), int(nthreads))
    _check(rc, "cam_prep")
    return out


def cam_prep_bwd(qkv, q_norm_w, k_norm_w, proj_q, proj_kv, rope_cos, rope_sin, k_scale, eps,
                 dq, dk, dv, dpre=None, dpost=None, dinfl=None, nthreads=0):
    """O8.  Gradients of :func:`cam_prep` under the upstream gradients dq,
    dk, dv (B,H,N,D) of its q, k, v outputs and, each optional, dpre, dpost,
    dinfl (B,H,N) of k_pre_sq, k_post_sq, inflation_sq.  Returns a dict of
    float64 arrays: dqkv (B,N,3,H,D), dq_norm_w and dk_norm_w (H*D),
    dproj_q and dproj_kv (B,N,4,4)."""
    qkv, q_norm_w, k_norm_w, proj_q, proj_kv, rope_cos, rope_sin, dq, dk, dv, dpre, dpost, dinfl = map(
        _f32, (qkv, q_norm_w, k_norm_w, proj_q, proj_kv, rope_cos, rope_sin, dq, dk, dv, dpre, dpost, dinfl))
    B, N, three, H, D = qkv.shape
    assert three == 3 and dq.shape == (B, H, N, D) and dk.shape == dq.shape and dv.shape == dq.shape
    out = {"dqkv": np.zeros((B, N, 3, H, D), np.float64),
           "dq_norm_w": np.zeros(H * D, np.float64), "dk_norm_w": np.zeros(H * D, np.float64),
           "dproj_q": np.zeros((B, N, 4, 4), np.float64), "dproj_kv": np.zeros((B, N, 4, 4), np.float64)}
    rc = _load().oracle_cam_prep_bwd(B, N, H, D, _ptr(qkv), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(proj_q),
                                     _ptr(proj_kv), _ptr(rope_cos), _ptr(rope_sin), float(k_scale), float(eps),
                                     _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dpre), _ptr(dpost), _ptr(dinfl),
                                     _ptr(out["dqkv"]), _ptr(out["dq_norm_w"]), _ptr(out["dk_norm_w"]),
                                     _ptr(out["dproj_q"]), _ptr(out["dproj_kv"]), int(nthreads))
    _check(rc, "cam_prep_bwd")
    return out


def frame_scan(q, k, v, beta, g, F, scale=1.0, h0=None, nthreads=0):
    """O4.  q,k,v (B,H,N,D) with N = F*S; beta (B,H,N); g (B,H,F) per frame;
    h0 (B,H,D,D).  Returns (out (B,H,N,D), hT (B,H,D,D)) in float64."""
    q, k, v, beta, g, h0 = map(_f32, (q, k, v, beta, g, h0))
    B, H, N, D = q.shape
    assert N % F == 0
    S = N // F
    assert beta.shape == (B, H, N) and g.shape == (B, H, F)
    out = np.zeros((B, H, N, D), np.float64)
    hT = np.zeros((B, H, D, D), np.float64)
    rc = _load().oracle_frame_scan(B, H, F, S, D, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
                                   float(scale), _ptr(h0), _ptr(out), _ptr(hT), int(nthreads))
    _check(rc, "frame_scan")
    return out, hT


def frame_scan_bwd(q, k, v, beta, g, F, dout, scale=1.0, h0=None, dhT=None, nthreads=0):
    """O7.  Gradients of :func:`frame_scan`'s (out, hT) under the upstream
    gradients dout (B,H,N,D) and dhT (B,H,D,D, or None = 0).  Returns
    (dq, dk, dv, dbeta (B,H,N), dg (B,H,F), dh0) in float64."""
    q, k, v, beta, g, dout, h0, dhT = map(_f32, (q, k, v, beta, g, dout, h0, dhT))
    B, H, N, D = q.shape
    assert F > 0 and N % F == 0
    S = N // F
    assert beta.shape == (B, H, N) and g.shape == (B, H, F) and dout.shape == q.shape
    dq, dk, dv = (np.zeros((B, H, N, D), np.float64) for _ in range(3))
    dbeta = np.zeros((B, H, N), np.float64)
    dg = np.zeros((B, H, F), np.float64)
    dh0 = np.zeros((B, H, D, D), np.float64)
    rc = _load().oracle_frame_scan_bwd(B, H, F, S, D, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
                                       float(scale), _ptr(h0), _ptr(dout), _ptr(dhT), _ptr(dq), _ptr(dk),
                                       _ptr(dv), _ptr(dbeta), _ptr(dg), _ptr(dh0), int(nthreads))
    _check(rc, "frame_scan_bwd")
    return dq, dk, dv, dbeta, dg, dh0


def _flip_and_shift(x, axis, pad):
    """Reverse ``x`` along ``axis`` and move it one place later, filling the
    first place with ``pad`` (the last element drops off) - the frame
    re-indexing of [cam] ``_flip_and_shift``."""
    xf = np.flip(x, axis=axis)
    lead = np.full_like(np.take(xf, [0], axis=axis), pad)
    return np.concatenate([lead, np.take(xf, np.arange(x.shape[axis] - 1), axis=axis)], axis=axis)


def frame_scan_reverse(q, k, v, beta, g, F, scale=1.0, nthreads=0):
    """O4, reverse direction, as [cam] defines it for ``cam_scan_func(...,
    reverse=True)`` (its pure-torch reference): frames are reversed; q is only
    flipped, k, v and beta are flipped and shifted by one frame with zeros,
    the per-frame gates are flipped and shifted with a gate factor of 1
    (log-decay 0); the forward scan O4 runs on that, and its output is
    flipped back.  No initial or final state (the page rejects them).
    Shapes as :func:`frame_scan`; returns out (B,H,N,D) float64."""
    q, k, v, beta, g = map(_f32, (q, k, v, beta, g))
    B, H, N, D = q.shape
    assert N % F == 0
    S = N // F
    fr = lambda x: x.reshape(B, H, F, S, D)
    q_b = np.flip(fr(q), axis=2)
    k_b = _flip_and_shift(fr(k), 2, 0.0)
    v_b = _flip_and_shift(fr(v), 2, 0.0)
    beta_b = _flip_and_shift(beta.reshape(B, H, F, S), 2, 0.0)
    g_b = _flip_and_shift(g, 2, 0.0)
    flat = lambda x: np.ascontiguousarray(x.reshape(B, H, N, D))
    out_b, _ = frame_scan(flat(q_b), flat(k_b), flat(v_b), np.ascontiguousarray(beta_b.reshape(B, H, N)),
                          np.ascontiguousarray(g_b), F, scale, None, nthreads)
    return np.ascontiguousarray(np.flip(out_b.reshape(B, H, F, S, D), axis=2).reshape(B, H, N, D))


def frame_den(q_den, k_z, beta, g, F, scale=1.0, z0=None, reverse=False, nthreads=0):
    """Normaliser stream ([cp] module docstring: z_f = decay_f (I - P_z) z_{f-1}
    + B_z with P_z = sum beta k k^T and B_z = sum beta k over the frame, read
    out as den = q . z).  It is O4 with every value equal to 1: H_f = sum
    beta_s k_s 1^T has B_z in every column, so each column of the O4 state is
    z; den is column 0 of the O4 output.  q_den, k_z (B,H,N,D); z0 (B,H,D).
    Returns (den (B,H,N), zT (B,H,D) or None for the reverse direction)."""
    q_den, k_z, beta, g, z0 = map(_f32, (q_den, k_z, beta, g, z0))
    B, H, N, D = q_den.shape
    ones = np.ones((B, H, N, D), np.float32)
    if reverse:
        assert z0 is None
        out = frame_scan_reverse(q_den, k_z, ones, beta, g, F, scale, nthreads)
        return np.ascontiguousarray(out[..., 0]), None
    h0 = None if z0 is None else np.ascontiguousarray(np.repeat(z0[..., :, None], D, axis=-1))
    out, hT = frame_scan(q_den, k_z, ones, beta, g, F, scale, h0, nthreads)
    return np.ascontiguousarray(out[..., 0]), np.ascontiguousarray(hT[..., :, 0])


def invert_se3(P):
    """Closed-form inverse of rigid transforms; P (..., 4, 4) float64."""
    P = np.ascontiguousarray(P, dtype=np.float64)
    out = np.zeros_like(P)
    n = P.size // 16
    _load().oracle_invert_se3(n, _ptr(P), _ptr(out))
    return out
