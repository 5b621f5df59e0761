"""Seeded synthetic inputs for the gated delta rule forward pass.

This module draws random inputs and nothing else: it holds none of the
method's arithmetic, and both the HIP path and the fp64 oracle consume what it
returns.  Every array is drawn in float64 with ``numpy.random.default_rng``
in the order the docstrings list, then cast.  A "bf16" array is returned as
float32 holding bf16 values exactly (float64 -> float32 -> bf16, each step
round-to-nearest-even), so the oracle and the GPU see identical numbers.

Workloads (the sizes and distributions of the method's configurations):

* ``gdn_tiny``        B=1 H=2  T=64    Dk=Dv=16  chunk 16, fp32
* ``gdn``             B=2 H=16 T=4096  Dk=Dv=128 chunk 64, bf16
* ``deltaproduct``    B=2 H=8  T=2048  K=2x128 Dv=128 chunk 32, r=2, bf16
* ``camera``          B=1 F=8 frames of 30x52 tokens, H=16 D=64, bf16
* ``gdn_long``        B=1 H=16 T=65536 Dk=Dv=128 chunk 64, bf16, h0 ~ N(0, 0.02^2)
"""
from __future__ import annotations

import numpy as np

WORKLOADS = {
    "gdn_tiny": dict(kind="gdn", B=1, H=2, T=64, Dk=16, Dv=16, chunk=16, dtype="f32",
                     h0_std=0.0, seed=20260),
    "gdn": dict(kind="gdn", B=2, H=16, T=4096, Dk=128, Dv=128, chunk=64, dtype="bf16",
                h0_std=0.0, seed=20261),
    "deltaproduct": dict(kind="deltaproduct", B=2, H=8, T=2048, r=2, dk=128, Dv=128, chunk=32,
                         dtype="bf16", seed=20262),
    "camera": dict(kind="camera", B=1, F=8, S=30 * 52, H=16, D=64, dtype="bf16", seed=20263),
    "gdn_long": dict(kind="gdn", B=1, H=16, T=65536, Dk=128, Dv=128, chunk=64, dtype="bf16",
                     h0_std=0.02, seed=20264),
}


def round_bf16(x) -> np.ndarray:
    """float64/float32 -> float32 holding the round-to-nearest-even bf16 value."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    out = u.astype(np.uint32).view(np.float32)
    out = np.where(nan, np.float32(np.nan), out)
    return np.ascontiguousarray(out, dtype=np.float32)


def cast(x, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def _l2n(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _sigmoid(x):
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def _logsigmoid(x):
    return -np.logaddexp(0.0, -x)


def gdn_inputs(B, T, H, Dk, Dv, seed, dtype="bf16", h0_std=0.0, decay_mean=2.0,
               decay_std=0.5, normalize=True):
    """Draw order: q, k ~ N(0,1) (B,T,H,Dk), L2-normalised per (b,t,h) when
    ``normalize``; v ~ N(0,1) (B,T,H,Dv); beta = sigmoid(N(0,1)) (B,T,H);
    g = logsigmoid(N(decay_mean, decay_std)) (B,T,H); h0 ~ N(0, h0_std^2)
    (B,H,Dk,Dv) when h0_std > 0 (else None).  beta, g, h0 are float32."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk))
    if normalize:
        q, k = _l2n(q), _l2n(k)
    v = rng.standard_normal((B, T, H, Dv))
    beta = _sigmoid(rng.standard_normal((B, T, H)))
    g = _logsigmoid(rng.normal(decay_mean, decay_std, (B, T, H)))
    h0 = rng.normal(0.0, h0_std, (B, H, Dk, Dv)) if h0_std > 0 else None
    return dict(q=cast(q, dtype), k=cast(k, dtype), v=cast(v, dtype),
                beta=beta.astype(np.float32), g=g.astype(np.float32),
                h0=None if h0 is None else h0.astype(np.float32))


def gdn_upstream(B, T, H, Dk, Dv, seed, dtype="bf16", dhT_std=0.0):
    """Upstream gradients for the backward: dout ~ N(0,1) (B,T,H,Dv) in
    ``dtype``; dhT ~ N(0, dhT_std^2) (B,H,Dk,Dv) float32 when dhT_std > 0
    (else None)."""
    rng = np.random.default_rng(seed)
    dout = rng.standard_normal((B, T, H, Dv))
    dhT = rng.normal(0.0, dhT_std, (B, H, Dk, Dv)) if dhT_std > 0 else None
    return dict(dout=cast(dout, dtype), dhT=None if dhT is None else dhT.astype(np.float32))


def deltaproduct_inputs(B, T, H, r, dk, Dv, seed, dtype="bf16", h0_std=0.0, mask=None,
                        decay_mean=2.0, decay_std=0.5):
    """Draw order: q, k ~ N(0,1) (B,T,H,r*dk), each dk-wide sub-key
    L2-normalised; v ~ N(0,1) (B,T,H,Dv); beta = sigmoid(N(0,1)) (B,T,H,r),
    one per step; g = logsigmoid(N(decay_mean, decay_std)) (B,T,H); h0 as in
    :func:`gdn_inputs`.  The step mask defaults to lower-triangular ones."""
    rng = np.random.default_rng(seed)
    q = _l2n(rng.standard_normal((B, T, H, r, dk))).reshape(B, T, H, r * dk)
    k = _l2n(rng.standard_normal((B, T, H, r, dk))).reshape(B, T, H, r * dk)
    v = rng.standard_normal((B, T, H, Dv))
    beta = _sigmoid(rng.standard_normal((B, T, H, r)))
    g = _logsigmoid(rng.normal(decay_mean, decay_std, (B, T, H)))
    h0 = rng.normal(0.0, h0_std, (B, H, r * dk, Dv)) if h0_std > 0 else None
    if mask is None:
        mask = np.tril(np.ones((r, r)))
    return dict(q=cast(q, dtype), k=cast(k, dtype), v=cast(v, dtype),
                beta=beta.astype(np.float32), g=g.astype(np.float32),
                h0=None if h0 is None else h0.astype(np.float32),
                mask=np.asarray(mask, np.float32))


def _random_rotation(rng, n):
    """n rotations in SO(3): Q of the QR factorisation of a Gaussian 3x3,
    columns sign-fixed by diag(R), one column negated when det Q = -1."""
    A = rng.standard_normal((n, 3, 3))
    Q, R = np.linalg.qr(A)
    d = np.sign(np.diagonal(R, axis1=1, axis2=2))
    d[d == 0] = 1.0
    Q = Q * d[:, None, :]
    neg = np.linalg.det(Q) < 0
    Q[neg, :, 0] *= -1.0
    return Q


def rope_tables(N, D_half, base=10000.0):
    """Interleaved-pair RoPE tables (N, D_half) float32 over the token index
    n: angle_i = n * base^(-2i/D_half) for pair i; cos repeated per pair,
    sin stored as (-sin, +sin).  Built in float64, then cast."""
    i = np.arange(D_half // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / D_half)
    ang = np.arange(N, dtype=np.float64)[:, None] * theta[None, :]
    c, s = np.cos(ang), np.sin(ang)
    cos_t = np.repeat(c, 2, axis=1)
    sin_t = np.stack([-s, s], axis=-1).reshape(N, D_half)
    return cos_t.astype(np.float32), sin_t.astype(np.float32)


def camera_inputs(B, F, S, H, D, seed, dtype="bf16", decay_mean=3.0, decay_std=0.5,
                  k_scale=None, eps=1e-6):
    """Camera-branch inputs.  Draw order: qkv ~ N(0,1) (B,N,3,H,D) with
    N = F*S; per-token rotation (see :func:`_random_rotation`) and
    translation ~ N(0,1)^3 giving P = [R t; 0 1]; scan beta =
    sigmoid(N(0,1)) (B,H,N); scan g = logsigmoid(N(decay_mean, decay_std))
    (B,H,F), one per frame.  proj_q = P^T and proj_kv = P^-1 (numpy inverse)
    as float32; norm weights are ones; k_scale = 1/sqrt(D); RoPE tables from
    :func:`rope_tables`."""
    rng = np.random.default_rng(seed)
    N = F * S
    qkv = rng.standard_normal((B, N, 3, H, D))
    Rm = _random_rotation(rng, B * N)
    t = rng.standard_normal((B * N, 3))
    P = np.zeros((B * N, 4, 4))
    P[:, :3, :3] = Rm
    P[:, :3, 3] = t
    P[:, 3, 3] = 1.0
    beta = _sigmoid(rng.standard_normal((B, H, N)))
    g = _logsigmoid(rng.normal(decay_mean, decay_std, (B, H, F)))
    cos_t, sin_t = rope_tables(N, D // 2)
    if k_scale is None:
        k_scale = 1.0 / np.sqrt(D)
    return dict(
        qkv=cast(qkv, dtype),
        q_norm_w=np.ones(H * D, np.float32), k_norm_w=np.ones(H * D, np.float32),
        P=P.reshape(B, N, 4, 4),
        proj_q=np.ascontiguousarray(np.transpose(P, (0, 2, 1)).reshape(B, N, 4, 4), np.float32),
        proj_kv=np.linalg.inv(P).reshape(B, N, 4, 4).astype(np.float32),
        rope_cos=cos_t, rope_sin=sin_t,
        k_scale=float(np.float32(k_scale)), eps=float(np.float32(eps)),
        beta=beta.astype(np.float32), g=g.astype(np.float32), F=F, S=S)


def workload_inputs(name, **overrides):
    """Inputs of a named workload (see the module docstring)."""
    cfg = dict(WORKLOADS[name])
    cfg.update(overrides)
    kind = cfg.pop("kind")
    cfg.pop("chunk", None)
    if kind == "gdn":
        return gdn_inputs(cfg["B"], cfg["T"], cfg["H"], cfg["Dk"], cfg["Dv"], cfg["seed"],
                          cfg["dtype"], cfg.get("h0_std", 0.0))
    if kind == "deltaproduct":
        return deltaproduct_inputs(cfg["B"], cfg["T"], cfg["H"], cfg["r"], cfg["dk"], cfg["Dv"],
                                   cfg["seed"], cfg["dtype"])
    if kind == "camera":
        return camera_inputs(cfg["B"], cfg["F"], cfg["S"], cfg["H"], cfg["D"], cfg["seed"],
                             cfg["dtype"])
    raise ValueError(kind)
