"""Pins of the fp64 camera-prep backward oracle (O8, gradients of O3).

O8 is checked against the forward oracle O3 (pinned in
``test_oracle_pins.py``) by finite differences of every input it returns a
gradient for, and its linear v path against the Jacobian of O3's v output,
built column by column from unit inputs.  No GPU is needed.
"""
import numpy as np

import oracle


def _grid(rng, shape, lo=-1.0, hi=1.0, step=2.0 ** -10):
    """Values on a 2^-10 grid: exact in float32, and so is x +- 2^-9."""
    return np.round(rng.uniform(lo, hi, size=shape) / step) * step


def _away(rng, shape, step=2.0 ** -10):
    """Grid values with |x| in [1/8, 1] and random signs: a perturbation of
    2^-8 never moves a post-norm value across the ReLU kink."""
    mag = np.round(rng.uniform(0.125, 1.0, size=shape) / step) * step
    return np.where(rng.uniform(size=shape) < 0.5, -mag, mag)


def _case(seed, B=1, N=3, H=2, D=16):
    rng = np.random.default_rng(seed)
    C = H * D
    d = dict(qkv=_away(rng, (B, N, 3, H, D)),
             q_norm_w=_grid(rng, C, 0.5, 1.5), k_norm_w=_grid(rng, C, 0.5, 1.5),
             proj_q=_grid(rng, (B, N, 4, 4)), proj_kv=_grid(rng, (B, N, 4, 4)),
             rope_cos=_grid(rng, (N, D // 2)), rope_sin=_grid(rng, (N, D // 2)))
    up = dict(dq=_grid(rng, (B, H, N, D)), dk=_grid(rng, (B, H, N, D)), dv=_grid(rng, (B, H, N, D)),
              dpre=_grid(rng, (B, H, N)), dpost=_grid(rng, (B, H, N)), dinfl=_grid(rng, (B, H, N)))
    return d, up


K_SCALE, EPS = 0.5, 2.0 ** -6


def _loss(d, up):
    o = oracle.cam_prep(d["qkv"], d["q_norm_w"], d["k_norm_w"], d["proj_q"], d["proj_kv"], d["rope_cos"],
                        d["rope_sin"], K_SCALE, EPS)
    L = np.sum(o["q"] * up["dq"]) + np.sum(o["k"] * up["dk"]) + np.sum(o["v"] * up["dv"])
    L += np.sum(o["k_pre_sq"] * up["dpre"]) + np.sum(o["k_post_sq"] * up["dpost"])
    L += np.sum(o["inflation_sq"] * up["dinfl"])
    return float(L)


def _fd(d, up, name, idx):
    def central(h):
        dp = {n: x.copy() for n, x in d.items()}
        dm = {n: x.copy() for n, x in d.items()}
        dp[name][idx] += h
        dm[name][idx] -= h
        return (_loss(dp, up) - _loss(dm, up)) / (2 * h)
    h = 2.0 ** -8
    return (4 * central(h / 2) - central(h)) / 3


def _grads(d, up):
    return oracle.cam_prep_bwd(d["qkv"], d["q_norm_w"], d["k_norm_w"], d["proj_q"], d["proj_kv"],
                               d["rope_cos"], d["rope_sin"], K_SCALE, EPS, up["dq"], up["dk"], up["dv"],
                               up["dpre"], up["dpost"], up["dinfl"])


def test_prep_bwd_matches_finite_differences():
    d, up = _case(11)
    g = _grads(d, up)
    pairs = (("qkv", "dqkv"), ("q_norm_w", "dq_norm_w"), ("k_norm_w", "dk_norm_w"),
             ("proj_q", "dproj_q"), ("proj_kv", "dproj_kv"))
    for name, gname in pairs:
        for idx in np.ndindex(d[name].shape):
            fd = _fd(d, up, name, idx)
            assert abs(g[gname][idx] - fd) <= 1e-7 + 1e-6 * abs(fd), (name, idx, g[gname][idx], fd)


def test_prep_bwd_without_norm_outputs_matches_finite_differences():
    """Only the q, k, v outputs carry gradient (no pre/post/inflation terms);
    two batches, unit weights passed as None."""
    d, up = _case(12, B=2, N=2, H=1, D=8)
    d["q_norm_w"] = np.ones_like(d["q_norm_w"])
    d["k_norm_w"] = np.ones_like(d["k_norm_w"])
    for n in ("dpre", "dpost", "dinfl"):
        up[n] = np.zeros_like(up[n])
    g = oracle.cam_prep_bwd(d["qkv"], None, None, d["proj_q"], d["proj_kv"], d["rope_cos"], d["rope_sin"],
                            K_SCALE, EPS, up["dq"], up["dk"], up["dv"])
    for idx in np.ndindex(d["qkv"].shape):
        fd = _fd(d, up, "qkv", idx)
        assert abs(g["dqkv"][idx] - fd) <= 1e-7 + 1e-6 * abs(fd), (idx, g["dqkv"][idx], fd)


def test_prep_bwd_v_path_is_the_transposed_map():
    """v_out is linear in v_raw (UCPE on the first half, RoPE on the second):
    its gradient must be J^T dv with J built from unit inputs through O3."""
    B, N, H, D = 1, 2, 2, 16
    d, up = _case(13, B=B, N=N, H=H, D=D)
    g = _grads(d, up)
    C = H * D
    for n in range(N):
        J = np.zeros((C, C))
        for c in range(C):
            x = d["qkv"].copy()
            x[0, n, 2] = 0.0
            x[0, n, 2].reshape(-1)[c] = 1.0
            o = oracle.cam_prep(x, d["q_norm_w"], d["k_norm_w"], d["proj_q"], d["proj_kv"], d["rope_cos"],
                                d["rope_sin"], K_SCALE, EPS)
            J[:, c] = o["v"][0, :, n, :].reshape(-1)
        want = J.T @ up["dv"][0, :, n, :].reshape(-1)
        np.testing.assert_allclose(g["dqkv"][0, n, 2].reshape(-1), want, rtol=0, atol=1e-12)
