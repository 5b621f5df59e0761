"""Pins of the fp64 DeltaProduct backward oracle (O9, gradients of O2).

O9 is checked against the forward oracle O2 (pinned in
``test_oracle_pins.py``) by finite differences of every input, with a
general step mask and with the lower unitriangular one, and against the
gated delta rule's backward (O6) for one step per token.  No GPU is
needed.
"""
import numpy as np
import pytest

import oracle


def _grid(rng, shape, lo=-1.0, hi=1.0, step=2.0 ** -10):
    return np.round(rng.uniform(lo, hi, size=shape) / step) * step


def _case(seed, B, T, H, r, dk, Dv):
    rng = np.random.default_rng(seed)
    K = r * dk
    d = dict(q=_grid(rng, (B, T, H, K)), k=_grid(rng, (B, T, H, K), -0.7, 0.7), v=_grid(rng, (B, T, H, Dv)),
             beta=_grid(rng, (B, T, H, r), 0.05, 0.95), g=_grid(rng, (B, T, H), -0.6, -0.01),
             h0=_grid(rng, (B, H, K, Dv)))
    up = dict(dout=_grid(rng, (B, T, H, Dv)), dhT=_grid(rng, (B, H, K, Dv)))
    return d, up


def _loss(d, up, mask, scale):
    o, hT = oracle.deltaproduct_recurrent(d["q"], d["k"], d["v"], d["beta"], d["g"], mask, scale, d["h0"])
    return float(np.sum(o * up["dout"]) + np.sum(hT * up["dhT"]))


def _fd(d, up, mask, scale, name, idx):
    def central(h):
        dp = {n: x.copy() for n, x in d.items()}
        dm = {n: x.copy() for n, x in d.items()}
        dp[name][idx] += h
        dm[name][idx] -= h
        return (_loss(dp, up, mask, scale) - _loss(dm, up, mask, scale)) / (2 * h)
    h = 2.0 ** -8
    return (4 * central(h / 2) - central(h)) / 3


@pytest.mark.parametrize("seed,mask", [
    (21, np.array([[0.75, -0.5], [0.25, 1.0]])),       # a general mask (upper entry too)
    (22, np.array([[1.0, 0.0], [1.0, 1.0]])),          # lower unitriangular, m = 1
    (23, np.array([[1.0, 0.0], [0.5, 1.0]])),          # lower unitriangular, m = 1/2
])
def test_dp_bwd_matches_finite_differences(seed, mask):
    scale = 0.7
    d, up = _case(seed, 1, 4, 2, 2, 2, 3)
    grads = oracle.deltaproduct_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], mask, up["dout"], scale, d["h0"],
                                    up["dhT"])
    for name, gr in zip(("q", "k", "v", "beta", "g", "h0"), grads):
        for idx in np.ndindex(d[name].shape):
            fd = _fd(d, up, mask, scale, name, idx)
            assert abs(gr[idx] - fd) <= 1e-7 + 1e-6 * abs(fd), (name, idx, gr[idx], fd)


def test_dp_bwd_across_segments_matches_finite_differences():
    """T = 70 spans two of the oracle's 64-token recompute segments."""
    mask = np.array([[1.0, 0.0], [1.0, 1.0]])
    d, up = _case(24, 1, 70, 1, 2, 1, 2)
    grads = dict(zip(("q", "k", "v", "beta", "g", "h0"),
                     oracle.deltaproduct_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], mask, up["dout"], 1.0,
                                             d["h0"], up["dhT"])))
    for t in (0, 1, 62, 63, 64, 65, 69):
        for name in ("q", "k", "v", "beta", "g"):
            idx = (0, t, 0) + ((1,) if d[name].ndim == 4 else ())
            fd = _fd(d, up, mask, 1.0, name, idx)
            assert abs(grads[name][idx] - fd) <= 1e-7 + 1e-6 * abs(fd), (name, t)


def test_dp_bwd_one_step_is_the_gated_delta_rule():
    """r = 1 with M = [[1]] is the gated delta rule: O9 equals O6."""
    d, up = _case(25, 2, 9, 2, 1, 3, 2)
    mask = np.array([[1.0]])
    got = oracle.deltaproduct_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], mask, up["dout"], 0.8, d["h0"],
                                  up["dhT"])
    ref = oracle.gdn_recurrent_bwd(d["q"], d["k"], d["v"], d["beta"][..., 0], d["g"], up["dout"], 0.8, d["h0"],
                                   up["dhT"])
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a.reshape(b.shape), b, rtol=1e-12, atol=1e-13)
