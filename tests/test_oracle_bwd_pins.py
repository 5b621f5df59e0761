"""Pins of the fp64 backward oracle (O6, gradients of the gated delta rule).

O6 is checked against the forward oracle O1 (itself pinned in
``test_oracle_pins.py``) by finite differences, and against closed forms of
the special case beta = 0, where the rule is a gated linear read-out of h0.
No GPU is needed.
"""
import numpy as np
import pytest

import oracle


def _grid(rng, shape, lo=-1.0, hi=1.0, step=2.0 ** -10):
    """Values on a 2^-10 grid: exact in float32, and so is x +- 2^-9."""
    return np.round(rng.uniform(lo, hi, size=shape) / step) * step


def _case(seed, B, T, H, Dk, Dv, with_h0=True, with_dhT=True):
    rng = np.random.default_rng(seed)
    d = {
        "q": _grid(rng, (B, T, H, Dk)),
        "k": _grid(rng, (B, T, H, Dk), -0.7, 0.7),
        "v": _grid(rng, (B, T, H, Dv)),
        "beta": _grid(rng, (B, T, H), 0.05, 0.95),
        "g": _grid(rng, (B, T, H), -0.6, -0.01),
        "h0": _grid(rng, (B, H, Dk, Dv)) if with_h0 else None,
    }
    up = {"dout": _grid(rng, (B, T, H, Dv)),
          "dhT": _grid(rng, (B, H, Dk, Dv)) if with_dhT else None}
    return d, up


def _loss(d, up, scale):
    o, hT = oracle.gdn_recurrent(d["q"], d["k"], d["v"], d["beta"], d["g"], scale, d["h0"])
    L = float(np.sum(o * up["dout"]))
    if up["dhT"] is not None:
        L += float(np.sum(hT * up["dhT"]))
    return L


def _fd(d, up, scale, name, idx):
    """dL/dx by central differences at steps h and h/2, combined by
    Richardson extrapolation (error O(h^4))."""
    def central(h):
        dp = {n: (None if x is None else x.copy()) for n, x in d.items()}
        dm = {n: (None if x is None else x.copy()) for n, x in d.items()}
        dp[name][idx] += h
        dm[name][idx] -= h
        return (_loss(dp, up, scale) - _loss(dm, up, scale)) / (2 * h)
    h = 2.0 ** -8
    return (4 * central(h / 2) - central(h)) / 3


@pytest.mark.parametrize("seed,B,T,H,Dk,Dv", [(1, 1, 5, 2, 3, 2), (2, 2, 3, 1, 2, 4)])
def test_bwd_matches_finite_differences(seed, B, T, H, Dk, Dv):
    scale = 0.75
    d, up = _case(seed, B, T, H, Dk, Dv)
    grads = oracle.gdn_recurrent_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], up["dout"],
                                     scale, d["h0"], up["dhT"])
    for name, gr in zip(("q", "k", "v", "beta", "g", "h0"), grads):
        for idx in np.ndindex(d[name].shape):
            fd = _fd(d, up, scale, name, idx)
            assert abs(gr[idx] - fd) <= 1e-7 + 1e-6 * abs(fd), (name, idx, gr[idx], fd)


def test_bwd_across_segments_matches_finite_differences():
    """T = 150 spans three of the oracle's 64-token recompute segments; a
    sample of entries on both sides of each boundary."""
    scale = 1.0
    d, up = _case(3, 1, 150, 1, 2, 2)
    grads = dict(zip(("q", "k", "v", "beta", "g", "h0"),
                     oracle.gdn_recurrent_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"],
                                              up["dout"], scale, d["h0"], up["dhT"])))
    for t in (0, 1, 62, 63, 64, 65, 127, 128, 129, 149):
        for name in ("q", "k", "v", "beta", "g"):
            idx = (0, t, 0) + ((1,) if d[name].ndim == 4 else ())
            fd = _fd(d, up, scale, name, idx)
            assert abs(grads[name][idx] - fd) <= 1e-7 + 1e-6 * abs(fd), (name, t)
    fd = _fd(d, up, scale, "h0", (0, 0, 1, 0))
    assert abs(grads["h0"][0, 0, 1, 0] - fd) <= 1e-7 + 1e-6 * abs(fd)


def test_bwd_beta_zero_closed_forms():
    """With beta = 0 nothing is written or erased: S_t = A_t h0 with
    A_t = exp(g_1 + ... + g_t), o_t = scale A_t h0^T q_t.  Then
      dq_t  = scale A_t h0 do_t,          dk = dv = 0,
      dS_t  = sum_{t' >= t} (A_t'/A_t) scale q_t' do_t'^T + (A_T/A_t) dhT,
      dbeta_t = k_t^T dS_t (v_t - A_t h0^T k_t),
      dg_t  = sum_{t' >= t} scale A_t' q_t'^T h0 do_t' + A_T <dhT, h0>,
      dh0   = sum_t scale A_t q_t do_t^T + A_T dhT."""
    B, T, H, Dk, Dv = 1, 7, 2, 3, 4
    scale = 0.5
    d, up = _case(4, B, T, H, Dk, Dv)
    d["beta"][:] = 0.0
    dq, dk, dv, dbeta, dg, dh0 = oracle.gdn_recurrent_bwd(
        d["q"], d["k"], d["v"], d["beta"], d["g"], up["dout"], scale, d["h0"], up["dhT"])
    assert np.all(dk == 0) and np.all(dv == 0)
    for h in range(H):
        h0 = d["h0"][0, h]
        A = np.exp(np.cumsum(d["g"][0, :, h]))
        q, k, v, do = d["q"][0, :, h], d["k"][0, :, h], d["v"][0, :, h], up["dout"][0, :, h]
        dhT = up["dhT"][0, h]
        for t in range(T):
            np.testing.assert_allclose(dq[0, t, h], scale * A[t] * h0 @ do[t], rtol=1e-12, atol=1e-14)
            dS = sum(A[s] / A[t] * scale * np.outer(q[s], do[s]) for s in range(t, T)) + A[-1] / A[t] * dhT
            np.testing.assert_allclose(dbeta[0, t, h], k[t] @ dS @ (v[t] - A[t] * h0.T @ k[t]),
                                       rtol=1e-11, atol=1e-13)
            dgt = sum(scale * A[s] * q[s] @ h0 @ do[s] for s in range(t, T)) + A[-1] * np.sum(dhT * h0)
            np.testing.assert_allclose(dg[0, t, h], dgt, rtol=1e-11, atol=1e-13)
        dh0_ref = sum(scale * A[t] * np.outer(q[t], do[t]) for t in range(T)) + A[-1] * dhT
        np.testing.assert_allclose(dh0[0, h], dh0_ref, rtol=1e-12, atol=1e-14)


def test_bwd_empty_sequence():
    """T = 0: the final state is h0, so dh0 = dhT and there is nothing else."""
    d, up = _case(5, 2, 0, 3, 4, 2)
    dq, dk, dv, dbeta, dg, dh0 = oracle.gdn_recurrent_bwd(
        d["q"], d["k"], d["v"], d["beta"], d["g"], up["dout"], 1.0, d["h0"], up["dhT"])
    assert dq.shape == (2, 0, 3, 4) and dv.shape == (2, 0, 3, 2) and dg.shape == (2, 0, 3)
    np.testing.assert_array_equal(dh0, up["dhT"])


def test_bwd_without_upstream_state_gradient():
    """dhT = None is the same as dhT = 0, and h0 = None the same as h0 = 0."""
    d, up = _case(6, 1, 9, 2, 3, 3, with_h0=False, with_dhT=False)
    a = oracle.gdn_recurrent_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], up["dout"], 1.0)
    z0 = np.zeros((1, 2, 3, 3))
    b = oracle.gdn_recurrent_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], up["dout"], 1.0, z0, z0)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


# ---------------------------------------------------------------------------
# O7: gradients of the frame-synchronous scan (O4)
# ---------------------------------------------------------------------------
def _frame_case(seed, B, H, F, S, D, with_h0=True, with_dhT=True):
    rng = np.random.default_rng(seed)
    N = F * S
    d = {
        "q": _grid(rng, (B, H, N, D)),
        "k": _grid(rng, (B, H, N, D), -0.5, 0.5),
        "v": _grid(rng, (B, H, N, D)),
        "beta": _grid(rng, (B, H, N), 0.05, 0.95),
        "g": _grid(rng, (B, H, F), -0.6, -0.01),
        "h0": _grid(rng, (B, H, D, D)) if with_h0 else None,
    }
    up = {"dout": _grid(rng, (B, H, N, D)),
          "dhT": _grid(rng, (B, H, D, D)) if with_dhT else None}
    return d, up


def _frame_loss(d, up, F, scale):
    out, hT = oracle.frame_scan(d["q"], d["k"], d["v"], d["beta"], d["g"], F, scale, d["h0"])
    L = float(np.sum(out * up["dout"]))
    if up["dhT"] is not None:
        L += float(np.sum(hT * up["dhT"]))
    return L


def _frame_fd(d, up, F, scale, name, idx):
    def central(h):
        dp = {n: (None if x is None else x.copy()) for n, x in d.items()}
        dm = {n: (None if x is None else x.copy()) for n, x in d.items()}
        dp[name][idx] += h
        dm[name][idx] -= h
        return (_frame_loss(dp, up, F, scale) - _frame_loss(dm, up, F, scale)) / (2 * h)
    h = 2.0 ** -8
    return (4 * central(h / 2) - central(h)) / 3


def test_frame_bwd_matches_finite_differences():
    """Every gradient entry of O7 against central differences of O4: three
    frames of four tokens, with h0 and dhT."""
    B, H, F, S, D = 1, 2, 3, 4, 3
    scale = 0.75
    d, up = _frame_case(11, B, H, F, S, D)
    grads = oracle.frame_scan_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], F, up["dout"], scale,
                                  d["h0"], up["dhT"])
    for name, gr in zip(("q", "k", "v", "beta", "g", "h0"), grads):
        for idx in np.ndindex(d[name].shape):
            fd = _frame_fd(d, up, F, scale, name, idx)
            assert abs(gr[idx] - fd) <= 1e-7 + 1e-6 * abs(fd), (name, idx, gr[idx], fd)


def test_frame_bwd_one_token_per_frame_is_the_token_backward():
    """With S = 1 the frame scan is the token recurrence (O1), so O7 equals
    O6 once the (B,H,N,D) and (B,T,H,D) layouts are matched."""
    B, H, T, D = 2, 3, 9, 4
    d, up = _frame_case(12, B, H, T, 1, D)
    f = oracle.frame_scan_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], T, up["dout"], 0.5,
                              d["h0"], up["dhT"])
    tr = lambda x: np.ascontiguousarray(np.swapaxes(x, 1, 2))      # (B,H,T,...) <-> (B,T,H,...)
    t = oracle.gdn_recurrent_bwd(tr(d["q"]), tr(d["k"]), tr(d["v"]), tr(d["beta"]), tr(d["g"]),
                                 tr(up["dout"]), 0.5, d["h0"], up["dhT"])
    for a, b in zip(f[:5], t[:5]):
        np.testing.assert_allclose(a, tr(b), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(f[5], t[5], rtol=1e-12, atol=1e-14)


def test_frame_bwd_without_upstream_state_gradient():
    """dhT = None is the same as dhT = 0, and h0 = None the same as h0 = 0."""
    d, up = _frame_case(13, 1, 2, 2, 5, 3, with_h0=False, with_dhT=False)
    a = oracle.frame_scan_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], 2, up["dout"], 1.0)
    z0 = np.zeros((1, 2, 3, 3))
    b = oracle.frame_scan_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], 2, up["dout"], 1.0, z0, z0)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_frame_bwd_matches_the_matrix_form():
    """O7 against the frame-level matrix form of the same gradients (a
    different algorithm): with G_f = sum_s beta_s k_s k_s^T,
    A_f = scale Q_f^T dO_f, X_F-1 = dhT + A_F-1 and
    X_f-1 = e^{g_f} (I - G_f) X_f + A_f-1, dh0 = e^{g_0} (I - G_0) X_0;
    per token dq = scale S_f do, u = X_f^T k, r = v - P_f^T k, dv = beta u,
    dbeta = u . r, dk = beta X_f r - beta P_f u; dg_f = <(I - G_f) X_f, P_f>."""
    B, H, F, S, D = 1, 2, 4, 6, 5
    scale = 0.6
    d, up = _frame_case(14, B, H, F, S, D)
    got = oracle.frame_scan_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], F, up["dout"], scale,
                                d["h0"], up["dhT"])
    f64 = lambda x: np.asarray(x, np.float64)
    for h in range(H):
        q, k, v = (f64(d[n][0, h]).reshape(F, S, D) for n in ("q", "k", "v"))
        beta = f64(d["beta"][0, h]).reshape(F, S)
        g, do = f64(d["g"][0, h]), f64(up["dout"][0, h]).reshape(F, S, D)
        I = np.eye(D)
        # forward states with the frame matrices
        G = [np.einsum("s,si,sj->ij", beta[f], k[f], k[f]) for f in range(F)]
        Hm = [np.einsum("s,si,sj->ij", beta[f], k[f], v[f]) for f in range(F)]
        Sst = [f64(d["h0"][0, h])]
        for f in range(F):
            Sst.append(np.exp(g[f]) * (I - G[f]) @ Sst[-1] + Hm[f])
        A = [scale * q[f].T @ do[f] for f in range(F)]
        X = [None] * F
        X[F - 1] = f64(up["dhT"][0, h]) + A[F - 1]
        for f in range(F - 1, 0, -1):
            X[f - 1] = np.exp(g[f]) * (I - G[f]) @ X[f] + A[f - 1]
        dh0 = np.exp(g[0]) * (I - G[0]) @ X[0]
        for f in range(F):
            P = np.exp(g[f]) * Sst[f]
            U = k[f] @ X[f]                              # rows u_s = X_f^T k_s
            R = v[f] - k[f] @ P                          # rows r_s = v_s - P^T k_s
            sl = slice(f * S, (f + 1) * S)
            np.testing.assert_allclose(got[0][0, h, sl], scale * do[f] @ Sst[f + 1].T, rtol=1e-11, atol=1e-13)
            np.testing.assert_allclose(got[2][0, h, sl], beta[f][:, None] * U, rtol=1e-11, atol=1e-13)
            np.testing.assert_allclose(got[3][0, h, sl], np.sum(U * R, axis=1), rtol=1e-11, atol=1e-13)
            dk = beta[f][:, None] * (R @ X[f].T - U @ P.T)
            np.testing.assert_allclose(got[1][0, h, sl], dk, rtol=1e-11, atol=1e-13)
            np.testing.assert_allclose(got[4][0, h, f], np.sum(((I - G[f]) @ X[f]) * P), rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(got[5][0, h], dh0, rtol=1e-11, atol=1e-13)
