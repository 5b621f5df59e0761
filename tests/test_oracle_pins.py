"""Pins of the fp64 oracle against what the method and the mathematics fix.

Each test checks the oracle against something other than itself: a closed
form, an invariant, a special case that reduces to a textbook computation, a
hand-worked example (``tests/golden``) or a different algorithm (the
chunkwise WY form) by brute force.  No GPU is needed.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import chunkwise_ref
from chunkwise_gated_delta_gdn_amd import inputs as synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _f32(x):
    return np.asarray(x, np.float32)


def _orthonormal_rows(rng, n, count):
    """``count`` mutually orthogonal unit vectors of length n = 16, exact in
    float32: rows of the Sylvester Hadamard matrix over 4, with random signs."""
    assert n == 16
    Hm = np.array([[1.0]])
    while Hm.shape[0] < n:
        Hm = np.block([[Hm, Hm], [Hm, -Hm]])
    rows = Hm[rng.permutation(n)[:count]] / 4.0
    return rows * rng.choice([-1.0, 1.0], size=(count, 1))


# --------------------------------------------------------------------------
# O1: gated delta rule token recurrence
# --------------------------------------------------------------------------

def test_gdn_hand_worked_example():
    fx = json.load(open(os.path.join(GOLDEN, "gdn_hand_d2.json")))
    inp = fx["inputs"]
    T = len(inp["beta"])
    q = _f32(inp["q"]).reshape(1, T, 1, 2)
    k = _f32(inp["k"]).reshape(1, T, 1, 2)
    v = _f32(inp["v"]).reshape(1, T, 1, 2)
    beta = _f32(inp["beta"]).reshape(1, T, 1)
    g = _f32(np.log(inp["decay"])).reshape(1, T, 1)
    o, hT = oracle.gdn_recurrent(q, k, v, beta, g, inp["scale"])
    np.testing.assert_allclose(o[0, :, 0], fx["expected"]["o"], atol=1e-6)
    np.testing.assert_allclose(hT[0, 0], fx["expected"]["hT"], atol=1e-6)


def test_gdn_beta_zero_is_pure_decayed_carry():
    B, T, H, Dk, Dv = 2, 37, 3, 8, 5
    d = synth.gdn_inputs(B, T, H, Dk, Dv, seed=1, dtype="f32", h0_std=0.5)
    beta = np.zeros((B, T, H), np.float32)
    o, hT = oracle.gdn_recurrent(d["q"], d["k"], d["v"], beta, d["g"], 0.75, d["h0"])
    Gc = np.cumsum(d["g"].astype(np.float64), axis=1)           # (B,T,H)
    h0 = d["h0"].astype(np.float64)
    ref = 0.75 * np.exp(Gc)[..., None] * np.einsum("bthk,bhkv->bthv", d["q"].astype(np.float64), h0)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(hT, np.exp(Gc[:, -1])[..., None, None] * h0, rtol=1e-12, atol=1e-14)


def test_gdn_delta_rule_overwrites_unit_key():
    # gamma = 0, beta = 1, ||k|| = 1: after token t the state maps k_t to v_t
    # exactly (S_t^T k_t = v_t), whatever the earlier state was.
    B, T, H, D = 1, 20, 2, 6
    d = synth.gdn_inputs(B, T, H, D, D, seed=2, dtype="f32", h0_std=1.0)
    g = np.zeros((B, T, H), np.float32)
    beta = np.ones((B, T, H), np.float32)
    k = d["k"] / np.linalg.norm(d["k"].astype(np.float64), axis=-1, keepdims=True)
    k = _f32(k)
    o, _ = oracle.gdn_recurrent(k, k, d["v"], beta, g, 1.0, d["h0"])  # q = k
    np.testing.assert_allclose(o, d["v"], atol=2e-6)


def test_gdn_orthonormal_keys_reduce_to_decayed_linear_attention():
    # Mutually orthogonal unit keys and h0 = 0: the prediction p = P^T k_t is
    # always zero, so o_t = sum_{s<=t} exp(G_t - G_s) beta_s (q_t . k_s) v_s.
    B, T, H, Dk, Dv = 1, 12, 2, 16, 7
    rng = _rng(3)
    k = _f32(np.stack([_orthonormal_rows(rng, Dk, T) for _ in range(H)], axis=1)[None])  # (1,T,H,Dk)
    q = _f32(rng.standard_normal((B, T, H, Dk)))
    v = _f32(rng.standard_normal((B, T, H, Dv)))
    beta = _f32(rng.uniform(0.1, 1.0, (B, T, H)))
    g = _f32(-rng.uniform(0.0, 0.5, (B, T, H)))
    o, _ = oracle.gdn_recurrent(q, k, v, beta, g, 1.0)
    k64, q64, v64 = (x.astype(np.float64) for x in (k, q, v))
    G = np.cumsum(g.astype(np.float64), axis=1)
    ref = np.zeros_like(o)
    for h in range(H):
        Gh = G[0, :, h]
        Dm = np.tril(np.exp(Gh[:, None] - Gh[None, :]))
        A = Dm * (q64[0, :, h] @ k64[0, :, h].T) * beta[0, :, h][None, :].astype(np.float64)
        ref[0, :, h] = A @ v64[0, :, h]
    np.testing.assert_allclose(o, ref, rtol=1e-10, atol=1e-12)


def test_gdn_householder_beta_two_preserves_state_norm():
    # gamma = 0, beta = 2, ||k|| = 1, v = 0: each step applies the reflection
    # I - 2 k k^T, an orthogonal map, so ||S||_F never changes.
    B, T, H, D = 1, 30, 2, 16
    d = synth.gdn_inputs(B, T, H, D, D, seed=4, dtype="f32", h0_std=1.0)
    rng = _rng(4)
    k = _f32(np.stack([_orthonormal_rows(rng, D, 1)[0] for _ in range(B * T * H)]).reshape(B, T, H, D))
    o, hT = oracle.gdn_recurrent(d["q"], k, np.zeros_like(d["v"]), np.full((B, T, H), 2, np.float32),
                                 np.zeros((B, T, H), np.float32), 1.0, d["h0"])
    n0 = np.linalg.norm(d["h0"].astype(np.float64), axis=(-2, -1))
    np.testing.assert_allclose(np.linalg.norm(hT, axis=(-2, -1)), n0, rtol=1e-12)
    # and the state really moved (it is not the identity map)
    assert np.abs(hT - d["h0"]).max() > 1e-2


def test_gdn_split_and_resume_matches_one_pass():
    B, T, H, Dk, Dv = 2, 50, 2, 8, 4
    d = synth.gdn_inputs(B, T, H, Dk, Dv, seed=5, dtype="f32", h0_std=0.3)
    o, hT = oracle.gdn_recurrent(d["q"], d["k"], d["v"], d["beta"], d["g"], 0.5, d["h0"])
    T1 = 23
    s = lambda x, a, b: np.ascontiguousarray(x[:, a:b])
    o1, h1 = oracle.gdn_recurrent(s(d["q"], 0, T1), s(d["k"], 0, T1), s(d["v"], 0, T1),
                                  s(d["beta"], 0, T1), s(d["g"], 0, T1), 0.5, d["h0"])
    o2, h2 = oracle.gdn_recurrent(s(d["q"], T1, T), s(d["k"], T1, T), s(d["v"], T1, T),
                                  s(d["beta"], T1, T), s(d["g"], T1, T), 0.5, _f32(h1))
    # h1 goes through float32 on the way back in: compare at that precision
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), o, atol=1e-6)
    np.testing.assert_allclose(h2, hT, atol=1e-6)


def test_gdn_scale_is_linear():
    d = synth.gdn_inputs(1, 19, 2, 8, 8, seed=6, dtype="f32")
    o1, h1 = oracle.gdn_recurrent(d["q"], d["k"], d["v"], d["beta"], d["g"], 1.0)
    o2, h2 = oracle.gdn_recurrent(d["q"], d["k"], d["v"], d["beta"], d["g"], 0.125)
    np.testing.assert_allclose(o2, 0.125 * o1, rtol=1e-14)
    np.testing.assert_array_equal(h1, h2)


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("T", [1, 15, 16, 17, 33, 64, 70])
def test_gdn_chunkwise_form_equals_recurrence(chunk, T):
    d = synth.gdn_inputs(1, T, 2, 16, 8, seed=100 + T, dtype="f32", h0_std=0.2)
    o, hT = oracle.gdn_recurrent(d["q"], d["k"], d["v"], d["beta"], d["g"], 0.3, d["h0"])
    o2, h2 = chunkwise_ref.chunkwise_forward(d["q"], d["k"], d["v"], d["beta"][..., None], d["g"],
                                             np.ones((1, 1)), chunk, 0.3, d["h0"])
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(h2, hT, atol=1e-12)


def test_unit_lower_inverse_blocked_matches_library_inverse():
    # Pins the block merge (including the T_22 / T_33 terms of a 64x64 merge).
    rng = _rng(7)
    for n in (16, 31, 48, 64):
        A = np.tril(rng.standard_normal((n, n)) * 0.3, -1)
        M = np.eye(n) + A
        Tm = chunkwise_ref.unit_lower_inverse_blocked(M, 16)
        np.testing.assert_allclose(Tm, np.linalg.inv(M), atol=1e-10)
        np.testing.assert_allclose(M @ Tm, np.eye(n), atol=1e-10)


# --------------------------------------------------------------------------
# O2: gated DeltaProduct token recurrence
# --------------------------------------------------------------------------

def test_deltaproduct_r1_equals_gdn():
    d = synth.gdn_inputs(2, 29, 2, 8, 6, seed=8, dtype="f32", h0_std=0.4)
    o, hT = oracle.gdn_recurrent(d["q"], d["k"], d["v"], d["beta"], d["g"], 0.6, d["h0"])
    o2, h2 = oracle.deltaproduct_recurrent(d["q"], d["k"], d["v"], d["beta"][..., None], d["g"],
                                           np.ones((1, 1)), 0.6, d["h0"])
    np.testing.assert_allclose(o2, o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(h2, hT, rtol=1e-13, atol=1e-14)


def test_deltaproduct_identity_mask_is_independent_sub_blocks():
    # M = I: step a erases and writes only in row block a, so the state is r
    # independent GDN states on the sub-keys; the read-out sums them.
    B, T, H, r, dk, Dv = 1, 25, 2, 2, 8, 6
    d = synth.deltaproduct_inputs(B, T, H, r, dk, Dv, seed=9, dtype="f32", h0_std=0.3,
                                  mask=np.eye(r))
    o, hT = oracle.deltaproduct_recurrent(d["q"], d["k"], d["v"], d["beta"], d["g"], d["mask"],
                                          1.0, d["h0"])
    osum = np.zeros_like(o)
    for a in range(r):
        sl = slice(a * dk, (a + 1) * dk)
        oa, ha = oracle.gdn_recurrent(np.ascontiguousarray(d["q"][..., sl]),
                                      np.ascontiguousarray(d["k"][..., sl]), d["v"],
                                      np.ascontiguousarray(d["beta"][..., a]), d["g"], 1.0,
                                      np.ascontiguousarray(d["h0"][:, :, sl]))
        osum += oa
        np.testing.assert_allclose(hT[:, :, sl], ha, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(o, osum, rtol=1e-12, atol=1e-13)


def test_deltaproduct_all_ones_mask_equal_betas_is_gdn_on_full_key():
    # M = ones and beta_{t,a} = beta_t: every step erases along the full key
    # and the writes add up to beta_t k_t (v_t - P^T k_t)^T: GDN with K = r*dk.
    B, T, H, r, dk, Dv = 1, 31, 2, 2, 8, 5
    d = synth.deltaproduct_inputs(B, T, H, r, dk, Dv, seed=10, dtype="f32", h0_std=0.3,
                                  mask=np.ones((r, r)))
    beta1 = d["beta"][..., 0]
    beta = np.ascontiguousarray(np.repeat(beta1[..., None], r, axis=-1))
    o, hT = oracle.deltaproduct_recurrent(d["q"], d["k"], d["v"], beta, d["g"], d["mask"], 0.5, d["h0"])
    o2, h2 = oracle.gdn_recurrent(d["q"], d["k"], d["v"], np.ascontiguousarray(beta1), d["g"], 0.5, d["h0"])
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(hT, h2, rtol=1e-12, atol=1e-13)


def test_deltaproduct_mask_orientation_closed_form():
    # M = [[0,0],[1,0]]: step 0 erases along nothing and writes k_0 v^T into
    # block 0; step 1 erases along sub-key 0 (block 0 of the gated state) and
    # writes into block 1.  Closed form with h0 = 0, D_ts = exp(G_t - G_s):
    #   p1_t = sum_{s<t} D_ts beta_{s,0} (k_{s,0} . k_{t,0}) v_s,  u_t = v_t - p1_t
    #   o_t  = sum_{s<=t} D_ts [beta_{s,0} (q_{t,0}.k_{s,0}) v_s + beta_{s,1} (q_{t,1}.k_{s,1}) u_s]
    # Reading the mask transposed would erase step 0 along sub-key 1 instead.
    B, T, H, r, dk, Dv = 1, 21, 1, 2, 6, 4
    M = np.array([[0.0, 0.0], [1.0, 0.0]])
    d = synth.deltaproduct_inputs(B, T, H, r, dk, Dv, seed=11, dtype="f32", mask=M)
    o, _ = oracle.deltaproduct_recurrent(d["q"], d["k"], d["v"], d["beta"], d["g"], M, 1.0)
    q, k, v, beta = (x[0, :, 0].astype(np.float64) for x in (d["q"], d["k"], d["v"], d["beta"]))
    G = np.cumsum(d["g"][0, :, 0].astype(np.float64))
    Dm = np.exp(G[:, None] - G[None, :])
    incl = np.tril(np.ones((T, T)))
    strict = np.tril(np.ones((T, T)), -1)
    k0, k1, q0, q1 = k[:, :dk], k[:, dk:], q[:, :dk], q[:, dk:]
    p1 = (strict * Dm * (k0 @ k0.T) * beta[None, :, 0]) @ v
    u = v - p1
    ref = (incl * Dm * (q0 @ k0.T) * beta[None, :, 0]) @ v + (incl * Dm * (q1 @ k1.T) * beta[None, :, 1]) @ u
    np.testing.assert_allclose(o[0, :, 0], ref, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("chunk", [16, 32])
@pytest.mark.parametrize("T", [1, 9, 16, 40])
def test_deltaproduct_chunkwise_form_equals_recurrence(chunk, T):
    rng = _rng(200 + T)
    M = np.tril(rng.uniform(-1, 1, (2, 2)))
    d = synth.deltaproduct_inputs(1, T, 2, 2, 8, 6, seed=300 + T, dtype="f32", h0_std=0.2, mask=M)
    o, hT = oracle.deltaproduct_recurrent(d["q"], d["k"], d["v"], d["beta"], d["g"], d["mask"], 0.4, d["h0"])
    o2, h2 = chunkwise_ref.chunkwise_forward(d["q"], d["k"], d["v"], d["beta"], d["g"], d["mask"],
                                             chunk, 0.4, d["h0"])
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(h2, hT, atol=1e-12)


# --------------------------------------------------------------------------
# O3: camera prep
# --------------------------------------------------------------------------

def test_cam_prep_hand_worked_example():
    fx = json.load(open(os.path.join(GOLDEN, "cam_prep_hand_d8.json")))
    i = fx["inputs"]
    qkv = _f32([i["q"], i["k"], i["v"]]).reshape(1, 1, 3, 1, 8)
    out = oracle.cam_prep(qkv, None, None, _f32(i["proj_q"]).reshape(1, 1, 4, 4),
                          _f32(i["proj_kv"]).reshape(1, 1, 4, 4), _f32(i["rope_cos"]).reshape(1, 4),
                          _f32(i["rope_sin"]).reshape(1, 4), i["k_scale"], i["eps"])
    e = fx["expected"]
    for name in ("q", "k", "v"):
        np.testing.assert_allclose(out[name][0, 0, 0], e[name], atol=1e-12)
    for name in ("k_pre_sq", "k_post_sq", "inflation_sq"):
        np.testing.assert_allclose(out[name][0, 0, 0], e[name], rtol=1e-12)


def test_cam_prep_hand_worked_norm_weights():
    """The per-channel RMSNorm weight path: weights indexed over all H*D
    channels, applied before the ReLU and before the projection."""
    fx = json.load(open(os.path.join(GOLDEN, "cam_prep_hand_weights_h2d8.json")))
    i = fx["inputs"]
    H, D = i["H"], i["D"]
    qkv = _f32([i["q"], i["k"], i["v"]]).reshape(1, 1, 3, H, D)
    out = oracle.cam_prep(qkv, _f32(i["q_norm_w"]), _f32(i["k_norm_w"]), _f32(i["proj_q"]).reshape(1, 1, 4, 4),
                          _f32(i["proj_kv"]).reshape(1, 1, 4, 4), _f32(i["rope_cos"]).reshape(1, D // 2),
                          _f32(i["rope_sin"]).reshape(1, D // 2), i["k_scale"], i["eps"])
    e = fx["expected"]
    for name in ("q", "k", "v"):
        np.testing.assert_allclose(out[name][0, :, 0], e[name], atol=1e-12, err_msg=name)
    for name in ("k_pre_sq", "k_post_sq", "inflation_sq"):
        np.testing.assert_allclose(out[name][0, :, 0], e[name], rtol=1e-12, err_msg=name)


def test_se3_inverse_round_trips():
    d = synth.camera_inputs(1, 2, 5, 1, 8, seed=12, dtype="f32")
    P = d["P"].astype(np.float64)
    Pi = oracle.invert_se3(P)
    eye = np.broadcast_to(np.eye(4), P.shape)
    np.testing.assert_allclose(Pi @ P, eye, atol=1e-12)
    np.testing.assert_allclose(P @ Pi, eye, atol=1e-12)
    np.testing.assert_allclose(oracle.invert_se3(Pi), P, atol=1e-12)
    np.testing.assert_allclose(Pi, np.linalg.inv(P), atol=1e-12)
    R = P[..., :3, :3]
    np.testing.assert_allclose(np.swapaxes(R, -1, -2) @ R, np.broadcast_to(np.eye(3), R.shape), atol=1e-12)
    np.testing.assert_allclose(np.linalg.det(R), 1.0, atol=1e-12)


def _identity_prep_tables(N, D, B=1):
    eye = np.broadcast_to(np.eye(4, dtype=np.float32), (B, N, 4, 4)).copy()
    return eye, np.ones((N, D // 2), np.float32), np.zeros((N, D // 2), np.float32)


def test_cam_prep_rmsnorm_over_all_channels():
    # Identity projection and RoPE, positive inputs (ReLU inactive), w = 1:
    # per token, sum_c q_out_c^2 / C = ms / (ms + eps) over all H*D channels,
    # and q_out is proportional to q_in with one factor for all heads.
    B, N, H, D = 1, 7, 3, 16
    rng = _rng(13)
    qkv = _f32(np.abs(rng.standard_normal((B, N, 3, H, D))) + 0.01)
    eye, cs, sn = _identity_prep_tables(N, D, B)
    eps = 1e-3
    out = oracle.cam_prep(qkv, None, None, eye, eye, cs, sn, 0.25, eps)
    x = qkv.astype(np.float64)
    C = H * D
    for slot, name, sc in ((0, "q", 1.0), (1, "k", 0.25)):
        ms = (x[:, :, slot] ** 2).sum(axis=(-1, -2)) / C                      # (B,N)
        y = np.transpose(out[name], (0, 2, 1, 3)) / sc                           # (B,N,H,D)
        np.testing.assert_allclose((y ** 2).sum(axis=(-1, -2)) / C, ms / (ms + eps), rtol=1e-12)
        ratio = y / x[:, :, slot]
        np.testing.assert_allclose(ratio, np.broadcast_to(ratio[..., :1, :1], ratio.shape), rtol=1e-12)
    np.testing.assert_allclose(np.transpose(out["v"], (0, 2, 1, 3)), x[:, :, 2], rtol=0, atol=0)
    np.testing.assert_allclose(out["k_pre_sq"], out["k_post_sq"], rtol=1e-12)
    np.testing.assert_allclose(out["inflation_sq"], 1.0, rtol=1e-12)


def test_cam_prep_relu_zeroes_negative_q_k_only():
    B, N, H, D = 1, 5, 2, 16
    rng = _rng(14)
    qkv = _f32(rng.standard_normal((B, N, 3, H, D)))
    eye, cs, sn = _identity_prep_tables(N, D, B)
    out = oracle.cam_prep(qkv, None, None, eye, eye, cs, sn, 0.125, 1e-6)
    neg = np.transpose(qkv, (0, 2, 3, 1, 4)) < 0                              # (B,3,H,N,D)
    assert np.all(out["q"][neg[:, 0]] == 0) and np.all(out["k"][neg[:, 1]] == 0)
    assert np.all(out["q"][~neg[:, 0]] > 0) and np.all(out["k"][~neg[:, 1]] > 0)
    np.testing.assert_array_equal(out["v"], np.transpose(qkv[:, :, 2], (0, 2, 1, 3)))


def test_cam_prep_rope_is_complex_rotation():
    # Second half: (y_2i + i y_2i+1) = (x_2i + i x_2i+1) * exp(i n theta_i)
    # for the tables of the workload, on v (no norm in the way).
    B, N, H, D = 1, 40, 2, 32
    rng = _rng(15)
    qkv = _f32(rng.standard_normal((B, N, 3, H, D)))
    eye = np.broadcast_to(np.eye(4, dtype=np.float32), (B, N, 4, 4)).copy()
    cs, sn = synth.rope_tables(N, D // 2)
    out = oracle.cam_prep(qkv, None, None, eye, eye, cs, sn, 1.0, 1e-6)
    x = qkv[0, :, 2, :, D // 2:].astype(np.float64)                            # (N,H,D/2)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    ang = np.arctan2(sn[:, 1::2].astype(np.float64), cs[:, 0::2].astype(np.float64))  # (N, D/4)
    rad = np.hypot(sn[:, 1::2].astype(np.float64), cs[:, 0::2].astype(np.float64))
    w = z * (rad * np.exp(1j * ang))[:, None, :]
    y = np.transpose(out["v"][0], (1, 0, 2))[..., D // 2:]                   # (N,H,D/2)
    np.testing.assert_allclose(y[..., 0::2], w.real, atol=1e-12)
    np.testing.assert_allclose(y[..., 1::2], w.imag, atol=1e-12)
    # n = 0 is the identity, and every pair keeps its norm (to the table's rounding)
    np.testing.assert_allclose(y[0], x[0], atol=0)
    np.testing.assert_allclose(np.hypot(y[..., 0::2], y[..., 1::2]), np.abs(z), rtol=1e-6)


def test_cam_prep_ucpe_permutation_and_rigid_invariance():
    B, N, H, D = 1, 6, 2, 16
    rng = _rng(16)
    qkv = _f32(np.abs(rng.standard_normal((B, N, 3, H, D))) + 0.01)
    perm = np.stack([np.eye(4)[rng.permutation(4)] for _ in range(N)])[None].astype(np.float32)
    _, cs, sn = _identity_prep_tables(N, D, B)
    out = oracle.cam_prep(qkv, None, None, perm, perm, cs, sn, 1.0, 1e-6)
    # v first half: y[4g+i] = x[4g + pi(i)] where perm[i, pi(i)] = 1
    pi = perm[0].argmax(axis=-1)                                            # (N,4)
    x = qkv[0, :, 2, :, :D // 2].reshape(N, H, D // 8, 4)
    y = np.transpose(out["v"][0], (1, 0, 2))[..., :D // 2].reshape(N, H, D // 8, 4)
    np.testing.assert_array_equal(y, np.take_along_axis(x, pi[:, None, None, :].repeat(H, 1).repeat(D // 8, 2), -1))
    # a rotation about the origin (t = 0) keeps ||k||: inflation is one
    d = synth.camera_inputs(B, 1, N, H, D, seed=17, dtype="f32")
    Pr = d["P"].copy()
    Pr[..., :3, 3] = 0.0
    Pinv = oracle.invert_se3(Pr).astype(np.float32)
    out = oracle.cam_prep(d["qkv"], None, None, np.swapaxes(Pr, -1, -2).astype(np.float32).copy(), Pinv,
                          d["rope_cos"], d["rope_sin"], 0.125, 1e-6)
    np.testing.assert_allclose(out["inflation_sq"], 1.0, rtol=1e-6)


def test_cam_prep_inflation_clamps_zero_key():
    B, N, H, D = 1, 3, 1, 8
    qkv = np.ones((B, N, 3, H, D), np.float32)
    qkv[:, :, 1] = -1.0                                                     # relu kills all of k
    eye, cs, sn = _identity_prep_tables(N, D, B)
    out = oracle.cam_prep(qkv, None, None, eye, eye, cs, sn, 0.125, 1e-6)
    assert np.all(out["k"] == 0) and np.all(out["k_pre_sq"] == 0)
    np.testing.assert_array_equal(out["inflation_sq"], 1.0)


# --------------------------------------------------------------------------
# O4: frame-synchronous camera scan
# --------------------------------------------------------------------------

def _bhnd(x):
    return np.ascontiguousarray(np.transpose(x, (0, 2, 1, 3)))


def test_frame_scan_one_token_per_frame_is_gdn():
    B, T, H, D = 1, 33, 2, 8
    d = synth.gdn_inputs(B, T, H, D, D, seed=18, dtype="f32", h0_std=0.3)
    o, hT = oracle.gdn_recurrent(d["q"], d["k"], d["v"], d["beta"], d["g"], 1.0, d["h0"])
    out, hT2 = oracle.frame_scan(_bhnd(d["q"]), _bhnd(d["k"]), _bhnd(d["v"]),
                                 np.ascontiguousarray(d["beta"].transpose(0, 2, 1)),
                                 np.ascontiguousarray(d["g"].transpose(0, 2, 1)), T, 1.0, d["h0"])
    np.testing.assert_allclose(out, _bhnd(o), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(hT2, hT, rtol=1e-13, atol=1e-14)


def test_frame_scan_matches_matrix_form():
    # S_f = (I - sum_s beta_s k_s k_s^T) (d_f S_{f-1}) + sum_s beta_s k_s v_s^T
    B, H, F, S, D = 1, 2, 5, 7, 6
    rng = _rng(19)
    q, k, v = (_f32(rng.standard_normal((B, H, F * S, D)) * 0.4) for _ in range(3))
    beta = _f32(rng.uniform(0, 1, (B, H, F * S)))
    g = _f32(-rng.uniform(0, 1, (B, H, F)))
    h0 = _f32(rng.standard_normal((B, H, D, D)))
    out, hT = oracle.frame_scan(q, k, v, beta, g, F, 0.9, h0)
    for h in range(H):
        St = h0[0, h].astype(np.float64)
        for f in range(F):
            sl = slice(f * S, (f + 1) * S)
            kk, vv, bb = (x[0, h, sl].astype(np.float64) for x in (k, v, beta))
            Gm = (kk * bb[:, None]).T @ kk
            Hm = (kk * bb[:, None]).T @ vv
            St = (np.eye(D) - Gm) @ (np.exp(float(g[0, h, f])) * St) + Hm
            np.testing.assert_allclose(out[0, h, sl], 0.9 * q[0, h, sl].astype(np.float64) @ St, atol=1e-12)
        np.testing.assert_allclose(hT[0, h], St, atol=1e-12)


def test_frame_scan_beta_zero_is_pure_decayed_carry():
    B, H, F, S, D = 1, 2, 4, 3, 5
    rng = _rng(20)
    q, k, v = (_f32(rng.standard_normal((B, H, F * S, D))) for _ in range(3))
    g = _f32(-rng.uniform(0, 1, (B, H, F)))
    h0 = _f32(rng.standard_normal((B, H, D, D)))
    out, hT = oracle.frame_scan(q, k, v, np.zeros((B, H, F * S), np.float32), g, F, 1.0, h0)
    Gc = np.cumsum(g.astype(np.float64), axis=-1)
    fr = np.repeat(Gc, S, axis=-1)                                           # (B,H,N)
    ref = np.exp(fr)[..., None] * np.einsum("bhnk,bhkv->bhnv", q.astype(np.float64), h0.astype(np.float64))
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(hT, np.exp(Gc[..., -1])[..., None, None] * h0, rtol=1e-12)


def test_frame_scan_orthogonal_keys_in_frame_match_token_order():
    # Keys that are mutually orthogonal within a frame do not see each other's
    # writes, so the frame-synchronous update equals the token-sequential one
    # (gate on the first token of each frame, none on the others).
    B, H, F, S, D = 1, 1, 3, 5, 16
    rng = _rng(21)
    k = _f32(np.concatenate([_orthonormal_rows(rng, D, S) for _ in range(F)])[None, None])
    q = _f32(rng.standard_normal((B, H, F * S, D)))
    v = _f32(rng.standard_normal((B, H, F * S, D)))
    beta = _f32(rng.uniform(0.2, 1, (B, H, F * S)))
    g = _f32(-rng.uniform(0, 0.5, (B, H, F)))
    h0 = _f32(rng.standard_normal((B, H, D, D)) * 0.3)
    out, hT = oracle.frame_scan(q, k, v, beta, g, F, 1.0, h0)
    gt = np.zeros((B, H, F * S), np.float32)
    gt[..., ::S] = g
    tr = lambda x: np.ascontiguousarray(np.transpose(x, (0, 2, 1, 3)))
    o_tok, hT_tok = oracle.gdn_recurrent(tr(q), tr(k), tr(v), np.ascontiguousarray(beta.transpose(0, 2, 1)),
                                         np.ascontiguousarray(gt.transpose(0, 2, 1)), 1.0, h0)
    np.testing.assert_allclose(hT, hT_tok, atol=1e-12)
    last = np.arange(S - 1, F * S, S)
    np.testing.assert_allclose(out[:, :, last], tr(o_tok)[:, :, last], atol=1e-12)


def test_frame_scan_split_and_resume():
    B, H, F, S, D = 1, 2, 6, 5, 4
    rng = _rng(22)
    q, k, v = (_f32(rng.standard_normal((B, H, F * S, D)) * 0.5) for _ in range(3))
    beta = _f32(rng.uniform(0, 1, (B, H, F * S)))
    g = _f32(-rng.uniform(0, 1, (B, H, F)))
    out, hT = oracle.frame_scan(q, k, v, beta, g, F, 1.0)
    F1 = 2
    a = lambda x, lo, hi: np.ascontiguousarray(x[:, :, lo * S:hi * S])
    o1, h1 = oracle.frame_scan(a(q, 0, F1), a(k, 0, F1), a(v, 0, F1), np.ascontiguousarray(beta[..., :F1 * S]),
                               np.ascontiguousarray(g[..., :F1]), F1, 1.0)
    o2, h2 = oracle.frame_scan(a(q, F1, F), a(k, F1, F), a(v, F1, F), np.ascontiguousarray(beta[..., F1 * S:]),
                               np.ascontiguousarray(g[..., F1:]), F - F1, 1.0, _f32(h1))
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=2), out, atol=1e-6)
    np.testing.assert_allclose(h2, hT, atol=1e-6)


# --------------------------------------------------------------------------
# O4 reverse ([cam] REVERSE branch / flip-and-shift reference of cam_scan_func)
# --------------------------------------------------------------------------

def _frame_GH(k, v, beta, F, S):
    """G_j = sum beta k k^T, H_j = sum beta k v^T per frame, fp64 (one (b, h))."""
    k, v, beta = (x.astype(np.float64) for x in (k, v, beta))
    G = np.stack([(k[j * S:(j + 1) * S] * beta[j * S:(j + 1) * S, None]).T @ k[j * S:(j + 1) * S] for j in range(F)])
    Hm = np.stack([(k[j * S:(j + 1) * S] * beta[j * S:(j + 1) * S, None]).T @ v[j * S:(j + 1) * S] for j in range(F)])
    return G, Hm


def test_frame_scan_reverse_is_the_unrolled_future_sum():
    # R_f = sum_{j > f} (A_{f+1} ... A_{j-1}) H_j with A_m = e^{g_m} (I - G_m):
    # only later frames enter, each frame's own gate applies to the state
    # before that frame's keys and values are folded in.
    B, H, F, S, D = 1, 2, 5, 3, 4
    rng = _rng(31)
    q, k, v = (_f32(rng.standard_normal((B, H, F * S, D)) * 0.6) for _ in range(3))
    beta = _f32(rng.uniform(0, 1, (B, H, F * S)))
    g = _f32(-rng.uniform(0.05, 1, (B, H, F)))
    out = oracle.frame_scan_reverse(q, k, v, beta, g, F, 0.7)
    for h in range(H):
        G, Hm = _frame_GH(k[0, h], v[0, h], beta[0, h], F, S)
        A = [np.exp(np.float64(g[0, h, m])) * (np.eye(D) - G[m]) for m in range(F)]
        for f in range(F):
            R = np.zeros((D, D))
            P = np.eye(D)
            for j in range(f + 1, F):
                R += P @ Hm[j]
                P = P @ A[j]
            ref = 0.7 * q[0, h, f * S:(f + 1) * S].astype(np.float64) @ R
            np.testing.assert_allclose(out[0, h, f * S:(f + 1) * S], ref, atol=1e-12)


def test_frame_scan_reverse_edge_frames():
    B, H, F, S, D = 1, 1, 4, 6, 8
    rng = _rng(32)
    q, k, v = (_f32(rng.standard_normal((B, H, F * S, D))) for _ in range(3))
    beta = _f32(rng.uniform(0, 1, (B, H, F * S)))
    g = _f32(-rng.uniform(0, 1, (B, H, F)))
    out = oracle.frame_scan_reverse(q, k, v, beta, g, F, 1.0)
    # the last frame has no future: exactly zero
    assert np.all(out[0, 0, (F - 1) * S:] == 0.0)
    # the frame before it sees only the last frame, from a zero state: plain
    # linear attention onto that frame, sum_s beta_s (q . k_s) v_s
    qf = q[0, 0, (F - 2) * S:(F - 1) * S].astype(np.float64)
    kl, vl = (x[0, 0, (F - 1) * S:].astype(np.float64) for x in (k, v))
    bl = beta[0, 0, (F - 1) * S:].astype(np.float64)
    np.testing.assert_allclose(out[0, 0, (F - 2) * S:(F - 1) * S], (qf @ kl.T * bl) @ vl, atol=1e-12)
    # one frame only: nothing to read
    o1 = oracle.frame_scan_reverse(q[..., :S, :], k[..., :S, :], v[..., :S, :], beta[..., :S], g[..., :1], 1, 1.0)
    assert np.all(o1 == 0.0)
    # beta = 0: nothing is written, nothing is read
    o0 = oracle.frame_scan_reverse(q, k, v, np.zeros_like(beta), g, F, 1.0)
    assert np.all(o0 == 0.0)


def test_frame_scan_reverse_mirrors_the_forward_scan():
    # Reversing the frame order of the inputs turns the reverse scan into the
    # forward scan with an exclusive read-out: frame f of the reverse scan of
    # the reversed sequence reads the forward state after frame f - 1 of the
    # original (gates shifted by one frame).
    B, H, F, S, D = 1, 1, 5, 4, 6
    rng = _rng(33)
    q, k, v = (_f32(rng.standard_normal((B, H, F * S, D)) * 0.5) for _ in range(3))
    beta = _f32(rng.uniform(0, 1, (B, H, F * S)))
    g = _f32(-rng.uniform(0, 1, (B, H, F)))
    rf = lambda x: np.ascontiguousarray(np.flip(x.reshape(B, H, F, S, -1), axis=2).reshape(x.shape))
    out_r = oracle.frame_scan_reverse(rf(q), rf(k), rf(v), rf(beta[..., None])[..., 0], np.ascontiguousarray(g[..., ::-1]), F, 1.0)
    out_r = rf(out_r)
    # forward states S_f of the original order, in fp64 from G, H directly
    G, Hm = _frame_GH(k[0, 0], v[0, 0], beta[0, 0], F, S)
    St = np.zeros((D, D))
    for f in range(F):
        ref = q[0, 0, f * S:(f + 1) * S].astype(np.float64) @ St      # reads the state before frame f
        np.testing.assert_allclose(out_r[0, 0, f * S:(f + 1) * S], ref, atol=1e-12)
        St = np.exp(np.float64(g[0, 0, f])) * (np.eye(D) - G[f]) @ St + Hm[f]


# --------------------------------------------------------------------------
# normaliser (Z) stream ([cp] module docstring)
# --------------------------------------------------------------------------

def test_frame_den_follows_the_vector_recurrence():
    # the page's Z recurrence written out for the vector state, in fp64
    B, H, F, S, D = 1, 2, 4, 5, 6
    rng = _rng(41)
    q, k = (_f32(rng.standard_normal((B, H, F * S, D)) * 0.5) for _ in range(2))
    beta = _f32(rng.uniform(0, 1, (B, H, F * S)))
    g = _f32(-rng.uniform(0, 1, (B, H, F)))
    z0 = _f32(rng.standard_normal((B, H, D)))
    den, zT = oracle.frame_den(q, k, beta, g, F, 0.6, z0)
    for h in range(H):
        z = z0[0, h].astype(np.float64)
        for f in range(F):
            sl = slice(f * S, (f + 1) * S)
            kf, bf = k[0, h, sl].astype(np.float64), beta[0, h, sl].astype(np.float64)
            P = (kf * bf[:, None]).T @ kf
            z = np.exp(np.float64(g[0, h, f])) * (np.eye(D) - P) @ z + kf.T @ bf
            np.testing.assert_allclose(den[0, h, sl], 0.6 * q[0, h, sl].astype(np.float64) @ z, atol=1e-12)
        np.testing.assert_allclose(zT[0, h], z, atol=1e-12)


def test_frame_den_closed_forms():
    B, H, F, S, D = 1, 1, 3, 7, 8
    rng = _rng(42)
    q, k = (_f32(rng.standard_normal((B, H, F * S, D))) for _ in range(2))
    beta = _f32(rng.uniform(0, 1, (B, H, F * S)))
    g = _f32(-rng.uniform(0, 1, (B, H, F)))
    # one frame from zero: den = q . sum_s beta_s k_s
    d1, _ = oracle.frame_den(q[..., :S, :], k[..., :S, :], beta[..., :S], g[..., :1], 1, 1.0)
    ref = q[0, 0, :S].astype(np.float64) @ (k[0, 0, :S].astype(np.float64).T @ beta[0, 0, :S].astype(np.float64))
    np.testing.assert_allclose(d1[0, 0], ref, atol=1e-12)
    # beta = 0: the decayed initial state only
    z0 = _f32(rng.standard_normal((B, H, D)))
    d0, zT = oracle.frame_den(q, k, np.zeros_like(beta), g, F, 1.0, z0)
    decay = np.exp(np.cumsum(g[0, 0].astype(np.float64)))
    for f in range(F):
        ref = decay[f] * (q[0, 0, f * S:(f + 1) * S].astype(np.float64) @ z0[0, 0].astype(np.float64))
        np.testing.assert_allclose(d0[0, 0, f * S:(f + 1) * S], ref, atol=1e-12)
    np.testing.assert_allclose(zT[0, 0], decay[-1] * z0[0, 0], atol=1e-12)
    # reverse: the last frame reads nothing; the one before reads b of the last frame
    dr, _ = oracle.frame_den(q, k, beta, g, F, 1.0, reverse=True)
    assert np.all(dr[0, 0, (F - 1) * S:] == 0.0)
    bl = k[0, 0, (F - 1) * S:].astype(np.float64).T @ beta[0, 0, (F - 1) * S:].astype(np.float64)
    np.testing.assert_allclose(dr[0, 0, (F - 2) * S:(F - 1) * S], q[0, 0, (F - 2) * S:(F - 1) * S].astype(np.float64) @ bl,
                               atol=1e-12)


# --------------------------------------------------------------------------
# A planted mistake must be caught: the pins are not vacuous.
# --------------------------------------------------------------------------

def test_pins_catch_a_planted_sign_error():
    # Flip the sign of the erase term in a copy of the token recurrence (pure
    # numpy, CPU only) and check that the overwrite pin would fail on it.
    B, T, H, D = 1, 6, 1, 4
    d = synth.gdn_inputs(B, T, H, D, D, seed=23, dtype="f32", h0_std=1.0)
    k = d["k"][0, :, 0].astype(np.float64)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = d["v"][0, :, 0].astype(np.float64)
    S = d["h0"][0, 0].astype(np.float64)
    bad = []
    for t in range(T):
        p = S.T @ k[t]
        S = S + np.outer(k[t], v[t] + p)                                   # planted: + instead of -
        bad.append(S.T @ k[t])
    assert np.abs(np.array(bad) - v).max() > 1e-3
