"""GPU parity of gdn_prep_bwd (gradients of the camera prep) against the
fp64 backward oracle O8, element by element, through the C ABI."""
import sys

import numpy as np
import pytest

import oracle
from chunkwise_gated_delta_gdn_amd import inputs as synth
from tests._helpers import TOL, max_rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu

GRADS = ("dqkv", "dq_norm_w", "dk_norm_w", "dproj_q", "dproj_kv")


@pytest.fixture(scope="module")
def gdn():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from chunkwise_gated_delta_gdn_amd import gdn as g
    return g


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _case(B, N, H, D, seed, dtype, gdtype, weights=True, norm_grads=True):
    """Camera-like prep inputs (qkv ~ N(0,1), rigid per-token projections,
    RoPE tables) with norm weights ~ U(0.5, 1.5) (or None) and upstream
    gradients ~ N(0,1) of q, k, v (and of the three norm outputs)."""
    d = synth.camera_inputs(B, 1, N, H, D, seed, dtype)
    rng = np.random.default_rng(seed + 1)
    if weights:
        d["q_norm_w"] = rng.uniform(0.5, 1.5, H * D).astype(np.float32)
        d["k_norm_w"] = rng.uniform(0.5, 1.5, H * D).astype(np.float32)
    else:
        d["q_norm_w"] = d["k_norm_w"] = None
    up = {n: synth.cast(rng.standard_normal((B, H, N, D)), gdtype) for n in ("dq", "dk", "dv")}
    for n in ("dpre", "dpost", "dinfl"):
        up[n] = rng.standard_normal((B, H, N)).astype(np.float32) if norm_grads else None
    return d, up


def _run(gdn, d, up, dtype, gdtype):
    import torch
    dev = lambda x: None if x is None else to_dev(x, "f32")
    out = gdn.gdn_prep_bwd(to_dev(d["qkv"], dtype), dev(d["q_norm_w"]), dev(d["k_norm_w"]), dev(d["proj_q"]),
                           dev(d["proj_kv"]), dev(d["rope_cos"]), dev(d["rope_sin"]), d["k_scale"], d["eps"],
                           to_dev(up["dq"], gdtype), to_dev(up["dk"], gdtype), to_dev(up["dv"], gdtype),
                           dev(up["dpre"]), dev(up["dpost"]), dev(up["dinfl"]))
    torch.cuda.synchronize()
    return {n: to_np(x) for n, x in out.items()}


def _ref(d, up):
    return oracle.cam_prep_bwd(d["qkv"], d["q_norm_w"], d["k_norm_w"], d["proj_q"], d["proj_kv"], d["rope_cos"],
                               d["rope_sin"], d["k_scale"], d["eps"], up["dq"], up["dk"], up["dv"], up["dpre"],
                               up["dpost"], up["dinfl"])


def _check(got, ref, bar, what):
    errs = {}
    for n in GRADS:
        assert np.all(np.isfinite(got[n])), n
        errs[n] = max_rel_err(got[n], ref[n])
    _say(f"  {what}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()) + f" (bar {bar:.0e})")
    for n, e in errs.items():
        assert e <= bar, (what, n, e)


@pytest.mark.parametrize("case", [
    # (B, N, H, D, dtype, grad dtype, weights, norm-output gradients)
    (1, 37, 2, 16, "f32", "f32", True, True),
    (2, 50, 3, 32, "f32", "f32", False, True),
    (1, 64, 4, 64, "f32", "f32", True, False),
    (1, 40, 2, 128, "f32", "f32", True, True),
    (2, 33, 16, 64, "bf16", "bf16", True, True),
    (1, 70, 5, 48, "bf16", "f32", True, True),
    (1, 25, 64, 64, "bf16", "bf16", True, True),        # eight heads per lane
    (1, 30, 7, 112, "f32", "bf16", False, True),
], ids=lambda c: "B{}N{}H{}D{}{}g{}w{}n{}".format(*c))
def test_prep_bwd_small(gdn, case):
    B, N, H, D, dtype, gdtype, weights, ng = case
    _say(f"gdn_prep_bwd {case}")
    d, up = _case(B, N, H, D, 1300 + N + D, dtype, gdtype, weights, ng)
    bar = TOL["f32"] if dtype == "f32" and gdtype == "f32" else TOL["bf16"]
    _check(_run(gdn, d, up, dtype, gdtype), _ref(d, up), bar, str(case))


def test_prep_bwd_camera_workload(gdn):
    """The camera workload's prep (B=1 N=12480 H=16 D=64, bf16 qkv), bf16
    upstream gradients of q, k, v and fp32 ones of the three norm outputs;
    every gradient (the weight gradients sum all 12480 tokens)."""
    _say("gdn_prep_bwd camera workload")
    w = synth.workload_inputs("camera")
    rng = np.random.default_rng(20263 + 11)
    B, N, H, D = 1, w["F"] * w["S"], 16, 64
    up = {n: synth.cast(rng.standard_normal((B, H, N, D)), "bf16") for n in ("dq", "dk", "dv")}
    for n in ("dpre", "dpost", "dinfl"):
        up[n] = rng.standard_normal((B, H, N)).astype(np.float32)
    _check(_run(gdn, w, up, "bf16", "bf16"), _ref(w, up), TOL["bf16"], "camera")


def test_prep_bwd_options_and_refusals(gdn):
    import torch
    d, up = _case(1, 20, 2, 32, 5, "bf16", "bf16")
    dev = lambda x: None if x is None else to_dev(x, "f32")
    args = (to_dev(d["qkv"], "bf16"), dev(d["q_norm_w"]), dev(d["k_norm_w"]), dev(d["proj_q"]), dev(d["proj_kv"]),
            dev(d["rope_cos"]), dev(d["rope_sin"]), d["k_scale"], d["eps"],
            to_dev(up["dq"], "bf16"), to_dev(up["dk"], "bf16"), to_dev(up["dv"], "bf16"))
    full = gdn.gdn_prep_bwd(*args, dev(up["dpre"]), dev(up["dpost"]), dev(up["dinfl"]))
    part = gdn.gdn_prep_bwd(*args, dev(up["dpre"]), dev(up["dpost"]), dev(up["dinfl"]), weight_grads=False,
                            proj_grads=False)
    torch.cuda.synchronize()
    assert part["dq_norm_w"] is None and part["dproj_q"] is None
    np.testing.assert_array_equal(to_np(part["dqkv"]), to_np(full["dqkv"]))
    lib, p = gdn.lib(), gdn._ptr
    x = full["dqkv"]
    # weight gradients without a work space; one projection gradient only; D = 40
    assert lib.gdn_prep_bwd(p(x), None, None, p(x), p(x), p(x), p(x), 1.0, 1e-6, p(x), p(x), p(x), None, None,
                            None, p(x), p(x), None, None, None, 1, 20, 2, 32, 1, 1, None, 0, None) == -3
    assert lib.gdn_prep_bwd(p(x), None, None, p(x), p(x), p(x), p(x), 1.0, 1e-6, p(x), p(x), p(x), None, None,
                            None, p(x), None, None, p(x), None, 1, 20, 2, 32, 1, 1, None, 0, None) == -1
    assert lib.gdn_prep_bwd(p(x), None, None, p(x), p(x), p(x), p(x), 1.0, 1e-6, p(x), p(x), p(x), None, None,
                            None, p(x), None, None, None, None, 1, 20, 2, 40, 1, 1, None, 0, None) == -2


def test_camera_backward_end_to_end(gdn):
    """The camera workload's whole backward on the GPU: gdn_recurrent_bwd on
    the GPU prep's bf16 outputs, its fp32 dq, dk, dv straight into
    gdn_prep_bwd; against the oracle's scan backward on the oracle prep's
    outputs (rounded to bf16) fed into the prep backward oracle."""
    import torch
    _say("camera backward end to end")
    w = synth.workload_inputs("camera")
    dev = lambda x: to_dev(x, "f32")
    t = {n: dev(w[n]) for n in ("q_norm_w", "k_norm_w", "proj_q", "proj_kv", "rope_cos", "rope_sin", "beta", "g")}
    pr = gdn.gdn_prep(to_dev(w["qkv"], "bf16"), t["q_norm_w"], t["k_norm_w"], t["proj_q"], t["proj_kv"],
                      t["rope_cos"], t["rope_sin"], w["k_scale"], w["eps"])
    rng = np.random.default_rng(20263 + 13)
    dout = synth.cast(rng.standard_normal(tuple(pr["q"].shape)), "bf16")
    sg = gdn.gdn_recurrent_bwd(pr["q"], pr["k"], pr["v"], t["beta"], t["g"], to_dev(dout, "bf16"), w["F"], 1.0)
    pg = gdn.gdn_prep_bwd(to_dev(w["qkv"], "bf16"), t["q_norm_w"], t["k_norm_w"], t["proj_q"], t["proj_kv"],
                          t["rope_cos"], t["rope_sin"], w["k_scale"], w["eps"], sg[0], sg[1], sg[2])
    torch.cuda.synchronize()
    got = {n: to_np(x) for n, x in pg.items()}
    ref_pr = oracle.cam_prep(w["qkv"], w["q_norm_w"], w["k_norm_w"], w["proj_q"], w["proj_kv"], w["rope_cos"],
                             w["rope_sin"], w["k_scale"], w["eps"])
    q, k, v = (synth.round_bf16(ref_pr[n]) for n in ("q", "k", "v"))
    rs = oracle.frame_scan_bwd(q, k, v, w["beta"], w["g"], w["F"], dout, 1.0)
    ref = oracle.cam_prep_bwd(w["qkv"], w["q_norm_w"], w["k_norm_w"], w["proj_q"], w["proj_kv"], w["rope_cos"],
                              w["rope_sin"], w["k_scale"], w["eps"], rs[0], rs[1], rs[2])
    _check(got, ref, TOL["bf16"], "end to end")
