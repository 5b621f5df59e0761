"""GPU parity of gdn_recurrent_bwd (gradients of the frame-synchronous
camera scan) against the fp64 backward oracle O7, element by element,
through the C ABI (ctypes binding)."""
import sys

import numpy as np
import pytest

import oracle
from chunkwise_gated_delta_gdn_amd import inputs as synth
from tests._helpers import TOL, max_rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dbeta", "dg", "dh0")


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


def _inputs(B, H, F, S, D, seed, h0_std=0.0, dhT_std=0.0):
    """Scan inputs in the (B,H,N,D) layout with keys scaled so that a frame's
    sum of beta k k^T stays below one; upstream gradients dout ~ N(0,1) and
    dhT ~ N(0, dhT_std)."""
    rng = np.random.default_rng(seed)
    N = F * S
    q = rng.standard_normal((B, H, N, D))
    k = rng.standard_normal((B, H, N, D))
    k /= np.linalg.norm(k, axis=-1, keepdims=True) * np.sqrt(max(S, 1))
    v = rng.standard_normal((B, H, N, D))
    beta = 0.5 * (1 + np.tanh(0.5 * rng.standard_normal((B, H, N))))
    g = -np.logaddexp(0.0, -rng.normal(3.0, 0.5, (B, H, F)))
    h0 = rng.normal(0, h0_std, (B, H, D, D)).astype(np.float32) if h0_std > 0 else None
    dout = rng.standard_normal((B, H, N, D))
    dhT = rng.normal(0, dhT_std, (B, H, D, D)).astype(np.float32) if dhT_std > 0 else None
    c = lambda x: synth.cast(x, "bf16")
    return dict(q=c(q), k=c(k), v=c(v), beta=beta.astype(np.float32), g=g.astype(np.float32), h0=h0,
                dout=c(dout), dhT=dhT, F=F)


def _run(gdn, d, scale, need_dh0=True):
    import torch
    q, k, v, dout = (to_dev(d[n], "bf16") for n in ("q", "k", "v", "dout"))
    beta, g = to_dev(d["beta"], "f32"), to_dev(d["g"], "f32")
    h0 = None if d["h0"] is None else to_dev(d["h0"], "f32")
    dhT = None if d["dhT"] is None else to_dev(d["dhT"], "f32")
    out = gdn.gdn_recurrent_bwd(q, k, v, beta, g, dout, d["F"], scale, h0, dhT, need_dh0=need_dh0)
    torch.cuda.synchronize()
    return [None if x is None else to_np(x) for x in out]


def _ref(d, scale):
    return oracle.frame_scan_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["F"], d["dout"], scale, d["h0"],
                                 d["dhT"])


def _check(got, ref, what):
    errs = {}
    for n, a, r in zip(NAMES, got, ref):
        if a is None:
            continue
        assert np.all(np.isfinite(a)), n
        errs[n] = max_rel_err(a, r)
    _say(f"  {what}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()) + f" (bar {TOL['bf16']:.0e})")
    for n, e in errs.items():
        assert e <= TOL["bf16"], (what, n, e)


@pytest.mark.parametrize("case", [
    # (B, H, F, S, D, h0_std, dhT_std)
    (1, 2, 3, 50, 32, 0.3, 0.5),
    (2, 2, 4, 100, 64, 0.1, 0.2),
    (1, 2, 3, 257, 128, 0.1, 0.0),
    (1, 1, 1, 600, 64, 0.0, 0.3),      # one frame, two 512-token blocks
    (1, 2, 5, 33, 64, 0.2, 0.2),
    (1, 1, 6, 1, 32, 0.2, 0.1),        # one token per frame: the token-level rule
], ids=lambda c: "B{}H{}F{}S{}D{}h{}d{}".format(*c))
def test_scan_bwd_small(gdn, case):
    B, H, F, S, D, h0s, dhs = case
    _say(f"gdn_recurrent_bwd {case}")
    d = _inputs(B, H, F, S, D, 900 + S + D, h0s, dhs)
    _check(_run(gdn, d, 0.7), _ref(d, 0.7), str(case))


def test_scan_bwd_camera_workload(gdn):
    """The camera workload (B=1 H=16 F=8 S=1560 D=64): q, k, v the oracle's
    prep outputs in bf16, beta and per-frame log-decay from the workload,
    dout ~ N(0,1) in bf16; every gradient of every head and frame."""
    _say("gdn_recurrent_bwd camera workload")
    w = synth.workload_inputs("camera")
    pr = oracle.cam_prep(w["qkv"], w["q_norm_w"], w["k_norm_w"], w["proj_q"], w["proj_kv"], w["rope_cos"],
                         w["rope_sin"], w["k_scale"], w["eps"])
    rng = np.random.default_rng(20263 + 7)
    d = dict(q=synth.round_bf16(pr["q"]), k=synth.round_bf16(pr["k"]), v=synth.round_bf16(pr["v"]),
             beta=w["beta"], g=w["g"], h0=None, dhT=None, F=w["F"],
             dout=synth.cast(rng.standard_normal(pr["q"].shape), "bf16"))
    _check(_run(gdn, d, 1.0), _ref(d, 1.0), "camera")


def test_scan_bwd_edges(gdn):
    import torch
    # no frames: dh0 = dhT (or zero)
    d = _inputs(1, 2, 1, 4, 32, 5, 0.2, 0.3)
    z = torch.zeros((1, 2, 0, 32), dtype=torch.bfloat16, device="cuda")
    zb = torch.zeros((1, 2, 0), device="cuda")
    zg = torch.zeros((1, 2, 0), device="cuda")
    lib = gdn.lib()
    dh0 = torch.full((1, 2, 32, 32), 7.0, device="cuda")
    dhT = to_dev(d["dhT"], "f32")
    p = gdn._ptr
    rc = lib.gdn_recurrent_bwd(p(z), p(z), p(z), p(zb), p(zg), 1.0, None, p(z), p(dhT), p(z), p(z), p(z), p(zb),
                               p(zg), p(dh0), 1, 2, 0, 4, 32, 1, None, 0, None)
    torch.cuda.synchronize()
    assert rc == 0
    np.testing.assert_array_equal(to_np(dh0), d["dhT"])
    # unsupported shapes and dtypes are refused before anything runs
    fake = p(dh0)
    assert lib.gdn_recurrent_bwd(fake, fake, fake, fake, fake, 1.0, None, fake, None, fake, fake, fake, fake,
                                 fake, None, 1, 1, 1, 4, 48, 1, None, 0, None) == -2
    assert lib.gdn_recurrent_bwd(fake, fake, fake, fake, fake, 1.0, None, fake, None, fake, fake, fake, fake,
                                 fake, None, 1, 1, 1, 4, 64, 0, None, 0, None) == -2
    # dh0 not requested
    d = _inputs(1, 1, 2, 20, 64, 6, 0.1, 0.1)
    got = _run(gdn, d, 1.0, need_dh0=False)
    assert got[5] is None
    _check(got, _ref(d, 1.0), "no dh0")
