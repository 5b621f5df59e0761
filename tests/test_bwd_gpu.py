"""GPU parity of gdn_bwd (gradients of the gated delta rule) against the
fp64 backward oracle, element by element, through the C ABI."""
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


def _run(gdn, d, up, dtype, scale, need_dh0=True):
    import torch
    q, k, v = (to_dev(d[n], dtype) for n in ("q", "k", "v"))
    dout = to_dev(up["dout"], dtype)
    beta, g = to_dev(d["beta"], "f32"), to_dev(d["g"], "f32")
    h0 = None if d.get("h0") is None else to_dev(d["h0"], "f32")
    dhT = None if up.get("dhT") is None else to_dev(up["dhT"], "f32")
    out = gdn.gdn_bwd(q, k, v, beta, g, dout, scale, h0, dhT, need_dh0=need_dh0)
    torch.cuda.synchronize()
    return [None if x is None else to_np(x) for x in out]


def _ref(d, up, scale, heads=None):
    sel = (lambda x: x) if heads is None else (lambda x: x[:, :, heads])
    sel_s = (lambda x: x) if heads is None else (lambda x: x[:, heads])
    h0 = None if d.get("h0") is None else sel_s(d["h0"])
    dhT = None if up.get("dhT") is None else sel_s(up["dhT"])
    return oracle.gdn_recurrent_bwd(sel(d["q"]), sel(d["k"]), sel(d["v"]), sel(d["beta"]),
                                    sel(d["g"]), sel(up["dout"]), scale, h0, dhT)


def _check(got, ref, dtype, what):
    errs = {}
    for n, a, r in zip(NAMES, got, ref):
        if a is None:
            continue
        assert np.all(np.isfinite(a)), n
        errs[n] = max_rel_err(a, r)
    _say(f"  {what}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()) + f" (bar {TOL[dtype]:.0e})")
    for n, e in errs.items():
        assert e <= TOL[dtype], (n, e)


CASES = [
    # (B, T, H, Dk, Dv, dtype, h0_std, dhT_std)
    (1, 70, 2, 16, 16, "f32", 0.3, 0.5),
    (2, 100, 3, 32, 32, "f32", 0.0, 0.0),
    (1, 130, 2, 64, 64, "f32", 0.3, 0.5),      # 12-token segments, ragged last one
    (1, 90, 1, 128, 32, "f32", 0.1, 0.2),
    (1, 33, 1, 128, 128, "f32", 0.1, 0.2),
    (1, 100, 2, 32, 48, "bf16", 0.3, 0.5),
    (2, 150, 2, 64, 64, "bf16", 0.0, 0.5),
    (1, 77, 2, 128, 128, "bf16", 0.1, 0.0),
    (1, 2000, 1, 64, 64, "bf16", 0.1, 0.3),    # 167 segments: error across a long walk back
    (1, 96, 2, 128, 64, "bf16", 0.2, 0.3),     # a whole number of segments (8 x 12 tokens)
    (1, 1001, 1, 128, 16, "f32", 0.1, 0.3),
]


@pytest.mark.parametrize("B,T,H,Dk,Dv,dtype,h0_std,dhT_std", CASES)
def test_bwd_matches_oracle(gdn, B, T, H, Dk, Dv, dtype, h0_std, dhT_std):
    _say(f"gdn_bwd B={B} T={T} H={H} Dk={Dk} Dv={Dv} {dtype} h0={h0_std} dhT={dhT_std}")
    seed = 31000 + T + Dk + Dv
    d = synth.gdn_inputs(B, T, H, Dk, Dv, seed, dtype, h0_std=h0_std)
    up = synth.gdn_upstream(B, T, H, Dk, Dv, seed + 1, dtype, dhT_std=dhT_std)
    scale = Dk ** -0.5
    _check(_run(gdn, d, up, dtype, scale), _ref(d, up, scale), dtype, "all")


def test_bwd_edge_cases(gdn):
    import torch
    # T = 0: dh0 = dhT (or 0), nothing else
    d = synth.gdn_inputs(1, 0, 2, 32, 32, 31101, "f32", h0_std=0.3)
    up = synth.gdn_upstream(1, 0, 2, 32, 32, 31102, "f32", dhT_std=0.5)
    got = _run(gdn, d, up, "f32", 1.0)
    assert got[0].shape == (1, 0, 2, 32)
    np.testing.assert_array_equal(got[5], up["dhT"])
    up0 = dict(up, dhT=None)
    np.testing.assert_array_equal(_run(gdn, d, up0, "f32", 1.0)[5], 0.0)
    # one token; no h0, no dhT; dh0 not requested
    d = synth.gdn_inputs(2, 1, 3, 64, 32, 31103, "f32")
    up = synth.gdn_upstream(2, 1, 3, 64, 32, 31104, "f32")
    got = _run(gdn, d, up, "f32", 0.5, need_dh0=False)
    assert got[5] is None
    _check(got, _ref(d, up, 0.5), "f32", "T=1")
    # a token count that is an exact multiple of the 12-token segments
    d = synth.gdn_inputs(1, 48, 1, 16, 32, 31105, "bf16", h0_std=0.2)
    up = synth.gdn_upstream(1, 48, 1, 16, 32, 31106, "bf16", dhT_std=0.2)
    _check(_run(gdn, d, up, "bf16", 1.0), _ref(d, up, 1.0), "bf16", "T=48")
    # a work space that is too small is rejected before anything is launched
    q = torch.zeros((1, 8, 1, 16), device="cuda")
    p = gdn._ptr(q)
    rc = gdn.lib().gdn_bwd(p, p, p, p, p, 1.0, None, p, None, p, p, p, p, p, None,
                           1, 8, 1, 16, 16, 0, None, 0, None)
    assert rc == -3


def test_bwd_gdn_workload(gdn):
    """The gdn workload (B=2 H=16 T=4096 D=128, bf16), in the launch shape
    the benchmark times; the oracle on all 32 (batch, head) pairs (one
    thread per pair)."""
    B, T, H, D = 2, 4096, 16, 128
    _say(f"gdn_bwd gdn workload B={B} T={T} H={H} D={D}, all pairs")
    d = synth.gdn_inputs(B, T, H, D, D, 20261, "bf16")
    up = synth.gdn_upstream(B, T, H, D, D, 20265, "bf16")
    scale = D ** -0.5
    got = _run(gdn, d, up, "bf16", scale)
    _check(got, _ref(d, up, scale), "bf16", "all pairs")
    # the same call again gives bit-identical gradients (no atomics, fixed
    # summation order)
    again = _run(gdn, d, up, "bf16", scale)
    for n, a, b in zip(NAMES, got, again):
        np.testing.assert_array_equal(a, b, err_msg=n)
