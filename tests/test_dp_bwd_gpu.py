"""GPU parity of deltaproduct_bwd (gradients of the two-step gated
DeltaProduct with a lower unitriangular step mask) against the fp64
backward oracle O9, element by element, through the C ABI."""
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


def _inputs(B, T, H, dk, Dv, m, seed, h0_std, dhT_std):
    mask = np.array([[1.0, 0.0], [m, 1.0]], np.float32)
    d = synth.deltaproduct_inputs(B, T, H, 2, dk, Dv, seed, "bf16", h0_std=h0_std, mask=mask)
    up = synth.gdn_upstream(B, T, H, 2 * dk, Dv, seed + 1, "bf16", dhT_std=dhT_std)
    return d, up


def _run(gdn, d, up, scale, need_dh0=True):
    import torch
    q, k, v = (to_dev(d[n], "bf16") for n in ("q", "k", "v"))
    dout = to_dev(up["dout"], "bf16")
    beta, g = to_dev(d["beta"], "f32"), to_dev(d["g"], "f32")
    h0 = None if d.get("h0") is None else to_dev(d["h0"], "f32")
    dhT = None if up.get("dhT") is None else to_dev(up["dhT"], "f32")
    out = gdn.deltaproduct_bwd(q, k, v, beta, g, d["mask"], dout, scale, h0, dhT, need_dh0=need_dh0)
    torch.cuda.synchronize()
    return [None if x is None else to_np(x) for x in out]


def _ref(d, up, scale):
    return oracle.deltaproduct_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["mask"], up["dout"], scale,
                                   d.get("h0"), up.get("dhT"))


def _check(got, ref, what):
    errs = {}
    for n, a, r in zip(NAMES, got, ref):
        if a is None:
            continue
        assert np.all(np.isfinite(a)), n
        errs[n] = max_rel_err(a, r)
    _say(f"  {what}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()) + f" (bar {TOL['bf16']:.0e})")
    for n, e in errs.items():
        assert e <= TOL["bf16"], (n, e)


CASES = [
    # (B, T, H, dk, Dv, m, h0_std, dhT_std)
    (1, 70, 2, 32, 32, 1.0, 0.3, 0.5),          # two chunks, ragged tail
    (2, 130, 2, 64, 64, 0.5, 0.0, 0.3),         # three chunks, no h0
    (1, 200, 1, 128, 128, 1.0, 0.1, 0.0),       # no dhT
    (1, 64, 2, 32, 96, -0.7, 0.2, 0.2),         # one whole chunk, a negative mask entry
    (1, 300, 2, 128, 64, 0.25, 0.1, 0.3),
    (1, 1000, 1, 64, 32, 1.0, 0.1, 0.3),        # 16 chunks: error across a long walk back
]


@pytest.mark.parametrize("B,T,H,dk,Dv,m,h0_std,dhT_std", CASES)
def test_dp_bwd_matches_oracle(gdn, B, T, H, dk, Dv, m, h0_std, dhT_std):
    _say(f"deltaproduct_bwd B={B} T={T} H={H} dk={dk} Dv={Dv} m={m} h0={h0_std} dhT={dhT_std}")
    d, up = _inputs(B, T, H, dk, Dv, m, 41000 + T + dk + Dv, h0_std, dhT_std)
    scale = (2 * dk) ** -0.5
    _check(_run(gdn, d, up, scale), _ref(d, up, scale), "all")


def test_dp_bwd_edge_cases(gdn):
    import torch
    # T = 0: dh0 = dhT (or 0)
    d, up = _inputs(1, 0, 2, 32, 32, 1.0, 41101, 0.3, 0.5)
    got = _run(gdn, d, up, 1.0)
    assert got[0].shape == (1, 0, 2, 64)
    np.testing.assert_array_equal(got[5], up["dhT"])
    np.testing.assert_array_equal(_run(gdn, d, dict(up, dhT=None), 1.0)[5], 0.0)
    # one token; dh0 not requested
    d, up = _inputs(2, 1, 3, 64, 32, 0.5, 41103, 0.2, 0.2)
    got = _run(gdn, d, up, 0.5, need_dh0=False)
    assert got[5] is None
    _check(got, _ref(d, up, 0.5), "T=1")
    # m = 0: two independent gated delta rules; the second block's values are v
    d, up = _inputs(1, 100, 2, 64, 64, 0.0, 41105, 0.2, 0.3)
    _check(_run(gdn, d, up, 0.125), _ref(d, up, 0.125), "m=0")
    # masks off the lower unitriangular form, fp32 inputs, unsupported widths
    q = torch.zeros((1, 8, 1, 64), device="cuda", dtype=torch.bfloat16)
    v = torch.zeros((1, 8, 1, 32), device="cuda", dtype=torch.bfloat16)
    b = torch.zeros((1, 8, 1, 2), device="cuda")
    g = torch.zeros((1, 8, 1), device="cuda")
    for mask in ([[0.75, -0.5], [0.25, 1.0]], [[1.0, 0.0], [1.0, 0.5]]):
        with pytest.raises(gdn.GdnError) as e:
            gdn.deltaproduct_bwd(q, q, v, b, g, mask, v)
        assert e.value.code == -2
    with pytest.raises(gdn.GdnError) as e:
        gdn.deltaproduct_bwd(q.float(), q.float(), v.float(), b, g, [[1, 0], [1, 1]], v.float())
    assert e.value.code == -2
    q48 = torch.zeros((1, 8, 1, 96), device="cuda", dtype=torch.bfloat16)
    with pytest.raises(gdn.GdnError) as e:
        gdn.deltaproduct_bwd(q48, q48, v, b, g, [[1, 0], [1, 1]], v)
    assert e.value.code == -2
    # a work space that is too small is rejected before anything is launched
    p = gdn._ptr(q)
    m = np.array([[1, 0], [1, 1]], np.float32)
    import ctypes
    rc = gdn.lib().deltaproduct_bwd(p, p, p, p, p, m.ctypes.data_as(ctypes.c_void_p), 2, 1.0, None, p, None,
                                    p, p, p, p, p, None, 1, 8, 1, 32, 32, 1, None, 0, None)
    assert rc == -3


def test_dp_bwd_workload(gdn):
    """The DeltaProduct workload (B=2 H=8 T=2048, two 128-wide sub-keys,
    Dv=128, lower unitriangular ones, bf16) in the launch shape the
    benchmark times; the oracle on all 16 (batch, head) pairs."""
    d = synth.workload_inputs("deltaproduct")
    B, T, H, K = d["q"].shape
    Dv = d["v"].shape[-1]
    _say(f"deltaproduct_bwd deltaproduct workload B={B} T={T} H={H} K={K} Dv={Dv}, all pairs")
    up = synth.gdn_upstream(B, T, H, K, Dv, 20266, "bf16", dhT_std=0.1)
    scale = K ** -0.5
    got = _run(gdn, d, up, scale)
    _check(got, _ref(d, up, scale), "all pairs")
    again = _run(gdn, d, up, scale)
    for n, a, b in zip(NAMES, got, again):
        np.testing.assert_array_equal(a, b, err_msg=n)
