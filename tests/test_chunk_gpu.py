"""GPU parity of gdn_chunk_fwd and deltaproduct_chunk_fwd against the fp64
oracle, element by element, through the C ABI (ctypes binding)."""
import sys

import numpy as np
import pytest

import oracle
from chunkwise_gated_delta_gdn_amd import inputs as synth
from tests._helpers import TOL, max_rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu


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


def _run_gdn(gdn, d, dtype, chunk, scale=1.0, out_dtype=None):
    import torch
    out_dtype = out_dtype or torch.float32
    q, k, v = (to_dev(d[n], dtype) for n in ("q", "k", "v"))
    beta, g = to_dev(d["beta"], "f32"), to_dev(d["g"], "f32")
    h0 = None if d.get("h0") is None else to_dev(d["h0"], "f32")
    o, hT = gdn.gdn_chunk_fwd(q, k, v, beta, g, scale, h0, chunk=chunk, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return to_np(o), to_np(hT)


def _check(o, hT, oref, href, dtype, what):
    eo, eh = max_rel_err(o, oref), max_rel_err(hT, href)
    _say(f"  {what}: max rel err o={eo:.3e} hT={eh:.3e} (bar {TOL[dtype]:.0e})")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(hT))
    assert eo <= TOL[dtype] and eh <= TOL[dtype], (eo, eh)


# ---------------------------------------------------------------------------
# small cases: several tiles, ragged last chunk, random initial state
# ---------------------------------------------------------------------------
SMALL = [
    # (B, T, H, Dk, Dv, chunk, dtype, h0_std)
    (1, 64, 2, 16, 16, 16, "f32", 0.0),       # the tiny fp32 workload
    (1, 70, 2, 16, 32, 16, "f32", 0.3),
    (2, 100, 3, 32, 32, 32, "f32", 0.3),
    (1, 130, 2, 64, 64, 64, "f32", 0.3),
    (1, 90, 1, 128, 32, 32, "f32", 0.1),
    (1, 77, 2, 128, 64, 32, "f32", 0.1),
    (1, 64, 2, 16, 16, 16, "bf16", 0.0),
    (1, 100, 2, 32, 48, 16, "bf16", 0.3),
    (2, 150, 2, 64, 64, 32, "bf16", 0.3),
    (1, 200, 3, 64, 128, 64, "bf16", 0.2),
    (1, 257, 2, 128, 128, 64, "bf16", 0.05),
    (1, 129, 2, 128, 256, 32, "bf16", 0.05),
    (1, 95, 2, 256, 64, 32, "bf16", 0.05),
    (1, 33, 1, 256, 128, 16, "bf16", 0.05),
    # key and value widths that are multiples of 16 but not powers of two
    # (run on the next power of two's kernels, the extra features zero)
    (1, 150, 2, 112, 112, 64, "bf16", 0.1),
    (2, 77, 2, 48, 80, 32, "bf16", 0.2),
    (1, 100, 2, 176, 48, 32, "bf16", 0.05),
    (1, 90, 2, 80, 112, 16, "f32", 0.2),
    (1, 70, 2, 112, 32, 32, "f32", 0.1),
    (1, 40, 1, 240, 16, 16, "f32", 0.05),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B{}T{}H{}K{}V{}C{}{}h{}".format(*c))
def test_gdn_chunk_small(gdn, case):
    B, T, H, Dk, Dv, chunk, dtype, h0s = case
    _say(f"gdn_chunk_fwd small case {case}")
    d = synth.gdn_inputs(B, T, H, Dk, Dv, seed=1000 + T + Dk, dtype=dtype, h0_std=h0s)
    o, hT = _run_gdn(gdn, d, dtype, chunk, scale=0.7)
    oref, href = oracle.gdn_recurrent(d["q"], d["k"], d["v"], d["beta"], d["g"], 0.7, d["h0"])
    _check(o, hT, oref, href, dtype, str(case))


# More (batch, head, 16-column slice) chains than compute units: the state
# pass runs in its two-workgroups-per-CU configuration (four waves, two
# staging buffers).  Key widths 32...128 (112 padded), value widths 48...128,
# ragged last chunks, one-token and one-chunk sequences, nonzero initial
# state, fp32 and bf16 output.
DUAL = [
    # (B, T, H, Dk, Dv, h0_std, out)
    (4, 300, 16, 128, 128, 0.05, "bf16"),
    (2, 200, 40, 64, 64, 0.1, "f32"),
    (3, 130, 32, 32, 128, 0.2, "bf16"),
    (2, 257, 48, 112, 48, 0.1, "f32"),
    (4, 1, 16, 128, 128, 0.1, "f32"),
    (4, 64, 16, 128, 128, 0.1, "f32"),
]


@pytest.mark.parametrize("case", DUAL, ids=lambda c: "B{}T{}H{}K{}V{}h{}{}".format(*c))
def test_gdn_chunk_two_workgroups_per_cu(gdn, case):
    import torch
    B, T, H, Dk, Dv, h0s, out = case
    _say(f"gdn_chunk_fwd two workgroups per CU {case}")
    d = synth.gdn_inputs(B, T, H, Dk, Dv, seed=5000 + T + Dk + Dv + H, dtype="bf16", h0_std=h0s)
    od = torch.bfloat16 if out == "bf16" else torch.float32
    o, hT = _run_gdn(gdn, d, "bf16", 64, scale=Dk ** -0.5, out_dtype=od)
    oref, href = oracle.gdn_recurrent(d["q"], d["k"], d["v"], d["beta"], d["g"], Dk ** -0.5, d["h0"])
    if out == "bf16":
        bar = _bf16_out_bar(o, oref, TOL["bf16"])
        err = np.abs(o.astype(np.float64) - oref)
        _say(f"  o: max err / bar {np.max(err / bar):.3f}")
        assert np.all(err <= bar)
        eh = max_rel_err(hT, href)
        _say(f"  hT: max rel err {eh:.3e}")
        assert eh <= TOL["bf16"]
    else:
        _check(o, hT, oref, href, "bf16", str(case))


# Long sequences over few heads, where the dispatch takes the segment-parallel
# state pass (segment summaries, their composition, then the output pass per
# segment; 24-29 segments here): key widths 32...128 (112 padded), value
# widths 64...256 (two 128-column groups at 256), ragged last chunk and
# segment, nonzero initial state.
SEG = [
    # (B, T, H, Dk, Dv, h0_std)
    (1, 16384, 2, 128, 128, 0.02),
    (1, 16384, 1, 112, 256, 0.05),
    (1, 12288, 2, 64, 80, 0.1),
    (1, 16384, 1, 32, 64, 0.1),
    (1, 20000, 1, 128, 112, 0.05),
    (1, 16384, 1, 48, 128, 0.1),
]


@pytest.mark.parametrize("case", SEG, ids=lambda c: "B{}T{}H{}K{}V{}h{}".format(*c))
def test_gdn_chunk_segment_pass(gdn, case):
    B, T, H, Dk, Dv, h0s = case
    _say(f"gdn_chunk_fwd segment pass {case}")
    d = synth.gdn_inputs(B, T, H, Dk, Dv, seed=3000 + T + Dk + Dv, dtype="bf16", h0_std=h0s)
    o, hT = _run_gdn(gdn, d, "bf16", 64)
    oref, href = oracle.gdn_recurrent(d["q"], d["k"], d["v"], d["beta"], d["g"], 1.0, d["h0"])
    _check(o, hT, oref, href, "bf16", str(case))


def test_gdn_chunk_tiny_workload(gdn):
    """The tiny fp32 workload exactly: B=1 H=2 T=64 D=16 chunk 16."""
    _say("gdn_chunk_fwd gdn_tiny workload")
    d = synth.workload_inputs("gdn_tiny")
    o, hT = _run_gdn(gdn, d, "f32", 16)
    oref, href = oracle.gdn_recurrent(d["q"], d["k"], d["v"], d["beta"], d["g"], 1.0, d["h0"])
    _check(o, hT, oref, href, "f32", "gdn_tiny")


def _bf16_out_bar(o, oref, tol):
    """Element-wise bar for an output stored in bf16: the fp32 bar on the
    whole tensor plus half an ulp of bf16 at the element's own magnitude (the
    rounding of the store itself; the larger of |o| and |oref| decides the
    binade, as the stored value may sit just across a power of two)."""
    mag = np.maximum(np.abs(o), np.abs(oref)).astype(np.float64)
    ex = np.floor(np.log2(np.maximum(mag, np.finfo(np.float32).tiny)))
    half_ulp = np.exp2(ex - 8)
    return tol * np.abs(oref).max() + half_ulp


def test_gdn_chunk_full_workload(gdn):
    """B=2 H=16 T=4096 D=128 chunk 64 bf16, every output element, with the
    output stored in fp32 and in bf16 (the call the benchmark times)."""
    import torch
    _say("gdn_chunk_fwd gdn workload (B=2 H=16 T=4096 D=128), full comparison, fp32 and bf16 output")
    d = synth.workload_inputs("gdn")
    oref, href = oracle.gdn_recurrent(d["q"], d["k"], d["v"], d["beta"], d["g"], 1.0, d["h0"])
    o, hT = _run_gdn(gdn, d, "bf16", 64)
    _check(o, hT, oref, href, "bf16", "gdn full, fp32 output")
    ob, hTb = _run_gdn(gdn, d, "bf16", 64, out_dtype=torch.bfloat16)
    eb = max_rel_err(ob, oref)
    over = np.abs(ob - oref) - _bf16_out_bar(ob, oref, TOL["bf16"])
    _say(f"  gdn full, bf16 output: max rel err o={eb:.3e} (bar {TOL['bf16'] + 2.0 ** -8:.2e}); "
         f"element-wise margin to fp32 bar + half ulp: {-over.max():.3e}")
    assert np.all(np.isfinite(ob))
    assert eb <= TOL["bf16"] + 2.0 ** -8
    assert np.all(over <= 0.0)
    # the state does not depend on the output's storage type
    np.testing.assert_array_equal(hTb, hT)


def test_gdn_chunk_long_workload(gdn):
    """B=1 H=16 T=65536 D=128 chunk 64 bf16 with h0 ~ N(0, 0.02^2): every
    head, every output element (the oracle runs one thread per head)."""
    _say("gdn_chunk_fwd gdn_long workload (T=65536), full comparison on all 16 heads")
    d = synth.workload_inputs("gdn_long")
    o, hT = _run_gdn(gdn, d, "bf16", 64)
    oref, href = oracle.gdn_recurrent(d["q"], d["k"], d["v"], d["beta"], d["g"], 1.0, d["h0"])
    _check(o, hT, oref, href, "bf16", "gdn_long all heads")
    per_head = [max_rel_err(o[:, :, h], oref[:, :, h]) for h in range(o.shape[2])]
    _say("  per head: " + " ".join(f"{e:.1e}" for e in per_head))


def test_gdn_chunk_head_dim_112(gdn):
    """D = 112 (the width of the pages' reference model) at a workload-like
    size: B=1 H=8 T=2048 Dk=Dv=112 chunk 64 bf16, h0 ~ N(0, 0.02^2), every
    output element."""
    _say("gdn_chunk_fwd D=112 B=1 H=8 T=2048 chunk 64, full comparison")
    d = synth.gdn_inputs(1, 2048, 8, 112, 112, seed=20266, dtype="bf16", h0_std=0.02)
    o, hT = _run_gdn(gdn, d, "bf16", 64)
    oref, href = oracle.gdn_recurrent(d["q"], d["k"], d["v"], d["beta"], d["g"], 1.0, d["h0"])
    _check(o, hT, oref, href, "bf16", "D=112")


def test_gdn_chunk_split_resume_on_gpu(gdn):
    import torch
    _say("gdn_chunk_fwd split/resume")
    d = synth.gdn_inputs(1, 300, 2, 64, 64, seed=31, dtype="bf16", h0_std=0.1)
    o, hT = _run_gdn(gdn, d, "bf16", 64)
    T1 = 128   # a chunk boundary: the chunked arithmetic is then identical
    d1 = {n: (np.ascontiguousarray(d[n][:, :T1]) if n in ("q", "k", "v", "beta", "g") else d[n]) for n in d}
    d2 = {n: (np.ascontiguousarray(d[n][:, T1:]) if n in ("q", "k", "v", "beta", "g") else d[n]) for n in d}
    o1, h1 = _run_gdn(gdn, d1, "bf16", 64)
    d2["h0"] = h1
    o2, h2 = _run_gdn(gdn, d2, "bf16", 64)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), o, rtol=0, atol=1e-6)
    np.testing.assert_allclose(h2, hT, rtol=0, atol=1e-6)


def test_gdn_chunk_edge_cases(gdn):
    import torch
    _say("gdn_chunk_fwd edge cases: T=0, T=1, beta=0 closed form, bf16 output")
    # T = 0: hT is h0
    d = synth.gdn_inputs(1, 0, 2, 64, 64, seed=32, dtype="bf16", h0_std=0.5)
    o, hT = _run_gdn(gdn, d, "bf16", 64)
    assert o.shape == (1, 0, 2, 64)
    np.testing.assert_array_equal(hT, d["h0"])
    # T = 1
    d = synth.gdn_inputs(2, 1, 3, 128, 128, seed=33, dtype="bf16", h0_std=0.5)
    o, hT = _run_gdn(gdn, d, "bf16", 64)
    oref, href = oracle.gdn_recurrent(d["q"], d["k"], d["v"], d["beta"], d["g"], 1.0, d["h0"])
    _check(o, hT, oref, href, "bf16", "T=1")
    # beta = 0 and h0 = 0: the output is exactly zero
    d = synth.gdn_inputs(1, 100, 2, 64, 64, seed=34, dtype="bf16")
    d["beta"][:] = 0
    o, hT = _run_gdn(gdn, d, "bf16", 64)
    assert np.all(o == 0) and np.all(hT == 0)
    # bf16 output: the oracle within the output's own rounding (half an ulp,
    # 2^-8 of the largest magnitude) plus the fp32-output bar
    d = synth.gdn_inputs(1, 200, 2, 128, 128, seed=35, dtype="bf16", h0_std=0.05)
    o, hT = _run_gdn(gdn, d, "bf16", 64, out_dtype=torch.bfloat16)
    oref, href = oracle.gdn_recurrent(d["q"], d["k"], d["v"], d["beta"], d["g"], 1.0, d["h0"])
    assert max_rel_err(o, oref) <= 2.0 ** -8 + TOL["bf16"]
    assert max_rel_err(hT, href) <= TOL["bf16"]


# ---------------------------------------------------------------------------
# DeltaProduct
# ---------------------------------------------------------------------------
DP_SMALL = [
    # (B, T, H, r, dk, Dv, chunk, dtype, mask)
    (1, 50, 2, 2, 16, 16, 16, "f32", "tril"),
    (1, 70, 2, 2, 32, 32, 32, "f32", "rand"),
    (1, 45, 1, 2, 64, 48, 16, "f32", "tril"),
    (1, 90, 2, 2, 32, 32, 16, "bf16", "tril"),
    (2, 100, 2, 2, 64, 64, 32, "bf16", "rand"),
    (1, 130, 2, 2, 128, 128, 32, "bf16", "tril"),
    (1, 77, 2, 1, 128, 64, 64, "bf16", "one"),
    # lower unitriangular masks [[1, 0], [m, 1]] in bf16 run as two passes of
    # the single-chain kernels: m = 1, 0.5, 0 (M = I), several chunks, ragged
    (1, 300, 2, 2, 128, 128, 32, "bf16", "tril"),
    (2, 200, 3, 2, 64, 48, 16, "bf16", "half"),
    (1, 150, 2, 2, 32, 64, 32, "bf16", "eye"),
    (1, 1000, 1, 2, 128, 80, 32, "bf16", "half"),
]


@pytest.mark.parametrize("case", DP_SMALL, ids=lambda c: "B{}T{}H{}r{}dk{}V{}C{}{}{}".format(*c))
def test_deltaproduct_small(gdn, case):
    import torch
    B, T, H, r, dk, Dv, chunk, dtype, mk = case
    _say(f"deltaproduct_chunk_fwd small case {case}")
    rng = np.random.default_rng(T + dk)
    mask = {"tril": np.tril(np.ones((r, r))), "rand": np.tril(rng.uniform(-1, 1, (r, r))),
            "one": np.ones((1, 1)), "half": np.array([[1.0, 0.0], [0.5, 1.0]]),
            "eye": np.eye(2)}[mk].astype(np.float32)
    d = synth.deltaproduct_inputs(B, T, H, r, dk, Dv, seed=2000 + T, dtype=dtype, h0_std=0.1, mask=mask)
    q, k, v = (to_dev(d[n], dtype) for n in ("q", "k", "v"))
    o, hT = gdn.deltaproduct_chunk_fwd(q, k, v, to_dev(d["beta"], "f32"), to_dev(d["g"], "f32"), mask,
                                       scale=(r * dk) ** -0.5, h0=to_dev(d["h0"], "f32"), chunk=chunk)
    torch.cuda.synchronize()
    oref, href = oracle.deltaproduct_recurrent(d["q"], d["k"], d["v"], d["beta"], d["g"], mask,
                                               (r * dk) ** -0.5, d["h0"])
    _check(to_np(o), to_np(hT), oref, href, dtype, str(case))


def test_deltaproduct_full_workload(gdn):
    """B=2 H=8 T=2048 K=2x128 Dv=128 chunk 32 r=2 bf16, lower-triangular mask."""
    import torch
    _say("deltaproduct_chunk_fwd deltaproduct workload, full comparison")
    d = synth.workload_inputs("deltaproduct")
    q, k, v = (to_dev(d[n], "bf16") for n in ("q", "k", "v"))
    o, hT = gdn.deltaproduct_chunk_fwd(q, k, v, to_dev(d["beta"], "f32"), to_dev(d["g"], "f32"),
                                       d["mask"], scale=256 ** -0.5, chunk=32)
    torch.cuda.synchronize()
    oref, href = oracle.deltaproduct_recurrent(d["q"], d["k"], d["v"], d["beta"], d["g"], d["mask"],
                                               256 ** -0.5)
    _check(to_np(o), to_np(hT), oref, href, "bf16", "deltaproduct full")


def test_deltaproduct_r1_equals_gdn_on_gpu(gdn):
    import torch
    _say("deltaproduct_chunk_fwd r=1 vs gdn_chunk_fwd")
    d = synth.gdn_inputs(1, 150, 2, 128, 64, seed=36, dtype="bf16", h0_std=0.1)
    o1, h1 = _run_gdn(gdn, d, "bf16", 64, scale=0.5)
    q, k, v = (to_dev(d[n], "bf16") for n in ("q", "k", "v"))
    o2, h2 = gdn.deltaproduct_chunk_fwd(q, k, v, to_dev(d["beta"][..., None], "f32"), to_dev(d["g"], "f32"),
                                        [[1.0]], scale=0.5, h0=to_dev(d["h0"], "f32"), chunk=64)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(o2), o1)
    np.testing.assert_array_equal(to_np(h2), h1)
