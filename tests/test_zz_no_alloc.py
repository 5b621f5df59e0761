"""gdn_chunk_fwd_noalloc (the entry point for callers that cannot allocate)
called through the C ABI: its outputs equal gdn_chunk_fwd's, bit for bit
(the same kernels on the library's static scratch instead of a caller work
space), on two calls in a row, the second with a smaller input; a shape
whose work space exceeds the scratch is rejected before anything runs."""
import ctypes

import numpy as np
import pytest

from chunkwise_gated_delta_gdn_amd import inputs as synth
from tests._helpers import TOL, max_rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu

GDN_DTYPE_F32, GDN_DTYPE_BF16 = 0, 1
NOALLOC_MAX = 128 * 1024 * 1024


@pytest.fixture(scope="module")
def gdn():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from chunkwise_gated_delta_gdn_amd import gdn as g
    return g


def _noalloc_abi(gdn, t, scale, chunk, out_dtype):
    """Call the C entry point directly with preallocated outputs."""
    import torch
    q = t["q"]
    B, T, H, Dk = q.shape
    Dv = t["v"].shape[-1]
    o = torch.full((B, T, H, Dv), float("nan"), dtype=out_dtype, device=q.device)
    hT = torch.full((B, H, Dk, Dv), float("nan"), dtype=torch.float32, device=q.device)
    P = lambda x: ctypes.c_void_p(x.data_ptr()) if x is not None else None
    rc = gdn.lib().gdn_chunk_fwd_noalloc(
        P(q), P(t["k"]), P(t["v"]), P(t["beta"]), P(t["g"]), ctypes.c_float(scale), P(t.get("h0")), P(hT), P(o),
        B, T, H, Dk, Dv, chunk, GDN_DTYPE_BF16 if q.dtype == torch.bfloat16 else GDN_DTYPE_F32,
        GDN_DTYPE_BF16 if out_dtype == torch.bfloat16 else GDN_DTYPE_F32,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, gdn.lib().gdn_last_error()
    torch.cuda.synchronize()
    return o, hT


def _inputs(B, T, H, D, seed, dtype):
    d = synth.gdn_inputs(B, T, H, D, D, seed=seed, dtype=dtype, h0_std=0.1)
    return d, {n: to_dev(d[n], dtype if n in ("q", "k", "v") else "f32") for n in ("q", "k", "v", "beta", "g", "h0")}


@pytest.mark.parametrize("dtype,D,chunk", [("bf16", 128, 64), ("f32", 32, 16)])
def test_noalloc_equals_workspace_entry_on_two_calls(gdn, dtype, D, chunk):
    import oracle
    import torch
    print(f"gdn_chunk_fwd_noalloc vs gdn_chunk_fwd {dtype} D={D} chunk={chunk}", flush=True)
    out_dtype = torch.bfloat16 if dtype == "bf16" else torch.float32
    # first call: the gdn workload's shape (B=2 H=16 T=4096 at D=128), then a smaller one
    shapes = [(2, 4096, 16, 20261), (1, 333, 3, 7)] if D == 128 else [(2, 700, 4, 11), (1, 50, 2, 12)]
    for B, T, H, seed in shapes:
        need = gdn.lib().gdn_chunk_fwd_workspace_bytes(B, T, H, D, D, chunk, GDN_DTYPE_BF16 if dtype == "bf16"
                                                       else GDN_DTYPE_F32)
        assert 0 < need <= NOALLOC_MAX
        d, t = _inputs(B, T, H, D, seed, dtype)
        o1, h1 = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["beta"], t["g"], 0.9, t["h0"], chunk=chunk,
                                   out_dtype=out_dtype)
        torch.cuda.synchronize()
        o2, h2 = _noalloc_abi(gdn, t, 0.9, chunk, out_dtype)
        np.testing.assert_array_equal(to_np(o2), to_np(o1))
        np.testing.assert_array_equal(to_np(h2), to_np(h1))
        # and both within the parity bar of the oracle
        oref, href = oracle.gdn_recurrent(d["q"], d["k"], d["v"], d["beta"], d["g"], 0.9, d["h0"])
        bar = TOL[dtype] + (2.0 ** -8 if out_dtype == torch.bfloat16 else 0.0)
        eo, eh = max_rel_err(to_np(o2), oref), max_rel_err(to_np(h2), href)
        print(f"  B={B} T={T} H={H}: work space {need} B, max rel err o={eo:.2e} hT={eh:.2e}", flush=True)
        assert eo <= bar and eh <= TOL[dtype]


def test_noalloc_rejects_a_shape_beyond_its_scratch(gdn):
    import torch
    print("gdn_chunk_fwd_noalloc rejects an oversized shape", flush=True)
    B, T, H, D = 1, 65536, 16, 128          # the long-context shape: ~315 MB of work space
    need = gdn.lib().gdn_chunk_fwd_workspace_bytes(B, T, H, D, D, 64, GDN_DTYPE_BF16)
    assert need > NOALLOC_MAX
    x = torch.zeros(16, device="cuda")
    p = ctypes.c_void_p(x.data_ptr())      # never dereferenced: the call is rejected first
    rc = gdn.lib().gdn_chunk_fwd_noalloc(p, p, p, p, p, ctypes.c_float(1.0), None, None, p, B, T, H, D, D, 64,
                                         GDN_DTYPE_BF16, GDN_DTYPE_BF16, None)
    assert rc == -3                         # GDN_EWORKSPACE
    assert b"no-allocation" in gdn.lib().gdn_last_error()
