"""Thin ctypes binding over the libgdn C ABI (``include/gdn.h``).

Argument marshalling only: each function checks that the tensors sit on the
GPU with the expected dtype and shape, allocates the outputs with torch, and
passes raw device pointers and the current HIP stream to the library.  Every
step of the computation runs in the library's HIP kernels; there is no
fallback.  Importing this module raises if ``libgdn.so`` has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_DTYPE_F32 = 0
GDN_DTYPE_BF16 = 1

# every symbol declared in include/gdn.h
EXPORTS = (
    "gdn_last_error", "gdn_abi_version",
    "gdn_chunk_fwd", "gdn_chunk_fwd_workspace_bytes", "gdn_chunk_fwd_noalloc",
    "deltaproduct_chunk_fwd", "deltaproduct_chunk_fwd_workspace_bytes",
    "gdn_recurrent_fwd", "gdn_recurrent_fwd_workspace_bytes",
    "gdn_recurrent_den_fwd", "gdn_recurrent_den_fwd_workspace_bytes",
    "gdn_prep",
    "gdn_bwd", "gdn_bwd_workspace_bytes",
    "gdn_recurrent_bwd", "gdn_recurrent_bwd_workspace_bytes",
    "gdn_prep_bwd", "gdn_prep_bwd_workspace_bytes",
    "deltaproduct_bwd", "deltaproduct_bwd_workspace_bytes",
)


class GdnError(RuntimeError):
    """A non-zero return code from the library, with its message."""

    def __init__(self, name, code, msg):
        super().__init__(f"{name} failed ({code}): {msg}")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it first "
                          "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.gdn_last_error.restype = ctypes.c_char_p
    lib.gdn_last_error.argtypes = []
    lib.gdn_abi_version.restype = I
    lib.gdn_chunk_fwd.argtypes = [P, P, P, P, P, F, P, P, P, I, I, I, I, I, I, I, I, P, Z, P]
    lib.gdn_chunk_fwd.restype = I
    lib.gdn_chunk_fwd_noalloc.argtypes = [P, P, P, P, P, F, P, P, P, I, I, I, I, I, I, I, I, P]
    lib.gdn_chunk_fwd_noalloc.restype = I
    lib.gdn_chunk_fwd_workspace_bytes.argtypes = [I] * 7
    lib.gdn_chunk_fwd_workspace_bytes.restype = Z
    lib.deltaproduct_chunk_fwd.argtypes = [P, P, P, P, P, P, I, F, P, P, P, I, I, I, I, I, I, I, I, P, Z, P]
    lib.deltaproduct_chunk_fwd.restype = I
    lib.deltaproduct_chunk_fwd_workspace_bytes.argtypes = [I] * 8
    lib.deltaproduct_chunk_fwd_workspace_bytes.restype = Z
    lib.gdn_recurrent_fwd.argtypes = [P, P, P, P, P, F, P, P, P, I, I, I, I, I, I, I, P, Z, P]
    lib.gdn_recurrent_fwd.restype = I
    lib.gdn_recurrent_fwd_workspace_bytes.argtypes = [I] * 6
    lib.gdn_recurrent_fwd_workspace_bytes.restype = Z
    lib.gdn_recurrent_den_fwd.argtypes = [P, P, P, P, F, P, P, P, I, I, I, I, I, I, I, P, Z, P]
    lib.gdn_recurrent_den_fwd.restype = I
    lib.gdn_recurrent_den_fwd_workspace_bytes.argtypes = [I] * 6
    lib.gdn_recurrent_den_fwd_workspace_bytes.restype = Z
    lib.gdn_prep.argtypes = [P, P, P, P, P, P, P, F, F, P, P, P, P, P, P, I, I, I, I, I, I, P]
    lib.gdn_prep.restype = I
    lib.gdn_bwd.argtypes = [P, P, P, P, P, F, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, P, Z, P]
    lib.gdn_bwd.restype = I
    lib.gdn_bwd_workspace_bytes.argtypes = [I] * 6
    lib.gdn_bwd_workspace_bytes.restype = Z
    lib.gdn_recurrent_bwd.argtypes = [P, P, P, P, P, F, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, P, Z, P]
    lib.gdn_recurrent_bwd.restype = I
    lib.gdn_recurrent_bwd_workspace_bytes.argtypes = [I] * 6
    lib.gdn_recurrent_bwd_workspace_bytes.restype = Z
    lib.gdn_prep_bwd.argtypes = [P, P, P, P, P, P, P, F, F, P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I,
                                 P, Z, P]
    lib.gdn_prep_bwd.restype = I
    lib.gdn_prep_bwd_workspace_bytes.argtypes = [I] * 4
    lib.gdn_prep_bwd_workspace_bytes.restype = Z
    lib.deltaproduct_bwd.argtypes = [P, P, P, P, P, P, I, F, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, P, Z, P]
    lib.deltaproduct_bwd.restype = I
    lib.deltaproduct_bwd_workspace_bytes.argtypes = [I] * 7
    lib.deltaproduct_bwd_workspace_bytes.restype = Z
    return lib


_lib = _load()


def lib():
    return _lib


def _check(name, rc):
    if rc != 0:
        raise GdnError(name, rc, _lib.gdn_last_error().decode())


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return GDN_DTYPE_F32
    if t == torch.bfloat16:
        return GDN_DTYPE_BF16
    raise TypeError(f"unsupported dtype {t} (float32 or bfloat16)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("libgdn takes GPU tensors only")
            if not t.is_contiguous():
                raise ValueError("libgdn takes contiguous tensors only")


def _f32(t, name):
    if t is not None and t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32")


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _workspace(nbytes, device):
    if nbytes == 0:
        return None, 0
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def gdn_chunk_fwd(q, k, v, beta, log_decay, scale=1.0, h0=None, output_final_state=True,
                  chunk=64, out_dtype=torch.float32):
    """Chunkwise gated delta rule forward.  q,k (B,T,H,Dk); v (B,T,H,Dv);
    beta, log_decay (B,T,H) fp32; h0 (B,H,Dk,Dv) fp32 or None.
    Returns (o (B,T,H,Dv) out_dtype, hT (B,H,Dk,Dv) fp32 or None)."""
    _dev(q, k, v, beta, log_decay, h0)
    _f32(beta, "beta"), _f32(log_decay, "log_decay"), _f32(h0, "h0")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != (B, T, H) or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v shapes or dtypes disagree")
    if beta.shape != (B, T, H) or log_decay.shape != (B, T, H):
        raise ValueError("beta and log_decay must be (B, T, H)")
    if h0 is not None and h0.shape != (B, H, Dk, Dv):
        raise ValueError("h0 must be (B, H, Dk, Dv)")
    o = torch.empty((B, T, H, Dv), dtype=out_dtype, device=q.device)
    hT = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device) if output_final_state else None
    dt = _dtype_code(q.dtype)
    ws, nws = _workspace(_lib.gdn_chunk_fwd_workspace_bytes(B, T, H, Dk, Dv, chunk, dt), q.device)
    rc = _lib.gdn_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_decay), float(scale),
                            _ptr(h0), _ptr(hT), _ptr(o), B, T, H, Dk, Dv, int(chunk), dt,
                            _dtype_code(out_dtype), _ptr(ws), nws, _stream(q.device))
    _check("gdn_chunk_fwd", rc)
    return o, hT


def gdn_chunk_fwd_noalloc(q, k, v, beta, log_decay, scale=1.0, h0=None, output_final_state=True,
                          chunk=64, out_dtype=torch.float32, o=None, hT=None):
    """:func:`gdn_chunk_fwd` on the library's own static scratch (no work-space
    allocation).  ``o`` and ``hT`` may be passed in preallocated, so that the
    call itself allocates nothing.  Calls that overlap on one device race."""
    _dev(q, k, v, beta, log_decay, h0, o, hT)
    _f32(beta, "beta"), _f32(log_decay, "log_decay"), _f32(h0, "h0"), _f32(hT, "hT")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != (B, T, H) or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v shapes or dtypes disagree")
    if beta.shape != (B, T, H) or log_decay.shape != (B, T, H):
        raise ValueError("beta and log_decay must be (B, T, H)")
    if h0 is not None and h0.shape != (B, H, Dk, Dv):
        raise ValueError("h0 must be (B, H, Dk, Dv)")
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=out_dtype, device=q.device)
    elif o.shape != (B, T, H, Dv):
        raise ValueError("o must be (B, T, H, Dv)")
    if hT is None and output_final_state:
        hT = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device)
    elif hT is not None and hT.shape != (B, H, Dk, Dv):
        raise ValueError("hT must be (B, H, Dk, Dv)")
    rc = _lib.gdn_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_decay), float(scale),
                                    _ptr(h0), _ptr(hT), _ptr(o), B, T, H, Dk, Dv, int(chunk),
                                    _dtype_code(q.dtype), _dtype_code(o.dtype), _stream(q.device))
    _check("gdn_chunk_fwd_noalloc", rc)
    return o, hT


def deltaproduct_chunk_fwd(q, k, v, beta, log_decay, step_mask, scale=1.0, h0=None,
                           output_final_state=True, chunk=32, out_dtype=torch.float32):
    """Chunkwise gated DeltaProduct forward.  q,k (B,T,H,r*dk); v (B,T,H,Dv);
    beta (B,T,H,r) fp32; log_decay (B,T,H) fp32; step_mask (r,r) host
    sequence; h0 (B,H,r*dk,Dv) fp32 or None.  Returns (o, hT)."""
    _dev(q, k, v, beta, log_decay, h0)
    _f32(beta, "beta"), _f32(log_decay, "log_decay"), _f32(h0, "h0")
    import numpy as np
    m = np.ascontiguousarray(np.asarray(step_mask, dtype=np.float32))
    r = m.shape[0]
    if m.shape != (r, r):
        raise ValueError("step_mask must be square")
    B, T, H, K = q.shape
    Dv = v.shape[-1]
    if K % r:
        raise ValueError("key width must be a multiple of r")
    dk = K // r
    if k.shape != q.shape or v.shape[:3] != (B, T, H) or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v shapes or dtypes disagree")
    if beta.shape != (B, T, H, r) or log_decay.shape != (B, T, H):
        raise ValueError("beta must be (B,T,H,r) and log_decay (B,T,H)")
    if h0 is not None and h0.shape != (B, H, K, Dv):
        raise ValueError("h0 must be (B, H, r*dk, Dv)")
    o = torch.empty((B, T, H, Dv), dtype=out_dtype, device=q.device)
    hT = torch.empty((B, H, K, Dv), dtype=torch.float32, device=q.device) if output_final_state else None
    dt = _dtype_code(q.dtype)
    ws, nws = _workspace(_lib.deltaproduct_chunk_fwd_workspace_bytes(B, T, H, r, dk, Dv, chunk, dt), q.device)
    rc = _lib.deltaproduct_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_decay),
                                     m.ctypes.data_as(ctypes.c_void_p), r, float(scale), _ptr(h0),
                                     _ptr(hT), _ptr(o), B, T, H, dk, Dv, int(chunk), dt,
                                     _dtype_code(out_dtype), _ptr(ws), nws, _stream(q.device))
    _check("deltaproduct_chunk_fwd", rc)
    return o, hT


def gdn_recurrent_fwd(q, k, v, beta, log_decay, scale=1.0, h0=None, output_final_state=True, reverse=False):
    """Camera-branch frame-synchronous numerator-only scan.  q,k,v (B,H,N,D);
    beta (B,H,N) fp32; log_decay (B,H,F) fp32 (one gate per frame, N = F*S);
    h0 (B,H,D,D) fp32 or None.  Returns (out (B,H,N,D) fp32, hT or None).
    reverse=True runs the anti-causal scan (frame f reads frames f+1..F-1);
    it takes no h0 and returns no hT."""
    if reverse:
        output_final_state = False
    _dev(q, k, v, beta, log_decay, h0)
    _f32(beta, "beta"), _f32(log_decay, "log_decay"), _f32(h0, "h0")
    B, H, N, D = q.shape
    F = log_decay.shape[-1]
    if F == 0 and N == 0:
        S = 1                        # no frames: only hT = h0 is produced
    elif F <= 0 or N % F:
        raise ValueError("N must be a multiple of the number of frames")
    else:
        S = N // F
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v shapes or dtypes disagree")
    if beta.shape != (B, H, N) or log_decay.shape != (B, H, F):
        raise ValueError("beta must be (B,H,N) and log_decay (B,H,F)")
    out = torch.empty((B, H, N, D), dtype=torch.float32, device=q.device)
    hT = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device) if output_final_state else None
    dt = _dtype_code(q.dtype)
    ws, nws = _workspace(_lib.gdn_recurrent_fwd_workspace_bytes(B, H, F, S, D, dt), q.device)
    rc = _lib.gdn_recurrent_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_decay), float(scale),
                                _ptr(h0), _ptr(hT), _ptr(out), B, H, F, S, D, dt, int(bool(reverse)),
                                _ptr(ws), nws, _stream(q.device))
    _check("gdn_recurrent_fwd", rc)
    return out, hT


def gdn_recurrent_den_fwd(q_den, k_z, beta, log_decay, scale=1.0, z0=None, output_final_state=True,
                          reverse=False):
    """Normaliser stream of the frame scan.  q_den, k_z (B,H,N,D); beta (B,H,N)
    fp32; log_decay (B,H,F) fp32; z0 (B,H,D) fp32 or None.  Returns
    (den (B,H,N) fp32, zT (B,H,D) or None).  reverse=True runs the
    anti-causal direction (no z0, no zT)."""
    if reverse:
        output_final_state = False
    _dev(q_den, k_z, beta, log_decay, z0)
    _f32(beta, "beta"), _f32(log_decay, "log_decay"), _f32(z0, "z0")
    B, H, N, D = q_den.shape
    F = log_decay.shape[-1]
    if F == 0 and N == 0:
        S = 1
    elif F <= 0 or N % F:
        raise ValueError("N must be a multiple of the number of frames")
    else:
        S = N // F
    if k_z.shape != q_den.shape or k_z.dtype != q_den.dtype:
        raise ValueError("q_den and k_z shapes or dtypes disagree")
    if beta.shape != (B, H, N) or log_decay.shape != (B, H, F):
        raise ValueError("beta must be (B,H,N) and log_decay (B,H,F)")
    if z0 is not None and z0.shape != (B, H, D):
        raise ValueError("z0 must be (B,H,D)")
    den = torch.empty((B, H, N), dtype=torch.float32, device=q_den.device)
    zT = torch.empty((B, H, D), dtype=torch.float32, device=q_den.device) if output_final_state else None
    dt = _dtype_code(q_den.dtype)
    ws, nws = _workspace(_lib.gdn_recurrent_den_fwd_workspace_bytes(B, H, F, S, D, dt), q_den.device)
    rc = _lib.gdn_recurrent_den_fwd(_ptr(q_den), _ptr(k_z), _ptr(beta), _ptr(log_decay), float(scale), _ptr(z0),
                                    _ptr(zT), _ptr(den), B, H, F, S, D, dt, int(bool(reverse)), _ptr(ws), nws,
                                    _stream(q_den.device))
    _check("gdn_recurrent_den_fwd", rc)
    return den, zT


def gdn_prep(qkv, q_norm_w, k_norm_w, proj_q, proj_kv, rope_cos, rope_sin, k_scale, norm_eps,
             want_inflation=True, out_dtype=None):
    """Camera-branch prep.  qkv (B,N,3,H,D); norm weights (H*D,) fp32 or None;
    proj (B,N,4,4) fp32; rope tables (N,D/2) fp32.  Returns a dict with q, k, v
    (B,H,N,D) in out_dtype (default: qkv's dtype) and k_pre_sq, k_post_sq,
    inflation_sq (B,H,N) fp32."""
    _dev(qkv, q_norm_w, k_norm_w, proj_q, proj_kv, rope_cos, rope_sin)
    for t, n in ((q_norm_w, "q_norm_w"), (k_norm_w, "k_norm_w"), (proj_q, "proj_q"),
                 (proj_kv, "proj_kv"), (rope_cos, "rope_cos"), (rope_sin, "rope_sin")):
        _f32(t, n)
    B, N, three, H, D = qkv.shape
    if three != 3:
        raise ValueError("qkv must be (B, N, 3, H, D)")
    if proj_q.shape != (B, N, 4, 4) or proj_kv.shape != (B, N, 4, 4):
        raise ValueError("projections must be (B, N, 4, 4)")
    if rope_cos.shape != (N, D // 2) or rope_sin.shape != (N, D // 2):
        raise ValueError("rope tables must be (N, D/2)")
    dev = qkv.device
    out_dtype = out_dtype or qkv.dtype
    out = {n: torch.empty((B, H, N, D), dtype=out_dtype, device=dev) for n in ("q", "k", "v")}
    for n in ("k_pre_sq", "k_post_sq"):
        out[n] = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    out["inflation_sq"] = torch.empty((B, H, N), dtype=torch.float32, device=dev) if want_inflation else None
    rc = _lib.gdn_prep(_ptr(qkv), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(proj_q), _ptr(proj_kv),
                       _ptr(rope_cos), _ptr(rope_sin), float(k_scale), float(norm_eps),
                       _ptr(out["q"]), _ptr(out["k"]), _ptr(out["v"]), _ptr(out["k_pre_sq"]),
                       _ptr(out["k_post_sq"]), _ptr(out["inflation_sq"]), B, N, H, D,
                       _dtype_code(qkv.dtype), _dtype_code(out_dtype), _stream(dev))
    _check("gdn_prep", rc)
    return out


def gdn_bwd(q, k, v, beta, log_decay, dout, scale=1.0, h0=None, dhT=None, need_dh0=True):
    """Gradients of :func:`gdn_chunk_fwd`'s (o, hT).  q,k (B,T,H,Dk); v and
    dout (B,T,H,Dv), all of one dtype; beta, log_decay (B,T,H) fp32; h0, dhT
    (B,H,Dk,Dv) fp32 or None.  Returns (dq, dk, dv, dbeta, dlog_decay, dh0),
    fp32 (dh0 None unless need_dh0)."""
    _dev(q, k, v, beta, log_decay, dout, h0, dhT)
    _f32(beta, "beta"), _f32(log_decay, "log_decay"), _f32(h0, "h0"), _f32(dhT, "dhT")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if (k.shape != q.shape or v.shape[:3] != (B, T, H) or dout.shape != v.shape
            or k.dtype != q.dtype or v.dtype != q.dtype or dout.dtype != q.dtype):
        raise ValueError("q, k, v, dout shapes or dtypes disagree")
    if beta.shape != (B, T, H) or log_decay.shape != (B, T, H):
        raise ValueError("beta and log_decay must be (B, T, H)")
    for name, st in (("h0", h0), ("dhT", dhT)):
        if st is not None and st.shape != (B, H, Dk, Dv):
            raise ValueError(f"{name} must be (B, H, Dk, Dv)")
    dev = q.device
    dq = torch.empty((B, T, H, Dk), dtype=torch.float32, device=dev)
    dk = torch.empty((B, T, H, Dk), dtype=torch.float32, device=dev)
    dv = torch.empty((B, T, H, Dv), dtype=torch.float32, device=dev)
    dbeta = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    dg = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    dh0 = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev) if need_dh0 else None
    ws, nws = _workspace(_lib.gdn_bwd_workspace_bytes(B, T, H, Dk, Dv, _dtype_code(q.dtype)), dev)
    rc = _lib.gdn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_decay), float(scale), _ptr(h0),
                      _ptr(dout), _ptr(dhT), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbeta), _ptr(dg),
                      _ptr(dh0), B, T, H, Dk, Dv, _dtype_code(q.dtype), _ptr(ws), nws, _stream(dev))
    _check("gdn_bwd", rc)
    return dq, dk, dv, dbeta, dg, dh0


def deltaproduct_bwd(q, k, v, beta, log_decay, step_mask, dout, scale=1.0, h0=None, dhT=None, need_dh0=True):
    """Gradients of :func:`deltaproduct_chunk_fwd`'s (o, hT) for r = 2 with a
    lower unitriangular step mask [[1, 0], [m, 1]] (bf16).  q,k (B,T,H,2*dk);
    v and dout (B,T,H,Dv); beta (B,T,H,2) and log_decay (B,T,H) fp32; h0, dhT
    (B,H,2*dk,Dv) fp32 or None.  Returns (dq, dk, dv, dbeta, dlog_decay, dh0),
    fp32 (dh0 None unless need_dh0)."""
    _dev(q, k, v, beta, log_decay, dout, h0, dhT)
    _f32(beta, "beta"), _f32(log_decay, "log_decay"), _f32(h0, "h0"), _f32(dhT, "dhT")
    import numpy as np
    m = np.ascontiguousarray(np.asarray(step_mask, dtype=np.float32))
    r = m.shape[0]
    if m.shape != (r, r):
        raise ValueError("step_mask must be square")
    B, T, H, K = q.shape
    Dv = v.shape[-1]
    if K % r:
        raise ValueError("key width must be a multiple of r")
    dk_ = K // r
    if (k.shape != q.shape or v.shape[:3] != (B, T, H) or dout.shape != v.shape
            or k.dtype != q.dtype or v.dtype != q.dtype or dout.dtype != q.dtype):
        raise ValueError("q, k, v, dout shapes or dtypes disagree")
    if beta.shape != (B, T, H, r) or log_decay.shape != (B, T, H):
        raise ValueError("beta must be (B,T,H,r) and log_decay (B,T,H)")
    for name, st in (("h0", h0), ("dhT", dhT)):
        if st is not None and st.shape != (B, H, K, Dv):
            raise ValueError(f"{name} must be (B, H, r*dk, Dv)")
    dev = q.device
    dq = torch.empty((B, T, H, K), dtype=torch.float32, device=dev)
    dk = torch.empty((B, T, H, K), dtype=torch.float32, device=dev)
    dv = torch.empty((B, T, H, Dv), dtype=torch.float32, device=dev)
    dbeta = torch.empty((B, T, H, r), dtype=torch.float32, device=dev)
    dg = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    dh0 = torch.empty((B, H, K, Dv), dtype=torch.float32, device=dev) if need_dh0 else None
    dt = _dtype_code(q.dtype)
    ws, nws = _workspace(_lib.deltaproduct_bwd_workspace_bytes(B, T, H, r, dk_, Dv, dt), dev)
    rc = _lib.deltaproduct_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_decay),
                               m.ctypes.data_as(ctypes.c_void_p), r, float(scale), _ptr(h0), _ptr(dout),
                               _ptr(dhT), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbeta), _ptr(dg), _ptr(dh0),
                               B, T, H, dk_, Dv, dt, _ptr(ws), nws, _stream(dev))
    _check("deltaproduct_bwd", rc)
    return dq, dk, dv, dbeta, dg, dh0


def gdn_recurrent_bwd(q, k, v, beta, log_decay, dout, frames, scale=1.0, h0=None, dhT=None, need_dh0=True):
    """Gradients of :func:`gdn_recurrent_fwd`'s (out, hT), forward direction.
    q, k, v, dout (B,H,N,D) of one dtype; beta (B,H,N) and log_decay
    (B,H,F) fp32; h0, dhT (B,H,D,D) fp32 or None.  Returns (dq, dk, dv,
    dbeta, dlog_decay, dh0), fp32 (dh0 None unless need_dh0)."""
    _dev(q, k, v, beta, log_decay, dout, h0, dhT)
    _f32(beta, "beta"), _f32(log_decay, "log_decay"), _f32(h0, "h0"), _f32(dhT, "dhT")
    B, H, N, D = q.shape
    F = int(frames)
    if F <= 0 or N % F:
        raise ValueError("frames must divide N")
    if (k.shape != q.shape or v.shape != q.shape or dout.shape != q.shape
            or k.dtype != q.dtype or v.dtype != q.dtype or dout.dtype != q.dtype):
        raise ValueError("q, k, v, dout shapes or dtypes disagree")
    if beta.shape != (B, H, N) or log_decay.shape != (B, H, F):
        raise ValueError("beta must be (B, H, N) and log_decay (B, H, F)")
    for name, st in (("h0", h0), ("dhT", dhT)):
        if st is not None and st.shape != (B, H, D, D):
            raise ValueError(f"{name} must be (B, H, D, D)")
    dev = q.device
    dq, dk, dv = (torch.empty((B, H, N, D), dtype=torch.float32, device=dev) for _ in range(3))
    dbeta = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dg = torch.empty((B, H, F), dtype=torch.float32, device=dev)
    dh0 = torch.empty((B, H, D, D), dtype=torch.float32, device=dev) if need_dh0 else None
    dt = _dtype_code(q.dtype)
    ws, nws = _workspace(_lib.gdn_recurrent_bwd_workspace_bytes(B, H, F, N // F, D, dt), dev)
    rc = _lib.gdn_recurrent_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_decay), float(scale), _ptr(h0),
                                _ptr(dout), _ptr(dhT), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbeta), _ptr(dg),
                                _ptr(dh0), B, H, F, N // F, D, dt, _ptr(ws), nws, _stream(dev))
    _check("gdn_recurrent_bwd", rc)
    return dq, dk, dv, dbeta, dg, dh0


def gdn_prep_bwd(qkv, q_norm_w, k_norm_w, proj_q, proj_kv, rope_cos, rope_sin, k_scale, norm_eps,
                 dq, dk, dv, dk_pre_sq=None, dk_post_sq=None, dinflation_sq=None, weight_grads=True,
                 proj_grads=True):
    """Gradients of :func:`gdn_prep`.  Forward arguments as there; dq, dk, dv
    (B,H,N,D) gradients of its q, k, v outputs (bf16 or fp32, one dtype);
    dk_pre_sq, dk_post_sq, dinflation_sq (B,H,N) fp32 or None.  Returns a
    dict: dqkv (B,N,3,H,D) fp32, dq_norm_w and dk_norm_w (H*D) (None unless
    weight_grads), dproj_q and dproj_kv (B,N,4,4) (None unless proj_grads)."""
    _dev(qkv, q_norm_w, k_norm_w, proj_q, proj_kv, rope_cos, rope_sin, dq, dk, dv, dk_pre_sq, dk_post_sq,
         dinflation_sq)
    for name, t in (("q_norm_w", q_norm_w), ("k_norm_w", k_norm_w), ("proj_q", proj_q), ("proj_kv", proj_kv),
                    ("rope_cos", rope_cos), ("rope_sin", rope_sin), ("dk_pre_sq", dk_pre_sq),
                    ("dk_post_sq", dk_post_sq), ("dinflation_sq", dinflation_sq)):
        _f32(t, name)
    B, N, three, H, D = qkv.shape
    if three != 3:
        raise ValueError("qkv must be (B, N, 3, H, D)")
    if dq.shape != (B, H, N, D) or dk.shape != dq.shape or dv.shape != dq.shape:
        raise ValueError("dq, dk, dv must be (B, H, N, D)")
    if dk.dtype != dq.dtype or dv.dtype != dq.dtype:
        raise ValueError("dq, dk, dv must share one dtype")
    dev = qkv.device
    out = {"dqkv": torch.empty((B, N, 3, H, D), dtype=torch.float32, device=dev)}
    out["dq_norm_w"] = torch.empty(H * D, dtype=torch.float32, device=dev) if weight_grads else None
    out["dk_norm_w"] = torch.empty(H * D, dtype=torch.float32, device=dev) if weight_grads else None
    out["dproj_q"] = torch.empty((B, N, 4, 4), dtype=torch.float32, device=dev) if proj_grads else None
    out["dproj_kv"] = torch.empty((B, N, 4, 4), dtype=torch.float32, device=dev) if proj_grads else None
    nws = _lib.gdn_prep_bwd_workspace_bytes(B, N, H, D) if weight_grads else 0
    ws, nws = _workspace(nws, dev)
    rc = _lib.gdn_prep_bwd(_ptr(qkv), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(proj_q), _ptr(proj_kv),
                           _ptr(rope_cos), _ptr(rope_sin), float(k_scale), float(norm_eps), _ptr(dq), _ptr(dk),
                           _ptr(dv), _ptr(dk_pre_sq), _ptr(dk_post_sq), _ptr(dinflation_sq), _ptr(out["dqkv"]),
                           _ptr(out["dq_norm_w"]), _ptr(out["dk_norm_w"]), _ptr(out["dproj_q"]),
                           _ptr(out["dproj_kv"]), B, N, H, D, _dtype_code(qkv.dtype), _dtype_code(dq.dtype),
                           _ptr(ws), nws, _stream(dev))
    _check("gdn_prep_bwd", rc)
    return out
