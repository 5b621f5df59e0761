"""MI355X (gfx950) gated delta rule forward: chunkwise GDN, gated
DeltaProduct, and the camera-branch prep and frame-synchronous scan.

The compute lives in ``libgdn.so`` (HIP kernels behind the C ABI of
``include/gdn.h``); :mod:`.gdn` is its ctypes binding and :mod:`.inputs` the
seeded synthetic input generator.  The binding functions are re-exported
here on first use.
"""

_BINDING = ("gdn_chunk_fwd", "deltaproduct_chunk_fwd", "gdn_recurrent_fwd", "gdn_recurrent_den_fwd", "gdn_prep",
            "gdn_bwd", "gdn_recurrent_bwd", "gdn_prep_bwd", "deltaproduct_bwd")


def __getattr__(name):
    if name in _BINDING:
        from . import gdn as _g
        return getattr(_g, name)
    raise AttributeError(name)
