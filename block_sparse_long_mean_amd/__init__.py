"""FlashPrefill V2 block-sparse causal prefill attention, native to AMD MI355X (gfx950).

The compute path is the C-ABI library ``libfp.so`` (hand-written HIP kernels,
declared in ``include/fp.h``); :mod:`block_sparse_long_mean_amd.fp` is its thin
ctypes binding and raises if the library has not been built.  :mod:`synth` and
:mod:`configs` draw the seeded synthetic workloads.
"""
from . import configs, synth  # noqa: F401

__all__ = ["configs", "synth"]
