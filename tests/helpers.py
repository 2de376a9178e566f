"""Shared test helpers: bridges from seeded batches to the oracle and the binding."""
from __future__ import annotations

import numpy as np
import torch

import oracle


def oracle_problem(batch, **kw) -> "oracle.Problem":
    return oracle.Problem(batch.cu, batch.hq, batch.hkv, batch.d, batch.dtype,
                          batch.storage(batch.q), batch.storage(batch.k), batch.storage(batch.v),
                          descale=batch.descale, cu_kv=batch.cu_kv, **kw)


def f32_problem(lengths, hq, hkv, d, q, k, v, **kw) -> "oracle.Problem":
    """Oracle problem over explicit float32 numpy arrays [total, H, d]."""
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return oracle.Problem(cu, hq, hkv, d, "f32", np.asarray(q, np.float32),
                          np.asarray(k, np.float32), np.asarray(v, np.float32), **kw)


def to_f64(batch, t: torch.Tensor, which: str) -> torch.Tensor:
    """Decode a batch tensor to float64 (E4M3 codes through torch's own decoder)."""
    if t.dtype == torch.uint8:
        c = batch.descale["qkv".index(which)]
        return t.view(torch.float8_e4m3fn).double() * c
    return t.double()
