"""fp_sparse_attn_static (the no-allocation entry point) against fp_sparse_attn.

For callers that cannot allocate device memory.  Both calls go through the C
ABI on the same inputs and index.  With KV splitting off in the regular call
(FP_MAX_SPLITS=1) the two must agree bit for bit; with the regular call's
default splits they must agree within the attention bars (both are also
checked against the oracle).  Two static calls run in a row on one device, the
second on a smaller batch, so the second sees the first one's leftovers in the
shared scratch.
"""
import os

import numpy as np
import pytest
import torch

from block_sparse_long_mean_amd import synth
from tests.gpu_harness import GpuRun, check_rows, oracle_for, sample_segments

pytestmark = pytest.mark.gpu


def _static(run, correction=True):
    from block_sparse_long_mean_amd import fp

    out = torch.full((run.batch.total, run.batch.hq, 128), float("nan"), dtype=run.out_dtype, device=run.q.device)
    lse = torch.full((run.batch.total, run.batch.hq), float("nan"), dtype=torch.float32, device=run.q.device)
    fp.sparse_attn_static(run.B, run.params, run.q, run.k, run.v, run.bufs.cu, run.bufs.idx, run.bufs.means, out,
                          lse, correction=correction)
    torch.cuda.synchronize()
    return out, lse


def _regular_unsplit(run, correction=True):
    old = os.environ.get("FP_MAX_SPLITS")
    os.environ["FP_MAX_SPLITS"] = "1"
    try:
        return run.attn(correction=correction)
    finally:
        if old is None:
            del os.environ["FP_MAX_SPLITS"]
        else:
            os.environ["FP_MAX_SPLITS"] = old


@pytest.mark.parametrize("first,second", [(("bf16", (1000, 2500, 333)), ("e4m3", (700,))),
                                          (("e4m3", (1300, 900)), ("bf16", (257, 64)))])
def test_static_scratch_matches_workspace_call(first, second):
    for dtype, lengths in (first, second):
        print(f"[case] static scratch {dtype} lengths={lengths}", flush=True)
        b = synth.make_batch(list(lengths), 32, 4, 128, seed=11, dtype="bf16", clusters=True, diag_bias=True)
        if dtype == "e4m3":
            b = synth.to_e4m3(b)
        run = GpuRun(b)
        cu, idx = run.select()
        for corr in (True, False):
            o_s, l_s = _static(run, corr)
            o_u, l_u = _regular_unsplit(run, corr)
            assert torch.isfinite(o_s.float()).all()
            assert torch.equal(o_s, o_u) and torch.equal(l_s, l_u), "static scratch differs from the unsplit call"
            o_r, l_r = run.attn(correction=corr)
            d = float((o_s.float() - o_r.float()).abs().max())
            print(f"  corr={corr}: static == unsplit bit for bit; static vs default splits max {d:.2e}", flush=True)
            P = oracle_for(run)
            segs = sample_segments(P, 32, seed=4)
            check_rows(run, P, o_s, l_s, segs, cu, idx, correction=corr)
        assert run.device_error() == 0
