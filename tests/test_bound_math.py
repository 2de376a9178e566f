"""The index stage scores most blocks with the bf16 hi part of the pooled key
alone and bounds the term it leaves out: for a query row q and a block J with
kbar_J = hi_J + r_J (r_J the exact fp32 remainder),
|q . r_J| <= |q|_2 |lo_J|_2 (1 + 2^-7), where lo_J is r_J rounded to bf16 (the
operand the GPU stores and whose norm pooling writes).  This checks that
inequality on CPU for every (row, block) pair of sampled tiles of the seeded
workloads, with the pooled means from the oracle rounded to fp32 as the GPU
stores them; no GPU code is involved.
"""
import numpy as np
import pytest
import torch

from block_sparse_long_mean_amd import configs, synth
from tests.helpers import oracle_problem


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


@pytest.mark.parametrize("name", ["tiny_2k_f32", "qwen3_30b_a3b_32k_bf16"])
def test_hi_only_error_bound_holds(name):
    w = configs.ALL[name]
    if w.lengths[0] > 4096:
        # the 32K layer's first 4K tokens (same generator, same structure)
        b = synth.make_batch([4096], w.hq, w.hkv, w.d, w.seed, w.dtype, clusters=w.clusters,
                             diag_bias=w.diag_bias)
    else:
        b, _ = w.make()
    P = oracle_problem(b)
    kb, _ = P.pool()
    k32 = kb.astype(np.float32)
    hi = _bf16(k32)
    rem = (k32.astype(np.float64) - hi.astype(np.float64))      # what hi leaves out
    lo = _bf16((k32 - hi).astype(np.float32)).astype(np.float64)  # the stored lo operand
    lo_norm = np.sqrt((lo ** 2).sum(-1))                         # [blocks][hkv]
    q = b.q.float().numpy().astype(np.float64)
    rng = np.random.default_rng(0)
    nseg = P.num_segments()
    worst = 0.0
    for s in sorted(rng.choice(nseg, min(nseg, 24), replace=False)):
        bq, h, I = P.segment_coords(s)
        pos, heads, valid = P.rows_of_segment(s)
        Q = q[pos[valid], heads[valid]]
        nc = P.candidates(bq, I)
        off = P.block_offset(bq)
        R = rem[off:off + nc, h]                                 # [nc, d]
        err = np.abs(Q @ R.T)                                    # [rows, nc]
        bound = np.linalg.norm(Q, axis=1)[:, None] * lo_norm[off:off + nc, h][None, :] * (1 + 2 ** -7)
        assert np.all(err <= bound + 1e-30), float((err - bound).max())
        nz = bound > 0
        worst = max(worst, float((err[nz] / bound[nz]).max()))
    # the bound is not vacuous: the worst case uses a sizeable part of it
    assert 0.05 < worst <= 1.0, worst
