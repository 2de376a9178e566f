"""Host arithmetic of bench.py: the FLOP counts it reports, checked by brute
force on small fresh and chunked problems (CSR from the oracle)."""
import numpy as np
import pytest

import bench
from block_sparse_long_mean_amd import synth
from tests.helpers import oracle_problem


def _brute(P, batch, cu, idx, correction):
    """4 d per (packed row, visible key of a listed tile) + 4 d per (packed row,
    block before the tile's first block that no listed tile covers)."""
    tot = 0
    for s in range(P.num_segments()):
        b, h, I = P.segment_coords(s)
        n, t0, t1, beta = P.tile_info(b, I)
        off = batch.lengths[b] - batch.q_lengths[b]
        lst = idx[cu[s]:cu[s + 1]]
        rows, _, valid = P.rows_of_segment(s)
        for r in rows[valid]:
            t = off + int(r) - int(P.cu[b])
            keys = sum(min(64, max(0, t - 64 * int(p) + 1)) for p in lst)
            corr = len(set(range(beta)) - set((lst // 2).tolist())) if correction else 0
            tot += keys + corr
    return 4.0 * 128 * tot


@pytest.mark.parametrize("lengths,qlens", [([700, 300], None), ([1500, 600], [411, 600])])
@pytest.mark.parametrize("correction", [True, False])
def test_csr_work_matches_brute_force(lengths, qlens, correction):
    b = synth.make_batch(lengths, 8, 2, 128, seed=11, dtype="f32", clusters=True, diag_bias=True,
                         q_lengths=qlens)
    P = oracle_problem(b)
    for alpha in (0.0, 0.3):
        cu, idx = P.select_all(alpha, 1, 2)
        alg, execd, dens = bench.csr_work(b.lengths, b.hq, b.hkv, cu, idx, correction, b.q_lengths)
        assert alg == _brute(P, b, cu, idx, correction)
        if alpha == 0.0:
            assert alg == bench.dense_flops(b.lengths, b.hq, b.q_lengths)
            assert dens == 1.0
        assert execd >= alg
