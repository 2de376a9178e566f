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


def test_segment_geometry_and_recall_stats():
    """bench.py's segment positions match the oracle's tiles; its recall figures
    match per-segment loops over the oracle's masses and index."""
    b = synth.make_batch([1500, 700], 8, 2, 128, seed=12, dtype="f32", clusters=True, diag_bias=True,
                         q_lengths=[411, 700])
    P = oracle_problem(b)
    nseg = P.num_segments()
    t0, t1 = bench.segment_geometry(b.lengths, b.q_lengths, b.hq, b.hkv)
    for s in range(nseg):
        bb, _, I = P.segment_coords(s)
        _, o0, o1, _ = P.tile_info(bb, I)
        assert (t0[s], t1[s]) == (o0, o1)
    cu, idx = P.select_all(0.3, 1, 2)
    m, su = P.block_mass_segments(range(nseg))
    st = bench.recall_stats(m, su, cu, idx, t0, t1, 0.3, 1, 2)
    kept, miss_c, corr_m, corr_s, rec_n, rec_d = [], [], 0.0, 0.0, 0, 0
    for s in range(nseg):
        bb, _, I = P.segment_coords(s)
        beta, nc = P.tile_info(bb, I)[3], P.candidates(bb, I)
        sel = set((idx[cu[s]:cu[s + 1]] // 2).tolist())
        kept.append(sum(m[s, J] for J in sel))
        cj = [J for J in range(beta) if J not in sel]
        miss_c.append(sum(m[s, J] - su[s, J] for J in cj))
        corr_m += sum(m[s, J] for J in cj)
        corr_s += sum(su[s, J] for J in cj)
        mx = m[s, :nc].max()
        star = {J for J in range(nc) if J < 1 or beta - 2 <= J < beta or J >= beta or m[s, J] >= 0.3 * mx}
        rec_n += len(star & sel)
        rec_d += len(star)
    assert abs(st["mass_kept"] - np.mean(kept)) < 1e-12
    assert abs(st["missed_after_correction"] - np.mean(miss_c)) < 1e-12
    assert abs(st["am_gm_ratio_corrected"] - corr_s / corr_m) < 1e-12
    assert st["exact_rule_block_recall"] == rec_n / rec_d
    assert 0 <= st["missed_after_correction"] <= st["missed_without_correction"]


def test_segment_list_selection_matches_the_whole_index():
    """The CPU baseline's OpenMP selection over a segment list gives each listed
    segment exactly the tile list of the whole-problem selection."""
    b = synth.make_batch([900, 2100, 333], 16, 4, 128, seed=13, dtype="bf16", clusters=True, diag_bias=True)
    P = oracle_problem(b)
    cu, idx = P.select_all(0.1, 2, 4)
    segs = [0, 3, 40, 41, P.num_segments() - 1]
    cu2, idx2 = P.select_segments(segs, 0.1, 2, 4)
    for s in range(P.num_segments()):
        want = idx[cu[s]:cu[s + 1]] if s in segs else idx[:0]
        np.testing.assert_array_equal(idx2[cu2[s]:cu2[s + 1]], want)
