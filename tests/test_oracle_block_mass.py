"""Pins of the oracle's exact block mass (the selection-recall diagnostic).

FlashPrefill (V1) summary page, §3.1: exact identification scores every query
against every key, sums the attention within each block and averages over the
tile's queries; its AM-GM argument bounds the pooled surrogate |B| exp(q.k_bar)
by the true block sum.  Pinned against: the softmax normalisation (masses of a
tile sum to 1), torch's softmax by brute force, the closed form for equal
logits, AM-GM equality for constant blocks and the inequality otherwise, and
the (separately pinned) attention oracle's log-sum-exp, which must equal the
mass it keeps exactly plus the surrogate mass it substitutes.
"""
import math

import numpy as np
import pytest
import torch

from block_sparse_long_mean_amd import synth
from tests.helpers import f32_problem, oracle_problem


def _batch(chunked):
    if chunked:
        return synth.make_batch([1500, 700], 8, 2, 128, seed=61, dtype="f32", clusters=True, diag_bias=True,
                                q_lengths=[411, 700])
    return synth.make_batch([1100, 300], 8, 2, 128, seed=62, dtype="f32", clusters=True, diag_bias=True)


@pytest.mark.parametrize("chunked", [False, True])
def test_masses_sum_to_one(chunked):
    P = oracle_problem(_batch(chunked))
    m, s = P.block_mass_segments(range(P.num_segments()))
    for n in range(P.num_segments()):
        b, _, I = P.segment_coords(n)
        nc = P.candidates(b, I)
        assert abs(m[n, :nc].sum() - 1.0) < 1e-12
        assert np.all(m[n, :nc] >= 0) and np.all(m[n, nc:] == -1)


def test_mass_matches_torch_softmax():
    b = _batch(True)
    P = oracle_problem(b)
    g = b.hq // b.hkv
    q, k = b.q.double(), b.k.double()
    for s in (0, 3, P.num_segments() - 1):
        bb, h, I = P.segment_coords(s)
        rows, heads, valid = P.rows_of_segment(s)
        off = b.lengths[bb] - b.q_lengths[bb]
        kv0 = int(b.kv_cu[bb])
        nc = P.candidates(bb, I)
        want = np.zeros(nc)
        for r, hd in zip(rows[valid], heads[valid]):
            t = off + int(r) - int(b.cu[bb])
            p = torch.softmax((k[kv0:kv0 + t + 1, hd // g] @ q[r, hd]) / math.sqrt(b.d), 0).numpy()
            np.add.at(want, np.arange(t + 1) // 128, p)
        want /= valid.sum()
        got, _ = P.block_mass_tile(bb, h, I)
        np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-15)


def test_equal_logits_closed_form():
    """q = 0: every visible key gets 1/(t+1), so mass_J = mean_r |{i in B_J, i <= t_r}| / (t_r + 1)."""
    L, Lq, d = 900, 300, 128
    rng = np.random.default_rng(1)
    q = np.zeros((Lq, 2, d), np.float32)
    k = rng.standard_normal((L, 1, d)).astype(np.float32)
    v = rng.standard_normal((L, 1, d)).astype(np.float32)
    P = f32_problem([Lq], 2, 1, d, q, k, v, cu_kv=np.array([0, L]))
    for s in range(P.num_segments()):
        _, _, I = P.segment_coords(s)
        rows, _, valid = P.rows_of_segment(s)
        ts = L - Lq + rows[valid]
        nc = P.candidates(0, I)
        want = np.zeros(nc)
        for t in ts:
            for J in range(nc):
                want[J] += max(0, min(t + 1, 128 * (J + 1)) - 128 * J) / (t + 1)
        want /= len(ts)
        got, _ = P.block_mass_tile(0, 0, I)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-15)


def test_surrogate_exact_for_constant_blocks_and_below_otherwise():
    rng = np.random.default_rng(4)
    L, hq, hkv, d = 1024 + 256, 4, 1, 128
    kb = rng.standard_normal((L // 128, hkv, d)).astype(np.float32)
    q = rng.standard_normal((L, hq, d)).astype(np.float32)
    v = rng.standard_normal((L, hkv, d)).astype(np.float32)
    const = f32_problem([L], hq, hkv, d, q, np.repeat(kb, 128, axis=0), v)
    noisy = f32_problem([L], hq, hkv, d, q, np.repeat(kb, 128, axis=0)
                        + rng.standard_normal((L, hkv, d)).astype(np.float32), v)
    gap = 0.0
    for s in range(const.num_segments()):
        b, h, I = const.segment_coords(s)
        beta = const.tile_info(b, I)[3]
        m, su = const.block_mass_tile(b, h, I)
        np.testing.assert_allclose(su[:beta], m[:beta], rtol=1e-11)
        assert np.all(su[beta:] == 0)
        m, su = noisy.block_mass_tile(b, h, I)
        assert np.all(su[:beta] <= m[:beta] * (1 + 1e-12))
        gap = max(gap, float(np.max(m[:beta] - su[:beta], initial=0.0)))
    assert gap > 1e-3


@pytest.mark.parametrize("chunked", [False, True])
def test_mass_accounts_for_the_attention_lse(chunked):
    """Per tile, mean_r exp(LSE_sparse,r - LSE_dense,r) = sum of mass over selected blocks
    (+ sum of the surrogate over corrected blocks when correction is on)."""
    b = _batch(chunked)
    P = oracle_problem(b)
    cu, idx = P.select_all(0.3, 1, 2)
    segs = list(range(P.num_segments()))
    _, l_d = P.attend_segments(segs, dense=True)
    m, su = P.block_mass_segments(segs)
    for corr in (True, False):
        _, l_s = P.attend_segments(segs, cu, idx, correction=corr)
        for n, s in enumerate(segs):
            bb, _, I = P.segment_coords(s)
            beta = P.tile_info(bb, I)[3]
            valid = P.rows_of_segment(s)[2]
            sel = np.unique(idx[cu[s]:cu[s + 1]] // 2)
            want = m[n, sel].sum()
            if corr:
                cj = np.setdiff1d(np.arange(beta), sel)
                want += su[n, cj].sum()
            got = np.mean(np.exp(l_s[n][valid] - l_d[n][valid]))
            assert abs(got - want) < 1e-12, (s, corr, got, want)
