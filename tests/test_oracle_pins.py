"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test names what it pins: library routines (torch's E4M3 decoder and
softmax), closed forms, identities the pages state (AM-GM bound, exactness of
the mean surrogate for constant blocks, second-order accuracy of the mass
surrogate, cancellation of the 2^8 FP8 offset), values the pages print
(Table 7 index sizes), and brute force on tiny inputs.  Sources:
"FlashPrefill V2: Block-Sparse Prefill Attention for Long-Context LLM
Serving" (arXiv 2608.19758) and the FlashPrefill (V1) summary page.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from block_sparse_long_mean_amd import synth
from tests.helpers import f32_problem, oracle_problem

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- E4M3 codec
def test_e4m3_decode_matches_torch_for_all_codes():
    """OCP E4M3FN decode vs torch.float8_e4m3fn, all 256 codes."""
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for c in range(256):
        got = oracle.e4m3_decode(c)
        if math.isnan(ref[c]):
            assert math.isnan(got), c
        else:
            assert got == ref[c], (c, got, ref[c])
    assert oracle.e4m3_decode(0x7E) == 448.0


def test_e4m3_round_nearest_even_and_saturating():
    vals = sorted({oracle.e4m3_decode(c) for c in range(0x7F)})
    for v in vals:
        assert oracle.e4m3_round(v) == v and oracle.e4m3_round(-v) == -v
    # midpoints go to the code with an even mantissa
    for a, b in zip(vals[:-1], vals[1:]):
        mid = 0.5 * (a + b)
        got = oracle.e4m3_round(mid)
        codes = {oracle.e4m3_decode(c): c for c in range(0x7F)}
        assert got in (a, b)
        assert codes[got] % 2 == 0, (a, b, got)
    assert oracle.e4m3_round(500.0) == 448.0 and oracle.e4m3_round(-1e9) == -448.0
    # agrees with torch's round-to-nearest-even conversion inside the range
    rng = np.random.default_rng(3)
    xs = np.concatenate([rng.uniform(-448, 448, 2000), rng.normal(0, 0.01, 500)])
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.e4m3_round(float(x)) for x in xs])
    np.testing.assert_array_equal(got, ref)


# ---------------------------------------------------------------- pooling
def test_pool_closed_forms():
    """Block means of a linear ramp are the midpoints; short last block uses its own count."""
    L, hkv, d = 300, 2, 128
    t = np.arange(L, dtype=np.float32)
    k = np.zeros((L, hkv, d), np.float32)
    v = np.zeros((L, hkv, d), np.float32)
    for h in range(hkv):
        k[:, h, :] = t[:, None] * (h + 1) + np.arange(d, dtype=np.float32)[None, :]
        v[:, h, :] = (t[:, None] // 128) * 10 + h  # constant inside each block
    q = np.zeros((L, 2 * hkv, d), np.float32)
    P = f32_problem([L], 2 * hkv, hkv, d, q, k, v)
    kb, vb = P.pool()
    assert kb.shape == (3, hkv, d)
    mids = [63.5, 191.5, (256 + 299) / 2.0]
    for J in range(3):
        for h in range(hkv):
            np.testing.assert_allclose(kb[J, h], mids[J] * (h + 1) + np.arange(d), rtol=0, atol=1e-9)
            np.testing.assert_allclose(vb[J, h], J * 10 + h, rtol=0, atol=1e-12)


def test_pool_bf16_decodes_like_torch():
    b = synth.make_batch([260], 4, 2, 128, seed=5, dtype="bf16")
    P = oracle_problem(b)
    kb, vb = P.pool()
    kd = b.k.double().numpy()
    vd = b.v.double().numpy()
    for J, (lo, hi) in enumerate([(0, 128), (128, 256), (256, 260)]):
        np.testing.assert_allclose(kb[J], kd[lo:hi].mean(0), rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(vb[J], vd[lo:hi].mean(0), rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- scoring
@pytest.mark.parametrize("lengths,hq,hkv,rows", [([700, 300], 8, 2, 128), ([513], 4, 4, 128),
                                                  ([900], 8, 1, 128), ([1000, 77], 4, 1, 32)])
def test_three_score_forms_agree(lengths, hq, hkv, rows):
    """Direct, V1 (Eq. 1-2) and V2 chunked (Eq. 19-20) energies agree to 1e-12."""
    b = synth.make_batch(lengths, hq, hkv, 128, seed=11, dtype="f32", clusters=True, diag_bias=True)
    P = oracle_problem(b, rows=rows)
    for s in range(P.num_segments()):
        bb, h, I = P.segment_coords(s)
        e0 = P.score_tile(bb, h, I, 0)
        e1 = P.score_tile(bb, h, I, 1)
        e2 = P.score_tile(bb, h, I, 2)
        assert e0.max() == 1.0
        np.testing.assert_allclose(e1, e0, rtol=1e-12, atol=1e-300)
        np.testing.assert_allclose(e2, e0, rtol=1e-12, atol=1e-300)


def test_score_chunked_form_crosses_chunks():
    """More than 64 candidate blocks exercise the chunk rescale of Eq. 20."""
    b = synth.make_batch([64 * 128 + 200], 2, 1, 128, seed=12, dtype="f32", clusters=True)
    P = oracle_problem(b)
    s = P.num_segments() - 1
    bb, h, I = P.segment_coords(s)
    e0 = P.score_tile(bb, h, I, 0)
    assert len(e0) > 64
    np.testing.assert_allclose(P.score_tile(bb, h, I, 2), e0, rtol=1e-12, atol=1e-300)


def test_score_closed_form_one_hot():
    """q_r = a_r e0 and constant blocks k = b_J e0 give s_rJ = sigma a_r b_J exactly."""
    B, R, L, d = 4, 4, 16, 8
    a = np.array([0.5, -1.0, 2.0, 1.5, 0.25, 3.0, -0.5, 1.0, 2.5, 0.0, 1.0, -2.0, 0.75, 1.25, -1.5, 2.0],
                 np.float32)
    bJ = np.array([1.0, -2.0, 0.5, 3.0], np.float32)
    q = np.zeros((L, 1, d), np.float32)
    k = np.zeros((L, 1, d), np.float32)
    q[:, 0, 0] = a
    for J in range(4):
        k[J * B:(J + 1) * B, 0, 0] = bJ[J]
    v = np.zeros_like(k)
    P = f32_problem([L], 1, 1, d, q, k, v, scale=0.5, block=B, rows=R, phys=2)
    for I in range(4):
        rows = range(I * R, I * R + R)
        E = [sum(math.exp(0.5 * float(a[r]) * float(bJ[J])) for r in rows) for J in range(I + 1)]
        mx = max(E)
        want = np.array(E) / mx
        for form in (0, 1, 2):
            np.testing.assert_allclose(P.score_tile(0, 0, I, form), want, rtol=1e-13)


def test_score_shift_invariance_and_stability():
    """A logit offset common to every (row, block) leaves e_J unchanged, even at +1000."""
    rng = np.random.default_rng(7)
    L, g, d = 600, 4, 128
    q = rng.standard_normal((L, g, d)).astype(np.float32)
    k = rng.standard_normal((L, 1, d)).astype(np.float32)
    q[:, :, -1] = 1.0
    k0 = k.copy()
    k0[:, :, -1] = 0.0
    k1 = k.copy()
    k1[:, :, -1] = 1000.0 * math.sqrt(d)
    v = np.zeros_like(k)
    P0 = f32_problem([L], g, 1, d, q, k0, v)
    P1 = f32_problem([L], g, 1, d, q, k1, v)
    for s in range(P0.num_segments()):
        _, _, I = P0.segment_coords(s)
        base = P0.score_tile(0, 0, I, 0)
        for form in (0, 1, 2):
            np.testing.assert_allclose(P1.score_tile(0, 0, I, form), base, rtol=1e-9, atol=1e-300)


# ---------------------------------------------------------------- threshold / CSR
def _forced(beta, n_sink, n_win):
    return {J for J in range(beta + 1) if J < n_sink or beta - n_win <= J < beta or J == beta}


def test_threshold_extremes_and_nesting():
    rng = np.random.default_rng(1)
    for beta in [0, 1, 3, 10, 70]:
        e = rng.uniform(0, 1, beta + 1)
        e[rng.integers(0, beta + 1)] = 1.0
        forced = _forced(beta, 2, 4)
        sel, _ = oracle.Problem.select_tile(e, 0.0, 2, 4)
        assert sel.all()
        sel, _ = oracle.Problem.select_tile(e, 1.5, 2, 4)
        assert set(np.nonzero(sel)[0]) == forced
        sel, _ = oracle.Problem.select_tile(e, 1.0, 2, 4)
        assert set(np.nonzero(sel)[0]) == forced | set(np.nonzero(e == 1.0)[0])
        prev = None
        for alpha in [0.01, 0.05, 0.1, 0.2, 0.5, 0.9]:
            cur = set(np.nonzero(oracle.Problem.select_tile(e, alpha, 2, 4)[0])[0])
            if prev is not None:
                assert cur <= prev
            prev = cur
    # the comparison is inclusive and the band flags near-threshold unforced blocks
    e = np.array([0.1, 0.3, 0.1, 0.10000001, 0.2, 0.05, 0.07, 1.0, 0.5, 0.3])
    sel, amb = oracle.Problem.select_tile(e, 0.1, 0, 0)
    assert sel[2] and sel[3] and not sel[5]
    assert amb[2] and amb[3] and not amb[4] and not amb[9]


def test_csr_structure():
    b = synth.make_batch([1500, 333], 8, 2, 128, seed=3, dtype="f32", clusters=True, diag_bias=True)
    P = oracle_problem(b)
    cu, idx = P.select_all(0.1, 2, 4)
    assert cu[0] == 0 and np.all(np.diff(cu) > 0)
    for s in range(P.num_segments()):
        bb, h, I = P.segment_coords(s)
        _, t0, t1, beta = P.tile_info(bb, I)
        seg = idx[cu[s]:cu[s + 1]]
        assert np.all(np.diff(seg) > 0)
        assert seg.min() >= 0 and seg.max() * 64 <= t1
        blocks = set((seg // 2).tolist())
        assert _forced(beta, 2, 4) <= blocks
        for J in blocks:  # both halves of every kept block, unless causally trimmed
            for p in (2 * J, 2 * J + 1):
                assert (p in seg) == (p * 64 <= t1)


def test_table7_index_memory_golden():
    """CSR per PackGQA M-tile reproduces the printed index sizes; a per-block tile does not."""
    g = json.load(open(os.path.join(GOLDEN, "table7_index_memory.json")))
    for case in g["cases"]:
        L = case["L"]
        P = oracle.Problem.geometry([L], g["hq"], g["hkv"])
        cand = 0
        for s in range(P.num_segments()):
            b, h, I = P.segment_coords(s)
            cand += P.tile_info(b, I)[3] + 1
        csr = 4 * 2 * case["density"] * cand / 2**20
        assert round(csr) == case["csr_mib"], csr
        # one byte per (q head, 128-token q tile, 128-token kv tile)
        mask = g["hq"] * (L // 128) ** 2 / 2**20
        assert round(mask) == case["mask_mib"]
        # the other reading (one segment per 128 positions per KV head) is far off
        Pb = oracle.Problem.geometry([L], g["hq"], g["hkv"], rows=128 * (g["hq"] // g["hkv"]))
        cand_b = sum(Pb.tile_info(*Pb.segment_coords(s)[::2])[3] + 1 for s in range(Pb.num_segments()))
        assert round(4 * 2 * case["density"] * cand_b / 2**20) != case["csr_mib"]


# ---------------------------------------------------------------- attention
def _torch_dense(batch, b, pos_abs, heads):
    """Brute-force causal softmax attention (torch, float64) for given absolute rows."""
    q = batch.q.double()
    k = batch.k.double()
    v = batch.v.double()
    g = batch.hq // batch.hkv
    lo = int(batch.cu[b])
    out = np.zeros((len(pos_abs), batch.d))
    lse = np.zeros(len(pos_abs))
    for n, (p, hd) in enumerate(zip(pos_abs, heads)):
        kk = k[lo:p + 1, hd // g]
        s = (kk @ q[p, hd]) / math.sqrt(batch.d)
        w = torch.softmax(s, 0)
        out[n] = (w[:, None] * v[lo:p + 1, hd // g]).sum(0).numpy()
        lse[n] = float(torch.logsumexp(s, 0))
    return out, lse


def test_dense_matches_torch_softmax():
    b = synth.make_batch([300, 129], 4, 2, 128, seed=21, dtype="f32", clusters=True, diag_bias=True)
    P = oracle_problem(b)
    segs = list(range(P.num_segments()))
    out, lse = P.attend_segments(segs, dense=True)
    for n, s in enumerate(segs):
        bb, _, _ = P.segment_coords(s)
        pos, heads, valid = P.rows_of_segment(s)
        ro, rl = _torch_dense(b, bb, pos[valid], heads[valid])
        np.testing.assert_allclose(out[n][valid], ro, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(lse[n][valid], rl, rtol=1e-12, atol=1e-12)
        assert np.all(out[n][~valid] == 0)


@pytest.mark.parametrize("correction", [True, False])
def test_alpha_zero_equals_dense(correction):
    b = synth.make_batch([1100, 260], 8, 2, 128, seed=22, dtype="f32", clusters=True, diag_bias=True)
    P = oracle_problem(b)
    cu, idx = P.select_all(0.0, 2, 4)
    segs = list(range(P.num_segments()))
    o_s, l_s = P.attend_segments(segs, cu, idx, correction=correction)
    o_d, l_d = P.attend_segments(segs, dense=True)
    np.testing.assert_allclose(o_s, o_d, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l_s, l_d, rtol=1e-13, atol=1e-13)


def test_identical_keys_values_make_correction_exact():
    """Constant blocks: the surrogate |B| e^{s_bar} v_bar is the block's exact term (Eq. 7, delta = 0)."""
    rng = np.random.default_rng(4)
    L, hq, hkv, d = 1024 + 256, 8, 2, 128
    kb = rng.standard_normal((L // 128, hkv, d)).astype(np.float32)
    vb = rng.standard_normal((L // 128, hkv, d)).astype(np.float32)
    k = np.repeat(kb, 128, axis=0)
    v = np.repeat(vb, 128, axis=0)
    q = rng.standard_normal((L, hq, d)).astype(np.float32) * 2
    P = f32_problem([L], hq, hkv, d, q, k, v)
    cu, idx = P.select_all(0.5, 1, 1)
    segs = list(range(P.num_segments()))
    assert len(idx) < sum(2 * (P.tile_info(*P.segment_coords(s)[::2])[3] + 1) for s in segs)
    o_c, l_c = P.attend_segments(segs, cu, idx, correction=True)
    o_n, l_n = P.attend_segments(segs, cu, idx, correction=False)
    o_d, l_d = P.attend_segments(segs, dense=True)
    np.testing.assert_allclose(o_c, o_d, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(l_c, l_d, rtol=1e-12, atol=1e-12)
    assert np.abs(o_n - o_d).max() > 1e-3  # dropping the blocks is visibly wrong


def test_am_gm_orders_the_denominators():
    """n e^{s_bar} <= sum e^{s_i} per block (AM-GM), so LSE_drop <= LSE_corrected <= LSE_dense."""
    b = synth.make_batch([1400], 8, 2, 128, seed=23, dtype="f32", clusters=True, diag_bias=True)
    P = oracle_problem(b)
    cu, idx = P.select_all(0.2, 2, 4)
    segs = list(range(P.num_segments()))
    _, l_c = P.attend_segments(segs, cu, idx, correction=True)
    _, l_n = P.attend_segments(segs, cu, idx, correction=False)
    _, l_d = P.attend_segments(segs, dense=True)
    assert np.all(l_n <= l_c + 1e-12)
    assert np.all(l_c <= l_d + 1e-12)
    assert np.any(l_c > l_n + 1e-3)


def test_mass_surrogate_is_second_order():
    """Halving the within-block spread quarters the mass gap (Eq. 7: 1 + mean(delta^2)/2)."""
    rng = np.random.default_rng(9)
    L, d = 1024, 128
    m = rng.standard_normal((L // 128, 1, d)).astype(np.float64)
    noise = rng.standard_normal((L, 1, d))
    q = rng.standard_normal((L, 1, d))
    v = rng.standard_normal((L, 1, d)).astype(np.float32)
    gaps = []
    for eps in (0.2, 0.1, 0.05):
        k = (np.repeat(m, 128, axis=0) + eps * noise).astype(np.float32)
        P = f32_problem([L], 1, 1, d, q.astype(np.float32), k, v)
        I = P.num_segments() - 1
        _, t0, t1, beta = P.tile_info(0, I)
        # only the diagonal block is exact; every other block is corrected
        idx = [t for t in (2 * beta, 2 * beta + 1) if 64 * t <= t1]
        _, l_c = P.attend_tile(0, 0, I, idx, correction=True)
        _, l_d = P.dense_tile(0, 0, I)
        gaps.append(float(np.mean(l_d - l_c)))
    assert gaps[0] > 0
    r1, r2 = gaps[0] / gaps[1], gaps[1] / gaps[2]
    assert 3.4 < r1 < 4.6 and 3.7 < r2 < 4.3, gaps


def test_fp8_offset_cancels_when_weights_are_exact():
    """With 2^8 e^{a-m} exactly representable, the E4M3 weights reproduce the exact output (Eq. 15)."""
    L, d = 128, 128
    ks = np.arange(L) % 9  # logit -k ln 2 -> weight 2^-k
    q = np.zeros((L, 1, d), np.float32)
    q[:, 0, 0] = 1.0
    k = np.zeros((L, 1, d), np.float32)
    k[:, 0, 0] = -ks * math.log(2.0)
    rng = np.random.default_rng(2)
    v = rng.standard_normal((L, 1, d)).astype(np.float32)
    P = f32_problem([L], 1, 1, d, q, k, v, scale=1.0, rows=8)
    I = P.num_segments() - 1
    idx = [0, 1]
    o, l = P.attend_tile(0, 0, I, idx, correction=False, p8=False)
    o8, l8 = P.attend_tile(0, 0, I, idx, correction=False, p8=True)
    np.testing.assert_allclose(o8, o, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(l8, l, rtol=0, atol=1e-6)


def test_causality():
    """Changing keys/values after a row's position leaves that row unchanged."""
    b = synth.make_batch([700], 4, 1, 128, seed=31, dtype="f32")
    P = oracle_problem(b)
    cu, idx = P.select_all(0.1, 1, 2)
    s = 10
    o1, l1 = P.attend_segments([s], cu, idx)
    o1d, _ = P.attend_segments([s], dense=True)
    pos, _, valid = P.rows_of_segment(s)
    tmax = int(pos[valid].max())
    b.k[tmax + 1:] = 7.0
    b.v[tmax + 1:] = -7.0
    P2 = oracle_problem(b)
    o2, l2 = P2.attend_segments([s], cu, idx)
    o2d, _ = P2.attend_segments([s], dense=True)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    np.testing.assert_array_equal(o1d, o2d)


# ---------------------------------------------------------------- generator
def test_generator_is_seeded_and_structured():
    a = synth.make_batch([500, 260], 8, 2, 128, seed=9, dtype="bf16", clusters=True, diag_bias=True)
    b = synth.make_batch([500, 260], 8, 2, 128, seed=9, dtype="bf16", clusters=True, diag_bias=True)
    assert torch.equal(a.q, b.q) and torch.equal(a.k, b.k) and torch.equal(a.v, b.v)
    c = synth.make_batch([500, 260], 8, 2, 128, seed=10, dtype="bf16")
    assert not torch.equal(a.k, c.k)
    # sinks: the first four keys carry a common direction u that every query also leans on
    k = c.k.float()[:500, 0]
    q = c.q.float()[:500, :4]
    du = k[:4].mean(0) - k[4:128].mean(0)
    qm = q.mean((0, 1))
    assert float(torch.nn.functional.cosine_similarity(du, qm, dim=0)) > 0.6
    e = synth.to_e4m3(a)
    assert e.q.dtype == torch.uint8 and abs(e.descale[1] - float(a.k.abs().max()) / 448) < 1e-6
