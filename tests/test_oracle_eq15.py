"""Pins of the oracle's step-by-step [V2] Eq. 15 mode (E4M3 weights rounded
against the running row maximum, "FlashPrefill V2: Block-Sparse Prefill
Attention for Long-Context LLM Serving", §3.3 "FP8 Execution", with the step
order of Eq. 17 and the split partition of Eq. 18).

What pins it, independently of the mode itself:
- unrounded, the same recurrence must give the exact rows of the plain
  attention function for any split count (rescales and merges are exact);
- when every row's maximum sits in its first visited step, the running
  maximum is the final one, so the mode must equal the final-maximum
  evaluation;
- weights 2^8 e^{x - m} that are powers of two are E4M3 values, so rounding
  changes nothing even while the running maximum moves;
- two hand-built rows (one head dimension, scale 1) whose expected outputs
  and log-sum-exps are written out below with torch's own E4M3 conversion:
  a later step raising the maximum rescales the earlier step's rounded sums
  instead of re-rounding its weights, and a correction chunk is a step of
  its own after the listed tiles whose weights carry the 2^7 block factor
  before rounding.
"""
import math

import numpy as np
import pytest
import torch

from block_sparse_long_mean_amd import synth
from tests.helpers import f32_problem, oracle_problem


def _e4m3(x: float) -> float:
    """Round to OCP E4M3FN with torch's conversion (round to nearest even)."""
    return float(torch.tensor([x], dtype=torch.float64).to(torch.float8_e4m3fn).double()[0])


@pytest.mark.parametrize("correction", [True, False])
def test_unrounded_recurrence_equals_exact_rows(correction):
    b = synth.to_e4m3(synth.make_batch([600, 1100, 190], 8, 2, 128, seed=41, dtype="bf16",
                                       clusters=True, diag_bias=True))
    P = oracle_problem(b)
    cu, idx = P.select_all(0.2, 2, 4)
    segs = list(range(P.num_segments()))
    o_ref, l_ref = P.attend_segments(segs, cu, idx, correction=correction)
    rng = np.random.default_rng(5)
    for U in (1, 3, 7):
        ns = rng.integers(1, U + 1, size=len(segs)) if U > 1 else None
        o, l = P.attend_segments_eq15(segs, cu, idx, correction=correction, rounding=False, nsplit=ns)
        np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(l, l_ref, rtol=0, atol=1e-11)
    # rounded, the rows move (the mode is not the exact softmax) but stay close
    o8, l8 = P.attend_segments_eq15(segs, cu, idx, correction=correction)
    assert 1e-4 < np.abs(o8 - o_ref).max() < 0.1


def test_equals_final_max_mode_when_the_first_step_holds_the_maximum():
    """Keys along one direction with logits rising with position: every row's
    maximum is its own key, which lies in the first visited tile (its own 64-key
    tile, listed last); corrected blocks stay far below it."""
    L, d = 512, 128
    rng = np.random.default_rng(8)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    q = np.tile(u, (L, 1))[:, None, :].astype(np.float32)
    coef = 0.45 * np.arange(L) + 0.3 * rng.standard_normal(L)
    coef = np.maximum.accumulate(coef)  # non-decreasing
    k = (coef[:, None] * u[None, :])[:, None, :].astype(np.float32)
    v = rng.standard_normal((L, 1, d)).astype(np.float32)
    P = f32_problem([L], 1, 1, d, q, k, v, scale=1.0, rows=64)
    checked = 0
    for I in range(P.num_segments()):
        _, t0, t1, beta = P.tile_info(0, I)
        # the diagonal block's tiles that start at or before t1, plus one earlier tile
        idx = sorted({t for t in (2 * beta, 2 * beta + 1) if 64 * t <= t1} | ({0} if I >= 3 else set()))
        assert idx[-1] == t0 // 64  # the first visited step is the row's own tile
        for corr in (True, False):
            o, l = P.attend_tile_eq15(0, 0, I, idx, correction=corr)
            of, lf = P.attend_tile(0, 0, I, idx, correction=corr, p8=True)
            np.testing.assert_allclose(o, of, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(l, lf, rtol=0, atol=1e-12)
            checked += 1
    assert checked == 2 * P.num_segments()


def test_power_of_two_weights_are_exact_while_the_maximum_moves():
    """Logits -j ln 2 inside a tile and a step of -3 ln 2 per tile: visited
    backwards, each step raises the running maximum by 2^3, and every rounded
    weight 2^(8 - j) is an E4M3 value."""
    L, d = 256, 1
    j = np.arange(L) % 9
    tile = np.arange(L) // 64
    q = np.ones((L, 1, d), np.float32)
    k = (-(j + 3 * tile)).astype(np.float32)[:, None, None]
    v = np.random.default_rng(6).standard_normal((L, 1, d)).astype(np.float32)
    P = f32_problem([L], 1, 1, d, q, k, v, scale=math.log(2.0), rows=64)
    for I in range(P.num_segments()):
        idx = list(range(I + 1))
        o, l = P.attend_tile(0, 0, I, idx, correction=False)
        for U in (1, 2):
            o8, l8 = P.attend_tile_eq15(0, 0, I, idx, correction=False, nsplit=U)
            np.testing.assert_allclose(o8, o, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(l8, l, rtol=0, atol=1e-12)


def test_hand_case_running_maximum_rescales_rounded_sums():
    """One request of 128 tokens, d = 1, scale 1, 64-row tiles; tile 1 (positions
    64..127) lists key tiles [0, 1].  Row 1 (position 65) sees keys 0..65:
    key 0 has logit x1 = 2 (value 1), keys 1..63 logit -60 (value 0.5), key 64
    logit 0 (value 2), key 65 logit -y with 2^8 e^-y = 2.9 (value 4).
    Eq. 15, visiting tile 1 then tile 0:
      step 1 (m = 0):  P64 = 256, P65 = e4m3(2.9) = 3
      step 2 (m = 2):  sums scaled by e^-2, P0 = 256, the others round to 0
      O = (e^-2 (256*2 + 3*4) + 256*1) / (e^-2 (256 + 3) + 256),
      LSE = 2 + ln(e^-2 (256 + 3) + 256) - ln 256.
    Rounding at the final maximum instead gives e4m3(256 e^-2) and
    e4m3(2.9 e^-2) for keys 64 and 65, a different row."""
    L = 128
    y = math.log(256.0 / 2.9)
    k = np.full(L, -60.0)
    v = np.full(L, 0.5)
    k[0], v[0] = 2.0, 1.0
    k[64], v[64] = 0.0, 2.0
    k[65], v[65] = -y, 4.0
    f = lambda a: np.asarray(a, np.float32).reshape(L, 1, 1)
    q = np.ones((L, 1, 1), np.float32)
    P = f32_problem([L], 1, 1, 1, q, f(k), f(v), scale=1.0, rows=64)
    x1 = float(np.float32(2.0))
    p65 = _e4m3(256.0 * math.exp(float(np.float32(-y))))
    assert p65 == 3.0
    e = math.exp(-x1)
    want_o = (e * (256 * 2 + p65 * 4) + 256 * 1) / (e * (256 + p65) + 256)
    want_l = x1 + math.log(e * (256 + p65) + 256) - math.log(256.0)
    for U in (1, 2):
        o, l = P.attend_tile_eq15(0, 0, 1, [0, 1], correction=True, nsplit=U)
        assert abs(o[1, 0] - want_o) < 1e-12 and abs(l[1] - want_l) < 1e-12, (U, o[1, 0], want_o)
    w64 = _e4m3(256 * e)
    w65 = _e4m3(256 * math.exp(float(np.float32(-y)) - x1))
    final = (2 * w64 + 4 * w65 + 256) / (w64 + w65 + 256)
    of, _ = P.attend_tile(0, 0, 1, [0, 1], correction=True, p8=True)
    assert abs(of[1, 0] - final) < 1e-12
    assert abs(final - want_o) > 1e-3


def test_hand_case_correction_chunk_is_a_later_step():
    """Three blocks of 128 tokens, d = 1, scale 1, 64-row tiles; tile 4
    (positions 256..319, block 2) lists only key tile 4, so blocks 0 and 1 are
    corrected in one chunk visited after it.  Keys are constant per block
    (block 0: a0, block 1: a1), key 256 has logit 0 and value 3.  Row 0
    (position 256) sees key 256 and the two corrected blocks, whose logits
    are c_J = a_J + ln 128 with c0 = ln(2.9 / 256), c1 = 1:
      step 1 (m = 0): P256 = 256
      step 2 (m = 1): sums scaled by e^-1; P_c0 = e4m3(2.9 e^-1), P_c1 = 256
      O = (e^-1 256*3 + P_c0 vb0 + 256 vb1) / (e^-1 256 + P_c0 + 256)."""
    L = 384
    a0 = math.log(2.9 / 256.0) - math.log(128.0)
    a1 = 1.0 - math.log(128.0)
    k = np.zeros(L)
    v = np.zeros(L)
    k[:128], v[:128] = a0, -1.5
    k[128:256], v[128:256] = a1, 0.25
    k[256:], v[256:] = -30.0, 7.0
    k[256], v[256] = 0.0, 3.0
    f = lambda a: np.asarray(a, np.float32).reshape(L, 1, 1)
    q = np.ones((L, 1, 1), np.float32)
    P = f32_problem([L], 1, 1, 1, q, f(k), f(v), scale=1.0, rows=64)
    kb, vb = P.pool()
    c0 = float(kb[0, 0, 0]) + math.log(128.0)
    c1 = float(kb[1, 0, 0]) + math.log(128.0)
    assert abs(c0 - math.log(2.9 / 256)) < 1e-6 and abs(c1 - 1.0) < 1e-6
    m = c1
    pc0 = _e4m3(256 * math.exp(c0 - m))
    pc1 = _e4m3(256 * math.exp(c1 - m))
    e = math.exp(-m)
    vb0, vb1 = float(vb[0, 0, 0]), float(vb[1, 0, 0])
    den = e * 256 + pc0 + pc1
    want_o = (e * 256 * 3.0 + pc0 * vb0 + pc1 * vb1) / den
    want_l = m + math.log(den) - math.log(256.0)
    o, l = P.attend_tile_eq15(0, 0, 4, [4], correction=True)
    assert abs(o[0, 0] - want_o) < 1e-12 and abs(l[0] - want_l) < 1e-12, (o[0, 0], want_o)
    # without correction only key 256 remains
    o, l = P.attend_tile_eq15(0, 0, 4, [4], correction=False)
    assert abs(o[0, 0] - 3.0) < 1e-12 and abs(l[0] - 0.0) < 1e-12


def test_tie_allowance_hand_case():
    """The running-maximum hand case again, with key 65's weight 2^8 e^-y placed on
    the midpoint 2.875 between the E4M3 values 2.75 and 3: an implementation whose
    logits carry any error may take either rounding.  The allowance of row 1 must be the first-order bound on what the
    other rounding changes, written out here for either choice the rounding made:
    S = 0.25 e^-2 (the gap, rescaled into the merged sums), SV = 4 S,
    allow = (SV + S |O|) / (D - S), lallow = -ln(1 - S / D).  Row 0 has no tie."""
    L = 128
    y = math.log(256.0 / 2.875)
    k = np.full(L, -60.0)
    v = np.full(L, 0.5)
    k[0], v[0] = 2.0, 1.0
    k[64], v[64] = 0.0, 2.0
    k[65], v[65] = -y, 4.0
    f = lambda a: np.asarray(a, np.float64).reshape(L, 1, 1)
    q = np.ones((L, 1, 1), np.float64)
    # float64 storage is not an oracle dtype: keep the values exact in float32
    k32 = np.float32(k).astype(np.float64)
    P = f32_problem([L], 1, 1, 1, q.astype(np.float32), f(k32).astype(np.float32), f(v).astype(np.float32),
                    scale=1.0, rows=64)
    # logit error bound 2^-13 sigma sum|q_i k_i|: key 65's weight is known only to a
    # factor e^(+-2^-13 * 4.49), which straddles the midpoint; no other weight is near one
    o, l, allow, lallow = P.attend_tile_eq15(0, 0, 1, [0, 1], correction=True, logit_err=2.0 ** -13)
    w65 = 256.0 * math.exp(float(k32[65]))
    assert abs(w65 - 2.875) < 1e-5
    x1 = float(k32[0])
    e = math.exp(-x1)
    S = 0.25 * e
    hits = 0
    for p65 in (2.75, 3.0):
        D = e * (256 + p65) + 256
        want_o = (e * (256 * 2 + p65 * 4) + 256) / D
        if abs(o[1, 0] - want_o) < 1e-12:
            hits += 1
            assert abs(l[1] - (x1 + math.log(D) - math.log(256.0))) < 1e-12
            assert abs(allow[1] - (4 * S + S * abs(want_o)) / (D - S)) < 1e-14
            assert abs(lallow[1] + math.log(1 - S / D)) < 1e-14
    assert hits == 1
    assert allow[0] == 0.0 and lallow[0] == 0.0
    # the stored key is the float32 rounding of -y, ~1e-7 off the midpoint: a
    # logit error bound far below that leaves no tie
    _, _, allow_s, _ = P.attend_tile_eq15(0, 0, 1, [0, 1], correction=True, logit_err=1e-12)
    assert abs(math.log(w65 / 2.875)) > 4.49 * 1e-12 and allow_s[1] == 0.0
    # no band, no allowance; and the rows themselves do not depend on the band
    o0, l0 = P.attend_tile_eq15(0, 0, 1, [0, 1], correction=True)
    np.testing.assert_array_equal(o0, o)
    np.testing.assert_array_equal(l0, l)
