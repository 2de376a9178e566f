"""GPU parity of the column-major FP8 V path (v_layout = FP_V_COLS).

FlashPrefill V2 page, §3.3 Eq. 16 (first case): a V that is stored
transposed is consumed as it is and the probabilities are re-arranged in
registers instead.  The values are the same as in the row-major layout, so
the oracle is unchanged; the checks are the E4M3 bars against the oracle,
agreement with the row-major path, and paged (64- and 128-token pages,
unused slots NaN-poisoned) equal bit for bit to contiguous.
"""
import numpy as np
import pytest
import torch

from block_sparse_long_mean_amd import configs, synth
from tests.gpu_harness import GpuRun, check_rows, oracle_for, sample_segments

pytestmark = pytest.mark.gpu

def _note(msg):
    print(msg, flush=True)


def _batch():
    # K/V offsets multiples of 16 (contiguous transposed V); chunks of every kind
    lengths, qlens = (3008, 1312, 784, 2512), (1000, 660, 1, 2512)
    b = synth.make_batch(list(lengths), 32, 4, 128, seed=29, dtype="bf16", clusters=True, diag_bias=True,
                         q_lengths=list(qlens))
    return synth.to_e4m3(b)


def test_vcols_contiguous_matches_oracle_and_rows():
    b = _batch()
    _note("[case] transposed V, contiguous, e4m3 mix")
    rr = GpuRun(b)
    rc = GpuRun(b, v_cols=True)
    cu, idx = rr.select()
    cu2, idx2 = rc.select()
    np.testing.assert_array_equal(cu, cu2)
    np.testing.assert_array_equal(idx, idx2)
    # pooled means from the transposed rows
    from block_sparse_long_mean_amd import fp

    nb_pad = sum((((L + 127) // 128) + 63) // 64 * 64 for L in b.lengths)
    vr = fp.means_f32(rr.bufs, nb_pad, b.hkv)[1]
    vc = fp.means_f32(rc.bufs, nb_pad, b.hkv)[1]
    dv = float((vr - vc).abs().max())
    _note(f"  vbar rows vs columns: {dv:.2e}")
    assert dv <= 1e-5
    P = oracle_for(rc)
    segs = sample_segments(P, 96, seed=6)
    for corr in (True, False):
        oc, lc = rc.attn(correction=corr)
        orow, lrow = rr.attn(correction=corr)
        check_rows(rc, P, oc, lc, segs, cu, idx, correction=corr, note=_note)
        d = float((oc.float() - orow.float()).abs().max())
        _note(f"  corr={corr}: columns vs rows max {d:.2e}")
        assert torch.isfinite(oc.float()).all() and d <= 2e-2
    od, ld = rc.attn(dense=True)
    check_rows(rc, P, od, ld, segs, dense=True, note=_note)
    assert rc.device_error() == 0 and rr.device_error() == 0


@pytest.mark.parametrize("page_size", [64, 128])
def test_vcols_paged_equals_contiguous(page_size):
    b = _batch()
    _note(f"[case] transposed V, paged {page_size} vs contiguous")
    pg = synth.page_kv(b, page_size, seed=3, v_cols=True)
    rp = GpuRun(b, paged=pg, v_cols=True)
    rc = GpuRun(b, v_cols=True)
    cu, idx = rp.select()
    rc.select()
    for corr in (True, False):
        op, lp = rp.attn(correction=corr)
        oc, lc = rc.attn(correction=corr)
        assert torch.isfinite(op.float()).all()
        assert torch.equal(op, oc) and torch.equal(lp, lc)
    op, lp = rp.attn(dense=True)
    oc, lc = rc.attn(dense=True)
    assert torch.equal(op, oc)
    assert rp.device_error() == 0


def test_vcols_128k_sampled():
    w = configs.L128K_FP8
    _note(f"[case] {w.name} transposed V")
    b, _ = w.make()
    run = GpuRun(b, alpha=w.alpha, sink=w.sink_blocks, win=w.window_blocks, v_cols=True)
    cu, idx = run.select()
    P = oracle_for(run)
    segs = sample_segments(P, 48, seed=7)
    out, lse = run.attn(correction=True)
    check_rows(run, P, out, lse, segs, cu, idx, correction=True, note=_note)
    assert run.device_error() == 0
