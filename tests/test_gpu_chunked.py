"""GPU parity of chunked prefill: requests with L_kv keys and L_q <= L_kv
queries at positions L_kv - L_q .. L_kv - 1, the index rebuilt for the chunk
(FlashPrefill V2 page, §4.3 "Compatibility with Chunked Prefill").

- 1000-query chunk of a 3000-token fp32 prompt (offset on no tile or block
  edge, so some tiles span two blocks): full CSR, every segment, correction on
  and off, and the dense path; fp32 bar 1e-4.
- Small bf16 and E4M3 batches mixing chunks, a fresh request, a one-query chunk
  and a request with no queries: full CSR, sampled attention, dense.
- A chunk on a tile edge against the fresh prefill of the same prompt on the
  GPU: the same index and the same rows.
- The last 8K chunk of the 128K layer prompt, and a paged (64-token pages,
  NaN-poisoned pool) varlen mix: sampled segments.
"""
import dataclasses

import numpy as np
import pytest
import torch

from block_sparse_long_mean_amd import configs, synth
from tests.gpu_harness import GpuRun, check_rows, compare_attn, compare_csr, oracle_for, sample_segments

pytestmark = pytest.mark.gpu

def _note(msg):
    print(msg, flush=True)


def _check_pool(run, P):
    from block_sparse_long_mean_amd import fp

    b = run.batch
    kb_o, vb_o = P.pool()
    nb_pad = sum((((L + 127) // 128) + 63) // 64 * 64 for L in b.lengths)
    kb, vb = fp.means_f32(run.bufs, nb_pad, b.hkv)
    kb, vb = kb.cpu().numpy(), vb.cpu().numpy()
    worst = 0.0
    for r in range(len(b.lengths)):
        base = fp.block_base(run.B, r)
        nj = (b.lengths[r] + 127) // 128
        o0 = P.block_offset(r)
        for arr, ref in ((kb, kb_o), (vb, vb_o)):
            d = np.abs(arr[base:base + nj] - ref[o0:o0 + nj]).max() / max(1.0, np.abs(ref[o0:o0 + nj]).max())
            worst = max(worst, float(d))
    assert worst < 2e-6, worst


def _attn_check(run, P, segs, cu, idx, dtype, correction=True):
    assert run.batch.dtype == dtype
    out, lse = run.attn(correction=correction)
    check_rows(run, P, out, lse, segs, cu, idx, correction=correction, note=_note)
    return out, lse


def _rows_untouched(run, out):
    """Every query row is written; the output has exactly total_q rows."""
    assert out.shape[0] == run.batch.total
    assert torch.isfinite(out.float()).all()


def test_chunk_tiny_full_parity():
    w = configs.CHUNK_TINY
    _note(f"[case] {w.name}")
    b, _ = w.make()
    run = GpuRun(b, alpha=w.alpha, sink=w.sink_blocks, win=w.window_blocks)
    cu, idx = run.select()
    P = oracle_for(run)
    _check_pool(run, P)
    n, amb = compare_csr(P, cu, idx, w.alpha, w.sink_blocks, w.window_blocks)
    assert n == P.num_segments() == 32
    segs = list(range(P.num_segments()))
    for corr in (True, False):
        out, lse = run.attn(correction=corr)
        _rows_untouched(run, out)
        mx, mean, lmx = compare_attn(P, out, lse, segs, cu, idx, correction=corr)
        _note(f"  corr={corr}: max {mx:.2e} mean {mean:.2e} lse {lmx:.2e}")
        assert mx < 1e-4 and mean < 1e-5 and lmx < 1e-4
    out, lse = run.attn(dense=True)
    mx, mean, lmx = compare_attn(P, out, lse, segs, dense=True)
    _note(f"  dense: max {mx:.2e} lse {lmx:.2e}")
    assert mx < 1e-4 and lmx < 1e-4
    assert run.device_error() == 0


@pytest.mark.parametrize("dtype", ["bf16", "e4m3"])
def test_chunk_mix_small(dtype):
    lengths, qlens = (3000, 1300, 777, 2500, 640), (1000, 660, 1, 2500, 0)
    _note(f"[case] chunk mix {dtype} lengths={lengths} q_lengths={qlens}")
    b = synth.make_batch(list(lengths), 32, 4, 128, seed=17, dtype="bf16", clusters=True, diag_bias=True,
                         q_lengths=list(qlens))
    if dtype == "e4m3":
        b = synth.to_e4m3(b)
    run = GpuRun(b)
    cu, idx = run.select()
    P = oracle_for(run)
    _check_pool(run, P)
    n, amb = compare_csr(P, cu, idx, 0.1, 2, 4)
    _note(f"  CSR: {n} segments, {amb} band differences")
    segs = sample_segments(P, 96, seed=3)
    for corr in (True, False):
        out, _ = _attn_check(run, P, segs, cu, idx, dtype, correction=corr)
        _rows_untouched(run, out)
    out, lse = run.attn(dense=True)
    check_rows(run, P, out, lse, segs, dense=True, note=_note)
    assert run.device_error() == 0


def test_chunk_on_tile_edge_equals_fresh_on_gpu():
    L, Lq = 5000, 2600  # g = 8: 16 positions per tile; offset 2400 = 150 tiles
    _note(f"[case] chunk {Lq} of {L} vs fresh {L}")
    fresh = synth.make_batch([L], 32, 4, 128, seed=19, dtype="bf16", clusters=True, diag_bias=True)
    chunk = synth.make_batch([L], 32, 4, 128, seed=19, dtype="bf16", clusters=True, diag_bias=True,
                             q_lengths=[Lq])
    rf, rc = GpuRun(fresh), GpuRun(chunk)
    cu_f, idx_f = rf.select()
    cu_c, idx_c = rc.select()
    shift = (L - Lq) * 8 // 128
    nt_f, nt_c = -(-8 * L // 128), -(-8 * Lq // 128)
    for h in range(4):
        for I in range(nt_c):
            sc, sf = h * nt_c + I, h * nt_f + I + shift
            np.testing.assert_array_equal(idx_c[cu_c[sc]:cu_c[sc + 1]], idx_f[cu_f[sf]:cu_f[sf + 1]])
    of, lf = rf.attn()
    oc, lc = rc.attn()
    d = (oc.float() - of[L - Lq:].float()).abs()
    _note(f"  chunk vs fresh rows: max {float(d.max()):.3e}")
    assert float(d.max()) <= 1e-2
    assert float((lc - lf[L - Lq:]).abs().max()) <= 1e-3


@pytest.mark.parametrize("w", [configs.CHUNK_8K, configs.CHUNK_16K], ids=lambda w: w.name)
def test_chunk_of_128k_sampled(w):
    _note(f"[case] {w.name}")
    b, _ = w.make()
    run = GpuRun(b, alpha=w.alpha, sink=w.sink_blocks, win=w.window_blocks)
    cu, idx = run.select()
    P = oracle_for(run)
    _check_pool(run, P)
    segs = sample_segments(P, 48, seed=8)
    n, amb = compare_csr(P, cu, idx, w.alpha, w.sink_blocks, w.window_blocks, segs=segs)
    _note(f"  CSR: {n} sampled segments, {amb} band differences; entries {len(idx)}")
    for corr in (True, False):
        _attn_check(run, P, segs, cu, idx, "bf16", correction=corr)
    out, lse = run.attn(dense=True)
    ds = segs[:: max(1, len(segs) // 8)]
    _note(f"  dense on {len(ds)} segments")
    check_rows(run, P, out, lse, ds, dense=True, note=_note)
    assert run.device_error() == 0


@pytest.mark.parametrize("dtype", ["bf16", "e4m3"])
def test_chunk_mix_paged(dtype):
    """The paged chunk mix (64-token pages; chunks of 8192 queries over 20000
    and 65613 keys, a whole 9001-token prompt, a single query, a request with
    keys only), in bf16 and in E4M3 (per-tensor scales, pooled means on their
    own scale): sampled segments of every request against the oracle."""
    w = dataclasses.replace(configs.CHUNK_MIX, name=configs.CHUNK_MIX.name.replace("bf16", dtype), dtype=dtype)
    _note(f"[case] {w.name} lengths={list(w.lengths)} q_lengths={list(w.q_lengths)}")
    b, pg = w.make()
    run = GpuRun(b, paged=pg, alpha=w.alpha, sink=w.sink_blocks, win=w.window_blocks)
    cu, idx = run.select()
    P = oracle_for(run)
    _check_pool(run, P)
    rng = np.random.default_rng(5)
    segs, start = [], 0
    for r in range(P.num_reqs):
        ns = P.hkv * P.tiles_in_req(r)
        if ns:
            pick = set(rng.choice(ns, size=min(6, ns), replace=False).tolist()) | {0, ns - 1}
            segs.extend(start + x for x in sorted(pick))
        start += ns
    n, amb = compare_csr(P, cu, idx, w.alpha, w.sink_blocks, w.window_blocks, segs=segs)
    _note(f"  CSR: {n} sampled segments, {amb} band differences")
    out, _ = _attn_check(run, P, segs, cu, idx, dtype, correction=True)
    _rows_untouched(run, out)
    assert run.device_error() == 0
