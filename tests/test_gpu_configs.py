"""Parity at the workloads' full sizes, in the launch configuration bench.py times.

- 32K bf16: CSR checked for every segment; attention on 256 sampled segments.
- 128K bf16 (alpha 0.1 and 0.2, correction on and off) and 128K E4M3: CSR and
  attention on 64 seeded (KV head, query tile) segments, the first and the
  ragged last tile included; pooled means for every block.
- Paged varlen (16 requests, 64-token pages, NaN-poisoned pool): 4 segments
  per request.
- Length sweep, 4 requests of 4K (full CSR, 256 sampled segments) and of 16K
  (64 sampled segments), correction on and off.
The oracle computes each sampled segment on its own (pooling of all blocks,
scoring, selection, corrected attention on the GPU's own index).
"""
import numpy as np
import pytest
import torch

from block_sparse_long_mean_amd import configs
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
    return check_rows(run, P, out, lse, segs, cu, idx, correction=correction, note=_note)


def test_32k_full_csr_sampled_attention():
    w = configs.L32K
    _note(f"[case] {w.name}")
    b, _ = w.make()
    run = GpuRun(b, alpha=w.alpha, sink=w.sink_blocks, win=w.window_blocks)
    cu, idx = run.select()
    P = oracle_for(run)
    _check_pool(run, P)
    n, amb = compare_csr(P, cu, idx, w.alpha, w.sink_blocks, w.window_blocks)
    _note(f"  CSR: {n} segments, {amb} ambiguous-band differences, density "
          f"{len(idx) / float(run.sizes.idx_capacity):.4f}")
    _attn_check(run, P, sample_segments(P, 256, seed=32), cu, idx, "bf16")
    assert run.device_error() == 0


@pytest.mark.parametrize("alpha", [0.1, 0.2])
def test_128k_bf16_sampled(alpha):
    w = configs.L128K
    _note(f"[case] {w.name} alpha={alpha}")
    b, _ = w.make()
    run = GpuRun(b, alpha=alpha, sink=w.sink_blocks, win=w.window_blocks)
    cu, idx = run.select()
    P = oracle_for(run)
    _check_pool(run, P)
    segs = sample_segments(P, 64, seed=128)
    n, amb = compare_csr(P, cu, idx, alpha, w.sink_blocks, w.window_blocks, segs=segs)
    _note(f"  CSR: {n} sampled segments, {amb} band differences; density "
          f"{len(idx) / float(run.sizes.idx_capacity):.4f}")
    for corr in (True, False):
        _attn_check(run, P, segs, cu, idx, "bf16", correction=corr)
    assert run.device_error() == 0


@pytest.mark.parametrize("alpha", [0.1, 0.2])
def test_128k_fp8_sampled(alpha):
    w = configs.L128K_FP8
    _note(f"[case] {w.name} alpha={alpha}")
    b, _ = w.make()
    run = GpuRun(b, alpha=alpha, sink=w.sink_blocks, win=w.window_blocks)
    cu, idx = run.select()
    P = oracle_for(run)
    _check_pool(run, P)
    segs = sample_segments(P, 64, seed=256)
    n, amb = compare_csr(P, cu, idx, alpha, w.sink_blocks, w.window_blocks, segs=segs)
    _note(f"  CSR: {n} sampled segments, {amb} band differences")
    _attn_check(run, P, segs, cu, idx, "e4m3", correction=True)
    assert run.device_error() == 0


def test_paged_varlen_sampled():
    w = configs.VARLEN
    _note(f"[case] {w.name} lengths={list(w.lengths)}")
    b, pg = w.make()
    run = GpuRun(b, paged=pg, alpha=w.alpha, sink=w.sink_blocks, win=w.window_blocks)
    cu, idx = run.select()
    P = oracle_for(run)
    _check_pool(run, P)
    rng = np.random.default_rng(16)
    segs = []
    start = 0
    for r in range(P.num_reqs):
        ns = P.hkv * P.tiles_in_req(r)
        pick = set(rng.choice(ns, size=min(4, ns), replace=False).tolist())
        pick.add(ns - 1)  # the request's ragged last tile
        segs.extend(start + x for x in sorted(pick))
        start += ns
    n, amb = compare_csr(P, cu, idx, w.alpha, w.sink_blocks, w.window_blocks, segs=segs)
    _note(f"  CSR: {n} sampled segments, {amb} band differences")
    _attn_check(run, P, segs, cu, idx, "bf16", correction=True)
    assert run.device_error() == 0
    # per-request density
    dens = []
    for r in range(P.num_reqs):
        s0 = sum(P.hkv * P.tiles_in_req(x) for x in range(r))
        s1 = s0 + P.hkv * P.tiles_in_req(r)
        cand = sum(2 * (P.tile_info(r, P.segment_coords(s)[2])[3] + 1) for s in range(s0, s1, 97))
        got = sum(int(cu[s + 1] - cu[s]) for s in range(s0, s1, 97))
        dens.append(got / max(1, cand))
    _note("  per-request density (every 97th segment): " + " ".join(f"{d:.3f}" for d in dens))


@pytest.mark.parametrize("name,n_attn,full_csr", [("sweep_4k_x4_bf16", 256, True),
                                                  ("sweep_16k_x4_bf16", 64, False)])
def test_length_sweep_sampled(name, n_attn, full_csr):
    """Length-sweep workloads (4 requests of equal length): the short end of the
    sweep, where every request has few blocks and the forced set dominates."""
    w = configs.ALL[name]
    _note(f"[case] {w.name}")
    b, _ = w.make()
    run = GpuRun(b, alpha=w.alpha, sink=w.sink_blocks, win=w.window_blocks)
    cu, idx = run.select()
    P = oracle_for(run)
    _check_pool(run, P)
    segs = sample_segments(P, n_attn, seed=7)
    n, amb = compare_csr(P, cu, idx, w.alpha, w.sink_blocks, w.window_blocks, segs=None if full_csr else segs)
    _note(f"  CSR: {n} segments, {amb} band differences")
    _attn_check(run, P, segs, cu, idx, "bf16", correction=True)
    _attn_check(run, P, segs, cu, idx, "bf16", correction=False)
    assert run.device_error() == 0
