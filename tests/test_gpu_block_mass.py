"""GPU parity of the exact block-mass diagnostic (fp_block_mass) against the oracle.

FlashPrefill (V1) summary page, §3.1 (exact identification; the AM-GM pair
of the pooled surrogate and the true block sum).  The GPU's LSE comes from its
own dense path (for E4M3 inputs, the fp32 path on the decoded values); the
oracle computes its own in fp64.  Bars: masses and
surrogates within 2e-5 absolute and 1e-4 relative where above 1e-3 (fp32
logits from exact bf16 operand products, k_bar and fp32 inputs split into bf16
hi + lo; exp2 of fp32 arguments; fp32 sums of up to 16K terms; observed ~1e-6);
every segment's masses sum to 1 within 1e-4 at full size.
"""
import numpy as np
import pytest
import torch

from block_sparse_long_mean_amd import configs, synth
from tests.gpu_harness import GpuRun, oracle_for, sample_segments

pytestmark = pytest.mark.gpu


def _note(msg):
    print(msg, flush=True)


def _exact_lse(run):
    """Dense LSE of the batch on the GPU.  E4M3 inputs go through the fp32 path on
    their decoded, descaled values: the E4M3 dense path's LSE carries Eq. 15's
    rounding of the weights, and the mass is defined against the exact one."""
    from block_sparse_long_mean_amd import fp

    b = run.batch
    lse = torch.empty((b.total, b.hq), dtype=torch.float32, device="cuda")
    if b.dtype != "e4m3":
        out = torch.empty((b.total, b.hq, 128), dtype=run.out_dtype, device="cuda")
        fp.dense_attn(run.B, run.q, run.k, run.v, run.bufs, out, lse)
        return lse
    dec = [t.view(torch.float8_e4m3fn).float() * c for t, c in zip((run.q, run.k, run.v), b.descale)]
    B32 = fp.make_batch(b.cu, b.hq, b.hkv, torch.float32, cu_seqlens_kv=b.cu_kv)
    bufs = fp.Buffers(B32)
    out = torch.empty((b.total, b.hq, 128), dtype=torch.float32, device="cuda")
    fp.dense_attn(B32, dec[0], dec[1], dec[2], bufs, out, lse)
    return lse


def _gpu_mass(run, surrogate=True):
    from block_sparse_long_mean_amd import fp

    b = run.batch
    assert run.paged is None or b.dtype != "e4m3"
    lse = _exact_lse(run)
    n, mx = run.sizes.n_segments, run.sizes.max_blocks
    mass = torch.full((n, mx), float("nan"), dtype=torch.float32, device="cuda")
    sur = torch.full((n, mx), float("nan"), dtype=torch.float32, device="cuda") if surrogate else None
    fp.block_mass(run.B, run.q, run.k, lse, run.bufs, mass, sur)
    torch.cuda.synchronize()
    assert run.device_error() == 0
    return mass.cpu().numpy(), None if sur is None else sur.cpu().numpy()


def _compare(P, mass, sur, segs, tag):
    m_o, s_o = P.block_mass_segments(segs, max_nc=mass.shape[1])
    worst = [0.0, 0.0, 0.0, 0.0]
    for n, s in enumerate(segs):
        b, _, I = P.segment_coords(s)
        nc = P.candidates(b, I)
        assert np.all(mass[s, nc:] == -1) and np.all(sur[s, nc:] == -1)
        for k, (g, o) in enumerate(((mass[s, :nc], m_o[n, :nc]), (sur[s, :nc], s_o[n, :nc]))):
            d = np.abs(g - o)
            big = o > 1e-3
            worst[2 * k] = max(worst[2 * k], float(d.max()))
            if big.any():
                worst[2 * k + 1] = max(worst[2 * k + 1], float((d[big] / o[big]).max()))
    _note(f"  {tag}: mass max-abs {worst[0]:.2e} rel {worst[1]:.2e}; surrogate max-abs {worst[2]:.2e} "
          f"rel {worst[3]:.2e}")
    assert worst[0] <= 2e-5 and worst[1] <= 1e-4 and worst[2] <= 2e-5 and worst[3] <= 1e-4


@pytest.mark.parametrize("w", [configs.TINY, configs.CHUNK_TINY], ids=lambda w: w.name)
def test_block_mass_fp32_all_segments(w):
    _note(f"[case] block mass {w.name}")
    b, _ = w.make()
    run = GpuRun(b, alpha=w.alpha, sink=w.sink_blocks, win=w.window_blocks)
    run.select()
    mass, sur = _gpu_mass(run)
    P = oracle_for(run)
    _compare(P, mass, sur, list(range(P.num_segments())), w.name)


@pytest.mark.parametrize("dtype", ["bf16", "e4m3"])
def test_block_mass_small_mix(dtype):
    lengths, qlens = (3000, 1300, 777, 2500), (1000, 660, 1, 2500)
    _note(f"[case] block mass mix {dtype}")
    b = synth.make_batch(list(lengths), 32, 4, 128, seed=23, dtype="bf16", clusters=True, diag_bias=True,
                         q_lengths=list(qlens))
    if dtype == "e4m3":
        b = synth.to_e4m3(b)
    run = GpuRun(b)
    run.select()
    mass, sur = _gpu_mass(run)
    P = oracle_for(run)
    _compare(P, mass, sur, sample_segments(P, 64, seed=4), f"mix {dtype}")


def test_block_mass_paged_equals_contiguous():
    w = configs.CHUNK_MIX
    _note(f"[case] block mass {w.name} paged vs contiguous")
    b, pg = w.make()
    rp = GpuRun(b, paged=pg)
    rp.select()
    mp, sp = _gpu_mass(rp)
    rc = GpuRun(b)
    rc.select()
    mc, sc = _gpu_mass(rc)
    np.testing.assert_array_equal(mp, mc)
    np.testing.assert_array_equal(sp, sc)


def test_block_mass_32k_sampled_and_sums():
    w = configs.L32K
    _note(f"[case] block mass {w.name}")
    b, _ = w.make()
    run = GpuRun(b)
    run.select()
    mass, sur = _gpu_mass(run)
    P = oracle_for(run)
    _compare(P, mass, sur, sample_segments(P, 24, seed=5), w.name)
    sums = np.where(mass >= 0, mass, 0).sum(1)
    _note(f"  mass sums: min {sums.min():.6f} max {sums.max():.6f}")
    assert np.abs(sums - 1).max() <= 1e-4
