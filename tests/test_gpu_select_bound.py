"""The index stage scores most blocks with the bf16 hi part of the pooled keys
alone and re-scores with hi + lo only the blocks that its bound on the missing
lo term leaves undecided (and the possible maxima).  Requesting the energies
switches every block to hi + lo scoring.  The two must produce the same CSR on
every segment: these tests run both on whole workloads (no oracle involved; the
CSR parity against the oracle is in test_gpu_parity.py and the workload tests).
"""
import numpy as np
import pytest

from block_sparse_long_mean_amd import configs, synth
from tests.gpu_harness import GpuRun

pytestmark = pytest.mark.gpu


def _both(run):
    cu_f, idx_f = run.select()
    cu_e, idx_e, _ = run.select(energies=True)
    return cu_f, idx_f, cu_e, idx_e


@pytest.mark.parametrize("name,alpha,sink,win", [
    ("qwen3_30b_a3b_32k_bf16", 0.1, 2, 4),
    ("qwen3_30b_a3b_32k_bf16", 0.2, 1, 1),
    ("qwen3_30b_a3b_128k_e4m3", 0.1, 2, 4),
    ("chunk_mix_paged_bf16", 0.1, 2, 4),
    ("paged_varlen_16req_bf16", 0.1, 2, 4),
])
def test_bounded_scoring_keeps_the_exact_set(name, alpha, sink, win):
    w = configs.ALL[name]
    print(f"[case] bounded vs exact scoring {name} alpha={alpha}", flush=True)
    b, pg = w.make()
    run = GpuRun(b, paged=pg, alpha=alpha, sink=sink, win=win)
    cu_f, idx_f, cu_e, idx_e = _both(run)
    nseg = len(cu_f) - 1
    same = np.array_equal(cu_f, cu_e) and np.array_equal(idx_f, idx_e)
    if not same:
        diff = [s for s in range(nseg)
                if not np.array_equal(idx_f[cu_f[s]:cu_f[s + 1]], idx_e[cu_e[s]:cu_e[s + 1]])]
        raise AssertionError(f"{len(diff)} of {nseg} segments differ, first {diff[:5]}")
    print(f"  {nseg} segments, {len(idx_f)} entries: identical", flush=True)
    assert run.device_error() == 0


def test_bounded_scoring_extremes():
    """Ragged and single-row tiles, alpha 0 (everything kept) and alpha 1 (only
    blocks tied with the maximum), on tiles from one candidate block (the
    1-token request) to 157 (the 20000-token request)."""
    b = synth.make_batch([1, 130, 2500, 7000, 20000], 32, 4, 128, seed=53, dtype="bf16", clusters=True,
                         diag_bias=True)
    for alpha in (0.0, 1.0, 0.5):
        print(f"[case] extremes alpha={alpha}", flush=True)
        run = GpuRun(b, alpha=alpha, sink=1, win=1)
        cu_f, idx_f, cu_e, idx_e = _both(run)
        assert np.array_equal(cu_f, cu_e) and np.array_equal(idx_f, idx_e)
        assert run.device_error() == 0


def test_random_configurations():
    """Seeded random batches (lengths, head counts, chunk offsets, alpha,
    forced-block counts, bf16 / E4M3): bounded scoring must give the CSR of
    hi + lo scoring of every block, segment for segment."""
    rng = np.random.default_rng(2024)
    for case in range(12):
        hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([1, 2, 4, 8]))
        n = int(rng.integers(1, 4))
        lengths = [int(x) for x in rng.integers(8000, 24000, size=n)]
        qlens = [int(rng.integers(1, L + 1)) if rng.random() < 0.4 else L for L in lengths]
        alpha = float(rng.choice([0.02, 0.1, 0.3, 0.7]))
        sink, win = int(rng.integers(0, 3)), int(rng.integers(0, 5))
        dtype = "e4m3" if rng.random() < 0.3 else "bf16"
        print(f"[case] random {case}: lengths={lengths} q={qlens} hkv={hkv} g={g} alpha={alpha} "
              f"sink={sink} win={win} {dtype}", flush=True)
        b = synth.make_batch(lengths, hkv * g, hkv, 128, seed=100 + case, dtype="bf16", clusters=True,
                             diag_bias=bool(rng.random() < 0.7), q_lengths=qlens)
        if dtype == "e4m3":
            b = synth.to_e4m3(b)
        run = GpuRun(b, alpha=alpha, sink=sink, win=win)
        cu_f, idx_f, cu_e, idx_e = _both(run)
        assert np.array_equal(cu_f, cu_e) and np.array_equal(idx_f, idx_e), case
        assert run.device_error() == 0


@pytest.mark.parametrize("qscale,kscale", [(8.0, 4.0), (0.125, 0.25)])
def test_bounded_scoring_large_and_small_logits(qscale, kscale):
    """Logits scaled up 32x (energies concentrated on few blocks, a wide bound
    that leaves many blocks to re-score) and down 32x (nearly flat energies):
    the CSR still equals that of hi + lo scoring of every block."""
    print(f"[case] scaled logits q x{qscale} k x{kscale}", flush=True)
    b = synth.make_batch([20000, 9000], 16, 2, 128, seed=61, dtype="bf16", clusters=True, diag_bias=True)
    b.q = (b.q.float() * qscale).to(b.q.dtype)  # powers of two: exact in bf16
    b.k = (b.k.float() * kscale).to(b.k.dtype)
    run = GpuRun(b, alpha=0.1, sink=2, win=4)
    cu_f, idx_f, cu_e, idx_e = _both(run)
    assert np.array_equal(cu_f, cu_e) and np.array_equal(idx_f, idx_e)
    assert run.device_error() == 0
