"""The error model behind the E4M3 rounding-tie allowance, checked on the GPU.

The E4M3 attention kernel forms its logits with v_mfma_scale_f32_32x32x64_f8f6f4.
Its fp32 results are not the exact sums: the accumulation keeps about 15 bits
relative to the sum of absolute products.  The Eq. 15 comparisons in the other
tests treat a weight as a rounding tie when an error of 2^-13 sigma sum|q_i k_i|
in its logit could move it across an E4M3 midpoint; this test checks that bound
on tiles of the workloads' own E4M3 keys and queries (the small test batch and
the 128K FP8 layer, sinks and 3x-norm clusters included), using the same MFMA
and lane layout (tests/native/fp8_mfma_probe.hip).
"""
import ctypes as C
import os

import numpy as np
import pytest
import torch

from block_sparse_long_mean_amd import configs, synth

pytestmark = pytest.mark.gpu

LOGIT_ERR = 2.0 ** -13  # the bound the E4M3 tie allowance assumes (tests/gpu_harness.py)


def _probe():
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "libfp8_mfma_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m tests.native.build` or __graft_entry__.build()")
    lib = C.CDLL(path)
    lib.fp8_mfma_probe.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int, C.c_void_p]
    lib.fp8_mfma_probe.restype = C.c_int
    return lib


def _tiles(b, nt, seed):
    rng = np.random.default_rng(seed)
    kc, qc = b.k.numpy(), b.q.numpy()
    g = b.hq // b.hkv
    A = np.zeros((nt, 32, 128), np.uint8)
    B = np.zeros((nt, 32, 128), np.uint8)
    for t in range(nt):
        h = int(rng.integers(0, b.hkv))
        A[t] = kc[rng.integers(0, kc.shape[0], 32), h]
        B[t] = qc[rng.integers(0, qc.shape[0], 32), h * g + rng.integers(0, g, 32)]
    return A, B


@pytest.mark.parametrize("which", ["small", "128k_e4m3"])
def test_fp8_mfma_error_within_tie_model(which):
    print(f"[case] fp8 MFMA accuracy, {which}", flush=True)
    if which == "small":
        b = synth.to_e4m3(synth.make_batch([700, 1400], 32, 4, 128, seed=7, dtype="bf16", clusters=True,
                                           diag_bias=True))
    else:
        b, _ = configs.L128K_FP8.make()
    nt = 1024
    A, B = _tiles(b, nt, seed=3)
    lib = _probe()
    dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    dD = torch.zeros((nt, 32, 32), dtype=torch.float32, device="cuda")
    assert dA.shape == dB.shape == (nt, 32, 128) and dD.shape == (nt, 32, 32)
    rc = lib.fp8_mfma_probe(dA.data_ptr(), dB.data_ptr(), dD.data_ptr(), nt, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0, rc
    D = dD.cpu().double().numpy()
    fa = torch.from_numpy(A).view(torch.float8_e4m3fn).double().numpy()
    fb = torch.from_numpy(B).view(torch.float8_e4m3fn).double().numpy()
    exact = np.einsum("tik,tjk->tij", fa, fb)
    absum = np.einsum("tik,tjk->tij", np.abs(fa), np.abs(fb))
    rel = np.abs(D - exact) / absum
    print(f"  error / sum|products|: max {rel.max():.3e} (2^{np.log2(rel.max()):.2f}), mean {rel.mean():.3e}; "
          f"exact results {(D == exact).mean():.3f}", flush=True)
    assert rel.max() <= LOGIT_ERR, rel.max()
    assert rel.max() > 0  # the accumulation is not exact: the allowance is needed
