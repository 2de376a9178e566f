"""Runs the HIP path through the C ABI on seeded batches and compares it with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from tests.helpers import oracle_problem

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "e4m3": torch.uint8}


def fp():
    from block_sparse_long_mean_amd import fp as _fp  # raises if libfp.so is missing
    return _fp


class GpuRun:
    """Device copies of a batch plus the library's buffers and results."""

    def __init__(self, batch, paged=None, alpha=0.1, sink=2, win=4, device="cuda", v_cols=False):
        F = fp()
        self.batch = batch
        self.paged = paged
        dt = TORCH_DT[batch.dtype]
        self.q = batch.q.to(device)
        if paged is None:
            from block_sparse_long_mean_amd import synth

            self.k = batch.k.to(device)
            self.v = (synth.v_columns(batch) if v_cols else batch.v).to(device)
            self.B = F.make_batch(batch.cu, batch.hq, batch.hkv, dt, cu_seqlens_kv=batch.cu_kv,
                                  descale=batch.descale if batch.dtype == "e4m3" else None, v_cols=v_cols)
        else:
            self.k = paged.k_pool.to(device)
            self.v = paged.v_pool.to(device)
            self.B = F.make_batch(batch.cu, batch.hq, batch.hkv, dt, page_table=paged.page_table,
                                  page_size=paged.page_size, num_pool_slots=paged.num_slots,
                                  cu_seqlens_kv=batch.cu_kv, v_cols=v_cols,
                                  descale=batch.descale if batch.dtype == "e4m3" else None)
        self.params = F.select_params(alpha, sink, win)
        self.bufs = F.Buffers(self.B, self.params)
        self.sizes = self.bufs.sizes
        self.out_dtype = torch.float32 if batch.dtype == "f32" else torch.bfloat16

    def select(self, energies=False):
        F = fp()
        e = None
        if energies:
            e = torch.empty(self.sizes.n_segments * self.sizes.max_blocks, dtype=torch.float32,
                            device=self.q.device)
        F.select(self.B, self.params, self.q, self.k, self.v, self.bufs, energies=e)
        torch.cuda.synchronize()
        cu = self.bufs.cu.cpu().numpy()
        idx = self.bufs.idx[: int(cu[-1])].cpu().numpy()
        self.cu_np, self.idx_np = cu, idx
        if e is not None:
            return cu, idx, e.view(self.sizes.n_segments, self.sizes.max_blocks).cpu().numpy()
        return cu, idx

    def attn(self, correction=True, dense=False):
        F = fp()
        out = torch.full((self.batch.total, self.batch.hq, 128), float("nan"), dtype=self.out_dtype,
                         device=self.q.device)
        lse = torch.full((self.batch.total, self.batch.hq), float("nan"), dtype=torch.float32,
                         device=self.q.device)
        if dense:
            F.dense_attn(self.B, self.q, self.k, self.v, self.bufs, out, lse)
        else:
            F.sparse_attn(self.B, self.params, self.q, self.k, self.v, self.bufs, out, lse,
                          correction=correction)
        torch.cuda.synchronize()
        return out, lse

    def device_error(self):
        return fp().read_device_error(self.bufs)


def compare_csr(P: "oracle.Problem", cu, idx, alpha, sink, win, segs=None):
    """CSR parity: per segment the kept block set must equal the oracle's except at
    ambiguous blocks (|e - alpha| <= 1e-4 alpha); the tile list must be the exact
    expansion of the GPU's own block set.  Returns (n_checked, n_ambiguous_diffs)."""
    segs = range(P.num_segments()) if segs is None else segs
    amb_diffs = 0
    for s in segs:
        b, h, I = P.segment_coords(s)
        _, t0, t1, beta = P.tile_info(b, I)
        e, sel, amb, want = P.segment_select(s, alpha, sink, win)
        got = idx[cu[s]:cu[s + 1]]
        assert np.all(np.diff(got) > 0), f"segment {s}: idx not ascending"
        blocks = np.zeros(P.candidates(b, I), bool)
        blocks[np.unique(got // 2)] = True
        # the list must be exactly the expansion of its blocks
        exp = P.csr_tile(blocks.astype(np.uint8), t1)
        np.testing.assert_array_equal(got, exp, err_msg=f"segment {s}: malformed expansion")
        diff = blocks != sel
        bad = diff & ~amb
        assert not bad.any(), (f"segment {s} (b={b},h={h},I={I}): blocks {np.nonzero(bad)[0][:10]} differ "
                               f"outside the band; e={e[bad][:5]}, alpha={alpha}")
        amb_diffs += int(diff.sum())
    return len(list(segs)), amb_diffs


def compare_attn(P, gpu_out, gpu_lse, segs, cu=None, idx=None, dense=False, correction=True, p8=False,
                 ref=None):
    """Oracle rows for the listed segments vs the GPU output; returns (max_abs, mean_abs, lse_max).
    ``ref``: the oracle's (out, lse) of these segments when already computed."""
    if ref is None:
        ref = P.attend_segments(segs, cu, idx, dense=dense, correction=correction, p8=p8)
    ref, ref_lse = ref
    out = gpu_out.float().cpu().numpy()
    lse = gpu_lse.cpu().numpy()
    errs = []
    lerrs = []
    for n, s in enumerate(segs):
        pos, heads, valid = P.rows_of_segment(s)
        g = out[pos[valid], heads[valid]]
        r = ref[n][valid]
        assert np.all(np.isfinite(g)), f"segment {s}: non-finite GPU output"
        errs.append(np.abs(g - r).ravel())
        lerrs.append(np.abs(lse[pos[valid], heads[valid]] - ref_lse[n][valid]))
    e = np.concatenate(errs)
    le = np.concatenate(lerrs)
    return float(e.max()), float(e.mean()), float(le.max())


def check_e4m3(P, gpu_out, gpu_lse, segs, cu, idx, correction, tmax, tmean, note=print):
    """E4M3 bars.  The page's Eq. 15 rounds 2^8 exp(S - m) to E4M3 with m the
    running row maximum, so the kernel's weights are roundings at scales that
    depend on the visiting order; the oracle's Eq. 15 evaluation rounds at the
    final maximum.  Both are roundings of the same weights, so the kernel may sit
    as far from the oracle's Eq. 15 rows as those sit from the exact softmax
    (their mean gap, floor 1e-3); against the exact rows the max bar widens to
    1.25x that gap's max when it exceeds the base bar."""
    ref = P.attend_segments(segs, cu, idx, correction=correction)
    ref8 = P.attend_segments(segs, cu, idx, correction=correction, p8=True)
    mx, mean, lmx = compare_attn(P, gpu_out, gpu_lse, segs, ref=ref)
    mx8, mean8, _ = compare_attn(P, gpu_out, gpu_lse, segs, ref=ref8)
    gaps = []
    for n, s in enumerate(segs):
        valid = P.rows_of_segment(s)[2]
        gaps.append(np.abs(ref8[0][n][valid] - ref[0][n][valid]).ravel())
    gap = np.concatenate(gaps)
    gmax, gmean = float(gap.max()), float(gap.mean())
    note(f"  attention corr={correction}: max {mx:.3e} mean {mean:.3e} lse {lmx:.3e}")
    note(f"  vs Eq.15 oracle: max {mx8:.3e} mean {mean8:.3e}; Eq.15 itself vs exact: max {gmax:.3e} "
         f"mean {gmean:.3e}")
    assert mx8 <= tmax and mean8 <= max(1e-3, gmean), (mx8, mean8, gmean)
    assert mx <= max(tmax, 1.25 * gmax) and mean <= tmean, (mx, mean, gmax)
    return mx, mean


def sample_segments(P, n, seed):
    rng = np.random.default_rng(seed)
    nseg = P.num_segments()
    if nseg <= n:
        return list(range(nseg))
    pick = set(rng.choice(nseg, size=n - 2, replace=False).tolist())
    pick.update({0, nseg - 1})  # first tile and ragged last tile
    return sorted(pick)


def oracle_for(run: GpuRun):
    return oracle_problem(run.batch)
