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


# Bars of the attention checks; every bar is a fixed number.
#   bf16 (and fp32 inputs graded the same way): the target bar of max-abs 2e-2 and
#   mean-abs 2e-3 on O; LSE max-abs 2e-2 (the correction logits use the bf16
#   rounding of the pooled keys, relative error <= 2^-9, which the oracle keeps
#   exact; the 128K layer shows ~1.3e-2).
BAR = {"bf16": {"max": 2e-2, "mean": 2e-3, "lse": 2e-2},
       "f32": {"max": 2e-2, "mean": 2e-3, "lse": 2e-2}}
#   E4M3 against the oracle's Eq. 15 rows (every weight rounded at the running
#   row maximum, in the kernel's step order and KV splits): the kernel differs
#   from them by the E4M3 storage of the pooled means (k-bar as hi + 2^-4 lo,
#   v-bar as one code) and fp32 sums, and where a weight sits on a rounding
#   tie.  The kernel's logits come from FP8 MFMAs whose accumulation keeps
#   about 15 bits relative to the sum of absolute products (measured:
#   <= 2.8e-5 sum|q_i k_i|, tests/test_gpu_fp8_mfma.py asserts 2^-13); a weight
#   that an error of 2^-13 sigma sum|q_i k_i| in its logit (and in the running
#   maximum's) could carry across a midpoint between two E4M3 values has two
#   valid roundings.  The oracle reports per row how far taking the other ones
#   can move the row (max-abs) and its LSE; that allowance is added to the
#   row's max and LSE bars.  The mean bar takes no allowance.
E4M3_EQ15 = {"max": 2e-2, "mean": 5e-4, "lse": 3e-2}
E4M3_LOGIT_ERR = 2.0 ** -13
#   E4M3 against the exact rows: the target bar of max-abs 6e-2, mean-abs 5e-3,
#   LSE 5e-2.  On one test batch (requests of 1000, 2500 and 333 tokens, seed
#   7) Eq. 15 itself, evaluated by the oracle, lies 6.64e-2 from the exact rows;
#   that batch is graded at max-abs 8e-2 against them (E4M3_EXACT_MAX_EQ15_OVER).
E4M3_EXACT = {"max": 6e-2, "mean": 5e-3, "lse": 5e-2}
E4M3_EXACT_MAX_EQ15_OVER = 8e-2


def row_errors(P, gpu_out, gpu_lse, segs, ref_out, ref_lse, allow, lallow):
    """Per valid row: max-abs output error, LSE error, and the oracle's allowances;
    plus the mean-abs error over every element."""
    out = gpu_out.float().cpu().numpy()
    lse = gpu_lse.cpu().numpy()
    err, lerr, al, lal = [], [], [], []
    tot, cnt = 0.0, 0
    for n, s in enumerate(segs):
        pos, heads, valid = P.rows_of_segment(s)
        g = out[pos[valid], heads[valid]]
        assert np.all(np.isfinite(g)), f"segment {s}: non-finite GPU output"
        d = np.abs(g - ref_out[n][valid])
        err.append(d.max(axis=1))
        tot += float(d.sum())
        cnt += d.size
        lerr.append(np.abs(lse[pos[valid], heads[valid]] - ref_lse[n][valid]))
        al.append(allow[n][valid])
        lal.append(lallow[n][valid])
    cat = np.concatenate
    return cat(err), cat(lerr), cat(al), cat(lal), tot / max(cnt, 1)


def split_counts(run, P, segs, cu, idx, correction, dense=False):
    """KV split count U of each listed segment, as the attention scheduler
    assigns it (the launch configuration, restated on the host): with S
    segments, C compute units and w attention workgroups per CU (1 for fp32
    inputs, else 2), at most Umax = min(16, ceil(4 C w / S)) splits (lowered to
    FP_MAX_SPLITS when that is set), and U = min(Umax, ceil(W / 4)) for a
    segment with W steps: its listed tiles (clamped to the causal maximum) plus
    ceil(beta / 64) correction chunks, or every causal tile when dense.  Split u
    takes steps [u ceil(W/U), (u+1) ceil(W/U)) ([V2] §3.3 Eq. 18)."""
    import os
    cus = torch.cuda.get_device_properties(run.q.device).multi_processor_count
    wgs = 1 if run.batch.dtype == "f32" else 2
    nseg = P.num_segments()
    umax = max(1, min(16, -(-4 * cus * wgs // nseg)))
    cap = os.environ.get("FP_MAX_SPLITS")
    if cap and int(cap) >= 1:
        umax = min(umax, min(int(cap), 16))
    out = []
    for s in segs:
        b, _, I = P.segment_coords(s)
        _, _, t1, beta = P.tile_info(b, I)
        if dense:
            W = t1 // 64 + 1
        else:
            T = max(0, min(int(cu[s + 1] - cu[s]), 2 * (t1 // 128 + 1)))
            W = T + ((beta + 63) // 64 if correction else 0)
        out.append(min(umax, max(1, -(-max(W, 1) // 4))))
    return out


def causal_csr(P):
    """The all-causal tile lists (what dense attention visits): every tile p <= t1/64."""
    nseg = P.num_segments()
    lists = []
    for s in range(nseg):
        b, _, I = P.segment_coords(s)
        t1 = P.tile_info(b, I)[2]
        lists.append(np.arange(t1 // 64 + 1, dtype=np.int32))
    cu = np.zeros(nseg + 1, np.int32)
    cu[1:] = np.cumsum([len(x) for x in lists])
    return cu, np.concatenate(lists) if lists else np.zeros(0, np.int32)


def check_e4m3(run, P, gpu_out, gpu_lse, segs, cu, idx, correction, exact_max=None, dense=False,
               note=print):
    """E4M3 rows against the oracle's Eq. 15 rows (tight bar) and its exact rows."""
    exact_max = E4M3_EXACT["max"] if exact_max is None else exact_max
    if dense:
        ref = P.attend_segments(segs, dense=True)
        cu, idx = causal_csr(P)
        correction = False
    else:
        ref = P.attend_segments(segs, cu, idx, correction=correction)
    ns = split_counts(run, P, segs, cu, idx, correction, dense=dense)
    o15, l15, allow, lallow = P.attend_segments_eq15(segs, cu, idx, correction=correction, nsplit=ns,
                                                     logit_err=E4M3_LOGIT_ERR)
    mx, mean, lmx = compare_attn(P, gpu_out, gpu_lse, segs, ref=ref)
    err, lerr, al, lal, mean8 = row_errors(P, gpu_out, gpu_lse, segs, o15, l15, allow, lallow)
    tag = "dense" if dense else f"corr={correction}"
    tied = al > 0
    over = err > E4M3_EQ15["max"]
    note(f"  attention {tag}: vs exact max {mx:.3e} mean {mean:.3e} lse {lmx:.3e}")
    note(f"  vs Eq.15 rows (splits up to {max(ns)}): max {err.max():.3e} (untied rows {err[~tied].max(initial=0):.3e}) "
         f"mean {mean8:.3e} lse {lerr.max():.3e}; {int(tied.sum())}/{len(err)} rows with a rounding tie, "
         f"{int(over.sum())} over the bar within their allowance (largest allowance {al.max():.2e})")
    bad = err > E4M3_EQ15["max"] + al
    lbad = lerr > E4M3_EQ15["lse"] + lal
    assert not bad.any(), (err[bad][:5], al[bad][:5])
    assert not lbad.any(), (lerr[lbad][:5], lal[lbad][:5])
    assert mean8 <= E4M3_EQ15["mean"], mean8
    assert mx <= exact_max and mean <= E4M3_EXACT["mean"] and lmx <= E4M3_EXACT["lse"], (mx, mean, lmx)
    return mx, mean


def check_rows(run, P, gpu_out, gpu_lse, segs, cu=None, idx=None, correction=True, dense=False,
               exact_max=None, note=print):
    """Sampled rows of one attention call against the oracle, at the bars above."""
    if run.batch.dtype == "e4m3":
        return check_e4m3(run, P, gpu_out, gpu_lse, segs, cu, idx, correction, exact_max=exact_max,
                          dense=dense, note=note)
    bar = BAR[run.batch.dtype]
    mx, mean, lmx = compare_attn(P, gpu_out, gpu_lse, segs, cu, idx, dense=dense, correction=correction)
    tag = "dense" if dense else f"corr={correction}"
    note(f"  attention {tag}: max {mx:.3e} mean {mean:.3e} lse {lmx:.3e}")
    assert mx <= bar["max"] and mean <= bar["mean"] and lmx <= bar["lse"], (mx, mean, lmx)
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
