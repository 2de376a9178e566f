"""Benchmark of the block-sparse prefill path on one MI355X.

One step = the whole hot path over one batch: fp_select (pooling, scoring,
selection, CSR) + fp_sparse_attn (sparse attention with mean correction), on
the 128K-token Qwen3-30B-A3B-shaped layer (Hq=32, Hkv=4, d=128, bf16,
alpha=0.1, 2 sink + 4 window blocks).  Inputs are seeded synthetic tensors
already resident in HBM.  Prints ONE JSON line.

  value      effective dense-equivalent TFLOP/s = 2 d Hq sum L(L+1) / t_step
  roofline   the attention kernel's algorithmic FLOP rate vs the bf16 MFMA peak
  extra      per-stage times, the dense baseline on the same kernel, FP8 and
             alpha / correction variants, density
  cpu_baseline  the fp64 oracle on a bounded sample of the same workload
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from block_sparse_long_mean_amd import configs, synth  # noqa: E402

METRIC = "128K sparse-prefill attn ms, eff. TFLOP/s (bf16/fp8), MFMA util vs peak"
PEAK = {"bf16": 2500.0, "e4m3": 5000.0, "f32": 157.3}  # dense MFMA TFLOP/s, MI355X
D = 128


def dense_flops(lengths, hq, q_lengths=None):
    """Causal attention FLOPs (QK^T and PV, 2 flops per multiply-add) of queries at
    positions L - L_q .. L - 1 over keys 0 .. t."""
    q_lengths = lengths if q_lengths is None else q_lengths
    tot = 0.0
    for L, Lq in zip(lengths, q_lengths):
        off = L - Lq
        tot += 2.0 * D * hq * (L * (L + 1) - off * (off + 1))
    return tot


def algorithmic_bytes(batch):
    """Least HBM bytes one attention launch must move: Q and O once, K and V once."""
    eb = {"bf16": 2, "e4m3": 1, "f32": 4}[batch.dtype]
    ob = 4 if batch.dtype == "f32" else 2
    return float(batch.total * batch.hq * D * (eb + ob) + 2 * batch.total_kv * batch.hkv * D * eb)


def csr_work(lengths, hq, hkv, cu, idx, correction, q_lengths=None):
    """Algorithmic and executed attention FLOPs of a CSR (host arithmetic on the index).

    algorithmic: 4 d per (packed row, visible key in a listed tile) + 4 d per
    (packed row, corrected block); executed: 4 d x 128 rows x 64 per step the
    kernel runs (listed tiles + correction chunks with something to correct).
    Queries sit at positions L - L_q .. L - 1 of their request."""
    g = hq // hkv
    q_lengths = lengths if q_lengths is None else q_lengths
    alg = 0.0
    steps = 0
    nsel_blocks = 0
    ncand = 0
    s = 0
    for L, Lq in zip(lengths, q_lengths):
        nt = -(-g * Lq // 128)
        off = L - Lq
        for h in range(hkv):
            for I in range(nt):
                r0, r1 = I * 128, min((I + 1) * 128, g * Lq)
                pos = off + np.arange(r0, r1) // g
                t0, t1 = int(pos[0]), int(pos[-1])
                beta, beta1 = t0 // 128, t1 // 128
                lst = idx[cu[s]:cu[s + 1]]
                full = int(np.count_nonzero(lst < 2 * beta))
                keys = 64 * full + np.zeros(len(pos))
                for p in lst[lst >= 2 * beta]:
                    keys += np.clip(pos - 64 * int(p) + 1, 0, 64)
                blocks = np.unique(lst // 2)
                sel_before = int(np.count_nonzero(blocks < beta))
                corr = (beta - sel_before) if correction else 0
                alg += 4.0 * D * float(keys.sum() + corr * len(pos))
                st = len(lst)
                if correction and beta > 0:
                    selmask = np.zeros(beta, bool)
                    selmask[blocks[blocks < beta]] = True
                    for c0 in range(0, beta, 64):
                        if not selmask[c0:c0 + 64].all():
                            st += 1
                steps += st
                nsel_blocks += len(blocks)
                ncand += beta1 + 1
                s += 1
    execd = 4.0 * D * 128 * 64 * steps
    return alg, execd, nsel_blocks / max(1, ncand)


def recorded_traffic(workload):
    """HBM bytes per attention launch from the committed rocprofv3 byte counters,
    only while the kernel source is the one that was profiled (else None)."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "attn_traffic_128k_bf16.json")
    src = os.path.join(ROOT, "block_sparse_long_mean_amd", "csrc", "attn.hip")
    try:
        rec = json.load(open(path))
        cur = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("workload") != workload or rec.get("attn_hip_sha256") != cur:
        return None
    return float(rec["read_bytes_per_launch"] + rec["write_bytes_per_launch"])


def time_calls(fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record(st)
        fn()
        b.record(st)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


class Case:
    def __init__(self, batch, paged=None, alpha=0.1, sink=2, win=4, dev=None, v_cols=False):
        """``dev``: (q, k, v) already on the device (views are fine), else uploaded.
        ``v_cols``: E4M3 V stored transposed (contiguous only)."""
        from block_sparse_long_mean_amd import fp

        self.fp = fp
        self.batch = batch
        tdt = {"bf16": torch.bfloat16, "e4m3": torch.uint8, "f32": torch.float32}[batch.dtype]
        if dev is not None:
            self.q, self.k, self.v = dev
            self.B = fp.make_batch(batch.cu, batch.hq, batch.hkv, tdt, cu_seqlens_kv=batch.cu_kv,
                                   descale=batch.descale if batch.dtype == "e4m3" else None)
        elif paged is None:
            self.q = batch.q.cuda()
            self.k = batch.k.cuda()
            self.v = (synth.v_columns(batch) if v_cols else batch.v).cuda()
            self.B = fp.make_batch(batch.cu, batch.hq, batch.hkv, tdt, cu_seqlens_kv=batch.cu_kv,
                                   descale=batch.descale if batch.dtype == "e4m3" else None, v_cols=v_cols)
        else:
            self.q = batch.q.cuda()
            self.k, self.v = paged.k_pool.cuda(), paged.v_pool.cuda()
            self.B = fp.make_batch(batch.cu, batch.hq, batch.hkv, tdt, page_table=paged.page_table,
                                   page_size=paged.page_size, num_pool_slots=paged.num_slots,
                                   cu_seqlens_kv=batch.cu_kv,
                                   descale=batch.descale if batch.dtype == "e4m3" else None)
        self.params = fp.select_params(alpha, sink, win)
        self.bufs = fp.Buffers(self.B, self.params)
        odt = torch.float32 if batch.dtype == "f32" else torch.bfloat16
        self.out = torch.empty((batch.total, batch.hq, D), dtype=odt, device="cuda")
        self.lse = torch.empty((batch.total, batch.hq), dtype=torch.float32, device="cuda")

    def select(self):
        self.fp.select(self.B, self.params, self.q, self.k, self.v, self.bufs)

    def attn(self, correction=True):
        self.fp.sparse_attn(self.B, self.params, self.q, self.k, self.v, self.bufs, self.out, self.lse,
                            correction=correction)

    def dense(self):
        self.fp.dense_attn(self.B, self.q, self.k, self.v, self.bufs, self.out, self.lse)

    def csr(self):
        torch.cuda.synchronize()
        cu = self.bufs.cu.cpu().numpy()
        return cu, self.bufs.idx[: int(cu[-1])].cpu().numpy()


def measure(case, steps, warmup, correction=True):
    sel = time_calls(case.select, steps, warmup)
    att = time_calls(lambda: case.attn(correction), steps, warmup)
    cu, idx = case.csr()
    b = case.batch
    alg, execd, density = csr_work(b.lengths, b.hq, b.hkv, cu, idx, correction, b.q_lengths)
    sel_ms, att_ms = float(np.median(sel)), float(np.median(att))
    return {"select_ms": sel_ms, "attn_ms": att_ms, "step_ms": sel_ms + att_ms, "density": density,
            "attn_alg_flop": alg, "attn_exec_flop": execd, "csr_entries": int(len(idx)),
            "csr_mib": len(idx) * 4 / 2**20}


def cpu_baseline(batch, w, n_seg=64):
    """The oracle (fp64, OpenMP over segments on every host thread) on a bounded
    sample: pooling of every block, then scoring, selection and mean-corrected
    attention of n_seg segments.  Also reports the labelled extrapolation of one
    whole call: pooling time + the sample's wall time scaled to every segment."""
    import oracle
    from tests.helpers import oracle_problem

    P = oracle_problem(batch)
    t0 = time.time()
    P.pool()
    t_pool = time.time() - t0
    nseg = P.num_segments()
    rng = np.random.default_rng(0)
    n_seg = min(n_seg, nseg // 2)
    segs = sorted(2 * x for x in rng.choice(nseg // 2, size=n_seg, replace=False).tolist())  # non-adjacent
    t1 = time.time()
    cu, idx = P.select_segments(segs, w.alpha, w.sink_blocks, w.window_blocks)
    t_sel = time.time() - t1
    P.attend_segments(segs, cu, idx, correction=True)
    t_seg = time.time() - t1
    flops = 0.0
    for s in segs:
        b, _, _ = P.segment_coords(s)
        rows, _, valid = P.rows_of_segment(s)
        off = batch.lengths[b] - batch.q_lengths[b]
        flops += float(np.sum(4.0 * D * (off + rows[valid] - P.cu[b] + 1)))
    # dense-equivalent rate of the sampled rows, charging the pooling pro rata
    total_rows = batch.total * batch.hq
    sample_rows = n_seg * 128
    t = t_seg + t_pool * sample_rows / total_rows
    full_s = t_pool + t_seg * nseg / n_seg
    return {"value": flops / t / 1e12, "unit": "TFLOP/s (dense-equivalent)", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{n_seg} of {nseg} (KV head, query tile) segments: scoring, selection and "
                      f"mean-corrected attention (all OpenMP over segments), plus pooling of all blocks "
                      f"charged pro rata (pool {t_pool:.2f} s, selection {t_sel:.1f} s, segments {t_seg:.1f} s)",
            "extrapolated_full_call_s": full_s,
            "extrapolated_note": "extrapolation, not a measurement: pooling of every block + the sampled "
                                 "segments' wall time x (all segments / sampled segments), on the same threads",
            "nproc": os.cpu_count()}


def other_workloads(args):
    """The 32K layer and the paged varlen batch, timed like the headline workload
    (select, attention, density, algorithmic attention TFLOP/s and its fraction
    of the bf16 MFMA peak, dense-equivalent rate of the step)."""
    out = {}
    for w in (configs.L32K, configs.VARLEN):
        batch, paged = w.make()
        case = Case(batch, paged, w.alpha, w.sink_blocks, w.window_blocks)
        m = measure(case, max(3, args.steps // 2), max(1, args.warmup))
        F = dense_flops(batch.lengths, batch.hq, batch.q_lengths)
        alg = m["attn_alg_flop"] / (m["attn_ms"] / 1e3) / 1e12
        out[w.name] = {"num_reqs": len(batch.lengths), "total_tokens": int(sum(batch.lengths)),
                       "paged": bool(w.page_size), "select_ms": m["select_ms"], "attn_ms": m["attn_ms"],
                       "step_ms": m["step_ms"], "density": m["density"],
                       "eff_tflops": F / (m["step_ms"] / 1e3) / 1e12, "attn_alg_tflops": alg,
                       "attn_roofline_frac": alg / PEAK[batch.dtype],
                       "mfma_util_executed": m["attn_exec_flop"] / (m["attn_ms"] / 1e3) / 1e12 / PEAK[batch.dtype]}
        del case, batch, paged
        torch.cuda.empty_cache()
    return out


def sweep(args):
    """Speedup over the dense baseline and density against length (4 requests
    of L tokens each, 4K..128K), one JSON line per length."""
    for w in configs.SWEEP:
        batch, _ = w.make()
        case = Case(batch, None, w.alpha, w.sink_blocks, w.window_blocks)
        m = measure(case, max(3, args.steps // 2), max(1, args.warmup))
        d_ms = float(np.median(time_calls(case.dense, 3, 1)))
        F = dense_flops(batch.lengths, batch.hq, batch.q_lengths)
        print(json.dumps({
            "sweep": w.name, "L": batch.lengths[0], "num_reqs": len(batch.lengths),
            "select_ms": m["select_ms"], "attn_ms": m["attn_ms"], "step_ms": m["step_ms"],
            "dense_ms": d_ms, "speedup_vs_dense": d_ms / m["step_ms"],
            "select_share": m["select_ms"] / m["step_ms"], "density": m["density"],
            "eff_tflops": F / (m["step_ms"] / 1e3) / 1e12,
            "attn_alg_tflops": m["attn_alg_flop"] / (m["attn_ms"] / 1e3) / 1e12}), flush=True)
        del case, batch
        torch.cuda.empty_cache()


def chunked(args):
    """The 128K prompt of the headline layer prefilled in chunks of 8K and 16K
    tokens, the index rebuilt for every chunk: per chunk size, the summed select,
    attention and dense-baseline times over all chunks, next to the same prompt
    in one pass.  One JSON line per chunk size."""
    w = configs.L128K
    batch, _ = w.make()
    L = batch.lengths[0]
    dq, dk, dv = batch.q.cuda(), batch.k.cuda(), batch.v.cuda()
    reps, warm = max(3, args.steps // 2), max(1, args.warmup)
    whole = Case(batch, None, w.alpha, w.sink_blocks, w.window_blocks, dev=(dq, dk, dv))
    m = measure(whole, reps, warm)
    whole_dense = float(np.median(time_calls(whole.dense, 3, 1)))
    del whole
    for C in (8192, 16384):
        tot = {"select_ms": 0.0, "attn_ms": 0.0, "dense_ms": 0.0, "alg": 0.0, "sel": 0.0, "cand": 0.0}
        for stop in range(C, L + 1, C):
            ch = synth.prefix_chunk(batch, stop, C)
            case = Case(ch, None, w.alpha, w.sink_blocks, w.window_blocks,
                        dev=(dq[stop - C:stop], dk[:stop], dv[:stop]))
            mc = measure(case, reps, warm)
            tot["select_ms"] += mc["select_ms"]
            tot["attn_ms"] += mc["attn_ms"]
            tot["dense_ms"] += float(np.median(time_calls(case.dense, 3, 1)))
            tot["alg"] += mc["attn_alg_flop"]
            del case
        step = tot["select_ms"] + tot["attn_ms"]
        print(json.dumps({
            "chunked": w.name, "chunk": C, "n_chunks": L // C,
            "select_ms": tot["select_ms"], "attn_ms": tot["attn_ms"], "step_ms": step,
            "dense_ms": tot["dense_ms"], "speedup_vs_dense": tot["dense_ms"] / step,
            "select_share": tot["select_ms"] / step,
            "attn_alg_tflops": tot["alg"] / (tot["attn_ms"] / 1e3) / 1e12,
            "unchunked_step_ms": m["step_ms"], "unchunked_dense_ms": whole_dense,
            "unchunked_speedup_vs_dense": whole_dense / m["step_ms"]}), flush=True)
        torch.cuda.empty_cache()


def segment_geometry(lengths, q_lengths, hq, hkv):
    """(t0, t1) of every segment in (request, KV head, tile) order (host arithmetic)."""
    g = hq // hkv
    t0s, t1s = [], []
    for L, Lq in zip(lengths, q_lengths):
        nt = -(-g * Lq // 128)
        r0 = 128 * np.arange(nt)
        r1 = np.minimum(r0 + 128, g * Lq)
        t0 = (L - Lq) + r0 // g
        t1 = (L - Lq) + (r1 - 1) // g
        for _ in range(hkv):
            t0s.append(t0)
            t1s.append(t1)
    return np.concatenate(t0s), np.concatenate(t1s)


def recall_stats(mass, sur, cu, idx, t0, t1, alpha, sink, win):
    """What the selection keeps of the exact block mass ([V1] §3.1 exact identification)."""
    nseg, mx = mass.shape
    J = np.arange(mx)[None, :]
    beta, nc = (t0 // 128)[:, None], (t1 // 128 + 1)[:, None]
    cand = J < nc
    sel = np.zeros((nseg, mx), bool)
    seg_of = np.repeat(np.arange(nseg), np.diff(cu))
    sel[seg_of, idx // 2] = True
    m = np.where(cand, mass, 0.0).astype(np.float64)
    su = np.where(cand, sur, 0.0).astype(np.float64)
    corr = cand & ~sel & (J < beta)
    forced = cand & ((J < sink) | ((J >= beta - win) & (J < beta)) | (J >= beta))
    star = cand & (forced | (m >= alpha * m.max(1, keepdims=True)))
    kept = (m * sel).sum(1)
    return {
        "mass_kept": float(kept.mean()), "mass_kept_min": float(kept.min()),
        "missed_without_correction": float((1 - kept).mean()),
        "missed_after_correction": float(((m - su) * corr).sum(1).mean()),
        "am_gm_ratio_corrected": float((su * corr).sum() / max((m * corr).sum(), 1e-300)),
        "exact_rule_block_recall": float((sel & star).sum() / star.sum()),
        "exact_rule_density": float(star.sum() / cand.sum()), "density": float(sel.sum() / cand.sum()),
    }


def recall(args):
    """Selection recall against the exact block mass for the 32K and 128K layers:
    one JSON line per workload (fp_block_mass timed on the GPU)."""
    from block_sparse_long_mean_amd import fp

    for w in (configs.L32K, configs.L128K):
        batch, _ = w.make()
        case = Case(batch, None, w.alpha, w.sink_blocks, w.window_blocks)
        case.select()
        case.dense()
        cu, idx = case.csr()
        lse = case.lse.clone()
        n, mx = case.bufs.sizes.n_segments, case.bufs.sizes.max_blocks
        mass = torch.empty((n, mx), dtype=torch.float32, device="cuda")
        sur = torch.empty((n, mx), dtype=torch.float32, device="cuda")
        ms = float(np.median(time_calls(lambda: fp.block_mass(case.B, case.q, case.k, lse, case.bufs, mass, sur),
                                        3, 1)))
        t0, t1 = segment_geometry(batch.lengths, batch.q_lengths, batch.hq, batch.hkv)
        st = recall_stats(mass.cpu().numpy(), sur.cpu().numpy(), cu, idx, t0, t1, w.alpha, w.sink_blocks,
                          w.window_blocks)
        qk = dense_flops(batch.lengths, batch.hq, batch.q_lengths) / 2  # Q K^T of every visible pair
        print(json.dumps({"recall": w.name, "alpha": w.alpha, "block_mass_ms": ms,
                          "block_mass_tflops": qk / (ms / 1e3) / 1e12,
                          "block_mass_mfma_frac": qk / (ms / 1e3) / 1e12 / PEAK[batch.dtype], **st}), flush=True)
        del case, mass, sur
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default=configs.L128K.name, choices=sorted(configs.ALL))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip dense / fp8 / alpha variants")
    ap.add_argument("--cpu-segments", type=int, default=4096)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (scale for HBM byte counters)")
    ap.add_argument("--sweep", action="store_true",
                    help="length sweep 4K..128K at 4 requests: one JSON line per length (select, attention, "
                         "dense baseline, speedup, density)")
    ap.add_argument("--chunked", action="store_true",
                    help="the 128K prompt in 8K and 16K chunks (index rebuilt per chunk) against one pass: "
                         "one JSON line per chunk size")
    ap.add_argument("--recall", action="store_true",
                    help="selection recall against the exact block mass (32K and 128K layers): one JSON line each")
    args = ap.parse_args()
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 1 << 30, "copies": 5}))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the operator runs on one GPU (sharding across GPUs is a design note, not code); --gpus must be 1"}))
        sys.exit(2)
    if args.sweep:
        sweep(args)
        return
    if args.chunked:
        chunked(args)
        return
    if args.recall:
        recall(args)
        return

    w = configs.ALL[args.config]
    t0 = time.time()
    batch, paged = w.make()
    gen_s = time.time() - t0
    case = Case(batch, paged, w.alpha, w.sink_blocks, w.window_blocks)
    main_m = measure(case, args.steps, args.warmup, correction=True)
    F = dense_flops(batch.lengths, batch.hq, batch.q_lengths)
    peak = PEAK[batch.dtype]
    attn_s = main_m["attn_ms"] / 1e3
    achieved = main_m["attn_alg_flop"] / attn_s / 1e12
    extra = {
        "select_ms": main_m["select_ms"], "sparse_attn_ms": main_m["attn_ms"],
        "density": main_m["density"], "csr_mib": main_m["csr_mib"],
        "attn_alg_tflop": main_m["attn_alg_flop"] / 1e12, "attn_exec_tflop": main_m["attn_exec_flop"] / 1e12,
        "mfma_util_executed": main_m["attn_exec_flop"] / attn_s / 1e12 / peak,
        "dense_equiv_tflop": F / 1e12, "input_gen_s": gen_s,
    }
    if not args.no_extra:
        d_ms = float(np.median(time_calls(case.dense, 3, 1)))
        extra["dense_ms"] = d_ms
        extra["dense_tflops"] = F / (d_ms / 1e3) / 1e12
        extra["dense_mfma_util"] = extra["dense_tflops"] / peak
        extra["speedup_vs_dense"] = d_ms / main_m["step_ms"]
        variants = {}
        m = measure(case, 3, 1, correction=False)
        variants["alpha0.1_nocorr"] = {k: m[k] for k in ("select_ms", "attn_ms", "step_ms", "density")}
        c2 = Case(batch, paged, 0.2, w.sink_blocks, w.window_blocks)
        for corr in (True, False):
            m = measure(c2, 3, 1, correction=corr)
            variants[f"alpha0.2_{'corr' if corr else 'nocorr'}"] = {
                k: m[k] for k in ("select_ms", "attn_ms", "step_ms", "density")}
        del c2
        if batch.dtype == "bf16" and w.page_size == 0:
            b8 = synth.to_e4m3(batch)
            for a in (0.1, 0.2):
                c8 = Case(b8, None, a, w.sink_blocks, w.window_blocks)
                m = measure(c8, 5, 2, correction=True)
                variants[f"fp8_alpha{a}"] = {
                    "select_ms": m["select_ms"], "attn_ms": m["attn_ms"], "step_ms": m["step_ms"],
                    "density": m["density"], "eff_tflops": F / (m["step_ms"] / 1e3) / 1e12,
                    "attn_alg_tflops": m["attn_alg_flop"] / (m["attn_ms"] / 1e3) / 1e12,
                    "mfma_util_executed": m["attn_exec_flop"] / (m["attn_ms"] / 1e3) / 1e12 / PEAK["e4m3"]}
                if a == 0.1:
                    dd = float(np.median(time_calls(c8.dense, 3, 1)))
                    variants["fp8_dense_ms"] = dd
                    variants["fp8_speedup_vs_dense"] = dd / m["step_ms"]
                del c8
            # V stored transposed (the column-major FP8 layout, consumed without a transpose)
            c8 = Case(b8, None, 0.1, w.sink_blocks, w.window_blocks, v_cols=True)
            m = measure(c8, 5, 2, correction=True)
            variants["fp8_vcols_alpha0.1"] = {
                "select_ms": m["select_ms"], "attn_ms": m["attn_ms"], "step_ms": m["step_ms"],
                "density": m["density"], "eff_tflops": F / (m["step_ms"] / 1e3) / 1e12,
                "attn_alg_tflops": m["attn_alg_flop"] / (m["attn_ms"] / 1e3) / 1e12}
            dd = float(np.median(time_calls(c8.dense, 3, 1)))
            variants["fp8_vcols_dense_ms"] = dd
            del c8
        extra["variants"] = variants
        extra["other_workloads"] = other_workloads(args)
    res = {
        "metric": METRIC,
        "value": F / (main_m["step_ms"] / 1e3) / 1e12,
        "unit": "TFLOP/s (dense-equivalent)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": main_m["step_ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": batch.dtype, "data": "synthetic (seeded generator standing in for RULER needle-in-a-haystack)",
        "config": {"workload": w.name, "lengths": list(batch.lengths)[:4] + (["..."] if len(batch.lengths) > 4 else []),
                   "q_lengths": None if not batch.chunked else list(batch.q_lengths)[:4] + (
                       ["..."] if len(batch.q_lengths) > 4 else []),
                   "num_reqs": len(batch.lengths), "hq": batch.hq, "hkv": batch.hkv, "d": D, "alpha": w.alpha,
                   "sink_blocks": w.sink_blocks, "window_blocks": w.window_blocks,
                   "paged": bool(w.page_size), "mean_correction": True},
        "roofline": {"bound": "mfma", "kernel": "attn_kernel (fp_sparse_attn)", "achieved": achieved,
                     "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
                     "traffic": recorded_traffic(w.name), "traffic_unit": "HBM bytes per launch",
                     "algorithmic_bytes": algorithmic_bytes(batch)},
        "extra": extra,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(batch, w, args.cpu_segments)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
