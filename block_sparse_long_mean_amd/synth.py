"""Seeded synthetic inputs for the block-sparse prefill path.

This module only draws and lays out random tensors; it holds none of the
method's arithmetic, so both the HIP path and the CPU oracle may consume what
it makes.  The inputs stand in for the needle-in-a-haystack / RULER prompts
run through real models on the FlashPrefill V2 page (§4.1, Table 1), which are
not available here.

Recipe, per request b and KV head h (numpy PCG64 seeded by (seed, b, h)):
  m_J ~ N(0, I_d) per 128-token block J;   with ``clusters``, ceil(1% n_J)
  blocks chosen without replacement get m_J <- 3 m_J.
  u = z/|z|, z ~ N(0, I_d)                 (one direction per KV head)
  k_t = m_{t//128} + 0.5 n_t,  n_t ~ N(0, I_d);  k_t += 3u for t < 4 (sinks)
  v_t ~ N(0, I_d)
and for the j-th query head of the group (seeded by (seed, b, h, 1+j)):
  q_t = N(0, I_d) + 1.5u;  with ``diag_bias``, r ~ U{1..64} and
  q_t += 0.5 k_{t-r} for t >= r.
A request with L_q < L queries (a prefill chunk after a cached prefix) keeps
the last L_q rows of the same q_t draws, so its queries are exactly those of
the fresh request at positions L-L_q..L-1.
Everything is drawn in float32, then cast with round-to-nearest-even.  E4M3
inputs are quantised from the bf16 tensors with per-tensor scales
c = amax|X| / 448 (OCP E4M3FN, saturated at +-448).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

BLOCK = 128


def _workers() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def _rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(x) for x in key])))


@dataclass
class Batch:
    """One batch of requests, contiguous layout: Q [total_q, Hq, d] ragged by
    ``cu``, K/V [total_kv, Hkv, d] ragged by ``cu_kv`` (None: by ``cu``).
    ``lengths`` are the K/V lengths, ``q_lengths`` the query lengths."""

    lengths: list
    hq: int
    hkv: int
    d: int
    dtype: str                       # "f32" | "bf16" | "e4m3"
    q: torch.Tensor                  # float32 / bfloat16 / uint8 (E4M3 codes)
    k: torch.Tensor
    v: torch.Tensor
    descale: tuple = (1.0, 1.0, 1.0)
    cu: np.ndarray = field(default=None)
    q_lengths: list = field(default=None)
    cu_kv: np.ndarray = field(default=None)

    def __post_init__(self):
        if self.q_lengths is None:
            self.q_lengths = list(self.lengths)
        if self.cu is None:
            self.cu = np.concatenate([[0], np.cumsum(self.q_lengths)]).astype(np.int64)
        if self.cu_kv is None and list(self.q_lengths) != list(self.lengths):
            self.cu_kv = np.concatenate([[0], np.cumsum(self.lengths)]).astype(np.int64)

    @property
    def chunked(self) -> bool:
        return self.cu_kv is not None

    @property
    def kv_cu(self) -> np.ndarray:
        return self.cu if self.cu_kv is None else self.cu_kv

    @property
    def total(self) -> int:
        """Query rows."""
        return int(self.cu[-1])

    @property
    def total_kv(self) -> int:
        return int(self.kv_cu[-1])

    def storage(self, t: torch.Tensor) -> np.ndarray:
        """Raw host view for the oracle: float32, uint16 (bf16 bits) or uint8."""
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()


def _gen_head(seed, b, h, L, Lq, d, g, clusters, diag_bias, q_out, k_out, v_out, q_dtype, kv_dtype):
    rng = _rng(seed, b, h)
    nJ = (L + BLOCK - 1) // BLOCK
    m = rng.standard_normal((nJ, d), dtype=np.float32)
    if clusters:
        nc = int(math.ceil(0.01 * nJ))
        pick = rng.choice(nJ, size=nc, replace=False)
        m[pick] *= 3.0
    z = rng.standard_normal(d, dtype=np.float32)
    u = (z / np.linalg.norm(z)).astype(np.float32)
    k = rng.standard_normal((L, d), dtype=np.float32)
    k *= 0.5
    k += np.repeat(m, BLOCK, axis=0)[:L]
    k[: min(4, L)] += 3.0 * u
    v = rng.standard_normal((L, d), dtype=np.float32)
    k_out[:, h, :] = torch.from_numpy(k).to(kv_dtype)
    v_out[:, h, :] = torch.from_numpy(v).to(kv_dtype)
    for j in range(g):
        rq = _rng(seed, b, h, 1 + j)
        r = int(rq.integers(1, 65)) if diag_bias else 0
        q = rq.standard_normal((L, d), dtype=np.float32)
        q += 1.5 * u
        if diag_bias and r < L:
            q[r:] += 0.5 * k[: L - r]
        q_out[:, h * g + j, :] = torch.from_numpy(q[L - Lq:]).to(q_dtype)


def make_batch(lengths, hq, hkv, d, seed, dtype="bf16", clusters=False, diag_bias=False,
               q_lengths=None) -> Batch:
    """Draw a batch; ``dtype`` "f32" or "bf16" (use :func:`to_e4m3` for E4M3).
    ``lengths`` are the K/V lengths; ``q_lengths`` (None: the same) the number of
    trailing positions of each request that carry queries."""
    lengths = [int(x) for x in lengths]
    qls = list(lengths) if q_lengths is None else [int(x) for x in q_lengths]
    assert len(qls) == len(lengths) and all(0 <= a <= L for a, L in zip(qls, lengths))
    g = hq // hkv
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    q = torch.empty((sum(qls), hq, d), dtype=tdt)
    k = torch.empty((sum(lengths), hkv, d), dtype=tdt)
    v = torch.empty((sum(lengths), hkv, d), dtype=tdt)
    jobs = []
    off = qoff = 0
    for b, (L, Lq) in enumerate(zip(lengths, qls)):
        for h in range(hkv):
            jobs.append((b, h, L, Lq, off, qoff))
        off += L
        qoff += Lq
    with ThreadPoolExecutor(_workers()) as ex:
        futs = [ex.submit(_gen_head, seed, b, h, L, Lq, d, g, clusters, diag_bias,
                          q[qo:qo + Lq], k[o:o + L], v[o:o + L], tdt, tdt)
                for (b, h, L, Lq, o, qo) in jobs]
        for f in futs:
            f.result()
    return Batch(lengths, hq, hkv, d, dtype, q, k, v,
                 q_lengths=None if q_lengths is None else qls)


def _quant_e4m3(x: torch.Tensor):
    amax = float(x.abs().max().float())
    c = amax / 448.0 if amax > 0 else 1.0
    codes = torch.empty(x.shape, dtype=torch.uint8)
    n = x.shape[0]
    step = max(1, n // 64)

    def work(i):
        xs = (x[i:i + step].float() / c).clamp_(-448.0, 448.0)
        codes[i:i + step] = xs.to(torch.float8_e4m3fn).view(torch.uint8)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(work, range(0, n, step)))
    return codes, c


def to_e4m3(batch: Batch) -> Batch:
    """Per-tensor E4M3 quantisation of a bf16 batch (c = amax/448)."""
    qc, cq = _quant_e4m3(batch.q)
    kc, ck = _quant_e4m3(batch.k)
    vc, cv = _quant_e4m3(batch.v)
    return Batch(batch.lengths, batch.hq, batch.hkv, batch.d, "e4m3", qc, kc, vc,
                 descale=(cq, ck, cv), cu=batch.cu, q_lengths=batch.q_lengths, cu_kv=batch.cu_kv)


def prefix_chunk(batch: Batch, stop: int, size: int) -> Batch:
    """Chunk [stop - size, stop) of a one-request batch's prompt: its queries and
    every key/value before ``stop`` (views, no copy)."""
    assert len(batch.lengths) == 1 and not batch.chunked and 0 < size <= stop <= batch.lengths[0]
    return Batch([stop], batch.hq, batch.hkv, batch.d, batch.dtype, batch.q[stop - size:stop],
                 batch.k[:stop], batch.v[:stop], descale=batch.descale, q_lengths=[size])


def varlen_lengths(n, lo, hi, seed):
    """n lengths log-uniform in [lo, hi] (seeded)."""
    rng = _rng(seed, 0x5EED)
    x = rng.uniform(math.log(lo), math.log(hi), size=n)
    return [int(math.floor(math.exp(t))) for t in x]


def v_columns(batch: Batch) -> torch.Tensor:
    """V stored transposed, [Hkv][d][total_kv]: each head's value vectors as
    columns (the column-major FP8 V layout; layout only)."""
    return batch.v.permute(1, 2, 0).contiguous()


@dataclass
class Paged:
    """K/V scattered into a pool of pages through a page table ([V2] §3.3 Eq. 22)."""

    k_pool: torch.Tensor          # [num_slots, hkv, d]
    v_pool: torch.Tensor          # [num_slots, hkv, d], or [num_pages, hkv, d, page_size] (v_cols)
    page_table: np.ndarray        # [num_reqs, max_pages] int32 (-1 = unused)
    page_size: int
    num_slots: int


def page_kv(batch: Batch, page_size, seed, spare=0.05, poison=True, v_cols=False) -> Paged:
    """Scatter K/V into a page pool with a random permutation of page ids.

    The pool holds sum ceil(L_b/p) pages plus ``spare`` extra, and every slot
    no request owns is filled with NaN so a stray read shows in the output.
    ``v_cols``: each V page is stored transposed, [Hkv][d][page_size].
    """
    need = [(L + page_size - 1) // page_size for L in batch.lengths]
    npages = int(sum(need) + math.ceil(spare * sum(need)))
    rng = _rng(seed, 0xFA6E)
    perm = rng.permutation(npages).astype(np.int32)
    maxp = max(need)
    pt = np.full((len(need), maxp), -1, np.int32)
    o = 0
    for b, n in enumerate(need):
        pt[b, :n] = perm[o:o + n]
        o += n
    slots = npages * page_size
    shape = (slots, batch.hkv, batch.d)
    kp = torch.empty(shape, dtype=batch.k.dtype)
    vp = torch.empty((npages, batch.hkv, batch.d, page_size) if v_cols else shape, dtype=batch.v.dtype)
    if poison:
        if batch.k.dtype == torch.uint8:
            kp.fill_(0x7F)  # E4M3 NaN code
            vp.fill_(0x7F)
        else:
            kp.fill_(float("nan"))
            vp.fill_(float("nan"))
    for b, L in enumerate(batch.lengths):
        base = int(batch.kv_cu[b])
        for j in range(need[b]):
            lo = j * page_size
            hi = min(L, lo + page_size)
            s0 = int(pt[b, j]) * page_size
            kp[s0:s0 + hi - lo] = batch.k[base + lo:base + hi]
            if v_cols:
                vp[int(pt[b, j]), :, :, :hi - lo] = batch.v[base + lo:base + hi].permute(1, 2, 0)
            else:
                vp[s0:s0 + hi - lo] = batch.v[base + lo:base + hi]
    return Paged(kp, vp, pt, page_size, slots)
