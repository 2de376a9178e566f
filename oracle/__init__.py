"""ctypes front end of the fp64 CPU oracle (``oracle/fpo.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of ``bench.py`` are the only callers.  The product library never imports
this package and shares no code with it.

All arrays are host numpy arrays.  Element storage follows the problem dtype:
``f32`` -> float32, ``bf16`` -> uint16 (raw bits), ``e4m3`` -> uint8 (raw OCP
E4M3 codes, decoded by the oracle itself and multiplied by the descale).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fpo.c")
_LIB = os.path.join(_HERE, "libfpo.so")

DTYPES = {"f32": 0, "bf16": 1, "e4m3": 2}
_NP_STORAGE = {"f32": np.float32, "bf16": np.uint16, "e4m3": np.uint8}


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", "-Wall", "-o", tmp, _SRC, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


class _Prob(C.Structure):
    _fields_ = [
        ("num_reqs", C.c_int32), ("hq", C.c_int32), ("hkv", C.c_int32), ("d", C.c_int32),
        ("cu", C.POINTER(C.c_int64)),
        ("dtype", C.c_int32),
        ("cq", C.c_double), ("ck", C.c_double), ("cv", C.c_double),
        ("q", C.c_void_p), ("k", C.c_void_p), ("v", C.c_void_p),
        ("scale", C.c_double),
        ("block", C.c_int32), ("rows", C.c_int32), ("phys", C.c_int32),
        ("cu_kv", C.POINTER(C.c_int64)),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = C.CDLL(build())
        L = _lib
        P = C.POINTER(_Prob)
        dp = C.POINTER(C.c_double)
        i32p = C.POINTER(C.c_int32)
        i64p = C.POINTER(C.c_int64)
        u8p = C.POINTER(C.c_uint8)
        L.fpo_e4m3_decode.restype = C.c_double
        L.fpo_e4m3_decode.argtypes = [C.c_uint8]
        L.fpo_e4m3_round.restype = C.c_double
        L.fpo_e4m3_round.argtypes = [C.c_double]
        L.fpo_blocks_in_req.restype = C.c_int64
        L.fpo_blocks_in_req.argtypes = [P, C.c_int]
        L.fpo_block_offset.restype = C.c_int64
        L.fpo_block_offset.argtypes = [P, C.c_int]
        L.fpo_tiles_in_req.restype = C.c_int64
        L.fpo_tiles_in_req.argtypes = [P, C.c_int]
        L.fpo_num_segments.restype = C.c_int64
        L.fpo_num_segments.argtypes = [P]
        L.fpo_segment_coords.restype = None
        L.fpo_segment_coords.argtypes = [P, C.c_int64, i32p, i32p, i64p]
        L.fpo_tile_info.restype = C.c_int
        L.fpo_tile_info.argtypes = [P, C.c_int, C.c_int64, i64p, i64p, i64p]
        L.fpo_pool_all.restype = None
        L.fpo_pool_all.argtypes = [P, dp, dp]
        L.fpo_score_tile.restype = C.c_int64
        L.fpo_score_tile.argtypes = [P, dp, C.c_int, C.c_int, C.c_int64, C.c_int, dp]
        L.fpo_select_tile.restype = None
        L.fpo_select_tile.argtypes = [dp, C.c_int64, C.c_int64, C.c_double, C.c_int, C.c_int, u8p, u8p]
        L.fpo_csr_tile.restype = C.c_int64
        L.fpo_csr_tile.argtypes = [u8p, C.c_int64, C.c_int64, C.c_int, C.c_int, i32p]
        L.fpo_select_all.restype = C.c_int64
        L.fpo_select_all.argtypes = [P, dp, C.c_double, C.c_int, C.c_int, C.c_int, i32p, i32p,
                                     C.c_int64, dp, u8p, C.c_int64]
        L.fpo_select_list.restype = None
        L.fpo_select_list.argtypes = [P, dp, C.c_double, C.c_int, C.c_int, C.c_int, C.c_int64, i64p, C.c_int64,
                                      i32p, i32p]
        L.fpo_attend_tile.restype = None
        L.fpo_attend_tile.argtypes = [P, dp, dp, C.c_int, C.c_int, C.c_int64, i32p, C.c_int64,
                                      C.c_int, C.c_int, dp, dp]
        L.fpo_dense_tile.restype = None
        L.fpo_dense_tile.argtypes = [P, C.c_int, C.c_int, C.c_int64, dp, dp]
        L.fpo_attend_list.restype = None
        L.fpo_attend_list.argtypes = [P, dp, dp, C.c_int64, i64p, i32p, i32p, C.c_int, C.c_int,
                                      C.c_int, dp, dp]
        L.fpo_attend_tile_eq15.restype = None
        L.fpo_attend_tile_eq15.argtypes = [P, dp, dp, C.c_int, C.c_int, C.c_int64, i32p, C.c_int64,
                                           C.c_int, C.c_int, C.c_int, C.c_double, dp, dp, dp, dp]
        L.fpo_attend_list_eq15.restype = None
        L.fpo_attend_list_eq15.argtypes = [P, dp, dp, C.c_int64, i64p, i32p, i32p, C.c_int, C.c_int,
                                           i32p, C.c_double, dp, dp, dp, dp]
        L.fpo_block_mass_tile.restype = C.c_int64
        L.fpo_block_mass_tile.argtypes = [P, dp, C.c_int, C.c_int, C.c_int64, dp, dp]
        L.fpo_block_mass_list.restype = None
        L.fpo_block_mass_list.argtypes = [P, dp, C.c_int64, i64p, C.c_int64, dp, dp]
        L.fpo_num_threads.restype = C.c_int
        L.fpo_num_threads.argtypes = []
    return _lib


def _ptr(a, ctype):
    return a.ctypes.data_as(C.POINTER(ctype))


def e4m3_decode(code: int) -> float:
    return lib().fpo_e4m3_decode(code)


def e4m3_round(x: float) -> float:
    return lib().fpo_e4m3_round(x)


def num_threads() -> int:
    return lib().fpo_num_threads()


class Problem:
    """Host description of one batch for the oracle.

    ``q`` is [total_q, hq, d] ragged by ``cu``; ``k``/``v`` are [total_kv, hkv, d]
    ragged by ``cu_kv`` (None: by ``cu``), contiguous, stored as described in
    the module docstring.  A request with more keys than queries holds a prefill
    chunk: its queries are its last L_q positions.
    """

    def __init__(self, cu, hq, hkv, d, dtype, q, k, v, descale=(1.0, 1.0, 1.0), scale=None,
                 block=128, rows=128, phys=64, cu_kv=None, _geometry_only=False):
        if dtype not in DTYPES:
            raise ValueError(dtype)
        st = _NP_STORAGE[dtype]
        self.q = np.ascontiguousarray(q).view(st) if q.dtype != st else np.ascontiguousarray(q)
        self.k = np.ascontiguousarray(k).view(st) if k.dtype != st else np.ascontiguousarray(k)
        self.v = np.ascontiguousarray(v).view(st) if v.dtype != st else np.ascontiguousarray(v)
        self.cu = np.ascontiguousarray(np.asarray(cu, dtype=np.int64))
        self.cu_kv = None if cu_kv is None else np.ascontiguousarray(np.asarray(cu_kv, dtype=np.int64))
        kvc = self.cu if self.cu_kv is None else self.cu_kv
        assert len(kvc) == len(self.cu) and kvc[0] == 0
        assert np.all(np.diff(kvc) >= np.diff(self.cu)), "every request needs L_kv >= L_q"
        total, total_kv = int(self.cu[-1]), int(kvc[-1])
        if not _geometry_only:
            assert self.q.shape == (total, hq, d), (self.q.shape, total, hq, d)
            assert self.k.shape == (total_kv, hkv, d) and self.v.shape == (total_kv, hkv, d)
        self.hq, self.hkv, self.d, self.dtype = hq, hkv, d, dtype
        self.block, self.rows, self.phys = block, rows, phys
        self.scale = float(scale) if scale is not None else 1.0 / float(np.sqrt(d))
        self.descale = tuple(float(x) for x in descale)
        self._s = _Prob(
            len(self.cu) - 1, hq, hkv, d, _ptr(self.cu, C.c_int64), DTYPES[dtype],
            self.descale[0], self.descale[1], self.descale[2],
            self.q.ctypes.data, self.k.ctypes.data, self.v.ctypes.data,
            self.scale, block, rows, phys,
            None if self.cu_kv is None else _ptr(self.cu_kv, C.c_int64),
        )
        self._kbar = None
        self._vbar = None

    @classmethod
    def geometry(cls, lengths, hq, hkv, d=128, block=128, rows=128, phys=64, q_lengths=None):
        """A problem usable only for its geometry (segments, tiles, blocks).
        ``lengths`` are the K/V lengths, ``q_lengths`` the query lengths (None: the same)."""
        cu_kv = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
        cu = cu_kv if q_lengths is None else np.concatenate([[0], np.cumsum(q_lengths)]).astype(np.int64)
        z = np.zeros((1, 1, 1), np.float32)
        return cls(cu, hq, hkv, d, "f32", z, z, z, block=block, rows=rows, phys=phys,
                   cu_kv=None if q_lengths is None else cu_kv, _geometry_only=True)

    # -- geometry -------------------------------------------------------
    @property
    def num_reqs(self):
        return len(self.cu) - 1

    @property
    def g(self):
        return self.hq // self.hkv

    def num_segments(self) -> int:
        return int(lib().fpo_num_segments(C.byref(self._s)))

    def blocks_in_req(self, b) -> int:
        return int(lib().fpo_blocks_in_req(C.byref(self._s), b))

    def block_offset(self, b) -> int:
        return int(lib().fpo_block_offset(C.byref(self._s), b))

    def tiles_in_req(self, b) -> int:
        return int(lib().fpo_tiles_in_req(C.byref(self._s), b))

    def segment_coords(self, s):
        b, h, i = C.c_int32(), C.c_int32(), C.c_int64()
        lib().fpo_segment_coords(C.byref(self._s), s, C.byref(b), C.byref(h), C.byref(i))
        return b.value, h.value, i.value

    def tile_info(self, b, I):
        t0, t1, beta = C.c_int64(), C.c_int64(), C.c_int64()
        n = lib().fpo_tile_info(C.byref(self._s), b, I, C.byref(t0), C.byref(t1), C.byref(beta))
        return n, t0.value, t1.value, beta.value

    # -- pooling --------------------------------------------------------
    def pool(self):
        if self._kbar is None:
            nb = self.block_offset(self.num_reqs)
            kb = np.zeros((nb, self.hkv, self.d), np.float64)
            vb = np.zeros((nb, self.hkv, self.d), np.float64)
            lib().fpo_pool_all(C.byref(self._s), _ptr(kb, C.c_double), _ptr(vb, C.c_double))
            self._kbar, self._vbar = kb, vb
        return self._kbar, self._vbar

    # -- scoring / selection -------------------------------------------
    def candidates(self, b, I) -> int:
        """Candidate blocks of tile I: every block up to that of its last position."""
        _, _, t1, _ = self.tile_info(b, I)
        return t1 // self.block + 1

    def score_tile(self, b, h, I, form=2):
        kb, _ = self.pool()
        e = np.zeros(self.candidates(b, I), np.float64)
        lib().fpo_score_tile(C.byref(self._s), _ptr(kb, C.c_double), b, h, I, form,
                             _ptr(e, C.c_double))
        return e

    @staticmethod
    def select_tile(e, alpha, n_sink, n_win, beta=None):
        """``beta``: the block of the tile's first position (None: the last candidate)."""
        e = np.ascontiguousarray(e, np.float64)
        sel = np.zeros(len(e), np.uint8)
        amb = np.zeros(len(e), np.uint8)
        beta = len(e) - 1 if beta is None else beta
        lib().fpo_select_tile(_ptr(e, C.c_double), len(e), beta, alpha, n_sink, n_win,
                              _ptr(sel, C.c_uint8), _ptr(amb, C.c_uint8))
        return sel.astype(bool), amb.astype(bool)

    def csr_tile(self, sel, t1):
        sel = np.ascontiguousarray(sel, np.uint8)
        n = lib().fpo_csr_tile(_ptr(sel, C.c_uint8), len(sel), t1, self.phys, self.block, None)
        out = np.zeros(max(n, 1), np.int32)
        lib().fpo_csr_tile(_ptr(sel, C.c_uint8), len(sel), t1, self.phys, self.block,
                           _ptr(out, C.c_int32))
        return out[:n]

    def segment_select(self, s, alpha, n_sink, n_win, form=2):
        """(e, sel, ambig, idx) of one segment."""
        b, h, I = self.segment_coords(s)
        _, _, t1, beta = self.tile_info(b, I)
        e = self.score_tile(b, h, I, form)
        sel, amb = self.select_tile(e, alpha, n_sink, n_win, beta)
        return e, sel, amb, self.csr_tile(sel, t1)

    def max_candidates(self) -> int:
        return max(self.blocks_in_req(b) for b in range(self.num_reqs))

    def select_all(self, alpha, n_sink, n_win, form=2, want_energies=False):
        """Full CSR of the problem: (cu, idx[, e, ambig])."""
        kb, _ = self.pool()
        nseg = self.num_segments()
        cap = 0
        for s in range(nseg):
            b, h, I = self.segment_coords(s)
            cap += self.candidates(b, I) * (self.block // self.phys)
        cu = np.zeros(nseg + 1, np.int32)
        idx = np.zeros(max(cap, 1), np.int32)
        mx = self.max_candidates()
        e = np.zeros((nseg, mx), np.float64) if want_energies else None
        amb = np.zeros((nseg, mx), np.uint8) if want_energies else None
        n = lib().fpo_select_all(
            C.byref(self._s), _ptr(kb, C.c_double), alpha, n_sink, n_win, form,
            _ptr(cu, C.c_int32), _ptr(idx, C.c_int32), cap,
            _ptr(e, C.c_double) if e is not None else None,
            _ptr(amb, C.c_uint8) if amb is not None else None, mx)
        assert n >= 0
        if want_energies:
            return cu, idx[:n], e, amb.astype(bool)
        return cu, idx[:n]

    def select_segments(self, segs, alpha, n_sink, n_win, form=2):
        """Tile lists of the listed segments (OpenMP over them): a CSR (cu, idx)
        over ALL segments of the problem in which only the listed ones are
        non-empty."""
        kb, _ = self.pool()
        segs = np.ascontiguousarray(np.asarray(segs, np.int64))
        stride = 2 * self.max_candidates()
        lists = np.zeros((len(segs), stride), np.int32)
        counts = np.zeros(len(segs), np.int32)
        lib().fpo_select_list(C.byref(self._s), _ptr(kb, C.c_double), alpha, n_sink, n_win, form, len(segs),
                              _ptr(segs, C.c_int64), stride, _ptr(lists, C.c_int32), _ptr(counts, C.c_int32))
        nseg = self.num_segments()
        cnt = np.zeros(nseg, np.int64)
        cnt[segs] = counts
        cu = np.zeros(nseg + 1, np.int32)
        cu[1:] = np.cumsum(cnt)
        idx = np.zeros(max(int(cu[-1]), 1), np.int32)
        for n, s in enumerate(segs):
            idx[cu[s]:cu[s + 1]] = lists[n, :counts[n]]
        return cu, idx[: int(cu[-1])]

    # -- attention ------------------------------------------------------
    def attend_segments(self, segs, cu=None, idx=None, dense=False, correction=True, p8=False):
        """Oracle output rows of the listed segments: (out [n,R,d], lse [n,R])."""
        kb, vb = self.pool()
        segs = np.ascontiguousarray(np.asarray(segs, np.int64))
        n = len(segs)
        out = np.zeros((n, self.rows, self.d), np.float64)
        lse = np.zeros((n, self.rows), np.float64)
        if dense:
            cu_a = np.zeros(1, np.int32)
            idx_a = np.zeros(1, np.int32)
        else:
            cu_a = np.ascontiguousarray(np.asarray(cu, np.int32))
            idx_a = np.ascontiguousarray(np.asarray(idx, np.int32))
            if idx_a.size == 0:
                idx_a = np.zeros(1, np.int32)
        lib().fpo_attend_list(
            C.byref(self._s), _ptr(kb, C.c_double), _ptr(vb, C.c_double), n, _ptr(segs, C.c_int64),
            _ptr(cu_a, C.c_int32), _ptr(idx_a, C.c_int32), 1 if dense else 0,
            1 if correction else 0, 1 if p8 else 0, _ptr(out, C.c_double), _ptr(lse, C.c_double))
        return out, lse

    def attend_segments_eq15(self, segs, cu, idx, correction=True, rounding=True, nsplit=None, logit_err=0.0):
        """[V2] Eq. 15 as printed (E4M3 weights rounded against the running row
        maximum, steps in Eq. 17 order then the correction chunks; ``nsplit``: the
        KV split count of each listed segment, None = 1): (out [n,R,d], lse [n,R]).
        ``rounding=False`` runs the same recurrence unrounded.  With ``logit_err`` > 0
        also returns (allow [n,R], lallow [n,R]): how far each row's output (max-abs)
        and LSE can move if every weight whose rounding an implementation with logits
        off by up to logit_err * sigma * sum|q_i k_i| could flip took its other
        rounding."""
        kb, vb = self.pool()
        segs = np.ascontiguousarray(np.asarray(segs, np.int64))
        n = len(segs)
        out = np.zeros((n, self.rows, self.d), np.float64)
        lse = np.zeros((n, self.rows), np.float64)
        cu_a = np.ascontiguousarray(np.asarray(cu, np.int32))
        idx_a = np.ascontiguousarray(np.asarray(idx, np.int32))
        if idx_a.size == 0:
            idx_a = np.zeros(1, np.int32)
        ns = None
        if nsplit is not None:
            ns = np.ascontiguousarray(np.asarray(nsplit, np.int32))
            assert ns.shape == (n,) and np.all(ns >= 1)
        allow = np.zeros((n, self.rows), np.float64)
        lallow = np.zeros((n, self.rows), np.float64)
        lib().fpo_attend_list_eq15(
            C.byref(self._s), _ptr(kb, C.c_double), _ptr(vb, C.c_double), n, _ptr(segs, C.c_int64),
            _ptr(cu_a, C.c_int32), _ptr(idx_a, C.c_int32), 1 if correction else 0, 1 if rounding else 0,
            None if ns is None else _ptr(ns, C.c_int32), float(logit_err), _ptr(out, C.c_double),
            _ptr(lse, C.c_double), _ptr(allow, C.c_double), _ptr(lallow, C.c_double))
        if logit_err > 0:
            return out, lse, allow, lallow
        return out, lse

    def attend_tile_eq15(self, b, h, I, idx, correction=True, rounding=True, nsplit=1, logit_err=0.0):
        kb, vb = self.pool()
        idx = np.ascontiguousarray(np.asarray(idx, np.int32))
        out = np.zeros((self.rows, self.d), np.float64)
        lse = np.zeros(self.rows, np.float64)
        buf = idx if idx.size else np.zeros(1, np.int32)
        allow = np.zeros(self.rows, np.float64)
        lallow = np.zeros(self.rows, np.float64)
        lib().fpo_attend_tile_eq15(C.byref(self._s), _ptr(kb, C.c_double), _ptr(vb, C.c_double), b, h, I,
                                   _ptr(buf, C.c_int32), idx.size, 1 if correction else 0,
                                   1 if rounding else 0, int(nsplit), float(logit_err), _ptr(out, C.c_double),
                                   _ptr(lse, C.c_double), _ptr(allow, C.c_double), _ptr(lallow, C.c_double))
        if logit_err > 0:
            return out, lse, allow, lallow
        return out, lse

    def attend_tile(self, b, h, I, idx, correction=True, p8=False):
        kb, vb = self.pool()
        idx = np.ascontiguousarray(np.asarray(idx, np.int32))
        out = np.zeros((self.rows, self.d), np.float64)
        lse = np.zeros(self.rows, np.float64)
        buf = idx if idx.size else np.zeros(1, np.int32)
        lib().fpo_attend_tile(C.byref(self._s), _ptr(kb, C.c_double), _ptr(vb, C.c_double), b, h, I,
                              _ptr(buf, C.c_int32), idx.size, 1 if correction else 0, 1 if p8 else 0,
                              _ptr(out, C.c_double), _ptr(lse, C.c_double))
        return out, lse

    def dense_tile(self, b, h, I):
        out = np.zeros((self.rows, self.d), np.float64)
        lse = np.zeros(self.rows, np.float64)
        lib().fpo_dense_tile(C.byref(self._s), b, h, I, _ptr(out, C.c_double), _ptr(lse, C.c_double))
        return out, lse

    # -- exact block mass (selection-recall diagnostic) -------------------
    def block_mass_tile(self, b, h, I):
        """(mass, sur) over the tile's candidate blocks: the exact per-block attention
        mass averaged over the tile's rows, and the mean surrogate for blocks J < beta."""
        kb, _ = self.pool()
        nc = self.candidates(b, I)
        m = np.zeros(nc, np.float64)
        su = np.zeros(nc, np.float64)
        lib().fpo_block_mass_tile(C.byref(self._s), _ptr(kb, C.c_double), b, h, I,
                                  _ptr(m, C.c_double), _ptr(su, C.c_double))
        return m, su

    def block_mass_segments(self, segs, max_nc=None):
        """(mass, sur) of the listed segments, [n][max_nc] padded with -1 (OpenMP)."""
        kb, _ = self.pool()
        segs = np.ascontiguousarray(np.asarray(segs, np.int64))
        mx = self.max_candidates() if max_nc is None else max_nc
        m = np.zeros((len(segs), mx), np.float64)
        su = np.zeros((len(segs), mx), np.float64)
        lib().fpo_block_mass_list(C.byref(self._s), _ptr(kb, C.c_double), len(segs), _ptr(segs, C.c_int64),
                                  mx, _ptr(m, C.c_double), _ptr(su, C.c_double))
        return m, su

    # -- row mapping (definition of PackGQA, [V2] §3.3 Eq. 13) -----------
    def rows_of_segment(self, s):
        """(Q rows, heads, valid) of the R packed rows of segment s."""
        b, h, I = self.segment_coords(s)
        r = I * self.rows + np.arange(self.rows)
        Lq = int(self.cu[b + 1] - self.cu[b])
        valid = r < self.g * Lq
        qi = r // self.g
        head = h * self.g + r % self.g
        return self.cu[b] + qi, head, valid
