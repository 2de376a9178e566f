"""ctypes binding of libfp.so (include/fp.h).

Argument marshalling only: tensors are passed as raw device pointers with
torch's current stream; every step of the computation runs in the library's
HIP kernels.  Importing this module fails loudly if the library is missing.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m block_sparse_long_mean_amd.build` "
        "(there is no fallback path)")

_lib = C.CDLL(LIB_PATH)

FP_F32, FP_BF16, FP_E4M3 = 0, 1, 2
STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported", -3: "workspace too small",
          -4: "idx capacity too small", -5: "kernel launch failed", -6: "device reported malformed input"}


class Problem(C.Structure):
    _fields_ = [
        ("num_reqs", C.c_int32), ("num_heads_q", C.c_int32), ("num_heads_kv", C.c_int32),
        ("head_dim", C.c_int32),
        ("cu_seqlens_q", C.c_void_p), ("cu_seqlens_q_host", C.c_void_p),
        ("page_table", C.c_void_p), ("page_size", C.c_int32), ("max_pages_per_req", C.c_int32),
        ("num_pool_slots", C.c_int64), ("dtype", C.c_int32), ("descale", C.c_void_p),
        ("softmax_scale", C.c_float),
        ("cu_seqlens_kv", C.c_void_p), ("cu_seqlens_kv_host", C.c_void_p),
        ("v_layout", C.c_int32),
    ]


class SelectParams(C.Structure):
    _fields_ = [("alpha", C.c_float), ("block_size", C.c_int32), ("sink_blocks", C.c_int32),
                ("window_blocks", C.c_int32)]


class Sizes(C.Structure):
    _fields_ = [("n_segments", C.c_int64), ("idx_capacity", C.c_int64), ("means_bytes", C.c_size_t),
                ("workspace_bytes", C.c_size_t), ("max_blocks", C.c_int64)]


_P = C.POINTER(Problem)
_SP = C.POINTER(SelectParams)
_vp = C.c_void_p
_lib.fp_query_sizes.restype = C.c_int
_lib.fp_query_sizes.argtypes = [_P, _SP, C.POINTER(Sizes)]
_lib.fp_pool.restype = C.c_int
_lib.fp_pool.argtypes = [_P, _vp, _vp, _vp, _vp, C.c_size_t, _vp]
_lib.fp_select.restype = C.c_int
_lib.fp_select.argtypes = [_P, _SP, _vp, _vp, _vp, _vp, _vp, C.c_int64, _vp, _vp, _vp, C.c_size_t, _vp]
_lib.fp_sparse_attn.restype = C.c_int
_lib.fp_sparse_attn.argtypes = [_P, _SP, _vp, _vp, _vp, _vp, _vp, _vp, C.c_int32, _vp, _vp, _vp,
                                C.c_size_t, _vp]
_lib.fp_sparse_attn_static.restype = C.c_int
_lib.fp_sparse_attn_static.argtypes = [_P, _SP, _vp, _vp, _vp, _vp, _vp, _vp, C.c_int32, _vp, _vp, _vp]
_lib.fp_dense_attn.restype = C.c_int
_lib.fp_dense_attn.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, C.c_size_t, _vp]
_lib.fp_block_mass.restype = C.c_int
_lib.fp_block_mass.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, C.c_size_t, _vp]
_lib.fp_read_device_error.restype = C.c_int
_lib.fp_read_device_error.argtypes = [_vp, _vp, C.POINTER(C.c_int32)]
_lib.fp_block_base.restype = C.c_int64
_lib.fp_block_base.argtypes = [_P, C.c_int32]
_lib.fp_status_string.restype = C.c_char_p
_lib.fp_status_string.argtypes = [C.c_int]
_lib.fp_last_error.restype = C.c_char_p
_lib.fp_last_error.argtypes = []

EXPORTS = ["fp_query_sizes", "fp_pool", "fp_select", "fp_sparse_attn", "fp_sparse_attn_static", "fp_dense_attn",
           "fp_block_mass",
           "fp_read_device_error", "fp_block_base", "fp_status_string", "fp_last_error"]


class FPError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {_lib.fp_last_error().decode()}")


def _check(st: int):
    if st != 0:
        raise FPError(st)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


_DT = {torch.float32: FP_F32, torch.bfloat16: FP_BF16, torch.uint8: FP_E4M3}


@dataclass
class Batch:
    """Device-side description of one batch; keeps every referenced tensor alive."""

    prob: Problem
    cu_dev: torch.Tensor
    cu_host: np.ndarray
    page_table: torch.Tensor | None
    descale: torch.Tensor | None
    cu_kv_dev: torch.Tensor | None = None
    cu_kv_host: np.ndarray | None = None

    @property
    def ptr(self):
        return C.byref(self.prob)


def make_batch(cu_seqlens, num_heads_q, num_heads_kv, dtype, device="cuda", head_dim=128,
               page_table=None, page_size=0, num_pool_slots=0, descale=None, softmax_scale=0.0,
               cu_seqlens_kv=None, v_cols=False) -> Batch:
    """Build the C problem struct.  ``cu_seqlens`` (query rows) and ``cu_seqlens_kv`` (K/V
    lengths; None = the same) are host sequences; ``dtype`` a torch dtype (float32, bfloat16,
    or uint8 for E4M3 codes); ``page_table`` a host int array or None; ``v_cols``: V is stored
    transposed (E4M3 only, see fp.h)."""
    cu_host = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    cu_dev = torch.from_numpy(cu_host.copy()).to(device)
    kv_host = kv_dev = None
    if cu_seqlens_kv is not None:
        kv_host = np.ascontiguousarray(np.asarray(cu_seqlens_kv, dtype=np.int32))
        kv_dev = torch.from_numpy(kv_host.copy()).to(device)
    pt = None
    max_pages = 0
    if page_table is not None:
        pt_np = np.ascontiguousarray(np.asarray(page_table, dtype=np.int32))
        max_pages = pt_np.shape[1]
        pt = torch.from_numpy(pt_np).to(device)
    ds = None
    if descale is not None:
        ds = torch.tensor(list(descale), dtype=torch.float32, device=device)
    prob = Problem(len(cu_host) - 1, num_heads_q, num_heads_kv, head_dim, cu_dev.data_ptr(),
                   cu_host.ctypes.data, _ptr(pt), page_size if pt is not None else 0, max_pages,
                   num_pool_slots if pt is not None else 0, _DT[dtype], _ptr(ds), softmax_scale,
                   _ptr(kv_dev), None if kv_host is None else kv_host.ctypes.data, 1 if v_cols else 0)
    return Batch(prob, cu_dev, cu_host, pt, ds, kv_dev, kv_host)


def select_params(alpha=0.1, sink_blocks=2, window_blocks=4, block_size=128) -> SelectParams:
    return SelectParams(alpha, block_size, sink_blocks, window_blocks)


def query_sizes(batch: Batch, params: SelectParams | None = None) -> Sizes:
    out = Sizes()
    _check(_lib.fp_query_sizes(batch.ptr, C.byref(params) if params is not None else None, C.byref(out)))
    return out


def block_base(batch: Batch, b: int) -> int:
    return int(_lib.fp_block_base(batch.ptr, b))


class Buffers:
    """Caller-owned device buffers sized by fp_query_sizes."""

    def __init__(self, batch: Batch, params: SelectParams | None = None, device="cuda"):
        s = query_sizes(batch, params)
        self.sizes = s
        self.cu = torch.zeros(s.n_segments + 1, dtype=torch.int32, device=device)
        self.idx = torch.zeros(max(1, s.idx_capacity), dtype=torch.int32, device=device)
        self.means = torch.zeros(max(1, s.means_bytes), dtype=torch.uint8, device=device)
        self.ws = torch.zeros(max(1, s.workspace_bytes), dtype=torch.uint8, device=device)


def pool(batch: Batch, k, v, bufs: Buffers):
    _check(_lib.fp_pool(batch.ptr, _ptr(k), _ptr(v), _ptr(bufs.means), _ptr(bufs.ws), bufs.ws.numel(),
                        _stream()))


def select(batch: Batch, params: SelectParams, q, k, v, bufs: Buffers, energies=None):
    _check(_lib.fp_select(batch.ptr, C.byref(params), _ptr(q), _ptr(k), _ptr(v), _ptr(bufs.cu),
                          _ptr(bufs.idx), bufs.idx.numel(), _ptr(bufs.means), _ptr(energies),
                          _ptr(bufs.ws), bufs.ws.numel(), _stream()))


def sparse_attn(batch: Batch, params: SelectParams, q, k, v, bufs: Buffers, out, lse=None, correction=True):
    _check(_lib.fp_sparse_attn(batch.ptr, C.byref(params), _ptr(q), _ptr(k), _ptr(v), _ptr(bufs.cu),
                               _ptr(bufs.idx), _ptr(bufs.means), 1 if correction else 0, _ptr(out),
                               _ptr(lse), _ptr(bufs.ws), bufs.ws.numel(), _stream()))


def sparse_attn_static(batch: Batch, params: SelectParams, q, k, v, cu, idx, means, out, lse=None,
                       correction=True):
    """fp_sparse_attn on the library's static scratch (no workspace argument)."""
    _check(_lib.fp_sparse_attn_static(batch.ptr, C.byref(params), _ptr(q), _ptr(k), _ptr(v), _ptr(cu), _ptr(idx),
                                      _ptr(means), 1 if correction else 0, _ptr(out), _ptr(lse), _stream()))


def dense_attn(batch: Batch, q, k, v, bufs: Buffers, out, lse=None):
    _check(_lib.fp_dense_attn(batch.ptr, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(bufs.ws),
                              bufs.ws.numel(), _stream()))


def block_mass(batch: Batch, q, k, lse, bufs: Buffers, mass, surrogate=None):
    """Exact per-block attention mass [n_segments, max_blocks] (and the mean surrogate);
    ``lse`` from :func:`dense_attn`, ``bufs.means`` from :func:`select` or :func:`pool`."""
    _check(_lib.fp_block_mass(batch.ptr, _ptr(q), _ptr(k), _ptr(lse), _ptr(bufs.means), _ptr(mass),
                              _ptr(surrogate), _ptr(bufs.ws), bufs.ws.numel(), _stream()))


def read_device_error(bufs: Buffers) -> int:
    flag = C.c_int32(0)
    st = _lib.fp_read_device_error(_ptr(bufs.ws), _stream(), C.byref(flag))
    if st not in (0, -6):
        raise FPError(st)
    return flag.value


def means_f32(bufs: Buffers, nb_pad: int, hkv: int):
    """(kbar, vbar) float views [nb_pad, hkv, 128] of the pooled-statistics buffer."""
    n = nb_pad * hkv * 128
    f = bufs.means.view(torch.float32)
    kb = f[:n].view(nb_pad, hkv, 128)
    off = ((n * 4 + 255) // 256 * 256) // 4
    vb = f[off:off + n].view(nb_pad, hkv, 128)
    return kb, vb


def lib_handle():
    return _lib
