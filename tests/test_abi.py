"""CPU checks of the C ABI: the library loads, exports every declared entry
point, and rejects bad host arguments before launching anything."""
import ctypes as C
import math
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp.h")


def _fp():
    from block_sparse_long_mean_amd import fp
    return fp


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fp_[a-z_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["fp_query_sizes", "fp_pool", "fp_select", "fp_sparse_attn", "fp_dense_attn",
              "fp_read_device_error", "fp_status_string", "fp_last_error", "fp_block_base"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    fp = _fp()
    lib = fp.lib_handle()
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_binding_lists_exactly_the_declared_functions():
    """The binding's export list names every function the header declares, and nothing else."""
    assert sorted(_fp().EXPORTS) == declared_functions()


def test_library_exports_match_the_header():
    """The shared object's exported fp_* functions are exactly the header's."""
    lib = os.path.join(ROOT, "block_sparse_long_mean_amd", "libfp.so")
    out = subprocess.run(["nm", "-D", "--defined-only", lib], capture_output=True, text=True, check=True).stdout
    exported = sorted({ln.split()[-1] for ln in out.splitlines()
                       if ln.split() and ln.split()[-1].startswith("fp_") and " T " in ln})
    assert exported == declared_functions()


def _problem(fp, lengths=(1000, 300), hq=32, hkv=4, dtype=1, **kw):
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    p = fp.Problem()
    p.num_reqs = len(lengths)
    p.num_heads_q = hq
    p.num_heads_kv = hkv
    p.head_dim = kw.get("head_dim", 128)
    p.cu_seqlens_q = 0x1000  # never dereferenced on the host
    p.cu_seqlens_q_host = cu.ctypes.data
    p.page_table = kw.get("page_table", None)
    p.page_size = kw.get("page_size", 0)
    p.max_pages_per_req = kw.get("max_pages", 0)
    p.num_pool_slots = kw.get("slots", 0)
    p.dtype = dtype
    p.descale = kw.get("descale", None)
    p.softmax_scale = kw.get("scale", 0.0)
    return p, cu


def _sizes(fp, p, params=None):
    out = fp.Sizes()
    st = fp.lib_handle().fp_query_sizes(C.byref(p), C.byref(params) if params else None, C.byref(out))
    return st, out


def test_query_sizes_geometry():
    fp = _fp()
    p, cu = _problem(fp, lengths=(1000, 300))
    st, s = _sizes(fp, p, fp.select_params())
    assert st == 0
    g = 8
    nseg = 4 * (math.ceil(g * 1000 / 128) + math.ceil(g * 300 / 128))
    assert s.n_segments == nseg
    assert s.max_blocks == 8
    # worst-case CSR: every causal 64-token tile of every segment
    cap = 0
    for L in (1000, 300):
        for I in range(math.ceil(g * L / 128)):
            t1 = (min((I + 1) * 128, g * L) - 1) // g
            cap += 4 * (t1 // 64 + 1)
    assert s.idx_capacity == cap
    assert s.means_bytes > 0 and s.workspace_bytes > 0
    assert fp.lib_handle().fp_block_base(C.byref(p), 1) == 64


@pytest.mark.parametrize("field,value,code", [
    ("head_dim", 64, -2),
    ("num_heads_q", 30, -1),
    ("num_heads_q", 4 * 3, -2),
    ("dtype", 7, -1),
    ("num_reqs", 0, -1),
    ("softmax_scale", float("nan"), -1),
])
def test_invalid_problems_are_rejected(field, value, code):
    fp = _fp()
    p, cu = _problem(fp)
    setattr(p, field, value)
    st, _ = _sizes(fp, p)
    assert st == code, fp.lib_handle().fp_last_error()
    assert fp.lib_handle().fp_last_error()


def test_decreasing_offsets_and_missing_descale_are_rejected():
    fp = _fp()
    p, cu = _problem(fp, lengths=(100, 200))
    cu[2] = 50
    assert _sizes(fp, p)[0] == -1
    p, cu = _problem(fp, dtype=2)
    assert _sizes(fp, p)[0] == -1
    p, cu = _problem(fp, lengths=(1 << 21,))
    assert _sizes(fp, p)[0] == -2


def test_paged_arguments_are_checked():
    fp = _fp()
    pt = np.zeros((2, 4), np.int32)
    p, cu = _problem(fp, lengths=(1000, 300), page_table=pt.ctypes.data, page_size=64, max_pages=4, slots=1 << 20)
    assert _sizes(fp, p)[0] == -1  # 4 pages of 64 cannot hold 1000 tokens
    p.max_pages_per_req = 16
    assert _sizes(fp, p)[0] == 0
    p.page_size = 0
    assert _sizes(fp, p)[0] == -1


@pytest.mark.parametrize("alpha,block,sink,code", [(float("nan"), 128, 2, -1), (-0.1, 128, 2, -1),
                                                    (0.1, 64, 2, -2), (0.1, 128, -1, -1)])
def test_invalid_select_params(alpha, block, sink, code):
    fp = _fp()
    p, cu = _problem(fp)
    sp = fp.SelectParams(alpha, block, sink, 4)
    assert _sizes(fp, p, sp)[0] == code


def test_calls_fail_before_launch_on_small_buffers():
    fp = _fp()
    lib = fp.lib_handle()
    p, cu = _problem(fp)
    sp = fp.select_params()
    st, s = _sizes(fp, p, sp)
    dummy = C.c_void_p(0x1000)
    # workspace too small
    r = lib.fp_select(C.byref(p), C.byref(sp), dummy, dummy, dummy, dummy, dummy, s.idx_capacity, dummy, None,
                      dummy, s.workspace_bytes - 1, None)
    assert r == -3
    # idx capacity too small
    r = lib.fp_select(C.byref(p), C.byref(sp), dummy, dummy, dummy, dummy, dummy, s.idx_capacity - 1, dummy,
                      None, dummy, s.workspace_bytes, None)
    assert r == -4
    # missing tensors
    r = lib.fp_sparse_attn(C.byref(p), C.byref(sp), None, dummy, dummy, dummy, dummy, dummy, 1, dummy, None,
                           dummy, s.workspace_bytes, None)
    assert r == -1
    r = lib.fp_dense_attn(C.byref(p), dummy, dummy, dummy, dummy, None, None, s.workspace_bytes, None)
    assert r == -1
    assert lib.fp_status_string(-3) == b"workspace too small"
    # block mass: lse and mass are required; the surrogate needs the means
    r = lib.fp_block_mass(C.byref(p), dummy, dummy, None, dummy, dummy, None, dummy, s.workspace_bytes, None)
    assert r == -1
    r = lib.fp_block_mass(C.byref(p), dummy, dummy, dummy, None, dummy, dummy, dummy, s.workspace_bytes, None)
    assert r == -1
    r = lib.fp_block_mass(C.byref(p), dummy, dummy, dummy, None, dummy, None, dummy, s.workspace_bytes - 1,
                          None)
    assert r == -3


def test_chunked_problem_geometry_and_checks():
    """K/V lengths from cu_seqlens_kv: segments from the queries, blocks and the
    worst-case CSR from the keys (queries at positions L_kv - L_q ..)."""
    fp = _fp()
    p, cu = _problem(fp, lengths=(1000, 300))
    ckv = np.array([0, 3000, 3300], np.int32)
    p.cu_seqlens_kv = 0x2000  # never dereferenced on the host
    p.cu_seqlens_kv_host = ckv.ctypes.data
    st, s = _sizes(fp, p, fp.select_params())
    assert st == 0, fp.lib_handle().fp_last_error()
    g = 8
    assert s.n_segments == 4 * (math.ceil(g * 1000 / 128) + math.ceil(g * 300 / 128))
    assert s.max_blocks == math.ceil(3000 / 128)
    cap = 0
    for L, Lq in ((3000, 1000), (300, 300)):
        for I in range(math.ceil(g * Lq / 128)):
            t1 = L - Lq + (min((I + 1) * 128, g * Lq) - 1) // g
            cap += 4 * (t1 // 64 + 1)
    assert s.idx_capacity == cap
    assert fp.lib_handle().fp_block_base(C.byref(p), 1) == 64  # ceil(24 / 64) * 64
    # fewer keys than queries
    ckv[1] = 999
    assert _sizes(fp, p)[0] == -1
    ckv[1] = 3000
    # the two K/V offset pointers go together
    p.cu_seqlens_kv_host = None
    assert _sizes(fp, p)[0] == -1


def test_problem_struct_matches_the_header(tmp_path):
    """The binding's ctypes layout of fp_problem equals the C compiler's."""
    fp = _fp()
    src = tmp_path / "lay.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "fp.h"\n'
                   'int main(void){printf("%zu %zu %zu %zu\\n", sizeof(fp_problem),'
                   ' offsetof(fp_problem, softmax_scale), offsetof(fp_problem, cu_seqlens_kv),'
                   ' offsetof(fp_problem, cu_seqlens_kv_host)); return 0;}\n')
    exe = tmp_path / "lay"
    subprocess.check_call(["gcc", "-I", os.path.join(ROOT, "include"), "-o", str(exe), str(src)])
    got = [int(x) for x in subprocess.check_output([str(exe)]).split()]
    P = fp.Problem
    assert got == [C.sizeof(P), P.softmax_scale.offset, P.cu_seqlens_kv.offset,
                   P.cu_seqlens_kv_host.offset]


def test_column_major_v_checks():
    fp = _fp()
    p, cu = _problem(fp, lengths=(1008, 304), dtype=2, descale=0x3000)
    p.v_layout = 1
    assert _sizes(fp, p)[0] == 0, fp.lib_handle().fp_last_error()
    p.v_layout = 2
    assert _sizes(fp, p)[0] == -1
    # an E4M3 layout only
    p, cu = _problem(fp, lengths=(1008, 304), dtype=1)
    p.v_layout = 1
    assert _sizes(fp, p)[0] == -2
    # contiguous: every K/V offset a multiple of 16
    p, cu = _problem(fp, lengths=(1000, 304), dtype=2, descale=0x3000)
    p.v_layout = 1
    assert _sizes(fp, p)[0] == -2
    # paged: pages a multiple of 64 tokens, the pool a whole number of pages
    pt = np.zeros((2, 32), np.int32)
    p, cu = _problem(fp, lengths=(1000, 300), dtype=2, descale=0x3000, page_table=pt.ctypes.data,
                     page_size=64, max_pages=32, slots=64 * 40)
    p.v_layout = 1
    assert _sizes(fp, p)[0] == 0, fp.lib_handle().fp_last_error()
    p.page_size, p.max_pages_per_req = 48, 32
    assert _sizes(fp, p)[0] == -2
    p.page_size, p.num_pool_slots = 64, 64 * 40 + 3
    assert _sizes(fp, p)[0] == -2


def test_empty_batch_launches_nothing():
    """Every request empty: the calls return before launching anything."""
    fp = _fp()
    lib = fp.lib_handle()
    p, cu = _problem(fp, lengths=(0, 0))
    sp = fp.select_params()
    st, s = _sizes(fp, p, sp)
    assert st == 0 and s.n_segments == 0
    dummy = C.c_void_p(0x1000)
    ws = max(1, s.workspace_bytes)
    assert lib.fp_select(C.byref(p), C.byref(sp), dummy, dummy, dummy, dummy, dummy, max(1, s.idx_capacity),
                         dummy, None, dummy, ws, None) == 0
    assert lib.fp_sparse_attn(C.byref(p), C.byref(sp), dummy, dummy, dummy, dummy, dummy, dummy, 1, dummy, None,
                              dummy, ws, None) == 0
    assert lib.fp_dense_attn(C.byref(p), dummy, dummy, dummy, dummy, None, dummy, ws, None) == 0


def test_step_count_bound_near_int32_limit():
    """The scheduler sums per-segment step counts (listed tiles plus correction
    chunks) in int32.  Two E4M3 requests of 1,048,576 and L2 tokens with 31
    heads, g = 1: for some L2 the worst-case index still fits int32 but the
    worst-case step count does not; such a problem is refused before anything
    is sized, while a slightly shorter L2 is accepted."""
    fp = _fp()
    refused = accepted = None
    for L2 in range(147456, 188416, 4096):
        p, cu = _problem(fp, lengths=(8192 * 128, L2), hq=31, hkv=31, dtype=2, descale=0x1000)
        st, out = _sizes(fp, p)
        msg = fp.lib_handle().fp_last_error().decode()
        if st == 0:
            accepted = (L2, out.idx_capacity)
        elif "attention steps" in msg:
            assert st == -2
            refused = L2
            break
    assert accepted is not None and refused is not None, (accepted, refused)
    assert accepted[1] <= 2**31 - 1 and accepted[0] < refused


def test_static_scratch_entry_point_checks_on_the_host():
    """fp_sparse_attn_static: missing buffers and problems whose workspace exceeds
    the static scratch are refused before anything touches a device."""
    fp = _fp()
    lib = fp.lib_handle()
    params = fp.select_params(0.1, 2, 4)
    p, cu = _problem(fp)
    st = lib.fp_sparse_attn_static(C.byref(p), C.byref(params), None, None, None, None, None, None, 1, None,
                                   None, None)
    assert st == -1
    # 4096 requests of 16K tokens, MHA with one head: 524,288 segments need ~42 MB of scratch
    lengths = (16384,) * 4096
    p, cu = _problem(fp, lengths=lengths, hq=1, hkv=1)
    st, out = _sizes(fp, p)
    assert st == 0 and out.n_segments == 4096 * 128
    dummy = 0x1000  # never dereferenced: the size check refuses first
    st = lib.fp_sparse_attn_static(C.byref(p), C.byref(params), dummy, dummy, dummy, dummy, dummy, dummy, 1,
                                   dummy, None, None)
    assert st == -3 and "static scratch" in lib.fp_last_error().decode()
