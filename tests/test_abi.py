"""The C-ABI library: it loads, exports what include/hstu.h declares, its host
logic (edge table, validation, workspace sizing) is right.  CPU only: no call
here reaches a kernel launch (validation rejects every argument set first)."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import jagged_hstu_attention_amd as hstu
from jagged_hstu_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hstu.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hstu_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = declared_functions()
    assert len(names) >= 7
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.EXPORTS)


def test_version():
    assert hstu.version() == 100


@pytest.mark.parametrize("nb", [1, 2, 7, 32, 100, 128, 256, 512])
def test_library_edge_table_equals_oracle(nb):
    got = hstu.bucket_edges(nb)
    want = [0] + oracle.bucket_edges(nb) + [0xFFFFFFFF]
    assert got == want


def test_edge_table_rejects_bad_sizes():
    with pytest.raises(hstu.HstuError) as e:
        hstu.bucket_edges(0)
    assert e.value.status == 1
    with pytest.raises(hstu.HstuError) as e:
        hstu.bucket_edges(513)
    assert e.value.status == 2


def make_problem(**kw):
    p = hstu.Problem()
    base = dict(dtype=0, flags=0, num_seqs=4, num_heads=2, d_qk=64, d_v=64, num_buckets=128,
                max_seq_len=100, total_kv=300, total_q=300, cp_size=1, cp_rank=0)
    base.update(kw)
    for k, v in base.items():
        setattr(p, k, v)
    return p


def test_workspace_size_valid_and_monotone():
    small = hstu.workspace_size(make_problem(), False)
    bwd = hstu.workspace_size(make_problem(), True)
    big = hstu.workspace_size(make_problem(total_kv=30000, total_q=30000, max_seq_len=10000), False)
    assert 0 < small <= bwd
    assert big > small
    assert small % 256 == 0


@pytest.mark.parametrize("kw,stored", [
    (dict(), True), (dict(d_qk=128, d_v=128, max_seq_len=300, num_seqs=1), True),
    (dict(dtype=1), False), (dict(d_qk=32, d_v=32), False), (dict(cp_size=2, total_q=150), False),
])
def test_backward_workspace_holds_score_gradient_blocks(kw, stored):
    # bf16, d >= 64, one CP rank: the backward workspace holds the stored score
    # gradient, 16 KiB blocks of 64 keys x 128 query rows, bounded by
    # H (N + 1) (ceil(T / 128) + B) with N = ceil(max_seq_len / 128), plus the
    # per-sequence block offsets (int64 [B + 1], 256-byte aligned); the
    # memory-efficient flag drops both.  Otherwise the flag changes nothing.
    p = make_problem(**kw)
    lean = make_problem(flags=hstu.HSTU_FLAG_RECOMPUTE_BWD, **kw)
    full, small = hstu.workspace_size(p, True), hstu.workspace_size(lean, True)
    assert hstu.workspace_size(p, False) == hstu.workspace_size(lean, False)
    if not stored:
        assert full == small
        return
    n = -(-p.max_seq_len // 128)
    blocks = p.num_heads * (n + 1) * (-(-p.total_kv // 128) + p.num_seqs)
    offsets = -(-(p.num_seqs + 1) * 8 // 256) * 256
    assert full - small == blocks * 64 * 128 * 2 + offsets


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=5), 1), (dict(flags=2), 1), (dict(flags=-1), 1), (dict(num_seqs=-1), 1), (dict(num_heads=0), 1),
    (dict(d_qk=48, d_v=48), 2), (dict(d_v=32), 2), (dict(num_buckets=0), 1), (dict(num_buckets=1000), 2),
    (dict(cp_size=0), 1), (dict(cp_size=2, cp_rank=2), 1), (dict(cp_rank=-1), 1),
    (dict(total_q=10), 1), (dict(max_seq_len=400), 1), (dict(max_seq_len=0), 1),
    (dict(cp_size=2, cp_rank=0, total_q=400), 1),
])
def test_validation_errors(kw, status):
    p = make_problem(**kw)
    lib = _lib.load()
    assert lib.hstu_workspace_size(ctypes.byref(p), 1) == 0
    dummy = ctypes.c_void_p(16)
    rc = lib.hstu_jagged_attn_fwd(ctypes.byref(p), dummy, dummy, dummy, dummy, dummy, dummy, dummy, dummy,
                                  1 << 30, None)
    assert rc == status
    assert lib.hstu_last_error()


def test_null_and_misaligned_pointers_rejected():
    p = make_problem()
    lib = _lib.load()
    good = ctypes.c_void_p(1 << 20)
    bad = ctypes.c_void_p((1 << 20) + 2)
    ws = hstu.workspace_size(p, False)
    args = [good] * 8
    rc = lib.hstu_jagged_attn_fwd(ctypes.byref(p), None, *args[1:7], good, ws, None)
    assert rc == 1 and b"q is NULL" in lib.hstu_last_error()
    rc = lib.hstu_jagged_attn_fwd(ctypes.byref(p), bad, *args[1:7], good, ws, None)
    assert rc == 1 and b"aligned" in lib.hstu_last_error()
    # workspace too small
    rc = lib.hstu_jagged_attn_fwd(ctypes.byref(p), *args[:7], good, ws - 1, None)
    assert rc == 3
    rc = lib.hstu_jagged_attn_fwd(ctypes.byref(p), *args[:7], None, ws, None)
    assert rc == 3
    # backward: d_ts_weights NULL
    wsb = hstu.workspace_size(p, True)
    rc = lib.hstu_jagged_attn_bwd(ctypes.byref(p), *([good] * 10), None, good, wsb, None)
    assert rc == 1 and b"d_ts_weights" in lib.hstu_last_error()


def test_reorder_validation():
    lib = _lib.load()
    g = ctypes.c_void_p(1 << 20)
    o = ctypes.c_void_p(1 << 21)
    assert lib.hstu_cp_reorder(g, o, 0, g, 2, 10, 5, 2, 0, None, None) == 1    # row_bytes
    assert lib.hstu_cp_reorder(g, o, 8, g, 2, 10, 5, 0, 0, None, None) == 1    # cp_size
    assert lib.hstu_cp_reorder(g, o, 8, g, 2, 10, 11, 2, 0, None, None) == 1   # max_seq_len > rows
    assert lib.hstu_cp_reorder(g, g, 8, g, 2, 10, 5, 2, 0, None, None) == 1    # overlap
    assert lib.hstu_cp_reorder(None, o, 8, g, 2, 10, 5, 2, 0, None, None) == 1
    # nothing to do: no launch, OK
    assert lib.hstu_cp_reorder(g, o, 8, g, 0, 0, 0, 2, 0, None, None) == 0


def test_timing_api_without_launches():
    import jagged_hstu_attention_amd as m
    m.timing_reset()
    m.timing_enable(True)
    m.timing_enable(False)
    for k in ("sched", "fwd", "bwd_kv", "bwd_q", "reorder", "reduce"):
        assert m.timing_read(k) == (0.0, 0)
    lib = _lib.load()
    ms, n = ctypes.c_double(), ctypes.c_int64()
    assert lib.hstu_timing_read(5, ctypes.byref(ms), ctypes.byref(n)) == 0  # the split-sum kernel
    assert lib.hstu_timing_read(6, ctypes.byref(ms), ctypes.byref(n)) == 1  # one past the last id
    assert lib.hstu_timing_read(-1, ctypes.byref(ms), ctypes.byref(n)) == 1


def _lut_model(edges, nb):
    """Host model of the kernels' exact-bucket table: entry (z << 5) | j covers
    the integers with z leading zeros and sub-bin j; bucket = b + [m >= E]."""
    e_arr = np.array(edges[1:nb], dtype=np.uint64)
    table = []
    for idx in range(1024):
        e, j = 31 - (idx >> 5), idx & 31
        if e >= 5:
            lo = (32 + j) << (e - 5)
            hi = lo + (1 << (e - 5)) - 1
        else:
            step = 1 << (5 - e)
            if j % step:
                table.append((0, 0xFFFFFFFF))
                continue
            lo = hi = (1 << e) + j // step
        b0 = int(np.searchsorted(e_arr, lo, side="right"))
        if b0 + 1 < nb and edges[b0 + 1] <= hi:
            table.append((edges[b0 + 1], b0))
        else:
            table.append((0, (b0 - 1) & 0xFFFFFFFF))
    return table


def _lut_lookup(table, m):
    m = max(int(m), 1)
    z = 32 - m.bit_length()
    t = (m << z) & 0xFFFFFFFF
    E, b = table[(z << 5) | ((t >> 26) & 31)]
    return ((b + (1 if m >= E else 0)) & 0xFFFFFFFF)


@pytest.mark.parametrize("nb", [1, 2, 3, 31, 32, 33, 100, 128, 256, 300, 511, 512])
def test_exact_bucket_table_model_matches_oracle(nb):
    edges = hstu.bucket_edges(nb)
    table = _lut_model(edges, nb)
    rng = np.random.default_rng(nb)
    vals = set(range(0, 300))
    for k in range(1, nb):
        E = edges[k]
        vals.update(x for x in (E - 1, E, E + 1) if 0 <= x < 2 ** 32)
    for p in range(33):
        vals.update(x for x in ((1 << p) - 1, 1 << p, (1 << p) + 1) if 0 <= x < 2 ** 32)
    vals.update(int(x) for x in rng.integers(0, 2 ** 32, size=2000, dtype=np.uint64))
    vals = np.array(sorted(vals), dtype=np.int64)
    want = oracle.bucketize(vals, nb)
    got = np.array([_lut_lookup(table, v) for v in vals])
    assert np.array_equal(got, want)


def test_every_sub_bin_holds_at_most_one_edge():
    for nb in range(1, 513):
        e = np.array(hstu.bucket_edges(nb)[1:nb], dtype=np.int64)
        for oct_ in range(5, 32):
            lo = (32 + np.arange(32, dtype=np.int64)) << (oct_ - 5)
            hi = lo + (1 << (oct_ - 5)) - 1
            inside = np.searchsorted(e, hi, side="right") - np.searchsorted(e, lo, side="right")
            assert inside.max() <= 1, (nb, oct_)


def test_candidates_forward_validation():
    lib = _lib.load()
    dummy = ctypes.c_void_p(16)

    def call(p, num_targets=dummy, only=0):
        return lib.hstu_jagged_attn_fwd_targets(ctypes.byref(p), dummy, dummy, dummy, dummy, num_targets, only,
                                                dummy, dummy, dummy, dummy, 1 << 30, None)

    # a forward may query a subset of the rows (the candidates-only pass)
    assert lib.hstu_workspace_size(ctypes.byref(make_problem(total_q=10)), 0) > 0
    assert call(make_problem(cp_size=2, cp_rank=0, total_q=150)) == 2
    assert call(make_problem(), only=2) == 1
    assert call(make_problem(total_q=10), only=0) == 1
    assert call(make_problem(total_q=400), only=1) == 1
    assert call(make_problem(), num_targets=None) == 1
    assert call(make_problem(), num_targets=ctypes.c_void_p(20)) == 1
    # the plain forward still requires all rows
    p = make_problem(total_q=10)
    assert lib.hstu_jagged_attn_fwd(ctypes.byref(p), dummy, dummy, dummy, dummy, dummy, dummy, dummy, dummy,
                                    1 << 30, None) == 1
