"""GPU tests of the boundary's options: the device check of the offsets
(HSTU_VALIDATE), the schedule shared by a step's forward and backward, and the
stored score gradient sized from a stated sum of squared lengths.  Every
malformed offsets array here stays inside the tensors it describes, so a
check that failed to fire could not address memory out of bounds."""

import numpy as np
import pytest

import oracle
import synth
from hstu_testlib import assert_close, to_f64, upload

pytestmark = pytest.mark.gpu


def hstu():
    import jagged_hstu_attention_amd as m
    return m


def wl_small(seed=71):
    return synth.custom([300, 1, 129, 0, 500], num_heads=2, d_qk=128, d_v=128, num_buckets=128, dtype="bf16",
                        gap_mean=3600.0, seed=seed, w_std=0.5)


def test_validate_accepts_good_offsets_and_changes_nothing(monkeypatch):
    import torch
    wl = wl_small()
    d = upload(wl)
    m = hstu()
    args = (d["q"], d["k"], d["v"], d["offsets"], d["ts"], d["w"], wl.max_seq_len)
    plain = m.jagged_attn_fwd(*args)
    bplain = m.jagged_attn_bwd(d["dout"], *args)
    monkeypatch.setenv("HSTU_VALIDATE", "1")
    checked = m.jagged_attn_fwd(*args)
    bchecked = m.jagged_attn_bwd(d["dout"], *args)
    assert torch.equal(plain, checked)
    for a, b in zip(bplain[:3], bchecked[:3]):
        assert torch.equal(a, b)
    assert_close(to_f64(bchecked[3]), to_f64(bplain[3]), "bf16", "dw")


@pytest.mark.parametrize("case", ["short_total", "decreasing", "too_long", "nonzero_first"])
def test_validate_rejects_bad_offsets(monkeypatch, case):
    import torch
    wl = wl_small()
    d = upload(wl)
    m = hstu()
    off = wl.offsets.copy()
    max_len = wl.max_seq_len
    if case == "short_total":        # offsets[B] < total_kv: rows left over
        off[-1] -= 7
        want = "offsets[B]"
    elif case == "decreasing":       # a sequence of negative length, inside [0, T]
        off[2] = off[3] + 5
        want = "decrease"
    elif case == "too_long":         # a sequence longer than the stated maximum
        max_len = 400
        want = "max_seq_len"
    else:
        off[0] = 3
        want = "offsets[0]"
    dev_off = torch.from_numpy(off).cuda()
    monkeypatch.setenv("HSTU_VALIDATE", "1")
    args = (d["q"], d["k"], d["v"], dev_off, d["ts"], d["w"], max_len)
    for call in (lambda: m.jagged_attn_fwd(*args), lambda: m.jagged_attn_bwd(d["dout"], *args)):
        with pytest.raises(m.HstuError) as e:
            call()
        assert e.value.status == 1 and want in str(e.value), str(e.value)
    with pytest.raises(m.HstuError) as e:
        m.cp_reorder(d["q"], dev_off, max_len, 2)
    assert e.value.status == 1 and want in str(e.value)
    torch.cuda.synchronize()


def test_validate_checks_the_rank_row_count(monkeypatch):
    wl = wl_small()
    d = upload(wl)
    m = hstu()
    monkeypatch.setenv("HSTU_VALIDATE", "1")
    q, seg = m.cp_reorder(d["q"], d["offsets"], wl.max_seq_len, 2)
    seg = seg.cpu().numpy()
    lo, hi = int(seg[0]), int(seg[wl.num_seqs])
    ql = q[lo:hi].contiguous()
    m.jagged_attn_fwd(ql, d["k"], d["v"], d["offsets"], d["ts"], d["w"], wl.max_seq_len, cp_size=2, cp_rank=0)
    with pytest.raises(m.HstuError) as e:  # rank 1's problem given rank 0's rows
        m.jagged_attn_fwd(ql[:-1].contiguous(), d["k"], d["v"], d["offsets"], d["ts"], d["w"], wl.max_seq_len,
                          cp_size=2, cp_rank=1)
    assert "query row count" in str(e.value)


@pytest.mark.parametrize("dtype,dim,recompute", [("bf16", 128, False), ("bf16", 64, True), ("fp32", 32, False)])
def test_shared_schedule_equals_separate_schedules(dtype, dim, recompute):
    # one scheduler launch per step: the forward builds both passes' lists in a
    # backward-sized workspace, the backward reuses them; three steps in a row
    # give the same bits as calls that schedule for themselves
    import torch
    wl = synth.custom([4000, 100, 1, 700], num_heads=2, d_qk=dim, d_v=dim, num_buckets=128, dtype=dtype,
                      gap_mean=600.0, seed=72 + dim, w_std=0.5)
    d = upload(wl)
    m = hstu()
    args = (d["q"], d["k"], d["v"], d["offsets"], d["ts"], d["w"], wl.max_seq_len)
    o_ref = m.jagged_attn_fwd(*args)
    g_ref = m.jagged_attn_bwd(d["dout"], *args, recompute=recompute)
    p = m.problem(d["q"], d["k"], d["v"], d["offsets"], d["w"], wl.max_seq_len, shared_schedule=True,
                  recompute_bwd=recompute)
    ws = torch.empty(m.workspace_size(p, True), dtype=torch.uint8, device="cuda")
    for _ in range(3):
        o = m.jagged_attn_fwd(*args, workspace=ws, shared_schedule=True, recompute_bwd=recompute)
        g = m.jagged_attn_bwd(d["dout"], *args, workspace=ws, shared_schedule=True, recompute=recompute)
        assert torch.equal(o, o_ref)
        for name, a, b in zip(("dq", "dk", "dv"), g, g_ref):
            assert torch.equal(a, b), name
        assert_close(to_f64(g[3]), to_f64(g_ref[3]), dtype, "dw")
    rq, rk, rv, rw = oracle.attn_bwd(wl.dout.f64, wl.q.f64, wl.k.f64, wl.v.f64, wl.offsets, wl.ts, wl.w.f64, 128)
    assert_close(to_f64(g[3]), rw, dtype, "dw vs oracle")
    assert_close(to_f64(g[0]), rq, dtype, "dq vs oracle")


def test_stated_sum_of_squares_gives_the_same_gradients():
    import torch
    wl = synth.config("skewed_powerlaw", num_seqs=48)
    d = upload(wl)
    m = hstu()
    args = (d["dout"], d["q"], d["k"], d["v"], d["offsets"], d["ts"], d["w"], wl.max_seq_len)
    sq = int(sum(int(L) ** 2 for L in wl.lengths))
    p_loose = m.problem(d["q"], d["k"], d["v"], d["offsets"], d["w"], wl.max_seq_len)
    p_tight = m.problem(d["q"], d["k"], d["v"], d["offsets"], d["w"], wl.max_seq_len, sum_sq_len=sq)
    assert m.workspace_size(p_tight, True) < m.workspace_size(p_loose, True)
    a = m.jagged_attn_bwd(*args)
    b = m.jagged_attn_bwd(*args, sum_sq_len=sq)
    for name, x, y in zip(("dq", "dk", "dv"), a, b):
        assert torch.equal(x, y), name
    rq, rk, rv, rw = oracle.attn_bwd(wl.dout.f64, wl.q.f64, wl.k.f64, wl.v.f64, wl.offsets, wl.ts, wl.w.f64,
                                     wl.num_buckets)
    for name, got, r in [("dq", b[0], rq), ("dk", b[1], rk), ("dv", b[2], rv), ("dw", b[3], rw)]:
        assert_close(to_f64(got), r, "bf16", name)
