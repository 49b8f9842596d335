"""GPU parity of the context-parallel share and the chunk-pair reorder."""

import numpy as np
import pytest

import oracle
import synth
from hstu_testlib import assert_close, to_f64, upload, upload_array

pytestmark = pytest.mark.gpu


def hstu():
    import jagged_hstu_attention_amd as m
    return m


# --------------------------------------------------------------------------
# Reorder: bit-exact against the oracle's index permutation.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("lengths,cp", [([16, 16, 16], 2), ([13, 1, 0, 22, 5, 64], 4), ([7, 31, 100], 8),
                                        ([1000, 17], 1), ([5, 3], 8)])
@pytest.mark.parametrize("row_shape,dtype", [((4, 128), "bf16"), ((1,), "i64"), ((3,), "u8"), ((2, 5), "f32")])
def test_reorder_bit_exact(lengths, cp, row_shape, dtype):
    import torch
    off = synth.offsets_from_lengths(lengths)
    T = int(off[-1])
    rng = np.random.default_rng(T + cp)
    if dtype == "bf16":
        x = rng.integers(0, 1 << 16, size=(T, *row_shape), dtype=np.uint16).view(np.int16)
    elif dtype == "i64":
        x = rng.integers(-(1 << 62), 1 << 62, size=(T, *row_shape), dtype=np.int64)
    elif dtype == "u8":
        x = rng.integers(0, 256, size=(T, *row_shape), dtype=np.uint8)
    else:
        x = rng.standard_normal(size=(T, *row_shape)).astype(np.float32)
    dx = upload_array(x)
    doff = upload_array(off)
    y, seg = hstu().cp_reorder(dx, doff, int(max(lengths)), cp)
    want, want_off = oracle.reorder(x, off, cp)
    assert np.array_equal(y.cpu().numpy().view(np.uint8), want.view(np.uint8))
    assert np.array_equal(seg.cpu().numpy(), want_off)
    back, _ = hstu().cp_reorder(y, doff, int(max(lengths)), cp, inverse=True)
    assert np.array_equal(back.cpu().numpy().view(np.uint8), x.view(np.uint8))
    if cp == 1:
        assert torch.equal(y, dx)


def test_reorder_len16384_cp8_bit_exact():
    wl = synth.config("cp8_rank3_len16384", with_dout=False)
    d = upload(wl)
    m = hstu()
    for t, name in [(d["q"], "q"), (d["ts"], "ts")]:
        y, seg = m.cp_reorder(t, d["offsets"], wl.max_seq_len, synth.CP_SIZE)
        idx, want_off = oracle.reorder_index(wl.offsets, synth.CP_SIZE)
        host = t.cpu()
        assert np.array_equal(seg.cpu().numpy(), want_off), name
        import torch
        assert torch.equal(y.cpu(), host[torch.from_numpy(idx)]), name
        back, _ = m.cp_reorder(y, d["offsets"], wl.max_seq_len, synth.CP_SIZE, inverse=True)
        assert torch.equal(back, t), name


# --------------------------------------------------------------------------
# CP share: each rank's forward/backward against the oracle and the unsharded
# run.
# --------------------------------------------------------------------------

def rank_inputs(m, d, wl, cp, r):
    q_re, seg = m.cp_reorder(d["q"], d["offsets"], wl.max_seq_len, cp)
    do_re, _ = m.cp_reorder(d["dout"], d["offsets"], wl.max_seq_len, cp)
    seg = seg.cpu().numpy()
    B = wl.num_seqs
    lo, hi = int(seg[r * B]), int(seg[(r + 1) * B])
    return q_re[lo:hi].contiguous(), do_re[lo:hi].contiguous(), lo, hi


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("lengths,cps", [([160, 90, 210], [1, 2, 4, 8]), ([400, 3], [2, 8])])
def test_cp_share_matches_oracle_and_unsharded(dtype, lengths, cps):
    import torch
    wl = synth.custom(lengths, num_heads=2, d_qk=64, d_v=64, num_buckets=128, dtype=dtype, seed=31, w_std=0.5)
    d = upload(wl)
    m = hstu()
    full_o = m.jagged_attn_fwd(d["q"], d["k"], d["v"], d["offsets"], d["ts"], d["w"], wl.max_seq_len)
    fdq, fdk, fdv, fdw = m.jagged_attn_bwd(d["dout"], d["q"], d["k"], d["v"], d["offsets"], d["ts"], d["w"],
                                           wl.max_seq_len)
    for cp in cps:
        outs, dqs = [], []
        sdk = torch.zeros_like(fdk, dtype=torch.float64)
        sdv = torch.zeros_like(fdv, dtype=torch.float64)
        sdw = torch.zeros_like(fdw, dtype=torch.float64)
        for r in range(cp):
            ql, dol, lo, hi = rank_inputs(m, d, wl, cp, r)
            o = m.jagged_attn_fwd(ql, d["k"], d["v"], d["offsets"], d["ts"], d["w"], wl.max_seq_len,
                                  cp_size=cp, cp_rank=r)
            dq, dk, dv, dw = m.jagged_attn_bwd(dol, ql, d["k"], d["v"], d["offsets"], d["ts"], d["w"],
                                               wl.max_seq_len, cp_size=cp, cp_rank=r)
            # oracle for this rank
            q_re, _ = oracle.reorder(wl.q.f64, wl.offsets, cp)
            d_re, _ = oracle.reorder(wl.dout.f64, wl.offsets, cp)
            ro = oracle.cp_attn_fwd(q_re[lo:hi], wl.k.f64, wl.v.f64, wl.offsets, wl.ts, wl.w.f64, 128, cp, r)
            rq, rk, rv, rw = oracle.cp_attn_bwd(d_re[lo:hi], q_re[lo:hi], wl.k.f64, wl.v.f64, wl.offsets, wl.ts,
                                                wl.w.f64, 128, cp, r)
            tag = f"cp{cp} r{r}"
            assert_close(to_f64(o), ro, dtype, tag + " out")
            assert_close(to_f64(dq), rq, dtype, tag + " dq")
            if np.abs(rk).max() > 0:
                assert_close(to_f64(dk), rk, dtype, tag + " dk")
                assert_close(to_f64(dv), rv, dtype, tag + " dv")
            assert_close(to_f64(dw), rw, dtype, tag + " dw")
            outs.append(o)
            dqs.append(dq)
            sdk += dk.double()
            sdv += dv.double()
            sdw += dw.double()
        o_all, _ = m.cp_reorder(torch.cat(outs), d["offsets"], wl.max_seq_len, cp, inverse=True)
        dq_all, _ = m.cp_reorder(torch.cat(dqs), d["offsets"], wl.max_seq_len, cp, inverse=True)
        ref_o = oracle.attn_fwd(wl.q.f64, wl.k.f64, wl.v.f64, wl.offsets, wl.ts, wl.w.f64, 128)
        assert_close(to_f64(o_all), ref_o, dtype, f"cp{cp} gathered out")
        if cp == 1:
            assert torch.equal(o_all, full_o)
        assert_close(to_f64(dq_all), to_f64(fdq), dtype, f"cp{cp} gathered dq vs unsharded")
        assert_close(sdk.cpu().numpy(), to_f64(fdk), dtype, f"cp{cp} summed dk vs unsharded")
        assert_close(sdv.cpu().numpy(), to_f64(fdv), dtype, f"cp{cp} summed dv vs unsharded")
        assert_close(sdw.cpu().numpy(), to_f64(fdw), dtype, f"cp{cp} summed dw vs unsharded")


# With bf16 and d >= 64 a share whose chunk boundaries all fall on 128-row
# boundaries uses the stored score gradient for dQ; any other share
# recomputes it.  The scheduler takes that decision on the device and leaves
# it in the workspace's counters (the first 64 int32 of the workspace; the
# decision is counter 6), which the test reads back.
@pytest.mark.parametrize("lengths,cp,aligned", [([512, 1024, 1536], 2, True), ([1024, 2048], 4, True),
                                                ([1024, 2048, 640], 4, False), ([512, 1000], 2, False)])
def test_cp_share_stored_gradient(lengths, cp, aligned):
    import torch
    wl = synth.custom(lengths, num_heads=2, d_qk=64, d_v=64, num_buckets=128, dtype="bf16", seed=33, w_std=0.5)
    d = upload(wl)
    m = hstu()
    for r in range(cp):
        ql, dol, lo, hi = rank_inputs(m, d, wl, cp, r)
        args = (dol, ql, d["k"], d["v"], d["offsets"], d["ts"], d["w"], wl.max_seq_len)
        p = m.problem(ql, d["k"], d["v"], d["offsets"], d["w"], wl.max_seq_len, cp_size=cp, cp_rank=r)
        ws = torch.zeros(m.workspace_size(p, True), dtype=torch.uint8, device=ql.device)
        dq, dk, dv, dw = m.jagged_attn_bwd(*args, cp_size=cp, cp_rank=r, workspace=ws)
        torch.cuda.synchronize()
        assert ws[24:28].view(torch.int32).item() == int(aligned), f"cp{cp} r{r} stored-gradient decision"
        lq, lk, lv, lw = m.jagged_attn_bwd(*args, cp_size=cp, cp_rank=r, recompute=True)
        q_re, _ = oracle.reorder(wl.q.f64, wl.offsets, cp)
        d_re, _ = oracle.reorder(wl.dout.f64, wl.offsets, cp)
        rq, rk, rv, rw = oracle.cp_attn_bwd(d_re[lo:hi], q_re[lo:hi], wl.k.f64, wl.v.f64, wl.offsets, wl.ts,
                                            wl.w.f64, 128, cp, r)
        tag = f"cp{cp} r{r}"
        assert_close(to_f64(dq), rq, "bf16", tag + " dq")
        assert_close(to_f64(dk), rk, "bf16", tag + " dk")
        assert_close(to_f64(dv), rv, "bf16", tag + " dv")
        assert_close(to_f64(dw), rw, "bf16", tag + " dw")
        # dK and dV come from the same key pass either way (d(ts_weights) too,
        # but its sums are fp32 atomics whose order varies from run to run)
        assert torch.equal(dk, lk) and torch.equal(dv, lv), tag
        assert_close(to_f64(lq), rq, "bf16", tag + " dq (recomputed)")


@pytest.mark.parametrize("lengths,cp,r", [([1024, 2048], 4, 1), ([512, 1000], 2, 1)])
def test_cp_share_shared_schedule(lengths, cp, r):
    # one schedule per step for a share too: the forward builds both passes'
    # lists (and the stored-gradient decision) in a backward-sized workspace,
    # the backward reuses them; two steps give the bits of separately
    # scheduled calls
    import torch
    wl = synth.custom(lengths, num_heads=2, d_qk=128, d_v=128, num_buckets=128, dtype="bf16", seed=35, w_std=0.5)
    d = upload(wl)
    m = hstu()
    ql, dol, lo, hi = rank_inputs(m, d, wl, cp, r)
    args = (ql, d["k"], d["v"], d["offsets"], d["ts"], d["w"], wl.max_seq_len)
    o_ref = m.jagged_attn_fwd(*args, cp_size=cp, cp_rank=r)
    g_ref = m.jagged_attn_bwd(dol, *args, cp_size=cp, cp_rank=r)
    p = m.problem(ql, d["k"], d["v"], d["offsets"], d["w"], wl.max_seq_len, cp_size=cp, cp_rank=r,
                  shared_schedule=True)
    ws = torch.empty(m.workspace_size(p, True), dtype=torch.uint8, device="cuda")
    for _ in range(2):
        o = m.jagged_attn_fwd(*args, cp_size=cp, cp_rank=r, workspace=ws, shared_schedule=True)
        g = m.jagged_attn_bwd(dol, *args, cp_size=cp, cp_rank=r, workspace=ws, shared_schedule=True)
        assert torch.equal(o, o_ref)
        for name, a, b in zip(("dq", "dk", "dv"), g, g_ref):
            assert torch.equal(a, b), name
        assert_close(to_f64(g[3]), to_f64(g_ref[3]), "bf16", "dw")
    q_re, _ = oracle.reorder(wl.q.f64, wl.offsets, cp)
    d_re, _ = oracle.reorder(wl.dout.f64, wl.offsets, cp)
    rq, rk, rv, rw = oracle.cp_attn_bwd(d_re[lo:hi], q_re[lo:hi], wl.k.f64, wl.v.f64, wl.offsets, wl.ts, wl.w.f64,
                                        128, cp, r)
    assert_close(to_f64(g[0]), rq, "bf16", "dq vs oracle")
    assert_close(to_f64(g[3]), rw, "bf16", "dw vs oracle")


@pytest.mark.parametrize("seed", [1004, 1104])
def test_cp8_rank3_len16384_full(seed):
    # every element of the rank's O and dQ and of its partial dK, dV and
    # d(ts_weights) over all keys and heads, against the oracle's block form of
    # the share
    wl = synth.config("cp8_rank3_len16384", seed=seed)
    d = upload(wl)
    m = hstu()
    cp, r = synth.CP_SIZE, synth.CP_RANK
    ql, dol, lo, hi = rank_inputs(m, d, wl, cp, r)
    assert hi - lo == 4 * 2048
    o = to_f64(m.jagged_attn_fwd(ql, d["k"], d["v"], d["offsets"], d["ts"], d["w"], wl.max_seq_len,
                                 cp_size=cp, cp_rank=r))
    dq, dk, dv, dw = [to_f64(x) for x in m.jagged_attn_bwd(dol, ql, d["k"], d["v"], d["offsets"], d["ts"], d["w"],
                                                           wl.max_seq_len, cp_size=cp, cp_rank=r)]
    idx, _ = oracle.reorder_index(wl.offsets, cp)
    q_loc, d_loc = wl.q.f64[idx[lo:hi]], wl.dout.f64[idx[lo:hi]]
    ro, rq, rk, rv, rw = oracle.cp_attn_blocks(d_loc, q_loc, wl.k.f64, wl.v.f64, wl.offsets, wl.ts, wl.w.f64,
                                               wl.num_buckets, cp, r)
    assert_close(o, ro, "bf16", "out")
    for name, got, ref in [("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv), ("dw", dw, rw)]:
        assert_close(got, ref, "bf16", name)
    # keys past the rank's last chunk (chunk 12 ends at 13*1024) get no gradient
    for b in range(4):
        tail = slice(int(wl.offsets[b]) + 13 * 1024, int(wl.offsets[b + 1]))
        assert np.all(dk[tail] == 0) and np.all(dv[tail] == 0)
