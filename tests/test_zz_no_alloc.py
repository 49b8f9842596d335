"""The forward that allocates nothing (static per-GPU scratch) against the
forward with a caller workspace, through the C ABI."""

import pytest

import oracle
import synth
from hstu_testlib import assert_close, to_f64, upload

pytestmark = pytest.mark.gpu


def hstu():
    import jagged_hstu_attention_amd as m
    return m


def run_both(wl):
    d = upload(wl)
    m = hstu()
    args = (d["q"], d["k"], d["v"], d["offsets"], d["ts"], d["w"], wl.max_seq_len)
    return m.jagged_attn_fwd(*args), m.jagged_attn_fwd_noalloc(*args)


def test_noalloc_forward_matches_workspace_forward_twice():
    # two calls in a row on the shared scratch, the second with a smaller
    # problem: each equals the forward with a caller workspace bit for bit
    # (neither splits key walks here) and the oracle within tolerance
    import torch
    first = synth.custom([300, 1, 129, 0, 500, 64], num_heads=4, d_qk=128, d_v=128, num_buckets=128,
                         dtype="bf16", gap_mean=3600.0, seed=81, w_std=0.5)
    second = synth.custom([77, 3], num_heads=2, d_qk=64, d_v=64, num_buckets=256, dtype="bf16",
                          gap_mean=600.0, seed=82, w_std=0.5)
    for wl in (first, second):
        ref, got = run_both(wl)
        torch.cuda.synchronize()
        assert torch.equal(ref, got)
        want = oracle.attn_fwd(wl.q.f64, wl.k.f64, wl.v.f64, wl.offsets, wl.ts, wl.w.f64, wl.num_buckets)
        assert_close(to_f64(got), want, "bf16", "out")


def test_noalloc_forward_long_tiles_without_split_room():
    # few long query tiles: the workspace forward splits their key walks, the
    # scratch has no room for the partial sums, so the no-allocation forward
    # walks each tile in one item; both match the oracle, then a smaller fp32
    # call follows on the same scratch
    import torch
    wl = synth.custom([4000, 100], num_heads=2, d_qk=128, d_v=128, num_buckets=128, dtype="bf16",
                      gap_mean=600.0, seed=83, w_std=0.5)
    ref, got = run_both(wl)
    want = oracle.attn_fwd(wl.q.f64, wl.k.f64, wl.v.f64, wl.offsets, wl.ts, wl.w.f64, wl.num_buckets)
    assert_close(to_f64(got), want, "bf16", "out")
    assert_close(to_f64(got), to_f64(ref), "bf16", "out vs workspace forward")
    small = synth.custom([33, 64, 1], num_heads=2, d_qk=32, d_v=32, num_buckets=128, dtype="fp32", seed=84)
    ref, got = run_both(small)
    assert torch.equal(ref, got)
    want = oracle.attn_fwd(small.q.f64, small.k.f64, small.v.f64, small.offsets, small.ts, small.w.f64, 128)
    assert_close(to_f64(got), want, "fp32", "out")
