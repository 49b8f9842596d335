"""GPU parity of the candidates forward (target-aware mask for scoring
candidates: Actions Speak Louder than Words, App. H) against the float64
oracle, through the C ABI."""

import numpy as np
import pytest

import oracle
import synth
from hstu_testlib import assert_close, to_f64, upload, upload_array

pytestmark = pytest.mark.gpu

# ragged lengths with candidates: several tiles, a tile boundary inside the
# candidates, no history, no candidates, a single row, empty sequences
LENGTHS = [300, 1, 129, 0, 700, 64, 65, 200, 3]
TARGETS = [100, 1, 0, 0, 257, 64, 1, 200, 2]


def hstu():
    import jagged_hstu_attention_amd as m
    return m


def run(wl, d, targets, only=False, rows=None):
    import torch
    nt = upload_array(np.asarray(targets, np.int64))
    q = d["q"]
    if only:
        q = q[torch.from_numpy(np.asarray(rows, np.int64)).to(q.device)].contiguous()
    return hstu().jagged_attn_fwd_targets(q, d["k"], d["v"], d["offsets"], nt, d["ts"], d["w"], wl.max_seq_len,
                                          q_targets_only=only)


@pytest.mark.parametrize("dtype,dim,nb", [("bf16", 128, 128), ("bf16", 64, 256), ("bf16", 32, 7),
                                          ("fp32", 64, 128), ("fp32", 32, 100)])
def test_candidates_full_and_cached(dtype, dim, nb):
    wl = synth.custom(LENGTHS, num_heads=3, d_qk=dim, d_v=dim, num_buckets=nb, dtype=dtype, gap_mean=3600.0,
                      seed=dim + nb + 7, w_std=0.5, with_dout=False)
    d = upload(wl)
    full = run(wl, d, TARGETS)
    ref = oracle.attn_fwd_targets(wl.q.f64, wl.k.f64, wl.v.f64, wl.offsets, TARGETS, wl.ts, wl.w.f64, nb)
    assert_close(to_f64(full), ref, dtype, "full")
    rows = oracle.target_rows(wl.offsets, TARGETS)
    cached = run(wl, d, TARGETS, only=True, rows=rows)
    ref_c = oracle.attn_fwd_cached(wl.q.f64[rows], wl.k.f64, wl.v.f64, wl.offsets, TARGETS, wl.ts, wl.w.f64, nb)
    assert_close(to_f64(cached), ref_c, dtype, "cached")
    # both passes walk the same key tiles in the same order for a candidate
    np.testing.assert_array_equal(to_f64(cached), to_f64(full)[rows])


def test_no_candidates_is_the_causal_forward():
    wl = synth.custom(LENGTHS, num_heads=2, d_qk=128, d_v=128, dtype="bf16", seed=31, w_std=0.5, with_dout=False)
    d = upload(wl)
    got = run(wl, d, [0] * len(LENGTHS))
    plain = hstu().jagged_attn_fwd(d["q"], d["k"], d["v"], d["offsets"], d["ts"], d["w"], wl.max_seq_len)
    np.testing.assert_array_equal(to_f64(got), to_f64(plain))


def test_all_rows_candidates():
    lengths = [130, 7, 64]
    wl = synth.custom(lengths, num_heads=2, d_qk=64, d_v=64, dtype="fp32", seed=32, w_std=0.5, with_dout=False)
    d = upload(wl)
    got = run(wl, d, lengths)
    ref = oracle.attn_fwd_targets(wl.q.f64, wl.k.f64, wl.v.f64, wl.offsets, lengths, wl.ts, wl.w.f64, 128)
    assert_close(to_f64(got), ref, "fp32", "out")


def test_microbatch_of_1024_candidates_sampled():
    # a 3072-row history per user and a micro-batch of 1024 candidates (App. H
    # evaluates b_m = 1024): sampled candidates against their own causal pass
    # over history plus themselves
    hist, m = 3072, 1024
    lengths = [hist + m, hist + m]
    wl = synth.custom(lengths, num_heads=4, d_qk=128, d_v=128, dtype="bf16", seed=33, w_std=0.5, with_dout=False)
    d = upload(wl)
    targets = [m, m]
    rows = oracle.target_rows(wl.offsets, targets)
    got = to_f64(run(wl, d, targets, only=True, rows=rows))
    rng = np.random.default_rng(5)
    picks = sorted(set([0, m - 1, m, 2 * m - 1, 63, 64, 127, 128] + rng.integers(0, 2 * m, 24).tolist()))
    for n in picks:
        c = int(rows[n])
        b = 0 if c < int(wl.offsets[1]) else 1
        lo = int(wl.offsets[b])
        sub = list(range(lo, lo + hist)) + [c]
        alone = oracle.attn_fwd(wl.q.f64[sub], wl.k.f64[sub], wl.v.f64[sub], [0, len(sub)], wl.ts[sub], wl.w.f64,
                                wl.num_buckets)
        assert_close(got[n], alone[-1], "bf16", f"candidate {n}")


@pytest.mark.parametrize("dtype,dim", [("bf16", 128), ("fp32", 64)])
def test_candidates_long_history_split(dtype, dim):
    # one user with a long history: few query tiles, whose key walks (the
    # history prefix, then the tiles holding the tile's own candidates) are
    # split over several items and summed by a second kernel
    lengths, targets = [3300, 40], [300, 10]
    wl = synth.custom(lengths, num_heads=2, d_qk=dim, d_v=dim, num_buckets=128, dtype=dtype, gap_mean=600.0,
                      seed=dim + 3, w_std=0.5, with_dout=False)
    d = upload(wl)
    full = run(wl, d, targets)
    ref = oracle.attn_fwd_targets(wl.q.f64, wl.k.f64, wl.v.f64, wl.offsets, targets, wl.ts, wl.w.f64, 128)
    assert_close(to_f64(full), ref, dtype, "full")
    rows = oracle.target_rows(wl.offsets, targets)
    cached = run(wl, d, targets, only=True, rows=rows)
    ref_c = oracle.attn_fwd_cached(wl.q.f64[rows], wl.k.f64, wl.v.f64, wl.offsets, targets, wl.ts, wl.w.f64, 128)
    assert_close(to_f64(cached), ref_c, dtype, "cached")
