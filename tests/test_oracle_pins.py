"""Pins of the float64 oracle against facts that do not come from the oracle.

Each test checks the oracle against one of: a closed form, a library routine, a
brute-force loop written independently in the test, an invariant of the
mathematics, or numbers printed on the pages (tests/golden).  CPU only.
"""

import math
import os
from decimal import ROUND_FLOOR, Decimal, getcontext

import numpy as np
import pytest

import oracle
from oracle import hstu_oracle as ho
import synth

getcontext().prec = 90
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# Independent bucket function: via a high-precision logarithm, not via integer
# roots and counting as the oracle does.  floor(NB*log2|x|/32) clamped to
# [0, NB-1]; ties (x^NB == 2^(32k)) decided exactly.
# --------------------------------------------------------------------------

LN2 = Decimal(2).ln()


def bucket_by_log(x: int, nb: int) -> int:
    x = abs(int(x))
    if x <= 1:
        return 0
    y = Decimal(nb) * (Decimal(x).ln() / LN2) / Decimal(32)
    k = int(y.to_integral_value(rounding=ROUND_FLOOR))
    kr = int(y.to_integral_value())
    if abs(y - kr) < Decimal(10) ** -50:
        k = kr if x ** nb >= 2 ** (32 * kr) else kr - 1
    return min(max(k, 0), nb - 1)


NBS = [1, 2, 7, 32, 100, 128, 256, 512]


@pytest.mark.parametrize("nb", NBS)
def test_bucket_powers_of_two_closed_form(nb):
    # |Δ| = 2^m  ->  bucket min(floor(m*NB/32), NB-1)
    m = np.arange(0, 63)
    delta = (np.int64(1) << m.astype(np.int64))
    got = oracle.bucketize(delta, nb)
    want = np.minimum((m * nb) // 32, nb - 1)
    assert np.array_equal(got, want)
    assert np.array_equal(oracle.bucketize(-delta, nb), want)
    assert oracle.bucketize(np.array([0]), nb)[0] == 0


@pytest.mark.parametrize("nb", [128, 256])
def test_bucket_just_below_powers_of_two(nb):
    # 2^m - 1 lies strictly below the edge at exactly 2^m when m*NB/32 is an
    # integer k, so its bucket is k-1 (for m large enough that the previous edge
    # is <= 2^m - 1, i.e. 2^m * (1 - 2^(-32/NB)) >= 1: m >= 4 for both NB here).
    per_octave = nb // 32
    for m in range(5, 32):
        k = m * per_octave
        x = (1 << m) - 1
        assert oracle.bucketize(np.array([x]), nb)[0] == min(k - 1, nb - 1)


@pytest.mark.parametrize("nb", NBS)
def test_bucket_vs_high_precision_log(nb):
    rng = np.random.default_rng(7 + nb)
    xs = list(range(0, 600)) + [int(v) for v in rng.integers(1, 1 << 40, size=400)]
    xs += [int(v) for v in np.exp2(rng.uniform(0, 62, size=200)).astype(np.int64)]
    # values right at and next to every edge
    for e in oracle.bucket_edges(nb)[:: max(1, nb // 64)]:
        xs += [e - 1, e, e + 1]
    got = oracle.bucketize(np.array(xs, dtype=np.int64), nb)
    want = [bucket_by_log(x, nb) for x in xs]
    assert list(got) == want


def test_bucket_monotone_and_range():
    for nb in NBS:
        x = np.unique(np.concatenate([np.arange(0, 5000), np.exp2(np.arange(0, 62, 0.37)).astype(np.int64)]))
        b = oracle.bucketize(x, nb)
        assert np.all(np.diff(b) >= 0)
        assert b.min() >= 0 and b.max() <= nb - 1
        assert oracle.bucketize(np.array([1 << 62]), nb)[0] == nb - 1


def test_bucket_edges_are_ceil_of_real_edges():
    # E_k = ceil(2^(32k/NB)): check (E_k - 1)^NB < 2^(32k) <= E_k^NB exactly.
    for nb in [7, 128, 256]:
        for k, e in enumerate(oracle.bucket_edges(nb), start=1):
            assert e ** nb >= 2 ** (32 * k)
            assert (e - 1) ** nb < 2 ** (32 * k)


# --------------------------------------------------------------------------
# Forward
# --------------------------------------------------------------------------

def brute_force_fwd(q, k, v, offsets, ts, w, nb):
    """Per-pair pure-Python loop: out_i = sum_{j<=i} silu(alpha*(q_i.k_j + w[bucket])) v_j."""
    T, H, d = q.shape
    dv = v.shape[2]
    alpha = 1.0 / math.sqrt(d)
    out = np.zeros((T, H, dv))
    for b in range(len(offsets) - 1):
        lo, hi = int(offsets[b]), int(offsets[b + 1])
        for h in range(H):
            for i in range(lo, hi):
                for j in range(lo, i + 1):
                    dot = 0.0
                    for e in range(d):
                        dot += float(q[i, h, e]) * float(k[j, h, e])
                    s = alpha * (dot + float(w[h, bucket_by_log(int(ts[i]) - int(ts[j]), nb)]))
                    a = s / (1.0 + math.exp(-s))
                    for e in range(dv):
                        out[i, h, e] += a * float(v[j, h, e])
    return out


def small(lengths, *, nb=128, H=2, d=4, dv=None, gap=3600.0, seed=0, w_std=0.02):
    return synth.custom(lengths, num_heads=H, d_qk=d, d_v=dv or d, num_buckets=nb,
                        dtype="fp32", gap_mean=gap, seed=seed, w_std=w_std)


def fwd(wl, q=None, k=None, v=None, w=None, ts=None, offsets=None):
    return oracle.attn_fwd(wl.q.f64 if q is None else q, wl.k.f64 if k is None else k,
                           wl.v.f64 if v is None else v,
                           wl.offsets if offsets is None else offsets,
                           wl.ts if ts is None else ts,
                           wl.w.f64 if w is None else w, wl.num_buckets)


@pytest.mark.parametrize("nb,gap,w_std", [(128, 3600.0, 0.5), (7, 3.0, 1.0), (256, 600.0, 0.3)])
def test_fwd_matches_brute_force(nb, gap, w_std):
    wl = small([5, 1, 7, 0, 3], nb=nb, H=2, d=4, dv=3, gap=gap, w_std=w_std, seed=nb)
    got = fwd(wl)
    want = brute_force_fwd(wl.q.f64, wl.k.f64, wl.v.f64, wl.offsets, wl.ts, wl.w.f64, nb)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_fwd_zero_bias_equals_dense_silu_attention():
    import torch
    wl = small([37, 64, 5], H=3, d=16, seed=3)
    got = fwd(wl, w=np.zeros_like(wl.w.f64))
    alpha = 1.0 / math.sqrt(16)
    for b in range(3):
        lo, hi = wl.offsets[b], wl.offsets[b + 1]
        for h in range(3):
            q = torch.from_numpy(wl.q.f64[lo:hi, h])
            k = torch.from_numpy(wl.k.f64[lo:hi, h])
            v = torch.from_numpy(wl.v.f64[lo:hi, h])
            a = torch.tril(torch.nn.functional.silu(alpha * (q @ k.T)))
            np.testing.assert_allclose(got[lo:hi, h], (a @ v).numpy(), rtol=0, atol=1e-12)


def test_fwd_q_zero_constant_bias_is_cumsum():
    wl = small([20, 33], H=2, d=8, seed=4)
    c = 1.7
    w = np.full_like(wl.w.f64, c)
    got = fwd(wl, q=np.zeros_like(wl.q.f64), w=w)
    alpha = 1.0 / math.sqrt(8)
    sc = alpha * c / (1.0 + math.exp(-alpha * c))
    for b in range(2):
        lo, hi = wl.offsets[b], wl.offsets[b + 1]
        np.testing.assert_allclose(got[lo:hi], sc * np.cumsum(wl.v.f64[lo:hi], axis=0), rtol=1e-13, atol=1e-12)


@pytest.mark.parametrize("nb", [128, 256])
def test_fwd_q_zero_one_hot_bias_selects_bucket(nb):
    wl = small([40, 25], nb=nb, H=2, d=8, gap=50_000.0, seed=5)
    alpha = 1.0 / math.sqrt(8)
    c = 2.5
    for target in [0, nb // 2, int(nb * 0.6)]:
        w = np.zeros_like(wl.w.f64)
        w[:, target] = c
        got = fwd(wl, q=np.zeros_like(wl.q.f64), w=w)
        sc = alpha * c / (1.0 + math.exp(-alpha * c))
        want = np.zeros_like(got)
        for b in range(2):
            lo, hi = int(wl.offsets[b]), int(wl.offsets[b + 1])
            for i in range(lo, hi):
                for j in range(lo, i + 1):
                    if bucket_by_log(int(wl.ts[i]) - int(wl.ts[j]), nb) == target:
                        want[i] += sc * wl.v.f64[j]
        np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-12)


def test_fwd_single_token_closed_form():
    wl = small([1, 1, 1], H=2, d=8, seed=6, w_std=0.7)
    got = fwd(wl)
    alpha = 1.0 / math.sqrt(8)
    for i in range(3):
        for h in range(2):
            s = alpha * (wl.q.f64[i, h] @ wl.k.f64[i, h] + wl.w.f64[h, 0])
            np.testing.assert_allclose(got[i, h], s / (1 + math.exp(-s)) * wl.v.f64[i, h], rtol=1e-14, atol=1e-14)


def test_fwd_causality_by_perturbation():
    wl = small([30], H=2, d=8, seed=8)
    base = fwd(wl)
    for cut in [0, 7, 29]:
        k2 = wl.k.f64.copy()
        v2 = wl.v.f64.copy()
        k2[cut + 1:] += 3.0
        v2[cut + 1:] -= 5.0
        pert = fwd(wl, k=k2, v=v2)
        assert np.array_equal(pert[:cut + 1], base[:cut + 1])
        if cut + 1 < 30:
            assert not np.allclose(pert[cut + 1:], base[cut + 1:])


def test_fwd_jagged_equals_independent_sequences():
    wl = small([9, 0, 14, 3], H=2, d=8, seed=9)
    got = fwd(wl)
    for b in range(4):
        lo, hi = int(wl.offsets[b]), int(wl.offsets[b + 1])
        one = oracle.attn_fwd(wl.q.f64[lo:hi], wl.k.f64[lo:hi], wl.v.f64[lo:hi],
                              np.array([0, hi - lo]), wl.ts[lo:hi], wl.w.f64, wl.num_buckets)
        assert np.array_equal(got[lo:hi], one)


def test_fwd_linear_in_v():
    wl = small([12, 17], H=2, d=8, seed=10)
    v2 = np.random.default_rng(0).standard_normal(wl.v.f64.shape)
    lhs = fwd(wl, v=2.0 * wl.v.f64 - 3.0 * v2)
    rhs = 2.0 * fwd(wl) - 3.0 * fwd(wl, v=v2)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def test_fwd_timestamp_shift_invariance():
    # Only differences of timestamps enter: shifting a sequence's timestamps
    # by a constant leaves its output unchanged.
    wl = small([15, 11], H=2, d=8, seed=11, w_std=0.5)
    ts2 = wl.ts.copy()
    ts2[:15] += 123_456_789
    assert np.array_equal(fwd(wl), fwd(wl, ts=ts2))


# --------------------------------------------------------------------------
# Backward
# --------------------------------------------------------------------------

def loss(wl, dout, **kw):
    return float(np.sum(dout * fwd(wl, **kw)))


@pytest.mark.parametrize("nb,seed", [(128, 12), (7, 13)])
def test_bwd_central_finite_differences(nb, seed):
    wl = small([4, 6, 1], nb=nb, H=2, d=3, dv=2, gap=5.0 if nb == 7 else 3600.0, seed=seed, w_std=0.4)
    dout = np.random.default_rng(seed).standard_normal((wl.total, 2, 2))
    dq, dk, dv, dw = oracle.attn_bwd(dout, wl.q.f64, wl.k.f64, wl.v.f64, wl.offsets, wl.ts, wl.w.f64, nb)
    h = 1e-6
    for name, base, grad in [("q", wl.q.f64, dq), ("k", wl.k.f64, dk), ("v", wl.v.f64, dv), ("w", wl.w.f64, dw)]:
        num = np.zeros_like(base)
        it = np.nditer(base, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            p = base.copy()
            m = base.copy()
            p[idx] += h
            m[idx] -= h
            num[idx] = (loss(wl, dout, **{name: p}) - loss(wl, dout, **{name: m})) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-7, err_msg=name)


def test_bwd_adjoint_identities():
    wl = small([23, 9, 31], H=3, d=8, seed=14, w_std=0.3)
    dout = np.random.default_rng(1).standard_normal(wl.v.f64.shape)
    o = fwd(wl)
    dq, dk, dv, dw = oracle.attn_bwd(dout, wl.q.f64, wl.k.f64, wl.v.f64, wl.offsets, wl.ts, wl.w.f64, wl.num_buckets)
    # O is linear in V:  <dV, V> = <dO, O>
    np.testing.assert_allclose(np.sum(dv * wl.v.f64), np.sum(dout * o), rtol=1e-12)
    # both equal sum_ij G_ij q_i.k_j
    np.testing.assert_allclose(np.sum(dq * wl.q.f64), np.sum(dk * wl.k.f64), rtol=1e-11)


def test_bwd_q_zero_one_hot_dw_closed_form():
    wl = small([18, 26], H=2, d=8, gap=50_000.0, seed=15)
    nb = wl.num_buckets
    alpha = 1.0 / math.sqrt(8)
    c, target = 1.3, 80
    w = np.zeros_like(wl.w.f64)
    w[:, target] = c
    dout = np.random.default_rng(2).standard_normal(wl.v.f64.shape)
    _, _, _, dw = oracle.attn_bwd(dout, np.zeros_like(wl.q.f64), wl.k.f64, wl.v.f64, wl.offsets, wl.ts, w, nb)
    # s = alpha*c on target-bucket pairs, 0 elsewhere; SiLU'(0) = 1/2.
    sg = 1.0 / (1.0 + math.exp(-alpha * c))
    dsilu_c = sg * (1.0 + alpha * c * (1.0 - sg))
    want = np.zeros((2, nb))
    for b in range(2):
        lo, hi = int(wl.offsets[b]), int(wl.offsets[b + 1])
        for i in range(lo, hi):
            for j in range(lo, i + 1):
                bk = bucket_by_log(int(wl.ts[i]) - int(wl.ts[j]), nb)
                dp = np.sum(dout[i] * wl.v.f64[j], axis=-1)  # per head
                want[:, bk] += alpha * dp * (dsilu_c if bk == target else 0.5)
    np.testing.assert_allclose(dw, want, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# Context-parallel share and reorder
# --------------------------------------------------------------------------

def load_table1():
    rows = []
    with open(os.path.join(GOLDEN, "cp_max_seq_len_table.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                c, n = line.split()
                rows.append((int(c), int(n)))
    return rows


def test_table1_lengths_split_into_balanced_chunk_pairs():
    # The pages print these (CP size, max length) pairs; each length splits into
    # 2C equal mini-chunks and every rank's pair (r, 2C-1-r) carries exactly 1/C
    # of the causal pairs: n(L+1) with n = L/2C.
    for c, length in load_table1():
        assert length % (2 * c) == 0
        n = length // (2 * c)
        total = oracle.causal_pairs([length])
        assert total == length * (length + 1) // 2
        for r in range(c):
            assert oracle.cp_rank_pairs([length], c, r) == n * (length + 1)
        assert sum(oracle.cp_rank_pairs([length], c, r) for r in range(c)) == total


def test_cp8_rank3_pairs_closed_form():
    # chunks 3 and 12 of a 16384-long sequence (n = 1024)
    n = 1024
    p3 = sum(p + 1 for p in range(3 * n, 4 * n))
    p12 = sum(p + 1 for p in range(12 * n, 13 * n))
    assert (p3, p12) == (3_670_528, 13_107_712)
    assert oracle.cp_rank_pairs([16384], 8, 3) == p3 + p12 == 16_778_240


@pytest.mark.parametrize("lengths", [[16, 16], [13, 1, 0, 22, 5], [7, 31]])
def test_reorder_permutation_properties(lengths):
    off = synth.offsets_from_lengths(lengths)
    T = int(off[-1])
    x = np.arange(T) * 10 + 3
    for c in [1, 2, 4, 8]:
        y, out_off = oracle.reorder(x, off, c)
        assert sorted(y.tolist()) == sorted(x.tolist())
        back, _ = oracle.reorder(y, off, c, inverse=True)
        assert np.array_equal(back, x)
        assert len(out_off) == c * len(lengths) + 1 and out_off[-1] == T
        if c == 1:
            assert np.array_equal(y, x)
        # segment (r, b) holds exactly the two mini-chunks' row counts
        for r in range(c):
            for b, n in enumerate(lengths):
                seg = int(out_off[r * len(lengths) + b + 1] - out_off[r * len(lengths) + b])
                want = sum((k + 1) * n // (2 * c) - k * n // (2 * c) for k in (r, 2 * c - 1 - r))
                assert seg == want


def test_reorder_uniform_closed_form():
    # Equal lengths L = 2Cn: output row (r, b, half, j) is input row b*L + chunk*n + j.
    B, C, n = 3, 4, 5
    L = 2 * C * n
    off = synth.offsets_from_lengths([L] * B)
    idx, _ = oracle.reorder_index(off, C)
    want = []
    for r in range(C):
        for b in range(B):
            for chunk in (r, 2 * C - 1 - r):
                want.extend(b * L + chunk * n + j for j in range(n))
    assert idx.tolist() == want


@pytest.mark.parametrize("lengths,cps", [([16, 9, 21], [1, 2, 4, 8]), ([40, 3], [2, 8])])
def test_cp_share_equals_unsharded(lengths, cps):
    wl = small(lengths, H=2, d=4, seed=21, w_std=0.5)
    dout = np.random.default_rng(3).standard_normal(wl.v.f64.shape)
    full_o = fwd(wl)
    fdq, fdk, fdv, fdw = oracle.attn_bwd(dout, wl.q.f64, wl.k.f64, wl.v.f64, wl.offsets, wl.ts, wl.w.f64, wl.num_buckets)
    for c in cps:
        outs, dqs = [], []
        sdk = np.zeros_like(fdk)
        sdv = np.zeros_like(fdv)
        sdw = np.zeros_like(fdw)
        q_re, out_off = oracle.reorder(wl.q.f64, wl.offsets, c)
        d_re, _ = oracle.reorder(dout, wl.offsets, c)
        B = len(lengths)
        for r in range(c):
            lo, hi = int(out_off[r * B]), int(out_off[(r + 1) * B])
            o = oracle.cp_attn_fwd(q_re[lo:hi], wl.k.f64, wl.v.f64, wl.offsets, wl.ts, wl.w.f64, wl.num_buckets, c, r)
            dq, dk, dv, dw = oracle.cp_attn_bwd(d_re[lo:hi], q_re[lo:hi], wl.k.f64, wl.v.f64, wl.offsets, wl.ts,
                                                wl.w.f64, wl.num_buckets, c, r)
            outs.append(o)
            dqs.append(dq)
            sdk += dk
            sdv += dv
            sdw += dw
        o_all, _ = oracle.reorder(np.concatenate(outs), wl.offsets, c, inverse=True)
        dq_all, _ = oracle.reorder(np.concatenate(dqs), wl.offsets, c, inverse=True)
        np.testing.assert_allclose(o_all, full_o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(dq_all, fdq, rtol=0, atol=1e-12)
        np.testing.assert_allclose(sdk, fdk, rtol=0, atol=1e-12)
        np.testing.assert_allclose(sdv, fdv, rtol=0, atol=1e-12)
        np.testing.assert_allclose(sdw, fdw, rtol=0, atol=1e-12)


def test_cp_local_offsets():
    off = synth.offsets_from_lengths([16, 9, 21])
    lo = oracle.cp_local_offsets(off, 2, 1)
    # rank 1 of C=2 holds chunks 1 and 2 of 4
    want = [0]
    for n in [16, 9, 21]:
        want.append(want[-1] + sum((k + 1) * n // 4 - k * n // 4 for k in (1, 2)))
    assert lo.tolist() == want


# --------------------------------------------------------------------------
# The pins catch plausible mistakes: plant one in the oracle and check that at
# least one pin fails.
# --------------------------------------------------------------------------

def _pins_fail(monkeypatch, attr, bad):
    monkeypatch.setattr(ho, attr, bad)
    failures = 0
    for fn in [lambda: test_fwd_matches_brute_force(128, 3600.0, 0.5),
               lambda: test_fwd_zero_bias_equals_dense_silu_attention(),
               lambda: test_fwd_q_zero_one_hot_bias_selects_bucket(128),
               lambda: test_fwd_causality_by_perturbation(),
               lambda: test_bwd_central_finite_differences(128, 12)]:
        try:
            fn()
        except AssertionError:
            failures += 1
    return failures


def test_planted_mistakes_are_caught(monkeypatch):
    orig_scores = ho._seq_scores
    orig_silu = ho.silu

    def no_scale_on_bias(qb, kb, tsq, tsk, wh, nb, alpha):
        s, b = orig_scores(qb, kb, tsq, tsk, wh, nb, alpha)
        return s - alpha * wh[b] + wh[b], b

    def off_by_one_bucket(qb, kb, tsq, tsk, wh, nb, alpha):
        raw = qb @ kb.T
        b = np.minimum(ho.bucketize(tsq[:, None] - tsk[None, :], nb) + 1, nb - 1)
        return alpha * (raw + wh[b]), b

    def transposed(qb, kb, tsq, tsk, wh, nb, alpha):
        s, b = orig_scores(qb, kb, tsq, tsk, wh, nb, alpha)
        return s.T, b.T

    for attr, bad in [("_seq_scores", no_scale_on_bias), ("_seq_scores", off_by_one_bucket),
                      ("_seq_scores", transposed), ("silu", lambda x: x / (1.0 + np.exp(x)))]:
        assert _pins_fail(monkeypatch, attr, bad) > 0, attr
        monkeypatch.setattr(ho, "_seq_scores", orig_scores)
        monkeypatch.setattr(ho, "silu", orig_silu)


# --------------------------------------------------------------------------
# Target-aware attention for candidates ([HSTU] App. H, M-FALCON)
# --------------------------------------------------------------------------

T_LENGTHS = [9, 1, 6, 0, 12, 5]
T_TARGETS = [3, 1, 0, 0, 12, 2]


def brute_force_fwd_targets(q, k, v, offsets, num_targets, ts, w, nb):
    """Per-pair loop; key j is visible to query i iff j <= i and j is a history
    row or i itself."""
    T, H, d = q.shape
    alpha = 1.0 / math.sqrt(d)
    out = np.zeros((T, H, v.shape[2]))
    for b in range(len(offsets) - 1):
        lo, hi = int(offsets[b]), int(offsets[b + 1])
        hist = hi - int(num_targets[b])
        for h in range(H):
            for i in range(lo, hi):
                for j in range(lo, i + 1):
                    if j >= hist and j != i:
                        continue
                    dot = sum(float(q[i, h, e]) * float(k[j, h, e]) for e in range(d))
                    s = alpha * (dot + float(w[h, bucket_by_log(int(ts[i]) - int(ts[j]), nb)]))
                    out[i, h] += (s / (1.0 + math.exp(-s))) * v[j, h]
    return out


def targets_wl(seed=5, nb=128, w_std=0.5):
    return small(T_LENGTHS, nb=nb, H=2, d=4, dv=3, w_std=w_std, seed=seed)


def test_targets_match_brute_force():
    wl = targets_wl()
    got = oracle.attn_fwd_targets(wl.q.f64, wl.k.f64, wl.v.f64, wl.offsets, T_TARGETS, wl.ts, wl.w.f64, 128)
    want = brute_force_fwd_targets(wl.q.f64, wl.k.f64, wl.v.f64, wl.offsets, T_TARGETS, wl.ts, wl.w.f64, 128)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_each_candidate_equals_its_own_pass():
    # App. H: one pass over history plus all candidates gives each candidate
    # what its own causal pass over history plus that candidate gives.
    wl = targets_wl(seed=6)
    got = oracle.attn_fwd_targets(wl.q.f64, wl.k.f64, wl.v.f64, wl.offsets, T_TARGETS, wl.ts, wl.w.f64, 128)
    for b in range(len(T_LENGTHS)):
        lo, hi = int(wl.offsets[b]), int(wl.offsets[b + 1])
        hist = hi - T_TARGETS[b]
        for c in range(hist, hi):
            rows = list(range(lo, hist)) + [c]
            alone = oracle.attn_fwd(wl.q.f64[rows], wl.k.f64[rows], wl.v.f64[rows], [0, len(rows)],
                                    wl.ts[rows], wl.w.f64, 128)
            np.testing.assert_allclose(got[c], alone[-1], rtol=0, atol=1e-12)


def test_targets_zero_is_causal_and_history_rows_are_causal():
    wl = targets_wl(seed=7)
    plain = fwd(wl)
    none = oracle.attn_fwd_targets(wl.q.f64, wl.k.f64, wl.v.f64, wl.offsets, [0] * len(T_LENGTHS), wl.ts,
                                   wl.w.f64, 128)
    np.testing.assert_allclose(none, plain, rtol=0, atol=1e-12)
    got = oracle.attn_fwd_targets(wl.q.f64, wl.k.f64, wl.v.f64, wl.offsets, T_TARGETS, wl.ts, wl.w.f64, 128)
    cand = set(oracle.target_rows(wl.offsets, T_TARGETS).tolist())
    hist_rows = [i for i in range(int(wl.offsets[-1])) if i not in cand]
    np.testing.assert_allclose(got[hist_rows], plain[hist_rows], rtol=0, atol=1e-12)


def test_all_candidates_closed_form():
    # no history: each row sees only itself, O_i = silu(alpha (q_i.k_i + w[h, bucket 0])) v_i
    wl = small([4, 7], nb=128, H=2, d=4, dv=3, w_std=0.5, seed=8)
    got = oracle.attn_fwd_targets(wl.q.f64, wl.k.f64, wl.v.f64, wl.offsets, [4, 7], wl.ts, wl.w.f64, 128)
    alpha = 0.5
    s = alpha * (np.einsum("thd,thd->th", wl.q.f64, wl.k.f64) + wl.w.f64[:, 0][None, :])
    np.testing.assert_allclose(got, (s / (1.0 + np.exp(-s)))[:, :, None] * wl.v.f64, rtol=0, atol=1e-12)


def test_cached_candidates_equal_full_pass():
    wl = targets_wl(seed=9)
    full = oracle.attn_fwd_targets(wl.q.f64, wl.k.f64, wl.v.f64, wl.offsets, T_TARGETS, wl.ts, wl.w.f64, 128)
    rows = oracle.target_rows(wl.offsets, T_TARGETS)
    cached = oracle.attn_fwd_cached(wl.q.f64[rows], wl.k.f64, wl.v.f64, wl.offsets, T_TARGETS, wl.ts, wl.w.f64, 128)
    np.testing.assert_allclose(cached, full[rows], rtol=0, atol=1e-12)


def test_planted_target_mask_mistakes_are_caught(monkeypatch):
    orig = ho.target_mask

    def candidates_see_each_other(n, m):
        return np.tril(np.ones((n, n), dtype=bool))

    def no_self(n, m):
        out = orig(n, m)
        idx = np.arange(n - m, n)
        out[idx, idx] = False
        return out

    def history_off_by_one(n, m):
        return orig(n, min(m + 1, n))

    pins = [test_targets_match_brute_force, test_each_candidate_equals_its_own_pass,
            test_all_candidates_closed_form]
    for bad in (candidates_see_each_other, no_self, history_off_by_one):
        monkeypatch.setattr(ho, "target_mask", bad)
        failures = 0
        for fn in pins:
            try:
                fn()
            except AssertionError:
                failures += 1
        monkeypatch.setattr(ho, "target_mask", orig)
        assert failures > 0, bad.__name__


# --------------------------------------------------------------------------
# Per-row forms.  attn_fwd_rows, attn_bwd_q_rows and attn_bwd_kv_rows are the
# checkers for sampled rows of problems too large for the whole-batch oracle,
# so each is pinned to the whole-batch form (itself pinned above) at every row
# of a ragged batch: empty and single-token sequences, first and last rows.
# --------------------------------------------------------------------------

ROW_LENGTHS = [5, 0, 1, 9, 0, 0, 7, 1, 3, 2]


def row_forms_agree(wl, atol=1e-12):
    """True when every row of the per-row forms equals the batch forms."""
    rows = list(range(wl.total))
    args = (wl.q.f64, wl.k.f64, wl.v.f64, wl.offsets, wl.ts, wl.w.f64, wl.num_buckets)
    o = oracle.attn_fwd(*args)
    dq, dk, dv, _ = oracle.attn_bwd(wl.dout.f64, *args)
    ro = oracle.attn_fwd_rows(*args, rows)
    rq = oracle.attn_bwd_q_rows(wl.dout.f64, *args, rows)
    rk, rv = oracle.attn_bwd_kv_rows(wl.dout.f64, *args, rows)
    return all(np.allclose(a, b, rtol=1e-12, atol=atol) for a, b in [(ro, o), (rq, dq), (rk, dk), (rv, dv)])


@pytest.mark.parametrize("nb,gap,seed", [(128, 3600.0, 21), (7, 3.0, 22), (256, 600.0, 23)])
def test_row_forms_equal_batch_forms_at_every_row(nb, gap, seed):
    wl = small(ROW_LENGTHS, nb=nb, H=2, d=4, gap=gap, seed=seed, w_std=0.5)
    assert wl.dout is not None
    rows = list(range(wl.total))
    args = (wl.q.f64, wl.k.f64, wl.v.f64, wl.offsets, wl.ts, wl.w.f64, wl.num_buckets)
    o = oracle.attn_fwd(*args)
    dq, dk, dv, _ = oracle.attn_bwd(wl.dout.f64, *args)
    np.testing.assert_allclose(oracle.attn_fwd_rows(*args, rows), o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.attn_bwd_q_rows(wl.dout.f64, *args, rows), dq, rtol=1e-12, atol=1e-12)
    rk, rv = oracle.attn_bwd_kv_rows(wl.dout.f64, *args, rows)
    np.testing.assert_allclose(rk, dk, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(rv, dv, rtol=1e-12, atol=1e-12)
    # a subset in any order gives the same rows
    sub = [wl.total - 1, 0, 6, 7, 15]
    np.testing.assert_allclose(oracle.attn_fwd_rows(*args, sub), o[sub], rtol=1e-12, atol=1e-12)


def test_row_form_pins_catch_planted_mistakes(monkeypatch):
    wl = small(ROW_LENGTHS, nb=128, H=2, d=4, gap=3600.0, seed=21, w_std=0.5)
    assert row_forms_agree(wl)
    orig_row_seq = ho._row_seq
    orig_kv_rows = ho.attn_bwd_kv_rows

    # a row at a sequence's first position assigned to the sequence before it
    def row_seq_left(offsets, row):
        b = int(np.searchsorted(np.asarray(offsets), row, side="left")) - 1
        b = max(b, 0)
        return b, int(offsets[b]), int(offsets[b + 1])

    monkeypatch.setattr(ho, "_row_seq", row_seq_left)
    assert not row_forms_agree(wl)
    monkeypatch.setattr(ho, "_row_seq", orig_row_seq)

    # the diagonal pair dropped from a key's query range
    def kv_rows_no_diagonal(dout, q, k, v, offsets, ts, w, num_buckets, rows):
        dk, dv = orig_kv_rows(dout, q, k, v, offsets, ts, w, num_buckets, rows)
        alpha = 1.0 / math.sqrt(q.shape[2])
        for n, j in enumerate(rows):
            for h in range(q.shape[1]):
                s = alpha * (q[j, h] @ k[j, h] + w[h, 0])
                sg = 1.0 / (1.0 + math.exp(-s))
                dp = dout[j, h] @ v[j, h]
                dv[n, h] -= s * sg * dout[j, h]
                dk[n, h] -= alpha * dp * sg * (1.0 + s * (1.0 - sg)) * q[j, h]
        return dk, dv

    monkeypatch.setattr(ho, "attn_bwd_kv_rows", kv_rows_no_diagonal)
    monkeypatch.setattr(oracle, "attn_bwd_kv_rows", kv_rows_no_diagonal)
    assert not row_forms_agree(wl)

    # the causal prefix of a query row stopping one key short
    monkeypatch.setattr(ho, "attn_bwd_kv_rows", orig_kv_rows)
    monkeypatch.setattr(oracle, "attn_bwd_kv_rows", orig_kv_rows)
    orig_scores = ho._seq_scores

    def short_prefix_scores(qb, kb, tsq, tsk, wh, nb, alpha):
        s, b = orig_scores(qb, kb, tsq, tsk, wh, nb, alpha)
        if s.shape[0] == 1 and s.shape[1] > 1:  # a query row against its prefix
            s = s.copy()
            s[0, -1] = -700.0                   # silu(-700) ~ 0: the diagonal drops out
        return s, b

    monkeypatch.setattr(ho, "_seq_scores", short_prefix_scores)
    assert not row_forms_agree(wl)


# --------------------------------------------------------------------------
# Block form of a CP rank's share (the checker of the full-size share): equal
# to the per-row CP forms and to the rows of the unsharded oracle.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("lengths,cp", [([37, 16, 0, 1], 2), ([37, 16, 0, 1], 4), ([64, 23], 8), ([5, 50], 1)])
def test_cp_block_form_equals_row_form_and_unsharded(lengths, cp):
    wl = small(lengths, nb=128, H=2, d=4, gap=3600.0, seed=31 + cp, w_std=0.5)
    args = (wl.k.f64, wl.v.f64, wl.offsets, wl.ts, wl.w.f64, 128)
    q_re, _ = oracle.reorder(wl.q.f64, wl.offsets, cp)
    d_re, _ = oracle.reorder(wl.dout.f64, wl.offsets, cp)
    full_o = oracle.attn_fwd(wl.q.f64, *args)
    full_g = oracle.attn_bwd(wl.dout.f64, wl.q.f64, *args)
    idx, seg = oracle.reorder_index(wl.offsets, cp)
    B = len(lengths)
    sums = [np.zeros_like(full_g[1]), np.zeros_like(full_g[2]), np.zeros_like(full_g[3])]
    for r in range(cp):
        lo, hi = int(seg[r * B]), int(seg[(r + 1) * B])
        o, dq, dk, dv, dw = oracle.cp_attn_blocks(d_re[lo:hi], q_re[lo:hi], *args, cp, r)
        np.testing.assert_allclose(o, oracle.cp_attn_fwd(q_re[lo:hi], *args, cp, r), rtol=1e-12, atol=1e-12)
        rq, rk, rv, rw = oracle.cp_attn_bwd(d_re[lo:hi], q_re[lo:hi], *args, cp, r)
        for got, want in [(dq, rq), (dk, rk), (dv, rv), (dw, rw)]:
            np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
        # rows of the unsharded problem
        np.testing.assert_allclose(o, full_o[idx[lo:hi]], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dq, full_g[0][idx[lo:hi]], rtol=1e-12, atol=1e-12)
        for acc, part in zip(sums, (dk, dv, dw)):
            acc += part
    for acc, want in zip(sums, full_g[1:]):
        np.testing.assert_allclose(acc, want, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# Stochastic Length ([HSTU] §3.2, §4.2, App. E)
# --------------------------------------------------------------------------

def iroot(x: int, k: int) -> int:
    """floor(x^(1/k)) for integers, by bisection on exact integer powers."""
    lo, hi = 0, 1
    while hi ** k <= x:
        hi *= 2
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if mid ** k <= x:
            lo = mid
        else:
            hi = mid
    return lo


def test_sl_printed_length_after_sampling():
    # the pages' one printed case: alpha = 1.6, length 4096 -> 776
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "sl_length_at_alpha_1_6.txt"))
            if ln.strip() and not ln.startswith("#")]
    assert rows
    for alpha, n, want in rows:
        assert oracle.sl_target_length(int(n), float(alpha)) == int(want)


@pytest.mark.parametrize("alpha,k,p", [(1.0, 2, 1), (1.5, 4, 3), (1.75, 8, 7), (0.5, 4, 1), (1.25, 8, 5)])
def test_sl_target_length_equals_integer_roots(alpha, k, p):
    # alpha/2 = p/k exactly (dyadic alphas), so floor(n^(alpha/2)) is the
    # integer k-th root of n^p: a different route from the decimal power
    for n in list(range(1, 3000)) + [4095, 4096, 4097, 8191, 8192, 16384, 65535, 65536, 1 << 20]:
        assert oracle.sl_target_length(n, alpha) == min(iroot(n ** p, k), n), n


def test_sl_float_alpha_at_perfect_powers():
    # alpha = 1.2 as a float is slightly below 6/5: the length at perfect
    # fifth powers is still the integer k^3 (the 2^-40 tolerance), and away
    # from integers the floor is unchanged
    for k in range(2, 9):
        assert oracle.sl_target_length(k ** 5, 1.2) == k ** 3
    assert oracle.sl_target_length(4096, 1.2) == 147  # 2^7.2 = 147.03
    for n in range(2, 5000):
        exact = n ** 0.6
        if abs(exact - round(exact)) > 1e-6:
            assert oracle.sl_target_length(n, 1.2) == math.floor(exact), n


def test_sl_keep_whole_rule():
    from fractions import Fraction
    # alpha = 1: kept whole iff u < n^-1 = 1/n (exact rational compare)
    rng = np.random.default_rng(3)
    for n in [2, 3, 7, 100, 4096]:
        for u in list(rng.random(50)) + [1.0 / n, np.nextafter(1.0 / n, 0.0), np.nextafter(1.0 / n, 1.0)]:
            assert oracle.sl_keeps_whole(n, 1.0, float(u)) == (Fraction(float(u)) < Fraction(1, n)), (n, u)
    # alpha >= 2 never shortens; length 1 and 0 are untouched
    assert all(oracle.sl_keeps_whole(n, 2.0, 0.999) for n in (1, 5, 4096))
    assert oracle.sl_keeps_whole(1, 1.6, 0.5)
    # the printed case is shortened "most of the time": for u spread over
    # [0, 1) it is kept whole only below 4096^-0.4 = 0.0359
    us = (np.arange(10000) + 0.5) / 10000
    kept = np.mean([oracle.sl_keeps_whole(4096, 1.6, float(u)) for u in us])
    assert abs(kept - 4096 ** -0.4) < 1e-3 and kept < 0.5


def sl_brute(offsets, alpha, u, keys):
    idx, off = [], [0]
    for b in range(len(offsets) - 1):
        lo, hi = int(offsets[b]), int(offsets[b + 1])
        n = hi - lo
        if n > 0 and not oracle.sl_keeps_whole(n, alpha, float(u[b])):
            L = oracle.sl_target_length(n, alpha)
            if keys is None:
                rows = np.arange(hi - L, hi)
            else:
                order = np.lexsort((np.arange(lo, hi), keys[lo:hi]))  # by key, then position
                rows = lo + np.sort(order[:L])
        else:
            rows = np.arange(lo, hi)
        idx.extend(int(r) for r in rows)
        off.append(len(idx))
    return np.asarray(off), np.asarray(idx, dtype=np.int64)


@pytest.mark.parametrize("mode", ["random", "recency", "random_ties"])
def test_sl_selection_matches_brute_force(mode):
    rng = np.random.default_rng(11)
    lengths = [0, 1, 2, 5, 64, 300, 1000, 4096, 17]
    off = synth.offsets_from_lengths(lengths)
    T = int(off[-1])
    u = rng.random(len(lengths))
    u[7] = 0.5  # the 4096-row sequence is cut
    keys = None
    if mode == "random":
        keys = rng.integers(0, 1 << 32, size=T, dtype=np.uint64).astype(np.uint32)
    elif mode == "random_ties":
        keys = rng.integers(0, 7, size=T).astype(np.uint32)  # many equal keys
    for alpha in (1.6, 1.2, 1.0):
        got_off, got = oracle.sl_select(off, alpha, u, keys)
        want_off, want = sl_brute(off, alpha, u, keys)
        assert np.array_equal(got_off, want_off) and np.array_equal(got, want)
        # structure: per sequence a sorted subset of its rows
        for b in range(len(lengths)):
            seg = got[got_off[b]:got_off[b + 1]]
            assert np.all(np.diff(seg) > 0) and np.all((seg >= off[b]) & (seg < off[b + 1]))
        if alpha == 1.6:
            assert got_off[8] - got_off[7] == 776


def test_sl_random_selection_is_uniform():
    # with uniform random keys every position of a sequence is kept with
    # probability L/n (here 776/4096), whatever its place
    rng = np.random.default_rng(12)
    off = np.array([0, 4096])
    hits = np.zeros(4096)
    for _ in range(200):
        keys = rng.integers(0, 1 << 32, size=4096, dtype=np.uint64).astype(np.uint32)
        _, idx = oracle.sl_select(off, 1.6, [0.9], keys)
        hits[idx] += 1
    p = hits / 200
    assert abs(p.mean() - 776 / 4096) < 1e-9
    assert abs(p[:2048].mean() - p[2048:].mean()) < 0.01


def test_sl_gather_rows():
    x = np.arange(40, dtype=np.int64).reshape(10, 4)
    assert np.array_equal(oracle.gather_rows(x, [3, 0, 9]), x[[3, 0, 9]])


def test_sl_planted_mistakes_are_caught(monkeypatch):
    orig = ho.sl_target_length

    def ceil_length(n, alpha):
        return min(int(math.ceil(float(ho._pow_exact(n, ho.Fraction(alpha) / 2)))), n)

    def full_alpha(n, alpha):
        return min(int(math.floor(float(ho._pow_exact(n, ho.Fraction(alpha))))), n)

    for bad in (ceil_length, full_alpha):
        monkeypatch.setattr(ho, "sl_target_length", bad)
        monkeypatch.setattr(oracle, "sl_target_length", bad)
        with pytest.raises(AssertionError):
            test_sl_printed_length_after_sampling()
    monkeypatch.setattr(ho, "sl_target_length", orig)
    monkeypatch.setattr(oracle, "sl_target_length", orig)
    # ties broken the wrong way, and kept rows not in their original order
    orig_select = ho.sl_select

    def unordered(offsets, alpha, u, keys=None):
        o, idx = orig_select(offsets, alpha, u, keys)
        for b in range(len(o) - 1):
            idx[o[b]:o[b + 1]] = idx[o[b]:o[b + 1]][::-1].copy()
        return o, idx

    monkeypatch.setattr(oracle, "sl_select", unordered)
    with pytest.raises(AssertionError):
        test_sl_selection_matches_brute_force("random")

    def late_ties(offsets, alpha, u, keys=None):
        if keys is None:
            return orig_select(offsets, alpha, u, keys)
        out_off, idx = [0], []
        for b in range(len(offsets) - 1):
            lo, hi = int(offsets[b]), int(offsets[b + 1])
            n = hi - lo
            if n and not ho.sl_keeps_whole(n, alpha, float(u[b])):
                order = sorted(range(lo, hi), key=lambda r: (int(keys[r]), -r))
                idx.extend(sorted(order[:ho.sl_target_length(n, alpha)]))
            else:
                idx.extend(range(lo, hi))
            out_off.append(len(idx))
        return np.asarray(out_off), np.asarray(idx, dtype=np.int64)

    monkeypatch.setattr(oracle, "sl_select", late_ties)
    with pytest.raises(AssertionError):
        test_sl_selection_matches_brute_force("random_ties")


# --------------------------------------------------------------------------
# HSTU layer steps ([HSTU] §3): projection with SiLU, Norm(O) ⊙ U
# --------------------------------------------------------------------------

def test_projection_matches_brute_force_and_split_order():
    rng = np.random.default_rng(41)
    T, Dm, H, dqk, dv = 5, 6, 2, 3, 4
    x = rng.standard_normal((T, Dm))
    w = rng.standard_normal((H * (2 * dv + 2 * dqk), Dm))
    u, v, q, k = oracle.hstu_projection(x, w, H, dqk, dv)
    # per-element loop: column c of the projection, SiLU, then the split
    cols = []
    for t in range(T):
        row = []
        for c in range(w.shape[0]):
            acc = 0.0
            for e in range(Dm):
                acc += x[t, e] * w[c, e]
            row.append(acc / (1.0 + math.exp(-acc)))
        cols.append(row)
    h = np.array(cols)
    np.testing.assert_allclose(u.reshape(T, -1), h[:, :H * dv], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(v.reshape(T, -1), h[:, H * dv:2 * H * dv], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(q.reshape(T, -1), h[:, 2 * H * dv:2 * H * dv + H * dqk], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(k.reshape(T, -1), h[:, 2 * H * dv + H * dqk:], rtol=1e-12, atol=1e-12)
    # one-hot input column: each output is SiLU of one weight column
    e0 = np.zeros((1, Dm)); e0[0, 2] = 1.0
    uu, vv, qq, kk = oracle.hstu_projection(e0, w, H, dqk, dv)
    np.testing.assert_allclose(np.concatenate([a.reshape(1, -1) for a in (uu, vv, qq, kk)], axis=1)[0],
                               oracle.silu(w[:, 2]), rtol=1e-14, atol=1e-14)


def test_norm_gate_against_library_layer_norm():
    import torch
    rng = np.random.default_rng(42)
    T, H, dv = 7, 3, 8
    o = rng.standard_normal((T, H, dv)) * 5 + 2
    u = rng.standard_normal((T, H, dv))
    got = oracle.hstu_norm_gate(o, u)
    ln = torch.nn.functional.layer_norm(torch.from_numpy(o.reshape(T, -1)), (H * dv,), eps=1e-6)
    np.testing.assert_allclose(got, ln.numpy() * u.reshape(T, -1), rtol=1e-12, atol=1e-12)
    # invariants: with U = 1 every row has mean 0 and variance var/(var+eps);
    # a positive scale and a shift of O do not change the result (eps aside)
    ones = np.ones_like(u)
    n1 = oracle.hstu_norm_gate(o, ones)
    np.testing.assert_allclose(n1.mean(axis=1), 0.0, atol=1e-12)
    var = o.reshape(T, -1).var(axis=1)
    np.testing.assert_allclose(n1.var(axis=1), var / (var + 1e-6), rtol=1e-12)
    np.testing.assert_allclose(oracle.hstu_norm_gate(3.0 * o + 7.0, u, eps=0.0), oracle.hstu_norm_gate(o, u, eps=0.0),
                               rtol=1e-10, atol=1e-12)


def test_layer_step_planted_mistakes_are_caught(monkeypatch):
    # a norm over each head instead of the whole row, and U and V swapped
    def per_head(o, u, eps=1e-6):
        o = np.asarray(o, np.float64)
        m = o.mean(axis=2, keepdims=True)
        va = ((o - m) ** 2).mean(axis=2, keepdims=True)
        return ((o - m) / np.sqrt(va + eps) * u).reshape(o.shape[0], -1)

    monkeypatch.setattr(oracle, "hstu_norm_gate", per_head)
    with pytest.raises(AssertionError):
        test_norm_gate_against_library_layer_norm()
    orig = ho.hstu_projection

    def swapped(x, w, H, dqk, dv):
        u, v, q, k = orig(x, w, H, dqk, dv)
        return v, u, q, k

    monkeypatch.setattr(oracle, "hstu_projection", swapped)
    with pytest.raises(AssertionError):
        test_projection_matches_brute_force_and_split_order()
