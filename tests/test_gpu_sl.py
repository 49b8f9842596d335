"""GPU parity of Stochastic Length: selection and row gather against the
oracle, bit for bit (integer and byte work)."""

import numpy as np
import pytest

import oracle
import synth
from hstu_testlib import upload, upload_array

pytestmark = pytest.mark.gpu


def hstu():
    import jagged_hstu_attention_amd as m
    return m


def run_select(offsets, alpha, u, keys):
    import torch
    m = hstu()
    T = int(offsets[-1])
    d_off = upload_array(np.asarray(offsets, dtype=np.int64))
    d_u = upload_array(np.asarray(u, dtype=np.float32))
    d_keys = upload_array(keys.view(np.int32)) if keys is not None else None
    out_index = torch.full((max(T, 1),), -1, dtype=torch.int64, device="cuda")
    max_len = int(np.max(np.diff(offsets))) if len(offsets) > 1 else 0
    o, idx = m.sl_select(d_off, max_len, alpha, d_u, d_keys, out_index=out_index[:T] if T else out_index[:0])
    o = o.cpu().numpy()
    return o, out_index[: int(o[-1])].cpu().numpy(), out_index


LENGTHS = [0, 1, 2, 3, 5, 64, 300, 1000, 4096, 17, 8192, 777]


@pytest.mark.parametrize("mode", ["random", "recency", "ties"])
@pytest.mark.parametrize("alpha", [1.6, 1.0, 1.3, 1.9])
def test_sl_select_matches_oracle(mode, alpha):
    rng = np.random.default_rng(21)
    off = synth.offsets_from_lengths(LENGTHS)
    T = int(off[-1])
    u = rng.random(len(LENGTHS)).astype(np.float32)
    u[8] = 0.5  # the 4096-row sequence is cut at alpha 1.6
    keys = None
    if mode == "random":
        keys = rng.integers(0, 1 << 32, size=T, dtype=np.uint64).astype(np.uint32)
    elif mode == "ties":
        keys = rng.integers(0, 5, size=T).astype(np.uint32)
    got_off, got_idx, _ = run_select(off, alpha, u, keys)
    want_off, want_idx = oracle.sl_select(off, alpha, u, keys)
    assert np.array_equal(got_off, want_off)
    assert np.array_equal(got_idx, want_idx)
    if alpha == 1.6:
        assert got_off[9] - got_off[8] == 776


@pytest.mark.parametrize("alpha", [1.6, 1.0, 1.5, 1.2])
def test_sl_lengths_for_every_length_up_to_4096(alpha):
    # one sequence of every length 1..4096, always cut: the kept lengths equal
    # the oracle's exact floor(n^(alpha/2)) for every n
    lengths = np.arange(1, 4097)
    off = synth.offsets_from_lengths(lengths)
    u = np.full(len(lengths), 0.999999, dtype=np.float32)
    got_off, got_idx, _ = run_select(off, alpha, u, None)
    want = np.array([n if oracle.sl_keeps_whole(int(n), alpha, 0.999999) else oracle.sl_target_length(int(n), alpha)
                     for n in lengths])
    assert np.array_equal(np.diff(got_off), want)
    # recency keeps the last rows of each sequence
    want_off, want_idx = oracle.sl_select(off, alpha, u, None)
    assert np.array_equal(got_idx, want_idx)


@pytest.mark.parametrize("row_shape,dtype", [((8, 64), "bf16"), ((1,), "i64"), ((3,), "u8"), ((5,), "f32")])
def test_gather_rows_bit_exact(row_shape, dtype):
    import torch
    rng = np.random.default_rng(22)
    off = synth.offsets_from_lengths([100, 0, 513, 7, 2048])
    T = int(off[-1])
    if dtype == "bf16":
        x = rng.integers(0, 1 << 16, size=(T, *row_shape), dtype=np.uint16).view(np.int16)
    elif dtype == "i64":
        x = rng.integers(-(1 << 62), 1 << 62, size=(T, *row_shape), dtype=np.int64)
    elif dtype == "u8":
        x = rng.integers(0, 256, size=(T, *row_shape), dtype=np.uint8)
    else:
        x = rng.standard_normal(size=(T, *row_shape)).astype(np.float32)
    keys = rng.integers(0, 1 << 32, size=T, dtype=np.uint64).astype(np.uint32)
    u = np.full(5, 0.9, dtype=np.float32)
    got_off, got_idx, d_idx = run_select(off, 1.6, u, keys)
    dx = upload_array(x)
    d_cnt = upload_array(got_off[-1:].astype(np.int64))
    out = torch.zeros_like(dx)
    hstu().gather_rows(dx, d_idx[:T], d_cnt, out=out)
    n = int(got_off[-1])
    want = oracle.gather_rows(x, oracle.sl_select(off, 1.6, u, keys)[1])
    assert np.array_equal(out[:n].cpu().numpy().view(np.uint8), want.view(np.uint8))
    assert np.all(out[n:].cpu().numpy().view(np.uint8) == 0)  # rows past the count untouched


@pytest.mark.parametrize("seed", [1005, 1105])
def test_sl_skewed_batch_select_and_gather(seed):
    # the skewed power-law batch (B = 256, lengths 16..8192) at alpha 1.6,
    # random selection: the sampled q, k, v and timestamps, bit for bit
    import torch
    wl = synth.config("skewed_powerlaw", seed=seed)
    d = upload(wl)
    rng = np.random.default_rng(seed)
    u = rng.random(wl.num_seqs).astype(np.float32)
    keys = rng.integers(0, 1 << 32, size=wl.total, dtype=np.uint64).astype(np.uint32)
    got_off, got_idx, d_idx = run_select(wl.offsets, 1.6, u, keys)
    want_off, want_idx = oracle.sl_select(wl.offsets, 1.6, u, keys)
    assert np.array_equal(got_off, want_off) and np.array_equal(got_idx, want_idx)
    d_cnt = upload_array(got_off[-1:].astype(np.int64))
    n = int(got_off[-1])
    for name in ("q", "k", "v", "ts"):
        out = hstu().gather_rows(d[name], d_idx[: wl.total], d_cnt)
        host = d[name].cpu()
        assert torch.equal(out[:n].cpu(), host[torch.from_numpy(want_idx)]), name
