"""GPU parity of the HSTU layer steps either side of the attention (the
projection with SiLU and the Norm(O) ⊙ U transformation) against the oracle."""

import numpy as np
import pytest

import oracle
import synth
from hstu_testlib import assert_close, to_f64, upload, upload_tensor

pytestmark = pytest.mark.gpu


def hstu():
    import jagged_hstu_attention_amd as m
    return m


@pytest.mark.parametrize("T,Dm,H,d", [(300, 128, 2, 64), (1, 64, 1, 128), (129, 256, 4, 32), (1300, 64, 2, 64),
                                     (49152, 512, 4, 128)])
def test_projection_matches_oracle(T, Dm, H, d):
    li = synth.layer_inputs(T, Dm, H, d, d, seed=T + Dm)
    x, w = upload_tensor(li.x), upload_tensor(li.w)
    got = hstu().layer_projection(x, w, H, d, d)
    want = oracle.hstu_projection(li.x.f64, li.w.f64, H, d, d)
    for name, g, r in zip("uvqk", got, want):
        assert tuple(g.shape) == (T, H, d)
        assert_close(to_f64(g), r, "bf16", name)


@pytest.mark.parametrize("T,width", [(300, 512), (7, 8), (64, 1024), (5, 1536), (33, 2048), (1000, 4096), (49152, 512)])
def test_norm_gate_matches_oracle(T, width):
    rng = np.random.default_rng(T + width)
    o = synth.from_f32((rng.standard_normal((T, width)) * 3 + 1).astype(np.float32), "bf16")
    u = synth.from_f32(rng.standard_normal((T, width)).astype(np.float32), "bf16")
    got = hstu().layer_norm_gate(upload_tensor(o), upload_tensor(u))
    want = oracle.hstu_norm_gate(o.f64.reshape(T, 1, width), u.f64.reshape(T, 1, width))
    assert_close(to_f64(got), want, "bf16", "y")


def test_layer_chain_projection_attention_norm_gate():
    # X -> U, V, Q, K -> jagged attention with the timestamp bias -> Norm(O) ⊙ U,
    # each step on the GPU, against the oracle's chain in float64
    import torch
    H, d, Dm = 2, 128, 256
    wl = synth.custom([300, 1, 129, 0, 64], num_heads=H, d_qk=d, d_v=d, num_buckets=128, dtype="bf16", seed=91,
                      w_std=0.5, with_dout=False)
    li = synth.layer_inputs(wl.total, Dm, H, d, d, seed=92)
    d_in = upload(wl)
    m = hstu()
    u, v, q, k = m.layer_projection(upload_tensor(li.x), upload_tensor(li.w), H, d, d)
    o = m.jagged_attn_fwd(q, k, v, d_in["offsets"], d_in["ts"], d_in["w"], wl.max_seq_len)
    y = m.layer_norm_gate(o, u)
    # the interface stores U, V, Q, K and O in bf16 between the steps: the
    # oracle's chain rounds its own float64 intermediates the same way
    # (round to nearest even), so each step is compared at its own tolerance
    def bf16(a):
        return synth.bf16_bits_to_f64(synth.f32_to_bf16_bits(np.asarray(a, np.float64).astype(np.float32)))

    ru, rv, rq, rk = (bf16(a) for a in oracle.hstu_projection(li.x.f64, li.w.f64, H, d, d))
    ro = oracle.attn_fwd(rq, rk, rv, wl.offsets, wl.ts, wl.w.f64, 128)
    ry = oracle.hstu_norm_gate(bf16(ro), ru)
    assert_close(to_f64(o), ro, "bf16", "attention output")
    assert_close(to_f64(y), ry, "bf16", "layer output")
    torch.cuda.synchronize()
