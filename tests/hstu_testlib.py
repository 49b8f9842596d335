"""Shared helpers for the GPU tests: upload seeded workloads, compare with the
oracle at the stated tolerances."""

from __future__ import annotations

import math

import numpy as np

# Tolerances.  fp32: relative L2 <= 1e-5 and max absolute error <= 1e-5 —
# literally for the tiny fp32 workload (outputs of magnitude <~ 20), and scaled
# by max(1, max|ref|) for larger fp32 outputs, whose own rounding (about
# |x| * 2^-24 * sqrt(terms)) exceeds 1e-5 once |x| passes ~40.
# bf16: relative L2 <= 5e-3 and max|x - ref| / max|ref| <= 2e-2 per tensor.
FP32_ABS = 1e-5
FP32_REL_L2 = 1e-5
BF16_REL_L2 = 5e-3
BF16_MAX_REL = 2e-2


def torch_mod():
    import torch
    return torch


def upload_tensor(t, device="cuda"):
    torch = torch_mod()
    if t.dtype == "bf16":
        x = torch.from_numpy(t.raw.view(np.int16).copy()).view(torch.bfloat16)
    else:
        x = torch.from_numpy(np.ascontiguousarray(t.raw, dtype=np.float32))
    return x.to(device)


def upload_array(a, device="cuda"):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def upload(wl, device="cuda"):
    d = dict(q=upload_tensor(wl.q, device), k=upload_tensor(wl.k, device), v=upload_tensor(wl.v, device),
             w=upload_tensor(wl.w, device), offsets=upload_array(wl.offsets.astype(np.int64), device),
             ts=upload_array(wl.ts.astype(np.int64), device))
    if wl.dout is not None:
        d["dout"] = upload_tensor(wl.dout, device)
    return d


def to_f64(x) -> np.ndarray:
    torch = torch_mod()
    return x.detach().to(torch.float64).cpu().numpy()


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = got - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    ref_norm = float(np.linalg.norm(ref))
    rel_l2 = float(np.linalg.norm(diff) / ref_norm) if ref_norm > 0 else float(np.linalg.norm(diff))
    ref_max = float(np.max(np.abs(ref))) if ref.size else 0.0
    max_rel = max_abs / ref_max if ref_max > 0 else max_abs
    return dict(max_abs=max_abs, rel_l2=rel_l2, max_rel=max_rel)


def assert_close(got, ref, dtype: str, name: str = "", literal: bool = False):
    e = errors(got, ref)
    assert np.all(np.isfinite(np.asarray(got, np.float64))), f"{name}: non-finite values"
    if dtype == "fp32":
        scale = 1.0 if literal else max(1.0, float(np.max(np.abs(ref))) if np.size(ref) else 1.0)
        assert e["max_abs"] <= FP32_ABS * scale and e["rel_l2"] <= FP32_REL_L2, f"{name}: {e}"
    else:
        assert e["rel_l2"] <= BF16_REL_L2 and e["max_rel"] <= BF16_MAX_REL, f"{name}: {e}"
    return e


def sample_rows(offsets, n, seed, include_edges=True):
    """Row indices spread over all sequences, including first/last rows and
    rows at tile boundaries, deterministic in seed."""
    rng = np.random.default_rng(seed)
    T = int(offsets[-1])
    rows = set(int(x) for x in rng.integers(0, T, size=n)) if T else set()
    if include_edges:
        for b in range(len(offsets) - 1):
            lo, hi = int(offsets[b]), int(offsets[b + 1])
            if hi > lo:
                for r in (lo, hi - 1, lo + 63, lo + 64, lo + 127, lo + 128, hi - 65):
                    if lo <= r < hi:
                        rows.add(r)
                if len(rows) > 4 * n:
                    break
    return sorted(rows)
