"""Benchmark of the jagged HSTU attention hot path on one MI355X.

A step is one forward plus one backward of jagged HSTU attention over the
3072-length batch: B=16 sequences of length 3072, H=4 heads, d_qk=d_v=128,
bf16 inputs with fp32 accumulation, 128 timestamp buckets (synthetic, seeded).
The printed `value` is causal-effective TFLOP/s of the whole step: counted
FLOPs are 2*(d_qk+d_v) per causal pair and head for the forward and
2*(3*d_qk+2*d_v) for the backward, over pairs j <= i inside each sequence.

Inputs, outputs and workspaces are allocated before the timed region; each
step calls the C ABI (forward, then backward) on torch's current stream.

Besides the JSON contract fields it reports:
  roofline      the kernel with the largest time (timed alone with HIP events
                on the stream it runs on) against the bf16 dense MFMA peak;
  cpu_baseline  the float64 oracle on a bounded sample of the same workload;
  extra         the other workloads: the CP=8 rank-3 share at length 16384
                (forward+backward), its chunk-pair reorder in GB/s, the skewed
                power-law batch (forward+backward), the uniform 256..1024
                forward, and the candidates pass: 16 users with a 3072-row
                history and a micro-batch of 1024 candidates each, candidates
                only against cached history K/V (candidates/s and TFLOP/s), and
                Stochastic Length on the skewed batch (selection time, gather
                GB/s against the HBM peak), and the layer steps around the
                attention (projection TFLOP/s, norm-gate GB/s).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extra]
       python bench.py --counter-run          (the program profiled for HBM counters)
       python bench.py --traffic-summary FETCH_CSV WRITE_CSV   (CPU: writes the counter summary)
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2516.6   # 256 CU x 4096 FLOP/clk x 2.4 GHz (published 2.5 PFLOP/s dense)
HBM_PEAK_GBS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def causal_pairs(lengths):
    return int(sum(int(n) * (int(n) + 1) // 2 for n in lengths))


def cp_rank_pairs(lengths, cp_size, rank):
    """Causal pairs whose query row lies in mini-chunks r and 2C-1-r."""
    total = 0
    for n in lengths:
        n = int(n)
        for c in (rank, 2 * cp_size - 1 - rank):
            lo, hi = c * n // (2 * cp_size), (c + 1) * n // (2 * cp_size)
            total += (hi * (hi + 1) - lo * (lo + 1)) // 2
    return total


def flops(pairs, heads, dqk, dv):
    fwd = 2 * (dqk + dv) * pairs * heads
    bwd = 2 * (3 * dqk + 2 * dv) * pairs * heads
    return fwd, bwd


class Case:
    """A workload uploaded once, with preallocated outputs and workspaces."""

    def __init__(self, wl, *, cp_size=1, cp_rank=0):
        import numpy as np
        import torch
        import jagged_hstu_attention_amd as m
        self.m = m
        self.wl = wl

        def up(t):
            if t.dtype == "bf16":
                return torch.from_numpy(t.raw.view(np.int16).copy()).view(torch.bfloat16).cuda()
            return torch.from_numpy(t.raw.copy()).cuda()

        self.k, self.v, self.w = up(wl.k), up(wl.v), up(wl.w)
        self.offsets = torch.from_numpy(wl.offsets).cuda()
        self.ts = torch.from_numpy(wl.ts).cuda()
        q, do = up(wl.q), up(wl.dout)
        self.cp_size, self.cp_rank = cp_size, cp_rank
        if cp_size > 1:
            qr, seg = m.cp_reorder(q, self.offsets, wl.max_seq_len, cp_size)
            dr, _ = m.cp_reorder(do, self.offsets, wl.max_seq_len, cp_size)
            seg = seg.cpu().numpy()
            B = wl.num_seqs
            lo, hi = int(seg[cp_rank * B]), int(seg[(cp_rank + 1) * B])
            q, do = qr[lo:hi].contiguous(), dr[lo:hi].contiguous()
        self.q, self.dout = q, do
        self.out = torch.empty((q.shape[0], q.shape[1], self.v.shape[2]), dtype=q.dtype, device="cuda")
        self.dq = torch.empty_like(q)
        self.dk = torch.empty_like(self.k)
        self.dv = torch.empty_like(self.v)
        self.dw = torch.empty(self.w.shape, dtype=torch.float32, device="cuda")
        # host metadata a caller has from its host copy of the offsets
        self.sum_sq = int(sum(int(L) * int(L) for L in wl.lengths))
        p = m.problem(q, self.k, self.v, self.offsets, self.w, wl.max_seq_len, cp_size=cp_size, cp_rank=cp_rank,
                      sum_sq_len=self.sum_sq)
        self.ws_f = torch.empty(m.workspace_size(p, False), dtype=torch.uint8, device="cuda")
        self.ws_b = torch.empty(m.workspace_size(p, True), dtype=torch.uint8, device="cuda")

    def fwd(self, shared=False, recompute=False):
        self.m.jagged_attn_fwd(self.q, self.k, self.v, self.offsets, self.ts, self.w, self.wl.max_seq_len,
                               cp_size=self.cp_size, cp_rank=self.cp_rank, out=self.out,
                               workspace=self.ws_b if shared else self.ws_f, shared_schedule=shared,
                               sum_sq_len=self.sum_sq, recompute_bwd=recompute)

    def bwd(self, shared=False, recompute=False):
        self.m.jagged_attn_bwd(self.dout, self.q, self.k, self.v, self.offsets, self.ts, self.w,
                               self.wl.max_seq_len, cp_size=self.cp_size, cp_rank=self.cp_rank, dq=self.dq,
                               dk=self.dk, dv=self.dv, dw=self.dw, workspace=self.ws_b, recompute=recompute,
                               shared_schedule=shared, sum_sq_len=self.sum_sq)

    def step(self):
        """One training step of the attention: forward then backward, one
        schedule shared by both (the backward stores the score gradient)."""
        self.fwd(shared=True)
        self.bwd(shared=True)

    def step_recompute(self):
        """The same step with the memory-efficient backward (nothing of the
        size of the attention matrix stored; the dQ pass recomputes G)."""
        self.fwd(shared=True, recompute=True)
        self.bwd(shared=True, recompute=True)


def kernel_flops(pairs, heads, dqk, dv):
    """Algorithmic FLOPs per launch of each attention kernel.  The dK/dV pass
    computes S, dP, dV and dK; the dQ pass is credited with dQ only (with bf16
    and d >= 64 it reads the score gradient the dK/dV pass stored; otherwise its
    S and dP are recomputation).  fwd + bwd_kv + bwd_q equals the counted
    total."""
    return {"fwd": 2 * (dqk + dv) * pairs * heads,
            "bwd_kv": 4 * (dqk + dv) * pairs * heads,
            "bwd_q": 2 * dqk * pairs * heads}


ATTN_SOURCES = ("api.hip", "attn.h", "attn.hip", "bias.h", "common.h", "sched.hip", "swtile.h")


def source_digest():
    """sha256 over the sources of the attention kernels and their launches (to
    tell whether the stored counters of those kernels are current)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "jagged_hstu_attention_amd", "csrc")
    for f in sorted(os.path.join(csrc, n) for n in ATTN_SOURCES):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic(kernel):
    """HBM bytes per launch from the committed counter summary, or None when it
    is missing or was taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic_len3072.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != source_digest():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else int(k["fetch_bytes"] + k["write_bytes"])


COUNTER_CMD = ("rocprofv3 --pmc {counter} --output-format csv -d <dir> -o <name> -- "
               "python bench.py --counter-run")
# Substrings of the kernel symbols (for bf16 with d >= 64 the backward runs
# bwd_kv_half_kernel and bwd_q_g_kernel, otherwise bwd_kv_kernel and
# bwd_q_kernel).
KERNEL_SYMBOLS = {"fwd": "fwd_kernel", "bwd_kv": "bwd_kv_", "bwd_q": "bwd_q_", "sched": "sched_kernel",
                  "reorder": "reorder_kernel", "proj": "proj_kernel", "norm_gate": "norm_gate_kernel"}


def traffic_summary(fetch_csv, write_csv, out_path):
    """Per-launch HBM bytes of each kernel from two rocprofv3 --pmc runs of
    `bench.py --counter-run` (FETCH_SIZE, then WRITE_SIZE; both in KiB per
    dispatch).  Each counter is scaled by what it reads for the 256 MiB device
    copy (the largest copyBuffer dispatch) of that same run: the copy moves
    exactly 256 MiB each way."""
    import csv
    import statistics
    copy_kib = (256 << 20) / 1024.0
    out = {"source_sha256": source_digest(), "workload": "bf16, B=16 x length 3072, H=4, d=128, 128 buckets",
           "commands": [COUNTER_CMD.format(counter=c) for c in ("FETCH_SIZE", "WRITE_SIZE")],
           "calibration": {}, "kernels": {}}
    for counter, path, key in (("FETCH_SIZE", fetch_csv, "fetch_bytes"), ("WRITE_SIZE", write_csv, "write_bytes")):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        copy = max(float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"])
        scale = copy_kib / copy
        out["calibration"][counter] = {"copy_counter_kib": copy, "copy_true_kib": copy_kib,
                                       "scale": round(scale, 4)}
        for k, sym in KERNEL_SYMBOLS.items():
            vals = [float(r["Counter_Value"]) for r in rows if sym in r["Kernel_Name"]]
            if vals:
                ent = out["kernels"].setdefault(k, {})
                ent[key] = int(statistics.mean(vals) * scale * 1024)
                ent[counter.lower() + "_kib_raw_per_dispatch"] = [round(v, 1) for v in vals]
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    return out


def profile_workload(m, name, steps, warmup):
    """W warmup steps, then K steps timed per kernel with the library's HIP
    events (the program rocprofv3 traces; its last K dispatches of each
    kernel are the timed ones)."""
    import torch
    import synth
    cp = {}
    if name == "len3072":
        wl = synth.config("bf16_len3072")
    elif name == "skewed":
        wl = synth.config("skewed_powerlaw")
    elif name == "cp8":  # rank 3's share of the CP=8 batch of length 16384
        wl = synth.config("cp8_rank3_len16384")
        cp = dict(cp_size=synth.CP_SIZE, cp_rank=synth.CP_RANK)
    else:  # the skewed batch's head shape on uniform lengths: 16 x 3072, H = 8, d = 64, 256 buckets
        wl = synth.custom([3072] * 16, num_heads=8, d_qk=64, d_v=64, num_buckets=256, dtype="bf16",
                          gap_mean=600.0, seed=1008)
    case = Case(wl, **cp)
    for _ in range(warmup):
        case.step()
    kms = time_kernels(case, steps)
    pairs = cp_rank_pairs(wl.lengths, cp["cp_size"], cp["cp_rank"]) if cp else causal_pairs(wl.lengths)
    kfl = kernel_flops(pairs, wl.num_heads, wl.d_qk, wl.d_v)
    torch.cuda.synchronize()
    return {"profile": name, "warmup": warmup, "steps": steps, "kernels_ms": {k: round(v, 4) for k, v in kms.items()},
            "kernels_tflops": {k: round(kfl[k] / kms[k] / 1e9, 2) for k in kfl if kms.get(k)},
            "pairs": pairs, "heads": wl.num_heads, "d": wl.d_qk}


def trace_summary(path, last):
    """Average duration (us) of the last `last` dispatches of each kernel in a
    rocprofv3 kernel_trace.csv, next to the average over all of them."""
    import csv
    import re
    rows = list(csv.DictReader(open(path)))
    by = {}
    for r in sorted(rows, key=lambda r: int(r["Start_Timestamp"])):
        name = re.sub(r"\(.*", "", r["Kernel_Name"])[:80]
        by.setdefault(name, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    return {k: {"dispatches": len(v), "avg_us_all": round(sum(v) / len(v), 2),
                f"avg_us_last_{min(last, len(v))}": round(sum(v[-last:]) / len(v[-last:]), 2)}
            for k, v in sorted(by.items(), key=lambda kv: -sum(kv[1]))}


def balance_model(name):
    """Longest-first (descending cost, each item to the earliest-free slot)
    schedule of the attention items, from the scheduler's cost rules: a
    (128-row query tile, head) item costs the 64-key tiles of its causal
    prefix (forward, dQ); a (128-key tile, head) item costs the 64-row query
    steps from its first key on (dK/dV).  Slots: 512 for the forward and dQ
    passes (two workgroups per compute unit at d = 128; three for the d = 64
    forward), 256 for the dK/dV pass."""
    import heapq
    import synth
    wl = synth.config("bf16_len3072" if name == "len3072" else "skewed_powerlaw", with_dout=False)
    H = wl.num_heads
    q_items, k_items = [], []
    for L in map(int, wl.lengths):
        for i in range(0, L, 128):
            q_items += [(min(i + 128, L) + 63) // 64] * H
        for k0 in range(0, L, 128):
            k_items += [(L - k0 + 63) // 64] * H

    def lpt(costs, slots):
        heap = [0] * slots
        for c in sorted(costs, reverse=True):
            t = heapq.heappop(heap)
            heapq.heappush(heap, t + c)
        makespan = max(heap)
        mean = sum(costs) / slots
        return {"items": len(costs), "slots": slots, "total_cost": sum(costs), "max_item": max(costs),
                "makespan": makespan, "mean_load": round(mean, 2), "makespan_over_mean": round(makespan / mean, 4)}

    fwd_slots = 768 if wl.d_qk <= 64 else 512
    return {"workload": name, "lengths": {"B": len(wl.lengths), "max": int(max(wl.lengths)),
                                          "sum": int(sum(wl.lengths))},
            "forward": lpt(q_items, fwd_slots), "dq": lpt(q_items, 512), "dkdv": lpt(k_items, 256)}


def time_kernels(case, steps):
    """Per-kernel average milliseconds, from HIP events the library records on
    the launch stream around each kernel (one forward + one backward per call)."""
    import torch
    m = case.m
    torch.cuda.synchronize()
    m.timing_reset()
    m.timing_enable(True)
    for _ in range(steps):
        case.step()
    torch.cuda.synchronize()
    m.timing_enable(False)
    out = {}
    for k in ("sched", "fwd", "bwd_kv", "bwd_q", "reduce"):  # reduce: sums of split key walks (0 if none)
        ms, n = m.timing_read(k)
        out[k] = ms / max(n, 1)
    m.timing_reset()
    return out


def time_loop(fn, steps, warmup):
    """Average ms per call over `steps` calls, bracketed by HIP events on the
    current stream (the stream every launch goes to)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def candidates_pass(m, steps, users=16, hist=3072, cands=1024):
    """Candidates-only forward against cached history K/V: each user's 3072
    history rows plus a micro-batch of 1024 candidates, H=4, d=128, bf16.
    Counted work: each candidate attends to its history and itself,
    2*(d_qk+d_v) FLOP per pair and head."""
    import numpy as np
    import torch
    import synth
    wl = synth.custom([hist + cands] * users, num_heads=4, d_qk=128, d_v=128, num_buckets=128, dtype="bf16",
                      gap_mean=3600.0, seed=1006, w_std=0.02, with_dout=False)

    def up(t):
        return torch.from_numpy(t.raw.view(np.int16).copy()).view(torch.bfloat16).cuda()

    k, v, w = up(wl.k), up(wl.v), up(wl.w)
    offsets = torch.from_numpy(wl.offsets).cuda()
    ts = torch.from_numpy(wl.ts).cuda()
    rows = np.concatenate([np.arange(int(wl.offsets[b + 1]) - cands, int(wl.offsets[b + 1])) for b in range(users)])
    q = up(wl.q)[torch.from_numpy(rows).cuda()].contiguous()
    nt = torch.full((users,), cands, dtype=torch.int64, device="cuda")
    out = torch.empty_like(q)
    p = m.problem(q, k, v, offsets, w, wl.max_seq_len)
    ws = torch.empty(m.workspace_size(p, False), dtype=torch.uint8, device="cuda")

    def run():
        m.jagged_attn_fwd_targets(q, k, v, offsets, nt, ts, w, wl.max_seq_len, q_targets_only=True, out=out,
                                  workspace=ws)

    t = time_loop(run, steps, 2)
    fl = 2 * (128 + 128) * users * cands * (hist + 1) * 4
    return {"fwd_ms": round(t, 4), "candidates_per_s": round(users * cands / t * 1e3, 1),
            "tflops": round(fl / t / 1e9, 2)}


def stochastic_length(m, steps):
    """Stochastic Length on the skewed power-law batch (B = 256, lengths
    16..8192, H = 8, d = 64, bf16) at alpha = 1.6 with random selection:
    the selection (kept lengths, offsets, row index) and the gather of q, k,
    v and the timestamps into the sampled jagged batch.  The gather moves
    2 x kept rows x row bytes per tensor (read + write) against the 8 TB/s
    HBM peak."""
    import numpy as np
    import torch
    import synth
    wl = synth.config("skewed_powerlaw", with_dout=False)

    def up(t):
        return torch.from_numpy(t.raw.view(np.int16).copy()).view(torch.bfloat16).cuda()

    q, k, v = up(wl.q), up(wl.k), up(wl.v)
    ts = torch.from_numpy(wl.ts).cuda()
    off = torch.from_numpy(wl.offsets).cuda()
    rng = np.random.default_rng(1006)
    u = torch.from_numpy(rng.random(wl.num_seqs).astype(np.float32)).cuda()
    keys = torch.from_numpy(rng.integers(0, 1 << 32, size=wl.total, dtype=np.uint64).astype(np.uint32)
                            .view(np.int32)).cuda()
    out_off = torch.empty(wl.num_seqs + 1, dtype=torch.int64, device="cuda")
    out_idx = torch.empty(wl.total, dtype=torch.int64, device="cuda")
    outs = [torch.empty_like(t) for t in (q, k, v, ts)]

    def select():
        m.sl_select(off, wl.max_seq_len, 1.6, u, keys, out_offsets=out_off, out_index=out_idx)

    def gather():
        for src, dst in zip((q, k, v, ts), outs):
            m.gather_rows(src, out_idx, out_off[-1:], out=dst)

    t_sel = time_loop(select, steps, 3)
    t_gat = time_loop(gather, steps, 3)
    kept = int(out_off[-1].item())
    row_bytes = sum(t.element_size() * int(np.prod(t.shape[1:])) for t in (q, k, v, ts))
    moved = 2 * kept * row_bytes
    return {"alpha": 1.6, "rows_in": wl.total, "rows_kept": kept, "select_ms": round(t_sel, 4),
            "gather_ms": round(t_gat, 4), "gather_gbs": round(moved / t_gat / 1e6, 1),
            "gather_frac_hbm": round(moved / t_gat / 1e6 / HBM_PEAK_GBS, 4),
            "rows_per_s": round(wl.total / ((t_sel + t_gat) * 1e-3), 1)}


def layer_steps(m, steps):
    """The HSTU layer steps around the attention at the 3072-length workload's
    shape (T = 49152 rows, d_model = 512, H = 4, d = 128, bf16): the projection
    GEMM with SiLU (2 T d_model N FLOP, N = H (2 d_v + 2 d_qk) = 2048, against
    the bf16 dense peak) and the norm-gate (reads O and U, writes Y: 3 T H d_v
    x 2 bytes, against the HBM peak)."""
    import torch
    import synth
    T, Dm, H, d = 49152, 512, 4, 128
    li = synth.layer_inputs(T, Dm, H, d, d, seed=1007)

    def up(t):
        import numpy as np
        return torch.from_numpy(t.raw.view(np.int16).copy()).view(torch.bfloat16).cuda()

    x, w = up(li.x), up(li.w)
    outs = tuple(torch.empty((T, H, d), dtype=torch.bfloat16, device="cuda") for _ in range(4))
    y = torch.empty((T, H * d), dtype=torch.bfloat16, device="cuda")

    def proj():
        m.layer_projection(x, w, H, d, d, out=outs)

    def gate():
        m.layer_norm_gate(outs[1], outs[0], out=y)

    t_p = time_loop(proj, steps, 3)
    t_g = time_loop(gate, steps, 3)
    fl = 2 * T * Dm * H * 4 * d
    nbytes = 3 * T * H * d * 2
    return {"workload": "T=49152, d_model=512, H=4, d=128, bf16", "projection_ms": round(t_p, 4),
            "projection_tflops": round(fl / t_p / 1e9, 2), "projection_frac_bf16_peak": round(fl / t_p / 1e9 / BF16_PEAK_TFLOPS, 4),
            "norm_gate_ms": round(t_g, 4), "norm_gate_gbs": round(nbytes / t_g / 1e6, 1),
            "norm_gate_frac_hbm": round(nbytes / t_g / 1e6 / HBM_PEAK_GBS, 4)}


def cpu_baseline(max_seconds=30.0):
    """The float64 oracle, as it stands, on a bounded sample of the 3072-length
    workload: whole sequences (all 4 heads, forward + backward), as many as fit
    in about 15 s, scaled to causal-effective TFLOP/s."""
    import oracle
    import synth
    try:
        import threadpoolctl
        blas_threads = max(p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()) or 1
    except Exception:
        blas_threads = os.cpu_count() or 1
    n_done, t_total = 0, 0.0
    wl = synth.config("bf16_len3072", num_seqs=4)
    for b in range(4):
        lo, hi = int(wl.offsets[b]), int(wl.offsets[b + 1])
        off = [0, hi - lo]
        sl = slice(lo, hi)
        t0 = time.perf_counter()
        oracle.attn_fwd(wl.q.f64[sl], wl.k.f64[sl], wl.v.f64[sl], off, wl.ts[sl], wl.w.f64, wl.num_buckets)
        oracle.attn_bwd(wl.dout.f64[sl], wl.q.f64[sl], wl.k.f64[sl], wl.v.f64[sl], off, wl.ts[sl], wl.w.f64,
                        wl.num_buckets)
        t_total += time.perf_counter() - t0
        n_done += 1
        if t_total > max_seconds / 2:
            break
    f, bw = flops(causal_pairs([3072] * n_done), 4, 128, 128)
    return {
        "value": (f + bw) / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": f"{n_done} of 16 sequences (length 3072, 4 heads, d=128), forward+backward in float64 numpy, "
                  f"{t_total:.1f} s; BLAS threads={blas_threads}, elementwise numpy single-threaded; "
                  f"host has {os.cpu_count()} logical CPUs",
    }


def reorder_bandwidth(m, steps):
    """Chunk-pair reorder of the CP=8, length-16384 bf16 [65536, 4, 128] tensor.
    Buffer pairs are rotated so the working set (5 x 128 MiB) exceeds the
    256 MB last-level cache; a plain device copy of the same bytes is timed
    the same way."""
    import torch
    import synth
    B, L, C = 4, 16384, 8
    off = torch.from_numpy(synth.offsets_from_lengths([L] * B)).cuda()
    nbuf = 5
    src = [torch.randn(B * L, 4, 128, device="cuda").to(torch.bfloat16) for _ in range(nbuf)]
    dst = [torch.empty_like(s) for s in src]
    seg = torch.empty(C * B + 1, dtype=torch.int64, device="cuda")
    it = [0]

    def one():
        i = it[0] % nbuf
        it[0] += 1
        m.cp_reorder(src[i], off, L, C, out=dst[i], out_offsets=seg)

    def cp():
        i = it[0] % nbuf
        it[0] += 1
        dst[i].copy_(src[i])

    ms = time_loop(one, steps, 3)
    ms_copy = time_loop(cp, steps, 3)
    nbytes = 2 * src[0].numel() * 2
    return {"gbs": nbytes / ms / 1e6, "ms": ms, "copy_gbs": nbytes / ms_copy / 1e6, "bytes_moved": nbytes}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--counter-run", action="store_true",
                    help="for rocprofv3 --pmc: a 256 MiB device copy (calibration), then 3 forward+backward "
                         "steps of the 3072-length workload, 15 chunk-pair reorders and 3 calls of each layer "
                         "step; no timing")
    ap.add_argument("--profile", choices=["len3072", "skewed", "uniform_d64", "cp8", "layer"],
                    help="for rocprofv3 --kernel-trace: W warmup then K timed steps of one workload (one schedule "
                         "per step); prints the per-kernel HIP-event averages of the timed steps as JSON")
    ap.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV",
                    help="CPU only: per-kernel average duration of the last --last dispatches of each kernel in a "
                         "rocprofv3 kernel_trace.csv")
    ap.add_argument("--last", type=int, default=20)
    ap.add_argument("--balance-model", choices=["len3072", "skewed"],
                    help="CPU only: longest-first schedule of the attention work items over the workgroup slots "
                         "(makespan against the mean load), from the scheduler's cost rules")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="CPU only: turn the two --pmc counter CSVs of --counter-run into "
                         "profiles/traffic_len3072.json and exit")
    args = ap.parse_args()
    if args.trace_summary:
        print(json.dumps(trace_summary(args.trace_summary, args.last), indent=1))
        return
    if args.balance_model:
        print(json.dumps(balance_model(args.balance_model), indent=1))
        return
    if args.traffic_summary:
        t = traffic_summary(*args.traffic_summary, os.path.join(ROOT, "profiles", "traffic_len3072.json"))
        print(json.dumps({k: {kk: vv for kk, vv in v.items() if kk.endswith("bytes")}
                          for k, v in t["kernels"].items()}))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import jagged_hstu_attention_amd as m
    import synth

    m._lib.load()
    torch.cuda.set_device(0)
    if args.counter_run:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        case = Case(synth.config("bf16_len3072"))
        for _ in range(3):
            case.step()
        torch.cuda.synchronize()
        del case, dst
        torch.cuda.empty_cache()
        # the chunk-pair reorder of the CP=8 length-16384 bf16 tensor, on 5
        # rotating buffer pairs (640 MiB, past the last-level cache), 3 passes
        off = torch.from_numpy(synth.offsets_from_lengths([16384] * 4)).cuda()
        bufs = [(torch.randn(65536, 4, 128, device="cuda").to(torch.bfloat16),
                 torch.empty(65536, 4, 128, dtype=torch.bfloat16, device="cuda")) for _ in range(5)]
        seg = torch.empty(8 * 4 + 1, dtype=torch.int64, device="cuda")
        for _ in range(3):
            for a, b in bufs:
                m.cp_reorder(a, off, 16384, 8, out=b, out_offsets=seg)
        torch.cuda.synchronize()
        del bufs
        torch.cuda.empty_cache()
        # the layer steps at the 3072-length shape (T = 49152, d_model = 512,
        # H = 4, d = 128), 3 calls each on freshly written inputs
        T, Dm, H, d = 49152, 512, 4, 128
        for i in range(3):
            x = torch.randn(T, Dm, device="cuda").to(torch.bfloat16)
            w = (torch.randn(4 * H * d, Dm, device="cuda") * 0.05).to(torch.bfloat16)
            outs = m.layer_projection(x, w, H, d, d)
            o = torch.randn(T, H * d, device="cuda").to(torch.bfloat16)
            u = torch.randn(T, H * d, device="cuda").to(torch.bfloat16)
            m.layer_norm_gate(o, u)
            torch.cuda.synchronize()
            del x, w, outs, o, u
        print(json.dumps({"counter_run": True, "copy_bytes": src.numel()}), flush=True)
        return
    if args.profile == "layer":  # the layer steps' launches, timed as in the bench line
        print(json.dumps({"profile": "layer", **layer_steps(m, args.steps)}), flush=True)
        return
    if args.profile:
        print(json.dumps(profile_workload(m, args.profile, args.steps, args.warmup)), flush=True)
        return
    log("uploading the 3072-length workload")
    wl = synth.config("bf16_len3072")
    case = Case(wl)
    pairs = causal_pairs(wl.lengths)
    f_fwd, f_bwd = flops(pairs, wl.num_heads, wl.d_qk, wl.d_v)

    log(f"timing {args.steps} steps after {args.warmup} warmup")
    ms_step = time_loop(case.step, args.steps, args.warmup)
    value = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12
    log(f"step {ms_step:.3f} ms -> {value:.1f} TFLOP/s")

    ms_fwd = time_loop(case.fwd, args.steps, 2)
    ms_bwd = time_loop(case.bwd, args.steps, 2)
    ms_rec = time_loop(case.step_recompute, args.steps, 2)
    log(f"forward {ms_fwd:.3f} ms, backward {ms_bwd:.3f} ms, step with the recompute backward {ms_rec:.3f} ms")
    kms = time_kernels(case, args.steps)
    kfl = kernel_flops(pairs, wl.num_heads, wl.d_qk, wl.d_v)
    log("per kernel (ms): " + ", ".join(f"{k} {v:.4f}" for k, v in kms.items()))
    dom = max(("fwd", "bwd_kv", "bwd_q"), key=lambda k: kms[k])
    achieved = kfl[dom] / (kms[dom] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": stored_traffic(dom),
                "kernel": {"fwd": "fwd_kernel", "bwd_kv": "bwd_kv_half_kernel", "bwd_q": "bwd_q_g_kernel"}[dom],
                "ms_per_launch": round(kms[dom], 4), "flop_per_launch": kfl[dom]}

    extra = {
        "value_backward": "stored score gradient (the dK/dV pass writes G = dS, the dQ pass reads it); "
                          "one schedule shared by the forward and backward",
        "len3072_step_recompute": {"ms": round(ms_rec, 4), "tflops": round((f_fwd + f_bwd) / ms_rec / 1e9, 2),
                                   "backward": "memory-efficient: nothing of the size of the attention matrix "
                                               "stored, the dQ pass recomputes S, dP and G"},
        "len3072_forward": {"ms": round(ms_fwd, 4), "tflops": round(f_fwd / ms_fwd / 1e9, 2)},
        "len3072_backward": {"ms": round(ms_bwd, 4), "tflops": round(f_bwd / ms_bwd / 1e9, 2)},
        "len3072_kernels_ms": {k: round(v, 4) for k, v in kms.items()},
        "len3072_kernels_tflops": {k: round(kfl[k] / kms[k] / 1e9, 2) for k in kfl},
    }
    if not args.no_extra:
        del case
        torch.cuda.empty_cache()
        log("CP=8 rank-3 share, length 16384")
        wl4 = synth.config("cp8_rank3_len16384")
        c4 = Case(wl4, cp_size=synth.CP_SIZE, cp_rank=synth.CP_RANK)
        p4 = cp_rank_pairs(wl4.lengths, synth.CP_SIZE, synth.CP_RANK)
        f4f, f4b = flops(p4, wl4.num_heads, wl4.d_qk, wl4.d_v)
        t4f = time_loop(c4.fwd, args.steps, 2)
        t4b = time_loop(c4.bwd, args.steps, 2)
        k4 = time_kernels(c4, args.steps)
        extra["cp8_rank3_len16384"] = {"fwd_ms": round(t4f, 4), "bwd_ms": round(t4b, 4),
                                       "tflops": round((f4f + f4b) / (t4f + t4b) / 1e9, 2),
                                       "kernels_ms": {k: round(v, 4) for k, v in k4.items()}}
        del c4
        torch.cuda.empty_cache()
        log("reorder bandwidth")
        rb = reorder_bandwidth(m, args.steps)
        extra["cp8_reorder_len16384"] = {"gbs": round(rb["gbs"], 1), "frac_hbm": round(rb["gbs"] / HBM_PEAK_GBS, 4),
                                         "copy_gbs": round(rb["copy_gbs"], 1), "ms": round(rb["ms"], 4)}
        torch.cuda.empty_cache()
        log("skewed power-law batch")
        wl5 = synth.config("skewed_powerlaw")
        c5 = Case(wl5)
        f5f, f5b = flops(causal_pairs(wl5.lengths), wl5.num_heads, wl5.d_qk, wl5.d_v)
        t5f = time_loop(c5.fwd, args.steps, 2)
        t5b = time_loop(c5.bwd, args.steps, 2)
        extra["skewed_powerlaw"] = {"fwd_ms": round(t5f, 4), "bwd_ms": round(t5b, 4),
                                    "tflops": round((f5f + f5b) / (t5f + t5b) / 1e9, 2)}
        del c5
        torch.cuda.empty_cache()
        log("uniform 256..1024 forward")
        wl2 = synth.config("bf16_fwd_u256_1024", with_dout=True)
        c2 = Case(wl2)
        f2f, _ = flops(causal_pairs(wl2.lengths), wl2.num_heads, wl2.d_qk, wl2.d_v)
        t2f = time_loop(c2.fwd, args.steps, 2)
        extra["u256_1024_forward"] = {"fwd_ms": round(t2f, 4), "tflops": round(f2f / t2f / 1e9, 2)}
        del c2
        torch.cuda.empty_cache()
        log("candidates against cached history")
        extra["candidates_b16_hist3072_m1024"] = candidates_pass(m, args.steps)
        torch.cuda.empty_cache()
        log("stochastic length on the skewed batch")
        extra["stochastic_length_skewed_alpha1.6"] = stochastic_length(m, args.steps)
        torch.cuda.empty_cache()
        log("layer steps (projection, norm-gate)")
        extra["layer_steps_len3072_shape"] = layer_steps(m, args.steps)

    cpu = None
    if not args.no_cpu:
        log("CPU oracle baseline (bounded sample)")
        cpu = cpu_baseline()

    line = {
        "metric": "jagged HSTU attention TFLOPS (causal-effective) and % of bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "bf16 forward+backward, B=16 x length 3072, H=4, d_qk=d_v=128, 128 buckets",
                   "global_batch": 16, "seq_len": 3072, "parallelism": "none (1 GPU)",
                   "pct_of_bf16_peak": round(100 * value / BF16_PEAK_TFLOPS, 2)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
