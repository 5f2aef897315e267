#!/usr/bin/env python3
"""Throughput of batched draft verification on one MI355X.

Default workload: the heavy-load batch -- B=512 requests, K=8, budgets
2..8 (mean 4), V=151,936, bf16 target and drafter logits, T=1 -- verified
back to back with a fresh Philox seed per step, inputs resident in HBM.

Prints one JSON line: verified draft tokens/s (sum of budgets per step over
the step time); the roofline of the whole verify call (algorithmic HBM bytes
per call over the streaming pass's plus the draw pass's duration, from the
library's own per-pass HIP events, against the 8 TB/s HBM peak), with the
streaming pass's own figure beside it; the timed step's outputs against the
fp64 CPU oracle on every request (near-ties excused and counted); the oracle
as a CPU baseline on a pool of host processes (every workload's step); and,
on the same batch shape, the verify-budget scheduler (per call, beside its
oracle), the fused output head (TFLOP/s against the 2.5 PFLOP/s dense bf16
peak, beside its oracle), a whole verify step from hidden states through that
head, and the drafter's low-rank Markov head over a drafted block (each per
call, beside its oracle); the other synthetic workloads (Qwen3- and
Gemma-shaped vocabularies, the ragged batch) and, as context, a plain
read-only reduction over the same logits.

  python bench.py [--steps K] [--warmup W] [--warmup-settle S] [--workload heavy]
                  [--no-cpu-baseline] [--verify-only]
  python bench.py --copy-probe GIB   # plain copies of a known size (counter scale)
  python bench.py --markov-only      # the Markov head alone at the heavy shape (profiling)
  python bench.py --head-only        # the output head alone at the heavy rows (profiling)
  python bench.py --hidden-only      # the whole step from hidden states alone (profiling)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E peak, GB/s
WARMUP_SETTLE_S = 0.2           # minimum busy time before the timed steps
KERNEL_SRC = os.path.join(ROOT, "draft_verify_sampling_spec_amd", "csrc", "spec_verify.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "verify_kernel_heavy_traffic.json")
WORKLOAD_INDEX = {"tiny": 1, "qwen3": 2, "ragged": 3, "gemma": 4, "heavy": 5}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(budgets, K, V, elem_bytes, greedy):
    """HBM bytes the method must move once per step: every budgeted logit row
    read once (k_b+1 target rows, k_b drafter rows; greedy reads no drafter
    rows), drafted tokens and budgets read, tokens and counts written."""
    ksum = int(sum(int(k) for k in budgets))
    B = len(budgets)
    rows = ksum + B if greedy else 2 * ksum + B
    return rows * V * elem_bytes + 4 * (B * K + B) + 4 * (B * (K + 1) + B), rows


def kernel_source_hash():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def load_traffic():
    """HBM traffic per launch of each pass and per call, from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    ks = rec.get("kernels", {})
    stream = ks.get("streaming pass", {}).get("hbm_bytes_per_launch")
    draw = ks.get("draw pass", {}).get("hbm_bytes_per_launch")
    if stream is None or draw is None:
        return None
    return {"stream": stream, "draw": draw, "call": stream + draw}


def cpu_baseline(inp, seeds, n_requests, min_seconds=5.0, max_seconds=15.0):
    """The fp64 oracle, as it stands, in this one process on the first
    n_requests of the batch, repeated with fresh Philox seeds until about
    min_seconds of CPU work (never starting a pass after max_seconds).
    Returns (tokens/s, seconds, passes)."""
    import numpy as np
    import torch
    from oracle import verify as ov

    def bits(x):
        return x.cpu().view(torch.int16).numpy().view(np.uint16)

    budgets = inp["budgets"].cpu().numpy()
    tokens = inp["tokens"].cpu().numpy()
    T = inp["temperature"]
    rows = [(bits(inp["target"][b, : int(budgets[b]) + 1]), bits(inp["draft"][b, : int(budgets[b])]))
            for b in range(n_requests)]
    verified = 0
    passes = 0
    t0 = time.perf_counter()
    for seed in seeds:
        for b in range(n_requests):
            kb = int(budgets[b])
            zt = ov.decode_bf16(rows[b][0])
            zd = ov.decode_bf16(rows[b][1])
            ov.verify_request(b, zt, zd, tokens[b, :kb], T, seed)
            verified += kb
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or dt >= max_seconds:
            break
    dt = time.perf_counter() - t0
    return verified / dt, dt, passes


# ------------------------------------------------------- oracle on a pool ---

def cpu_workers():
    """Worker processes for the oracle pool: the host cores this process may
    run on, at most 16 (the CPU share of one GPU on the benchmark hosts)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


_WORKER_MAPS = {}


def _worker_array(path, shape, dtype):
    import numpy as np
    key = (path, tuple(shape), dtype)
    if key not in _WORKER_MAPS:
        _WORKER_MAPS[key] = np.memmap(path, dtype=dtype, mode="r", shape=tuple(shape))
    return _WORKER_MAPS[key]


def _oracle_task(args):
    """Pool worker: the oracle on requests [b0, b1) of a stored batch."""
    desc, T, seed, b0, b1 = args
    from oracle import verify as ov
    target = _worker_array(*desc["target"])
    draft = _worker_array(*desc["draft"]) if desc["draft"] else None
    tokens = _worker_array(*desc["tokens"])
    budgets = _worker_array(*desc["budgets"])
    fmt = desc["fmt"]
    out = []
    for b in range(b0, b1):
        k = int(budgets[b])
        zt = ov.as_f64_rows(target[b, : k + 1], fmt)
        zd = ov.as_f64_rows(draft[b, :k], fmt) if T > 0 else None
        out.append(ov.verify_request(b, zt, zd, tokens[b, :k], T, seed))
    return out


class OraclePool:
    """The fp64 oracle, unchanged, run over the requests of a batch on a pool
    of worker processes. The pool is forked before this process touches the
    GPU; batches reach the workers as files they map read-only (the exact
    bytes the GPU was given), so nothing large is pickled."""

    def __init__(self, workers):
        import multiprocessing as mp
        import tempfile
        self.workers = workers
        self.pool = mp.get_context("fork").Pool(workers)
        self.dir = tempfile.mkdtemp(prefix="sv_oracle_")
        self.files = []

    def _store(self, name, arr):
        import numpy as np
        path = os.path.join(self.dir, name)
        mm = np.memmap(path, dtype=arr.dtype, mode="w+", shape=arr.shape)
        mm[...] = arr
        mm.flush()
        del mm
        self.files.append(path)
        return (path, arr.shape, arr.dtype.str)

    def store(self, name, inp):
        """Copy a batch's tensors to the host files the workers read."""
        import numpy as np
        import torch

        def host(x):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy().view(np.uint16), "bf16"
            return x.numpy(), "f32"
        t, fmt = host(inp["target"])
        d, _ = host(inp["draft"])
        return {"target": self._store(name + ".t", t), "draft": self._store(name + ".d", d),
                "tokens": self._store(name + ".x", inp["tokens"].cpu().numpy()),
                "budgets": self._store(name + ".k", inp["budgets"].cpu().numpy()),
                "fmt": fmt, "B": int(t.shape[0])}

    def step(self, desc, T, seed):
        """One verify step of the oracle over every request: (decisions in
        request order, wall seconds)."""
        B = desc["B"]
        parts = max(1, min(B, 4 * self.workers))
        cuts = [B * i // parts for i in range(parts + 1)]
        tasks = [(desc, T, seed, cuts[i], cuts[i + 1]) for i in range(parts) if cuts[i] < cuts[i + 1]]
        t0 = time.perf_counter()
        res = self.pool.map(_oracle_task, tasks)
        dt = time.perf_counter() - t0
        return [d for part in res for d in part], dt

    def close(self):
        self.pool.terminate()
        self.pool.join()
        for f in self.files:
            try:
                os.remove(f)
            except OSError:
                pass
        try:
            os.rmdir(self.dir)
        except OSError:
            pass


def near_ties_on_step(inp, decisions, gpu_out, T):
    """The bench step's outputs against the oracle's decisions under the
    parity bar (tests/helpers.py): excused near-ties, unexcused mismatches,
    the smallest residual mass, and the largest relative error of p(x), q(x)."""
    import numpy as np
    from tests.helpers import PROB_FLOOR, compare_sampled, logits_mass_fn
    toks, nacc, p, q = (x.cpu().numpy() for x in gpu_out)
    budgets = inp["budgets"].cpu().numpy()
    reqs = np.arange(len(budgets))
    mass_fn = logits_mass_fn(inp["target"], inp["draft"], budgets, reqs, decisions, T)
    cmp = compare_sampled(toks, nacc, decisions, inp["tokens"].shape[1],
                          inp["tokens"].cpu().numpy(), mass_fn)
    worst = 0.0
    for n, d in enumerate(decisions):
        for i, (po, qo) in enumerate(zip(d.p_x, d.q_x)):
            for g, o in ((p[n, i], po), (q[n, i], qo)):
                if o >= PROB_FLOOR:
                    worst = max(worst, abs(float(g) - o) / o)
    return {"requests": cmp.requests,
            "excused_accept": sum(1 for e in cmp.excused if e[1] == "accept"),
            "excused_sample": sum(1 for e in cmp.excused if e[1] == "sample"),
            "unexcused": len(cmp.unexcused),
            "min_residual_R": cmp.min_residual_R,
            "max_rel_err_p_q": worst,
            "band": 1e-6}


def bench_scheduler(B, K, steps, seed=5):
    """The verify-budget scheduler on the workload's batch shape: per-position
    confidences for B requests and K drafted positions, a batch verify budget
    of 4 positions per request (the heavy batch's mean), tau = 0. Per-call
    durations from HIP events around each launch; the oracle timed beside it
    on the same confidences."""
    import torch
    from draft_verify_sampling_spec_amd import schedule_budgets
    from workloads import make_confidences
    conf_cpu = make_confidences(B, K, seed)
    conf = conf_cpu.to("cuda")
    out = torch.empty(B, dtype=torch.int32, device="cuda")
    n_total = 4 * B
    for _ in range(20):
        schedule_budgets(conf, n_total, 0.0, out=out)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record()
        schedule_budgets(conf, n_total, 0.0, out=out)
        b.record()
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    from oracle import schedule as osch
    t0 = time.perf_counter()
    reps = 0
    while True:
        want = osch.schedule(conf_cpu.numpy(), n_total, 0.0)
        reps += 1
        if time.perf_counter() - t0 > 1.0:
            break
    cpu_us = (time.perf_counter() - t0) / reps * 1e6
    same = out.cpu().numpy().tolist() == want.tolist()
    return {
        "config": f"B={B} K={K} N={n_total} tau=0, synthetic sigmoid confidences (chat and math/code halves)",
        "us_per_call": {"mean": sum(us) / len(us), "median": us[len(us) // 2],
                        "p5": us[int(0.05 * (len(us) - 1))], "p95": us[int(0.95 * (len(us) - 1))]},
        "calls": steps,
        "bound": "latency",
        "bytes_per_call": 4 * B * K + 4 * B,
        "budgets_match_oracle": same,
        "cpu_oracle_us_per_call": cpu_us,
        "cpu_oracle_cores": 1,
    }


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak


def warm_up(fn, min_s=0.25, min_calls=3):
    """Untimed calls until the clocks have settled under the load: at least
    `min_calls`, and at least `min_s` seconds of work."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while n < min_calls or time.perf_counter() - t0 < min_s:
        fn(n)
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def bench_head(R, H, V, steps, T=1.0, seed=5):
    """The shared output head with its statistics epilogue on the verify
    batch's rows (target and drafter positions), synthetic bf16 hidden states
    and head. Per-call durations from HIP events; the dense-MFMA roofline in
    TFLOP/s; the oracle timed beside it on a few rows, scaled to the call."""
    import numpy as np
    import torch
    from draft_verify_sampling_spec_amd import head_stats
    from workloads import make_head_inputs
    h, w, tok = make_head_inputs(R, H, V, seed)
    warm_up(lambda n: head_stats(h, w, tok, T))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record()
        head_stats(h, w, tok, T)
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    mean_ms = sum(ms) / len(ms)
    flops = 2.0 * R * H * V
    achieved = flops / (mean_ms * 1e-3) / 1e12
    from oracle import head as oh
    rows = 2
    hb = h[:rows].cpu().view(torch.int16).numpy().view(np.uint16)
    wb = w.cpu().view(torch.int16).numpy().view(np.uint16)
    t0 = time.perf_counter()
    h64 = oh.bf16_bits_to_f64(hb)
    for v0 in range(0, V, 16384):
        oh.logits(h64, oh.bf16_bits_to_f64(wb[v0:v0 + 16384]))
    cpu_s = (time.perf_counter() - t0) / rows * R
    return {
        "config": f"R={R} rows (target + drafter positions) H={H} V={V} bf16, T={T}",
        "ms_per_call": {"mean": mean_ms, "median": ms[len(ms) // 2],
                        "p5": ms[int(0.05 * (len(ms) - 1))], "p95": ms[int(0.95 * (len(ms) - 1))]},
        "calls": steps,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                     "flops_per_call": flops},
        "cpu_oracle_s_per_call": cpu_s,
        "cpu_oracle_sample": f"fp64 NumPy logits of {rows} rows, scaled to {R} rows",
    }


def bench_hidden(B, K, H, V, steps, T=1.0, seed=5):
    """A whole verify step from hidden states through the shared head at the
    verify batch's shape (budgets 2 + Binomial(6, 1/3)): plan, the head
    product with the statistics epilogue over every budgeted row, decide,
    the head product again over each request's paired draw rows (its
    epilogue leaves per-block draw masses, no logits), and the inverse-CDF
    draw. Per-call durations from HIP events. The matrix
    work is 2 H V flops per scored row plus per draw row; its rate over the
    whole call is a lower bound on the product kernels' own rate. The oracle
    is timed on one request and scaled to the batch."""
    import numpy as np
    import torch
    from draft_verify_sampling_spec_amd import HiddenVerify
    from workloads import make_hidden_inputs, philox_seed
    inp = make_hidden_inputs(B, K, H, V, seed, device="cuda:0", variant="heavy", temperature=T)
    hv = HiddenVerify("cuda:0", B, K, V)
    args = (inp["target_hidden"], inp["draft_hidden"], inp["head"], inp["tokens"], inp["budgets"], T)
    warm_up(lambda n: hv.run(*args, philox_seed(WORKLOAD_INDEX["heavy"], 3_000_000 + n)))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    outs = []
    for i, (a, b) in enumerate(ev):
        a.record()
        outs.append(hv.run(*args, philox_seed(WORKLOAD_INDEX["heavy"], 3_100_000 + i)))
        b.record()
    torch.cuda.synchronize()
    if any(int(o[4].item()) != 0 for o in outs):
        raise RuntimeError("spec_verify_hidden set device status flags")
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    mean_ms = sum(ms) / len(ms)
    budgets = inp["budgets"].cpu().numpy()
    scored = int(np.sum(2 * budgets + 1))
    n_acc = outs[-1][1].cpu().numpy()
    draw_rows = int(np.sum(np.where(n_acc < budgets, 2, 1)))
    flops = 2.0 * (scored + draw_rows) * H * V
    achieved = flops / (mean_ms * 1e-3) / 1e12
    from oracle import hidden as ohid

    def bits(x):
        return x.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    th, dh, w = bits(inp["target_hidden"][:1]), bits(inp["draft_hidden"][:1]), bits(inp["head"])
    t0 = time.perf_counter()
    ohid.verify_from_hidden(th, dh, w, inp["tokens"][:1].cpu().numpy(), budgets[:1], T,
                            philox_seed(WORKLOAD_INDEX["heavy"], 3_100_000))
    cpu_s = (time.perf_counter() - t0) * B
    verified = int(budgets.sum())
    return {
        "config": f"B={B} K={K} H={H} V={V} bf16 hidden states and head, budgets 2..8 "
                  f"(mean 4), T={T}; {scored} scored rows, {draw_rows} draw rows (last call)",
        "ms_per_call": {"mean": mean_ms, "median": ms[len(ms) // 2],
                        "p5": ms[int(0.05 * (len(ms) - 1))], "p95": ms[int(0.95 * (len(ms) - 1))]},
        "calls": steps,
        "verified_draft_tokens_per_s": verified / (mean_ms * 1e-3),
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                     "flops_per_call": flops, "note": "whole call, all five launches"},
        "cpu_oracle_s_per_call": cpu_s,
        "cpu_oracle_sample": f"fp64 oracle on request 0 ({int(budgets[0])} drafted), scaled to {B} requests",
    }


def bench_markov(B, K, V, r, steps, seed=5):
    """The drafter's low-rank Markov head over a drafted block at the verify
    batch's shape: K positions in order, each the rank-r transition product
    of the previous tokens plus the backbone row, stored as bf16, with the
    first argmax drafted. Per-call durations from HIP events. Algorithmic HBM
    bytes per call: backbone logits read and drafter logits written once
    (B K V bf16 each), the vocabulary factor read once per position (V r
    bf16), the previous tokens' rows of the other factor. The argmax follows
    the stored values inside the product's epilogue, so no row is read back
    (only the 32 columns of each request's best tile); each group of 256
    requests after the first may read the vocabulary factor again where the
    L2 has not kept it, which is implementation traffic (counted in full
    below, as an upper bound). Untimed calls first bring the clocks to their
    sustained state. The oracle is timed on one request's block and
    scaled to the batch."""
    import numpy as np
    import torch
    from draft_verify_sampling_spec_amd import MarkovDraft
    from workloads import make_markov_inputs
    inp = make_markov_inputs(B, K, V, r, seed, device="cuda:0")
    md = MarkovDraft("cuda:0", B, K, V)
    out_z = torch.empty((B, K, V), dtype=torch.bfloat16, device="cuda:0")
    out_x = torch.empty((B, K), dtype=torch.int32, device="cuda:0")
    args = (inp["base"], inp["markov_a"], inp["markov_b"], inp["prev"])
    warm_up(lambda n: md.run(*args, out_logits=out_z, out_tokens=out_x), min_calls=10)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record()
        _, _, st = md.run(*args, out_logits=out_z, out_tokens=out_x)
        b.record()
    torch.cuda.synchronize()
    if int(st.item()) != 0:
        raise RuntimeError("spec_markov_draft set device status flags")
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    mean_ms = sum(ms) / len(ms)
    alg = 2 * (2 * B * K * V) + K * (2 * V * r + 2 * B * r) + 4 * B + 4 * B * K
    groups = 1
    while groups * 256 < B:
        groups *= 2
    impl_extra = K * (groups - 1) * 2 * V * r
    achieved = alg / (mean_ms * 1e-3) / 1e9
    from oracle import markov as om

    def vals(t):
        return om.bf16_bits_to_f64(t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16))
    A, Bm = vals(inp["markov_a"]), vals(inp["markov_b"])
    base0 = vals(inp["base"][:1])
    t0 = time.perf_counter()
    om.draft_block(base0, A, Bm, inp["prev"][:1].cpu().numpy())
    cpu_s = (time.perf_counter() - t0) * B
    return {
        "config": f"B={B} K={K} V={V} r={r} bf16 backbone logits and factors",
        "ms_per_call": {"mean": mean_ms, "median": ms[len(ms) // 2],
                        "p5": ms[int(0.05 * (len(ms) - 1))], "p95": ms[int(0.95 * (len(ms) - 1))]},
        "calls": steps,
        "drafted_tokens_per_s": B * K / (mean_ms * 1e-3),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "algorithmic_bytes_per_call": alg,
                     "implementation_factor_rereads_bytes_per_call": impl_extra,
                     "note": "whole call, K + 2 launches"},
        "cpu_oracle_s_per_call": cpu_s,
        "cpu_oracle_sample": f"fp64 oracle on request 0's block of {K} positions, scaled to {B} requests",
    }


def bench_workloads(steps=50, settle_s=0.1):
    """The other synthetic workloads at one GPU, each verified back to back
    with a fresh Philox seed per step: the Qwen3-4B-shaped batch (fp32) at
    T = 0 and T = 1, the ragged moderate-load batch and the Gemma-shaped
    vocabulary (bf16). Distinct input sets (other data seeds) rotate from
    step to step, more than 512 MB in all, so no step finds its logits in the
    last-level cache. Per workload: step time (HIP events around each step),
    verified draft tokens/s, the path's algorithmic GB/s, and the streaming
    pass's roofline from the library's per-pass events."""
    import torch
    from draft_verify_sampling_spec_amd import SpecVerify
    from workloads import make_inputs, philox_seed
    dev = torch.device("cuda:0")
    out = {}
    for name, T_over, nsets in (("qwen3", 0.0, 12), ("qwen3", 1.0, 12), ("ragged", None, 3),
                                ("gemma", None, 2)):
        widx = WORKLOAD_INDEX[name]
        sets = [make_inputs(name, device=dev, seed=100 * widx + j) for j in range(nsets)]
        T = sets[0]["temperature"] if T_over is None else T_over
        greedy = T == 0.0
        B, K1, V = sets[0]["target"].shape
        K = K1 - 1
        elem = sets[0]["target"].element_size()
        sv = SpecVerify(dev, max_batch=B, max_k=K, vocab=V, dtype=sets[0]["target"].dtype)
        out_t = torch.empty(B, K + 1, dtype=torch.int32, device=dev)
        out_n = torch.empty(B, dtype=torch.int32, device=dev)
        args = [(x["target"], None if greedy else x["draft"], x["tokens"], x["budgets"]) for x in sets]
        alg = [algorithmic_bytes(x["budgets"].cpu().tolist(), K, V, elem, greedy)[0] for x in sets]
        ver = [int(x["budgets"].sum().item()) for x in sets]
        n = 0
        t0 = time.perf_counter()
        while n < 20 or time.perf_counter() - t0 < settle_s:
            a = args[n % nsets]
            sv.run(a[0], a[1], a[2], a[3], T, philox_seed(widx, n), out_t, out_n, want_probs=False)
            n += 1
            if n % 16 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        stream = torch.cuda.current_stream(dev)
        for s_, (e0, e1) in enumerate(ev):
            a = args[s_ % nsets]
            e0.record(stream)
            sv.run(a[0], a[1], a[2], a[3], T, philox_seed(widx, 1_000_000 + s_), out_t, out_n,
                   want_probs=False)
            e1.record(stream)
        torch.cuda.synchronize()
        sv.timing(True)
        for s_ in range(steps):
            a = args[s_ % nsets]
            sv.run(a[0], a[1], a[2], a[3], T, philox_seed(widx, 2_000_000 + s_), out_t, out_n,
                   want_probs=False)
        counts, pass_ms = sv.pass_times()
        sv.timing(False)
        if sv.status() != 0:
            raise RuntimeError(f"device status flags set on workload {name}")
        ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
        mean_ms = sum(ms) / len(ms)
        mean_alg = sum(alg[s_ % nsets] for s_ in range(steps)) / steps
        mean_ver = sum(ver[s_ % nsets] for s_ in range(steps)) / steps
        stream_ms = pass_ms[0] / max(counts[0], 1)
        sv.close()
        out[f"{name} T={T:g}"] = {
            "config": sets[0]["workload"].summary,
            "input_sets": nsets,
            "ms_per_step": {"mean": mean_ms, "median": ms[len(ms) // 2],
                            "p5": ms[int(0.05 * (len(ms) - 1))], "p95": ms[int(0.95 * (len(ms) - 1))]},
            "verified_draft_tokens_per_s": mean_ver / (mean_ms * 1e-3),
            "algorithmic_bytes_per_step": mean_alg,
            "path_gbs": mean_alg / (mean_ms * 1e-3) / 1e9,
            "stream_pass_ms": stream_ms,
            "stream_pass_frac_of_peak": mean_alg / (stream_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        }
        del sets, args
        torch.cuda.empty_cache()
    return out


def read_ceiling(t, d, reps=10):
    """Context: a plain read-only streaming reduction (torch's sum in fp32)
    over the same logit buffers, whole tensors, as the achievable read rate."""
    import torch
    for _ in range(2):
        t.sum(dtype=torch.float32)
        d.sum(dtype=torch.float32)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        t.sum(dtype=torch.float32)
        d.sum(dtype=torch.float32)
    b.record()
    torch.cuda.synchronize()
    nbytes = (t.numel() * t.element_size() + d.numel() * d.element_size()) * reps
    return {"gbs": nbytes / (a.elapsed_time(b) * 1e-3) / 1e9, "bytes_per_pass": nbytes // reps,
            "kernel": "torch sum (fp32 accumulation) over the target and drafter logits"}


def copy_probe(gib):
    import torch
    n = int(gib * (1 << 30))
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 5}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warmup-settle", type=float, default=WARMUP_SETTLE_S,
                    help="minimum seconds of warmup (0: exactly --warmup steps)")
    ap.add_argument("--workload", default="heavy", choices=sorted(WORKLOAD_INDEX))
    ap.add_argument("--temperature", type=float, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--verify-only", action="store_true",
                    help="time the verify step only (no scheduler, head or hidden-state legs)")
    ap.add_argument("--cpu-requests", type=int, default=512)
    ap.add_argument("--copy-probe", type=float, default=None)
    ap.add_argument("--markov-only", action="store_true",
                    help="time only the Markov head over a heavy-shape block (3 calls)")
    ap.add_argument("--head-only", action="store_true",
                    help="time only the output head at the heavy rows (3 calls per temperature)")
    ap.add_argument("--hidden-only", action="store_true",
                    help="time only the verify step from hidden states (3 calls)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    # The oracle's worker pool is forked here, before this process touches
    # the GPU (torch is not imported yet).
    pool = None
    want_cpu = (not args.no_cpu_baseline and args.workload == "heavy" and args.copy_probe is None
                and not (args.markov_only or args.head_only or args.hidden_only))
    if want_cpu:
        pool = OraclePool(cpu_workers())
    try:
        run(args, pool)
    finally:
        if pool is not None:
            pool.close()


def run(args, pool):
    import torch
    from draft_verify_sampling_spec_amd import SpecVerify
    from workloads import make_inputs, philox_seed

    if args.copy_probe is not None:
        copy_probe(args.copy_probe)
        return
    if args.markov_only:
        print(json.dumps({"markov": bench_markov(512, 8, 151936, 256, 3)}), flush=True)
        return
    if args.head_only:
        out = {f"T={T}": bench_head(4592, 2560, 151936, 3, T=T) for T in (1.0, 0.0)}
        print(json.dumps({"head": out}), flush=True)
        return
    if args.hidden_only:
        print(json.dumps({"hidden": bench_hidden(512, 8, 2560, 151936, 3)}), flush=True)
        return

    dev = torch.device("cuda:0")
    log(f"[bench] drawing workload {args.workload} on {torch.cuda.get_device_name(dev)}")
    inp = make_inputs(args.workload, device=dev)
    w = inp["workload"]
    T = inp["temperature"] if args.temperature is None else args.temperature
    greedy = T == 0.0
    t, x, k = inp["target"], inp["tokens"], inp["budgets"]
    d = inp["draft"] if not greedy else None
    B, K1, V = t.shape
    K = K1 - 1
    elem = t.element_size()
    sv = SpecVerify(dev, max_batch=B, max_k=K, vocab=V, dtype=t.dtype)
    out_t = torch.empty(B, K + 1, dtype=torch.int32, device=dev)
    out_n = torch.empty(B, dtype=torch.int32, device=dev)
    widx = WORKLOAD_INDEX[args.workload]

    budgets = k.cpu().tolist()
    alg_bytes, rows = algorithmic_bytes(budgets, K, V, elem, greedy)
    verified_per_step = int(sum(budgets))

    # Everything the timed regions use is set up before the warmup, so that
    # the first timed step follows the last warmup step with no idle gap.
    stream = torch.cuda.current_stream(dev)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for e in starts + ends:
        e.record(stream)
    accepted = torch.zeros((), dtype=torch.int64, device=dev)
    acc_sum = torch.zeros((), dtype=torch.int64, device=dev)
    torch.cuda.synchronize()

    # Warmup: W steps, continued (untimed) until the GPU has been busy for
    # WARMUP_SETTLE_S -- its clocks ramp over the first tens of milliseconds
    # of sustained load, and a short warmup would time the ramp.
    log(f"[bench] warmup {args.warmup} steps (at least {args.warmup_settle} s)")
    warm_steps = 0
    w0 = time.perf_counter()
    while warm_steps < args.warmup or time.perf_counter() - w0 < args.warmup_settle:
        sv.run(t, d, x, k, T, philox_seed(widx, warm_steps), out_t, out_n, want_probs=False)
        warm_steps += 1
        if warm_steps % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    # The timed steps: nothing but the verify calls between the two
    # synchronisations (wall clock).
    t0 = time.perf_counter()
    for s in range(args.steps):
        sv.run(t, d, x, k, T, philox_seed(widx, 1_000_000 + s), out_t, out_n,
               want_probs=False)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    accepted += out_n.sum()
    # The same steps again with a HIP event pair around each, for the
    # per-step distribution (the event packets add a little time per step).
    log(f"[bench] timing {args.steps} steps with per-step events")
    for s in range(args.steps):
        starts[s].record(stream)
        sv.run(t, d, x, k, T, philox_seed(widx, 1_000_000 + s), out_t, out_n,
               want_probs=False)
        ends[s].record(stream)
    torch.cuda.synchronize()
    # Third timed region, same steps: per-pass HIP events that the library
    # records on this stream around each launch (pass 0: the streaming pass,
    # the dominant kernel; pass 1: the draw pass). Kept apart from the regions
    # above because the event markers add a little time between the passes.
    log(f"[bench] timing {args.steps} steps per pass")
    sv.timing(True)
    for s in range(args.steps):
        sv.run(t, d, x, k, T, philox_seed(widx, 1_000_000 + s), out_t, out_n,
               want_probs=False)
        acc_sum += out_n.sum()
    pass_counts, pass_ms = sv.pass_times()
    accepted_per_step = float(acc_sum.item()) / args.steps
    sv.timing(False)
    kernel_ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    kernel_ms.sort()
    mean_kernel_ms = sum(kernel_ms) / len(kernel_ms)
    ms_per_step = elapsed * 1e3 / args.steps
    if sv.status() != 0:
        log("[bench] device status flags set")
        sys.exit(1)

    path_gbs = alg_bytes / (mean_kernel_ms * 1e-3) / 1e9
    stream_ms = pass_ms[0] / max(pass_counts[0], 1)
    draw_ms = pass_ms[1] / pass_counts[1] if pass_counts[1] else 0.0
    call_ms = stream_ms + draw_ms
    # Roofline of the whole call (streaming pass + draw pass): the
    # algorithmic bytes are read once by the streaming pass; the draw pass
    # re-reads each first-rejected row pair, which is implementation cost.
    achieved = alg_bytes / (call_ms * 1e-3) / 1e9
    stream_achieved = alg_bytes / (stream_ms * 1e-3) / 1e9
    traffic = load_traffic()
    result = {
        "metric": "verified draft tokens/s + achieved HBM GB/s (% peak), B=512 V=151936 bf16",
        "value": verified_per_step / (ms_per_step * 1e-3),
        "unit": "verified draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warm_steps,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if elem == 2 else "f32",
        "data": "synthetic (seeded; see workloads/)",
        "config": {
            "workload": f"{w.name}: {w.summary}",
            "B": B, "K": K, "V": V, "temperature": T,
            "verified_draft_tokens_per_step": verified_per_step,
            "logit_rows_per_step": rows,
            "accepted_last_step": int(accepted.item()),
            "accepted_per_step_mean": accepted_per_step,
        },
        "accepted_draft_tokens_per_s": accepted_per_step / (ms_per_step * 1e-3),
        "emitted_tokens_per_s": (accepted_per_step + B) / (ms_per_step * 1e-3),
        "hbm_gbs": path_gbs,
        "hbm_frac_of_peak": path_gbs / HBM_PEAK_GBS,
        "kernel_ms": {"mean": mean_kernel_ms, "median": kernel_ms[len(kernel_ms) // 2],
                      "p5": kernel_ms[int(0.05 * (len(kernel_ms) - 1))],
                      "p95": kernel_ms[int(0.95 * (len(kernel_ms) - 1))]},
        "pass_ms": {"stream": stream_ms, "draw": draw_ms if pass_counts[1] else None,
                    "launches": pass_counts},
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic["call"] if traffic else None,
            "algorithmic_bytes_per_launch": alg_bytes,
            "kernel": ("verify call: verify_kernel (streaming pass) + draw_kernel (draw pass)"
                       if not greedy else "verify call: verify_kernel (greedy, one pass)"),
            "streaming_pass": {"kernel": "verify_kernel", "ms": stream_ms,
                               "achieved": stream_achieved,
                               "frac": stream_achieved / HBM_PEAK_GBS,
                               "traffic": traffic["stream"] if traffic else None},
            "draw_pass": None if greedy else {
                "kernel": "draw_kernel", "ms": draw_ms,
                "traffic": traffic["draw"] if traffic else None,
                "note": "re-reads each first-rejected row pair (implementation bytes)"},
        },
        "cpu_baseline": None,
    }
    if pool is not None and not greedy:
        s0 = philox_seed(widx, 1_000_000)
        gpu_out = sv.run(t, d, x, k, T, s0)
        torch.cuda.synchronize()
        log(f"[bench] oracle pool ({pool.workers} processes): heavy step")
        desc = pool.store("heavy", inp)
        decisions, dt0 = pool.step(desc, T, s0)
        result["near_ties"] = near_ties_on_step(inp, decisions, gpu_out, T)
        result["near_ties"]["seed"] = s0
        if result["near_ties"]["unexcused"]:
            log(f"[bench] PARITY: {result['near_ties']['unexcused']} unexcused mismatches")
        heavy_s = [dt0] + [pool.step(desc, T, philox_seed(widx, 1_000_001 + i))[1]
                           for i in range(2)]
        cpu = {"heavy": sum(heavy_s) / len(heavy_s)}
        for name in ("qwen3", "ragged", "gemma"):
            other = make_inputs(name, device=dev)
            cpu[name] = pool.step(pool.store(name, other), other["temperature"],
                                  philox_seed(WORKLOAD_INDEX[name], 5))[1]
            del other
            torch.cuda.empty_cache()
        single_rate, single_s, single_passes = cpu_baseline(
            inp, [philox_seed(widx, 2_000_000 + i) for i in range(64)], min(args.cpu_requests, B))
        result["cpu_baseline"] = {
            "value": verified_per_step / cpu["heavy"], "unit": "verified draft tokens/s",
            "cores": pool.workers, "kind": "oracle",
            "sample": f"the whole heavy step ({B} requests) on {pool.workers} worker processes, "
                      f"mean of 3 steps with fresh seeds; one step of each other workload",
            "s_per_step": cpu,
            "single_process": {"value": single_rate, "cores": 1,
                               "sample": f"{single_passes} passes over the first "
                                         f"{min(args.cpu_requests, B)} requests "
                                         f"({single_s:.1f} s)"},
        }
    if not greedy and not args.verify_only:
        log("[bench] budget scheduler")
        result["scheduler"] = bench_scheduler(B, K, args.steps)
        if args.workload == "heavy":
            # One hidden state per scored row (the step's budgeted target and
            # drafter rows), Qwen3-4B's hidden size.
            log("[bench] output head")
            result["head"] = bench_head(rows, 2560, V, min(args.steps, 10))
            log("[bench] verify from hidden states")
            result["hidden"] = bench_hidden(B, K, 2560, V, min(args.steps, 10), T)
            log("[bench] Markov head draft")
            result["markov"] = bench_markov(B, K, V, 256, min(args.steps, 10))
    if not greedy and not args.verify_only and args.workload == "heavy":
        log("[bench] read ceiling")
        result["read_ceiling"] = read_ceiling(t, d)
        log("[bench] other workloads")
        result["workloads"] = bench_workloads()
    print(json.dumps(result), flush=True)
    sv.close()


if __name__ == "__main__":
    main()
