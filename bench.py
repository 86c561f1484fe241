#!/usr/bin/env python3
"""Benchmark of the gfx950 fused dequantise-and-dot GEMV and MoE FFN.

Prints ONE JSON line.  The headline workload is the Q4_K 4096 x 4096 GEMV at
batch 1; a step is one qgemv over that matrix.  The other workloads (Q8_0
256 x 1024, the Q6_K 151936 x 2048 lm_head, the Q5_K / Q4_0 batch sweep,
batches above 8, the int8-activation variant, the Qwen3-30B-A3B-shaped MoE
FFN, and the plain streaming read that bounds every batch-1 GEMV) are
measured in the same run and reported under "workloads".

Cold weights: consecutive launches read different copies of the weights
(the copies of a workload cover at least 1 GiB, four times the 256 MB
Infinity Cache), and right before every timed replay a 1 GiB device copy
(1 GiB read, 1 GiB written) scrubs the Infinity Cache and the L2s, so every
timed launch streams its weights from HBM whatever the step count: a copy
is read again only after at least 1 GiB of other traffic.  Inputs are
resident in HBM before the timed region starts.

Timing: the K launches of a workload are captured in one HIP graph (the
host cannot issue launches as fast as the kernels run).  Untimed replays
come first, for at least --warm-seconds: under sustained load the GPU takes
a while to reach its steady clocks.  Then the scrub, then the timed region:
one replay of that graph, bracketed by torch.cuda.synchronize().  Its wall
time gives the whole-job rate (`value`), and a HIP event pair recorded on
the replay stream gives the average launch duration behind `roofline`.
The rocprofv3 kernel-trace mean of the same kernel, from the committed
summary under profiles/ (when it was taken on these kernel sources), is
printed beside it.  `cpu_baseline` times the C oracle on a bounded sample
of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
COLD_BYTES = 1 << 30       # weight copies per workload cover at least 1 GiB


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=2, help="untimed graph replays")
    ap.add_argument("--warm-seconds", type=float, default=0.3,
                    help="keep replaying untimed until this long has passed (clocks and power "
                         "management settle under sustained load)")
    ap.add_argument("--quick", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--moe-tokens", type=int, default=256)
    ap.add_argument("--only", default="", help="comma list of workload names (profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run plain device copies of 256 MiB (scale for the HBM byte "
                         "counters under rocprofv3 --pmc)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "q4_k_4096x4096_b1_hbm_traffic.md")
TRACE_FILE = os.path.join(ROOT, "profiles", "q4_k_4096x4096_b1_kernel_trace.md")
CSRC = os.path.join(ROOT, "gguf_quant_dequant_amd", "csrc")


def source_digest():
    """sha256 over the kernel sources (every file under csrc/, in name
    order), to tell whether counters taken on an earlier build still
    describe this one."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(CSRC, "*"))):
        if f.endswith((".hip", ".hpp")):
            with open(f, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def _summary_fields(path):
    """The '- key: value' lines of a committed profile summary."""
    try:
        with open(path) as fh:
            text = fh.read()
    except OSError:
        return {}
    fields = {}
    for line in text.splitlines():
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].split(": ", 1)
            fields[k.strip()] = v.strip().strip("`")
    return fields


def measured_trace_us():
    """Mean kernel-trace duration (us) of the headline kernel over the timed
    replay, from the committed rocprofv3 summary; None when missing or taken
    on other kernel sources."""
    f = _summary_fields(TRACE_FILE)
    if f.get("kernel sources sha256") != source_digest():
        return None
    try:
        return float(f["trace mean dispatch us, timed replay"])
    except (KeyError, ValueError):
        return None


def measured_traffic():
    """HBM bytes per launch of the headline kernel from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, each scaled by what the counter reads
    for a copy of known size); None when the summary is missing or was taken
    on other kernel sources."""
    f = _summary_fields(TRAFFIC_FILE)
    if f.get("kernel sources sha256") != source_digest():
        return None
    try:
        return int(f["HBM bytes per launch"])
    except (KeyError, ValueError):
        return None


class Gemv:
    """A GEMV workload with enough device copies of W to stay cold."""

    def __init__(self, case, batch, torch, q, q8act=False, ws=False):
        import synth
        self.case, self.batch, self.q, self.torch = case, batch, q, torch
        W, X = synth.gemv_inputs(case, batch)
        self.wbytes = W.nbytes
        ncopy = max(2, -(-COLD_BYTES // self.wbytes))
        first = torch.from_numpy(W.reshape(-1)).cuda()
        self.copies = [first] + [first.clone() for _ in range(ncopy - 1)]
        self.X = torch.from_numpy(X).cuda()
        self.Y = torch.empty(batch, case.rows, device="cuda")
        self.i = 0
        self.q8act = q8act
        # qgemv_ws: the caller-provided workspace, allocated once
        self.ws = None
        if ws:
            need = q.qgemv_ws_bytes(case.fmt, case.rows, case.cols, batch)
            self.ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        self.use_ws = ws

    def launch(self):
        W = self.copies[self.i % len(self.copies)]
        self.i += 1
        if self.q8act:
            self.q.qgemv_q8act(self.case.fmt, W, self.case.rows, self.case.cols, self.X, self.Y)
        elif self.use_ws:
            self.q.qgemv_ws(self.case.fmt, W, self.case.rows, self.case.cols, self.X, self.Y,
                            self.batch, self.ws)
        else:
            self.q.qgemv(self.case.fmt, W, self.case.rows, self.case.cols, self.X, self.Y,
                         self.batch)


class Stream:
    """The plain streaming read of `nbytes` (qg_stream_read) over rotating
    cold copies: the floor of any kernel that must read that many bytes."""

    def __init__(self, nbytes, torch, q, grid=0):
        self.q, self.torch, self.grid = q, torch, grid
        self.wbytes = nbytes
        ncopy = max(2, -(-COLD_BYTES // nbytes))
        first = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device="cuda")
        self.copies = [first] + [first.clone() for _ in range(ncopy - 1)]
        self.out = torch.empty(4096, dtype=torch.int32, device="cuda")
        self.i = 0

    def launch(self):
        W = self.copies[self.i % len(self.copies)]
        self.i += 1
        self.q.qg_stream_read(W, self.wbytes, self.out, self.grid)


class Moe:
    """The MoE FFN for one token per call; several device copies of the
    stacked weights (one per emulated layer) keep the expert reads cold."""

    def __init__(self, case, torch, q, tokens):
        import synth
        self.case, self.q, self.torch = case, q, torch
        router, gate, up, down = synth.moe_weights(case)
        per = router.nbytes + gate.nbytes + up.nbytes + down.nbytes
        layers = max(2, -(-4 * COLD_BYTES // per))
        r0 = torch.from_numpy(router).cuda()
        g0 = torch.from_numpy(gate.reshape(-1)).cuda()
        u0 = torch.from_numpy(up.reshape(-1)).cuda()
        d0 = torch.from_numpy(down.reshape(-1)).cuda()
        self.layers = [(r0, g0, u0, d0)] + [(r0.clone(), g0.clone(), u0.clone(), d0.clone())
                                            for _ in range(layers - 1)]
        xs, rs = synth.moe_tokens(case)
        reps = -(-tokens // xs.shape[0])
        self.x = torch.from_numpy(np.tile(xs, (reps, 1))[:tokens]).cuda()
        self.res = torch.from_numpy(np.tile(rs, (reps, 1))[:tokens]).cuda()
        self.y = torch.empty_like(self.x)
        self.sel = torch.empty(tokens, case.top_k, dtype=torch.int32, device="cuda")
        self.w = torch.empty(tokens, case.top_k, device="cuda")
        self.wsb = q.moe_ffn_workspace_bytes(case.n_experts, case.top_k, case.expert_dim)
        self.ws = torch.empty(self.wsb, dtype=torch.uint8, device="cuda")
        self.i = 0
        self.tokens = tokens
        # algorithmic bytes per token: router + k experts' gate, up and down
        c = case
        rb_g = q.qg_row_bytes(c.gate_fmt, c.hidden)
        rb_d = q.qg_row_bytes(c.down_fmt, c.expert_dim)
        self.bytes_per_token = (4 * c.n_experts * c.hidden
                                + c.top_k * (2 * c.expert_dim * rb_g + c.hidden * rb_d))

    def launch(self):
        c = self.case
        t = self.i % self.tokens
        r, g, u, d = self.layers[self.i % len(self.layers)]
        self.i += 1
        self.q.moe_ffn(self.x[t], self.res[t], self.y[t], r, c.gate_fmt, g, c.up_fmt, u,
                       c.down_fmt, d, c.hidden, c.n_experts, c.top_k, c.expert_dim,
                       self.sel[t], self.w[t], self.ws, self.wsb)


class MoeQ8(Moe):
    """moe_ffn_q8act: the same chain with the expert GEMVs on int8 activations."""

    def launch(self):
        c = self.case
        t = self.i % self.tokens
        r, g, u, d = self.layers[self.i % len(self.layers)]
        self.i += 1
        self.q.moe_ffn_q8act(self.x[t], self.res[t], self.y[t], r, c.gate_fmt, g, c.up_fmt, u,
                             c.down_fmt, d, c.hidden, c.n_experts, c.top_k, c.expert_dim,
                             self.sel[t], self.w[t], self.ws, self.wsb)


class MoeNorm(Moe):
    """The MoE FFN behind the fused residual add + RMSNorm (moe_ffn_norm):
    per token its own attention output and hidden state, one norm weight."""

    def __init__(self, case, torch, q, tokens):
        import synth
        super().__init__(case, torch, q, tokens)
        attn, hid, wn = synth.moe_norm_inputs(case)
        reps = -(-tokens // attn.shape[0])
        self.attn = torch.from_numpy(np.tile(attn, (reps, 1))[:tokens]).cuda()
        self.hid = torch.from_numpy(np.tile(hid, (reps, 1))[:tokens]).cuda()
        self.wn = torch.from_numpy(wn).cuda()
        self.eps = float(np.float32(synth.NORM_EPS))
        self.xn = torch.empty_like(self.attn)
        self.wsb = q.moe_ffn_norm_workspace_bytes(case.hidden, case.n_experts, case.top_k,
                                                  case.expert_dim)
        self.ws = torch.empty(self.wsb, dtype=torch.uint8, device="cuda")
        # plus the norm's reads: attention output, hidden state, norm weight
        self.bytes_per_token += 3 * 4 * case.hidden

    def launch(self):
        c = self.case
        t = self.i % self.tokens
        r, g, u, d = self.layers[self.i % len(self.layers)]
        self.i += 1
        self.q.moe_ffn_norm(self.attn[t], self.hid[t], self.y[t], self.wn, self.eps, self.xn[t],
                            r, c.gate_fmt, g, c.up_fmt, u, c.down_fmt, d, c.hidden,
                            c.n_experts, c.top_k, c.expert_dim, self.sel[t], self.w[t],
                            self.ws, self.wsb)


class MoeTokens(Moe):
    """T decode tokens per call through moe_ffn_tokens (each routed on its
    own); the token window rotates over the 64 distinct synthetic tokens."""

    def __init__(self, case, torch, q, tokens, T):
        super().__init__(case, torch, q, tokens)
        self.T = T
        self.sel = torch.empty(tokens + T, case.top_k, dtype=torch.int32, device="cuda")
        self.w = torch.empty(tokens + T, case.top_k, device="cuda")
        self.x = torch.cat([self.x, self.x[:T]])
        self.res = torch.cat([self.res, self.res[:T]])
        self.y = torch.empty_like(self.x)
        self.wsb = q.moe_ffn_tokens_workspace_bytes(T, case.n_experts, case.top_k,
                                                    case.expert_dim)
        self.ws = torch.empty(self.wsb, dtype=torch.uint8, device="cuda")

    def launch(self):
        c = self.case
        t = (self.i * self.T) % self.tokens
        r, g, u, d = self.layers[self.i % len(self.layers)]
        self.i += 1
        T = self.T
        self.q.moe_ffn_tokens(self.x[t:t + T], self.res[t:t + T], self.y[t:t + T], r,
                              c.gate_fmt, g, c.up_fmt, u, c.down_fmt, d, T, c.hidden,
                              c.n_experts, c.top_k, c.expert_dim, self.sel[t:t + T],
                              self.w[t:t + T], self.ws, self.wsb)


class Scrub:
    """A 1 GiB device copy (1 GiB read + 1 GiB written): run right before a
    timed replay, it evicts the 256 MB Infinity Cache and the L2s."""

    def __init__(self, torch):
        self.src = torch.ones(COLD_BYTES, dtype=torch.uint8, device="cuda")
        self.dst = torch.empty_like(self.src)

    def run(self):
        self.dst.copy_(self.src)


def time_launches(torch, work, steps, warmup, warm_seconds=0.0, scrub=None):
    """Capture `steps` back-to-back launches in one HIP graph, replay it
    `warmup` times untimed (and further until `warm_seconds` have passed:
    the GPU reaches its sustained clocks only after some time under load),
    scrub the caches, then time one replay: wall clock between two
    synchronisations and a HIP event pair on the replay stream.  Returns
    (wall seconds, event milliseconds)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            work.launch()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(steps):
            work.launch()
    t_warm = time.perf_counter()
    for _ in range(max(1, warmup)):
        graph.replay()
    torch.cuda.synchronize()
    while time.perf_counter() - t_warm < warm_seconds:
        graph.replay()
        torch.cuda.synchronize()
    if scrub is not None:
        scrub.run()
        torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, e0.elapsed_time(e1)


def host_cpu():
    """(model name from /proc/cpuinfo, logical CPUs usable by this process)."""
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return model, n


def cpu_baseline(seconds):
    """The oracle (single-threaded C) on the headline workload: whole
    Q4_K 4096 x 4096 GEMVs repeated until `seconds` have passed."""
    import oracle
    import synth
    case = synth.GEMV_CASES["q4_k_4096x4096"]
    W, X = synth.gemv_inputs(case, 1)
    oracle.gemv(case.fmt, W[:8], 8, case.cols, X)  # load / warm
    n, t0 = 0, time.perf_counter()
    while True:
        oracle.gemv(case.fmt, W, case.rows, case.cols, X)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    gbs = n * W.nbytes / el / 1e9
    model, ncpu = host_cpu()
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} full Q4_K 4096x4096 batch-1 GEMVs in {el:.1f} s "
                      f"(f64 dequantise-and-dot, one thread)",
            "cpu_model": model, "host_logical_cpus": ncpu}


def cpu_baseline_moe(seconds):
    """The oracle (single-threaded C) on the MoE workload: tokens of the
    Qwen3-30B-A3B-shaped MoE FFN one after another (router, routing, the 8
    experts' gate / up / down, residual) until `seconds` have passed."""
    import oracle
    import synth
    c = synth.MOE_CASE
    router, gate, up, down = synth.moe_weights(c)
    xs, rs = synth.moe_tokens(c)
    n, t0 = 0, time.perf_counter()
    while True:
        t = n % xs.shape[0]
        oracle.moe_ffn(xs[t], rs[t], router, c.gate_fmt, gate, c.up_fmt, up, c.down_fmt, down,
                       c.hidden, c.n_experts, c.top_k, c.expert_dim)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(n / el, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} tokens of the Qwen3-30B-A3B-shaped MoE FFN in {el:.1f} s, one "
                      f"thread ({el / n * 1e3:.1f} ms per token)"}


def _oracle_rows(args):
    import oracle
    import synth
    lo, hi, seconds = args
    case = synth.GEMV_CASES["q4_k_4096x4096"]
    W, X = synth.gemv_inputs(case, 1)
    idx = np.arange(lo, hi, dtype=np.int64)
    n, t0 = 0, time.perf_counter()
    while True:
        oracle.gemv(case.fmt, W, case.rows, case.cols, X, row_idx=idx)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return n * (hi - lo), el


# Worker processes for the many-core oracle run: this machine gives one GPU
# a share of 16 host CPUs, whatever the host's CPU count.
CPU_SHARE = 16


def cpu_baseline_all_cores(seconds):
    """The same oracle on the host CPUs this GPU's share allows: one process
    per CPU (up to 16), each running the single-threaded oracle over its own
    contiguous row range of the headline matrix (the oracle itself is
    unchanged)."""
    import multiprocessing as mp
    import synth
    case = synth.GEMV_CASES["q4_k_4096x4096"]
    model, ncpu = host_cpu()
    cores = max(1, min(ncpu, CPU_SHARE))
    bounds = np.linspace(0, case.rows, cores + 1).astype(int)
    # fresh interpreters that import the oracle only (no GPU runtime)
    ctx = mp.get_context("spawn")
    with ctx.Pool(cores) as pool:
        done = pool.map(_oracle_rows, [(int(bounds[i]), int(bounds[i + 1]), seconds)
                                       for i in range(cores)])
    row_bytes = (case.cols // 256) * 144
    # the processes run side by side: the aggregate rate is the sum of theirs
    gbs = sum(n * row_bytes / el for n, el in done) / 1e9
    rows = sum(n for n, _ in done)
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{rows} rows of Q4_K 4096x4096 batch-1 GEMVs, {cores} processes side by "
                      f"side for ~{seconds:.0f} s each, every one the single-threaded oracle over "
                      f"its own rows ({cores} = min(host logical CPUs {ncpu}, the 16-CPU share "
                      f"of one GPU on this machine))",
            "cpu_model": model, "host_logical_cpus": ncpu}


# What each workload's kernel computes in (the "dtype" of the line is the
# headline's).
ARITH = {
    "valu_f32": "f32 products and sums on the vector ALUs",
    "valu_q6k_int": "int8 codes x integer activations (rint at 2^21..2^22 of each 16-column "
                    "run's max), exact int32 sums, f32 per run",
    "mfma_i8_q6k": "int8 codes x integer activations (rint at 2^21..2^22 of each 16-column "
                   "run's max) on the matrix cores, exact int32 sums, f32 per run",
    "mfma_f16": "f16 codes x f16 hi + lo activation parts on the matrix cores, f32 sums",
    "mfma_bf16": "bf16 codes x bf16 hi + lo activation parts on the matrix cores, f32 sums",
    "mfma_bf16_ws": "bf16 codes x bf16 hi + lo activation parts on the matrix cores, f32 sums, "
                    "column ranges added in a second kernel",
    "mfma_bf16_ks2": "bf16 codes x bf16 hi + lo activation parts on the matrix cores, f32 sums, "
                     "activations shared by 4 row tiles, two column ranges added in the workgroup",
    "q8act": "int8 codes x int8 activations (per 16 columns), exact int32 sums, f32 per group",
    "moe": "f64 router, f32 expert GEMVs on the vector ALUs",
    "moe_tokens": "f64 router, gate/up as bf16 codes x bf16 hi + lo activation parts on the "
                  "matrix cores (f32 sums, each distinct expert's rows read once per call), "
                  "down f32 on the vector ALUs",
    "moe_q8": "f64 router, expert GEMVs as int8 codes x int8 activations (per 16 columns), "
              "exact int32 sums, f32 per group",
    "read": "plain read, no arithmetic",
}


def gemv_arith(q):
    """The arithmetic the library reports for its last GEMV call."""
    return ARITH[{"valu_f32": "valu_f32", "valu_q6k_int": "valu_q6k_int",
                  "mfma_i8_q6k": "mfma_i8_q6k", "mx_f16": "mfma_f16", "gemm_bf16": "mfma_bf16",
                  "gemm_ws_bf16": "mfma_bf16_ws", "gemm_ks2_bf16": "mfma_bf16_ks2",
                  "valu_q8act": "q8act"}[q.qg_last_kernel()]]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "sharding of this path is described, not built", file=sys.stderr)
        sys.exit(2)
    import torch
    import gguf_quant_dequant_amd as q
    import synth

    q.load_library()
    torch.cuda.set_device(0)
    only = set(filter(None, args.only.split(",")))
    scrub = Scrub(torch)

    head_case = synth.GEMV_CASES["q4_k_4096x4096"]
    results = {}
    if not only or "q4_k_4096x4096_b1" in only:
        head = Gemv(head_case, 1, torch, q)
        wall, ev_ms = time_launches(torch, head, args.steps, args.warmup, args.warm_seconds,
                                    scrub)
        per_us = ev_ms * 1e3 / args.steps
        results["q4_k_4096x4096_b1"] = dict(
            weight_bytes=head.wbytes, launches=args.steps,
            wall_gbs=round(args.steps * head.wbytes / wall / 1e9, 1),
            event_us_per_launch=round(per_us, 3),
            event_gbs=round(head.wbytes / (per_us * 1e-6) / 1e9, 1),
            arith=gemv_arith(q))
        head_wall, head_us = wall, per_us
        del head

    if not args.quick:
        # (workload, batch, variant): "" qgemv, "q8act" qgemv_q8act, "ws" qgemv_ws
        sweep = [("q8_0_256x1024", 1, ""), ("q6_k_151936x2048", 1, "")]
        # the lm_head for two and four sequences
        sweep += [("q6_k_151936x2048", b, "") for b in (2, 4)]
        sweep += [("q5_k_14336x4096", b, "") for b in (1, 4, 8)]
        sweep += [("q4_0_4096x14336", b, "") for b in (1, 4, 8)]
        # prefill-sized batches
        sweep += [("q4_k_4096x4096", b, "") for b in (16, 32, 64)]
        # the batched shapes again through qgemv_ws (activations shared
        # through LDS, a workspace)
        sweep += [("q5_k_14336x4096", b, "ws") for b in (4, 8)]
        sweep += [("q4_0_4096x14336", b, "ws") for b in (4, 8)]
        sweep += [("q4_k_4096x4096", b, "ws") for b in (16, 32, 64)]
        # the int8-activation variant (batch 1)
        sweep += [("q4_k_4096x4096", 1, "q8act"), ("q6_k_151936x2048", 1, "q8act")]
        for name, b, var in sweep:
            key = f"{name}_b{b}" + (f"_{var}" if var else "")
            if only and key not in only:
                continue
            case = synth.GEMV_CASES[name]
            w = Gemv(case, b, torch, q, q8act=var == "q8act", ws=var == "ws")
            steps = max(50, min(args.steps, int(4e9 // w.wbytes)))
            wall, ev_ms = time_launches(torch, w, steps, args.warmup, args.warm_seconds, scrub)
            per_us = ev_ms * 1e3 / steps
            results[key] = dict(
                weight_bytes=w.wbytes, launches=steps,
                wall_gbs=round(steps * w.wbytes / wall / 1e9, 1),
                event_us_per_launch=round(per_us, 3),
                event_gbs=round(w.wbytes / (per_us * 1e-6) / 1e9, 1),
                event_frac_hbm=round(w.wbytes / (per_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 3),
                # multiply-adds of the product, as TFLOP/s (2 flops each)
                tflops=round(2.0 * case.rows * case.cols * b / (per_us * 1e-6) / 1e12, 2),
                arith=gemv_arith(q))
            del w
            torch.cuda.empty_cache()
        # the streaming floor: a plain read of the headline's and the lm_head's
        # weight bytes, cold, at a few grid sizes
        for name in ("q4_k_4096x4096", "q6_k_151936x2048"):
            case = synth.GEMV_CASES[name]
            nbytes = case.rows * q.qg_row_bytes(case.fmt, case.cols)
            key = f"stream_read_{name}_bytes"
            if only and key not in only:
                continue
            best = None
            for grid in (0, 256, 512, 1024):
                sw = Stream(nbytes, torch, q, grid)
                steps = max(50, min(args.steps, int(4e9 // nbytes)))
                wall, ev_ms = time_launches(torch, sw, steps, args.warmup, args.warm_seconds,
                                            scrub)
                per_us = ev_ms * 1e3 / steps
                if best is None or per_us < best[1]:
                    best = (grid, per_us, steps)
                del sw
                torch.cuda.empty_cache()
            grid, per_us, steps = best
            results[key] = dict(
                bytes=nbytes, launches=steps, best_grid=grid or "auto",
                event_us_per_launch=round(per_us, 3),
                event_gbs=round(nbytes / (per_us * 1e-6) / 1e9, 1),
                event_frac_hbm=round(nbytes / (per_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 3),
                arith=ARITH["read"])
        if not only or "moe_ffn_qwen3_30b_a3b" in only:
            m = Moe(synth.MOE_CASE, torch, q, args.moe_tokens)
            steps = max(64, min(args.steps, 1000))
            wall, ev_ms = time_launches(torch, m, steps, args.warmup, args.warm_seconds, scrub)
            per_us = ev_ms * 1e3 / steps
            results["moe_ffn_qwen3_30b_a3b"] = dict(
                bytes_per_token=m.bytes_per_token, tokens=steps,
                wall_tokens_per_s=round(steps / wall, 1),
                event_us_per_token=round(per_us, 3),
                tokens_per_s=round(1e6 / per_us, 1),
                effective_gbs=round(m.bytes_per_token / (per_us * 1e-6) / 1e9, 1),
                arith=ARITH["moe"])
            del m
        if not only or "moe_ffn_q8act_qwen3_30b_a3b" in only:
            m = MoeQ8(synth.MOE_CASE, torch, q, args.moe_tokens)
            steps = max(64, min(args.steps, 1000))
            wall, ev_ms = time_launches(torch, m, steps, args.warmup, args.warm_seconds, scrub)
            per_us = ev_ms * 1e3 / steps
            results["moe_ffn_q8act_qwen3_30b_a3b"] = dict(
                bytes_per_token=m.bytes_per_token, tokens=steps,
                wall_tokens_per_s=round(steps / wall, 1),
                event_us_per_token=round(per_us, 3),
                tokens_per_s=round(1e6 / per_us, 1),
                effective_gbs=round(m.bytes_per_token / (per_us * 1e-6) / 1e9, 1),
                arith=ARITH["moe_q8"])
            del m
        if not only or "moe_ffn_norm_qwen3_30b_a3b" in only:
            m = MoeNorm(synth.MOE_CASE, torch, q, args.moe_tokens)
            steps = max(64, min(args.steps, 1000))
            wall, ev_ms = time_launches(torch, m, steps, args.warmup, args.warm_seconds, scrub)
            per_us = ev_ms * 1e3 / steps
            results["moe_ffn_norm_qwen3_30b_a3b"] = dict(
                bytes_per_token=m.bytes_per_token, tokens=steps,
                wall_tokens_per_s=round(steps / wall, 1),
                event_us_per_token=round(per_us, 3),
                tokens_per_s=round(1e6 / per_us, 1),
                effective_gbs=round(m.bytes_per_token / (per_us * 1e-6) / 1e9, 1),
                arith=ARITH["moe"])
            del m

        for T in (4, 8):
            key = f"moe_ffn_tokens{T}_qwen3_30b_a3b"
            if only and key not in only:
                continue
            m = MoeTokens(synth.MOE_CASE, torch, q, args.moe_tokens, T)
            steps = max(64, min(args.steps, 500))
            wall, ev_ms = time_launches(torch, m, steps, args.warmup, args.warm_seconds, scrub)
            per_us = ev_ms * 1e3 / steps
            results[key] = dict(
                tokens_per_call=T, calls=steps,
                wall_tokens_per_s=round(steps * T / wall, 1),
                event_us_per_call=round(per_us, 3),
                tokens_per_s=round(T * 1e6 / per_us, 1),
                arith=ARITH["moe_tokens"])
            del m

    line = {
        "metric": "quantized GEMV weight GB/s (Q4_K 4096x4096, batch 1)",
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic, seeded (Q4_K fields: d, dmin ~ U[1e-3,1e-2], 6-bit scales and "
                "nibbles uniform; x ~ N(0,1)); weights cold in HBM (rotating copies >= 1 GiB "
                "and a 1 GiB cache scrub before the timed replay)",
        "config": {"workload": "Q4_K GEMV 4096 x 4096, batch 1", "rows": 4096, "cols": 4096,
                   "batch": 1, "format": "Q4_K", "weight_bytes": head_case.rows * 2304,
                   "cold_copies": True},
    }
    if "q4_k_4096x4096_b1" in results:
        r = results["q4_k_4096x4096_b1"]
        wb = r["weight_bytes"]
        line["value"] = r["wall_gbs"]
        line["ms_per_step"] = round(head_wall / args.steps * 1e3, 6)
        achieved = wb / (head_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(),
                "kernel": "qgemv_lds_kernel, Q4_K, 64-column lane tiles, batch 1",
                "bytes_per_launch": wb, "event_us_per_launch": round(head_us, 3)}
        # the same kernel's mean duration in the committed rocprofv3 trace
        tu = measured_trace_us()
        roof["trace_us_per_launch"] = tu
        if tu:
            roof["trace_achieved"] = round(wb / (tu * 1e-6) / 1e9, 1)
            roof["trace_frac"] = round(wb / (tu * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
        line["roofline"] = roof
    line["workloads"] = results
    if args.copy_calibration:
        n = 256 << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        line["copy_calibration_bytes"] = n
        del src, dst
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
        line["cpu_baseline_all_cores"] = cpu_baseline_all_cores(args.cpu_seconds / 2)
        if not args.quick:
            line["cpu_baseline_moe"] = cpu_baseline_moe(args.cpu_seconds / 2)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
