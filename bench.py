"""Benchmark of the chunked Mamba-2 SSD forward pass on one MI355X.

One step = one mamba2_ssd_forward (chunk_cumsum -> fwd_pass_state ->
chunk_scan; at L = 64K fwd_pass_state runs over spans of chunks: span_end ->
span_pass) over the whole workload, inputs resident in HBM.
Prints one JSON line with tokens/s, the roofline position of the dominant
kernel (per-kernel durations measured here with HIP events on the launch
stream) and the CPU oracle's throughput on the host as a reported baseline.

    python bench.py [--gpus 1] [--steps 100] [--warmup 100] [--workload long_L64k_N256]
    python bench.py --backward      (the backward pass on the same workload)
    python bench.py --decode-batch B (the one-token recurrent step)
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SSD forward tokens/s at L=64K,N=256 on 1 MI355X; % of MFMA/HBM roofline"
HEADLINE = "long_L64k_N256"


def metric_name(w, backward=False):
    """The headline metric for the headline workload; other workloads name
    themselves (their numbers are not the headline's)."""
    if backward:
        if w.name == HEADLINE:
            return "SSD backward tokens/s at L=64K,N=256 on 1 MI355X (forward states recomputed)"
        return f"SSD backward tokens/s, {w.name} on 1 MI355X (forward states recomputed)"
    return METRIC if w.name == HEADLINE else f"SSD forward tokens/s, {w.name} on 1 MI355X; % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA, TFLOP/s
FP32_VALU_PEAK_TFLOPS = 157.3  # float32 vector FMA, TFLOP/s
RIDGE = BF16_MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
STAGES = ("chunk_cumsum", "chunk_state", "state_passing", "chunk_scan")


def grouped_path(w):
    """The fused forward hands the chunk-start states to the output stage as
    bfloat16 for these sizes (same rule as the library's dispatch)."""
    return (w.dtype == "bf16" and w.headdim == 64 and w.dstate in (64, 128, 256, 512)
            and w.chunk_size in (64, 128, 256))


def span_scan_chunks(w, cus=256):
    """The forward's span length at state size 64 (span_scan, an even number
    of heads per group): the longest span of 8, 4 or 2 chunks whose
    span_scan grid gives every CU a workgroup; 0 where none does and at every
    other state size (same rule as the library)."""
    if not (grouped_path(w) and w.dstate == 64):
        return 0
    hg = w.nheads // w.ngroups
    if hg % 2:
        return 0
    for K in (8, 4, 2):
        if w.nchunks < K:
            continue
        ng = -(-w.nchunks // K)
        R = 4 if (hg % 4 == 0 and w.batch * ng * w.nheads // 4 >= cus) else 2
        if w.batch * ng * w.nheads // R >= cus:
            return K
    return 0


def span_plan(w, cus=256, forward=True):
    """(span length K, heads per workgroup R of span_end and the replay) of
    the span path, or None where the library runs chunk_state +
    state_passing (same rule as the library's dispatch: spans of 8, else 4,
    chunks while the grid gives every CU two (batch, span, head) units, else
    one; in the forward at state size 64, the span length span_scan's grid
    asks for; R = 4, 2 or 1 heads of a group likewise, at most 2 at N = 128
    and 1 at N = 64).  forward=False: the backward's recompute, which keeps
    the first rule."""
    if not grouped_path(w):
        return None
    nc = w.nchunks
    max_r = 1 if w.dstate == 64 else 2 if w.dstate == 128 else 4

    def heads(K):
        ng = -(-nc // K)
        for R in (4, 2):
            if (R <= max_r and (w.nheads // w.ngroups) % R == 0
                    and w.batch * ng * w.nheads // R >= cus):
                return R
        return 1

    if forward:
        K = span_scan_chunks(w, cus)
        if K:
            return K, heads(K)
    for want in (2 * cus, cus):
        for K in (8, 4):
            ng = -(-nc // K)
            if nc >= K and w.batch * w.nheads * ng >= want:
                return K, heads(K)
    return None


def workload(name):
    """A named workload, or a shape of the sequence-length x state-size sweep
    named sweep_L<k>k_N<n> (batch 1, 32 heads of 64, one B/C group, chunk 256,
    bf16, no initial state, as --sweep runs it)."""
    import ssd_inputs
    if name in ssd_inputs.WORKLOADS:
        return ssd_inputs.WORKLOADS[name]
    m = re.fullmatch(r"sweep_L(\d+)k_N(\d+)", name)
    if not m:
        raise SystemExit(f"unknown workload {name!r}: one of {list(ssd_inputs.WORKLOADS)} "
                         "or sweep_L<k>k_N<n>")
    L, N = int(m.group(1)) * 1024, int(m.group(2))
    return ssd_inputs.custom(name=name, batch=1, seqlen=L, nheads=32, headdim=64, dstate=N,
                             ngroups=1, chunk_size=256, dtype="bf16", init_state=False,
                             seed=2000 + N + L // 1024)


def scan_plan(w, cus=256):
    """Heads per workgroup of span_scan (the span replay fused with the output
    stage), or None where the forward runs the replay and the grouped
    chunk_scan instead (same rule as the library: state size 64 or 128 on the
    span path; 4 heads where the grid still gives every CU a workgroup, else 2;
    an even number of heads per group)."""
    plan = span_plan(w, cus)
    if not plan or w.dstate not in (64, 128):
        return None
    K = plan[0]
    hg = w.nheads // w.ngroups
    ng = -(-w.nchunks // K)
    if hg % 4 == 0 and w.batch * ng * w.nheads // 4 >= cus:
        return 4
    return 2 if hg % 2 == 0 else None


def forward_stages(w, cus=256):
    """Names of the four timed slots of mamba2_ssd_forward_profile."""
    if span_plan(w, cus):
        if scan_plan(w, cus):
            return ("chunk_cumsum", "span_end", "span_jump", "span_scan")
        return ("chunk_cumsum", "span_end", "span_pass", "chunk_scan")
    return STAGES


def stage_model(w, cus=256):
    """Algorithmic flops and HBM bytes per launch of each stage of the fused
    forward: every input read once and every output written once, in the
    dtypes that stage consumes and produces; flops count the causal triangle
    (diagonal included) and nothing above it, and the C B^T products once per
    (chunk, group), since every head of the group shares them.  On the span
    path, span_end is the span-end kernel and span_pass the jump across spans
    plus the replay that writes the chunk-start states (x rows of every
    chunk but each span's last, which needs no contraction)."""
    B, L, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk_size
    nc = w.nchunks
    e = 4 if w.dtype == "f32" else 2
    tok, csb = B * L, B * H * nc * Q * 4
    st = B * nc * H * P * N * 4                      # per-chunk states, float32
    hs = st // 2 if grouped_path(w) else st          # chunk-start states as handed on
    fin = B * H * P * N * 4
    x = tok * H * P * e
    bc = tok * G * N * e
    m = {}
    m["chunk_cumsum"] = dict(flops=2 * tok * H, bytes=tok * H * e + H * 4 + 2 * csb)
    m["chunk_state"] = dict(flops=2 * N * P * tok * H, bytes=x + bc + 2 * csb + st)
    m["state_passing"] = dict(flops=2 * st // 4, bytes=st + hs + B * H * nc * 4 + fin)
    m["chunk_scan"] = dict(
        # C B^T depends only on the (chunk, group): counted once per group
        flops=tok * H * (2 * N * P + (Q + 1) * P + 2 * P) + tok * G * (Q + 1) * N,
        bytes=x + 2 * bc + 2 * csb + hs + H * 4 + x)
    plan = span_plan(w, cus)
    if plan:
        K = plan[0]
        ng = -(-nc // K)
        ss = B * ng * H * P * N * 4                  # span states, float32
        dec = B * H * ng * 4
        init = fin if w.init_state else 0
        frac = (nc - ng) / nc                         # chunks the replay contracts
        m["span_end"] = dict(flops=2 * N * P * tok * H, bytes=x + bc + 2 * csb + ss + dec)
        m["span_pass"] = dict(
            flops=2 * ss // 4 + 2 * N * P * tok * H * frac,
            bytes=(ss + dec + init + ss + fin) + (x * frac + bc * frac + 2 * csb + ss + hs))
        # fused path: the jump alone, then span_scan (replay and output in one
        # pass over blocks of 32 steps: x, B, C, sums and the span start
        # states read once, y written once; C B^T of each block once per group)
        m["span_jump"] = dict(flops=2 * ss // 4, bytes=ss + dec + init + ss + fin)
        rb = 32
        nblk = nc * (Q // rb)
        ufrac = (nblk - ng) / nblk                    # blocks whose state update runs
        m["span_scan"] = dict(
            flops=tok * H * (2 * N * P + 2 * N * P * ufrac + (rb + 1) * P + 2 * P)
            + tok * G * (rb + 1) * N,
            bytes=x + 2 * bc + 2 * csb + ss + H * 4 + x)
    return m


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=int(os.environ.get("WORLD_SIZE", "1")))
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens per head for the CPU oracle sample (0 = whole sequence)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--decode-batch", type=int, default=0,
                    help="only measure the one-token recurrent step at this batch size "
                         "(H=32, P=64, N=256, bf16)")
    ap.add_argument("--backward", action="store_true",
                    help="only measure the backward pass (mamba2_ssd_backward) on the workload")
    ap.add_argument("--sweep", action="store_true",
                    help="only measure the forward over sequence lengths 1K-256K and state "
                         "sizes 64-512 (H=32, P=64, G=1, Q=256, bf16): one JSON line per shape")
    ap.add_argument("--state-path", choices=("default", "fused"), default="default",
                    help="fused: measure mamba2_ssd_forward_fused (one-kernel fwd_pass_state)")
    args = ap.parse_args()
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return
    if args.sweep:
        sweep_bench(args)
        return
    if args.decode_batch:
        decode_bench(args)
        return
    if args.backward:
        if args.gpus != 1:
            print(json.dumps({"error": "this benchmark runs on one GPU only; run with --gpus 1",
                              "n_gpus": args.gpus}))
            sys.exit(2)
        backward_bench(args)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; run with --gpus 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.state_path == "fused":
        fused_state_bench(args)
        return

    import torch

    import ssd_inputs
    import state_space_sequence_02_amd as m2

    w = workload(args.workload)
    inp = ssd_inputs.make_inputs(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = {k: (None if v is None else v.to(dev)) for k, v in inp.items()}
    dims = m2.dims_of(g["x"], g["B"], w.chunk_size)
    y = torch.empty_like(g["x"])
    fin = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.float32, device=dev)
    need = m2.mamba2_ssd_workspace_bytes(dims)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        m2.mamba2_ssd_forward(dims, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"],
                              g["init_state"], y, fin, ws, need, stream)

    # Per-stage durations of the same forward first: HIP events recorded on the
    # launch stream between its kernels (mamba2_ssd_forward_profile), at least
    # 50 calls and 0.25 s.  This also brings the GPU's clocks to their steady
    # state before the warm-up and timed steps below (they take tens of
    # milliseconds of load to settle).
    stage_sum, n_prof = [0.0] * 4, 0
    t_prof = time.perf_counter()
    while n_prof < 50 or time.perf_counter() - t_prof < 0.25:
        ms4 = m2.mamba2_ssd_forward_profile(dims, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"],
                                            g["init_state"], y, fin, ws, need, stream)
        stage_sum = [a + b for a, b in zip(stage_sum, ms4)]
        n_prof += 1

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ms = ev0.elapsed_time(ev1) / args.steps

    # Per-step spread: 20 more steps, each bracketed by its own events on the
    # launch stream (the events sit between steps, so the steps still run
    # back to back); reported beside the mean, not used for `value`.
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(21)]
    evs[0].record(stream)
    for k in range(20):
        step()
        evs[k + 1].record(stream)
    torch.cuda.synchronize()
    per_step = sorted(evs[k].elapsed_time(evs[k + 1]) for k in range(20))

    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    names = forward_stages(w, cus)
    stage_ms = {s: stage_sum[i] / n_prof for i, s in enumerate(names)}
    model = stage_model(w, cus)
    dom = max(names, key=lambda s: stage_ms[s])
    dm = model[dom]
    ai = dm["flops"] / dm["bytes"]
    bound = "hbm" if ai < RIDGE else "mfma"
    if bound == "hbm":
        achieved = dm["bytes"] / (stage_ms[dom] * 1e-3) / 1e9
        peak, unit = HBM_PEAK_GBS, "GB/s"
    else:
        achieved = dm["flops"] / (stage_ms[dom] * 1e-3) / 1e12
        peak, unit = BF16_MFMA_PEAK_TFLOPS, "TFLOP/s"
    stages = {}
    for s in names:
        t = stage_ms[s] * 1e-3
        stages[s] = {"ms": round(stage_ms[s], 4),
                     "GB/s": round(model[s]["bytes"] / t / 1e9, 1),
                     "TFLOP/s": round(model[s]["flops"] / t / 1e12, 2),
                     "hbm_frac": round(model[s]["bytes"] / t / 1e9 / HBM_PEAK_GBS, 3)}

    tokens = w.tokens
    out = {
        "metric": metric_name(w),
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_spread": {"median": (per_step[9] + per_step[10]) / 2, "min": per_step[0],
                               "max": per_step[-1], "steps": 20},
        "wall_ms_per_step": wall_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "nheads": w.nheads,
                   "headdim": w.headdim, "dstate": w.dstate, "ngroups": w.ngroups,
                   "chunk_size": w.chunk_size, "parallelism": "none (1 GPU)"},
        "roofline": {"kernel": dom, "bound": bound, "achieved": achieved, "peak": peak,
                     "unit": unit, "frac": achieved / peak,
                     "traffic": profiled_traffic(w.name, dom),
                     "algorithmic_bytes": dm["bytes"], "algorithmic_flops": dm["flops"],
                     "mfma": mfma_fractions(w, dom, stage_ms[dom])},
        "stages": stages,
        "stage_timing_calls": n_prof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, w, args.cpu_tokens)
    print(json.dumps(out), flush=True)


def effective_flops(w, stage):
    """Flops of `stage` counted per head, as a kernel that did not share the
    group's C B^T across heads would execute them: 4NP + (Q+1)(N+P) + 2P per
    (token, head) for the whole forward, of which the output stage's share is
    2NP + (Q+1)(N+P) + 2P.  Other stages have nothing shared, so their count
    equals the issued one."""
    B, L, H, P, N, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.chunk_size
    tok = B * L
    if stage == "chunk_scan":
        return tok * H * (2 * N * P + (Q + 1) * (N + P) + 2 * P)
    if stage == "span_scan":
        m = stage_model(w)["span_scan"]
        return m["flops"] - tok * w.ngroups * 33 * N + tok * H * 33 * N
    return stage_model(w)[stage]["flops"]


def mfma_fractions(w, stage, ms):
    """The dominant kernel against the dense bf16 MFMA peak, both ways:
    issued = the flops the kernel performs (C B^T once per (chunk, group)),
    effective = the per-head count of the same work."""
    issued = stage_model(w)[stage]["flops"]
    eff = effective_flops(w, stage)
    t = ms * 1e-3
    return {"issued_flops": issued, "issued_TFLOP/s": issued / t / 1e12,
            "issued_frac": issued / t / 1e12 / BF16_MFMA_PEAK_TFLOPS,
            "effective_flops": eff, "effective_TFLOP/s": eff / t / 1e12,
            "effective_frac": eff / t / 1e12 / BF16_MFMA_PEAK_TFLOPS,
            "peak_TFLOP/s": BF16_MFMA_PEAK_TFLOPS}


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def fused_state_model(w):
    """Algorithmic flops and HBM bytes of one mamba2_fwd_pass_state call: the
    weights kernel (reads the cumulative sums and dt, writes the weights) and
    the one-kernel state pass (reads x, B, the sums and weights, writes the
    bfloat16 chunk-start states and the float32 final state).  Every head of a
    group reads the group's B rows, so B counts once per head."""
    B, L, H, P, N, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.chunk_size
    tok, csb = B * L, B * H * w.nchunks * Q * 4
    hs = B * w.nchunks * H * P * N * 2
    fin = B * H * P * N * 4
    init = fin if w.init_state else 0
    return dict(flops=2 * N * P * tok * H,
                bytes=3 * csb + tok * H * P * 2 + tok * H * N * 2 + 2 * csb + hs + fin + init)


def fused_state_bench(args):
    import torch

    import ssd_inputs
    import state_space_sequence_02_amd as m2

    w = workload(args.workload)
    inp = ssd_inputs.make_inputs(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = {k: (None if v is None else v.to(dev)) for k, v in inp.items()}
    dims = m2.dims_of(g["x"], g["B"], w.chunk_size)
    y = torch.empty_like(g["x"])
    fin = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.float32, device=dev)
    need = m2.mamba2_ssd_workspace_bytes(dims)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        m2.mamba2_ssd_forward_fused(dims, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"],
                                    g["init_state"], y, fin, ws, need, stream)

    def timed(fn, n):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(n):
            fn()
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / n

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = timed(step, args.steps)
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps

    # the state pass alone, on the same stream: weights kernel + one-kernel pass
    cs, dtt, _ = m2.stage_buffers(dims, dev)
    m2.mamba2_chunk_cumsum(dims, g["dt"], g["A"], cs, dtt, stream)
    wT = torch.empty_like(cs)
    hst = torch.empty((w.batch, w.nchunks, w.nheads, w.headdim, w.dstate), dtype=torch.bfloat16,
                      device=dev)
    fin2 = torch.empty_like(fin)

    def state_pass():
        m2.mamba2_fwd_pass_state(dims, g["x"], g["B"], cs, dtt, g["init_state"], wT, hst, fin2,
                                 stream)

    state_pass()
    torch.cuda.synchronize()
    sp_ms = timed(state_pass, args.steps)
    dm = fused_state_model(w)
    achieved = dm["bytes"] / (sp_ms * 1e-3) / 1e9
    out = {
        "metric": metric_name(w),
        "value": w.tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "wall_ms_per_step": wall_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "nheads": w.nheads,
                   "headdim": w.headdim, "dstate": w.dstate, "ngroups": w.ngroups,
                   "chunk_size": w.chunk_size, "state_path": "one-kernel fwd_pass_state",
                   "parallelism": "none (1 GPU)"},
        "roofline": {"kernel": "fwd_pass_state (weights + state pass)", "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes": dm["bytes"], "algorithmic_flops": dm["flops"],
                     "ms": sp_ms, "TFLOP/s": dm["flops"] / (sp_ms * 1e-3) / 1e12},
    }
    print(json.dumps(out), flush=True)


# Source files that define each stage's kernel (with the shared helpers): a
# profile's byte counts stand for the kernel only while these are unchanged.
KERNEL_SOURCES = {
    "chunk_cumsum": ("chunk_cumsum.hip", "common.h"),
    "chunk_state": ("chunk_state_grouped.hip", "common.h"),
    "state_passing": ("state_passing.hip", "common.h"),
    "span_end": ("state_span.hip", "common.h"),
    "span_pass": ("state_span.hip", "common.h"),
    "span_jump": ("state_span.hip", "common.h"),
    "span_scan": ("span_scan.hip", "common.h"),
    "chunk_scan": ("chunk_scan_grouped.hip", "common.h"),
    "adjoint_state": ("chunk_state_grouped.hip", "common.h"),
    "reverse_pass": ("state_passing.hip", "common.h"),
    "dB_dC": ("chunk_bwd.hip", "common.h"),
    "dx": ("chunk_bwd.hip", "common.h"),
    "param_sums": ("chunk_bwd.hip", "common.h"),
}


def stage_sources(stage, direction="forward", workload_name=None):
    """The source files of `stage`'s kernel.  The backward's recompute stages
    (chunk_state, state_passing) run the forward's span kernels where the
    workload takes the span path."""
    if (direction == "backward" and stage in ("chunk_state", "state_passing")
            and workload_name is not None and span_plan(workload(workload_name), forward=False)):
        return KERNEL_SOURCES["span_end"]
    return KERNEL_SOURCES[stage]


def sources_digest(stage, direction="forward", workload_name=None):
    """sha256 over the files that define `stage`'s kernel (names and bytes)."""
    import hashlib
    d = os.path.join(ROOT, "state_space_sequence_02_amd", "csrc")
    h = hashlib.sha256()
    for f in stage_sources(stage, direction, workload_name):
        h.update(f.encode())
        with open(os.path.join(d, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def profiled_traffic(workload, stage, direction="forward"):
    """HBM bytes per launch of `stage` from the committed rocprofv3 summary of
    this workload (FETCH_SIZE and WRITE_SIZE, each scaled by the copy-kernel
    calibration), or None when there is none or the kernel's sources changed
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"ssd_{direction}_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(rf"sources-sha256 {stage}: ([0-9a-f]{{64}})", text)
    if not m or m.group(1) != sources_digest(stage, direction, workload):
        return None
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 8 and cells[0].startswith(stage):
            try:
                return float(cells[5]) * 1e6
            except ValueError:
                return None
    return None


SWEEP_L = (1024, 4096, 16384, 65536, 262144)
SWEEP_N = (64, 128, 256, 512)


def sweep_bench(args):
    """Forward throughput over the pages' sweep of sequence lengths and state
    sizes (1K-256K tokens, N = 64-512): batch 1, 32 heads of 64, one B/C
    group, chunk 256, bf16, inputs resident.  Each shape is warmed up for at
    least 0.3 s of back-to-back steps (clocks settle) and then timed over at
    least 100 steps and 0.2 s with HIP events on the launch stream.  The
    roofline fraction is the path's algorithmic HBM bytes (the stages the
    library runs for that shape, as in stage_model) over the step time,
    against 8 TB/s; MFMA is the algorithmic flops over the step time against
    the dense bf16 peak."""
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; run with --gpus 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import ssd_inputs
    import state_space_sequence_02_amd as m2

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = torch.cuda.current_stream()
    for N in SWEEP_N:
        for L in SWEEP_L:
            w = ssd_inputs.custom(name=f"sweep_L{L // 1024}k_N{N}", batch=1, seqlen=L, nheads=32,
                                  headdim=64, dstate=N, ngroups=1, chunk_size=256,
                                  dtype="bf16", init_state=False, seed=2000 + N + L // 1024)
            g = {k: (None if v is None else v.to(dev))
                 for k, v in ssd_inputs.make_inputs(w).items()}
            dims = m2.dims_of(g["x"], g["B"], w.chunk_size)
            y = torch.empty_like(g["x"])
            fin = torch.empty((1, w.nheads, w.headdim, w.dstate), dtype=torch.float32, device=dev)
            need = m2.mamba2_ssd_workspace_bytes(dims)
            ws = torch.empty(need, dtype=torch.uint8, device=dev)

            def step():
                m2.mamba2_ssd_forward(dims, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"],
                                      g["init_state"], y, fin, ws, need, stream)

            t_end = time.perf_counter() + 0.3
            while time.perf_counter() < t_end:
                for _ in range(10):
                    step()
                torch.cuda.synchronize()
            step()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            e0.record(stream)
            n = 0
            while n < 100 or time.perf_counter() - t0 < 0.2:
                step()
                n += 1
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / n
            model = stage_model(w, cus)
            names = forward_stages(w, cus)
            st_ms = [0.0] * 4
            for _ in range(10):
                ms4 = m2.mamba2_ssd_forward_profile(dims, g["x"], g["dt"], g["A"], g["B"], g["C"],
                                                    g["D"], g["init_state"], y, fin, ws, need,
                                                    stream)
                st_ms = [a + b / 10 for a, b in zip(st_ms, ms4)]
            byt = sum(model[s]["bytes"] for s in names)
            flo = sum(model[s]["flops"] for s in names)
            plan = span_plan(w, cus)
            sp = scan_plan(w, cus)
            path = (f"span K={plan[0]} R={plan[1]}" + (f", span_scan R={sp}" if sp else "")
                    if plan else
                    ("split, bf16 start states" if grouped_path(w) else "split, per head"))
            print(json.dumps({
                "workload": w.name, "seqlen": L, "dstate": N, "nheads": w.nheads,
                "headdim": w.headdim, "ngroups": w.ngroups, "chunk_size": w.chunk_size,
                "path": path, "steps": n, "ms_per_step": round(ms, 4),
                "tokens_per_s": L / (ms * 1e-3),
                "algorithmic_bytes": byt, "GB/s": round(byt / (ms * 1e-3) / 1e9, 1),
                "hbm_frac": round(byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 3),
                "TFLOP/s": round(flo / (ms * 1e-3) / 1e12, 1),
                "mfma_frac": round(flo / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 3),
                "stage_ms": {s: round(t, 4) for s, t in zip(names, st_ms)}}),
                flush=True)
            del g, y, fin, ws
            torch.cuda.empty_cache()


def copy_probe(mib):
    """A plain device-to-device copy of known size, used to calibrate the HBM
    byte counters (each launch reads and writes `mib` MiB)."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4,
                      "launches": 5}), flush=True)


def decode_bench(args):
    """One-token recurrent step (mamba2_decode_step) on a serving-sized batch:
    tokens/s = batch / step time, and the state's HBM roofline (the float32
    state is read and written once per step; the per-token inputs are
    negligible next to it)."""
    import torch

    import ssd_inputs
    import state_space_sequence_02_amd as m2

    w = ssd_inputs.custom(name=f"decode_B{args.decode_batch}_H32_P64_N256", batch=args.decode_batch,
                          seqlen=1, nheads=32, headdim=64, dstate=256, ngroups=1, chunk_size=64,
                          init_state=True, seed=48)
    inp = ssd_inputs.make_inputs(w)
    g = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    x, dt, Bm, C = (g[k][:, 0].clone() for k in ("x", "dt", "B", "C"))
    state = g["init_state"].clone()
    y = torch.empty_like(x)
    dims = m2.make_dims(w.batch, 1, w.nheads, w.headdim, w.dstate, 1, 64, torch.bfloat16)
    for _ in range(args.warmup):
        m2.mamba2_decode_step(dims, x, dt, g["A"], Bm, C, g["D"], state, y)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        m2.mamba2_decode_step(dims, x, dt, g["A"], Bm, C, g["D"], state, y)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    sbytes = 2 * state.numel() * 4
    ibytes = (x.numel() + dt.numel() + Bm.numel() + C.numel() + y.numel()) * 2
    gbs = (sbytes + ibytes) / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "SSD one-token decode step tokens/s (B sequences, H=32, P=64, N=256) on 1 MI355X",
        "value": w.batch / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "dtype": "bf16",
        "data": "synthetic", "config": {"workload": w.name, "batch": w.batch},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None},
        "cpu_baseline": None if args.no_cpu_baseline else decode_cpu_baseline(inp, w),
    }), flush=True)


def decode_cpu_baseline(inp, w):
    """The CPU oracle advancing the same batch by one token (its recurrence
    over a one-token sequence from the given state), repeated for at least a
    second; tokens/s over the batch."""
    import oracle
    o = {k: (None if v is None else v.float().numpy()) for k, v in inp.items()}
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.ssd_recurrence(o["x"], o["dt"], o["A"], o["B"], o["C"], o["D"], o["init_state"],
                              chunk_size=64, want_final=True)
        reps += 1
        sec = time.perf_counter() - t0
        if sec >= 1.0:
            break
    return {"value": w.batch * reps / sec, "unit": "tokens/s", "cores": oracle.num_threads(),
            "cpu_model": cpu_model(), "kind": "oracle", "seconds": sec,
            "sample": f"{reps} one-token steps of the whole batch ({w.batch} sequences, "
                      f"{w.nheads} heads)"}


BWD_STAGES = ("chunk_cumsum", "chunk_state", "state_passing", "adjoint_state", "reverse_pass",
              "dB_dC", "dx", "param_sums")


def backward_model(w):
    """Algorithmic flops and HBM bytes per launch of each backward stage
    (inputs read once, outputs written once; flops over the causal triangle,
    the group-shared products once per (chunk, group))."""
    B, L, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk_size
    nc = w.nchunks
    tok, csb = B * L, B * H * nc * Q * 4
    st = B * nc * H * P * N * 4
    hs = st // 2
    fin = B * H * P * N * 4
    x = tok * H * P * 2
    bc = tok * G * N * 2
    th = B * nc * H * (N // 64) * Q * 4
    fwd = stage_model(w)
    m = {k: fwd[k] for k in ("chunk_cumsum", "chunk_state", "state_passing")}
    if span_plan(w, forward=False):
        # the chunk-start states recomputed over spans, as the forward does:
        # the profile's two stages are span_end and the jump plus the replay
        m["chunk_state"], m["state_passing"] = fwd["span_end"], fwd["span_pass"]
    m["adjoint_state"] = dict(flops=2 * N * P * tok * H, bytes=x + bc + 2 * csb + st)
    m["reverse_pass"] = dict(flops=2 * st // 4 + 2 * st // 4,
                             bytes=st + hs + B * H * nc * 4 + 2 * fin + hs)
    rs = B * H * nc * Q * 4                           # rectangle sums of the decay gradient
    # dB_dC: the summed-W kernel (W, its rectangle sums, C B^T once per
    # (chunk, group)) and the dB/dC kernel (state terms, summed W times B, C)
    m["dB_dC"] = dict(
        flops=tok * H * ((Q + 1) * P + 4 * P * N) + tok * G * 3 * (Q + 1) * N,
        bytes=2 * x + 2 * bc + 2 * hs + 2 * csb + 2 * bc + th + rs)
    m["dx"] = dict(flops=tok * G * (Q + 1) * N + tok * H * (2 * P * N + (Q + 1) * P),
                   bytes=2 * x + 2 * bc + hs + 2 * csb + th + rs + x + tok * H * 2)
    if N > 256:
        # the state term B g^T by its own kernel (g and B read, float32 dU
        # part written), which dx then reads instead of g
        m["dx"]["bytes"] += bc + 2 * tok * H * P * 4
    m["param_sums"] = dict(flops=4 * B * nc * H, bytes=2 * B * nc * H * 4 + 2 * H * 4)
    return m


def backward_fast(w):
    """Whether the MFMA backward kernels cover the workload (else the generic
    float32 backward runs)."""
    return (w.dtype == "bf16" and w.headdim == 64
            and ((w.dstate in (64, 128, 256) and w.chunk_size in (64, 128, 256))
                 or (w.dstate == 512 and w.chunk_size == 256)))


def generic_backward_flops(w):
    """Flops the generic backward's contractions issue (float32 FMAs, 2 flops
    each; the causal triangles counted at half the square, the group-shared
    C B^T once per group): adjoint states, the g B^T and h C^T products, the
    in-chunk dU contraction, dy x^T for the decay gradient, and dB, dC (their
    dy x^T tiles recomputed once per 64 state columns)."""
    B, L, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk_size
    tok = B * L
    per_head = (3 * P * N          # adjoint states, g B^T, h C^T
                + Q / 2 * P        # dU in-chunk
                + Q / 2 * P        # dy x^T for the decay gradient
                + 2 * (P * N + Q / 2 * P * -(-N // 64) + Q / 2 * N))  # dC and dB
    return 2 * tok * (H * per_head + G * Q / 2 * N)


def backward_bench(args):
    """Backward pass over the workload: tokens/s of one mamba2_ssd_backward
    (it recomputes the forward's chunk states inside), per-stage times from
    HIP events on the launch stream, the dominant kernel's roofline, and the
    CPU oracle's back-propagation through the recurrence as the baseline."""
    import torch

    import ssd_inputs
    import state_space_sequence_02_amd as m2

    w = workload(args.workload)
    inp = ssd_inputs.make_inputs(w)
    cot = ssd_inputs.make_cotangents(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = {k: (None if v is None else v.to(dev)) for k, v in inp.items()}
    dy, dfin = cot["dy"].to(dev), cot["dfinal"].to(dev)
    dims = m2.dims_of(g["x"], g["B"], w.chunk_size)
    need = m2.mamba2_ssd_backward_workspace_bytes(dims)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    o = {"dx": torch.empty_like(g["x"]), "ddt": torch.empty_like(g["dt"]),
         "dA": torch.empty_like(g["A"]), "dB": torch.empty_like(g["B"]),
         "dC": torch.empty_like(g["C"]), "dD": torch.empty_like(g["D"]),
         "dinit": torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.float32,
                              device=dev)}
    stream = torch.cuda.current_stream()
    a = (dims, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["init_state"], dy, dfin,
         o["dx"], o["ddt"], o["dA"], o["dB"], o["dC"], o["dD"], o["dinit"], ws, need, stream)

    for _ in range(args.warmup):
        m2.mamba2_ssd_backward(*a)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        m2.mamba2_ssd_backward(*a)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    if not backward_fast(w):
        # generic backward: one pass of float32 vector-ALU kernels, measured as
        # a whole against the fp32 vector peak
        fl = generic_backward_flops(w)
        achieved = fl / (ms * 1e-3) / 1e12
        out = {
            "metric": metric_name(w, backward=True),
            "value": w.tokens / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "f32" if w.dtype == "f32" else "f32 (bf16 operands)", "data": "synthetic",
            "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen,
                       "nheads": w.nheads, "headdim": w.headdim, "dstate": w.dstate,
                       "ngroups": w.ngroups, "chunk_size": w.chunk_size, "path": "generic",
                       "parallelism": "none (1 GPU)"},
            "roofline": {"kernel": "generic backward (all kernels)", "bound": "alu",
                         "achieved": achieved, "peak": FP32_VALU_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": achieved / FP32_VALU_PEAK_TFLOPS,
                         "traffic": None, "algorithmic_flops": fl},
        }
        print(json.dumps(out), flush=True)
        return
    ssum = [0.0] * len(BWD_STAGES)
    for _ in range(args.steps):
        ssum = [u + v for u, v in zip(ssum, m2.mamba2_ssd_backward_profile(*a))]
    stage_ms = {s: ssum[i] / args.steps for i, s in enumerate(BWD_STAGES)}
    model = backward_model(w)
    dom = max(BWD_STAGES, key=lambda s: stage_ms[s])
    dm = model[dom]
    bound = "hbm" if dm["flops"] / dm["bytes"] < RIDGE else "mfma"
    if bound == "hbm":
        achieved, peak, unit = dm["bytes"] / (stage_ms[dom] * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        achieved = dm["flops"] / (stage_ms[dom] * 1e-3) / 1e12
        peak, unit = BF16_MFMA_PEAK_TFLOPS, "TFLOP/s"
    stages = {}
    for s in BWD_STAGES:
        t = stage_ms[s] * 1e-3
        stages[s] = {"ms": round(stage_ms[s], 4),
                     "GB/s": round(model[s]["bytes"] / t / 1e9, 1),
                     "TFLOP/s": round(model[s]["flops"] / t / 1e12, 2),
                     "hbm_frac": round(model[s]["bytes"] / t / 1e9 / HBM_PEAK_GBS, 3)}
    out = {
        "metric": metric_name(w, backward=True),
        "value": w.tokens / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "nheads": w.nheads,
                   "headdim": w.headdim, "dstate": w.dstate, "ngroups": w.ngroups,
                   "chunk_size": w.chunk_size, "parallelism": "none (1 GPU)"},
        "roofline": {"kernel": dom, "bound": bound, "achieved": achieved, "peak": peak,
                     "unit": unit, "frac": achieved / peak,
                     "traffic": profiled_traffic(w.name, dom, "backward"),
                     "algorithmic_bytes": dm["bytes"], "algorithmic_flops": dm["flops"]},
        "stages": stages,
    }
    if not args.no_cpu_baseline:
        import oracle
        Ls = w.seqlen if args.cpu_tokens <= 0 else min(w.seqlen, args.cpu_tokens)
        oc = {k: (None if v is None else v[:, :Ls].float().numpy() if k in ("x", "dt", "B", "C")
                  else v.float().numpy()) for k, v in inp.items()}
        t0 = time.perf_counter()
        oracle.ssd_backward(oc["x"], oc["dt"], oc["A"], oc["B"], oc["C"], oc["D"],
                            oc["init_state"], cot["dy"][:, :Ls].float().numpy(),
                            cot["dfinal"].numpy(), chunk_size=w.chunk_size)
        sec = time.perf_counter() - t0
        out["cpu_baseline"] = {
            "value": w.batch * Ls / sec, "unit": "tokens/s", "cores": oracle.num_threads(),
            "cpu_model": cpu_model(), "kind": "oracle", "seconds": sec,
            "sample": f"first {Ls} of {w.seqlen} tokens, all {w.nheads} heads, batch {w.batch}"}
    print(json.dumps(out), flush=True)


def cpu_baseline(inp, w, tokens_per_head):
    """The CPU oracle (direct float64 recurrence, OpenMP) on the host, on a
    bounded prefix of the same inputs; tokens/s over all heads."""
    import oracle
    Ls = w.seqlen if tokens_per_head <= 0 else min(w.seqlen, tokens_per_head)
    o = {k: (None if v is None else v[:, :Ls].float().numpy() if k in ("x", "dt", "B", "C")
             else v.float().numpy()) for k, v in inp.items()}
    t0 = time.perf_counter()
    oracle.ssd_recurrence(o["x"], o["dt"], o["A"], o["B"], o["C"], o["D"], o["init_state"],
                          chunk_size=w.chunk_size, want_final=True)
    dt = time.perf_counter() - t0
    # the oracle's independent chunked form on the same sample: per-chunk
    # local states, the jump across chunks, outputs of each chunk restarted
    # from its start state
    import numpy as np
    t1 = time.perf_counter()
    cs, _ = oracle.chunk_cumsum(o["dt"], o["A"], w.chunk_size)
    S = oracle.chunk_local_states(o["x"], o["dt"], o["A"], o["B"], chunk_size=w.chunk_size)
    hs, _ = oracle.state_passing(S, np.exp2(cs[..., -1]), o["init_state"])
    del S
    oracle.chunk_outputs(o["x"], o["dt"], o["A"], o["B"], o["C"], o["D"], hs,
                         chunk_size=w.chunk_size)
    dt_chunked = time.perf_counter() - t1
    return {"value": w.batch * Ls / dt, "unit": "tokens/s", "cores": oracle.num_threads(),
            "cpu_model": cpu_model(), "kind": "oracle", "seconds": dt,
            "sample": f"first {Ls} of {w.seqlen} tokens, all {w.nheads} heads, batch {w.batch}",
            "chunked_form": {"value": w.batch * Ls / dt_chunked, "unit": "tokens/s",
                             "seconds": dt_chunked}}


if __name__ == "__main__":
    main()
