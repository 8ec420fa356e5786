"""Host-side checks of bench.py (no GPU): its one-GPU contract, its mirror of
the library's path choice (checked against the workspace the library plans
for the same sizes), its per-stage byte model and its reading of the
committed profiles."""
import json
import os
import subprocess
import sys

import pytest

import ssd_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

m2 = pytest.importorskip("state_space_sequence_02_amd")


def _r256(v):
    return (v + 255) & ~255


def _expected_workspace(w):
    """The forward workspace for the path bench.py predicts: cumulative sums
    and dt, then per path the state slot, the bf16 chunk-start states and the
    N = 512 partial y (none of the two when span_scan runs); the one-kernel
    forward's layout where it is supported."""
    B, L, H, P, N, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.chunk_size
    nc = -(-L // Q)
    cs = _r256(B * H * nc * Q * 4)
    hst = _r256(B * nc * H * P * N * 2)
    part = _r256(B * L * H * P * 2) if N == 512 else 0
    plan = bench.span_plan(w)
    grouped = bench.grouped_path(w)
    if plan:
        K = plan[0]
        ng = -(-nc // K)
        st = _r256(B * ng * H * P * N * 4) + _r256(B * H * ng * 4)
        rs = bench.scan_plan(w)
        total = 2 * cs + st + (0 if rs else hst + part)
    else:
        st = _r256(B * nc * H * P * N * 4)
        total = 2 * cs + st + (hst + part if grouped else 0)
    if w.dtype == "bf16" and P == 64 and N in (64, 128, 256) and Q in (64, 128, 256):
        total = max(total, 3 * cs + hst)
    return total


SHAPES = [ssd_inputs.custom(name=f"ws_{B}_{L}_{H}_{N}_{G}_{Q}", batch=B, seqlen=L, nheads=H,
                            headdim=64, dstate=N, ngroups=G, chunk_size=Q)
          for B in (1, 2) for L in (1000, 8192, 65536) for H in (8, 24, 32, 64)
          for N in (64, 128, 256, 512) for G in (1, 2) for Q in (64, 256)]


def test_bench_path_model_matches_the_library_workspace():
    """bench.py's copy of the span / span_scan rules (it names the stages and
    prices the bytes with them) agrees with the library's dispatch, as seen
    in the workspace the library asks for (the library assumes 256 CUs when
    no device is visible)."""
    bad = []
    for w in SHAPES:
        d = m2.Mamba2Dims(batch=w.batch, seqlen=w.seqlen, nheads=w.nheads, headdim=w.headdim,
                          dstate=w.dstate, ngroups=w.ngroups, chunk_size=w.chunk_size,
                          dtype=m2.MAMBA2_DTYPE_BF16, reserved=0)
        got = m2.mamba2_ssd_workspace_bytes(d)
        if got != _expected_workspace(w):
            bad.append((w.name, got, _expected_workspace(w)))
    assert not bad, bad[:5]


def test_stage_model_per_unit_bytes():
    """The per-(token, head) byte figures of the L = 64K, N = 256 path."""
    w = ssd_inputs.WORKLOADS["long_L64k_N256"]
    u = w.batch * w.seqlen * w.nheads
    m = bench.stage_model(w)
    assert bench.span_plan(w) == (8, 4) and bench.scan_plan(w) is None
    assert m["chunk_scan"]["bytes"] / u == pytest.approx(424, abs=0.01)
    assert m["span_end"]["bytes"] / u == pytest.approx(184, abs=0.01)
    assert m["chunk_cumsum"]["bytes"] / u == pytest.approx(10, abs=0.01)
    assert bench.forward_stages(w) == ("chunk_cumsum", "span_end", "span_pass", "chunk_scan")
    w2 = bench.workload("sweep_L64k_N128")
    assert bench.scan_plan(w2) == 4
    assert bench.forward_stages(w2) == ("chunk_cumsum", "span_end", "span_jump", "span_scan")
    assert bench.stage_model(w2)["span_scan"]["bytes"] / u == pytest.approx(296, abs=0.01)


def test_committed_profiles_parse():
    """Each committed forward summary yields the traffic of every stage whose
    sources still match the digest recorded with it."""
    for name in ("long_L64k_N256", "longest_L256k_N512", "sweep_L64k_N128"):
        w = bench.workload(name)
        text = open(os.path.join(ROOT, "profiles", f"ssd_forward_{name}.md")).read()
        for st in bench.forward_stages(w):
            t = bench.profiled_traffic(name, st)
            current = f"sources-sha256 {st}: {bench.sources_digest(st)}" in text
            assert (t is not None) == current, (name, st)
            if t is not None:
                assert 0.9 < t / bench.stage_model(w)[st]["bytes"] < 1.6, (name, st, t)


def test_committed_backward_profile_parses():
    """The backward summary yields every stage's traffic while its sources
    match; its recompute stages are the forward's span kernels at this shape,
    so their digests cover state_span.hip."""
    name = "long_L64k_N256"
    w = bench.workload(name)
    text = open(os.path.join(ROOT, "profiles", f"ssd_backward_{name}.md")).read()
    assert bench.stage_sources("chunk_state", "backward", name) == bench.KERNEL_SOURCES["span_end"]
    assert bench.stage_sources("chunk_state") == bench.KERNEL_SOURCES["chunk_state"]
    model = bench.backward_model(w)
    for st in ("chunk_cumsum", "chunk_state", "state_passing", "adjoint_state", "reverse_pass",
               "dB_dC", "dx"):
        t = bench.profiled_traffic(name, st, "backward")
        current = f"sources-sha256 {st}: {bench.sources_digest(st, 'backward', name)}" in text
        assert (t is not None) == current, st
        if t is not None:
            assert 0.9 < t / model[st]["bytes"] < 1.6, (st, t)


def test_workload_names():
    w = bench.workload("sweep_L16k_N64")
    assert (w.seqlen, w.dstate, w.nheads, w.headdim, w.chunk_size) == (16384, 64, 32, 64, 256)
    with pytest.raises(SystemExit):
        bench.workload("nonsense")


def test_metric_names():
    """The headline workload reports the headline metric; any other workload
    names itself, so its line is never mistaken for the headline's."""
    head = bench.workload(bench.HEADLINE)
    assert bench.metric_name(head) == bench.METRIC
    other = bench.workload("longest_L256k_N512")
    assert "longest_L256k_N512" in bench.metric_name(other)
    assert "longest_L256k_N512" in bench.metric_name(other, backward=True)
    assert "L=64K,N=256" in bench.metric_name(head, backward=True)


def test_backward_fast_path_rule():
    """bench's model of which sizes take the MFMA backward matches the
    library's rule: bf16, head size 64, state 64/128/256 with chunk 64-256,
    or state 512 with chunk 256."""
    cases = [((64, 256, "bf16", 64), True), ((512, 256, "bf16", 64), True),
             ((512, 128, "bf16", 64), False), ((256, 64, "f32", 64), False),
             ((256, 256, "bf16", 32), False), ((96, 128, "bf16", 64), False)]
    for (N, Q, dt, P), fast in cases:
        w = ssd_inputs.custom(name="m", batch=1, seqlen=512, nheads=2, headdim=P, dstate=N,
                              ngroups=1, chunk_size=Q, dtype=dt, init_state=False, seed=0)
        assert bench.backward_fast(w) == fast, (N, Q, dt, P)


@pytest.mark.parametrize("extra", [[], ["--backward"]])
def test_more_than_one_gpu_is_refused(extra):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", *extra],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]
