"""Parity of the forward's span path with the oracle.

For bfloat16 with headdim 64, state size 64, 128 or 256 and enough
(batch, head, span) work to give every CU a workgroup, mamba2_ssd_forward
runs fwd_pass_state over spans of K = 8 (else 4) chunks, or, at state size
64, the longest of 8, 4 or 2 chunks that fills the device with span_scan
workgroups: span-end states,
the jump across spans, and then either a replay of every span that writes the
chunk-start states for the grouped chunk_scan (state size 256 and 512), or
span_scan, the replay fused with the output stage (state size 64 and 128),
with 1, 2 or 4 heads of a group per workgroup.  These shapes meet
that rule (checked below with the device's CU count) and cover every (chunk
size, state size) pair, 1, 2 and 4 heads per workgroup, ragged last chunks, a
last span of one chunk, several groups and batches, with and without the
initial state.  y and the final state are compared with the oracle at the
bfloat16 bar (2e-2 normwise); the full-size workload (L = 64K, N = 256,
spans of 8) is covered on sampled heads by the full-size tests."""
import pytest
import torch

import oracle
import ssd_inputs
from gpu_helpers import TOL, assert_within, errors, f64, oracle_inputs, run_forward, say, to_gpu

pytestmark = pytest.mark.gpu

BT = TOL["bf16"]


@pytest.fixture(scope="module")
def m2():
    import state_space_sequence_02_amd as lib
    return lib


def _w(name, L, H, N, G, Q, Bn=1, init=True, seed=0):
    return ssd_inputs.custom(name=name, batch=Bn, seqlen=L, nheads=H, headdim=64, dstate=N,
                             ngroups=G, chunk_size=Q, init_state=init, seed=seed)


SHAPES = [
    _w("span_Q64_N64_G2_K2", 1000, 64, 64, 2, 64, seed=91),
    _w("span_Q64_N256_last_span_one_chunk", 2085, 32, 256, 1, 64, Bn=2, seed=92),
    _w("span_Q128_N128_G3_K4", 5115, 48, 128, 3, 128, init=False, seed=93),
    _w("span_Q256_N64_G4_ragged", 3996, 64, 64, 4, 256, seed=94),
    _w("span_Q128_N256_B2_K4", 4097, 16, 256, 1, 128, Bn=2, seed=95),
    _w("span_Q256_N128_K4", 4096, 64, 128, 2, 256, init=False, seed=96),
    _w("span_Q64_N128_B4", 1024, 16, 128, 1, 64, Bn=4, seed=97),
    _w("span_Q256_N256_K4", 4096, 64, 256, 1, 256, seed=98),
    # several heads per workgroup (sharing the B rows)
    _w("span_Q64_N256_R4_ragged", 8155, 64, 256, 1, 64, seed=99),
    _w("span_Q128_N128_G2_R2", 8192, 64, 128, 2, 128, Bn=2, init=False, seed=100),
    _w("span_Q256_N64_G4_R1", 8192, 32, 64, 4, 256, Bn=4, seed=101),
    # N = 64, one head per workgroup, four workgroups per CU
    _w("span_Q64_N64_R1_ragged", 2000, 64, 64, 1, 64, Bn=4, seed=102),
    # N = 512: two launches over halves of the state columns
    _w("span_Q64_N512_G4_R4_ragged", 4096 - 19, 32, 512, 4, 64, Bn=4, seed=103),
    _w("span_Q256_N512_G3_K4", 3000, 96, 512, 3, 256, init=False, seed=104),
    # N = 256, one head per workgroup, two workgroups per CU (three-buffer ring)
    _w("span_Q64_N256_G2_R1_two_per_cu", 4096 - 3, 66, 256, 2, 64, seed=105),
    # span_scan with four heads per workgroup at the chunk sizes not covered above
    _w("span_scan_Q64_N128_R4_ragged", 8192 - 45, 32, 128, 2, 64, Bn=2, seed=106),
    _w("span_scan_Q256_N64_R4", 16384 - 7, 64, 64, 4, 256, Bn=2, init=False, seed=107),
    _w("span_scan_Q128_N64_G2", 4096 + 100, 32, 64, 2, 128, Bn=2, seed=108),
]

# (span length, heads per workgroup) each shape reaches on a 256-CU device
EXPECT = {"span_Q64_N64_G2_K2": (2, 1), "span_Q64_N256_last_span_one_chunk": (4, 2), "span_Q64_N256_R4_ragged": (8, 4),
          "span_Q128_N128_G2_R2": (8, 2), "span_Q256_N64_G4_R1": (8, 1),
          "span_Q64_N64_R1_ragged": (8, 1), "span_Q64_N512_G4_R4_ragged": (8, 4),
          "span_Q256_N512_G3_K4": (4, 1), "span_Q64_N256_G2_R1_two_per_cu": (8, 1)}


def span_chunks(w, cus, forward=True):
    """The span length the forward picks for these sizes (0: no span path);
    forward=False: the backward's recompute, which keeps span_end's rule.
    At state size 64 with an even number of heads per group (span_scan): the
    longest span of 8, 4 or 2 chunks whose span_scan grid gives every CU a
    workgroup.  Otherwise, or if none does: 8 chunks if that gives every CU
    two (batch, span, head) units, else 4 if that does, else the longest span
    that gives every CU one."""
    if not (w.dtype == "bf16" and w.headdim == 64 and w.dstate in (64, 128, 256, 512)
            and w.chunk_size in (64, 128, 256)):
        return 0
    nc = -(-w.seqlen // w.chunk_size)
    hg = w.nheads // w.ngroups
    if forward and w.dstate == 64 and hg % 2 == 0:
        for K in (8, 4, 2):
            if nc < K:
                continue
            ng = -(-nc // K)
            R = 4 if (hg % 4 == 0 and w.batch * ng * w.nheads // 4 >= cus) else 2
            if w.batch * ng * w.nheads // R >= cus:
                return K
    for want in (2 * cus, cus):
        for K in (8, 4):
            if nc >= K and w.batch * w.nheads * (-(-nc // K)) >= want:
                return K
    return 0


def span_heads(w, K, cus):
    """Heads per workgroup the library picks: 4, 2 or 1 (at most 2 at N = 128
    and 1 at N = 64), a divisor of the group's heads, while the grid still
    gives every CU a workgroup."""
    nc = -(-w.seqlen // w.chunk_size)
    ng = -(-nc // K)
    max_r = 1 if w.dstate == 64 else 2 if w.dstate == 128 else 4
    for R in (4, 2):
        if (R <= max_r and (w.nheads // w.ngroups) % R == 0
                and w.batch * ng * w.nheads // R >= cus):
            return R
    return 1


def scan_heads(w, K, cus):
    """Heads per workgroup of span_scan, the span replay fused with the output
    stage (0: the replay and the grouped chunk_scan run instead): state size
    64 or 128; 4 heads where the grid still gives every CU a workgroup, else
    2; an even number of heads per group."""
    if not K or w.dstate not in (64, 128):
        return 0
    hg = w.nheads // w.ngroups
    ng = -(-(-(-w.seqlen // w.chunk_size)) // K)
    if hg % 4 == 0 and w.batch * ng * w.nheads // 4 >= cus:
        return 4
    return 2 if hg % 2 == 0 else 0


def test_span_scan_cases_cover_every_variant():
    """The shapes above reach span_scan with 2 and 4 heads per workgroup at
    state sizes 64 and 128, over every chunk size (on a 256-CU device)."""
    seen = set()
    for w in SHAPES:
        K = span_chunks(w, 256)
        r = scan_heads(w, K, 256)
        if r:
            seen.add((w.dstate, r, w.chunk_size))
    for n in (64, 128):
        for r in (2, 4):
            assert any((n, r, q) in seen for q in (64, 128, 256)), (n, r)
        assert {q for (nn, _, q) in seen if nn == n} == {64, 128, 256}, n


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
def test_span_forward_matches_oracle(m2, w):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    K = span_chunks(w, cus)
    R = span_heads(w, K, cus) if K else 0
    say(f"[span] {w} K={K} R={R} span_scan R={scan_heads(w, K, cus)}")
    assert K > 0, "shape does not reach the span path on this device"
    if cus == 256 and w.name in EXPECT:
        assert (K, R) == EXPECT[w.name]
    inp = ssd_inputs.make_inputs(w)
    o = oracle_inputs(inp)
    g = to_gpu(inp)
    y, fin = run_forward(m2, g, w.chunk_size)
    oy, ofin, _ = oracle.ssd_recurrence(o["x"], o["dt"], o["A"], o["B"], o["C"], o["D"],
                                        o["init_state"], chunk_size=w.chunk_size)
    errs = errors({"y": (f64(y), oy), "final_state": (f64(fin), ofin)})
    say(f"  errors (tensor, worst head) {errs}")
    assert_within(errs, BT)


def test_span_forward_is_deterministic(m2):
    w = SHAPES[1]
    g = to_gpu(ssd_inputs.make_inputs(w))
    y1, f1 = run_forward(m2, g, w.chunk_size)
    y2, f2 = run_forward(m2, g, w.chunk_size)
    assert torch.equal(y1, y2) and torch.equal(f1, f2)
