"""Library state across calls: per-stream scratch, split-K stamps, prepared activations.

Every call on a stream reuses that stream's scratch block (tile counters, stamped split-K
slices, prepared activations), and the block grows when a later call needs more. These tests
interleave shapes and launches so that stale state from an earlier call would show up in a
later one, and run two streams at once.
"""
import numpy as np
import pytest
import torch

import oracle
import verify_matmul_amd as vm
from tests import parity
from verify_matmul_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gu():
    from tests import gpu_util
    vm.load()
    return gpu_util


# (K, N, g, symmetric, M, splits, waves_k): small and large slices, staged and prepared
# activations, growing and shrinking scratch, the same shape again after a different one.
SEQUENCE = [
    (1024, 520, 64, False, 1, 4, 2),
    (2048, 776, 128, True, 16, 8, 2),     # many rows: partials, prepared activations
    (1024, 520, 64, False, 1, 4, 2),      # same shape again: a fresh stamp must be waited for
    (4096, 264, 4096, False, 16, 1, 1),   # one piece per tile: a 128-step slice, prepared
    (512, 256, 128, True, 5, 2, 8),
    (2048, 776, 128, True, 16, 8, 2),
    (768, 1000, 64, True, 3, 3, 1),
    (2048, 776, 128, True, 9, 16, 4),     # grows the partials again
    (1024, 520, 64, False, 2, 4, 2),
]


def test_interleaved_shapes_on_one_stream(gu):
    cache = {}
    for i, (K, N, g, sym, M, splits, wk) in enumerate(SEQUENCE):
        key = (K, N, g, sym)
        if key not in cache:
            inp = synth.make_random(K + 3 * N + g, 16, K, N, g, sym)
            cache[key] = (inp, gu.DevInputs(inp))
        inp, d = cache[key]
        gu.say(f"[sequence {i}] K={K} N={N} g={g} sym={sym} M={M} splits={splits} waves_k={wk}")
        y_ref, bound = oracle.gemm(inp.act[:M], inp.qweight, inp.scales, inp.qzeros, g)
        y = d.run(M, splits=splits, waves_k=wk)
        parity.check_close(y, y_ref, bound, f"sequence step {i}")
        # the same call again gives the same bits
        assert np.array_equal(d.run(M, splits=splits, waves_k=wk), y)


def test_two_streams_at_once(gu):
    """Calls on two streams share no scratch: both run concurrently and both are right."""
    a = synth.make_random(11, 16, 2048, 1032, 128, True)
    b = synth.make_random(12, 16, 1024, 776, 64, False)
    da, db = gu.DevInputs(a), gu.DevInputs(b)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for rep in range(3):
        oa = torch.empty((16, a.N), dtype=torch.float32, device=gu.DEV)
        ob = torch.empty((1, b.N), dtype=torch.float32, device=gu.DEV)
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            vm.w4a16_gemm_ex(da.act[:16], da.qweight, da.scales, None, 128, oa, 4, 8, stream=s1)
        with torch.cuda.stream(s2):
            vm.w4a16_gemm_ex(db.act[:1], db.qweight, db.scales, db.qzeros, 64, ob, 8, 4, stream=s2)
        torch.cuda.synchronize()
        outs.append((oa.double().cpu().numpy(), ob.double().cpu().numpy()))
    ya, ba = oracle.gemm(a.act[:16], a.qweight, a.scales, None, 128)
    yb, bb = oracle.gemm(b.act[:1], b.qweight, b.scales, b.qzeros, 64)
    for rep, (oa, ob) in enumerate(outs):
        gu.say(f"[two streams] repeat {rep}")
        parity.check_close(oa, ya, ba, f"stream 1 repeat {rep}")
        parity.check_close(ob, yb, bb, f"stream 2 repeat {rep}")
        assert np.array_equal(oa, outs[0][0]) and np.array_equal(ob, outs[0][1])


def test_release_scratch_then_call_again(gu):
    """After the library frees its scratch, the next call allocates a fresh block and is right."""
    inp = synth.make_random(13, 16, 2048, 520, 128, False)
    d = gu.DevInputs(inp)
    y_ref, bound = oracle.gemm(inp.act[:4], inp.qweight, inp.scales, inp.qzeros, 128)
    first = d.run(4, splits=4, waves_k=4)
    torch.cuda.synchronize()
    vm.w4a16_release_scratch()
    second = d.run(4, splits=4, waves_k=4)
    parity.check_close(second, y_ref, bound, "after release")
    assert np.array_equal(first, second)


def test_every_entry_point_interleaved_on_one_stream(gu):
    """The small-row GEMM, the gated pair and the many-row GEMM share one stream's scratch
    (counters, stamped slices, prepared activations, K-slice sums) and grow it in turn: each
    call's result equals the same call made alone on a fresh scratch block."""
    K, N, g = 2048, 1032, 64
    gate = synth.make_random(41, 300, K, N, g, symmetric=False)
    up = synth.make_random(42, 300, K, N, g, symmetric=False)
    up = synth.Inputs(up.qweight, up.scales, up.qzeros, gate.act, g)
    dg, du = gu.DevInputs(gate), gu.DevInputs(up)

    def small(M):
        out = torch.empty((M, N), dtype=torch.float32, device=gu.DEV)
        vm.w4a16_gemm(du.act[:M], du.qweight, du.scales, du.qzeros, g, out)
        return out

    def pair(M):
        out = torch.empty((M, N), dtype=torch.float32, device=gu.DEV)
        vm.w4a16_gemm_gate_up(du.act[:M], (dg.qweight, dg.scales, dg.qzeros), (du.qweight, du.scales, du.qzeros),
                              g, out)
        return out

    def many(M):
        out = torch.empty((M, N), dtype=torch.float32, device=gu.DEV)
        vm.w4a16_gemm_prefill(du.act[:M], du.qweight, du.scales, du.qzeros, g, out)
        return out

    calls = [(small, 16), (many, 300), (pair, 5), (small, 1), (many, 40), (pair, 16), (many, 300), (small, 16)]
    alone = {}
    for fn, M in set(calls):
        torch.cuda.synchronize()
        vm.w4a16_release_scratch()
        r = fn(M)
        torch.cuda.synchronize()
        alone[(fn.__name__, M)] = r.cpu().numpy()
    torch.cuda.synchronize()
    vm.w4a16_release_scratch()
    outs = [(fn.__name__, M, fn(M)) for fn, M in calls]   # queued back to back, one stream
    torch.cuda.synchronize()
    for i, (name, M, o) in enumerate(outs):
        gu.say(f"[interleaved] call {i}: {name} M={M}")
        assert np.array_equal(o.cpu().numpy(), alone[(name, M)]), (i, name, M)
    y_ref, bound = oracle.gemm(up.act[:300], up.qweight, up.scales, up.qzeros, g)
    parity.check_close(alone[("many", 300)].astype(np.float64), y_ref, bound, "many-row alone")
