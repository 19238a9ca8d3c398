"""Calls captured into a HIP graph and replayed: every replay gives the oracle's results.

The decode loops of the pages capture a step once and replay it for every token (lucebox PR
#823, commit messages: one graph launch per steady-state token; TensorFold PR #859, commit
messages: forwards captured the first time a shape is seen and replayed after). A replay runs
the captured kernels with the captured arguments, so nothing a call needs may come from host
state that changes between calls: the split-K reduction keeps its counters and slice flags on
the device and returns them to zero in every call. Here a stream is warmed up (its scratch is
allocated then), the calls are captured, and the graph is replayed twelve times with new
activations copied into the captured input buffer between replays (outside the graph, with
the program's own eager work and synchronisations in between); every replay is checked
against the oracle, and the fused pick against the host's pick over the replay's own logits.
"""
import numpy as np
import pytest
import torch

import oracle
import verify_matmul_amd as vm
from tests import parity
from verify_matmul_amd import synth

pytestmark = pytest.mark.gpu

REPLAYS = 12


@pytest.fixture(scope="module")
def gu():
    from tests import gpu_util
    vm.load()
    return gpu_util


def test_graph_replay_matches_the_oracle(gu):
    K, N, g = 2048, 1000, 128            # 16 tiles of 64 columns, the last one ragged
    Mg, Ma, Mp = 5, 5, 3                 # rows of the plain GEMMs, the fused pick, the gated pair
    w = synth.make_random(9101, 16, K, N, g, symmetric=False)
    w_sym = synth.make_random(9102, 16, K, N, g, symmetric=True)
    gate = synth.make_random(9103, 16, K, N, g, symmetric=True)
    dw, ds, dg = gu.DevInputs(w), gu.DevInputs(w_sym), gu.DevInputs(gate)
    a_buf = torch.zeros((16, K), dtype=torch.int16, device=gu.DEV)   # the captured input

    o_split = torch.empty((Mg, N), dtype=torch.float32, device=gu.DEV)
    o_one = torch.empty((1, N), dtype=torch.float32, device=gu.DEV)
    o_def = torch.empty((16, N), dtype=torch.float32, device=gu.DEV)
    o_amax = torch.empty((Ma, N), dtype=torch.float32, device=gu.DEV)
    idx = torch.full((Ma,), -1, dtype=torch.int32, device=gu.DEV)
    o_pair = torch.empty((Mp, N), dtype=torch.float32, device=gu.DEV)

    def calls():
        # an explicit split-K launch (4 workgroups per tile, 2 waves each), the default launches at
        # one and sixteen rows, the fused pick, and the gated pair split along K
        vm.w4a16_gemm_ex(a_buf[:Mg], dw.qweight, dw.scales, dw.qzeros, g, o_split, 4, 2)
        vm.w4a16_gemm(a_buf[:1], ds.qweight, ds.scales, None, g, o_one)
        vm.w4a16_gemm(a_buf[:16], dw.qweight, dw.scales, dw.qzeros, g, o_def)
        vm.w4a16_gemm_argmax(a_buf[:Ma], ds.qweight, ds.scales, None, g, o_amax, idx)
        vm.w4a16_gemm_gate_up(a_buf[:Mp], (dg.qweight, dg.scales, None), (ds.qweight, ds.scales, None), g,
                              o_pair, splits=4, waves_k=2)

    for M in (1, 16):
        kern, splits, wk, cols = vm.w4a16_plan(M, N, K, g)
        gu.say(f"[graph] default plan M={M}: kernel={kern} splits={splits} waves_k={wk} tile_cols={cols}")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        calls()   # warm-up: allocates the stream's scratch
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        calls()
    torch.cuda.synchronize()

    rng = np.random.default_rng(9104)
    for r in range(REPLAYS):
        act = synth.f32_to_bf16_bits(rng.standard_normal((16, K)).astype(np.float32) * np.float32(1 + r))
        a_buf.copy_(torch.from_numpy(act.view(np.int16)))
        for t in (o_split, o_one, o_def, o_amax, o_pair):
            t.fill_(float("nan"))
        idx.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        gu.say(f"[graph] replay {r}")
        y, b = oracle.gemm(act[:Mg], w.qweight, w.scales, w.qzeros, g)
        parity.check_close(o_split.cpu().numpy(), y, b, f"replay {r}: split-K GEMM")
        y, b = oracle.gemm(act[:1], w_sym.qweight, w_sym.scales, None, g)
        parity.check_close(o_one.cpu().numpy(), y, b, f"replay {r}: one-row GEMM")
        y, b = oracle.gemm(act[:16], w.qweight, w.scales, w.qzeros, g)
        parity.check_close(o_def.cpu().numpy(), y, b, f"replay {r}: 16-row GEMM")
        y, b = oracle.gemm(act[:Ma], w_sym.qweight, w_sym.scales, None, g)
        logits = o_amax.cpu().numpy()
        parity.check_close(logits, y, b, f"replay {r}: fused pick's logits")
        assert np.array_equal(idx.cpu().numpy().astype(np.int64), oracle.argmax_rows_f32(logits)), f"replay {r}"
        h = oracle.gate_up(act[:Mp], (gate.qweight, gate.scales, None), (w_sym.qweight, w_sym.scales, None), g)
        parity.check_gate_up(o_pair.cpu().numpy(), *h, f"replay {r}: gated pair")


def test_graph_replay_of_the_wide_matrix_kernel(gu):
    """The same on a matrix wide enough for the decode kernel (the output layer's path): default
    launches at one, five and sixteen rows (K slices exchanged through slice flags), the fused
    greedy pick and the fused top-8 on it (the last group to finish lowers the pick's counter in
    every replay), and an explicit launch of three slices with a top-4."""
    K, N, g = 1024, 70000, 128           # 137 groups of 512 columns, the last one ragged
    w = synth.make_random(9201, 16, K, N, g, symmetric=False)
    d = gu.DevInputs(w)
    a_buf = torch.zeros((16, K), dtype=torch.int16, device=gu.DEV)
    outs = {M: torch.empty((M, N), dtype=torch.float32, device=gu.DEV) for M in (1, 5, 16)}
    o_pick = torch.empty((5, N), dtype=torch.float32, device=gu.DEV)
    o_ex = torch.empty((16, N), dtype=torch.float32, device=gu.DEV)
    idx = torch.full((5,), -1, dtype=torch.int32, device=gu.DEV)
    idx_ex = torch.full((16, 4), -1, dtype=torch.int32, device=gu.DEV)
    o_top = torch.empty((5, N), dtype=torch.float32, device=gu.DEV)
    idx_top = torch.full((5, 8), -1, dtype=torch.int32, device=gu.DEV)
    for M in (1, 5, 16):
        kern, slices, kw, cols = vm.w4a16_plan(M, N, K, g)
        gu.say(f"[graph wide] default plan M={M}: kernel={kern} slices={slices} kw={kw} tile_cols={cols}")
        assert kern == (2 if M == 1 else 3)

    def calls():
        for M in (1, 5, 16):
            vm.w4a16_gemm(a_buf[:M], d.qweight, d.scales, d.qzeros, g, outs[M])
        vm.w4a16_gemm_argmax(a_buf[:5], d.qweight, d.scales, d.qzeros, g, o_pick, idx)
        vm.w4a16_gemm_decode_ex(a_buf[:16], d.qweight, d.scales, d.qzeros, g, o_ex, 3, 8, 1, 64, 4, idx=idx_ex)
        vm.w4a16_gemm_topk(a_buf[:5], d.qweight, d.scales, d.qzeros, g, o_top, idx_top)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        calls()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        calls()
    torch.cuda.synchronize()

    rng = np.random.default_rng(9202)
    for r in range(REPLAYS):
        act = synth.f32_to_bf16_bits(rng.standard_normal((16, K)).astype(np.float32) * np.float32(1 + r))
        a_buf.copy_(torch.from_numpy(act.view(np.int16)))
        for t in (*outs.values(), o_pick, o_ex, o_top):
            t.fill_(float("nan"))
        idx.fill_(-1)
        idx_ex.fill_(-1)
        idx_top.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        gu.say(f"[graph wide] replay {r}")
        y16, b16 = oracle.gemm(act, w.qweight, w.scales, w.qzeros, g)
        for M in (1, 5, 16):
            y, b = (y16, b16) if M == 16 else oracle.gemm(act[:M], w.qweight, w.scales, w.qzeros, g)
            parity.check_close(outs[M].cpu().numpy(), y, b, f"replay {r}: {M}-row GEMM")
        y5, b5 = oracle.gemm(act[:5], w.qweight, w.scales, w.qzeros, g)
        logits = o_pick.cpu().numpy()
        parity.check_close(logits, y5, b5, f"replay {r}: fused pick's logits")
        assert np.array_equal(idx.cpu().numpy().astype(np.int64), oracle.argmax_rows_f32(logits)), f"replay {r}"
        logits = o_ex.cpu().numpy()
        parity.check_close(logits, y16, b16, f"replay {r}: three-slice launch")
        assert np.array_equal(idx_ex.cpu().numpy().astype(np.int64), oracle.topk_rows_f32(logits, 4)), f"replay {r}"
        logits = o_top.cpu().numpy()
        parity.check_close(logits, y5, b5, f"replay {r}: top-8 logits")
        assert np.array_equal(idx_top.cpu().numpy().astype(np.int64), oracle.topk_rows_f32(logits, 8)), f"replay {r}"


def test_capture_that_needs_scratch_is_refused(gu):
    """A call that would have to allocate scratch during capture fails cleanly instead."""
    K, N, g = 1024, 512, 128
    w = synth.make_random(9105, 4, K, N, g, symmetric=True)
    d = gu.DevInputs(w)
    out = torch.empty((4, N), dtype=torch.float32, device=gu.DEV)
    s = torch.cuda.Stream()   # never used before: it holds no scratch
    graph = torch.cuda.CUDAGraph()
    with pytest.raises(vm.W4A16Error) as err:
        with torch.cuda.graph(graph, stream=s):
            vm.w4a16_gemm_ex(d.act[:4], d.qweight, d.scales, None, g, out, 4, 2)
    assert err.value.status == -2
    torch.cuda.synchronize()
    # the stream still works once warmed up eagerly
    with torch.cuda.stream(s):
        vm.w4a16_gemm_ex(d.act[:4], d.qweight, d.scales, None, g, out, 4, 2)
    torch.cuda.synchronize()
    y, b = oracle.gemm(w.act[:4], w.qweight, w.scales, None, g)
    parity.check_close(out.cpu().numpy(), y, b, "after a refused capture")
