"""The output-layer call with the greedy pick fused into the GEMM epilogue (w4a16_gemm_argmax).

Its logits must equal w4a16_gemm's bit for bit (same launch, same arithmetic) and its indices
must equal the standalone pick (w4a16_argmax_rows) over those fp32 logits; the logits are also
checked against the oracle.
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


def fused_vs_separate(gu, d, M, out_dtype=torch.float32):
    out_f = torch.empty((M, d.N), dtype=out_dtype, device=gu.DEV)
    idx_f = torch.full((M,), -7, dtype=torch.int32, device=gu.DEV)
    vm.w4a16_gemm_argmax(d.act[:M], d.qweight, d.scales, d.qzeros, d.group, out_f, idx_f)
    out_s = torch.empty((M, d.N), dtype=out_dtype, device=gu.DEV)
    vm.w4a16_gemm(d.act[:M], d.qweight, d.scales, d.qzeros, d.group, out_s)
    # the standalone pick runs on fp32 logits: take them from the fp32 call
    out32 = torch.empty((M, d.N), dtype=torch.float32, device=gu.DEV)
    vm.w4a16_gemm(d.act[:M], d.qweight, d.scales, d.qzeros, d.group, out32)
    idx_s = torch.empty((M,), dtype=torch.int32, device=gu.DEV)
    vm.w4a16_argmax_rows(out32, idx_s)
    torch.cuda.synchronize()
    assert torch.equal(out_f.view(torch.int16) if out_dtype == torch.bfloat16 else out_f.view(torch.int32),
                       out_s.view(torch.int16) if out_dtype == torch.bfloat16 else out_s.view(torch.int32))
    assert idx_f.cpu().tolist() == idx_s.cpu().tolist()
    return out32.double().cpu().numpy(), idx_f.cpu().numpy()


SHAPES = [(512, 256, 128, True), (1024, 1000, 64, False), (2048, 40, 128, True), (5120, 5120, 128, True),
          (4096, 33000, 64, False)]


@pytest.mark.parametrize("K,N,g,sym", SHAPES)
def test_fused_pick_matches_separate(gu, K, N, g, sym):
    inp = synth.make_random(K + N, 16, K, N, g, sym)
    d = gu.DevInputs(inp)
    for M in (1, 2, 5, 8, 16):
        gu.say(f"[fused argmax] K={K} N={N} g={g} sym={sym} M={M} plan={vm.w4a16_plan(M, N, K, g)}")
        y, idx = fused_vs_separate(gu, d, M)
        y_ref, bound = oracle.gemm(inp.act[:M], inp.qweight, inp.scales, inp.qzeros, g)
        parity.check_close(y, y_ref, bound, f"fused K={K} N={N} M={M}")
        assert idx.tolist() == np.argmax(y, axis=1).tolist()   # numpy: first maximum of the same values
    fused_vs_separate(gu, d, 5, torch.bfloat16)


def test_fused_pick_output_layer(gu):
    inp = synth.make_inputs("lm_head")
    d = gu.DevInputs(inp)
    for M in (5, 1):
        gu.say(f"[fused argmax] output layer M={M}")
        y, idx = fused_vs_separate(gu, d, M)
        assert idx.tolist() == np.argmax(y, axis=1).tolist()


def test_fused_pick_ties_take_the_lowest_index(gu):
    """Zero scales make every logit 0: every row picks column 0. Equal columns tie exactly."""
    rng = np.random.default_rng(31)
    K, N, g = 1024, 520, 128
    inp = synth.make_random(32, 16, K, N, g, True)
    zero = synth.Inputs(inp.qweight, np.zeros_like(inp.scales), None, inp.act, g)
    _, idx = fused_vs_separate(gu, gu.DevInputs(zero), 4)
    assert idx.tolist() == [0, 0, 0, 0]
    # copy column 7 over columns 300 and 519: the maximum (if it is column 7) ties three ways
    qw = inp.qweight.copy()
    sc = inp.scales.copy()
    for c in (300, 519):
        qw[:, c] = qw[:, 7]
        sc[:, c] = sc[:, 7]
    act = inp.act.copy()
    tie = synth.Inputs(qw, sc, None, act, g)
    y, idx = fused_vs_separate(gu, gu.DevInputs(tie), 16)
    for m in range(16):
        if y[m, 7] == y[m].max():
            assert idx[m] == 7


def test_draft_vocabulary_subset(gu):
    """Drafted tokens scored against only the first n rows of the output layer: strix-llama.cpp
    PR #105 (commit messages) copies those rows once at load time. In this layout that copy is a
    [K/8, n] matrix of the head's first n columns, so the fused pick over it is the greedy choice
    among those n tokens of the full head: its logits meet the bar against the full head's first
    n columns, and its index is the oracle's wherever the top-2 gap exceeds the error bound."""
    K, N_full, g, n, M = 2048, 40000, 128, 16384, 16
    inp = synth.make_random(31, M, K, N_full, g, symmetric=True)
    draft = synth.Inputs(np.ascontiguousarray(inp.qweight[:, :n]), np.ascontiguousarray(inp.scales[:, :n]), None,
                         inp.act, g)
    d = gu.DevInputs(draft)
    logits, idx = fused_vs_separate(gu, d, M)
    y_ref, bound = oracle.gemm(inp.act[:M], inp.qweight, inp.scales, None, g, cols=np.arange(n))
    parity.check_close(logits, y_ref, bound, "draft head")
    checked = 0
    for m in range(M):
        top, second = np.argsort(-y_ref[m], kind="stable")[:2]
        if y_ref[m, top] - y_ref[m, second] > 2 * parity.tolerance(bound[m, [top, second]]).max():
            assert idx[m] == top
            checked += 1
    assert checked >= 2
