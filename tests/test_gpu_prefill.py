"""GPU parity of the many-row (prompt-processing) GEMM, w4a16_gemm_prefill, against the oracle.

Same bar as the small-row path (tests/parity.py). Rows are independent, so permuting the rows
of A permutes the output rows bit for bit; integer inputs with unit scales give exact results.
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


def run(gu, d, act, out_dtype=torch.float32):
    M = act.shape[0]
    out = torch.empty((M, d.N), dtype=out_dtype, device=gu.DEV)
    vm.w4a16_gemm_prefill(act, d.qweight, d.scales, d.qzeros, d.group, out)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


# (M, K, N, g, sym): ragged M and N (not multiples of the 128 x 128 tile), both zero-point forms
SHAPES = [(17, 512, 200, 128, True), (130, 1024, 264, 64, False), (300, 2048, 136, 128, True),
          (256, 512, 512, 32, False), (1, 256, 72, 64, True), (513, 1024, 392, 128, False)]


@pytest.mark.parametrize("M,K,N,g,sym", SHAPES)
def test_prefill_parity(gu, M, K, N, g, sym):
    inp = synth.make_random(90 + M, M, K, N, g, symmetric=sym)
    d = gu.DevInputs(inp)
    gu.say(f"[prefill] M={M} K={K} N={N} g={g} sym={sym}")
    y = run(gu, d, d.act)
    y_ref, bound = oracle.gemm(inp.act, inp.qweight, inp.scales, inp.qzeros, g)
    frac = parity.check_close(y, y_ref, bound, f"prefill M={M} K={K} N={N}")
    gu.say(f"  worst err/tol {frac:.3e}")
    yb = run(gu, d, d.act, torch.bfloat16)
    assert np.array_equal(yb, torch.from_numpy(y.astype(np.float32)).to(torch.bfloat16).double().numpy())


def test_prefill_integer_exact_and_row_permutation(gu):
    rng = np.random.default_rng(91)
    M, K, N, g = 200, 2048, 264, 64
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    zeros = rng.integers(0, 16, size=(K // g, N), dtype=np.uint8)
    ai = rng.integers(-8, 9, size=(M, K))
    inp = synth.Inputs(synth.pack_rows(codes), np.full((K // g, N), 0x3C00, np.uint16), synth.pack_cols(zeros),
                       synth.f32_to_bf16_bits(ai.astype(np.float32)), g)
    d = gu.DevInputs(inp)
    y = run(gu, d, d.act)
    dq = codes.astype(np.int64) - np.repeat(zeros.astype(np.int64), g, axis=0)
    assert np.array_equal(y, (ai.astype(np.int64) @ dq).astype(np.float64))
    perm = rng.permutation(M)
    assert np.array_equal(run(gu, d, gu.dev_u16(inp.act[perm])), y[perm])
    for _ in range(3):
        assert np.array_equal(run(gu, d, d.act), y)


def test_prefill_matches_small_row_path_within_the_bar(gu):
    """Rows 0..15 through the prompt kernel and through the small-row kernel: both within the bar
    of the oracle (different K splits round differently)."""
    inp = synth.make_random(92, 16, 2048, 520, 128, symmetric=False)
    d = gu.DevInputs(inp)
    y_ref, bound = oracle.gemm(inp.act, inp.qweight, inp.scales, inp.qzeros, 128)
    parity.check_close(run(gu, d, d.act), y_ref, bound, "prefill 16 rows")
    parity.check_close(d.run(16), y_ref, bound, "small-row 16 rows")


@pytest.mark.parametrize("name,M", [("ffn_up", 512), ("ffn_down", 300)])
def test_prefill_workloads(gu, name, M):
    """The FFN matrices with a prompt-sized block of rows (activations drawn with the workload's
    distribution), on a sample of columns that spans every tile position and the last tile."""
    wl = synth.WORKLOADS[name]
    inp = synth.make_inputs(wl)
    rng = np.random.Generator(np.random.PCG64(1000 * wl.index + 8))
    act = synth.draw_activations(rng, M, wl.K, wl.act_sigma, wl.outlier_frac, wl.outlier_mul)
    d = gu.DevInputs(inp)
    gu.say(f"[prefill workload] {name} M={M}")
    y = run(gu, d, gu.dev_u16(act))
    cols = np.unique(np.concatenate([rng.choice(inp.N, 600, replace=False), np.arange(inp.N - 130, inp.N)]))
    y_ref, bound = oracle.gemm(act, inp.qweight, inp.scales, inp.qzeros, wl.group, cols)
    frac = parity.check_close(y[:, cols], y_ref, bound, f"prefill {name} M={M}")
    gu.say(f"  worst err/tol {frac:.3e}")
