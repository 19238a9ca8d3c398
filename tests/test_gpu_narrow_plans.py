"""GPU parity of the default launches on matrices of at most 256 column tiles, where the planner
balances the compute units: the K splits per tile that minimise the busiest CU's share of the
work, 16 waves per workgroup (8 for short pieces up to 8 rows). Each shape's launch is checked
against the rule, its fp32 output against the oracle on sampled columns that include the last
tile, and a repeat for bit-identity.
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


# (M, K, N, g, symmetric, (splits, waves_k) of the default launch)
CASES = [
    (16, 5120, 5120, 128, True, (3, 16)),     # attention, 80 tiles
    (2, 5120, 5120, 128, True, (3, 8)),       # short pieces at few rows: 8 waves
    (1, 5120, 13824, 128, True, (1, 16)),     # 216 tiles: whole K in one workgroup (the GEMV)
    (16, 2048, 13824, 128, False, (1, 16)),   # the same on the matrix cores, stored zero points
    (1, 3072, 2048, 64, False, (8, 8)),       # 32 tiles
    (16, 5120, 4096, 128, True, (4, 16)),     # 64 tiles
    (12, 4096, 8192, 64, False, (2, 16)),     # 128 tiles
    (5, 1024, 1000, 32, False, (16, 2)),      # 16 tiles (ragged), 32 K steps
]


@pytest.mark.parametrize("M,K,N,g,sym,launch", CASES)
def test_narrow_default_launch_parity(gu, M, K, N, g, sym, launch):
    kern, splits, wk, cols = vm.w4a16_plan(M, N, K, g)
    assert (splits, wk) == launch and cols == 64 and kern == (0 if M == 1 else 1), (kern, splits, wk, cols)
    inp = synth.make_random(9500 + M + K // 64 + N // 8, M, K, N, g, symmetric=sym)
    d = gu.DevInputs(inp)
    gu.say(f"[narrow plan] M={M} K={K} N={N} g={g} sym={sym} plan={(kern, splits, wk, cols)}")
    y = d.run(M)
    rng = np.random.default_rng(M + N)
    c = np.unique(np.concatenate([rng.choice(N, min(N, 400), replace=False), np.arange(max(0, N - 70), N)]))
    y_ref, bound = oracle.gemm(inp.act, inp.qweight, inp.scales, inp.qzeros, g, c)
    frac = parity.check_close(y[:, c], y_ref, bound, f"narrow plan M={M} K={K} N={N}")
    gu.say(f"  worst err/tol {frac:.3e}")
    assert np.array_equal(d.run(M), y)   # bit-identical repeat


def test_prompt_gemm_two_slices_just_past_a_round(gu):
    """Stored zero points at 2048 rows x 5120 columns: 640 tiles, one and a quarter rounds of the
    2 workgroups a CU holds, so the call cuts K in two. Checked on sampled rows (the oracle's rows
    are independent) and sampled columns that include the last tile, and for bit-identity."""
    M, K, N, g = 2048, 2048, 5120, 64
    inp = synth.make_random(9600, M, K, N, g, symmetric=False)
    d = gu.DevInputs(inp)
    gu.say(f"[prompt GEMM two slices] M={M} K={K} N={N} g={g}")

    def run():
        out = torch.empty((M, N), dtype=torch.float32, device=gu.DEV)
        vm.w4a16_gemm_prefill(d.act, d.qweight, d.scales, d.qzeros, g, out)
        torch.cuda.synchronize()
        return out.cpu().numpy().astype(np.float64)

    y = run()
    rng = np.random.default_rng(9600)
    rows = np.unique(np.concatenate([rng.choice(M, 48, replace=False), np.arange(M - 32, M)]))
    cols = np.unique(np.concatenate([rng.choice(N, 300, replace=False), np.arange(N - 70, N)]))
    y_ref, bound = oracle.gemm(inp.act[rows], inp.qweight, inp.scales, inp.qzeros, g, cols)
    frac = parity.check_close(y[rows][:, cols], y_ref, bound, "prompt GEMM two slices")
    gu.say(f"  worst err/tol {frac:.3e}")
    assert np.array_equal(run(), y)   # bit-identical repeat
