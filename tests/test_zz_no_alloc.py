"""w4a16_gemm_noalloc, the entry point that allocates nothing, against w4a16_gemm.

Called through the C ABI (the ctypes binding) twice in a row on the same GPU, the second call
with a smaller input than the first, so the second runs on the array the first left behind.
Each output must be within the parity bar of w4a16_gemm's output for the same inputs (the bound
is the oracle's sum of |a * w|), and within the bar of the oracle itself.
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


# (seed, M, K, N, group, symmetric), each call smaller than the one before: two matrices wide
# enough for the decode kernel (the first, 16 rows over 70000 columns, needs fewer K slices than
# its default launch to fit the array; the second is one row of 65536 columns), then the
# small-row kernel: split-K partials of 1 MiB at 16 rows with packed zero points, a ragged N,
# and the one-row GEMV
CALLS = [(9204, 16, 1024, 70000, 128, False), (9205, 1, 512, 65536, 64, True), (9201, 16, 2048, 8192, 128, False),
         (9202, 3, 1024, 520, 64, True), (9203, 1, 512, 256, 128, True)]


def test_noalloc_matches_gemm_on_consecutive_calls(gu):
    s = torch.cuda.Stream()
    for seed, M, K, N, g, sym in CALLS:
        inp = synth.make_random(seed, M, K, N, g, symmetric=sym)
        d = gu.DevInputs(inp)
        kern, splits, wk, cols = vm.w4a16_plan(M, N, K, g)
        gu.say(f"[noalloc] M={M} K={K} N={N} g={g} sym={sym} plan kernel={kern} splits={splits} waves_k={wk}")
        out_na = torch.full((M, N), float("nan"), dtype=torch.float32, device=gu.DEV)
        out_ref = torch.full((M, N), float("nan"), dtype=torch.float32, device=gu.DEV)
        with torch.cuda.stream(s):
            vm.w4a16_gemm_noalloc(d.act[:M], d.qweight, d.scales, d.qzeros, g, out_na)
            vm.w4a16_gemm(d.act[:M], d.qweight, d.scales, d.qzeros, g, out_ref)
        torch.cuda.synchronize()
        y_na = out_na.cpu().numpy().astype(np.float64)
        y_gemm = out_ref.cpu().numpy().astype(np.float64)
        y, bound = oracle.gemm(inp.act[:M], inp.qweight, inp.scales, inp.qzeros, g)
        frac = parity.check_close(y_na, y_gemm, bound, f"noalloc vs gemm M={M} N={N}")
        parity.check_close(y_na, y, bound, f"noalloc vs oracle M={M} N={N}")
        gu.say(f"  worst |noalloc - gemm| / bar {frac:.3e}")


def test_noalloc_refuses_a_call_too_large_for_its_array(gu):
    """A launch whose scratch cannot fit even at one workgroup per tile is refused, not run."""
    M, K, N, g = 16, 1 << 20, 64, 128   # prepared activations alone: 16 x 2^20 x 2 bytes = 32 MiB
    A = torch.zeros((M, K), dtype=torch.int16, device=gu.DEV)
    qw = torch.zeros((K // 8, N), dtype=torch.int32, device=gu.DEV)
    sc = torch.zeros((K // g, N), dtype=torch.int16, device=gu.DEV)
    out = torch.empty((M, N), dtype=torch.float32, device=gu.DEV)
    kern, splits, wk, cols = vm.w4a16_plan(M, N, K, g)
    gu.say(f"[noalloc] too large: plan kernel={kern} splits={splits} waves_k={wk}")
    with pytest.raises(vm.W4A16Error) as err:
        vm.w4a16_gemm_noalloc(A, qw, sc, None, g, out)
    assert err.value.status == -2
    torch.cuda.synchronize()
