"""GPU parity of plain calls of 9-16 rows on matrices of 16384-65535 columns, which take the
decode kernel by default (4 tiles x 2 K pieces per workgroup over the fewest K slices that run in
one round), against the oracle, and of the neighbouring shapes that keep the small-row kernel.

For each shape: the launch the library reports (`w4a16_plan`); fp32 outputs on a sample of
columns that spans every tile position and the last tile, within the bar; the bf16 output equal
to the fp32 output rounded once; bit-identical repeats; the fused greedy pick (`w4a16_gemm_argmax`)
equal to the separate pick on the same launch's logits; and `w4a16_gemm_noalloc` within the bar.
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


# (M, K, N, g, symmetric, decode kernel by default)
CASES = [
    (9, 1024, 16384, 128, True, True),
    (12, 2048, 20008, 64, False, True),
    (13, 3072, 24000, 32, False, True),
    (16, 4096, 32768, 128, True, True),
    (16, 5120, 17408, 128, True, True),
    (11, 1536, 65528, 64, True, True),
    (8, 2048, 16384, 128, True, False),     # 8 rows: the small-row kernel
    (16, 2048, 16376, 128, False, False),   # below 16384 columns: the small-row kernel
]


def _cols(rng, N):
    return np.unique(np.concatenate([rng.choice(N, min(N, 500), replace=False), np.arange(N - 300, N)]))


@pytest.mark.parametrize("M,K,N,g,sym,dec", CASES)
def test_mid_width_parity(gu, M, K, N, g, sym, dec):
    inp = synth.make_random(6000 + M + K // 32 + N // 8, M, K, N, g, symmetric=sym)
    kern, splits, wk, cols = vm.w4a16_plan(M, N, K, g)
    assert (kern == 3) == dec, (M, N, K, kern)
    if dec:
        assert wk == 2 and cols == 64 and splits * -(-N // 256) >= 192
    d = gu.DevInputs(inp)
    gu.say(f"[mid width] M={M} K={K} N={N} g={g} sym={sym} plan={(kern, splits, wk, cols)}")
    y = d.run(M)
    rng = np.random.default_rng(M + N)
    c = _cols(rng, N)
    y_ref, bound = oracle.gemm(inp.act, inp.qweight, inp.scales, inp.qzeros, g, c)
    frac = parity.check_close(y[:, c], y_ref, bound, f"mid width M={M} K={K} N={N}")
    gu.say(f"  worst err/tol {frac:.3e}")
    assert np.array_equal(d.run(M), y)   # bit-identical repeat
    yb = d.run(M, out_dtype=torch.bfloat16)
    assert np.array_equal(yb, torch.from_numpy(y.astype(np.float32)).to(torch.bfloat16).double().numpy())


@pytest.mark.parametrize("M,K,N,g,sym,dec", [c for c in CASES if c[5]][:4])
def test_mid_width_fused_pick_and_noalloc(gu, M, K, N, g, sym, dec):
    inp = synth.make_random(6100 + M + N // 8, M, K, N, g, symmetric=sym)
    d = gu.DevInputs(inp)
    gu.say(f"[mid width pick/noalloc] M={M} K={K} N={N} g={g} sym={sym}")
    out = torch.empty((M, N), dtype=torch.float32, device=gu.DEV)
    idx = torch.full((M,), -7, dtype=torch.int32, device=gu.DEV)
    vm.w4a16_gemm_argmax(d.act, d.qweight, d.scales, d.qzeros, g, out, idx)
    sep = torch.full((M,), -7, dtype=torch.int32, device=gu.DEV)
    vm.w4a16_argmax_rows(out, sep)
    torch.cuda.synchronize()
    assert torch.equal(idx, sep), (idx.cpu().numpy(), sep.cpu().numpy())
    logits = out.double().cpu().numpy()
    assert np.array_equal(idx.cpu().numpy(), oracle.argmax_rows_f32(logits.astype(np.float32)))
    y = d.run(M)
    assert np.array_equal(logits, y)   # the fused pick leaves the product as the plain call computes it
    na = torch.empty((M, N), dtype=torch.float32, device=gu.DEV)
    vm.w4a16_gemm_noalloc(d.act, d.qweight, d.scales, d.qzeros, g, na)
    torch.cuda.synchronize()
    c = _cols(np.random.default_rng(N), N)
    y_ref, bound = oracle.gemm(inp.act, inp.qweight, inp.scales, inp.qzeros, g, c)
    parity.check_close(na.double().cpu().numpy()[:, c], y_ref, bound, f"noalloc M={M} N={N}")
