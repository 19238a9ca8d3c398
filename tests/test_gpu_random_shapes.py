"""Seeded random shapes through every matmul entry point, each against the oracle.

Shapes are drawn once from a fixed seed: K a multiple of a group size from {32, 64, 128, 256},
N a multiple of 8 (rarely of 64), zero points present or not, M over each entry point's range.
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


def _cases(seed, count, m_lo, m_hi):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        g = int(rng.choice([32, 64, 128, 256]))
        K = g * int(rng.integers(1, 12))
        N = 8 * int(rng.integers(1, 160))
        M = int(rng.integers(m_lo, m_hi + 1))
        out.append((M, K, N, g, bool(rng.integers(0, 2)), int(rng.integers(0, 1 << 30))))
    return out


def _dev(gu, inp):
    return gu.DevInputs(inp)


@pytest.mark.parametrize("M,K,N,g,sym,seed", _cases(500, 10, 1, 16))
def test_random_small_rows(gu, M, K, N, g, sym, seed):
    inp = synth.make_random(seed, M, K, N, g, symmetric=sym)
    gu.say(f"[random gemm] M={M} K={K} N={N} g={g} sym={sym}")
    y_ref, bound = oracle.gemm(inp.act, inp.qweight, inp.scales, inp.qzeros, g)
    parity.check_close(_dev(gu, inp).run(M), y_ref, bound, f"gemm M={M} K={K} N={N} g={g}")


@pytest.mark.parametrize("M,K,N,g,sym,seed", _cases(501, 8, 1, 200))
def test_random_many_rows(gu, M, K, N, g, sym, seed):
    inp = synth.make_random(seed, M, K, N, g, symmetric=sym)
    d = _dev(gu, inp)
    gu.say(f"[random prefill] M={M} K={K} N={N} g={g} sym={sym}")
    out = torch.empty((M, N), dtype=torch.float32, device=gu.DEV)
    vm.w4a16_gemm_prefill(d.act, d.qweight, d.scales, d.qzeros, g, out)
    torch.cuda.synchronize()
    y_ref, bound = oracle.gemm(inp.act, inp.qweight, inp.scales, inp.qzeros, g)
    parity.check_close(out.double().cpu().numpy(), y_ref, bound, f"prefill M={M} K={K} N={N} g={g}")


@pytest.mark.parametrize("M,K,N,g,sym,seed", _cases(502, 6, 1, 16) + _cases(503, 4, 17, 150))
def test_random_gated_pair(gu, M, K, N, g, sym, seed):
    gate = synth.make_random(seed, M, K, N, g, symmetric=sym)
    up = synth.make_random(seed + 1, M, K, N, g, symmetric=sym)
    up = synth.Inputs(up.qweight, up.scales, up.qzeros, gate.act, g)
    dg, du = _dev(gu, gate), _dev(gu, up)
    gu.say(f"[random pair] M={M} K={K} N={N} g={g} sym={sym}")
    out = torch.empty((M, N), dtype=torch.float32, device=gu.DEV)
    fn = vm.w4a16_gemm_gate_up if M <= 16 else vm.w4a16_gemm_gate_up_prefill
    fn(du.act, (dg.qweight, dg.scales, dg.qzeros), (du.qweight, du.scales, du.qzeros), g, out)
    torch.cuda.synchronize()
    h, yg, bg, yu, bu = oracle.gate_up(gate.act, (gate.qweight, gate.scales, gate.qzeros),
                                        (up.qweight, up.scales, up.qzeros), g)
    parity.check_gate_up(out.double().cpu().numpy(), h, yg, bg, yu, bu, f"pair M={M} K={K} N={N} g={g}")
