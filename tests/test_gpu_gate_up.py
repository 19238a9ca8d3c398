"""GPU parity of the gated pair, out = silu(A x W_gate) * (A x W_up), against the oracle.

Bar: the gated-product bar of tests/parity.py (each product within the matmul bar, carried
through silu and the product). The fused launch is also checked against the two products of
single-matrix launches of the same shape, which it must reproduce up to the fp32 evaluation of
silu and the product, and its bf16 output against its own fp32 output rounded once.
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


class Pair:
    def __init__(self, gu, gate, up):
        self.gate, self.up = gate, up
        self.dg, self.du = gu.DevInputs(gate), gu.DevInputs(up)
        self.K, self.N, self.group = up.K, up.N, up.group
        self.gu = gu

    def run(self, M, out_dtype=torch.float32, splits=0, waves_k=0):
        out = torch.empty((M, self.N), dtype=out_dtype, device=self.gu.DEV)
        vm.w4a16_gemm_gate_up(self.du.act[:M], (self.dg.qweight, self.dg.scales, self.dg.qzeros),
                              (self.du.qweight, self.du.scales, self.du.qzeros), self.group, out,
                              splits=splits, waves_k=waves_k)
        torch.cuda.synchronize()
        return out.float().cpu().numpy().astype(np.float64)

    def ref(self, M, cols=None):
        return oracle.gate_up(self.up.act[:M], (self.gate.qweight, self.gate.scales, self.gate.qzeros),
                              (self.up.qweight, self.up.scales, self.up.qzeros), self.group, cols)


def _pair(seed, K, N, g, sym):
    gate = synth.make_random(seed, 16, K, N, g, symmetric=sym)
    up = synth.make_random(seed + 1, 16, K, N, g, symmetric=sym)
    return gate, synth.Inputs(up.qweight, up.scales, up.qzeros, gate.act, g)


# (K, N, g, sym): ragged widths (N not a multiple of 64), both zero-point forms, group 64/128
SHAPES = [(512, 200, 128, True), (2048, 520, 64, False), (1024, 1032, 128, True), (4096, 264, 128, False)]
# (splits, waves_k): default; one wave per tile (direct store); LDS and split-K reductions;
# one long slice per wave (prepared activations at 16 rows)
LAUNCHES = [(0, 0), (1, 1), (1, 4), (3, 2), (8, 8)]


@pytest.mark.parametrize("K,N,g,sym", SHAPES)
def test_gate_up_parity_sweep(gu, K, N, g, sym):
    gate, up = _pair(40 + K % 97, K, N, g, sym)
    p = Pair(gu, gate, up)
    for M in (1, 2, 5, 16):
        h_ref, yg, bg, yu, bu = p.ref(M)
        for splits, wk in LAUNCHES:
            if splits * max(wk, 1) > K // 32:
                continue
            gu.say(f"[gate_up] K={K} N={N} g={g} sym={sym} M={M} splits={splits} waves_k={wk}")
            h = p.run(M, splits=splits, waves_k=wk)
            parity.check_gate_up(h, h_ref, yg, bg, yu, bu, f"K={K} N={N} M={M} splits={splits} waves_k={wk}")


@pytest.mark.parametrize("sym", [True, False])
def test_gate_up_equals_two_launches(gu, sym):
    """Same K split for the pair and for each matrix alone on the matrix cores: every column's sum
    depends only on its own weights, the activations and the K split, so the pair's sums are the
    single launches' sums and the fused output is silu(g) * u of those up to fp32 evaluation."""
    K, N, g = 2048, 328, 128
    gate, up = _pair(60, K, N, g, sym)
    p = Pair(gu, gate, up)
    for M in (1, 3, 16):
        for splits, wk in ((1, 1), (2, 4), (4, 8)):
            gu.say(f"[gate_up=two] sym={sym} M={M} splits={splits} waves_k={wk}")
            h = p.run(M, splits=splits, waves_k=wk)
            yg = p.dg.run(M, splits=splits, waves_k=wk, tile_cols=128)
            yu = p.du.run(M, splits=splits, waves_k=wk, tile_cols=128)
            expect = oracle.silu_mul(yg, yu)
            err = np.abs(h - expect)
            assert np.all(err <= 4e-6 * np.abs(expect) + 1e-30), float((err / (np.abs(expect) + 1e-30)).max())


def test_gate_up_bf16_and_repeat(gu):
    gate, up = _pair(70, 1024, 1032, 128, False)
    p = Pair(gu, gate, up)
    for M in (1, 16):
        h = p.run(M)
        for _ in range(3):
            assert np.array_equal(p.run(M), h)   # deterministic
        hb = p.run(M, out_dtype=torch.bfloat16)
        assert np.array_equal(hb, torch.from_numpy(h.astype(np.float32)).to(torch.bfloat16).double().numpy())


def test_gate_up_zero_gate_or_up(gu):
    """A zero gate product gives silu(0) = 0, a zero up product gives 0: exact zeros out."""
    K, N, g = 512, 256, 128
    gate, up = _pair(80, K, N, g, True)
    eights = np.full((K // 8, N), 0x88888888, np.uint32)   # q = 8 = z: every weight is 0
    for zg in (True, False):
        gg = synth.Inputs(eights, gate.scales, None, gate.act, g) if zg else gate
        uu = up if zg else synth.Inputs(eights, up.scales, None, up.act, g)
        p = Pair(gu, gg, uu)
        for M in (1, 16):
            assert np.all(p.run(M) == 0.0)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_gate_up_ffn_workload(gu, M):
    """The 5120 x 17408 FFN pair (group 128, symmetric) in the default launch, on a sample of
    columns spanning every tile position and the last tile."""
    up = synth.make_inputs("ffn_up")
    gate = synth.make_gate_inputs("ffn_up")
    p = Pair(gu, gate, up)
    gu.say(f"[gate_up ffn] M={M}")
    h = p.run(M)
    rng = np.random.default_rng(M)
    cols = np.unique(np.concatenate([rng.choice(up.N, 1500, replace=False), np.arange(up.N - 64, up.N)]))
    h_ref, yg, bg, yu, bu = p.ref(M, cols)
    frac = parity.check_gate_up(h[:, cols], h_ref, yg, bg, yu, bu, f"ffn gate_up M={M}")
    gu.say(f"  worst err/tol {frac:.3e}")


def run_prefill_pair(gu, p, M, out_dtype=torch.float32, act=None):
    out = torch.empty((M, p.N), dtype=out_dtype, device=gu.DEV)
    a = p.du.act[:M] if act is None else act
    vm.w4a16_gemm_gate_up_prefill(a, (p.dg.qweight, p.dg.scales, p.dg.qzeros),
                                  (p.du.qweight, p.du.scales, p.du.qzeros), p.group, out)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


# (M, K, N, g, sym): ragged M and N; few tiles (K slices, 2N-wide partials) and many (LDS hand-over)
PREFILL_SHAPES = [(17, 512, 200, 128, True), (130, 2048, 264, 64, False), (300, 1024, 1032, 128, True),
                  (640, 512, 5120, 64, False)]


@pytest.mark.parametrize("M,K,N,g,sym", PREFILL_SHAPES)
def test_gate_up_prefill_parity(gu, M, K, N, g, sym):
    gate = synth.make_random(100 + M, M, K, N, g, symmetric=sym)
    up = synth.make_random(101 + M, M, K, N, g, symmetric=sym)
    up = synth.Inputs(up.qweight, up.scales, up.qzeros, gate.act, g)
    p = Pair(gu, gate, up)
    gu.say(f"[gate_up prefill] M={M} K={K} N={N} g={g} sym={sym}")
    h = run_prefill_pair(gu, p, M)
    h_ref, yg, bg, yu, bu = p.ref(M)
    frac = parity.check_gate_up(h, h_ref, yg, bg, yu, bu, f"prefill pair M={M} K={K} N={N}")
    gu.say(f"  worst err/tol {frac:.3e}")
    hb = run_prefill_pair(gu, p, M, torch.bfloat16)
    assert np.array_equal(hb, torch.from_numpy(h.astype(np.float32)).to(torch.bfloat16).double().numpy())
    assert np.array_equal(run_prefill_pair(gu, p, M), h)   # deterministic


def test_gate_up_prefill_ffn_workload(gu):
    """The 5120 x 17408 FFN pair with 512 prompt rows, sampled columns."""
    up = synth.make_inputs("ffn_up")
    gate = synth.make_gate_inputs("ffn_up")
    wl = synth.WORKLOADS["ffn_up"]
    M = 512
    rng = np.random.Generator(np.random.PCG64(1000 * wl.index + 9))
    act = synth.draw_activations(rng, M, wl.K, wl.act_sigma, wl.outlier_frac, wl.outlier_mul)
    gate = synth.Inputs(gate.qweight, gate.scales, gate.qzeros, act, gate.group)
    up = synth.Inputs(up.qweight, up.scales, up.qzeros, act, up.group)
    p = Pair(gu, gate, up)
    gu.say(f"[gate_up prefill ffn] M={M}")
    h = run_prefill_pair(gu, p, M)
    cols = np.unique(np.concatenate([rng.choice(up.N, 400, replace=False), np.arange(up.N - 130, up.N)]))
    h_ref, yg, bg, yu, bu = p.ref(M, cols)
    frac = parity.check_gate_up(h[:, cols], h_ref, yg, bg, yu, bu, "ffn prefill pair")
    gu.say(f"  worst err/tol {frac:.3e}")
