"""GPU parity of the affine codes (w = s * q + b, MLX affine format) against the oracle, and the
exact widening of narrower codes onto the 4-bit layout.

Bar: |y - y_oracle| <= 4e-3 * sum_k |a_k| (|s q_k| + |b|) + 1e-6 (the oracle's affine bound:
the kernel applies scale and bias to two separate sums, whose sizes set its rounding). The
widening is integer work and must be bit-exact.
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


class Aff:
    """Device copies of 4-bit affine inputs (codes of fewer bits are widened on the host by the
    generator's encoder for these tests; the device widening has its own test)."""

    def __init__(self, gu, x):
        self.x, self.gu = x, gu
        codes = oracle.affine_unpack(x.packed, x.bits, x.K)
        self.qweight = gu.dev_u32(synth.pack_rows(codes))
        self.scales = gu.dev_u16(x.scales)
        self.biases = gu.dev_u16(x.biases)
        self.act = gu.dev_u16(x.act)

    def run(self, M, out_dtype=torch.float32, splits=0, waves_k=0, tile_cols=0, act=None):
        out = torch.empty((M, self.x.N), dtype=out_dtype, device=self.gu.DEV)
        vm.w4a16_gemm_affine(self.act[:M] if act is None else act, self.qweight, self.scales, self.biases,
                             self.x.group, out, splits, waves_k, tile_cols)
        torch.cuda.synchronize()
        return out.float().cpu().numpy().astype(np.float64)

    def ref(self, M, cols=None):
        x = self.x
        return oracle.affine_gemm(x.act[:M], x.packed, x.bits, x.scales, x.biases, x.group, cols)


# (K, N, g, bits): ragged widths (N not a multiple of 64), groups of 32 / 64 / 128, narrower codes
SHAPES = [(512, 200, 64, 4), (2048, 520, 64, 4), (1024, 1032, 128, 3), (4096, 264, 32, 2), (64, 72, 32, 4)]
# (splits, waves_k, tile_cols): default; one wave per tile (direct store); LDS and split-K
# reductions; one long slice per wave (prepared activations at 16 rows); 128-column tiles
LAUNCHES = [(0, 0, 0), (1, 1, 0), (1, 4, 0), (3, 2, 0), (8, 8, 0), (2, 2, 128)]


@pytest.mark.parametrize("K,N,g,bits", SHAPES)
def test_affine_parity_sweep(gu, K, N, g, bits):
    x = synth.make_affine_random(300 + K % 251 + bits, 16, K, N, g, bits)
    p = Aff(gu, x)
    for M in (1, 2, 5, 16):
        y_ref, bound = p.ref(M)
        for splits, wk, tc in LAUNCHES:
            if splits * max(wk, 1) > K // 32:
                continue
            gu.say(f"[affine] K={K} N={N} g={g} bits={bits} M={M} splits={splits} waves_k={wk} tile_cols={tc}")
            y = p.run(M, splits=splits, waves_k=wk, tile_cols=tc)
            frac = parity.check_close(y, y_ref, bound, f"affine K={K} N={N} M={M} {splits}/{wk}/{tc}")
    gu.say(f"  worst err/tol {frac:.3e}")


def test_affine_bf16_repeat_and_row_permutation(gu):
    x = synth.make_affine_random(91, 16, 2048, 328, 64, 4)
    p = Aff(gu, x)
    for M in (1, 16):
        y = p.run(M)
        for _ in range(2):
            assert np.array_equal(p.run(M), y)   # deterministic
        yb = p.run(M, out_dtype=torch.bfloat16)
        assert np.array_equal(yb, torch.from_numpy(y.astype(np.float32)).to(torch.bfloat16).double().numpy())
    perm = np.random.default_rng(3).permutation(16)
    act_p = gu.dev_u16(np.ascontiguousarray(x.act[perm]))
    assert np.array_equal(p.run(16, act=act_p), p.run(16)[perm])


def test_affine_zero_scale_leaves_the_bias_term(gu):
    """Every scale 0: out = bias x group sums of the activations (the ones product alone)."""
    x = synth.make_affine_random(92, 16, 1024, 256, 64, 4)
    x0 = synth.AffineInputs(x.packed, 4, np.zeros_like(x.scales), x.biases, x.act, 64)
    p = Aff(gu, x0)
    for M in (1, 7, 16):
        y_ref, bound = p.ref(M)
        parity.check_close(p.run(M), y_ref, bound, f"zero scale M={M}")


@pytest.mark.parametrize("M", [1, 4, 16])
def test_affine_ffn_workload(gu, M):
    """The affine-4 FFN up projection 5120 x 17408 (groups of 64) in the default launch, on a
    sample of columns spanning every tile position and the last tile."""
    x = synth.make_affine_inputs("ffn_up_affine4")
    p = Aff(gu, x)
    gu.say(f"[affine ffn] M={M}")
    y = p.run(M)
    rng = np.random.default_rng(M)
    cols = np.unique(np.concatenate([rng.choice(x.N, 1200, replace=False), np.arange(x.N - 64, x.N)]))
    y_ref, bound = p.ref(M, cols)
    frac = parity.check_close(y[:, cols], y_ref, bound, f"affine ffn M={M}")
    gu.say(f"  worst err/tol {frac:.3e}")


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_affine_widen_is_exact(gu, bits):
    """The device widening gives the 4-bit words of the oracle's codes, bit for bit."""
    for K, N in ((32, 8), (640, 264), (4096, 1032)):
        rng = np.random.default_rng(bits * 1000 + K)
        packed = rng.integers(0, 1 << 32, size=(K * bits // 32, N), dtype=np.uint32)
        gu.say(f"[widen] bits={bits} K={K} N={N}")
        out = torch.empty((K // 8, N), dtype=torch.int32, device=gu.DEV)
        vm.w4a16_affine_widen(gu.dev_u32(packed), bits, K, out)
        torch.cuda.synchronize()
        expect = synth.pack_rows(oracle.affine_unpack(packed, bits, K))
        assert np.array_equal(out.cpu().numpy().view(np.uint32), expect)


def test_affine_widened_codes_through_the_gemm(gu):
    """3-bit codes widened on the device, then the affine GEMM, against the oracle on the 3-bit
    stream itself."""
    K, N, g = 2048, 392, 64
    x = synth.make_affine_random(93, 16, K, N, g, 3)
    qw = torch.empty((K // 8, N), dtype=torch.int32, device=gu.DEV)
    vm.w4a16_affine_widen(gu.dev_u32(x.packed), 3, K, qw)
    out = torch.empty((16, N), dtype=torch.float32, device=gu.DEV)
    vm.w4a16_gemm_affine(gu.dev_u16(x.act), qw, gu.dev_u16(x.scales), gu.dev_u16(x.biases), g, out)
    torch.cuda.synchronize()
    y_ref, bound = oracle.affine_gemm(x.act, x.packed, 3, x.scales, x.biases, g)
    parity.check_close(out.cpu().numpy().astype(np.float64), y_ref, bound, "widened 3-bit")


def _split_on_device(gu, x):
    K, N, g = x.K, x.N, x.group
    qw = torch.empty((2 * K // 8, N), dtype=torch.int32, device=gu.DEV)
    so = torch.empty((2 * K // g, N), dtype=torch.int16, device=gu.DEV)
    bo = torch.empty((2 * K // g, N), dtype=torch.int16, device=gu.DEV)
    vm.w4a16_affine_split(gu.dev_u32(x.packed), x.bits, gu.dev_u16(x.scales), gu.dev_u16(x.biases), g, K, qw, so, bo)
    torch.cuda.synchronize()
    return qw, so, bo


@pytest.mark.parametrize("bits", [5, 6, 7, 8])
def test_affine_split_is_exact(gu, bits):
    """The two 4-bit planes of every code (low nibbles, then high), the scales s then 16 s and the
    biases b then 0, bit for bit."""
    K, N, g = 640, 264, 64
    x = synth.make_affine_random(500 + bits, 1, K, N, g, bits)
    qw, so, bo = _split_on_device(gu, x)
    codes = oracle.affine_unpack(x.packed, bits, K)
    expect = synth.pack_rows(np.concatenate([codes & 15, codes >> 4], axis=0))
    assert np.array_equal(qw.cpu().numpy().view(np.uint32), expect)
    s16 = (torch.from_numpy(x.scales.view(np.int16)).view(torch.bfloat16) * 16).view(torch.int16).numpy()
    assert np.array_equal(so.cpu().numpy(), np.concatenate([x.scales.view(np.int16), s16], axis=0))
    assert np.array_equal(bo.cpu().numpy(), np.concatenate([x.biases.view(np.int16), np.zeros_like(s16)], axis=0))


@pytest.mark.parametrize("K,N,g,bits", [(512, 200, 64, 8), (2048, 520, 64, 5), (1024, 1032, 128, 6), (64, 72, 32, 8)])
def test_affine_split_gemm_parity(gu, K, N, g, bits):
    """Codes of 5..8 bits through the split planes against the oracle on the original stream."""
    x = synth.make_affine_random(600 + K % 251 + bits, 16, K, N, g, bits)
    qw, so, bo = _split_on_device(gu, x)
    act = gu.dev_u16(x.act)
    for M in (1, 2, 5, 16):
        gu.say(f"[affine split] K={K} N={N} g={g} bits={bits} M={M}")
        out = torch.empty((M, N), dtype=torch.float32, device=gu.DEV)
        vm.w4a16_gemm_affine_split(act[:M], qw, so, bo, g, out)
        torch.cuda.synchronize()
        y_ref, bound = oracle.affine_gemm(x.act[:M], x.packed, bits, x.scales, x.biases, g)
        frac = parity.check_close(out.cpu().numpy().astype(np.float64), y_ref, bound, f"split bits={bits} M={M}")
    gu.say(f"  worst err/tol {frac:.3e}")


@pytest.mark.parametrize("M", [1, 16])
def test_affine8_ffn_workload(gu, M):
    """The 8-bit affine FFN up projection 5120 x 17408 (groups of 64), sampled columns."""
    x = synth.make_affine_inputs("ffn_up_affine8")
    qw, so, bo = _split_on_device(gu, x)
    out = torch.empty((M, x.N), dtype=torch.float32, device=gu.DEV)
    vm.w4a16_gemm_affine_split(gu.dev_u16(x.act)[:M], qw, so, bo, x.group, out)
    torch.cuda.synchronize()
    rng = np.random.default_rng(10 + M)
    cols = np.unique(np.concatenate([rng.choice(x.N, 800, replace=False), np.arange(x.N - 64, x.N)]))
    y_ref, bound = oracle.affine_gemm(x.act[:M], x.packed, 8, x.scales, x.biases, x.group, cols)
    frac = parity.check_close(out.cpu().numpy().astype(np.float64)[:, cols], y_ref, bound, f"affine8 ffn M={M}")
    gu.say(f"[affine8 ffn] M={M} worst err/tol {frac:.3e}")


def _gate_up_on_device(gu, gate, up, M, out_dtype=torch.float32):
    dg = [gu.dev_u32(synth.pack_rows(oracle.affine_unpack(gate.packed, gate.bits, gate.K))),
          gu.dev_u16(gate.scales), gu.dev_u16(gate.biases)]
    du = [gu.dev_u32(synth.pack_rows(oracle.affine_unpack(up.packed, up.bits, up.K))),
          gu.dev_u16(up.scales), gu.dev_u16(up.biases)]
    out = torch.empty((M, up.N), dtype=out_dtype, device=gu.DEV)
    vm.w4a16_gemm_affine_gate_up(gu.dev_u16(up.act)[:M], tuple(dg), tuple(du), up.group, out)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("K,N,g", [(512, 200, 64), (2048, 520, 64), (1024, 1032, 128)])
def test_affine_gate_up_parity(gu, K, N, g):
    gate = synth.make_affine_random(700 + K % 97, 16, K, N, g, 4)
    up = synth.make_affine_random(701 + K % 97, 16, K, N, g, 4)
    up = synth.AffineInputs(up.packed, 4, up.scales, up.biases, gate.act, g)
    for M in (1, 2, 5, 16):
        gu.say(f"[affine gate_up] K={K} N={N} g={g} M={M}")
        h = _gate_up_on_device(gu, gate, up, M)
        ref = oracle.affine_gate_up(gate.act[:M], (gate.packed, 4, gate.scales, gate.biases),
                                    (up.packed, 4, up.scales, up.biases), g)
        frac = parity.check_gate_up(h, *ref, f"affine gate_up K={K} M={M}")
        hb = _gate_up_on_device(gu, gate, up, M, torch.bfloat16)
        assert np.array_equal(hb, torch.from_numpy(h.astype(np.float32)).to(torch.bfloat16).double().numpy())
    gu.say(f"  worst err/tol {frac:.3e}")


@pytest.mark.parametrize("M", [1, 16])
def test_affine_gate_up_ffn_workload(gu, M):
    up = synth.make_affine_inputs("ffn_up_affine4")
    gate = synth.make_affine_gate_inputs("ffn_up_affine4")
    h = _gate_up_on_device(gu, gate, up, M)
    rng = np.random.default_rng(20 + M)
    cols = np.unique(np.concatenate([rng.choice(up.N, 800, replace=False), np.arange(up.N - 64, up.N)]))
    ref = oracle.affine_gate_up(up.act[:M], (gate.packed, 4, gate.scales, gate.biases),
                                (up.packed, 4, up.scales, up.biases), up.group, cols)
    frac = parity.check_gate_up(h[:, cols], *ref, f"affine ffn gate_up M={M}")
    gu.say(f"[affine gate_up ffn] M={M} worst err/tol {frac:.3e}")
