"""GPU parity of affine codes read at their own width (w4a16_gemm_affine_bits: w = s * q + b,
codes of 1, 2, 3, 4, 5, 6 and 8 bits streamed as stored, nothing widened) against the oracle.

Every width over ragged shapes (N not a multiple of 64 or of a workgroup's columns, groups of 32,
64 and 128), every row count class (the one-row GEMV, 2..4, 5..8 and 9..16 rows on the matrix
cores), and launches that split K across workgroups (slices through the flag exchange), across the
waves of a workgroup, and over 1 to 8 adjacent tiles. Bar: the affine bar of the oracle,
|y - y_oracle| <= 4e-3 * sum_k |a_k| (|s q_k| + |b|) + 1e-6. Also bit-exact invariants: an integer
matmul (unit scales, zero biases, integer activations), every code at every width through a bias-
only and a scale-only matrix, bit-identical repeats, the bf16 output equal to the fp32 output
rounded once, and the native-width result equal to the same matrix through the 4-bit and 8-bit
paths within the bar.
"""
import numpy as np
import pytest
import torch

import oracle
import verify_matmul_amd as vm
from tests import parity
from verify_matmul_amd import synth

pytestmark = pytest.mark.gpu

BITS = (1, 2, 3, 4, 5, 6, 8)


@pytest.fixture(scope="module")
def gu():
    from tests import gpu_util
    vm.load()
    return gpu_util


class Dev:
    def __init__(self, gu, x):
        self.x, self.gu = x, gu
        self.packed = gu.dev_u32(x.packed)
        self.scales = gu.dev_u16(x.scales)
        self.biases = gu.dev_u16(x.biases)
        self.act = gu.dev_u16(x.act)

    def run(self, M, launch=(0, 0, 0, 0), out_dtype=torch.float32, act=None, scales=None, biases=None):
        out = torch.full((M, self.x.N), float("nan"), dtype=out_dtype, device=self.gu.DEV)
        vm.w4a16_gemm_affine_bits(self.act[:M] if act is None else act, self.packed, self.x.bits,
                                  self.scales if scales is None else scales, self.biases if biases is None else biases,
                                  self.x.group, out, *launch)
        torch.cuda.synchronize()
        return out.float().cpu().numpy().astype(np.float64)


def refused(M, N, K, g, bits, launch):
    slices, tiles, kw, ring = launch
    try:
        vm.w4a16_decode_plan(M, N, K, g, False, slices, tiles, kw, 0, ring, affine_bits=bits)
    except vm.W4A16Error:
        return True
    return False


SHAPES = [(512, 256, 64), (1024, 520, 32), (2048, 1000, 128), (3072, 136, 64)]
# (slices, tiles, kw, ring); 0 = the default for that knob
LAUNCHES = [(0, 0, 0, 0), (1, 4, 1, 4), (3, 2, 2, 4), (4, 4, 1, 4), (2, 1, 4, 4), (5, 8, 1, 4), (1, 1, 1, 4)]


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("K,N,g", SHAPES)
def test_affine_bits_sweep(gu, K, N, g, bits):
    x = synth.make_affine_random(7000 + 13 * bits + K % 97 + N, 16, K, N, g, bits)
    d = Dev(gu, x)
    for M in (1, 2, 5, 16):
        y_ref, bound = oracle.affine_gemm(x.act[:M], x.packed, bits, x.scales, x.biases, g)
        worst = 0.0
        for launch in LAUNCHES:
            if refused(M, N, K, g, bits, launch):
                continue
            gu.say(f"[affine bits] K={K} N={N} g={g} bits={bits} M={M} (slices, tiles, kw, ring)={launch}")
            y = d.run(M, launch)
            worst = max(worst, parity.check_close(y, y_ref, bound, f"bits={bits} K={K} N={N} M={M} {launch}"))
        gu.say(f"  bits={bits} M={M} worst err/tol {worst:.3e}")


@pytest.mark.parametrize("bits", BITS)
def test_affine_bits_exact_cases(gu, bits):
    """Unit scales, zero biases and integer activations: an exact integer matmul at every row
    count. A scale-only matrix with activation rows that pick single K rows returns every code of
    every column exactly (each code value appears); zero scales and unit biases give the group
    sums of the activations."""
    K, N, g = 512, 264, 64
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 1 << bits, size=(K, N), dtype=np.uint32)
    codes[:1 << bits, 0] = np.arange(1 << bits)   # every code value in column 0
    packed = synth.pack_stream(codes, bits)
    one = np.full((K // g, N), 0x3F80, np.uint16)   # bf16 1.0
    zero = np.zeros((K // g, N), np.uint16)
    ai = rng.integers(-8, 9, size=(16, K)).astype(np.float32)
    x = synth.AffineInputs(packed, bits, one, zero, synth.f32_to_bf16_bits(ai), g)
    d = Dev(gu, x)
    for M in (1, 5, 16):
        ref = ai[:M].astype(np.int64) @ codes.astype(np.int64)
        for launch in ((0, 0, 0, 0), (3, 2, 2, 4), (4, 4, 1, 4)):
            assert np.array_equal(d.run(M, launch), ref.astype(np.float64)), (bits, M, launch)
    # rows of the identity pick single K rows: out[m][n] = q[row m][n] for 16 rows at a time
    for r0 in range(0, max(64, 1 << bits), 16):
        eye = np.zeros((16, K), np.float32)
        eye[np.arange(16), r0 + np.arange(16)] = 1.0
        a = gu.dev_u16(synth.f32_to_bf16_bits(eye))
        y = d.run(16, act=a)
        assert np.array_equal(y, codes[r0:r0 + 16].astype(np.float64)), (bits, r0)
    # zero scales, unit biases: each output is the sum of the row's activations
    y = d.run(16, scales=gu.dev_u16(zero), biases=gu.dev_u16(one))
    assert np.array_equal(y, np.repeat(ai.sum(axis=1, keepdims=True).astype(np.float64), N, axis=1)), bits


def test_affine_bits_invariants(gu):
    """Bit-identical repeats; the bf16 output is the fp32 output rounded once; the native-width
    product agrees with the same codes through the 4-bit path (widened) and the 8-bit planes
    (split), each within the bar."""
    K, N, g = 1024, 520, 64
    for bits in (2, 3, 5, 6):
        x = synth.make_affine_random(900 + bits, 16, K, N, g, bits)
        d = Dev(gu, x)
        y_ref, bound = oracle.affine_gemm(x.act, x.packed, bits, x.scales, x.biases, g)
        y1 = d.run(16, (3, 2, 2, 4))
        assert np.array_equal(d.run(16, (3, 2, 2, 4)), y1)
        yb = d.run(16, (3, 2, 2, 4), out_dtype=torch.bfloat16)
        assert np.array_equal(yb, torch.from_numpy(y1.astype(np.float32)).to(torch.bfloat16).double().numpy())
        if bits < 4:   # widened onto 4 bits, on the small-row kernel
            qw = torch.empty((K // 8, N), dtype=torch.int32, device=gu.DEV)
            vm.w4a16_affine_widen(d.packed, bits, K, qw)
            out = torch.empty((16, N), dtype=torch.float32, device=gu.DEV)
            vm.w4a16_gemm_affine(d.act, qw, d.scales, d.biases, g, out)
        else:          # split into two 4-bit planes
            qw = torch.empty((2 * K // 8, N), dtype=torch.int32, device=gu.DEV)
            sc = torch.empty((2 * K // g, N), dtype=torch.int16, device=gu.DEV)
            bi = torch.empty((2 * K // g, N), dtype=torch.int16, device=gu.DEV)
            vm.w4a16_affine_split(d.packed, bits, d.scales, d.biases, g, K, qw, sc, bi)
            out = torch.empty((16, N), dtype=torch.float32, device=gu.DEV)
            vm.w4a16_gemm_affine_split(d.act, qw, sc, bi, g, out)
        torch.cuda.synchronize()
        parity.check_close(out.cpu().numpy().astype(np.float64), y_ref, bound, f"bits={bits} other path")
        parity.check_close(y1, y_ref, bound, f"bits={bits} native")


@pytest.mark.parametrize("name,M", [("ffn_up_affine4", 1), ("ffn_up_affine4", 16)])
def test_affine_bits_workload(gu, name, M):
    """The affine-4 FFN up projection (5120 x 17408, groups of 64) read natively."""
    x = synth.make_affine_inputs(name)
    d = Dev(gu, x)
    y_ref, bound = oracle.affine_gemm(x.act[:M], x.packed, x.bits, x.scales, x.biases, x.group)
    frac = parity.check_close(d.run(M), y_ref, bound, f"{name} M={M}")
    gu.say(f"[affine bits workload] {name} M={M} worst err/tol {frac:.3e}")
