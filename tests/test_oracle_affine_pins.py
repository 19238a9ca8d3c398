"""Pins of the oracle's affine form (w = s * q + b, codes of 1..8 bits in column bit streams)
against facts that do not come from the oracle itself: hand-written streams, numpy's own bit
unpacking, the independently pinned GPTQ path, exact rational sums and closed forms.
"""
import ctypes
from fractions import Fraction

import numpy as np
import pytest
import torch

from tests import parity
from verify_matmul_amd import synth


def _bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double().numpy()


# ---- unpacking ------------------------------------------------------------------------------

def test_affine_unpack_spec_literal(orc):
    # 2 bits: byte 0b11100100 holds codes 0, 1, 2, 3 from the low end
    q = orc.affine_unpack(np.array([[0xE4E4E4E4]], dtype=np.uint32), 2, 16)
    assert q[:, 0].tolist() == [0, 1, 2, 3] * 4
    # 8 bits: one byte per row, lowest byte first
    q = orc.affine_unpack(np.array([[0x03020100], [0xFFFEFD80]], dtype=np.uint32), 8, 8)
    assert q[:, 0].tolist() == [0, 1, 2, 3, 0x80, 0xFD, 0xFE, 0xFF]
    # 3 bits: row 10 takes stream bits 30, 31 (word 0) and 32 (bit 0 of word 1); row 11 bits 33..35
    pk = np.zeros((3, 1), dtype=np.uint32)
    pk[0, 0] = 0xC0000000
    pk[1, 0] = 0x00000001 | 0x00000002   # bit 32 -> row 10's top bit, bit 33 -> row 11's low bit
    q = orc.affine_unpack(pk, 3, 32)[:, 0].tolist()
    assert q[10] == 7 and q[11] == 1 and sum(q) == 8


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 7, 8])
def test_affine_unpack_matches_numpy_bit_view(orc, bits):
    """Any words are a valid stream: numpy's little-endian unpackbits of each column's bytes,
    cut into fields of `bits`, must give the oracle's codes."""
    rng = np.random.default_rng(bits)
    K, N = 64 * 3, 5
    pk = rng.integers(0, 1 << 32, size=(K * bits // 32, N), dtype=np.uint32)
    q = orc.affine_unpack(pk, bits, K)
    for n in range(N):
        raw = np.ascontiguousarray(pk[:, n]).astype("<u4").view(np.uint8)
        stream = np.unpackbits(raw, bitorder="little")[: K * bits].reshape(K, bits)
        codes = (stream.astype(np.int64) << np.arange(bits)).sum(axis=1)
        assert np.array_equal(q[:, n], codes), n


def test_affine_four_bits_is_the_qweight_layout(orc):
    rng = np.random.default_rng(4)
    qw = rng.integers(0, 1 << 32, size=(32, 24), dtype=np.uint32)
    assert np.array_equal(orc.affine_unpack(qw, 4, 256), orc.unpack_qweight(qw))


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
def test_affine_roundtrip_with_encoder(orc, bits):
    rng = np.random.default_rng(10 + bits)
    codes = rng.integers(0, 1 << bits, size=(96, 8), dtype=np.uint8)
    assert np.array_equal(orc.affine_unpack(synth.pack_stream(codes, bits), bits, 96), codes)


# ---- the matmul -----------------------------------------------------------------------------

@pytest.mark.parametrize("M,K,N,g,bits", [(1, 32, 8, 32, 4), (2, 64, 8, 32, 3), (3, 128, 16, 64, 2),
                                          (2, 64, 8, 64, 8), (1, 96, 8, 32, 5)])
def test_affine_gemm_bruteforce_tiny(orc, M, K, N, g, bits):
    x = synth.make_affine_random(200 + K + bits, M, K, N, g, bits)
    y, b = orc.affine_gemm(x.act, x.packed, bits, x.scales, x.biases, g)
    raw = np.ascontiguousarray(x.packed).astype("<u4")
    a, s, bb = _bf16(x.act), _bf16(x.scales), _bf16(x.biases)
    for n in range(N):
        stream = np.unpackbits(np.ascontiguousarray(raw[:, n]).view(np.uint8), bitorder="little")
        codes = [int(sum(int(stream[k * bits + i]) << i for i in range(bits))) for k in range(K)]
        for m in range(M):
            ye = be = Fraction(0)
            for k in range(K):
                sq = Fraction(s[k // g, n]) * codes[k]
                w = sq + Fraction(bb[k // g, n])
                ye += Fraction(a[m, k]) * w
                be += abs(Fraction(a[m, k])) * (abs(sq) + abs(Fraction(bb[k // g, n])))
            slack = K * 2.0 ** -52 * float(be)
            assert abs(Fraction(y[m, n]) - ye) <= slack
            assert abs(Fraction(b[m, n]) - be) <= slack


def test_affine_without_bias_is_the_gptq_product(orc):
    """Biases 0 and scales exact in both fp16 and bf16: the affine product must equal the
    (separately pinned) GPTQ product with every zero point 0, bit for bit."""
    rng = np.random.default_rng(77)
    K, N, g = 256, 16, 64
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    vals = rng.integers(1, 256, size=(K // g, N)) * 2.0 ** -12          # 8 significant bits
    s_bf16 = synth.f32_to_bf16_bits(vals.astype(np.float32))
    s_fp16 = synth.f64_to_fp16_bits(vals)
    assert np.array_equal(_bf16(s_bf16), s_fp16.view(np.float16).astype(np.float64))
    act = synth.f32_to_bf16_bits(rng.standard_normal((3, K)).astype(np.float32))
    zeros = synth.pack_cols(np.zeros((K // g, N), dtype=np.uint8))
    y_gptq, _ = orc.gemm(act, synth.pack_rows(codes), s_fp16, zeros, g)
    y_aff, _ = orc.affine_gemm(act, synth.pack_stream(codes, 4), 4, s_bf16,
                               np.zeros((K // g, N), np.uint16), g)
    assert np.array_equal(y_aff, y_gptq)


def test_affine_zero_scale_is_bias_times_group_sums(orc):
    """s = 0: y[m][n] = sum over groups of b[g][n] * (sum of the group's activations)."""
    x = synth.make_affine_random(31, 4, 512, 24, 64, 4)
    zs = np.zeros_like(x.scales)
    y, _ = orc.affine_gemm(x.act, x.packed, 4, zs, x.biases, 64)
    gs = _bf16(x.act).reshape(4, 512 // 64, 64).sum(axis=2)              # [M, groups]
    expect = gs @ _bf16(x.biases)
    assert np.allclose(y, expect, rtol=1e-12, atol=1e-12)


def test_affine_constant_code_and_linearity(orc):
    """All codes c: w = s c + b per group; doubling scales and biases doubles y exactly."""
    rng = np.random.default_rng(5)
    K, N, g = 128, 8, 32
    act = synth.f32_to_bf16_bits(rng.standard_normal((2, K)).astype(np.float32))
    s = synth.f32_to_bf16_bits(rng.uniform(0.01, 0.02, size=(K // g, N)).astype(np.float32))
    b = synth.f32_to_bf16_bits(-rng.uniform(0.05, 0.1, size=(K // g, N)).astype(np.float32))
    pk = synth.pack_stream(np.full((K, N), 9, np.uint8), 4)
    y, _ = orc.affine_gemm(act, pk, 4, s, b, g)
    w = np.repeat(_bf16(s) * 9 + _bf16(b), g, axis=0)                     # [K, N]
    assert np.allclose(y, _bf16(act) @ w, rtol=1e-13, atol=1e-13)
    s2 = synth.f32_to_bf16_bits((_bf16(s) * 2).astype(np.float32))
    b2 = synth.f32_to_bf16_bits((_bf16(b) * 2).astype(np.float32))
    y2, _ = orc.affine_gemm(act, pk, 4, s2, b2, g)
    assert np.array_equal(y2, 2 * y)


def test_affine_bar_rejects_plausible_mistakes(orc):
    """The parity bar on an FFN-width slice rejects a dropped bias, a bias of the wrong sign,
    the bias taken from the neighbouring group, and codes read one bit wide of their field."""
    x = synth.make_affine_random(9, 4, 2048, 64, 64, 4)
    y, b = orc.affine_gemm(x.act, x.packed, 4, x.scales, x.biases, 64)
    neg = (x.biases ^ np.uint16(0x8000))
    wrong = {
        "no bias": orc.affine_gemm(x.act, x.packed, 4, x.scales, np.zeros_like(x.biases), 64)[0],
        "bias sign": orc.affine_gemm(x.act, x.packed, 4, x.scales, neg, 64)[0],
        "bias group": orc.affine_gemm(x.act, x.packed, 4, x.scales, np.roll(x.biases, 1, axis=0), 64)[0],
        "field width": orc.affine_gemm(x.act, synth.pack_stream(orc.affine_unpack(x.packed, 4, 2048) >> 1, 3),
                                       3, x.scales, x.biases, 64)[0],
    }
    for name, yw in wrong.items():
        with pytest.raises(AssertionError):
            parity.check_close(yw, y, b, name)


def test_affine_oracle_rejects_bad_arguments(orc):
    x = synth.make_affine_random(3, 1, 64, 8, 32, 4)
    lib = orc._load()
    y = np.empty((1, 8))
    P = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    args = [P(x.act), P(x.packed), 4, P(x.scales), P(x.biases), 32, 1, 8, 64, None, 8, P(y), None]
    assert lib.w4o_affine_gemm(*args) == 0
    for i, bad in ((5, 48), (2, 9), (2, 0), (8, 60), (5, 0)):   # K % g, bits, K * bits % 32, g
        a = list(args)
        a[i] = bad
        assert lib.w4o_affine_gemm(*a) == -1, (i, bad)


def test_affine_gate_up_orientation(orc):
    """Scales 0 make every weight its bias: gate biases 1 give y_gate = sum(a), up biases 2 give
    y_up = 2 sum(a), so h = silu(sum a) * 2 sum(a) -- and not silu(2 sum a) * sum(a)."""
    K, N, g = 64, 8, 32
    rng = np.random.default_rng(8)
    act = synth.f32_to_bf16_bits(rng.standard_normal((2, K)).astype(np.float32))
    pk = synth.pack_stream(rng.integers(0, 16, size=(K, N), dtype=np.uint8), 4)
    zs = np.zeros((K // g, N), np.uint16)
    one, two = np.full_like(zs, 0x3F80), np.full_like(zs, 0x4000)   # bf16 1.0 and 2.0
    h, yg, _, yu, _ = orc.affine_gate_up(act, (pk, 4, zs, one), (pk, 4, zs, two), g)
    sa = _bf16(act).sum(axis=1)[:, None] * np.ones((1, N))
    assert np.allclose(yg, sa, rtol=1e-15, atol=1e-15) and np.allclose(yu, 2 * sa, rtol=1e-15, atol=1e-15)
    expect = sa / (1 + np.exp(-sa)) * 2 * sa
    assert np.allclose(h, expect, rtol=1e-14, atol=1e-15)
    swapped = 2 * sa / (1 + np.exp(-2 * sa)) * sa
    assert not np.allclose(h, swapped, rtol=1e-6)
