"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test would fail on a plausible mistake in the oracle: a wrong nibble order, a wrong
group index, a dropped zero point, a transposed operand, a sign error, a wrong fp16 decode.
The pages print no worked example or test vector, so the pins are the storage convention
written out by hand, library conversions, exhaustive enumeration, exact rational brute force
and algebraic invariants.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from verify_matmul_amd import synth


# ---- unpacking: the GPTQ storage convention, written out by hand -------------------------

def test_unpack_spec_literal_word(orc):
    # nibble j of word i holds row 8i+j, lowest nibble first: 0x76543210 -> rows 0..7 = 0..7
    qw = np.array([[0x76543210, 0xFEDCBA98], [0x01234567, 0x89ABCDEF]], dtype=np.uint32)
    q = orc.unpack_qweight(qw)
    assert q[:8, 0].tolist() == [0, 1, 2, 3, 4, 5, 6, 7]
    assert q[:8, 1].tolist() == [8, 9, 10, 11, 12, 13, 14, 15]
    assert q[8:, 0].tolist() == [7, 6, 5, 4, 3, 2, 1, 0]
    assert q[8:, 1].tolist() == [15, 14, 13, 12, 11, 10, 9, 8]


def test_unpack_every_value_every_position(orc):
    # a word holding only value v at nibble j unpacks to v at row 8i+j and 0 elsewhere
    K, N = 16, 8
    for j in range(8):
        for v in range(16):
            qw = np.zeros((K // 8, N), dtype=np.uint32)
            qw[1, 3] = np.uint32(v << (4 * j))
            q = orc.unpack_qweight(qw)
            expect = np.zeros((K, N), dtype=np.uint8)
            expect[8 + j, 3] = v
            assert np.array_equal(q, expect), (j, v)


def test_unpack_zeros_every_value_every_position(orc):
    G, N = 3, 16
    for j in range(8):
        for v in range(16):
            qz = np.zeros((G, N // 8), dtype=np.uint32)
            qz[2, 1] = np.uint32(v << (4 * j))
            z = orc.unpack_qzeros(qz, G, N)
            expect = np.zeros((G, N), dtype=np.uint8)
            expect[2, 8 + j] = v
            assert np.array_equal(z, expect), (j, v)


def test_unpack_zeros_absent_means_eight(orc):
    assert np.all(orc.unpack_qzeros(None, 4, 16) == 8)


def test_unpack_roundtrip_with_encoder(orc):
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 16, size=(64, 24), dtype=np.uint8)
    assert np.array_equal(orc.unpack_qweight(synth.pack_rows(codes)), codes)
    zc = rng.integers(0, 16, size=(5, 24), dtype=np.uint8)
    assert np.array_equal(orc.unpack_qzeros(synth.pack_cols(zc), 5, 24), zc)


# ---- scalar conversions against library conversions --------------------------------------

def test_fp16_decode_all_patterns(orc):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    ours = np.array([orc.fp16_to_f32(int(b)) for b in bits], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_decode_all_patterns(orc):
    bits = np.arange(1 << 16, dtype=np.int64).astype(np.int16)
    ref = torch.from_numpy(bits).view(torch.bfloat16).to(torch.float32).numpy()
    ours = np.array([orc.bf16_to_f32(int(b) & 0xFFFF) for b in bits], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


# ---- dequantisation: exhaustive (q, z, scale) -------------------------------------------

def test_dequant_exhaustive_exact(orc):
    """Every code q, every zero z and every finite fp16 scale: w == (q - z) * s exactly."""
    fin = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    fin = fin[np.isfinite(fin.view(np.float16))]
    N = fin.size - fin.size % 8                      # 63488 finite patterns, a multiple of 8
    assert N == 63488
    g = 16
    K = 16 * g                                       # group gi has zero gi; row k has code k % 16
    k = np.arange(K)
    d = (k % 16 - k // g).astype(np.float64)         # q - z
    C = N // 8                                       # the scales in 8 column blocks (bounded memory)
    qweight = np.empty((K // 8, C), dtype=np.uint32)
    qweight[0::2] = 0x76543210
    qweight[1::2] = 0xFEDCBA98
    qzeros = np.repeat((np.arange(16, dtype=np.uint32) * 0x11111111)[:, None], C // 8, axis=1)
    for c0 in range(0, N, C):
        blk = fin[c0:c0 + C]
        scales = np.broadcast_to(blk, (K // g, C)).copy()
        w = orc.dequant(qweight, scales, qzeros, g)
        s = blk.view(np.float16).astype(np.float64)
        exact = d[:, None] * s[None, :]               # exact in fp64 (<= 5 x 11 bits)
        assert np.array_equal(exact.astype(np.float32).astype(np.float64), exact)   # fits fp32
        assert np.array_equal(w.astype(np.float64), exact), c0


# ---- the matmul against exact rational arithmetic -----------------------------------------

def _exact(act_bits, codes, zeros, scales_bits, g):
    """sum_k a*(q-z)*s over the rationals, from unpacked codes (independent of the packing)."""
    a = torch.from_numpy(act_bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    s = scales_bits.view(np.float16).astype(np.float64)
    M, K = a.shape
    N = codes.shape[1]
    y = [[Fraction(0)] * N for _ in range(M)]
    b = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            acc_abs = Fraction(0)
            for k in range(K):
                t = Fraction(a[m, k]) * (int(codes[k, n]) - int(zeros[k // g, n])) * Fraction(s[k // g, n])
                acc += t
                acc_abs += abs(t)
            y[m][n] = acc
            b[m][n] = acc_abs
    return y, b


@pytest.mark.parametrize("M,K,N,g,sym", [
    (1, 8, 8, 8, True), (2, 32, 16, 8, False), (3, 64, 8, 32, False),
    (3, 128, 16, 64, True), (2, 128, 8, 32, False),
])
def test_gemm_bruteforce_tiny(orc, M, K, N, g, sym):
    rng = np.random.default_rng(1000 + K + N + g)
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    zeros = np.full((K // g, N), 8, dtype=np.uint8) if sym else \
        rng.integers(0, 16, size=(K // g, N), dtype=np.uint8)
    scales = synth.draw_scales(rng, (K // g, N), 0.001, 0.05)
    act = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    y, b = orc.gemm(act, synth.pack_rows(codes), scales, None if sym else synth.pack_cols(zeros), g)
    ye, be = _exact(act, codes, zeros, scales, g)
    for m in range(M):
        for n in range(N):
            slack = K * 2.0 ** -52 * float(be[m][n])
            assert abs(Fraction(y[m, n]) - ye[m][n]) <= slack
            assert abs(Fraction(b[m, n]) - be[m][n]) <= slack


def test_gemm_bruteforce_tiny_workload(orc):
    """The whole tiny workload (1 x 512 x 256, group 128, symmetric): 131072 exact products."""
    inp = synth.make_inputs("tiny")
    act = inp.act[:1]
    y, b = orc.gemm(act, inp.qweight, inp.scales, None, inp.group)
    codes = np.zeros((512, 256), dtype=np.uint8)
    for j in range(8):                                      # unpack by hand, not via the oracle
        codes[j::8] = (inp.qweight >> np.uint32(4 * j)) & np.uint32(0xF)
    ye, be = _exact(act, codes, np.full((4, 256), 8, np.uint8), inp.scales, 128)
    for n in range(256):
        slack = 512 * 2.0 ** -52 * float(be[0][n])
        assert abs(Fraction(y[0, n]) - ye[0][n]) <= slack
        assert abs(Fraction(b[0, n]) - be[0][n]) <= slack


def test_gemm_column_subset_matches_full(orc):
    inp = synth.make_random(5, 3, 256, 64, 64, symmetric=False)
    y, b = orc.gemm(inp.act, inp.qweight, inp.scales, inp.qzeros, inp.group)
    cols = [63, 0, 17, 17, 40]
    ys, bs = orc.gemm(inp.act, inp.qweight, inp.scales, inp.qzeros, inp.group, cols=cols)
    assert np.array_equal(ys, y[:, cols]) and np.array_equal(bs, b[:, cols])


# ---- invariants -------------------------------------------------------------------------

def test_codes_equal_zeros_give_exact_zero(orc):
    rng = np.random.default_rng(11)
    K, N, g = 256, 32, 64
    zeros = rng.integers(0, 16, size=(K // g, N), dtype=np.uint8)
    codes = np.repeat(zeros, g, axis=0)
    scales = synth.draw_scales(rng, (K // g, N), 0.001, 0.05)
    act = synth.f32_to_bf16_bits(rng.standard_normal((4, K)).astype(np.float32) * 50)
    y, b = orc.gemm(act, synth.pack_rows(codes), scales, synth.pack_cols(zeros), g)
    assert np.all(y == 0.0) and np.all(b == 0.0)
    y8, _ = orc.gemm(act, np.full((K // 8, N), 0x88888888, np.uint32), scales, None, g)
    assert np.all(y8 == 0.0)


def test_unit_scale_zero_point_is_integer_matmul(orc):
    rng = np.random.default_rng(12)
    M, K, N, g = 3, 512, 40, 128
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    ai = rng.integers(-8, 9, size=(M, K))
    act = synth.f32_to_bf16_bits(ai.astype(np.float32))
    scales = np.full((K // g, N), 0x3C00, dtype=np.uint16)            # fp16 1.0
    qzeros = np.zeros((K // g, N // 8), dtype=np.uint32)              # every zero 0
    y, _ = orc.gemm(act, synth.pack_rows(codes), scales, qzeros, g)
    ref = ai.astype(np.int64) @ codes.astype(np.int64)
    assert np.array_equal(y, ref.astype(np.float64))


def test_many_rows_integer_matmul(orc):
    """The prompt-sized case: 300 rows (more than any small-row launch), unit scales and zero
    points drawn per group and column, integer activations: an exact int64 matmul of the codes
    minus their zeros."""
    rng = np.random.default_rng(16)
    M, K, N, g = 300, 256, 72, 64
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    zeros = rng.integers(0, 16, size=(K // g, N), dtype=np.uint8)
    ai = rng.integers(-8, 9, size=(M, K))
    act = synth.f32_to_bf16_bits(ai.astype(np.float32))
    scales = np.full((K // g, N), 0x3C00, dtype=np.uint16)
    y, _ = orc.gemm(act, synth.pack_rows(codes), scales, synth.pack_cols(zeros), g)
    d = codes.astype(np.int64) - np.repeat(zeros.astype(np.int64), g, axis=0)
    assert np.array_equal(y, (ai.astype(np.int64) @ d).astype(np.float64))


def test_scaling_and_negation(orc):
    inp = synth.make_random(13, 4, 384, 48, 128, symmetric=False)
    y, b = orc.gemm(inp.act, inp.qweight, inp.scales, inp.qzeros, inp.group)
    doubled = (inp.scales + np.uint16(0x0400)).astype(np.uint16)      # fp16 exponent + 1
    assert np.all(np.isfinite(doubled.view(np.float16)))
    y2, b2 = orc.gemm(inp.act, inp.qweight, doubled, inp.qzeros, inp.group)
    assert np.array_equal(y2, 2 * y) and np.array_equal(b2, 2 * b)
    neg = (inp.act ^ np.uint16(0x8000)).astype(np.uint16)              # bf16 sign flip
    yn, bn = orc.gemm(neg, inp.qweight, inp.scales, inp.qzeros, inp.group)
    assert np.array_equal(yn, -y) and np.array_equal(bn, b)


def test_transpose_sensitivity(orc):
    """Swapping the roles of rows and columns must change the result (catches a transposed read)."""
    rng = np.random.default_rng(14)
    K = N = 64
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    act = synth.f32_to_bf16_bits(rng.standard_normal((1, K)).astype(np.float32))
    scales = np.full((1, N), 0x3C00, dtype=np.uint16)
    y, _ = orc.gemm(act, synth.pack_rows(codes), scales, None, 64)
    yt, _ = orc.gemm(act, synth.pack_rows(np.ascontiguousarray(codes.T)), scales, None, 64)
    a = torch.from_numpy(act.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.allclose(y, a @ (codes.astype(np.float64) - 8), rtol=1e-12, atol=1e-12)
    assert not np.allclose(y, yt)


# ---- argmax ----------------------------------------------------------------------------

def test_argmax_ties_take_lowest_index(orc):
    v = np.array([[1, 5, 5, 2], [3, 3, 3, 3], [-1, -7, -1, -2], [0, np.nan, 4, 4]], dtype=np.float32)
    assert orc.argmax_rows_f32(v).tolist() == [1, 0, 0, 2]
    rng = np.random.default_rng(15)
    r = rng.integers(0, 5, size=(6, 300)).astype(np.float32)
    assert orc.argmax_rows_f32(r).tolist() == np.argmax(r, axis=1).tolist()   # numpy: first max


def test_topk_hand_cases(orc):
    """Worked by hand: best first, equal values by lowest column, -0 equal to +0, NaN never
    chosen, -1 once a row has run out."""
    v = np.array([[1, 5, 5, 2],
                  [3, 3, 3, 3],
                  [0.0, -0.0, 0.0, -1],
                  [np.nan, 4, np.nan, 2],
                  [np.nan, np.nan, np.nan, np.nan]], dtype=np.float32)
    assert orc.topk_rows_f32(v, 3).tolist() == [[1, 2, 3], [0, 1, 2], [0, 1, 2], [1, 3, -1], [-1, -1, -1]]
    assert orc.topk_rows_f32(v, 6).tolist()[0] == [1, 2, 3, 0, -1, -1]


def test_topk_against_a_stable_sort(orc):
    """Brute force on small rows by another route: numpy's stable argsort of the negated values
    orders the non-NaN entries largest first with ties by lowest column (negation maps -0 and +0
    to the same key as +0 and -0 do to each other); the first k of it, padded with -1, and k = 1
    is the greedy pick."""
    rng = np.random.default_rng(16)
    for trial in range(40):
        M, N = int(rng.integers(1, 5)), int(rng.integers(1, 40))
        r = rng.integers(-3, 4, size=(M, N)).astype(np.float32)   # many ties
        r[rng.random((M, N)) < 0.1] = np.nan
        r[rng.random((M, N)) < 0.1] = -0.0
        for k in (1, 2, 5, N, N + 3):
            got = orc.topk_rows_f32(r, k)
            for m in range(M):
                ok = np.flatnonzero(~np.isnan(r[m]))
                order = ok[np.argsort(-r[m][ok], kind="stable")].tolist()
                want = (order + [-1] * k)[:k]
                assert got[m].tolist() == want, (trial, m, k)
            if k == 1:
                greedy = orc.argmax_rows_f32(r)
                has = ~np.all(np.isnan(r), axis=1)
                assert got[has, 0].tolist() == greedy[has].tolist()


def test_oracle_rejects_bad_arguments(orc):
    inp = synth.make_random(16, 1, 64, 16, 32, symmetric=True)
    with pytest.raises(ValueError):
        orc.gemm(inp.act, inp.qweight, inp.scales, None, 48)                 # K % g != 0
    with pytest.raises(ValueError):
        orc.gemm(inp.act, inp.qweight, inp.scales, None, 32, cols=[16])      # column out of range


# ---- the gated feed-forward input: silu(A x W_gate) * (A x W_up) --------------------------

def test_silu_closed_forms(orc):
    """silu(x) = x * logistic(x): logistic(1) = e / (1 + e), silu(0) = 0, silu(x) -> x for large
    x and -> 0 for large -x, and the odd part silu(x) - silu(-x) = x."""
    e = float(np.e)
    assert orc.silu(0.0) == 0.0
    assert abs(orc.silu(1.0) - e / (1.0 + e)) <= 1e-16
    assert abs(orc.silu(2.0) - 2.0 * e * e / (1.0 + e * e)) <= 1e-15
    assert orc.silu(64.0) == 64.0
    assert -1e-20 < orc.silu(-64.0) < 0.0
    for x in (0.25, 1.5, 3.0, 7.0, 20.0):
        assert abs((orc.silu(x) - orc.silu(-x)) - x) <= 4e-15 * max(1.0, x)


def test_silu_slope_bound(orc):
    """The test tolerance for the gated product uses max |silu'| <= 1.1 (the true maximum is
    about 1.0998, reached near x = 2.4): checked by finite differences on a fine grid."""
    x = np.linspace(-20.0, 20.0, 40001)
    s = np.array([orc.silu(v) for v in x])
    slope = np.abs(np.diff(s) / np.diff(x))
    assert 1.09 < slope.max() < 1.1


def test_silu_mul_elementwise(orc):
    e = float(np.e)
    g = np.array([[0.0, 1.0, -1.0], [64.0, 2.0, -64.0]])
    u = np.array([[5.0, 2.0, 3.0], [-1.0, 0.5, 7.0]])
    h = orc.silu_mul(g, u)
    expect = np.array([[0.0, 2.0 * e / (1 + e), -3.0 / (1 + e)], [-64.0, e * e / (1 + e * e), 0.0]])
    assert np.allclose(h, expect, rtol=1e-15, atol=1e-18)


def test_gate_up_orientation(orc):
    """All-ones activations, gate weights +1 and up weights -1 (unit scales): gate = K, up = -K
    in every column, so h = silu(K) * (-K) = -K^2 exactly; with gate and up swapped the
    result would be silu(-K) * K, about -K^2 e^-K."""
    K, N, g = 64, 16, 32
    ones = np.full((1, K), 0x3F80, np.uint16)            # bf16 1.0
    unit = np.full((K // g, N), 0x3C00, np.uint16)       # fp16 1.0
    gate = (synth.pack_rows(np.full((K, N), 9)), unit, None)   # 9 - 8 = +1
    up = (synth.pack_rows(np.full((K, N), 7)), unit, None)     # 7 - 8 = -1
    h, yg, bg, yu, bu = orc.gate_up(ones, gate, up, g)
    assert np.all(yg == K) and np.all(yu == -K) and np.all(bg == K) and np.all(bu == K)
    assert np.all(h == -float(K * K))
    h2 = orc.gate_up(ones, up, gate, g)[0]
    assert np.all((h2 < 0) & (h2 > -1e-20))


def test_gate_up_column_subset(orc):
    inp = synth.make_random(17, 3, 256, 64, 64, symmetric=False)
    inp2 = synth.make_random(18, 3, 256, 64, 64, symmetric=False)
    gate = (inp.qweight, inp.scales, inp.qzeros)
    up = (inp2.qweight, inp2.scales, inp2.qzeros)
    full = orc.gate_up(inp.act, gate, up, 64)[0]
    cols = [0, 7, 8, 33, 63]
    assert np.array_equal(orc.gate_up(inp.act, gate, up, 64, cols=cols)[0], full[:, cols])


def test_gate_up_bar_rejects_plausible_mistakes(orc):
    """The gated-product bar passes the exact product rounded to fp32 and rejects a missing
    nonlinearity, swapped operands and a bare logistic gate."""
    from tests import parity
    inp = synth.make_random(19, 4, 512, 128, 128, symmetric=True)
    inp2 = synth.make_random(20, 4, 512, 128, 128, symmetric=True)
    h, yg, bg, yu, bu = orc.gate_up(inp.act, (inp.qweight, inp.scales, None), (inp2.qweight, inp2.scales, None), 128)
    parity.check_gate_up(h.astype(np.float32), h, yg, bg, yu, bu, "fp32 rounding")
    logistic = orc.silu_mul(yg, np.ones_like(yg)) / np.where(yg == 0, 1.0, yg)
    for wrong in (yg * yu, orc.silu_mul(yu, yg), logistic * yu):
        with pytest.raises(AssertionError):
            parity.check_gate_up(wrong, h, yg, bg, yu, bu, "planted")
