"""GPU parity of the affine prompt GEMM (w4a16_gemm_affine_bits_prefill: w = s * q + b, codes of 1,
2, 3, 4, 5, 6 and 8 bits read at their own width on the many-row kernel) against the oracle.

Every width over ragged shapes (M and N not multiples of the 64 x 256 tile, groups of 32, 64 and
128), launches with K slices (few tiles) and without (a full round of tiles, checked on sampled
rows and columns), the affine bar of the oracle, |y - y_oracle| <= 4e-3 * sum_k |a_k|
(|s q_k| + |b|) + 1e-6. Bit-exact invariants: an integer matmul (unit scales, zero biases,
integer activations), the group sums of the activations through a bias-only matrix, a row
permutation of A permuting the output rows, bit-identical repeats, and the bf16 output equal to
the fp32 output rounded once. Rows 0..15 also agree with the small-row path within the bar.
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
        self.N = x.packed.shape[1]
        self.packed = gu.dev_u32(x.packed)
        self.scales = gu.dev_u16(x.scales)
        self.biases = gu.dev_u16(x.biases)
        self.act = gu.dev_u16(x.act)

    def run(self, act=None, out_dtype=torch.float32, scales=None, biases=None):
        act = self.act if act is None else act
        out = torch.full((act.shape[0], self.N), float("nan"), dtype=out_dtype, device=self.gu.DEV)
        vm.w4a16_gemm_affine_bits_prefill(act, self.packed, self.x.bits, self.scales if scales is None else scales,
                                          self.biases if biases is None else biases, self.x.group, out)
        torch.cuda.synchronize()
        return out.float().cpu().numpy().astype(np.float64)


# (M, K, N, g): ragged M and N; every one of these has fewer tiles than the device runs at once,
# so the call cuts K into whole-group slices
SHAPES = [(37, 512, 264, 64), (130, 1024, 520, 32), (200, 2048, 1000, 128), (1, 256, 72, 64), (65, 1024, 136, 128)]


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("M,K,N,g", SHAPES)
def test_affine_prefill_parity(gu, M, K, N, g, bits):
    x = synth.make_affine_random(8000 + 17 * bits + M + N, M, K, N, g, bits)
    d = Dev(gu, x)
    gu.say(f"[affine prefill] M={M} K={K} N={N} g={g} bits={bits}")
    y = d.run()
    y_ref, bound = oracle.affine_gemm(x.act, x.packed, bits, x.scales, x.biases, g)
    frac = parity.check_close(y, y_ref, bound, f"affine prefill bits={bits} M={M} K={K} N={N}")
    gu.say(f"  worst err/tol {frac:.3e}")
    yb = d.run(out_dtype=torch.bfloat16)
    assert np.array_equal(yb, torch.from_numpy(y.astype(np.float32)).to(torch.bfloat16).double().numpy())
    assert np.array_equal(d.run(), y)


@pytest.mark.parametrize("bits", (2, 3, 4, 8))
def test_affine_prefill_whole_k(gu, bits):
    """A full round of tiles (2048 x 4096: 512 tiles of 64 x 256), so no K slices, checked on
    sampled rows (the oracle's rows are independent) and on sampled columns that include the last
    tile."""
    M, K, N, g = 2048, 512, 4096, 64
    x = synth.make_affine_random(8100 + bits, M, K, N, g, bits)
    d = Dev(gu, x)
    gu.say(f"[affine prefill whole K] M={M} K={K} N={N} bits={bits}")
    y = d.run()
    rng = np.random.default_rng(bits)
    rows = np.unique(np.concatenate([rng.choice(M, 48, replace=False), np.arange(M - 64, M)]))
    y_ref, bound = oracle.affine_gemm(x.act[rows], x.packed, bits, x.scales, x.biases, g)
    frac = parity.check_close(y[rows], y_ref, bound, f"affine prefill whole K bits={bits}")
    cols = np.unique(np.concatenate([rng.choice(N, 300, replace=False), np.arange(N - 260, N)]))
    y_ref, bound = oracle.affine_gemm(x.act[:64], x.packed, bits, x.scales, x.biases, g, cols)
    frac = max(frac, parity.check_close(y[:64][:, cols], y_ref, bound, f"affine prefill whole K cols bits={bits}"))
    gu.say(f"  worst err/tol {frac:.3e}")


@pytest.mark.parametrize("bits", BITS)
def test_affine_prefill_exact_cases(gu, bits):
    """Unit scales, zero biases and integer activations: an exact integer matmul, every code value
    present; a row permutation of A permutes the output rows bit for bit; zero scales and unit
    biases give each row's activation sum in every column."""
    M, K, N, g = 150, 1024, 264, 64
    rng = np.random.default_rng(100 + bits)
    codes = rng.integers(0, 1 << bits, size=(K, N), dtype=np.uint32)
    codes[:1 << bits, 0] = np.arange(1 << bits)
    packed = synth.pack_stream(codes, bits)
    one = np.full((K // g, N), 0x3F80, np.uint16)   # bf16 1.0
    zero = np.zeros((K // g, N), np.uint16)
    ai = rng.integers(-8, 9, size=(M, K)).astype(np.float32)
    x = synth.AffineInputs(packed, bits, one, zero, synth.f32_to_bf16_bits(ai), g)
    d = Dev(gu, x)
    y = d.run()
    assert np.array_equal(y, (ai.astype(np.int64) @ codes.astype(np.int64)).astype(np.float64)), bits
    perm = rng.permutation(M)
    assert np.array_equal(d.run(act=gu.dev_u16(x.act[perm])), y[perm])
    ys = d.run(scales=gu.dev_u16(zero), biases=gu.dev_u16(one))
    assert np.array_equal(ys, np.repeat(ai.sum(axis=1, keepdims=True).astype(np.float64), N, axis=1)), bits


@pytest.mark.parametrize("bits", (3, 4, 6))
def test_affine_prefill_matches_small_row_path_within_the_bar(gu, bits):
    """Rows 0..15 through the prompt kernel and through w4a16_gemm_affine_bits: both within the
    bar of the oracle (the two kernels split and round K differently)."""
    K, N, g = 2048, 520, 64
    x = synth.make_affine_random(8200 + bits, 16, K, N, g, bits)
    d = Dev(gu, x)
    y_ref, bound = oracle.affine_gemm(x.act, x.packed, bits, x.scales, x.biases, g)
    parity.check_close(d.run(), y_ref, bound, f"affine prefill 16 rows bits={bits}")
    out = torch.empty((16, N), dtype=torch.float32, device=gu.DEV)
    vm.w4a16_gemm_affine_bits(d.act, d.packed, bits, d.scales, d.biases, g, out)
    torch.cuda.synchronize()
    parity.check_close(out.cpu().numpy().astype(np.float64), y_ref, bound, f"affine small-row 16 rows bits={bits}")


def test_affine_prefill_workload(gu):
    """The affine-4 FFN up projection (5120 x 17408, groups of 64) with 512 prompt rows, on sampled
    columns that span every tile position and the last tile."""
    x = synth.make_affine_inputs("ffn_up_affine4")
    K = x.packed.shape[0] * 32 // x.bits
    rng = np.random.Generator(np.random.PCG64(8300))
    act = synth.draw_activations(rng, 512, K, 1.0, 0.0, 1.0)
    d = Dev(gu, x)
    gu.say("[affine prefill workload] ffn_up_affine4 M=512")
    y = d.run(act=gu.dev_u16(act))
    N = d.N
    cols = np.unique(np.concatenate([rng.choice(N, 400, replace=False), np.arange(N - 130, N)]))
    y_ref, bound = oracle.affine_gemm(act, x.packed, x.bits, x.scales, x.biases, x.group, cols)
    frac = parity.check_close(y[:, cols], y_ref, bound, "affine prefill ffn_up_affine4 M=512")
    gu.say(f"  worst err/tol {frac:.3e}")
