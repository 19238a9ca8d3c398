"""GPU invariants and edge cases that hold exactly (bit for bit), plus degenerate inputs."""
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


ROWS = [1, 2, 5, 16]


def test_codes_equal_zeros_give_zero(gu):
    """q == z everywhere: every product is exactly zero, so every output is exactly zero."""
    rng = np.random.default_rng(21)
    K, N, g = 1024, 520, 64
    zeros = rng.integers(0, 16, size=(K // g, N), dtype=np.uint8)
    inp = synth.Inputs(synth.pack_rows(np.repeat(zeros, g, axis=0)), synth.draw_scales(rng, (K // g, N), 0.001, 0.05),
                       synth.pack_cols(zeros), synth.f32_to_bf16_bits(rng.standard_normal((16, K)).astype(np.float32) * 100),
                       g)
    d = gu.DevInputs(inp)
    sym = synth.Inputs(np.full((K // 8, N), 0x88888888, np.uint32), inp.scales, None, inp.act, g)
    ds = gu.DevInputs(sym)
    for M in ROWS:
        for splits, wk, cols in ((1, 1, 0), (3, 2, 0), (0, 0, 0), (3, 2, 128)):
            gu.say(f"[q==z] M={M} splits={splits} waves_k={wk} tile_cols={cols}")
            assert np.all(d.run(M, splits=splits, waves_k=wk, tile_cols=cols) == 0.0)
            assert np.all(ds.run(M, splits=splits, waves_k=wk, tile_cols=cols) == 0.0)


def test_integer_matmul_is_exact(gu):
    """scale 1, zero 0, integer activations: every partial sum is an integer below 2^24."""
    rng = np.random.default_rng(22)
    K, N, g = 17408, 264, 64
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    ai = rng.integers(-8, 9, size=(16, K))
    inp = synth.Inputs(synth.pack_rows(codes), np.full((K // g, N), 0x3C00, np.uint16),
                       np.zeros((K // g, N // 8), np.uint32), synth.f32_to_bf16_bits(ai.astype(np.float32)), g)
    d = gu.DevInputs(inp)
    for M in ROWS:
        ref = (ai[:M].astype(np.int64) @ codes.astype(np.int64)).astype(np.float64)
        assert np.abs(ref).max() < 2 ** 24
        for splits, wk, cols in ((0, 0, 0), (17, 2, 0), (40, 8, 0), (1, 16, 0), (0, 0, 128), (17, 2, 128)):
            gu.say(f"[integer] M={M} splits={splits} waves_k={wk} tile_cols={cols}")
            assert np.array_equal(d.run(M, splits=splits, waves_k=wk, tile_cols=cols), ref)


def test_scaling_negation_permutation_and_repeat(gu):
    inp = synth.make_random(23, 16, 2048, 1032, 128, symmetric=False)
    d = gu.DevInputs(inp)
    doubled = gu.DevInputs(synth.Inputs(inp.qweight, (inp.scales + np.uint16(0x0400)).astype(np.uint16),
                                        inp.qzeros, inp.act, inp.group))
    neg_act = gu.dev_u16((inp.act ^ np.uint16(0x8000)).astype(np.uint16))
    for M in ROWS:
        gu.say(f"[invariants] M={M}")
        y = d.run(M)
        assert np.array_equal(doubled.run(M), 2 * y)
        assert np.array_equal(d.run(M, act=neg_act[:M]), -y)
        for _ in range(5):
            assert np.array_equal(d.run(M), y)          # deterministic split-K
        if M > 1:
            perm = np.random.default_rng(M).permutation(M)
            yp = d.run(M, act=gu.dev_u16(inp.act[:M][perm]))
            assert np.array_equal(yp, y[perm])


def test_explicit_zero_eight_equals_symmetric(gu):
    inp = synth.make_random(24, 16, 1024, 512, 128, symmetric=True)
    d = gu.DevInputs(inp)
    z8 = gu.DevInputs(synth.Inputs(inp.qweight, inp.scales, np.full((8, 64), 0x88888888, np.uint32), inp.act, 128))
    for M in ROWS:
        assert np.array_equal(d.run(M), z8.run(M))


def test_zero_activations_and_zero_scales(gu):
    inp = synth.make_random(25, 16, 512, 256, 64, symmetric=False)
    zero_act = gu.DevInputs(synth.Inputs(inp.qweight, inp.scales, inp.qzeros, np.zeros_like(inp.act), 64))
    zero_sc = gu.DevInputs(synth.Inputs(inp.qweight, np.zeros_like(inp.scales), inp.qzeros, inp.act, 64))
    for M in ROWS:
        assert np.all(zero_act.run(M) == 0.0)
        assert np.all(zero_sc.run(M) == 0.0)


def test_wide_dynamic_range_rows(gu):
    """Rows with exponents spread over 2^+-14, and whole rows far outside fp16's range, stay within
    the bar (the per-row power-of-two rescale keeps them representable)."""
    rng = np.random.default_rng(26)
    K, N, g = 2048, 512, 128
    base = rng.standard_normal((16, K)).astype(np.float32)
    expo = rng.integers(-14, 15, size=(16, K)).astype(np.float32)
    a = base * np.exp2(expo)
    a[3] *= np.float32(2.0 ** 40)     # whole row far above fp16's largest value
    a[4] *= np.float32(2.0 ** -60)    # whole row far below fp16's smallest normal
    inp = synth.Inputs(synth.random_words(rng, (K // 8, N)), synth.draw_scales(rng, (K // g, N), 0.002, 0.02),
                       synth.random_words(rng, (K // g, N // 8)), synth.f32_to_bf16_bits(a), g)
    d = gu.DevInputs(inp)
    for M in (1, 5, 16):
        y_ref, bound = oracle.gemm(inp.act[:M], inp.qweight, inp.scales, inp.qzeros, g)
        for splits, wk in ((1, 1), (2, 4), (0, 0)):
            gu.say(f"[range] M={M} splits={splits} waves_k={wk}")
            parity.check_close(d.run(M, splits=splits, waves_k=wk), y_ref, bound, f"range M={M}")


def test_activation_span_at_the_documented_edge(gu):
    """The accuracy contract holds for rows whose nonzero activations span up to 2^29 within one
    K slice. Each row carries one outlier 2^29 times larger than its other entries (which lie in
    [1, 2)), and in about half of the columns the outlier's code equals its zero point, so the
    outlier contributes nothing there and the bound is made of the small entries alone: they
    must reach the matrix cores without losing a bit for those columns to pass."""
    rng = np.random.default_rng(27)
    K, N, g = 1024, 512, 64
    a = (1.0 + rng.random((16, K))).astype(np.float32) * rng.choice([-1.0, 1.0], size=(16, K)).astype(np.float32)
    pos = rng.integers(0, K, size=16)
    a[np.arange(16), pos] *= np.float32(2.0 ** 29)
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    zeros = rng.integers(0, 16, size=(K // g, N), dtype=np.uint8)
    half = rng.random(N) < 0.5
    for m in range(16):   # the outlier's code equals the zero point in the chosen columns
        codes[pos[m], half] = zeros[pos[m] // g, half]
    inp = synth.Inputs(synth.pack_rows(codes), synth.draw_scales(rng, (K // g, N), 0.002, 0.02),
                       synth.pack_cols(zeros), synth.f32_to_bf16_bits(a), g)
    d = gu.DevInputs(inp)
    for M in (1, 4, 16):
        y_ref, bound = oracle.gemm(inp.act[:M], inp.qweight, inp.scales, inp.qzeros, g)
        for splits, wk, cols in ((0, 0, 0), (1, 1, 0), (4, 2, 0), (2, 4, 128)):
            gu.say(f"[span 2^29] M={M} splits={splits} waves_k={wk} tile_cols={cols}")
            frac = parity.check_close(d.run(M, splits=splits, waves_k=wk, tile_cols=cols), y_ref, bound,
                                      f"span M={M} {splits}/{wk}/{cols}")
            gu.say(f"  worst err/tol {frac:.3e}")


def test_power_of_two_activation_scaling_is_exact(gu):
    """Scaling every activation by 2^k scales every output by exactly 2^k: the per-slice rescale
    into fp16 is exact, so it absorbs any power of two, from slices far below fp16's range to
    slices above it, and for held and LDS-staged slices alike."""
    rng = np.random.default_rng(27)
    K, N, g = 2048, 520, 128
    mag = np.exp2(rng.uniform(-6.0, 2.0, size=(16, K))).astype(np.float32)
    a = np.where(rng.integers(0, 2, size=(16, K)) == 1, mag, -mag).astype(np.float32)
    a[rng.random((16, K)) < 0.05] = 0.0       # exact zeros: must stay zero in either form
    a[:, ::32] = 3.0                          # every slice's largest magnitude is in [2, 4)
    a = a.view(np.uint32) & np.uint32(0xFFFF0000)   # already bf16: scaling by 2^k stays exact
    base = synth.f32_to_bf16_bits(a.view(np.float32))
    inp = synth.Inputs(synth.random_words(rng, (K // 8, N)), synth.draw_scales(rng, (K // g, N), 0.002, 0.02),
                       synth.random_words(rng, (K // g, N // 8)), base, g)
    d = gu.DevInputs(inp)
    launches = ((0, 0, 0), (1, 1, 0), (4, 2, 0), (0, 0, 128))
    for M in (1, 5, 16):
        ys = {c: d.run(M, splits=c[0], waves_k=c[1], tile_cols=c[2]) for c in launches}
        for k in (-90, -89, -40, 13, 14, 20):
            scaled = synth.f32_to_bf16_bits(a.view(np.float32)[:M] * np.float32(2.0 ** k))
            act = gu.dev_u16(scaled)
            for c in launches:
                gu.say(f"[2^k] M={M} k={k} splits={c[0]} waves_k={c[1]} tile_cols={c[2]}")
                assert np.array_equal(d.run(M, act=act, splits=c[0], waves_k=c[1], tile_cols=c[2]),
                                      ys[c] * 2.0 ** k)


def test_argmax_edge_cases(gu):
    rows = []
    N = 40000                                   # more than two argmax chunks, ragged tail
    r = np.zeros(N, np.float32); r[[17, 39999, 20000]] = 3.0; rows.append(r)       # ties -> 17
    r = np.full(N, -np.inf, np.float32); r[39999] = -1e30; rows.append(r)           # max at the end
    r = np.full(N, np.nan, np.float32); r[123] = -5.0; r[5] = -7.0; rows.append(r)   # NaNs ignored
    r = np.full(N, -0.0, np.float32); r[9] = 0.0; rows.append(r)                    # -0 == +0 -> 0
    r = np.full(N, np.nan, np.float32); rows.append(r)                              # all NaN -> 0
    r = np.random.default_rng(27).standard_normal(N).astype(np.float32); rows.append(r)
    v = np.stack(rows)
    t = torch.from_numpy(v).to(gu.DEV)
    idx = torch.empty((v.shape[0],), dtype=torch.int32, device=gu.DEV)
    for _ in range(3):   # keys and counters must be left clean for the next call
        vm.w4a16_argmax_rows(t, idx)
        torch.cuda.synchronize()
        got = idx.cpu().numpy()
        assert got.tolist()[:5] == [17, 39999, 123, 0, 0]
        assert np.array_equal(got.astype(np.int64), oracle.argmax_rows_f32(v))
    one = torch.tensor([[2.5]], device=gu.DEV)
    i1 = torch.empty((1,), dtype=torch.int32, device=gu.DEV)
    vm.w4a16_argmax_rows(one, i1)
    torch.cuda.synchronize()
    assert int(i1.item()) == 0


def test_errors_do_not_touch_the_device(gu):
    inp = synth.make_random(28, 1, 512, 256, 128, symmetric=True)
    d = gu.DevInputs(inp)
    out = torch.zeros((1, 256), dtype=torch.float32, device=gu.DEV)
    with pytest.raises(vm.W4A16Error):
        vm.w4a16_gemm_ex(d.act[:1], d.qweight, d.scales, None, 128, out, 999, 1)
    torch.cuda.synchronize()
    assert torch.all(out == 0)


def test_stream_read_hook_reads_without_writing(gu):
    """The read-ceiling hook reads any size (a ragged last workgroup included) and leaves its
    inputs and, unless the fold hits its constant, its sink untouched."""
    for nbytes in (16, 16 * 1024, 16 * 1024 + 48, 3 * 2 ** 20 + 16 * 77):
        buf = torch.arange(nbytes // 4, dtype=torch.int32, device=gu.DEV)
        before = buf.clone()
        sink = torch.full((4,), 7, dtype=torch.int32, device=gu.DEV)
        vm.w4a16_stream_read(buf, sink)
        torch.cuda.synchronize()
        assert torch.equal(buf, before)
        assert sink.cpu().tolist() == [7, 7, 7, 7]
