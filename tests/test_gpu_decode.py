"""GPU parity of the decode kernel (w4a16_gemm_decode_ex) against the oracle.

Every launch knob (slices along K, waves per workgroup, tile width, weight ring) over ragged
shapes: N not a multiple of a workgroup's columns, K slices that do not divide K or the groups,
group sizes from 32 to 4096, both zero-point forms, every row count from 1 to 16. Bar: the
matmul bar of tests/parity.py. Also the invariants that hold bit for bit: outputs exactly zero
when every code equals its zero point, an exact integer matmul, bit-identical repeats, row
permutation, the bf16 output equal to the fp32 output rounded once.
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


def run(gu, d, M, slices=0, tiles=0, kw=0, cols=0, ring=0, out_dtype=torch.float32, act=None):
    a = d.act[:M] if act is None else act
    out = torch.full((M, d.N), float("nan"), dtype=out_dtype, device=gu.DEV)
    vm.w4a16_gemm_decode_ex(a, d.qweight, d.scales, d.qzeros, d.group, out, slices, tiles, kw, cols, ring)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def refused(launch, M, N, K, g, packed):
    """Whether the library refuses an explicit launch; asked of the host-only planner, which does
    no device work (the same checks as the call)."""
    slices, tiles, kw, cols, ring = launch
    try:
        vm.w4a16_decode_plan(M, N, K, g, packed, slices, tiles, kw, cols, ring)
    except vm.W4A16Error as e:
        assert e.status == -1 and ("LDS" in str(e) or "activation items" in str(e) or "K-steps" in str(e)), str(e)
        return True
    return False


SHAPES = [  # K, N, g, symmetric
    (512, 256, 128, True),
    (1024, 520, 64, False),
    (2048, 1000, 128, True),
    (4096, 2056, 32, False),
    (1536, 136, 128, False),
    (8192, 264, 4096, True),
]
# (slices, tiles, kw, tile_cols, ring); 0 = the default for that knob
LAUNCHES = [(0, 0, 0, 0, 0), (1, 1, 1, 64, 2), (3, 2, 1, 64, 3), (16, 4, 1, 64, 4), (5, 8, 1, 128, 2),
            (2, 3, 1, 128, 4), (7, 1, 1, 64, 8), (4, 4, 1, 64, 6), (11, 5, 1, 64, 3), (1, 8, 1, 64, 4),
            (2, 2, 4, 64, 4), (1, 1, 8, 64, 3), (3, 4, 2, 64, 8), (2, 1, 3, 128, 2), (4, 2, 2, 128, 4),
            (1, 2, 4, 64, 6), (0, 2, 4, 0, 0), (0, 1, 8, 0, 0)]


@pytest.mark.parametrize("K,N,g,sym", SHAPES)
def test_decode_sweep(gu, K, N, g, sym):
    steps = K // 32
    inp = synth.make_random(1000 + K + N + g, 16, K, N, g, symmetric=sym)
    d = gu.DevInputs(inp)
    for M in (1, 2, 3, 5, 8, 13, 16):
        y_ref, bound = oracle.gemm(inp.act[:M], inp.qweight, inp.scales, inp.qzeros, g)
        worst = 0.0
        for launch in LAUNCHES:
            if refused(launch, M, N, K, g, not sym):
                continue   # refused on the host (K steps, LDS or registers); tested on the CPU
            gu.say(f"[decode] K={K} N={N} g={g} sym={sym} M={M} (slices, tiles, kw, cols, ring)={launch}")
            y = run(gu, d, M, *launch)
            worst = max(worst, parity.check_close(y, y_ref, bound, f"K={K} N={N} g={g} M={M} {launch}"))
        gu.say(f"  M={M} worst err/tol {worst:.3e}")


def test_decode_bf16_is_fp32_rounded_once(gu):
    inp = synth.make_random(77, 16, 2048, 1000, 128, symmetric=False)
    d = gu.DevInputs(inp)
    for M in (1, 7, 16):
        for launch in ((0, 0, 0, 0, 0), (4, 2, 1, 128, 2), (2, 2, 2, 64, 4)):
            y = run(gu, d, M, *launch)
            yb = run(gu, d, M, *launch, out_dtype=torch.bfloat16)
            assert np.array_equal(yb, torch.from_numpy(y.astype(np.float32)).to(torch.bfloat16).double().numpy())


def test_decode_invariants(gu):
    K, N, g = 2048, 776, 64
    rng = np.random.default_rng(31)
    # q == z everywhere: exactly zero
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    zeros = rng.integers(0, 16, size=(K // g, N), dtype=np.uint8)
    codes = np.repeat(zeros, g, axis=0)
    act = synth.f32_to_bf16_bits(rng.standard_normal((16, K)).astype(np.float32) * 30)
    qz = synth.Inputs(synth.pack_rows(codes), synth.draw_scales(rng, (K // g, N), 0.002, 0.02), synth.pack_cols(zeros),
                      act, g)
    d = gu.DevInputs(qz)
    for M in (1, 4, 16):
        for launch in ((0, 0, 0, 0, 0), (16, 4, 1, 64, 4), (3, 4, 2, 128, 2), (2, 2, 4, 64, 4)):
            assert np.all(run(gu, d, M, *launch) == 0.0)
    # unit scales, zero point 0, integer activations in [-8, 8]: an exact integer matmul
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    ai = rng.integers(-8, 9, size=(16, K)).astype(np.float32)
    one = synth.f64_to_fp16_bits(np.ones((K // g, N)))
    ex = synth.Inputs(synth.pack_rows(codes), one, synth.pack_cols(np.zeros((K // g, N), np.uint8)),
                      synth.f32_to_bf16_bits(ai), g)
    d = gu.DevInputs(ex)
    for M in (1, 5, 16):
        ref = ai[:M].astype(np.int64) @ codes.astype(np.int64)
        for launch in ((0, 0, 0, 0, 0), (16, 4, 1, 64, 4), (5, 8, 1, 128, 2), (4, 1, 2, 64, 2), (2, 2, 4, 64, 3)):
            assert np.array_equal(run(gu, d, M, *launch), ref.astype(np.float64)), (M, launch)
    # repeats are bit-identical; permuting rows permutes outputs bit for bit
    inp = synth.make_random(32, 16, K, N, g, symmetric=False)
    d = gu.DevInputs(inp)
    perm = rng.permutation(16)
    a_perm = d.act[torch.from_numpy(perm).to(gu.DEV)].contiguous()
    for launch in ((0, 0, 0, 0, 0), (16, 4, 1, 64, 4), (3, 4, 2, 128, 2), (2, 2, 4, 64, 4)):
        y1 = run(gu, d, 16, *launch)
        assert np.array_equal(run(gu, d, 16, *launch), y1)
        assert np.array_equal(run(gu, d, 16, *launch, act=a_perm), y1[perm])


_WL_CASES = [("tiny", 1), ("attn", 1), ("attn", 16)] + [("ffn_up", m) for m in (1, 2, 4, 8, 16)] + \
            [("ffn_down", m) for m in (1, 4, 8, 16)]


@pytest.mark.parametrize("name,M", _WL_CASES)
def test_decode_workloads(gu, name, M):
    inp = synth.make_inputs(name)
    d = gu.DevInputs(inp)
    y_ref, bound = oracle.gemm(inp.act[:M], inp.qweight, inp.scales, inp.qzeros, inp.group)
    y = run(gu, d, M)
    frac = parity.check_close(y, y_ref, bound, f"{name} M={M}")
    gu.say(f"[decode workload] {name} M={M} worst err/tol {frac:.3e}")


@pytest.mark.parametrize("K,N,g,sym", [(512, 1000, 128, True), (1024, 4104, 64, False), (512, 131072, 128, True),
                                      (64, 256, 32, False)])
def test_decode_fused_topk(gu, K, N, g, sym):
    """The k best columns per row picked inside the decode kernel's launch, single-slice and
    through the slice reducer, on every launch knob: logits bit-identical to the same launch
    without the pick and within the bar against the oracle, indices equal to the oracle's k best
    over those fp32 logits (both sides decide in fp32: bit-exact), k = 1 equal to the separate
    greedy pick. Ragged groups of columns; K = 64 gives slices too short to hold the outputs in
    the fragments' LDS, which the plan enlarges."""
    inp = synth.make_random(K + N + 7, 16, K, N, g, symmetric=sym)
    d = gu.DevInputs(inp)
    for M in (1, 2, 5, 16):
        y_ref, bound = oracle.gemm(inp.act[:M], inp.qweight, inp.scales, inp.qzeros, g)
        for launch in ((0, 0, 0, 0, 0), (1, 4, 1, 64, 4), (3, 2, 2, 64, 3), (4, 4, 1, 128, 2), (1, 8, 1, 128, 4)):
            for k in (1, 3, 8):
                try:
                    vm.w4a16_decode_plan(M, N, K, g, not sym, *launch, topk=k)
                except vm.W4A16Error:
                    continue   # refused on the host (K steps or LDS); tested on the CPU
                gu.say(f"[decode topk] K={K} N={N} M={M} launch={launch} k={k}")
                plain = run(gu, d, M, *launch)
                out = torch.full((M, N), float("nan"), dtype=torch.float32, device=gu.DEV)
                idx = torch.full((M, k), -5, dtype=torch.int32, device=gu.DEV)
                vm.w4a16_gemm_decode_ex(d.act[:M], d.qweight, d.scales, d.qzeros, g, out, *launch, idx=idx)
                torch.cuda.synchronize()
                y = out.double().cpu().numpy()
                assert np.array_equal(y, plain)
                got = idx.cpu().numpy().astype(np.int64)
                assert np.array_equal(got, oracle.topk_rows_f32(out.cpu().numpy(), k)), (M, launch, k)
                if k == 1:
                    sep = torch.empty((M,), dtype=torch.int32, device=gu.DEV)
                    vm.w4a16_argmax_rows(out, sep)
                    torch.cuda.synchronize()
                    assert got[:, 0].tolist() == sep.cpu().tolist()
                parity.check_close(y, y_ref, bound, f"topk K={K} N={N} M={M} {launch} k={k}")


def test_decode_topk_rows_that_run_out(gu):
    """Ties and rows with fewer numbers than k: all-zero activations make every output of a row
    equal (picked by lowest column); NaN scales make their columns' outputs NaN, never picked, so a
    row with four numbers gives four columns and then -1, and a row with none gives -1 throughout
    (w4a16_gemm_argmax gives 0 there)."""
    K, N, g = 32, 8, 32
    inp = synth.make_random(4242, 4, K, N, g, symmetric=True)
    d = gu.DevInputs(inp)
    out = torch.empty((4, N), dtype=torch.float32, device=gu.DEV)
    idx = torch.full((4, 8), -5, dtype=torch.int32, device=gu.DEV)
    vm.w4a16_gemm_topk(d.act[:4], d.qweight, d.scales, None, g, out, idx)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy().astype(np.int64), oracle.topk_rows_f32(out.cpu().numpy(), 8))
    zero = torch.zeros((4, K), dtype=torch.int16, device=gu.DEV)
    vm.w4a16_gemm_topk(zero, d.qweight, d.scales, None, g, out, idx)
    torch.cuda.synchronize()
    assert idx.cpu().tolist() == [list(range(8))] * 4
    nan_half = d.scales.clone()
    nan_half[:, 1::2] = 0x7E00   # fp16 NaN scale on the odd columns
    vm.w4a16_gemm_topk(d.act[:4], d.qweight, nan_half, None, g, out, idx)
    torch.cuda.synchronize()
    logits = out.cpu().numpy()
    assert np.all(np.isnan(logits[:, 1::2])) and not np.any(np.isnan(logits[:, 0::2]))
    got = idx.cpu().numpy().astype(np.int64)
    assert np.array_equal(got, oracle.topk_rows_f32(logits, 8))
    assert np.all(got[:, 4:] == -1) and np.all(got[:, :4] % 2 == 0)
    nan_all = torch.full_like(d.scales, 0x7E00)
    vm.w4a16_gemm_topk(d.act[:4], d.qweight, nan_all, None, g, out, idx)
    torch.cuda.synchronize()
    assert idx.cpu().tolist() == [[-1] * 8] * 4
