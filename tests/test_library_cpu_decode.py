"""Host-side checks of the decode kernel's explicit launch (no GPU needed): refused knobs fail
with INVALID_ARG, asked of the host-only planner w4a16_decode_plan (the checks w4a16_gemm_decode_ex
makes before any device work)."""
import ctypes
import os

import pytest


@pytest.fixture(scope="module")
def lib():
    import verify_matmul_amd as vm
    if not os.path.exists(vm.lib_path):
        from verify_matmul_amd import _build
        _build.build()
    return vm.load()


def dec(lib, slices=0, tiles=0, kw=0, cols=0, ring=0, M=4, N=256, K=512, g=128, topk=0, bits=0):
    """The host-only planner: the same checks as w4a16_gemm_decode_ex, no device work."""
    return lib.w4a16_decode_plan(M, N, K, g, 0, slices, tiles, kw, cols, ring, topk, bits, None)


@pytest.mark.parametrize("kw,msg", [
    (dict(slices=17), b"slices"),            # above the 16 the kernel adds
    (dict(slices=17, K=1024), b"slices"),
    (dict(slices=20, K=512), b"slices"),     # 512 / 32 = 16 steps
    (dict(slices=5, tiles=2, kw=4, K=512), b"K-steps"),   # 5 x 4 pieces > 16 steps
    (dict(tiles=9), b"waves"),
    (dict(tiles=4, kw=3), b"waves"),         # 12 waves
    (dict(cols=96), b"tile_cols"),
    (dict(ring=5), b"ring"),
    (dict(ring=3, cols=128), b"ring"),
    (dict(slices=-1), b"must be >= 0"),
    (dict(slices=1, tiles=1, M=16, K=8192, g=4096), b"LDS"),   # 256 steps of 1 KB fragments
    (dict(slices=1, tiles=4, kw=2, M=16, K=5120), b"LDS"),                 # 160 steps of 1 KB fragments
    (dict(topk=9), b"k=9"),
    (dict(topk=-1), b"k=-1"),
    (dict(bits=7), b"affine_bits=7"),
    (dict(bits=9), b"affine_bits=9"),
    (dict(bits=2, cols=128), b"64-column"),
    (dict(bits=3, ring=2), b"ring"),
    (dict(bits=2, ring=3), b"ring"),
    (dict(bits=5, ring=8), b"ring"),
])
def test_decode_launch_is_checked(lib, kw, msg):
    assert dec(lib, **kw) == -1
    assert msg in lib.w4a16_last_error(), lib.w4a16_last_error()


def test_default_plans_are_accepted(lib):
    """The default launch of every workload shape and row count is one the kernel takes."""
    out = (ctypes.c_int * 7)()
    for K, N, g, packed in ((512, 256, 128, 0), (5120, 5120, 128, 0), (5120, 17408, 128, 0), (17408, 5120, 64, 1),
                            (5120, 248320, 128, 0)):
        for M in range(1, 17):
            for topk in (0, 1, 8):
                assert lib.w4a16_decode_plan(M, N, K, g, packed, 0, 0, 0, 0, 0, topk, 0, out) == 0, \
                    (K, N, M, topk, lib.w4a16_last_error())
                assert out[5] <= 160 * 1024 - 256


def test_fused_pick_reserves_lds_for_the_outputs(lib):
    """A fused pick stages the group's finished outputs, M x (tiles x tile_cols) fp32, over the
    activation fragments: a slice too short to hold them gets the room anyway."""
    out = (ctypes.c_int * 7)()
    assert lib.w4a16_decode_plan(1, 256, 64, 32, 0, 1, 4, 1, 64, 2, 0, 0, out) == 0
    plain = out[5]
    assert lib.w4a16_decode_plan(1, 256, 64, 32, 0, 1, 4, 1, 64, 2, 1, 0, out) == 0
    assert out[5] - plain == 1 * 256 * 4 - 2 * 64   # two steps of one-row fragments -> one row of 256 outputs



def test_topk_checks_its_arguments(lib):
    A = O = 4096
    assert lib.w4a16_gemm_topk(A, A, A, None, 128, 2, 256, 512, O, 0, 4, None, None) == -1
    assert b"idx" in lib.w4a16_last_error()
    for k in (0, 9, -3):
        assert lib.w4a16_gemm_topk(A, A, A, None, 128, 2, 256, 512, O, 0, k, O, None) == -1
        assert b"k=" in lib.w4a16_last_error()
    assert lib.w4a16_gemm_topk(A, A, A, None, 128, 17, 256, 512, O, 0, 2, O, None) == -1   # M
    assert lib.w4a16_gemm_decode_ex(A, A, A, None, 128, 2, 256, 512, O, 0, 0, 0, 0, 0, 0, 2, None, None) == -1
    assert lib.w4a16_gemm_decode_ex(A, A, A, None, 128, 2, 256, 512, O, 0, 0, 0, 0, 0, 0, 0, O, None) == -1


def test_affine_bits_plans(lib):
    """Affine codes read at their own width: every width the kernel takes, at the affine
    workloads' shapes and every row count, has a default launch that fits; its scales and biases
    both sit in LDS (more than the GPTQ launch of the same shape)."""
    out = (ctypes.c_int * 7)()
    for K, N, g in ((5120, 17408, 64), (512, 256, 64), (1024, 520, 32), (5120, 248320, 64)):
        for bits in (1, 2, 3, 4, 5, 6, 8):
            for M in (1, 2, 5, 9, 16):
                assert lib.w4a16_decode_plan(M, N, K, g, 0, 0, 0, 0, 0, 0, 0, bits, out) == 0, \
                    (K, N, bits, M, lib.w4a16_last_error())
                assert out[3] == 64 and out[4] == 4 and out[5] <= 160 * 1024 - 256
    assert lib.w4a16_decode_plan(4, 256, 512, 64, 1, 0, 0, 0, 0, 0, 0, 2, out) == -1   # no zero points


def test_affine_bits_checks_its_arguments(lib):
    A = O = 4096
    f = lib.w4a16_gemm_affine_bits
    assert f(A, A, 2, A, None, 64, 2, 256, 512, O, 0, None) == -1
    assert b"biases" in lib.w4a16_last_error()
    for bits in (0, 7, 9, -1):
        assert f(A, A, bits, A, A, 64, 2, 256, 512, O, 0, None) == -1
        assert b"bits=" in lib.w4a16_last_error()
    assert f(A, A, 2, A, A + 8, 64, 2, 256, 512, O, 0, None) == -2   # biases not 16-byte aligned
    assert f(A, A, 2, A, A, 48, 2, 256, 512, O, 0, None) == -1       # group size
    assert f(A, A, 2, A, A, 64, 17, 256, 512, O, 0, None) == -1      # M
    assert lib.w4a16_gemm_affine_bits_ex(A, A, 3, A, A, 64, 2, 256, 512, O, 0, 0, 0, 0, 3, None) == -1
    assert b"ring" in lib.w4a16_last_error()


def test_affine_bits_prefill_checks_its_arguments(lib):
    """The affine prompt GEMM refuses what w4a16_gemm_affine_bits refuses, with M up to
    W4A16_PREFILL_MAX_M, before any device work."""
    A = O = 4096
    f = lib.w4a16_gemm_affine_bits_prefill
    assert f(A, A, 2, A, None, 64, 300, 256, 512, O, 0, None) == -1
    assert b"biases" in lib.w4a16_last_error()
    for bits in (0, 7, 9, -1):
        assert f(A, A, bits, A, A, 64, 300, 256, 512, O, 0, None) == -1
        assert b"bits=" in lib.w4a16_last_error()
    assert f(A, A, 2, A, A + 8, 64, 300, 256, 512, O, 0, None) == -2   # biases not 16-byte aligned
    assert f(A, A, 2, A, A, 48, 300, 256, 512, O, 0, None) == -1       # group size
    assert f(A, A, 2, A, A, 64, 0, 256, 512, O, 0, None) == -1         # M
    assert f(A, A, 2, A, A, 64, 65537, 256, 512, O, 0, None) == -1
    assert b"M=65537" in lib.w4a16_last_error()
    assert f(A, A, 8, A, A, 64, 300, 260, 512, O, 0, None) == -1       # N % 8
    assert f(A, A, 8, A, A, 64, 300, 256, 512, O, 2, None) == -1       # out_dtype


def test_affine_word_per_lane_blocks(lib):
    """1- and 2-bit codes read a word per lane over blocks of 4 and 2 steps when the quantisation
    groups hold whole blocks; otherwise (and for every other width) one step per ring slot. A
    block is never split: slices and K pieces are whole blocks."""
    import verify_matmul_amd as vm
    for bits, g, sub in ((2, 64, 2), (2, 128, 2), (2, 32, 1), (1, 128, 4), (1, 256, 4), (1, 64, 1), (1, 32, 1),
                         (3, 128, 1), (4, 128, 1), (8, 64, 1)):
        assert vm.w4a16_decode_plan(4, 512, 1024, g, affine_bits=bits)["sub"] == sub, (bits, g)
    assert vm.w4a16_decode_plan(4, 512, 1024, 128, packed_zeros=True)["sub"] == 1   # GPTQ codes
    # K = 512: 16 steps = 8 blocks of 2-bit codes or 4 of 1-bit codes
    assert vm.w4a16_decode_plan(4, 512, 512, 64, slices=8, affine_bits=2)["slices"] == 8
    with pytest.raises(vm.W4A16Error):
        vm.w4a16_decode_plan(4, 512, 512, 64, slices=9, affine_bits=2)
    with pytest.raises(vm.W4A16Error):
        vm.w4a16_decode_plan(4, 512, 512, 128, slices=5, affine_bits=1)
    with pytest.raises(vm.W4A16Error):
        vm.w4a16_decode_plan(4, 512, 512, 128, slices=2, kw=4, affine_bits=1)
