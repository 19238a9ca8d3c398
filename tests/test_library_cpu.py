"""The HIP library builds, loads, exports every declared symbol, and rejects bad arguments on
the host before touching a device (no GPU needed)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")


@pytest.fixture(scope="module")
def lib():
    import verify_matmul_amd as vm
    if not os.path.exists(vm.lib_path):
        from verify_matmul_amd import _build
        _build.build()
    return vm.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a16_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_api():
    names = declared_functions()
    for n in ("w4a16_gemm", "w4a16_argmax_rows", "w4a16_unpack_u8", "w4a16_dequant_f32", "w4a16_gemm_gate_up"):
        assert n in names


def test_exports_every_declared_symbol(lib):
    import verify_matmul_amd as vm
    names = declared_functions()
    assert sorted(vm.EXPORTS) == names
    out = subprocess.run(["nm", "-D", "--defined-only", vm.lib_path], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(w4a16_\w+)$", out, flags=re.M))
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


A = 0x10000   # fake, 16-byte-aligned device addresses: the checks below fail before any use
Q = 0x20000
S = 0x30000
Z = 0x40000
O = 0x50000


def gemm(lib, a=A, q=Q, s=S, z=None, g=128, M=1, N=256, K=512, o=O, dt=0):
    return lib.w4a16_gemm(a, q, s, z, g, M, N, K, o, dt, None)


@pytest.mark.parametrize("kw,status", [
    (dict(a=None), -1), (dict(q=None), -1), (dict(s=None), -1), (dict(o=None), -1),
    (dict(M=0), -1), (dict(M=17), -1), (dict(N=0), -1), (dict(K=0), -1), (dict(g=0), -1),
    (dict(N=-8), -1), (dict(g=48), -1), (dict(g=96), -1), (dict(K=520, g=32), -1),
    (dict(N=260), -1), (dict(a=A + 2), -2), (dict(q=Q + 4), -2), (dict(s=S + 8), -2),
    (dict(z=Z + 4), -2), (dict(o=O + 8), -2), (dict(dt=2), -1), (dict(dt=-1), -1),
    (dict(N=1 << 20, K=1 << 22), -2),   # qweight of 2^39 words: beyond the 32-bit word offsets
])
def test_gemm_rejects_bad_arguments(lib, kw, status):
    assert gemm(lib, **kw) == status
    assert lib.w4a16_last_error().decode()


def test_validation_order_is_fixed(lib):
    # null pointer is reported before a bad M, bad M before a bad group, group before alignment
    assert gemm(lib, a=None, M=0) == -1 and b"null" in lib.w4a16_last_error()
    assert gemm(lib, M=0, g=48) == -1 and b"M=0" in lib.w4a16_last_error()
    assert gemm(lib, g=48, a=A + 2) == -1 and b"multiple of 32" in lib.w4a16_last_error()


def ex(lib, splits, wk, K=512, cols=0):
    return lib.w4a16_gemm_ex(A, Q, S, None, 128, 1, 256, K, O, 0, splits, wk, cols, None)


def test_explicit_launch_is_checked(lib):
    # K=512 has 16 steps of 32: splits * waves_k may not exceed 16; waves_k in {1,2,4,8,16}
    assert ex(lib, 17, 1) == -1
    assert ex(lib, 4, 8) == -1
    assert ex(lib, -1, 0) == -1
    assert ex(lib, 0, -1) == -1
    assert ex(lib, 1, 3) == -1
    assert ex(lib, 1, 32) == -1
    assert ex(lib, 1, 1, cols=96) == -1 and b"tile_cols" in lib.w4a16_last_error()
    assert ex(lib, 1, 1, cols=-64) == -1


def test_plan_host_only(lib):
    import ctypes
    k, s, w, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    # (M, N, K, g, whether the decode kernel takes it): the widest matrices at every row count; from
    # 16384 columns 9-16 rows when its launch of 4 tiles x 2 K pieces runs in one round (FFN 5120 x
    # 17408: 3 slices, 204 workgroups; 8192 x 28672 has none and stays on the small-row kernel)
    for M, N, K, g, dec in ((1, 17408, 5120, 128, False), (8, 17408, 5120, 128, False), (9, 17408, 5120, 128, True),
                            (16, 17408, 5120, 128, True), (5, 248320, 5120, 128, True), (1, 248320, 5120, 128, True),
                            (16, 248320, 5120, 128, True), (9, 65536, 4096, 64, True), (1, 65528, 4096, 64, False),
                            (16, 32768, 5120, 128, True), (16, 28672, 8192, 128, False), (1, 5120, 5120, 128, False),
                            (16, 5120, 17408, 64, False), (16, 5120, 5120, 128, False), (1, 256, 512, 128, False),
                            (16, 8, 64, 32, False)):
        assert lib.w4a16_plan(M, N, K, g, ctypes.byref(k), ctypes.byref(s), ctypes.byref(w), ctypes.byref(c)) == 0
        assert (k.value >= 2) == dec, (M, N, K)
        if k.value >= 2:
            assert k.value == (2 if M == 1 else 3) and 1 <= s.value <= 16
            assert w.value == (2 if 8 < M and N < 65536 else 1)
            if N < 65536:   # one round of at least 192 workgroups of 4 x 64 columns
                assert s.value * -(-N // 256) >= 192 and c.value == 64
        else:
            assert k.value == (0 if M == 1 and c.value == 64 else 1)   # one row on 128 columns: matrix cores
            assert s.value >= 1 and w.value in (1, 2, 4, 8, 16) and s.value * w.value <= K // 32
        assert c.value in (64, 128)
    assert lib.w4a16_plan(0, 256, 512, 128, None, None, None, None) == -1
    assert lib.w4a16_plan(1, 256, 512, 48, None, None, None, None) == -1


def test_plan_balances_narrow_matrices(lib):
    """At most 256 column tiles (one per compute unit): the default launch takes the workgroups
    per tile s that minimise ceil(tiles * s / 256) / s (the busiest CU's share of the work), the
    fewest on a tie, with at most two workgroups per CU; 16 waves per workgroup, or 8 for up to 8
    rows when the pieces would be shorter than 8 steps."""
    import ctypes
    k, s, w, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int()

    def plan(M, N, K, g):
        assert lib.w4a16_plan(M, N, K, g, ctypes.byref(k), ctypes.byref(s), ctypes.byref(w), ctypes.byref(c)) == 0
        return k.value, s.value, w.value, c.value

    # (M, N, K, g) -> (splits, waves_k): attention and FFN down (80 tiles), 5120 x 4096 (64 tiles),
    # 5120 x 8192 (128), 5120 x 13824 (216: whole K in a workgroup), 3072 x 2048 (32)
    for M, N, K, g, want in ((1, 5120, 5120, 128, (3, 8)), (8, 5120, 5120, 128, (3, 8)),
                             (16, 5120, 5120, 128, (3, 16)), (1, 5120, 17408, 64, (3, 16)),
                             (16, 5120, 17408, 64, (3, 16)), (1, 4096, 5120, 128, (4, 8)),
                             (16, 4096, 5120, 128, (4, 16)), (4, 8192, 5120, 128, (2, 8)),
                             (16, 8192, 5120, 128, (2, 16)), (1, 13824, 5120, 128, (1, 16)),
                             (16, 13824, 5120, 128, (1, 16)), (1, 2048, 3072, 64, (8, 8))):
        kern, splits, wk, cols = plan(M, N, K, g)
        assert kern == (0 if M == 1 else 1) and cols == 64, (M, N, K)
        assert (splits, wk) == want, (M, N, K, (splits, wk))
        tiles = -(-N // 64)
        cost = lambda x: -(-tiles * x // 256) / x
        assert all(cost(splits) <= cost(x) for x in range(1, min(16, 512 // tiles) + 1)), (M, N, K)
    # more than 256 tiles keep the wave-count rule (FFN up 5120 x 17408: 4 workgroups of 4 waves)
    assert plan(1, 17408, 5120, 128)[1:3] == (4, 4)


def test_fused_pick_checks_its_arguments(lib):
    assert lib.w4a16_gemm_argmax(A, Q, S, None, 128, 1, 256, 512, O, 0, None, None) == -1
    assert b"idx" in lib.w4a16_last_error()
    assert lib.w4a16_gemm_argmax(A, Q, S, None, 128, 17, 256, 512, O, 0, O, None) == -1
    assert lib.w4a16_gemm_argmax(A, Q, S, None, 48, 1, 256, 512, O, 0, O, None) == -1


def test_aux_entry_points_reject_bad_arguments(lib):
    assert lib.w4a16_argmax_rows(None, 1, 10, O, None) == -1
    assert lib.w4a16_argmax_rows(A, 0, 10, O, None) == -1
    assert lib.w4a16_argmax_rows(A, 1, 0, O, None) == -1
    assert lib.w4a16_argmax_rows(A + 4, 1, 10, O, None) == -2
    assert lib.w4a16_stream_read(None, 64, O, None) == -1
    assert lib.w4a16_stream_read(A, 64, None, None) == -1
    assert lib.w4a16_stream_read(A, 0, O, None) == -1
    assert lib.w4a16_stream_read(A, 40, O, None) == -1
    assert lib.w4a16_stream_read(A + 4, 64, O, None) == -2
    assert lib.w4a16_unpack_u8(Q, 12, 8, O, None) == -1
    assert lib.w4a16_unpack_u8(Q, 16, 6, O, None) == -1
    assert lib.w4a16_dequant_f32(Q, S, None, 64, 96, 8, O, None) == -1
    assert lib.w4a16_dequant_f32(Q, S, None, 32, 64, 12, O, None) == -1


def test_status_strings(lib):
    for st in (0, -1, -2, -3, -4, 7):
        assert lib.w4a16_status_string(st)
    assert lib.w4a16_version() >= 100


def test_bench_refuses_more_than_one_gpu():
    # the refusal comes before any GPU or torch import, so it runs on the CPU
    import subprocess
    import sys
    from pathlib import Path
    root = Path(__file__).resolve().parents[1]
    r = subprocess.run([sys.executable, str(root / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=60)
    assert r.returncode == 2
    assert "--gpus 2 is not supported" in r.stderr
    assert r.stdout == ""


Q2, S2, Z2 = 0x60000, 0x70000, 0x80000


def gate_up(lib, q=Q, s=S, z=None, q2=Q2, s2=S2, z2=None, g=128, M=1, N=256, K=512, o=O, dt=0, splits=0, wk=0):
    return lib.w4a16_gemm_gate_up_ex(A, q, s, z, q2, s2, z2, g, M, N, K, o, dt, splits, wk, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(s2=None), -1), (dict(q2=None), -1),
    (dict(z=Z), -1), (dict(z2=Z2), -1),                 # zeros given for one matrix only
    (dict(q2=Q2 + 4), -2), (dict(z=Z, z2=Z2 + 4), -2), (dict(M=17), -1), (dict(N=260), -1),
    (dict(splits=17, wk=1), -1),                        # 17 x 1 > 512/32 steps
    (dict(wk=3, splits=1), -1),
])
def test_gate_up_rejects_bad_arguments(lib, kw, status):
    assert gate_up(lib, **kw) == status
    assert lib.w4a16_last_error().decode()
    assert lib.w4a16_gemm_gate_up(A, Q, S, None, None, S2, None, 128, 1, 256, 512, O, 0, None) == -1


def test_prefill_rejects_bad_arguments(lib):
    def pre(a=A, q=Q, s=S, z=None, g=128, M=300, N=256, K=512, o=O, dt=0):
        return lib.w4a16_gemm_prefill(a, q, s, z, g, M, N, K, o, dt, None)
    assert pre(M=0) == -1 and pre(M=65537) == -1 and pre(N=260) == -1 and pre(g=48) == -1
    assert pre(q=None) == -1 and pre(a=A + 2) == -2 and pre(dt=3) == -1
    assert pre(M=65537) == -1 and b"M=65537" in lib.w4a16_last_error()


def test_gate_up_prefill_rejects_bad_arguments(lib):
    def pre(q2=Q2, z=None, z2=None, M=300, N=256):
        return lib.w4a16_gemm_gate_up_prefill(A, Q, S, z, q2, S2, z2, 128, M, N, 512, O, 0, None)
    assert pre(q2=None) == -1 and pre(z=Z) == -1 and pre(z2=Z2) == -1
    assert pre(M=65537) == -1 and pre(N=260) == -1 and pre(q2=Q2 + 4) == -2


B = 0x60000   # fake bias address


def test_affine_rejects_bad_arguments(lib):
    def aff(a=A, q=Q, s=S, b=B, g=64, M=1, N=256, K=512, o=O, dt=0):
        return lib.w4a16_gemm_affine(a, q, s, b, g, M, N, K, o, dt, None)
    assert aff(b=None) == -1 and b"biases" in lib.w4a16_last_error()
    assert aff(q=None) == -1 and aff(M=17) == -1 and aff(g=48) == -1 and aff(N=260) == -1
    assert aff(b=B + 2) == -2 and aff(s=S + 4) == -2 and aff(dt=2) == -1
    ex = lambda **kw: lib.w4a16_gemm_affine_ex(A, Q, S, B, 64, 1, 256, 512, O, 0, kw.get("sp", 0),
                                               kw.get("wk", 0), kw.get("tc", 0), None)
    assert ex(wk=3) == -1 and ex(tc=96) == -1 and ex(sp=17, wk=1) == -1


def test_affine_widen_rejects_bad_arguments(lib):
    def widen(p=Q, bits=3, K=512, N=256, o=O):
        return lib.w4a16_affine_widen(p, bits, K, N, o, None)
    assert widen(bits=0) == -1 and widen(bits=5) == -1 and b"bits=5" in lib.w4a16_last_error()
    assert widen(p=None) == -1 and widen(o=None) == -1 and widen(K=520) == -1 and widen(N=260) == -1
    assert widen(p=Q + 4) == -2 and widen(o=O + 8) == -2


def test_affine_split_rejects_bad_arguments(lib):
    def split(p=Q, bits=8, s=S, b=B, g=64, K=512, N=256, qo=O, so=Z, bo=A):
        return lib.w4a16_affine_split(p, bits, s, b, g, K, N, qo, so, bo, None)
    assert split(bits=4) == -1 and split(bits=9) == -1 and b"bits=9" in lib.w4a16_last_error()
    assert split(p=None) == -1 and split(so=None) == -1 and split(g=48) == -1 and split(K=544) == -1
    assert split(N=260) == -1 and split(qo=O + 4) == -2 and split(b=B + 2) == -2

    def gemm_split(K=512, g=64, M=1, b=B):
        return lib.w4a16_gemm_affine_split(A, Q, S, b, g, M, 256, K, O, 0, None)
    assert gemm_split(b=None) == -1 and gemm_split(K=96) == -1 and gemm_split(M=17) == -1
    assert gemm_split(K=96, g=64) == -1 and b"group_size" in lib.w4a16_last_error()


def test_load_refuses_a_library_built_from_other_sources(monkeypatch):
    """The binding compares the hash embedded at build time with the hash of the sources beside it."""
    import verify_matmul_amd as vm
    from verify_matmul_amd import _build
    assert vm.load().w4a16_source_hash().decode() == _build.source_hash()
    monkeypatch.setattr(vm, "_lib", None)
    monkeypatch.setattr(_build, "source_hash", lambda: "0" * 16)
    with pytest.raises(ImportError, match="other sources"):
        vm.load()
