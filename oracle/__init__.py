"""CPU oracle for the W4A16 matmul (int4 GPTQ-packed weights x bf16 activations).

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT: only ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package. The HIP library never
imports, links or calls it, and it shares no code with the HIP library.

The arithmetic lives in ``w4a16_oracle.c`` (plain C, fp32 exact dequantisation, fp64
accumulation; the affine form w = s * q + b of MLX checkpoints in fp64); this module only
builds that file with gcc and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "w4a16_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libw4a16_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP over output columns)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC",
                               "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.w4o_fp16_to_f32.argtypes = [ctypes.c_uint16]
        lib.w4o_fp16_to_f32.restype = ctypes.c_float
        lib.w4o_bf16_to_f32.argtypes = [ctypes.c_uint16]
        lib.w4o_bf16_to_f32.restype = ctypes.c_float
        lib.w4o_unpack_qweight.argtypes = [P, I64, I64, P]
        lib.w4o_unpack_qzeros.argtypes = [P, I64, I64, P]
        lib.w4o_dequant.argtypes = [P, P, P, I64, I64, I64, P]
        lib.w4o_gemm.argtypes = [P, P, P, P, I64, I64, I64, I64, P, I64, P, P]
        lib.w4o_argmax_rows_f32.argtypes = [P, I64, I64, P]
        lib.w4o_topk_rows_f32.argtypes = [P, I64, I64, I64, P]
        lib.w4o_silu.argtypes = [ctypes.c_double]
        lib.w4o_silu.restype = ctypes.c_double
        lib.w4o_silu_mul.argtypes = [P, P, I64, P]
        lib.w4o_affine_unpack.argtypes = [P, ctypes.c_int, I64, I64, P]
        lib.w4o_affine_gemm.argtypes = [P, P, ctypes.c_int, P, P, I64, I64, I64, I64, P, I64, P, P]
        for f in (lib.w4o_unpack_qweight, lib.w4o_unpack_qzeros, lib.w4o_dequant,
                  lib.w4o_gemm, lib.w4o_argmax_rows_f32, lib.w4o_topk_rows_f32, lib.w4o_silu_mul,
                  lib.w4o_affine_unpack, lib.w4o_affine_gemm):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (status {rc})")


def fp16_to_f32(bits: int) -> float:
    return _load().w4o_fp16_to_f32(int(bits))


def bf16_to_f32(bits: int) -> float:
    return _load().w4o_bf16_to_f32(int(bits))


def unpack_qweight(qweight: np.ndarray) -> np.ndarray:
    """Codes [K, N] (uint8) from qweight [K/8, N]."""
    qw = _c(qweight, np.uint32)
    K, N = qw.shape[0] * 8, qw.shape[1]
    q = np.empty((K, N), dtype=np.uint8)
    _check(_load().w4o_unpack_qweight(_ptr(qw), K, N, _ptr(q)), "unpack_qweight")
    return q


def unpack_qzeros(qzeros: Optional[np.ndarray], groups: int, N: int) -> np.ndarray:
    """Zeros [G, N] (uint8) from qzeros [G, N/8]; all 8 when qzeros is None."""
    qz = _c(qzeros, np.uint32)
    if qz is not None:
        assert qz.shape == (groups, N // 8)
    z = np.empty((groups, N), dtype=np.uint8)
    _check(_load().w4o_unpack_qzeros(_ptr(qz), groups, N, _ptr(z)), "unpack_qzeros")
    return z


def dequant(qweight, scales, qzeros, group: int) -> np.ndarray:
    """Dequantised weights [K, N] in fp32."""
    qw = _c(qweight, np.uint32)
    sc = _c(scales, np.uint16)
    qz = _c(qzeros, np.uint32)
    K, N = qw.shape[0] * 8, qw.shape[1]
    w = np.empty((K, N), dtype=np.float32)
    _check(_load().w4o_dequant(_ptr(qw), _ptr(sc), _ptr(qz), group, K, N, _ptr(w)), "dequant")
    return w


def gemm(act, qweight, scales, qzeros, group: int, cols: Optional[Sequence[int]] = None,
         with_bound: bool = True):
    """y (fp64 [M, C]) and bound (fp64 [M, C]) for columns ``cols`` (all when None).

    ``act`` is bf16 bits [M, K] (uint16)."""
    a = _c(act, np.uint16)
    qw = _c(qweight, np.uint32)
    sc = _c(scales, np.uint16)
    qz = _c(qzeros, np.uint32)
    M, K = a.shape
    N = qw.shape[1]
    assert qw.shape[0] * 8 == K
    cc = None if cols is None else np.ascontiguousarray(cols, dtype=np.int64)
    C = N if cc is None else cc.shape[0]
    y = np.empty((M, C), dtype=np.float64)
    b = np.empty((M, C), dtype=np.float64) if with_bound else None
    _check(_load().w4o_gemm(_ptr(a), _ptr(qw), _ptr(sc), _ptr(qz), group, M, N, K,
                            _ptr(cc), C, _ptr(y), _ptr(b)), "gemm")
    return (y, b) if with_bound else y


def argmax_rows_f32(v: np.ndarray) -> np.ndarray:
    """Per-row argmax (ties -> lowest index) of fp32 values [M, N]."""
    x = _c(v, np.float32)
    M, N = x.shape
    idx = np.empty(M, dtype=np.int64)
    _check(_load().w4o_argmax_rows_f32(_ptr(x), M, N, _ptr(idx)), "argmax")
    return idx



def topk_rows_f32(v: np.ndarray, k: int) -> np.ndarray:
    """Per-row k best columns of fp32 values [M, N], best first (ties -> lowest index, NaN never
    chosen, -1 once a row has nothing left): [M, k] int64."""
    x = _c(v, np.float32)
    M, N = x.shape
    idx = np.empty((M, k), dtype=np.int64)
    _check(_load().w4o_topk_rows_f32(_ptr(x), M, N, int(k), _ptr(idx)), "topk")
    return idx


def silu(x: float) -> float:
    """x / (1 + e^-x) in fp64."""
    return _load().w4o_silu(float(x))


def silu_mul(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """silu(g) * u elementwise, fp64 (same shapes)."""
    gg = _c(g, np.float64)
    uu = _c(u, np.float64)
    assert gg.shape == uu.shape
    h = np.empty(gg.shape, dtype=np.float64)
    _check(_load().w4o_silu_mul(_ptr(gg), _ptr(uu), gg.size, _ptr(h)), "silu_mul")
    return h


def gate_up(act, gate, up, group: int, cols: Optional[Sequence[int]] = None):
    """Gated feed-forward input silu(A x W_gate) * (A x W_up) for columns ``cols`` (all when None).

    ``gate`` and ``up`` are (qweight, scales, qzeros) triples of the same shape. Returns h, and
    the two products with their bounds: (h, y_gate, bound_gate, y_up, bound_up), all fp64."""
    yg, bg = gemm(act, gate[0], gate[1], gate[2], group, cols)
    yu, bu = gemm(act, up[0], up[1], up[2], group, cols)
    return silu_mul(yg, yu), yg, bg, yu, bu


def affine_unpack(packed: np.ndarray, bits: int, K: int) -> np.ndarray:
    """Codes [K, N] (uint8) of ``bits`` bits each from the column bit streams [K*bits/32, N]."""
    pk = _c(packed, np.uint32)
    N = pk.shape[1]
    assert pk.shape[0] * 32 == K * bits
    q = np.empty((K, N), dtype=np.uint8)
    _check(_load().w4o_affine_unpack(_ptr(pk), bits, K, N, _ptr(q)), "affine_unpack")
    return q


def affine_gemm(act, packed, bits: int, scales, biases, group: int,
                cols: Optional[Sequence[int]] = None):
    """y and bound (fp64 [M, C]) of A x W with W = s * q + b, codes of ``bits`` bits.

    ``act``, ``scales`` and ``biases`` are bf16 bits (uint16); the bound is
    sum |a| * (|s * q| + |b|)."""
    a = _c(act, np.uint16)
    pk = _c(packed, np.uint32)
    sc = _c(scales, np.uint16)
    bi = _c(biases, np.uint16)
    M, K = a.shape
    N = pk.shape[1]
    assert pk.shape[0] * 32 == K * bits and sc.shape == bi.shape == (K // group, N)
    cc = None if cols is None else np.ascontiguousarray(cols, dtype=np.int64)
    C = N if cc is None else cc.shape[0]
    y = np.empty((M, C), dtype=np.float64)
    b = np.empty((M, C), dtype=np.float64)
    _check(_load().w4o_affine_gemm(_ptr(a), _ptr(pk), bits, _ptr(sc), _ptr(bi), group, M, N, K,
                                   _ptr(cc), C, _ptr(y), _ptr(b)), "affine_gemm")
    return y, b


def affine_gate_up(act, gate, up, group: int, cols: Optional[Sequence[int]] = None):
    """silu(A x W_gate) * (A x W_up) for affine matrices; gate and up are (packed, bits, scales,
    biases). Returns (h, y_gate, bound_gate, y_up, bound_up), all fp64."""
    yg, bg = affine_gemm(act, gate[0], gate[1], gate[2], gate[3], group, cols)
    yu, bu = affine_gemm(act, up[0], up[1], up[2], up[3], group, cols)
    return silu_mul(yg, yu), yg, bg, yu, bu
