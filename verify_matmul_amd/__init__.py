"""Python binding of libw4a16.so: group-quantised int4 x bf16 matmul on AMD MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP library. PyTorch
provides the device buffers and the stream; tensors are passed by pointer to the C ABI in
``include/w4a16.h``. There is no CPU fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "W4A16Error", "lib_path", "load", "w4a16_gemm", "w4a16_gemm_noalloc", "w4a16_gemm_ex", "w4a16_gemm_decode_ex",
    "w4a16_decode_plan", "w4a16_gemm_argmax", "w4a16_gemm_topk",
    "w4a16_gemm_gate_up", "w4a16_gemm_prefill", "w4a16_gemm_gate_up_prefill", "w4a16_plan",
    "w4a16_argmax_rows", "w4a16_unpack_u8", "w4a16_dequant_f32", "w4a16_release_scratch",
    "w4a16_gemm_affine", "w4a16_affine_widen", "w4a16_affine_split", "w4a16_gemm_affine_split",
    "w4a16_gemm_affine_bits", "w4a16_gemm_affine_bits_prefill",
    "w4a16_gemm_affine_gate_up", "w4a16_stream_read", "EXPORTS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libw4a16.so")
_lib = None

# every symbol the header declares
EXPORTS = (
    "w4a16_gemm", "w4a16_gemm_noalloc", "w4a16_gemm_ex", "w4a16_gemm_decode_ex", "w4a16_decode_plan", "w4a16_gemm_argmax", "w4a16_gemm_topk", "w4a16_gemm_prefill",
    "w4a16_gemm_gate_up", "w4a16_gemm_gate_up_ex", "w4a16_gemm_gate_up_prefill", "w4a16_gemm_affine", "w4a16_gemm_affine_ex",
    "w4a16_affine_widen", "w4a16_affine_split", "w4a16_gemm_affine_split", "w4a16_gemm_affine_bits",
    "w4a16_gemm_affine_bits_ex", "w4a16_gemm_affine_bits_prefill", "w4a16_gemm_affine_gate_up", "w4a16_plan", "w4a16_argmax_rows", "w4a16_unpack_u8", "w4a16_dequant_f32", "w4a16_stream_read", "w4a16_release_scratch", "w4a16_status_string",
    "w4a16_last_error", "w4a16_version", "w4a16_source_hash",
)

OUT_F32 = 0
OUT_BF16 = 1


class W4A16Error(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status}: {detail}")
        self.status = status


def load():
    """Load libw4a16.so (built in-tree by ``__graft_entry__.build()``); raise if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise ImportError(f"{lib_path} is missing: build it with __graft_entry__.build() "
                          f"(hipcc --offload-arch=gfx950); there is no fallback implementation")
    lib = ctypes.CDLL(lib_path)
    from . import _build
    lib.w4a16_source_hash.argtypes = []
    lib.w4a16_source_hash.restype = ctypes.c_char_p
    built, want = lib.w4a16_source_hash().decode(), _build.source_hash()
    if built != want:
        raise ImportError(f"{lib_path} was built from other sources (hash {built}, these sources {want}): "
                          f"rebuild it with __graft_entry__.build()")
    P, I = ctypes.c_void_p, ctypes.c_int
    lib.w4a16_gemm.argtypes = [P, P, P, P, I, I, I, I, P, I, P]
    lib.w4a16_gemm_noalloc.argtypes = [P, P, P, P, I, I, I, I, P, I, P]
    lib.w4a16_gemm_decode_ex.argtypes = [P, P, P, P, I, I, I, I, P, I, I, I, I, I, I, I, P, P]
    lib.w4a16_decode_plan.argtypes = [I, I, I, I, I, I, I, I, I, I, I, I, P]
    lib.w4a16_gemm_affine_bits.argtypes = [P, P, I, P, P, I, I, I, I, P, I, P]
    lib.w4a16_gemm_affine_bits_ex.argtypes = [P, P, I, P, P, I, I, I, I, P, I, I, I, I, I, P]
    lib.w4a16_gemm_affine_bits_prefill.argtypes = [P, P, I, P, P, I, I, I, I, P, I, P]
    lib.w4a16_gemm_topk.argtypes = [P, P, P, P, I, I, I, I, P, I, I, P, P]
    lib.w4a16_gemm_ex.argtypes = [P, P, P, P, I, I, I, I, P, I, I, I, I, P]
    lib.w4a16_gemm_argmax.argtypes = [P, P, P, P, I, I, I, I, P, I, P, P]
    lib.w4a16_gemm_prefill.argtypes = [P, P, P, P, I, I, I, I, P, I, P]
    lib.w4a16_gemm_gate_up.argtypes = [P, P, P, P, P, P, P, I, I, I, I, P, I, P]
    lib.w4a16_gemm_gate_up_prefill.argtypes = [P, P, P, P, P, P, P, I, I, I, I, P, I, P]
    lib.w4a16_gemm_gate_up_ex.argtypes = [P, P, P, P, P, P, P, I, I, I, I, P, I, I, I, P]
    lib.w4a16_gemm_affine.argtypes = [P, P, P, P, I, I, I, I, P, I, P]
    lib.w4a16_gemm_affine_ex.argtypes = [P, P, P, P, I, I, I, I, P, I, I, I, I, P]
    lib.w4a16_affine_widen.argtypes = [P, I, I, I, P, P]
    lib.w4a16_affine_split.argtypes = [P, I, P, P, I, I, I, P, P, P, P]
    lib.w4a16_gemm_affine_split.argtypes = [P, P, P, P, I, I, I, I, P, I, P]
    lib.w4a16_gemm_affine_gate_up.argtypes = [P, P, P, P, P, P, P, I, I, I, I, P, I, P]
    lib.w4a16_plan.argtypes = [I, I, I, I, P, P, P, P]
    lib.w4a16_argmax_rows.argtypes = [P, I, I, P, P]
    lib.w4a16_unpack_u8.argtypes = [P, I, I, P, P]
    lib.w4a16_dequant_f32.argtypes = [P, P, P, I, I, I, P, P]
    lib.w4a16_stream_read.argtypes = [P, ctypes.c_size_t, P, P]
    lib.w4a16_release_scratch.argtypes = []
    lib.w4a16_status_string.argtypes = [I]
    lib.w4a16_status_string.restype = ctypes.c_char_p
    lib.w4a16_last_error.argtypes = []
    lib.w4a16_last_error.restype = ctypes.c_char_p
    lib.w4a16_version.argtypes = []
    for f in ("w4a16_gemm", "w4a16_gemm_noalloc", "w4a16_gemm_ex", "w4a16_gemm_decode_ex", "w4a16_decode_plan", "w4a16_gemm_argmax", "w4a16_gemm_topk", "w4a16_gemm_affine_bits", "w4a16_gemm_affine_bits_ex", "w4a16_gemm_affine_bits_prefill", "w4a16_gemm_prefill", "w4a16_gemm_gate_up",
              "w4a16_gemm_gate_up_ex", "w4a16_gemm_gate_up_prefill",
              "w4a16_plan", "w4a16_argmax_rows",
              "w4a16_unpack_u8", "w4a16_dequant_f32", "w4a16_stream_read", "w4a16_release_scratch",
              "w4a16_version"):
        getattr(lib, f).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(rc: int, where: str):
    if rc < 0:
        lib = load()
        raise W4A16Error(rc, where, f"{lib.w4a16_status_string(rc).decode()}: "
                                    f"{lib.w4a16_last_error().decode()}")
    return rc


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: Optional[torch.Tensor], name: str, dtypes) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


_I32 = (torch.int32, torch.uint32)
_I16 = (torch.float16, torch.int16, torch.uint16)


def _gemm_args(A, qweight, scales, qzeros, group_size, out):
    M, K = A.shape
    N = qweight.shape[1]
    if qweight.shape[0] * 8 != K:
        raise ValueError(f"qweight {tuple(qweight.shape)} does not match K={K}")
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out {tuple(out.shape)} is not [{M}, {N}]")
    if tuple(scales.shape) != (K // group_size, N):
        raise ValueError(f"scales {tuple(scales.shape)} is not [{K // group_size}, {N}]")
    if qzeros is not None and tuple(qzeros.shape) != (K // group_size, N // 8):
        raise ValueError(f"qzeros {tuple(qzeros.shape)} is not [{K // group_size}, {N // 8}]")
    dt = {torch.float32: OUT_F32, torch.bfloat16: OUT_BF16}.get(out.dtype)
    if dt is None:
        raise TypeError("out must be float32 or bfloat16")
    return (_ptr(A, "A", (torch.bfloat16, torch.int16, torch.uint16)), _ptr(qweight, "qweight", _I32),
            _ptr(scales, "scales", _I16), _ptr(qzeros, "qzeros", _I32), int(group_size), M, N, K,
            _ptr(out, "out", (torch.float32, torch.bfloat16)), dt)


def w4a16_gemm(A, qweight, scales, qzeros, group_size, out, stream=None):
    """out[M,N] = A[M,K] (bf16) x dequant(qweight, scales, qzeros); qzeros None = symmetric 8."""
    args = _gemm_args(A, qweight, scales, qzeros, group_size, out)
    _check(load().w4a16_gemm(*args, _stream(stream)), "w4a16_gemm")
    return out


def w4a16_gemm_decode_ex(A, qweight, scales, qzeros, group_size, out, slices=0, tiles=0, kw=0, tile_cols=0, ring=0,
                         idx=None, stream=None):
    """w4a16_gemm on the decode kernel with an explicit launch (0 = its default for that knob); idx
    (int32 [M, k]) adds the fused pick of the k best columns per row."""
    args = _gemm_args(A, qweight, scales, qzeros, group_size, out)
    k = 0
    if idx is not None:
        if idx.dim() != 2 or idx.shape[0] != A.shape[0]:
            raise ValueError("idx must be [M, k]")
        k = int(idx.shape[1])
    _check(load().w4a16_gemm_decode_ex(*args, int(slices), int(tiles), int(kw), int(tile_cols), int(ring), k,
                                       _ptr(idx, "idx", (torch.int32,)), _stream(stream)), "w4a16_gemm_decode_ex")
    return out


def w4a16_decode_plan(M, N, K, group_size, packed_zeros=False, slices=0, tiles=0, kw=0, tile_cols=0, ring=0, topk=0,
                      affine_bits=0):
    """The decode kernel's launch for a shape (host only, no device work): a dict of slices, tiles,
    kw, tile_cols, ring, lds bytes and sub (32-row steps per ring slot), or W4A16Error with the status
    w4a16_gemm_decode_ex would return."""
    out = (ctypes.c_int * 7)()
    _check(load().w4a16_decode_plan(int(M), int(N), int(K), int(group_size), int(bool(packed_zeros)), int(slices),
                                    int(tiles), int(kw), int(tile_cols), int(ring), int(topk), int(affine_bits), out),
           "w4a16_decode_plan")
    return dict(zip(("slices", "tiles", "kw", "tile_cols", "ring", "lds", "sub"), list(out)))


def w4a16_gemm_noalloc(A, qweight, scales, qzeros, group_size, out, stream=None):
    """w4a16_gemm on the library's fixed per-GPU scratch array: allocates nothing."""
    args = _gemm_args(A, qweight, scales, qzeros, group_size, out)
    _check(load().w4a16_gemm_noalloc(*args, _stream(stream)), "w4a16_gemm_noalloc")
    return out


def w4a16_gemm_ex(A, qweight, scales, qzeros, group_size, out, splits=0, waves_k=0, tile_cols=0, stream=None):
    """w4a16_gemm with an explicit launch (0 = the default choice for that knob)."""
    args = _gemm_args(A, qweight, scales, qzeros, group_size, out)
    _check(load().w4a16_gemm_ex(*args, int(splits), int(waves_k), int(tile_cols), _stream(stream)),
           "w4a16_gemm_ex")
    return out


def w4a16_gemm_topk(A, qweight, scales, qzeros, group_size, out, idx, stream=None):
    """w4a16_gemm plus the k best columns per row (fp32 values, best first; -1 when a row runs out)
    in the same launch; idx: int32 [M, k], k in 1..8."""
    args = _gemm_args(A, qweight, scales, qzeros, group_size, out)
    if idx.dim() != 2 or idx.shape[0] != A.shape[0]:
        raise ValueError("idx must be [M, k]")
    _check(load().w4a16_gemm_topk(*args, int(idx.shape[1]), _ptr(idx, "idx", (torch.int32,)), _stream(stream)),
           "w4a16_gemm_topk")
    return out, idx


def w4a16_gemm_argmax(A, qweight, scales, qzeros, group_size, out, idx, stream=None):
    """w4a16_gemm plus the greedy pick per row (fp32 values) in the same launch."""
    args = _gemm_args(A, qweight, scales, qzeros, group_size, out)
    if tuple(idx.shape) != (A.shape[0],):
        raise ValueError("idx must be [M]")
    _check(load().w4a16_gemm_argmax(*args, _ptr(idx, "idx", (torch.int32,)), _stream(stream)),
           "w4a16_gemm_argmax")
    return out, idx


def w4a16_gemm_prefill(A, qweight, scales, qzeros, group_size, out, stream=None):
    """w4a16_gemm for many rows (prompt processing, M up to 65536) on the matrix cores."""
    args = _gemm_args(A, qweight, scales, qzeros, group_size, out)
    _check(load().w4a16_gemm_prefill(*args, _stream(stream)), "w4a16_gemm_prefill")
    return out


def w4a16_gemm_gate_up(A, gate, up, group_size, out, splits=0, waves_k=0, stream=None):
    """out[M,N] = silu(A x W_gate) * (A x W_up) in one launch. ``gate`` and ``up`` are
    (qweight, scales, qzeros) triples of the same shape (qzeros None = symmetric 8 for both);
    splits / waves_k > 0 fix the launch as in w4a16_gemm_ex."""
    ga = _gemm_args(A, gate[0], gate[1], gate[2], group_size, out)
    ua = _gemm_args(A, up[0], up[1], up[2], group_size, out)
    _check(load().w4a16_gemm_gate_up_ex(ga[0], ga[1], ga[2], ga[3], ua[1], ua[2], ua[3], *ga[4:],
                                        int(splits), int(waves_k), _stream(stream)),
           "w4a16_gemm_gate_up")
    return out


def w4a16_gemm_gate_up_prefill(A, gate, up, group_size, out, stream=None):
    """silu(A x W_gate) * (A x W_up) for many rows (prompt processing) on the matrix cores."""
    ga = _gemm_args(A, gate[0], gate[1], gate[2], group_size, out)
    ua = _gemm_args(A, up[0], up[1], up[2], group_size, out)
    _check(load().w4a16_gemm_gate_up_prefill(ga[0], ga[1], ga[2], ga[3], ua[1], ua[2], ua[3], *ga[4:],
                                             _stream(stream)), "w4a16_gemm_gate_up_prefill")
    return out


def w4a16_plan(M, N, K, group_size):
    """(kernel, splits, waves_k, tile_cols) that w4a16_gemm uses for a shape; kernel 0 = GEMV,
    1 = MFMA GEMM."""
    k, s, w, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(load().w4a16_plan(int(M), int(N), int(K), int(group_size), ctypes.byref(k), ctypes.byref(s),
                             ctypes.byref(w), ctypes.byref(c)), "w4a16_plan")
    return k.value, s.value, w.value, c.value


def w4a16_stream_read(buf, sink, stream=None):
    """Measurement hook: one plain streaming read of the tensor's bytes (sink: int32 [>= 1])."""
    _check(load().w4a16_stream_read(_ptr(buf, "buf", (buf.dtype,)), buf.numel() * buf.element_size(),
                                    _ptr(sink, "sink", (torch.int32,)), _stream(stream)), "w4a16_stream_read")


def w4a16_argmax_rows(logits, idx, stream=None):
    M, N = logits.shape
    if tuple(idx.shape) != (M,):
        raise ValueError("idx must be [M]")
    _check(load().w4a16_argmax_rows(_ptr(logits, "logits", (torch.float32,)), M, N,
                                    _ptr(idx, "idx", (torch.int32,)), _stream(stream)),
           "w4a16_argmax_rows")
    return idx


def w4a16_gemm_affine(A, qweight, scales, biases, group_size, out, splits=0, waves_k=0, tile_cols=0,
                      stream=None):
    """out[M,N] = A[M,K] (bf16) x W, W = scales * q + biases (4-bit codes in qweight, bf16 scales
    and biases [K/g, N]); splits / waves_k / tile_cols as w4a16_gemm_ex (0 = default)."""
    args = list(_gemm_args(A, qweight, scales, None, group_size, out))
    if tuple(biases.shape) != tuple(scales.shape):
        raise ValueError(f"biases {tuple(biases.shape)} is not {tuple(scales.shape)}")
    _sb = (torch.bfloat16, torch.int16, torch.uint16)
    args[2] = _ptr(scales, "scales", _sb)
    args[3] = _ptr(biases, "biases", _sb)
    if splits or waves_k or tile_cols:
        rc = load().w4a16_gemm_affine_ex(*args, int(splits), int(waves_k), int(tile_cols), _stream(stream))
    else:
        rc = load().w4a16_gemm_affine(*args, _stream(stream))
    _check(rc, "w4a16_gemm_affine")
    return out


def w4a16_gemm_affine_gate_up(A, gate, up, group_size, out, stream=None):
    """out = silu(A x W_gate) * (A x W_up) for affine matrices; gate and up are
    (qweight, scales, biases) triples (4-bit codes, bf16 scales and biases)."""
    M, K = A.shape
    N = gate[0].shape[1]
    _sb = (torch.bfloat16, torch.int16, torch.uint16)
    for name, (qw, sc, bi) in (("gate", gate), ("up", up)):
        if qw.shape[0] * 8 != K or qw.shape[1] != N:
            raise ValueError(f"{name} qweight {tuple(qw.shape)} is not [{K // 8}, {N}]")
        if tuple(sc.shape) != (K // group_size, N) or tuple(bi.shape) != tuple(sc.shape):
            raise ValueError(f"{name} scales and biases must be [{K // group_size}, {N}]")
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out {tuple(out.shape)} is not [{M}, {N}]")
    dt = {torch.float32: OUT_F32, torch.bfloat16: OUT_BF16}.get(out.dtype)
    if dt is None:
        raise TypeError("out must be float32 or bfloat16")
    ptrs = []
    for qw, sc, bi in (gate, up):
        ptrs += [_ptr(qw, "qweight", _I32), _ptr(sc, "scales", _sb), _ptr(bi, "biases", _sb)]
    _check(load().w4a16_gemm_affine_gate_up(_ptr(A, "A", _sb), *ptrs, int(group_size), M, N, K,
                                            _ptr(out, "out", (torch.float32, torch.bfloat16)), dt,
                                            _stream(stream)),
           "w4a16_gemm_affine_gate_up")
    return out


def w4a16_affine_widen(packed, bits, K, qweight_out, stream=None):
    """Codes of ``bits`` (1..4) bits in column bit streams [K*bits/32, N] -> 4-bit qweight [K/8, N]."""
    N = packed.shape[1]
    if packed.shape[0] * 32 != K * bits:
        raise ValueError(f"packed {tuple(packed.shape)} does not hold K={K} codes of {bits} bits")
    if tuple(qweight_out.shape) != (K // 8, N):
        raise ValueError("qweight_out must be [K/8, N]")
    _check(load().w4a16_affine_widen(_ptr(packed, "packed", _I32), int(bits), int(K), N,
                                     _ptr(qweight_out, "qweight_out", _I32), _stream(stream)),
           "w4a16_affine_widen")
    return qweight_out


def w4a16_affine_split(packed, bits, scales, biases, group_size, K, qweight_out, scales_out, biases_out,
                       stream=None):
    """Codes of ``bits`` (5..8) bits -> two 4-bit planes over 2K rows (low, then high) with their
    scales (s, then 16 s) and biases (b, then 0), for w4a16_gemm_affine_split."""
    N = packed.shape[1]
    G = K // group_size
    if packed.shape[0] * 32 != K * bits:
        raise ValueError(f"packed {tuple(packed.shape)} does not hold K={K} codes of {bits} bits")
    if tuple(scales.shape) != (G, N) or tuple(biases.shape) != (G, N):
        raise ValueError(f"scales and biases must be [{G}, {N}]")
    if tuple(qweight_out.shape) != (2 * K // 8, N):
        raise ValueError("qweight_out must be [2K/8, N]")
    if tuple(scales_out.shape) != (2 * G, N) or tuple(biases_out.shape) != (2 * G, N):
        raise ValueError("scales_out and biases_out must be [2K/g, N]")
    _sb = (torch.bfloat16, torch.int16, torch.uint16)
    _check(load().w4a16_affine_split(_ptr(packed, "packed", _I32), int(bits), _ptr(scales, "scales", _sb),
                                     _ptr(biases, "biases", _sb), int(group_size), int(K), N,
                                     _ptr(qweight_out, "qweight_out", _I32), _ptr(scales_out, "scales_out", _sb),
                                     _ptr(biases_out, "biases_out", _sb), _stream(stream)),
           "w4a16_affine_split")
    return qweight_out, scales_out, biases_out


def w4a16_gemm_affine_split(A, qweight, scales, biases, group_size, out, stream=None):
    """out[M,N] = A[M,K] x W, W = s * q + b from the split planes of w4a16_affine_split."""
    M, K = A.shape
    N = qweight.shape[1]
    if qweight.shape[0] * 8 != 2 * K:
        raise ValueError(f"qweight {tuple(qweight.shape)} is not the [2K/8, N] planes for K={K}")
    if tuple(scales.shape) != (2 * K // group_size, N) or tuple(biases.shape) != tuple(scales.shape):
        raise ValueError("scales and biases must be [2K/g, N]")
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out {tuple(out.shape)} is not [{M}, {N}]")
    dt = {torch.float32: OUT_F32, torch.bfloat16: OUT_BF16}.get(out.dtype)
    if dt is None:
        raise TypeError("out must be float32 or bfloat16")
    _sb = (torch.bfloat16, torch.int16, torch.uint16)
    _check(load().w4a16_gemm_affine_split(_ptr(A, "A", _sb), _ptr(qweight, "qweight", _I32),
                                          _ptr(scales, "scales", _sb), _ptr(biases, "biases", _sb),
                                          int(group_size), M, N, K, _ptr(out, "out", (torch.float32, torch.bfloat16)),
                                          dt, _stream(stream)),
           "w4a16_gemm_affine_split")
    return out


def w4a16_gemm_affine_bits(A, packed, bits, scales, biases, group_size, out, slices=0, tiles=0, kw=0, ring=0,
                           stream=None):
    """out[M,N] = A[M,K] (bf16) x W, W = scales * q + biases, the codes read at their own width
    from the column bit streams `packed` (uint32 [K*bits/32, N]; bits 1..6 or 8), bf16 scales and
    biases [K/g, N]; slices / tiles / kw / ring as w4a16_gemm_decode_ex (0 = default)."""
    M, K = A.shape
    N = packed.shape[1]
    if packed.shape[0] * 32 != K * bits:
        raise ValueError(f"packed {tuple(packed.shape)} is not [{K * bits // 32}, {N}] for {bits}-bit codes")
    if tuple(scales.shape) != (K // group_size, N) or tuple(biases.shape) != tuple(scales.shape):
        raise ValueError("scales and biases must be [K/g, N]")
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out {tuple(out.shape)} is not [{M}, {N}]")
    dt = {torch.float32: OUT_F32, torch.bfloat16: OUT_BF16}.get(out.dtype)
    if dt is None:
        raise TypeError("out must be float32 or bfloat16")
    _sb = (torch.bfloat16, torch.int16, torch.uint16)
    _check(load().w4a16_gemm_affine_bits_ex(_ptr(A, "A", _sb), _ptr(packed, "packed", _I32), int(bits),
                                            _ptr(scales, "scales", _sb), _ptr(biases, "biases", _sb), int(group_size),
                                            M, N, K, _ptr(out, "out", (torch.float32, torch.bfloat16)), dt,
                                            int(slices), int(tiles), int(kw), int(ring), _stream(stream)),
           "w4a16_gemm_affine_bits")
    return out


def w4a16_gemm_affine_bits_prefill(A, packed, bits, scales, biases, group_size, out, stream=None):
    """The product of w4a16_gemm_affine_bits for many rows (M up to 65536), on the prompt GEMM."""
    M, K = A.shape
    N = packed.shape[1]
    if packed.shape[0] * 32 != K * bits:
        raise ValueError(f"packed {tuple(packed.shape)} is not [{K * bits // 32}, {N}] for {bits}-bit codes")
    if tuple(scales.shape) != (K // group_size, N) or tuple(biases.shape) != tuple(scales.shape):
        raise ValueError("scales and biases must be [K/g, N]")
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out {tuple(out.shape)} is not [{M}, {N}]")
    dt = {torch.float32: OUT_F32, torch.bfloat16: OUT_BF16}.get(out.dtype)
    if dt is None:
        raise TypeError("out must be float32 or bfloat16")
    _sb = (torch.bfloat16, torch.int16, torch.uint16)
    _check(load().w4a16_gemm_affine_bits_prefill(_ptr(A, "A", _sb), _ptr(packed, "packed", _I32), int(bits),
                                                 _ptr(scales, "scales", _sb), _ptr(biases, "biases", _sb),
                                                 int(group_size), M, N, K,
                                                 _ptr(out, "out", (torch.float32, torch.bfloat16)), dt,
                                                 _stream(stream)),
           "w4a16_gemm_affine_bits_prefill")
    return out


def w4a16_unpack_u8(qweight, q_out, stream=None):
    K, N = qweight.shape[0] * 8, qweight.shape[1]
    if tuple(q_out.shape) != (K, N):
        raise ValueError("q_out must be [K, N]")
    _check(load().w4a16_unpack_u8(_ptr(qweight, "qweight", _I32), K, N,
                                  _ptr(q_out, "q_out", (torch.uint8,)), _stream(stream)),
           "w4a16_unpack_u8")
    return q_out


def w4a16_dequant_f32(qweight, scales, qzeros, group_size, w_out, stream=None):
    K, N = qweight.shape[0] * 8, qweight.shape[1]
    if tuple(w_out.shape) != (K, N):
        raise ValueError("w_out must be [K, N]")
    _check(load().w4a16_dequant_f32(_ptr(qweight, "qweight", _I32), _ptr(scales, "scales", _I16),
                                    _ptr(qzeros, "qzeros", _I32), int(group_size), K, N,
                                    _ptr(w_out, "w_out", (torch.float32,)), _stream(stream)),
           "w4a16_dequant_f32")
    return w_out


def w4a16_release_scratch():
    _check(load().w4a16_release_scratch(), "w4a16_release_scratch")
