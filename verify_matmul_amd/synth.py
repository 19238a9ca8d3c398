"""Seeded synthetic inputs for the W4A16 matmul (GPTQ-packed int4 weights x bf16 activations).

This module only draws random numbers and lays them out in the storage format; it holds
none of the matmul's arithmetic (no unpacking, no dequantisation, no accumulation). Both
the CPU oracle's tests and the HIP path take their inputs from here, so the two never
share anything else.

Storage format (the GPTQ convention for 4-bit weights):
  qweight  uint32 [K/8, N]   nibble j (bits 4j..4j+3) of word [i, n] is the code of row 8i+j
  scales   fp16   [K/g, N]   stored here as uint16 bit patterns
  qzeros   uint32 [K/g, N/8] nibble j of word [gi, c] is the zero of column 8c+j; absent
                             (None) means every zero is 8 (the symmetric checkpoints)
  A        bf16   [M, K]     stored here as uint16 bit patterns, row-major

The workloads mirror the checkpoints the GRIMOIRE v1.7 release notes benchmark in
'What changed' (GPTQ int4 group 128 symmetric; W4A16 group 64) at the hidden/FFN widths of
a 27B-class model, the 248k-row output layer named in strix-llama.cpp PR #105, and the
1 + 4 drafted rows of the v1.8 MTP check (GRIMOIRE v1.8 release notes, 'What changed').
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

# tensor ids mixed into the seed: seed = 1000 * config_index + tensor_id
_T_QWEIGHT, _T_SCALES, _T_ZEROS, _T_ACT = 1, 2, 3, 4
# the second matrix of a gated pair (the gate beside the up projection): its own draws
_T_QWEIGHT2, _T_SCALES2, _T_ZEROS2 = 5, 6, 7


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes plus the value distributions of its tensors."""
    index: int            # 1-based configuration number, part of every seed
    name: str
    K: int
    N: int
    group: int
    symmetric: bool       # True: no qzeros, every zero is 8
    ms: tuple             # row counts the workload is run at
    scale_lo: float
    scale_hi: float
    act_sigma: float
    outlier_frac: float   # fraction of activation entries multiplied by outlier_mul
    outlier_mul: float
    argmax: bool          # the output layer also checks a per-row argmax

    @property
    def groups(self) -> int:
        return self.K // self.group


WORKLOADS = {
    "tiny": Workload(1, "tiny 512x256 g128 sym", 512, 256, 128, True, (1,),
                     0.002, 0.02, 1.0, 0.0, 1.0, False),
    "attn": Workload(2, "attention projection 5120x5120 g128 sym", 5120, 5120, 128, True, (1,),
                     0.002, 0.02, 1.0, 0.0, 1.0, False),
    "ffn_up": Workload(3, "FFN up/gate 5120x17408 g128 sym", 5120, 17408, 128, True,
                       (1, 2, 4, 8, 16), 0.002, 0.02, 1.0, 0.0, 1.0, False),
    "ffn_down": Workload(4, "FFN down 17408x5120 g64 asym", 17408, 5120, 64, False,
                         (1, 4, 8, 16), 0.001, 0.01, 2.0, 0.01, 20.0, False),
    "lm_head": Workload(5, "LM head 5120x248320 g128 sym", 5120, 248320, 128, True,
                        (5, 1), 0.002, 0.02, 1.0, 0.0, 1.0, True),
}

MAX_ROWS = 16


@dataclass
class Inputs:
    """Host copies of one workload's tensors (numpy arrays in storage format)."""
    qweight: np.ndarray            # uint32 [K/8, N]
    scales: np.ndarray             # uint16 [K/g, N] (fp16 bits)
    qzeros: Optional[np.ndarray]   # uint32 [K/g, N/8] or None
    act: np.ndarray                # uint16 [16, K] (bf16 bits); a call with M rows uses act[:M]
    group: int

    @property
    def K(self) -> int:
        return self.qweight.shape[0] * 8

    @property
    def N(self) -> int:
        return self.qweight.shape[1]


def _rng(index: int, tensor: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * index + tensor))


def random_words(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniform uint32 words: every nibble is an independent uniform draw from 0..15."""
    return rng.integers(0, 1 << 32, size=shape, dtype=np.uint32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even, via torch) and return bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def f64_to_fp16_bits(x: np.ndarray) -> np.ndarray:
    """Round to fp16 (numpy's round-to-nearest-even) and return bit patterns."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def draw_scales(rng: np.random.Generator, shape, lo: float, hi: float) -> np.ndarray:
    return f64_to_fp16_bits(rng.uniform(lo, hi, size=shape))


def draw_activations(rng: np.random.Generator, rows: int, K: int, sigma: float,
                     outlier_frac: float, outlier_mul: float) -> np.ndarray:
    """sigma * N(0,1) in fp32, an exact count of outlier entries scaled, one rounding to bf16."""
    a = rng.standard_normal((rows, K), dtype=np.float32) * np.float32(sigma)
    if outlier_frac > 0.0:
        count = int(round(outlier_frac * rows * K))
        pos = rng.permutation(rows * K)[:count]
        flat = a.reshape(-1)
        flat[pos] *= np.float32(outlier_mul)
    return f32_to_bf16_bits(a)


def make_inputs(wl: Workload | str, N: Optional[int] = None) -> Inputs:
    """Draw a workload's tensors. ``N`` overrides the width (a leading slice of columns is
    NOT taken: the draw itself is made at the given width), used for quick variants."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    n = wl.N if N is None else N
    qweight = random_words(_rng(wl.index, _T_QWEIGHT), (wl.K // 8, n))
    scales = draw_scales(_rng(wl.index, _T_SCALES), (wl.groups, n), wl.scale_lo, wl.scale_hi)
    qzeros = None if wl.symmetric else random_words(_rng(wl.index, _T_ZEROS), (wl.groups, n // 8))
    act = draw_activations(_rng(wl.index, _T_ACT), MAX_ROWS, wl.K, wl.act_sigma,
                           wl.outlier_frac, wl.outlier_mul)
    return Inputs(qweight, scales, qzeros, act, wl.group)


def make_gate_inputs(wl: Workload | str, N: Optional[int] = None) -> Inputs:
    """The gate matrix that pairs with ``make_inputs(wl)`` (taken as the up projection) in a
    gated feed-forward input: same shapes and distributions, its own draws, the same
    activations."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    n = wl.N if N is None else N
    up = make_inputs(wl, N)
    qweight = random_words(_rng(wl.index, _T_QWEIGHT2), (wl.K // 8, n))
    scales = draw_scales(_rng(wl.index, _T_SCALES2), (wl.groups, n), wl.scale_lo, wl.scale_hi)
    qzeros = None if wl.symmetric else random_words(_rng(wl.index, _T_ZEROS2), (wl.groups, n // 8))
    return Inputs(qweight, scales, qzeros, up.act, wl.group)


def make_random(seed: int, M: int, K: int, N: int, group: int, symmetric: bool,
                scale_lo: float = 0.002, scale_hi: float = 0.02, sigma: float = 1.0) -> Inputs:
    """Free-form seeded inputs for parity sweeps over arbitrary shapes."""
    rng = np.random.Generator(np.random.PCG64(seed))
    qweight = random_words(rng, (K // 8, N))
    scales = draw_scales(rng, (K // group, N), scale_lo, scale_hi)
    qzeros = None if symmetric else random_words(rng, (K // group, N // 8))
    act = draw_activations(rng, M, K, sigma, 0.0, 1.0)
    return Inputs(qweight, scales, qzeros, act, group)


# ---- encoders for hand-built codes (tests that need a chosen code pattern) -------------

def pack_rows(codes: np.ndarray) -> np.ndarray:
    """Encode codes [K, N] (values 0..15) as qweight [K/8, N]: row 8i+j -> nibble j of word i."""
    c = np.asarray(codes, dtype=np.uint32)
    K, N = c.shape
    assert K % 8 == 0 and c.max(initial=0) < 16
    c = c.reshape(K // 8, 8, N)
    out = np.zeros((K // 8, N), dtype=np.uint32)
    for j in range(8):
        out |= c[:, j, :] << np.uint32(4 * j)
    return out


def pack_cols(codes: np.ndarray) -> np.ndarray:
    """Encode zeros [G, N] (values 0..15) as qzeros [G, N/8]: column 8c+j -> nibble j of word c."""
    c = np.asarray(codes, dtype=np.uint32)
    G, N = c.shape
    assert N % 8 == 0 and c.max(initial=0) < 16
    c = c.reshape(G, N // 8, 8)
    out = np.zeros((G, N // 8), dtype=np.uint32)
    for j in range(8):
        out |= c[:, :, j] << np.uint32(4 * j)
    return out


# ---- affine codes (MLX affine quantisation: w = s * q + b) ------------------------------
#
# Storage format of an affine matrix with codes of `bits` bits (TensorFold PR #859, commit
# messages: mixed-width MLX checkpoints, 2 to 8 bits in groups of 64):
#   packed   uint32 [K*bits/32, N]  for column n the codes of rows 0, 1, 2, ... form one
#                                   little-endian bit stream (row k at stream bits
#                                   k*bits .. k*bits+bits-1); stream bit i is bit i % 32 of
#                                   word [i / 32, n]. At 4 bits this is the qweight layout.
#   scales   bf16   [K/g, N]        stored as uint16 bit patterns
#   biases   bf16   [K/g, N]        stored as uint16 bit patterns

_T_AFF_CODES, _T_AFF_SCALES, _T_AFF_BIASES, _T_AFF_ACT = 11, 12, 13, 14
# the gate matrix beside an affine up projection: its own draws
_T_AFF_CODES2, _T_AFF_SCALES2, _T_AFF_BIASES2 = 15, 16, 17


@dataclass
class AffineInputs:
    packed: np.ndarray   # uint32 [K*bits/32, N]
    bits: int
    scales: np.ndarray   # uint16 [K/g, N] (bf16 bits)
    biases: np.ndarray   # uint16 [K/g, N] (bf16 bits)
    act: np.ndarray      # uint16 [rows, K] (bf16 bits)
    group: int

    @property
    def K(self) -> int:
        return self.packed.shape[0] * 32 // self.bits

    @property
    def N(self) -> int:
        return self.packed.shape[1]


@dataclass(frozen=True)
class AffineWorkload:
    index: int
    name: str
    K: int
    N: int
    group: int
    bits: int
    ms: tuple


# An MLX affine-4 checkpoint's FFN up/gate projection (groups of 64) at the 27B-class widths.
AFFINE_WORKLOADS = {
    "ffn_up_affine4": AffineWorkload(6, "FFN up/gate 5120x17408 affine-4 g64", 5120, 17408, 64, 4,
                                     (1, 2, 4, 8, 16)),
    # the same projection of an 8-bit MLX checkpoint
    "ffn_up_affine8": AffineWorkload(7, "FFN up/gate 5120x17408 affine-8 g64", 5120, 17408, 64, 8,
                                     (1, 2, 4, 8, 16)),
    # and of 2, 3, 5 and 6-bit ones (mixed-width checkpoints)
    "ffn_up_affine2": AffineWorkload(8, "FFN up/gate 5120x17408 affine-2 g64", 5120, 17408, 64, 2,
                                     (1, 2, 4, 8, 16)),
    "ffn_up_affine3": AffineWorkload(9, "FFN up/gate 5120x17408 affine-3 g64", 5120, 17408, 64, 3,
                                     (1, 2, 4, 8, 16)),
    "ffn_up_affine5": AffineWorkload(10, "FFN up/gate 5120x17408 affine-5 g64", 5120, 17408, 64, 5,
                                     (1, 2, 4, 8, 16)),
    "ffn_up_affine6": AffineWorkload(11, "FFN up/gate 5120x17408 affine-6 g64", 5120, 17408, 64, 6,
                                     (1, 2, 4, 8, 16)),
}


def pack_stream(codes: np.ndarray, bits: int) -> np.ndarray:
    """Encode codes [K, N] (values < 2^bits) as column bit streams [K*bits/32, N]."""
    c = np.asarray(codes, dtype=np.uint32)
    K, N = c.shape
    assert (K * bits) % 32 == 0 and c.max(initial=0) < (1 << bits)
    stream = ((c[:, None, :] >> np.arange(bits, dtype=np.uint32)[None, :, None]) & 1)   # [K, bits, N]
    stream = stream.reshape(K * bits // 32, 32, N)
    out = np.zeros((K * bits // 32, N), dtype=np.uint32)
    for i in range(32):
        out |= stream[:, i, :] << np.uint32(i)
    return out


def draw_affine(rng_codes, rng_scales, rng_biases, K: int, N: int, group: int, bits: int):
    """Codes uniform on 0..2^bits-1; scales uniform on [0.002, 0.02] x 15 / (2^bits - 1) (the
    same weight spread at every width) and biases -s * (2^bits - 1) * U(0.4, 0.6) (a group's
    minimum, as affine quantisation stores it, about half the range below zero), both rounded
    once to bf16."""
    top = (1 << bits) - 1
    codes = rng_codes.integers(0, top + 1, size=(K, N), dtype=np.uint32)
    s = rng_scales.uniform(0.002, 0.02, size=(K // group, N)) * (15.0 / top)
    b = -s * top * rng_biases.uniform(0.4, 0.6, size=(K // group, N))
    return pack_stream(codes, bits), f32_to_bf16_bits(s.astype(np.float32)), f32_to_bf16_bits(b.astype(np.float32))


def make_affine_inputs(wl: AffineWorkload | str) -> AffineInputs:
    if isinstance(wl, str):
        wl = AFFINE_WORKLOADS[wl]
    packed, scales, biases = draw_affine(_rng(wl.index, _T_AFF_CODES), _rng(wl.index, _T_AFF_SCALES),
                                         _rng(wl.index, _T_AFF_BIASES), wl.K, wl.N, wl.group, wl.bits)
    act = draw_activations(_rng(wl.index, _T_AFF_ACT), MAX_ROWS, wl.K, 1.0, 0.0, 1.0)
    return AffineInputs(packed, wl.bits, scales, biases, act, wl.group)


def make_affine_random(seed: int, M: int, K: int, N: int, group: int, bits: int,
                       sigma: float = 1.0) -> AffineInputs:
    """Free-form seeded affine inputs for parity sweeps."""
    rng = np.random.Generator(np.random.PCG64(seed))
    packed, scales, biases = draw_affine(rng, rng, rng, K, N, group, bits)
    act = draw_activations(rng, M, K, sigma, 0.0, 1.0)
    return AffineInputs(packed, bits, scales, biases, act, group)


def make_affine_gate_inputs(wl: AffineWorkload | str) -> AffineInputs:
    """The gate matrix that pairs with ``make_affine_inputs(wl)`` (the up projection): same shape
    and distributions, its own draws, the same activations."""
    if isinstance(wl, str):
        wl = AFFINE_WORKLOADS[wl]
    up = make_affine_inputs(wl)
    packed, scales, biases = draw_affine(_rng(wl.index, _T_AFF_CODES2), _rng(wl.index, _T_AFF_SCALES2),
                                         _rng(wl.index, _T_AFF_BIASES2), wl.K, wl.N, wl.group, wl.bits)
    return AffineInputs(packed, wl.bits, scales, biases, up.act, wl.group)
