"""Seeded synthetic inputs for the EQ-Linear workloads.

This module is shared by the tests, the benchmark and the CPU oracle's callers.
It holds the workload shapes and draws Gaussian tensors; it contains none of the
layer's arithmetic (no transform, no product, no expansion).

Workloads stand in for the token batches the pages benchmark on: ViT token
batches of 64 images x 196/197 tokens at ViT-B widths ("Quick ViTs", Table 2 in
the key findings; "Flash EQ-Linear", Experimental Results / Network Level).
No image data is involved: tokens are i.i.d. N(0, 1) and weights are
N(0, 1/fan_in), drawn from numpy's PCG64 generator.

Draw order per workload: x first, then the weight tensor(s), each as fp64
standard normals scaled by the std, then rounded once to the workload dtype
(fp32: IEEE round-to-nearest-even; bf16: round-to-nearest-even applied to the
fp32 bit pattern). The rounded values, converted exactly back to fp64, are what
both the GPU path and the oracle consume.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass

import numpy as np

F32 = "f32"
BF16 = "bf16"
F16 = "f16"


@dataclass(frozen=True)
class Workload:
    """One layer workload: a cyclic-group layer (group='C'), the D8 variant
    (group='D8', N = 8) or another dihedral group D_n (group='D', N = 2n)."""

    name: str
    group: str  # "C" (cyclic C_N), "D8", or "D" (dihedral D_n)
    N: int  # group order (8 for D8, 2n for D_n)
    C_in: int  # C: channels per group element; D8: full width
    C_out: int
    T: int  # tokens
    dtype: str
    note: str = ""

    @property
    def x_shape(self):
        if self.group == "C":
            return (self.T, self.C_in, self.N)
        return (self.T, self.C_in)

    @property
    def y_shape(self):
        if self.group == "C":
            return (self.T, self.C_out, self.N)
        return (self.T, self.C_out)


# The five benchmark layers.  c3 is the ViT-B MLP trio (768->768, 768->3072,
# 3072->768 at 8 group elements, i.e. 96 and 384 channels per element).
WORKLOADS = {
    "c1": Workload("c1", "C", 4, 8, 8, 64, F32, "C4, 64 tokens, width 32"),
    "c2": Workload("c2", "C", 8, 32, 32, 4096, F32, "C8, 4096 tokens, width 256"),
    "c3a": Workload("c3a", "C", 8, 96, 96, 64 * 197, BF16, "C8 ViT-B 768->768"),
    "c3b": Workload("c3b", "C", 8, 96, 384, 64 * 197, BF16, "C8 ViT-B MLP 768->3072"),
    "c3c": Workload("c3c", "C", 8, 384, 96, 64 * 197, BF16, "C8 ViT-B MLP 3072->768"),
    "c4": Workload("c4", "C", 7, 160, 160, 32768, BF16, "C7 odd order, width 1120"),
    "c5": Workload("c5", "D8", 8, 1280, 1280, 16 * 257, BF16, "D8 Fourier-domain, width 1280"),
    # the extension to other shapes: the hexagon's symmetries (order 12), c5's batch
    "d6": Workload("d6", "D", 12, 1152, 1152, 16 * 257, BF16, "D6 (hexagon) Fourier-domain, width 1152"),
}


def round_f32(a64: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 bit pattern (numpy's conversion rounds to nearest even)."""
    return np.ascontiguousarray(a64, dtype=np.float64).astype(np.float32)


def round_bf16_bits(a64: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bit pattern (uint16): fp32 first, then RNE on the upper half."""
    u = round_f32(a64).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) & 0xFFFF
    return r.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def quantize(a64: np.ndarray, dtype: str):
    """Return (device_array, exact_fp64) for the workload dtype.

    device_array is float32 (f32), or uint16 bit patterns (bf16, f16).
    exact_fp64 holds the same values exactly in fp64.  fp16 takes numpy's
    fp64 -> float16 conversion (round-to-nearest-even, correctly rounded).
    """
    if dtype == F32:
        d = round_f32(a64)
        return d, d.astype(np.float64)
    if dtype == BF16:
        b = round_bf16_bits(a64)
        return b, bf16_bits_to_f64(b)
    if dtype == F16:
        h = np.ascontiguousarray(a64, dtype=np.float64).astype(np.float16)
        return h.view(np.uint16), h.astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def _normal(rng, shape, std):
    return rng.standard_normal(size=shape, dtype=np.float64) * std


def cn_inputs(N: int, C_in: int, C_out: int, T: int, dtype: str, seed: int = 0):
    """x[T][C_in][N] ~ N(0,1), w[C_out][C_in][N] ~ N(0, 1/(C_in*N)).

    Returns a dict with device arrays ('x', 'w') and exact fp64 copies
    ('x64', 'w64').
    """
    rng = np.random.default_rng(seed)
    x = _normal(rng, (T, C_in, N), 1.0)
    w = _normal(rng, (C_out, C_in, N), 1.0 / np.sqrt(C_in * N))
    xd, x64 = quantize(x, dtype)
    wd, w64 = quantize(w, dtype)
    return {"x": xd, "x64": x64, "w": wd, "w64": w64}


def channel_bias(C_out: int, dtype: str, seed: int = 0):
    """A per-output-channel bias b[C_out] ~ N(0, 0.5^2): ('b', 'b64') like quantize().

    Its spread keeps layer output + bias on both sides of 0, where GELU bends."""
    rng = np.random.default_rng(seed)
    return quantize(_normal(rng, (C_out,), 0.5), dtype)


def d8_block_shapes(C_in: int, C_out: int):
    """Shapes of the five D8 weight blocks, in packing order A1, A2, B1, B2, E."""
    mi, mo = C_in // 8, C_out // 8
    return [(mo, mi)] * 4 + [(2 * mo, 2 * mi)]


def dn_block_shapes(n: int, C_in: int, C_out: int):
    """Shapes of the D_n weight blocks in packing order: one (C_out/2n, C_in/2n)
    per 1-D irrep (4 for even n, 2 for odd), then one (C_out/n, C_in/n) per E_k."""
    mi, mo = C_in // (2 * n), C_out // (2 * n)
    n1 = 4 if n % 2 == 0 else 2
    n2 = n // 2 - 1 if n % 2 == 0 else (n - 1) // 2
    return [(mo, mi)] * n1 + [(2 * mo, 2 * mi)] * n2


def dn_inputs(n: int, C_in: int, C_out: int, T: int, dtype: str, seed: int = 0):
    """x[T][C_in] ~ N(0,1) and the D_n blocks ~ N(0, 1/fan_in), packed flat ('wb')."""
    if C_in % (2 * n) or C_out % (2 * n):
        raise ValueError("D_n widths must be multiples of 2n")
    rng = np.random.default_rng(seed)
    x = _normal(rng, (T, C_in), 1.0)
    wb = np.concatenate([_normal(rng, shp, 1.0 / np.sqrt(shp[1])).ravel() for shp in dn_block_shapes(n, C_in, C_out)])
    xd, x64 = quantize(x, dtype)
    wd, w64 = quantize(wb, dtype)
    return {"x": xd, "x64": x64, "w": wd, "w64": w64}


def d8_inputs(C_in: int, C_out: int, T: int, dtype: str, seed: int = 0):
    """x[T][C_in] ~ N(0,1); blocks W_A1, W_A2, W_B1, W_B2 (std 1/sqrt(C_in/8))
    and W_E (std 1/sqrt(C_in/4)), packed flat in that order ('wb')."""
    if C_in % 8 or C_out % 8:
        raise ValueError("D8 widths must be multiples of 8")
    rng = np.random.default_rng(seed)
    x = _normal(rng, (T, C_in), 1.0)
    blocks = []
    for shp in d8_block_shapes(C_in, C_out):
        blocks.append(_normal(rng, shp, 1.0 / np.sqrt(shp[1])).ravel())
    wb = np.concatenate(blocks)
    xd, x64 = quantize(x, dtype)
    wd, w64 = quantize(wb, dtype)
    return {"x": xd, "x64": x64, "w": wd, "w64": w64}


def workload_inputs(wl: Workload, seed: int = 0, T: int | None = None):
    T = wl.T if T is None else T
    if wl.group == "C":
        return cn_inputs(wl.N, wl.C_in, wl.C_out, T, wl.dtype, seed)
    if wl.group == "D8":
        return d8_inputs(wl.C_in, wl.C_out, T, wl.dtype, seed)
    return dn_inputs(wl.N // 2, wl.C_in, wl.C_out, T, wl.dtype, seed)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
