"""Seeded synthetic inputs shared by the CPU oracle and the HIP path.

This package holds no arithmetic of the attention method: only a
counter-based pseudo-random generator, the value mappings that turn its
words into tensor elements, and the workload shapes.  Both sides draw
their inputs from it; the GPU side additionally has a device-side filler
(``synth/csrc/synth_fill.hip``) that implements the same published
generator independently, so multi-GiB tensors can be produced in HBM and
any element regenerated on the host.

Generator (SplitMix64, Steele, Lea & Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014; finaliser constants as in Vigna's
public-domain ``splitmix64.c``):

* ``mix64(z)``: ``z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
  z *= 0x94D049BB133111EB; z ^= z >> 31`` (all mod 2**64).
* The j-th output (j = 0, 1, ...) of a SplitMix64 stream seeded with ``s``
  is ``mix64(s + (j + 1) * GAMMA)``, ``GAMMA = 0x9E3779B97F4A7C15``.
* Tensor ``tid`` under run seed ``seed`` (both < 2**32) uses the stream
  seeded with ``key = mix64((seed | tid << 32) + GAMMA)``; its word ``j`` is
  output ``j`` of that stream.

Value mappings (element ``e`` is the flat row-major index):

* ``I8U4``  int8 uniform on [-8, 7]: nibble ``e % 16`` of word ``e // 16``,
  minus 8.
* ``BF16U4`` the same integers stored exactly as bfloat16.
* ``BF16N`` approximately N(0, 1) by Irwin-Hall(12): words ``3e .. 3e+2``
  give twelve 16-bit fields ``u_i``; ``x = (sum u_i - 6 * 65536) / 65536``
  is exact in float32 and is rounded to bfloat16 to nearest-even.  Mean
  ~0, variance ~1, bounded by +-6, integer-only, hence bit-identical on
  any machine.
"""

from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

I8U4 = 0
BF16U4 = 1
BF16N = 2

KIND_NAMES = {I8U4: "i8u4", BF16U4: "bf16u4", BF16N: "bf16n"}


def mix64(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = z ^ (z >> np.uint64(30))
        z = z * _M1
        z = z ^ (z >> np.uint64(27))
        z = z * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def stream_key(seed: int, tid: int) -> np.uint64:
    if not (0 <= seed < 2**32 and 0 <= tid < 2**32):
        raise ValueError("seed and tensor id must fit in 32 bits")
    x = np.uint64(seed | (tid << 32))
    with np.errstate(over="ignore"):
        return mix64(np.array([x + GAMMA], dtype=np.uint64))[0]


def words(key: np.uint64, j: np.ndarray) -> np.ndarray:
    """Outputs ``j`` of the SplitMix64 stream seeded with ``key``."""
    j = np.asarray(j, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return mix64(key + (j + np.uint64(1)) * GAMMA)


def _u4(key, e: np.ndarray) -> np.ndarray:
    e = np.asarray(e, dtype=np.int64)
    w = words(key, (e >> 4).astype(np.uint64))
    sh = ((e & 15) * 4).astype(np.uint64)
    return ((w >> sh) & np.uint64(15)).astype(np.int64) - 8


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bfloat16 bit pattern (finite inputs)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16_bits(key, e: np.ndarray) -> np.ndarray:
    e = np.asarray(e, dtype=np.int64).astype(np.uint64)
    s = np.zeros(e.shape, dtype=np.int64)
    for t in range(3):
        w = words(key, e * np.uint64(3) + np.uint64(t))
        for i in range(4):
            s += ((w >> np.uint64(16 * i)) & np.uint64(0xFFFF)).astype(np.int64)
    d = s - 6 * 65536
    f = d.astype(np.float32) * np.float32(1.0 / 65536.0)  # exact: |d| < 2**20
    return f32_to_bf16_bits(f)


def values(kind: int, seed: int, tid: int, flat_index) -> np.ndarray:
    """Elements at the given flat indices.

    Returns int8 for ``I8U4`` and the uint16 bfloat16 bit pattern for the
    bf16 kinds (use :func:`bf16_bits_to_f32` to read them as numbers).
    """
    key = stream_key(seed, tid)
    e = np.asarray(flat_index, dtype=np.int64)
    if kind == I8U4:
        return _u4(key, e).astype(np.int8)
    if kind == BF16U4:
        return f32_to_bf16_bits(_u4(key, e).astype(np.float32))
    if kind == BF16N:
        return _normal_bf16_bits(key, e)
    raise ValueError(f"unknown kind {kind}")


def tensor(kind: int, seed: int, tid: int, shape) -> np.ndarray:
    """A whole tensor (row-major) generated on the host."""
    n = int(np.prod(shape)) if len(shape) else 1
    return values(kind, seed, tid, np.arange(n, dtype=np.int64)).reshape(shape)


def as_float(kind: int, raw: np.ndarray) -> np.ndarray:
    """Numeric value (float64) of generated elements."""
    if kind == I8U4:
        return raw.astype(np.float64)
    return bf16_bits_to_f32(raw).astype(np.float64)
