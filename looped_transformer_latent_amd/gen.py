"""Seeded, counter-based synthetic input generator (host side).

This module holds random-number generation only -- none of the attention,
encoder or decoder arithmetic.  It is the one piece shared by the oracle tests
and the GPU tests: both draw their inputs from it.  ``csrc/gen/lla_gen.hip`` implements
the same generator on the device (for inputs too large to upload, such as a
100 GB latent pool), and tests check that both give identical bits.

Definition (counter-based, so any element can be regenerated on its own):

* 64-bit mixer: the SplitMix64 output function (Steele, Lea & Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014):
  ``z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27; z *= 0x94D049BB133111EB;
  z ^= z >> 31`` (all mod 2**64).
* key(seed, stream) = mix(seed * 0x9E3779B97F4A7C15 + stream * 0xD1B54A32D192ED03).
* word(seed, stream, i) = mix(key + (i + 1) * 0x9E3779B97F4A7C15): 64 random bits
  for element i of the tensor named by ``stream``.
* Approximately standard normal value: split the word into four 16-bit
  unsigned integers, sum them (Irwin-Hall with 4 terms), subtract the mean
  131070 and convert to fp32 (exact), then multiply in fp32 by
  ``mult = fp32(1/sqrt((65536**2 - 1)/3)) * fp32(scale)`` (one rounding on each
  side, computed on the host and passed to the device as-is).  The result has
  mean 0 and standard deviation ``scale`` and lies within +-3.46 * scale.
* bf16 storage: round the fp32 value to nearest-even on its bit pattern.
"""
from __future__ import annotations

import numpy as np

MASK64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15
STREAM_MULT = 0xD1B54A32D192ED03
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
IH_MEAN = 131070
IH_INV_STD = np.float32(1.0 / np.sqrt((65536.0 ** 2 - 1.0) / 3.0))


def _mix_int(z: int) -> int:
    z &= MASK64
    z ^= z >> 30
    z = (z * _M1) & MASK64
    z ^= z >> 27
    z = (z * _M2) & MASK64
    z ^= z >> 31
    return z


def _mix_np(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.uint64, copy=True)
    z ^= z >> np.uint64(30)
    z *= np.uint64(_M1)
    z ^= z >> np.uint64(27)
    z *= np.uint64(_M2)
    z ^= z >> np.uint64(31)
    return z


def key(seed: int, stream: int) -> int:
    return _mix_int((seed * GOLDEN + stream * STREAM_MULT) & MASK64)


def words(seed: int, stream: int, idx: np.ndarray) -> np.ndarray:
    """64-bit words for element indices ``idx`` (any integer array)."""
    k = np.uint64(key(seed, stream))
    i = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = k + (i + np.uint64(1)) * np.uint64(GOLDEN)
    return _mix_np(z)


def mult_for(scale: float) -> np.float32:
    """The single fp32 multiplier applied to the centred Irwin-Hall sum."""
    return np.float32(IH_INV_STD * np.float32(scale))


def normal_f32(seed: int, stream: int, idx, scale: float = 1.0) -> np.ndarray:
    """fp32 values of elements ``idx`` (an int array, or an int n for 0..n-1)."""
    if np.isscalar(idx):
        idx = np.arange(int(idx), dtype=np.uint64)
    w = words(seed, stream, idx)
    s = ((w & np.uint64(0xFFFF)) + ((w >> np.uint64(16)) & np.uint64(0xFFFF)) +
         ((w >> np.uint64(32)) & np.uint64(0xFFFF)) + (w >> np.uint64(48)))
    centred = (s.astype(np.int64) - IH_MEAN).astype(np.float32)  # exact (|v| < 2**18)
    return (centred * mult_for(scale)).astype(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    r = r.astype(np.uint16)
    r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal(seed: int, stream: int, shape, scale: float = 1.0, dtype: str = "bf16",
           offset: int = 0) -> np.ndarray:
    """A tensor of the given shape: bf16 bit patterns (uint16) or fp32 values."""
    n = int(np.prod(shape))
    v = normal_f32(seed, stream, np.arange(offset, offset + n, dtype=np.uint64), scale)
    v = v.reshape(shape)
    return f32_to_bf16_bits(v) if dtype == "bf16" else v


def storage_to_f64(a: np.ndarray) -> np.ndarray:
    """Exact float64 values of a stored tensor (uint16 = bf16 bits, or fp32)."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def shuffled_page_table(seed: int, batch: int, pages_per_seq: int, num_pages: int | None = None
                        ) -> np.ndarray:
    """[batch][pages_per_seq] int32: a seeded Fisher-Yates permutation of the
    physical pages (numpy's PCG64 generator), dealt out row by row."""
    total = batch * pages_per_seq if num_pages is None else num_pages
    perm = np.random.default_rng(seed).permutation(total).astype(np.int32)
    return np.ascontiguousarray(perm[: batch * pages_per_seq].reshape(batch, pages_per_seq))


def identity_page_table(batch: int, pages_per_seq: int) -> np.ndarray:
    return np.arange(batch * pages_per_seq, dtype=np.int32).reshape(batch, pages_per_seq)
