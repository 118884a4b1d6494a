"""Counter-based random streams for the synthetic workloads (CPU side).

This module holds no attention or merge arithmetic.  It defines the random
numbers every test and benchmark input is drawn from, so that the CPU oracle
and the GPU path can be fed bit-identical inputs without either side reading
the other's results.  ``synth/csrc/synth.hip`` implements the same definition
on the GPU; the two agree bit for bit (checked by the GPU tests).

Generator: Philox4x32-10, as published by Salmon, Moraes, Dror and Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11).  One call maps a
128-bit counter and a 64-bit key to four 32-bit words through ten rounds of
two 32x32->64 multiplies, with the key bumped by the Weyl constants between
rounds.

Streams.  A stream is named by ``(seed, tag)``: key = (seed, tag).  Element
``i`` (a 64-bit logical index) of a stream is lane ``i % 4`` of block
``i // 4``, and block ``b`` uses counter ``(b mod 2^32, b >> 32, 0, 0)``.  Any
slice of any stream can therefore be regenerated on its own.

Normal deviates come from Box-Muller in float64 on consecutive word pairs
(w0, w1) and (w2, w3) of a block:
    u1 = (w_even + 1) * 2^-32          in (0, 1]
    u2 =  w_odd       * 2^-32          in [0, 1)
    z_even = sqrt(-2 ln u1) * cos(2 pi u2)
    z_odd  = sqrt(-2 ln u1) * sin(2 pi u2)
and are then rounded to float32 (round to nearest even).  Storage types are
reached from that float32 value by one more round-to-nearest-even step.
"""
from __future__ import annotations

import numpy as np

# Philox4x32 multipliers and Weyl key increments (Salmon et al., SC'11).
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
ROUNDS = 10

_MASK32 = np.uint64(0xFFFFFFFF)
TWO_PI = 6.283185307179586  # float64 nearest to 2*pi
INV_2_32 = 2.0 ** -32


def philox4x32(c0, c1, c2, c3, k0: int, k1: int):
    """Philox4x32-10 on arrays of counters; returns four uint32 arrays."""
    c0 = np.asarray(c0, dtype=np.uint64)
    c1 = np.asarray(c1, dtype=np.uint64)
    c2 = np.asarray(c2, dtype=np.uint64)
    c3 = np.asarray(c3, dtype=np.uint64)
    m0 = np.uint64(PHILOX_M0)
    m1 = np.uint64(PHILOX_M1)
    k0 &= 0xFFFFFFFF
    k1 &= 0xFFFFFFFF
    for _ in range(ROUNDS):
        p0 = m0 * c0
        p1 = m1 * c2
        hi0 = p0 >> np.uint64(32)
        lo0 = p0 & _MASK32
        hi1 = p1 >> np.uint64(32)
        lo1 = p1 & _MASK32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(k0), lo1,
                          hi0 ^ c3 ^ np.uint64(k1), lo0)
        k0 = (k0 + PHILOX_W0) & 0xFFFFFFFF
        k1 = (k1 + PHILOX_W1) & 0xFFFFFFFF
    return (c0.astype(np.uint32), c1.astype(np.uint32),
            c2.astype(np.uint32), c3.astype(np.uint32))


def _blocks(seed: int, tag: int, first_block: int, nblocks: int):
    b = np.arange(first_block, first_block + nblocks, dtype=np.uint64)
    zero = np.zeros_like(b)
    return philox4x32(b & _MASK32, b >> np.uint64(32), zero, zero, seed, tag)


def words(seed: int, tag: int, start: int, count: int) -> np.ndarray:
    """Raw uint32 words ``start .. start+count-1`` of stream (seed, tag)."""
    if count <= 0:
        return np.zeros(0, dtype=np.uint32)
    fb = start // 4
    lb = (start + count - 1) // 4
    w = np.stack(_blocks(seed, tag, fb, lb - fb + 1), axis=1).reshape(-1)
    off = start - 4 * fb
    return w[off:off + count]


def normal_f32(seed: int, tag: int, start: int, count: int) -> np.ndarray:
    """float32 standard-normal deviates ``start .. start+count-1``."""
    if count <= 0:
        return np.zeros(0, dtype=np.float32)
    fb = start // 4
    lb = (start + count - 1) // 4
    w0, w1, w2, w3 = _blocks(seed, tag, fb, lb - fb + 1)
    out = np.empty((lb - fb + 1, 4), dtype=np.float32)
    for (we, wo, col) in ((w0, w1, 0), (w2, w3, 2)):
        u1 = (we.astype(np.float64) + 1.0) * INV_2_32
        u2 = wo.astype(np.float64) * INV_2_32
        rad = np.sqrt(-2.0 * np.log(u1))
        ang = TWO_PI * u2
        out[:, col] = (rad * np.cos(ang)).astype(np.float32)
        out[:, col + 1] = (rad * np.sin(ang)).astype(np.float32)
    out = out.reshape(-1)
    off = start - 4 * fb
    return out[off:off + count]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest even); returns uint16 bit patterns.

    Inputs here are finite; NaN handling is not needed by the generators."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to(x_f32: np.ndarray, dtype: str):
    """Round float32 values to the storage dtype.

    Returns (bits, values): ``bits`` is the raw storage (uint16 for bf16,
    float16 for fp16, float32 for fp32) and ``values`` the same numbers as
    float32 (exact: every bf16/fp16 value is a float32 value)."""
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x_f32)
        return bits, bf16_bits_to_f32(bits)
    if dtype == "fp16":
        h = np.asarray(x_f32, dtype=np.float32).astype(np.float16)
        return h, h.astype(np.float32)
    if dtype == "fp32":
        f = np.asarray(x_f32, dtype=np.float32)
        return f, f
    raise ValueError(dtype)


def uniform_int(seed: int, tag: int, start: int, count: int, n: int) -> np.ndarray:
    """Integers in [0, n) from words: floor(w * n / 2^32) (multiply-shift)."""
    w = words(seed, tag, start, count).astype(np.uint64)
    return ((w * np.uint64(n)) >> np.uint64(32)).astype(np.int64)


def bernoulli(seed: int, tag: int, start: int, count: int, p: float) -> np.ndarray:
    """True with probability p: word < ceil(p * 2^32)."""
    thr = int(np.ceil(p * 2.0 ** 32))
    return words(seed, tag, start, count).astype(np.uint64) < np.uint64(thr)
