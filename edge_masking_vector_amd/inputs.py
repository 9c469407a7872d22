"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds random numbers only: none of the maps, copies or reductions.  Inputs are drawn
once on the host and the same array feeds both the CPU oracle and the device copy, so parity never
depends on how the numbers were drawn.

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
OOPSLA 2014; the 64-bit finaliser constants as published by Vigna), evaluated in closed form for
element k of a stream: state_k = seed + (k + 1) * 0x9E3779B97F4A7C15 (mod 2**64).

Derived draws, all exactly reproducible:
  * u32 = upper 32 bits of the 64-bit output;
  * U[0,1) = (u32 >> 8) * 2**-24, so every value is a multiple of 2**-24 and none is subnormal;
  * U[lo,hi) = lo + (hi - lo) * U[0,1), evaluated in double and rounded once to f32;
  * N(0,1) = Box-Muller in double on two U draws (the first shifted off zero), rounded to f32.
"""
import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(seed: int, n: int, offset: int = 0) -> np.ndarray:
    """Outputs offset .. offset+n-1 of the SplitMix64 stream started at `seed` (uint64)."""
    k = np.arange(offset + 1, offset + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + k * _GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def u32(seed: int, n: int, offset: int = 0) -> np.ndarray:
    return (splitmix64(seed, n, offset) >> np.uint64(32)).astype(np.uint32)


def u24(seed: int, n: int, offset: int = 0) -> np.ndarray:
    """The 24-bit integers k = u32 >> 8 behind every U[0,1) draw."""
    return (u32(seed, n, offset) >> np.uint32(8)).astype(np.int64)


def uniform(seed: int, n: int, lo: float = 0.0, hi: float = 1.0) -> np.ndarray:
    u = u24(seed, n).astype(np.float64) * 2.0 ** -24
    return (lo + (hi - lo) * u).astype(np.float32)


def normal(seed: int, n: int) -> np.ndarray:
    k = u24(seed, 2 * n)
    u1 = (k[0::2].astype(np.float64) + 1.0) * 2.0 ** -24   # (0, 1]
    u2 = k[1::2].astype(np.float64) * 2.0 ** -24           # [0, 1)
    return (np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)).astype(np.float32)


def integers(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    """Integers in [lo, hi) as f32 (exact while |value| < 2**24)."""
    k = u32(seed, n).astype(np.int64)
    return (lo + k % (hi - lo)).astype(np.float32)


def matrix(values: np.ndarray, M: int, N: int, ld: int, pad: float = 0.0) -> np.ndarray:
    """Lay M*N values out as a flat row-major buffer with row stride ld (padding = `pad`)."""
    buf = np.full(max(M, 0) * ld if M > 0 else 0, pad, np.float32)
    if M > 0 and N > 0:
        buf.reshape(M, ld)[:, :N] = values.reshape(M, N)
    return buf


# ---- the workloads' synthetic inputs -------------------------------------------------------------
# Shapes follow the workloads the pages describe: the 1M-element a*2+1 map, a 4096 x 4096 matrix
# walked by rows and by columns, a ragged 4100 x 1000 tensor under 64 x 64 tiles and a ragged
# 8192 x 1000 score matrix under 64-column tiles.

def map1d_input(n: int = 1 << 20, seed: int = 1) -> np.ndarray:
    """a ~ U[-1, 1): a = (k - 2**23) * 2**-23 exactly, k a 24-bit integer."""
    return uniform(seed, n, -1.0, 1.0)


def scale_input(M: int = 4096, N: int = 4096, seed: int = 2) -> np.ndarray:
    """X ~ N(0, 1), row-major, ld = N."""
    return normal(seed, M * N)


def ragged_input(M: int = 4100, N: int = 1000, seed: int = 3) -> np.ndarray:
    """X ~ U[-8, 8), row-major, ld = N."""
    return uniform(seed, M * N, -8.0, 8.0)


def colrow_input(M: int = 4096, N: int = 4096, seed: int = 4) -> np.ndarray:
    """X ~ U[0, 1), row-major, ld = N."""
    return uniform(seed, M * N, 0.0, 1.0)


def scores_input(M: int = 8192, N: int = 1000, seed: int = 5) -> np.ndarray:
    """S ~ U[-10, -1), row-major, ld = N: every score negative."""
    return uniform(seed, M * N, -10.0, -1.0)
