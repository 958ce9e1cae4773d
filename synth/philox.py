"""Counter-based Gaussian input generator with a device twin (input preparation only).

One generator, written twice from its published definition: here in numpy for the
oracle's side, and in ``synth/csrc/fill.hip`` for filling device tensors, so that any
device draw can be regenerated on the host bit for bit.  No attention, cache or
quantisation arithmetic lives here.

Definition
----------
* Philox4x32-10 (J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel random
  numbers: as easy as 1, 2, 3", SC'11): a 4 x 32-bit counter and a 2 x 32-bit key; each
  of 10 rounds multiplies counter words 0 and 2 by 0xD2511F53 and 0xCD9E8D57 and
  recombines the 64-bit products' halves with words 1 and 3 and the key, then adds
  0x9E3779B9 and 0xBB67AE85 to the key words.
* Element i of a tensor takes 32-bit word i mod 4 of the block with counter
  (i div 4 mod 2^32, i div 2^34, 0, 0) under key (key64 mod 2^32, key64 div 2^32), where
  key64 is ``synth.key64`` of the caller's integer tuple.
* The word's top 16 bits index a table of the 65 536 standard-normal quantiles
  Phi^-1((j + 1/2) / 65536), computed in float64 and stored as float32; the value is
  float32(table[j] * sigma) rounded to bf16 (nearest, ties to even).
"""

import numpy as np

M0, M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
W0, W1 = 0x9E3779B9, 0xBB67AE85
_MASK = np.uint64(0xFFFFFFFF)
TABLE_SIZE = 65536


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32-10 of counters (c0, c1, c2, c3) (uint32 arrays or scalars) under key
    (k0, k1) (ints); returns the four output words as uint32 arrays."""
    c = [np.asarray(x, dtype=np.uint64) & _MASK for x in (c0, c1, c2, c3)]
    k0, k1 = int(k0) & 0xFFFFFFFF, int(k1) & 0xFFFFFFFF
    for _ in range(10):
        p0 = M0 * c[0]                      # 32 x 32 -> 64-bit product, exact in uint64
        p1 = M1 * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK
        c = [hi1 ^ c[1] ^ np.uint64(k0), lo1, hi0 ^ c[3] ^ np.uint64(k1), lo0]
        k0 = (k0 + W0) & 0xFFFFFFFF
        k1 = (k1 + W1) & 0xFFFFFFFF
    return [x.astype(np.uint32) for x in c]


_table = None


def normal_table() -> np.ndarray:
    """float32 [65536]: Phi^-1((j + 1/2) / 65536), evaluated in float64."""
    global _table
    if _table is None:
        from scipy.special import ndtri
        j = np.arange(TABLE_SIZE, dtype=np.float64)
        _table = ndtri((j + 0.5) / TABLE_SIZE).astype(np.float32)
    return _table


def words(n: int, key64: int) -> np.ndarray:
    """The 32-bit Philox word of each of n elements (element i: word i mod 4 of block i div 4)."""
    nb = (n + 3) // 4
    b = np.arange(nb, dtype=np.uint64)
    out = philox4x32_10(b & _MASK, b >> np.uint64(32), 0, 0, key64 & 0xFFFFFFFF, key64 >> 32)
    return np.stack(out, axis=1).reshape(-1)[:n]


def _bf16_rne(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def normal_bf16(shape, sigma, key64: int) -> np.ndarray:
    """bf16 bits (uint16) of N(0, sigma^2) draws of the generator above."""
    n = int(np.prod(shape))
    j = words(n, key64) >> np.uint32(16)
    vals = normal_table()[j] * np.float32(sigma)           # float32 product, one rounding
    return _bf16_rne(vals).reshape(shape)
