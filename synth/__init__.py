"""Seeded synthetic inputs shared by the tests, ``bench.py`` and ``smoke()``.

This module holds no attention, cache or quantisation arithmetic: it only
draws Gaussian numbers from counter-based generators and rounds them to
bfloat16 as input preparation.  Both the HIP path and the CPU oracle consume
the same bytes produced here.

* ``normal_bf16`` draws on the host with numpy's Philox4x32-10 bit generator
  (Salmon et al., SC'11), keyed by a tuple of integers (seed, tensor id,
  layer, chunk, pass, ...).  Reproducible on any machine.
* ``normal_bf16_device`` draws on the GPU with the counter-based generator of
  ``synth.philox`` (Philox4x32-10 and a normal-quantile table) through its
  device twin ``libsynthfill.so``; ``normal_bf16_philox`` draws the same bits
  on the host, so any device draw can be regenerated from its key.  Used where
  host generation would be too slow (30-layer rollouts, bench inputs).
"""

import hashlib
import struct

import numpy as np

from . import configs  # noqa: F401


def key64(*parts) -> int:
    """Deterministic 63-bit key from a tuple of integers."""
    data = b"".join(struct.pack("<q", int(p)) for p in parts)
    return int.from_bytes(hashlib.blake2b(data, digest_size=8).digest(), "little") >> 1


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even) as input preparation; uint16 bits."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_f32(shape, sigma, *key) -> np.ndarray:
    """float32 N(0, sigma^2) drawn with Philox keyed by ``key``."""
    rng = np.random.Generator(np.random.Philox(key=key64(*key)))
    return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(sigma)).astype(np.float32)


def normal_bf16(shape, sigma, *key) -> np.ndarray:
    """bf16 bits (uint16) of N(0, sigma^2) drawn in float32 then rounded."""
    return f32_to_bf16_bits(normal_f32(shape, sigma, *key))


def normal_bf16_philox(shape, sigma, *key) -> np.ndarray:
    """bf16 bits (uint16) of the counter-based generator's N(0, sigma^2) draws for key
    (the host twin of normal_bf16_device: the same bits)."""
    from . import philox
    return philox.normal_bf16(shape, sigma, key64(*key))


def normal_bf16_device(shape, sigma, *key, device="cuda"):
    """torch.bfloat16 tensor of N(0, sigma^2) drawn on the device by the counter-based
    generator (bit-identical to normal_bf16_philox of the same key)."""
    from . import device as _dev
    return _dev.fill_normal_bf16(shape, sigma, key64(*key), device)


def to_device(bits, device="cuda"):
    """uint16 bf16 bits (numpy) -> torch.bfloat16 tensor on ``device``."""
    import torch
    a = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)


def to_bits(t) -> np.ndarray:
    """torch.bfloat16 tensor (any device) -> uint16 bf16 bits on the host."""
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
