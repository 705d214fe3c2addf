"""Counter-based 32-bit hashing used by every generator in this package.

Values are carried in int64 tensors holding numbers in [0, 2^32). Each
multiplier is below 2^31, so no product overflows int64 and the integer results
are identical on every torch device. ``mix32`` is a xorshift-multiply
finaliser in the style of the public "hash prospector" family.
"""

import torch

M32 = 0xFFFFFFFF
_C1 = 0x21F0AAAD
_C2 = 0x735A2D97


def mix32_int(x: int) -> int:
    """Python-int version of :func:`mix32` (for scalar keys)."""
    x &= M32
    x ^= x >> 16
    x = (x * _C1) & M32
    x ^= x >> 15
    x = (x * _C2) & M32
    x ^= x >> 15
    return x


def mix32(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 16)
    x = (x * _C1) & M32
    x = x ^ (x >> 15)
    x = (x * _C2) & M32
    x = x ^ (x >> 15)
    return x


def stream_key(seed: int, stream: int) -> int:
    """A 32-bit key for (seed, stream)."""
    return mix32_int(mix32_int(seed * 0x9E3779B1 + 0x632BE5AB) ^ mix32_int(stream + 0x85EBCA6B))


def hash_range(seed: int, stream: int, start: int, count: int, device="cpu") -> torch.Tensor:
    """32-bit hashes of element indices [start, start+count) of (seed, stream)."""
    key = stream_key(seed, stream)
    key2 = mix32_int(key ^ 0x27D4EB2F)
    i = torch.arange(start, start + count, dtype=torch.int64, device=device)
    lo = i & M32
    hi = i >> 32
    h = mix32(lo ^ key)
    h = mix32(h ^ ((hi + key2) & M32))
    return h
