"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random numbers; it holds none of the method's
arithmetic.  Every tensor has a name; its values come from NumPy's PCG64
seeded by ``SeedSequence(seed, spawn_key=(crc32(name), chunk))`` for chunks of
2**24 elements, so any tensor can be regenerated alone, in parallel, and the
same name always gives the same values.

Activations handed to the device are bfloat16.  ``bf16_exact`` clears the low
16 bits of fp32 draws (a truncation, so the values are exactly representable
in bfloat16 and both sides receive the very same numbers).
"""
import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

SEED = 1234
_CHUNK = 1 << 24
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        _POOL = ThreadPoolExecutor(max_workers=8)
    return _POOL


def _gen(name, chunk, seed):
    key = (zlib.crc32(name.encode("utf-8")), chunk)
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def _fill(name, shape, seed, draw):
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.float32)
    chunks = [(c, c * _CHUNK, min(n, (c + 1) * _CHUNK)) for c in range((n + _CHUNK - 1) // _CHUNK)]

    def work(item):
        c, lo, hi = item
        out[lo:hi] = draw(_gen(name, c, seed), hi - lo)

    if len(chunks) > 1:
        list(_pool().map(work, chunks))
    elif chunks:
        work(chunks[0])
    return out.reshape(shape)


def normal(name, shape, std=1.0, seed=SEED):
    """fp32 draws from N(0, std^2) (std is the standard deviation)."""
    std = np.float32(std)
    return _fill(name, tuple(shape), seed,
                 lambda g, m: g.standard_normal(m, dtype=np.float32) * std)


def uniform(name, shape, lo, hi, seed=SEED):
    """fp32 draws from U[lo, hi)."""
    lo32, span = np.float32(lo), np.float32(hi - lo)
    return _fill(name, tuple(shape), seed,
                 lambda g, m: g.random(m, dtype=np.float32) * span + lo32)


def token_ids(name, shape, vocab, seed=SEED):
    """int32 token ids drawn uniformly from [0, vocab)."""
    g = _gen(name, 0, seed)
    return g.integers(0, vocab, size=shape, dtype=np.int64).astype(np.int32)


def preference_pairs(name, pairs, seq, vocab, prompt_len, seed=SEED):
    """int32 ids [2 * pairs, seq] for preference training: rows 0..pairs-1 are
    the chosen sequences, rows pairs..2*pairs-1 the rejected ones; pair p
    shares its first prompt_len tokens (the prompt) and draws the two
    responses independently."""
    prompt = token_ids(name + ".prompt", (pairs, prompt_len), vocab, seed)
    resp = token_ids(name + ".response", (2 * pairs, seq - prompt_len), vocab, seed)
    ids = np.concatenate([np.concatenate([prompt, prompt]), resp], axis=1)
    return np.ascontiguousarray(ids, dtype=np.int32)


def bf16_exact(x):
    """Clear the low 16 bits: returns (fp32 values, uint16 bfloat16 bits)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
    return u.view(np.float32), (u >> np.uint32(16)).astype(np.uint16)
