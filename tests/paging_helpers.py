"""Test-local builders of paged layouts from logically contiguous K/V.

These scatter with numpy fancy indexing and are written independently of the
oracle's gather, so a gather mistake in the oracle shows up as a mismatch
against attention on the unpaged data.
"""

import numpy as np


def paginate(logical, block_size, num_blocks, rng, fill=0.0):
    """logical: list of [L_i, Hkv, D] float arrays. Returns (cache, tables)
    with blocks taken in a random physical order."""
    Hkv, D = logical[0].shape[1], logical[0].shape[2]
    cache = np.full((num_blocks, block_size, Hkv, D), fill, dtype=logical[0].dtype)
    perm = rng.permutation(num_blocks)
    nxt = 0
    max_blocks = max(-(-x.shape[0] // block_size) for x in logical)
    tables = np.full((len(logical), max(max_blocks, 1)), -1, dtype=np.int32)
    for i, seq in enumerate(logical):
        L = seq.shape[0]
        nb = -(-L // block_size)
        ids = perm[nxt:nxt + nb]
        nxt += nb
        tables[i, :nb] = ids
        padded = np.full((nb * block_size, Hkv, D), fill, dtype=seq.dtype)
        padded[:L] = seq
        cache[ids] = padded.reshape(nb, block_size, Hkv, D)
    return cache, tables


def paginate_kv(ks, vs, block_size, num_blocks, rng, fill=0.0):
    """K and V sequences placed into blocks through the same tables."""
    kc, tables = paginate(ks, block_size, num_blocks, rng, fill)
    vc = np.full_like(kc, fill)
    for i, v in enumerate(vs):
        nb = -(-v.shape[0] // block_size)
        padded = np.full((nb * block_size,) + v.shape[1:], fill, dtype=v.dtype)
        padded[:v.shape[0]] = v
        vc[tables[i, :nb]] = padded.reshape((nb, block_size) + v.shape[1:])
    return kc, vc, tables
