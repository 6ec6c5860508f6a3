"""Run the fp64 oracle over whole batches in a thread pool (test harness).

The oracle itself is unchanged: these helpers only cut a batch into
independent pieces - one (sequence, kv head) for decode, one request for
prefill - call the oracle on each with the caches' views of that piece, and
put the results back in place. numpy releases the interpreter lock in its
array loops and matrix products, so the pieces run side by side on the host's
cores and full-size batches are checked in seconds to minutes.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle


def workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def decode_all(query, key_cache, value_cache, block_tables, context_lens, scale, dtype,
               pieces=None):
    """oracle.decode of every (sequence, kv head) pair, or of the listed
    (sequence, kv head) pairs; returns float64 [B, Hq, D] (unlisted pairs 0)."""
    B, Hq, D = query.shape
    Hkv = key_cache.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    if pieces is None:
        pieces = [(i, kv) for i in range(B) for kv in range(Hkv)]

    def one(piece):
        i, kv = piece
        qh = slice(kv * G, (kv + 1) * G)
        out[i, qh] = oracle.decode(query[i:i + 1, qh], key_cache[:, :, kv:kv + 1],
                                   value_cache[:, :, kv:kv + 1], block_tables[i:i + 1],
                                   context_lens[i:i + 1], scale, dtype)[0]

    # longest contexts first, so the pool does not end on one long piece
    order = sorted(pieces, key=lambda p: -int(context_lens[p[0]]))
    with ThreadPoolExecutor(workers()) as ex:
        list(ex.map(one, order))
    return out


def prefill_all(query, key_cache, value_cache, block_tables, context_lens, query_start, scale,
                dtype, requests=None):
    """oracle.prefill of every request (or the listed ones), one (request,
    kv head) pair per task; returns float64 [T, Hq, D] (rows of unlisted
    requests 0)."""
    T, Hq, D = query.shape
    Hkv = key_cache.shape[2]
    G = Hq // Hkv
    out = np.zeros((T, Hq, D), dtype=np.float64)
    qs = np.asarray(query_start)
    if requests is None:
        requests = range(len(context_lens))

    def one(piece):
        i, kv = piece
        a, b = int(qs[i]), int(qs[i + 1])
        if b == a:
            return
        qh = slice(kv * G, (kv + 1) * G)
        out[a:b, qh] = oracle.prefill(query[a:b, qh], key_cache[:, :, kv:kv + 1],
                                      value_cache[:, :, kv:kv + 1], block_tables[i:i + 1],
                                      context_lens[i:i + 1], np.array([0, b - a], dtype=np.int32),
                                      scale, dtype)

    pieces = [(i, kv) for i in requests for kv in range(Hkv)]
    pieces.sort(key=lambda p: -int(qs[p[0] + 1] - qs[p[0]]) * int(context_lens[p[0]]))
    with ThreadPoolExecutor(workers()) as ex:
        list(ex.map(one, pieces))
    return out
