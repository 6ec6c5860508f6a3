"""pa_decode_split_noalloc - the split path whose partial rows go to the
library's own scratch array instead of a caller workspace (for callers that
cannot allocate) - gives pa_decode_split's outputs bit for bit, call after
call on one GPU, the later calls smaller than the earlier ones (the array
keeps the previous call's rows)."""

import os

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_138_amd import lib as palib
from paged_kv_cache_138_amd import workloads as W
from paged_kv_cache_138_amd.pipeline import DeviceBatch, to_host_f64

pytestmark = pytest.mark.gpu

ATOL = 2e-3

# (workload fields, partition size, output dtype), run in this order: each
# call after the first is smaller than the one before it
CALLS = [
    # 64 x 16 rows x 32 partitions of 128: a 17 MB layout, over half the array
    (dict(num_seqs=64, num_heads=16, num_kv_heads=2, head_dim=128, dtype="bf16", block_size=16,
          num_blocks=2560, max_blocks_per_seq=256, lens="uniform:1:600"), 128, torch.float32),
    (dict(num_seqs=12, num_heads=8, num_kv_heads=8, head_dim=128, dtype="f16", block_size=16,
          num_blocks=640, max_blocks_per_seq=64, lens="uniform:1:1000"), 256, None),
    (dict(num_seqs=3, num_heads=4, num_kv_heads=4, head_dim=64, dtype="f16", block_size=32,
          num_blocks=64, max_blocks_per_seq=16, lens="uniform:1:500"), 64, torch.float32),
]


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def test_noalloc_split_matches_split_call_after_call():
    assert os.path.exists(palib.LIB_PATH)
    palib.load()
    sizes = []
    for n, (kw, P, od) in enumerate(CALLS):
        w = W.custom_workload("noalloc%d" % n, **kw)
        print("noalloc call %d: %s P=%d out=%s" % (n, kw, P, od), flush=True)
        b = W.make_batch(w, seed=50 + n)
        db = DeviceBatch(b, out_dtype=od, split=True, partition_size=P)
        db.write_cache()
        B, Hq, D = db.query.shape
        ws_bytes = palib.decode_split_workspace_bytes(B, Hq, D, db.block_tables.shape[1],
                                                      w.block_size, P)
        assert ws_bytes <= palib.NOALLOC_MAX_WORKSPACE
        sizes.append(ws_bytes)
        ref = palib.decode_split(db.query, db.key_cache, db.value_cache, db.block_tables,
                                 db.context_lens, db.scale, P, workspace=db.workspace,
                                 out=torch.empty_like(db.out))
        got = torch.full_like(db.out, float("nan"))
        palib.decode_split_noalloc(db.query, db.key_cache, db.value_cache, db.block_tables,
                                   db.context_lens, db.scale, P, out=got)
        torch.cuda.synchronize()
        assert torch.equal(_bits(got), _bits(ref)), "call %d differs from pa_decode_split" % n
        # and both meet the oracle's bar
        kc, vc = oracle.reshape_and_cache(b.new_key, b.new_value, b.key_cache, b.value_cache,
                                          b.slot_mapping)
        exp = oracle.decode(b.query, kc, vc, b.block_tables, b.context_lens, b.scale, b.dtype)
        err = np.abs(to_host_f64(got) - exp)
        bound = ATOL if od == torch.float32 else ATOL + 2.0 ** (
            np.floor(np.log2(np.maximum(np.abs(exp), 2.0 ** -14))) - 10)
        assert (err <= bound).all(), "call %d: max err %.3g" % (n, err.max())
    assert sizes == sorted(sizes, reverse=True) and len(set(sizes)) == len(sizes)


def test_noalloc_split_refuses_a_workspace_past_its_array():
    palib.load()
    w = W.custom_workload("noalloc_big", num_seqs=128, num_heads=64, num_kv_heads=8,
                          head_dim=128, dtype="bf16", block_size=16, num_blocks=256,
                          max_blocks_per_seq=512, lens="uniform:1:16")
    b = W.make_batch(w, seed=3)
    db = DeviceBatch(b, out_dtype=torch.float32, split=False)
    with pytest.raises(palib.PaError) as e:
        palib.decode_split_noalloc(db.query, db.key_cache, db.value_cache, db.block_tables,
                                   db.context_lens, db.scale, 512, out=db.out)
    assert e.value.status == 5 and "scratch" in str(e.value)
