"""One decode step on the GPU, as the benchmark times it.

A step appends the new token's K/V into its slot (pa_reshape_and_cache),
then runs paged decode attention over every sequence's context, the new
token included (append first, then attend: "vLLM PagedAttention深度解析与
工程实践" §二). Attention uses the split path (partitions + log-sum-exp
merge) with the workload's partition size, or the single-launch path when
`split` is False.
"""

import numpy as np
import torch

from . import lib as palib

_TORCH = {"f16": torch.float16, "bf16": torch.bfloat16}


def to_device_tensor(arr, dtype, device):
    """Host array (fp16, or bf16 as uint16 bits) -> GPU tensor of `dtype`."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    elif dtype == "f16":
        t = torch.from_numpy(np.ascontiguousarray(arr))
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.to(device)


def to_host_bits(t):
    """GPU fp16/bf16 tensor -> host uint16 bit patterns."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def to_host_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


class DeviceBatch:
    """GPU copies of a workloads.Batch plus the step's output buffers."""

    def __init__(self, batch, device="cuda", out_dtype=None, split=True, partition_size=None,
                 shared_prefix=False, fused=False):
        w = batch.workload
        self.batch = batch
        self.device = device
        dt = w.dtype
        self.query = to_device_tensor(batch.query, dt, device)
        self.key_cache = to_device_tensor(batch.key_cache, dt, device)
        self.value_cache = to_device_tensor(batch.value_cache, dt, device)
        self.new_key = to_device_tensor(batch.new_key, dt, device)
        self.new_value = to_device_tensor(batch.new_value, dt, device)
        self.block_tables = torch.from_numpy(batch.block_tables).to(device)
        self.context_lens = torch.from_numpy(batch.context_lens).to(device)
        self.slot_mapping = torch.from_numpy(batch.slot_mapping).to(device)
        self.scale = batch.scale
        self.split = split
        self.partition_size = partition_size or w.partition_size
        # shared-prefix launches when every sequence starts with the same
        # blocks and the prefix is a whole number of partitions
        pt = w.shared_prefix_tokens
        self.prefix_tokens = pt if (shared_prefix and split and pt > 0
                                    and pt % self.partition_size == 0) else 0
        # one launch pair per step: the scatter runs inside the partition launch
        self.fused = bool(fused and split and not self.prefix_tokens)
        B, Hq, D = self.query.shape
        od = out_dtype if out_dtype is not None else self.query.dtype
        self.out = torch.empty((B, Hq, D), dtype=od, device=device)
        self.workspace = None
        if split:
            self.workspace = palib.make_workspace(B, Hq, D, self.block_tables.shape[1],
                                                  w.block_size, self.partition_size, device)

    def write_cache(self):
        palib.reshape_and_cache(self.new_key, self.new_value, self.key_cache, self.value_cache,
                                self.slot_mapping)

    def partitions(self):
        """Split path, partition launches only (see lib.decode_partitions)."""
        if self.fused:
            palib.decode_partitions_append(
                self.query, self.key_cache, self.value_cache, self.block_tables, self.context_lens,
                self.new_key, self.new_value, self.slot_mapping, self.scale, self.partition_size,
                workspace=self.workspace, out=self.out)
            return
        if self.prefix_tokens:
            palib.decode_partitions_shared_prefix(
                self.query, self.key_cache, self.value_cache, self.block_tables, self.context_lens,
                self.scale, self.prefix_tokens, self.partition_size, workspace=self.workspace,
                out=self.out)
            return
        palib.decode_partitions(self.query, self.key_cache, self.value_cache, self.block_tables,
                                self.context_lens, self.scale, self.partition_size,
                                workspace=self.workspace, out=self.out)

    def merge(self):
        """Split path, second launch: log-sum-exp merge over the workspace."""
        B, Hq, D = self.query.shape
        pm, ps, po = palib.workspace_views(self.workspace, B, Hq, D, self.block_tables.shape[1],
                                           self.key_cache.shape[1], self.partition_size)
        palib.lse_merge(po, pm, ps, self.context_lens, self.partition_size, out=self.out)

    def attend(self):
        if self.split and self.prefix_tokens:
            palib.decode_split_shared_prefix(
                self.query, self.key_cache, self.value_cache, self.block_tables, self.context_lens,
                self.scale, self.prefix_tokens, self.partition_size, workspace=self.workspace,
                out=self.out)
        elif self.split:
            palib.decode_split(self.query, self.key_cache, self.value_cache, self.block_tables,
                               self.context_lens, self.scale, self.partition_size,
                               workspace=self.workspace, out=self.out)
        else:
            palib.decode(self.query, self.key_cache, self.value_cache, self.block_tables,
                         self.context_lens, self.scale, out=self.out)
        return self.out

    def step(self):
        if self.fused:
            palib.decode_split_append(
                self.query, self.key_cache, self.value_cache, self.block_tables, self.context_lens,
                self.new_key, self.new_value, self.slot_mapping, self.scale, self.partition_size,
                workspace=self.workspace, out=self.out)
            return self.out
        self.write_cache()
        return self.attend()


class RotatedBatch(DeviceBatch):
    """A copy of a DeviceBatch whose whole pool is permuted: block b of the
    source is block perm[b] here, for every one of the pool's blocks.

    The logical content of every sequence is unchanged, so the outputs are
    bit-identical to the source batch's, and the blocks in use stay spread
    over a pool of the workload's full size (the same address range and
    page spread as the source); timing loops cycle through several such
    copies so that no step finds the previous step's cache blocks in the
    GPU's last-level cache.
    """

    def __init__(self, src, seed):  # noqa: D401 - no DeviceBatch.__init__
        self.batch = src.batch
        self.device = src.device
        self.query, self.new_key, self.new_value = src.query, src.new_key, src.new_value
        self.context_lens = src.context_lens
        self.scale = src.scale
        self.split = src.split
        self.partition_size = src.partition_size
        self.prefix_tokens = src.prefix_tokens
        self.fused = src.fused
        NB, BS = src.key_cache.shape[0], src.key_cache.shape[1]
        g = torch.Generator(device="cpu").manual_seed(seed)
        perm = torch.randperm(NB, generator=g).to(src.device)
        self.key_cache = torch.empty_like(src.key_cache)
        self.value_cache = torch.empty_like(src.value_cache)
        self.key_cache[perm] = src.key_cache
        self.value_cache[perm] = src.value_cache
        bt = src.block_tables
        # table entries outside the pool (padding) keep their value
        ok = (bt >= 0) & (bt < NB)
        self.block_tables = torch.where(ok, perm[bt.clamp(0, NB - 1).long()].to(torch.int32), bt)
        sm = src.slot_mapping
        blk = torch.div(sm.clamp(min=0), BS, rounding_mode="floor")
        sok = (sm >= 0) & (blk < NB)
        self.slot_mapping = torch.where(sok, perm[blk.clamp(max=NB - 1)] * BS + sm.clamp(min=0) % BS,
                                        sm)
        self.out = torch.empty_like(src.out)
        self.workspace = None if src.workspace is None else torch.empty_like(src.workspace)


class DevicePrefill:
    """GPU copies of a workloads.PrefillBatch. A step stores the new tokens'
    K/V into their slots (pa_reshape_and_cache), then runs pa_prefill: the
    new tokens attend over the cached prompt blocks and themselves, causally
    (lqnn.cn/news/170268 §3.4: prefill from the first missing position on
    top of the hit blocks). With shared_prefix_tokens set (the cached
    prompt's tokens, which every table starts with), the attention is
    pa_prefill_shared_prefix, which reads the shared blocks once per group
    of rows of all requests."""

    def __init__(self, batch, device="cuda", out_dtype=None, shared_prefix_tokens=None):
        self.shared_prefix_tokens = shared_prefix_tokens
        dt = batch.workload.dtype
        self.batch = batch
        self.query = to_device_tensor(batch.query, dt, device)
        self.key_cache = to_device_tensor(batch.key_cache, dt, device)
        self.value_cache = to_device_tensor(batch.value_cache, dt, device)
        self.new_key = to_device_tensor(batch.new_key, dt, device)
        self.new_value = to_device_tensor(batch.new_value, dt, device)
        self.block_tables = torch.from_numpy(batch.block_tables).to(device)
        self.context_lens = torch.from_numpy(batch.context_lens).to(device)
        self.query_start = torch.from_numpy(batch.query_start).to(device)
        self.slot_mapping = torch.from_numpy(batch.slot_mapping).to(device)
        self.scale = batch.scale
        self.max_query_len = batch.max_query_len
        od = out_dtype if out_dtype is not None else self.query.dtype
        self.out = torch.empty(tuple(self.query.shape), dtype=od, device=device)

    def write_cache(self):
        palib.reshape_and_cache(self.new_key, self.new_value, self.key_cache, self.value_cache,
                                self.slot_mapping)

    def attend(self):
        return palib.prefill(self.query, self.key_cache, self.value_cache, self.block_tables,
                             self.context_lens, self.query_start, self.scale, self.max_query_len,
                             out=self.out, shared_prefix_tokens=self.shared_prefix_tokens)

    def step(self):
        self.write_cache()
        return self.attend()
