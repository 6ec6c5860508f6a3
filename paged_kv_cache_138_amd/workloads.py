"""Seeded synthetic decode batches and the host-side block bookkeeping.

This module builds inputs only: block tables popped from a shuffled free
list, context lengths, query / cache contents and the new token's K/V with
its slot. It holds none of the attention arithmetic, so the HIP path and the
CPU oracle can both be fed from it.

Host bookkeeping follows the pages:

* Free-list order: blocks are handed out in the order of the (shuffled)
  free list and freed blocks rejoin it at the end; a request that needs more
  blocks than are free fails with an out-of-memory error ("vLLM
  PagedAttention深度解析与工程实践" §3.2, the block manager's flow).
* Table growth: a token whose position is a multiple of the block size
  opens a new block; the others fill the sequence's last block
  (lqnn.cn/news/170268 §2.2, appending a token to a block table).
* Shared prefix blocks are referenced by several tables at once and carry a
  reference count (lqnn.cn/news/170268 §3.2; "vLLM 核心：PagedAttention 与
  Continuous Batching" §3 Prefix Caching).

Randomness: context lengths and the free-list shuffle come from
numpy.random.default_rng(seed) (PCG64), in that order. Element data q, K, V
and the new token's K/V ~ N(0, 1) are drawn in float32 from independent PCG64
streams keyed SeedSequence(seed, spawn_key=(stream, chunk)) - one stream per
tensor, one chunk per 256 cache blocks in allocation order - so generation
can run on several threads and still give the same bits; values are rounded
to nearest-even into fp16 / bf16. bf16 arrays are carried as uint16 bit
patterns.
"""

from collections import deque
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import math
import os

import numpy as np

# ---------------------------------------------------------------------------
# Named workloads
# ---------------------------------------------------------------------------


@dataclass(frozen=True)
class Workload:
    name: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str            # "f16" or "bf16"
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    lens: str             # length-distribution recipe, see draw_context_lens
    # split-path partition size: the GQA long-context workload names 512; the
    # others leave it open and take the size measured fastest for the shape
    partition_size: int = 512
    shared_prefix_tokens: int = 0
    long_seqs: int = 0        # extra sequences of long_len tokens
    long_len: int = 0
    description: str = ""


WORKLOADS = {
    "tiny": Workload(
        "tiny", 4, 8, 8, 64, "f16", 16, 64, 8, "uniform:1:128",
        description="4 seqs, 8 MHA heads, head_dim 64, fp16, block 16, "
                    "64 permuted physical blocks, context U[1,128]"),
    "llama13b": Workload(
        "llama13b", 32, 40, 40, 128, "f16", 16, 8192, 128, "uniform:32:2048",
        partition_size=256,
        description="LLaMA-13B-like decode: 32 seqs, 40 heads, head_dim 128, "
                    "fp16, block 16, 8192-block shuffled free list, "
                    "context U[32,2048]"),
    "llama7b": Workload(
        "llama7b", 64, 32, 32, 128, "bf16", 16, 16384, 256,
        "lognormal:512:1.0:16:4096",
        description="LLaMA-7B-like decode: 64 seqs, 32 heads, head_dim 128, "
                    "bf16, block 16, context lognormal(median 512, sigma 1) "
                    "clipped to [16,4096], new K/V scattered by slot"),
    "gqa_long": Workload(
        "gqa_long", 128, 64, 8, 128, "bf16", 16, 65536, 512,
        "uniform:1024:8192", partition_size=512,
        description="GQA long context: 128 seqs, 64 q / 8 kv heads, head_dim "
                    "128, bf16, block 16, context U[1024,8192], split-K 512"),
    "shared_prefix": Workload(
        "shared_prefix", 256, 32, 32, 128, "f16", 32, 16384, 1024,
        "uniform:1:1024", shared_prefix_tokens=2048, long_seqs=4,
        long_len=32768, partition_size=1024,
        description="shared prefix: 256 seqs share a 2048-token prefix "
                    "(same physical blocks) then private suffixes U[1,1024]; "
                    "plus 4 seqs of 32768 tokens; 32 heads, head_dim 128, "
                    "fp16, block 32, split-K 1024"),
}

WORKLOAD_ORDER = ["tiny", "llama13b", "llama7b", "gqa_long", "shared_prefix"]

# ---------------------------------------------------------------------------
# Block bookkeeping
# ---------------------------------------------------------------------------


class OutOfBlocks(RuntimeError):
    """The free list cannot satisfy an allocation (preemption territory)."""


def blocks_for(num_tokens, block_size):
    """Blocks of block_size slots that hold num_tokens tokens."""
    return -(-int(num_tokens) // int(block_size))


class BlockManager:
    """Reference-counted physical blocks over a first-in first-out free list.

    Blocks leave the free list from its head and return to its tail, so a
    freshly shuffled list hands out blocks in its shuffled order and a freed
    block is reused only after every block that was free before it. A block
    returns to the list when the last table holding it lets it go.
    """

    def __init__(self, free_blocks, block_size):
        self.free_blocks = deque(int(b) for b in free_blocks)
        self.block_size = int(block_size)
        self.allocated = {}   # seq id -> its table: physical blocks in logical order
        self.refcount = {}    # physical block -> number of tables holding it

    def take(self, n):
        """The n blocks at the head of the free list, each held once."""
        if n > len(self.free_blocks):
            raise OutOfBlocks("need %d blocks, %d free" % (n, len(self.free_blocks)))
        got = [self.free_blocks.popleft() for _ in range(n)]
        self.refcount.update((b, 1) for b in got)
        return got

    def release(self, blocks):
        """Drop one reference to each block; blocks nobody holds go back to
        the tail of the free list, in the order given."""
        for b in blocks:
            self.refcount[b] -= 1
        idle = [b for b in blocks if self.refcount[b] == 0]
        for b in idle:
            del self.refcount[b]
        self.free_blocks.extend(idle)

    def allocate(self, seq_id, num_tokens):
        """Extend seq_id's table to cover num_tokens tokens (never shrinks)."""
        table = self.allocated.setdefault(seq_id, [])
        table.extend(self.take(max(blocks_for(num_tokens, self.block_size) - len(table), 0)))

    def share(self, seq_id, blocks):
        """Append existing blocks to seq_id's table (held, not copied)."""
        for b in blocks:
            self.refcount[b] = self.refcount.get(b, 0) + 1
        self.allocated.setdefault(seq_id, []).extend(int(b) for b in blocks)

    def fork(self, parent_id, child_id):
        """child_id starts as a copy of parent_id's table: every block shared.

        The parallel-sampling case of the copy-on-write section of "优化大模型
        推理：PagedAttention 如何实现 GPU 显存高效管理": the candidates reference the
        prompt's physical blocks until their answers diverge."""
        self.share(child_id, list(self.allocated.get(parent_id, [])))

    def append_slot(self, seq_id, position):
        """Slot of seq_id's token at `position` (tokens 0 .. position-1 held).

        A position past the table's last block gets a new block. A token that
        lands in a block other tables still reference is written to a fresh
        copy of that block instead (copy-on-write: shared content stays
        read-only and is copied only when written); the copy replaces the
        block in this table and the pair (source block, new block) is
        returned for the device copy. The last table still holding a block
        writes in place. Returns (slot, (src, dst) or None)."""
        table = self.allocated.setdefault(seq_id, [])
        idx, off = divmod(int(position), self.block_size)
        if idx == len(table):
            table.extend(self.take(1))
            return table[idx] * self.block_size + off, None
        if idx != len(table) - 1:
            raise ValueError("position %d is not the next token of the table" % position)
        held = table[idx]
        if self.refcount[held] == 1:
            return held * self.block_size + off, None
        (copy,) = self.take(1)
        self.release([held])
        table[idx] = copy
        return copy * self.block_size + off, (held, copy)

    def move_out(self, seq_id, other):
        """Move seq_id's blocks into the pool managed by `other` (the swap-out
        of "vLLM 核心：PagedAttention 与 Continuous Batching" §5: a preempted
        request's KV blocks are copied to CPU memory and its GPU blocks freed).
        Returns the (block here, block there) pairs to copy. The blocks keep
        their logical order in the sequence's new table."""
        mine = list(self.allocated.get(seq_id, []))
        if any(self.refcount[b] > 1 for b in mine):
            raise ValueError("shared blocks stay resident: only a table's private blocks move")
        theirs = other.take(len(mine))
        other.allocated[seq_id] = theirs
        self.free(seq_id)
        return list(zip(mine, theirs))

    def free(self, seq_id):
        """Let go of seq_id's whole table."""
        self.release(self.allocated.pop(seq_id, []))


def kv_bytes_per_token(num_layers, num_kv_heads, head_dim, dtype_bytes):
    """K and V bytes one token occupies: 2 · layers · kv_heads · head_dim · bytes."""
    return 2 * num_layers * num_kv_heads * head_dim * dtype_bytes


def reservation_utilisation(used_tokens, reserved_per_request):
    """Fraction of a max-length contiguous reservation that holds tokens."""
    return sum(used_tokens) / float(reserved_per_request * len(used_tokens))


# ---------------------------------------------------------------------------
# Element encodings
# ---------------------------------------------------------------------------

F16_NAN = np.uint16(0x7E00)
BF16_NAN = np.uint16(0x7FC0)


def f32_to_bf16_bits(x):
    """Round-to-nearest-even fp32 -> bf16, returned as uint16 bits (finite x)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def encode(x, dtype):
    if dtype == "f16":
        return np.asarray(x, dtype=np.float32).astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def element_numpy_dtype(dtype):
    return {"f16": np.float16, "bf16": np.uint16}[dtype]


def nan_bits(dtype):
    return {"f16": F16_NAN, "bf16": BF16_NAN}[dtype]


# ---------------------------------------------------------------------------
# Batch construction
# ---------------------------------------------------------------------------


def draw_context_lens(rng, recipe, n):
    kind, *args = recipe.split(":")
    if kind == "uniform":
        lo, hi = int(args[0]), int(args[1])
        return rng.integers(lo, hi, endpoint=True, size=n).astype(np.int64)
    if kind == "lognormal":
        median, sigma, lo, hi = float(args[0]), float(args[1]), int(args[2]), int(args[3])
        z = rng.standard_normal(n)
        return np.clip(np.floor(np.exp(math.log(median) + sigma * z)), lo, hi).astype(np.int64)
    if kind == "fixed":
        return np.full(n, int(args[0]), dtype=np.int64)
    raise ValueError(recipe)


@dataclass
class Batch:
    """One decode step's inputs. Caches hold the history (positions < L-1);
    the new token (position L-1) arrives as new_key/new_value + slot_mapping."""
    workload: Workload
    query: np.ndarray          # [B, Hq, D]
    key_cache: np.ndarray      # [NB, BS, Hkv, D]
    value_cache: np.ndarray    # [NB, BS, Hkv, D]
    block_tables: np.ndarray   # int32 [B, MB], -1 past each table's end
    context_lens: np.ndarray   # int32 [B]
    new_key: np.ndarray        # [B, Hkv, D]
    new_value: np.ndarray      # [B, Hkv, D]
    slot_mapping: np.ndarray   # int64 [B]
    scale: float
    allocated_blocks: np.ndarray  # int64, every block some table uses (unique)
    shared_blocks: np.ndarray     # int64, blocks referenced by several tables
    refcount: dict = field(default_factory=dict)

    @property
    def dtype(self):
        return self.workload.dtype


def _bits(a):
    return a.view(np.uint16)


STREAM_Q, STREAM_K, STREAM_V, STREAM_NEW_K, STREAM_NEW_V = range(5)
BLOCKS_PER_CHUNK = 256


def _normal(seed, stream, chunk, shape):
    ss = np.random.SeedSequence(seed, spawn_key=(stream, chunk))
    return np.random.Generator(np.random.PCG64(ss)).standard_normal(shape, dtype=np.float32)


def _workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _fill_blocks(seed, stream, cache_bits, blocks, dtype):
    """Draw N(0,1) contents for whole blocks, chunk by chunk in parallel."""
    shape = cache_bits.shape[1:]
    starts = list(range(0, len(blocks), BLOCKS_PER_CHUNK))

    def one(c):
        ids = blocks[starts[c]:starts[c] + BLOCKS_PER_CHUNK]
        vals = _normal(seed, stream, c, (len(ids),) + shape)
        cache_bits[ids] = _bits(encode(vals, dtype))

    if len(starts) <= 1:
        for c in range(len(starts)):
            one(c)
        return
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(one, range(len(starts))))


def make_batch(workload, seed=0, lens=None, poison="nan", unallocated="zero"):
    """Build the seeded batch for a Workload.

    lens overrides the drawn context lengths (shared-prefix workloads take
    suffix lengths here). poison fills the new token's slot and the idle tail
    of each last block ("nan" or "zero"); unallocated blocks are "zero" or
    "nan".
    """
    w = workload
    rng = np.random.default_rng(seed)
    B = w.num_seqs + w.long_seqs
    BS = w.block_size
    # -- context lengths (each includes the new token) ---------------------
    if lens is None:
        drawn = draw_context_lens(rng, w.lens, w.num_seqs)
    else:
        drawn = np.asarray(lens, dtype=np.int64)
        if len(drawn) != w.num_seqs:
            raise ValueError("expected %d lengths" % w.num_seqs)
    if w.shared_prefix_tokens:
        ctx = np.concatenate([w.shared_prefix_tokens + drawn,
                              np.full(w.long_seqs, w.long_len, dtype=np.int64)])
    else:
        ctx = np.concatenate([drawn, np.full(w.long_seqs, w.long_len, dtype=np.int64)])
    if ctx.max(initial=0) > w.max_blocks_per_seq * BS:
        raise ValueError("context longer than max_blocks_per_seq * block_size")
    # -- block tables --------------------------------------------------------
    # The pool hands out blocks in the order of a seeded shuffle of its ids.
    # Every sequence holds its history (positions 0 .. L-2) from earlier
    # steps: first the shared prefix blocks, if any, then its private
    # blocks, taken in sequence order. This step's token (position L-1)
    # takes one more block, after all the histories, when it is the first
    # token of a block (L-1 a multiple of BS); otherwise it fills the last
    # history block.
    free = rng.permutation(w.num_blocks)
    npre = -(-w.shared_prefix_tokens // BS)
    if w.shared_prefix_tokens % BS:
        raise ValueError("shared prefix must be whole blocks")
    hist = np.maximum(ctx - 1, 0)
    own_hist = -(-np.maximum(hist - w.shared_prefix_tokens, 0) // BS)  # private history blocks
    opens = (ctx > 0) & (hist % BS == 0) & (hist >= w.shared_prefix_tokens)
    need = npre + int(own_hist.sum()) + int(opens.sum())
    if need > w.num_blocks:
        raise OutOfBlocks("need %d blocks, %d in the pool" % (need, w.num_blocks))
    shared = [int(b) for b in free[:npre]]
    hist_start = npre + np.concatenate([[0], np.cumsum(own_hist)[:-1]]).astype(np.int64)
    new_at = npre + int(own_hist.sum()) + np.cumsum(opens) - 1
    bt = np.full((B, w.max_blocks_per_seq), -1, dtype=np.int32)
    slots = np.full(B, -1, dtype=np.int64)
    # every block in use, the shared ones first, then each sequence's own
    # in table order (the order their contents are drawn in)
    order = list(shared)
    refcount = {b: B for b in shared}
    tables_blocks = []
    for i in range(B):
        own = [int(b) for b in free[hist_start[i]:hist_start[i] + own_hist[i]]]
        if opens[i]:
            own.append(int(free[new_at[i]]))
        row = shared + own
        bt[i, :len(row)] = row
        tables_blocks.append(row)
        if ctx[i] > 0:
            slots[i] = row[hist[i] // BS] * BS + hist[i] % BS
        refcount.update((b, 1) for b in own)
        order += own
    # -- element data (built as uint16 bit patterns) -------------------------
    D, Hq, Hkv = w.head_dim, w.num_heads, w.num_kv_heads
    q = _bits(encode(_normal(seed, STREAM_Q, 0, (B, Hq, D)), w.dtype))
    pool = (w.num_blocks, BS, Hkv, D)
    if unallocated == "nan":
        key_cache = np.full(pool, nan_bits(w.dtype), dtype=np.uint16)
        value_cache = np.full(pool, nan_bits(w.dtype), dtype=np.uint16)
    else:
        key_cache = np.zeros(pool, dtype=np.uint16)
        value_cache = np.zeros(pool, dtype=np.uint16)
    order = np.asarray(order, dtype=np.int64)
    _fill_blocks(seed, STREAM_K, key_cache, order, w.dtype)
    _fill_blocks(seed, STREAM_V, value_cache, order, w.dtype)
    new_key = _bits(encode(_normal(seed, STREAM_NEW_K, 0, (B, Hkv, D)), w.dtype))
    new_value = _bits(encode(_normal(seed, STREAM_NEW_V, 0, (B, Hkv, D)), w.dtype))
    # -- poison the new token's slot and every idle tail slot ----------------
    if poison is not None:
        pv = nan_bits(w.dtype) if poison == "nan" else np.uint16(0)
        for i in range(B):
            L = int(ctx[i])
            if L <= 0:
                continue
            last = tables_blocks[i][(L - 1) // BS]
            off = (L - 1) % BS
            key_cache[last, off:] = pv
            value_cache[last, off:] = pv
    edt = element_numpy_dtype(w.dtype)
    q, key_cache, value_cache, new_key, new_value = (
        a.view(edt) for a in (q, key_cache, value_cache, new_key, new_value))
    scale = 1.0 / math.sqrt(D)
    return Batch(w, q, key_cache, value_cache, bt, ctx.astype(np.int32), new_key,
                 new_value, slots, scale, order, np.asarray(shared, dtype=np.int64),
                 refcount)


# ---------------------------------------------------------------------------
# Prefill after a prefix-cache hit (lqnn.cn/news/170268 §3.4, §4.3)
# ---------------------------------------------------------------------------


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    cached_tokens: int    # whole blocks of a shared prompt found in the prefix cache
    new_lens: str         # new tokens per request, a draw_context_lens recipe
    description: str = ""


PREFILL_WORKLOADS = {
    "prefill_tiny": PrefillWorkload(
        "prefill_tiny", 4, 8, 8, 64, "f16", 16, 64, 12, 64, "uniform:1:64",
        description="4 requests share 64 cached prompt tokens, then 1..64 new tokens each; "
                    "8 MHA heads, head_dim 64, fp16, block 16"),
    "prefix_prefill": PrefillWorkload(
        "prefix_prefill", 100, 32, 32, 128, "f16", 16, 2048, 128, 1488, "uniform:16:80",
        description="100 requests share a ~1500-token system prompt whose 93 whole blocks "
                    "(1488 tokens) hit the prefix cache; each prefills the prompt's tail and "
                    "its question, 16..80 new tokens; 32 heads, head_dim 128, fp16, block 16, "
                    "2048-block shuffled free list"),
    "prefix_prefill_gqa": PrefillWorkload(
        "prefix_prefill_gqa", 100, 28, 4, 128, "bf16", 16, 2048, 128, 1488, "uniform:16:80",
        description="the same requests on a 28-query / 4-kv-head model, head_dim 128, bf16, "
                    "block 16"),
}

PREFILL_ORDER = ["prefill_tiny", "prefix_prefill", "prefix_prefill_gqa"]


@dataclass
class PrefillBatch:
    workload: PrefillWorkload
    query: np.ndarray          # [T, Hq, D], the new tokens of every request in order
    key_cache: np.ndarray      # [NB, BS, Hkv, D]: cached prompt blocks; new slots poisoned
    value_cache: np.ndarray
    block_tables: np.ndarray   # int32 [B, MB]
    context_lens: np.ndarray   # int32 [B]: cached + new tokens
    query_start: np.ndarray    # int32 [B + 1]
    new_key: np.ndarray        # [T, Hkv, D], K/V of the new tokens, stored by the scatter
    new_value: np.ndarray
    slot_mapping: np.ndarray   # int64 [T]
    scale: float
    shared_blocks: np.ndarray  # the cached prompt's blocks, in every table

    @property
    def dtype(self):
        return self.workload.dtype

    @property
    def max_query_len(self):
        return int(np.diff(self.query_start).max(initial=0))


def make_prefill_batch(workload, seed=0, lens=None, unallocated="nan"):
    """Seeded prefill batch: every request's table starts with the cached
    prompt's blocks (the same physical blocks, shared), then the blocks its
    new tokens need, taken from a shuffled free list. The new tokens' slots
    hold NaN until the scatter stores their K/V. lens overrides the drawn
    new-token counts."""
    w = workload
    rng = np.random.default_rng(seed)
    BS, B = w.block_size, w.num_seqs
    if w.cached_tokens % BS:
        raise ValueError("cached prompt tokens must be whole blocks")
    S = (draw_context_lens(rng, w.new_lens, B) if lens is None
         else np.asarray(lens, dtype=np.int64))
    if len(S) != B:
        raise ValueError("expected %d lengths" % B)
    ctx = w.cached_tokens + S
    if ctx.max(initial=0) > w.max_blocks_per_seq * BS:
        raise ValueError("context longer than max_blocks_per_seq * block_size")
    mgr = BlockManager(rng.permutation(w.num_blocks), BS)
    shared = []
    if w.cached_tokens:
        mgr.allocate("prompt", w.cached_tokens)
        shared = list(mgr.allocated["prompt"])
    bt = np.full((B, w.max_blocks_per_seq), -1, dtype=np.int32)
    for i in range(B):
        if shared:
            mgr.share(i, shared)
        mgr.allocate(i, int(ctx[i]))
        blocks = mgr.allocated.get(i, [])
        bt[i, :len(blocks)] = blocks
    if shared:
        mgr.free("prompt")
    qs = np.concatenate([[0], np.cumsum(S)]).astype(np.int32)
    T = int(qs[-1])
    slots = np.empty(T, dtype=np.int64)
    for i in range(B):
        for t in range(int(S[i])):
            p = w.cached_tokens + t
            slots[qs[i] + t] = int(bt[i, p // BS]) * BS + p % BS
    D, Hq, Hkv = w.head_dim, w.num_heads, w.num_kv_heads
    pool = (w.num_blocks, BS, Hkv, D)
    fill = nan_bits(w.dtype) if unallocated == "nan" else np.uint16(0)
    key_cache = np.full(pool, fill, dtype=np.uint16)
    value_cache = np.full(pool, fill, dtype=np.uint16)
    if shared:
        ids = np.asarray(shared, dtype=np.int64)
        _fill_blocks(seed, STREAM_K, key_cache, ids, w.dtype)
        _fill_blocks(seed, STREAM_V, value_cache, ids, w.dtype)
    # every slot of the new tokens' blocks is NaN until written
    for i in range(B):
        for j in range(w.cached_tokens // BS, -(-int(ctx[i]) // BS)):
            key_cache[bt[i, j]] = nan_bits(w.dtype)
            value_cache[bt[i, j]] = nan_bits(w.dtype)
    q = _bits(encode(_normal(seed, STREAM_Q, 0, (T, Hq, D)), w.dtype))
    nk = _bits(encode(_normal(seed, STREAM_NEW_K, 0, (T, Hkv, D)), w.dtype))
    nv = _bits(encode(_normal(seed, STREAM_NEW_V, 0, (T, Hkv, D)), w.dtype))
    edt = element_numpy_dtype(w.dtype)
    q, key_cache, value_cache, nk, nv = (a.view(edt) for a in (q, key_cache, value_cache, nk, nv))
    return PrefillBatch(w, q, key_cache, value_cache, bt, ctx.astype(np.int32), qs, nk, nv, slots,
                        1.0 / math.sqrt(D), np.asarray(shared, dtype=np.int64))


def prefill_flops(batch):
    """Algorithmic flops of the attention of a prefill batch: new token t of
    request i attends to L_i - S_i + t + 1 positions, each costing a q·k and
    a p·v multiply-add per head_dim element and query head (4 flops)."""
    w = batch.workload
    n = 0
    for i in range(len(batch.context_lens)):
        S = int(batch.query_start[i + 1] - batch.query_start[i])
        L = int(batch.context_lens[i])
        n += sum(max(L - S + t + 1, 0) for t in range(S))
    return 4 * n * w.num_heads * w.head_dim


def prefill_bytes(batch, out_dtype=None):
    """Algorithmic HBM bytes of the attention: each request's K/V rows once
    per kv head (a shared prompt block once for the whole batch), plus q and
    the output. Returns (unique, per_request)."""
    w = batch.workload
    e = element_bytes(w.dtype)
    eo = element_bytes(out_dtype or w.dtype)
    per_tok = 2 * w.num_kv_heads * w.head_dim * e
    T = int(batch.query_start[-1])
    qo = T * w.num_heads * w.head_dim * (e + eo)
    L = batch.context_lens.astype(np.int64)
    per_request = int(L.sum()) * per_tok + qo
    unique = (int(L.sum()) - (len(L) - 1) * w.cached_tokens) * per_tok + qo if len(L) else qo
    return unique, per_request


def custom_workload(name="custom", **kw):
    base = dict(num_seqs=2, num_heads=4, num_kv_heads=4, head_dim=64, dtype="f16",
                block_size=16, num_blocks=64, max_blocks_per_seq=8,
                lens="uniform:1:128")
    base.update(kw)
    return Workload(name, **base)


# ---------------------------------------------------------------------------
# Byte accounting for the measurement
# ---------------------------------------------------------------------------


def element_bytes(dtype):
    return {"f16": 2, "bf16": 2, "f32": 4}[dtype]


def step_bytes(batch, out_dtype=None):
    """Algorithmic bytes of one decode step (attention part).

    Σ L_i · 2·Hkv·D·e for K and V, plus q, the output, the block-table entries
    actually used and the context lengths. Returns (unique, logical): unique
    counts each shared physical block once.
    """
    w = batch.workload
    e = element_bytes(w.dtype)
    eo = element_bytes(out_dtype or w.dtype)
    B = len(batch.context_lens)
    per_tok = 2 * w.num_kv_heads * w.head_dim * e
    L = batch.context_lens.astype(np.int64)
    logical_tokens = int(L.sum())
    shared_tokens = len(batch.shared_blocks) * w.block_size
    n_sharing = int((L > shared_tokens).sum()) if shared_tokens else 0
    unique_tokens = logical_tokens - max(n_sharing - 1, 0) * shared_tokens if shared_tokens else logical_tokens
    nblk = int(sum(-(-int(x) // w.block_size) for x in L))
    fixed = B * w.num_heads * w.head_dim * (e + eo) + 4 * nblk + 4 * B
    return unique_tokens * per_tok + fixed, logical_tokens * per_tok + fixed


def kv_read_bytes(batch):
    """K and V bytes the attention must read: every attended position once
    per kv head (a shared prefix once), nothing else."""
    w = batch.workload
    per_tok = 2 * w.num_kv_heads * w.head_dim * element_bytes(w.dtype)
    L = batch.context_lens.astype(np.int64)
    shared_tokens = len(batch.shared_blocks) * w.block_size
    n_sharing = int((L > shared_tokens).sum()) if shared_tokens else 0
    return (int(L.sum()) - max(n_sharing - 1, 0) * shared_tokens) * per_tok


def cache_write_bytes(batch):
    """reshape_and_cache bytes: new K/V read + written, plus 8-byte slots."""
    w = batch.workload
    e = element_bytes(w.dtype)
    T = len(batch.slot_mapping)
    return 2 * (2 * T * w.num_kv_heads * w.head_dim * e) + 8 * T
