"""Plain float64 oracle for paged decode attention (test infrastructure only).

Sources (cited by page title and section):

* [P1] "LLM推理优化：vLLM PagedAttention深度解析与工程实践" (CSDN):
  §二 (the attention formula softmax(Q·Kᵀ/√d)·V and the per-step KV append),
  §3.1 (the block table: logical block -> physical block, blocks fill 16/16
  before the next is taken, only the last block is partial),
  §4.1 (cache layout [num_blocks, block_size, num_heads, head_dim]; the v2
  kernel "partially accumulates, then merges").
* [P2] "vLLM 核心：PagedAttention 与 Continuous Batching": §3 architecture
  diagram (logical blocks 0,1,2 -> physical 5,12,3 with block size 4) and
  "内存管理优势" (at most block_size-1 slots of the last block are idle).
* [P3] lqnn.cn/news/170268 (nano-vllm walkthrough): §2.2 (cache dimensions,
  append into the current block or a new one), §2.3 (the three kernel steps:
  walk the block table, score every cached token and weight V, write out),
  §6 (ignore unfilled slots of a block; accumulate in fp32 or better).
* [P3] also §3.2 (prefix-cache hits are whole blocks: a block's hash
  depends on its tokens only, matched in order) and §3.4 (on a hit the
  request's block table points at the cached blocks, prefill runs from the
  first missing position, new blocks are taken as it goes, and decoding then
  continues on the blocks); §1.1 (each generated token attends to itself and
  every earlier token).
* [P4] "优化大模型推理：PagedAttention 如何实现 GPU 显存高效管理":
  "按需分配" (35 tokens at block size 16 -> 3 blocks, 13 idle slots),
  Figure 2 (logical 0,1,2 -> physical 7,1,12), "写时复制" (copy-on-write:
  candidates share the prompt's blocks, a block is copied only when written;
  also [P1] §3.1's list of the design's benefits).

Readings where the pages are silent (each is listed with its reason in the
design notes): query head h reads kv head h // (Hq/Hkv); a context length of 0
gives a zero output; block-table entries past ceil(L/BS) are never read;
slots with a negative slot_mapping entry are skipped; a split partition p
covers logical tokens [p·P, (p+1)·P) and partitions are combined with the
textbook log-sum-exp rule. Prefill: the new tokens' K/V are stored into
their slots before attention, and new token t of a sequence whose context
(cached plus new) is L tokens, S of them new, sits at position L - S + t and
attends to positions 0 .. L - S + t, itself included.

Array conventions: fp16 data arrive as numpy float16; bf16 data arrive as
their raw uint16 bit patterns (numpy has no bfloat16); fp32 as float32.
"""

import numpy as np

# ---------------------------------------------------------------------------
# Block arithmetic ([P1] §3.1, [P4] "按需分配", [P3] §5.1)
# ---------------------------------------------------------------------------


def blocks_needed(num_tokens, block_size):
    """Number of fixed-size blocks that hold num_tokens tokens: ceil(n / bs)."""
    n = int(num_tokens)
    bs = int(block_size)
    if n < 0 or bs <= 0:
        raise ValueError("num_tokens must be >= 0 and block_size > 0")
    count = 0
    filled = 0
    while filled < n:  # one block at a time, as the pages describe the fill
        count += 1
        filled += bs
    return count


def unused_slots(num_tokens, block_size):
    """Idle slots at the end of the last block (at most block_size - 1)."""
    return blocks_needed(num_tokens, block_size) * int(block_size) - int(num_tokens)


def slot_of_token(block_table_row, token_index, block_size):
    """Physical slot of a logical token: the token's logical block is
    token // bs; the table names its physical block; the offset inside the
    block is token % bs ([P1] §3.1, [P2] §3 diagram)."""
    logical_block = int(token_index) // int(block_size)
    offset = int(token_index) - logical_block * int(block_size)
    physical_block = int(block_table_row[logical_block])
    return physical_block * int(block_size) + offset


# ---------------------------------------------------------------------------
# Exact upcast of the stored element types
# ---------------------------------------------------------------------------


def upcast(arr, dtype):
    """Exact float64 copy of an fp16 / bf16-bits / fp32 array."""
    if dtype == "f16":
        a = np.asarray(arr)
        if a.dtype != np.float16:
            raise TypeError("f16 data must be numpy float16")
        return a.astype(np.float64)
    if dtype == "bf16":
        a = np.asarray(arr)
        if a.dtype != np.uint16:
            raise TypeError("bf16 data must be passed as uint16 bit patterns")
        # a bf16 value is the top half of the fp32 with the same bits
        wide = a.astype(np.uint32) << np.uint32(16)
        return wide.view(np.float32).astype(np.float64)
    if dtype == "f32":
        a = np.asarray(arr)
        if a.dtype != np.float32:
            raise TypeError("f32 data must be numpy float32")
        return a.astype(np.float64)
    raise ValueError("unknown dtype %r" % (dtype,))


# ---------------------------------------------------------------------------
# reshape_and_cache: write each new token's K/V into its slot
# ([P1] §二 per-step append, [P3] §2.2 "write into the current block")
# ---------------------------------------------------------------------------


def reshape_and_cache(key, value, key_cache, value_cache, slot_mapping):
    """Return copies of the caches with token n's K/V stored at its slot.

    key, value: [T, Hkv, D]; caches: [NB, BS, Hkv, D] (any element type, the
    copy is bitwise); slot_mapping: [T] integers, a negative entry means
    "no slot" and the token is skipped.
    """
    key = np.asarray(key)
    value = np.asarray(value)
    kc = np.array(key_cache, copy=True)
    vc = np.array(value_cache, copy=True)
    num_blocks, block_size = kc.shape[0], kc.shape[1]
    slots = np.asarray(slot_mapping)
    if key.shape[0] != slots.shape[0] or value.shape[0] != slots.shape[0]:
        raise ValueError("one slot per new token")
    for n in range(slots.shape[0]):
        s = int(slots[n])
        if s < 0:
            continue
        if s >= num_blocks * block_size:
            raise IndexError("slot %d outside the cache" % s)
        blk = s // block_size
        off = s % block_size
        kc[blk, off] = key[n]
        vc[blk, off] = value[n]
    return kc, vc


# ---------------------------------------------------------------------------
# Decode attention ([P1] §二 formula; [P3] §2.3 three steps; [P3] §6 masking)
# ---------------------------------------------------------------------------


def gather_sequence(cache, block_table_row, context_len, block_size):
    """Logically contiguous [L, Hkv, D] view of one sequence's cache rows.

    Walks the first ceil(L/BS) table entries in logical order and keeps the
    first L slots; later entries and the idle tail of the last block are
    never touched.
    """
    L = int(context_len)
    nb = blocks_needed(L, block_size)
    if nb == 0:
        return cache[:0, 0]  # [0, Hkv, D]
    rows = [cache[int(block_table_row[j])] for j in range(nb)]  # each [BS, Hkv, D]
    seq = np.concatenate(rows, axis=0)
    return seq[:L]


def decode(query, key_cache, value_cache, block_tables, context_lens, scale,
           kv_dtype):
    """out[i, h] = softmax(scale · K_i q_ih) · V_i for every sequence i, head h.

    query [B, Hq, D] and caches [NB, BS, Hkv, D] of element type kv_dtype;
    block_tables [B, MB] ints; context_lens [B] ints; returns float64 [B, Hq, D].
    """
    q64 = upcast(query, kv_dtype)
    B, Hq, D = q64.shape
    Hkv = key_cache.shape[2]
    if Hq % Hkv != 0:
        raise ValueError("query heads must be a multiple of kv heads")
    group = Hq // Hkv
    block_size = key_cache.shape[1]
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for i in range(B):
        L = int(context_lens[i])
        if L <= 0:
            continue  # empty context: zero output
        K = upcast(gather_sequence(key_cache, block_tables[i], L, block_size), kv_dtype)
        V = upcast(gather_sequence(value_cache, block_tables[i], L, block_size), kv_dtype)
        for h in range(Hq):
            g = h // group
            s = scale * (K[:, g, :] @ q64[i, h])  # [L] logits
            p = np.exp(s - s.max())
            p = p / p.sum()
            out[i, h] = p @ V[:, g, :]
    return out


def decode_partitions(query, key_cache, value_cache, block_tables, context_lens,
                      scale, kv_dtype, partition_size, max_partitions=None):
    """Per-partition softmax statistics ([P1] §4.1, "partial accumulate").

    Partition p of sequence i covers logical tokens [p·P, min((p+1)·P, L)).
    Returns (m, l, o): m [B, Hq, NP] the partition's largest logit,
    l [B, Hq, NP] = Σ exp(s_t - m), o [B, Hq, NP, D] = Σ exp(s_t - m)·v_t / l.
    Partitions holding no token have m = -inf, l = 0, o = 0.
    """
    q64 = upcast(query, kv_dtype)
    B, Hq, D = q64.shape
    Hkv = key_cache.shape[2]
    group = Hq // Hkv
    block_size = key_cache.shape[1]
    P = int(partition_size)
    if max_partitions is None:
        max_partitions = max([blocks_needed(max(int(x), 0), P) for x in context_lens] + [1])
    NP = int(max_partitions)
    m = np.full((B, Hq, NP), -np.inf)
    l = np.zeros((B, Hq, NP))
    o = np.zeros((B, Hq, NP, D))
    for i in range(B):
        L = int(context_lens[i])
        if L <= 0:
            continue
        K = upcast(gather_sequence(key_cache, block_tables[i], L, block_size), kv_dtype)
        V = upcast(gather_sequence(value_cache, block_tables[i], L, block_size), kv_dtype)
        for p in range(blocks_needed(L, P)):
            lo, hi = p * P, min((p + 1) * P, L)
            for h in range(Hq):
                g = h // group
                s = scale * (K[lo:hi, g, :] @ q64[i, h])
                mp = s.max()
                w = np.exp(s - mp)
                m[i, h, p] = mp
                l[i, h, p] = w.sum()
                o[i, h, p] = (w @ V[lo:hi, g, :]) / w.sum()
    return m, l, o


def lse_merge(m, l, o, context_lens, partition_size):
    """Combine partitions by log-sum-exp: with M = max_p m_p and
    w_p = l_p·exp(m_p - M), out = Σ_p w_p·o_p / Σ_p w_p over the partitions
    that hold tokens. A sequence with no tokens gives zeros."""
    B, Hq, NP, D = o.shape
    out = np.zeros((B, Hq, D))
    P = int(partition_size)
    for i in range(B):
        L = int(context_lens[i])
        n_parts = blocks_needed(max(L, 0), P)
        if n_parts == 0:
            continue
        for h in range(Hq):
            mp = m[i, h, :n_parts]
            M = mp.max()
            w = l[i, h, :n_parts] * np.exp(mp - M)
            out[i, h] = (w[:, None] * o[i, h, :n_parts]).sum(axis=0) / w.sum()
    return out


def decode_split(query, key_cache, value_cache, block_tables, context_lens, scale,
                 kv_dtype, partition_size):
    """decode() computed as partitions followed by the log-sum-exp merge."""
    m, l, o = decode_partitions(query, key_cache, value_cache, block_tables,
                                context_lens, scale, kv_dtype, partition_size)
    return lse_merge(m, l, o, context_lens, partition_size)


# ---------------------------------------------------------------------------
# Copy-on-write block copy ([P4] "写时复制", [P1] §3.1)
# ---------------------------------------------------------------------------


def copy_blocks(key_cache, value_cache, block_mapping):
    """Return copies of the caches where, for every pair (src, dst) of
    block_mapping ([N, 2] integers), physical block dst holds the contents of
    physical block src, for K and for V (all block_size rows, all heads).

    A shared block that one sequence is about to write is copied first, and
    the sequence's table then points at the copy ([P4] "写时复制"). All pairs
    read the caches as they were before the call (destinations are fresh
    blocks, never a source of another pair, each used once); the copy is
    bitwise, for any element type.
    """
    kc = np.array(key_cache, copy=True)
    vc = np.array(value_cache, copy=True)
    src_k = np.asarray(key_cache)
    src_v = np.asarray(value_cache)
    pairs = np.asarray(block_mapping).reshape(-1, 2)
    for n in range(pairs.shape[0]):
        src, dst = int(pairs[n, 0]), int(pairs[n, 1])
        kc[dst] = src_k[src]
        vc[dst] = src_v[src]
    return kc, vc


# ---------------------------------------------------------------------------
# Swapping blocks between pools ("vLLM 核心：PagedAttention 与 Continuous
# Batching" §5, strategy 1)
# ---------------------------------------------------------------------------


def swap_blocks(dst_key_cache, dst_value_cache, src_key_cache, src_value_cache, block_mapping):
    """Return copies of the destination pool's caches where, for every pair
    (s, d) of block_mapping ([N, 2]), block d holds block s of the source pool
    (K and V, bitwise). The swap-out of a preempted request copies its KV
    blocks from GPU to CPU memory; the swap-in copies them back, possibly to
    other physical blocks. The destinations are distinct."""
    kd = np.array(dst_key_cache, copy=True)
    vd = np.array(dst_value_cache, copy=True)
    pairs = np.asarray(block_mapping).reshape(-1, 2)
    for n in range(pairs.shape[0]):
        src, dst = int(pairs[n, 0]), int(pairs[n, 1])
        kd[dst] = np.asarray(src_key_cache)[src]
        vd[dst] = np.asarray(src_value_cache)[src]
    return kd, vd


# ---------------------------------------------------------------------------
# Prefill over cached prefix blocks ([P3] §3.4 flow, §3.2 block-level hits,
# §1.1 each token attends to itself and all earlier tokens; [P1] §二 formula)
# ---------------------------------------------------------------------------


def prefill(query, key_cache, value_cache, block_tables, context_lens, query_start,
            scale, kv_dtype):
    """Causal attention of every sequence's new tokens over its paged context.

    query [T, Hq, D]: the new tokens of all sequences, packed in sequence
    order; sequence i owns rows query_start[i] .. query_start[i+1] - 1
    (query_start has B + 1 ascending entries, the first 0, the last T).
    context_lens[i] = L_i counts the cached tokens plus the S_i new ones,
    whose K/V are already in the caches at positions L_i - S_i .. L_i - 1.
    Row t of sequence i (position p = L_i - S_i + t) attends to the cache
    positions 0..p. Returns float64 [T, Hq, D]; a row with no position to
    attend (p < 0, a caller error) is zero.
    """
    q64 = upcast(query, kv_dtype)
    T, Hq, D = q64.shape
    Hkv = key_cache.shape[2]
    if Hq % Hkv != 0:
        raise ValueError("query heads must be a multiple of kv heads")
    group = Hq // Hkv
    block_size = key_cache.shape[1]
    qs = [int(x) for x in query_start]
    if qs[0] != 0 or qs[-1] != T or any(b < a for a, b in zip(qs, qs[1:])):
        raise ValueError("query_start must ascend from 0 to the number of query rows")
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for i in range(len(qs) - 1):
        S = qs[i + 1] - qs[i]
        L = int(context_lens[i])
        if S == 0 or L <= 0:
            continue
        K = upcast(gather_sequence(key_cache, block_tables[i], L, block_size), kv_dtype)
        V = upcast(gather_sequence(value_cache, block_tables[i], L, block_size), kv_dtype)
        for t in range(S):
            p = L - S + t  # the token's position in its sequence
            if p < 0:
                continue
            for h in range(Hq):
                g = h // group
                s = scale * (K[: p + 1, g, :] @ q64[qs[i] + t, h])  # logits of 0..p
                w = np.exp(s - s.max())
                w = w / w.sum()
                out[qs[i] + t, h] = w @ V[: p + 1, g, :]
    return out

