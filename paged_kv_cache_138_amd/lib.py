"""ctypes binding of libpa.so: argument marshalling only.

Every function here checks devices, element types, contiguity and shapes of
torch tensors (a block table kept on the host, or in the wrong integer type,
silently reads the wrong blocks - lqnn.cn/news/170268 §6), then calls the
C entry point of the same name on the current HIP stream. All compute runs
in the library's HIP kernels; there is no fallback path. If libpa.so is not
built, the first call raises.
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("PA_LIBRARY", os.path.join(_PKG, "libpa.so"))

PA_F16, PA_BF16, PA_F32 = 0, 1, 2
_DT = {torch.float16: PA_F16, torch.bfloat16: PA_BF16, torch.float32: PA_F32}
_TORCH_DT = {v: k for k, v in _DT.items()}


class PaError(RuntimeError):
    def __init__(self, status, what, detail):
        super().__init__("%s failed: status %d (%s): %s" % (what, status, _status_str(status), detail))
        self.status = status


_lib = None


def _status_str(s):
    try:
        return load().pa_status_string(s).decode()
    except Exception:  # pragma: no cover
        return "?"


def load():
    """Load libpa.so once (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libpa.so not found at %s; build it with "
                           "`python -m paged_kv_cache_138_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.pa_reshape_and_cache.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i32, i32, i32, i32, i32, vp]
    lib.pa_reshape_and_cache.restype = i32
    dec = [vp, i32, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i32]
    lib.pa_decode.argtypes = dec + [vp]
    lib.pa_prefill.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                               i32, i32, f32, i32, vp]
    lib.pa_prefill.restype = i32
    lib.pa_prefill_shared_prefix.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                             i32, i32, i32, i32, i32, f32, i32, i32, vp]
    lib.pa_prefill_shared_prefix.restype = i32
    lib.pa_decode.restype = i32
    lib.pa_decode_split.argtypes = dec + [i32, vp, sz, vp]
    lib.pa_decode_split.restype = i32
    lib.pa_decode_split_noalloc.argtypes = dec + [i32, vp]
    lib.pa_decode_split_noalloc.restype = i32
    lib.pa_decode_partitions.argtypes = dec + [i32, vp, sz, vp]
    lib.pa_decode_partitions.restype = i32
    lib.pa_decode_partitions_shared_prefix.argtypes = dec + [i32, i32, vp, sz, vp]
    lib.pa_decode_partitions_shared_prefix.restype = i32
    lib.pa_decode_split_shared_prefix.argtypes = dec + [i32, i32, vp, sz, vp]
    lib.pa_decode_split_shared_prefix.restype = i32
    lib.pa_decode_split_append.argtypes = ([vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64]
                                           + [i32] * 7 + [f32, i32, i32, vp, sz, vp])
    lib.pa_decode_split_append.restype = i32
    lib.pa_decode_partitions_append.argtypes = lib.pa_decode_split_append.argtypes
    lib.pa_decode_partitions_append.restype = i32
    lib.pa_decode_split_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.pa_decode_split_workspace_bytes.restype = sz
    lib.pa_lse_merge.argtypes = [vp, i32, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
    lib.pa_lse_merge.restype = i32
    lib.pa_copy_blocks.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
    lib.pa_copy_blocks.restype = i32
    lib.pa_swap_blocks.argtypes = [vp, vp, i32, vp, vp, i32, vp, i32, i32, i32, i32, i32, vp]
    lib.pa_swap_blocks.restype = i32
    lib.pa_stream_read.argtypes = [vp, sz, vp, vp]
    lib.pa_stream_read.restype = i32
    lib.pa_status_string.argtypes = [i32]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_last_error.argtypes = []
    lib.pa_last_error.restype = ctypes.c_char_p
    lib.pa_version.argtypes = []
    lib.pa_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status, what):
    if status != 0:
        raise PaError(status, what, load().pa_last_error().decode())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _on_gpu(*ts):
    dev = ts[0].device
    for t in ts:
        _need(t.is_cuda, "all tensors must be on the GPU (got %s)" % t.device)
        _need(t.device == dev, "all tensors must be on one device")


def _kv_checks(query, key_cache, value_cache):
    _need(key_cache.dtype in (torch.float16, torch.bfloat16), "cache dtype must be fp16 or bf16")
    _need(query.dtype == key_cache.dtype == value_cache.dtype, "query and caches must share a dtype")
    _need(key_cache.dim() == 4 and key_cache.shape == value_cache.shape,
          "caches must be [num_blocks, block_size, num_kv_heads, head_dim]")
    for t in (query, key_cache, value_cache):
        _need(t.is_contiguous(), "query and caches must be contiguous")


def version():
    return load().pa_version().decode()


def reshape_and_cache(key, value, key_cache, value_cache, slot_mapping):
    """Store key[n], value[n] ([T, Hkv, D]) at slot_mapping[n] (int64) of the
    caches [NB, BS, Hkv, D], in place. Negative slots are skipped."""
    _on_gpu(key, value, key_cache, value_cache, slot_mapping)
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.dim() == 1 and slot_mapping.is_contiguous(),
          "slot_mapping must be a contiguous int64 vector")
    _need(key.dtype == value.dtype == key_cache.dtype == value_cache.dtype, "dtypes differ")
    _need(key_cache.dtype in (torch.float16, torch.bfloat16), "cache dtype must be fp16 or bf16")
    _need(key_cache.is_contiguous() and value_cache.is_contiguous(), "caches must be contiguous")
    NB, BS, Hkv, D = key_cache.shape
    _need(value_cache.shape == key_cache.shape, "caches differ in shape")
    T = slot_mapping.shape[0]
    for t in (key, value):
        _need(t.dim() == 3 and tuple(t.shape) == (T, Hkv, D), "key/value must be [T, Hkv, D]")
        _need(t.stride(2) == 1 and t.stride(1) == D, "heads and dims of a token must be dense")
    st = load().pa_reshape_and_cache(
        _ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache), _ptr(slot_mapping), T,
        key.stride(0) if T else Hkv * D, value.stride(0) if T else Hkv * D, Hkv, D, NB, BS,
        _DT[key_cache.dtype], _stream(key_cache))
    _check(st, "pa_reshape_and_cache")


def copy_blocks(key_cache, value_cache, block_mapping):
    """Copy block src to block dst of both caches for every row (src, dst) of
    block_mapping (int64 [N, 2]), in place; see pa_copy_blocks."""
    _on_gpu(key_cache, value_cache, block_mapping)
    _need(block_mapping.dtype == torch.int64 and block_mapping.dim() == 2
          and block_mapping.shape[1] == 2 and block_mapping.is_contiguous(),
          "block_mapping must be a contiguous int64 [N, 2] tensor")
    _need(key_cache.dtype == value_cache.dtype and key_cache.dtype in (torch.float16, torch.bfloat16),
          "caches must share an fp16/bf16 dtype")
    _need(key_cache.is_contiguous() and value_cache.is_contiguous()
          and key_cache.shape == value_cache.shape and key_cache.dim() == 4, "caches must be contiguous "
          "[num_blocks, block_size, num_kv_heads, head_dim] tensors of one shape")
    NB, BS, Hkv, D = key_cache.shape
    st = load().pa_copy_blocks(_ptr(key_cache), _ptr(value_cache), _ptr(block_mapping),
                               block_mapping.shape[0], Hkv, D, BS, NB, _DT[key_cache.dtype],
                               _stream(key_cache))
    _check(st, "pa_copy_blocks")


def swap_blocks(dst_key_cache, dst_value_cache, src_key_cache, src_value_cache, block_mapping):
    """Copy block s of the source pool to block d of the destination pool for
    every row (s, d) of block_mapping (int64 [N, 2]); either pool may be a
    pinned CPU tensor (pin_memory=True), see pa_swap_blocks."""
    caches = (dst_key_cache, dst_value_cache, src_key_cache, src_value_cache)
    for t in caches + (block_mapping,):
        _need(t.is_contiguous(), "tensors must be contiguous")
        _need(t.is_cuda or t.is_pinned(), "tensors must be on the GPU or in pinned host memory")
    _need(block_mapping.dtype == torch.int64 and block_mapping.dim() == 2
          and block_mapping.shape[1] == 2, "block_mapping must be an int64 [N, 2] tensor")
    dt = dst_key_cache.dtype
    _need(all(t.dtype == dt for t in caches) and dt in (torch.float16, torch.bfloat16),
          "caches must share an fp16/bf16 dtype")
    _need(dst_key_cache.shape == dst_value_cache.shape and src_key_cache.shape == src_value_cache.shape
          and dst_key_cache.dim() == 4 and dst_key_cache.shape[1:] == src_key_cache.shape[1:],
          "pools must be [num_blocks, block_size, num_kv_heads, head_dim] of one row shape")
    NBd, BS, Hkv, D = dst_key_cache.shape
    NBs = src_key_cache.shape[0]
    cuda = [t.device for t in caches + (block_mapping,) if t.is_cuda]
    dev = cuda[0] if cuda else torch.device("cuda", torch.cuda.current_device())
    st = load().pa_swap_blocks(_ptr(dst_key_cache), _ptr(dst_value_cache), NBd, _ptr(src_key_cache),
                               _ptr(src_value_cache), NBs, _ptr(block_mapping), block_mapping.shape[0],
                               Hkv, D, BS, _DT[dt], torch.cuda.current_stream(dev).cuda_stream)
    _check(st, "pa_swap_blocks")


def _decode_common(query, key_cache, value_cache, block_tables, context_lens, out, out_dtype):
    _on_gpu(query, key_cache, value_cache, block_tables, context_lens)
    _kv_checks(query, key_cache, value_cache)
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and block_tables.is_contiguous(),
          "block_tables must be a contiguous int32 [num_seqs, max_blocks_per_seq] tensor")
    _need(context_lens.dtype == torch.int32 and context_lens.dim() == 1 and context_lens.is_contiguous(),
          "context_lens must be a contiguous int32 vector")
    B, Hq, D = query.shape
    NB, BS, Hkv, D2 = key_cache.shape
    _need(D == D2, "head_dim of query and caches differ")
    _need(block_tables.shape[0] == B and context_lens.shape[0] == B, "batch sizes differ")
    if out is None:
        od = out_dtype if out_dtype is not None else query.dtype
        out = torch.empty((B, Hq, D), dtype=od, device=query.device)
    _on_gpu(query, out)
    _need(out.shape == (B, Hq, D) and out.is_contiguous(), "out must be a contiguous [B, Hq, D] tensor")
    _need(out.dtype in _DT, "unsupported out dtype")
    return out, (B, Hq, Hkv, D, BS, block_tables.shape[1], NB)


def decode(query, key_cache, value_cache, block_tables, context_lens, scale, out=None, out_dtype=None):
    """Single-launch paged decode attention; returns out [B, Hq, D]."""
    out, (B, Hq, Hkv, D, BS, MB, NB) = _decode_common(
        query, key_cache, value_cache, block_tables, context_lens, out, out_dtype)
    st = load().pa_decode(_ptr(out), _DT[out.dtype], _ptr(query), _ptr(key_cache), _ptr(value_cache),
                          _ptr(block_tables), _ptr(context_lens), B, Hq, Hkv, D, BS, MB, NB,
                          float(scale), _DT[key_cache.dtype], _stream(query))
    _check(st, "pa_decode")
    return out


def prefill(query, key_cache, value_cache, block_tables, context_lens, query_start, scale,
            max_query_len, out=None, out_dtype=None, shared_prefix_tokens=None):
    """Causal attention of the new tokens query [T, Hq, D] (sequence i owns
    rows query_start[i] .. query_start[i+1] - 1, the last positions of its
    context_lens[i] tokens, whose K/V are already cached) over each
    sequence's paged context; returns out [T, Hq, D]. max_query_len bounds
    every sequence's new-token count; see pa_prefill. With
    shared_prefix_tokens set, pa_prefill_shared_prefix: every sequence's
    first shared_prefix_tokens positions are the blocks of row 0 of
    block_tables."""
    _on_gpu(query, key_cache, value_cache, block_tables, context_lens, query_start)
    _kv_checks(query, key_cache, value_cache)
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and block_tables.is_contiguous(),
          "block_tables must be a contiguous int32 [num_seqs, max_blocks_per_seq] tensor")
    _need(context_lens.dtype == torch.int32 and context_lens.dim() == 1 and context_lens.is_contiguous(),
          "context_lens must be a contiguous int32 vector")
    B = context_lens.shape[0]
    _need(query_start.dtype == torch.int32 and query_start.dim() == 1 and query_start.is_contiguous()
          and query_start.shape[0] == B + 1, "query_start must be a contiguous int32 [num_seqs + 1] vector")
    _need(block_tables.shape[0] == B, "batch sizes differ")
    T, Hq, D = query.shape
    NB, BS, Hkv, D2 = key_cache.shape
    _need(D == D2, "head_dim of query and caches differ")
    if out is None:
        od = out_dtype if out_dtype is not None else query.dtype
        out = torch.empty((T, Hq, D), dtype=od, device=query.device)
    _on_gpu(query, out)
    _need(out.shape == (T, Hq, D) and out.is_contiguous(), "out must be a contiguous [T, Hq, D] tensor")
    _need(out.dtype in _DT, "unsupported out dtype")
    args = (_ptr(out), _DT[out.dtype], _ptr(query), _ptr(key_cache), _ptr(value_cache),
            _ptr(block_tables), _ptr(context_lens), _ptr(query_start), B, T, int(max_query_len),
            Hq, Hkv, D, BS, block_tables.shape[1], NB, float(scale), _DT[key_cache.dtype])
    if shared_prefix_tokens is None:
        _check(load().pa_prefill(*args, _stream(query)), "pa_prefill")
    else:
        _check(load().pa_prefill_shared_prefix(*args, int(shared_prefix_tokens), _stream(query)),
               "pa_prefill_shared_prefix")
    return out


def decode_split_workspace_bytes(num_seqs, num_heads, head_dim, max_blocks_per_seq, block_size,
                                 partition_size):
    return int(load().pa_decode_split_workspace_bytes(num_seqs, num_heads, head_dim,
                                                      max_blocks_per_seq, block_size, partition_size))


def make_workspace(num_seqs, num_heads, head_dim, max_blocks_per_seq, block_size, partition_size,
                   device="cuda"):
    n = decode_split_workspace_bytes(num_seqs, num_heads, head_dim, max_blocks_per_seq, block_size,
                                     partition_size)
    _need(n > 0, "invalid sizes for the split workspace")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _split_call(name, query, key_cache, value_cache, block_tables, context_lens, scale, partition_size,
                workspace, out, out_dtype, prefix=None):
    out, (B, Hq, Hkv, D, BS, MB, NB) = _decode_common(
        query, key_cache, value_cache, block_tables, context_lens, out, out_dtype)
    if workspace is None:
        workspace = make_workspace(B, Hq, D, MB, BS, partition_size, query.device)
    _need(workspace.is_cuda and workspace.is_contiguous(), "workspace must be a contiguous GPU tensor")
    nbytes = workspace.numel() * workspace.element_size()
    extra = [] if prefix is None else [int(prefix)]
    st = getattr(load(), name)(_ptr(out), _DT[out.dtype], _ptr(query), _ptr(key_cache),
                               _ptr(value_cache), _ptr(block_tables), _ptr(context_lens), B, Hq, Hkv,
                               D, BS, MB, NB, float(scale), _DT[key_cache.dtype], int(partition_size),
                               *extra, _ptr(workspace), nbytes, _stream(query))
    _check(st, name)
    return out


def decode_split(query, key_cache, value_cache, block_tables, context_lens, scale, partition_size=512,
                 workspace=None, out=None, out_dtype=None):
    """Paged decode attention as partitions + log-sum-exp merge."""
    return _split_call("pa_decode_split", query, key_cache, value_cache, block_tables, context_lens,
                       scale, partition_size, workspace, out, out_dtype)


# bytes of the scratch array pa_decode_split_noalloc uses (PA_DECODE_NOALLOC_MAX_WORKSPACE)
NOALLOC_MAX_WORKSPACE = 32 << 20


def decode_split_noalloc(query, key_cache, value_cache, block_tables, context_lens, scale,
                         partition_size=512, out=None):
    """decode_split without a workspace: the partials go to the library's own
    scratch array on the device (pa_decode_split_noalloc), so nothing is
    allocated when `out` is given. Calls overlapping in time on one GPU race."""
    out, (B, Hq, Hkv, D, BS, MB, NB) = _decode_common(
        query, key_cache, value_cache, block_tables, context_lens, out, None)
    st = load().pa_decode_split_noalloc(
        _ptr(out), _DT[out.dtype], _ptr(query), _ptr(key_cache), _ptr(value_cache),
        _ptr(block_tables), _ptr(context_lens), B, Hq, Hkv, D, BS, MB, NB, float(scale),
        _DT[key_cache.dtype], int(partition_size), _stream(query))
    _check(st, "pa_decode_split_noalloc")
    return out


def decode_split_append(query, key_cache, value_cache, block_tables, context_lens, new_key, new_value,
                        slot_mapping, scale, partition_size=512, workspace=None, out=None,
                        out_dtype=None, _name="pa_decode_split_append"):
    """One decode step: store new_key[i] / new_value[i] ([B, Hkv, D], one new
    token per sequence) at slot_mapping[i] of the caches and attend, the new
    token being position L_i - 1 of sequence i (see pa.h)."""
    out, (B, Hq, Hkv, D, BS, MB, NB) = _decode_common(
        query, key_cache, value_cache, block_tables, context_lens, out, out_dtype)
    _on_gpu(new_key, new_value, slot_mapping)
    _need(slot_mapping.dtype == torch.int64 and tuple(slot_mapping.shape) == (B,)
          and slot_mapping.is_contiguous(), "slot_mapping must be a contiguous int64 [num_seqs] vector")
    for t in (new_key, new_value):
        _need(t.dtype == key_cache.dtype, "new rows must have the cache dtype")
        _need(t.dim() == 3 and tuple(t.shape) == (B, Hkv, D), "new_key/new_value must be [B, Hkv, D]")
        _need(t.stride(2) == 1 and t.stride(1) == D, "heads and dims of a token must be dense")
    if workspace is None:
        workspace = make_workspace(B, Hq, D, MB, BS, partition_size, query.device)
    _need(workspace.is_cuda and workspace.is_contiguous(), "workspace must be a contiguous GPU tensor")
    nbytes = workspace.numel() * workspace.element_size()
    st = getattr(load(), _name)(
        _ptr(out), _DT[out.dtype], _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(context_lens), _ptr(new_key), _ptr(new_value), _ptr(slot_mapping),
        new_key.stride(0) if B else Hkv * D, new_value.stride(0) if B else Hkv * D, B, Hq, Hkv, D, BS,
        MB, NB, float(scale), _DT[key_cache.dtype], int(partition_size), _ptr(workspace), nbytes,
        _stream(query))
    _check(st, _name)
    return out


def decode_partitions_append(query, key_cache, value_cache, block_tables, context_lens, new_key,
                             new_value, slot_mapping, scale, partition_size=512, workspace=None,
                             out=None, out_dtype=None):
    """The partition launch of decode_split_append (merge with lse_merge)."""
    return decode_split_append(query, key_cache, value_cache, block_tables, context_lens, new_key,
                               new_value, slot_mapping, scale, partition_size, workspace, out,
                               out_dtype, _name="pa_decode_partitions_append")


def decode_partitions(query, key_cache, value_cache, block_tables, context_lens, scale,
                      partition_size=512, workspace=None, out=None, out_dtype=None):
    """The partition launch of decode_split alone: single-partition sequences
    get their output, the others leave per-partition rows in `workspace`."""
    return _split_call("pa_decode_partitions", query, key_cache, value_cache, block_tables,
                       context_lens, scale, partition_size, workspace, out, out_dtype)


def decode_split_shared_prefix(query, key_cache, value_cache, block_tables, context_lens, scale,
                               shared_prefix_tokens, partition_size=512, workspace=None, out=None,
                               out_dtype=None):
    """decode_split for a batch whose sequences all begin with the same
    shared_prefix_tokens tokens (the blocks of block_tables row 0); the prefix
    partitions are computed once per 64 or 128 query rows."""
    return _split_call("pa_decode_split_shared_prefix", query, key_cache, value_cache, block_tables,
                       context_lens, scale, partition_size, workspace, out, out_dtype,
                       prefix=shared_prefix_tokens)


def decode_partitions_shared_prefix(query, key_cache, value_cache, block_tables, context_lens, scale,
                                    shared_prefix_tokens, partition_size=512, workspace=None,
                                    out=None, out_dtype=None):
    """The partition launches of decode_split_shared_prefix alone."""
    return _split_call("pa_decode_partitions_shared_prefix", query, key_cache, value_cache,
                       block_tables, context_lens, scale, partition_size, workspace, out, out_dtype,
                       prefix=shared_prefix_tokens)


def workspace_views(workspace, num_seqs, num_heads, head_dim, max_blocks_per_seq, block_size,
                    partition_size):
    """(part_max, part_sum, part_out) float32 views of a split workspace."""
    lmax = max_blocks_per_seq * block_size
    NP = -(-lmax // partition_size)
    rows = num_seqs * num_heads * NP
    up = lambda x: (x + 255) // 256 * 256
    f = workspace.view(torch.uint8)
    o_max, o_sum = 0, up(rows * 4)
    o_out = o_sum + up(rows * 4)
    view = lambda off, n: f[off:off + 4 * n].view(torch.float32)
    return (view(o_max, rows).view(num_seqs, num_heads, NP), view(o_sum, rows).view(num_seqs, num_heads, NP),
            view(o_out, rows * head_dim).view(num_seqs, num_heads, NP, head_dim))


def lse_merge(part_out, part_max, part_sum, context_lens, partition_size, out=None, out_dtype=torch.float32):
    """Merge per-partition (max, sum, normalised output) by log-sum-exp.
    part_out [B, Hq, NP, D], part_max / part_sum [B, Hq, NP] (float32)."""
    _on_gpu(part_out, part_max, part_sum, context_lens)
    for t in (part_out, part_max, part_sum):
        _need(t.dtype == torch.float32 and t.is_contiguous(), "partials must be contiguous float32")
    _need(context_lens.dtype == torch.int32 and context_lens.is_contiguous(), "context_lens must be int32")
    B, Hq, NP, D = part_out.shape
    _need(part_max.shape == (B, Hq, NP) and part_sum.shape == (B, Hq, NP), "partial shapes differ")
    if out is None:
        out = torch.zeros((B, Hq, D), dtype=out_dtype, device=part_out.device)
    st = load().pa_lse_merge(_ptr(out), _DT[out.dtype], _ptr(part_out), _ptr(part_max), _ptr(part_sum),
                             _ptr(context_lens), B, Hq, D, NP, int(partition_size), _stream(part_out))
    _check(st, "pa_lse_merge")
    return out


def stream_read(data, sink):
    """Read all of `data` (a contiguous GPU tensor) once; see pa_stream_read."""
    _on_gpu(data, sink)
    _need(data.is_contiguous() and sink.is_contiguous(), "tensors must be contiguous")
    _need(sink.dtype == torch.int32 and sink.numel() >= 64, "sink must hold 64 int32")
    nbytes = data.numel() * data.element_size()
    _check(load().pa_stream_read(_ptr(data), nbytes, _ptr(sink), _stream(data)), "pa_stream_read")
