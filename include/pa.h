/*
 * pa.h - C ABI of libpa: paged decode attention and the KV-cache scatter on
 * MI355X (gfx950).
 *
 * The operations follow the pages' statement of the problem:
 *   - KV cache per layer laid out [num_blocks, block_size, num_kv_heads,
 *     head_dim]; physical blocks are not contiguous per sequence and are
 *     found through a per-sequence block table ("vLLM PagedAttention深度解析
 *     与工程实践" §3.1 Block Table and §4.1 注意力计算的修改;
 *     lqnn.cn/news/170268 §2.2).
 *   - Each decode step appends the new token's K/V into a free slot of the
 *     sequence's current block or of a newly taken block (same pages, §二
 *     and §2.2): pa_reshape_and_cache.
 *   - Decode attention walks the block table, scores the query against every
 *     cached token, weights V by softmax(q·Kᵀ·scale) and writes the output
 *     ("vLLM PagedAttention深度解析与工程实践" §二 formula;
 *     lqnn.cn/news/170268 §2.3 three steps): pa_decode.
 *   - The long-context variant accumulates per context partition and then
 *     merges ("vLLM PagedAttention深度解析与工程实践" §4.1, the v2 kernel):
 *     pa_decode_split, with the merge exported as pa_lse_merge.
 *
 * Conventions for every entry point:
 *   - All data pointers are DEVICE memory owned by the caller; tensors are
 *     dense and row-major in the layouts stated below, 16-byte aligned.
 *     The library allocates nothing and keeps no data between calls. It
 *     does cache, per process, facts of each device it has run on (the
 *     number of compute units, each kernel's resident workgroups, the
 *     address of pa_decode_split_noalloc's scratch array), under a lock;
 *     they never change while the process runs.
 *   - Calls are asynchronous on `stream` (a hipStream_t, NULL = the default
 *     stream); nothing is synchronised. Calls that write the same buffers
 *     race if they overlap on different streams.
 *   - Host-side validation happens before any launch. A non-zero status
 *     means nothing was launched and nothing was written; pa_last_error()
 *     gives the detail (thread-local, valid until the next call on the
 *     same thread). No C++ exception crosses this boundary.
 *   - Device data the host cannot see without a synchronisation (block ids,
 *     context lengths, slots) are the caller's contract; the kernels still
 *     never touch memory outside the buffers: a block id outside
 *     [0, num_blocks) makes its tokens count as absent, a context length is
 *     clamped to [0, max_blocks_per_seq * block_size], a slot outside
 *     [0, num_blocks * block_size) is skipped.
 *   - Element types: KV cache, query and new K/V share `dtype`
 *     (PA_F16 or PA_BF16). Outputs may be that type (rounded to nearest
 *     even from fp32) or PA_F32. All accumulation is fp32
 *     (lqnn.cn/news/170268 §6: half-precision accumulation of the scores
 *     degrades long sequences). The softmax weights enter the p·v
 *     products on the matrix cores as 16-bit values: for fp16 caches in
 *     the prefill kernel (pa_prefill, pa_prefill_shared_prefix, and decode
 *     at head_dim 256) one rounded fp16 value per weight, whose sum is the
 *     softmax denominator (an exact average of the V rows with weights
 *     within 2^-10 relative of the true ones); otherwise hi + lo halves,
 *     about 16 bits of each weight.
 *   - Supported shapes: head_dim in {64, 80, 96, 128, 256}; block_size in
 *     {8, 16, 32, 64}; num_heads a multiple of num_kv_heads (query head h
 *     reads kv head h / (num_heads / num_kv_heads)), at most 16 query heads
 *     per kv head at head_dim 256; one block of a cache (block_size *
 *     num_kv_heads * head_dim elements) below 128 MiB. At head_dim 256 the
 *     decode calls run on the prefill kernel (one new token per sequence):
 *     the fused-append calls then launch the scatter first, and the
 *     shared-prefix calls read the prefix per sequence; the results are
 *     those of the other widths' paths.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PA_OK = 0,
    PA_ERR_NULL = 1,         /* a required pointer is NULL */
    PA_ERR_SHAPE = 2,        /* sizes out of range or inconsistent */
    PA_ERR_DTYPE = 3,        /* element type not accepted here */
    PA_ERR_UNSUPPORTED = 4,  /* valid request without a compiled instance */
    PA_ERR_WORKSPACE = 5,    /* workspace NULL, too small or misaligned */
    PA_ERR_LAUNCH = 6,       /* the HIP runtime refused the launch */
    PA_ERR_ALIGNMENT = 7     /* a data pointer is not 16-byte aligned */
} pa_status;

typedef enum { PA_F16 = 0, PA_BF16 = 1, PA_F32 = 2 } pa_dtype;

/*
 * pa_reshape_and_cache - store each new token's K and V in its cache slot.
 *
 *   key, value        [num_tokens, num_kv_heads, head_dim] of `dtype`; token n
 *                     starts at key + n * key_token_stride elements (use
 *                     num_kv_heads * head_dim for a dense tensor; larger
 *                     strides let K/V be read straight out of a fused QKV
 *                     projection). Heads and dims of one token are dense.
 *   key_cache,
 *   value_cache       [num_blocks, block_size, num_kv_heads, head_dim], written
 *                     in place.
 *   slot_mapping      int64 [num_tokens]; slot s means block s / block_size,
 *                     row s % block_size. s < 0 marks padding: the token is
 *                     skipped. Slots must be distinct (else the result for
 *                     the duplicated slot is one of the writers, unspecified).
 *
 * Bit-exact copy; no arithmetic on the elements. num_tokens == 0 is a no-op.
 */
pa_status pa_reshape_and_cache(const void* key, const void* value,
                               void* key_cache, void* value_cache,
                               const int64_t* slot_mapping, int num_tokens,
                               int64_t key_token_stride, int64_t value_token_stride,
                               int num_kv_heads, int head_dim, int num_blocks,
                               int block_size, pa_dtype dtype, void* stream);

/*
 * pa_copy_blocks - copy-on-write block copy ("优化大模型推理：PagedAttention 如何
 * 实现 GPU 显存高效管理", 写时复制: sequences share physical blocks until one
 * of them is about to write into a shared block, which it first copies).
 *
 *   key_cache, value_cache  [num_blocks, block_size, num_kv_heads, head_dim]
 *                     fp16/bf16 (dtype), written in place.
 *   block_mapping     int64 [num_pairs, 2], device: row n = (src, dst). After
 *                     the call block dst of both caches holds what block src
 *                     held before it (all rows and heads, bitwise).
 * Pairs with an id outside [0, num_blocks) are skipped. Caller contract (not
 * checked on the device): the destinations are distinct and none is also a
 * source; otherwise the copies race and the result is unspecified. One
 * launch on `stream`; no host synchronisation.
 */
pa_status pa_copy_blocks(void* key_cache, void* value_cache, const int64_t* block_mapping,
                         int num_pairs, int num_kv_heads, int head_dim, int block_size,
                         int num_blocks, pa_dtype dtype, void* stream);

/*
 * pa_swap_blocks - copy blocks between two pools, one of which may live in
 * pinned host memory ("vLLM 核心：PagedAttention 与 Continuous Batching" §5,
 * strategy 1: a preempted request's KV blocks are copied to CPU memory and
 * back when it resumes).
 *
 *   dst_key_cache, dst_value_cache  [dst_num_blocks, block_size,
 *                     num_kv_heads, head_dim]: the destination pool.
 *   src_key_cache, src_value_cache  [src_num_blocks, ...]: the source pool.
 *   block_mapping     int64 [num_pairs, 2]: row n = (src block, dst block).
 * Each pool and the mapping must be device memory or pinned host memory the
 * device can address (e.g. hipHostMalloc'd); anything else returns
 * PA_ERR_UNSUPPORTED before any launch. Pairs with an id outside their pool
 * are skipped; destinations must be distinct (caller contract). One kernel
 * launch on `stream` moves all pairs; for a host pool its bandwidth is that
 * of the host link.
 */
pa_status pa_swap_blocks(void* dst_key_cache, void* dst_value_cache, int dst_num_blocks,
                         const void* src_key_cache, const void* src_value_cache,
                         int src_num_blocks, const int64_t* block_mapping, int num_pairs,
                         int num_kv_heads, int head_dim, int block_size, pa_dtype dtype,
                         void* stream);

/*
 * pa_decode - one query token per sequence attends over its paged context,
 * in a single launch (no workspace).
 *
 *   out               [num_seqs, num_heads, head_dim] of `out_dtype`
 *                     (PA_F32 or the cache's dtype).
 *   query             [num_seqs, num_heads, head_dim] of `kv_dtype`.
 *   key_cache,
 *   value_cache       [num_blocks, block_size, num_kv_heads, head_dim].
 *   block_tables      int32 [num_seqs, max_blocks_per_seq]; entry j of row i
 *                     is the physical block of sequence i's logical block j.
 *                     Only the first ceil(L_i / block_size) entries are read.
 *   context_lens      int32 [num_seqs]; L_i counts every cached token of
 *                     sequence i, the one written this step included.
 *   scale             multiplies q·k before the softmax (1/sqrt(head_dim) in
 *                     the usual attention).
 *
 * out[i, h, :] = Σ_t softmax_t(scale · q_ih · K_i[t]) · V_i[t] over t < L_i;
 * a sequence with L_i == 0 gets zeros. Slots at or past L_i in the last
 * block are never read, whatever they hold.
 */
pa_status pa_decode(void* out, pa_dtype out_dtype, const void* query,
                    const void* key_cache, const void* value_cache,
                    const int32_t* block_tables, const int32_t* context_lens,
                    int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                    int block_size, int max_blocks_per_seq, int num_blocks,
                    float scale, pa_dtype kv_dtype, void* stream);

/*
 * Workspace of pa_decode_split, in bytes, for these sizes. With
 * NP = ceil(max_blocks_per_seq * block_size / partition_size) it holds, each
 * region starting on a 256-byte boundary in this order:
 *   part_max  float [num_seqs, num_heads, NP]
 *   part_sum  float [num_seqs, num_heads, NP]
 *   part_out  float [num_seqs, num_heads, NP, head_dim]
 * Returns 0 for invalid sizes.
 */
size_t pa_decode_split_workspace_bytes(int num_seqs, int num_heads, int head_dim,
                                       int max_blocks_per_seq, int block_size,
                                       int partition_size);

/*
 * pa_decode_split - pa_decode computed as context partitions and a merge.
 *
 * Same arguments and result as pa_decode, plus:
 *   partition_size    tokens per partition, a positive multiple of
 *                     block_size; partition p of sequence i covers logical
 *                     tokens [p*P, min((p+1)*P, L_i)).
 *   workspace         device buffer of at least
 *                     pa_decode_split_workspace_bytes(...) bytes, 256-byte
 *                     aligned, owned by the caller; its contents on entry are
 *                     ignored and on exit unspecified. Calls that share a
 *                     workspace must not overlap in time.
 *
 * Two launches on `stream`: pa_decode_partitions, then pa_lse_merge over the
 * workspace (the merge skips sequences that one workgroup covered whole).
 */
pa_status pa_decode_split(void* out, pa_dtype out_dtype, const void* query,
                          const void* key_cache, const void* value_cache,
                          const int32_t* block_tables, const int32_t* context_lens,
                          int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                          int block_size, int max_blocks_per_seq, int num_blocks,
                          float scale, pa_dtype kv_dtype, int partition_size,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_split_noalloc - pa_decode_split for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.
 *
 * Same arguments and result as pa_decode_split, without the workspace: the
 * partitions' rows go to a scratch array that the library keeps in device
 * memory, PA_DECODE_NOALLOC_MAX_WORKSPACE bytes on each GPU it runs on,
 * from the first call on that GPU until the process ends. Sizes whose
 * pa_decode_split_workspace_bytes(...) exceeds that return PA_ERR_WORKSPACE
 * before anything touches the device. Nothing is allocated: no hipMalloc,
 * no hipFree, no allocating library call (the first call on a device looks
 * up the array's address once). Every call on one GPU shares its array,
 * which keeps the last call's partial rows; nothing in it needs to start at
 * zero. Calls that overlap in time on one GPU (on different streams, or
 * from different host threads) race on the array and give unspecified
 * results: serialise them, e.g. on one stream. Two launches on `stream`, as
 * pa_decode_split.
 */
#define PA_DECODE_NOALLOC_MAX_WORKSPACE ((size_t)32 << 20)
pa_status pa_decode_split_noalloc(void* out, pa_dtype out_dtype, const void* query,
                                  const void* key_cache, const void* value_cache,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                  int block_size, int max_blocks_per_seq, int num_blocks,
                                  float scale, pa_dtype kv_dtype, int partition_size,
                                  void* stream);

/*
 * pa_prefill - causal attention of each sequence's new tokens over its paged
 * context, the prefill that follows a prefix-cache hit (lqnn.cn/news/170268
 * §3.4: hit blocks enter the request's block table as they are, prefill
 * runs from the first missing position and takes new blocks as it goes;
 * §3.2: hits are whole blocks; §1.1: a token attends to itself and every
 * earlier token).
 *
 *   out          [num_tokens, num_heads, head_dim] of out_dtype: row r of
 *                query's attention result.
 *   query        [num_tokens, num_heads, head_dim] in kv_dtype: the new
 *                tokens of every sequence, packed in sequence order.
 *   query_start  int32 [num_seqs + 1], ascending, query_start[0] = 0 and
 *                query_start[num_seqs] = num_tokens: sequence i's new tokens
 *                are rows query_start[i] .. query_start[i+1] - 1, S_i of
 *                them, with S_i <= max_query_len.
 *   context_lens int32 [num_seqs]: L_i = cached tokens + S_i. New token t of
 *                sequence i sits at position L_i - S_i + t, and its K/V must
 *                already be in the caches there (pa_reshape_and_cache with
 *                the new tokens' slots, before this call).
 *   key_cache, value_cache, block_tables, the shape arguments, scale and
 *                kv_dtype: as for pa_decode; num_heads / num_kv_heads <= 16.
 * Row t of sequence i is softmax(scale · K q) · V over positions
 * 0 .. L_i - S_i + t. Rows of a sequence with S_i > L_i whose position is
 * negative, and rows of a sequence with L_i = 0, are zero. Rows past
 * max_query_len of a sequence (a caller error) are not written; the device
 * data query_start and context_lens are not checked. Nothing is allocated;
 * one launch, one workgroup per (sequence, kv head, 4 or 8 x 16/G new
 * tokens) over the whole context on the matrix cores (G = num_heads /
 * num_kv_heads).
 */
pa_status pa_prefill(void* out, pa_dtype out_dtype, const void* query, const void* key_cache,
                     const void* value_cache, const int32_t* block_tables,
                     const int32_t* context_lens, const int32_t* query_start, int num_seqs,
                     int num_tokens, int max_query_len, int num_heads, int num_kv_heads,
                     int head_dim, int block_size, int max_blocks_per_seq, int num_blocks,
                     float scale, pa_dtype kv_dtype, void* stream);

/*
 * pa_prefill_shared_prefix - pa_prefill for sequences whose contexts start
 * with the same cached blocks, e.g. requests that share a system prompt
 * (lqnn.cn/news/170268 §3.4 and §4.3: many requests hit the same cached
 * prompt blocks, the shared blocks counted once).
 *
 * Same arguments and result as pa_prefill (up to rounding order), plus:
 *   shared_prefix_tokens  positions every sequence shares, a multiple of
 *                     block_size and at most max_blocks_per_seq * block_size;
 *                     0 is allowed (nothing shared).
 * The new tokens of all sequences form one list of rows; a workgroup takes
 * 4 or 8 x 16/G consecutive rows, whichever sequences they belong to, reads
 * the shared positions once for all of them (through row 0 of
 * block_tables), then each of its sequences' own positions past the prefix
 * for that sequence's rows. Without sharing the shared blocks are read once
 * per sequence and kv head instead, and a sequence whose new tokens do not
 * fill its workgroups leaves waves idle.
 * Caller contract (not checked on the device): for every sequence i,
 * block_tables[i][j] == block_tables[0][j] for
 * j < shared_prefix_tokens / block_size, and context_lens[i] >=
 * shared_prefix_tokens. max_query_len is not used for the grid (num_tokens
 * is). One launch; nothing is allocated.
 */
pa_status pa_prefill_shared_prefix(void* out, pa_dtype out_dtype, const void* query,
                                   const void* key_cache, const void* value_cache,
                                   const int32_t* block_tables, const int32_t* context_lens,
                                   const int32_t* query_start, int num_seqs, int num_tokens,
                                   int max_query_len, int num_heads, int num_kv_heads,
                                   int head_dim, int block_size, int max_blocks_per_seq,
                                   int num_blocks, float scale, pa_dtype kv_dtype,
                                   int shared_prefix_tokens, void* stream);

/*
 * pa_decode_split_append - one decode step's scatter and attention in the
 * launches of pa_decode_split ("vLLM PagedAttention深度解析与工程实践" §二:
 * each step appends the new token's K/V, then attends over the sequence).
 *
 * Same arguments as pa_decode_split (the caches are written), plus the step's
 * new rows, one token per sequence:
 *   new_key, new_value  [num_seqs, num_kv_heads, head_dim] in kv_dtype, token
 *                     i at element offset i * new_*_token_stride (16-byte
 *                     aligned, strides >= num_kv_heads*head_dim and multiples
 *                     of 8, so fused QKV buffers can be passed directly).
 *   slot_mapping      int64 [num_seqs]: the cache slot of sequence i's new
 *                     token; negative = no token (padding).
 * Effect: pa_reshape_and_cache(new_key, new_value, key_cache, value_cache,
 * slot_mapping, num_seqs, ...) followed by pa_decode_split(...), with the
 * same result up to rounding order, provided that, for every sequence with a
 * slot in [0, num_blocks*block_size) and L_i >= 1, that slot is the one its
 * block table gives position L_i - 1 (block_tables[i][(L_i-1)/block_size] *
 * block_size + (L_i-1) % block_size): the new token is the last one
 * attended to. The workgroups of the partition that holds position L_i - 1
 * take the token's rows from new_key/new_value rather than from the cache,
 * and store them into the slot; slots outside the cache are skipped, as the
 * scatter skips them. Not checked on the device.
 */
pa_status pa_decode_split_append(void* out, pa_dtype out_dtype, const void* query,
                                 void* key_cache, void* value_cache,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 const void* new_key, const void* new_value,
                                 const int64_t* slot_mapping, int64_t new_key_token_stride,
                                 int64_t new_value_token_stride, int num_seqs, int num_heads,
                                 int num_kv_heads, int head_dim, int block_size,
                                 int max_blocks_per_seq, int num_blocks, float scale,
                                 pa_dtype kv_dtype, int partition_size, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* The partition launch of pa_decode_split_append on its own (the merge is
 * pa_lse_merge), as pa_decode_partitions is for pa_decode_split. */
pa_status pa_decode_partitions_append(void* out, pa_dtype out_dtype, const void* query,
                                      void* key_cache, void* value_cache,
                                      const int32_t* block_tables,
                                      const int32_t* context_lens, const void* new_key,
                                      const void* new_value, const int64_t* slot_mapping,
                                      int64_t new_key_token_stride,
                                      int64_t new_value_token_stride, int num_seqs,
                                      int num_heads, int num_kv_heads, int head_dim,
                                      int block_size, int max_blocks_per_seq, int num_blocks,
                                      float scale, pa_dtype kv_dtype, int partition_size,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_partitions - the first launch of pa_decode_split on its own.
 *
 * Same arguments as pa_decode_split. One workgroup handles one partition of
 * one (sequence, head) - of two adjacent heads when the grid is large
 * compared with the device, and of one (sequence, kv head) when 2..16 query
 * heads share a kv head; when the grid is large a grouped-query workgroup
 * may walk a group of consecutive partitions (a sequence's n partitions
 * then form ceil(n / k) groups of nearly equal size, k = 2 or 4, group i
 * starting at partition floor(i * n / groups)). Every partition
 * p < ceil(L_i / partition_size) of every row gets its workspace row:
 * part_max = the largest scaled logit (natural-log units), part_sum =
 * Σ exp(s - part_max), part_out = the normalised partial output, over the
 * partition's tokens - or over a group of consecutive partitions, whose
 * first row then holds the group and whose other rows are marked empty
 * (part_max = -inf, part_sum = 0, part_out not written). A sequence that one
 * workgroup covered whole (L_i <= partition_size, or within one group) also
 * gets its final output in `out`. pa_lse_merge over the workspace then
 * gives `out` for every row.
 */
pa_status pa_decode_partitions(void* out, pa_dtype out_dtype, const void* query,
                               const void* key_cache, const void* value_cache,
                               const int32_t* block_tables, const int32_t* context_lens,
                               int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                               int block_size, int max_blocks_per_seq, int num_blocks,
                               float scale, pa_dtype kv_dtype, int partition_size,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Shared-prefix variants. When every sequence of the batch begins with the
 * same physical blocks - a prompt prefix cached once and referenced by all
 * tables ("vLLM 核心：PagedAttention 与 Continuous Batching" §3 Prefix
 * Caching; lqnn.cn/news/170268 §3.2-§3.4) - the partitions covering that
 * prefix are computed once per 64 or 128 query rows: one workgroup takes
 * that many sequences x G query heads of a kv head (G = num_heads /
 * num_kv_heads, at most 16; 128 rows at head_dim 128) and one prefix
 * partition, and reads each prefix block once for all of them on the matrix
 * cores. The remaining partitions, the workspace and the merge are those of
 * pa_decode_split, and the result is the same up to rounding order.
 *
 *   shared_prefix_tokens  tokens every sequence shares; a multiple of
 *                     partition_size (hence of block_size); 0 gives plain
 *                     pa_decode_partitions / pa_decode_split.
 * Caller contract (not checked on the device): for every sequence i,
 * block_tables[i][j] == block_tables[0][j] for j < shared_prefix_tokens /
 * block_size, and context_lens[i] >= shared_prefix_tokens. The prefix blocks
 * are read through row 0 of block_tables.
 */
pa_status pa_decode_partitions_shared_prefix(void* out, pa_dtype out_dtype, const void* query,
                                             const void* key_cache, const void* value_cache,
                                             const int32_t* block_tables,
                                             const int32_t* context_lens, int num_seqs,
                                             int num_heads, int num_kv_heads, int head_dim,
                                             int block_size, int max_blocks_per_seq,
                                             int num_blocks, float scale, pa_dtype kv_dtype,
                                             int partition_size, int shared_prefix_tokens,
                                             void* workspace, size_t workspace_bytes,
                                             void* stream);

pa_status pa_decode_split_shared_prefix(void* out, pa_dtype out_dtype, const void* query,
                                        const void* key_cache, const void* value_cache,
                                        const int32_t* block_tables,
                                        const int32_t* context_lens, int num_seqs,
                                        int num_heads, int num_kv_heads, int head_dim,
                                        int block_size, int max_blocks_per_seq, int num_blocks,
                                        float scale, pa_dtype kv_dtype, int partition_size,
                                        int shared_prefix_tokens, void* workspace,
                                        size_t workspace_bytes, void* stream);

/*
 * pa_lse_merge - combine per-partition results (the second launch of
 * pa_decode_split).
 *
 *   part_max  float [num_seqs, num_heads, max_partitions]: m_p, the largest
 *             scaled logit scale·q·k of partition p (natural-log units).
 *   part_sum  float [num_seqs, num_heads, max_partitions]: l_p = Σ exp(s - m_p).
 *   part_out  float [num_seqs, num_heads, max_partitions, head_dim]:
 *             o_p = Σ exp(s - m_p) v / l_p. A partition with m_p = -inf is
 *             empty: it adds nothing and its o_p is not read.
 *   context_lens  int32 [num_seqs]; sequence i uses partitions
 *             p < ceil(L_i / partition_size).
 *
 * With M = max_p m_p and w_p = l_p exp(m_p - M):
 * out = Σ_p w_p o_p / Σ_p w_p over the np_i = ceil(L_i / partition_size)
 * partitions of sequence i (at most max_partitions). Every row of `out` is
 * written: a sequence with one partition gets o_0 as it is (the merge of a
 * single partition), one with L_i <= 0 gets zeros. (The split calls run the
 * same kernel but leave single-partition rows to their partition launch,
 * which wrote the final output there.)
 */
pa_status pa_lse_merge(void* out, pa_dtype out_dtype, const float* part_out,
                       const float* part_max, const float* part_sum,
                       const int32_t* context_lens, int num_seqs, int num_heads,
                       int head_dim, int max_partitions, int partition_size,
                       void* stream);

/*
 * pa_stream_read - measurement aid: read every byte of a device buffer once
 * with the 16-byte non-temporal loads the attention kernels use, writing
 * (practically) nothing. Timed over a buffer much larger than the
 * last-level cache it gives the device's streaming-read ceiling, the
 * measured counterpart of the HBM peak that the attention kernels' bandwidth
 * is compared with.
 *   data   device buffer, 16-byte aligned, bytes a multiple of 16.
 *   sink   device buffer of at least 64 uint32 (almost never written).
 */
pa_status pa_stream_read(const void* data, size_t bytes, uint32_t* sink, void* stream);

/* Static text for a status code. */
const char* pa_status_string(pa_status s);

/* Detail of the last failure on this thread ("" if none). */
const char* pa_last_error(void);

/* Library version, "major.minor.patch". */
const char* pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
