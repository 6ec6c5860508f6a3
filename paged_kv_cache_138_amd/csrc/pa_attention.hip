// Paged decode attention: pa_decode, the split path (pa_decode_split,
// pa_decode_partitions, their shared-prefix and fused-append forms) and
// pa_lse_merge.
//
// What is computed ("vLLM PagedAttention深度解析与工程实践" §二 formula and
// §4.1; lqnn.cn/news/170268 §2.3 and §6): for sequence i and query head h,
// out = softmax(scale · K_i q_ih) · V_i over the sequence's first L_i logical
// tokens, whose rows sit in physical blocks named by the block table. Slots
// at or past L_i in the last block are never read.
//
// The kernels live in pa_attn_mha.h (one head per workgroup) and
// pa_attn_gqa.h (matrix cores); their instances are compiled in the
// pa_inst_*.hip files, in parallel, and reached through pa_kernels.h.
#include "pa_attn_args.h"
#include "pa_kernels.h"
#include "pa_merge.h"
#include "pa_device.h"
#include "pa_host.h"

#include <math.h>

#include <algorithm>
#include <mutex>
#include <unordered_map>

namespace pa {
namespace {


struct MergeArgs {
    void* out;
    const float* part_out;
    const float* part_max;
    const float* part_sum;
    const int32_t* context_lens;
    int num_seqs;
    int num_heads;
    int max_partitions;
    int partition_size;
    // rows of sequences with at most this many partitions are left alone:
    // the split paths' partition launch wrote their output (one workgroup
    // covered the whole context); 0 writes every row (pa_lse_merge). Above
    // 1, partitions were walked in ceil(np / skip_parts) groups of nearly
    // equal size, and only the groups' first rows are read.
    int skip_parts;
};

// A row (one query head of one sequence) with np <= 1 partitions: whether
// the merge writes it, and the element it writes (np = 1: the partition's
// output o_0 as it is, the merge of one partition; np = 0: zero).
__device__ __forceinline__ bool merge_trivial_row(const MergeArgs& a, int np, size_t r, int D,
                                                  int d, float* v) {
    if (np > 1) return false;
    *v = np == 1 ? a.part_out[r * D + d] : 0.f;
    return true;
}

// 256 threads merge 1024 / head_dim workspace rows (row = one query head of
// one sequence), four consecutive output elements per thread, each
// partition's four read by one 16-byte load.
template <class OUT, int D>
__global__ __launch_bounds__(256) void lse_merge_kernel(MergeArgs a) {
    constexpr int TPR = D / 4;      // threads per row
    constexpr int RPW = 256 / TPR;  // rows per workgroup
    const int row = blockIdx.x * RPW + threadIdx.x / TPR;
    const int d = (threadIdx.x % TPR) * 4;
    if (row >= a.num_seqs * a.num_heads) return;
    const int seq = row / a.num_heads;
    int L = a.context_lens[seq];
    if (L < 0) L = 0;
    int np = (int)(((int64_t)L + a.partition_size - 1) / a.partition_size);
    if (np > a.max_partitions) np = a.max_partitions;
    if (a.skip_parts > 0 && np <= a.skip_parts) return;
    const size_t r = (size_t)row * a.max_partitions;
    f32x4 o;
    if (np <= 1) {  // the merge of one partition is its output; of none, zeros
        o = np == 1 ? *(const f32x4*)(a.part_out + r * D + d) : f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
        o = merge_row_element4(a.part_max + r, a.part_sum + r, a.part_out + r * D + d, np, D,
                               a.skip_parts > 1 ? a.skip_parts : 1);
    }
    const size_t e = (size_t)row * D + d;
    OUT::store2(a.out, e, o[0], o[1]);
    OUT::store2(a.out, e + 2, o[2], o[3]);
}

// head_dim 80 and 96: one row per wavefront, each lane merging the
// elements lane and lane + 64 of it.
template <class OUT, int D>
__global__ __launch_bounds__(256) void lse_merge_wave_kernel(MergeArgs a) {
    static_assert(D <= 128, "two elements per lane at most");
    const int row = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    if (row >= a.num_seqs * a.num_heads) return;
    const int seq = row / a.num_heads;
    int L = a.context_lens[seq];
    if (L < 0) L = 0;
    int np = (int)(((int64_t)L + a.partition_size - 1) / a.partition_size);
    if (np > a.max_partitions) np = a.max_partitions;
    if (a.skip_parts > 0 && np <= a.skip_parts) return;
    const size_t r = (size_t)row * a.max_partitions;
#pragma unroll
    for (int d = lane; d < D; d += 64) {
        float o;
        if (!merge_trivial_row(a, np, r, D, d, &o))
            o = merge_row_element(a.part_max + r, a.part_sum + r, a.part_out + r * D + d, np, D,
                                  a.skip_parts > 1 ? a.skip_parts : 1);
        OUT::store(a.out, (size_t)row * D + d, o);
    }
}

// ---------------------------------------------------------------------------
// Host dispatch
// ---------------------------------------------------------------------------

typedef void (*merge_fn)(MergeArgs);

constexpr int kMaxGroupMfma = 16;

bool use_gqa(int num_heads, int num_kv_heads) {
    const int g = num_heads / num_kv_heads;
    return g >= 2 && g <= kMaxGroupMfma;
}

// Adjacent heads (log2, at most max_log2) whose row slices together are a
// whole number of 128-byte cache lines. A head slice of 160 or 192 bytes
// (head_dim 80, 96) shares a line with the next head's; workgroups that
// serve single heads then fetch those lines twice (measured on MI355X:
// 1.39x the algorithmic bytes at head_dim 80 with two heads per
// workgroup), while 4 (head_dim 80) or 2 (head_dim 96) heads together start
// and end on line boundaries.
int whole_line_heads_log2(int heads, int head_dim, int max_log2) {
    int hl = 0;
    while (((head_dim * 2) << hl) % 128 != 0 && hl < max_log2) ++hl;
    return ((head_dim * 2) << hl) % 128 == 0 && heads % (1 << hl) == 0 ? hl : 0;
}

// Query heads per workgroup of the MHA kernel on the split path (log2).
// One head per workgroup gives the finest work units, which matters when
// the grid is only a few times what the device holds at once (the last,
// ragged units then decide the end of the kernel). When the grid is many
// times larger - many sequences or long maximum contexts, where most of the
// (sequence, partition) rectangle may be empty - two adjacent heads per
// workgroup halve the workgroups to dispatch and read each block row's
// heads side by side. More heads are served when a partition holds fewer
// chunks than a head would get waves, so that no wave idles. The
// single-pass path keeps one head per workgroup, so that a sequence's
// context is spread over all the waves of its workgroup.
#ifndef PA_MHA_MIN_HEADS_LOG2
#define PA_MHA_MIN_HEADS_LOG2 0
#endif
int mha_heads_log2(int num_heads, int64_t rect_workgroups, int resident, bool split,
                   int head_dim, int block_size, int partition_size) {
    if (!split || num_heads % 2 != 0) return 0;
    int hl = rect_workgroups / 2 >= (int64_t)6 * resident ? 1 : 0;
    while (hl < PA_MHA_MIN_HEADS_LOG2 && (1 << hl) < kWaves && num_heads % (2 << hl) == 0) ++hl;
    const int chunk = mha_chunk_tokens(head_dim, block_size);
    while ((1 << hl) < kWaves && (kWaves >> hl) * chunk > partition_size &&
           num_heads % (2 << hl) == 0)
        ++hl;
    return std::max(hl, whole_line_heads_log2(num_heads, head_dim, 2));
}

#ifndef PA_GQA_HEADS
#define PA_GQA_HEADS 2
#endif
// kv heads per workgroup of the grouped-query kernel on the split path (log2)
int gqa_heads_log2(int num_kv_heads, int head_dim) {
    int hl = 0;
    while ((2 << hl) <= PA_GQA_HEADS && (2 << hl) <= kGqaWaves && num_kv_heads % (2 << hl) == 0)
        ++hl;
    int max_log2 = 0;
    while ((2 << max_log2) <= kGqaWaves) ++max_log2;
    return std::max(hl, whole_line_heads_log2(num_kv_heads, head_dim, max_log2));
}

// Consecutive partitions one grouped-query workgroup walks, at most (1, 2 or
// 4): a sequence's n partitions form ceil(n / k) groups of nearly equal
// size. Each workgroup writes one fp32 row per query head to the workspace; such
// stores, arriving while the device streams the cache at full bandwidth,
// cost far more time than their share of the bytes (measured on MI355X with
// 64 q / 8 kv heads, contexts of 1k-8k tokens: 452 / 431 / 416 us per launch
// for partitions walked in groups of 1 / 2 / 4). Grouping keeps the
// partition as the unit of the workspace and the merge; it is used while the
// grid of groups (for the longest table) still holds at least two rounds of
// the workgroups the device runs at once.
#ifndef PA_GQA_MAX_GROUP
#define PA_GQA_MAX_GROUP 4
#endif
// rounds of resident workgroups the grid of groups must still hold
#ifndef PA_GQA_GROUP_ROUNDS
#define PA_GQA_GROUP_ROUNDS 2
#endif
int gqa_group(int parts, int64_t units, int resident) {
    for (int k = PA_GQA_MAX_GROUP; k > 1; k /= 2)
        if (parts >= 2 * k &&
            units * ceil_div(parts, k) >= (int64_t)PA_GQA_GROUP_ROUNDS * resident)
            return k;
    return 1;
}

// Sequence slots of a split-path grid, whose units run (sequence slot, head
// or kv-head group, partition) with the group fastest. The dispatcher hands
// workgroup i to XCD i mod 8, so a (sequence, partition) block of, say, 20
// head groups starts on XCD (20 * block index) mod 8: with one slot per
// sequence, the sequence's parity alone would pick the XCDs that take each
// block's 4 extra units, and the even and odd sequences' lengths would load
// the XCDs unevenly. With slots = 1 (mod 8) the block index mod 8 is
// (partition + sequence) mod 8, so each sequence's partitions rotate over
// the XCDs. The padding slots' workgroups return at once. (Built with
// PA_SPLIT_SEQ_SLOTS=0 the grids keep one slot per sequence, for comparison.)
#ifndef PA_SPLIT_SEQ_SLOTS
#define PA_SPLIT_SEQ_SLOTS 1
#endif
int xcd_seq_slots(int num_seqs) {
    return PA_SPLIT_SEQ_SLOTS ? num_seqs + (9 - num_seqs % 8) % 8 : num_seqs;
}

// Waves per workgroup of the prefill kernel's shared-prefix mode (16 rows
// each; every wave reads every chunk from LDS, so more waves fetch each
// prefix row for more rows)
#ifndef PA_PREFILL_SHARED_WAVES
#define PA_PREFILL_SHARED_WAVES 8
#endif
int prefill_shared_waves(int head_dim) { return head_dim == 128 ? PA_PREFILL_SHARED_WAVES : 4; }

// The shared-prefix decode's prefix partitions: on the prefill kernel's
// prefix-only decode mode (1), whose workgroups read each prefix chunk once
// into LDS for 64 or 128 query rows, or on the grouped-query kernel's
// prefix mode (0, built for comparison), one 16-row MFMA tile per read.
#ifndef PA_PREFIX_ON_PREFILL
#define PA_PREFIX_ON_PREFILL 1
#endif

// Workgroups of fn that fit on the current device at once (at least 1).
int resident_workgroups(const void* fn, int threads) {
    static std::mutex mu;
    static std::unordered_map<const void*, int> per_cu;
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
    std::lock_guard<std::mutex> lock(mu);
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 1;
        cus[dev] = n > 0 ? n : 1;
    }
    auto it = per_cu.find(fn);
    if (it == per_cu.end()) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, threads, 0) != hipSuccess)
            n = 1;
        it = per_cu.emplace(fn, n > 0 ? n : 1).first;
    }
    return it->second * cus[dev];
}

// kernel and grid width (workgroups per sequence and partition)
attn_fn pick_kernel(pa_dtype kv, pa_dtype out, int d, int bs, int num_heads, int num_kv_heads,
                    int heads_log2, int* per_seq, int* threads) {
    *threads = kWaves * 64;
    if (use_gqa(num_heads, num_kv_heads)) {
        *per_seq = num_kv_heads;
        *threads = kGqaWaves * 64;
        return pick_gqa(kv, out, d, bs);
    }
    *per_seq = num_heads >> heads_log2;
    return pick_attn(kv, out, d, bs);
}

template <class OUT>
merge_fn pick_merge_d(int d) {
    switch (d) {
        case 64: return lse_merge_kernel<OUT, 64>;
        case 80: return lse_merge_wave_kernel<OUT, 80>;
        case 96: return lse_merge_wave_kernel<OUT, 96>;
        case 128: return lse_merge_kernel<OUT, 128>;
        case 256: return lse_merge_kernel<OUT, 256>;
    }
    return nullptr;
}

merge_fn pick_merge(pa_dtype out, int d) {
    switch (out) {
        case PA_F32: return pick_merge_d<OutF32>(d);
        case PA_F16: return pick_merge_d<OutF16>(d);
        case PA_BF16: return pick_merge_d<OutBF16>(d);
    }
    return nullptr;
}

struct DecodeShape {
    int num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
        num_blocks;
};

pa_status validate_decode(void* out, pa_dtype out_dtype, const void* query, const void* kc,
                          const void* vc, const int32_t* bt, const int32_t* cl,
                          const DecodeShape& s, float scale, pa_dtype kv_dtype) {
    PA_REQUIRE(s.num_seqs >= 0, PA_ERR_SHAPE, "num_seqs %d < 0", s.num_seqs);
    PA_REQUIRE(s.num_heads > 0 && s.num_kv_heads > 0, PA_ERR_SHAPE,
               "num_heads and num_kv_heads must be > 0");
    PA_REQUIRE(s.num_heads % s.num_kv_heads == 0, PA_ERR_SHAPE,
               "num_heads %d is not a multiple of num_kv_heads %d", s.num_heads,
               s.num_kv_heads);
    PA_REQUIRE(s.block_size > 0 && s.max_blocks_per_seq > 0 && s.num_blocks > 0,
               PA_ERR_SHAPE, "block_size, max_blocks_per_seq, num_blocks must be > 0");
    PA_REQUIRE((int64_t)s.max_blocks_per_seq * s.block_size <= (int64_t)1 << 30, PA_ERR_SHAPE,
               "max_blocks_per_seq * block_size too large");
    PA_REQUIRE(kv_dtype == PA_F16 || kv_dtype == PA_BF16, PA_ERR_DTYPE,
               "kv dtype must be PA_F16 or PA_BF16");
    PA_REQUIRE(out_dtype == PA_F32 || out_dtype == kv_dtype, PA_ERR_DTYPE,
               "out dtype must be PA_F32 or the kv dtype");
    PA_REQUIRE(isfinite(scale), PA_ERR_SHAPE, "scale must be finite");
    PA_REQUIRE(s.head_dim == 64 || s.head_dim == 80 || s.head_dim == 96 || s.head_dim == 128 ||
                   s.head_dim == 256,
               PA_ERR_UNSUPPORTED, "head_dim %d not in {64, 80, 96, 128, 256}", s.head_dim);
    PA_REQUIRE(s.head_dim != 256 || s.num_heads / s.num_kv_heads <= kMaxGroupMfma,
               PA_ERR_UNSUPPORTED, "head_dim 256 takes at most %d query heads per kv head",
               kMaxGroupMfma);
    // lanes of missing 16-byte slices (head_dim 80, 96) read past a block's
    // range with a fixed offset, which must stay past every block
    PA_REQUIRE((int64_t)s.block_size * s.num_kv_heads * s.head_dim * 2 < ((int64_t)1 << 27),
               PA_ERR_SHAPE, "a block of more than 128 MiB");
    PA_REQUIRE(s.block_size == 8 || s.block_size == 16 || s.block_size == 32 ||
                   s.block_size == 64,
               PA_ERR_UNSUPPORTED, "block_size %d not in {8, 16, 32, 64}", s.block_size);
    if (s.num_seqs == 0) return PA_OK;
    PA_REQUIRE(out && query && kc && vc && bt && cl, PA_ERR_NULL, "null pointer argument");
    PA_REQUIRE(aligned16(out) && aligned16(query) && aligned16(kc) && aligned16(vc),
               PA_ERR_ALIGNMENT, "out, query and caches must be 16-byte aligned");
    return PA_OK;
}

AttnArgs make_args(void* out, const void* query, const void* kc, const void* vc,
                   const int32_t* bt, const int32_t* cl, const DecodeShape& s, float scale) {
    AttnArgs a{};
    a.out = out;
    a.query = (const uint16_t*)query;
    a.key_cache = (const uint16_t*)kc;
    a.value_cache = (const uint16_t*)vc;
    a.block_tables = bt;
    a.context_lens = cl;
    a.num_seqs = s.num_seqs;
    a.num_heads = s.num_heads;
    a.num_kv_heads = s.num_kv_heads;
    a.max_blocks_per_seq = s.max_blocks_per_seq;
    a.num_blocks = s.num_blocks;
    a.scale_log2 = scale * kLog2e;
    return a;
}

// head_dim 256: the decode paths run on the prefill kernel in its decode
// mode (one new token per sequence, `nparts` partitions of
// a.partition_size), whose registers stretch to that width; the one-head
// and grouped-query decode kernels stop at 128.
pa_status launch_wide(AttnArgs a, const DecodeShape& s, pa_dtype kv_dtype, pa_dtype out_dtype,
                      int nparts, void* stream, const char* what) {
    attn_fn fn = pick_prefill_kernel(kv_dtype, out_dtype, s.head_dim, s.block_size, 4);
    PA_REQUIRE(fn, PA_ERR_UNSUPPORTED, "no kernel instance for this dtype/shape");
    a.query_start = nullptr;  // decode mode
    a.num_q_tiles = nparts;
    const int64_t grid = (int64_t)s.num_seqs * nparts * s.num_kv_heads;
    PA_REQUIRE(grid < ((int64_t)1 << 31), PA_ERR_SHAPE, "grid too large");
    if (grid == 0) return PA_OK;
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(4 * 64), 0, (hipStream_t)stream, a);
    return check_launch(what);
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }



struct SplitLayout {
    int np;
    size_t off_max, off_sum, off_out, total;
    int group;  // partitions one workgroup walked (set by the partition launch)
};

bool split_layout(int num_seqs, int num_heads, int head_dim, int max_blocks_per_seq,
                  int block_size, int partition_size, SplitLayout* lay) {
    if (num_seqs < 0 || num_heads <= 0 || head_dim <= 0 || max_blocks_per_seq <= 0 ||
        block_size <= 0 || partition_size <= 0)
        return false;
    const int64_t lmax = (int64_t)max_blocks_per_seq * block_size;
    const int np = (int)((lmax + partition_size - 1) / partition_size);
    const size_t rows = (size_t)num_seqs * num_heads * np;
    lay->np = np;
    lay->group = 1;
    lay->off_max = 0;
    lay->off_sum = lay->off_max + align256(rows * sizeof(float));
    lay->off_out = lay->off_sum + align256(rows * sizeof(float));
    lay->total = lay->off_out + align256(rows * head_dim * sizeof(float));
    return true;
}


}  // namespace
}  // namespace pa

using namespace pa;

extern "C" pa_status pa_decode(void* out, pa_dtype out_dtype, const void* query,
                               const void* key_cache, const void* value_cache,
                               const int32_t* block_tables, const int32_t* context_lens,
                               int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                               int block_size, int max_blocks_per_seq, int num_blocks,
                               float scale, pa_dtype kv_dtype, void* stream) {
    clear_error();
    const DecodeShape s{num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                        max_blocks_per_seq, num_blocks};
    pa_status st = validate_decode(out, out_dtype, query, key_cache, value_cache, block_tables,
                                   context_lens, s, scale, kv_dtype);
    if (st != PA_OK || num_seqs == 0) return st;
    if (head_dim == 256) {
        AttnArgs a = make_args(out, query, key_cache, value_cache, block_tables, context_lens, s,
                               scale);
        a.partition_size = max_blocks_per_seq * block_size;  // one partition per sequence
        a.max_partitions = 1;
        return launch_wide(a, s, kv_dtype, out_dtype, 1, stream, "pa_decode");
    }
    int per_seq = 0, threads = 0;
    const int hl = 0;  // one head per workgroup: its waves share the whole context
    attn_fn fn = pick_kernel(kv_dtype, out_dtype, head_dim, block_size, num_heads, num_kv_heads,
                             hl, &per_seq, &threads);
    PA_REQUIRE(fn, PA_ERR_UNSUPPORTED, "no kernel instance for this dtype/shape");
    AttnArgs a = make_args(out, query, key_cache, value_cache, block_tables, context_lens, s,
                           scale);
    a.heads_log2 = hl;
    a.partition_size = max_blocks_per_seq * block_size;  // one partition per sequence
    a.max_partitions = 1;
    const int64_t grid = (int64_t)num_seqs * per_seq;
    PA_REQUIRE(grid < ((int64_t)1 << 31), PA_ERR_SHAPE, "grid too large");
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(threads), 0, (hipStream_t)stream, a);
    return check_launch("pa_decode");
}

extern "C" size_t pa_decode_split_workspace_bytes(int num_seqs, int num_heads, int head_dim,
                                                  int max_blocks_per_seq, int block_size,
                                                  int partition_size) {
    SplitLayout lay;
    if (!split_layout(num_seqs, num_heads, head_dim, max_blocks_per_seq, block_size,
                      partition_size, &lay))
        return 0;
    return lay.total;
}

namespace {

// the decode step's new rows, for the fused-append calls
struct AppendRows {
    const void* new_key;
    const void* new_value;
    const int64_t* slot_mapping;
    int64_t key_stride, value_stride;  // elements between tokens
};

pa_status launch_partitions(void* out, pa_dtype out_dtype, const void* query,
                            const void* key_cache, const void* value_cache,
                            const int32_t* block_tables, const int32_t* context_lens,
                            const DecodeShape& s, float scale, pa_dtype kv_dtype,
                            int partition_size, int prefix_tokens, void* workspace,
                            size_t workspace_bytes, void* stream, const char* what,
                            SplitLayout* lay_out, const AppendRows* app = nullptr) {
    pa_status st = validate_decode(out, out_dtype, query, key_cache, value_cache, block_tables,
                                   context_lens, s, scale, kv_dtype);
    if (st != PA_OK) return st;
    PA_REQUIRE(partition_size > 0 && partition_size % s.block_size == 0, PA_ERR_SHAPE,
               "partition_size %d must be a positive multiple of block_size %d",
               partition_size, s.block_size);
    PA_REQUIRE(prefix_tokens >= 0 && prefix_tokens % partition_size == 0 &&
                   (int64_t)prefix_tokens <= (int64_t)s.max_blocks_per_seq * s.block_size,
               PA_ERR_SHAPE,
               "shared_prefix_tokens %d must be a multiple of partition_size %d and fit "
               "max_blocks_per_seq * block_size", prefix_tokens, partition_size);
    PA_REQUIRE(prefix_tokens == 0 || s.num_heads / s.num_kv_heads <= kMaxGroupMfma,
               PA_ERR_UNSUPPORTED, "shared-prefix mode needs num_heads / num_kv_heads <= %d",
               kMaxGroupMfma);
    SplitLayout lay;
    split_layout(s.num_seqs, s.num_heads, s.head_dim, s.max_blocks_per_seq, s.block_size,
                 partition_size, &lay);
    *lay_out = lay;
    if (s.num_seqs == 0) return PA_OK;
    PA_REQUIRE(workspace, PA_ERR_WORKSPACE, "workspace is NULL");
    PA_REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, PA_ERR_WORKSPACE,
               "workspace must be 256-byte aligned");
    PA_REQUIRE(workspace_bytes >= lay.total, PA_ERR_WORKSPACE,
               "workspace has %zu bytes, needs %zu", workspace_bytes, lay.total);
    char* ws = (char*)workspace;
    if (s.head_dim == 256) {
        // the step's scatter first, then every partition of every context
        // (a shared prefix is read per sequence: same results)
        if (app) {
            st = pa_reshape_and_cache(app->new_key, app->new_value, (void*)key_cache,
                                      (void*)value_cache, app->slot_mapping, s.num_seqs,
                                      app->key_stride, app->value_stride, s.num_kv_heads,
                                      s.head_dim, s.num_blocks, s.block_size, kv_dtype, stream);
            if (st != PA_OK) return st;
        }
        AttnArgs a = make_args(out, query, key_cache, value_cache, block_tables, context_lens, s,
                               scale);
        a.part_max = (float*)(ws + lay.off_max);
        a.part_sum = (float*)(ws + lay.off_sum);
        a.part_out = (float*)(ws + lay.off_out);
        a.partition_size = partition_size;
        a.max_partitions = lay.np;
        return launch_wide(a, s, kv_dtype, out_dtype, lay.np, stream, what);
    }
    const int prefix_parts = prefix_tokens / partition_size;
    int per_seq = 0, threads = 0;
    attn_fn fn = pick_kernel(kv_dtype, out_dtype, s.head_dim, s.block_size, s.num_heads,
                             s.num_kv_heads, 0, &per_seq, &threads);
    int hl = 0, group = 1;
    if (fn && !use_gqa(s.num_heads, s.num_kv_heads)) {
        const int64_t rect = (int64_t)s.num_seqs * s.num_heads * (lay.np - prefix_parts);
        hl = mha_heads_log2(s.num_heads, rect, resident_workgroups((const void*)fn, threads),
                            true, s.head_dim, s.block_size, partition_size);
        per_seq = s.num_heads >> hl;
    } else if (fn) {
        hl = gqa_heads_log2(s.num_kv_heads, s.head_dim);
        per_seq = s.num_kv_heads >> hl;
        // (not after a shared prefix, whose partitions stay single: the
        // merge then reads every row)
        if (prefix_parts == 0)
            group = gqa_group(lay.np, (int64_t)s.num_seqs * per_seq,
                              resident_workgroups((const void*)fn, threads));
    }
    attn_fn pfn = nullptr;
    int pthreads = 0, prows = 0;  // prefix launch: threads, sequences per workgroup
    if (prefix_tokens > 0) {
        const int G = s.num_heads / s.num_kv_heads;
        if (PA_PREFIX_ON_PREFILL) {
            const int waves = prefill_shared_waves(s.head_dim);
            pfn = pick_prefill_shared_kernel(kv_dtype, out_dtype, s.head_dim, s.block_size,
                                             waves);
            pthreads = waves * 64;
            prows = waves * PA_PREFILL_SHARED_TR * (16 / G);
        } else {
            pfn = pick_prefix_kernel(kv_dtype, out_dtype, s.head_dim, s.block_size);
            pthreads = kGqaWaves * 64;
            prows = 16 / G;
        }
    }
    PA_REQUIRE(fn && (prefix_tokens == 0 || pfn), PA_ERR_UNSUPPORTED,
               "no kernel instance for this dtype/shape");
    AttnArgs a = make_args(out, query, key_cache, value_cache, block_tables, context_lens, s,
                           scale);
    a.part_max = (float*)(ws + lay.off_max);
    a.part_sum = (float*)(ws + lay.off_sum);
    a.part_out = (float*)(ws + lay.off_out);
    a.partition_size = partition_size;
    a.max_partitions = lay.np;
    a.prefix_tokens = prefix_tokens;
    a.heads_log2 = hl;
    a.parts_per_wg = group;
    lay_out->group = group;
    if (app) {
        a.new_key = (const uint16_t*)app->new_key;
        a.new_value = (const uint16_t*)app->new_value;
        a.slot_mapping = app->slot_mapping;
        a.new_key_stride = app->key_stride;
        a.new_value_stride = app->value_stride;
    }
    if (prefix_parts > 0) {
        // shared prefix: prows sequences x G heads of one kv head per
        // workgroup, one prefix partition each (the prefill kernel takes a
        // null query_start for one query row per sequence)
        const int64_t tiles = (s.num_seqs + prows - 1) / prows;
        const int64_t grid = (int64_t)s.num_kv_heads * tiles * prefix_parts;
        PA_REQUIRE(grid < ((int64_t)1 << 31), PA_ERR_SHAPE, "grid too large");
        a.part_begin = 0;
        a.query_start = nullptr;
        hipLaunchKernelGGL(pfn, dim3((unsigned)grid), dim3(pthreads), 0, (hipStream_t)stream,
                           a);
        st = check_launch(what);
        if (st != PA_OK) return st;
    }
    a.seq_slots = xcd_seq_slots(s.num_seqs);
    const int64_t grid =
        (int64_t)a.seq_slots * per_seq * ceil_div(lay.np - prefix_parts, group);
    PA_REQUIRE(grid < ((int64_t)1 << 31), PA_ERR_SHAPE, "grid too large");
    if (grid == 0) return PA_OK;
    a.part_begin = prefix_parts;
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(threads), 0, (hipStream_t)stream, a);
    return check_launch(what);
}

pa_status launch_merge(void* out, pa_dtype out_dtype, const float* part_out,
                       const float* part_max, const float* part_sum,
                       const int32_t* context_lens, int num_seqs, int num_heads, int head_dim,
                       int max_partitions, int partition_size, void* stream, const char* what,
                       int skip_parts) {
    merge_fn mfn = pick_merge(out_dtype, head_dim);
    PA_REQUIRE(mfn, PA_ERR_UNSUPPORTED, "no merge instance");
    MergeArgs m{out,      part_out,      part_max, part_sum, context_lens, num_seqs,
                num_heads, max_partitions, partition_size, skip_parts};
    const int64_t rows = (int64_t)num_seqs * num_heads;
    const int64_t rpw = head_dim % 64 == 0 ? 1024 / head_dim : 4;  // rows per workgroup
    const int64_t grid = (rows + rpw - 1) / rpw;
    PA_REQUIRE(grid < ((int64_t)1 << 31), PA_ERR_SHAPE, "grid too large");
    hipLaunchKernelGGL(mfn, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, m);
    return check_launch(what);
}

}  // namespace

extern "C" pa_status pa_decode_partitions(void* out, pa_dtype out_dtype, const void* query,
                                          const void* key_cache, const void* value_cache,
                                          const int32_t* block_tables,
                                          const int32_t* context_lens, int num_seqs,
                                          int num_heads, int num_kv_heads, int head_dim,
                                          int block_size, int max_blocks_per_seq,
                                          int num_blocks, float scale, pa_dtype kv_dtype,
                                          int partition_size, void* workspace,
                                          size_t workspace_bytes, void* stream) {
    clear_error();
    const DecodeShape s{num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                        max_blocks_per_seq, num_blocks};
    SplitLayout lay;
    return launch_partitions(out, out_dtype, query, key_cache, value_cache, block_tables,
                             context_lens, s, scale, kv_dtype, partition_size, 0, workspace,
                             workspace_bytes, stream, "pa_decode_partitions", &lay);
}

extern "C" pa_status pa_decode_partitions_shared_prefix(
    void* out, pa_dtype out_dtype, const void* query, const void* key_cache,
    const void* value_cache, const int32_t* block_tables, const int32_t* context_lens,
    int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
    int max_blocks_per_seq, int num_blocks, float scale, pa_dtype kv_dtype, int partition_size,
    int shared_prefix_tokens, void* workspace, size_t workspace_bytes, void* stream) {
    clear_error();
    const DecodeShape s{num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                        max_blocks_per_seq, num_blocks};
    SplitLayout lay;
    return launch_partitions(out, out_dtype, query, key_cache, value_cache, block_tables,
                             context_lens, s, scale, kv_dtype, partition_size,
                             shared_prefix_tokens, workspace, workspace_bytes, stream,
                             "pa_decode_partitions_shared_prefix", &lay);
}

extern "C" pa_status pa_decode_split(void* out, pa_dtype out_dtype, const void* query,
                                     const void* key_cache, const void* value_cache,
                                     const int32_t* block_tables, const int32_t* context_lens,
                                     int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                     int block_size, int max_blocks_per_seq, int num_blocks,
                                     float scale, pa_dtype kv_dtype, int partition_size,
                                     void* workspace, size_t workspace_bytes, void* stream) {
    clear_error();
    const DecodeShape s{num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                        max_blocks_per_seq, num_blocks};
    SplitLayout lay;
    pa_status st = launch_partitions(out, out_dtype, query, key_cache, value_cache, block_tables,
                                     context_lens, s, scale, kv_dtype, partition_size, 0,
                                     workspace, workspace_bytes, stream,
                                     "pa_decode_split (partitions)", &lay);
    if (st != PA_OK || num_seqs == 0) return st;
    char* ws = (char*)workspace;
    return launch_merge(out, out_dtype, (const float*)(ws + lay.off_out),
                        (const float*)(ws + lay.off_max), (const float*)(ws + lay.off_sum),
                        context_lens, num_seqs, num_heads, head_dim, lay.np, partition_size,
                        stream, "pa_decode_split (merge)", lay.group);
}

// ---------------------------------------------------------------------------
// pa_decode_split_noalloc: the split path with its workspace in a scratch
// array of the library's own, for callers that cannot allocate
// ---------------------------------------------------------------------------

// The partitions' (max, sum, output) rows of pa_decode_split_noalloc. Each
// GPU the library runs on holds its own copy, from the code object's load
// until the process ends. In host code `scratch` names a host-side stand-in,
// not device memory: kernels get the address hipGetSymbolAddress returns for
// the current device (scratch_address), never the array's name.
static constexpr size_t kScratchBytes = PA_DECODE_NOALLOC_MAX_WORKSPACE;  // pa.h
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // per device, set on its first call

// Device address of the current device's scratch array (looked up once per
// device, with that device current).
pa_status scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    PA_REQUIRE(e == hipSuccess, PA_ERR_LAUNCH, "hipGetDevice failed: %s", hipGetErrorString(e));
    PA_REQUIRE(dev >= 0 && dev < kMaxDevices, PA_ERR_UNSUPPORTED, "device %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        PA_REQUIRE(e == hipSuccess && p, PA_ERR_LAUNCH,
                   "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                   hipGetErrorString(e));
        PA_REQUIRE((reinterpret_cast<uintptr_t>(p) & 255u) == 0, PA_ERR_LAUNCH,
                   "scratch array is not 256-byte aligned");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return PA_OK;
}

}  // namespace

extern "C" pa_status pa_decode_split_noalloc(void* out, pa_dtype out_dtype, const void* query,
                                             const void* key_cache, const void* value_cache,
                                             const int32_t* block_tables,
                                             const int32_t* context_lens, int num_seqs,
                                             int num_heads, int num_kv_heads, int head_dim,
                                             int block_size, int max_blocks_per_seq,
                                             int num_blocks, float scale, pa_dtype kv_dtype,
                                             int partition_size, void* stream) {
    clear_error();
    const DecodeShape s{num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                        max_blocks_per_seq, num_blocks};
    pa_status st = validate_decode(out, out_dtype, query, key_cache, value_cache, block_tables,
                                   context_lens, s, scale, kv_dtype);
    if (st != PA_OK) return st;
    PA_REQUIRE(partition_size > 0 && partition_size % block_size == 0, PA_ERR_SHAPE,
               "partition_size %d must be a positive multiple of block_size %d", partition_size,
               block_size);
    SplitLayout lay;
    split_layout(num_seqs, num_heads, head_dim, max_blocks_per_seq, block_size, partition_size,
                 &lay);
    // checked before the device is touched
    PA_REQUIRE(lay.total <= kScratchBytes, PA_ERR_WORKSPACE,
               "pa_decode_split_noalloc: these sizes need %zu bytes of workspace, more than the "
               "%zu-byte scratch array (use pa_decode_split with a caller workspace)",
               lay.total, kScratchBytes);
    if (num_seqs == 0) return PA_OK;
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st != PA_OK) return st;
    st = launch_partitions(out, out_dtype, query, key_cache, value_cache, block_tables,
                           context_lens, s, scale, kv_dtype, partition_size, 0, ws, lay.total,
                           stream, "pa_decode_split_noalloc (partitions)", &lay);
    if (st != PA_OK) return st;
    char* w = (char*)ws;
    return launch_merge(out, out_dtype, (const float*)(w + lay.off_out),
                        (const float*)(w + lay.off_max), (const float*)(w + lay.off_sum),
                        context_lens, num_seqs, num_heads, head_dim, lay.np, partition_size,
                        stream, "pa_decode_split_noalloc (merge)", lay.group);
}

namespace {

// the partition launch of the fused-append calls (validates the new rows)
pa_status launch_partitions_append(
    void* out, pa_dtype out_dtype, const void* query, void* key_cache, void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, const void* new_key,
    const void* new_value, const int64_t* slot_mapping, int64_t new_key_token_stride,
    int64_t new_value_token_stride, const DecodeShape& s, float scale, pa_dtype kv_dtype,
    int partition_size, void* workspace, size_t workspace_bytes, void* stream, const char* what,
    SplitLayout* lay) {
    const int64_t row = (int64_t)s.num_kv_heads * s.head_dim;
    PA_REQUIRE(new_key_token_stride >= row && new_value_token_stride >= row, PA_ERR_SHAPE,
               "new-token strides must be >= num_kv_heads * head_dim");
    PA_REQUIRE(new_key_token_stride % 8 == 0 && new_value_token_stride % 8 == 0,
               PA_ERR_ALIGNMENT, "new-token strides must be multiples of 8 elements");
    if (s.num_seqs > 0) {
        PA_REQUIRE(new_key && new_value && slot_mapping, PA_ERR_NULL, "null pointer argument");
        PA_REQUIRE(aligned16(new_key) && aligned16(new_value), PA_ERR_ALIGNMENT,
                   "new_key and new_value must be 16-byte aligned");
    }
    const AppendRows app{new_key, new_value, slot_mapping, new_key_token_stride,
                         new_value_token_stride};
    return launch_partitions(out, out_dtype, query, key_cache, value_cache, block_tables,
                             context_lens, s, scale, kv_dtype, partition_size, 0, workspace,
                             workspace_bytes, stream, what, lay, &app);
}

}  // namespace

extern "C" pa_status pa_decode_partitions_append(
    void* out, pa_dtype out_dtype, const void* query, void* key_cache, void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, const void* new_key,
    const void* new_value, const int64_t* slot_mapping, int64_t new_key_token_stride,
    int64_t new_value_token_stride, int num_seqs, int num_heads, int num_kv_heads,
    int head_dim, int block_size, int max_blocks_per_seq, int num_blocks, float scale,
    pa_dtype kv_dtype, int partition_size, void* workspace, size_t workspace_bytes,
    void* stream) {
    clear_error();
    const DecodeShape s{num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                        max_blocks_per_seq, num_blocks};
    SplitLayout lay;
    return launch_partitions_append(out, out_dtype, query, key_cache, value_cache, block_tables,
                                    context_lens, new_key, new_value, slot_mapping,
                                    new_key_token_stride, new_value_token_stride, s, scale,
                                    kv_dtype, partition_size, workspace, workspace_bytes, stream,
                                    "pa_decode_partitions_append", &lay);
}

extern "C" pa_status pa_decode_split_append(
    void* out, pa_dtype out_dtype, const void* query, void* key_cache, void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, const void* new_key,
    const void* new_value, const int64_t* slot_mapping, int64_t new_key_token_stride,
    int64_t new_value_token_stride, int num_seqs, int num_heads, int num_kv_heads,
    int head_dim, int block_size, int max_blocks_per_seq, int num_blocks, float scale,
    pa_dtype kv_dtype, int partition_size, void* workspace, size_t workspace_bytes,
    void* stream) {
    clear_error();
    const DecodeShape s{num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                        max_blocks_per_seq, num_blocks};
    SplitLayout lay;
    pa_status st = launch_partitions_append(
        out, out_dtype, query, key_cache, value_cache, block_tables, context_lens, new_key,
        new_value, slot_mapping, new_key_token_stride, new_value_token_stride, s, scale,
        kv_dtype, partition_size, workspace, workspace_bytes, stream,
        "pa_decode_split_append (partitions)", &lay);
    if (st != PA_OK || num_seqs == 0) return st;
    char* ws = (char*)workspace;
    return launch_merge(out, out_dtype, (const float*)(ws + lay.off_out),
                        (const float*)(ws + lay.off_max), (const float*)(ws + lay.off_sum),
                        context_lens, num_seqs, num_heads, head_dim, lay.np, partition_size,
                        stream, "pa_decode_split_append (merge)", lay.group);
}

extern "C" pa_status pa_decode_split_shared_prefix(
    void* out, pa_dtype out_dtype, const void* query, const void* key_cache,
    const void* value_cache, const int32_t* block_tables, const int32_t* context_lens,
    int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
    int max_blocks_per_seq, int num_blocks, float scale, pa_dtype kv_dtype, int partition_size,
    int shared_prefix_tokens, void* workspace, size_t workspace_bytes, void* stream) {
    clear_error();
    const DecodeShape s{num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                        max_blocks_per_seq, num_blocks};
    SplitLayout lay;
    pa_status st = launch_partitions(out, out_dtype, query, key_cache, value_cache, block_tables,
                                     context_lens, s, scale, kv_dtype, partition_size,
                                     shared_prefix_tokens, workspace, workspace_bytes, stream,
                                     "pa_decode_split_shared_prefix (partitions)", &lay);
    if (st != PA_OK || num_seqs == 0) return st;
    char* ws = (char*)workspace;
    return launch_merge(out, out_dtype, (const float*)(ws + lay.off_out),
                        (const float*)(ws + lay.off_max), (const float*)(ws + lay.off_sum),
                        context_lens, num_seqs, num_heads, head_dim, lay.np, partition_size,
                        stream, "pa_decode_split_shared_prefix (merge)", lay.group);
}

extern "C" pa_status pa_lse_merge(void* out, pa_dtype out_dtype, const float* part_out,
                                  const float* part_max, const float* part_sum,
                                  const int32_t* context_lens, int num_seqs, int num_heads,
                                  int head_dim, int max_partitions, int partition_size,
                                  void* stream) {
    clear_error();
    PA_REQUIRE(num_seqs >= 0 && num_heads > 0 && max_partitions > 0 && partition_size > 0,
               PA_ERR_SHAPE, "invalid sizes");
    PA_REQUIRE(head_dim == 64 || head_dim == 80 || head_dim == 96 || head_dim == 128 ||
                   head_dim == 256,
               PA_ERR_UNSUPPORTED, "head_dim %d not in {64, 80, 96, 128, 256}", head_dim);
    PA_REQUIRE(out_dtype == PA_F32 || out_dtype == PA_F16 || out_dtype == PA_BF16,
               PA_ERR_DTYPE, "invalid out dtype");
    if (num_seqs == 0) return PA_OK;
    PA_REQUIRE(out && part_out && part_max && part_sum && context_lens, PA_ERR_NULL,
               "null pointer argument");
    PA_REQUIRE(aligned16(out) && aligned16(part_out), PA_ERR_ALIGNMENT,
               "out and part_out must be 16-byte aligned");
    return launch_merge(out, out_dtype, part_out, part_max, part_sum, context_lens, num_seqs,
                        num_heads, head_dim, max_partitions, partition_size, stream,
                        "pa_lse_merge", /*skip_parts=*/0);
}

// ---------------------------------------------------------------------------
// Prefill over cached prefix blocks
// ---------------------------------------------------------------------------

namespace {
// Wavefronts (16 rows each) per prefill workgroup. Every wave of a
// workgroup reads every chunk of the context from LDS, so more waves means
// fewer fetches of each K/V row; but a wave whose rows lie past the
// sequence's last new token only loads and waits. Measured on MI355X with
// ~1500 cached tokens and 16..80 new tokens per request: one token per kv
// head row (MHA, 16 tokens a wave) is fastest with 4 waves, 7 heads per kv
// head (2 tokens a wave) with 8.
int prefill_waves(int tokens_per_wave, int head_dim, int max_query_len) {
    return head_dim == 128 && 8 * tokens_per_wave <= max_query_len ? 8 : 4;
}
}  // namespace

extern "C" pa_status pa_prefill(void* out, pa_dtype out_dtype, const void* query,
                                const void* key_cache, const void* value_cache,
                                const int32_t* block_tables, const int32_t* context_lens,
                                const int32_t* query_start, int num_seqs, int num_tokens,
                                int max_query_len, int num_heads, int num_kv_heads,
                                int head_dim, int block_size, int max_blocks_per_seq,
                                int num_blocks, float scale, pa_dtype kv_dtype, void* stream) {
    clear_error();
    const DecodeShape s{num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                        max_blocks_per_seq, num_blocks};
    pa_status st = validate_decode(out, out_dtype, query, key_cache, value_cache, block_tables,
                                   context_lens, s, scale, kv_dtype);
    if (st != PA_OK) return st;
    PA_REQUIRE(num_tokens >= 0 && max_query_len >= 0, PA_ERR_SHAPE,
               "num_tokens and max_query_len must be >= 0");
    PA_REQUIRE(max_query_len <= (int64_t)max_blocks_per_seq * block_size, PA_ERR_SHAPE,
               "max_query_len %d exceeds the longest context %d", max_query_len,
               max_blocks_per_seq * block_size);
    const int G = num_heads / num_kv_heads;
    PA_REQUIRE(G <= 16, PA_ERR_UNSUPPORTED,
               "prefill takes at most 16 query heads per kv head (got %d)", G);
    if (num_seqs == 0 || num_tokens == 0 || max_query_len == 0) return PA_OK;
    PA_REQUIRE(query_start, PA_ERR_NULL, "null query_start");
    const int waves = prefill_waves(16 / G, head_dim, max_query_len);
    attn_fn fn = pick_prefill_kernel(kv_dtype, out_dtype, head_dim, block_size, waves);
    PA_REQUIRE(fn, PA_ERR_UNSUPPORTED, "no kernel instance for this dtype/shape");
    AttnArgs a = make_args(out, query, key_cache, value_cache, block_tables, context_lens, s,
                           scale);
    const int rows = waves * (16 / G);  // new tokens per workgroup
    a.query_start = query_start;
    a.num_q_tiles = ceil_div(max_query_len, rows);
    const int64_t grid = (int64_t)num_seqs * a.num_q_tiles * num_kv_heads;
    PA_REQUIRE(grid < ((int64_t)1 << 31), PA_ERR_SHAPE, "grid too large");
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(waves * 64), 0, (hipStream_t)stream, a);
    return check_launch("pa_prefill");
}


extern "C" pa_status pa_prefill_shared_prefix(
    void* out, pa_dtype out_dtype, const void* query, const void* key_cache,
    const void* value_cache, const int32_t* block_tables, const int32_t* context_lens,
    const int32_t* query_start, int num_seqs, int num_tokens, int max_query_len, int num_heads,
    int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq, int num_blocks,
    float scale, pa_dtype kv_dtype, int shared_prefix_tokens, void* stream) {
    clear_error();
    const DecodeShape s{num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                        max_blocks_per_seq, num_blocks};
    pa_status st = validate_decode(out, out_dtype, query, key_cache, value_cache, block_tables,
                                   context_lens, s, scale, kv_dtype);
    if (st != PA_OK) return st;
    PA_REQUIRE(num_tokens >= 0 && max_query_len >= 0, PA_ERR_SHAPE,
               "num_tokens and max_query_len must be >= 0");
    PA_REQUIRE(max_query_len <= (int64_t)max_blocks_per_seq * block_size, PA_ERR_SHAPE,
               "max_query_len %d exceeds the longest context %d", max_query_len,
               max_blocks_per_seq * block_size);
    PA_REQUIRE(shared_prefix_tokens >= 0 && shared_prefix_tokens % block_size == 0 &&
                   shared_prefix_tokens <= (int64_t)max_blocks_per_seq * block_size,
               PA_ERR_SHAPE,
               "shared_prefix_tokens %d must be a multiple of block_size %d within "
               "max_blocks_per_seq * block_size", shared_prefix_tokens, block_size);
    const int G = num_heads / num_kv_heads;
    PA_REQUIRE(G <= 16, PA_ERR_UNSUPPORTED,
               "prefill takes at most 16 query heads per kv head (got %d)", G);
    if (num_seqs == 0 || num_tokens == 0 || max_query_len == 0) return PA_OK;
    PA_REQUIRE(query_start, PA_ERR_NULL, "null query_start");
    const int waves = prefill_shared_waves(head_dim);
    attn_fn fn = pick_prefill_shared_kernel(kv_dtype, out_dtype, head_dim, block_size, waves);
    PA_REQUIRE(fn, PA_ERR_UNSUPPORTED, "no kernel instance for this dtype/shape");
    AttnArgs a = make_args(out, query, key_cache, value_cache, block_tables, context_lens, s,
                           scale);
    a.query_start = query_start;
    a.prefix_tokens = shared_prefix_tokens;
    const int rows = waves * PA_PREFILL_SHARED_TR * (16 / G);  // new tokens per workgroup
    const int64_t grid = (int64_t)ceil_div(num_tokens, rows) * num_kv_heads;
    PA_REQUIRE(grid < ((int64_t)1 << 31), PA_ERR_SHAPE, "grid too large");
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(waves * 64), 0, (hipStream_t)stream, a);
    return check_launch("pa_prefill_shared_prefix");
}
