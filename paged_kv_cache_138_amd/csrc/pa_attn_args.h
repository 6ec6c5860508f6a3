// Arguments shared by the decode-attention kernels of libpa.
#pragma once

#include <stdint.h>

namespace pa {

// Tokens per chunk of the one-head decode kernel, from the host's view as
// well (it sizes the heads per workgroup so that every wave gets a chunk).
// A lane keeps 16 loads of 16 bytes of K (and as many of V) in flight: 64
// tokens of 128-element rows (head_dim 80 and 96 are laid out as 128), and
// 128 tokens of 64-element rows, where each lane then holds two scores. At
// block size 8 such a chunk would span 16 blocks, whose ids and ranges no
// longer fit the scalar registers: there it stays at 64 tokens.
#ifndef PA_MHA_CHUNK_64
#define PA_MHA_CHUNK_64 128
#endif
constexpr int mha_chunk_tokens(int head_dim, int block_size) {
    return head_dim <= 64 && block_size >= 16 ? PA_MHA_CHUNK_64 : 64;
}

// Grouped-query partition groups: a sequence's n partitions in ceil(n / k)
// groups of nearly equal size (1), or groups of k from partition 0 with a
// short last one (0, built for comparison). The partition kernel and the
// merge read the same setting.
#ifndef PA_GQA_EVEN_GROUPS
#define PA_GQA_EVEN_GROUPS 1
#endif

struct AttnArgs {
    void* out;
    const uint16_t* query;
    const uint16_t* key_cache;
    const uint16_t* value_cache;
    const int32_t* block_tables;
    const int32_t* context_lens;
    float* part_max;
    float* part_sum;
    float* part_out;
    int num_seqs;
    int num_heads;
    int num_kv_heads;
    int max_blocks_per_seq;
    int num_blocks;
    int partition_size;
    int max_partitions;
    int part_begin;     // first partition index the grid covers
    // split paths: sequence slots of the grid (>= num_seqs; 0 means
    // num_seqs); the units of slots past num_seqs return at once
    int seq_slots;
    // grouped-query decode: the most consecutive partitions one workgroup
    // walks (1, 2 or 4; 0 counts as 1). A sequence's n partitions form
    // ceil(n / k) groups of nearly equal size; a group's combined state goes
    // to its first partition's workspace row, and its other rows are marked
    // empty.
    int parts_per_wg;
    int prefix_tokens;  // shared-prefix mode: tokens every sequence shares (block_tables row 0)
    int heads_log2;     // MHA kernel: log2 of the query heads one workgroup serves (0, 1, 2)
    float scale_log2;  // scale * log2(e)
    // Fused append (decode step). When new_key is set, row i of new_key /
    // new_value is sequence i's token at position L_i - 1: the workgroups of
    // the partition holding that position use it in place of the cache row
    // and store it into slot slot_mapping[i] (skipped when the slot is
    // negative or outside the cache, and then the cache row is used).
    const uint16_t* new_key;
    const uint16_t* new_value;
    const int64_t* slot_mapping;
    int64_t new_key_stride;    // elements between consecutive tokens of new_key
    int64_t new_value_stride;  // and of new_value
    // Prefill: sequence i's new tokens are rows query_start[i] ..
    // query_start[i+1] - 1 of query and out, the last positions of its
    // context; the grid has num_q_tiles tiles of new tokens per sequence.
    const int32_t* query_start;
    int num_q_tiles;
};

}  // namespace pa
