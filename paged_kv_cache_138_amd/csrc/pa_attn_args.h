// Arguments shared by the decode-attention kernels of libpa.
#pragma once

#include <stdint.h>

namespace pa {


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
    int prefix_tokens;  // shared-prefix mode: tokens every sequence shares (block_tables row 0)
    int heads_log2;     // MHA kernel: log2 of the query heads one workgroup serves (0, 1, 2)
    float scale_log2;  // scale * log2(e)
};

}  // namespace pa
