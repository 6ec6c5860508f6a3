// The attention kernels' instances, as the host code reaches them. Each
// picker returns the kernel instance for an element type, output type,
// head_dim and block size, or null when there is none; each is defined in
// its own pa_inst_*.hip file so that the instances compile in parallel.
#pragma once

#include "pa.h"
#include "pa_attn_args.h"

#ifndef PA_WAVES
#define PA_WAVES 4
#endif
#ifndef PA_GQA_WAVES
#define PA_GQA_WAVES 4
#endif

// 16-row tiles per wave of the prefill kernel in shared-prefix mode
#ifndef PA_PREFILL_SHARED_TR
#define PA_PREFILL_SHARED_TR 1
#endif

namespace pa {

constexpr int kWaves = PA_WAVES;         // wavefronts per workgroup, one-head kernel
constexpr int kGqaWaves = PA_GQA_WAVES;  // and matrix-core kernel

// what a grouped-query decode kernel instance computes
enum GqaMode {
    kModeDecode = 0,  // one sequence's query heads of a kv head per workgroup
    kModePrefix = 1,  // over a shared prefix: several sequences per workgroup
};

typedef void (*attn_fn)(AttnArgs);

attn_fn pick_attn(pa_dtype kv, pa_dtype out, int d, int bs);            // pa_inst_mha.hip
attn_fn pick_gqa(pa_dtype kv, pa_dtype out, int d, int bs);             // pa_inst_gqa.hip
attn_fn pick_prefix_kernel(pa_dtype kv, pa_dtype out, int d, int bs);   // pa_inst_prefix.hip
// prefill kernel with `waves` (4 or 8) wavefronts of 16 rows per workgroup
attn_fn pick_prefill_kernel(pa_dtype kv, pa_dtype out, int d, int bs,
                            int waves);  // pa_inst_prefill.hip
// the same kernel in shared-prefix mode (rows of every request in one list)
attn_fn pick_prefill_shared_kernel(pa_dtype kv, pa_dtype out, int d, int bs,
                                   int waves);  // pa_inst_prefill_shared.hip

}  // namespace pa
