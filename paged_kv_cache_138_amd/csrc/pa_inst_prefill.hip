// Instances of the matrix-core kernel for prefill.
#include "pa_attn_gqa.h"
#include "pa_kernels.h"

namespace pa {

attn_fn pick_prefill_kernel(pa_dtype kv, pa_dtype out, int d, int bs) {
    return pick_gqa_mode<kModePrefill>(kv, out, d, bs);
}

}  // namespace pa
