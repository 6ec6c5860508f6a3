// Instances of the prefill kernel in shared-prefix mode.
#include "pa_attn_prefill.h"
#include "pa_kernels.h"

namespace pa {

namespace {
template <int NW>
attn_fn pick_cfg(pa_dtype kv, pa_dtype out, int d, int bs) {
    if (kv == PA_F16) return pick_prefill_out<KvF16, NW, PA_PREFILL_SHARED_TR, true>(out, kv, d, bs);
    if (kv == PA_BF16) return pick_prefill_out<KvBF16, NW, PA_PREFILL_SHARED_TR, true>(out, kv, d, bs);
    return nullptr;
}
}  // namespace

attn_fn pick_prefill_shared_kernel(pa_dtype kv, pa_dtype out, int d, int bs, int waves) {
    if (waves == 4) return pick_cfg<4>(kv, out, d, bs);
    if (waves == 8) return pick_cfg<8>(kv, out, d, bs);
    return nullptr;
}

}  // namespace pa
