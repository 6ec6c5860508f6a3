// Instances of the one-head-per-workgroup decode kernel.
#include "pa_attn_mha.h"
#include "pa_kernels.h"

namespace pa {
namespace {

template <class KV, class OUT, int D>
attn_fn pick_attn_bs(int bs) {
    switch (bs) {
        case 8: return attn_partition_kernel<KV, OUT, D, 8, kWaves>;
        case 16: return attn_partition_kernel<KV, OUT, D, 16, kWaves>;
        case 32: return attn_partition_kernel<KV, OUT, D, 32, kWaves>;
        case 64: return attn_partition_kernel<KV, OUT, D, 64, kWaves>;
    }
    return nullptr;
}

template <class KV, class OUT>
attn_fn pick_attn_d(int d, int bs) {
    switch (d) {
        case 64: return pick_attn_bs<KV, OUT, 64>(bs);
        case 80: return pick_attn_bs<KV, OUT, 80>(bs);
        case 96: return pick_attn_bs<KV, OUT, 96>(bs);
        case 128: return pick_attn_bs<KV, OUT, 128>(bs);
    }
    return nullptr;
}

template <class KV>
attn_fn pick_attn_out(pa_dtype out, pa_dtype kv, int d, int bs) {
    if (out == PA_F32) return pick_attn_d<KV, OutF32>(d, bs);
    if (out != kv) return nullptr;
    if (kv == PA_F16) return pick_attn_d<KV, OutF16>(d, bs);
    return pick_attn_d<KV, OutBF16>(d, bs);
}

}  // namespace

attn_fn pick_attn(pa_dtype kv, pa_dtype out, int d, int bs) {
    if (kv == PA_F16) return pick_attn_out<KvF16>(out, kv, d, bs);
    if (kv == PA_BF16) return pick_attn_out<KvBF16>(out, kv, d, bs);
    return nullptr;
}

}  // namespace pa
