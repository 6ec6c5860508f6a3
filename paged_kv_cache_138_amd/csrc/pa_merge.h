// Log-sum-exp merge of per-partition decode results, shared by the
// standalone merge kernel and the in-kernel merge of the split path.
//
// Partition p of a query head carries m_p (largest scaled logit, natural-log
// units), l_p = Σ exp(s - m_p) and o_p = Σ exp(s - m_p) v / l_p. With
// M = max_p m_p and w_p = l_p exp(m_p - M) the head's output is
// Σ_p w_p o_p / Σ_p w_p ("vLLM PagedAttention深度解析与工程实践" §4.1: the
// v2 kernel accumulates partial results, then merges them; the combination
// rule is the textbook one for softmax over a union of disjoint sets).
#pragma once

#include "pa_device.h"

namespace pa {

// Merge element d of one workspace row (one query head of one sequence)
// over its np partitions: first the largest m_p, then the weighted sums.
// Both loops are free of data-dependent branches, so the loads of successive
// partitions can be in flight together. A partition whose m_p is -inf holds
// no token (its l_p is 0) and its o_p is never used: it may be unwritten.
__device__ __forceinline__ float merge_row_element(const float* pm, const float* ps,
                                                  const float* po, int np, int D) {
    constexpr int kFew = 16;
    if (np <= kFew) {
        // up to 16 partitions: every load is issued before any arithmetic
        float m[kFew], l[kFew], o[kFew];
#pragma unroll
        for (int p = 0; p < kFew; ++p) {
            const bool in = p < np;
            m[p] = in ? pm[p] : -INFINITY;
            l[p] = in ? ps[p] : 0.f;
            o[p] = in ? po[(size_t)p * D] : 0.f;
        }
        float M = -INFINITY;
#pragma unroll
        for (int p = 0; p < kFew; ++p) M = fmaxf(M, m[p]);
        if (M == -INFINITY) return 0.f;
        float tot = 0.f, acc = 0.f;
#pragma unroll
        for (int p = 0; p < kFew; ++p) {
            const bool live = m[p] != -INFINITY;
            const float w = live ? l[p] * fast_exp2((m[p] - M) * kLog2e) : 0.f;
            tot += w;
            acc = live ? fmaf(w, o[p], acc) : acc;
        }
        return tot > 0.f ? acc / tot : 0.f;
    }
    float M = -INFINITY;
#pragma unroll 8
    for (int p = 0; p < np; ++p) M = fmaxf(M, pm[p]);
    if (M == -INFINITY) return 0.f;
    float tot = 0.f, acc = 0.f;
#pragma unroll 8
    for (int p = 0; p < np; ++p) {
        const float mp = pm[p];
        const bool live = mp != -INFINITY;
        const float w = live ? ps[p] * fast_exp2((mp - M) * kLog2e) : 0.f;
        tot += w;
        acc = live ? fmaf(w, po[(size_t)p * D], acc) : acc;
    }
    return tot > 0.f ? acc / tot : 0.f;
}

}  // namespace pa
