// Log-sum-exp merge of per-partition decode results, shared by the merge
// kernels (four elements of a row per thread, or one row per wavefront).
//
// Partition p of a query head carries m_p (largest scaled logit, natural-log
// units), l_p = Σ exp(s - m_p) and o_p = Σ exp(s - m_p) v / l_p. With
// M = max_p m_p and w_p = l_p exp(m_p - M) the head's output is
// Σ_p w_p o_p / Σ_p w_p ("vLLM PagedAttention深度解析与工程实践" §4.1: the
// v2 kernel accumulates partial results, then merges them; the combination
// rule is the textbook one for softmax over a union of disjoint sets).
#pragma once

#include "pa_attn_args.h"
#include "pa_device.h"

namespace pa {

// First rows floor(i * np / nq) of the groups i = 0, 1, ...: with
// np = q * nq + rem, each step adds q, and one more when the running
// remainder i * rem mod nq wraps (no division per group).
struct GroupRows {
    int q, rem, nq, p = 0, acc = 0;
    __device__ GroupRows(int np, int nq_) : q(np / nq_), rem(np - (np / nq_) * nq_), nq(nq_) {}
    // groups of `step` from partition 0 (PA_GQA_EVEN_GROUPS=0): q = step, no remainder
    __device__ GroupRows(int step) : q(step), rem(0), nq(1) {}
    __device__ __forceinline__ int next() {
        const int r = p;
        p += q;
        acc += rem;
        if (acc >= nq) {
            acc -= nq;
            ++p;
        }
        return r;
    }
};

// Merge element d of one workspace row (one query head of one sequence)
// over its np partitions: the largest m_p, then the weighted sums.
// Partitions walked in groups of up to `step` form nq = ceil(np / step)
// groups of nearly equal size, group i starting at partition
// floor(i * np / nq), which holds the group's state; the other rows are not
// read (step 1: every partition is its own group). A partition whose m_p
// is -inf holds no token (its l_p is 0) and its o_p is never used: it may
// be unwritten.
// KB groups at a time: their loads are free of data-dependent branches and
// all in flight together; a row of more groups takes them in blocks of KB,
// rescaling its running sums to each block's maximum.
template <int KB>
__device__ __forceinline__ float merge_blocks(const float* pm, const float* ps, const float* po,
                                             int np, int D, int step) {
    const int nq = (np + step - 1) / step;  // np >= 1
    GroupRows rows = PA_GQA_EVEN_GROUPS ? GroupRows(np, nq) : GroupRows(step);
    float M = -INFINITY, tot = 0.f, acc = 0.f;
    for (int i0 = 0; i0 < nq; i0 += KB) {
        float m[KB], l[KB], o[KB];
#pragma unroll
        for (int q = 0; q < KB; ++q) {
            const bool in = i0 + q < nq;
            const int p = in ? rows.next() : 0;
            m[q] = in ? pm[p] : -INFINITY;
            l[q] = in ? ps[p] : 0.f;
            o[q] = in ? po[(size_t)p * D] : 0.f;
        }
        float Mb = M;
#pragma unroll
        for (int q = 0; q < KB; ++q) Mb = fmaxf(Mb, m[q]);
        if (Mb == -INFINITY) continue;  // nothing yet (uniform over the row)
        const float r = M == -INFINITY ? 0.f : fast_exp2((M - Mb) * kLog2e);
        tot *= r;
        acc *= r;
        M = Mb;
#pragma unroll
        for (int q = 0; q < KB; ++q) {
            const bool live = m[q] != -INFINITY;
            const float w = live ? l[q] * fast_exp2((m[q] - M) * kLog2e) : 0.f;
            tot += w;
            acc = live ? fmaf(w, o[q], acc) : acc;
        }
    }
    return tot > 0.f ? acc / tot : 0.f;
}

// merge_blocks for four consecutive elements of the row at once: one
// 16-byte load of each partition's output.
template <int KB>
__device__ __forceinline__ f32x4 merge_blocks4(const float* pm, const float* ps, const float* po,
                                              int np, int D, int step) {
    const int nq = (np + step - 1) / step;  // np >= 1
    GroupRows rows = PA_GQA_EVEN_GROUPS ? GroupRows(np, nq) : GroupRows(step);
    float M = -INFINITY, tot = 0.f;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int i0 = 0; i0 < nq; i0 += KB) {
        float m[KB], l[KB];
        f32x4 o[KB];
#pragma unroll
        for (int q = 0; q < KB; ++q) {
            const bool in = i0 + q < nq;
            const int p = in ? rows.next() : 0;
            m[q] = in ? pm[p] : -INFINITY;
            l[q] = in ? ps[p] : 0.f;
            o[q] = in ? *(const f32x4*)(po + (size_t)p * D) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        float Mb = M;
#pragma unroll
        for (int q = 0; q < KB; ++q) Mb = fmaxf(Mb, m[q]);
        if (Mb == -INFINITY) continue;
        const float r = M == -INFINITY ? 0.f : fast_exp2((M - Mb) * kLog2e);
        tot *= r;
        acc *= r;
        M = Mb;
#pragma unroll
        for (int q = 0; q < KB; ++q) {
            const bool live = m[q] != -INFINITY;
            const float w = live ? l[q] * fast_exp2((m[q] - M) * kLog2e) : 0.f;
            tot += w;
            if (live) acc += w * o[q];
        }
    }
    return tot > 0.f ? acc / tot : f32x4{0.f, 0.f, 0.f, 0.f};
}

__device__ __forceinline__ f32x4 merge_row_element4(const float* pm, const float* ps,
                                                   const float* po, int np, int D, int step) {
    const int nq = (np + step - 1) / step;
    if (nq <= 4) return merge_blocks4<4>(pm, ps, po, np, D, step);
    if (nq <= 8) return merge_blocks4<8>(pm, ps, po, np, D, step);
    return merge_blocks4<16>(pm, ps, po, np, D, step);
}

// The block width follows the row's partition count (uniform over a wave,
// which covers part of one row).
__device__ __forceinline__ float merge_row_element(const float* pm, const float* ps,
                                                  const float* po, int np, int D, int step) {
    const int nq = (np + step - 1) / step;
    if (nq <= 4) return merge_blocks<4>(pm, ps, po, np, D, step);
    if (nq <= 8) return merge_blocks<8>(pm, ps, po, np, D, step);
    return merge_blocks<16>(pm, ps, po, np, D, step);
}

}  // namespace pa
