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
// Work decomposition (MI355X, 64-lane wavefronts):
//   * one workgroup = one (sequence, group of 1 or 2 adjacent query heads,
//     context partition) with NW wavefronts; each head's waves take 64-token
//     chunks of the partition in turn and their softmax states are merged in
//     LDS at the end. The single-pass pa_decode is the same kernel with one
//     head per workgroup and one partition covering the context.
//   * inside a chunk, one 16-byte load per lane brings 8 elements of a K (or
//     V) row: head_dim/8 lanes cover a row, 64 lanes cover 64*8/head_dim
//     rows of one physical block per load instruction, so each load is a
//     set of dense head_dim*2-byte row segments and the block's base address
//     is uniform across the wavefront.
//   * q·k: fp32 dot2 of packed fp16/bf16 pairs, then a transpose-reduce over
//     the lanes of a row that leaves lane c of each row group holding the
//     full score of that group's c-th load; softmax max/sum by wavefront
//     shuffles; exp2 with log2(e) folded into the scale.
//   * p·V: each lane scales its 8 V elements by the broadcast weight of its
//     row; the rows are summed at the end of the partition.
#include "pa_attn_args.h"
#include "pa_attn_gqa.h"
#include "pa_merge.h"
#include "pa_device.h"
#include "pa_host.h"

#include <math.h>

#include <mutex>
#include <unordered_map>

namespace pa {
namespace {

#ifndef PA_WAVES
#define PA_WAVES 4
#endif
constexpr int kWaves = PA_WAVES;  // wavefronts per workgroup
#ifndef PA_GQA_WAVES
#define PA_GQA_WAVES 4
#endif
constexpr int kGqaWaves = PA_GQA_WAVES;

// One transpose-reduce step over groups of lanes: lanes whose index has
// bit HALF set keep the upper half of their list, the others the lower half,
// and each adds its partner's copy of the half it keeps.
template <int HALF, int N>
__device__ __forceinline__ void tr_step(float (&pd)[N], int c) {
    const bool upper = (c & HALF) != 0;
#pragma unroll
    for (int k = 0; k < HALF; ++k) {
        const float send = upper ? pd[k] : pd[k + HALF];
        const float keep = upper ? pd[k + HALF] : pd[k];
        pd[k] = keep + tr_partner<HALF>(send);
    }
}

#ifndef PA_MHA_WAVES_PER_EU
#define PA_MHA_WAVES_PER_EU 3
#endif

template <class KV, class OUT, int D, int BS, int NW>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(PA_MHA_WAVES_PER_EU))) void attn_partition_kernel(AttnArgs a) {
    constexpr int LPR = D / 8;          // lanes per cache row
    constexpr int RPI = 64 / LPR;       // rows per load instruction
    constexpr int NI = LPR;             // load instructions per chunk
    constexpr int CHUNK = RPI * NI;     // tokens per chunk (64)
    constexpr int RPB = BS < 32 ? BS : 32;  // rows one load descriptor covers
    constexpr int IPB = RPB / RPI;      // load instructions per descriptor
    constexpr int BPC = CHUNK / RPB;    // descriptors per chunk
    // with more than 4 blocks per chunk the descriptors of two chunks would
    // not fit the scalar registers: keep each block's offset and range and
    // build its descriptor when its loads are issued
    constexpr bool LAZY = BPC > 4;
    static_assert(CHUNK == 64, "one score per lane per chunk");
    static_assert(RPB % RPI == 0 && CHUNK % BS == 0 && BS % RPB == 0,
                  "blocks tile the chunk, descriptors the block");
    static_assert(LPR == 8 || LPR == 16, "head_dim 64 or 128");

    __shared__ float sm_m[NW];
    __shared__ float sm_l[NW];
    __shared__ float sm_acc[NW][D];
    __shared__ __attribute__((aligned(16))) uint16_t sm_new[NW][2][D];  // fused append: new K, V rows

    // the wave index is uniform inside a wavefront; saying so keeps every
    // chunk, block-table and address computation in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // the workgroup serves 2^heads_log2 adjacent query heads of one
    // (sequence, partition); each head gets NW / 2^heads_log2 waves, which
    // take the partition's 64-token chunks in turn. Adjacent heads' rows are
    // adjacent in a cache row, so serving several heads at once reads longer
    // contiguous runs of each block at about the same time.
    constexpr int LOG_NW = NW == 4 ? 2 : (NW == 2 ? 1 : 0);
    static_assert((1 << LOG_NW) == NW, "NW must be 1, 2 or 4");
    const int hl = a.heads_log2;
    const int nwh = NW >> hl;                     // waves per head
    const int hslot = wave >> (LOG_NW - hl);      // head within the workgroup
    const int sub = wave & (nwh - 1);             // wave within the head
    const int Hq = a.num_heads;
    const int ngroups = Hq >> hl;

    int bid = blockIdx.x;  // (sequence, head group, partition), head group fastest
    const int head = (bid % ngroups) * (1 << hl) + hslot;
    bid /= ngroups;
    const int seq = bid % a.num_seqs;
    const int part = bid / a.num_seqs + a.part_begin;
    const int lane = threadIdx.x & 63;
    const int r = lane / LPR;  // row within a load instruction
    const int c = lane % LPR;  // 8-element slice of the row

    const int Lmax = a.max_blocks_per_seq * BS;
    int L = a.context_lens[seq];
    L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
    const int P = a.partition_size;
    const int nparts = (L + P - 1) / P;
    if (part > 0 && part >= nparts) return;  // uniform over the workgroup
    const int start = part * P;
    const int end = min(start + P, L);
    const int nb = (L + BS - 1) / BS;

    const int kvh = head / (Hq / a.num_kv_heads);
    const size_t row_bytes = (size_t)a.num_kv_heads * D * 2;
    const size_t block_bytes = row_bytes * BS;
    const char* kbase = (const char*)a.key_cache + (size_t)kvh * D * 2;
    const char* vbase = (const char*)a.value_cache + (size_t)kvh * D * 2;
    const int32_t* bt = a.block_tables + (size_t)seq * a.max_blocks_per_seq;
    // byte offset, inside a block, of the first row this lane reads; load j
    // of a block reads RPI * j rows further
    const uint32_t loff0 = (uint32_t)(r * row_bytes + c * 16);

    const u32x4 q = *(const u32x4*)(a.query + ((size_t)seq * Hq + head) * D + c * 8);

    // Fused append: position L - 1 of the partition that holds it is the new
    // token, whose rows come from new_key / new_value instead of the cache.
    // The chunk loop then stops before it (end_c), and one wave per head
    // folds it in after the loop. That wave keeps its copy of the rows in
    // LDS (written and read by itself, so no barrier), and at the very end
    // stores them into the cache slot when its head is the first of its kv
    // head: a global store ahead of the chunk loop would stop the compiler
    // from reading the block table with scalar loads.
    // A sequence with L = 0 has no token to attend, but its row is still
    // stored (by the workgroups of its partition 0), as the scatter would.
    const bool owner = a.new_key && part == max(nparts, 1) - 1;
    const bool slot_ok = owner && a.slot_mapping[seq] >= 0 &&
                         a.slot_mapping[seq] < (int64_t)a.num_blocks * BS;
    const bool has_new = slot_ok && L > 0;  // every wave of the head
    const bool app = has_new && sub == 0;   // the wave that folds it in
    if (slot_ok && sub == 0 && r == 0) {
        *(u32x4*)&sm_new[hslot][0][c * 8] =
            *(const u32x4*)(a.new_key + seq * a.new_key_stride + kvh * D + c * 8);
        *(u32x4*)&sm_new[hslot][1][c * 8] =
            *(const u32x4*)(a.new_value + seq * a.new_value_stride + kvh * D + c * 8);
    }
    const int end_c = has_new ? L - 1 : end;  // end of the tokens read from the cache

    float m = -INFINITY;  // running max of scores (log2 units)
    float lsum = 0.f;     // this lane's share of Σ exp2(s - m)
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;

    // load descriptors of the chunk starting at token cs, one per RPB rows
    // (a whole block, or a block's slice when blocks are longer): the range
    // of each covers exactly its rows below `end`, so rows past the context
    // and blocks past the table (or with an id outside the pool) read as
    // zeros and are never fetched
    struct IdsEager {
        __amdgpu_buffer_rsrc_t k[BPC], v[BPC];
        bool ok[BPC];
    };
    struct IdsLazy {
        int pid[BPC];        // block id (0 when absent)
        uint32_t nrec[BPC];  // bytes in range; 0 when absent
        uint32_t okm;        // bit b: block b present
    };
    using ChunkIds = std::conditional_t<LAZY, IdsLazy, IdsEager>;
    auto fetch_ids = [&](int cs, ChunkIds& ci) {
        if constexpr (LAZY) ci.okm = 0;
#pragma unroll
        for (int b = 0; b < BPC; ++b) {
            // chunks start on block boundaries (a block is never longer
            // than a chunk), so block and row offset are known per b
            const int lb = cs / BS + (b * RPB) / BS;
            const int pid = lb < nb ? bt[lb] : -1;
            const int rows = min(max(end_c - (cs + b * RPB), 0), RPB);
            const bool ok = pid >= 0 && pid < a.num_blocks && rows > 0;
            const uint32_t nrec = ok ? (uint32_t)((rows - 1) * row_bytes + D * 2) : 0u;
            if constexpr (LAZY) {
                ci.pid[b] = __builtin_amdgcn_readfirstlane(ok ? pid : 0);
                ci.nrec[b] = __builtin_amdgcn_readfirstlane(nrec);
                ci.okm |= (uint32_t)ok << b;
            } else {
                const size_t boff =
                    (size_t)(ok ? pid : 0) * block_bytes + ((b * RPB) % BS) * row_bytes;
                ci.k[b] = make_rsrc(kbase + boff, nrec);
                ci.v[b] = make_rsrc(vbase + boff, nrec);
                ci.ok[b] = ok;
            }
        }
    };
    auto issue = [&](const ChunkIds& ci, auto is_v, u32x4 (&buf)[NI]) {
        // recomputing the IPB offsets here (one add each) keeps them out of
        // the registers that live across the chunk loop
        uint32_t o = loff0;
        asm("" : "+v"(o));
#pragma unroll
        for (int b = 0; b < BPC; ++b) {
            __amdgpu_buffer_rsrc_t rs;
            if constexpr (LAZY)
                rs = make_rsrc((is_v ? vbase : kbase) + (size_t)ci.pid[b] * block_bytes +
                                   ((b * RPB) % BS) * row_bytes,
                               ci.nrec[b]);
            else
                rs = is_v ? ci.v[b] : ci.k[b];
#pragma unroll
            for (int j = 0; j < IPB; ++j)
                buf[b * IPB + j] = buffer_load16(rs, o + (uint32_t)(j * RPI * row_bytes));
        }
    };
    constexpr std::false_type kK{};
    constexpr std::true_type kV{};
    // scores of the chunk's 64 tokens, one per lane (log2 units, -inf if absent)
    auto scores = [&](const u32x4 (&kr)[NI], int cs, const ChunkIds& ci) -> float {
        float pd[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            float t = KV::dot2(kr[i].x, q.x, 0.f);
            t = KV::dot2(kr[i].y, q.y, t);
            t = KV::dot2(kr[i].z, q.z, t);
            pd[i] = KV::dot2(kr[i].w, q.w, t);
        }
        // lane c of each row group ends up with the full score of load c
        if constexpr (NI >= 16) tr_step<8>(pd, c);
        tr_step<4>(pd, c);
        tr_step<2>(pd, c);
        tr_step<1>(pd, c);
        const int myb = c / IPB;
        const int mytok = cs + myb * RPB + (c % IPB) * RPI + r;
        bool ok;
        if constexpr (LAZY) {
            ok = (__builtin_amdgcn_readfirstlane(ci.okm) >> myb) & 1u;
        } else {
            ok = ci.ok[0];
#pragma unroll
            for (int b = 1; b < BPC; ++b)
                if (myb == b) ok = ci.ok[b];
        }
        ok = ok && mytok < end_c;
        return ok ? pd[0] * a.scale_log2 : -INFINITY;
    };
    // online softmax update; returns this lane's weight exp2(s - m)
    auto update = [&](float s) -> float {
        const float mn = fmaxf(m, wave_max(s));
        float alpha, pr;
        if (mn == -INFINITY) {  // nothing valid yet (uniform)
            alpha = 1.f;
            pr = 0.f;
        } else {
            alpha = fast_exp2(m - mn);
            pr = fast_exp2(s - mn);
        }
        m = mn;
        lsum = lsum * alpha + pr;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= alpha;
        return pr;
    };
    // acc += Σ_rows weight(row) · V(row) for this lane's 8 elements
    auto pv = [&](const u32x4 (&vr)[NI], float pr) {
        static_for<0, NI>([&](auto I) {
            constexpr int i = decltype(I)::value;
            const float pb = group_bcast<LPR, i>(pr);
            // tie the row to its weight so its unpacking (explicit shifts for
            // bf16) is not hoisted ahead of the softmax, where all 16 rows'
            // unpacked values would be live at once
            uint32_t x = vr[i].x, y = vr[i].y, z = vr[i].z, w = vr[i].w;
            if constexpr (std::is_same<KV, KvBF16>::value)
                asm("" : "+v"(x), "+v"(y), "+v"(z), "+v"(w) : "v"(pb));
            acc[0] += pb * KV::lo(x);
            acc[1] += pb * KV::hi(x);
            acc[2] += pb * KV::lo(y);
            acc[3] += pb * KV::hi(y);
            acc[4] += pb * KV::lo(z);
            acc[5] += pb * KV::hi(z);
            acc[6] += pb * KV::lo(w);
            acc[7] += pb * KV::hi(w);
        });
    };

    // ---- chunks, software-pipelined: the next chunk's K is in flight during
    // this chunk's p·V, and its V during the next score pass -----------------
    int cs = start + sub * CHUNK;
    const int cstep = nwh * CHUNK;
    if (cs < end_c) {
        ChunkIds cur;
        u32x4 kr[NI], vr[NI];
        fetch_ids(cs, cur);
        issue(cur, kK, kr);
        issue(cur, kV, vr);
        for (;;) {
            const int nx = cs + cstep;
            const bool more = nx < end_c;
            ChunkIds nxt;
            if (more) fetch_ids(nx, nxt);
            const float pr = update(scores(kr, cs, cur));
            if (!more) {
                pv(vr, pr);
                break;
            }
            issue(nxt, kK, kr);
            pv(vr, pr);
            issue(nxt, kV, vr);
            cur = nxt;
            cs = nx;
        }
    }

    // ---- the fused-append token, once per head -----------------------------
    if (app) {
        const u32x4 kn = *(const u32x4*)&sm_new[hslot][0][c * 8];
        float t = KV::dot2(kn.x, q.x, 0.f);
        t = KV::dot2(kn.y, q.y, t);
        t = KV::dot2(kn.z, q.z, t);
        t = KV::dot2(kn.w, q.w, t);
#pragma unroll
        for (int msk = 1; msk < LPR; msk <<= 1) t += __shfl_xor(t, msk, 64);
        const float sn = t * a.scale_log2;  // the same in every row group
        const float mn = fmaxf(m, sn);
        const float alpha = m == -INFINITY ? 0.f : fast_exp2(m - mn);
        const float pn = fast_exp2(sn - mn);
        m = mn;
        lsum = lsum * alpha + (lane == 0 ? pn : 0.f);
        const u32x4 vn = *(const u32x4*)&sm_new[hslot][1][c * 8];
        const float w = r == 0 ? pn : 0.f;  // row group 0 carries the token
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= alpha;
        acc[0] += w * KV::lo(vn.x);
        acc[1] += w * KV::hi(vn.x);
        acc[2] += w * KV::lo(vn.y);
        acc[3] += w * KV::hi(vn.y);
        acc[4] += w * KV::lo(vn.z);
        acc[5] += w * KV::hi(vn.z);
        acc[6] += w * KV::lo(vn.w);
        acc[7] += w * KV::hi(vn.w);
    }

    // ---- fold the wavefront's rows, then the workgroup's waves -------------
    lsum = wave_sum(lsum);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
#pragma unroll
        for (int msk = LPR; msk < 64; msk <<= 1) acc[e] += __shfl_xor(acc[e], msk, 64);
    }
    if (lane == 0) {
        sm_m[wave] = m;
        sm_l[wave] = lsum;
    }
    if (r == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sm_acc[wave][c * 8 + e] = acc[e];
    }
    __syncthreads();

    // the waves hslot*nwh .. hslot*nwh + nwh - 1 hold this head's states
    const int w0 = hslot * nwh;
    float M = -INFINITY;
    for (int w = 0; w < nwh; ++w) M = fmaxf(M, sm_m[w0 + w]);
    float wt[NW];
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        wt[w] = 0.f;
        if (w < nwh) {
            const float mw = sm_m[w0 + w];
            if (mw != -INFINITY) wt[w] = fast_exp2(mw - M);
            tot += wt[w] * sm_l[w0 + w];
        }
    }
    const size_t sh = (size_t)seq * Hq + head;
    const size_t pidx = sh * a.max_partitions + part;
    for (int d = sub * 64 + lane; d < D; d += nwh * 64) {
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w)
            if (w < nwh) t += wt[w] * sm_acc[w0 + w][d];
        const float o = tot > 0.f ? t / tot : 0.f;
        if (nparts <= 1) {
            OUT::store(a.out, sh * D + d, o);
        } else {
            a.part_out[pidx * D + d] = o;
        }
    }
    if (nparts > 1 && sub == 0 && lane == 0) {
        a.part_max[pidx] = M * kLn2;  // natural-log units
        a.part_sum[pidx] = tot;
    }
    if (slot_ok && sub == 0 && r == 0 && head % (Hq / a.num_kv_heads) == 0) {
        const size_t dst = (size_t)a.slot_mapping[seq] * (a.num_kv_heads * D) + kvh * D + c * 8;
        *(u32x4*)((uint16_t*)a.key_cache + dst) = *(const u32x4*)&sm_new[hslot][0][c * 8];
        *(u32x4*)((uint16_t*)a.value_cache + dst) = *(const u32x4*)&sm_new[hslot][1][c * 8];
    }
}

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
};

// 256 threads merge 256 / head_dim workspace rows (row = one query head of
// one sequence), one output element per thread; rows of sequences with at
// most one partition are skipped (the partition kernel wrote them).
template <class OUT, int D>
__global__ __launch_bounds__(256) void lse_merge_kernel(MergeArgs a) {
    constexpr int RPW = 256 / D;
    // a wavefront covers 64 consecutive elements of one row (D >= 64)
    const int row = __builtin_amdgcn_readfirstlane(blockIdx.x * RPW + threadIdx.x / D);
    const int d = threadIdx.x % D;
    if (row >= a.num_seqs * a.num_heads) return;
    const int seq = row / a.num_heads;
    int L = a.context_lens[seq];
    if (L < 0) L = 0;
    int np = (int)(((int64_t)L + a.partition_size - 1) / a.partition_size);
    if (np > a.max_partitions) np = a.max_partitions;
    if (np <= 1) return;
    const size_t r = (size_t)row * a.max_partitions;
    const float o = merge_row_element(a.part_max + r, a.part_sum + r, a.part_out + r * D + d, np, D);
    OUT::store(a.out, (size_t)row * D + d, o);
}

// ---------------------------------------------------------------------------
// Host dispatch
// ---------------------------------------------------------------------------

typedef void (*attn_fn)(AttnArgs);
typedef void (*merge_fn)(MergeArgs);

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

attn_fn pick_attn(pa_dtype kv, pa_dtype out, int d, int bs) {
    if (kv == PA_F16) return pick_attn_out<KvF16>(out, kv, d, bs);
    if (kv == PA_BF16) return pick_attn_out<KvBF16>(out, kv, d, bs);
    return nullptr;
}

// grouped-query instances (MFMA), 2 <= num_heads / num_kv_heads <= 16, and
// the shared-prefix mode of the same kernel (1 <= G <= 16)
template <class KV, class OUT, int D, bool PREFIX>
attn_fn pick_gqa_bs(int bs) {
    switch (bs) {
        case 8: return attn_gqa_kernel<KV, OUT, D, 8, kGqaWaves, PREFIX>;
        case 16: return attn_gqa_kernel<KV, OUT, D, 16, kGqaWaves, PREFIX>;
        case 32: return attn_gqa_kernel<KV, OUT, D, 32, kGqaWaves, PREFIX>;
        case 64: return attn_gqa_kernel<KV, OUT, D, 64, kGqaWaves, PREFIX>;
    }
    return nullptr;
}

template <class KV, class OUT, bool PREFIX>
attn_fn pick_gqa_d(int d, int bs) {
    switch (d) {
        case 64: return pick_gqa_bs<KV, OUT, 64, PREFIX>(bs);
        case 128: return pick_gqa_bs<KV, OUT, 128, PREFIX>(bs);
    }
    return nullptr;
}

template <class KV, bool PREFIX = false>
attn_fn pick_gqa_out(pa_dtype out, pa_dtype kv, int d, int bs) {
    if (out == PA_F32) return pick_gqa_d<KV, OutF32, PREFIX>(d, bs);
    if (out != kv) return nullptr;
    if (kv == PA_F16) return pick_gqa_d<KV, OutF16, PREFIX>(d, bs);
    return pick_gqa_d<KV, OutBF16, PREFIX>(d, bs);
}

attn_fn pick_prefix_kernel(pa_dtype kv, pa_dtype out, int d, int bs) {
    if (kv == PA_F16) return pick_gqa_out<KvF16, true>(out, kv, d, bs);
    if (kv == PA_BF16) return pick_gqa_out<KvBF16, true>(out, kv, d, bs);
    return nullptr;
}

constexpr int kMaxGroupMfma = 16;

bool use_gqa(int num_heads, int num_kv_heads) {
    const int g = num_heads / num_kv_heads;
    return g >= 2 && g <= kMaxGroupMfma;
}

// Query heads per workgroup of the MHA kernel on the split path (log2).
// One head per workgroup gives the finest work units, which matters when
// the grid is only a few times what the device holds at once (the last,
// ragged units then decide the end of the kernel). When the grid is many
// times larger - many sequences or long maximum contexts, where most of the
// (sequence, partition) rectangle may be empty - two adjacent heads per
// workgroup halve the workgroups to dispatch and read each block row's
// heads side by side. The single-pass path keeps one head per workgroup, so
// that a sequence's context is spread over all the waves of its workgroup.
int mha_heads_log2(int num_heads, int64_t rect_workgroups, int resident, bool split) {
    if (!split || num_heads % 2 != 0) return 0;
    return rect_workgroups / 2 >= (int64_t)6 * resident ? 1 : 0;
}

#ifndef PA_GQA_HEADS
#define PA_GQA_HEADS 2
#endif
// kv heads per workgroup of the grouped-query kernel on the split path (log2)
int gqa_heads_log2(int num_kv_heads) {
    int hl = 0;
    while ((2 << hl) <= PA_GQA_HEADS && (2 << hl) <= kGqaWaves && num_kv_heads % (2 << hl) == 0)
        ++hl;
    return hl;
}

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
        if (kv == PA_F16) return pick_gqa_out<KvF16>(out, kv, d, bs);
        if (kv == PA_BF16) return pick_gqa_out<KvBF16>(out, kv, d, bs);
        return nullptr;
    }
    *per_seq = num_heads >> heads_log2;
    return pick_attn(kv, out, d, bs);
}

template <class OUT>
merge_fn pick_merge_d(int d) {
    switch (d) {
        case 64: return lse_merge_kernel<OUT, 64>;
        case 128: return lse_merge_kernel<OUT, 128>;
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
    PA_REQUIRE(s.head_dim == 64 || s.head_dim == 128, PA_ERR_UNSUPPORTED,
               "head_dim %d not in {64, 128}", s.head_dim);
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

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }



struct SplitLayout {
    int np;
    size_t off_max, off_sum, off_out, total;
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
    const int prefix_parts = prefix_tokens / partition_size;
    int per_seq = 0, threads = 0;
    attn_fn fn = pick_kernel(kv_dtype, out_dtype, s.head_dim, s.block_size, s.num_heads,
                             s.num_kv_heads, 0, &per_seq, &threads);
    int hl = 0;
    if (fn && !use_gqa(s.num_heads, s.num_kv_heads)) {
        const int64_t rect = (int64_t)s.num_seqs * s.num_heads * (lay.np - prefix_parts);
        hl = mha_heads_log2(s.num_heads, rect, resident_workgroups((const void*)fn, threads),
                            true);
        per_seq = s.num_heads >> hl;
    } else if (fn) {
        hl = gqa_heads_log2(s.num_kv_heads);
        per_seq = s.num_kv_heads >> hl;
    }
    attn_fn pfn = prefix_tokens > 0 ? pick_prefix_kernel(kv_dtype, out_dtype, s.head_dim,
                                                         s.block_size)
                                    : nullptr;
    PA_REQUIRE(fn && (prefix_tokens == 0 || pfn), PA_ERR_UNSUPPORTED,
               "no kernel instance for this dtype/shape");
    char* ws = (char*)workspace;
    AttnArgs a = make_args(out, query, key_cache, value_cache, block_tables, context_lens, s,
                           scale);
    a.part_max = (float*)(ws + lay.off_max);
    a.part_sum = (float*)(ws + lay.off_sum);
    a.part_out = (float*)(ws + lay.off_out);
    a.partition_size = partition_size;
    a.max_partitions = lay.np;
    a.prefix_tokens = prefix_tokens;
    a.heads_log2 = hl;
    if (app) {
        a.new_key = (const uint16_t*)app->new_key;
        a.new_value = (const uint16_t*)app->new_value;
        a.slot_mapping = app->slot_mapping;
        a.new_key_stride = app->key_stride;
        a.new_value_stride = app->value_stride;
    }
    if (prefix_parts > 0) {
        // shared prefix: 16 / G sequences x G heads per workgroup
        const int rows = 16 / (s.num_heads / s.num_kv_heads);
        const int64_t tiles = (s.num_seqs + rows - 1) / rows;
        const int64_t grid = (int64_t)s.num_kv_heads * tiles * prefix_parts;
        PA_REQUIRE(grid < ((int64_t)1 << 31), PA_ERR_SHAPE, "grid too large");
        a.part_begin = 0;
        hipLaunchKernelGGL(pfn, dim3((unsigned)grid), dim3(kGqaWaves * 64), 0,
                           (hipStream_t)stream, a);
        st = check_launch(what);
        if (st != PA_OK) return st;
    }
    const int64_t grid = (int64_t)s.num_seqs * per_seq * (lay.np - prefix_parts);
    PA_REQUIRE(grid < ((int64_t)1 << 31), PA_ERR_SHAPE, "grid too large");
    if (grid == 0) return PA_OK;
    a.part_begin = prefix_parts;
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(threads), 0, (hipStream_t)stream, a);
    return check_launch(what);
}

pa_status launch_merge(void* out, pa_dtype out_dtype, const float* part_out,
                       const float* part_max, const float* part_sum,
                       const int32_t* context_lens, int num_seqs, int num_heads, int head_dim,
                       int max_partitions, int partition_size, void* stream, const char* what) {
    merge_fn mfn = pick_merge(out_dtype, head_dim);
    PA_REQUIRE(mfn, PA_ERR_UNSUPPORTED, "no merge instance");
    MergeArgs m{out, part_out, part_max, part_sum, context_lens,
                num_seqs, num_heads, max_partitions, partition_size};
    const int64_t rows = (int64_t)num_seqs * num_heads;
    const int64_t rpw = 256 / head_dim;
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
                        stream, "pa_decode_split (merge)");
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
                        stream, "pa_decode_split_append (merge)");
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
                        stream, "pa_decode_split_shared_prefix (merge)");
}

extern "C" pa_status pa_lse_merge(void* out, pa_dtype out_dtype, const float* part_out,
                                  const float* part_max, const float* part_sum,
                                  const int32_t* context_lens, int num_seqs, int num_heads,
                                  int head_dim, int max_partitions, int partition_size,
                                  void* stream) {
    clear_error();
    PA_REQUIRE(num_seqs >= 0 && num_heads > 0 && max_partitions > 0 && partition_size > 0,
               PA_ERR_SHAPE, "invalid sizes");
    PA_REQUIRE(head_dim == 64 || head_dim == 128, PA_ERR_UNSUPPORTED,
               "head_dim %d not in {64, 128}", head_dim);
    PA_REQUIRE(out_dtype == PA_F32 || out_dtype == PA_F16 || out_dtype == PA_BF16,
               PA_ERR_DTYPE, "invalid out dtype");
    if (num_seqs == 0) return PA_OK;
    PA_REQUIRE(out && part_out && part_max && part_sum && context_lens, PA_ERR_NULL,
               "null pointer argument");
    PA_REQUIRE(aligned16(out) && aligned16(part_out), PA_ERR_ALIGNMENT,
               "out and part_out must be 16-byte aligned");
    return launch_merge(out, out_dtype, part_out, part_max, part_sum, context_lens, num_seqs,
                        num_heads, head_dim, max_partitions, partition_size, stream,
                        "pa_lse_merge");
}
