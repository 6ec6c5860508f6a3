// The one-head-per-workgroup paged decode kernel (multi-head attention, and
// grouped-query shapes the matrix-core kernel does not take).
//
// Work decomposition (MI355X, 64-lane wavefronts):
//   * one workgroup = one (sequence, group of 1, 2 or 4 adjacent query
//     heads, context partition) with NW wavefronts; each head's waves take
//     chunks of the partition (64 tokens, 128 at head_dim 64) in turn and
//     their softmax states are merged in LDS at the end. The single-pass
//     pa_decode is the same kernel with one head per workgroup and one
//     partition covering the context.
//   * inside a chunk, one 16-byte load per lane brings 8 elements of a K (or
//     V) row: head_dim/8 lanes cover a row, 64 lanes cover 64*8/head_dim
//     rows of one physical block per load instruction, so each load is a
//     set of dense head_dim*2-byte row segments and the block's base address
//     is uniform across the wavefront. A chunk is 16 such loads of K and 16
//     of V, whatever the row width, so that each wave keeps as many bytes in
//     flight at head_dim 64 as at 128.
//   * q·k: fp32 dot2 of packed fp16/bf16 pairs, then a transpose-reduce over
//     the lanes of a row that leaves lane c of each row group holding the
//     full score of that group's c-th load; softmax max/sum by wavefront
//     shuffles; exp2 with log2(e) folded into the scale.
//   * p·V: each lane scales its 8 V elements by the broadcast weight of its
//     row; the rows are summed at the end of the partition.
#pragma once

#include "pa_attn_args.h"
#include "pa_device.h"

namespace pa {

// One transpose-reduce step over groups of lanes, on the list pd[OFF ..
// OFF + 2*HALF - 1]: lanes whose index has bit HALF set keep the upper half
// of the list, the others the lower half, and each adds its partner's copy
// of the half it keeps.
template <int HALF, int OFF, int N>
__device__ __forceinline__ void tr_step(float (&pd)[N], int c) {
    const bool upper = (c & HALF) != 0;
#pragma unroll
    for (int k = OFF; k < OFF + HALF; ++k) {
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
    // head_dim 80 and 96 are laid out as 128: the lanes of the missing
    // slices load nothing (an offset past every range reads zeros) and
    // store nothing, so every product and sum is the real one
    constexpr int DP = D <= 64 ? 64 : 128;
    constexpr int LPR = DP / 8;         // lanes per cache row
    constexpr int RPI = 64 / LPR;       // rows per load instruction
    constexpr int CHUNK = mha_chunk_tokens(D, BS);  // tokens per chunk
    constexpr int NI = CHUNK / RPI;     // load instructions per chunk (16; 8 at 64 / BS 8)
    constexpr int SPL = NI / LPR;       // scores per lane (2 at head_dim 64 unless BS 8)
    constexpr int RPB = BS < 32 ? BS : 32;  // rows one load descriptor covers
    constexpr int IPB = RPB / RPI;      // load instructions per descriptor
    constexpr int BPC = CHUNK / RPB;    // descriptors per chunk
    // with more than 4 blocks per chunk the descriptors of two chunks would
    // not fit the scalar registers: keep each block's offset and range and
    // build its descriptor when its loads are issued
    constexpr bool LAZY = BPC > 4;
    static_assert(NI % LPR == 0 && SPL >= 1 && SPL <= 2, "whole scores per lane");
    static_assert(RPB % RPI == 0 && CHUNK % BS == 0 && BS % RPB == 0,
                  "blocks tile the chunk, descriptors the block");
    static_assert(LPR == 8 || LPR == 16, "head_dim laid out as 64 or 128");
    static_assert(D % 16 == 0 && D <= DP, "head_dim a multiple of 16, at most the layout");

    __shared__ float sm_m[NW];
    __shared__ float sm_l[NW];
    __shared__ float sm_acc[NW][DP];
    __shared__ __attribute__((aligned(16))) uint16_t sm_new[NW][2][DP];  // fused append: new K, V rows

    // the wave index is uniform inside a wavefront; saying so keeps every
    // chunk, block-table and address computation in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // the workgroup serves 2^heads_log2 adjacent query heads of one
    // (sequence, partition); each head gets NW / 2^heads_log2 waves, which
    // take the partition's chunks in turn. Adjacent heads' rows are
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

    int bid = blockIdx.x;  // (sequence slot, head group, partition), head group fastest
    const int head = (bid % ngroups) * (1 << hl) + hslot;
    bid /= ngroups;
    const int slots = a.seq_slots > 0 ? a.seq_slots : a.num_seqs;
    const int seq = bid % slots;
    if (seq >= a.num_seqs) return;  // a padding slot (uniform over the workgroup)
    const int part = bid / slots + a.part_begin;
    const int lane = threadIdx.x & 63;
    const int r = lane / LPR;  // row within a load instruction
    const int c = lane % LPR;  // 8-element slice of the row
    const bool cv = c * 8 < D;  // the slice exists (head_dim 80, 96: not all do)

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
    const uint32_t loff0 = (uint32_t)(r * row_bytes) + (cv ? (uint32_t)(c * 16) : kNoSlice);

    u32x4 q = u32x4{0u, 0u, 0u, 0u};
    if (cv) q = *(const u32x4*)(a.query + ((size_t)seq * Hq + head) * D + c * 8);

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
        u32x4 nk = u32x4{0u, 0u, 0u, 0u}, nv = nk;
        if (cv) {
            nk = *(const u32x4*)(a.new_key + seq * a.new_key_stride + kvh * D + c * 8);
            nv = *(const u32x4*)(a.new_value + seq * a.new_value_stride + kvh * D + c * 8);
        }
        *(u32x4*)&sm_new[hslot][0][c * 8] = nk;
        *(u32x4*)&sm_new[hslot][1][c * 8] = nv;
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
    // cache policy: non-temporal for rows of whole lines; a head slice that
    // ends inside a line (head_dim 80, 96) shares it with the next head,
    // whose wave reads it soon after from L2 if the line is kept there
    constexpr int AUX = (D * 2) % 128 == 0 ? PA_LOAD_AUX : PA_LOAD_AUX_SHARED_LINES;
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
                buf[b * IPB + j] = buffer_load16<AUX>(rs, o + (uint32_t)(j * RPI * row_bytes));
        }
    };
    constexpr std::false_type kK{};
    constexpr std::true_type kV{};
    // scores of the chunk's tokens, SPL per lane (log2 units, -inf if
    // absent): slot h of lane (r, c) holds the token of load h*LPR + c, row r
    auto scores = [&](const u32x4 (&kr)[NI], int cs, const ChunkIds& ci, float (&sc)[SPL]) {
        float pd[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            float t = KV::dot2(kr[i].x, q.x, 0.f);
            t = KV::dot2(kr[i].y, q.y, t);
            t = KV::dot2(kr[i].z, q.z, t);
            pd[i] = KV::dot2(kr[i].w, q.w, t);
        }
        // per list of LPR loads: lane c of each row group ends up with the
        // full score of load c of the list
        static_for<0, SPL>([&](auto H) {
            constexpr int o = decltype(H)::value * LPR;
            if constexpr (LPR >= 16) tr_step<8, o>(pd, c);
            tr_step<4, o>(pd, c);
            tr_step<2, o>(pd, c);
            tr_step<1, o>(pd, c);
        });
#pragma unroll
        for (int h = 0; h < SPL; ++h) {
            const int i = h * LPR + c;
            const int myb = i / IPB;
            const int mytok = cs + myb * RPB + (i % IPB) * RPI + r;
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
            sc[h] = ok ? pd[h * LPR] * a.scale_log2 : -INFINITY;
        }
    };
    // online softmax update; leaves this lane's weights exp2(s - m) in pr
    auto update = [&](const float (&sc)[SPL], float (&pr)[SPL]) {
        float smax = sc[0];
#pragma unroll
        for (int h = 1; h < SPL; ++h) smax = fmaxf(smax, sc[h]);
        const float mn = fmaxf(m, wave_max(smax));
        float alpha;
        if (mn == -INFINITY) {  // nothing valid yet (uniform)
            alpha = 1.f;
#pragma unroll
            for (int h = 0; h < SPL; ++h) pr[h] = 0.f;
        } else {
            alpha = fast_exp2(m - mn);
#pragma unroll
            for (int h = 0; h < SPL; ++h) pr[h] = fast_exp2(sc[h] - mn);
        }
        m = mn;
        float psum = pr[0];
#pragma unroll
        for (int h = 1; h < SPL; ++h) psum += pr[h];
        lsum = lsum * alpha + psum;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= alpha;
    };
    // acc += Σ_rows weight(row) · V(row) for this lane's 8 elements
    auto pv = [&](const u32x4 (&vr)[NI], const float (&pr)[SPL]) {
        static_for<0, NI>([&](auto I) {
            constexpr int i = decltype(I)::value;
            const float pb = group_bcast<LPR, i % LPR>(pr[i / LPR]);
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
            float sc[SPL], pr[SPL];
            scores(kr, cs, cur, sc);
            update(sc, pr);
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
        // a single partition is the whole context: the output itself; on
        // the split path the partition's workspace row is written as well,
        // so the rows describe every context whoever merges them
        if (nparts <= 1) OUT::store(a.out, sh * D + d, o);
        if (a.part_out) a.part_out[pidx * D + d] = o;
    }
    if (a.part_out && sub == 0 && lane == 0) {
        a.part_max[pidx] = M * kLn2;  // natural-log units
        a.part_sum[pidx] = tot;
    }
    if (slot_ok && sub == 0 && r == 0 && cv && head % (Hq / a.num_kv_heads) == 0) {
        const size_t dst = (size_t)a.slot_mapping[seq] * (a.num_kv_heads * D) + kvh * D + c * 8;
        *(u32x4*)((uint16_t*)a.key_cache + dst) = *(const u32x4*)&sm_new[hslot][0][c * 8];
        *(u32x4*)((uint16_t*)a.value_cache + dst) = *(const u32x4*)&sm_new[hslot][1][c * 8];
    }
}

}  // namespace pa
