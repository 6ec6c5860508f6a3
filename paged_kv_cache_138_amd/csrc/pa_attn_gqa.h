// Grouped-query paged decode attention on MFMA (gfx950).
//
// When G = num_heads / num_kv_heads query heads share one kv head, the G
// query rows against one K/V block form a real small GEMM, so this kernel
// reads each K/V row once for all G heads and does both products on the
// matrix cores (v_mfma_f32_16x16x32_{bf16,f16}, fp32 accumulation):
//
//   Sᵀ[16 tokens x 16 heads] = K[16 x 32 d] · Qᵀ[32 d x 16 heads], 4 per
//       16-token sub-block for head_dim 128 (heads G..15 are zero padding);
//   Oᵀ[16 d x 16 heads] += Vᵀ[16 d x 32 tokens] · Pᵀ[32 tokens x 16 heads],
//       one per 16-column tile of head_dim, for each 32 tokens of a chunk
//       (chunks of 32 tokens; 64 at head_dim 64).
//
// Register layouts (lane l, g = l/16, n = l%16): an MFMA output leaves lane l
// holding column n and rows 4g..4g+3, so both products keep head n in lane
// n's column; the online softmax of head n is entirely lane-local apart from
// one max over the four lanes {n, n+16, n+32, n+48}. The contraction index of
// each product is free to permute as long as both operands use the same map,
// which is used twice:
//   * q·k: lane (g, n) holds d = 32j + 8g .. +7 of K row n and of q row n,
//     read from the wave's LDS copy of the chunk with ds_read_b128.
//   * p·v: the score registers themselves (tokens 4g..4g+3 and 16+4g..+3)
//     are the Pᵀ operand; Vᵀ with the matching token order is read from the
//     wave's LDS copy of the chunk's V rows by the gfx950 transpose read
//     ds_read_b64_tr_b16 (in each 16-lane group, lane 4e+q names 4 elements
//     of row e and lane j receives column j of the 4 rows).
// P is split into hi + lo halves in the 16-bit type before the p·v products,
// so the weights keep ~16 bits of precision.
//
// K and V rows reach LDS through the same coalesced loads as the
// head-per-workgroup kernel (head_dim/8 lanes per row, whole 128-byte lines
// per request). LDS rows are padded to 2*head_dim + 32 bytes, which spreads
// the 16-byte reads of K and the transpose reads of V over the banks. The
// work decomposition (1 or 2 adjacent kv heads per workgroup), masking by
// buffer ranges, partitions, the cross-wave merge and the fused append
// follow the head-per-workgroup kernel. On the split path a workgroup may
// also walk a group of consecutive partitions of its sequence (a sequence's
// partitions form groups of nearly equal size), whose combined state is one
// workspace row.
#pragma once

#include "pa_attn_args.h"
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

template <class KV>
struct Mma;

template <>
struct Mma<KvBF16> {
    static __device__ __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                      __builtin_bit_cast(bf16x8_t, b), c, 0, 0,
                                                      0);
    }
    // x rounded to the 16-bit type (bits) and the value it stands for
    static __device__ __forceinline__ uint32_t round16(float x, float* back) {
        const __bf16 h = (__bf16)x;  // v_cvt_pk_bf16_f32, round to nearest even
        const uint32_t b = (uint32_t)__builtin_bit_cast(uint16_t, h);
        *back = __uint_as_float(b << 16);
        return b;
    }
    // (x0, x1) as packed hi halves, and what is left of each, packed. The
    // remainders x - hi are exact in fp32 (hi is x rounded to 8 bits), so
    // the dot2 form x + (-1)·hi + (-0)·other computes them with no rounding,
    // one instruction each. (The pairs are (-1, -0) rather than (-1, 0):
    // the compiler encodes a bf16 pair (-1, 0) as the inline constant -1.0,
    // which the hardware reads as the fp32 bit pattern, -1 in the upper
    // half; (-1, -0) is a literal.)
    static __device__ __forceinline__ void split2(float x0, float x1, uint32_t* hi,
                                                  uint32_t* lo) {
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
        typedef float f2 __attribute__((ext_vector_type(2)));
        const b2 h = __builtin_convertvector(f2{x0, x1}, b2);
        const float r0 = __builtin_amdgcn_fdot2_f32_bf16(h, b2{(__bf16)-1.0f, (__bf16)-0.0f}, x0,
                                                         false);
        const float r1 = __builtin_amdgcn_fdot2_f32_bf16(h, b2{(__bf16)-0.0f, (__bf16)-1.0f}, x1,
                                                         false);
        *hi = __builtin_bit_cast(uint32_t, h);
        *lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{r0, r1}, b2));
    }
};

template <>
struct Mma<KvF16> {
    static __device__ __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                     __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t round16(float x, float* back) {
        const _Float16 h = (_Float16)x;
        *back = (float)h;
        return (uint32_t)__builtin_bit_cast(uint16_t, h);
    }
    // as for bf16: the remainders are exact, taken by dot2 with (-1, -0)
    static __device__ __forceinline__ void split2(float x0, float x1, uint32_t* hi,
                                                  uint32_t* lo) {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        typedef float f2 __attribute__((ext_vector_type(2)));
        const h2 h = __builtin_convertvector(f2{x0, x1}, h2);
        const float r0 =
            __builtin_amdgcn_fdot2(h, h2{(_Float16)-1.0f, (_Float16)-0.0f}, x0, false);
        const float r1 =
            __builtin_amdgcn_fdot2(h, h2{(_Float16)-0.0f, (_Float16)-1.0f}, x1, false);
        *hi = __builtin_bit_cast(uint32_t, h);
        *lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{r0, r1}, h2));
    }
};

__device__ __forceinline__ u32x2 lds_read_tr16(const char* p) {
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)(p));
    return __builtin_bit_cast(u32x2, v);
}

#ifndef PA_GQA_WAVES_PER_EU
#define PA_GQA_WAVES_PER_EU 3
#endif
#ifndef PA_GQA_CHUNK
#define PA_GQA_CHUNK 32
#endif
// Tokens per chunk at head_dim 64: 64, so that a wave stages as many bytes
// per chunk as at head_dim 128 (measured on MI355X, 64 q / 8 kv heads,
// contexts of 1k-8k tokens: 236 -> 229 us per launch).
#ifndef PA_GQA_CHUNK_64
#define PA_GQA_CHUNK_64 64
#endif

// MODE kModeDecode: a workgroup serves the G query heads of one (sequence,
// kv head) over one partition of that sequence's context.
// MODE kModePrefix (shared-prefix decode): every sequence's first
// prefix_tokens tokens are the same physical blocks (block_tables row 0). A
// workgroup then serves 16 / G sequences x G heads of one kv head over one
// partition of the shared prefix, so each prefix block is read once per 16
// query rows instead of once per (sequence, kv head).
template <class KV, class OUT, int D, int BS, int NW, int MODE>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(PA_GQA_WAVES_PER_EU))) void attn_gqa_kernel(AttnArgs a) {
    constexpr bool PREFIX = MODE == kModePrefix;
    static_assert(MODE == kModeDecode || MODE == kModePrefix, "decode modes");
    constexpr int CH = D <= 64 ? PA_GQA_CHUNK_64 : PA_GQA_CHUNK;  // tokens per chunk (32 or 64)
    constexpr int NS = CH / 16;         // 16-token sub-blocks of a chunk
    constexpr int NH = CH / 32;         // 32-token halves (one p·v contraction each)
    // head_dim 80 and 96 are laid out as 128: the missing slices read as
    // zeros, so they add nothing to q·k and give output columns never stored
    constexpr int DP = D <= 64 ? 64 : 128;
    constexpr int NJ = DP / 32;         // q·k products per 16-token sub-block
    constexpr int NT = DP / 16;         // 16-wide output tiles of head_dim
    constexpr int LPR = DP / 8;         // lanes per row in a coalesced V load
    constexpr int RPI = 64 / LPR;       // rows per coalesced V load
    constexpr int VL = CH / RPI;        // V loads per chunk
    constexpr int RPB = BS < CH ? BS : CH;  // rows one load descriptor covers
    constexpr int BPC = CH / RPB;       // descriptors per chunk (blocks, or one block's slice)
    // LDS bytes per K or V row: a 32-byte pad keeps the 16-byte K reads and
    // the transposed V reads free of bank conflicts (a 16-byte pad left both
    // 2-way on MI355X)
    constexpr int ROWB = DP * 2 + PA_LDS_ROW_PAD;
    constexpr int TILE = CH * ROWB;     // LDS bytes of one chunk's K (then V) rows
    constexpr int OROW = DP + 4;        // floats per row of the wave's partial output
    static_assert(BS == 8 || BS == 16 || BS == 32 || BS == 64, "block size 8, 16, 32 or 64");
    static_assert(RPB % RPI == 0, "the rows of one coalesced load share a block");
    static_assert(CH == 32 || CH == 64, "chunk of 32 or 64 tokens");
    static_assert(16 * OROW * 4 <= TILE, "the wave's LDS tile also holds its partial output");
    static_assert(VL * RPI == CH, "coalesced loads tile the chunk");

    __shared__ __attribute__((aligned(16))) char sm_v[NW][TILE];
    __shared__ float sm_m[NW][16];
    __shared__ float sm_l[NW][16];
    __shared__ __attribute__((aligned(16))) uint16_t sm_new[NW][2][DP];  // fused append: new K, V rows

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;   // lane group
    const int n = lane & 15;   // head inside the group (column of every product)
    const int vr = lane / LPR; // row of a coalesced V load
    const int vc = lane % LPR; // 16-byte slice of that row
    const bool vcv = vc * 8 < D;  // the slice exists (head_dim 80, 96: not all do)

    const int Hq = a.num_heads;
    const int Hkv = a.num_kv_heads;
    const int G = Hq / Hkv;
    const int P = a.partition_size;
    const int Lmax = a.max_blocks_per_seq * BS;
    auto ctx_len = [&](int sq) {
        const int l = a.context_lens[sq];
        return l < 0 ? 0 : (l > Lmax ? Lmax : l);
    };
    // Without a shared prefix the workgroup may serve 2^heads_log2 adjacent
    // kv heads of one (sequence, partition), each with NW / 2^heads_log2
    // waves taking the partition's chunks in turn: adjacent kv heads' rows
    // are adjacent in a cache row, so their reads run side by side.
    constexpr int LOG_NW = NW == 4 ? 2 : (NW == 2 ? 1 : 0);
    static_assert((1 << LOG_NW) == NW, "NW must be 1, 2 or 4");
    const int hl = PREFIX ? 0 : a.heads_log2;
    const int nwh = NW >> hl;                 // waves per kv head
    const int hslot = wave >> (LOG_NW - hl);  // kv head within the workgroup
    const int sub = wave & (nwh - 1);         // wave within the kv head
    const int ngroups = Hkv >> hl;
    int bid = blockIdx.x;  // kv head group fastest, then sequence (or row tile), then partition
    const int kvh0 = (bid % ngroups) << hl;
    const int kvh = kvh0 + hslot;
    bid /= ngroups;
    // rows of every product: row r is query head r_head of sequence r_seq
    const int R = PREFIX ? 16 / G : 1;  // sequences per workgroup
    int seq0, part, part_end, Lsrc, nparts = 0;
    // groups of up to K consecutive partitions (grouped decode mode)
    const int K = PREFIX || a.parts_per_wg < 1 ? 1 : a.parts_per_wg;
    const int32_t* bt;
    if constexpr (PREFIX) {
        const int ntiles = (a.num_seqs + R - 1) / R;
        seq0 = (bid % ntiles) * R;
        part = bid / ntiles + a.part_begin;
        part_end = part + 1;
        Lsrc = a.prefix_tokens;
        bt = a.block_tables;  // the shared prefix, as row 0 lists it
    } else {
        const int slots = a.seq_slots > 0 ? a.seq_slots : a.num_seqs;
        seq0 = bid % slots;
        if (seq0 >= a.num_seqs) return;  // a padding slot (uniform over the workgroup)
        // partition groups in descending order: the last workgroups
        // dispatched are group 0's, one per sequence and mostly full, rather
        // than the few high groups of the longest sequences (measured on the
        // GQA long-context batch: 457 -> 451 µs; the one-head kernel gained
        // nothing from it)
        const int pslots = (int)(gridDim.x / ((unsigned)ngroups * (unsigned)slots));
        const int gi = pslots - 1 - bid / slots;
        Lsrc = ctx_len(seq0);
        nparts = (Lsrc + P - 1) / P;
        if (K == 1) {
            part = gi + a.part_begin;
            part_end = part + 1;
            if (part > 0 && part >= nparts) return;  // uniform over the workgroup
        } else {
            // the sequence's partitions (one, if it has none) in
            // ceil(n / K) groups of nearly equal size: group gi starts at
            // partition floor(gi * n / groups). Groups of K with a short
            // last one would leave single-partition workgroups, which
            // unbalance the launch's end.
            const int n = max(nparts, 1);
            const int ng = (n + K - 1) / K;
            if (gi >= ng) return;  // uniform over the workgroup
            part = PA_GQA_EVEN_GROUPS ? gi * n / ng : gi * K;
            part_end = PA_GQA_EVEN_GROUPS ? (gi + 1) * n / ng : min(part + K, n);
        }
        bt = a.block_tables + (size_t)seq0 * a.max_blocks_per_seq;
    }
    const int start = part * P;
    // Fused append (not in prefix mode): position L - 1 of the partition
    // holding it is the new token, taken from new_key / new_value. The
    // chunk loop stops before it (end), and the first wave of each kv head
    // folds it in after the loop, from its own copy in LDS; that wave also
    // stores the rows into the cache slot, at the very end (a global store
    // ahead of the chunk loop would stop the compiler from reading the
    // block table with scalar loads).
    // (A sequence with L = 0 has no token to attend; its row is still
    // stored, by the workgroups of its partition 0, as the scatter would.)
    bool has_new = false, store_new = false;
    if constexpr (MODE == kModeDecode) {
        if (a.new_key && part_end >= max(nparts, 1)) {  // the group holding position L - 1
            const int64_t slot = a.slot_mapping[seq0];
            const bool slot_ok = slot >= 0 && slot < (int64_t)a.num_blocks * BS;
            has_new = slot_ok && Lsrc > 0;
            store_new = slot_ok && sub == 0 && vr == 0;
            if (store_new) {
                u32x4 nk = u32x4{0u, 0u, 0u, 0u}, nv = nk;
                if (vcv) {
                    nk = *(const u32x4*)(a.new_key + seq0 * a.new_key_stride + kvh * D + vc * 8);
                    nv = *(const u32x4*)(a.new_value + seq0 * a.new_value_stride + kvh * D +
                                         vc * 8);
                }
                *(u32x4*)&sm_new[wave][0][vc * 8] = nk;
                *(u32x4*)&sm_new[wave][1][vc * 8] = nv;
            }
        }
    }
    const int end = has_new ? Lsrc - 1 : min(part_end * P, Lsrc);
    const int nb = (Lsrc + BS - 1) / BS;
    auto row_seq = [&](int r) { return seq0 + r / G; };
    auto row_head = [&](int r) { return kvh * G + r % G; };
    auto row_ok = [&](int r) { return r < R * G && row_seq(r) < a.num_seqs; };

    const size_t row_bytes = (size_t)Hkv * D * 2;
    const size_t block_bytes = row_bytes * BS;
    const char* kbase = (const char*)a.key_cache + (size_t)kvh * D * 2;
    const char* vbase = (const char*)a.value_cache + (size_t)kvh * D * 2;
    // the wave's LDS tile holds the current chunk's K rows, then its V rows
    // (a wave's LDS operations complete in order)
    char* tile = sm_v[wave];

    // Qᵀ operand: lane (g, n) holds row n's q[32j + 8g .. +7]; unused rows are 0
    u32x4 qb[NJ];
    {
        const bool real = row_ok(n);
        const uint16_t* qrow =
            a.query + ((size_t)(real ? row_seq(n) : 0) * Hq + (real ? row_head(n) : 0)) * D;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            qb[j] = u32x4{0u, 0u, 0u, 0u};
            if (real && 32 * j + 8 * g < D) qb[j] = *(const u32x4*)(qrow + 32 * j + 8 * g);
        }
    }

    float m = -INFINITY;  // running max of head n's scores (log2 units)
    float lsum = 0.f;     // this lane's share of head n's Σ exp2(s - m)
    f32x4 oacc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    struct ChunkIds {
        __amdgpu_buffer_rsrc_t k[BPC], v[BPC];
        bool ok[BPC];
        uint32_t okm;  // bit b = ok[b] (read per lane when blocks are shorter than 16)
    };
    auto fetch_ids = [&](int cs, ChunkIds& ci) {
        ci.okm = 0;
#pragma unroll
        for (int b = 0; b < BPC; ++b) {
            // descriptor b covers the RPB rows from token tok0 on: a whole
            // block when blocks are no longer than a chunk, else the chunk's
            // slice of its (single) block
            const int tok0 = cs + b * RPB;
            const int lb = tok0 / BS;
            const int pid = lb < nb ? bt[lb] : -1;
            // the row count is uniform, but min/max compile to a vector
            // med3; read back as a scalar, the descriptors stay in scalar
            // registers (a descriptor the compiler takes for per-lane would
            // wrap every load in a readfirstlane loop)
            const int rows =
                __builtin_amdgcn_readfirstlane(min(max(end - tok0, 0), RPB));
            const bool ok = pid >= 0 && pid < a.num_blocks && rows > 0;
            const uint32_t nrec = ok ? (uint32_t)((rows - 1) * row_bytes + D * 2) : 0u;
            const size_t boff =
                ok ? (size_t)pid * block_bytes + (size_t)(tok0 - lb * BS) * row_bytes : 0;
            ci.k[b] = make_rsrc(kbase + boff, nrec);
            ci.v[b] = make_rsrc(vbase + boff, nrec);
            ci.ok[b] = ok;
            ci.okm |= (uint32_t)ok << b;
        }
    };
    // Chunks start on descriptor boundaries (partitions are whole blocks, and
    // a block longer than a chunk holds a whole number of chunks). Load i of
    // a chunk brings rows vr + RPI*i (the RPI rows of one load share a block).
    const uint32_t voff = vcv ? (uint32_t)(vc * 16) : kNoSlice;
    // cache policy as in the one-head kernel: head slices that end inside a
    // cache line keep it in L2 for the neighbouring head's wave
    constexpr int AUX = (D * 2) % 128 == 0 ? PA_LOAD_AUX : PA_LOAD_AUX_SHARED_LINES;
    auto issue_rows = [&](const __amdgpu_buffer_rsrc_t (&rs)[BPC], u32x4 (&buf)[VL]) {
#pragma unroll
        for (int i = 0; i < VL; ++i) {
            const int t = vr + RPI * i;
            const int b = (RPI * i) / RPB;
            const int row = t - b * RPB;
            buf[i] = buffer_load16<AUX>(rs[b], (uint32_t)(row * row_bytes) + voff);
        }
    };
    auto issue_k = [&](const ChunkIds& ci, u32x4 (&kb)[VL]) { issue_rows(ci.k, kb); };
    auto issue_v = [&](const ChunkIds& ci, u32x4 (&vb)[VL]) { issue_rows(ci.v, vb); };
    auto to_lds = [&](char* tile, const u32x4 (&buf)[VL]) {
#pragma unroll
        for (int i = 0; i < VL; ++i) *(u32x4*)(tile + (vr + RPI * i) * ROWB + vc * 16) = buf[i];
    };

    // The next chunk's loads are issued on every pass, also after the last
    // chunk, where its descriptors have no range and the loads return zeros
    // without touching memory: a load issued only on some paths would make
    // the wait counts of every path assume it absent, and each wait for
    // this chunk's V would then also wait for the next chunk's K.
    auto process = [&](int cs, const ChunkIds& ci, const u32x4 (&kb)[VL],
                       auto&& prefetch_k, const u32x4 (&vb)[VL], auto&& prefetch_v) {
        // ---- scores Sᵀ: lane (g, n) gets head n, tokens 16s + 4g + k ------
        to_lds(tile, kb);
        prefetch_k();
        f32x4 sc[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            sc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
            const char* krow = tile + (16 * s + n) * ROWB + 16 * g;
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                sc[s] = Mma<KV>::mma(*(const u32x4*)(krow + 64 * j), qb[j], sc[s]);
        }
        float sv[4 * NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            // descriptor of tokens 16s + 4g .. 16s + 4g + 3 (uniform unless
            // a descriptor covers fewer than 16 rows)
            bool bok;
            if constexpr (RPB >= 16) {
                bok = ci.ok[(16 * s) / RPB];
            } else {
                bok = (__builtin_amdgcn_readfirstlane(ci.okm) >> ((16 * s + 4 * g) / RPB)) & 1u;
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int tok = cs + 16 * s + 4 * g + k;
                const bool ok = bok && tok < end;
                sv[4 * s + k] = ok ? sc[s][k] * a.scale_log2 : -INFINITY;
            }
        }
        // ---- online softmax of head n ------------------------------------
        float cm = sv[0];
#pragma unroll
        for (int e = 1; e < 4 * NS; ++e) cm = fmaxf(cm, sv[e]);
        cm = fmaxf(cm, __shfl_xor(cm, 16, 64));
        cm = fmaxf(cm, __shfl_xor(cm, 32, 64));
        const float mn = fmaxf(m, cm);
        const float alpha = mn == -INFINITY ? 1.f : fast_exp2(m - mn);
        float pr[4 * NS];
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 4 * NS; ++e) {
            pr[e] = mn == -INFINITY ? 0.f : fast_exp2(sv[e] - mn);
            ps += pr[e];
        }
        m = mn;
        lsum = lsum * alpha + ps;
#pragma unroll
        for (int t = 0; t < NT; ++t) oacc[t] *= alpha;
        // Pᵀ operands (one per 32-token half) in hi + lo halves
        u32x4 phi[NH], plo[NH];
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            uint32_t hw[8], lw[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float back, back2;
                hw[e] = Mma<KV>::round16(pr[8 * h + e], &back);
                lw[e] = Mma<KV>::round16(pr[8 * h + e] - back, &back2);
            }
            phi[h] = u32x4{hw[0] | (hw[1] << 16), hw[2] | (hw[3] << 16), hw[4] | (hw[5] << 16),
                           hw[6] | (hw[7] << 16)};
            plo[h] = u32x4{lw[0] | (lw[1] << 16), lw[2] | (lw[3] << 16), lw[4] | (lw[5] << 16),
                           lw[6] | (lw[7] << 16)};
        }
        // ---- V rows into the tile (after the K reads), Vᵀ by transpose reads
        to_lds(tile, vb);
        prefetch_v();
        const int e4 = n >> 2, q4 = n & 3;
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            // half h: tokens 32h + 4g + e (e < 4) and 32h + 16 + 4g + e - 4
            const char* r0 = tile + (32 * h + 4 * g + e4) * ROWB + q4 * 8;
            const char* r1 = r0 + 16 * ROWB;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const u32x2 lo = lds_read_tr16(r0 + 32 * t);
                const u32x2 hi = lds_read_tr16(r1 + 32 * t);
                const u32x4 av = u32x4{lo.x, lo.y, hi.x, hi.y};
                oacc[t] = Mma<KV>::mma(av, phi[h], oacc[t]);
                oacc[t] = Mma<KV>::mma(av, plo[h], oacc[t]);
            }
        }
    };

    int cs = start + sub * CH;
    if (cs < end) {
        ChunkIds cur;
        u32x4 kb[VL], vb[VL];
        fetch_ids(cs, cur);
        issue_k(cur, kb);
        issue_v(cur, vb);
        for (;;) {
            const int nx = cs + nwh * CH;
            const bool more = nx < end;
            ChunkIds nxt;
            fetch_ids(nx, nxt);  // descriptors without range when !more
            process(cs, cur, kb, [&] { issue_k(nxt, kb); }, vb, [&] { issue_v(nxt, vb); });
            if (!more) break;
            cur = nxt;
            cs = nx;
        }
    }

    // ---- the fused-append token, once per kv head: head n's score is
    // q_n·k_new (lane group g holds 8 of every 32 elements, then the groups
    // are summed), and O[n][16t + 4g + k] (oacc[t][k]) gains p_n v_new -------
    if (has_new && sub == 0) {
        float t = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const u32x4 kn = *(const u32x4*)&sm_new[wave][0][32 * j + 8 * g];
            t = KV::dot2(kn.x, qb[j].x, t);
            t = KV::dot2(kn.y, qb[j].y, t);
            t = KV::dot2(kn.z, qb[j].z, t);
            t = KV::dot2(kn.w, qb[j].w, t);
        }
        t += __shfl_xor(t, 16, 64);
        t += __shfl_xor(t, 32, 64);
        const float sn = t * a.scale_log2;
        const float mn = fmaxf(m, sn);
        const float alpha = m == -INFINITY ? 0.f : fast_exp2(m - mn);
        const float pn = fast_exp2(sn - mn);
        m = mn;
        lsum = lsum * alpha + (g == 0 ? pn : 0.f);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            const u32x2 vv = *(const u32x2*)&sm_new[wave][1][16 * tt + 4 * g];
            oacc[tt][0] = oacc[tt][0] * alpha + pn * KV::lo(vv.x);
            oacc[tt][1] = oacc[tt][1] * alpha + pn * KV::hi(vv.x);
            oacc[tt][2] = oacc[tt][2] * alpha + pn * KV::lo(vv.y);
            oacc[tt][3] = oacc[tt][3] * alpha + pn * KV::hi(vv.y);
        }
    }

    // ---- per-wave results: head n's (max, sum) and its output rows --------
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    if (g == 0) {
        sm_m[wave][n] = m;
        sm_l[wave][n] = lsum;
    }
    // the wave's tiles are free now: they hold O[16 heads][D] as floats, in
    // rows of OROW floats so the 16 heads' stores fall in different banks
    float* so = (float*)tile;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int k = 0; k < 4; ++k) so[n * OROW + 16 * t + 4 * g + k] = oacc[t][k];
    }
    __syncthreads();

    // ---- merge the waves of each kv head; every thread finishes some
    // (kv head, row, dim) triples ------------------------------------------
    for (int idx = threadIdx.x; idx < (R * G * D << hl); idx += NW * 64) {
        const int hs = idx / (R * G * D);
        const int h = idx / D - hs * (R * G);
        const int d = idx % D;
        if (!row_ok(h)) continue;
        const int w0 = hs * nwh;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w)
            if (w < nwh) M = fmaxf(M, sm_m[w0 + w][h]);
        float tot = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            if (w < nwh) {
                const float mw = sm_m[w0 + w][h];
                const float wt = mw == -INFINITY ? 0.f : fast_exp2(mw - M);
                tot += wt * sm_l[w0 + w][h];
                o += wt * ((const float*)sm_v[w0 + w])[h * OROW + d];
            }
        }
        const float res = tot > 0.f ? o / tot : 0.f;
        const size_t sh = (size_t)row_seq(h) * Hq + (kvh0 + hs) * G + h % G;
        const int np = PREFIX ? (ctx_len(row_seq(h)) + P - 1) / P : nparts;
        // a workgroup that covered the whole context writes the output; on
        // the split path every partition's workspace row is written as well
        // (this group's state in its first partition's row, the group's
        // other partitions marked empty), so the rows describe the whole
        // context whoever merges them
        if (part == 0 && part_end >= np) OUT::store(a.out, sh * D + d, res);
        if (a.part_out) {
            const size_t pidx = sh * a.max_partitions + part;
            a.part_out[pidx * D + d] = res;
            if (d == 0) {
                a.part_max[pidx] = M * kLn2;
                a.part_sum[pidx] = tot;
                for (int q = 1; part + q < part_end && part + q < np; ++q) {
                    a.part_max[pidx + q] = -INFINITY;
                    a.part_sum[pidx + q] = 0.f;
                }
            }
        }
    }
    if (store_new && vcv) {
        const size_t dst = (size_t)a.slot_mapping[seq0] * (Hkv * D) + kvh * D + vc * 8;
        *(u32x4*)((uint16_t*)a.key_cache + dst) = *(const u32x4*)&sm_new[wave][0][vc * 8];
        *(u32x4*)((uint16_t*)a.value_cache + dst) = *(const u32x4*)&sm_new[wave][1][vc * 8];
    }
}

// Instances of one mode: 1 <= num_heads / num_kv_heads <= 16 (2 <= ... for
// plain decode, where a single head takes the one-head kernel).
template <class KV, class OUT, int D, int MODE>
attn_fn pick_gqa_bs(int bs) {
    switch (bs) {
        case 8: return attn_gqa_kernel<KV, OUT, D, 8, kGqaWaves, MODE>;
        case 16: return attn_gqa_kernel<KV, OUT, D, 16, kGqaWaves, MODE>;
        case 32: return attn_gqa_kernel<KV, OUT, D, 32, kGqaWaves, MODE>;
        case 64: return attn_gqa_kernel<KV, OUT, D, 64, kGqaWaves, MODE>;
    }
    return nullptr;
}

template <class KV, class OUT, int MODE>
attn_fn pick_gqa_d(int d, int bs) {
    switch (d) {
        case 64: return pick_gqa_bs<KV, OUT, 64, MODE>(bs);
        case 80: return pick_gqa_bs<KV, OUT, 80, MODE>(bs);
        case 96: return pick_gqa_bs<KV, OUT, 96, MODE>(bs);
        case 128: return pick_gqa_bs<KV, OUT, 128, MODE>(bs);
    }
    return nullptr;
}

template <class KV, int MODE>
attn_fn pick_gqa_out(pa_dtype out, pa_dtype kv, int d, int bs) {
    if (out == PA_F32) return pick_gqa_d<KV, OutF32, MODE>(d, bs);
    if (out != kv) return nullptr;
    if (kv == PA_F16) return pick_gqa_d<KV, OutF16, MODE>(d, bs);
    return pick_gqa_d<KV, OutBF16, MODE>(d, bs);
}

template <int MODE>
attn_fn pick_gqa_mode(pa_dtype kv, pa_dtype out, int d, int bs) {
    if (kv == PA_F16) return pick_gqa_out<KvF16, MODE>(out, kv, d, bs);
    if (kv == PA_BF16) return pick_gqa_out<KvBF16, MODE>(out, kv, d, bs);
    return nullptr;
}

}  // namespace pa
