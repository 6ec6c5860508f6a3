// Prefill over cached prefix blocks on the matrix cores (gfx950).
//
// What is computed (lqnn.cn/news/170268 §3.4 and §1.1): new token t of
// sequence i, at position L_i - S_i + t, attends to the positions 0 ..
// L_i - S_i + t of its paged context: the cached prompt blocks its table
// starts with, then the new tokens themselves (already stored in the cache).
//
// Work decomposition: one workgroup = one (sequence, kv head, tile of
// NW * TR * 16/G consecutive new tokens). Wave w owns TR tiles of 16 rows,
// each 16/G new tokens x the G query heads of the kv head, and keeps their
// online softmax and output in registers for the whole context; there is
// no cross-wave merge. (The instances built use TR = 1: two tiles per wave
// halve the LDS reads per product but measured slower, with fewer waves
// resident.)
// The workgroup walks the context in 32-token chunks, and all its waves
// read each chunk's K and V rows from LDS, so a row of the cache comes from
// memory once per NW * 16 rows rather than once per 16 (the 16-row
// grouped-query kernel's reuse). Chunks are double-buffered in LDS and
// staged through registers: the global loads of chunks c + 1 and c + 2 (of
// c + 1 only at head_dim 256) are in flight while chunk c is computed, and
// one barrier per chunk orders the buffer swap.
//
// Per chunk and tile, the products are those of the grouped-query decode
// kernel: Sᵀ[16 tokens x 16 rows] = K · Qᵀ on v_mfma_f32_16x16x32, the
// online softmax lane-local per row (lane (g, n) holds row n; the max and
// sum over a row's four lanes use the gfx950 lane swaps), and
// Oᵀ[16 d x 16 rows] += Vᵀ · Pᵀ with Vᵀ read by ds_read_b64_tr_b16; P is
// one rounded fp16 value per weight for fp16 caches (the softmax
// denominator sums the rounded weights) and hi + lo halves for bf16 caches,
// whose 8-bit significand is too coarse alone. Each row is masked to positions up to
// its own; a wave whose rows all sit before a chunk, or that has no rows,
// skips its products (it still loads and waits at the barrier).
//
// Shared-prefix mode (SH, lqnn.cn/news/170268 §4.3: requests that hit the
// same cached prompt): the new tokens of all sequences form one list of
// rows and a workgroup takes consecutive ones, whatever their sequences.
// It streams the shared prompt blocks once for all its rows, then each of
// its sequences' own positions for that sequence's rows only; the online
// softmax runs on across the streams, so no merge is needed.
//
// The same kernel has a decode mode (no query_start): one new token per
// sequence and context partitions with the split path's workspace rows.
// The decode calls use it at head_dim 256, where it has the registers the
// head_dim-128 decode kernels lack.
#pragma once

#include "pa_attn_gqa.h"
#include "pa_kernels.h"

namespace pa {

// Max and sum over the four lanes n, n + 16, n + 32, n + 48 (the row
// groups of an MFMA output) with the gfx950 lane swaps, on the VALU.
__device__ __forceinline__ float max_over_groups(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_groups(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Waves per SIMD the registers are budgeted for (measured on MI355X: 4
// rather than the 3 the compiler picks by itself took the 32-head prefill
// from 487 to 438 µs; 5, for 8-wave workgroups, was slower again).
#ifndef PA_PREFILL_WAVES_PER_EU
#define PA_PREFILL_WAVES_PER_EU 4
#endif

// Cache policy of the prefill's K/V loads (0: default, 2: non-temporal).
// Unlike decode, prefill re-reads a cached prompt shared by many requests
// (each kv head's prompt blocks by every request's workgroups), and the
// default policy keeps it in L2: measured on MI355X, the 32-head workload
// ran 406 µs with non-temporal loads and 321 µs with the default.
#ifndef PA_PREFILL_LOAD_AUX
#define PA_PREFILL_LOAD_AUX 0
#endif

// Chunks of K/V in flight per wave: 2 (two register sets) where a chunk
// takes at most two loads of K and of V per lane, else 1 (head_dim 256:
// two sets of four would cost 32 registers and the waves that hide
// latency).
#ifndef PA_PREFILL_MAX_DEPTH
#define PA_PREFILL_MAX_DEPTH 2
#endif

// Vᵀ operand tiles (of 8) read from LDS ahead of the softmax, in 8-wave
// workgroups (0: all after it)
#ifndef PA_PREFILL_V_EARLY
#define PA_PREFILL_V_EARLY 4
#endif
// Masked scores selected in their own registers (1: a select with a tied
// operand, so that the unmasked path, taken by most chunks, needs no copy
// of the scores where the paths join; measured on MI355X about 3% faster
// for both prefill workloads) or by the compiler's selects (0)
#ifndef PA_PREFILL_MASK_IN_PLACE
#define PA_PREFILL_MASK_IN_PLACE 1
#endif
// fp16 caches: weights as one rounded fp16 value (1) or hi + lo halves (0)
#ifndef PA_PREFILL_F16_SINGLE_P
#define PA_PREFILL_F16_SINGLE_P 1
#endif

// Finds the request of flattened new token tok among requests lo .. hi:
// the last r in that range with query_start[r] <= tok (requests without
// new tokens are passed over).
__device__ __forceinline__ int request_of(const int32_t* qs, int lo, int hi, int tok) {
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (qs[mid] <= tok) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

template <class KV, class OUT, int D, int BS, int NW, int TR, bool SH>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(PA_PREFILL_WAVES_PER_EU))) void attn_prefill_kernel(AttnArgs a) {
    constexpr int CH = 32;         // tokens per chunk
    constexpr int NS = CH / 16;    // 16-token sub-blocks of a chunk
    // head_dim 80 and 96 are laid out as 128 (the missing slices read as
    // zeros, so they add nothing to q·k and give output columns never
    // stored); 64, 128 and 256 as themselves
    constexpr int DP = D <= 64 ? 64 : (D <= 128 ? 128 : 256);
    constexpr int NJ = DP / 32;    // q·k products per 16-token sub-block
    constexpr int NT = DP / 16;    // 16-wide output tiles of head_dim
    constexpr int LPR = DP / 8;    // lanes per row of a 16-byte load
    constexpr int RPW = 64 / LPR;  // rows one wave loads per instruction (4 or 8)
    constexpr int RPL = NW * RPW;  // rows the workgroup loads per instruction
    constexpr int LPC = CH / RPL;  // load instructions per chunk, of K and of V
    // LDS bytes per row: 32 bytes of padding make the 16-byte K reads and
    // the transposed V reads free of bank conflicts (measured on MI355X,
    // 16 waves on a CU: 4.4 and 2.6 cycles per instruction; a 16-byte pad
    // left both 2-way, 8.1 and 4.1)
    constexpr int ROWB = DP * 2 + PA_LDS_ROW_PAD;
    constexpr int TILE = CH * ROWB;
    constexpr int BSC = BS < CH ? BS : CH;  // tokens of a chunk in one block
    constexpr uint32_t kBlockBits = BSC == 32 ? 0xffffffffu : (1u << BSC) - 1u;
    static_assert(LPC >= 1 && LPC * RPL == CH, "the workgroup's loads tile the chunk");
    static_assert(BS % RPW == 0, "the rows of one wave's load share a block");
    static_assert(NS == 2, "one p·v contraction (32 tokens) per chunk");
    constexpr int DEPTH = LPC <= 2 ? PA_PREFILL_MAX_DEPTH : 1;
    // fp16 caches: the weights enter the p·v product as one fp16 value each
    // (11 significant bits), and the softmax denominator sums those same
    // rounded weights, so the output is an exact weighted average of the V
    // rows whose weights differ from the true ones by at most 2^-10
    // relative; bf16 caches keep hi + lo halves (8 bits would not do)
    constexpr bool ONE_P = std::is_same<KV, KvF16>::value && PA_PREFILL_F16_SINGLE_P;

    __shared__ __attribute__((aligned(16))) char sm_k[2][TILE];
    __shared__ __attribute__((aligned(16))) char sm_v[2][TILE];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;      // lane group
    const int n = lane & 15;      // row of a tile (column of every product)
    const int lr = lane / LPR;    // row of a wave's load
    const int lc = lane % LPR;    // 16-byte slice of that row

    const int Hq = a.num_heads;
    const int Hkv = a.num_kv_heads;
    const int G = Hq / Hkv;
    const int R = 16 / G;  // new tokens per 16-row tile
    const int Lmax = a.max_blocks_per_seq * BS;

    // Decode mode (no query_start): one new token per sequence, query and
    // out rows indexed by sequence, the context split into partitions of
    // partition_size whose (max, sum, normalised output) go to the split
    // workspace when a sequence has several; the grid's second coordinate
    // is then the partition instead of the tile of new tokens.
    const bool dec = !SH && a.query_start == nullptr;
    // Prefix-only decode (shared-prefix mode without query_start): one new
    // token per sequence, rows indexed by sequence; the workgroup streams
    // one partition of the shared prefix for all its rows and writes each
    // row's (max, sum, normalised output) of that partition to the split
    // workspace. The grid's coordinates are the kv head, the tile of rows
    // and the prefix partition.
    const bool pfx = SH && a.query_start == nullptr;
    int kvh, seq = 0, part = 0, qb0 = 0, S = 0, L = 0, start = 0, end = 0, tw, wend = 0,
        first_pos;
    int pstart = 0, pend = 0;  // shared-prefix mode: the prefix positions streamed
    int nparts = 1;
    bool rowv[TR];
    int lim[TR];  // last position row n of tile u attends to (-1: padding row)
    int rq[TR];   // shared-prefix mode: the request of row n of tile u
    size_t orow[TR];
    // shared-prefix mode: the prefix, the workgroup's requests
    int ps = 0, r_lo = 0, r_hi = -1;
    if constexpr (!SH) {
        // Decode mode (no query_start): one new token per sequence, query
        // and out rows indexed by sequence, the context split into
        // partitions of partition_size whose (max, sum, normalised output)
        // go to the split workspace when a sequence has several; the
        // grid's second coordinate is then the partition instead of the
        // tile of new tokens.
        int bid = blockIdx.x;  // kv head fastest, then token tile (partition), then sequence
        kvh = bid % Hkv;
        bid /= Hkv;
        const int tile = dec ? 0 : bid % a.num_q_tiles;
        part = dec ? bid % a.num_q_tiles : 0;
        seq = bid / a.num_q_tiles;
        qb0 = dec ? seq : a.query_start[seq];
        S = dec ? 1 : a.query_start[seq + 1] - qb0;
        const int t0 = tile * NW * TR * R;  // the workgroup's first new token
        if (t0 >= S) return;                // uniform over the workgroup
        L = a.context_lens[seq];
        L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
        const int P = a.partition_size;
        nparts = dec ? (L + P - 1) / P : 1;
        if (part > 0 && part >= nparts) return;  // uniform over the workgroup
        start = part * P;
        // positions the workgroup reads: up to its last row's own position
        end = min(max(min(L, L - S + t0 + min(NW * TR * R, S - t0)), 0), dec ? start + P : L);
        // this wave's tiles: tile u holds new tokens tw + u*R .. + R - 1
        tw = t0 + wave * TR * R;
        const int nq = max(min(TR * R, S - tw), 0);  // new tokens of the wave
        wend = nq > 0 ? max(min(L, L - S + tw + nq), 0) : 0;  // 0: no rows
        first_pos = L - S + tw;  // position of the wave's first row
#pragma unroll
        for (int u = 0; u < TR; ++u) {
            const int tok = tw + u * R + n / G;  // the new token of row n
            rowv[u] = n < R * G && tok < S;
            lim[u] = rowv[u] ? L - S + tok : -1;
            rq[u] = seq;
            orow[u] = ((size_t)(qb0 + (rowv[u] ? tok : 0)) * Hq + kvh * G + n % G) * D;
        }
    } else {
        // Shared-prefix mode: the new tokens of all requests are one list of
        // rows (query_start[num_seqs] of them); a workgroup takes NW*TR*R
        // consecutive tokens, whatever their requests. The first ps
        // positions are the same blocks for every request (read through
        // block_tables row 0): the workgroup streams them once for all its
        // rows, then each of its requests' own positions ps .. L_r - 1 for
        // that request's rows.
        const int32_t* qs = a.query_start;
        const int B = a.num_seqs;
        const int T = pfx ? B : qs[B];
        kvh = blockIdx.x % Hkv;
        int tile = blockIdx.x / Hkv;
        const int rows_wg = NW * TR * R;  // new tokens (rows of one head) per workgroup
        if (pfx) {
            const int ntl = (T + rows_wg - 1) / rows_wg;
            part = tile / ntl;
            tile -= part * ntl;
        }
        const int t0 = tile * rows_wg;
        if (t0 >= T) return;  // uniform over the workgroup
        ps = min(a.prefix_tokens, Lmax);
        pstart = pfx ? part * a.partition_size : 0;
        pend = pfx ? min(pstart + a.partition_size, ps) : ps;
        r_lo = pfx ? t0 : __builtin_amdgcn_readfirstlane(request_of(qs, 0, B - 1, t0));
        r_hi = pfx ? min(t0 + rows_wg, T) - 1
                   : __builtin_amdgcn_readfirstlane(
                         request_of(qs, r_lo, B - 1, min(t0 + rows_wg, T) - 1));
        tw = t0 + wave * TR * R;
        int lo_pos = 0x7fffffff;
#pragma unroll
        for (int u = 0; u < TR; ++u) {
            const int tok = tw + u * R + n / G;
            rowv[u] = n < R * G && tok < T;
            // (a short search)
            const int r = pfx ? (rowv[u] ? tok : t0) : request_of(qs, r_lo, r_hi, rowv[u] ? tok : t0);
            int Lr = a.context_lens[r];
            Lr = Lr < 0 ? 0 : (Lr > Lmax ? Lmax : Lr);
            const int pos = pfx ? Lr - 1 : Lr - (qs[r + 1] - qs[r]) + (tok - qs[r]);
            lim[u] = rowv[u] ? pos : -1;
            rq[u] = r;
            orow[u] = ((size_t)(rowv[u] ? tok : 0) * Hq + kvh * G + n % G) * D;
            if (rowv[u]) lo_pos = min(lo_pos, pos);
        }
        // the wave's smallest row position (prefix chunks at or before it
        // need no mask)
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) lo_pos = min(lo_pos, __shfl_xor(lo_pos, o));
        first_pos = __builtin_amdgcn_readfirstlane(lo_pos);
    }
    const int head = kvh * G + n % G;
    const size_t row_bytes = (size_t)Hkv * D * 2;
    const size_t block_bytes = row_bytes * BS;
    const char* kbase = (const char*)a.key_cache + (size_t)kvh * D * 2;
    const char* vbase = (const char*)a.value_cache + (size_t)kvh * D * 2;
    const uint32_t loff = (uint32_t)(lr * row_bytes) + (lc * 8 < D ? (uint32_t)(lc * 16) : kNoSlice);

    // Qᵀ operands: lane (g, n) holds row n's q[32j + 8g .. +7]; padding rows are 0
    u32x4 qb[TR][NJ];
#pragma unroll
    for (int u = 0; u < TR; ++u) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            qb[u][j] = u32x4{0u, 0u, 0u, 0u};
            if (rowv[u] && 32 * j + 8 * g < D)
                qb[u][j] = *(const u32x4*)(a.query + orow[u] + 32 * j + 8 * g);
        }
    }

    // reference max of row n's scores (log2 units): a finite sentinel below
    // any score, so that exp2(s - m) of a masked score (-inf) is 0 before
    // the first real score arrives
    float m[TR], lsum[TR];  // lsum: this lane's share of row n's Σ exp2(s - m)
    // how far a chunk's max may pass the reference before it moves (log2
    // units); 0 in the decode modes, whose partitions report their exact max
    const float thr = dec || pfx ? 0.f : 8.f;
    f32x4 oacc[TR][NT];
#pragma unroll
    for (int u = 0; u < TR; ++u) {
        m[u] = -1e30f;
        lsum[u] = 0.f;
#pragma unroll
        for (int t = 0; t < NT; ++t) oacc[u][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // ---- the scale: scores are kept unscaled and the scale enters the
    // exponent, exp2(s·c - m) by one fma. c = |scale·log2 e| > 0 (a zero
    // scale as the smallest normal float: every weight then rounds to
    // exactly 1, the uniform average a zero scale means); a negative scale
    // negates q instead, which is exact ----------------------------------
    const float sl = fmaxf(fabsf(a.scale_log2), 1.17549435e-38f);
    if (a.scale_log2 < 0.f) {
#pragma unroll
        for (int u = 0; u < TR; ++u) {
#pragma unroll
            for (int j = 0; j < NJ; ++j) qb[u][j] ^= 0x80008000u;
        }
    }

    // ---- loads: instruction j of a chunk brings rows j*RPL + wave*RPW + lr,
    // through a descriptor whose range ends at the wave's last valid row (an
    // absent block, or rows at or past `end`, read as zeros) ---------------
    // The scalar unit issues as much per chunk as the vector units, so the
    // per-chunk address work is kept small: a chunk's table entries are read
    // once, together, at clamped indices (chunk starts are multiples of BSC,
    // partitions being multiples of the block size, so a chunk covers blocks
    // lb0 .. lb0 + NBC - 1), block offsets use 32-bit products (blocks are
    // below 2^27 bytes), and what depends only on the wave is computed once.
    constexpr int LOG_BS = BS == 8 ? 3 : (BS == 16 ? 4 : (BS == 32 ? 5 : 6));
    static_assert((1 << LOG_BS) == BS, "block size a power of two");
    constexpr int NBC = CH / BSC;  // blocks of a chunk
    const uint32_t nblk = (uint32_t)a.num_blocks;
    const uint32_t row32 = (uint32_t)row_bytes;
    const uint32_t block32 = (uint32_t)block_bytes;
    const int pad = (int)row32 - D * 2;  // bytes from a row's head slice to the next row
    // per load j: the wave's first row of the chunk, x_j = j*RPL + wave*RPW,
    // and the bases of its row within a block (for BS = 64 a chunk starts
    // at row 0 or 32 of its block, added per chunk)
    const char* kb_j[LPC];
    const char* vb_j[LPC];
#pragma unroll
    for (int j = 0; j < LPC; ++j) {
        const uint32_t x = (uint32_t)(j * RPL + wave * RPW);
        const size_t o = (size_t)((BS < CH ? x & (BS - 1) : x) * row32);
        kb_j[j] = kbase + o;
        vb_j[j] = vbase + o;
    }
    typedef u32x4 Stage[LPC];  // one chunk's rows of this lane, K or V
    // Issues the loads of chunk cs of a stream of positions below tend whose
    // table tb has tnb entries, into (kr, vr); returns bit e set when
    // position cs + e lies in a block of the pool (in decode mode and in
    // shared-prefix mode also below tend). Rows below tend lie in blocks
    // below tnb, so a block's place in the table needs no test of its own:
    // the row counts cover it.
    // Each select depends on one comparison (the compiler turns a
    // combination of comparisons into lane masks and several instructions).
    // With `full` true the caller knows the whole chunk lies below tend (so
    // within the table): no clamping, and every load's range is whole.
    const int full_bytes = RPW * (int)row32 - pad;
    auto issue = [&](int cs, const int32_t* tb, int tnb, int tend, Stage& kr, Stage& vr,
                     auto full) -> uint32_t {
        constexpr bool FULL = decltype(full)::value;
        const uint32_t lb0 = (uint32_t)cs >> LOG_BS;
        const uint32_t last = tnb > 0 ? (uint32_t)tnb - 1 : 0;  // a table entry that exists
        uint32_t pid[NBC];
#pragma unroll
        for (int b = 0; b < NBC; ++b) {
            const uint32_t lb = lb0 + b;
            pid[b] = (uint32_t)tb[FULL || lb < last ? lb : last];
        }
        uint32_t okm = 0;
#pragma unroll
        for (int b = 0; b < NBC; ++b) okm |= pid[b] < nblk ? kBlockBits << (b * BSC) : 0u;
        const int rest = tend - cs;  // rows of the chunk below tend
        // (per-request prefill: every row's limit is below tend; not so in
        // decode mode, nor for the shared prefix, which ends where each
        // request's own positions begin)
        if (!FULL && (dec || SH))
            okm &= rest >= CH ? 0xffffffffu : (rest > 0 ? (1u << rest) - 1u : 0u);
        const size_t coff = BS > CH ? (size_t)(((uint32_t)cs & (BS - 1)) * row32) : 0;
#pragma unroll
        for (int j = 0; j < LPC; ++j) {
            // the load's block within the chunk: fixed when a load's rows
            // never straddle blocks (BS a multiple of RPL)
            uint32_t p = pid[0];
            if constexpr (BS < CH) {
                if constexpr (BS % RPL == 0) {
                    p = pid[(j * RPL) >> LOG_BS];
                } else {
                    const int bi = (j * RPL + wave * RPW) >> LOG_BS;
#pragma unroll
                    for (int b = 1; b < NBC; ++b) p = bi == b ? pid[b] : p;
                }
            }
            // bytes of the wave's rows below `end`, up to the last row's
            // head slice (none: 0, whatever the base)
            // (readfirstlane: the compiler would keep it per lane, and a
            // per-lane range makes it loop over the lanes' values)
            const int rr = FULL ? RPW : min(rest - (j * RPL + wave * RPW), RPW);
            const int bytes = FULL ? full_bytes : max(rr * (int)row32 - pad, 0);
            const uint32_t nrec = __builtin_amdgcn_readfirstlane(p < nblk ? (uint32_t)bytes : 0u);
            const size_t boff = (size_t)p * block32 + coff;
            kr[j] = buffer_load16<PA_PREFILL_LOAD_AUX>(make_rsrc(kb_j[j] + boff, nrec), loff);
            vr[j] = buffer_load16<PA_PREFILL_LOAD_AUX>(make_rsrc(vb_j[j] + boff, nrec), loff);
        }
        return okm;
    };
    constexpr std::false_type kPart{};
    constexpr std::true_type kWhole{};
    auto stash = [&](int buf, const Stage& kr, const Stage& vr) {
#pragma unroll
        for (int j = 0; j < LPC; ++j) {
            const int row = j * RPL + wave * RPW + lr;
            *(u32x4*)(sm_k[buf] + row * ROWB + lc * 16) = kr[j];
            *(u32x4*)(sm_v[buf] + row * ROWB + lc * 16) = vr[j];
        }
    };

    // lane (g, n) holds tokens 16s + 4g + k of row n; dl: row n's limit
    // less 4g, so that token 16s + k of chunk cs is visible when
    // 16s + k <= dl - cs
    int dl[TR];
#pragma unroll
    for (int u = 0; u < TR; ++u) dl[u] = lim[u] - 4 * g;

    // rseg: shared-prefix mode, the request whose own positions the chunk
    // holds (its rows alone attend to it), or -1 for the shared prefix
    auto compute = [&](int cs, int rseg, uint32_t okm, const char* kt, const char* vt) {
        const bool all = okm == 0xffffffffu;
        // a chunk wholly present and at or before every row's own position
        // needs no mask (most chunks of a long cached prefix)
        const bool inside = all & (cs + CH - 1 <= first_pos) & (rseg < 0);
        // ---- scores Sᵀ: lane (g, n) gets row n, tokens 16s + 4g + k; each
        // K operand read from LDS serves every tile of the wave ------------
        // (the sub-blocks' products interleaved: two independent accumulation
        // chains, so each product's wait for the previous one overlaps)
        f32x4 sc[TR][NS];
        const char* krow = kt + n * ROWB + 16 * g;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
#pragma unroll
            for (int u = 0; u < TR; ++u) sc[u][s] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const u32x4 kv = *(const u32x4*)(krow + 16 * s * ROWB + 64 * j);
#pragma unroll
                for (int u = 0; u < TR; ++u) sc[u][s] = Mma<KV>::mma(kv, qb[u][j], sc[u][s]);
            }
        }
        // the Vᵀ operands of the first d tiles, read ahead of the softmax:
        // their LDS latency then overlaps its arithmetic
        const int e4 = n >> 2, q4 = n & 3;
        const char* r0 = vt + (4 * g + e4) * ROWB + q4 * 8;
        const char* r1 = r0 + 16 * ROWB;
        // (8-wave workgroups only: with 4, the staging registers leave no room)
        constexpr int VE = NW < 8 ? 0 : (PA_PREFILL_V_EARLY < NT ? PA_PREFILL_V_EARLY : NT);
        u32x4 ave[VE > 0 ? VE : 1];
#pragma unroll
        for (int t = 0; t < VE; ++t) {
            const u32x2 lo = lds_read_tr16(r0 + 32 * t);
            const u32x2 hi = lds_read_tr16(r1 + 32 * t);
            ave[t] = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
        u32x4 phi[TR], plo[TR];
#pragma unroll
        for (int u = 0; u < TR; ++u) {
            // unscaled scores, -inf where masked (the branches are uniform;
            // the masks are selects, no short-circuit)
            // (masked in place, so that every path leaves them in the same
            // registers)
            float sv[4 * NS];
#pragma unroll
            for (int e = 0; e < 4 * NS; ++e) sv[e] = sc[u][e / 4][e % 4];
            if (!inside) {
                int d = dl[u] - cs;
                if constexpr (SH) d = ((rseg < 0) | (rq[u] == rseg)) ? d : -1;
#if PA_PREFILL_MASK_IN_PLACE
                // v_cndmask writes the score's own register; the nop gives
                // it the two wait states a lane mask just written by a
                // vector compare needs before a vector instruction reads it
                const float ninf = -INFINITY;
                const uint32_t lm = all ? 0xffffffffu : okm >> (4 * g);
#pragma unroll
                for (int e = 0; e < 4 * NS; ++e) {
                    const int t = (e / 4) * 16 + e % 4;
                    const bool ok = (((lm >> t) & 1u) != 0u) & (t <= d);
                    const uint64_t off = __builtin_amdgcn_ballot_w64(!ok);
                    asm("s_nop 1\n\tv_cndmask_b32_e64 %0, %0, %1, %2"
                        : "+v"(sv[e])
                        : "v"(ninf), "s"(off));
                }
#else
                if (all) {  // every block present: the row limit alone
#pragma unroll
                    for (int e = 0; e < 4 * NS; ++e)
                        sv[e] = (e / 4) * 16 + e % 4 <= d ? sv[e] : -INFINITY;
                } else {
                    const uint32_t lm = okm >> (4 * g);
#pragma unroll
                    for (int e = 0; e < 4 * NS; ++e) {
                        const int t = (e / 4) * 16 + e % 4;
                        const bool ok = (((lm >> t) & 1u) != 0u) & (t <= d);
                        sv[e] = ok ? sv[e] : -INFINITY;
                    }
                }
#endif
            }
            // ---- online softmax of row n ---------------------------------
            // The reference m moves only when a score of the chunk passes it
            // by more than thr (log2 units), and then for every row of the
            // tile, to the row's max: the result is the same for any
            // reference, the weights stay below 2^thr, and most chunks skip
            // rescaling the accumulators (and the max across lanes).
            // The test uses this lane's own max; the row's max (across its
            // four lanes) is only needed when some reference moves.
            float cr = sv[0];
#pragma unroll
            for (int e = 1; e < 4 * NS; ++e) cr = fmaxf(cr, sv[e]);
            if (__builtin_amdgcn_ballot_w64(cr * sl > m[u] + thr) != 0) {
                const float cm = max_over_groups(cr) * sl;
                const float mn = fmaxf(m[u], cm);
                const float alpha = fast_exp2(m[u] - mn);  // 0 while m is the sentinel
                m[u] = mn;
                lsum[u] *= alpha;
#pragma unroll
                for (int t = 0; t < NT; ++t) oacc[u][t] *= alpha;
            }
            const float nm = -m[u];
            float pr[4 * NS];
#pragma unroll
            for (int e = 0; e < 4 * NS; ++e) pr[e] = fast_exp2(fmaf(sv[e], sl, nm));
            static_assert(4 * NS == 8, "the sums below add eight weights");
            if constexpr (ONE_P) {
                // Pᵀ operand: the weights rounded to fp16, and the row's sum
                // of exactly those values (dot2 with (1, 1): each pair
                // exactly, accumulated in fp32)
                typedef _Float16 h2 __attribute__((ext_vector_type(2)));
                typedef float f2 __attribute__((ext_vector_type(2)));
                uint32_t hw[4];
                float ps = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const h2 h = __builtin_convertvector(f2{pr[2 * e], pr[2 * e + 1]}, h2);
                    ps = __builtin_amdgcn_fdot2(h, h2{(_Float16)1.0f, (_Float16)1.0f}, ps, false);
                    hw[e] = __builtin_bit_cast(uint32_t, h);
                }
                lsum[u] += ps;
                phi[u] = u32x4{hw[0], hw[1], hw[2], hw[3]};
            } else {
                lsum[u] +=
                    ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
                // Pᵀ operand in hi + lo halves
                uint32_t hw[4], lw[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    Mma<KV>::split2(pr[2 * e], pr[2 * e + 1], &hw[e], &lw[e]);
                phi[u] = u32x4{hw[0], hw[1], hw[2], hw[3]};
                plo[u] = u32x4{lw[0], lw[1], lw[2], lw[3]};
            }
        }
        // ---- Oᵀ += Vᵀ · Pᵀ: tokens 4g + e (e < 4) and 16 + 4g + e - 4; each
        // Vᵀ operand serves every tile ------------------------------------
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            u32x4 av;
            if (t < VE) {
                av = ave[t < VE ? t : 0];
            } else {
                const u32x2 lo = lds_read_tr16(r0 + 32 * t);
                const u32x2 hi = lds_read_tr16(r1 + 32 * t);
                av = u32x4{lo.x, lo.y, hi.x, hi.y};
            }
#pragma unroll
            for (int u = 0; u < TR; ++u) {
                oacc[u][t] = Mma<KV>::mma(av, phi[u], oacc[u][t]);
                if constexpr (!ONE_P) oacc[u][t] = Mma<KV>::mma(av, plo[u], oacc[u][t]);
            }
        }
    };

    // ---- the context, chunk by chunk; every wave takes every iteration
    // (the barrier), a wave computes only chunks that hold a position one
    // of its rows attends to. The loads and stores run on every pass, also
    // past the last chunk, where their descriptors have no range (zeros, no
    // memory traffic): a load issued on some paths only would make the wait
    // counts of every path assume it absent, and the first product of a
    // chunk would then wait for the next chunk's loads. The table reads of
    // chunk c + 1 come with its loads, before chunk c's LDS reads, whose
    // wait counter they share. ---------------------------------------------
    const int32_t* bt = a.block_tables + (size_t)seq * a.max_blocks_per_seq;
    const int nb = (L + BS - 1) / BS;
    if constexpr (!SH) {
        const int nch = (max(end - start, 0) + CH - 1) / CH;
        if constexpr (DEPTH == 1) {
            Stage kr, vr;
            uint32_t okm = issue(start, bt, nb, end, kr, vr, kPart);
            stash(0, kr, vr);
            __syncthreads();
            for (int c = 0; c < nch; ++c) {
                const int cs = start + c * CH;
                const uint32_t okm_next = issue(cs + CH, bt, nb, end, kr, vr, kPart);
                if (cs < wend) compute(cs, -1, okm, sm_k[c & 1], sm_v[c & 1]);
                stash((c + 1) & 1, kr, vr);
                __syncthreads();
                okm = okm_next;
            }
        } else {
            // Two chunks in flight: register set 0 stages the even chunks,
            // set 1 the odd ones, and the loop is unrolled by two so that
            // both sets and both LDS buffers are fixed in each half. In step
            // c the loads of chunk c + 2 are issued, chunk c is computed
            // from LDS, and chunk c + 1 (issued a step earlier) is stored to
            // the other buffer; its wait leaves chunk c + 2's loads in
            // flight.
            Stage k0, v0, k1, v1;
            uint32_t okm0 = issue(start, bt, nb, end, k0, v0, kPart);
            uint32_t okm1 = issue(start + CH, bt, nb, end, k1, v1, kPart);
            stash(0, k0, v0);
            __syncthreads();
            int c = 0;
            // while the chunks two steps ahead lie wholly below end, their
            // loads are whole (no clamped table index, no per-load range)
            const int nwhole = (end - start) / CH;
            for (; c + 3 < nwhole; c += 2) {
                const int cs = start + c * CH;
                const uint32_t okm2 = issue(cs + 2 * CH, bt, nb, end, k0, v0, kWhole);
                if (cs < wend) compute(cs, -1, okm0, sm_k[0], sm_v[0]);
                stash(1, k1, v1);
                __syncthreads();
                okm0 = okm2;
                const uint32_t okm3 = issue(cs + 3 * CH, bt, nb, end, k1, v1, kWhole);
                if (cs + CH < wend) compute(cs + CH, -1, okm1, sm_k[1], sm_v[1]);
                stash(0, k0, v0);
                __syncthreads();
                okm1 = okm3;
            }
            for (; c < nch; c += 2) {
                {
                    const int cs = start + c * CH;
                    const uint32_t okm2 = issue(cs + 2 * CH, bt, nb, end, k0, v0, kPart);
                    if (cs < wend) compute(cs, -1, okm0, sm_k[0], sm_v[0]);
                    stash(1, k1, v1);
                    __syncthreads();
                    okm0 = okm2;
                }
                if (c + 1 >= nch) break;
                {
                    const int cs = start + (c + 1) * CH;
                    const uint32_t okm3 = issue(cs + 2 * CH, bt, nb, end, k1, v1, kPart);
                    if (cs < wend) compute(cs, -1, okm1, sm_k[1], sm_v[1]);
                    stash(0, k0, v0);
                    __syncthreads();
                    okm1 = okm3;
                }
            }
        }
    } else {
        // The workgroup's streams, one after another: the shared prefix
        // (positions 0 .. ps - 1, table row 0), then for each of its
        // requests r with positions past the prefix, positions ps .. L_r - 1
        // of r's table. A cursor is one chunk of one stream; a finished
        // cursor (r = kDone) has no positions and loads nothing.
        constexpr int kDone = 0x3fffffff;
        struct Cur {
            int r, cs, end, nb;
            const int32_t* tb;
        };
        const int32_t* qs = a.query_start;
        // the first stream of request r or a later one of the workgroup
        auto stream_from = [&](int r) -> Cur {
            if (pfx) r = r_hi + 1;  // the prefix partition is the only stream
            for (; r <= r_hi; ++r) {
                int Lr = a.context_lens[r];
                Lr = Lr < 0 ? 0 : (Lr > Lmax ? Lmax : Lr);
                if (qs[r + 1] > qs[r] && Lr > ps)
                    return Cur{r, ps, Lr, (Lr + BS - 1) / BS,
                               a.block_tables + (size_t)r * a.max_blocks_per_seq};
            }
            return Cur{kDone, 0, 0, 1, a.block_tables};
        };
        auto next = [&](Cur c) -> Cur {
            c.cs += CH;
            if (c.cs < c.end || c.r == kDone) return c;
            return stream_from(c.r < 0 ? r_lo : c.r + 1);
        };
        // does a row of this wave attend to a position of chunk c
        auto wanted = [&](const Cur& c) -> bool {
            bool any = false;
#pragma unroll
            for (int u = 0; u < TR; ++u)
                any |= ((c.r < 0) | (rq[u] == c.r)) & (lim[u] >= c.cs);
            return __builtin_amdgcn_ballot_w64(any) != 0;
        };
        Cur c0 = pend > pstart ? Cur{-1, pstart, pend, ps / BS, a.block_tables}
                               : stream_from(r_lo);
        Cur c1 = next(c0);
        if constexpr (DEPTH == 1) {
            Stage kr, vr;
            uint32_t okm = issue(c0.cs, c0.tb, c0.nb, c0.end, kr, vr, kPart);
            stash(0, kr, vr);
            __syncthreads();
            for (int buf = 0; c0.r != kDone; buf ^= 1) {
                const uint32_t okm_next = issue(c1.cs, c1.tb, c1.nb, c1.end, kr, vr, kPart);
                if (wanted(c0)) compute(c0.cs, c0.r, okm, sm_k[buf], sm_v[buf]);
                stash(buf ^ 1, kr, vr);
                __syncthreads();
                okm = okm_next;
                c0 = c1;
                c1 = next(c1);
            }
        } else {
            Stage k0, v0, k1, v1;
            uint32_t okm0 = issue(c0.cs, c0.tb, c0.nb, c0.end, k0, v0, kPart);
            uint32_t okm1 = issue(c1.cs, c1.tb, c1.nb, c1.end, k1, v1, kPart);
            stash(0, k0, v0);
            __syncthreads();
            // The shared prompt's chunks while the chunks two steps ahead are
            // still inside it: the cursor is the position alone, and no test
            // of the rows runs (a chunk that no row attends to would only be
            // masked out whole).
            if (c0.r < 0) {
                const int nb0 = ps / BS;
                int cs = c0.cs;
                while (cs + 4 * CH <= pend) {  // chunks cs .. cs + 3 CH whole in the prompt
                    const uint32_t okm2 = issue(cs + 2 * CH, a.block_tables, nb0, pend, k0, v0, kWhole);
                    compute(cs, -1, okm0, sm_k[0], sm_v[0]);
                    stash(1, k1, v1);
                    __syncthreads();
                    okm0 = okm2;
                    const uint32_t okm3 = issue(cs + 3 * CH, a.block_tables, nb0, pend, k1, v1, kWhole);
                    compute(cs + CH, -1, okm1, sm_k[1], sm_v[1]);
                    stash(0, k0, v0);
                    __syncthreads();
                    okm1 = okm3;
                    cs += 2 * CH;
                }
                c0.cs = cs;
                c1 = next(c0);
            }
            while (c0.r != kDone) {
                const Cur c2 = next(c1);
                {
                    const uint32_t okm2 = issue(c2.cs, c2.tb, c2.nb, c2.end, k0, v0, kPart);
                    if (wanted(c0)) compute(c0.cs, c0.r, okm0, sm_k[0], sm_v[0]);
                    stash(1, k1, v1);
                    __syncthreads();
                    okm0 = okm2;
                }
                if (c1.r == kDone) break;
                const Cur c3 = next(c2);
                {
                    const uint32_t okm3 = issue(c3.cs, c3.tb, c3.nb, c3.end, k1, v1, kPart);
                    if (wanted(c1)) compute(c1.cs, c1.r, okm1, sm_k[1], sm_v[1]);
                    stash(0, k0, v0);
                    __syncthreads();
                    okm1 = okm3;
                }
                c0 = c2;
                c1 = c3;
            }
        }
    }

    // ---- row n's output: O[n][16t + 4g + k] = oacc[t][k] / Σ. In decode
    // mode on the split path (a workspace is given) the partition's row of
    // the workspace is written too, and a single partition, which is the
    // whole context, also gives the output itself --------------------------
    // (prefix-only decode: the workspace row of the row's sequence and the
    // prefix partition, never the output)
    const bool partial = (dec || pfx) && a.part_out != nullptr;
    const bool whole = !pfx && (!dec || nparts <= 1);
#pragma unroll
    for (int u = 0; u < TR; ++u) {
        const float tot = sum_over_groups(lsum[u]);
        if (rowv[u]) {
            const float inv = tot > 0.f ? 1.f / tot : 0.f;
            const size_t pidx =
                ((size_t)(pfx ? rq[u] : seq) * Hq + head) * a.max_partitions + part;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if (16 * t >= D) break;  // columns of the layout only
                if (partial) {
                    float* po = a.part_out + pidx * D + 16 * t + 4 * g;
                    *(f32x4*)po = f32x4{oacc[u][t][0] * inv, oacc[u][t][1] * inv,
                                        oacc[u][t][2] * inv, oacc[u][t][3] * inv};
                }
                if (whole) {
                    const size_t o = orow[u] + 16 * t + 4 * g;
                    OUT::store2(a.out, o, oacc[u][t][0] * inv, oacc[u][t][1] * inv);
                    OUT::store2(a.out, o + 2, oacc[u][t][2] * inv, oacc[u][t][3] * inv);
                }
            }
            if (partial && g == 0) {
                a.part_max[pidx] = m[u] * kLn2;  // natural-log units
                a.part_sum[pidx] = tot;
            }
        }
    }
}

template <class KV, class OUT, int D, int NW, int TR, bool SH>
attn_fn pick_prefill_bs(int bs) {
    switch (bs) {
        case 8: return attn_prefill_kernel<KV, OUT, D, 8, NW, TR, SH>;
        case 16: return attn_prefill_kernel<KV, OUT, D, 16, NW, TR, SH>;
        case 32: return attn_prefill_kernel<KV, OUT, D, 32, NW, TR, SH>;
        case 64: return attn_prefill_kernel<KV, OUT, D, 64, NW, TR, SH>;
    }
    return nullptr;
}

template <class KV, class OUT, int NW, int TR, bool SH>
attn_fn pick_prefill_d(int d, int bs) {
    if (d == 128) return pick_prefill_bs<KV, OUT, 128, NW, TR, SH>(bs);
    if constexpr (NW == 4) {
        if (d == 256) return pick_prefill_bs<KV, OUT, 256, NW, TR, SH>(bs);
    }
    if (d == 96) return pick_prefill_bs<KV, OUT, 96, NW, TR, SH>(bs);
    if (d == 80) return pick_prefill_bs<KV, OUT, 80, NW, TR, SH>(bs);
    // head_dim 64: 8 rows per wave-load, at most 4 waves for a 32-token chunk
    if constexpr (NW <= 4) {
        if (d == 64) return pick_prefill_bs<KV, OUT, 64, NW, TR, SH>(bs);
    }
    return nullptr;
}

template <class KV, int NW, int TR, bool SH>
attn_fn pick_prefill_out(pa_dtype out, pa_dtype kv, int d, int bs) {
    if (out == PA_F32) return pick_prefill_d<KV, OutF32, NW, TR, SH>(d, bs);
    if (out != kv) return nullptr;
    if (kv == PA_F16) return pick_prefill_d<KV, OutF16, NW, TR, SH>(d, bs);
    return pick_prefill_d<KV, OutBF16, NW, TR, SH>(d, bs);
}

}  // namespace pa
