// pa_reshape_and_cache: scatter each new token's K/V rows into its cache
// slot ("vLLM PagedAttention深度解析与工程实践" §二, per-step KV append;
// lqnn.cn/news/170268 §2.2, write into the current block's free slot).
//
// One work item moves one 16-byte piece (8 elements) of one token's K row
// and the matching piece of its V row; consecutive work items cover
// consecutive pieces of the same token, so both the reads of key/value and
// the writes into the slot's [num_kv_heads, head_dim] row are coalesced.
#include "pa_device.h"
#include "pa_host.h"

namespace pa {
namespace {

__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const uint16_t* __restrict__ key, const uint16_t* __restrict__ value,
    uint16_t* __restrict__ key_cache, uint16_t* __restrict__ value_cache,
    const int64_t* __restrict__ slot_mapping, int num_tokens, int64_t key_stride,
    int64_t value_stride, int pieces_per_token, int64_t num_slots) {
    const int64_t total = (int64_t)num_tokens * pieces_per_token;
    const int64_t row_elems = (int64_t)pieces_per_token * 8;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t tok = idx / pieces_per_token;
        const int64_t piece = idx - tok * pieces_per_token;
        // the source pieces do not depend on the slot: their loads are issued
        // together with the slot's, not after it. Loads and stores are
        // non-temporal: the rows pass through once, and a prefill's scatter
        // would otherwise push the cached prompt, which the attention after
        // it re-reads, out of L2.
        const u32x4 k = __builtin_nontemporal_load((const u32x4*)(key + tok * key_stride + piece * 8));
        const u32x4 v =
            __builtin_nontemporal_load((const u32x4*)(value + tok * value_stride + piece * 8));
        const int64_t slot = slot_mapping[tok];
        if (slot < 0 || slot >= num_slots) continue;  // padding, or outside the cache
        // slot = block * block_size + row, and rows are dense inside a block,
        // so the destination row is simply `slot` rows into the cache
        const int64_t dst = slot * row_elems + piece * 8;
        __builtin_nontemporal_store(k, (u32x4*)(key_cache + dst));
        __builtin_nontemporal_store(v, (u32x4*)(value_cache + dst));
    }
}

// ---------------------------------------------------------------------------
// pa_copy_blocks: copy-on-write block copy ("优化大模型推理：PagedAttention 如何
// 实现 GPU 显存高效管理", 写时复制: shared blocks are copied only when a
// sequence is about to write into them).
//
// Work item = (pair, 16 KiB slice of a block). Each workgroup reads its slice
// of the source K and V blocks (8 independent 16-byte loads per thread) and
// writes them to the destination blocks; the descriptors' ranges end at the
// block's end, so the lanes past it neither read nor write.
// ---------------------------------------------------------------------------

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;  // per cache: 4 K + 4 V loads in flight per thread
constexpr uint32_t kCopySlice = kCopyThreads * kCopyUnroll * 16;

// Also the swap between two pools (pa_swap_blocks): source and destination
// caches are then different allocations, one of them in pinned host memory
// that the device reads or writes across the host link.
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    char* __restrict__ dst_key, char* __restrict__ dst_value, const char* src_key,
    const char* src_value, const int64_t* __restrict__ block_mapping, int slices_per_block,
    uint32_t block_bytes, int64_t src_blocks, int64_t dst_blocks) {
    const int pair = blockIdx.x / slices_per_block;
    const int slice = blockIdx.x - pair * slices_per_block;
    const int64_t src = block_mapping[2 * (int64_t)pair];
    const int64_t dst = block_mapping[2 * (int64_t)pair + 1];
    if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;  // uniform
    const uint32_t begin = (uint32_t)slice * kCopySlice;
    const uint32_t left = block_bytes - begin;
    const uint32_t range = left < kCopySlice ? left : kCopySlice;
    const size_t so = (size_t)src * block_bytes + begin, dof = (size_t)dst * block_bytes + begin;
    const __amdgpu_buffer_rsrc_t ks = make_rsrc(src_key + so, range);
    const __amdgpu_buffer_rsrc_t vs = make_rsrc(src_value + so, range);
    const __amdgpu_buffer_rsrc_t kd = make_rsrc(dst_key + dof, range);
    const __amdgpu_buffer_rsrc_t vd = make_rsrc(dst_value + dof, range);
    u32x4 k[kCopyUnroll], v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const uint32_t off = (uint32_t)(u * kCopyThreads + threadIdx.x) * 16;
        k[u] = buffer_load16(ks, off);
        v[u] = buffer_load16(vs, off);
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const uint32_t off = (uint32_t)(u * kCopyThreads + threadIdx.x) * 16;
        __builtin_amdgcn_raw_buffer_store_b128(k[u], kd, (int)off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(v[u], vd, (int)off, 0, 0);
    }
}

}  // namespace
}  // namespace pa

extern "C" pa_status pa_reshape_and_cache(const void* key, const void* value, void* key_cache,
                                          void* value_cache, const int64_t* slot_mapping,
                                          int num_tokens, int64_t key_token_stride,
                                          int64_t value_token_stride, int num_kv_heads,
                                          int head_dim, int num_blocks, int block_size,
                                          pa_dtype dtype, void* stream) {
    using namespace pa;
    clear_error();
    PA_REQUIRE(num_tokens >= 0, PA_ERR_SHAPE, "num_tokens %d < 0", num_tokens);
    PA_REQUIRE(num_kv_heads > 0 && head_dim > 0 && num_blocks > 0 && block_size > 0,
               PA_ERR_SHAPE, "num_kv_heads, head_dim, num_blocks, block_size must be > 0");
    PA_REQUIRE(dtype == PA_F16 || dtype == PA_BF16, PA_ERR_DTYPE,
               "cache dtype must be PA_F16 or PA_BF16");
    const int64_t row = (int64_t)num_kv_heads * head_dim;
    PA_REQUIRE(row % 8 == 0, PA_ERR_UNSUPPORTED,
               "num_kv_heads * head_dim must be a multiple of 8");
    PA_REQUIRE(key_token_stride >= row && value_token_stride >= row, PA_ERR_SHAPE,
               "token strides must be >= num_kv_heads * head_dim");
    PA_REQUIRE(key_token_stride % 8 == 0 && value_token_stride % 8 == 0, PA_ERR_ALIGNMENT,
               "token strides must be multiples of 8 elements");
    if (num_tokens == 0) return PA_OK;
    PA_REQUIRE(key && value && key_cache && value_cache && slot_mapping, PA_ERR_NULL,
               "null pointer argument");
    PA_REQUIRE(aligned16(key) && aligned16(value) && aligned16(key_cache) &&
                   aligned16(value_cache),
               PA_ERR_ALIGNMENT, "K/V and cache pointers must be 16-byte aligned");
    const int pieces = (int)(row / 8);
    const int64_t total = (int64_t)num_tokens * pieces;
    int64_t grid = (total + 255) / 256;
    if (grid > 1 << 20) grid = 1 << 20;
    hipLaunchKernelGGL(reshape_and_cache_kernel, dim3((unsigned)grid), dim3(256), 0,
                       (hipStream_t)stream, (const uint16_t*)key, (const uint16_t*)value,
                       (uint16_t*)key_cache, (uint16_t*)value_cache, slot_mapping, num_tokens,
                       key_token_stride, value_token_stride, pieces,
                       (int64_t)num_blocks * block_size);
    return check_launch("pa_reshape_and_cache");
}

extern "C" pa_status pa_copy_blocks(void* key_cache, void* value_cache,
                                    const int64_t* block_mapping, int num_pairs,
                                    int num_kv_heads, int head_dim, int block_size,
                                    int num_blocks, pa_dtype dtype, void* stream) {
    using namespace pa;
    clear_error();
    PA_REQUIRE(num_pairs >= 0, PA_ERR_SHAPE, "num_pairs %d < 0", num_pairs);
    PA_REQUIRE(num_kv_heads > 0 && head_dim > 0 && num_blocks > 0 && block_size > 0,
               PA_ERR_SHAPE, "num_kv_heads, head_dim, num_blocks, block_size must be > 0");
    PA_REQUIRE(dtype == PA_F16 || dtype == PA_BF16, PA_ERR_DTYPE,
               "cache dtype must be PA_F16 or PA_BF16");
    const int64_t block_bytes = (int64_t)block_size * num_kv_heads * head_dim * 2;
    PA_REQUIRE(block_bytes % 16 == 0 && block_bytes < ((int64_t)1 << 31), PA_ERR_UNSUPPORTED,
               "a block must be a multiple of 16 bytes and below 2 GiB");
    if (num_pairs == 0) return PA_OK;
    PA_REQUIRE(key_cache && value_cache && block_mapping, PA_ERR_NULL, "null pointer argument");
    PA_REQUIRE(aligned16(key_cache) && aligned16(value_cache), PA_ERR_ALIGNMENT,
               "caches must be 16-byte aligned");
    const int slices = (int)((block_bytes + kCopySlice - 1) / kCopySlice);
    const int64_t grid = (int64_t)num_pairs * slices;
    PA_REQUIRE(grid < ((int64_t)1 << 31), PA_ERR_SHAPE, "too many pairs");
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)grid), dim3(kCopyThreads), 0,
                       (hipStream_t)stream, (char*)key_cache, (char*)value_cache,
                       (const char*)key_cache, (const char*)value_cache, block_mapping, slices,
                       (uint32_t)block_bytes, (int64_t)num_blocks, (int64_t)num_blocks);
    return check_launch("pa_copy_blocks");
}

namespace {

// The address under which the device reaches p: device memory as is, pinned
// host memory through its mapping. Anything else (pageable host memory,
// unknown pointers) is refused before a kernel could fault on it.
bool device_address(const void* p, const void** dev) {
    hipPointerAttribute_t at;
    if (hipPointerGetAttributes(&at, p) != hipSuccess) {
        (void)hipGetLastError();  // clear the sticky error of the failed query
        return false;
    }
    if (at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeManaged) {
        *dev = p;
        return true;
    }
    if (at.type == hipMemoryTypeHost && at.devicePointer) {
        // p may point inside the allocation: keep its offset from the host base
        const char* hb = (const char*)at.hostPointer;
        const char* db = (const char*)at.devicePointer;
        *dev = hb ? db + ((const char*)p - hb) : db;
        return true;
    }
    return false;
}

}  // namespace

extern "C" pa_status pa_swap_blocks(void* dst_key_cache, void* dst_value_cache,
                                    int dst_num_blocks, const void* src_key_cache,
                                    const void* src_value_cache, int src_num_blocks,
                                    const int64_t* block_mapping, int num_pairs,
                                    int num_kv_heads, int head_dim, int block_size,
                                    pa_dtype dtype, void* stream) {
    using namespace pa;
    clear_error();
    PA_REQUIRE(num_pairs >= 0, PA_ERR_SHAPE, "num_pairs %d < 0", num_pairs);
    PA_REQUIRE(num_kv_heads > 0 && head_dim > 0 && block_size > 0 && src_num_blocks > 0 &&
                   dst_num_blocks > 0,
               PA_ERR_SHAPE, "sizes and block counts must be > 0");
    PA_REQUIRE(dtype == PA_F16 || dtype == PA_BF16, PA_ERR_DTYPE,
               "cache dtype must be PA_F16 or PA_BF16");
    const int64_t block_bytes = (int64_t)block_size * num_kv_heads * head_dim * 2;
    PA_REQUIRE(block_bytes % 16 == 0 && block_bytes < ((int64_t)1 << 31), PA_ERR_UNSUPPORTED,
               "a block must be a multiple of 16 bytes and below 2 GiB");
    if (num_pairs == 0) return PA_OK;
    PA_REQUIRE(dst_key_cache && dst_value_cache && src_key_cache && src_value_cache &&
                   block_mapping,
               PA_ERR_NULL, "null pointer argument");
    PA_REQUIRE(aligned16(dst_key_cache) && aligned16(dst_value_cache) &&
                   aligned16(src_key_cache) && aligned16(src_value_cache),
               PA_ERR_ALIGNMENT, "caches must be 16-byte aligned");
    const void *dk, *dv, *sk, *sv, *bm;
    PA_REQUIRE(device_address(dst_key_cache, &dk) && device_address(dst_value_cache, &dv) &&
                   device_address(src_key_cache, &sk) && device_address(src_value_cache, &sv) &&
                   device_address(block_mapping, &bm),
               PA_ERR_UNSUPPORTED,
               "every pool and the mapping must be device memory or pinned host memory "
               "mapped for the device");
    const int slices = (int)((block_bytes + kCopySlice - 1) / kCopySlice);
    const int64_t grid = (int64_t)num_pairs * slices;
    PA_REQUIRE(grid < ((int64_t)1 << 31), PA_ERR_SHAPE, "too many pairs");
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)grid), dim3(kCopyThreads), 0,
                       (hipStream_t)stream, (char*)dk, (char*)dv, (const char*)sk,
                       (const char*)sv, (const int64_t*)bm, slices, (uint32_t)block_bytes,
                       (int64_t)src_num_blocks, (int64_t)dst_num_blocks);
    return check_launch("pa_swap_blocks");
}

