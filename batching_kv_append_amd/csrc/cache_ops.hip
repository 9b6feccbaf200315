// Append (new K/V rows -> paged pool slots) and gather (paged pool ->
// contiguous per-sequence cache) kernels.
//
// Append is the block write of a paged cache: the new token's K/V go to the
// slot of position context_len + i inside the physical block that the block
// table names for that position (clvsit.github.io AWS SageMaker page, section
// "PagedAttention 批处理"; klklkl10086.github.io kv_cache post, section "Batch
// Decode", which models the same write with torch.cat on a contiguous cache).
// Both kernels are pure 16-byte copies: one wave per token row, each lane
// moving 16 B of one kv head's row, so a wave writes 4 heads x 256 B
// (head_dim 128) per instruction.
#include <hip/hip_runtime.h>

#include "kvc_launch.h"

namespace kvc {

namespace {

constexpr int ROWS_PER_WG = 4;  // one wave per row

__global__ __launch_bounds__(256) void append_kernel(
    const uint4* __restrict__ k_new, const uint4* __restrict__ v_new, uint4* __restrict__ k_cache,
    uint4* __restrict__ v_cache, int64_t num_blocks, const int32_t* __restrict__ table,
    int32_t max_blocks, const int32_t* __restrict__ cu, const int32_t* __restrict__ ctx,
    int32_t num_seqs, int32_t total_q, int32_t hkv, int32_t head_dim, int32_t block_size,
    int32_t* hdr) {
    const int64_t t = (int64_t)blockIdx.x * ROWS_PER_WG + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (t >= total_q) return;
    const int f = append_row(k_new, v_new, k_cache, v_cache, num_blocks, table, max_blocks, cu, ctx,
                             num_seqs, t, hkv, head_dim, block_size, lane);
    if (f && hdr && lane == 0) set_flag(hdr, f);
}

__global__ __launch_bounds__(256) void gather_kernel(
    const uint4* __restrict__ k_cache, const uint4* __restrict__ v_cache, int64_t num_blocks,
    const int32_t* __restrict__ table, int32_t max_blocks, const int32_t* __restrict__ seq_lens,
    const int64_t* __restrict__ cu, int64_t total, uint4* __restrict__ k_out,
    uint4* __restrict__ v_out, int32_t num_seqs, int32_t hkv, int32_t head_dim,
    int32_t block_size) {
    const int64_t t = (int64_t)blockIdx.x * ROWS_PER_WG + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (t >= total) return;
    const int s = find_seq(cu, num_seqs, t, lane);
    const int64_t p = t - cu[s];
    if (p < 0 || p >= seq_lens[s]) return;
    const int64_t lb = p / block_size;
    if (lb >= max_blocks) return;
    const int64_t blk = table[(int64_t)s * max_blocks + lb];
    if (blk < 0 || blk >= num_blocks) return;
    const int slot = (int)(p % block_size);
    const int cpr = head_dim >> 3;
    const int nchunk = hkv * cpr;
    for (int c = lane; c < nchunk; c += 64) {
        const int g = c / cpr, e = c - g * cpr;
        const int64_t src = ((blk * hkv + g) * block_size + slot) * cpr + e;
        const int64_t dst = (t * hkv + g) * cpr + e;
        k_out[dst] = k_cache[src];
        v_out[dst] = v_cache[src];
    }
}

// Block copy for copy-on-write: workgroup (i, pool) copies block src[i] of
// that pool to block dst[i] (all kv heads and slots), 16 bytes per thread
// per step.  A pair with an id outside [0, num_blocks) is skipped.
__global__ __launch_bounds__(256) void copy_blocks_kernel(
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, int64_t num_blocks,
    const int32_t* __restrict__ src, const int32_t* __restrict__ dst, int64_t block_chunks) {
    const int64_t s = src[blockIdx.x], d = dst[blockIdx.x];
    if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks) return;
    uint4* pool = blockIdx.y == 0 ? k_cache : v_cache;
    const uint4* from = pool + s * block_chunks;
    uint4* to = pool + d * block_chunks;
    for (int64_t c = threadIdx.x; c < block_chunks; c += 256) to[c] = from[c];
}

}  // namespace

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, int64_t num_blocks,
                              const int32_t* src, const int32_t* dst, int32_t n, int32_t hkv,
                              int32_t head_dim, int32_t block_size, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int64_t block_chunks = (int64_t)hkv * block_size * (head_dim / 8);
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)n, 2), dim3(256), 0, stream,
                       (uint4*)k_cache, (uint4*)v_cache, num_blocks, src, dst, block_chunks);
    return hipGetLastError();
}

hipError_t launch_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                         int64_t num_blocks, const int32_t* table, int32_t max_blocks,
                         const int32_t* cu, const int32_t* ctx, int32_t num_seqs,
                         int32_t total_q, int32_t hkv, int32_t head_dim, int32_t block_size,
                         int32_t* hdr, hipStream_t stream) {
    if (total_q <= 0 || num_seqs <= 0) return hipSuccess;
    const unsigned grid = (unsigned)((total_q + ROWS_PER_WG - 1) / ROWS_PER_WG);
    hipLaunchKernelGGL(append_kernel, dim3(grid), dim3(64 * ROWS_PER_WG), 0, stream,
                       (const uint4*)k_new, (const uint4*)v_new, (uint4*)k_cache,
                       (uint4*)v_cache, num_blocks, table, max_blocks, cu, ctx, num_seqs,
                       total_q, hkv, head_dim, block_size, hdr);
    return hipGetLastError();
}

hipError_t launch_gather(const void* k_cache, const void* v_cache, int64_t num_blocks,
                         const int32_t* table, int32_t max_blocks, const int32_t* seq_lens,
                         const int64_t* cu_seq_lens, int64_t total_tokens, void* k_out,
                         void* v_out, int32_t num_seqs, int32_t hkv, int32_t head_dim,
                         int32_t block_size, hipStream_t stream) {
    if (total_tokens <= 0 || num_seqs <= 0) return hipSuccess;
    const int64_t grid = (total_tokens + ROWS_PER_WG - 1) / ROWS_PER_WG;
    hipLaunchKernelGGL(gather_kernel, dim3((unsigned)grid), dim3(64 * ROWS_PER_WG), 0, stream,
                       (const uint4*)k_cache, (const uint4*)v_cache, num_blocks, table,
                       max_blocks, seq_lens, cu_seq_lens, total_tokens, (uint4*)k_out,
                       (uint4*)v_out, num_seqs, hkv, head_dim, block_size);
    return hipGetLastError();
}

}  // namespace kvc
