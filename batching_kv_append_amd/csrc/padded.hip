// kvc_padded_decode_attention: one decode step of a left-padded batch, the
// static batching that ragged continuous batching replaces.
//
// In a left-padded batch every sequence occupies the same number of
// positions, n_max: its real tokens are right-aligned and the positions
// before them hold padding, hidden from attention by a padding mask
// (news.myit.tw continuous-batching article, section "Continuous batching":
// prompts of one batch are padded on the left to a common length, and a
// prompt joining a batch of decoding sequences costs (n - 1)(B - 1) pad
// tokens).  The cache is the contiguous per-sequence reservation of the
// klklkl10086.github.io kv_cache post (section "连续内存分配"): sequence b owns
// positions b * n_max .. b * n_max + n_max - 1, stored in the pool's page
// format (pages of block_size positions, [page][kv head][slot][dim]), page j
// of sequence b being page b * (n_max / block_size) + j.
//
// The step appends the new token at position n_max - 1 of every sequence and
// attends over all n_max positions with the padding masked: the decode kernel
// streams every position (the cost of padding), excludes keys below
// pad_lens[b] by select and zeroes their V rows, so whatever the padding
// holds has weight exactly 0.  The result of row b equals attention over its
// own n_max - pad_lens[b] tokens.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>

#include "kvc.h"
#include "kvc_launch.h"
#include "kvc_status.h"

namespace {

// Identity page table, one row per sequence, and the row offsets / cached
// lengths of a batch of one new token per sequence.
__global__ __launch_bounds__(256) void padded_setup_kernel(int32_t* table, int32_t* cu, int32_t* ctx,
                                                           int32_t batch, int32_t pages, int32_t n_max) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < (int64_t)batch * pages) table[i] = (int32_t)i;
    if (i <= batch) cu[i] = (int32_t)i;
    if (i < batch) ctx[i] = n_max - 1;
}

struct PaddedLayout {
    size_t main, table, cu, ctx, total;
};

PaddedLayout padded_layout(int32_t batch, int32_t n_max, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size) {
    PaddedLayout p{};
    p.main = kvc_workspace_size(batch, batch, 1, n_max - 1, num_q_heads, num_kv_heads, head_dim,
                                block_size);
    const int64_t pages = (int64_t)n_max / block_size;
    size_t off = kvc::align_up(p.main, 256);
    p.table = off;
    off = kvc::align_up(off + (size_t)batch * pages * 4, 256);
    p.cu = off;
    off = kvc::align_up(off + (size_t)(batch + 1) * 4, 256);
    p.ctx = off;
    off = kvc::align_up(off + (size_t)batch * 4, 256);
    p.total = off;
    return p;
}

// Sizes the step accepts (n_max up to 2^24 keeps every later size check of
// the step from failing after the set-up launch).
bool padded_shape_ok(int32_t batch, int32_t n_max, int32_t head_dim, int32_t block_size) {
    return batch >= 0 && n_max >= 1 && n_max <= (1 << 24) && head_dim == 128 &&
           (block_size == 4 || block_size == 16) && n_max % block_size == 0 &&
           (int64_t)batch * (n_max / block_size) <= INT32_MAX;
}

}  // namespace

extern "C" size_t kvc_padded_workspace_size(int32_t batch, int32_t n_max, int32_t num_q_heads,
                                            int32_t num_kv_heads, int32_t head_dim,
                                            int32_t block_size) {
    if (!padded_shape_ok(batch, n_max, head_dim, block_size)) return 0;
    const PaddedLayout p =
        padded_layout(batch, n_max, num_q_heads, num_kv_heads, head_dim, block_size);
    return p.main == 0 ? 0 : p.total;
}

extern "C" int kvc_padded_decode_attention(void* out, const void* q, const void* k_new,
                                           const void* v_new, void* k_cache, void* v_cache,
                                           const int32_t* pad_lens, int32_t batch, int32_t n_max,
                                           int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size, float scale,
                                           void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "kvc_padded_decode_attention";
    char msg[256];
    if (batch < 0 || n_max < 1)
        return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_padded_decode_attention: batch < 0 or n_max < 1");
    if (head_dim != 128 || (block_size != 4 && block_size != 16)) {
        std::snprintf(msg, sizeof msg, "%s: head_dim %d / block_size %d unsupported (128; 4 or 16)",
                      fn, head_dim, block_size);
        return kvc_fail(KVC_ERR_UNSUPPORTED, msg);
    }
    if (!padded_shape_ok(batch, n_max, head_dim, block_size))
        return kvc_fail(KVC_ERR_INVALID_ARG,
                        "kvc_padded_decode_attention: n_max must be a multiple of block_size, at "
                        "most 2^24, with batch * n_max / block_size < 2^31");
    if (batch == 0) return KVC_OK;
    // every check that can fail runs before the set-up launch below
    auto al16 = [](const void* p) { return ((uintptr_t)p & 15u) == 0; };
    if (!pad_lens || !out || !q || !k_cache || !v_cache)
        return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_padded_decode_attention: NULL pointer");
    if ((k_new == nullptr) != (v_new == nullptr))
        return kvc_fail(KVC_ERR_INVALID_ARG,
                        "kvc_padded_decode_attention: k_new and v_new must both be set or both NULL");
    if (!al16(out) || !al16(q) || !al16(k_cache) || !al16(v_cache) ||
        (k_new && (!al16(k_new) || !al16(v_new))))
        return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_padded_decode_attention: tensors must be 16-byte aligned");
    if (!std::isfinite(scale))
        return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_padded_decode_attention: scale must be finite");
    const PaddedLayout lay =
        padded_layout(batch, n_max, num_q_heads, num_kv_heads, head_dim, block_size);
    if (lay.main == 0)  // head counts the step does not support: its own checks report why
        return kvc::paged_attention(fn, out, q, k_new, v_new, k_cache, v_cache, 1, nullptr, 1,
                                    nullptr, nullptr, batch, batch, 1, n_max - 1, num_q_heads,
                                    num_kv_heads, head_dim, block_size, scale, workspace,
                                    workspace_bytes, stream, false, pad_lens);
    if (!workspace || workspace_bytes < lay.total || ((uintptr_t)workspace & 255u) != 0) {
        std::snprintf(msg, sizeof msg,
                      "%s: workspace of %zu bytes (256-byte aligned) needed, %zu given", fn,
                      lay.total, workspace ? workspace_bytes : (size_t)0);
        return kvc_fail(KVC_ERR_WORKSPACE, msg);
    }
    char* ws = (char*)workspace;
    int32_t* table = (int32_t*)(ws + lay.table);
    int32_t* cu = (int32_t*)(ws + lay.cu);
    int32_t* ctx = (int32_t*)(ws + lay.ctx);
    const int32_t pages = n_max / block_size;
    const int64_t n = (int64_t)batch * pages + 1;
    const int64_t grid = (n + 255) / 256;
    if (grid > INT32_MAX) return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_padded_decode_attention: batch too large");
    hipLaunchKernelGGL(padded_setup_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream,
                       table, cu, ctx, batch, pages, n_max);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        std::snprintf(msg, sizeof msg, "%s: %s", fn, hipGetErrorString(e));
        return kvc_fail(KVC_ERR_HIP, msg);
    }
    return kvc::paged_attention(fn, out, q, k_new, v_new, k_cache, v_cache,
                                (int64_t)batch * pages, table, pages, cu, ctx, batch, batch, 1,
                                n_max - 1, num_q_heads, num_kv_heads, head_dim, block_size, scale,
                                workspace, lay.main, stream, false, pad_lens);
}
