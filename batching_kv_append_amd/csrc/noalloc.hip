// kvc_paged_attention_varlen_noalloc: the ragged paged-attention step for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// The step's scratch (plan header, work lists, split-K partials) lives in a
// file-scope __device__ array of KVC_NOALLOC_SCRATCH_BYTES.  Each GPU the
// library runs on holds its own copy of it from module load until the process
// ends.  In host code the array's name is only a host-side stand-in, so the
// array is never passed by name: on the first call on a device, with that
// device current, its device address is looked up with hipGetSymbolAddress
// and kept per device, and every kernel receives that address.
//
// Nothing in the scratch has to start at zero: the planning kernel writes
// the header (counts, and the flag word it zeroes first) before any other
// kernel of the step reads it, and every other region is written before it
// is read within the step.  All calls on one GPU share its array, so calls
// that overlap in time on one GPU (two streams, or two host threads) race.
// The step runs every kernel on the caller's stream (no side stream is
// created), and the call itself allocates nothing: no hipMalloc, hipFree,
// stream or event creation.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "kvc.h"
#include "kvc_launch.h"
#include "kvc_status.h"

static __device__ __align__(256) unsigned char scratch[KVC_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

struct ScratchAddr {
    std::once_flag once;
    void* ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchAddr g_scratch[kMaxDevices];

// Device address of the current device's scratch array (looked up once per
// device, with that device current).
hipError_t scratch_address(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    ScratchAddr& sa = g_scratch[dev];
    std::call_once(sa.once, [&sa] {
        sa.err = hipGetSymbolAddress(&sa.ptr, HIP_SYMBOL(scratch));
        if (sa.err == hipSuccess && sa.ptr == nullptr) sa.err = hipErrorInvalidSymbol;
    });
    *ptr = sa.ptr;
    return sa.err;
}

}  // namespace

extern "C" int kvc_paged_attention_varlen_noalloc(
    void* out, const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
    int64_t num_blocks, const int32_t* block_table, int32_t max_blocks_per_seq,
    const int32_t* cu_seqlens_q, const int32_t* context_lens, int32_t num_seqs, int32_t total_q,
    int32_t max_q_len, int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, float scale, void* stream) {
    const char* fn = "kvc_paged_attention_varlen_noalloc";
    // The size the step needs, from the same host bounds the workspace
    // version uses (0 for arguments kvc_paged_attention_varlen rejects; those
    // are reported by its own checks below).
    const size_t need = kvc_workspace_size(num_seqs, total_q, max_q_len, max_context_len,
                                           num_q_heads, num_kv_heads, head_dim, block_size);
    if (need > (size_t)KVC_NOALLOC_SCRATCH_BYTES) {
        char msg[256];
        std::snprintf(msg, sizeof msg,
                      "%s: the step needs %zu bytes of scratch, the static scratch holds %zu "
                      "(use kvc_paged_attention_varlen with a caller workspace)",
                      fn, need, (size_t)KVC_NOALLOC_SCRATCH_BYTES);
        return kvc_fail(KVC_ERR_WORKSPACE, msg);
    }
    void* ws = nullptr;
    if (num_seqs > 0 && total_q > 0) {
        const hipError_t e = scratch_address(&ws);
        if (e != hipSuccess) {
            char msg[256];
            std::snprintf(msg, sizeof msg, "%s: scratch address: %s", fn, hipGetErrorString(e));
            return kvc_fail(KVC_ERR_HIP, msg);
        }
    }
    return kvc::paged_attention(fn, out, q, k_new, v_new, k_cache, v_cache, num_blocks,
                                block_table, max_blocks_per_seq, cu_seqlens_q, context_lens,
                                num_seqs, total_q, max_q_len, max_context_len, num_q_heads,
                                num_kv_heads, head_dim, block_size, scale, ws,
                                (size_t)KVC_NOALLOC_SCRATCH_BYTES, stream, false);
}
