// Host-side launchers of the gfx950 kernels (one translation unit each).
// Arguments are validated by the C-ABI layer before any of these run.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvc_device.h"

namespace kvc {

struct StepArgs {
    void* out;
    const void* q;
    const void* k_new;
    const void* v_new;
    void* k_cache;
    void* v_cache;
    int64_t num_blocks;
    const int32_t* block_table;
    int32_t max_blocks;
    const int32_t* cu_seqlens_q;
    const int32_t* context_lens;
    int32_t num_seqs, total_q, max_q_len, max_context_len;
    int32_t num_q_heads, num_kv_heads, head_dim, block_size;
    float scale;
    const int32_t* key_start = nullptr;  // left-padded batch: first unpadded key per sequence
    int32_t prefill_waves = 4;  // prefill workgroup size: 8 when no decode runs beside it (head_dim <= 128)
    bool prefill_beside_decode = false;  // the prefill runs on the side stream next to the decode
    char* ws;  // workspace base
    WsLayout lay;
    hipStream_t stream;
};

// Append new K/V rows into the pools (hdr may be null: no flag reporting).
hipError_t launch_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                         int64_t num_blocks, const int32_t* table, int32_t max_blocks,
                         const int32_t* cu, const int32_t* ctx, int32_t num_seqs,
                         int32_t total_q, int32_t hkv, int32_t head_dim, int32_t block_size,
                         int32_t* hdr, hipStream_t stream);

hipError_t launch_gather(const void* k_cache, const void* v_cache, int64_t num_blocks,
                         const int32_t* table, int32_t max_blocks, const int32_t* seq_lens,
                         const int64_t* cu_seq_lens, int64_t total_tokens, void* k_out,
                         void* v_out, int32_t num_seqs, int32_t hkv, int32_t head_dim,
                         int32_t block_size, hipStream_t stream);

// One launch: work lists for the decode and prefill kernels (zeroes the
// header flags) and, with_append, the append of k_new / v_new.
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, int64_t num_blocks,
                              const int32_t* src, const int32_t* dst, int32_t n, int32_t hkv,
                              int32_t head_dim, int32_t block_size, hipStream_t stream);
// done (optional): an event that the planning kernel's own completion records
hipError_t launch_prep(const StepArgs& a, bool with_append, hipEvent_t done = nullptr);
// Split-K decode partials (+ direct output for one-partition sequences).
hipError_t launch_decode(const StepArgs& a);
// Log-sum-exp merge of the partials of multi-partition decode sequences.
hipError_t launch_merge(const StepArgs& a);
// MFMA prefill over chunks of >= 2 rows.
hipError_t launch_prefill(const StepArgs& a);

// Compute units of the current device (cached per device).
int device_cu_count();
// Query heads per decode wave for a group ratio G (the kv head's heads are cut
// into G / that many head chunks).
int decode_heads_per_wave(int G, int head_dim, int block_size);

// Argument checks and launches of one step, shared by the entry points that
// run it (kvc_paged_attention_varlen and its variants): `fn` names the entry
// point in error messages; `overlap` lets a step with chunks and decode rows
// run its prefill on the caller stream's side stream; `key_start` (device,
// one per sequence, or null) masks each sequence's keys below it (a
// left-padded batch; decode rows of head_dim 128 only).  Returns a
// kvc_status.
int paged_attention(const char* fn, void* out, const void* q, const void* k_new,
                    const void* v_new, void* k_cache, void* v_cache, int64_t num_blocks,
                    const int32_t* block_table, int32_t max_blocks_per_seq,
                    const int32_t* cu_seqlens_q, const int32_t* context_lens, int32_t num_seqs,
                    int32_t total_q, int32_t max_q_len, int32_t max_context_len,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, float scale, void* workspace, size_t workspace_bytes,
                    void* stream, bool overlap, const int32_t* key_start = nullptr);

}  // namespace kvc
