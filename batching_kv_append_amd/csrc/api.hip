// C-ABI entry points of libkvc.so: argument validation, workspace layout and
// the launch sequence of one ragged paged-attention step.
//
// Every check that can fail happens before the first launch, so a call that
// returns an error has enqueued nothing.  Values inside device arrays are not
// read here (that would need a device-to-host copy and a sync on every call);
// the kernels guard every table lookup instead, and KVC_DEBUG=1 adds a
// synchronous host-side check of the lengths and the table.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <atomic>
#include <memory>
#include <mutex>
#include <utility>
#include <algorithm>
#include <vector>

#include "kvc.h"
#include "kvc_launch.h"
#include "kvc_status.h"

namespace kvc {

int device_cu_count() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64 && cache[dev] > 0) return cache[dev];
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    if (dev < 64) cache[dev] = n;
    return n;
}

}  // namespace kvc

namespace {

using kvc::WsLayout;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool debug_mode() {
    const char* e = std::getenv("KVC_DEBUG");
    return e && e[0] && e[0] != '0';
}

int check_shape(int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                const char* fn) {
    char msg[256];
    if (num_kv_heads <= 0 || num_q_heads <= 0) {
        std::snprintf(msg, sizeof msg, "%s: head counts must be positive", fn);
        return kvc_fail(KVC_ERR_INVALID_ARG, msg);
    }
    if (num_q_heads % num_kv_heads != 0) {
        std::snprintf(msg, sizeof msg, "%s: num_q_heads %% num_kv_heads != 0", fn);
        return kvc_fail(KVC_ERR_INVALID_ARG, msg);
    }
    const int G = num_q_heads / num_kv_heads;
    if (!(G == 1 || G == 2 || G % 4 == 0)) {
        std::snprintf(msg, sizeof msg, "%s: head ratio %d unsupported (1, 2 or a multiple of 4)", fn, G);
        return kvc_fail(KVC_ERR_UNSUPPORTED, msg);
    }
    if (head_dim != 16 && head_dim != 64 && head_dim != 128 && head_dim != 256) {
        std::snprintf(msg, sizeof msg, "%s: head_dim %d unsupported (16, 64, 128 or 256)", fn,
                      head_dim);
        return kvc_fail(KVC_ERR_UNSUPPORTED, msg);
    }
    if (block_size != 4 && block_size != 16) {
        std::snprintf(msg, sizeof msg, "%s: block_size %d unsupported (4 or 16)", fn, block_size);
        return kvc_fail(KVC_ERR_UNSUPPORTED, msg);
    }
    return KVC_OK;
}

int check_kv_shape(int32_t num_kv_heads, int32_t head_dim, int32_t block_size, const char* fn) {
    return check_shape(num_kv_heads, num_kv_heads, head_dim, block_size, fn);
}

int hip_fail(hipError_t e, const char* fn) {
    char msg[256];
    std::snprintf(msg, sizeof msg, "%s: %s", fn, hipGetErrorString(e));
    return kvc_fail(KVC_ERR_HIP, msg);
}

// "<fn>: <detail>" in a thread-local buffer (kvc_fail copies it at once).
const char* fmt_msg(const char* fn, const char* detail) {
    thread_local char buf[256];
    std::snprintf(buf, sizeof buf, "%s: %s", fn, detail);
    return buf;
}

// KVC_DEBUG=1: copy lengths and table back and check them on the host.
int debug_check(const int32_t* cu_d, const int32_t* ctx_d, const int32_t* table_d, int32_t num_seqs,
                int32_t total_q, int32_t max_q_len, int32_t max_context_len, int32_t max_blocks,
                int64_t num_blocks, int32_t block_size, bool after_append_only, hipStream_t st) {
    std::vector<int32_t> cu(num_seqs + 1), ctx(num_seqs), tab((size_t)num_seqs * max_blocks);
    hipError_t e = hipMemcpyAsync(cu.data(), cu_d, cu.size() * 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipMemcpyAsync(ctx.data(), ctx_d, ctx.size() * 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipMemcpyAsync(tab.data(), table_d, tab.size() * 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "KVC_DEBUG check");
    if (cu[0] != 0 || cu[num_seqs] != total_q)
        return kvc_fail(KVC_ERR_INVALID_ARG, "KVC_DEBUG: cu_seqlens_q must start at 0 and end at total_q");
    for (int s = 0; s < num_seqs; ++s) {
        const int64_t q = (int64_t)cu[s + 1] - cu[s];
        if (q < 0) return kvc_fail(KVC_ERR_INVALID_ARG, "KVC_DEBUG: cu_seqlens_q decreases");
        if (ctx[s] < 0) return kvc_fail(KVC_ERR_INVALID_ARG, "KVC_DEBUG: negative context length");
        if (!after_append_only && (q > max_q_len || ctx[s] > max_context_len))
            return kvc_fail(KVC_ERR_INVALID_ARG, "KVC_DEBUG: a length exceeds max_q_len / max_context_len");
        const int64_t L = ctx[s] + q;
        const int64_t nb = (L + block_size - 1) / block_size;
        if (nb > max_blocks) return kvc_fail(KVC_ERR_INVALID_ARG, "KVC_DEBUG: table row too short");
        for (int64_t b = 0; b < nb; ++b) {
            const int32_t id = tab[(size_t)s * max_blocks + b];
            if (id < 0 || id >= num_blocks)
                return kvc_fail(KVC_ERR_INVALID_ARG, "KVC_DEBUG: block id out of range");
        }
    }
    return KVC_OK;
}

// Optional per-kernel timing: a start and an end HIP event around each kernel
// of kvc_paged_attention_varlen, recorded on the stream that kernel runs on
// (kvc_profile_begin/end).  g_prof_on is read without the lock; a call takes
// g_prof_mu only while timing is on, so untimed calls from several threads
// never wait for each other here.
struct Profiler {
    bool on = false;
    int32_t max_calls = 0, calls = 0;
    std::vector<hipEvent_t> ev;  // 2 * KVC_PROF_PHASES per call: (start, end) per phase
    std::vector<uint8_t> used;   // per call and phase: 1 both events recorded, 2 a record failed
};
Profiler g_prof;
std::mutex g_prof_mu;
std::atomic<bool> g_prof_on{false};

// Caller holds g_prof_mu.
void prof_mark(int phase, bool end, hipStream_t st) {
    if (!g_prof.on || g_prof.calls >= g_prof.max_calls) return;
    const size_t base = (size_t)g_prof.calls * KVC_PROF_PHASES + phase;
    if (hipEventRecord(g_prof.ev[base * 2 + (end ? 1 : 0)], st) != hipSuccess)
        g_prof.used[base] = 2;  // a phase with a failed record is left out of the sums
    else if (end && g_prof.used[base] == 0)
        g_prof.used[base] = 1;
}

// Side streams for the prefill kernel, so the matrix-bound prefill overlaps
// the memory-bound decode.  Each caller stream gets its own side stream and
// fork/join event pair (per device, created on first use, default priority,
// non-blocking), so steps issued on different caller streams are not chained
// through one shared side stream.  A call forks to the side stream with an
// event after the append and joins it back with another before returning,
// so the caller's stream still sees one ordered step.  The per-entry mutex
// keeps the event pair of two threads using the same caller stream apart.
// Past kMaxSides caller streams on a device, new callers share an existing
// entry (chosen by the stream handle); that only orders their prefills.
struct SideStream {
    std::mutex mu;
    hipStream_t stream = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
constexpr size_t kMaxSides = 64;
struct DeviceSides {
    std::mutex mu;
    std::vector<std::pair<hipStream_t, std::unique_ptr<SideStream>>> by_caller;
};
DeviceSides g_sides[64];

SideStream* side_stream(hipStream_t caller) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    DeviceSides& ds = g_sides[dev];
    std::lock_guard<std::mutex> lk(ds.mu);
    for (auto& e : ds.by_caller)
        if (e.first == caller) return e.second.get();
    if (ds.by_caller.size() >= kMaxSides)
        return ds.by_caller[((uintptr_t)caller >> 4) % ds.by_caller.size()].second.get();
    auto ss = std::make_unique<SideStream>();
    if (hipStreamCreateWithFlags(&ss->stream, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&ss->fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ss->join, hipEventDisableTiming) != hipSuccess) {
        if (ss->fork) (void)hipEventDestroy(ss->fork);
        (void)hipStreamDestroy(ss->stream);
        return nullptr;
    }
    ds.by_caller.emplace_back(caller, std::move(ss));
    return ds.by_caller.back().second.get();
}

bool overlap_enabled() {
    const char* e = std::getenv("KVC_SERIAL");  // 1: run every kernel on the caller's stream
    return !(e && e[0] && e[0] != '0');
}

}  // namespace

extern "C" int kvc_profile_begin(int32_t max_calls) {
    if (max_calls < 1 || max_calls > 100000)
        return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_profile_begin: max_calls out of range");
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_on.store(false, std::memory_order_release);
    for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
    g_prof = Profiler{};
    g_prof.ev.resize((size_t)max_calls * KVC_PROF_PHASES * 2);
    g_prof.used.assign((size_t)max_calls * KVC_PROF_PHASES, 0);
    for (auto& e : g_prof.ev) {
        hipError_t r = hipEventCreate(&e);
        if (r != hipSuccess) return hip_fail(r, "kvc_profile_begin");
    }
    g_prof.max_calls = max_calls;
    g_prof.on = true;
    g_prof_on.store(true, std::memory_order_release);
    return KVC_OK;
}

extern "C" int kvc_profile_end(double* ms_sum, int32_t* calls) {
    if (!ms_sum || !calls) return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_profile_end: NULL pointer");
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_on.store(false, std::memory_order_release);
    for (int p = 0; p < KVC_PROF_PHASES; ++p) ms_sum[p] = 0.0;
    *calls = 0;
    for (int32_t c = 0; c < g_prof.calls; ++c) {
        for (int p = 0; p < KVC_PROF_PHASES; ++p) {
            const size_t base = (size_t)c * KVC_PROF_PHASES + p;
            if (g_prof.used[base] != 1) continue;
            hipError_t r = hipEventSynchronize(g_prof.ev[base * 2 + 1]);
            float ms = 0.f;
            if (r == hipSuccess) r = hipEventElapsedTime(&ms, g_prof.ev[base * 2], g_prof.ev[base * 2 + 1]);
            if (r != hipSuccess) return hip_fail(r, "kvc_profile_end");
            ms_sum[p] += ms;
        }
    }
    *calls = g_prof.calls;
    for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
    g_prof = Profiler{};
    return KVC_OK;
}

extern "C" int kvc_append_kv(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                             int64_t num_blocks, const int32_t* block_table,
                             int32_t max_blocks_per_seq, const int32_t* cu_seqlens_q,
                             const int32_t* context_lens, int32_t num_seqs, int32_t total_q,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             void* stream) {
    const char* fn = "kvc_append_kv";
    if (num_seqs < 0 || total_q < 0) return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_append_kv: negative size");
    if (int rc = check_kv_shape(num_kv_heads, head_dim, block_size, fn)) return rc;
    if (num_seqs == 0 || total_q == 0) return KVC_OK;
    if (!k_new || !v_new || !k_cache || !v_cache || !block_table || !cu_seqlens_q || !context_lens)
        return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_append_kv: NULL pointer");
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
        return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_append_kv: K/V pointers must be 16-byte aligned");
    if (num_blocks < 1 || max_blocks_per_seq < 1)
        return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_append_kv: num_blocks and max_blocks_per_seq must be >= 1");
    hipStream_t st = (hipStream_t)stream;
    if (debug_mode()) {
        if (int rc = debug_check(cu_seqlens_q, context_lens, block_table, num_seqs, total_q, 0, 0,
                                 max_blocks_per_seq, num_blocks, block_size, true, st))
            return rc;
    }
    hipError_t e = kvc::launch_append(k_new, v_new, k_cache, v_cache, num_blocks, block_table,
                                      max_blocks_per_seq, cu_seqlens_q, context_lens, num_seqs,
                                      total_q, num_kv_heads, head_dim, block_size, nullptr, st);
    return e == hipSuccess ? KVC_OK : hip_fail(e, fn);
}

extern "C" int kvc_gather_kv(const void* k_cache, const void* v_cache, int64_t num_blocks,
                             const int32_t* block_table, int32_t max_blocks_per_seq,
                             const int32_t* seq_lens, const int64_t* cu_seq_lens,
                             int64_t total_tokens, void* k_out, void* v_out, int32_t num_seqs,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             void* stream) {
    const char* fn = "kvc_gather_kv";
    if (num_seqs < 0 || total_tokens < 0) return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_gather_kv: negative size");
    if (int rc = check_kv_shape(num_kv_heads, head_dim, block_size, fn)) return rc;
    if (num_seqs == 0 || total_tokens == 0) return KVC_OK;
    if (!k_cache || !v_cache || !block_table || !seq_lens || !cu_seq_lens || !k_out || !v_out)
        return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_gather_kv: NULL pointer");
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_out) || !aligned16(v_out))
        return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_gather_kv: K/V pointers must be 16-byte aligned");
    if (num_blocks < 1 || max_blocks_per_seq < 1)
        return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_gather_kv: num_blocks and max_blocks_per_seq must be >= 1");
    if (total_tokens > ((int64_t)1 << 40))
        return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_gather_kv: total_tokens too large");
    hipError_t e = kvc::launch_gather(k_cache, v_cache, num_blocks, block_table, max_blocks_per_seq,
                                      seq_lens, cu_seq_lens, total_tokens, k_out, v_out, num_seqs,
                                      num_kv_heads, head_dim, block_size, (hipStream_t)stream);
    return e == hipSuccess ? KVC_OK : hip_fail(e, fn);
}

extern "C" int kvc_copy_blocks(void* k_cache, void* v_cache, int64_t num_blocks,
                               const int32_t* src_ids, const int32_t* dst_ids, int32_t n,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               void* stream) {
    const char* fn = "kvc_copy_blocks";
    if (n < 0) return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_copy_blocks: negative count");
    if (int rc = check_kv_shape(num_kv_heads, head_dim, block_size, fn)) return rc;
    if (n == 0) return KVC_OK;
    if (!k_cache || !v_cache || !src_ids || !dst_ids)
        return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_copy_blocks: NULL pointer");
    if (!aligned16(k_cache) || !aligned16(v_cache))
        return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_copy_blocks: K/V pointers must be 16-byte aligned");
    if (num_blocks < 1) return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_copy_blocks: num_blocks must be >= 1");
    hipStream_t st = (hipStream_t)stream;
    if (debug_mode()) {  // ids in range, destinations distinct and not sources
        std::vector<int32_t> src(n), dst(n);
        hipError_t e = hipMemcpyAsync(src.data(), src_ids, (size_t)n * 4, hipMemcpyDeviceToHost, st);
        if (e == hipSuccess) e = hipMemcpyAsync(dst.data(), dst_ids, (size_t)n * 4, hipMemcpyDeviceToHost, st);
        if (e == hipSuccess) e = hipStreamSynchronize(st);
        if (e != hipSuccess) return hip_fail(e, "KVC_DEBUG check");
        std::vector<int32_t> seen(dst);
        std::sort(seen.begin(), seen.end());
        for (int32_t i = 0; i < n; ++i) {
            if (src[i] < 0 || src[i] >= num_blocks || dst[i] < 0 || dst[i] >= num_blocks)
                return kvc_fail(KVC_ERR_INVALID_ARG, "KVC_DEBUG: block id out of range");
            if (i > 0 && seen[i] == seen[i - 1])
                return kvc_fail(KVC_ERR_INVALID_ARG, "KVC_DEBUG: repeated destination block");
        }
        for (int32_t i = 0; i < n; ++i)
            if (std::binary_search(seen.begin(), seen.end(), src[i]))
                return kvc_fail(KVC_ERR_INVALID_ARG, "KVC_DEBUG: a destination is also a source");
    }
    hipError_t e = kvc::launch_copy_blocks(k_cache, v_cache, num_blocks, src_ids, dst_ids, n,
                                           num_kv_heads, head_dim, block_size, st);
    return e == hipSuccess ? KVC_OK : hip_fail(e, fn);
}

namespace {

// Enqueue one planned step: plan + append, then the prefill (on the caller
// stream's side stream when the step also has decode rows) beside the decode
// and merge on the caller's stream.  Once the side stream has been forked,
// the join is recorded on every path, launch failures included, and the
// caller's stream waits on it after the decode and merge launches; if the
// join cannot be recorded or waited on, the host waits for the side stream
// instead, so nothing queued there can outlive the call unordered.
int run_step(const kvc::StepArgs& a, bool has_decode, bool overlap, const char* fn) {
    const hipStream_t st = a.stream;
    const int32_t max_q_len = a.max_q_len;
    const bool profiling = g_prof_on.load(std::memory_order_acquire);
    std::unique_lock<std::mutex> prof_lk(g_prof_mu, std::defer_lock);
    if (profiling) prof_lk.lock();
    auto mark = [&](int phase, bool end, hipStream_t s) {
        if (profiling) prof_mark(phase, end, s);
    };
    // planning and append share one launch (counted under "plan")
    // The prefill kernel (rows of chunks with >= 2 new tokens) runs on the side
    // stream when there is one, concurrently with decode and merge.
    SideStream* ss =
        (max_q_len >= 2 && has_decode && overlap) ? side_stream(st) : nullptr;
    std::unique_lock<std::mutex> side_lk;
    if (ss) side_lk = std::unique_lock<std::mutex>(ss->mu);
    // With a side stream the planning kernel's launch records the fork event
    // itself (on its completion): a separate event record between it and the
    // decode left about 8 us with nothing running on the caller's stream
    // (mixed step 0.760 -> 0.752 ms).
    mark(KVC_PROF_PLAN, false, st);
    hipError_t e = kvc::launch_prep(a, a.k_new != nullptr, ss ? ss->fork : nullptr);
    mark(KVC_PROF_PLAN, true, st);
    bool forked = false;
    if (e == hipSuccess && max_q_len >= 2) {
        kvc::StepArgs ap = a;
        if (ss) {
            e = hipStreamWaitEvent(ss->stream, ss->fork, 0);
            forked = e == hipSuccess;
            ap.stream = ss->stream;
        }
        mark(KVC_PROF_PREFILL, false, ap.stream);
        if (e == hipSuccess) e = kvc::launch_prefill(ap);
        mark(KVC_PROF_PREFILL, true, ap.stream);
    }
    // the join is recorded even after a failed prefill launch
    hipError_t ej = forked ? hipEventRecord(ss->join, ss->stream) : hipSuccess;
    if (has_decode) {
        mark(KVC_PROF_DECODE, false, st);
        if (e == hipSuccess) e = kvc::launch_decode(a);
        mark(KVC_PROF_DECODE, true, st);
        mark(KVC_PROF_MERGE, false, st);
        if (e == hipSuccess) e = kvc::launch_merge(a);
        mark(KVC_PROF_MERGE, true, st);
    }
    if (forked) {
        // the caller's stream never runs ahead of work queued on the side
        // stream: it waits on this call's join, or the host waits for the
        // side stream when the join could not be recorded or waited on
        if (ej == hipSuccess) ej = hipStreamWaitEvent(st, ss->join, 0);
        if (ej != hipSuccess) {
            (void)hipStreamSynchronize(ss->stream);
            if (e == hipSuccess) e = ej;
        }
    }
    if (profiling && g_prof.on && g_prof.calls < g_prof.max_calls) ++g_prof.calls;
    return e == hipSuccess ? KVC_OK : hip_fail(e, fn);
}

}  // namespace

extern "C" size_t kvc_workspace_size(int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                                     int32_t max_context_len, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size) {
    if (num_seqs < 0 || total_q < 0 || max_q_len < 0 || max_context_len < 0) return 0;
    if (check_shape(num_q_heads, num_kv_heads, head_dim, block_size, "kvc_workspace_size") != KVC_OK)
        return 0;
    return kvc::ws_layout(num_seqs, total_q, max_context_len, num_q_heads, num_kv_heads, head_dim).total;
}

namespace kvc {

int paged_attention(const char* fn, void* out, const void* q, const void* k_new,
                    const void* v_new, void* k_cache, void* v_cache, int64_t num_blocks,
                    const int32_t* block_table, int32_t max_blocks_per_seq,
                    const int32_t* cu_seqlens_q, const int32_t* context_lens, int32_t num_seqs,
                    int32_t total_q, int32_t max_q_len, int32_t max_context_len,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, float scale, void* workspace, size_t workspace_bytes,
                    void* stream, bool overlap, const int32_t* key_start) {
    if (num_seqs < 0 || total_q < 0 || max_q_len < 0 || max_context_len < 0)
        return kvc_fail(KVC_ERR_INVALID_ARG, fmt_msg(fn, "negative size"));
    if (int rc = check_shape(num_q_heads, num_kv_heads, head_dim, block_size, fn)) return rc;
    if (!std::isfinite(scale))
        return kvc_fail(KVC_ERR_INVALID_ARG, fmt_msg(fn, "scale must be finite"));
    if ((k_new == nullptr) != (v_new == nullptr))
        return kvc_fail(KVC_ERR_INVALID_ARG, fmt_msg(fn, "k_new and v_new must both be set or both NULL"));
    if (key_start && (head_dim != 128 || max_q_len > 1))
        return kvc_fail(KVC_ERR_UNSUPPORTED, fmt_msg(fn, "a key mask needs decode rows of head_dim 128"));
    if (num_seqs == 0 || total_q == 0) return KVC_OK;
    if (!out || !q || !k_cache || !v_cache || !block_table || !cu_seqlens_q || !context_lens)
        return kvc_fail(KVC_ERR_INVALID_ARG, fmt_msg(fn, "NULL pointer"));
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
        (k_new && (!aligned16(k_new) || !aligned16(v_new))))
        return kvc_fail(KVC_ERR_INVALID_ARG, fmt_msg(fn, "tensors must be 16-byte aligned"));
    if (num_blocks < 1 || max_blocks_per_seq < 1)
        return kvc_fail(KVC_ERR_INVALID_ARG, fmt_msg(fn, "num_blocks and max_blocks_per_seq must be >= 1"));
    if (max_q_len > total_q)
        return kvc_fail(KVC_ERR_INVALID_ARG, fmt_msg(fn, "max_q_len > total_q"));
    if ((int64_t)max_context_len + max_q_len > INT32_MAX / 2)
        return kvc_fail(KVC_ERR_INVALID_ARG, fmt_msg(fn, "lengths too large"));
    const WsLayout lay = kvc::ws_layout(num_seqs, total_q, max_context_len, num_q_heads,
                                        num_kv_heads, head_dim);
    if (lay.cap_dec > INT32_MAX / 64 || lay.cap_pre > INT32_MAX / 64)
        return kvc_fail(KVC_ERR_INVALID_ARG, fmt_msg(fn, "step too large"));
    if (!workspace || workspace_bytes < lay.total) {
        char msg[256];
        std::snprintf(msg, sizeof msg, "%s: workspace of %zu bytes needed, %zu given", fn,
                      lay.total, workspace ? workspace_bytes : (size_t)0);
        return kvc_fail(KVC_ERR_WORKSPACE, msg);
    }
    if (((uintptr_t)workspace & 255u) != 0)
        return kvc_fail(KVC_ERR_WORKSPACE, fmt_msg(fn, "workspace must be 256-byte aligned"));
    hipStream_t st = (hipStream_t)stream;
    if (debug_mode()) {
        if (int rc = debug_check(cu_seqlens_q, context_lens, block_table, num_seqs, total_q,
                                 max_q_len, max_context_len, max_blocks_per_seq, num_blocks,
                                 block_size, false, st))
            return rc;
    }

    kvc::StepArgs a;
    a.out = out;
    a.q = q;
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.num_blocks = num_blocks;
    a.block_table = block_table;
    a.max_blocks = max_blocks_per_seq;
    a.cu_seqlens_q = cu_seqlens_q;
    a.context_lens = context_lens;
    a.num_seqs = num_seqs;
    a.total_q = total_q;
    a.max_q_len = max_q_len;
    a.max_context_len = max_context_len;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.block_size = block_size;
    a.scale = scale;
    a.key_start = key_start;
    a.ws = (char*)workspace;
    a.lay = lay;
    a.stream = st;

    // Rows of one new token (decode) can be ruled out from the host sizes
    // alone: with d such sequences and every other one holding at most
    // max_q_len rows, total_q <= d + (num_seqs - d) * max_q_len. When that
    // leaves d = 0 the step is chunks only, and it skips the decode and merge
    // launches and the side-stream fork. (A call whose cu_seqlens_q break the
    // host sizes is flagged by the planner either way.)
    const bool has_decode =
        max_q_len < 2 ||
        (int64_t)num_seqs * max_q_len - total_q >= (int64_t)max_q_len - 1;
    // The prefill overlaps the decode only when the decode's workgroups can
    // fill the chip beside it: the grid's upper bound (the host sizes' work
    // items x kv heads x head chunks) at least one per compute unit.  A few
    // decode rows next to a long chunk would otherwise hold compute units
    // that the prefill's single round of workgroups needs, and the workgroups
    // waiting for them finish that much later (a 2048-row chunk at 6144
    // cached keys beside 2 decode rows: 390 us overlapped, 330 us one after
    // the other).
    const int G = num_q_heads / num_kv_heads;
    const int64_t dec_wgs =
        lay.cap_dec * num_kv_heads * (G / kvc::decode_heads_per_wave(G, head_dim, block_size));
    const bool side = overlap && has_decode && dec_wgs >= kvc::device_cu_count();
    // A prefill that has the chip to itself (chunks only, or run before the
    // decode) takes the 8-wave workgroups (one per compute unit, every K/V
    // tile shared by 8 waves, P.V a tile late on half of them); beside a
    // decode the 4-wave ones, which leave the decode more of each unit (and
    // at head_dim 128 at most one of them per unit).
    a.prefill_waves = (!side && head_dim <= 128) ? 8 : 4;
    a.prefill_beside_decode = side;

    return run_step(a, has_decode, side, fn);
}

}  // namespace kvc

extern "C" int kvc_paged_attention_varlen(
    void* out, const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
    int64_t num_blocks, const int32_t* block_table, int32_t max_blocks_per_seq,
    const int32_t* cu_seqlens_q, const int32_t* context_lens, int32_t num_seqs, int32_t total_q,
    int32_t max_q_len, int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, float scale, void* workspace, size_t workspace_bytes,
    void* stream) {
    return kvc::paged_attention("kvc_paged_attention_varlen", out, q, k_new, v_new, k_cache,
                                v_cache, num_blocks, block_table, max_blocks_per_seq,
                                cu_seqlens_q, context_lens, num_seqs, total_q, max_q_len,
                                max_context_len, num_q_heads, num_kv_heads, head_dim, block_size,
                                scale, workspace, workspace_bytes, stream, overlap_enabled());
}

extern "C" int kvc_workspace_flags(const void* workspace, void* stream, int32_t* flags) {
    if (!workspace || !flags) return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_workspace_flags: NULL pointer");
    hipStream_t st = (hipStream_t)stream;
    int32_t v = 0;
    hipError_t e = hipMemcpyAsync(&v, (const char*)workspace + kvc::HDR_FLAGS * 4, 4,
                                  hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "kvc_workspace_flags");
    *flags = v;
    return KVC_OK;
}
