// Device-side helpers shared by the gfx950 kernels: bf16 packing, lane
// exchanges and the workspace layout.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

// ---------------------------------------------------------------------------
// Workspace layout (caller-owned scratch of kvc_paged_attention_varlen).
// ---------------------------------------------------------------------------
enum HeaderSlot : int {
    HDR_N_DEC = 0,       // decode work items (sequence, partition)
    HDR_N_PRE = 1,       // prefill work items (sequence, position tile)
    HDR_UNUSED = 2,
    HDR_N_MERGE = 3,     // decode sequences split into >1 partition
    HDR_FLAGS = 4,       // error flags (kvc_workspace_flags)
    HDR_WORDS = 64
};
enum Flag : int {
    FLAG_TABLE_SHORT = 1,
    FLAG_BAD_BLOCK = 2,
    FLAG_CAPACITY = 4,
    FLAG_CU_SEQLENS = 8
};

// Decode partition length in tokens: at most what one wave walks.  Fixed
// (never chosen per batch), so a sequence's partial sums depend only on its
// own logical positions and the output does not change with batch
// composition.  1024 rather than 256: fewer, longer waves write fewer split-K
// partials and pay their start-up (table slice, Q operand, first loads) and
// their combine less often (head_dim 128: GQA batch 237 -> 226 us, MQA
// 141 -> 130 us, mixed step 0.81 -> 0.77 ms; head_dim 16 MQA batch with the
// merge 47 -> 46 us).
constexpr int DECODE_PART = 1024;

// Prefill: each wave owns one query head and QW consecutive positions; a
// workgroup of NW waves (4, or 8 on calls without decode rows) covers HPW
// heads x (NW/HPW) position blocks.
constexpr int PREFILL_QW = 32;
constexpr int PREFILL_TK = 64;  // keys per LDS tile

// Position blocks of a prefill work item.  A sequence's q new rows form
// nb = ceil(q / QW) blocks of QW positions; an item takes npb of them (one
// per group of HPW waves), and the sequence's T = ceil(nb / npb) items deal
// them out in snake order: slot k of item t holds block k T + t for even k
// and k T + T - 1 - t for odd k.  Under the causal mask a block's key count
// grows with its index, so item 0 of a 2048-row chunk takes blocks 0 and 63
// rather than 0 and 1, and every item walks about the same number of key
// tiles with both of its wave groups busy for about the same share of them.
// A block index >= nb is an empty slot.
__host__ __device__ inline int prefill_block(int tile, int slot, int per_slot) {
    return slot * per_slot + ((slot & 1) ? per_slot - 1 - tile : tile);
}
// One past the last position that item `tile` of a sequence with q new rows
// covers (its causal key range ends that many keys past the cached ones).
__host__ __device__ inline int prefill_item_end(int tile, int q, int npb) {
    const int nb = (q + PREFILL_QW - 1) / PREFILL_QW;
    const int T = (nb + npb - 1) / npb;
    int end = 0;
    for (int k = 0; k < npb; ++k) {
        const int b = prefill_block(tile, k, T);
        if (b < nb) {
            const int e = (b + 1) * PREFILL_QW < q ? (b + 1) * PREFILL_QW : q;
            end = e > end ? e : end;
        }
    }
    return end;
}

// A prefill work item as the planner hands it to the prefill kernel: the
// sequence, the item's index among its T items, and the sequence's first row,
// new-row count and cached length, so a workgroup reads everything it needs
// before its table lookups in one memory round trip.
struct PreItem {
    int32_t s, tile, row0, qlen;
    int32_t ctx, pad0, pad1, pad2;
};

struct WsLayout {
    size_t hdr, dec_items, pre_items, pre_sorted, merge_list, ml, acc, total;
    int64_t cap_dec, cap_pre;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Prefill heads per workgroup for a group ratio G (G <= 4 divides 4, or G % 4 == 0).
inline int prefill_hpw(int G) { return G >= 4 ? 4 : G; }
inline int prefill_span(int G, int nw = 4) { return PREFILL_QW * (nw / prefill_hpw(G)); }

// Decode partitions per work item: the decode cuts a sequence into
// ceil(L / (4 * DECODE_PART)) equal items, gives each of a workgroup's four
// waves a quarter of one item and combines them in LDS, so split-K partials
// exist per item.
constexpr int DECODE_GROUP = 4;  // partitions per decode workgroup (its four waves)

// Split of a decode sequence of L keys (cached + the new one): `items` work
// items of equal length, each cut into DECODE_GROUP wave shares of
// `per_wave` keys (a multiple of 32, at most DECODE_PART), so wave w of item
// i covers keys [(i G + w) per_wave, min(L, (i G + w + 1) per_wave)) and
// waves starting at or past L have none.  It depends on L alone, so a
// sequence's partial sums never depend on the rest of the batch; the planner
// and the decode kernel both take it from here.
struct DecodeSplit {
    int items, per_wave;
};
__host__ __device__ inline DecodeSplit decode_split(int L) {
    const int items = (L + DECODE_GROUP * DECODE_PART - 1) / (DECODE_GROUP * DECODE_PART);
    const int share = (L + DECODE_GROUP * items - 1) / (DECODE_GROUP * items);
    return {items, (share + 31) / 32 * 32};
}

// Launch id -> decode unit: the (work item x kv head) pair and the head
// chunk.  The hardware deals launch ids to the 8 XCDs round-robin, each XCD
// with its own L2; with HC > 1 head chunks the chunks of one pair get ids 8
// apart, so they run on one XCD at about the same time and all but the
// first find the pair's K/V rows in its L2.  decode_grid is the launch size
// for `pairs` pairs (rounded up to 8 pairs when HC > 1); ids whose pair is
// at or past `pairs` have no unit.
struct DecodeUnit {
    int64_t pair;
    int hc;
};
__host__ __device__ inline DecodeUnit decode_unit(int64_t lid, int HC) {
    if (HC == 1) return {lid, 0};
    return {(lid >> 3) / HC * 8 + (lid & 7), (int)((lid >> 3) % HC)};
}
__host__ __device__ inline int64_t decode_grid(int64_t pairs, int HC) {
    return HC == 1 ? pairs : (pairs + 7) / 8 * 8 * HC;
}

inline WsLayout ws_layout(int32_t num_seqs, int32_t total_q, int32_t max_context_len,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim) {
    WsLayout w{};
    const int G = num_q_heads / num_kv_heads;
    const int64_t parts = ((int64_t)max_context_len + DECODE_PART) / DECODE_PART;  // of L = ctx + 1
    w.cap_dec = (int64_t)num_seqs * ((parts + DECODE_GROUP - 1) / DECODE_GROUP);
    w.cap_pre = (int64_t)total_q / prefill_span(G) + num_seqs;  // 4-wave span: the most items
    size_t off = 0;
    w.hdr = off;        off = align_up(off + HDR_WORDS * 4, 256);
    w.dec_items = off;  off = align_up(off + (size_t)w.cap_dec * 8, 256);
    w.pre_items = off;  off = align_up(off + (size_t)w.cap_pre * 8, 256);
    w.pre_sorted = off; off = align_up(off + (size_t)w.cap_pre * sizeof(PreItem), 256);
    w.merge_list = off; off = align_up(off + (size_t)num_seqs * 16, 256);
    w.ml = off;         off = align_up(off + (size_t)w.cap_dec * num_q_heads * 2 * 4, 256);
    w.acc = off;        off = align_up(off + (size_t)w.cap_dec * num_q_heads * head_dim * 4, 256);
    w.total = off;
    return w;
}

#ifdef __HIPCC__
// ---------------------------------------------------------------------------
// fp32 -> bf16.  Storage is raw uint16.  Narrowing uses the compiler's __bf16
// conversion, which is round-to-nearest-even and lowers to v_cvt_pk_bf16_f32
// on gfx950.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t v;
    v[0] = (__bf16)a;
    v[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, v);
}

// acc + lo + hi of a packed bf16 pair (v_dot2_f32_bf16 with (1, 1)): the
// softmax denominators sum the same bf16-rounded weights that the P.V matrix
// products multiply.
__device__ __forceinline__ float sum_bf16x2(uint32_t w, float acc) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), one, acc, false);
}

__device__ __forceinline__ void set_flag(int32_t* hdr, int flag) {
    atomicOr(hdr + HDR_FLAGS, flag);
}

// Index of the sequence that owns row t: the largest s with cu[s] <= t,
// found by the whole wave (every lane passes the same t).  Each round the 64
// lanes probe 64 evenly spaced entries of the bracket [lo, hi] and a ballot
// keeps the sub-bracket between the last probe <= t and the next one, so
// S sequences take about log64(S) dependent loads (2 up to 4096) instead of
// log2(S).  cu is non-decreasing; on any input the result stays in
// [0, num_seqs - 1] and every round shrinks the bracket.
template <typename T>
__device__ __forceinline__ int find_seq(const T* cu, int num_seqs, int64_t t, int lane) {
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {
        const int64_t span = hi - lo;
        const int idx = lo + (int)(((int64_t)(lane + 1) * span + 63) / 64);  // lo < idx <= hi
        const uint64_t le = __ballot((int64_t)cu[idx] <= t);
        if (le == 0) {
            hi = __shfl(idx, 0, 64) - 1;  // below the first probe
        } else {
            const int k = 63 - __builtin_clzll(le);  // last probe <= t
            const int next = __shfl(idx, k < 63 ? k + 1 : 63, 64);
            lo = __shfl(idx, k, 64);
            hi = k < 63 ? next - 1 : hi;
        }
    }
    return lo;
}
// Copy the K and V rows of new token t (kv heads x head_dim bf16, 16-byte
// chunks spread over the 64 lanes of the calling wave) into the pool slot of
// its position context_lens[s] + (t - cu[s]).  A position outside the table
// or a block id outside [0, num_blocks) is skipped: the return value is
// FLAG_TABLE_SHORT / FLAG_BAD_BLOCK (0 when the row was written).
__device__ __forceinline__ int append_row(const uint4* __restrict__ k_new,
                                          const uint4* __restrict__ v_new, uint4* __restrict__ k_cache,
                                          uint4* __restrict__ v_cache, int64_t num_blocks,
                                          const int32_t* __restrict__ table, int32_t max_blocks,
                                          const int32_t* __restrict__ cu, const int32_t* __restrict__ ctx,
                                          int32_t num_seqs, int64_t t, int32_t hkv, int32_t head_dim,
                                          int32_t block_size, int lane) {
    const int s = find_seq(cu, num_seqs, t, lane);
    const int64_t p = (int64_t)ctx[s] + (t - cu[s]);
    const int64_t lb = p / block_size;
    if (p < 0 || lb >= max_blocks) return FLAG_TABLE_SHORT;
    const int64_t blk = table[(int64_t)s * max_blocks + lb];
    if (blk < 0 || blk >= num_blocks) return FLAG_BAD_BLOCK;
    const int slot = (int)(p % block_size);
    const int cpr = head_dim >> 3;  // 16-byte chunks per head row
    const int nchunk = hkv * cpr;
    for (int c = lane; c < nchunk; c += 64) {
        const int g = c / cpr, e = c - g * cpr;
        const int64_t dst = ((blk * hkv + g) * block_size + slot) * cpr + e;
        const int64_t src = (t * hkv + g) * cpr + e;
        k_cache[dst] = k_new[src];
        v_cache[dst] = v_new[src];
    }
    return 0;
}
#endif  // __HIPCC__

}  // namespace kvc
