// Work planning and the split-K decode path.
//
// Decode rows (one new token) dominate a continuous-batching step: each one
// streams its whole cached K/V once, so the step is bound by memory traffic
// (klklkl10086.github.io kv_cache post, section on the decode bottleneck: the
// decode stage is limited by memory access; clvsit.github.io AWS SageMaker
// page: every step moves the parameters and the cache into the compute
// units).  The kernels therefore aim at HBM bandwidth:
//   * a sequence's context is cut into pieces of at most DECODE_PART tokens
//     (split-K), a cut that depends only on its own length, so even a
//     short batch of long contexts yields thousands of independent pieces of
//     work;
//     the partial softmax states are combined by an exact log-sum-exp merge
//     (an exact regrouping of the row-wise softmax of the "Attention" section
//     of the continuous-batching article);
//   * K and V are streamed with non-temporal loads whose instructions each
//     cover whole 128-byte lines;
//   * the GW query heads that share a kv head (GQA, e2hang/Notes "MQA与GQA")
//     are served from one read of K/V;
//   * every head size (16, 64, 128, 256) runs decode_mfma_kernel: a sequence
//     is cut into ceil(L / 4096) work items of equal length, and a workgroup
//     takes one item of one (sequence, kv head, head chunk), a quarter of it
//     per wave (at most one 1024-token partition), scores and P.V on bf16
//     MFMA; the four states are combined in LDS, so split-K partials (and the
//     merge) exist per item.
// The planning kernel lists the work items on the device, longest pieces
// first, so the host needs no copy of the lengths, and the hardware
// dispatcher hands the next workgroup to whichever compute unit frees up
// first.
#include <hip/hip_runtime.h>

#include <hip/hip_ext.h>

#include "kvc_launch.h"

namespace kvc {

namespace {

// ---------------------------------------------------------------------------
// Plan: classify sequences and write the work lists.
// ---------------------------------------------------------------------------
constexpr int PLAN_THREADS = 1024;

constexpr int COST_BUCKETS = 1024;  // prefill cost histogram (key tiles, clamped)
constexpr int DEC_BUCKETS = DECODE_PART / 32;  // decode order: 32-token steps per wave

struct PrepParams {
    // planning
    const int32_t* cu;
    const int32_t* ctx;
    int32_t num_seqs, total_q, max_q_len, max_context_len, span;
    int64_t cap_dec, cap_pre;
    int32_t* hdr;
    int2* dec_items;
    int2* pre_items;
    PreItem* pre_sorted;
    int4* merge_list;  // (sequence, first item, items, output row)
    // append (k_new == nullptr: nothing to append)
    const uint4* k_new;
    const uint4* v_new;
    uint4* k_cache;
    uint4* v_cache;
    int64_t num_blocks;
    const int32_t* table;
    int32_t max_blocks, hkv, head_dim, block_size;
};

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_scan(int x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}

// Workgroup 0 plans; workgroups 1.. append the new rows (one wave per row).
// Only the planner writes the flag word (it zeroes it first).  The append
// skips a row whose block is outside the table or the pool; every appended
// position is read by the attention kernels (a row always sees its own key),
// which report such blocks (TABLE_SHORT / BAD_BLOCK) when they read them.
__global__ __launch_bounds__(PLAN_THREADS) void prep_kernel(PrepParams P) {
    if (blockIdx.x > 0) {
        const int64_t t = (int64_t)(blockIdx.x - 1) * (PLAN_THREADS / 64) + (threadIdx.x >> 6);
        if (P.k_new == nullptr || t >= P.total_q) return;
        append_row(P.k_new, P.v_new, P.k_cache, P.v_cache, P.num_blocks, P.table, P.max_blocks,
                   P.cu, P.ctx, P.num_seqs, t, P.hkv, P.head_dim, P.block_size, threadIdx.x & 63);
        return;
    }
    constexpr int WAVES = PLAN_THREADS / 64;
    const int32_t* __restrict__ cu = P.cu;
    const int32_t* __restrict__ ctx = P.ctx;
    const int32_t num_seqs = P.num_seqs, total_q = P.total_q, max_q_len = P.max_q_len;
    const int32_t max_context_len = P.max_context_len, span = P.span;
    const int64_t cap_dec = P.cap_dec, cap_pre = P.cap_pre;
    int32_t* hdr = P.hdr;
    int2* dec_items = P.dec_items;
    int2* pre_items = P.pre_items;
    PreItem* pre_sorted = P.pre_sorted;
    int4* merge_list = P.merge_list;
    __shared__ int wsum[3][WAVES];
    __shared__ int hist[COST_BUCKETS];
    __shared__ int carry[3];
    __shared__ int flags;
    __shared__ int cu_ends[2];  // cu[0], cu[num_seqs], as the loop reads them
    __shared__ int dec_off[DEC_BUCKETS];  // decode items per bucket, then offsets
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    if (tid == 0) {
        carry[0] = carry[1] = carry[2] = 0;
        flags = 0;
        hdr[HDR_FLAGS] = 0;
    }
    for (int b = tid; b < COST_BUCKETS; b += PLAN_THREADS) hist[b] = 0;
    if (tid < DEC_BUCKETS) dec_off[tid] = 0;
    __syncthreads();
    // The lengths of sequence s, checked against the host bounds.  A
    // sequence whose rows are not inside [0, total_q) or whose lengths break
    // the host bounds is skipped (and flagged): no later kernel touches its
    // rows, so garbage lengths can never move an access out of bounds.
    // Returns q (0 when skipped); sets c and the first row.
    auto seq_lengths = [&](int s, int& c, int& row0, bool flag) -> int {
        const int r0 = cu[s], r1 = cu[s + 1];
        c = ctx[s];
        row0 = r0;
        if (r0 < 0 || r1 < r0 || r1 > total_q || c < 0) {
            if (flag) atomicOr(&flags, FLAG_CU_SEQLENS);
            return 0;
        }
        if (c > max_context_len || r1 - r0 > max_q_len) {
            if (flag) atomicOr(&flags, FLAG_CAPACITY);
            return 0;
        }
        return r1 - r0;
    };
    // Decode items of a sequence with c cached tokens, and the bucket that
    // orders them: the matrix decode gives each wave a quarter of an item,
    // and items with longer quarters run first, so short ones fill the end
    // of the launch.
    auto decode_items = [&](int c, int& bucket) -> int {
        const DecodeSplit sp = decode_split(c + 1);
        bucket = min(sp.per_wave / 32, DEC_BUCKETS) - 1;  // 32-token steps per wave
        return sp.items;
    };
    // Pass 1: count decode items per bucket; list the prefill items.
    for (int base = 0; base < num_seqs; base += PLAN_THREADS) {
        const int s = base + tid;
        int nd = 0, np = 0;
        if (s < num_seqs) {
            int c, row0;
            const int q = seq_lengths(s, c, row0, true);
            if (s == 0) cu_ends[0] = row0;
            if (s == num_seqs - 1) cu_ends[1] = cu[s + 1];
            if (q == 1) {
                int b;
                nd = decode_items(c, b);
                atomicAdd(&dec_off[b], nd);
            } else if (q >= 2) {
                np = (q + span - 1) / span;
            }
        }
        // exclusive offsets: scan inside the wave, then the wave totals
        const int id = wave_scan(nd, lane), ip = wave_scan(np, lane);
        if (lane == 63) {
            wsum[0][wave] = id;
            wsum[1][wave] = ip;
        }
        __syncthreads();
        int op = carry[1] + ip - np;
        for (int w = 0; w < wave; ++w) op += wsum[1][w];
        if (s < num_seqs) {
            // heavier (later) position tiles first
            for (int j = 0; j < np; ++j) {
                if (op + j < cap_pre) pre_items[op + j] = make_int2(s, np - 1 - j);
                else atomicOr(&flags, FLAG_CAPACITY);
            }
        }
        __syncthreads();  // every thread has read carry and wsum
        if (tid < 2) {
            int t = 0;
            for (int w = 0; w < WAVES; ++w) t += wsum[tid][w];
            carry[tid] += t;
        }
        __syncthreads();
    }
    // Bucket offsets, longest quarters first.
    if (tid == 0) {
        int o = 0;
        for (int b = DEC_BUCKETS - 1; b >= 0; --b) {
            const int n = dec_off[b];
            dec_off[b] = o;
            o += n;
        }
    }
    __syncthreads();
    // Pass 2: place each decode sequence's items (consecutive, in order, at
    // a position taken from its bucket) and write its merge descriptor.  The
    // order inside a bucket only changes which workgroup starts first: an
    // item's result does not depend on its position.
    for (int base = 0; base < num_seqs; base += PLAN_THREADS) {
        const int s = base + tid;
        int nd = 0, nm = 0, b = 0, row0 = 0;
        if (s < num_seqs) {
            int c;
            if (seq_lengths(s, c, row0, false) == 1) {
                nd = decode_items(c, b);
                nm = nd > 1;
            }
        }
        const int im = wave_scan(nm, lane);
        if (lane == 63) wsum[2][wave] = im;
        __syncthreads();
        int om = carry[2] + im - nm;
        for (int w = 0; w < wave; ++w) om += wsum[2][w];
        if (nd > 0) {
            const int pos = atomicAdd(&dec_off[b], nd);
            for (int j = 0; j < nd; ++j) {
                if (pos + j < cap_dec) dec_items[pos + j] = make_int2(s, j);
                else atomicOr(&flags, FLAG_CAPACITY);
            }
            if (nm) merge_list[om] = make_int4(s, pos, nd, row0);
        }
        __syncthreads();  // every thread has read carry and wsum
        if (tid == 0) {
            int t = 0;
            for (int w = 0; w < WAVES; ++w) t += wsum[2][w];
            carry[2] += t;
        }
        __syncthreads();
    }
    // Order the prefill work costliest first (counting sort on the number of
    // 64-key tiles a workgroup walks), so the longest workgroups start first
    // and the short ones fill the tail.
    const int npre = (int)min((int64_t)carry[1], cap_pre);
    auto bucket_of = [&](int2 item) {
        const int q = cu[item.x + 1] - cu[item.x];
        const int64_t keys = (int64_t)ctx[item.x] + prefill_item_end(item.y, q, span / PREFILL_QW);
        const int64_t tiles = (keys + PREFILL_TK - 1) / PREFILL_TK;
        return COST_BUCKETS - 1 - (int)min(tiles, (int64_t)COST_BUCKETS - 1);
    };
    for (int i = tid; i < npre; i += PLAN_THREADS) atomicAdd(&hist[bucket_of(pre_items[i])], 1);
    __syncthreads();
    {  // exclusive scan of the histogram (one bucket per thread)
        static_assert(COST_BUCKETS == PLAN_THREADS, "one bucket per thread");
        const int v = hist[tid];
        const int iv = wave_scan(v, lane);
        if (lane == 63) wsum[0][wave] = iv;
        __syncthreads();
        int o = iv - v;
        for (int w = 0; w < wave; ++w) o += wsum[0][w];
        hist[tid] = o;
    }
    __syncthreads();
    for (int i = tid; i < npre; i += PLAN_THREADS) {
        const int2 item = pre_items[i];
        const int at = atomicAdd(&hist[bucket_of(item)], 1);
        const int row0 = cu[item.x];
        PreItem rec;
        rec.s = item.x;
        rec.tile = item.y;
        rec.row0 = row0;
        rec.qlen = cu[item.x + 1] - row0;
        rec.ctx = ctx[item.x];
        rec.pad0 = rec.pad1 = rec.pad2 = 0;
        pre_sorted[at] = rec;
    }
    if (tid == 0) {
        const int first = num_seqs > 0 ? cu_ends[0] : cu[0];
        const int last = num_seqs > 0 ? cu_ends[1] : cu[0];
        if (first != 0 || last != total_q) flags |= FLAG_CU_SEQLENS;
        hdr[HDR_N_DEC] = (int)min((int64_t)carry[0], cap_dec);
        hdr[HDR_N_PRE] = npre;
        hdr[HDR_N_MERGE] = carry[2];
        if (flags) atomicOr(hdr + HDR_FLAGS, flags);
    }
}

// ---------------------------------------------------------------------------
// Decode partial kernel.
// ---------------------------------------------------------------------------
struct DecodeParams {
    const uint16_t* q;
    uint16_t* out;
    const uint4* k_cache;
    const uint4* v_cache;
    const int32_t* table;
    const int32_t* cu;
    const int32_t* ctx;
    int32_t* hdr;
    const int2* items;
    float* ws_ml;
    float* ws_acc;
    const int32_t* key_start;  // left-padded batch: first key each sequence sees (else null)
    int64_t num_blocks;
    int32_t max_blocks, hq, hkv, G, HC;
    float scale_log2;  // scale * log2(e): scores live in the exp2 domain
};

constexpr float NEG_BIG = -1.0e30f;  // "no key yet": finite, so exp2(NEG_BIG - m) == 0

// ---------------------------------------------------------------------------
// Decode partial kernel on the matrix cores (head_dims 16, 64, 128 and 256).
//
// Both products of a decode step are small matrix products once the query
// heads that share a kv head are stacked as columns (up to 16):
//   S^T[token][head] = K[token][:] . Q^T[:][head]      v_mfma_f32_16x16x32_bf16
//   O^T[dim][head]  += V^T[dim][token] . P^T[token][head]
// K rows are loaded whole and rearranged through a per-wave LDS tile (A x 64 B)
// into the A operand (lane l owns token l%16 of a 16-token block and 8 dims
// of each 32-dim step); the score registers of a lane (head l%16, tokens
// 4g..4g+3 of each block, g = l/16) are already the B operand of the second
// product for a 32-token step, with the key order {4g..4g+3, 16+4g..16+4g+3};
// V is transposed through the same tile in that same order.  The four lanes of a head
// column share one running maximum (two lane exchanges per step), so the
// weights summed by one matrix instruction share one scale.  The VALU work per
// 32-token step is about 80 instructions, far under the bytes' HBM time.
// Head_dim 16 is half of one 32-dim step: its K rows sit in the tile padded
// with 16 zero dims (and the Q^T operand's upper 16 dims are zero), so the
// same 16x16x32 products serve it.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));

// Max and sum of x over the lane pairs (l, l ^ 16) and (l, l ^ 32) with the
// gfx950 row swaps in the VALU, not through the LDS crossbar.
// v_permlane16_swap trades the odd 16-lane rows of its first operand with the
// even rows of its second, v_permlane32_swap the upper half-wave of the first
// with the lower half of the second; swapping x with itself leaves each lane
// with x of one of the pair in the first result and x of the other in the
// second (the same two values, in the same order, on both lanes of a pair).
__device__ __forceinline__ float max_x16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_x32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_x16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_x32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Max and sum over the whole wave, every lane ending with the result: DPP
// row operations inside each 16-lane row (swap neighbours, swap pairs, then
// row_half_mirror and row_mirror, each of which meets a lane of the half that
// does not yet hold its total), then the two row swaps above.  Each step adds
// or compares the same two values on both lanes it pairs, so every lane holds
// the same bits.
__device__ __forceinline__ float dpp_f(float x, int ctrl) {
    switch (ctrl) {  // the control word must be a constant
        case 0xB1: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
        case 0x4E: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
        case 0x141: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true));
        default: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, true));
    }
}
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp_f(x, 0xB1));   // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp_f(x, 0x4E));   // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp_f(x, 0x141));  // row_half_mirror
    x = fmaxf(x, dpp_f(x, 0x140));  // row_mirror
    return max_x32(max_x16(x));
}
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp_f(x, 0xB1);
    x += dpp_f(x, 0x4E);
    x += dpp_f(x, 0x141);
    x += dpp_f(x, 0x140);
    return sum_x32(sum_x16(x));
}

__device__ __forceinline__ f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// NG: 16-column groups of q heads per wave (1, or 2 for 32 heads on one kv
// head, as in MQA): the groups share every K fragment and the V^T tile, so
// the partition's K/V is read once for all of them.
// A workgroup is one work item of one (sequence, kv head, head chunk).  The
// sequence's ceil(L / (GP x DP)) items split it evenly, and wave w
// takes the w-th quarter of its item (a multiple of 32 tokens, at most one
// partition), so a short sequence keeps all four waves busy for a short time
// instead of one wave for a long one.  The last of the item's waves to finish
// combines their (max, sum, accumulator) in LDS, in wave order, into the
// output (a sequence of one item) or into one split-K partial per item.
// The two-group kernel is held to two waves per SIMD (at most 256 VGPRs; it
// fits in 228 without spills): left free it takes about 300 and runs one wave
// per SIMD, too few loads in flight for a memory-bound kernel.  Head_dim 256
// runs one wave per SIMD (about 320 registers with one group, 480 with two,
// its V rows requested only once the K rows are in LDS so the two staging
// sets are never live together); with 4-token blocks it takes one group, and
// 32 heads on one kv head then run as two head chunks whose workgroups share
// an XCD (the second reads K/V from its L2).
// MASKED (the left-padded batch): keys below key_start[s] are padding.  They
// are still read (a padded batch streams every position), their scores are
// excluded by select and their V rows are zeroed, so whatever the padding
// holds has weight exactly 0.
template <int A, int BS, int NG, bool MASKED>
__global__ __launch_bounds__(256, NG == 2 && A <= 128 ? 2 : 1) void decode_mfma_kernel(DecodeParams P) {
    static_assert(A == 16 || A == 64 || A == 128 || A == 256, "matrix decode: head_dim 16 to 256");
    constexpr int CPR = A / 8;              // 16-byte chunks per row
    constexpr int STEP = 32;                // tokens per matrix step
    constexpr int RPL = 64 / CPR;           // whole K rows per load instruction (2 to 32)
    constexpr int NKL = STEP / RPL;         // K load instructions per step
    constexpr int KS = (A + 31) / 32;       // 32-dim steps of S^T = K Q^T
    constexpr int DT = A / 16;              // 16-dim tiles of O^T
    // Head_dim 16: the K tile holds each row zero-padded to one 32-dim step
    // (chunks 2 and 3 zero), placed past the V^T tile so the zeros stay.
    constexpr int KCPR = A < 32 ? 4 : CPR;  // 16-byte chunks per K tile row
    constexpr int KOFF = A < 32 ? A * 4 : 0;  // K tile offset in the wave's tile
    // 4-token V row groups per load instruction (head_dim 16: lanes 16..63
    // repeat lanes 0..15, which already cover a 32-token step)
    constexpr int VPL = A < 32 ? 8 : 64 / CPR;
    constexpr int NVG = 8 / VPL;            // 4-token V row groups per lane (2, or 1 at head_dim <= 64)
    constexpr int DP = DECODE_PART;         // partition length: at most one wave's tokens
    constexpr int NT = DP / BS;             // table entries per wave, at most
    constexpr int NTV = (NT + 63) / 64;     // VGPRs holding them (4 for 4-token blocks)
    constexpr float RESCALE_SLACK = 8.0f;   // log2 units: weights stay < 2^8
    static_assert(BS % 4 == 0, "4 consecutive tokens must share a block");

    constexpr int GP = DECODE_GROUP;        // waves per work item (at most a partition each)
    static_assert(GP == 4, "one quarter of an item per wave of a 256-thread workgroup");

    // per wave: V^T of one 32-token step, [dim][4 chunks of 8 tokens], 64 B
    // rows; after the loop it holds the wave's accumulators (NG x 8 KiB) for
    // the combine
    constexpr int TILE = A < 32 ? A * 4 + 32 * KCPR : A * 4 * NG;  // per wave, 16-byte units
    static_assert(NG * DT * 64 <= TILE && KOFF + 32 * KCPR <= TILE, "wave tile");
    __shared__ uint4 sVt[GP][TILE];
    __shared__ float sML[GP][2][16 * NG];  // per wave: column max, column total
    __shared__ int arrived;                        // waves of the group done

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar loop control
    const int lane = threadIdx.x & 63;
    const int col = lane & 15;  // head column
    const int g = lane >> 4;    // token group: tokens 4g..4g+3 of each 16-token block
    const int lr = lane / CPR;  // K loads: row of this lane in one instruction
    const int lc = lane % CPR;  // loads: 16-byte chunk of this lane (dims 8 lc .. 8 lc + 7)
    const int vr = (A < 32 ? (lane & 15) : lane) / CPR;  // V loads: 4-row group
    // Workgroup -> (work item, kv head, head chunk) by decode_unit: the head
    // chunks of one (item, kv head) pair run on one XCD, 8 launch ids apart.
    // The grid covers the capacity; workgroups past the planned count leave
    // at once.
    const int64_t n_pairs = (int64_t)P.hdr[HDR_N_DEC] * P.hkv;
    const DecodeUnit unit = decode_unit(blockIdx.x, P.HC);
    if (unit.pair >= n_pairs) return;  // the whole workgroup
    if (threadIdx.x == 0) arrived = 0;
    __syncthreads();  // the only barrier: waves past the sequence leave below
    uint4* vt = &sVt[wave][0];
    if constexpr (A < 32) {  // the K tile's padding chunks (dims 16..31), zero for good
        const int r = lane >> 1, ch = 2 + (lane & 1);
        vt[KOFF + r * KCPR + (ch ^ (r % KCPR))] = make_uint4(0, 0, 0, 0);
    }

    const int GW = P.G / P.HC;  // heads of this wave (<= 16 * NG)
    const int hc = unit.hc;
    const int kvh = unit.pair % P.hkv;
    const int item = unit.pair / P.hkv;
    const int2 it = P.items[item];
    const int s = it.x;
    const int L = P.ctx[s] + 1;
    const int row = P.cu[s];
    // The sequence's items split it evenly (decode_split): each covers span
    // tokens (the last one fewer) and each wave a quarter of that, a
    // multiple of STEP tokens and at most one partition.  Item count and
    // split depend only on the sequence's own length.
    static_assert(STEP == 32 && DP == DECODE_PART && GP == DECODE_GROUP, "decode_split's shares");
    const DecodeSplit split = decode_split(L);
    const int ngroups = split.items;  // work items of the sequence
    const int per_wave = split.per_wave;
    const int span = GP * per_wave;
    const int i0 = it.y * span;
    const int t0 = i0 + wave * per_wave;
    if (t0 >= L) return;  // the item runs past the sequence
    const int nact = min(GP, (L - i0 + per_wave - 1) / per_wave);  // waves of this item with work
    const int nparts = ngroups == 1 ? nact : 2;  // 1: one wave holds the whole sequence
    const int t1 = min(L, t0 + per_wave);
    // first unpadded key (at most L - 1: the new token is never padding)
    const int kstart = MASKED ? min(max(P.key_start[s], 0), L - 1) : 0;
    const int h0 = kvh * P.G + hc * GW;
    const float cs = P.scale_log2;
    const bool pos_scale = cs > 0.f;

    // table slice: lane i of register v holds entry (t0 / BS + 64 v + i)
    const int lb0 = t0 / BS;
    const int nlb = (t1 - t0 + BS - 1) / BS;
    int tbl[NTV], short_tbl = 0;  // short_tbl: a needed block is past the table row
#pragma unroll
    for (int v = 0; v < NTV; ++v) {
        tbl[v] = -1;
        const int i = 64 * v + lane;
        if (i < nlb) {
            const int64_t lb = lb0 + i;
            if (lb < P.max_blocks) tbl[v] = P.table[(int64_t)s * P.max_blocks + lb];
            else short_tbl = 1;
        }
    }

    // Q^T operand of group ng: column col = head h0 + 16ng + col (zero past
    // GW), dims 32ks + 8g .. +7
    uint4 qb[NG][KS];
#pragma unroll
    for (int ng = 0; ng < NG; ++ng)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qb[ng][ks] = make_uint4(0, 0, 0, 0);
            if (16 * ng + col < GW && (A >= 32 || g * 8 < A))  // head_dim 16: dims 16.. are zero
                qb[ng][ks] = *reinterpret_cast<const uint4*>(
                    P.q + (((int64_t)row * P.hq + h0 + 16 * ng + col) * A + ks * 32 + g * 8));
        }

    f32x4_t o[NG][DT];  // O^T rows 16dt + 4g + r, column col of group ng
#pragma unroll
    for (int ng = 0; ng < NG; ++ng)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[ng][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m[NG], lsum[NG];
#pragma unroll
    for (int ng = 0; ng < NG; ++ng) {
        m[ng] = -1.0e30f;
        lsum[ng] = 0.f;
    }
    int bad = 0;

    // Block id of token t (< t1) through the table slice register tv, the
    // one that holds the current step's entries.  A step's entries never
    // straddle two registers: it starts a multiple of 32 tokens past t0, so
    // its first entry is a multiple of 32 / BS, which divides 64.  With
    // 16-token blocks every lane of a 16-token group asks for the same block,
    // so the caller passes the group's first (clamped) token and a uniform
    // readlane serves it; smaller blocks take a per-lane shuffle.
    auto block_of = [&](int tv, int t, int t_group) -> int64_t {
        if constexpr (BS == 16) {
            static_assert(NTV == 1, "one register of entries");
            return __builtin_amdgcn_readlane(tv, t_group / BS - lb0);
        } else {
            (void)t_group;
            return __shfl(tv, (t / BS - lb0) & 63, 64);
        }
    };

    // K and V are streamed with the non-temporal hint: each line is used
    // once, and the hint keeps it from displacing other data in L2 (V alone
    // gave 7 % more bandwidth, K as well 4 % more on the GQA batch).  The
    // hint only pays when one load instruction covers whole 128-byte lines:
    // loading K straight in the MFMA operand layout covers half of each line
    // per instruction, and the hint made the other half miss, so K rows are
    // loaded whole and rearranged through LDS.
    auto v_stream = [&](const uint4* ptr) -> uint4 {
        return __builtin_bit_cast(uint4, __builtin_nontemporal_load(
            reinterpret_cast<const u32x4_t*>(ptr)));
    };
    // The table register that holds the entries of the step at tc (a uniform
    // choice).  A step at or past t1 reads only token t1 - 1 (every token is
    // clamped to it), so it takes that token's register.
    static_assert(NTV == 1 || NTV == 4, "table slice registers");
    auto table_reg = [&](int tc) -> int {
        if constexpr (NTV == 1) {
            return tbl[0];
        } else {
            // a branch per register (a select chain can be turned into an
            // indexed stack array)
            switch (((min(tc, t1 - 1) - t0) / BS) >> 6) {
                case 0: return tbl[0];
                case 1: return tbl[1];
                case 2: return tbl[2];
                default: return tbl[3];
            }
        }
    };
    // ---- K: 32 rows, RPL per load, each row whole (CPR lanes x 16 B) --
    // Lane (lr, lc) of load j reads chunk lc of row RPL j + lr; the rows then
    // pass through the wave's LDS tile into the MFMA operand layout.  The
    // rows of one load share a 16-token block (head_dim 16 aside: 32 rows).
    uint4 kst[NKL];
    auto load_k = [&](int tc) __attribute__((always_inline)) {
        const int tv = table_reg(tc);
#pragma unroll
        for (int j = 0; j < NKL; ++j) {
            const int t = min(tc + RPL * j + lr, t1 - 1);
            int64_t blk;
            if constexpr (BS == 16 && RPL > 16) {  // head_dim 16: one load spans both blocks
                const int64_t b0 = block_of(tv, t, min(tc, t1 - 1));
                const int64_t b1 = block_of(tv, t, min(tc + 16, t1 - 1));
                blk = lr >= 16 ? b1 : b0;
            } else {
                blk = block_of(tv, t, min(tc + 16 * (RPL * j / 16), t1 - 1));
            }
            if (blk < 0 || blk >= P.num_blocks) { bad = 1; blk = 0; }
            kst[j] = v_stream(P.k_cache + ((blk * P.hkv + kvh) * BS + t % BS) * CPR + lc);
        }
    };
    // ---- V: 4-token groups lr + VPL h (h < NVG) x chunk lc ---------------
    // Each load instruction reads VPL whole rows; rows past the end repeat
    // the last row (their weight is 0).  No branch: the two sides of one
    // would load into the same registers, and the second side would wait for
    // every load in flight.  At head_dims 16 and 64 the 8 groups of one
    // instruction span both 16-token halves of the step, so with 16-token
    // blocks the lane picks one of the two halves' entries.
    uint4 vb[NVG][4];
    auto load_v = [&](int tc) __attribute__((always_inline)) {
        const int tv = table_reg(tc);
#pragma unroll
        for (int hh = 0; hh < NVG; ++hh) {
            const int tg = vr + VPL * hh;
            const int t = min(tc + 4 * tg, t1 - 1);
            int64_t blk;
            if constexpr (BS == 16 && VPL > 4) {
                const int64_t b0 = block_of(tv, t, min(tc, t1 - 1));
                const int64_t b1 = block_of(tv, t, min(tc + 16, t1 - 1));
                blk = tg >= 4 ? b1 : b0;
            } else {
                blk = block_of(tv, t, min(tc + 16 * (VPL * hh / 4), t1 - 1));
            }
            if (blk < 0 || blk >= P.num_blocks) { bad = 1; blk = 0; }
            const uint4* vp = P.v_cache + ((blk * P.hkv + kvh) * BS + t % BS) * CPR + lc;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                vb[hh][j] = v_stream(vp + (min(tc + 4 * tg + j, t1 - 1) - t) * CPR);
        }
    };
    // With two head groups (PF), and at head_dim 16, the next step's K rows
    // are requested as soon as this step's are in LDS and the K operands in
    // registers, and its V rows as soon as this step's V^T is in LDS, so they
    // are in flight during this step's products and softmax (the load
    // registers are free by then, and the kernel already runs two waves per
    // SIMD; head_dim 16 has registers to spare, and its 2 KiB steps are too
    // short to keep the memory busy one at a time: GQA batch 52.7 -> 49.5 us).
    constexpr bool PF = (NG == 2 && A <= 128) || A < 32;
    // Head_dim 256: V rows are requested once this step's K rows are in LDS,
    // so the K and V staging registers are never live together.
    constexpr bool SPLIT = A == 256;
    // Wait here for everything requested so far (the table slice and the Q^T
    // operand, whose loads are conditional), so the loop's waits count only
    // its own K/V loads.
    __builtin_amdgcn_s_waitcnt(0);
    if (PF) {
        load_k(t0);
        load_v(t0);
    }
    for (int tc = t0; tc < t1; tc += STEP) {
        // The next step's loads are issued unconditionally, so every path has
        // the same loads in flight and the waits stay partial; past the end
        // every lane reads row t1 - 1 (one row, then unused).
        const int tc_next = tc + STEP;
        if (!PF) {
            load_k(tc);
            if (!SPLIT) load_v(tc);
        }
        const bool padded = MASKED && tc < kstart;  // some key of this step is padding

        // K rows into this wave's tile ([row][chunk ^ row % CPR]), then the
        // A operands: lane (g, col) of block b, step ks takes chunk 4 ks + g
        // of row 16 b + col.  The V^T stores below reuse the tile after these
        // reads (same wave, in order).
#pragma unroll
        for (int j = 0; j < NKL; ++j) {
            const int r = RPL * j + lr;
            vt[KOFF + r * KCPR + (lc ^ (r % KCPR))] = kst[j];
        }
        if (!PF && SPLIT) load_v(tc);
        if (padded) {
#pragma unroll
            for (int hh = 0; hh < NVG; ++hh)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (tc + 4 * (vr + VPL * hh) + j < kstart) vb[hh][j] = make_uint4(0, 0, 0, 0);
        }
        uint4 kb[2][KS];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int r = 16 * b + col;
                kb[b][ks] = vt[KOFF + r * KCPR + ((4 * ks + g) ^ (r % KCPR))];
            }
        if (PF) load_k(tc_next);

        // ---- S^T for the two blocks, per head group ---------------------------
        f32x4_t sc[NG][2];
#pragma unroll
        for (int ng = 0; ng < NG; ++ng)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                sc[ng][b] = mfma16(kb[b][0], qb[ng][0], f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int ks = 1; ks < KS; ++ks) sc[ng][b] = mfma16(kb[b][ks], qb[ng][ks], sc[ng][b]);
            }

        // ---- V^T into LDS (this wave's tile): 8-byte units of 4 tokens ------
        // The 4x8 transpose is written as vector interleaves of whole rows
        // (element-wise extracts would let the optimizer split each 16-byte
        // row load into four 4-byte loads).
#pragma unroll
        for (int hh = 0; hh < NVG; ++hh) {
            const int tg = vr + VPL * hh;  // tokens 4 tg .. 4 tg + 3 of the step
            const u16x8_t r0 = __builtin_bit_cast(u16x8_t, vb[hh][0]);
            const u16x8_t r1 = __builtin_bit_cast(u16x8_t, vb[hh][1]);
            const u16x8_t r2 = __builtin_bit_cast(u16x8_t, vb[hh][2]);
            const u16x8_t r3 = __builtin_bit_cast(u16x8_t, vb[hh][3]);
            // word e of t01 = (row0[e], row1[e]); of t23 = (row2[e], row3[e])
            const u32x8_t t01 = __builtin_bit_cast(u32x8_t, __builtin_shufflevector(
                r0, r1, 0, 8, 1, 9, 2, 10, 3, 11, 4, 12, 5, 13, 6, 14, 7, 15));
            const u32x8_t t23 = __builtin_bit_cast(u32x8_t, __builtin_shufflevector(
                r2, r3, 0, 8, 1, 9, 2, 10, 3, 11, 4, 12, 5, 13, 6, 14, 7, 15));
            uint2* vt2 = reinterpret_cast<uint2*>(vt);
            // row d, 16-byte chunk tg % 4 (tokens 4(tg%4).. and 16+4(tg%4)..),
            // half tg / 4 (with 4 groups per instruction: lr and hh)
            const int gq = VPL == 4 ? vr : (tg & 3);
            const int half = VPL == 4 ? hh : (tg >> 2);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int d = lc * 8 + e;
                vt2[(d * 4 + (gq ^ ((d >> 2) & 3))) * 2 + half] = make_uint2(t01[e], t23[e]);
            }
        }
        if (PF) load_v(tc_next);

        // ---- online softmax of this lane's column, per head group ------------
        const bool tail = tc + STEP > t1;
        const float mc = pos_scale ? cs : 1.f;
        uint4 pb[NG];
#pragma unroll
        for (int ng = 0; ng < NG; ++ng) {
            float v8[8];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                v8[r] = sc[ng][0][r];
                v8[4 + r] = sc[ng][1][r];
            }
            if (!pos_scale) {
#pragma unroll
                for (int r = 0; r < 8; ++r) v8[r] *= cs;
            }
            if (tail || padded) {
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int t = tc + (r >> 2) * 16 + 4 * g + (r & 3);
                    if (t >= t1 || (MASKED && t < kstart)) v8[r] = -INFINITY;
                }
            }
            float mx = fmaxf(fmaxf(fmaxf(v8[0], v8[1]), fmaxf(v8[2], v8[3])),
                             fmaxf(fmaxf(v8[4], v8[5]), fmaxf(v8[6], v8[7])));
            mx = max_x32(max_x16(mx));
            const float cand = pos_scale ? mx * cs : mx;
            const bool grow = cand > m[ng] + RESCALE_SLACK;
            if (__any(grow)) {
                const float m_new = grow ? cand : m[ng];
                const float alpha = __builtin_amdgcn_exp2f(m[ng] - m_new);
                m[ng] = m_new;
                lsum[ng] *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) o[ng][dt] *= alpha;
            }
            float p[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(v8[r], mc, -m[ng]));
            pb[ng].x = pack_bf16x2(p[0], p[1]);
            pb[ng].y = pack_bf16x2(p[2], p[3]);
            pb[ng].z = pack_bf16x2(p[4], p[5]);
            pb[ng].w = pack_bf16x2(p[6], p[7]);
            // the denominator sums the bf16 weights the P.V product multiplies
            lsum[ng] = sum_bf16x2(pb[ng].x, lsum[ng]);
            lsum[ng] = sum_bf16x2(pb[ng].y, lsum[ng]);
            lsum[ng] = sum_bf16x2(pb[ng].z, lsum[ng]);
            lsum[ng] = sum_bf16x2(pb[ng].w, lsum[ng]);
        }

        // ---- O^T += V^T P^T (one V^T fragment for all head groups) ------------
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int d = dt * 16 + col;
            const uint4 a = vt[d * 4 + (g ^ ((d >> 2) & 3))];
#pragma unroll
            for (int ng = 0; ng < NG; ++ng) o[ng][dt] = mfma16(a, pb[ng], o[ng][dt]);
        }
    }
    // a block past the table reads as id -1: reported as a short table
    if (__any(short_tbl)) {
        if (lane == 0) set_flag(P.hdr, FLAG_TABLE_SHORT);
    } else if (__any(bad)) {
        if (lane == 0) set_flag(P.hdr, FLAG_BAD_BLOCK);
    }

    // ---- column totals and output ----------------------------------------------
    float lt[NG];
#pragma unroll
    for (int ng = 0; ng < NG; ++ng) {
        lt[ng] = sum_x32(sum_x16(lsum[ng]));
    }
    // normalised bf16 output of column group ng (scaled by inv)
    auto write_out = [&](int ng, const f32x4_t (&acc)[DT], float inv) {
        uint16_t* orow = P.out + ((int64_t)row * P.hq + h0 + 16 * ng + col) * A;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            uint2 v;
            v.x = pack_bf16x2(acc[dt][0] * inv, acc[dt][1] * inv);
            v.y = pack_bf16x2(acc[dt][2] * inv, acc[dt][3] * inv);
            *reinterpret_cast<uint2*>(orow + dt * 16 + 4 * g) = v;
        }
    };
    // split-K partial (max, total, fp32 accumulator) of work item `item`
    auto write_partial = [&](int ng, const f32x4_t (&acc)[DT], float mm, float ll) {
        const int64_t slot = (int64_t)item * P.hq + h0 + 16 * ng + col;
        float* dst = P.ws_acc + slot * A;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            *reinterpret_cast<float4*>(dst + dt * 16 + 4 * g) =
                make_float4(acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
        if (g == 0) {
            P.ws_ml[slot * 2] = mm;
            P.ws_ml[slot * 2 + 1] = ll;
        }
    };
    if (nparts == 1) {
#pragma unroll
        for (int ng = 0; ng < NG; ++ng)
            if (16 * ng + col < GW) write_out(ng, o[ng], 1.f / lt[ng]);
        return;
    }
    {
        // Combine the group in LDS.  Each wave leaves its column max and
        // total and its accumulator (in its own V^T tile, no longer read),
        // then counts itself in; the wave that arrives last combines the
        // group in wave order (fixed, so the result does not depend on which
        // wave that is).
        float4* mine = reinterpret_cast<float4*>(vt);
#pragma unroll
        for (int ng = 0; ng < NG; ++ng) {
            if (g == 0) {
                sML[wave][0][16 * ng + col] = m[ng];
                sML[wave][1][16 * ng + col] = lt[ng];
            }
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                mine[(ng * DT + dt) * 64 + lane] =
                    make_float4(o[ng][dt][0], o[ng][dt][1], o[ng][dt][2], o[ng][dt][3]);
        }
        __threadfence_block();  // this wave's LDS writes before its arrival
        int before = 0;
        if (lane == 0) before = atomicAdd(&arrived, 1);
        before = __shfl(before, 0, 64);
        if (before != nact - 1) return;
        __threadfence_block();  // every other wave's writes after the last arrival
#pragma unroll
        for (int ng = 0; ng < NG; ++ng) {
            const int c16 = 16 * ng + col;
            float mm = -INFINITY;
            for (int w = 0; w < nact; ++w) mm = fmaxf(mm, sML[w][0][c16]);
            float ll = 0.f;
            f32x4_t acc[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            for (int w = 0; w < nact; ++w) {
                const float sc = __builtin_amdgcn_exp2f(sML[w][0][c16] - mm);
                ll += sc * sML[w][1][c16];
                const float4* src = reinterpret_cast<const float4*>(&sVt[w][0]);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const float4 v = src[(ng * DT + dt) * 64 + lane];
                    acc[dt][0] += sc * v.x;
                    acc[dt][1] += sc * v.y;
                    acc[dt][2] += sc * v.z;
                    acc[dt][3] += sc * v.w;
                }
            }
            if (c16 < GW) {
                if (ngroups == 1) write_out(ng, acc, 1.f / ll);
                else write_partial(ng, acc, mm, ll);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Merge kernel: one wave per (decode sequence with several work items, query
// head); a work item's partial covers one partition group.
//   M = max_p m_p;  out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p
// The plan's descriptor carries everything the wave needs, and the (m, l)
// pairs and accumulators of up to 32 partials are requested together, so a
// wave waits for two round trips to memory (descriptor, then partials).
// ---------------------------------------------------------------------------
struct MergeParams {
    uint16_t* out;
    const int32_t* hdr;
    const int4* merge_list;
    const float* ws_ml;
    const float* ws_acc;
    int64_t cap_dec;
    int32_t hq;
};

template <int A>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams P) {
    constexpr int DPL = A >= 64 ? A / 64 : 1;  // dims per lane
    constexpr int CH = 32;                      // partitions per batch of loads
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int h = blockIdx.y * 4 + wave;
    const int n_merge = P.hdr[HDR_N_MERGE];
    // The descriptor is requested together with the count (both conditions
    // are evaluated, so neither load waits for the other); an entry at or
    // past the count is stale and is never used.
    const int4 desc = P.merge_list[blockIdx.x];
    if (((int)blockIdx.x >= n_merge) | (desc.z < 2) | (h >= P.hq)) return;
    const int64_t base = desc.y;
    const int np = desc.z;
    if (base < 0 || base + np > P.cap_dec) return;  // never true for a planned sequence
    const int d0 = min(lane * DPL, A - DPL);
    float M = NEG_BIG, den = 0.f, num[DPL];
#pragma unroll
    for (int i = 0; i < DPL; ++i) num[i] = 0.f;
    for (int c0 = 0; c0 < np; c0 += CH) {
        const int n = min(CH, np - c0);
        // lane p < n: (m, l) of partition c0 + p; every lane: its dims of all n
        float2 ml = make_float2(NEG_BIG, 0.f);
        if (lane < n)
            ml = *reinterpret_cast<const float2*>(P.ws_ml + ((base + c0 + lane) * P.hq + h) * 2);
        const float* accp = P.ws_acc + ((base + c0) * P.hq + h) * A + d0;
        float acc[CH][DPL];
#pragma unroll
        for (int p = 0; p < CH; ++p) {
            if (p < n) {
                if constexpr (DPL == 2) {
                    const float2 v = *reinterpret_cast<const float2*>(accp + (int64_t)p * P.hq * A);
                    acc[p][0] = v.x;
                    acc[p][1] = v.y;
                } else {
#pragma unroll
                    for (int i = 0; i < DPL; ++i) acc[p][i] = accp[(int64_t)p * P.hq * A + i];
                }
            } else {
#pragma unroll
                for (int i = 0; i < DPL; ++i) acc[p][i] = 0.f;
            }
        }
        float cm = ml.x;
        cm = wave_max(cm);
        const float Mn = fmaxf(M, cm);
        const float a = __builtin_amdgcn_exp2f(M - Mn);
        den *= a;
#pragma unroll
        for (int i = 0; i < DPL; ++i) num[i] *= a;
        M = Mn;
        const float w = lane < n ? __builtin_amdgcn_exp2f(ml.x - M) : 0.f;
        float wl = w * ml.y;
        wl = wave_sum(wl);
        den += wl;
#pragma unroll
        for (int p = 0; p < CH; ++p) {
            if (p < n) {
                const float wp = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), p));
#pragma unroll
                for (int i = 0; i < DPL; ++i) num[i] = fmaf(wp, acc[p][i], num[i]);
            }
        }
    }
    if (lane * DPL < A) {
        const float inv = 1.f / den;
        uint16_t* o = P.out + ((int64_t)desc.w * P.hq + h) * A + d0;
        if constexpr (DPL == 2) {
            *reinterpret_cast<uint32_t*>(o) = pack_bf16x2(num[0] * inv, num[1] * inv);
        } else {
#pragma unroll
            for (int i = 0; i < DPL; ++i)
                o[i] = (uint16_t)(pack_bf16x2(num[i] * inv, 0.f) & 0xffffu);
        }
    }
}

template <int A, int BS, bool MASKED>
void launch_decode_mfma(const StepArgs& a, const DecodeParams& p, bool two, int grid) {
    if constexpr (A <= 128 || BS == 16) {  // head_dim 256, 4-token blocks: one group (registers)
        if (two) {
            hipLaunchKernelGGL((decode_mfma_kernel<A, BS, 2, MASKED>), dim3(grid), dim3(256), 0, a.stream, p);
            return;
        }
    }
    hipLaunchKernelGGL((decode_mfma_kernel<A, BS, 1, MASKED>), dim3(grid), dim3(256), 0, a.stream, p);
}

}  // namespace

// 32 when G is a multiple of 32 (two column groups; not at head_dim 256 with
// 4-token blocks, whose table slice leaves no registers for them), else the
// largest divisor of G up to 16.
int decode_heads_per_wave(int G, int head_dim, int block_size) {
    if (G % 32 == 0 && (head_dim <= 128 || block_size == 16)) return 32;
    for (int gw = G < 16 ? G : 16; gw > 1; --gw)
        if (G % gw == 0) return gw;
    return 1;
}

hipError_t launch_prep(const StepArgs& a, bool with_append, hipEvent_t done) {
    char* ws = a.ws;
    const int G = a.num_q_heads / a.num_kv_heads;
    PrepParams p;
    p.cu = a.cu_seqlens_q;
    p.ctx = a.context_lens;
    p.num_seqs = a.num_seqs;
    p.total_q = a.total_q;
    p.max_q_len = a.max_q_len;
    p.max_context_len = a.max_context_len;
    p.span = prefill_span(G, a.prefill_waves);
    p.cap_dec = a.lay.cap_dec;
    p.cap_pre = a.lay.cap_pre;
    p.hdr = (int32_t*)(ws + a.lay.hdr);
    p.dec_items = (int2*)(ws + a.lay.dec_items);
    p.pre_items = (int2*)(ws + a.lay.pre_items);
    p.pre_sorted = (PreItem*)(ws + a.lay.pre_sorted);
    p.merge_list = (int4*)(ws + a.lay.merge_list);
    p.k_new = with_append ? (const uint4*)a.k_new : nullptr;
    p.v_new = with_append ? (const uint4*)a.v_new : nullptr;
    p.k_cache = (uint4*)a.k_cache;
    p.v_cache = (uint4*)a.v_cache;
    p.num_blocks = a.num_blocks;
    p.table = a.block_table;
    p.max_blocks = a.max_blocks;
    p.hkv = a.num_kv_heads;
    p.head_dim = a.head_dim;
    p.block_size = a.block_size;
    const int64_t rows_per_wg = PLAN_THREADS / 64;
    const int64_t grid = 1 + (with_append ? ((int64_t)a.total_q + rows_per_wg - 1) / rows_per_wg : 0);
    if (done)  // the launch itself records `done` when the kernel completes
        hipExtLaunchKernelGGL(prep_kernel, dim3((unsigned)grid), dim3(PLAN_THREADS), 0, a.stream, nullptr,
                              done, 0, p);
    else
        hipLaunchKernelGGL(prep_kernel, dim3((unsigned)grid), dim3(PLAN_THREADS), 0, a.stream, p);
    return hipGetLastError();
}

hipError_t launch_decode(const StepArgs& a) {
    char* ws = a.ws;
    const int G = a.num_q_heads / a.num_kv_heads;
    const int GW = decode_heads_per_wave(G, a.head_dim, a.block_size);
    DecodeParams p;
    p.q = (const uint16_t*)a.q;
    p.out = (uint16_t*)a.out;
    p.k_cache = (const uint4*)a.k_cache;
    p.v_cache = (const uint4*)a.v_cache;
    p.table = a.block_table;
    p.cu = a.cu_seqlens_q;
    p.ctx = a.context_lens;
    p.hdr = (int32_t*)(ws + a.lay.hdr);
    p.items = (const int2*)(ws + a.lay.dec_items);
    p.ws_ml = (float*)(ws + a.lay.ml);
    p.ws_acc = (float*)(ws + a.lay.acc);
    p.key_start = a.key_start;
    p.num_blocks = a.num_blocks;
    p.max_blocks = a.max_blocks;
    p.hq = a.num_q_heads;
    p.hkv = a.num_kv_heads;
    p.G = G;
    p.HC = G / GW;
    p.scale_log2 = a.scale * 1.4426950408889634f;
    // one workgroup per decode unit (decode_unit / decode_grid)
    const int64_t grid64 = decode_grid(a.lay.cap_dec * a.num_kv_heads, p.HC);
    if (grid64 <= 0) return hipSuccess;
    if (grid64 > INT32_MAX) return hipErrorInvalidValue;
    const int grid = (int)grid64;
    const bool two = GW > 16;  // 32 heads per wave: two MFMA column groups
    const bool bs16 = a.block_size == 16;
    if (a.key_start) {  // the left-padded batch (head_dim 128 only)
        if (a.head_dim != 128) return hipErrorInvalidValue;
        if (bs16) launch_decode_mfma<128, 16, true>(a, p, two, grid);
        else launch_decode_mfma<128, 4, true>(a, p, two, grid);
        return hipGetLastError();
    }
    switch (a.head_dim) {
        case 16:
            if (bs16) launch_decode_mfma<16, 16, false>(a, p, two, grid);
            else launch_decode_mfma<16, 4, false>(a, p, two, grid);
            break;
        case 64:
            if (bs16) launch_decode_mfma<64, 16, false>(a, p, two, grid);
            else launch_decode_mfma<64, 4, false>(a, p, two, grid);
            break;
        case 128:
            if (bs16) launch_decode_mfma<128, 16, false>(a, p, two, grid);
            else launch_decode_mfma<128, 4, false>(a, p, two, grid);
            break;
        case 256:
            if (bs16) launch_decode_mfma<256, 16, false>(a, p, two, grid);
            else launch_decode_mfma<256, 4, false>(a, p, two, grid);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_merge(const StepArgs& a) {
    char* ws = a.ws;
    MergeParams mp;
    mp.out = (uint16_t*)a.out;
    mp.hdr = (const int32_t*)(ws + a.lay.hdr);
    mp.merge_list = (const int4*)(ws + a.lay.merge_list);
    mp.ws_ml = (const float*)(ws + a.lay.ml);
    mp.ws_acc = (const float*)(ws + a.lay.acc);
    mp.cap_dec = a.lay.cap_dec;
    mp.hq = a.num_q_heads;
    dim3 mgrid((unsigned)a.num_seqs, (unsigned)((a.num_q_heads + 3) / 4));
    switch (a.head_dim) {
        case 128: hipLaunchKernelGGL(merge_kernel<128>, mgrid, dim3(256), 0, a.stream, mp); break;
        case 64: hipLaunchKernelGGL(merge_kernel<64>, mgrid, dim3(256), 0, a.stream, mp); break;
        case 256: hipLaunchKernelGGL(merge_kernel<256>, mgrid, dim3(256), 0, a.stream, mp); break;
        default: hipLaunchKernelGGL(merge_kernel<16>, mgrid, dim3(256), 0, a.stream, mp); break;
    }
    return hipGetLastError();
}

}  // namespace kvc
