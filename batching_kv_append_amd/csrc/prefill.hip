// Prefill-chunk path: rows of sequences that bring >= 2 new tokens.
//
// A chunk of m new rows attends over the sequence's cached keys followed by
// its own new keys, with the causal mask shifted by the cached length
// (news.myit.tw continuous-batching article, section "Chunked prefill": the
// cached K/V are prepended to the new ones and the mask is adjusted).  QK^T
// costs O(n^2 d) (same article, "Attention"), so this path is bound by matrix
// throughput and runs both products on gfx950 bf16 MFMA with fp32
// accumulation:
//
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16, A = K tile (LDS), B = Q^T (VGPRs)
//   O^T += V^T P^T   A = V^T tile (LDS), B = P^T (the softmax of S^T, bf16)
//
// Computing the transposed scores makes each lane own one query column: its
// 16 accumulator registers per 32-key block are exactly the 8+8 k-slots of the
// B operand of the next product (the key order inside a 16-key step only has
// to agree between P^T and V^T, which reads its keys in the same order), so P
// never leaves the registers.  Softmax statistics are per lane (one column)
// with one exchange with lane^32 per 64-key tile.  The running maximum is
// only moved when it grows by more than 2^8 (weights stay below 256); the
// numerator and the denominator share it, so the result is unchanged and the
// accumulator rescale is rare.
//
// Work: one workgroup = NW waves = HPW query heads of one kv group x (NW/HPW)
// blocks of QW = 32 positions; each wave owns one (head, 32 positions).  The
// blocks of a sequence are dealt to its workgroups in snake order (an early
// block with a late one), so their causal key ranges even out.  A prefill
// that runs beside a decode takes NW = 4, which leaves the co-running decode
// more of each unit (at head_dim 128 one such workgroup per compute unit, by
// an LDS reservation at launch).  One with the chip to
// itself (a call of chunks only, or one whose few decode rows run after it)
// takes NW = 8 up to head_dim 128: one workgroup per compute unit, two waves
// per SIMD, so every K/V tile brought into the unit feeds 8 waves instead of
// 4, and waves 4..7 (the second wave of each SIMD) run P.V one tile late, so
// the two waves of a SIMD are out of phase (about 5 % on a 32K prompt).  K/V
// tiles of 64 keys (gathered block by block through the block table) are
// staged in LDS once per workgroup and shared by the HPW heads of the group
// (GQA, e2hang/Notes "MQA与GQA"): K double-buffered, V in two buffers (four
// with the late waves).  K and V are both stored
// row-major, as they sit in the cache, each with its own 16-byte XOR swizzle:
// the K operand is one ds_read_b128 per lane, and the V^T operand is read
// with the transposing LDS load of gfx950 (ds_read_b64_tr_b16: within each
// 16-lane group, lane o receives element o % 4 of the 8-byte loads of lanes
// 4j + o / 4, j = 0..3), two per MFMA, so no transpose is done by the ALUs.
// Each loading thread owns KPT (1, 2 or 4) consecutive keys x 8 dims (twice
// for head_dim 256) and writes them with 16-byte stores.  The planning kernel
// lists the workgroups costliest first.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "kvc_launch.h"

namespace kvc {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));

struct PrefillParams {
    const uint16_t* q;
    uint16_t* out;
    const uint4* k_cache;
    const uint4* v_cache;
    const int32_t* table;
    int32_t* hdr;
    const PreItem* items;
    int64_t num_blocks;
    int32_t max_blocks, hq, hkv, G, HC;
    float scale_log2;  // scale * log2(e)
};

// Workgroups are handed to the 8 XCDs (each with its own L2) round-robin by
// linear id.  The grid is one-dimensional over (work item, head slot), head
// slot = kv head x head chunk, item-major: workgroup L is item L / slots,
// slot L % slots, so it runs on XCD (item x slots + slot) mod 8.  With a
// slot count that is a multiple of 8 that is slot mod 8, and with one that
// divides 8 the XCD fixes the slot (XCD mod slots): either way an XCD serves
// a fixed set of head slots, and the K/V of a kv head are fetched into one L2
// (or, with fewer than 8 slots, into 8 / slots of them) instead of all
// eight.  Within an XCD, items keep the planner's costliest-first order.

__device__ __forceinline__ f32x16_t mfma32(uint4 a, uint4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// XOR swizzle of the 16-byte chunks of V row `row` (a key of the tile):
// 0, 6, 10, 12 for row % 4 = 0..3, and 8 more when row % 16 >= 8.  A
// transposing read takes 4 consecutive rows x 2 (16 lanes) or 4 (32 lanes)
// consecutive chunks; bits 1-2 and bits 2-3 of the four swizzles are both
// all distinct, so either lane group hits distinct banks.  The tile loaders'
// 16-byte writes (16 lanes: the 16 chunks of one row, or with head_dim 64
// the 8 chunks of two adjacent rows) are conflict-free as well: the swizzle
// permutes the chunks within a row.
template <int CPR>
__device__ __forceinline__ int vswz(int row) {
    return (((row & 1) * 6) ^ (((row >> 1) & 1) * 10) ^ (row & 8)) & (CPR - 1);
}

// Combine x of lanes l and l ^ 32 with the gfx950 half-wave swap
// (v_permlane32_swap trades one half-wave of its first operand with the other
// half-wave of its second), in the VALU rather than through the LDS crossbar.
// Swapping x with itself leaves every lane holding its own value in one
// result and its partner's in the other, so max and sum of the pair are the
// same whichever result is which.
__device__ __forceinline__ float halves_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 8-byte transposing LDS read (ds_read_b64_tr_b16) at a byte address of a
// __shared__ array.
__device__ __forceinline__ i16x4_t lds_read_tr16(const char* p) {
    typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)const_cast<char*>(p));
}

// NW = 4: up to two workgroups per compute unit (one for head_dim 256, whose
// accumulators and Q^T operand double: 128 KiB of LDS, one wave per SIMD).
// NW = 8 (no decode beside it, head_dim <= 128): one workgroup per
// compute unit, two waves per SIMD, each K/V tile fetched once for 8 waves,
// and the second wave of each SIMD runs P.V one tile late.
template <int A, int BS, int HPW, int NW>
__global__ __launch_bounds__(64 * NW, A > 128 ? 1 : 2) void prefill_kernel(PrefillParams P) {
    static_assert(NW == 4 || (NW == 8 && A <= 128), "8-wave workgroups up to head_dim 128");
    constexpr int NT = 64 * NW;            // threads per workgroup
    constexpr int TK = PREFILL_TK;         // keys per tile (64)
    constexpr int CPR = A / 8;             // 16-byte chunks per K/V row
    constexpr int KK = A / 16;             // 16-dim MFMA steps of QK^T
    constexpr int DT = (A + 31) / 32;      // 32-dim output tiles
    constexpr int QW = PREFILL_QW;         // positions per wave (32)
    constexpr int SPAN = QW * (NW / HPW);  // positions per workgroup
    constexpr int CW = CPR < 16 ? CPR : 16;  // loading threads along one row
    constexpr int NKC = CPR / CW;          // 16-byte chunks per thread and row (2 for head_dim 256)
    constexpr int KPT = TK * CW / NT > 0 ? TK * CW / NT : 1;  // keys per loading thread
    constexpr int LOADERS = (TK / KPT) * CW;  // threads that load
    constexpr float NEG_BIG = -1.0e30f;
    constexpr float RESCALE_SLACK = 8.0f;  // log2 units: weights stay < 2^8
    static_assert(LOADERS <= NT && LOADERS * KPT * NKC == TK * CPR, "tile loaders");
    static_assert(BS % KPT == 0, "a thread's keys must share a block");

    __shared__ uint4 sK[2][TK * CPR];  // [key][chunk ^ (key % CPR)]
    constexpr int NVB = NW == 8 ? 4 : 2;  // V tiles in LDS (four: P.V runs a tile late on half the waves)
    __shared__ uint4 sV[NVB][TK * CPR];  // [key][chunk ^ vswz(key)]
    __shared__ int sTab[2][TK / BS];   // block ids of the next tile's blocks

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int hi = lane >> 5;   // which half of the wave
    const int col = lane & 31;  // query column of this lane

    const int slots = P.hkv * P.HC;
    const int item = (int)blockIdx.x / slots, slot = (int)blockIdx.x % slots;
    // The item's record (sequence, lengths) is read together with the
    // planned count: item is below the list's capacity, so the read is in
    // bounds either way, and testing both values keeps the two loads in one
    // round trip.
    const int n_pre = P.hdr[HDR_N_PRE];
    const PreItem it = P.items[item];
    if (item >= n_pre || it.s < 0) return;
    const int s = it.s, tile = it.tile;
    const int kvh = slot / P.HC;
    const int hc = slot % P.HC;
    const int h = kvh * P.G + hc * HPW + (wave % HPW);
    const int row0 = it.row0;
    const int qlen = it.qlen;
    const int c = it.ctx;
    const int L = c + qlen;
    constexpr int NPB = NW / HPW;  // position blocks per workgroup (snake order across items)
    const int p0 = prefill_block(tile, wave / HPW, (qlen + SPAN - 1) / SPAN) * QW;  // first position of this wave
    const int wg_last = prefill_item_end(tile, qlen, NPB) - 1;  // last position of the workgroup
    const int nkt = (c + wg_last + 1 + TK - 1) / TK;        // key tiles the workgroup needs
    const int kend_w = (p0 < qlen) ? c + min(p0 + QW, qlen) : 0;  // keys this wave needs
    const float cs = P.scale_log2;
    const bool pos_scale = cs > 0.f;

    // ---- Q^T operand: 32 columns, KK 16-dim steps -------------------------
    uint4 qreg[KK];
    {
        const int pos = p0 + col;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            qreg[kk] = make_uint4(0, 0, 0, 0);
            if (pos < qlen)
                qreg[kk] = *reinterpret_cast<const uint4*>(
                    P.q + (((int64_t)(row0 + pos) * P.hq + h) * A + kk * 16 + hi * 8));
        }
    }

    f32x16_t o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
    float m = NEG_BIG;  // running maximum, scaled log2 units
    float lsum[4] = {0.f, 0.f, 0.f, 0.f};  // partial denominators, one per 16-key step

    // ---- cooperative tile loads: thread = KPT consecutive keys x one chunk ---
    // The KPT keys of a thread share one cache block (k0 and its first key
    // are multiples of KPT, and so is the block size), so a thread reads KPT
    // rows of one block at fixed offsets.  A thread whose keys are at or past L
    // reads the rows of the block that holds key L-1 instead (memory of that
    // block, whatever it holds):
    // keys >= L are masked out of every stored row's scores by select, and
    // their V rows are zeroed before they reach LDS, so their weight of 0
    // never meets a non-finite value.
    const bool loader = LOADERS == NT || tid < LOADERS;  // a constant when every thread loads
    // Thread -> (keys kb .. kb+KPT-1, 16-byte chunk cc: dims 8cc .. 8cc+7;
    // with head_dim 256 also chunk cc + 16).  The CW threads of a row are
    // consecutive lanes, so a 16-byte store instruction writes whole rows
    // (16 distinct bank groups per row with the swizzles below) and a load
    // instruction reads whole 256-byte row segments.
    const int cc = tid % CW;
    const int kb = KPT * (tid / CW);
    // offset (16-byte units) of the thread's first row inside a cache block
    const uint32_t toff = (uint32_t)((kvh * BS + kb % BS) * CPR + cc);
    const uint32_t blk_stride = (uint32_t)(P.hkv * BS * CPR);
    u32x4_t kreg[KPT * NKC], vreg[KPT * NKC];  // native vectors: the staging stays in VGPRs
    int bad = 0;
    // Block-table entry of this thread's keys in the tile at k0 (tiles past
    // the end give the block of key L-1).  Entries are read two tiles ahead,
    // unconditionally (an index past the row is clamped into it and flagged),
    // and handed on through LDS: every thread publishes the entry of its
    // block with the tile's stores (the threads of one block compute the
    // same entry), and the next step reads it from there.  So no register
    // carries a global load across the loop, and no step waits for the table.
    const int kblk = loader ? kb / BS : 0;  // the thread's block within a tile
    int short_tbl = 0;  // a needed block is past the table row
    auto table_entry = [&](int k0) __attribute__((always_inline)) -> int {
        const int lb = min(k0 + kb, L - 1) / BS;
        short_tbl |= lb >= P.max_blocks;
        return P.table[(int64_t)s * P.max_blocks + min(lb, P.max_blocks - 1)];
    };
    auto load_tile = [&](int entry) __attribute__((always_inline)) {
        if (!loader) return;
        uint32_t blk = (uint32_t)entry;
        if (entry < 0 || (int64_t)entry >= P.num_blocks) {
            bad = 1;
            blk = 0;
        }
        const uint64_t base = (uint64_t)blk * blk_stride + toff;
        const uint4* kp = P.k_cache + base;
        const uint4* vp = P.v_cache + base;
#pragma unroll
        for (int c = 0; c < NKC; ++c)
#pragma unroll
            for (int j = 0; j < KPT; ++j) {
                kreg[c * KPT + j] = __builtin_bit_cast(u32x4_t, kp[j * CPR + c * 16]);
                vreg[c * KPT + j] = __builtin_bit_cast(u32x4_t, vp[j * CPR + c * 16]);
            }
    };
    auto store_tile = [&](int kbuf, int vbuf, int k0) __attribute__((always_inline)) {
        if (!loader) return;
        if (k0 + kb + KPT - 1 >= L) {  // the sequence's last keys: V rows past L are zero
#pragma unroll
            for (int c = 0; c < NKC; ++c)
#pragma unroll
                for (int j = 0; j < KPT; ++j)
                    if (k0 + kb + j >= L) vreg[c * KPT + j] = u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int c = 0; c < NKC; ++c)
#pragma unroll
            for (int j = 0; j < KPT; ++j) {
                const int key = kb + j;
                const int ch = cc + c * 16;
                sK[kbuf][key * CPR + (ch ^ (key % CPR))] = __builtin_bit_cast(uint4, kreg[c * KPT + j]);
                sV[vbuf][key * CPR + (ch ^ vswz<CPR>(key))] = __builtin_bit_cast(uint4, vreg[c * KPT + j]);
            }
    };
    // Transposing-read offsets (bytes inside a V tile) of this lane for the
    // V^T operand of output tile dt, keys 8 rd + {0..3} of a 16-key step: the
    // lane is source 4j + q of its 16-lane group g, so it points at key row
    // 4 (g / 2) + j + 8 rd, dims 32 dt + 16 (g % 2) + 4q .. +3.  Rows of the
    // other steps are 16 or 32 keys further, which keeps the swizzle, so they
    // are constant offsets.  With A = 16 the lanes of dims 16..31 read chunk 0
    // and their operand is replaced by zeros.
    int troff[DT][2];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int rd = 0; rd < 2; ++rd) {
            const int g = lane >> 4, q = lane & 3, j = (lane >> 2) & 3;
            const int row = 4 * (g >> 1) + j + 8 * rd;
            int chunk = dt * 4 + 2 * (g & 1) + (q >> 1);
            if (chunk >= CPR) chunk = 0;
            troff[dt][rd] = row * CPR * 16 + (chunk ^ vswz<CPR>(row)) * 16 + (q & 1) * 8;
        }

    {
        const int e1 = table_entry(TK);
        if (nkt > 0) {
            load_tile(table_entry(0));
            store_tile(0, 0, 0);
        }
        if (loader) sTab[1][kblk] = e1;
    }
    __syncthreads();
    // Explicit wait for everything issued so far (the Q^T operand loads are
    // conditional, and without it the compiler assumes they may still be in
    // flight inside the loop and waits for ALL loads, the next tile's
    // included, before the first MFMA of every tile).
    __builtin_amdgcn_s_waitcnt(0);
    // With 8 waves, waves 4..7 (the second wave of each SIMD) run P.V one
    // tile late: in step t they multiply the previous tile's weights by its V
    // tile (kept in its own buffer: V tiles rotate through four), then take
    // this tile's scores and softmax.  So the two waves of a SIMD are out of
    // phase: one issues matrix work while the other does its vector work.
    // Each tile step's buffer indices are compile-time constants (the loop
    // is unrolled by four), so every LDS address of a step is a per-lane
    // register plus an immediate.
    const bool late = NW == 8 && wave >= 4;
    uint4 pb[2][2];  // [kh][ks] bf16 P^T operands
    auto qk_soft = [&](const int k0, auto kbc) __attribute__((always_inline)) {
        constexpr int kbuf = decltype(kbc)::value;  // K tile buffer
        // Raised wave priority around the two MFMA blocks: a wave that
        // reaches its matrix work is issued ahead of the others' softmax
        // and LDS stores, so the matrix pipe idles less (about 2% on long
        // chunks).
        __builtin_amdgcn_s_setprio(2);
        // ---- S^T = K Q^T : two 32-key halves -------------------------
        f32x16_t sacc[2];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kh][r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const int key = kh * 32 + col;
                const int ch = kk * 2 + hi;
                const uint4 a = sK[kbuf][key * CPR + (ch ^ (key % CPR))];
                sacc[kh] = mfma32(a, qreg[kk], sacc[kh]);
            }
        }

        __builtin_amdgcn_s_setprio(0);
        // ---- online softmax of this lane's column ---------------------
        const int lim = c + p0 + col;               // last visible key of the column
        const bool diag = k0 + TK - 1 > c + p0;     // some key may be masked
        if (!pos_scale) {
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[kh][r] *= cs;
        }
        if (diag) {
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + kh * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                    if (key > lim) sacc[kh][r] = -INFINITY;
                }
        }
        // column maximum: four independent chains, then the other half-wave
        float mq[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            mq[i] = fmaxf(sacc[i >> 1][(i & 1) * 8], sacc[i >> 1][(i & 1) * 8 + 1]);
#pragma unroll
            for (int r = 2; r < 8; ++r) mq[i] = fmaxf(mq[i], sacc[i >> 1][(i & 1) * 8 + r]);
        }
        float mx = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
        mx = halves_max(mx);
        const float cand = pos_scale ? mx * cs : mx;  // column max, scaled log2 units
        const bool grow = cand > m + RESCALE_SLACK;
        if (__any(grow)) {
            const float m_new = grow ? cand : m;
            const float alpha = __builtin_amdgcn_exp2f(m - m_new);
            m = m_new;
#pragma unroll
            for (int i = 0; i < 4; ++i) lsum[i] *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
        }
        const float mc = pos_scale ? cs : 1.f;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            float p[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(sacc[kh][r], mc, -m));
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                pb[kh][ks].x = pack_bf16x2(p[ks * 8 + 0], p[ks * 8 + 1]);
                pb[kh][ks].y = pack_bf16x2(p[ks * 8 + 2], p[ks * 8 + 3]);
                pb[kh][ks].z = pack_bf16x2(p[ks * 8 + 4], p[ks * 8 + 5]);
                pb[kh][ks].w = pack_bf16x2(p[ks * 8 + 6], p[ks * 8 + 7]);
                // the denominator sums the same bf16 weights the P.V
                // product uses: one dot2 with (1, 1) per pair
                float& ls = lsum[kh * 2 + ks];
                ls = sum_bf16x2(pb[kh][ks].x, ls);
                ls = sum_bf16x2(pb[kh][ks].y, ls);
                ls = sum_bf16x2(pb[kh][ks].z, ls);
                ls = sum_bf16x2(pb[kh][ks].w, ls);
            }
        }

    };
    auto pv = [&](auto vbc) __attribute__((always_inline)) {
        constexpr int vbuf = decltype(vbc)::value;  // V tile buffer
        __builtin_amdgcn_s_setprio(2);
        // ---- O^T += V^T P^T ---------------------------------------------
        // Operand slot e of lane l holds V[key][32 dt + l % 32] for key
        // 32 kh + 16 ks + 8 (e / 4) + 4 (l / 32) + e % 4, the key order of
        // the P^T slots.
        const char* vb = reinterpret_cast<const char*>(&sV[vbuf][0]);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int rb = (kh * 32 + ks * 16) * CPR * 16;
                    const i16x4_t v0 = lds_read_tr16(vb + troff[dt][0] + rb);
                    const i16x4_t v1 = lds_read_tr16(vb + troff[dt][1] + rb);
                    i16x8_t a8 = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
                    if (A < 32 && (lane & 16)) a8 = i16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
                    o[dt] = mfma32(__builtin_bit_cast(uint4, a8), pb[kh][ks], o[dt]);
                }
        }
    };
    auto run = [&](auto latec) __attribute__((always_inline)) {
        constexpr bool LATE = decltype(latec)::value;
        bool prev = false;  // the previous tile's weights wait for their P.V
        auto tile_step = [&](const int t, auto bc) __attribute__((always_inline)) {
            constexpr int b = decltype(bc)::value;  // t % 4
            const int k0 = t * TK;
            const int entry2 = table_entry(k0 + 2 * TK);           // consumed by this step's stores
            if (t + 1 < nkt) load_tile(sTab[(b & 1) ^ 1][kblk]);  // in flight during this tile's math
            if (LATE) {
                if (prev) pv(std::integral_constant<int, (b + NVB - 1) % NVB>{});
                prev = k0 < kend_w;
                if (prev) qk_soft(k0, std::integral_constant<int, b & 1>{});
            } else if (k0 < kend_w) {
                qk_soft(k0, std::integral_constant<int, b & 1>{});
                pv(std::integral_constant<int, b % NVB>{});
            }
            __builtin_amdgcn_s_setprio(0);
            if (t + 1 < nkt) store_tile((b & 1) ^ 1, (b + 1) % NVB, k0 + TK);
            if (loader) sTab[b & 1][kblk] = entry2;  // the tile after next
            __syncthreads();
        };
        for (int t = 0; t < nkt; t += 4) {
            tile_step(t, std::integral_constant<int, 0>{});
            if (t + 1 < nkt) tile_step(t + 1, std::integral_constant<int, 1>{});
            if (t + 2 < nkt) tile_step(t + 2, std::integral_constant<int, 2>{});
            if (t + 3 < nkt) tile_step(t + 3, std::integral_constant<int, 3>{});
        }
        if (LATE && prev) {  // the last tile's P.V (its V tile is still in place)
            switch ((nkt - 1) % NVB) {
                case 0: pv(std::integral_constant<int, 0>{}); break;
                case 1: pv(std::integral_constant<int, 1 % NVB>{}); break;
                case 2: pv(std::integral_constant<int, 2 % NVB>{}); break;
                default: pv(std::integral_constant<int, 3 % NVB>{}); break;
            }
        }
    };
    if (late) run(std::true_type{});
    else run(std::false_type{});
    if (short_tbl) atomicOr(P.hdr + HDR_FLAGS, FLAG_TABLE_SHORT);
    if (bad) atomicOr(P.hdr + HDR_FLAGS, FLAG_BAD_BLOCK);

    // ---- normalise and store ------------------------------------------------
    // The wave's 32 output rows go out through LDS (the V tile buffers, free
    // once every wave is past its last P.V): each lane writes its 8-byte
    // pieces of its column's row (16-byte chunks XOR-swizzled by row), then
    // the wave stores whole rows, CPR lanes x 16 B each, so every global
    // store instruction writes complete 128-byte lines instead of 16-byte
    // pieces of 32 rows.  Rows past the chunk are not stored.
    constexpr int SWZ = CPR < 16 ? CPR : 16;    // chunk swizzle period
    constexpr int ORPI = 64 / CPR;              // rows per store instruction
    static_assert(NW * QW * A * 2 <= (int)sizeof(sV), "output rows fit the V tiles");
    const float lw = (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
    const float inv = 1.f / halves_sum(lw);  // columns past the chunk: never stored
    __syncthreads();  // every wave is done with the V tiles
    char* ob = reinterpret_cast<char*>(&sV[0][0]) + wave * (QW * A * 2);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const int d = dt * 32 + 8 * rg + 4 * hi;
            if (d < A) {
                uint2 v;
                v.x = pack_bf16x2(o[dt][rg * 4 + 0] * inv, o[dt][rg * 4 + 1] * inv);
                v.y = pack_bf16x2(o[dt][rg * 4 + 2] * inv, o[dt][rg * 4 + 3] * inv);
                const int ch = (d >> 3) ^ (col % SWZ);
                *reinterpret_cast<uint2*>(ob + col * (A * 2) + ch * 16 + hi * 8) = v;
            }
        }
#pragma unroll
    for (int i = 0; i < QW / ORPI; ++i) {
        const int r = i * ORPI + lane / CPR;  // row of the wave's block
        const int c = lane % CPR;             // 16-byte chunk: dims 8c .. 8c+7
        const uint4 v = *reinterpret_cast<const uint4*>(ob + r * (A * 2) + ((c ^ (r % SWZ)) * 16));
        if (p0 + r < qlen)
            *reinterpret_cast<uint4*>(P.out + ((int64_t)(row0 + p0 + r) * P.hq + h) * A + c * 8) = v;
    }
}

// Beside the decode at head_dim 128, a compute unit takes at most one prefill
// workgroup: the launch reserves 20 KiB of unused dynamic LDS, which brings
// the workgroup's 64 KiB past half of the unit's 160 KiB.  Two of them (464
// of a SIMD's 512 registers) would leave no room for a decode wave on that
// unit; one leaves room for a decode workgroup.  Mixed step 0.764 -> 0.756 ms
// (four runs each, one box).  At head_dim 64 the same cap costs 6 % (0.383 ->
// 0.406 ms on the same rows) and at 16 it changes nothing, so it is kept to 128.
constexpr unsigned PREFILL_ONE_PER_CU_PAD = 20 * 1024;

template <int A, int BS, int NW>
void launch_prefill_nw(const StepArgs& a, const PrefillParams& p, int hpw, dim3 grid) {
    const dim3 block(64 * NW);
    const unsigned pad = (A == 128 && NW == 4 && a.prefill_beside_decode) ? PREFILL_ONE_PER_CU_PAD : 0u;
    switch (hpw) {
        case 1: hipLaunchKernelGGL((prefill_kernel<A, BS, 1, NW>), grid, block, pad, a.stream, p); break;
        case 2: hipLaunchKernelGGL((prefill_kernel<A, BS, 2, NW>), grid, block, pad, a.stream, p); break;
        default: hipLaunchKernelGGL((prefill_kernel<A, BS, 4, NW>), grid, block, pad, a.stream, p); break;
    }
}

template <int A, int BS>
void launch_prefill_hpw(const StepArgs& a, const PrefillParams& p, int hpw, dim3 grid) {
    if constexpr (A <= 128) {
        if (a.prefill_waves == 8) {
            launch_prefill_nw<A, BS, 8>(a, p, hpw, grid);
            return;
        }
    }
    launch_prefill_nw<A, BS, 4>(a, p, hpw, grid);
}

}  // namespace

hipError_t launch_prefill(const StepArgs& a) {
    if (a.max_q_len < 2) return hipSuccess;
    char* ws = a.ws;
    const int G = a.num_q_heads / a.num_kv_heads;
    const int hpw = prefill_hpw(G);
    PrefillParams p;
    p.q = (const uint16_t*)a.q;
    p.out = (uint16_t*)a.out;
    p.k_cache = (const uint4*)a.k_cache;
    p.v_cache = (const uint4*)a.v_cache;
    p.table = a.block_table;
    p.hdr = (int32_t*)(ws + a.lay.hdr);
    p.items = (const PreItem*)(ws + a.lay.pre_sorted);
    p.num_blocks = a.num_blocks;
    p.max_blocks = a.max_blocks;
    p.hq = a.num_q_heads;
    p.hkv = a.num_kv_heads;
    p.G = G;
    p.HC = G / hpw;
    p.scale_log2 = a.scale * 1.4426950408889634f;
    const int slots = a.num_kv_heads * p.HC;
    const int64_t gx = a.lay.cap_pre * slots;
    if (gx <= 0) return hipSuccess;
    if (gx > INT32_MAX) return hipErrorInvalidValue;
    dim3 grid((unsigned)gx);
    const bool b16 = a.block_size == 16;
    switch (a.head_dim) {
        case 128:
            if (b16) launch_prefill_hpw<128, 16>(a, p, hpw, grid);
            else launch_prefill_hpw<128, 4>(a, p, hpw, grid);
            break;
        case 64:
            if (b16) launch_prefill_hpw<64, 16>(a, p, hpw, grid);
            else launch_prefill_hpw<64, 4>(a, p, hpw, grid);
            break;
        case 256:
            if (b16) launch_prefill_hpw<256, 16>(a, p, hpw, grid);
            else launch_prefill_hpw<256, 4>(a, p, hpw, grid);
            break;
        default:
            if (b16) launch_prefill_hpw<16, 16>(a, p, hpw, grid);
            else launch_prefill_hpw<16, 4>(a, p, hpw, grid);
            break;
    }
    return hipGetLastError();
}

}  // namespace kvc
