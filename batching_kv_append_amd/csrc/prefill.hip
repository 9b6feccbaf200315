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
// to agree between P^T and V^T, which reads its keys with the same order), so
// P never leaves the registers.  Softmax statistics are per lane (one column)
// with one exchange with lane^32 per 64-key tile.
//
// Work: one workgroup = 4 waves = HPW query heads of one kv group x (4/HPW)
// blocks of PREFILL_QW = 64 positions; each wave owns one (head, 64
// positions) and two 32-column MFMA tiles.  K/V tiles of 64 keys (four 16-token
// blocks, gathered through the block table) are staged in LDS once per
// workgroup and shared by the HPW heads of the group (GQA, e2hang/Notes
// "MQA与GQA").  K is stored row-major with a 16-byte XOR swizzle; V is stored
// transposed ([dim][key]) with an 8-byte XOR swizzle, so both operand reads
// are bank-conflict free.
#include <hip/hip_runtime.h>

#include "kvc_launch.h"

namespace kvc {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct PrefillParams {
    const uint16_t* q;
    uint16_t* out;
    const uint4* k_cache;
    const uint4* v_cache;
    const int32_t* table;
    const int32_t* cu;
    const int32_t* ctx;
    const int32_t* hdr;
    const int2* items;
    int64_t num_blocks;
    int32_t max_blocks, hq, hkv, G, HC;
    float scale_log2;
};

__device__ __forceinline__ f32x16_t mfma32(uint4 a, uint4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <int A, int BS, int HPW>
__global__ __launch_bounds__(256, 1) void prefill_kernel(PrefillParams P) {
    constexpr int TK = PREFILL_TK;         // keys per tile
    constexpr int CPR = A / 8;             // 16-byte chunks per K/V row
    constexpr int NCH = TK * CPR;          // chunks per tile
    constexpr int CPT = (NCH + 255) / 256; // chunks per thread
    constexpr int KK = A / 16;             // 16-dim MFMA steps of QK^T
    constexpr int DT = (A + 31) / 32;      // 32-dim output tiles
    constexpr int SPAN = PREFILL_QW * (4 / HPW);
    constexpr float NEG_BIG = -1.0e30f;

    __shared__ uint4 sK[TK * CPR];          // [key][chunk ^ (key % CPR)]
    __shared__ uint2 sVt[A * (TK / 4)];     // [dim][keygroup ^ ((dim >> 1) & 15)], 4 keys per uint2

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int hi = lane >> 5;   // which half of the wave
    const int col = lane & 31;  // query column inside a 32-wide tile

    if ((int)blockIdx.x >= P.hdr[HDR_N_PRE]) return;
    const int2 it = P.items[blockIdx.x];
    const int s = it.x, tile = it.y;
    const int kvh = blockIdx.y / P.HC;
    const int hc = blockIdx.y % P.HC;
    const int h = kvh * P.G + hc * HPW + (wave % HPW);
    const int row0 = P.cu[s];
    const int qlen = P.cu[s + 1] - row0;
    const int c = P.ctx[s];
    const int L = c + qlen;
    const int p0 = tile * SPAN + (wave / HPW) * PREFILL_QW;  // first position of this wave
    const int wg_last = min(tile * SPAN + SPAN, qlen) - 1;     // last position of the workgroup
    const int kend = c + wg_last + 1;                          // keys the workgroup needs
    const int nkt = (kend + TK - 1) / TK;
    const int w_last = min(p0 + PREFILL_QW, qlen) - 1;         // last position of this wave
    const int kend_w = (p0 < qlen) ? c + w_last + 1 : 0;

    // ---- Q^T operand: two 32-column tiles, KK 16-dim steps ----------------
    uint4 qreg[2][KK];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        const int pos = p0 + qt * 32 + col;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            qreg[qt][kk] = make_uint4(0, 0, 0, 0);
            if (pos < qlen)
                qreg[qt][kk] = *reinterpret_cast<const uint4*>(
                    P.q + (((int64_t)(row0 + pos) * P.hq + h) * A + kk * 16 + hi * 8));
        }
    }

    f32x16_t o[2][DT];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[qt][dt][r] = 0.f;
    float m[2] = {NEG_BIG, NEG_BIG};
    float lsum[2] = {0.f, 0.f};

    // ---- cooperative tile loads (global -> registers) ---------------------
    uint4 kreg[CPT], vreg[CPT];
    int bad = 0;
    auto load_tile = [&](int k0) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int ci = tid + i * 256;
            kreg[i] = make_uint4(0, 0, 0, 0);
            vreg[i] = make_uint4(0, 0, 0, 0);
            if (ci < NCH) {
                const int key = ci / CPR, cc = ci % CPR;
                const int kidx = k0 + key;
                if (kidx < L) {
                    const int lb = kidx / BS;
                    int64_t blk = -1;
                    if (lb < P.max_blocks) blk = P.table[(int64_t)s * P.max_blocks + lb];
                    if (blk >= 0 && blk < P.num_blocks) {
                        const int64_t off = ((blk * P.hkv + kvh) * BS + kidx % BS) * CPR + cc;
                        kreg[i] = P.k_cache[off];
                        vreg[i] = P.v_cache[off];
                    } else {
                        bad = 1;
                    }
                }
            }
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int ci = tid + i * 256;
            if (ci < NCH) {
                const int key = ci / CPR, cc = ci % CPR;
                sK[key * CPR + (cc ^ (key % CPR))] = kreg[i];
                const uint32_t w[4] = {vreg[i].x, vreg[i].y, vreg[i].z, vreg[i].w};
                uint16_t* vt = reinterpret_cast<uint16_t*>(sVt);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int d = cc * 8 + e;
                    const int unit = (key >> 2) ^ ((d >> 1) & 15);
                    const uint16_t val = (uint16_t)((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xffffu));
                    vt[(d * (TK / 4) + unit) * 4 + (key & 3)] = val;
                }
            }
        }
    };

    if (nkt > 0) load_tile(0);
    for (int t = 0; t < nkt; ++t) {
        const int k0 = t * TK;
        __syncthreads();
        store_tile();
        __syncthreads();
        if (t + 1 < nkt) load_tile(k0 + TK);
        if (k0 >= kend_w) continue;  // this wave's rows see no key of the tile

        // ---- S^T = K Q^T : 2 key halves x 2 query tiles -----------------
        f32x16_t sacc[2][2];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[qt][kh][r] = 0.f;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            const int key = kh * 32 + col;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const int cc = kk * 2 + hi;
                const uint4 a = sK[key * CPR + (cc ^ (key % CPR))];
#pragma unroll
                for (int qt = 0; qt < 2; ++qt) sacc[qt][kh] = mfma32(a, qreg[qt][kk], sacc[qt][kh]);
            }
        }

        // ---- online softmax per query column ----------------------------
        const bool diag = k0 + TK - 1 > c + p0;  // some key of the tile may be masked
        uint4 pb[2][2][2];  // [qt][kh][ks] bf16 P^T operands
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            const int pos = p0 + qt * 32 + col;
            const int lim = c + pos;  // last visible key
            float mx = -INFINITY;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + kh * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                    float v = sacc[qt][kh][r] * P.scale_log2;
                    if (diag && key > lim) v = -INFINITY;
                    sacc[qt][kh][r] = v;
                    mx = fmaxf(mx, v);
                }
            mx = fmaxf(mx, shfl_xor_f(mx, 32));
            const float m_new = fmaxf(m[qt], mx);
            const float alpha = __builtin_amdgcn_exp2f(m[qt] - m_new);
            m[qt] = m_new;
            float ps = 0.f;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                float p[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    p[r] = __builtin_amdgcn_exp2f(sacc[qt][kh][r] - m_new);
                    ps += p[r];
                }
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    pb[qt][kh][ks].x = pack_bf16x2(p[ks * 8 + 0], p[ks * 8 + 1]);
                    pb[qt][kh][ks].y = pack_bf16x2(p[ks * 8 + 2], p[ks * 8 + 3]);
                    pb[qt][kh][ks].z = pack_bf16x2(p[ks * 8 + 4], p[ks * 8 + 5]);
                    pb[qt][kh][ks].w = pack_bf16x2(p[ks * 8 + 6], p[ks * 8 + 7]);
                }
            }
            lsum[qt] = lsum[qt] * alpha + ps;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[qt][dt][r] *= alpha;
        }

        // ---- O^T += V^T P^T ----------------------------------------------
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int d = dt * 32 + col;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    uint4 a = make_uint4(0, 0, 0, 0);
                    if (d < A) {
                        const int base = kh * 32 + ks * 16 + hi * 4;  // keys base..base+3, base+8..+11
                        const int sw = (d >> 1) & 15;
                        const uint2 lo = sVt[d * (TK / 4) + ((base >> 2) ^ sw)];
                        const uint2 hi2 = sVt[d * (TK / 4) + (((base + 8) >> 2) ^ sw)];
                        a = make_uint4(lo.x, lo.y, hi2.x, hi2.y);
                    }
#pragma unroll
                    for (int qt = 0; qt < 2; ++qt) o[qt][dt] = mfma32(a, pb[qt][kh][ks], o[qt][dt]);
                }
        }
    }
    if (bad) atomicOr(const_cast<int32_t*>(P.hdr) + HDR_FLAGS, FLAG_BAD_BLOCK);

    // ---- normalise and store ------------------------------------------------
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        const int pos = p0 + qt * 32 + col;
        const float lt = lsum[qt] + shfl_xor_f(lsum[qt], 32);
        if (pos >= qlen) continue;
        const float inv = 1.f / lt;
        uint16_t* orow = P.out + ((int64_t)(row0 + pos) * P.hq + h) * A;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int d = dt * 32 + 8 * rg + 4 * hi;
                if (d < A) {
                    uint2 v;
                    v.x = pack_bf16x2(o[qt][dt][rg * 4 + 0] * inv, o[qt][dt][rg * 4 + 1] * inv);
                    v.y = pack_bf16x2(o[qt][dt][rg * 4 + 2] * inv, o[qt][dt][rg * 4 + 3] * inv);
                    *reinterpret_cast<uint2*>(orow + d) = v;
                }
            }
    }
}

template <int A, int BS>
void launch_prefill_hpw(const StepArgs& a, const PrefillParams& p, int hpw, dim3 grid) {
    switch (hpw) {
        case 1: hipLaunchKernelGGL((prefill_kernel<A, BS, 1>), grid, dim3(256), 0, a.stream, p); break;
        case 2: hipLaunchKernelGGL((prefill_kernel<A, BS, 2>), grid, dim3(256), 0, a.stream, p); break;
        default: hipLaunchKernelGGL((prefill_kernel<A, BS, 4>), grid, dim3(256), 0, a.stream, p); break;
    }
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
    p.cu = a.cu_seqlens_q;
    p.ctx = a.context_lens;
    p.hdr = (const int32_t*)(ws + a.lay.hdr);
    p.items = (const int2*)(ws + a.lay.pre_items);
    p.num_blocks = a.num_blocks;
    p.max_blocks = a.max_blocks;
    p.hq = a.num_q_heads;
    p.hkv = a.num_kv_heads;
    p.G = G;
    p.HC = G / hpw;
    p.scale_log2 = a.scale * 1.4426950408889634f;
    const int64_t gx = a.lay.cap_pre;
    if (gx <= 0) return hipSuccess;
    dim3 grid((unsigned)gx, (unsigned)(a.num_kv_heads * p.HC));
    if (a.head_dim == 128) {
        if (a.block_size == 16) launch_prefill_hpw<128, 16>(a, p, hpw, grid);
        else launch_prefill_hpw<128, 4>(a, p, hpw, grid);
    } else {
        if (a.block_size == 16) launch_prefill_hpw<16, 16>(a, p, hpw, grid);
        else launch_prefill_hpw<16, 4>(a, p, hpw, grid);
    }
    return hipGetLastError();
}

}  // namespace kvc
