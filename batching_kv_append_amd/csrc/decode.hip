// Work planning and the split-K decode path.
//
// Decode rows (one new token) dominate a continuous-batching step: each one
// streams its whole cached K/V once, so the step is bound by memory traffic
// (klklkl10086.github.io kv_cache post, section on the decode bottleneck: the
// decode stage is limited by memory access; clvsit.github.io AWS SageMaker
// page: every step moves the parameters and the cache into the compute
// units).  The kernel therefore aims at HBM bandwidth:
//   * a sequence's context is cut into fixed partitions of DECODE_PART tokens
//     (split-K), so even a short batch of long contexts yields thousands of
//     independent work units; the partial softmax states are combined by an
//     exact log-sum-exp merge (an exact regrouping of the row-wise softmax of
//     the "Attention" section of the continuous-batching article);
//   * one wavefront per (sequence, partition, kv head, head chunk): the GW
//     query heads that share a kv head (GQA, e2hang/Notes "MQA与GQA") are
//     served from one read of K/V;
//   * 16 lanes own one 128-dim bf16 token row (16 B = 8 values each), so each
//     load instruction reads 4 whole rows = 1 KiB contiguous from one block
//     (the block table gives each 16-token block as one 4 KiB run per head);
//   * q.k partial dots are reduced across the 16 lanes with DPP row
//     operations; softmax is online per lane group, with one cross-group
//     merge per work unit.
// The planning kernel lists the work units on the device, so the host needs no
// copy of the lengths; each wave takes one unit, and the hardware dispatcher
// hands the next workgroup to whichever compute unit frees up first.
#include <hip/hip_runtime.h>

#include "kvc_launch.h"

namespace kvc {

namespace {

// ---------------------------------------------------------------------------
// Plan: classify sequences and write the work lists.
// ---------------------------------------------------------------------------
constexpr int PLAN_THREADS = 1024;

__global__ __launch_bounds__(PLAN_THREADS) void plan_kernel(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ ctx, int32_t num_seqs,
    int32_t total_q, int32_t max_q_len, int32_t max_context_len, int32_t span, int64_t cap_dec,
    int64_t cap_pre, int32_t* hdr, int32_t* dec_base, int2* dec_items, int2* pre_items,
    int32_t* merge_list) {
    __shared__ int sc[3][PLAN_THREADS];
    __shared__ int carry[3];
    __shared__ int flags;
    const int tid = threadIdx.x;
    if (tid == 0) {
        carry[0] = carry[1] = carry[2] = 0;
        flags = 0;
        hdr[HDR_FLAGS] = 0;
    }
    __syncthreads();
    for (int base = 0; base < num_seqs; base += PLAN_THREADS) {
        const int s = base + tid;
        int nd = 0, np = 0, nm = 0, q = 0;
        if (s < num_seqs) {
            const int r0 = cu[s], r1 = cu[s + 1];
            const int c = ctx[s];
            q = r1 - r0;
            // A sequence whose rows are not inside [0, total_q) or whose
            // lengths break the host bounds is skipped (and flagged): no
            // later kernel touches its rows, so garbage lengths can never
            // move an access out of bounds.
            if (r0 < 0 || r1 < r0 || r1 > total_q || c < 0) {
                atomicOr(&flags, FLAG_CU_SEQLENS);
                q = 0;
            } else if (c > max_context_len || q > max_q_len) {
                atomicOr(&flags, FLAG_CAPACITY);
                q = 0;
            }
            if (q == 1) {
                nd = (c + 1 + DECODE_PART - 1) / DECODE_PART;
                nm = nd > 1;
            } else if (q >= 2) {
                np = (q + span - 1) / span;
            }
        }
        sc[0][tid] = nd;
        sc[1][tid] = np;
        sc[2][tid] = nm;
        __syncthreads();
        // inclusive Hillis-Steele scan of the three counts
        for (int off = 1; off < PLAN_THREADS; off <<= 1) {
            int a0 = 0, a1 = 0, a2 = 0;
            if (tid >= off) {
                a0 = sc[0][tid - off];
                a1 = sc[1][tid - off];
                a2 = sc[2][tid - off];
            }
            __syncthreads();
            sc[0][tid] += a0;
            sc[1][tid] += a1;
            sc[2][tid] += a2;
            __syncthreads();
        }
        const int od = carry[0] + sc[0][tid] - nd;
        const int op = carry[1] + sc[1][tid] - np;
        const int om = carry[2] + sc[2][tid] - nm;
        if (s < num_seqs) {
            dec_base[s] = q == 1 ? od : -1;
            for (int j = 0; j < nd; ++j) {
                if (od + j < cap_dec) dec_items[od + j] = make_int2(s, j);
                else atomicOr(&flags, FLAG_CAPACITY);
            }
            // heavier (later) position tiles first
            for (int j = 0; j < np; ++j) {
                if (op + j < cap_pre) pre_items[op + j] = make_int2(s, np - 1 - j);
                else atomicOr(&flags, FLAG_CAPACITY);
            }
            if (nm) merge_list[om] = s;
        }
        __syncthreads();
        if (tid == PLAN_THREADS - 1) {
            carry[0] += sc[0][tid];
            carry[1] += sc[1][tid];
            carry[2] += sc[2][tid];
        }
        __syncthreads();
    }
    if (tid == 0) {
        if (cu[0] != 0 || cu[num_seqs] != total_q) flags |= FLAG_CU_SEQLENS;
        hdr[HDR_N_DEC] = (int)min((int64_t)carry[0], cap_dec);
        hdr[HDR_N_PRE] = (int)min((int64_t)carry[1], cap_pre);
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
    int64_t num_blocks;
    int32_t max_blocks, hq, hkv, G, HC;
    float scale_log2;  // scale * log2(e): scores live in the exp2 domain
};

constexpr float NEG_BIG = -1.0e30f;  // "no key yet": finite, so exp2(NEG_BIG - m) == 0

template <int A, int BS, int GW>
__global__ __launch_bounds__(256) void decode_kernel(DecodeParams P) {
    constexpr int LPR = A / 8;      // lanes per token row (16 B per lane)
    constexpr int RPL = 64 / LPR;   // token rows per load instruction
    constexpr int NL = (A == 128) ? 8 : 2;  // loads per chunk
    constexpr int CH = RPL * NL;    // tokens per chunk
    constexpr int NT = DECODE_PART / BS;  // table entries per partition (<= 64)
    constexpr bool UNIFORM_BLOCK = (BS % RPL) == 0;  // one block per load instruction
    static_assert(DECODE_PART % CH == 0, "chunk must divide the partition");
    static_assert(NT <= 64, "table slice must fit one VGPR");

    const int lane = threadIdx.x & 63;
    const int r = lane / LPR;
    const int c8 = lane % LPR;
    const int64_t n_units = (int64_t)P.hdr[HDR_N_DEC] * P.hkv * P.HC;
    // One wave per work unit; the grid covers the host-side upper bound and
    // waves past the planned count leave at once.  The unit index comes from
    // the launch coordinates only, so it is uniform by construction.
    const int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (u >= n_units) return;
    {
        const int hc = u % P.HC;
        const int kvh = (u / P.HC) % P.hkv;
        const int item = u / (P.HC * P.hkv);
        const int2 it = P.items[item];
        const int s = it.x, part = it.y;
        const int L = P.ctx[s] + 1;
        const int row = P.cu[s];
        const int nparts = (L + DECODE_PART - 1) / DECODE_PART;
        const int t0 = part * DECODE_PART;
        const int t1 = min(L, t0 + DECODE_PART);
        const int h0 = kvh * P.G + hc * GW;

        // table slice of this partition: lane i holds entry (t0 / BS + i)
        const int lb0 = t0 / BS;
        const int nlb = (t1 - t0 + BS - 1) / BS;
        int tbl = -1;
        if (lane < nlb && lane < NT) {
            const int64_t lb = lb0 + lane;
            if (lb < P.max_blocks) tbl = P.table[(int64_t)s * P.max_blocks + lb];
        }

        // q for GW heads, pre-scaled into the exp2 domain
        float qf[GW][8];
#pragma unroll
        for (int g = 0; g < GW; ++g) {
            const uint4 qq = *reinterpret_cast<const uint4*>(
                P.q + (((int64_t)row * P.hq + h0 + g) * A + c8 * 8));
            const uint32_t w[4] = {qq.x, qq.y, qq.z, qq.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                qf[g][2 * e] = bf_lo(w[e]) * P.scale_log2;
                qf[g][2 * e + 1] = bf_hi(w[e]) * P.scale_log2;
            }
        }
        float m[GW], l[GW], acc[GW][8];
#pragma unroll
        for (int g = 0; g < GW; ++g) {
            m[g] = NEG_BIG;
            l[g] = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
        }
        int bad = 0;

        for (int tc = t0; tc < t1; tc += CH) {
            uint4 kr[NL], vr[NL];
            bool ok[NL];
#pragma unroll
            for (int j = 0; j < NL; ++j) {
                const int t = tc + j * RPL + r;
                int blk;
                if constexpr (UNIFORM_BLOCK) {
                    blk = __builtin_amdgcn_readlane(tbl, ((tc + j * RPL) / BS - lb0));
                } else {
                    blk = __shfl(tbl, (t / BS - lb0) & 63, 64);
                }
                const bool in_range = blk >= 0 && blk < P.num_blocks;
                ok[j] = (t < t1) && in_range;
                bad |= (t < t1) && !in_range;
                kr[j] = make_uint4(0, 0, 0, 0);
                vr[j] = make_uint4(0, 0, 0, 0);
                if (ok[j]) {
                    const int64_t off =
                        (((int64_t)blk * P.hkv + kvh) * BS + (t % BS)) * LPR + c8;
                    kr[j] = P.k_cache[off];
                    vr[j] = P.v_cache[off];
                }
            }
            float sc[NL][GW];
#pragma unroll
            for (int j = 0; j < NL; ++j) {
                const uint32_t w[4] = {kr[j].x, kr[j].y, kr[j].z, kr[j].w};
                float kf[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kf[2 * e] = bf_lo(w[e]);
                    kf[2 * e + 1] = bf_hi(w[e]);
                }
#pragma unroll
                for (int g = 0; g < GW; ++g) {
                    float d = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) d = fmaf(qf[g][e], kf[e], d);
                    d = group_sum<LPR>(d);
                    sc[j][g] = ok[j] ? d : -INFINITY;
                }
            }
#pragma unroll
            for (int g = 0; g < GW; ++g) {
                float mx = sc[0][g];
#pragma unroll
                for (int j = 1; j < NL; ++j) mx = fmaxf(mx, sc[j][g]);
                const float m_new = fmaxf(m[g], mx);
                const float alpha = __builtin_amdgcn_exp2f(m[g] - m_new);
                l[g] *= alpha;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[g][e] *= alpha;
                m[g] = m_new;
            }
#pragma unroll
            for (int j = 0; j < NL; ++j) {
                const uint32_t w[4] = {vr[j].x, vr[j].y, vr[j].z, vr[j].w};
                float vf[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    vf[2 * e] = bf_lo(w[e]);
                    vf[2 * e + 1] = bf_hi(w[e]);
                }
#pragma unroll
                for (int g = 0; g < GW; ++g) {
                    const float p = __builtin_amdgcn_exp2f(sc[j][g] - m[g]);
                    l[g] += p;
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(p, vf[e], acc[g][e]);
                }
            }
        }
        if (bad && lane == 0) set_flag(P.hdr, FLAG_BAD_BLOCK);

        // merge the RPL row groups of the wave (lanes c8, c8+LPR, ...)
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
            for (int g = 0; g < GW; ++g) {
                const float m2 = shfl_xor_f(m[g], off);
                const float l2 = shfl_xor_f(l[g], off);
                const float M = fmaxf(m[g], m2);
                const float a1 = __builtin_amdgcn_exp2f(m[g] - M);
                const float a2 = __builtin_amdgcn_exp2f(m2 - M);
                l[g] = l[g] * a1 + l2 * a2;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc[g][e] = acc[g][e] * a1 + shfl_xor_f(acc[g][e], off) * a2;
                m[g] = M;
            }
        }

        if (lane < LPR) {
            if (nparts == 1) {
#pragma unroll
                for (int g = 0; g < GW; ++g) {
                    const float inv = 1.f / l[g];
                    uint4 o;
                    o.x = pack_bf16x2(acc[g][0] * inv, acc[g][1] * inv);
                    o.y = pack_bf16x2(acc[g][2] * inv, acc[g][3] * inv);
                    o.z = pack_bf16x2(acc[g][4] * inv, acc[g][5] * inv);
                    o.w = pack_bf16x2(acc[g][6] * inv, acc[g][7] * inv);
                    *reinterpret_cast<uint4*>(P.out + (((int64_t)row * P.hq + h0 + g) * A + c8 * 8)) = o;
                }
            } else {
#pragma unroll
                for (int g = 0; g < GW; ++g) {
                    const int64_t slot = (int64_t)item * P.hq + h0 + g;
                    float4* dst = reinterpret_cast<float4*>(P.ws_acc + slot * A + c8 * 8);
                    dst[0] = make_float4(acc[g][0], acc[g][1], acc[g][2], acc[g][3]);
                    dst[1] = make_float4(acc[g][4], acc[g][5], acc[g][6], acc[g][7]);
                    if (lane == 0) {
                        P.ws_ml[slot * 2] = m[g];
                        P.ws_ml[slot * 2 + 1] = l[g];
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Merge kernel: one wave per (multi-partition decode sequence, query head).
//   M = max_p m_p;  out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p
// ---------------------------------------------------------------------------
struct MergeParams {
    uint16_t* out;
    const int32_t* cu;
    const int32_t* ctx;
    const int32_t* hdr;
    const int32_t* merge_list;
    const int32_t* dec_base;
    const float* ws_ml;
    const float* ws_acc;
    int64_t cap_dec;
    int32_t hq, A;
};

template <int A>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams P) {
    constexpr int DPL = A >= 64 ? A / 64 : 1;  // dims per lane
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    if ((int)blockIdx.x >= P.hdr[HDR_N_MERGE]) return;
    const int h = blockIdx.y * 4 + wave;
    if (h >= P.hq) return;
    const int s = P.merge_list[blockIdx.x];
    const int L = P.ctx[s] + 1;
    const int np = (L + DECODE_PART - 1) / DECODE_PART;
    const int64_t base = P.dec_base[s];
    if (base < 0 || base + np > P.cap_dec) return;  // never true for a planned sequence
    float M = NEG_BIG;
    for (int p = 0; p < np; ++p) M = fmaxf(M, P.ws_ml[((base + p) * P.hq + h) * 2]);
    float den = 0.f, num[DPL];
#pragma unroll
    for (int i = 0; i < DPL; ++i) num[i] = 0.f;
    const int d0 = lane * DPL;
    for (int p = 0; p < np; ++p) {
        const int64_t slot = (base + p) * P.hq + h;
        const float w = __builtin_amdgcn_exp2f(P.ws_ml[slot * 2] - M);
        den = fmaf(w, P.ws_ml[slot * 2 + 1], den);
        if (d0 < A) {
#pragma unroll
            for (int i = 0; i < DPL; ++i) num[i] = fmaf(w, P.ws_acc[slot * A + d0 + i], num[i]);
        }
    }
    if (d0 < A) {
        const float inv = 1.f / den;
        uint16_t* o = P.out + ((int64_t)P.cu[s] * P.hq + h) * A + d0;
        if constexpr (DPL == 2) {
            *reinterpret_cast<uint32_t*>(o) = pack_bf16x2(num[0] * inv, num[1] * inv);
        } else {
#pragma unroll
            for (int i = 0; i < DPL; ++i)
                o[i] = (uint16_t)(pack_bf16x2(num[i] * inv, 0.f) & 0xffffu);
        }
    }
}

template <int A, int BS, int GW>
void launch_decode_t(const StepArgs& a, const DecodeParams& p, int grid) {
    hipLaunchKernelGGL((decode_kernel<A, BS, GW>), dim3(grid), dim3(256), 0, a.stream, p);
}

template <int A, int BS>
void launch_decode_gw(const StepArgs& a, const DecodeParams& p, int GW, int grid) {
    switch (GW) {
        case 1: launch_decode_t<A, BS, 1>(a, p, grid); break;
        case 2: launch_decode_t<A, BS, 2>(a, p, grid); break;
        case 4: launch_decode_t<A, BS, 4>(a, p, grid); break;
        default: launch_decode_t<A, BS, 8>(a, p, grid); break;
    }
}

}  // namespace

int decode_heads_per_wave(int G) {
    return (G % 8 == 0) ? 8 : (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
}

hipError_t launch_plan(const StepArgs& a) {
    char* ws = a.ws;
    const int G = a.num_q_heads / a.num_kv_heads;
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(PLAN_THREADS), 0, a.stream, a.cu_seqlens_q,
                       a.context_lens, a.num_seqs, a.total_q, a.max_q_len, a.max_context_len,
                       prefill_span(G), a.lay.cap_dec, a.lay.cap_pre,
                       (int32_t*)(ws + a.lay.hdr), (int32_t*)(ws + a.lay.dec_base),
                       (int2*)(ws + a.lay.dec_items), (int2*)(ws + a.lay.pre_items),
                       (int32_t*)(ws + a.lay.merge_list));
    return hipGetLastError();
}

hipError_t launch_decode(const StepArgs& a) {
    char* ws = a.ws;
    const int G = a.num_q_heads / a.num_kv_heads;
    const int GW = decode_heads_per_wave(G);
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
    p.num_blocks = a.num_blocks;
    p.max_blocks = a.max_blocks;
    p.hq = a.num_q_heads;
    p.hkv = a.num_kv_heads;
    p.G = G;
    p.HC = G / GW;
    p.scale_log2 = a.scale * 1.4426950408889634f;
    // One wave per unit over the upper bound of units (4 waves per workgroup).
    const int64_t units = a.lay.cap_dec * a.num_kv_heads * p.HC;
    const int64_t grid64 = (units + 3) / 4;
    if (grid64 <= 0) return hipSuccess;
    if (grid64 > INT32_MAX) return hipErrorInvalidValue;
    const int grid = (int)grid64;
    if (a.head_dim == 128) {
        if (a.block_size == 16) launch_decode_gw<128, 16>(a, p, GW, grid);
        else launch_decode_gw<128, 4>(a, p, GW, grid);
    } else {
        if (a.block_size == 16) launch_decode_gw<16, 16>(a, p, GW, grid);
        else launch_decode_gw<16, 4>(a, p, GW, grid);
    }
    return hipGetLastError();
}

hipError_t launch_merge(const StepArgs& a) {
    char* ws = a.ws;
    MergeParams mp;
    mp.out = (uint16_t*)a.out;
    mp.cu = a.cu_seqlens_q;
    mp.ctx = a.context_lens;
    mp.hdr = (const int32_t*)(ws + a.lay.hdr);
    mp.merge_list = (const int32_t*)(ws + a.lay.merge_list);
    mp.dec_base = (const int32_t*)(ws + a.lay.dec_base);
    mp.ws_ml = (const float*)(ws + a.lay.ml);
    mp.ws_acc = (const float*)(ws + a.lay.acc);
    mp.cap_dec = a.lay.cap_dec;
    mp.hq = a.num_q_heads;
    mp.A = a.head_dim;
    dim3 mgrid((unsigned)a.num_seqs, (unsigned)((a.num_q_heads + 3) / 4));
    if (a.head_dim == 128)
        hipLaunchKernelGGL(merge_kernel<128>, mgrid, dim3(256), 0, a.stream, mp);
    else
        hipLaunchKernelGGL(merge_kernel<16>, mgrid, dim3(256), 0, a.stream, mp);
    return hipGetLastError();
}

}  // namespace kvc
