/*
 * CPU oracle for one ragged paged-attention step — TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  The product library never links, loads or calls it,
 * and it includes nothing from the product sources: it is a slow, plain,
 * obviously-correct statement of what the step computes, in fp64.
 *
 * Sources (the four pages on KV caches and continuous batching):
 *   [myit]  news.myit.tw/news/j9529p, the translated "continuous batching from
 *           first principles" article — sections "Attention", "KV cache",
 *           "Chunked prefill", "Continuous batching".
 *   [aws]   clvsit.github.io "AWS SageMaker 推理方案" — section
 *           "PagedAttention 批处理".
 *   [notes] e2hang/Notes "KV Cache与Continuous Batching" — sections
 *           "KV Cache内存占用" and "MQA与GQA".
 *   [kvpost] klklkl10086.github.io kv_cache post — sections "Paged Attention"
 *           and "Batch Decode".
 *
 * Conventions (readings of points the pages leave open):
 *   - bf16 values are passed as their raw 16-bit patterns; widening bf16 to
 *     fp64 is exact, so every product below is formed in fp64 from exact
 *     inputs and no intermediate is rounded to a narrower type.
 *   - context_lens[s] is the number of tokens of sequence s cached BEFORE the
 *     step; the step appends q_len_s = cu[s+1]-cu[s] new tokens at positions
 *     context_lens[s] .. context_lens[s]+q_len_s-1.
 *   - Token position p of a sequence lives in logical block p / block_size at
 *     slot p % block_size; the block table maps the logical block to the
 *     physical block ([aws] "PagedAttention 批处理": the table maps logical to
 *     physical blocks; [kvpost] "Paged Attention": the table maps a block's
 *     logical number to its real storage address).
 *   - Pool layout: [num_blocks][num_kv_heads][block_size][head_dim].
 *   - Query head h reads kv head h / (Hq/Hkv) (contiguous groups; [notes]
 *     "MQA与GQA" fixes only num_kv_heads = num_q_heads / ratio).
 *   - Row i of sequence s sees keys 0 .. context_lens[s]+i inclusive: the
 *     causal mask of [myit] "Attention" (token j may influence token i iff
 *     j <= i), shifted by the cached length as in [myit] "Chunked prefill".
 *
 * Every function here is pinned by tests/test_oracle_pins.py against
 * properties the pages and the mathematics fix (library special cases,
 * closed forms, the chunking/decode/permutation/ragged/GQA invariants, and
 * the pages' cache-size numbers); tests/test_oracle_mutants.py rebuilds this
 * file with planted mistakes (KVCO_MUTANT=n) and checks that a pin fails.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef KVCO_MUTANT
#define KVCO_MUTANT 0
#endif

static double bf16_bits_to_f64(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16; /* bf16 is the top half of an fp32 */
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Physical block and slot of token position p of sequence s. */
static int locate(const int32_t* block_table, int32_t max_blocks, int32_t s,
                  int64_t p, int32_t block_size, int64_t num_blocks,
                  int64_t* blk, int64_t* slot) {
    int64_t lb = p / block_size;
    if (lb >= max_blocks) return -1;
#if KVCO_MUTANT == 10
    *blk = lb; /* planted: ignores the block table */
#else
    *blk = block_table[(int64_t)s * max_blocks + lb];
#endif
#if KVCO_MUTANT == 4
    *slot = block_size - 1 - p % block_size; /* planted: wrong slot index */
#else
    *slot = p % block_size;
#endif
    if (*blk < 0 || *blk >= num_blocks) return -1;
    return 0;
}

/* Bytes of K and V one token occupies across all layers:
 * 2 (K and V) * layers * kv heads * head_dim * element bytes.
 * [myit] "KV cache" gives the per-token size as 2*L*H*A values; [notes]
 * "KV Cache内存占用" gives the same product times bytes per value. */
int64_t kvco_kv_bytes_per_token(int32_t num_layers, int32_t num_kv_heads,
                                int32_t head_dim, int32_t elem_bytes) {
    return 2 * (int64_t)num_layers * num_kv_heads * head_dim * elem_bytes;
}

/* Step 1 — append ([aws] "PagedAttention 批处理": prefill stores K/V in
 * non-contiguous blocks recorded in the table; [kvpost] "Batch Decode": the new
 * token's K/V joins the cache, a block write under paging).  Pure bit copy of
 * k_new/v_new [Tq][Hkv][A] into the pools at positions c_s + i.
 * Returns 0, or -1 if a position falls outside the table or a block id is out
 * of range (nothing after that token is written). */
int kvco_append(uint16_t* k_pool, uint16_t* v_pool, int64_t num_blocks,
                const uint16_t* k_new, const uint16_t* v_new,
                const int32_t* block_table, int32_t max_blocks,
                const int32_t* cu_seqlens_q, const int32_t* context_lens,
                int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim,
                int32_t block_size) {
    for (int32_t s = 0; s < num_seqs; ++s) {
        int32_t n = cu_seqlens_q[s + 1] - cu_seqlens_q[s];
        for (int32_t i = 0; i < n; ++i) {
#if KVCO_MUTANT == 5
            int64_t p = (int64_t)context_lens[s] + i + 1; /* planted: off by one */
#else
            int64_t p = (int64_t)context_lens[s] + i;
#endif
            int64_t blk, slot;
            if (locate(block_table, max_blocks, s, p, block_size, num_blocks,
                       &blk, &slot))
                return -1;
            int64_t row = (int64_t)cu_seqlens_q[s] + i;
            for (int32_t g = 0; g < num_kv_heads; ++g) {
                int64_t dst = ((blk * num_kv_heads + g) * block_size + slot) * head_dim;
                int64_t src = (row * num_kv_heads + g) * head_dim;
                for (int32_t a = 0; a < head_dim; ++a) {
                    k_pool[dst + a] = k_new[src + a];
                    v_pool[dst + a] = v_new[src + a];
                }
            }
        }
    }
    return 0;
}

/* Step 2 — gather: rebuild the contiguous cache of every sequence from the
 * pool through its table ([kvpost] "Paged Attention": logically contiguous,
 * physically scattered).  Output [sum L][Hkv][A] as raw bf16 bits, sequences
 * back to back at offsets cu_seq_lens[s].  Returns 0 or -1 as kvco_append. */
int kvco_gather(const uint16_t* k_pool, const uint16_t* v_pool, int64_t num_blocks,
                const int32_t* block_table, int32_t max_blocks,
                const int32_t* seq_lens, const int64_t* cu_seq_lens,
                uint16_t* k_out, uint16_t* v_out, int32_t num_seqs,
                int32_t num_kv_heads, int32_t head_dim, int32_t block_size) {
    for (int32_t s = 0; s < num_seqs; ++s) {
        for (int64_t p = 0; p < seq_lens[s]; ++p) {
            int64_t blk, slot;
            if (locate(block_table, max_blocks, s, p, block_size, num_blocks,
                       &blk, &slot))
                return -1;
            for (int32_t g = 0; g < num_kv_heads; ++g) {
                int64_t src = ((blk * num_kv_heads + g) * block_size + slot) * head_dim;
                int64_t dst = ((cu_seq_lens[s] + p) * num_kv_heads + g) * head_dim;
                memcpy(k_out + dst, k_pool + src, (size_t)head_dim * 2);
                memcpy(v_out + dst, v_pool + src, (size_t)head_dim * 2);
            }
        }
    }
    return 0;
}

/* Step 3 — attend, in fp64, over the pools AFTER the append.
 *
 * For every sequence s, new row i < q_len_s and query head h
 * ([myit] "Attention": scores QK^T, boolean mask, row-wise softmax, times V;
 *  [myit] "Chunked prefill": the cached K/V are prepended and the mask shifted;
 *  [myit] "Continuous batching": sequences concatenated without a batch
 *  dimension, each seeing only its own keys;
 *  [kvpost] "Batch Decode": scores scaled by 1/sqrt(head_dim) before softmax,
 *  here the explicit `scale`):
 *     g  = h / (Hq / Hkv)
 *     z_j = scale * sum_a q[row, h, a] * K_s[j, g, a]     for j = 0 .. c_s + i
 *     M  = max_j z_j,   w_j = exp(z_j - M)
 *     out[row, h, :] = sum_j w_j V_s[j, g, :] / sum_j w_j
 * Masked keys are excluded from the sums (never added as -inf).  The softmax is
 * the plain two-pass form: first every z_j and their maximum, then the
 * weights; no running rescale.
 *
 * row_select: NULL, or a [Tq] byte mask — rows with 0 are skipped and their
 * output is left untouched (for sampled checks of very large steps).
 * nthreads: OpenMP threads (<= 0: the OpenMP default).
 * Returns the number of threads used, or -1 on a table/shape error. */
int kvco_attention(double* out, const uint8_t* row_select, const uint16_t* q,
                   const uint16_t* k_pool, const uint16_t* v_pool, int64_t num_blocks,
                   const int32_t* block_table, int32_t max_blocks,
                   const int32_t* cu_seqlens_q, const int32_t* context_lens,
                   int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                   int32_t head_dim, int32_t block_size, double scale, int nthreads) {
    if (num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return -1;
    if (head_dim <= 0 || head_dim > 1024) return -1;
    const int32_t group = num_q_heads / num_kv_heads;
    int used = 1;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
    {
#pragma omp single
        used = omp_get_num_threads();
    }
#else
    nthreads = 1;
#endif
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int32_t n = cu_seqlens_q[s + 1] - cu_seqlens_q[s];
        if (n <= 0) continue;
        const int64_t c = context_lens[s];
        const int64_t L = c + n;
        /* does any selected row belong to this sequence? */
        int any = 0;
        for (int32_t i = 0; i < n && !any; ++i)
            any = row_select == NULL || row_select[cu_seqlens_q[s] + i];
        if (!any) continue;
        /* Rebuild this sequence's contiguous K and V in fp64. */
        double* K = (double*)malloc(sizeof(double) * (size_t)(L * num_kv_heads * head_dim));
        double* V = (double*)malloc(sizeof(double) * (size_t)(L * num_kv_heads * head_dim));
        if (!K || !V) { free(K); free(V); return -1; }
        int bad = 0;
        for (int64_t p = 0; p < L && !bad; ++p) {
            int64_t blk, slot;
            if (locate(block_table, max_blocks, s, p, block_size, num_blocks, &blk, &slot)) {
                bad = 1;
                break;
            }
            for (int32_t g = 0; g < num_kv_heads; ++g) {
                int64_t src = ((blk * num_kv_heads + g) * block_size + slot) * head_dim;
                int64_t dst = (p * num_kv_heads + g) * head_dim;
                for (int32_t a = 0; a < head_dim; ++a) {
                    K[dst + a] = bf16_bits_to_f64(k_pool[src + a]);
                    V[dst + a] = bf16_bits_to_f64(v_pool[src + a]);
                }
            }
        }
        if (bad) { free(K); free(V); return -1; }
        const int64_t tasks = (int64_t)n * num_q_heads;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
        for (int64_t t = 0; t < tasks; ++t) {
            const int32_t i = (int32_t)(t / num_q_heads);
            const int32_t h = (int32_t)(t % num_q_heads);
            const int64_t row = (int64_t)cu_seqlens_q[s] + i;
#if KVCO_MUTANT == 9
            const int64_t qrow = i; /* planted: ignores the row offset of s */
#else
            const int64_t qrow = row;
#endif
            if (row_select != NULL && !row_select[row]) continue;
#if KVCO_MUTANT == 3
            const int32_t g = h % num_kv_heads; /* planted: wrong group map */
#else
            const int32_t g = h / group;
#endif
#if KVCO_MUTANT == 1
            const int64_t nvis = c + i; /* planted: own key excluded */
#elif KVCO_MUTANT == 8
            const int64_t nvis = (int64_t)i + 1; /* planted: cache offset ignored */
#else
            const int64_t nvis = c + i + 1;
#endif
            double* z = (double*)malloc(sizeof(double) * (size_t)(nvis > 0 ? nvis : 1));
            double qv[1024];
            for (int32_t a = 0; a < head_dim; ++a)
                qv[a] = bf16_bits_to_f64(q[(qrow * num_q_heads + h) * head_dim + a]);
            /* pass 1: scores and their maximum */
            double M = -INFINITY;
            for (int64_t j = 0; j < nvis; ++j) {
                const double* kj = K + (j * num_kv_heads + g) * head_dim;
                double dot = 0.0;
                for (int32_t a = 0; a < head_dim; ++a) dot += qv[a] * kj[a];
#if KVCO_MUTANT == 2
                z[j] = dot; /* planted: scale dropped */
                (void)scale;
#else
                z[j] = scale * dot;
#endif
                if (z[j] > M) M = z[j];
            }
            /* pass 2: weights, weighted sum of values, normaliser */
            double* o = out + (row * num_q_heads + h) * head_dim;
            for (int32_t a = 0; a < head_dim; ++a) o[a] = 0.0;
            double den = 0.0;
            for (int64_t j = 0; j < nvis; ++j) {
                const double w = exp(z[j] - M);
#if KVCO_MUTANT == 6
                const double* vj = K + (j * num_kv_heads + g) * head_dim; /* planted: K for V */
#else
                const double* vj = V + (j * num_kv_heads + g) * head_dim;
#endif
                for (int32_t a = 0; a < head_dim; ++a) o[a] += w * vj[a];
                den += w;
            }
#if KVCO_MUTANT == 7
            (void)den; /* planted: normaliser dropped */
#else
            for (int32_t a = 0; a < head_dim; ++a) o[a] /= den;
#endif
            free(z);
        }
        free(K);
        free(V);
    }
    return used;
}
