/*
 * pkv_oracle.c -- float64 CPU reference for paged-KV attention over one packed
 * engine step, and for the slot-mapped KV append.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link or call this
 * file: only the tests, the smoke check and the benchmark's CPU-baseline leg
 * use it.  It shares no code, header or constant with the HIP library.
 *
 * What it computes (plain definitions, written out slowly):
 *
 *  - Append.  The step's new key/value rows are written in place into a pool
 *    that was reserved once, addressed through a slot per token (slot =
 *    physical page * page_size + offset in page; a negative slot means "skip").
 *    Sources: vllm-metal v0.4.0 release post, "Set a predictable memory budget"
 *    (one pool reserved at startup serves every request) and "Replacing
 *    attention, reusing the rest" (keys and values stay in fixed-size pages,
 *    so a request grows by filling its pages, without reshaping a cache).
 *
 *  - Attention.  One engine step packs the query tokens of many sequences on one
 *    token axis, with query_start_loc (cu_seqlens) marking where each sequence's
 *    tokens start; each sequence's keys and values live in fixed-size pages that
 *    its block-table row locates.  Sources: vllm-metal v0.4.0 release post,
 *    "Replacing attention, reusing the rest" (packed query axis, paged KV,
 *    block tables; one launch covers prefill chunks and decode tokens) and
 *    "How vllm-metal fits into vLLM" (the runner gets a packed step plus block
 *    tables; chunked prefill shares a step with decodes).
 *
 *    For sequence s with L = seq_lens[s] keys (this step's tokens included),
 *    a = kv_start[s] leading masked keys (0 when kv_start is NULL) and
 *    n = query_start_loc[s+1] - query_start_loc[s] query tokens, query token i
 *    sits at absolute position p = L - n + i and sees keys a..p (a chunk is the
 *    same tokens a later decode would see: causal, aligned to the end).  Query
 *    head h reads kv head h / (Hq / Hkv).  Its output is the softmax-weighted
 *    mean of the visible values:
 *        l_j = scale * sum_d q[d] * K_j[d]
 *        out = sum_j exp(l_j - max l) * V_j / sum_j exp(l_j - max l)
 *    all in float64, summed in ascending index order.  The left-padded form
 *    (leading keys masked by kv_start) follows the vllm-ios README,
 *    "How it works" (uniform-offset batches, left padding) and "What this is
 *    and isn't" (padding masks on the roadmap).
 *
 * Element types: 0 = float32, 1 = bfloat16 (upper half of a float32).  Both
 * convert to double exactly.  The result is returned in float64; rounding to
 * the output dtype is left to the caller.
 *
 * Parallelism: OpenMP over (sequence, kv head) units.  Every output element is
 * produced by one thread in a fixed order, so the result does not depend on the
 * thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F32 0
#define ORC_BF16 1

#define ORC_OK 0
#define ORC_E_ARG -1
#define ORC_E_META -2
#define ORC_E_NOMEM -3

static double orc_elem(const void *base, int64_t idx, int dtype)
{
    if (dtype == ORC_F32)
        return (double)((const float *)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static size_t orc_esize(int dtype) { return dtype == ORC_F32 ? 4u : 2u; }

/* Byte copy of each new row into its slot.  pool layout:
 * [num_blocks][num_kv_heads][block_size][head_dim]; new rows [T][Hkv][D]. */
int oracle_append(void *k_pool, void *v_pool, const void *k_new, const void *v_new,
                  const int64_t *slot_mapping, int64_t num_tokens, int num_kv_heads,
                  int head_dim, int block_size, int64_t num_blocks, int dtype)
{
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        num_blocks < 0 || (dtype != ORC_F32 && dtype != ORC_BF16))
        return ORC_E_ARG;
    const size_t row = (size_t)head_dim * orc_esize(dtype);
    for (int64_t t = 0; t < num_tokens; ++t) {
        int64_t slot = slot_mapping[t];
        if (slot < 0)
            continue;
        int64_t blk = slot / block_size, off = slot % block_size;
        if (blk >= num_blocks)
            return ORC_E_META;
        for (int h = 0; h < num_kv_heads; ++h) {
            size_t dst = ((size_t)(blk * num_kv_heads + h) * block_size + (size_t)off) * row;
            size_t src = ((size_t)t * num_kv_heads + h) * row;
            memcpy((char *)k_pool + dst, (const char *)k_new + src, row);
            memcpy((char *)v_pool + dst, (const char *)v_new + src, row);
        }
    }
    return ORC_OK;
}

/* Checks that every index the attention loop will follow stays inside its
 * array.  Returns ORC_OK or ORC_E_META. */
static int orc_check(const int32_t *block_tables, const int32_t *seq_lens,
                     const int32_t *qsl, const int32_t *kv_start, int num_seqs,
                     int max_blocks_per_seq, int block_size, int64_t num_blocks)
{
    if (qsl[0] != 0)
        return ORC_E_META;
    for (int s = 0; s < num_seqs; ++s) {
        int64_t n = (int64_t)qsl[s + 1] - qsl[s];
        int64_t L = seq_lens[s];
        int64_t a = kv_start ? kv_start[s] : 0;
        if (n < 0 || L < 0 || a < 0 || a > L || n > L - a)
            return ORC_E_META;
        if (L == 0)
            continue;
        int64_t last_page = (L - 1) / block_size;
        if (last_page >= max_blocks_per_seq)
            return ORC_E_META;
        for (int64_t pg = a / block_size; pg <= last_page; ++pg) {
            int32_t b = block_tables[(int64_t)s * max_blocks_per_seq + pg];
            if (b < 0 || b >= num_blocks)
                return ORC_E_META;
        }
    }
    return ORC_OK;
}

/* out: [total_q][Hq][D] float64, total_q = query_start_loc[num_seqs]. */
int oracle_attention(double *out, const void *q, const void *k_pool, const void *v_pool,
                     const int32_t *block_tables, const int32_t *seq_lens,
                     const int32_t *query_start_loc, const int32_t *kv_start, int num_seqs,
                     int max_blocks_per_seq, int num_q_heads, int num_kv_heads, int head_dim,
                     int block_size, int64_t num_blocks, double scale, int dtype,
                     int num_threads)
{
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || num_q_heads % num_kv_heads != 0 ||
        (dtype != ORC_F32 && dtype != ORC_BF16))
        return ORC_E_ARG;
    if (num_seqs == 0)
        return ORC_OK;
    int rc = orc_check(block_tables, seq_lens, query_start_loc, kv_start, num_seqs,
                       max_blocks_per_seq, block_size, num_blocks);
    if (rc != ORC_OK)
        return rc;

    const int G = num_q_heads / num_kv_heads;
    const int D = head_dim;
    const int64_t units = (int64_t)num_seqs * num_kv_heads;
    int failed = 0;
    /* num_threads > 0 limits this call only; 0 uses the OpenMP default */
#ifdef _OPENMP
    const int nthr = num_threads > 0 ? num_threads : omp_get_max_threads();
#else
    (void)num_threads;
#endif

#pragma omp parallel for num_threads(nthr) schedule(dynamic, 1) reduction(| : failed)
    for (int64_t u = 0; u < units; ++u) {
        const int s = (int)(u / num_kv_heads);
        const int g = (int)(u % num_kv_heads);
        const int64_t L = seq_lens[s];
        const int64_t a = kv_start ? kv_start[s] : 0;
        const int64_t q0 = query_start_loc[s];
        const int64_t n = (int64_t)query_start_loc[s + 1] - q0;
        if (n == 0)
            continue;
        const int64_t nk = L - a; /* keys a..L-1, gathered into contiguous rows */
        double *Kc = (double *)malloc((size_t)(nk > 0 ? nk : 1) * D * sizeof(double));
        double *Vc = (double *)malloc((size_t)(nk > 0 ? nk : 1) * D * sizeof(double));
        double *w = (double *)malloc((size_t)(nk > 0 ? nk : 1) * sizeof(double));
        double *qd = (double *)malloc((size_t)D * sizeof(double));
        if (!Kc || !Vc || !w || !qd) {
            free(Kc);
            free(Vc);
            free(w);
            free(qd);
            failed |= 1;
            continue;
        }
        /* Page gather: logical key j lives in physical page
         * block_tables[s][j / bs] at offset j % bs. */
        for (int64_t j = a; j < L; ++j) {
            int64_t blk = block_tables[(int64_t)s * max_blocks_per_seq + j / block_size];
            int64_t base = ((blk * num_kv_heads + g) * block_size + j % block_size) * D;
            for (int d = 0; d < D; ++d) {
                Kc[(j - a) * D + d] = orc_elem(k_pool, base + d, dtype);
                Vc[(j - a) * D + d] = orc_elem(v_pool, base + d, dtype);
            }
        }
        for (int64_t i = 0; i < n; ++i) {
            const int64_t t = q0 + i;
            const int64_t p = L - n + i; /* absolute position of this query token */
            for (int hh = 0; hh < G; ++hh) {
                const int h = g * G + hh;
                double *o = out + (t * num_q_heads + h) * D;
                for (int d = 0; d < D; ++d)
                    o[d] = 0.0;
                const int64_t last = p; /* keys a..p inclusive */
                if (last < a)
                    continue;
                const int64_t qb = (t * num_q_heads + h) * (int64_t)D;
                for (int d = 0; d < D; ++d)
                    qd[d] = orc_elem(q, qb + d, dtype);
                double m = -INFINITY;
                for (int64_t j = a; j <= last; ++j) {
                    double acc = 0.0;
                    for (int d = 0; d < D; ++d)
                        acc += qd[d] * Kc[(j - a) * D + d];
                    w[j - a] = scale * acc;
                    if (w[j - a] > m)
                        m = w[j - a];
                }
                double Z = 0.0;
                for (int64_t j = a; j <= last; ++j) {
                    w[j - a] = exp(w[j - a] - m);
                    Z += w[j - a];
                }
                for (int64_t j = a; j <= last; ++j) {
                    const double c = w[j - a];
                    for (int d = 0; d < D; ++d)
                        o[d] += c * Vc[(j - a) * D + d];
                }
                for (int d = 0; d < D; ++d)
                    o[d] /= Z;
            }
        }
        free(Kc);
        free(Vc);
        free(w);
        free(qd);
    }
    return failed ? ORC_E_NOMEM : ORC_OK;
}

/* Number of OpenMP threads a parallel region would use (for reporting). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
