/*
 * pkv.h -- C ABI of the paged-KV attention library for one continuous-batching
 * engine step on AMD Instinct MI355X (gfx950).
 *
 * The operation.  An engine step packs the query tokens of many sequences onto
 * one token axis, with query_start_loc marking where each sequence's tokens
 * begin; prefill chunks and single-token decodes share the step.  Keys and
 * values live in fixed-size pages of a pool reserved once; each sequence's
 * block-table row lists the physical pages of its logical pages.  (vllm-metal
 * v0.4.0 release post: "How vllm-metal fits into vLLM", the runner receives a
 * packed step plus block tables; "Replacing attention, reusing the rest",
 * packed query axis with cu_seqlens, paged KV, one launch for prefill chunks
 * and decode tokens; "Set a predictable memory budget", one pool reserved at
 * startup serves every request.)
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless the argument says "host".
 *   - All memory is owned by the caller.  The device calls allocate nothing and
 *     keep no state between calls except the thread-local error text.  The
 *     host-side pool manager (pkv_pool_*) keeps its page tables in host memory
 *     it owns, between pkv_pool_create and pkv_pool_destroy.
 *   - Calls only enqueue kernels on `stream` (a hipStream_t; NULL is the null
 *     stream) and never synchronise, so they can be captured in a HIP graph.
 *   - Return PKV_OK (0) or a negative PKV_E_* code; the reason is available
 *     from pkv_last_error().  Host arguments are validated before anything is
 *     launched; an invalid call launches nothing.
 *   - Device-array contents are not validated on the hot path.  Values outside
 *     the documented ranges give unspecified output, but the kernels clamp
 *     every index they follow, so they never access memory outside the
 *     buffers whose sizes the host arguments describe.  pkv_check_metadata()
 *     and pkv_check_slots() validate host copies when a caller wants that.
 *   - Three environment variables, read at each pkv_attention call, choose
 *     between launch forms of the same computation (the defaults are the
 *     faster forms measured): PKV_MIXED_STEP=fused|split runs a step with
 *     prefill chunks as one launch or as separate decode and prefill launches
 *     (bitwise the same output); PKV_STEP_TILE_FIRST=0..4 sets how many of
 *     every 4 workgroups of that one launch compute their prefill tile before
 *     their decode waves rather than after (default 2; bitwise the same
 *     output); PKV_DECODE_SEGMENTS=whole|split runs a
 *     decode-only step with one wave per (sequence, kv head) -- where the step
 *     has at most 1024 such segments and 512 sequences -- or spread evenly
 *     over the decode waves (the same result up to float32 summation order).
 *
 * Layouts (row-major, contiguous):
 *   q, out        [total_q][num_q_heads][head_dim]        element type `dtype`
 *   k_new, v_new  [num_tokens][num_kv_heads][head_dim]    element type `dtype`
 *   k_pool,v_pool [num_blocks][num_kv_heads][block_size][head_dim]
 *   block_tables  [num_seqs][max_blocks_per_seq] int32
 *   seq_lens      [num_seqs] int32: keys of the sequence, this step's tokens included
 *   query_start_loc [num_seqs + 1] int32, [0] = 0, [num_seqs] = total_q, non-decreasing
 *   kv_start      [num_seqs] int32 or NULL: keys below kv_start[s] are masked
 *   slot_mapping  [num_tokens] int64: block * block_size + offset, negative = skip
 *
 * Query token i of a sequence with n = query_start_loc[s+1] - query_start_loc[s]
 * tokens and L = seq_lens[s] keys sits at position L - n + i and attends to
 * keys kv_start[s] .. L - n + i (causal inside a chunk, aligned to its end).
 * Query head h reads kv head h / (num_q_heads / num_kv_heads).
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PKV_F32 = 0,  /* float32 q, K/V and out */
    PKV_BF16 = 1  /* bfloat16 q, K/V and out; float32 accumulation */
} pkv_dtype_t;

enum {
    PKV_OK = 0,
    PKV_E_ARG = -1,         /* a host argument is invalid (size, null pointer, ...) */
    PKV_E_UNSUPPORTED = -2, /* valid but not built: head_dim, block_size, dtype, group size */
    PKV_E_WORKSPACE = -3,   /* workspace missing or smaller than required */
    PKV_E_HIP = -4,         /* the HIP runtime reported an error at launch */
    PKV_E_METADATA = -5,    /* pkv_check_*: host metadata violates the contract */
    PKV_E_NOMEM = -6        /* pkv_pool_*: too few free pages; nothing was changed */
};

/*
 * pkv_append -- write this step's new key and value rows into their pool slots.
 *
 * For every token t with slot_mapping[t] >= 0, copies k_new[t][h][:] to
 * k_pool[slot / block_size][h][slot % block_size][:] for every kv head h, and
 * the same for v.  A pure byte copy: the pool is updated in place, never
 * copied as a whole (vllm-metal v0.4.0 release post, "Replacing attention,
 * reusing the rest": KV stays in fixed-size pages located by per-request
 * block tables, so admitted requests grow without reshaping a cache).
 *
 * slot_mapping entries must be unique among non-negative values and lie in
 * [0, num_blocks * block_size); a slot outside that range is skipped.  Pages
 * shared by several sequences (a common prefix) must not be targeted.
 * Supported: dtype F32/BF16, head_dim 64 or 128, any block_size in [1, 256].
 * num_tokens == 0 returns PKV_OK without launching.
 */
int pkv_append(const void *k_new, const void *v_new, void *k_pool, void *v_pool,
               const int64_t *slot_mapping, int64_t num_tokens, int num_kv_heads,
               int head_dim, int block_size, int64_t num_blocks, pkv_dtype_t dtype,
               void *stream);

/*
 * pkv_attention_workspace_size -- bytes of device workspace pkv_attention needs
 * for a step with these host bounds (host-only, pure; 0 if none is needed).
 * The same arguments must be passed to pkv_attention.  The workspace holds the
 * float32 partial results of the split-key decode pass (their size grows with
 * the decode window W, see pkv_attention).
 */
size_t pkv_attention_workspace_size(int num_seqs, int64_t total_q, int max_seqlen_q,
                                    int max_seqlen_k, int num_q_heads, int num_kv_heads,
                                    int head_dim, int block_size, pkv_dtype_t dtype);

/*
 * pkv_attention -- attention for one packed step through the block tables.
 *
 * out[t][h][:] = sum_j softmax_j(scale * q[t][h] . K_j) * V_j over the keys
 * the token sees (see the header comment), K_j and V_j read from kv head
 * h / (num_q_heads / num_kv_heads) of the page block_tables[s][j / block_size]
 * at offset j % block_size.  Pages may be shared by several sequences (a common
 * prefix); they are only read.  Bytes of the pool outside a sequence's keys
 * [kv_start, seq_len) -- the rest of its last page, pages below kv_start,
 * free pages -- never reach the output, whatever they hold (NaN included).
 * The keys inside that range are the sequence's own rows and must be finite:
 * the tokens of one chunk or window share each key's value row in one
 * matrix product, so a non-finite value in a later token's row of the same
 * chunk or window would turn the earlier tokens' outputs (which give it zero
 * weight) into NaN.
 * (vllm-metal v0.4.0 release post, "Replacing attention, reusing the rest";
 * left padding with masked leading keys: vllm-ios README, "How it works" and
 * "What this is and isn't".)
 *
 * Host bounds: max_seqlen_q >= every sequence's query count, max_seqlen_k >=
 * every seq_lens[s]; both size the launch grids.  total_q = query_start_loc
 * [num_seqs], so total_q <= num_seqs * max_seqlen_q (else PKV_E_ARG); when the
 * bounds leave no room for a sequence of W or fewer query tokens
 * (num_seqs * max_seqlen_q - total_q < max_seqlen_q - W), only the prefill
 * kernel is launched.  With G = num_q_heads / num_kv_heads and
 * W = min(16 / G, max_seqlen_q) (integer division), sequences with 1..W query
 * tokens -- decodes, and speculative-verify windows of a few draft tokens --
 * take the split-key decode path; sequences with more take the chunked-prefill
 * path (vllm-metal v0.4.0 release post, "How vllm-metal fits into vLLM": one
 * packed step holds prefill chunks, decode tokens and verify windows).  Both
 * apply the same causal rule.  A sequence with zero query tokens contributes
 * nothing.
 *
 * scale must be finite and positive (a softmax temperature; the kernels bound
 * the running maximum of the scaled logits through the maximum of the raw
 * ones), else PKV_E_ARG.
 *
 * Supported: dtype F32/BF16 (q, pools and out share it), head_dim 64 or 128,
 * block_size 16, num_q_heads % num_kv_heads == 0 and 1 <= group size <= 16,
 * and num_seqs <= 16384; otherwise PKV_E_UNSUPPORTED.
 * out must not alias q or the pools.  workspace must hold at least
 * pkv_attention_workspace_size(...) bytes (it may be NULL when that is 0).
 * num_seqs == 0 or total_q == 0 returns PKV_OK without launching.
 */
int pkv_attention(void *out, const void *q, const void *k_pool, const void *v_pool,
                  const int32_t *block_tables, const int32_t *seq_lens,
                  const int32_t *query_start_loc, const int32_t *kv_start, int num_seqs,
                  int64_t total_q, int max_blocks_per_seq, int max_seqlen_q, int max_seqlen_k,
                  int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                  int64_t num_blocks, float scale, pkv_dtype_t dtype, void *workspace,
                  size_t workspace_bytes, void *stream);

/*
 * pkv_attention_noalloc -- pkv_attention without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.
 *
 * The step's workspace is a static device array of the library's own, of
 * PKV_NOALLOC_SCRATCH_BYTES (24 MiB); every GPU the library runs on holds its
 * own copy until the process ends (its address is looked up on the first
 * call on each device).  The call itself allocates nothing.  Every argument
 * is as for pkv_attention; a step whose pkv_attention_workspace_size exceeds
 * PKV_NOALLOC_SCRATCH_BYTES returns PKV_E_WORKSPACE and launches nothing (a
 * decode window of 16 / G tokens at head_dim 128 takes ~16.3 MiB plus 36
 * bytes per (sequence, kv head)).  Nothing in the scratch needs to start at
 * zero: each call writes what it reads.  All calls on one GPU share its
 * scratch, so two calls that may overlap on one GPU (different streams
 * without an ordering between them, or several host threads) race; calls on
 * one stream are ordered and safe.
 */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)24 << 20)

int pkv_attention_noalloc(void *out, const void *q, const void *k_pool, const void *v_pool,
                          const int32_t *block_tables, const int32_t *seq_lens,
                          const int32_t *query_start_loc, const int32_t *kv_start, int num_seqs,
                          int64_t total_q, int max_blocks_per_seq, int max_seqlen_q,
                          int max_seqlen_k, int num_q_heads, int num_kv_heads, int head_dim,
                          int block_size, int64_t num_blocks, float scale, pkv_dtype_t dtype,
                          void *stream);

/*
 * pkv_attention_shared_prefix -- pkv_attention for a step in which groups of
 * decode sequences share their first keys through common pages, reading
 * each group's shared pages once per kv head instead of once per sequence.
 *
 * Requests that share a prompt prefix keep it in shared pages (vllm-metal
 * v0.4.0 release post, "Prefix caching on hybrid models"; the vllm-mlx paper
 * summary, results: prefix caching on 512-token shared prefixes).  Attention
 * over a sequence's keys is the log-sum-exp combination of attention over the
 * shared prefix and over the rest, so the result is the same as
 * pkv_attention's (up to rounding order): the prefix of each group is
 * attended once for all its members' query rows (matrix-core tiles, chunks
 * of the prefix in parallel), each member's own keys by the decode pass,
 * which starts from the prefix's softmax states.
 *
 * prefix_group [num_seqs] int32 (device): the group of sequence s in
 * [0, num_groups), or -1.  prefix_len [num_groups] int32 (device): the
 * group's shared keys, a multiple of block_size, at most max_prefix_len.
 * Contract for a member s of group g: one query token (a decode), seq_lens[s]
 * > prefix_len[g], and its first prefix_len[g] / block_size block-table
 * entries are the group's shared pages (the same physical ids in every
 * member's row).  Sequences that break the token or length condition, and
 * the members of a group beyond its first max_group_size (which ones is
 * unspecified), are computed as plain sequences.  Other sequences of the
 * step (prefill chunks, verify windows, unshared decodes) are computed as by
 * pkv_attention.
 * kv_start is not taken (no left padding in such a step).
 *
 * Reading a prefix once takes three more launches (group setup, prefix
 * states, their combination), so the prefix pass pays for long prefixes
 * shared by many sequences, whose re-reads the GPU's caches cannot absorb;
 * for short prefixes the plain path is faster.  prefix_pass selects:
 *   PKV_PREFIX_PASS_AUTO (0): the library runs the prefix pass only when the
 *     prefix re-reads it can avoid, estimated from the host bounds as
 *     num_groups * (min(max_group_size, num_seqs) - 1) * max_prefix_len keys
 *     of K and V, reach 256 MiB; otherwise the step runs exactly as
 *     pkv_attention (the group arrays are then not read).
 *   PKV_PREFIX_PASS_ALWAYS (1): always run the prefix pass.
 *
 * Host bounds: max_group_size > 0, max_prefix_len a positive multiple of
 * block_size below max_seqlen_k, 0 <= num_groups <= 1024 (num_groups == 0:
 * exactly pkv_attention).  Workspace: at least
 * pkv_attention_shared_prefix_workspace_size(...) bytes with the same bounds
 * (whichever path runs).  Errors and every other argument as for
 * pkv_attention.
 */
enum { PKV_PREFIX_PASS_AUTO = 0, PKV_PREFIX_PASS_ALWAYS = 1 };

size_t pkv_attention_shared_prefix_workspace_size(int num_seqs, int64_t total_q, int max_seqlen_q,
                                                  int max_seqlen_k, int num_q_heads,
                                                  int num_kv_heads, int head_dim, int block_size,
                                                  pkv_dtype_t dtype, int num_groups,
                                                  int max_group_size, int max_prefix_len);

int pkv_attention_shared_prefix(void *out, const void *q, const void *k_pool, const void *v_pool,
                                const int32_t *block_tables, const int32_t *seq_lens,
                                const int32_t *query_start_loc, const int32_t *prefix_group,
                                const int32_t *prefix_len, int num_groups, int max_group_size,
                                int max_prefix_len, int num_seqs, int64_t total_q,
                                int max_blocks_per_seq, int max_seqlen_q, int max_seqlen_k,
                                int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                                int64_t num_blocks, float scale, pkv_dtype_t dtype,
                                int prefix_pass, void *workspace, size_t workspace_bytes,
                                void *stream);

/*
 * pkv_check_metadata -- validate HOST copies of the step metadata against the
 * contract above: query_start_loc starts at 0, is non-decreasing and ends at
 * total_q; 0 <= kv_start[s] <= seq_lens[s]; each sequence's query count is at
 * most seq_lens[s] - kv_start[s] and at most max_seqlen_q; seq_lens[s] is at
 * most max_seqlen_k; every page a visible key lives on is listed and lies in
 * [0, num_blocks).  max_seqlen_q and max_seqlen_k are the host bounds that
 * will be passed to pkv_attention: a step that exceeds them would leave output
 * rows unwritten (too many query tokens) or lose keys (too long a sequence),
 * so both are checked.  Returns PKV_OK, PKV_E_METADATA (reason in
 * pkv_last_error()) or PKV_E_ARG for invalid sizes.  kv_start may be NULL.
 */
int pkv_check_metadata(const int32_t *block_tables, const int32_t *seq_lens,
                       const int32_t *query_start_loc, const int32_t *kv_start, int num_seqs,
                       int64_t total_q, int max_blocks_per_seq, int max_seqlen_q,
                       int max_seqlen_k, int block_size, int64_t num_blocks);

/*
 * pkv_check_shared_prefix -- validate HOST copies of a shared-prefix step's
 * groups against the contract of pkv_attention_shared_prefix: group ids in
 * [-1, num_groups); prefix lengths multiples of block_size, at most
 * max_prefix_len and inside the block table; every member a decode (one query
 * token) with more keys than its prefix; all members of a group list the same
 * physical pages for the prefix.  Returns PKV_OK or PKV_E_METADATA.
 */
int pkv_check_shared_prefix(const int32_t *block_tables, const int32_t *seq_lens,
                            const int32_t *query_start_loc, const int32_t *prefix_group,
                            const int32_t *prefix_len, int num_seqs, int num_groups,
                            int max_blocks_per_seq, int block_size, int max_prefix_len);

/*
 * pkv_check_slots -- validate a HOST copy of a slot mapping: every
 * non-negative slot lies in [0, num_blocks * block_size) and appears once.
 * Returns PKV_OK or PKV_E_METADATA.
 */
int pkv_check_slots(const int64_t *slot_mapping, int64_t num_tokens, int block_size,
                    int64_t num_blocks);

/* Text of the last error on the calling thread ("" if none).  Valid until the
 * next pkv_* call on the same thread. */
const char *pkv_last_error(void);

/* ------------------------------------------------------------------------
 * Host-side pool manager.
 *
 * Bookkeeping for a KV pool of num_blocks pages reserved once at startup and
 * serving every request: admission is checked against its free pages, so load
 * changes the queue rather than the memory footprint (vllm-metal v0.4.0
 * release post, "Set a predictable memory budget").  Sequences forked from a
 * common prefix hold the same physical pages (reference counts); a sequence
 * about to write into a page it shares first moves to a private copy of that
 * page (copy-on-write), so pages shared by several sequences are only read,
 * as pkv_append requires ("Prefix caching on hybrid models": reusing a
 * prefix goes through the paged path's block tables).  The manager produces slot_mapping, block-table rows and
 * seq_lens for the device calls above; it never touches device memory itself
 * (pkv_copy_blocks performs the page copies it asks for).  All pointers of
 * pkv_pool_* are HOST pointers.  A pool is not thread-safe: one host thread
 * drives it.  Sequence ids are in [0, max_seqs).
 * ------------------------------------------------------------------------ */
typedef struct pkv_pool pkv_pool_t;

/* Creates a manager for num_blocks pages of block_size tokens; a sequence may
 * hold at most max_blocks_per_seq pages.  Returns NULL on invalid sizes (the
 * reason in pkv_last_error()). */
pkv_pool_t *pkv_pool_create(int64_t num_blocks, int block_size, int max_seqs,
                            int max_blocks_per_seq);
void pkv_pool_destroy(pkv_pool_t *pool);

/* Sets the order in which the free pages are handed out (order[0] first):
 * order must list each of the n == pkv_pool_free_blocks() free pages once,
 * else PKV_E_ARG and nothing changes.  A pool that has served for a while
 * hands out pages in no particular order; this reproduces any placement. */
int pkv_pool_set_free_order(pkv_pool_t *pool, const int32_t *order, int64_t n);

/* Free pages, and whether a new sequence of num_tokens tokens fits now
 * (1 / 0; -1 for a NULL pool). */
int64_t pkv_pool_free_blocks(const pkv_pool_t *pool);
int pkv_pool_can_admit(const pkv_pool_t *pool, int64_t num_tokens);

/* Starts an empty sequence; PKV_E_ARG if seq is out of range or live. */
int pkv_pool_add_seq(pkv_pool_t *pool, int seq);

/* Starts sequence child as the first shared_tokens tokens of parent, on the
 * parent's pages (no copy; 0 <= shared_tokens <= the parent's length). */
int pkv_pool_fork(pkv_pool_t *pool, int parent, int child, int64_t shared_tokens);

/* Reserves num_tokens more tokens at the end of seq and writes their slots
 * (page * block_size + offset, token order) to slots[0..num_tokens).  If the
 * sequence's last page is partly filled and shared, the sequence first moves
 * to a fresh page: the (source, destination) page ids are written to
 * cow_src[0] / cow_dst[0] and *num_cow = 1 (else 0); the caller copies those
 * pages on the device (pkv_copy_blocks) before appending this step's rows.
 * cow_src, cow_dst and num_cow may be NULL only when no copy can be needed.
 * PKV_E_NOMEM if the free pages do not suffice, PKV_E_ARG if the sequence
 * would exceed max_blocks_per_seq; in both cases nothing changes. */
int pkv_pool_append(pkv_pool_t *pool, int seq, int64_t num_tokens, int64_t *slots,
                    int32_t *cow_src, int32_t *cow_dst, int *num_cow);

/* pkv_pool_append for num_seqs distinct sequences at once (one engine step):
 * counts[i] tokens for seqs[i]; their slots are written back to back to slots
 * in the order given (sum of counts entries), copy-on-write pairs to
 * cow_src / cow_dst (room for num_seqs entries each), their number to
 * *num_cow.  All-or-nothing: PKV_E_ARG (a sequence not live, listed twice or
 * past max_blocks_per_seq) or PKV_E_NOMEM leaves the pool unchanged. */
int pkv_pool_append_batch(pkv_pool_t *pool, const int *seqs, const int64_t *counts,
                          int num_seqs, int64_t *slots, int32_t *cow_src, int32_t *cow_dst,
                          int *num_cow);

/* Drops the tokens of seq past new_len (for example the rejected draft tokens
 * of a speculative-verify window); pages no longer used are released. */
int pkv_pool_truncate(pkv_pool_t *pool, int seq, int64_t new_len);

/* Ends seq and releases its pages (a shared page returns to the free list
 * when its last holder releases it). */
int pkv_pool_free_seq(pkv_pool_t *pool, int seq);

/* Length of seq in tokens, or -1 if it is not live. */
int64_t pkv_pool_seq_len(const pkv_pool_t *pool, int seq);

/* Block-table rows and lengths of seqs[0..num_seqs): table is
 * [num_seqs][width] int32, entries past a sequence's pages set to -1;
 * seq_lens[i] is its length (may be NULL).  PKV_E_ARG if a sequence is not
 * live or holds more than width pages. */
int pkv_pool_block_tables(const pkv_pool_t *pool, const int *seqs, int num_seqs, int32_t *table,
                          int width, int32_t *seq_lens);

/* DEVICE call: copies whole pages src[i] -> dst[i] (K and V, every kv head),
 * i < num_pairs; src and dst are device int32 arrays; pairs naming a page
 * outside [0, num_blocks) are skipped.  Destinations must be distinct and must
 * not be sources.  Pool layout and dtypes as for pkv_append.  num_pairs == 0
 * returns PKV_OK without launching. */
int pkv_copy_blocks(void *k_pool, void *v_pool, const int32_t *src, const int32_t *dst,
                    int64_t num_pairs, int num_kv_heads, int head_dim, int block_size,
                    int64_t num_blocks, pkv_dtype_t dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
