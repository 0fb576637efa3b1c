/*
 * libpagedkv -- single-token decode attention over a paged KV cache, for
 * AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The problem statement these calls follow:
 *
 *  - "TensorRT-LLM 深度实战：从 Blackwell 架构到 INT4 量化的 LLM 推理性能革命"
 *    (chenxutan.com), section 3.1 "Paged KV Cache": a pool of fixed-size
 *    pages, a free-page list, a per-sequence page table, allocate /
 *    append_tokens / release, and an out-of-memory error when the free list
 *    runs dry;
 *  - the same page, section 3.3 "融合 CUDA Kernel": the attention a decode
 *    step computes -- scores scale * q.k, max-subtracted softmax, softmax-
 *    weighted sum of V -- fused so that K and V are read once and the output
 *    written once;
 *  - "TensorRT-LLM 推理加速实战：从 engine 编译到 kernel 调优"
 *    (socake.github.io), section 7.2 (masked_mha: decode attention for one
 *    new token per sequence per step), section 8 (block sizes 64 and 16) and
 *    section 8.1 (KV size = 2 x layers x kv_heads x head_dim x bytes per
 *    token, with grouped KV heads);
 *  - the aiqz.cc TensorRT-LLM explainer, section "KV缓存管理" (the total
 *    M_kv = 2 x layers x heads x d_head x tokens x batch x bytes, and paging
 *    of the KV memory).
 *
 * Conventions shared by every call:
 *  - Every call returns pkv_status: PKV_OK (0) or a negative error code.  On
 *    error nothing observable has changed, and pkv_last_error() returns a
 *    message for the calling thread.
 *  - "host" pointers are CPU memory owned by the caller, read or written only
 *    during the call.  "device" pointers are GPU memory owned by the caller
 *    (for instance torch tensors); the library never allocates, frees or
 *    retains them.
 *  - Device work is enqueued on `stream` (a hipStream_t; NULL is the null
 *    stream) and is asynchronous: the call returns after launching.  Launch
 *    failures are PKV_ERR_DEVICE.
 *  - Layouts are dense, row-major, with no padding:
 *      q, out        [batch][num_q_heads][head_dim]
 *      k_pool/v_pool [num_pages][num_kv_heads][page_size][head_dim]
 *      k/v_scale     [num_pages][num_kv_heads][page_size]     (fp32, int8 / fp8 only)
 *      block_tables  [batch][max_blocks]                      (int32)
 *      context_lens  [batch]                                  (int32)
 *    One page id addresses the same page in every layer's pools; block
 *    tables are shared by all layers.
 *  - Query head h reads KV head h / (num_q_heads / num_kv_heads): query heads
 *    share KV heads in contiguous groups (GQA; MQA when num_kv_heads == 1).
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 1

typedef enum pkv_status {
    PKV_OK = 0,
    PKV_ERR_INVALID_ARG = -1, /* null pointer, bad size, misaligned buffer  */
    PKV_ERR_OOM = -2,         /* the free-page list cannot cover a request  */
    PKV_ERR_NO_SEQ = -3,      /* unknown sequence id                        */
    PKV_ERR_SEQ_EXISTS = -4,  /* sequence id already allocated              */
    PKV_ERR_UNSUPPORTED = -5, /* shape / dtype outside the compiled set     */
    PKV_ERR_WORKSPACE = -6,   /* workspace missing or too small             */
    PKV_ERR_DEVICE = -7,      /* HIP runtime error (no device, bad launch)  */
    PKV_ERR_SHARED_PAGE = -8  /* the append needs a copy-on-write of a shared
                                 page: use pkv_append_tokens_cow             */
} pkv_status;

typedef enum pkv_dtype {
    PKV_F16 = 0,  /* IEEE binary16                                          */
    PKV_BF16 = 1, /* bfloat16                                               */
    PKV_I8 = 2,   /* symmetric int8 code; value = fp32 scale x code, one
                     scale per (page, kv head, slot), i.e. per token per head */
    PKV_FP8_E4M3 = 3 /* OCP 8-bit float E4M3 ("e4m3fn": bias 7, no infinities,
                     S.1111.111 = NaN, max 448); value = fp32 scale x code,
                     scales laid out as for PKV_I8.  The FP8 KV cache of
                     "TensorRT-LLM 推理加速实战", sections 8 and 8.1 (half the
                     bytes of fp16 KV per token).                           */
} pkv_dtype;

int32_t pkv_abi_version(void);
const char *pkv_status_string(pkv_status status);
/* Message describing the last error raised on the calling thread ("" if none). */
const char *pkv_last_error(void);
/* Number of visible HIP devices (0 when there is none or the runtime fails). */
int32_t pkv_device_count(void);

/* ===================================================================== *
 * Host page pool (section 3.1 of the first page).  Pure host bookkeeping:
 * it hands out page ids; the K/V bytes live in caller-owned device pools.
 * A pool handle is not thread-safe: use it from one thread at a time.
 * ===================================================================== */

typedef struct pkv_pool pkv_pool;

typedef struct pkv_pool_desc {
    int32_t num_pages;                  /* > 0                                     */
    int32_t page_size;                  /* tokens per page, > 0 (16 and 64 are
                                           the sizes the decode kernel supports)   */
    const int32_t *initial_free_order;  /* host, num_pages entries, a permutation
                                           of [0, num_pages); NULL = 0, 1, ..., n-1.
                                           Pages are taken from the END of the list
                                           and released pages are pushed back onto
                                           its end, in the sequence's page order.  */
} pkv_pool_desc;

/* Creates a pool.  *out receives the handle (host memory owned by the
 * library until pkv_pool_destroy).  INVALID_ARG on a bad descriptor. */
pkv_status pkv_pool_create(const pkv_pool_desc *desc, pkv_pool **out);
void pkv_pool_destroy(pkv_pool *pool);

/* Admits sequence seq_id holding num_tokens tokens: takes
 * ceil(num_tokens / page_size) pages, all or nothing.  OOM if the free list
 * is too short, SEQ_EXISTS if seq_id is live; neither changes the pool.
 * slots_out (host, may be NULL) receives num_tokens slot ids
 * page * page_size + offset, in token order. */
pkv_status pkv_seq_alloc(pkv_pool *pool, int64_t seq_id, int32_t num_tokens,
                         int64_t *slots_out);

/* Adds n_new tokens to a live sequence, taking
 * ceil((count + n_new - capacity) / page_size) new pages when the current
 * pages overflow.  OOM (checked before any page is taken) or NO_SEQ leave the
 * pool unchanged.  slots_out (host, may be NULL) receives the n_new slot ids
 * of the new tokens.  SHARED_PAGE (pool unchanged) if the sequence's last
 * page is partly filled and shared with another sequence: that append needs
 * the copy pkv_append_tokens_cow reports. */
pkv_status pkv_append_tokens(pkv_pool *pool, int64_t seq_id, int32_t n_new,
                             int64_t *slots_out);

/* Block reuse (the KV-cache reuse and prefix caching of shared prompts that
 * "TensorRT-LLM 推理加速实战", section 8, enables): pages may be owned by
 * several sequences.
 *
 * pkv_seq_fork: child_id (new) gets parent_id's pages and token count; every
 * page gains an owner.  NO_SEQ / SEQ_EXISTS leave the pool unchanged.
 *
 * pkv_append_tokens_cow: pkv_append_tokens that also handles a shared,
 * partly filled last page: a fresh page (taken from the free list before any
 * overflow pages) replaces it in this sequence, *copy_src / *copy_dst
 * (host, may be NULL) receive (old page, new page), and the caller must copy
 * the page's contents (pkv_copy_pages, every layer) before writing the new
 * tokens; -1, -1 when no copy is needed.  OOM counts the copy's page too.
 *
 * pkv_page_owners: sequences holding a page (0 = free), -1 for a bad page. */
pkv_status pkv_seq_fork(pkv_pool *pool, int64_t parent_id, int64_t child_id);
pkv_status pkv_append_tokens_cow(pkv_pool *pool, int64_t seq_id, int32_t n_new, int64_t *slots_out,
                                 int32_t *copy_src, int32_t *copy_dst);
int32_t pkv_page_owners(const pkv_pool *pool, int32_t page);

/* Retires a sequence; each of its pages loses an owner and returns to the
 * free list (in the sequence's page order) when it has none left.  NO_SEQ
 * for an unknown id. */
pkv_status pkv_seq_release(pkv_pool *pool, int64_t seq_id);

/* Token and page count of a live sequence (either output may be NULL). */
pkv_status pkv_seq_info(const pkv_pool *pool, int64_t seq_id, int32_t *num_tokens,
                        int32_t *num_pages);

/* Copies a live sequence's page ids, in logical order, into pages_out (host,
 * capacity entries); *n_pages receives the count.  INVALID_ARG if capacity is
 * too small. */
pkv_status pkv_seq_pages(const pkv_pool *pool, int64_t seq_id, int32_t *pages_out,
                         int32_t capacity, int32_t *n_pages);

int32_t pkv_free_page_count(const pkv_pool *pool);

/* Copies the free list, bottom to top (the next page handed out is the last
 * entry), into out (host, capacity entries); *count receives its length. */
pkv_status pkv_free_pages(const pkv_pool *pool, int32_t *out, int32_t capacity,
                          int32_t *count);

/* Writes the block tables and context lengths of `batch` live sequences:
 * block_tables_out (host, [batch][max_blocks]) gets each sequence's page ids
 * followed by -1 padding; context_lens_out (host, [batch]) its token count.
 * NO_SEQ for an unknown id, INVALID_ARG if a sequence has more than
 * max_blocks pages. */
pkv_status pkv_build_block_tables(const pkv_pool *pool, const int64_t *seq_ids,
                                  int32_t batch, int32_t max_blocks,
                                  int32_t *block_tables_out, int32_t *context_lens_out);

/* KV-cache bytes 2 x layers x kv_heads x head_dim x tokens x batch x bytes(dtype)
 * (section 8.1 of the engine-to-kernel-tuning page; the M_kv equation of the
 * aiqz.cc explainer).  int8 and fp8 count the codes only (scales excluded);
 * fp8 is the page's 1-byte FP8 case.
 * Returns -1 for a negative argument or overflow. */
int64_t pkv_kv_bytes(int32_t layers, int32_t kv_heads, int32_t head_dim, int64_t tokens,
                     int32_t batch, pkv_dtype dtype);

/* ===================================================================== *
 * Device: decode attention (section 3.3 of the first page; masked_mha of
 * section 7.2 of the engine-to-kernel-tuning page).
 * ===================================================================== */

typedef struct pkv_decode_args {
    const void *q;              /* device [batch][num_q_heads][head_dim], q_dtype   */
    const void *k_pool;         /* device [num_pages][num_kv_heads][page_size][head_dim] */
    const void *v_pool;         /* device, same shape                                */
    const float *k_scale;       /* device [num_pages][num_kv_heads][page_size]; int8
                                   and fp8 KV only, otherwise NULL                   */
    const float *v_scale;
    const int32_t *block_tables;/* device [batch][max_blocks]; entry j of row b is the
                                   physical page of tokens [j*page_size, (j+1)*page_size)
                                   of sequence b.  Entries j >= ceil(len_b/page_size)
                                   are never read.                                   */
    const int32_t *context_lens;/* device [batch]: tokens in the cache for each
                                   sequence, including the one just appended; the
                                   single query attends to all of them.             */
    void *out;                  /* device [batch][num_q_heads][head_dim], q_dtype    */
    void *workspace;            /* device scratch of >= pkv_decode_workspace_bytes,
                                   256-byte aligned; its contents between calls do
                                   not matter; may be NULL when that size is 0     */
    size_t workspace_bytes;
    uint32_t *merge_counters;   /* device array of >= pkv_decode_counter_bytes bytes,
                                   4-byte aligned, ZERO-FILLED once when allocated
                                   and used for nothing else: the arrival counters
                                   of the in-kernel merge.  Every complete call
                                   leaves all of it zero again, whatever the
                                   shapes, so one array serves any later calls
                                   that do not overlap in time.  Only
                                   pkv_paged_attn_decode uses it (NULL is fine for
                                   the two-launch form).                             */
    size_t merge_counter_bytes;
    int32_t batch;              /* >= 0; 0 is a no-op                               */
    int32_t num_q_heads;
    int32_t num_kv_heads;       /* divides num_q_heads; group = Hq / Hkv in {1,2,4,8} */
    int32_t head_dim;           /* 64 or 128                                        */
    int32_t page_size;          /* 16 or 64                                         */
    int32_t num_pages;          /* pages in each pool                               */
    int32_t max_blocks;         /* row length of block_tables                       */
    int32_t max_context_len;    /* host bound on every context_lens entry;
                                   <= max_blocks * page_size                         */
    int32_t num_splits;         /* waves sharing the batch: the batch's 64-token tiles
                                   (all sequences, all KV heads) are divided into this
                                   many equal contiguous shares, one per wave of a
                                   persistent grid.  0 = library default (4 waves per
                                   compute unit, 8 for int8 / fp8 KV);
                                   always capped at the number of tiles the batch
                                   can have.                                         */
    pkv_dtype q_dtype;          /* PKV_F16 or PKV_BF16; out has the same type       */
    pkv_dtype kv_dtype;         /* PKV_F16 (with f16 q), PKV_BF16 (with bf16 q), or
                                   PKV_I8 or PKV_FP8_E4M3 (with either)              */
    float scale;                /* softmax scale applied to q.k (e.g. 1/sqrt(head_dim)) */
} pkv_decode_args;

/* Bytes of workspace the decode calls need for these arguments: one
 * (max, sum, head_dim-vector) slot per query head for every (sequence, KV
 * head) segment plus every wave, fp32, one 16-byte record per segment and a
 * 256-byte header (uses batch, num_q_heads, num_kv_heads, head_dim,
 * max_context_len, num_splits).  0 only for an empty batch. */
pkv_status pkv_decode_workspace_bytes(const pkv_decode_args *args, size_t *bytes);

/* Bytes of merge_counters pkv_paged_attn_decode needs for these arguments:
 * 4 x (segments + waves) x levels, with levels the depth of a fan-in-8 tree
 * over the waves (uses batch, num_kv_heads, max_context_len, num_splits).
 * 0 only for an empty batch. */
pkv_status pkv_decode_counter_bytes(const pkv_decode_args *args, size_t *bytes);

/* Number of waves the library uses for these arguments (resolves 0). */
int32_t pkv_decode_num_splits(const pkv_decode_args *args);

/* Checks the arguments without touching the GPU (pointer presence and
 * 16-byte alignment, shapes, dtype pair, workspace and counter sizes).
 * Returns what pkv_paged_attn_decode would return before launching. */
pkv_status pkv_decode_validate(const pkv_decode_args *args);

/* out[b][h][:] = softmax_t(scale * q[b][h] . K_t) . V_t over the
 * context_lens[b] cached tokens of sequence b, read through block_tables from
 * KV head h / group.  Sequences with context length 0 get zeros.  A sequence
 * whose context length is negative or above max_context_len, or whose block
 * table names a page outside [0, num_pages), gets NaN in every element of its
 * output instead of a memory access outside the pools.
 * One launch on `stream`: a persistent grid of num_splits waves, each
 * streaming an equal share of the batch's tiles.  A (sequence, KV head) a
 * wave covers whole is written directly; the pieces of one shared by several
 * waves go to the workspace and the last wave to finish a group of pieces
 * merges them (a fan-in-8 tree; no wave ever waits for another).  The result
 * does not depend on the order in which waves finish.  Stateless and
 * re-entrant; the workspace must not be shared by calls that may overlap. */
pkv_status pkv_paged_attn_decode(const pkv_decode_args *args, void *stream);

/* The same computation in two launches: the decode kernel leaves every piece
 * of a shared segment in the workspace (it merges nothing), and the merge
 * kernel combines them, one workgroup per (query head, sequence).  Calling
 * both in order on one stream gives the result of pkv_paged_attn_decode up to
 * fp32 rounding order.  This form is for callers that combine pieces
 * themselves or time the phases apart; it does not use the counters. */
pkv_status pkv_paged_attn_decode_partitions(const pkv_decode_args *args, void *stream);
pkv_status pkv_splitk_reduce(const pkv_decode_args *args, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * pkv_paged_attn_decode with the workspace and merge counters taken from a
 * static device array of the library instead of the caller.  `workspace`,
 * `workspace_bytes`, `merge_counters` and `merge_counter_bytes` of args are
 * ignored; everything else is as for pkv_paged_attn_decode, with the same
 * result.  The array holds 32 MiB of workspace and 1 MiB of counters:
 * shapes whose pkv_decode_workspace_bytes or pkv_decode_counter_bytes exceed
 * that return PKV_ERR_WORKSPACE (nothing launched).  Each GPU the library
 * runs on holds its own array until the process ends; the first call on a
 * device looks up its address and enqueues one small kernel that zeroes the
 * counters.  No call allocates or frees memory.  All calls on one GPU share
 * the array, so calls that may overlap in time on one GPU (two streams, two
 * threads) race and give wrong results; serialise them. */
pkv_status pkv_paged_attn_decode_noalloc(const pkv_decode_args *args, void *stream);

/* ===================================================================== *
 * Device: write appended tokens' K/V into their slots (the device side of
 * append_tokens, section 3.1 of the first page).
 * ===================================================================== */

typedef struct pkv_write_args {
    const void *k_new;          /* device [n][num_kv_heads][head_dim], src_dtype     */
    const void *v_new;
    const float *k_scale_new;   /* device [n][num_kv_heads] fp32: the scales of
                                   already-encoded int8 / fp8 rows (src_dtype ==
                                   kv_dtype); NULL otherwise                         */
    const float *v_scale_new;
    const int64_t *slots;       /* device [n]: page * page_size + offset, as returned by
                                   pkv_seq_alloc / pkv_append_tokens.  A slot outside
                                   [0, num_pages * page_size) is skipped.            */
    void *k_pool;               /* device pools, as in pkv_decode_args               */
    void *v_pool;
    float *k_scale;             /* device pool scales; int8 / fp8 only, else NULL    */
    float *v_scale;
    int32_t n;                  /* tokens to write, >= 0; n * num_kv_heads < 2^31    */
    int32_t num_kv_heads;
    int32_t head_dim;           /* 64 or 128                                        */
    int32_t page_size;
    int32_t num_pages;
    pkv_dtype kv_dtype;         /* type of the pools                                 */
    pkv_dtype src_dtype;        /* type of k_new / v_new: kv_dtype (rows are copied
                                   as they are), or PKV_F16 / PKV_BF16 with an int8
                                   or fp8 pool: each row (one token, one KV head) is
                                   quantised on the device, s = max(max|x|, 1e-5) /
                                   Q in fp32 (Q = 127 int8, 448 fp8), codes rounded
                                   half to even (int8 clipped to +-127, fp8 the
                                   nearest E4M3 value, saturating at 448), and s is
                                   stored in k_scale / v_scale                       */
} pkv_write_args;

/* Writes the n new tokens' K and V (all KV heads) at their slots; for an
 * int8 / fp8 pool fed f16 / bf16 rows, quantises them first (see src_dtype).
 * Asynchronous on `stream`.  Slots must be distinct. */
pkv_status pkv_write_kv(const pkv_write_args *args, void *stream);

/* Device: whole-page copies for copy-on-write (pkv_append_tokens_cow), one
 * layer's pools per call: for each pair i, page pairs[2i] is copied to page
 * pairs[2i+1] in k_pool and v_pool (all KV heads, all slots) and, for int8 /
 * fp8, in k_scale and v_scale.  pairs is a device int32 array; a pair naming
 * a page outside [0, num_pages) is skipped.  Destination pages must be
 * distinct and not sources.  INVALID_ARG when n times the page's 16 KiB
 * tiles (per pool) reaches 2^32.  Asynchronous on `stream`. */
typedef struct pkv_copy_args {
    void *k_pool;
    void *v_pool;
    float *k_scale;             /* int8 / fp8 only, else NULL                        */
    float *v_scale;
    const int32_t *pairs;       /* device [n][2]: (source page, destination page)    */
    int32_t n;
    int32_t num_pages;
    int32_t num_kv_heads;
    int32_t page_size;
    int32_t head_dim;
    pkv_dtype kv_dtype;
} pkv_copy_args;

pkv_status pkv_copy_pages(const pkv_copy_args *args, void *stream);

/* ===================================================================== *
 * Device: chunked prefill (context attention) over the paged cache -- the
 * chunked context of "TensorRT-LLM 深度实战", section 7.3: a long prompt is
 * processed a chunk at a time, each chunk's queries attending to every
 * earlier token of the sequence and causally to the chunk's own tokens, with
 * the scaled-dot-product softmax of section 3.3.
 * ===================================================================== */

typedef struct pkv_prefill_args {
    const void *q;              /* device [n_q][num_q_heads][head_dim], q_dtype: the
                                   new tokens' queries, sequence after sequence       */
    const void *k_pool;         /* device pools [num_pages][num_kv_heads][page_size]
                                   [head_dim], kv_dtype; the chunk's own K/V already
                                   written (pkv_write_kv)                             */
    const void *v_pool;
    const int32_t *block_tables; /* device [batch][max_blocks], as for decode         */
    const int32_t *q_start;     /* device [batch + 1]: sequence b's queries are rows
                                   q_start[b] .. q_start[b+1]-1; q_start[0] = 0,
                                   non-decreasing, q_start[batch] = n_q              */
    const int32_t *context_lens; /* device [batch]: tokens in the cache, the chunk
                                   included; query i of sequence b sits at position
                                   context_lens[b] - nq_b + i and attends to keys
                                   0 .. that position                                 */
    void *out;                  /* device [n_q][num_q_heads][head_dim], q_dtype     */
    int32_t batch;
    int32_t n_q;                /* total query rows                                  */
    int32_t num_q_heads;
    int32_t num_kv_heads;       /* num_q_heads / num_kv_heads in {1, 2, 4, 8}        */
    int32_t head_dim;           /* 64 or 128                                         */
    int32_t page_size;          /* 16 or 64                                          */
    int32_t num_pages;
    int32_t max_blocks;
    int32_t max_context_len;    /* host bound on context_lens (<= max_blocks *
                                   page_size)                                         */
    int32_t max_q_len;          /* host bound on every sequence's chunk length; a
                                   sequence with a longer chunk gets NaN rows where
                                   it is written, and its rows past max_q_len are
                                   not written at all                                */
    pkv_dtype q_dtype;          /* PKV_F16 or PKV_BF16                               */
    pkv_dtype kv_dtype;         /* == q_dtype, or PKV_I8 / PKV_FP8_E4M3 (then the
                                   value of a code is code x its token's scale)      */
    float scale;
    const float *k_scale;       /* device [num_pages][num_kv_heads][page_size] fp32,
                                   4-byte aligned: int8 / fp8 K/V only, else NULL.
                                   Any finite scale magnitude is handled: p.V runs
                                   in f16 on the V scales divided by a running
                                   power of two                                      */
    const float *v_scale;
} pkv_prefill_args;

/* Chunked prefill attention; one launch, asynchronous on `stream`.  A
 * sequence whose context length is negative, above max_context_len or shorter
 * than its chunk, or whose chunk is longer than max_q_len, gets NaN rows, as
 * does any block of rows that needs a page outside the pool; rows of a
 * sequence whose q_start entries are out of order or beyond n_q are not
 * written.  UNSUPPORTED outside the instantiated
 * shapes; INVALID_ARG for bad sizes (batch and num_kv_heads at most 65535
 * each) or null pointers. */
pkv_status pkv_paged_prefill(const pkv_prefill_args *args, void *stream);

/* ===================================================================== *
 * Host: continuous-batching step driver over a pool.  One step follows
 * "TensorRT-LLM 深度实战", section 3.2: finished sequences leave the batch
 * and release their pages, waiting requests join while there is room (their
 * prompt's pages are allocated), then every running sequence appends one
 * token.  The clock, arrival steps, the static-batching alternative and the
 * statistics follow the request simulator of the aiqz.cc TensorRT-LLM
 * explainer ("连续批处理", "Python 演示").  Readings where those pages are
 * silent:
 *   - the waiting queue is served first come, first served, in submission
 *     order; arrival steps must not decrease along it;
 *   - a request reserves the pages of its whole life,
 *     ceil((prompt_len + max_new_tokens) / page_size); the head of the queue
 *     is admitted only when the free pages minus the pages still owed to
 *     running sequences cover that, and nothing overtakes it -- so a running
 *     sequence never runs out of pages (if the scheduler is the pool's only
 *     user);
 *   - PKV_SCHED_STATIC admits only into an empty batch;
 *   - with nothing running and the head of the queue not yet arrived, the
 *     clock jumps to its arrival; it advances by one per step that runs;
 *   - the batch is listed in admission order.
 * The pool must outlive the scheduler; the scheduler's sequences live in it
 * (read their pages and block tables through the pool calls above).
 * ===================================================================== */

typedef struct pkv_sched pkv_sched;

typedef enum pkv_sched_policy {
    PKV_SCHED_CONTINUOUS = 0,
    PKV_SCHED_STATIC = 1
} pkv_sched_policy;

/* max_batch >= 1 sequences run per step.  INVALID_ARG on bad arguments. */
pkv_status pkv_sched_create(pkv_pool *pool, int32_t max_batch, pkv_sched_policy policy,
                            pkv_sched **out);
void pkv_sched_destroy(pkv_sched *sched);

/* Queues a request: prompt_len >= 0 tokens already computed when it is
 * admitted, then max_new_tokens >= 1 decode steps; it may be admitted from
 * step arrive_step on.  INVALID_ARG for bad sizes or an arrival before the
 * last queued one; SEQ_EXISTS if seq_id is queued, running or live in the
 * pool; OOM if its reservation exceeds the whole pool.  Nothing changes on
 * error. */
pkv_status pkv_sched_submit(pkv_sched *sched, int64_t seq_id, int32_t prompt_len,
                            int32_t max_new_tokens, int64_t arrive_step);

/* Ends a request early (an end token): a running one retires at the next
 * step, a queued one is dropped.  NO_SEQ if it is neither. */
pkv_status pkv_sched_finish(pkv_sched *sched, int64_t seq_id);

typedef struct pkv_sched_step_out {
    int64_t step;               /* the clock of this step (after an idle jump)       */
    int32_t n_running;          /* entries of seq_ids / new_slots / context_lens     */
    int32_t n_admitted;         /* entries of admitted                               */
    int32_t n_retired;          /* entries of retired                                */
} pkv_sched_step_out;

/* Runs one step.  Host output arrays of `capacity` >= max_batch entries:
 * seq_ids (the batch), new_slots (the slot of each sequence's new token, to
 * write its K/V at), context_lens (tokens after the append: what decode
 * attends over), admitted (joined this step: their prompt K/V goes to the
 * slots of tokens 0 .. prompt_len - 1), retired (left this step; their ids
 * may be reused).  With nothing to run, n_running is 0 and the clock stays.
 * INVALID_ARG for a short capacity or a NULL output (nothing changes); OOM
 * if the pool, used outside the scheduler, cannot cover the step -- then
 * only the retirements happened (n_retired and retired are valid). */
pkv_status pkv_sched_step(pkv_sched *sched, int32_t capacity, int64_t *seq_ids,
                          int64_t *new_slots, int32_t *context_lens, int64_t *admitted,
                          int64_t *retired, pkv_sched_step_out *out);

/* Block tables and context lengths of the batch the last step ran (the
 * running sequences, in batch order), as pkv_build_block_tables writes them:
 * block_tables_out (host, [capacity][max_blocks]), context_lens_out (host,
 * [capacity]); *n_out receives the batch size.  INVALID_ARG if capacity is
 * below it or a sequence has more than max_blocks pages. */
pkv_status pkv_sched_batch_tables(const pkv_sched *sched, int32_t capacity, int32_t max_blocks,
                                  int32_t *block_tables_out, int32_t *context_lens_out,
                                  int32_t *n_out);

typedef struct pkv_sched_stats {
    int64_t now;                /* the clock                                         */
    int32_t waiting;            /* queued requests                                   */
    int32_t running;            /* sequences in the batch (finished ones included
                                   until the step that retires them)                 */
    int64_t finished;           /* requests retired                                  */
    int64_t wait_sum;           /* over retired requests: step of the last token
                                   minus arrival step                                */
} pkv_sched_stats;

pkv_status pkv_sched_get_stats(const pkv_sched *sched, pkv_sched_stats *out);

/* ===================================================================== *
 * Host + device: one serving step per call over one layer's pools -- the
 * three parts of a step of "TensorRT-LLM 深度实战", section 3.2 (retire
 * finished sequences, admit waiting ones, one forward pass over the running
 * batch) with the attention of that pass: the scheduler step (pkv_sched_step),
 * the K/V of the admitted prompts' tokens and of every running sequence's new
 * token written at their slots (pkv_write_kv), and the decode of the batch
 * (pkv_paged_attn_decode).  The host work (scheduling, prompt slots, block
 * tables) runs in native code and lands in one slot of a caller-provided ring
 * of pinned host buffers, which one copy moves to device memory; the device
 * work is enqueued on `stream` without waiting for it, so the host may run up
 * to `ring` steps ahead of the GPU.  A slot is reused only after the copy
 * that read it has completed.  Use one stream for all steps of an object.
 * ===================================================================== */

typedef struct pkv_serve pkv_serve;

typedef struct pkv_serve_desc {
    pkv_sched *sched;           /* the step driver (and through it the pool); must
                                   outlive this object and be used by it alone      */
    int32_t max_blocks;         /* block-table row length of the decode; every
                                   sequence's pages must fit                        */
    int32_t max_prompt_tokens;  /* bound on the prompt tokens admitted in one step  */
    int32_t ring;               /* staging slots, >= 1                              */
    void *host_staging;         /* host, PINNED (hipHostMalloc or equivalent),
                                   ring x pkv_serve_slot_bytes bytes, 16-byte aligned */
    void *dev_staging;          /* device, pkv_serve_slot_bytes bytes, 16-byte aligned */
    pkv_decode_args decode;     /* template of each step's decode: q, pools,
                                   scales, out, workspace and merge counters (sized
                                   for batch = the scheduler's max_batch and
                                   max_context_len = max_blocks x page_size), head
                                   counts, head_dim, page_size, num_pages,
                                   num_splits, dtypes, scale.  batch, block_tables,
                                   context_lens, max_blocks and max_context_len are
                                   set by each step.                                 */
    pkv_write_args append;      /* template of each step's append of the new tokens:
                                   k_new / v_new [max_batch][Hkv][D] rows in batch
                                   order (and their scales for encoded rows), the
                                   pools and their scales, num_kv_heads, head_dim,
                                   page_size, num_pages, kv_dtype, src_dtype.  slots
                                   and n are set by each step.                       */
    const void *k_prompt;       /* device [max_prompt_tokens][Hkv][D], the append's
                                   src_dtype: the admitted prompts' K/V rows, packed
                                   prompt after prompt in admission order            */
    const void *v_prompt;
    const float *k_prompt_scale; /* their scales for encoded rows, else NULL        */
    const float *v_prompt_scale;
} pkv_serve_desc;

typedef struct pkv_serve_step_out {
    pkv_sched_step_out sched;   /* the scheduler step (clock, batch size, admitted,
                                   retired)                                          */
    int32_t prompt_tokens;      /* admitted prompts' tokens written this step       */
    int32_t max_context_len;    /* longest context of the batch after the append    */
    float slot_wait_us;         /* host time this call spent waiting for a staging
                                   slot (the host was `ring` steps ahead)            */
} pkv_serve_step_out;

/* Bytes of one staging slot for this descriptor (host_staging holds ring of
 * them, dev_staging one). */
pkv_status pkv_serve_slot_bytes(const pkv_serve_desc *desc, size_t *bytes);

/* Creates the step object (host memory and `ring` HIP events, owned until
 * pkv_serve_destroy).  INVALID_ARG for a bad descriptor, or the decode
 * template's own error for the largest step. */
pkv_status pkv_serve_create(const pkv_serve_desc *desc, pkv_serve **out);
void pkv_serve_destroy(pkv_serve *serve);

/* Runs one step.  seq_ids (host, may be NULL) receives the batch, in the order
 * of the rows of q, out and the new-token K/V; this step's admissions are its
 * last out->sched.n_admitted entries.  With nothing to run, no device work is
 * enqueued.  If the step's admitted prompts exceed max_prompt_tokens, or a
 * sequence has more pages than max_blocks, the scheduler step has happened but
 * nothing is enqueued (WORKSPACE / INVALID_ARG). */
pkv_status pkv_serve_step(pkv_serve *serve, void *stream, pkv_serve_step_out *out, int64_t *seq_ids);

#ifdef __cplusplus
}
#endif
#endif /* PAGEDKV_H */
