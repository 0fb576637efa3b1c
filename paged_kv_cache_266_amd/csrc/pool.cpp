// Host page pool: the free-page list and per-sequence page tables of
// "TensorRT-LLM 深度实战" (chenxutan.com), section 3.1.
//
// The free list is a stack: pages are handed out from its end and released
// pages are pushed back onto its end in the sequence's page order.  Every
// mutating call checks everything first and then commits, so an error leaves
// the pool exactly as it was (the section's sketch would orphan popped pages
// on a mid-allocation failure, and its append never checks for exhaustion).
//
// Block reuse: a page may be owned by several sequences (pkv_seq_fork); it
// returns to the free list with its last owner.  Appending into a partly
// filled shared last page first replaces it, in the appending sequence, by a
// fresh page (taken before any overflow pages) whose contents the caller
// copies on the device (pkv_copy_pages).
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "host.h"

struct pkv_pool {
    int32_t num_pages = 0;
    int32_t page_size = 0;
    std::vector<int32_t> free_list;  // bottom .. top; top is handed out next
    struct Seq {
        std::vector<int32_t> pages;
        int32_t tokens = 0;
    };
    std::unordered_map<int64_t, Seq> seqs;
    std::vector<int32_t> owners;     // per page: sequences holding it (0 = free)
};

using pkv::fail;

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

extern "C" pkv_status pkv_pool_create(const pkv_pool_desc *desc, pkv_pool **out)
{
    pkv::clear_error();
    if (!desc || !out)
        return fail(PKV_ERR_INVALID_ARG, "pkv_pool_create: null descriptor or output");
    if (desc->num_pages <= 0 || desc->page_size <= 0)
        return fail(PKV_ERR_INVALID_ARG, "pkv_pool_create: num_pages and page_size must be > 0");
    pkv_pool *p = new (std::nothrow) pkv_pool;
    if (!p)
        return fail(PKV_ERR_OOM, "pkv_pool_create: host allocation failed");
    p->num_pages = desc->num_pages;
    p->page_size = desc->page_size;
    p->free_list.resize((size_t)desc->num_pages);
    p->owners.assign((size_t)desc->num_pages, 0);
    if (desc->initial_free_order) {
        std::vector<char> seen((size_t)desc->num_pages, 0);
        for (int32_t i = 0; i < desc->num_pages; ++i) {
            int32_t pg = desc->initial_free_order[i];
            if (pg < 0 || pg >= desc->num_pages || seen[(size_t)pg]) {
                delete p;
                return fail(PKV_ERR_INVALID_ARG,
                            "pkv_pool_create: initial_free_order is not a permutation of the pages");
            }
            seen[(size_t)pg] = 1;
            p->free_list[(size_t)i] = pg;
        }
    } else {
        for (int32_t i = 0; i < desc->num_pages; ++i)
            p->free_list[(size_t)i] = i;
    }
    *out = p;
    return PKV_OK;
}

extern "C" void pkv_pool_destroy(pkv_pool *pool) { delete pool; }

int32_t pkv::pool_page_size(const pkv_pool *pool) { return pool->page_size; }
int32_t pkv::pool_num_pages(const pkv_pool *pool) { return pool->num_pages; }

static void write_slots(const pkv_pool::Seq &s, int32_t ps, int32_t first, int32_t count,
                        int64_t *slots_out)
{
    if (!slots_out)
        return;
    for (int32_t i = 0; i < count; ++i) {
        int32_t t = first + i;
        slots_out[i] = (int64_t)s.pages[(size_t)(t / ps)] * ps + t % ps;
    }
}

extern "C" pkv_status pkv_seq_alloc(pkv_pool *pool, int64_t seq_id, int32_t num_tokens,
                                    int64_t *slots_out)
{
    pkv::clear_error();
    if (!pool || num_tokens < 0)
        return fail(PKV_ERR_INVALID_ARG, "pkv_seq_alloc: null pool or negative token count");
    if (pool->seqs.count(seq_id))
        return fail(PKV_ERR_SEQ_EXISTS, "pkv_seq_alloc: sequence id already allocated");
    int64_t need = ceil_div(num_tokens, pool->page_size);
    if (need > (int64_t)pool->free_list.size())
        return fail(PKV_ERR_OOM, "pkv_seq_alloc: not enough free pages");
    pkv_pool::Seq s;
    s.pages.reserve((size_t)need);
    for (int64_t i = 0; i < need; ++i) {
        s.pages.push_back(pool->free_list.back());
        pool->owners[(size_t)pool->free_list.back()] = 1;
        pool->free_list.pop_back();
    }
    s.tokens = num_tokens;
    auto it = pool->seqs.emplace(seq_id, std::move(s)).first;
    write_slots(it->second, pool->page_size, 0, num_tokens, slots_out);
    return PKV_OK;
}

// Append n_new tokens; *copy_src / *copy_dst receive the page pair to copy
// (-1, -1 when none).  With allow_copy false an append that needs a copy is
// refused (PKV_ERR_SHARED_PAGE).
static pkv_status append(pkv_pool *pool, int64_t seq_id, int32_t n_new, int64_t *slots_out, bool allow_copy,
                         int32_t *copy_src, int32_t *copy_dst, const char *who)
{
    if (!pool || n_new < 0)
        return fail(PKV_ERR_INVALID_ARG, "append: null pool or negative token count");
    auto it = pool->seqs.find(seq_id);
    if (it == pool->seqs.end())
        return fail(PKV_ERR_NO_SEQ, "append: unknown sequence id");
    pkv_pool::Seq &s = it->second;
    const int64_t usage = s.tokens;
    const int64_t capacity = (int64_t)s.pages.size() * pool->page_size;
    if (usage + n_new > INT32_MAX)
        return fail(PKV_ERR_INVALID_ARG, "append: token count overflows int32");
    const bool copy = n_new > 0 && usage % pool->page_size != 0 && pool->owners[(size_t)s.pages.back()] > 1;
    if (copy && !allow_copy)
        return fail(PKV_ERR_SHARED_PAGE, who);
    const int64_t over = usage + n_new > capacity ? ceil_div(usage + n_new - capacity, pool->page_size) : 0;
    if (over + (copy ? 1 : 0) > (int64_t)pool->free_list.size())
        return fail(PKV_ERR_OOM, "append: not enough free pages");
    int32_t src = -1, dst = -1;
    if (copy) {
        src = s.pages.back();
        dst = pool->free_list.back();
        pool->free_list.pop_back();
        pool->owners[(size_t)src] -= 1;
        pool->owners[(size_t)dst] = 1;
        s.pages.back() = dst;
    }
    for (int64_t i = 0; i < over; ++i) {
        s.pages.push_back(pool->free_list.back());
        pool->owners[(size_t)pool->free_list.back()] = 1;
        pool->free_list.pop_back();
    }
    s.tokens = (int32_t)(usage + n_new);
    write_slots(s, pool->page_size, (int32_t)usage, n_new, slots_out);
    if (copy_src)
        *copy_src = src;
    if (copy_dst)
        *copy_dst = dst;
    return PKV_OK;
}

extern "C" pkv_status pkv_append_tokens(pkv_pool *pool, int64_t seq_id, int32_t n_new,
                                        int64_t *slots_out)
{
    pkv::clear_error();
    return append(pool, seq_id, n_new, slots_out, false, nullptr, nullptr,
                  "pkv_append_tokens: the last page is shared and partly filled; "
                  "use pkv_append_tokens_cow");
}

extern "C" pkv_status pkv_append_tokens_cow(pkv_pool *pool, int64_t seq_id, int32_t n_new,
                                            int64_t *slots_out, int32_t *copy_src, int32_t *copy_dst)
{
    pkv::clear_error();
    return append(pool, seq_id, n_new, slots_out, true, copy_src, copy_dst, "");
}

extern "C" pkv_status pkv_seq_fork(pkv_pool *pool, int64_t parent_id, int64_t child_id)
{
    pkv::clear_error();
    if (!pool)
        return fail(PKV_ERR_INVALID_ARG, "pkv_seq_fork: null pool");
    auto it = pool->seqs.find(parent_id);
    if (it == pool->seqs.end())
        return fail(PKV_ERR_NO_SEQ, "pkv_seq_fork: unknown parent sequence id");
    if (pool->seqs.count(child_id))
        return fail(PKV_ERR_SEQ_EXISTS, "pkv_seq_fork: child sequence id already allocated");
    pkv_pool::Seq child = it->second;   // copy before inserting (insertion may rehash)
    for (int32_t pg : child.pages)
        pool->owners[(size_t)pg] += 1;
    pool->seqs.emplace(child_id, std::move(child));
    return PKV_OK;
}

extern "C" int32_t pkv_page_owners(const pkv_pool *pool, int32_t page)
{
    if (!pool || page < 0 || page >= pool->num_pages)
        return -1;
    return pool->owners[(size_t)page];
}

extern "C" pkv_status pkv_seq_release(pkv_pool *pool, int64_t seq_id)
{
    pkv::clear_error();
    if (!pool)
        return fail(PKV_ERR_INVALID_ARG, "pkv_seq_release: null pool");
    auto it = pool->seqs.find(seq_id);
    if (it == pool->seqs.end())
        return fail(PKV_ERR_NO_SEQ, "pkv_seq_release: unknown sequence id");
    for (int32_t pg : it->second.pages)
        if (--pool->owners[(size_t)pg] == 0)
            pool->free_list.push_back(pg);
    pool->seqs.erase(it);
    return PKV_OK;
}

extern "C" pkv_status pkv_seq_info(const pkv_pool *pool, int64_t seq_id, int32_t *num_tokens,
                                   int32_t *num_pages)
{
    pkv::clear_error();
    if (!pool)
        return fail(PKV_ERR_INVALID_ARG, "pkv_seq_info: null pool");
    auto it = pool->seqs.find(seq_id);
    if (it == pool->seqs.end())
        return fail(PKV_ERR_NO_SEQ, "pkv_seq_info: unknown sequence id");
    if (num_tokens)
        *num_tokens = it->second.tokens;
    if (num_pages)
        *num_pages = (int32_t)it->second.pages.size();
    return PKV_OK;
}

extern "C" pkv_status pkv_seq_pages(const pkv_pool *pool, int64_t seq_id, int32_t *pages_out,
                                    int32_t capacity, int32_t *n_pages)
{
    pkv::clear_error();
    if (!pool || !n_pages || capacity < 0 || (capacity > 0 && !pages_out))
        return fail(PKV_ERR_INVALID_ARG, "pkv_seq_pages: bad arguments");
    auto it = pool->seqs.find(seq_id);
    if (it == pool->seqs.end())
        return fail(PKV_ERR_NO_SEQ, "pkv_seq_pages: unknown sequence id");
    const auto &pg = it->second.pages;
    if ((int64_t)pg.size() > capacity)
        return fail(PKV_ERR_INVALID_ARG, "pkv_seq_pages: capacity too small");
    if (!pg.empty())
        std::memcpy(pages_out, pg.data(), pg.size() * sizeof(int32_t));
    *n_pages = (int32_t)pg.size();
    return PKV_OK;
}

extern "C" int32_t pkv_free_page_count(const pkv_pool *pool)
{
    return pool ? (int32_t)pool->free_list.size() : 0;
}

extern "C" pkv_status pkv_free_pages(const pkv_pool *pool, int32_t *out, int32_t capacity,
                                     int32_t *count)
{
    pkv::clear_error();
    if (!pool || !count || capacity < 0 || (capacity > 0 && !out))
        return fail(PKV_ERR_INVALID_ARG, "pkv_free_pages: bad arguments");
    if ((int64_t)pool->free_list.size() > capacity)
        return fail(PKV_ERR_INVALID_ARG, "pkv_free_pages: capacity too small");
    if (!pool->free_list.empty())
        std::memcpy(out, pool->free_list.data(), pool->free_list.size() * sizeof(int32_t));
    *count = (int32_t)pool->free_list.size();
    return PKV_OK;
}

extern "C" pkv_status pkv_build_block_tables(const pkv_pool *pool, const int64_t *seq_ids,
                                             int32_t batch, int32_t max_blocks,
                                             int32_t *block_tables_out, int32_t *context_lens_out)
{
    pkv::clear_error();
    if (!pool || batch < 0 || max_blocks < 0 ||
        (batch > 0 && (!seq_ids || !block_tables_out || !context_lens_out)))
        return fail(PKV_ERR_INVALID_ARG, "pkv_build_block_tables: bad arguments");
    // check every sequence before writing anything
    for (int32_t b = 0; b < batch; ++b) {
        auto it = pool->seqs.find(seq_ids[b]);
        if (it == pool->seqs.end())
            return fail(PKV_ERR_NO_SEQ, "pkv_build_block_tables: unknown sequence id");
        if ((int64_t)it->second.pages.size() > max_blocks)
            return fail(PKV_ERR_INVALID_ARG, "pkv_build_block_tables: a sequence has more than max_blocks pages");
    }
    for (int32_t b = 0; b < batch; ++b) {
        const auto &s = pool->seqs.find(seq_ids[b])->second;
        int32_t *row = block_tables_out + (size_t)b * (size_t)max_blocks;
        size_t np = s.pages.size();
        for (size_t j = 0; j < (size_t)max_blocks; ++j)
            row[j] = j < np ? s.pages[j] : -1;
        context_lens_out[b] = s.tokens;
    }
    return PKV_OK;
}

extern "C" int64_t pkv_kv_bytes(int32_t layers, int32_t kv_heads, int32_t head_dim,
                                int64_t tokens, int32_t batch, pkv_dtype dtype)
{
    int64_t e;
    switch (dtype) {
    case PKV_F16:
    case PKV_BF16: e = 2; break;
    case PKV_I8:
    case PKV_FP8_E4M3: e = 1; break;
    default: return -1;
    }
    if (layers < 0 || kv_heads < 0 || head_dim < 0 || tokens < 0 || batch < 0)
        return -1;
    // 2 (K and V) x layers x heads x head_dim x tokens x batch x bytes, with
    // an overflow check at every product
    int64_t factors[] = {layers, kv_heads, head_dim, tokens, batch, e};
    int64_t acc = 2;
    for (int64_t f : factors) {
        if (f != 0 && acc > INT64_MAX / f)
            return -1;
        acc *= f;
    }
    return acc;
}
