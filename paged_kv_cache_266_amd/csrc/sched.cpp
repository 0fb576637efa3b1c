// Continuous-batching step driver over the host page pool.
//
// One step, after "TensorRT-LLM 深度实战" (chenxutan.com), section 3.2:
// retire the finished sequences (their pages go back to the pool), admit
// waiting requests while the batch has room, then every running sequence
// appends one token -- its slot is where the step's new K/V goes, and its
// token count is what decode attends over.  The clock, arrival steps, the
// static-batching alternative and the wait statistic follow the request
// simulator of the aiqz.cc TensorRT-LLM explainer ("Python 演示").
//
// Admission reserves a request's whole life in pages (prompt + new tokens)
// against the free pages minus what running sequences are still owed, first
// come first served, so appends never fail while the scheduler is the pool's
// only user.  Every call checks before it commits.
#include <deque>
#include <new>
#include <unordered_set>
#include <vector>

#include "host.h"

namespace {

struct Request {
    int64_t id;
    int32_t prompt;
    int32_t max_new;
    int64_t arrive;
    int32_t generated = 0;
    bool stop = false;
    int64_t last_step = -1;
    int32_t reserve = 0;    // pages of its whole life
};

}  // namespace

struct pkv_sched {
    pkv_pool *pool = nullptr;
    int32_t max_batch = 0;
    pkv_sched_policy policy = PKV_SCHED_CONTINUOUS;
    int32_t page_size = 0;
    int64_t now = 0;
    int64_t finished = 0;
    int64_t wait_sum = 0;
    std::deque<Request> waiting;
    std::vector<Request> running;   // admission order
    std::unordered_set<int64_t> ids; // queued or running
};

using pkv::fail;

pkv_pool *pkv::sched_pool(const pkv_sched *s) { return s->pool; }
int32_t pkv::sched_max_batch(const pkv_sched *s) { return s->max_batch; }

static int32_t held_pages(const pkv_sched *s, int64_t id)
{
    int32_t pages = 0;
    pkv_seq_info(s->pool, id, nullptr, &pages);
    return pages;
}

// Pages the running sequences may still take.
static int64_t owed(const pkv_sched *s)
{
    int64_t o = 0;
    for (const Request &r : s->running)
        o += r.reserve - held_pages(s, r.id);
    return o;
}

extern "C" pkv_status pkv_sched_create(pkv_pool *pool, int32_t max_batch, pkv_sched_policy policy,
                                       pkv_sched **out)
{
    pkv::clear_error();
    if (!pool || !out || max_batch <= 0 || (policy != PKV_SCHED_CONTINUOUS && policy != PKV_SCHED_STATIC))
        return fail(PKV_ERR_INVALID_ARG, "pkv_sched_create: null pool / output, max_batch < 1 or bad policy");
    pkv_sched *s = new (std::nothrow) pkv_sched;
    if (!s)
        return fail(PKV_ERR_OOM, "pkv_sched_create: host allocation failed");
    s->pool = pool;
    s->max_batch = max_batch;
    s->policy = policy;
    s->page_size = pkv::pool_page_size(pool);
    *out = s;
    return PKV_OK;
}

extern "C" void pkv_sched_destroy(pkv_sched *sched) { delete sched; }

extern "C" pkv_status pkv_sched_submit(pkv_sched *s, int64_t seq_id, int32_t prompt_len, int32_t max_new_tokens,
                                       int64_t arrive_step)
{
    pkv::clear_error();
    if (!s || prompt_len < 0 || max_new_tokens <= 0 || arrive_step < 0)
        return fail(PKV_ERR_INVALID_ARG, "pkv_sched_submit: bad request");
    if (!s->waiting.empty() && arrive_step < s->waiting.back().arrive)
        return fail(PKV_ERR_INVALID_ARG, "pkv_sched_submit: arrival before the last queued request's");
    if ((int64_t)prompt_len + max_new_tokens > INT32_MAX)
        return fail(PKV_ERR_INVALID_ARG, "pkv_sched_submit: request too long");
    if (s->ids.count(seq_id) || pkv_seq_info(s->pool, seq_id, nullptr, nullptr) == PKV_OK)
        return fail(PKV_ERR_SEQ_EXISTS, "pkv_sched_submit: sequence id in use");
    pkv::clear_error();
    Request r;
    r.id = seq_id;
    r.prompt = prompt_len;
    r.max_new = max_new_tokens;
    r.arrive = arrive_step;
    const int64_t reserve = ((int64_t)prompt_len + max_new_tokens + s->page_size - 1) / s->page_size;
    if (reserve > pkv::pool_num_pages(s->pool))
        return fail(PKV_ERR_OOM, "pkv_sched_submit: the request needs more pages than the pool has");
    r.reserve = (int32_t)reserve;
    s->waiting.push_back(r);
    s->ids.insert(seq_id);
    return PKV_OK;
}

extern "C" pkv_status pkv_sched_finish(pkv_sched *s, int64_t seq_id)
{
    pkv::clear_error();
    if (!s)
        return fail(PKV_ERR_INVALID_ARG, "pkv_sched_finish: null scheduler");
    for (Request &r : s->running)
        if (r.id == seq_id) {
            r.stop = true;
            return PKV_OK;
        }
    for (auto it = s->waiting.begin(); it != s->waiting.end(); ++it)
        if (it->id == seq_id) {
            s->waiting.erase(it);
            s->ids.erase(seq_id);
            return PKV_OK;
        }
    return fail(PKV_ERR_NO_SEQ, "pkv_sched_finish: not queued or running");
}

extern "C" pkv_status pkv_sched_step(pkv_sched *s, int32_t capacity, int64_t *seq_ids, int64_t *new_slots,
                                     int32_t *context_lens, int64_t *admitted, int64_t *retired,
                                     pkv_sched_step_out *out)
{
    pkv::clear_error();
    if (!s || !seq_ids || !new_slots || !context_lens || !admitted || !retired || !out)
        return fail(PKV_ERR_INVALID_ARG, "pkv_sched_step: null argument");
    if (capacity < s->max_batch)
        return fail(PKV_ERR_INVALID_ARG, "pkv_sched_step: output capacity below max_batch");
    *out = pkv_sched_step_out{};

    // 1. retire
    std::vector<Request> keep;
    keep.reserve(s->running.size());
    for (Request &r : s->running) {
        if (r.generated >= r.max_new || r.stop) {
            pkv_seq_release(s->pool, r.id);
            retired[out->n_retired++] = r.id;
            s->ids.erase(r.id);
            s->finished += 1;
            if (r.last_step >= 0)
                s->wait_sum += r.last_step - r.arrive;
        } else {
            keep.push_back(r);
        }
    }
    s->running.swap(keep);

    // idle: the clock jumps to the next arrival
    if (s->running.empty() && !s->waiting.empty() && s->waiting.front().arrive > s->now)
        s->now = s->waiting.front().arrive;

    // 2. plan the admissions (first come first served, batch room, reservations)
    const int64_t free_pages = pkv_free_page_count(s->pool);
    int64_t avail = free_pages - owed(s);
    size_t n_admit = 0;
    const bool may_admit = s->policy == PKV_SCHED_CONTINUOUS || s->running.empty();
    while (may_admit && s->running.size() + n_admit < (size_t)s->max_batch && n_admit < s->waiting.size()) {
        const Request &r = s->waiting[n_admit];
        if (r.arrive > s->now || avail < r.reserve)
            break;
        avail -= r.reserve;
        ++n_admit;
    }
    // pages the step takes: the admitted prompts, plus one for every
    // sequence whose next token starts a page
    int64_t need = 0;
    for (size_t i = 0; i < n_admit; ++i) {
        const Request &r = s->waiting[i];
        need += (r.prompt + s->page_size - 1) / s->page_size + (r.prompt % s->page_size == 0 ? 1 : 0);
    }
    for (const Request &r : s->running) {
        int32_t tokens = 0;
        pkv_seq_info(s->pool, r.id, &tokens, nullptr);
        need += tokens % s->page_size == 0 ? 1 : 0;
    }
    if (need > free_pages)
        return fail(PKV_ERR_OOM, "pkv_sched_step: the pool cannot cover this step (used outside the scheduler?)");

    // 3. commit: admit, then one token for every running sequence
    for (size_t i = 0; i < n_admit; ++i) {
        Request r = s->waiting.front();
        s->waiting.pop_front();
        const pkv_status st = pkv_seq_alloc(s->pool, r.id, r.prompt, nullptr);
        if (st != PKV_OK)   // excluded by the checks above
            return st;
        admitted[out->n_admitted++] = r.id;
        s->running.push_back(r);
    }
    out->step = s->now;
    if (s->running.empty())
        return PKV_OK;
    for (Request &r : s->running) {
        int64_t slot = -1;
        const pkv_status st = pkv_append_tokens(s->pool, r.id, 1, &slot);
        if (st != PKV_OK)   // excluded by the checks above
            return st;
        int32_t tokens = 0;
        pkv_seq_info(s->pool, r.id, &tokens, nullptr);
        r.generated += 1;
        r.last_step = s->now;
        seq_ids[out->n_running] = r.id;
        new_slots[out->n_running] = slot;
        context_lens[out->n_running] = tokens;
        out->n_running++;
    }
    s->now += 1;
    return PKV_OK;
}

extern "C" pkv_status pkv_sched_batch_tables(const pkv_sched *s, int32_t capacity, int32_t max_blocks,
                                             int32_t *block_tables_out, int32_t *context_lens_out,
                                             int32_t *n_out)
{
    pkv::clear_error();
    if (!s || !n_out || (!s->running.empty() && (!block_tables_out || !context_lens_out)))
        return fail(PKV_ERR_INVALID_ARG, "pkv_sched_batch_tables: null argument");
    const int32_t n = (int32_t)s->running.size();
    if (capacity < n)
        return fail(PKV_ERR_INVALID_ARG, "pkv_sched_batch_tables: capacity below the batch size");
    *n_out = n;
    if (n == 0)
        return PKV_OK;
    std::vector<int64_t> ids((size_t)n);
    for (int32_t i = 0; i < n; ++i)
        ids[(size_t)i] = s->running[(size_t)i].id;
    return pkv_build_block_tables(s->pool, ids.data(), n, max_blocks, block_tables_out, context_lens_out);
}

extern "C" pkv_status pkv_sched_get_stats(const pkv_sched *s, pkv_sched_stats *out)
{
    pkv::clear_error();
    if (!s || !out)
        return fail(PKV_ERR_INVALID_ARG, "pkv_sched_get_stats: null argument");
    out->now = s->now;
    out->waiting = (int32_t)s->waiting.size();
    out->running = (int32_t)s->running.size();
    out->finished = s->finished;
    out->wait_sum = s->wait_sum;
    return PKV_OK;
}
