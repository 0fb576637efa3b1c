// One serving step per call: the scheduler step, the staging of the step's
// per-sequence data into device memory, the K/V appends and the decode of
// the batch -- the three parts of a step of "TensorRT-LLM 深度实战"
// (chenxutan.com), section 3.2 (retire finished sequences, admit waiting
// ones, one forward pass over the running batch), for one layer's pools.
//
// The host part of a step runs here in native code: the scheduler step, the
// slots of the admitted prompts' tokens and the block tables are written
// straight into a slot of a caller-provided ring of pinned host buffers, and
// one copy moves that slot to device memory.  The device part is enqueued on
// the caller's stream without waiting for it, so the host runs up to `ring`
// steps ahead of the GPU; a slot is reused only once the copy that read it
// has completed (an event per slot, polled).
#include <hip/hip_runtime.h>

#include <chrono>
#include <cstdio>
#include <new>
#include <thread>
#include <vector>

#include "internal.h"

using pkv::fail;

struct pkv_serve {
    pkv_serve_desc d{};
    int32_t max_batch = 0;
    int32_t page_size = 0;
    size_t off_ctx = 0, off_bt = 0, off_prompt = 0, slot_bytes = 0;
    std::vector<hipEvent_t> copied;   // per slot: the copy that last read it
    std::vector<bool> pending;
    int64_t count = 0;                // steps staged so far
    std::vector<int64_t> ids, admitted, retired;
    std::vector<int32_t> pages;
};

namespace {

struct SlotLayout {
    size_t off_ctx, off_bt, off_prompt, bytes;
};

// One staging slot: new tokens' slots (int64 [max_batch]), context lengths
// (int32 [max_batch]), block tables (int32 [max_batch][max_blocks]), the
// admitted prompts' token slots (int64 [max_prompt_tokens]).
SlotLayout slot_layout(int32_t max_batch, int32_t max_blocks, int32_t max_prompt_tokens)
{
    auto up = [](size_t x, size_t a) { return (x + a - 1) / a * a; };
    SlotLayout L;
    L.off_ctx = up(8 * (size_t)max_batch, 16);
    L.off_bt = up(L.off_ctx + 4 * (size_t)max_batch, 16);
    L.off_prompt = up(L.off_bt + 4 * (size_t)max_batch * (size_t)max_blocks, 16);
    L.bytes = up(L.off_prompt + 8 * (size_t)max_prompt_tokens, 256);
    return L;
}

pkv_status check_desc(const pkv_serve_desc *d)
{
    if (!d || !d->sched)
        return fail(PKV_ERR_INVALID_ARG, "serve: null descriptor or scheduler");
    if (d->max_blocks <= 0 || d->max_prompt_tokens < 0 || d->ring < 1)
        return fail(PKV_ERR_INVALID_ARG, "serve: max_blocks >= 1, max_prompt_tokens >= 0 and ring >= 1 required");
    return PKV_OK;
}

pkv_status device_error(hipError_t e, const char *where)
{
    char buf[256];
    std::snprintf(buf, sizeof buf, "%s: %s", where, hipGetErrorString(e));
    return fail(PKV_ERR_DEVICE, buf);
}

}  // namespace

extern "C" pkv_status pkv_serve_slot_bytes(const pkv_serve_desc *d, size_t *bytes)
{
    pkv::clear_error();
    pkv_status st = check_desc(d);
    if (st != PKV_OK)
        return st;
    if (!bytes)
        return fail(PKV_ERR_INVALID_ARG, "pkv_serve_slot_bytes: null output");
    *bytes = slot_layout(pkv::sched_max_batch(d->sched), d->max_blocks, d->max_prompt_tokens).bytes;
    return PKV_OK;
}

extern "C" pkv_status pkv_serve_create(const pkv_serve_desc *d, pkv_serve **out)
{
    pkv::clear_error();
    pkv_status st = check_desc(d);
    if (st != PKV_OK)
        return st;
    if (!out)
        return fail(PKV_ERR_INVALID_ARG, "pkv_serve_create: null output");
    if (!d->host_staging || !d->dev_staging || ((uintptr_t)d->host_staging & 15u) || ((uintptr_t)d->dev_staging & 15u))
        return fail(PKV_ERR_INVALID_ARG, "pkv_serve_create: staging buffers missing or not 16-byte aligned");
    const int32_t max_batch = pkv::sched_max_batch(d->sched);
    const int32_t page_size = pkv::pool_page_size(pkv::sched_pool(d->sched));
    const SlotLayout L = slot_layout(max_batch, d->max_blocks, d->max_prompt_tokens);
    if (d->decode.page_size != page_size || d->append.page_size != page_size)
        return fail(PKV_ERR_INVALID_ARG, "pkv_serve_create: decode / append page_size differs from the pool's");
    if (!d->append.k_new || !d->append.v_new ||
        (d->max_prompt_tokens > 0 && (!d->k_prompt || !d->v_prompt)))
        return fail(PKV_ERR_INVALID_ARG, "pkv_serve_create: new-token or prompt K/V rows missing");
    // the decode template must be valid for the largest step
    pkv_decode_args a = d->decode;
    a.batch = max_batch;
    a.block_tables = (const int32_t *)((const char *)d->dev_staging + L.off_bt);
    a.context_lens = (const int32_t *)((const char *)d->dev_staging + L.off_ctx);
    a.max_blocks = d->max_blocks;
    a.max_context_len = d->max_blocks * page_size;
    st = pkv_decode_validate(&a);
    if (st != PKV_OK)
        return st;
    pkv_serve *s = new (std::nothrow) pkv_serve;
    if (!s)
        return fail(PKV_ERR_OOM, "pkv_serve_create: out of host memory");
    s->d = *d;
    s->max_batch = max_batch;
    s->page_size = page_size;
    s->off_ctx = L.off_ctx;
    s->off_bt = L.off_bt;
    s->off_prompt = L.off_prompt;
    s->slot_bytes = L.bytes;
    s->ids.resize((size_t)max_batch);
    s->admitted.resize((size_t)max_batch);
    s->retired.resize((size_t)max_batch);
    s->pages.resize((size_t)d->max_blocks);
    s->pending.assign((size_t)d->ring, false);
    for (int32_t i = 0; i < d->ring; ++i) {
        hipEvent_t e = nullptr;
        const hipError_t err = hipEventCreateWithFlags(&e, hipEventDisableTiming);
        if (err != hipSuccess) {
            pkv_serve_destroy(s);
            return device_error(err, "pkv_serve_create: hipEventCreateWithFlags");
        }
        s->copied.push_back(e);
    }
    *out = s;
    return PKV_OK;
}

extern "C" void pkv_serve_destroy(pkv_serve *s)
{
    if (!s)
        return;
    for (hipEvent_t e : s->copied)
        if (e)
            (void)hipEventDestroy(e);
    delete s;
}

extern "C" pkv_status pkv_serve_step(pkv_serve *s, void *stream, pkv_serve_step_out *out, int64_t *seq_ids)
{
    pkv::clear_error();
    if (!s || !out)
        return fail(PKV_ERR_INVALID_ARG, "pkv_serve_step: null argument");
    const pkv_serve_desc &d = s->d;
    const size_t k = (size_t)(s->count % d.ring);
    char *host = (char *)d.host_staging + k * s->slot_bytes;
    // this slot is free once the copy that last read it has completed
    out->slot_wait_us = 0.0f;
    if (s->pending[k]) {
        hipError_t e = hipEventQuery(s->copied[k]);
        if (e == hipErrorNotReady) {
            const auto t0 = std::chrono::steady_clock::now();
            while ((e = hipEventQuery(s->copied[k])) == hipErrorNotReady)
                std::this_thread::yield();
            out->slot_wait_us =
                std::chrono::duration<float, std::micro>(std::chrono::steady_clock::now() - t0).count();
        }
        if (e != hipSuccess)
            return device_error(e, "pkv_serve_step: waiting for a staging slot");
        s->pending[k] = false;
    }
    // the scheduler step writes the new tokens' slots and the context
    // lengths straight into the staging slot
    int64_t *new_slots = (int64_t *)host;
    int32_t *ctx = (int32_t *)(host + s->off_ctx);
    int32_t *bt = (int32_t *)(host + s->off_bt);
    int64_t *prompt_slots = (int64_t *)(host + s->off_prompt);
    pkv_status st = pkv_sched_step(d.sched, s->max_batch, s->ids.data(), new_slots, ctx, s->admitted.data(),
                                   s->retired.data(), &out->sched);
    out->prompt_tokens = 0;
    out->max_context_len = 0;
    if (st != PKV_OK)
        return st;
    const int32_t n = out->sched.n_running;
    if (seq_ids)
        for (int32_t i = 0; i < n; ++i)
            seq_ids[i] = s->ids[(size_t)i];
    if (n == 0)
        return PKV_OK;
    pkv_pool *pool = pkv::sched_pool(d.sched);
    const int32_t ps = s->page_size;
    int32_t max_ctx = 0;
    // block tables (the batch is in admission order: this step's admissions
    // are its last n_admitted entries) and the admitted prompts' slots
    int32_t prompt_tokens = 0;
    for (int32_t i = 0; i < n; ++i) {
        int32_t np = 0;
        st = pkv_seq_pages(pool, s->ids[(size_t)i], s->pages.data(), d.max_blocks, &np);
        if (st != PKV_OK)
            return fail(st, "pkv_serve_step: a sequence has more pages than max_blocks (the step was scheduled, "
                            "nothing was enqueued)");
        int32_t *row = bt + (size_t)i * d.max_blocks;
        for (int32_t j = 0; j < np; ++j)
            row[j] = s->pages[(size_t)j];
        for (int32_t j = np; j < d.max_blocks; ++j)
            row[j] = -1;
        max_ctx = ctx[i] > max_ctx ? ctx[i] : max_ctx;
        if (i >= n - out->sched.n_admitted) {
            const int32_t prompt = ctx[i] - 1;   // the prompt; the step appended one token after it
            if (prompt_tokens + prompt > d.max_prompt_tokens)
                return fail(PKV_ERR_WORKSPACE, "pkv_serve_step: admitted prompts exceed max_prompt_tokens (the "
                                               "step was scheduled, nothing was enqueued)");
            for (int32_t t = 0; t < prompt; ++t)
                prompt_slots[prompt_tokens + t] = (int64_t)s->pages[(size_t)(t / ps)] * ps + t % ps;
            prompt_tokens += prompt;
        }
    }
    out->prompt_tokens = prompt_tokens;
    out->max_context_len = max_ctx;
    hipStream_t hs = (hipStream_t)stream;
    const size_t bytes = s->off_prompt + 8 * (size_t)prompt_tokens;
    hipError_t e = hipMemcpyAsync(d.dev_staging, host, bytes, hipMemcpyHostToDevice, hs);
    if (e != hipSuccess)
        return device_error(e, "pkv_serve_step: hipMemcpyAsync");
    e = hipEventRecord(s->copied[k], hs);
    if (e != hipSuccess)
        return device_error(e, "pkv_serve_step: hipEventRecord");
    s->pending[k] = true;
    ++s->count;
    const char *dev = (const char *)d.dev_staging;
    if (prompt_tokens > 0) {
        pkv_write_args w = d.append;
        w.k_new = d.k_prompt;
        w.v_new = d.v_prompt;
        w.k_scale_new = d.k_prompt_scale;
        w.v_scale_new = d.v_prompt_scale;
        w.slots = (const int64_t *)(dev + s->off_prompt);
        w.n = prompt_tokens;
        st = pkv_write_kv(&w, stream);
        if (st != PKV_OK)
            return st;
    }
    pkv_write_args w = d.append;
    w.slots = (const int64_t *)dev;
    w.n = n;
    st = pkv_write_kv(&w, stream);
    if (st != PKV_OK)
        return st;
    pkv_decode_args a = d.decode;
    a.batch = n;
    a.block_tables = (const int32_t *)(dev + s->off_bt);
    a.context_lens = (const int32_t *)(dev + s->off_ctx);
    a.max_blocks = d.max_blocks;
    a.max_context_len = d.max_blocks * ps;
    return pkv_paged_attn_decode(&a, stream);
}
