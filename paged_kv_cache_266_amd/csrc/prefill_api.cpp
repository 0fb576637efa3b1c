// C entry of the chunked-prefill kernel: argument checks and launch.
#include <cmath>
#include <cstdio>

#include "internal.h"

using pkv::fail;

static pkv_status launch_failed(int err)
{
    char buf[256];
    std::snprintf(buf, sizeof buf, "pkv_paged_prefill: %s", hipGetErrorString((hipError_t)err));
    fail(PKV_ERR_DEVICE, buf);
    return PKV_ERR_DEVICE;
}

extern "C" pkv_status pkv_paged_prefill(const pkv_prefill_args *a, void *stream)
{
    pkv::clear_error();
    if (!a)
        return fail(PKV_ERR_INVALID_ARG, "pkv_paged_prefill: null argument struct");
    if (a->batch < 0 || a->n_q < 0 || a->num_q_heads <= 0 || a->num_kv_heads <= 0 || a->head_dim <= 0 ||
        a->page_size <= 0 || a->num_pages <= 0 || a->max_blocks < 0 || a->max_context_len < 0 || a->max_q_len < 0)
        return fail(PKV_ERR_INVALID_ARG, "pkv_paged_prefill: bad sizes");
    if (a->num_q_heads % a->num_kv_heads)
        return fail(PKV_ERR_INVALID_ARG, "pkv_paged_prefill: num_q_heads must be a multiple of num_kv_heads");
    if ((int64_t)a->max_context_len > (int64_t)a->max_blocks * a->page_size)
        return fail(PKV_ERR_INVALID_ARG, "pkv_paged_prefill: max_context_len exceeds max_blocks * page_size");
    if (a->max_q_len > a->max_context_len)
        return fail(PKV_ERR_INVALID_ARG, "pkv_paged_prefill: max_q_len exceeds max_context_len");
    if (!(std::isfinite(a->scale)))
        return fail(PKV_ERR_INVALID_ARG, "pkv_paged_prefill: scale must be finite");
    const int group = a->num_q_heads / a->num_kv_heads;
    if (!pkv::prefill_instantiated(a->head_dim, a->page_size, group, a->q_dtype, a->kv_dtype))
        return fail(PKV_ERR_UNSUPPORTED, "pkv_paged_prefill: head_dim 64 or 128, page_size 16 or 64, group 1/2/4/8, "
                                         "f16 or bf16 q with K/V of the same type, int8 or fp8 E4M3");
    if (a->batch == 0 || a->n_q == 0 || a->max_q_len == 0)
        return PKV_OK;
    if (!a->q || !a->k_pool || !a->v_pool || !a->block_tables || !a->q_start || !a->context_lens || !a->out)
        return fail(PKV_ERR_INVALID_ARG, "pkv_paged_prefill: null device pointer");
    if ((uintptr_t)a->q % 16 || (uintptr_t)a->k_pool % 16 || (uintptr_t)a->v_pool % 16 || (uintptr_t)a->out % 16)
        return fail(PKV_ERR_INVALID_ARG, "pkv_paged_prefill: q, pools and out must be 16-byte aligned");
    if (((uintptr_t)a->block_tables & 3u) || ((uintptr_t)a->q_start & 3u) || ((uintptr_t)a->context_lens & 3u))
        return fail(PKV_ERR_INVALID_ARG, "pkv_paged_prefill: int32 arrays must be 4-byte aligned");
    const bool byte_kv = a->kv_dtype == PKV_I8 || a->kv_dtype == PKV_FP8_E4M3;
    if (byte_kv && (!a->k_scale || !a->v_scale || (uintptr_t)a->k_scale % 4 || (uintptr_t)a->v_scale % 4))
        return fail(PKV_ERR_INVALID_ARG, "pkv_paged_prefill: int8 / fp8 K/V need 4-byte aligned k_scale and v_scale");
    // one launch: grid (query blocks, KV heads, sequences)
    if (a->batch > 65535 || a->num_kv_heads > 65535)
        return fail(PKV_ERR_INVALID_ARG, "pkv_paged_prefill: batch and num_kv_heads must be at most 65535");
    pkv::PrefillParams p{};
    p.q = a->q;
    p.k_pool = a->k_pool;
    p.v_pool = a->v_pool;
    p.block_tables = a->block_tables;
    p.q_start = a->q_start;
    p.context_lens = a->context_lens;
    p.out = a->out;
    p.batch = a->batch;
    p.n_q = a->n_q;
    p.num_q_heads = a->num_q_heads;
    p.num_kv_heads = a->num_kv_heads;
    p.num_pages = a->num_pages;
    p.max_blocks = a->max_blocks;
    p.max_context_len = a->max_context_len;
    p.max_q_len = a->max_q_len;
    p.q_dtype = a->q_dtype;
    p.kv_dtype = a->kv_dtype;
    p.head_dim = a->head_dim;
    p.k_scale = a->k_scale;
    p.v_scale = a->v_scale;
    p.scale_log2 = a->scale * 1.4426950408889634f;
    const int err = pkv::launch_prefill(p, a->page_size, group, stream);
    return err ? launch_failed(err) : PKV_OK;
}
