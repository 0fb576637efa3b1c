// C ABI entry points of libpagedkv for the device side: argument validation,
// choice of kernel instantiation and of the work split, launches.
//
// The decode step is the masked_mha role of "TensorRT-LLM 推理加速实战"
// (socake.github.io), section 7.2, computing the fused attention of
// "TensorRT-LLM 深度实战" (chenxutan.com), section 3.3, over K/V reached
// through the page tables of section 3.1 of the same page.  The batch's
// tiles are divided evenly among a persistent grid of waves; sequences longer
// than a wave's share -- the >128k-token contexts of "TensorRT-LLM 核心架构解析",
// section 1.2, among them -- are split over several waves whose partial
// softmax statistics a second kernel merges.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <mutex>
#include <string>

#include "internal.h"

namespace pkv {

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

static pkv_status device_fail(int err, const char *where)
{
    char buf[256];
    std::snprintf(buf, sizeof buf, "%s: %s", where, hipGetErrorString((hipError_t)err));
    return fail(PKV_ERR_DEVICE, buf);
}

// Compute units of the current device (256, an MI355X, when there is none).
static int device_cu_count()
{
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return 256;
    if (dev < 64 && cached[dev] > 0)
        return cached[dev];
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    if (dev < 64)
        cached[dev] = cus;
    return cus;
}

// Waves of the persistent grid: the caller's choice or the default per
// compute unit for the KV type, never more than the batch can have tiles
// (at least 1).
static int32_t resolve_splits(const pkv_decode_args *a)
{
    const int64_t tiles_per_seq = ((int64_t)a->max_context_len + kTileTokens - 1) / kTileTokens;
    const int64_t upper = std::max<int64_t>(1, (int64_t)a->batch * a->num_kv_heads * tiles_per_seq);
    const bool byte_kv = a->kv_dtype == PKV_I8 || a->kv_dtype == PKV_FP8_E4M3;
    const int64_t per_cu = byte_kv ? kDefaultWavesPerCUByte : kDefaultWavesPerCU;
    const int64_t want = a->num_splits > 0 ? a->num_splits : per_cu * device_cu_count();
    return (int32_t)std::min<int64_t>(std::min<int64_t>(want, upper), 1 << 24);
}

// Workspace layout: a 256-byte header (the tag of the last decode launch),
// one 16-byte geometry record per (sequence, KV head) segment, then one piece
// slot per (segment + wave) and query head: head_dim fp32 values, and a
// (max, sum) pair.
struct WorkspaceLayout {
    size_t geo, part_o, part_ml, total;
};

// Levels of the fan-in-8 merge tree needed for up to `splits` waves per segment.
static int merge_levels(int32_t splits)
{
    int levels = 1;
    for (int64_t span = 8; span < splits; span *= 8)
        ++levels;
    return levels;
}

static WorkspaceLayout workspace_layout(const pkv_decode_args *a, int32_t splits)
{
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t S = (size_t)a->batch * (size_t)a->num_kv_heads;
    const size_t G = (size_t)(a->num_q_heads / a->num_kv_heads);
    const size_t pieces = (S + (size_t)splits) * G;
    WorkspaceLayout L;
    L.geo = 256;
    L.part_o = L.geo + up(S * 16);
    L.part_ml = L.part_o + up(pieces * (size_t)a->head_dim * sizeof(float));
    L.total = L.part_ml + pieces * 2 * sizeof(float);
    return L;
}

static size_t workspace_bytes(const pkv_decode_args *a)
{
    return a->batch == 0 ? 0 : workspace_layout(a, resolve_splits(a)).total;
}

// Arrival counters of the in-kernel merge: one per piece slot (segment +
// wave) per level of the merge tree.
static size_t counter_bytes(const pkv_decode_args *a)
{
    if (a->batch == 0)
        return 0;
    const int32_t splits = resolve_splits(a);
    const size_t S = (size_t)a->batch * (size_t)a->num_kv_heads;
    return (size_t)merge_levels(splits) * (S + (size_t)splits) * sizeof(uint32_t);
}

// A nonzero 32-bit value that differs from call to call.
static uint32_t next_tag()
{
    static std::atomic<uint32_t> counter{
        (uint32_t)std::chrono::steady_clock::now().time_since_epoch().count() * 2654435761u};
    uint32_t t;
    do
        t = counter.fetch_add(1, std::memory_order_relaxed) * 2654435761u + 0x9E3779B9u;
    while (t == 0);
    return t;
}

// Shape, dtype and pointer checks of everything but the workspace and the
// merge counters; no GPU access.
static pkv_status validate_core(const pkv_decode_args *a)
{
    if (!a)
        return fail(PKV_ERR_INVALID_ARG, "decode: null argument struct");
    if (a->batch < 0 || a->num_q_heads <= 0 || a->num_kv_heads <= 0 || a->num_pages <= 0 ||
        a->max_blocks < 0 || a->max_context_len < 0)
        return fail(PKV_ERR_INVALID_ARG, "decode: sizes must be positive (batch, max_blocks, "
                                         "max_context_len non-negative)");
    if (a->num_q_heads % a->num_kv_heads)
        return fail(PKV_ERR_INVALID_ARG, "decode: num_kv_heads must divide num_q_heads");
    if ((int64_t)a->max_context_len > (int64_t)a->max_blocks * a->page_size)
        return fail(PKV_ERR_INVALID_ARG, "decode: max_context_len exceeds max_blocks * page_size");
    if (a->num_splits < 0)
        return fail(PKV_ERR_INVALID_ARG, "decode: num_splits must be >= 0");
    if (!std::isfinite(a->scale))
        return fail(PKV_ERR_INVALID_ARG, "decode: scale must be finite");
    const bool byte_kv = a->kv_dtype == PKV_I8 || a->kv_dtype == PKV_FP8_E4M3;
    bool kv_ok = (byte_kv && (a->q_dtype == PKV_F16 || a->q_dtype == PKV_BF16)) ||
                 (a->kv_dtype == PKV_F16 && a->q_dtype == PKV_F16) ||
                 (a->kv_dtype == PKV_BF16 && a->q_dtype == PKV_BF16);
    int group = a->num_q_heads / a->num_kv_heads;
    if (!kv_ok || !decode_instantiated(a->head_dim, a->page_size, group, a->q_dtype, a->kv_dtype))
        return fail(PKV_ERR_UNSUPPORTED,
                    "decode: supported set is head_dim {64,128}, page_size {16,64}, group {1,2,4,8}, "
                    "(q,kv) in {(f16,f16),(bf16,bf16),(f16|bf16, i8|fp8)}");
    if (a->batch == 0)
        return PKV_OK;
    if (!a->q || !a->k_pool || !a->v_pool || !a->block_tables || !a->context_lens || !a->out)
        return fail(PKV_ERR_INVALID_ARG, "decode: null device pointer");
    if (byte_kv && (!a->k_scale || !a->v_scale))
        return fail(PKV_ERR_INVALID_ARG, "decode: int8 / fp8 KV needs k_scale and v_scale");
    if (!aligned16(a->q) || !aligned16(a->k_pool) || !aligned16(a->v_pool) || !aligned16(a->out) ||
        ((uintptr_t)a->k_scale & 3u) || ((uintptr_t)a->v_scale & 3u) ||
        ((uintptr_t)a->block_tables & 3u) || ((uintptr_t)a->context_lens & 3u))
        return fail(PKV_ERR_INVALID_ARG, "decode: q, pools and out must be 16-byte aligned, "
                                         "scales and int32 arrays 4-byte aligned");
    return PKV_OK;
}

// validate_core, then the workspace (and, for the one-launch form, the merge
// counters) the caller passed.
static pkv_status validate(const pkv_decode_args *a, bool one_launch)
{
    const pkv_status st = validate_core(a);
    if (st != PKV_OK || a->batch == 0)
        return st;
    const size_t need = workspace_bytes(a);
    if (need > 0 && (!a->workspace || a->workspace_bytes < need || ((uintptr_t)a->workspace & 255u)))
        return fail(PKV_ERR_WORKSPACE, "decode: workspace missing, smaller than "
                                       "pkv_decode_workspace_bytes, or not 256-byte aligned");
    const size_t need_ctr = one_launch ? counter_bytes(a) : 0;
    if (need_ctr > 0 && (!a->merge_counters || a->merge_counter_bytes < need_ctr ||
                         ((uintptr_t)a->merge_counters & 3u)))
        return fail(PKV_ERR_WORKSPACE, "decode: merge_counters missing, smaller than "
                                       "pkv_decode_counter_bytes, or not 4-byte aligned");
    return PKV_OK;
}

static DecodeParams make_params(const pkv_decode_args *a)
{
    DecodeParams p{};
    p.q = a->q;
    p.k_pool = a->k_pool;
    p.v_pool = a->v_pool;
    p.k_scale = a->k_scale;
    p.v_scale = a->v_scale;
    p.block_tables = a->block_tables;
    p.context_lens = a->context_lens;
    p.out = a->out;
    p.batch = a->batch;
    p.num_q_heads = a->num_q_heads;
    p.num_kv_heads = a->num_kv_heads;
    p.num_pages = a->num_pages;
    p.max_blocks = a->max_blocks;
    p.max_context_len = a->max_context_len;
    p.num_splits = resolve_splits(a);
    p.first_round = std::min<int32_t>(p.num_splits, 4 * device_cu_count());   // four SIMDs per compute unit
    p.tag = next_tag();
    p.fused = 0;
    p.counters = a->merge_counters;
    // log2(e) folded into the scale once, in fp32, so the kernels use exp2
    p.scale_log2 = a->scale * 1.44269504088896340736f;
    if (a->workspace) {
        const WorkspaceLayout L = workspace_layout(a, p.num_splits);
        char *ws = (char *)a->workspace;
        p.ws_tag = (uint32_t *)ws;
        p.seg_geo = (int4 *)(ws + L.geo);
        p.part_o = (float *)(ws + L.part_o);
        p.part_ml = (float *)(ws + L.part_ml);
    }
    return p;
}

}  // namespace pkv

using namespace pkv;

extern "C" int32_t pkv_device_count(void)
{
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess)
        return 0;
    return n;
}

extern "C" pkv_status pkv_decode_workspace_bytes(const pkv_decode_args *a, size_t *bytes)
{
    clear_error();
    if (!a || !bytes)
        return fail(PKV_ERR_INVALID_ARG, "pkv_decode_workspace_bytes: null argument");
    if (a->batch < 0 || a->num_q_heads <= 0 || a->num_kv_heads <= 0 || a->num_q_heads % a->num_kv_heads ||
        a->max_context_len < 0 || a->num_splits < 0 || a->head_dim <= 0)
        return fail(PKV_ERR_INVALID_ARG, "pkv_decode_workspace_bytes: bad sizes");
    *bytes = workspace_bytes(a);
    return PKV_OK;
}

extern "C" pkv_status pkv_decode_counter_bytes(const pkv_decode_args *a, size_t *bytes)
{
    clear_error();
    if (!a || !bytes)
        return fail(PKV_ERR_INVALID_ARG, "pkv_decode_counter_bytes: null argument");
    if (a->batch < 0 || a->num_q_heads <= 0 || a->num_kv_heads <= 0 || a->num_q_heads % a->num_kv_heads ||
        a->max_context_len < 0 || a->num_splits < 0)
        return fail(PKV_ERR_INVALID_ARG, "pkv_decode_counter_bytes: bad sizes");
    *bytes = counter_bytes(a);
    return PKV_OK;
}

extern "C" int32_t pkv_decode_num_splits(const pkv_decode_args *a)
{
    if (!a || a->batch < 0 || a->num_kv_heads <= 0 || a->max_context_len < 0 || a->num_splits < 0)
        return 0;
    return resolve_splits(a);
}

extern "C" pkv_status pkv_decode_validate(const pkv_decode_args *a)
{
    clear_error();
    return validate(a, true);
}

extern "C" pkv_status pkv_paged_attn_decode_partitions(const pkv_decode_args *a, void *stream)
{
    clear_error();
    pkv_status st = validate(a, false);
    if (st != PKV_OK || a->batch == 0)
        return st;
    DecodeParams p = make_params(a);
    int err = launch_decode_partitions(p, a->head_dim, a->page_size, a->num_q_heads / a->num_kv_heads,
                                       a->q_dtype, a->kv_dtype, stream);
    return err ? device_fail(err, "pkv_paged_attn_decode_partitions") : PKV_OK;
}

extern "C" pkv_status pkv_splitk_reduce(const pkv_decode_args *a, void *stream)
{
    clear_error();
    pkv_status st = validate(a, false);
    if (st != PKV_OK || a->batch == 0)
        return st;
    DecodeParams p = make_params(a);
    int err = launch_splitk_reduce(p, a->head_dim, a->q_dtype, stream);
    return err ? device_fail(err, "pkv_splitk_reduce") : PKV_OK;
}

extern "C" pkv_status pkv_paged_attn_decode(const pkv_decode_args *a, void *stream)
{
    clear_error();
    pkv_status st = validate(a, true);
    if (st != PKV_OK || a->batch == 0)
        return st;
    DecodeParams p = make_params(a);
    p.fused = 1;   // one launch: the decode kernel merges shared segments itself
    int err = launch_decode_partitions(p, a->head_dim, a->page_size, a->num_q_heads / a->num_kv_heads,
                                       a->q_dtype, a->kv_dtype, stream);
    return err ? device_fail(err, "pkv_paged_attn_decode") : PKV_OK;
}

// ---- decode for callers that cannot allocate --------------------------------
//
// pkv_paged_attn_decode_noalloc keeps its workspace and merge counters in
// `scratch`, a file-scope device array: every GPU the library runs on holds
// its own copy, at its own address, until the process ends.  Host code never
// uses the array's name as an address (on the host it is only a stand-in):
// the device address is looked up once per device, at the entry point's first
// call there, and kept in g_scratch.

constexpr size_t kNoAllocWorkspaceBytes = (size_t)32 << 20;
constexpr size_t kNoAllocCounterBytes = (size_t)1 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocWorkspaceBytes + kNoAllocCounterBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mutex;
static char *g_scratch[kMaxDevices];

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t *p, uint32_t n)
{
    for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < n; i += gridDim.x * 256u)
        p[i] = 0u;
}

// Device address of this device's scratch.  On the first call for a device
// the merge counters are cleared (static device memory starts zeroed and
// every complete call leaves the counters zero, so this is belt and braces)
// by a kernel on `stream`, ahead of the decode launch that follows.
static pkv_status scratch_for_current_device(hipStream_t stream, char **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return device_fail((int)e, "pkv_paged_attn_decode_noalloc");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(PKV_ERR_DEVICE, "pkv_paged_attn_decode_noalloc: device index beyond 63");
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return device_fail((int)(e != hipSuccess ? e : hipErrorInvalidSymbol),
                               "pkv_paged_attn_decode_noalloc: hipGetSymbolAddress");
        char *base = (char *)ptr;
        hipLaunchKernelGGL(zero_words_kernel, dim3(256), dim3(256), 0, stream,
                           (uint32_t *)(base + kNoAllocWorkspaceBytes), (uint32_t)(kNoAllocCounterBytes / 4));
        e = hipGetLastError();
        if (e != hipSuccess)
            return device_fail((int)e, "pkv_paged_attn_decode_noalloc: clearing the merge counters");
        g_scratch[dev] = base;
    }
    *out = g_scratch[dev];
    return PKV_OK;
}

extern "C" pkv_status pkv_paged_attn_decode_noalloc(const pkv_decode_args *a, void *stream)
{
    clear_error();
    pkv_status st = validate_core(a);
    if (st != PKV_OK || a->batch == 0)
        return st;
    const size_t need = workspace_bytes(a), need_ctr = counter_bytes(a);
    if (need > kNoAllocWorkspaceBytes || need_ctr > kNoAllocCounterBytes) {
        char buf[256];
        std::snprintf(buf, sizeof buf,
                      "pkv_paged_attn_decode_noalloc: these shapes need %zu bytes of workspace and %zu of merge "
                      "counters; the static scratch holds %zu and %zu",
                      need, need_ctr, kNoAllocWorkspaceBytes, kNoAllocCounterBytes);
        return fail(PKV_ERR_WORKSPACE, buf);
    }
    char *base = nullptr;
    st = scratch_for_current_device((hipStream_t)stream, &base);
    if (st != PKV_OK)
        return st;
    pkv_decode_args b = *a;
    b.workspace = base;
    b.workspace_bytes = kNoAllocWorkspaceBytes;
    b.merge_counters = (uint32_t *)(base + kNoAllocWorkspaceBytes);
    b.merge_counter_bytes = kNoAllocCounterBytes;
    DecodeParams p = make_params(&b);
    p.fused = 1;
    int err = launch_decode_partitions(p, b.head_dim, b.page_size, b.num_q_heads / b.num_kv_heads, b.q_dtype,
                                       b.kv_dtype, stream);
    return err ? device_fail(err, "pkv_paged_attn_decode_noalloc") : PKV_OK;
}

extern "C" pkv_status pkv_write_kv(const pkv_write_args *a, void *stream)
{
    clear_error();
    if (!a)
        return fail(PKV_ERR_INVALID_ARG, "pkv_write_kv: null argument struct");
    if (a->n < 0 || a->num_kv_heads <= 0 || a->page_size <= 0 || a->num_pages <= 0)
        return fail(PKV_ERR_INVALID_ARG, "pkv_write_kv: bad sizes");
    if (a->head_dim != 64 && a->head_dim != 128)
        return fail(PKV_ERR_UNSUPPORTED, "pkv_write_kv: head_dim must be 64 or 128");
    if (a->kv_dtype != PKV_F16 && a->kv_dtype != PKV_BF16 && a->kv_dtype != PKV_I8 &&
        a->kv_dtype != PKV_FP8_E4M3)
        return fail(PKV_ERR_UNSUPPORTED, "pkv_write_kv: unknown kv dtype");
    const bool byte_kv = a->kv_dtype == PKV_I8 || a->kv_dtype == PKV_FP8_E4M3;   // one scale per row
    const bool quantise = byte_kv && (a->src_dtype == PKV_F16 || a->src_dtype == PKV_BF16);
    if (a->src_dtype != a->kv_dtype && !quantise)
        return fail(PKV_ERR_UNSUPPORTED, "pkv_write_kv: src_dtype must equal kv_dtype, or be f16 / bf16 "
                                         "with an int8 / fp8 pool");
    if ((int64_t)a->n * a->num_kv_heads >= ((int64_t)1 << 31))
        return fail(PKV_ERR_INVALID_ARG, "pkv_write_kv: n * num_kv_heads must be below 2^31");
    if (a->n == 0)
        return PKV_OK;
    if (!a->k_new || !a->v_new || !a->slots || !a->k_pool || !a->v_pool)
        return fail(PKV_ERR_INVALID_ARG, "pkv_write_kv: null device pointer");
    if (byte_kv && (!a->k_scale || !a->v_scale || (!quantise && (!a->k_scale_new || !a->v_scale_new))))
        return fail(PKV_ERR_INVALID_ARG, "pkv_write_kv: int8 / fp8 KV needs the pool scales (and, for "
                                         "encoded rows, their scales)");
    if (!aligned16(a->k_new) || !aligned16(a->v_new) || !aligned16(a->k_pool) || !aligned16(a->v_pool) ||
        ((uintptr_t)a->slots & 7u))
        return fail(PKV_ERR_INVALID_ARG, "pkv_write_kv: K/V buffers must be 16-byte aligned, slots 8-byte");
    WriteParams p{};
    p.k_new = a->k_new;
    p.v_new = a->v_new;
    p.k_scale_new = byte_kv && !quantise ? a->k_scale_new : nullptr;
    p.v_scale_new = byte_kv && !quantise ? a->v_scale_new : nullptr;
    p.slots = a->slots;
    p.k_pool = a->k_pool;
    p.v_pool = a->v_pool;
    p.k_scale = byte_kv ? a->k_scale : nullptr;
    p.v_scale = byte_kv ? a->v_scale : nullptr;
    p.n = a->n;
    p.num_kv_heads = a->num_kv_heads;
    p.page_size = a->page_size;
    p.num_pages = a->num_pages;
    p.row_bytes = a->head_dim * (byte_kv ? 1 : 2);
    p.head_dim = a->head_dim;
    p.src_dtype = a->src_dtype;
    p.kv_dtype = a->kv_dtype;
    int err = launch_write_kv(p, stream);
    return err ? device_fail(err, "pkv_write_kv") : PKV_OK;
}

extern "C" pkv_status pkv_copy_pages(const pkv_copy_args *a, void *stream)
{
    clear_error();
    if (!a)
        return fail(PKV_ERR_INVALID_ARG, "pkv_copy_pages: null argument struct");
    if (a->n < 0 || a->num_pages <= 0 || a->num_kv_heads <= 0 || a->page_size <= 0 || a->head_dim <= 0)
        return fail(PKV_ERR_INVALID_ARG, "pkv_copy_pages: bad sizes");
    if (a->kv_dtype != PKV_F16 && a->kv_dtype != PKV_BF16 && a->kv_dtype != PKV_I8 &&
        a->kv_dtype != PKV_FP8_E4M3)
        return fail(PKV_ERR_UNSUPPORTED, "pkv_copy_pages: unknown kv dtype");
    if (a->n == 0)
        return PKV_OK;
    const bool byte_kv = a->kv_dtype == PKV_I8 || a->kv_dtype == PKV_FP8_E4M3;
    if (!a->k_pool || !a->v_pool || !a->pairs || (byte_kv && (!a->k_scale || !a->v_scale)))
        return fail(PKV_ERR_INVALID_ARG, "pkv_copy_pages: null device pointer");
    const int64_t page_bytes =
        (int64_t)a->num_kv_heads * a->page_size * a->head_dim * (byte_kv ? 1 : 2);
    if (!aligned16(a->k_pool) || !aligned16(a->v_pool) || page_bytes % 16 || ((uintptr_t)a->pairs & 3u))
        return fail(PKV_ERR_INVALID_ARG, "pkv_copy_pages: pools must be 16-byte aligned");
    const int64_t tiles = (page_bytes / 16 + kCopyTileChunks - 1) / kCopyTileChunks;
    if ((int64_t)a->n * tiles > (int64_t)0xFFFFFFFF)
        return fail(PKV_ERR_INVALID_ARG, "pkv_copy_pages: too many pairs for the page size in one call");
    CopyParams p{};
    p.k_pool = a->k_pool;
    p.v_pool = a->v_pool;
    p.k_scale = byte_kv ? a->k_scale : nullptr;
    p.v_scale = byte_kv ? a->v_scale : nullptr;
    p.pairs = a->pairs;
    p.n = a->n;
    p.num_pages = a->num_pages;
    p.page_bytes = page_bytes;
    p.page_scales = (int64_t)a->num_kv_heads * a->page_size;
    int err = launch_copy_pages(p, stream);
    return err ? device_fail(err, "pkv_copy_pages") : PKV_OK;
}
