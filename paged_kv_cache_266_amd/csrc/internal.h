// Internal declarations shared by the host-side translation units of
// libpagedkv.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "host.h"

namespace pkv {

// Tokens per wave-iteration of the decode kernel.
constexpr int kTileTokens = 64;
// Default waves per compute unit of the persistent grid (measured on
// MI355X): one per SIMD for 16-bit KV, where a second co-resident wave on a
// SIMD only slows the first (and the grid ends on the slower one); two per
// SIMD for int8 and fp8 KV, whose conversions leave more arithmetic to
// overlap with memory latency (fp8, Llama-3-8B shape: 67 vs 78 us).
constexpr int kDefaultWavesPerCU = 4;
constexpr int kDefaultWavesPerCUByte = 8;
// Waves per workgroup of the decode kernels: independent waves (each streams
// its own share), grouped only so that the dispatcher has a quarter as many
// workgroups to place (measured: -1.5 us on the Llama-3-8B decode step).
constexpr int kWavesPerGroup = 4;
// Shares of the tile list taken by a wave dispatched first on its SIMD and
// by one dispatched second (two waves per SIMD): vector kernel, fp8 kernel.
#ifndef PKV_SHARE_A
#define PKV_SHARE_A 4
#define PKV_SHARE_B 3
#endif
#ifndef PKV_SHARE_FP8_A
#define PKV_SHARE_FP8_A 4
#define PKV_SHARE_FP8_B 3
#endif
constexpr int kShareA = PKV_SHARE_A, kShareB = PKV_SHARE_B;
constexpr int kShareFp8A = PKV_SHARE_FP8_A, kShareFp8B = PKV_SHARE_FP8_B;

enum DType : int { F16 = 0, BF16 = 1, I8 = 2, FP8 = 3 };

// Everything the decode kernels read; built by the host from pkv_decode_args.
struct DecodeParams {
    const void *q;
    const void *k_pool;
    const void *v_pool;
    const float *k_scale;
    const float *v_scale;
    const int32_t *block_tables;
    const int32_t *context_lens;
    void *out;
    uint32_t *ws_tag;  // workspace header: tag of the last decode launch
    int4 *seg_geo;     // [segments]: (tag, first wave, last wave, 0) of each segment
    float *part_o;     // [(segments + num_splits) * G][D] pieces
    float *part_ml;    // [(segments + num_splits) * G][2]: (max in log2 units, sum)
    uint32_t *counters;  // [merge levels][segments + num_splits] arrival counters, zero between calls
    int32_t batch;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t num_pages;
    int32_t max_blocks;
    int32_t max_context_len;
    int32_t num_splits;   // waves of the persistent grid
    int32_t first_round;  // waves dispatched first on their SIMD (one per SIMD)
    uint32_t tag;         // nonzero, different for every call
    int32_t fused;        // 1: the decode kernel merges shared segments itself
    float scale_log2;     // softmax scale * log2(e)
};

struct WriteParams {
    const void *k_new;
    const void *v_new;
    const float *k_scale_new;
    const float *v_scale_new;
    const int64_t *slots;
    void *k_pool;
    void *v_pool;
    float *k_scale;
    float *v_scale;
    int32_t n;
    int32_t num_kv_heads;
    int32_t page_size;
    int32_t num_pages;
    int32_t row_bytes;    // bytes of one pool row (one token, one KV head)
    int32_t head_dim;
    int32_t src_dtype;    // type of k_new / v_new
    int32_t kv_dtype;     // type of the pools
};

// Kernel launchers (device code lives in the .hip translation units).
// Each returns a hipError_t value as int (0 = success).
bool decode_instantiated(int head_dim, int page_size, int group, int q_dtype, int kv_dtype);
int launch_decode_partitions(const DecodeParams &p, int head_dim, int page_size, int group,
                             int q_dtype, int kv_dtype, void *stream);
int launch_splitk_reduce(const DecodeParams &p, int head_dim, int q_dtype, void *stream);
int launch_write_kv(const WriteParams &p, void *stream);

struct CopyParams {
    void *k_pool;
    void *v_pool;
    float *k_scale;
    float *v_scale;
    const int32_t *pairs;
    int32_t n;
    int32_t num_pages;
    int64_t page_bytes;    // bytes of one page of one pool (all heads)
    int64_t page_scales;   // scales per page (all heads), 0 without scales
    int32_t tiles_per_page;   // set by the launcher
};

// Everything the chunked-prefill kernel reads; built from pkv_prefill_args.
struct PrefillParams {
    const void *q;
    const void *k_pool;
    const void *v_pool;
    const float *k_scale;   // int8 / fp8 K/V: [num_pages][Hkv][page_size]
    const float *v_scale;
    const int32_t *block_tables;
    const int32_t *q_start;
    const int32_t *context_lens;
    void *out;
    int32_t batch;
    int32_t n_q;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t num_pages;
    int32_t max_blocks;
    int32_t max_context_len;
    int32_t max_q_len;
    int32_t q_dtype;
    int32_t kv_dtype;
    int32_t head_dim;     // 64 or 128
    float scale_log2;     // softmax scale * log2(e)
};

bool prefill_instantiated(int head_dim, int page_size, int group, int q_dtype, int kv_dtype);
int launch_prefill(const PrefillParams &p, int page_size, int group, void *stream);

// 16-byte chunks of one page that one block of copy_pages_kernel copies
constexpr int kCopyTileChunks = 1024;

int launch_copy_pages(const CopyParams &p, void *stream);

}  // namespace pkv
