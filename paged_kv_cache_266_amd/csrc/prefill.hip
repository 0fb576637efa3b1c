// Chunked prefill over a paged KV cache for gfx950 (MI355X, CDNA4, wave64).
//
// The chunked context of "TensorRT-LLM 深度实战" (chenxutan.com), section
// 7.3: a long prompt is processed a chunk of tokens at a time, each chunk's
// queries attending to every earlier token of the sequence and causally to
// the chunk's own tokens.  Sequence b's new tokens are rows q_start[b] ..
// q_start[b+1]-1 of q [n_q][Hq][D]; its cache already holds them (their K/V
// written by pkv_write_kv), so its context length n counts them and query i
// sits at position n - nq + i, attending to keys 0 .. that position with the
// decode path's scaled-dot-product softmax (section 3.3 of the same page).
//
// Design.  One workgroup of four waves per (block of query tokens, KV head,
// sequence).  Its 64 rows are (token, head of the group) pairs, token-major:
// 64 / G query tokens of the G heads sharing the KV head, 16 rows per wave.
// Both contractions run on the matrix cores (v_mfma_f32_16x16x32_{bf16,f16}:
// D[16][16] += A[16][32] . B[32][16]; lane l = (a, c) = (l/16, l%16) supplies
// A[c][8a + i] and B[8a + i][c], i < 8, and holds D[4a + v][c], v < 4):
//
//  * K and V of a 64-token key tile are loaded by the whole workgroup, 16
//    bytes per thread per chunk, gathered through the block table (tokens
//    past the context length read as zero), and staged in LDS: K row-major
//    (the B operand of q.k reads 8 consecutive dims of one key), V transposed
//    (the B operand of p.V reads 8 consecutive keys of one dim; the lanes of
//    a wave load one key each, so they write consecutive keys of a row).  The
//    loads run two tiles ahead of the arithmetic (two register sets).
//  * q.k: the wave's 16 query rows are the A operand (held in registers for
//    the whole block), 4 dim steps of 32; scores land as row 4a + v, key
//    16tb + c.  Keys after a row's position are masked.
//  * Online softmax per row (running max and sum in the exp2 domain),
//    probabilities rounded to q's type and passed through the wave's LDS slot
//    into the A layout of p.V; O[row][dim] accumulates in 8 x 4 registers.
//
// Key tiles after the block's last position are not visited.  A sequence
// whose context length is invalid (negative, above the bound, or shorter
// than its chunk) gets NaN rows, as does a block that needs a page outside
// the pool.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>
#include <utility>

#include "internal.h"

namespace pkv {
namespace {

typedef uint32_t u32;
typedef __attribute__((ext_vector_type(4))) u32 u32x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kKeyTile = 64;          // keys per tile
constexpr int kRows = 64;             // query rows per workgroup (4 waves x 16)
constexpr int kD = 128;               // head_dim
constexpr int kKStride = kD + 8;      // LDS row of K (16-bit elements), padded
constexpr int kVStride = kKeyTile + 8;  // LDS row of transposed V (16-bit elements), padded

template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF,
                                                                 false));
}

// Max / sum over the 16 lanes of a row; every lane of the row gets the result.
__device__ __forceinline__ float row_max16(float x)
{
    x = fmaxf(x, dpp<0x128>(x));
    x = fmaxf(x, dpp<0x124>(x));
    x = fmaxf(x, dpp<0x122>(x));
    x = fmaxf(x, dpp<0x121>(x));
    return x;
}

__device__ __forceinline__ float row_sum16(float x)
{
    x += dpp<0x128>(x);
    x += dpp<0x124>(x);
    x += dpp<0x122>(x);
    x += dpp<0x121>(x);
    return x;
}

template <int QT>
__device__ __forceinline__ u32 pack2(float a, float b)
{
    if constexpr (QT == BF16) {
        bf16x2 v = {(__bf16)a, (__bf16)b};
        return __builtin_bit_cast(u32, v);
    } else {
        f16x2 v = {(_Float16)a, (_Float16)b};
        return __builtin_bit_cast(u32, v);
    }
}

template <int QT>
__device__ __forceinline__ uint16_t pack1(float a)
{
    if constexpr (QT == BF16)
        return __builtin_bit_cast(uint16_t, (__bf16)a);
    else
        return __builtin_bit_cast(uint16_t, (_Float16)a);
}

template <int QT>
__device__ __forceinline__ f32x4 mfma32(u32x4 a, u32x4 b, f32x4 c)
{
    if constexpr (QT == BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
}

template <int N, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    [&]<int... I>(std::integer_sequence<int, I...>) { (f(std::integral_constant<int, I>{}), ...); }
        (std::make_integer_sequence<int, N>{});
}

template <int PS, int G, int QT>
__global__ __launch_bounds__(256) void paged_prefill_kernel(PrefillParams p)
{
    constexpr int QPB = kRows / G;    // query tokens per block
    __shared__ uint16_t s_k[kKeyTile * kKStride];
    __shared__ uint16_t s_vt[kD * kVStride];
    __shared__ float s_p[4][16][kKeyTile];

    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    const int a = lane / 16, c = lane % 16;
    const int qblk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int Hq = p.num_q_heads, Hkv = p.num_kv_heads;

    const int qs0 = p.q_start[b], qs1 = p.q_start[b + 1];
    if (qs0 < 0 || qs1 < qs0 || qs1 > p.n_q)
        return;   // no rows that can be written safely
    const int nq = qs1 - qs0;
    const int i0 = qblk * QPB;
    if (i0 >= nq)
        return;
    const int n = p.context_lens[b];
    const bool bad_len = n < 0 || n > p.max_context_len || nq > n;
    const int tok_hi = min(nq, i0 + QPB);   // this block's query tokens: [i0, tok_hi)

    // this lane's A-operand row (for q) and its query
    const int row_a = 16 * wave + c;
    const int tok_a = i0 + row_a / G, head_a = g * G + row_a % G;
    const bool valid_a = tok_a < tok_hi;
    u32x4 qa[4];
    {
        const char *qrow = (const char *)p.q + (((size_t)(qs0 + (valid_a ? tok_a : i0)) * Hq + head_a) * kD) * 2;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(qrow + (32 * s + 8 * a) * 2);
            qa[s] = valid_a ? v : u32x4{0u, 0u, 0u, 0u};
        }
    }
    // positions of the rows this lane holds in the D layout (row 4a + v of the wave)
    int pos_row[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int r = 16 * wave + 4 * a + v;
        const int tok = i0 + r / G;
        pos_row[v] = tok < tok_hi && !bad_len ? n - nq + tok : -1;   // -1: masks every key
    }
    const int last_pos = bad_len ? -1 : n - nq + tok_hi - 1;
    const int n_tiles = last_pos < 0 ? 0 : last_pos / kKeyTile + 1;

    // ---- key-tile loads, two tiles in flight (register sets 0 and 1).  K:
    // thread tid moves chunks tid + 256 j (j < 4), chunk q being dims
    // 8 (q % 16) .. +8 of key q / 16 (rows of consecutive 16-byte pieces).  V:
    // thread tid moves dims 8 (tid / 64 + 4 j) .. +8 of key tid % 64, so that
    // the lanes of a wave write consecutive keys of one transposed row.
    const size_t page_stride = (size_t)Hkv * PS * kD;   // elements
    const int32_t *bt = p.block_tables + (size_t)b * p.max_blocks;
    u32x4 kreg[2][4], vreg[2][4];
    bool bad = false;
    // element offset of key `key` (dims from 0) in the pools, or -1 if it is
    // not read (past the context / the block, or its page outside the pool)
    auto key_offset = [&](int key) -> long long {
        if (key >= n || key > last_pos)
            return -1;
        const int blk = key / PS;
        const int page = blk < p.max_blocks ? bt[blk] : -1;
        if ((unsigned)page >= (unsigned)p.num_pages) {
            bad = true;
            return -1;
        }
        return (long long)((size_t)page * page_stride + ((size_t)g * PS + key % PS) * kD);
    };
    auto load_tile = [&](int tile, u32x4 (&kr)[4], u32x4 (&vr)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int qc = tid + 256 * j;
            const long long ko = key_offset(tile * kKeyTile + qc / 16);
            kr[j] = ko < 0 ? u32x4{0u, 0u, 0u, 0u}
                           : *reinterpret_cast<const u32x4 *>((const uint16_t *)p.k_pool + ko + 8 * (qc % 16));
            const long long vo = key_offset(tile * kKeyTile + tid % 64);
            vr[j] = vo < 0 ? u32x4{0u, 0u, 0u, 0u}
                           : *reinterpret_cast<const u32x4 *>((const uint16_t *)p.v_pool + vo +
                                                              8 * (tid / 64 + 4 * j));
        }
    };
    auto store_tile = [&](const u32x4 (&kr)[4], const u32x4 (&vr)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int qc = tid + 256 * j;
            *reinterpret_cast<u32x4 *>(&s_k[(qc / 16) * kKStride + 8 * (qc % 16)]) = kr[j];
            const int key = tid % 64, d0 = 8 * (tid / 64 + 4 * j);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                s_vt[(d0 + e) * kVStride + key] = (uint16_t)(vr[j][e / 2] >> (16 * (e % 2)));
        }
    };

    f32x4 acc[8];   // O[row 4a + v][dim 16nb + c] in acc[nb][v]
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
        acc[nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float m_row[4], l_row[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        m_row[v] = -INFINITY;
        l_row[v] = 0.0f;
    }

    if (n_tiles > 0)
        load_tile(0, kreg[0], vreg[0]);
    if (n_tiles > 1)
        load_tile(1, kreg[1], vreg[1]);
    auto tile_body = [&](int tile, u32x4 (&kr)[4], u32x4 (&vr)[4]) {
        __syncthreads();                    // the previous tile's LDS reads are done
        store_tile(kr, vr);
        __syncthreads();
        if (tile + 2 < n_tiles)
            load_tile(tile + 2, kr, vr);    // two tiles ahead of the arithmetic

        // ---- scores: S[row 4a + v][key 16tb + c]
        f32x4 sc[4];
        static_for<4>([&](auto TBc) {
            constexpr int TB = decltype(TBc)::value;
            f32x4 x = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const u32x4 kop = *reinterpret_cast<const u32x4 *>(&s_k[(16 * TB + c) * kKStride + 32 * s + 8 * a]);
                x = mfma32<QT>(qa[s], kop, x);
            }
            sc[TB] = x;
        });

        // ---- online softmax (log2 domain) with the causal mask
        const int key0 = tile * kKeyTile;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float mx = -INFINITY;
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const float x = key0 + 16 * tb + c <= pos_row[v] ? sc[tb][v] * p.scale_log2 : -INFINITY;
                sc[tb][v] = x;
                mx = fmaxf(mx, x);
            }
            const float m_new = fmaxf(m_row[v], row_max16(mx));
            // a row with no key yet keeps m = -inf; exp2 of (-inf) - (-inf) is avoided
            const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_row[v] - m_new);
            float ls = 0.0f;
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const float e = m_new == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sc[tb][v] - m_new);
                sc[tb][v] = e;
                ls += e;
            }
            l_row[v] = l_row[v] * alpha + ls;
            m_row[v] = m_new;
#pragma unroll
            for (int nb = 0; nb < 8; ++nb)
                acc[nb][v] *= alpha;
        }
        // probabilities to the wave's LDS slot, [row][key]
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                s_p[wave][4 * a + v][16 * tb + c] = sc[tb][v];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- p.V: A[row c][key 32ks + 8a + i] from LDS, B[key][dim 16nb + c] from transposed V
        static_for<2>([&](auto KSc) {
            constexpr int KS = decltype(KSc)::value;
            const float *src = &s_p[wave][c][32 * KS + 8 * a];
            const float4 p0 = *reinterpret_cast<const float4 *>(src);
            const float4 p1 = *reinterpret_cast<const float4 *>(src + 4);
            const u32x4 aop = {pack2<QT>(p0.x, p0.y), pack2<QT>(p0.z, p0.w), pack2<QT>(p1.x, p1.y),
                               pack2<QT>(p1.z, p1.w)};
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                const u32x4 vop =
                    *reinterpret_cast<const u32x4 *>(&s_vt[(16 * nb + c) * kVStride + 32 * KS + 8 * a]);
                acc[nb] = mfma32<QT>(aop, vop, acc[nb]);
            }
        });
        __builtin_amdgcn_wave_barrier();
    };
    for (int tile = 0; tile < n_tiles; tile += 2) {
        tile_body(tile, kreg[0], vreg[0]);
        if (tile + 1 < n_tiles)
            tile_body(tile + 1, kreg[1], vreg[1]);
    }

    // ---- finalize: O / l, written in q's type
    const bool any_bad = __syncthreads_or(bad ? 1 : 0) != 0 || bad_len;
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int r = 16 * wave + 4 * a + v;
        const int tok = i0 + r / G;
        if (tok >= tok_hi)
            continue;
        const int head = g * G + r % G;
        const float l = row_sum16(l_row[v]);
        const float inv = any_bad ? nan : 1.0f / l;
        uint16_t *orow = (uint16_t *)p.out + ((size_t)(qs0 + tok) * Hq + head) * kD;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
            orow[16 * nb + c] = pack1<QT>(acc[nb][v] * inv);
    }
}

template <int PS, int G>
int launch_g(const PrefillParams &p, dim3 grid, hipStream_t s)
{
    void *args[] = {const_cast<PrefillParams *>(&p)};
    const void *fn = p.q_dtype == BF16 ? (const void *)&paged_prefill_kernel<PS, G, BF16>
                                       : (const void *)&paged_prefill_kernel<PS, G, F16>;
    return (int)hipLaunchKernel(fn, grid, dim3(256), args, 0, s);
}

template <int PS>
int launch_ps(const PrefillParams &p, int G, dim3 grid, hipStream_t s)
{
    switch (G) {
    case 1: return launch_g<PS, 1>(p, grid, s);
    case 2: return launch_g<PS, 2>(p, grid, s);
    case 4: return launch_g<PS, 4>(p, grid, s);
    case 8: return launch_g<PS, 8>(p, grid, s);
    }
    return (int)hipErrorInvalidValue;
}

}  // namespace

bool prefill_instantiated(int head_dim, int page_size, int group, int q_dtype, int kv_dtype)
{
    return head_dim == kD && (page_size == 16 || page_size == 64) &&
           (group == 1 || group == 2 || group == 4 || group == 8) && (q_dtype == F16 || q_dtype == BF16) &&
           kv_dtype == q_dtype;
}

int launch_prefill(const PrefillParams &p, int page_size, int group, void *stream)
{
    const int qpb = kRows / group;
    const dim3 grid((unsigned)((p.max_q_len + qpb - 1) / qpb), (unsigned)p.num_kv_heads, (unsigned)p.batch);
    hipStream_t s = (hipStream_t)stream;
    if (page_size == 16)
        return launch_ps<16>(p, group, grid, s);
    if (page_size == 64)
        return launch_ps<64>(p, group, grid, s);
    return (int)hipErrorInvalidValue;
}

}  // namespace pkv
