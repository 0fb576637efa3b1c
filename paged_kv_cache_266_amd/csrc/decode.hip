// Paged single-token decode attention for gfx950 (MI355X, CDNA4, wave64).
//
// What is computed is the fused attention of "TensorRT-LLM 深度实战"
// (chenxutan.com), section 3.3 -- scores scale * q.k, max-subtracted softmax,
// softmax-weighted sum of V -- for one new query token per sequence (the
// masked_mha role of "TensorRT-LLM 推理加速实战", section 7.2), with K and V
// gathered from fixed-size pages through the per-sequence page table of the
// first page's section 3.1, and query heads sharing KV heads in groups (GQA).
// The structure below is this library's own design for CDNA4; the pages'
// kernel (one thread per query, whole score matrix in shared memory) is not
// followed.
//
// Design (one workgroup = one sequence b, one KV head g, one partition of
// partition_tokens tokens; 4 waves, each wave taking every 4th 64-token tile):
//
//  * Loads.  A (page, KV head) tile is one contiguous run of page_size rows.
//    Each lane loads 16 bytes per instruction through a buffer descriptor
//    whose base is the page and whose size is the tile, so one instruction
//    reads 1 KiB of consecutive rows (R = row_bytes/16 lanes per token row,
//    64/R tokens per instruction).  Slots past the context length get an
//    out-of-range offset and read as zero without touching memory: no
//    garbage (or NaN) from a partly filled last page ever enters a product.
//    K and V of a tile (R instructions each) are issued together, so a wave
//    has 2 x 64 x R x 16 bytes in flight.
//  * q.k.  Lane (row r, column j) holds 16 bytes of one token row and the
//    matching slice of each of the G query heads of the group; dot2
//    instructions (f16/bf16) or byte conversions + FMAs (int8) give partial
//    dots.  A DPP reduce-scatter over the R lanes of a row leaves each lane
//    with the full scores of ONE token (token r + (64/R) j of the tile) for
//    all G heads -- no redundant softmax work.
//  * Online softmax.  Tile max per head by DPP row rotations and a
//    wave-uniform combine of the four rows; running max, per-lane running
//    sums, exp2 with
//    log2(e) folded into the scale.  For int8, the V scale of the token is
//    folded into its probability and the K scale into its score.
//  * p.V.  Probabilities go to a per-wave LDS slot; each lane then reads, per
//    chunk, the G probabilities of the token whose V bytes it holds
//    (broadcast reads) and accumulates G x (elements per lane) fp32 sums.
//  * Combine.  Rows, then waves (through LDS), then -- when the sequence
//    spans several partitions -- the split-K reduce kernel merges
//    (max, sum, unnormalised output) partials.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "internal.h"

namespace pkv {
namespace {

typedef uint32_t u32;
typedef __attribute__((ext_vector_type(4))) u32 u32x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;

constexpr u32 kBufferFlags = 0x00020000u;  // gfx9 raw buffer: 32-bit data format
constexpr int kOutOfRange = 0x7FFFFFF0;    // voffset that fails the range check

// ---- lane exchange ---------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                                 0xF, 0xF, false));
}

// DPP controls: partner lane for the reduce-scatter bit, and row rotations.
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // j <-> 7-j within each 8 lanes
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;       // j <-> j^8 within each 16 lanes

template <int BIT>
struct Partner;
template <> struct Partner<0> { static constexpr int ctrl = kQuadXor1; };
template <> struct Partner<1> { static constexpr int ctrl = kQuadXor2; };
template <> struct Partner<2> { static constexpr int ctrl = kRowHalfMirror; };
template <> struct Partner<3> { static constexpr int ctrl = kRowRor8; };

// Full reductions over the 64 lanes.  DPP rotations finish each 16-lane row;
// the four row results are then read as wave-uniform values.
__device__ __forceinline__ float lane_value(float x, int lane)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

__device__ __forceinline__ float wave_max(float x)
{
    x = fmaxf(x, dpp<0x128>(x));  // row_ror 8
    x = fmaxf(x, dpp<0x124>(x));  // row_ror 4
    x = fmaxf(x, dpp<0x122>(x));  // row_ror 2
    x = fmaxf(x, dpp<0x121>(x));  // row_ror 1
    return fmaxf(fmaxf(lane_value(x, 0), lane_value(x, 16)), fmaxf(lane_value(x, 32), lane_value(x, 48)));
}

__device__ __forceinline__ float wave_sum(float x)
{
    x += dpp<0x128>(x);
    x += dpp<0x124>(x);
    x += dpp<0x122>(x);
    x += dpp<0x121>(x);
    return (lane_value(x, 0) + lane_value(x, 16)) + (lane_value(x, 32) + lane_value(x, 48));
}

// Sum over the 64/R token rows of R lanes each (lanes with equal l % R); every
// lane receives the total of its column.
template <int R>
__device__ __forceinline__ float sum_over_rows(float x)
{
    if constexpr (R <= 4)
        x += dpp<kRowRor4>(x);
    if constexpr (R <= 8)
        x += dpp<kRowRor8>(x);
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

// One reduce-scatter step over lanes that differ in bit BIT of the column:
// lanes with that bit clear keep (and complete) the lower half of the
// values, lanes with it set the upper half.
template <int N, int BIT>
__device__ __forceinline__ void rs_step(const float (&in)[N], float (&out)[N / 2], bool upper)
{
#pragma unroll
    for (int x = 0; x < N / 2; ++x) {
        const float lo = in[x], up = in[x + N / 2];
        const float a = lo + dpp<Partner<BIT>::ctrl>(lo);
        const float c = up + dpp<Partner<BIT>::ctrl>(up);
        out[x] = upper ? c : a;
    }
}

// in[i * G + h] = partial of chunk i, head h on column j of an R-lane row;
// out[h] = full value of chunk j, head h.
template <int R, int G>
__device__ __forceinline__ void reduce_scatter(const float (&in)[R * G], float (&out)[G], int j)
{
    if constexpr (R == 16) {
        float t8[8 * G], t4[4 * G], t2[2 * G];
        rs_step<16 * G, 3>(in, t8, (j & 8) != 0);
        rs_step<8 * G, 2>(t8, t4, (j & 4) != 0);
        rs_step<4 * G, 1>(t4, t2, (j & 2) != 0);
        rs_step<2 * G, 0>(t2, out, (j & 1) != 0);
    } else if constexpr (R == 8) {
        float t4[4 * G], t2[2 * G];
        rs_step<8 * G, 2>(in, t4, (j & 4) != 0);
        rs_step<4 * G, 1>(t4, t2, (j & 2) != 0);
        rs_step<2 * G, 0>(t2, out, (j & 1) != 0);
    } else {
        static_assert(R == 4, "row split");
        float t2[2 * G];
        rs_step<4 * G, 1>(in, t2, (j & 2) != 0);
        rs_step<2 * G, 0>(t2, out, (j & 1) != 0);
    }
}

// ---- element conversion ------------------------------------------------------

__device__ __forceinline__ float bf16_lo(u32 w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(u32 w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }
__device__ __forceinline__ float f16_lo(u32 w) { return (float)__builtin_bit_cast(f16x2, w)[0]; }
__device__ __forceinline__ float f16_hi(u32 w) { return (float)__builtin_bit_cast(f16x2, w)[1]; }

template <int QT>
__device__ __forceinline__ float q_lo(u32 w) { return QT == BF16 ? bf16_lo(w) : f16_lo(w); }
template <int QT>
__device__ __forceinline__ float q_hi(u32 w) { return QT == BF16 ? bf16_hi(w) : f16_hi(w); }

// Two fp32 values -> packed output pair, round to nearest even.
template <int QT>
__device__ __forceinline__ u32 pack_out(float a, float b)
{
    if constexpr (QT == BF16) {
        bf16x2 v = {(__bf16)a, (__bf16)b};
        return __builtin_bit_cast(u32, v);
    } else {
        f16x2 v = {(_Float16)a, (_Float16)b};
        return __builtin_bit_cast(u32, v);
    }
}

template <int KVT>
__device__ __forceinline__ float dot2(u32 k, u32 q, float acc)
{
    if constexpr (KVT == BF16)
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k), __builtin_bit_cast(bf16x2, q),
                                               acc, false);
    else
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, k), __builtin_bit_cast(f16x2, q), acc,
                                      false);
}

// Unsigned byte e of w as float (v_cvt_f32_ubyteN).
template <int E>
__device__ __forceinline__ float ubyte(u32 w) { return (float)((w >> (8 * E)) & 0xFFu); }

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t rsrc, int voff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char *base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), (short)0, bytes, kBufferFlags);
}

// ---- the partition kernel ---------------------------------------------------

template <int D, int PS, int G, int QT, int KVT>
struct Shape {
    static constexpr int EB = KVT == I8 ? 1 : 2;   // bytes per KV element
    static constexpr int ROW = D * EB;             // bytes per token row
    static constexpr int R = ROW / 16;             // lanes per token row
    static constexpr int TPI = 64 / R;             // tokens per load instruction
    static constexpr int EPL = 16 / EB;            // elements per lane chunk
    static constexpr int TILE_BYTES = PS * ROW;    // one (page, KV head) tile
    static constexpr int PAGES_PER_TILE = kTileTokens / PS;
    static constexpr int PSTRIDE = 64 * G + (64 / R) * 4;  // floats per wave in the p buffer
    static_assert(R >= 4 && R <= 16, "row split");
    static_assert(PS % TPI == 0, "a load instruction must not straddle pages");
    static_assert(kTileTokens % PS == 0, "tiles hold whole pages");
};

template <int D, int PS, int G, int QT, int KVT>
__global__ __launch_bounds__(kWaves * 64) void paged_decode_kernel(DecodeParams p)
{
    using S = Shape<D, PS, G, QT, KVT>;
    constexpr int R = S::R, TPI = S::TPI, EPL = S::EPL;
    constexpr bool kI8 = KVT == I8;

    __shared__ float s_p[kWaves * S::PSTRIDE];
    __shared__ float s_m[kWaves][G];
    __shared__ float s_l[kWaves][G];
    __shared__ float s_o[kWaves][G][D];

    const int part = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int T = p.partition_tokens;
    const int Hq = p.num_q_heads;
    const int hq0 = g * G;

    int n = p.context_lens[b];
    bool bad = n < 0 || n > p.max_context_len;
    if (bad)
        n = 0;
    const int t_begin = part * T;
    if (part > 0 && t_begin >= n)
        return;                              // partition past the end (uniform)
    const bool single = n <= T;              // this workgroup owns the whole sequence

    if (n == 0) {                            // empty (or invalid) sequence: zeros (NaN)
        const float fill = bad ? __builtin_nanf("") : 0.0f;
        for (int i = threadIdx.x; i < G * D / 2; i += kWaves * 64) {
            int h = i / (D / 2), d2 = (i % (D / 2)) * 2;
            u32 *o = reinterpret_cast<u32 *>(p.out) + (((size_t)b * Hq + hq0 + h) * D + d2) / 2;
            *o = pack_out<QT>(fill, fill);
        }
        return;
    }

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int r = lane / R, j = lane % R;
    const int t_end = min(n, t_begin + T);
    const int n_tiles = (t_end - t_begin + kTileTokens - 1) / kTileTokens;
    const int tile_base = t_begin / kTileTokens;   // T is a multiple of 64

    // ---- this lane's slice of the G query heads
    u32 qw[G][4];         // 16-bit KV: packed pairs matching the K chunk
    float qf[kI8 ? G : 1][kI8 ? 16 : 1];
    float qbias[G];       // int8: -128 * sum of the lane's q slice
    {
        const char *qb = (const char *)p.q + (((size_t)b * Hq + hq0) * D) * 2;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            if constexpr (!kI8) {
                u32x4 v = *reinterpret_cast<const u32x4 *>(qb + ((size_t)h * D + EPL * j) * 2);
                qw[h][0] = v.x; qw[h][1] = v.y; qw[h][2] = v.z; qw[h][3] = v.w;
                qbias[h] = 0.0f;
            } else {
                const u32x4 *src = reinterpret_cast<const u32x4 *>(qb + ((size_t)h * D + 16 * j) * 2);
                u32x4 a = src[0], c = src[1];
                u32 w[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
                float s = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    qf[h][2 * e] = q_lo<QT>(w[e]);
                    qf[h][2 * e + 1] = q_hi<QT>(w[e]);
                    s += qf[h][2 * e] + qf[h][2 * e + 1];
                }
                qbias[h] = -128.0f * s;
            }
        }
    }

    float m_run[G], l_run[G], acc[G][EPL], psum[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m_run[h] = -INFINITY;
        l_run[h] = 0.0f;
        psum[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            acc[h][e] = 0.0f;
    }

    const int32_t *bt = p.block_tables + (size_t)b * p.max_blocks;
    const size_t page_stride = (size_t)p.num_kv_heads * S::TILE_BYTES;
    const char *k_head = (const char *)p.k_pool + (size_t)g * S::TILE_BYTES;
    const char *v_head = (const char *)p.v_pool + (size_t)g * S::TILE_BYTES;
    float *pbuf = s_p + wave * S::PSTRIDE;
    bool wave_bad = false;

    for (int tile = wave; tile < n_tiles; tile += kWaves) {
        const int tg = tile_base + tile;       // global tile index
        const int t0 = tg * kTileTokens;       // first token of the tile

        // ---- issue K and V loads of the whole tile
        u32x4 kr[R], vr[R];
        int phys_of_page[S::PAGES_PER_TILE];
#pragma unroll
        for (int pg = 0; pg < S::PAGES_PER_TILE; ++pg) {
            const int tp = t0 + pg * PS;
            int phys = -1;
            if (tp < t_end) {
                phys = bt[tg * S::PAGES_PER_TILE + pg];
                if ((unsigned)phys >= (unsigned)p.num_pages) {
                    wave_bad = true;
                    phys = -1;
                }
            }
            phys_of_page[pg] = phys;
        }
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int pg = (i * TPI) / PS;
            const int phys = phys_of_page[pg];
            const int tok = t0 + i * TPI + r;
            const bool valid = phys >= 0 && tok < t_end;
            const int voff = valid ? (((i * TPI) % PS + r) * S::ROW + 16 * j) : kOutOfRange;
            const size_t poff = (size_t)(phys < 0 ? 0 : phys) * page_stride;
            kr[i] = load16(tile_rsrc(k_head + poff, S::TILE_BYTES), voff);
            vr[i] = load16(tile_rsrc(v_head + poff, S::TILE_BYTES), voff);
        }

        // this lane's token after the reduce-scatter: r + TPI * j
        const int my_tok = t0 + TPI * j + r;
        const int my_pg = (TPI * j) / PS;
        int my_phys = -1;
#pragma unroll
        for (int pg = 0; pg < S::PAGES_PER_TILE; ++pg)
            if (pg == my_pg)
                my_phys = phys_of_page[pg];
        const bool my_valid = my_phys >= 0 && my_tok < t_end;
        float kscale = 1.0f, vscale = 1.0f;
        if constexpr (kI8) {
            if (my_valid) {
                size_t si = ((size_t)my_phys * p.num_kv_heads + g) * PS + (TPI * j) % PS + r;
                kscale = p.k_scale[si];
                vscale = p.v_scale[si];
            }
        }

        // ---- partial dots: part[i][h] over this lane's 16 bytes of chunk i
        float part_[R * G];
#pragma unroll
        for (int i = 0; i < R; ++i) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float a;
                if constexpr (!kI8) {
                    a = dot2<KVT>(kr[i].x, qw[h][0], 0.0f);
                    a = dot2<KVT>(kr[i].y, qw[h][1], a);
                    a = dot2<KVT>(kr[i].z, qw[h][2], a);
                    a = dot2<KVT>(kr[i].w, qw[h][3], a);
                } else {
                    // code + 128 as unsigned bytes; the -128 * sum(q) bias restores the sign
                    const u32 w0 = kr[i].x ^ 0x80808080u, w1 = kr[i].y ^ 0x80808080u;
                    const u32 w2 = kr[i].z ^ 0x80808080u, w3 = kr[i].w ^ 0x80808080u;
                    a = qbias[h];
                    a = fmaf(qf[h][0], ubyte<0>(w0), a);
                    a = fmaf(qf[h][1], ubyte<1>(w0), a);
                    a = fmaf(qf[h][2], ubyte<2>(w0), a);
                    a = fmaf(qf[h][3], ubyte<3>(w0), a);
                    a = fmaf(qf[h][4], ubyte<0>(w1), a);
                    a = fmaf(qf[h][5], ubyte<1>(w1), a);
                    a = fmaf(qf[h][6], ubyte<2>(w1), a);
                    a = fmaf(qf[h][7], ubyte<3>(w1), a);
                    a = fmaf(qf[h][8], ubyte<0>(w2), a);
                    a = fmaf(qf[h][9], ubyte<1>(w2), a);
                    a = fmaf(qf[h][10], ubyte<2>(w2), a);
                    a = fmaf(qf[h][11], ubyte<3>(w2), a);
                    a = fmaf(qf[h][12], ubyte<0>(w3), a);
                    a = fmaf(qf[h][13], ubyte<1>(w3), a);
                    a = fmaf(qf[h][14], ubyte<2>(w3), a);
                    a = fmaf(qf[h][15], ubyte<3>(w3), a);
                }
                part_[i * G + h] = a;
            }
        }

        // ---- reduce-scatter over the R lanes of a row: lane j keeps chunk j
        float sc[G];
        reduce_scatter<R, G>(part_, sc, j);

        // ---- online softmax (log2 domain)
        float pe[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float s = my_valid ? sc[h] * kscale * p.scale_log2 : -INFINITY;
            const float m_new = fmaxf(m_run[h], wave_max(s));
            const float alpha = __builtin_amdgcn_exp2f(m_run[h] - m_new);
            const float e = __builtin_amdgcn_exp2f(s - m_new);
            l_run[h] = l_run[h] * alpha + e;
            m_run[h] = m_new;
            psum[h] *= alpha;
#pragma unroll
            for (int x = 0; x < EPL; ++x)
                acc[h][x] *= alpha;
            pe[h] = e * vscale;
        }

        // ---- hand each probability to the lanes holding that token's V bytes
        float *mine = pbuf + lane * G + r * 4;
#pragma unroll
        for (int h = 0; h < G; ++h)
            mine[h] = pe[h];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

#pragma unroll
        for (int i = 0; i < R; ++i) {
            const float *src = pbuf + (r * R + i) * G + r * 4;
            float pv[G];
#pragma unroll
            for (int h = 0; h < G; ++h)
                pv[h] = src[h];
            float vf[EPL];
            const u32 w[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
            if constexpr (kI8) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const u32 u = w[q4] ^ 0x80808080u;
                    vf[4 * q4 + 0] = ubyte<0>(u);
                    vf[4 * q4 + 1] = ubyte<1>(u);
                    vf[4 * q4 + 2] = ubyte<2>(u);
                    vf[4 * q4 + 3] = ubyte<3>(u);
                }
            } else {
#pragma unroll
                for (int q2 = 0; q2 < 4; ++q2) {
                    vf[2 * q2] = KVT == BF16 ? bf16_lo(w[q2]) : f16_lo(w[q2]);
                    vf[2 * q2 + 1] = KVT == BF16 ? bf16_hi(w[q2]) : f16_hi(w[q2]);
                }
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                if constexpr (kI8)
                    psum[h] += pv[h];
#pragma unroll
                for (int x = 0; x < EPL; ++x)
                    acc[h][x] = fmaf(pv[h], vf[x], acc[h][x]);
            }
        }
        __builtin_amdgcn_wave_barrier();
    }

    // ---- wave totals
#pragma unroll
    for (int h = 0; h < G; ++h) {
        if constexpr (kI8) {
#pragma unroll
            for (int x = 0; x < EPL; ++x)
                acc[h][x] = fmaf(-128.0f, psum[h], acc[h][x]);
        }
        const float lt = wave_sum(l_run[h]);
#pragma unroll
        for (int x = 0; x < EPL; ++x)
            acc[h][x] = sum_over_rows<R>(acc[h][x]);
        if (lane == 0) {
            s_m[wave][h] = m_run[h];
            s_l[wave][h] = lt;
        }
        if (r == 0) {
#pragma unroll
            for (int x = 0; x < EPL; ++x)
                s_o[wave][h][EPL * j + x] = acc[h][x];
        }
    }
    // a bad page anywhere in the workgroup poisons the result
    const bool any_bad = __syncthreads_or(wave_bad ? 1 : 0) != 0;

    // ---- merge the waves; write the output or this partition's partials
    for (int i = threadIdx.x; i < G * D / 2; i += kWaves * 64) {
        const int h = i / (D / 2), d2 = (i % (D / 2)) * 2;
        float M = s_m[0][h];
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
            M = fmaxf(M, s_m[w][h]);
        float L = 0.0f, o0 = 0.0f, o1 = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = __builtin_amdgcn_exp2f(s_m[w][h] - M);
            L = fmaf(f, s_l[w][h], L);
            o0 = fmaf(f, s_o[w][h][d2], o0);
            o1 = fmaf(f, s_o[w][h][d2 + 1], o1);
        }
        if (any_bad) {
            L = __builtin_nanf("");
            o0 = o1 = __builtin_nanf("");
        }
        const size_t unit = (size_t)b * Hq + hq0 + h;
        if (single) {
            const float inv = 1.0f / L;
            u32 *o = reinterpret_cast<u32 *>(p.out) + (unit * D + d2) / 2;
            *o = pack_out<QT>(o0 * inv, o1 * inv);
        } else {
            const size_t pu = unit * p.num_partitions + part;
            float2 *po = reinterpret_cast<float2 *>(p.part_o + pu * D + d2);
            *po = make_float2(o0, o1);
            if (d2 == 0)
                *reinterpret_cast<float2 *>(p.part_ml + pu * 2) = make_float2(M, L);
        }
    }
}

// ---- the split-K reduce kernel ---------------------------------------------
//
// For a sequence spread over P partitions with partials (m_k, l_k, o_k)
// (m in log2 units): M = max m_k, L = sum l_k 2^(m_k - M),
// out = sum o_k 2^(m_k - M) / L.  One workgroup per (query head, sequence).

template <int D, int QT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(DecodeParams p)
{
    constexpr int NG = 256 / D;           // partition groups per workgroup
    __shared__ float s_red[256];
    __shared__ float s_L[NG];
    __shared__ float s_o[NG][D];

    const int h = blockIdx.x, b = blockIdx.y;
    const int n = p.context_lens[b];
    if (n < 0 || n > p.max_context_len)
        return;                           // the partition kernel wrote NaN
    const int T = p.partition_tokens;
    const int np_ = (n + T - 1) / T;
    if (np_ <= 1)
        return;                           // the partition kernel wrote the output
    const size_t unit = (size_t)b * p.num_q_heads + h;
    const float *ml = p.part_ml + unit * p.num_partitions * 2;
    const float *po = p.part_o + unit * p.num_partitions * D;
    const int tid = threadIdx.x;

    float mx = -INFINITY;
    for (int k = tid; k < np_; k += 256)
        mx = fmaxf(mx, ml[2 * k]);
    s_red[tid] = mx;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (tid < s)
            s_red[tid] = fmaxf(s_red[tid], s_red[tid + s]);
        __syncthreads();
    }
    const float M = s_red[0];

    const int d = tid % D, grp = tid / D;
    float L = 0.0f, o = 0.0f;
    for (int k = grp; k < np_; k += NG) {
        const float f = __builtin_amdgcn_exp2f(ml[2 * k] - M);
        L = fmaf(f, ml[2 * k + 1], L);
        o = fmaf(f, po[(size_t)k * D + d], o);
    }
    s_o[grp][d] = o;
    if (d == 0)
        s_L[grp] = L;
    __syncthreads();
    if (tid < D / 2) {
        float Lt = 0.0f, a0 = 0.0f, a1 = 0.0f;
#pragma unroll
        for (int q = 0; q < NG; ++q) {
            Lt += s_L[q];
            a0 += s_o[q][2 * tid];
            a1 += s_o[q][2 * tid + 1];
        }
        const float inv = 1.0f / Lt;
        u32 *out = reinterpret_cast<u32 *>(p.out) + (unit * D) / 2 + tid;
        *out = pack_out<QT>(a0 * inv, a1 * inv);
    }
}

// ---- K/V scatter for appended tokens -----------------------------------------

__global__ __launch_bounds__(256) void write_kv_kernel(WriteParams p)
{
    const int chunks = p.row_bytes / 16;
    const size_t total = (size_t)p.n * p.num_kv_heads * chunks;
    for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (size_t)gridDim.x * blockDim.x) {
        const int c = (int)(idx % chunks);
        const size_t ig = idx / chunks;
        const int g = (int)(ig % p.num_kv_heads);
        const size_t i = ig / p.num_kv_heads;
        const int64_t slot = p.slots[i];
        if (slot < 0 || slot >= (int64_t)p.num_pages * p.page_size)
            continue;
        const int64_t page = slot / p.page_size, off = slot % p.page_size;
        const size_t row = ((size_t)page * p.num_kv_heads + g) * p.page_size + off;
        const size_t src = (i * p.num_kv_heads + g) * (size_t)p.row_bytes + (size_t)c * 16;
        const size_t dst = row * p.row_bytes + (size_t)c * 16;
        *reinterpret_cast<u32x4 *>((char *)p.k_pool + dst) =
            *reinterpret_cast<const u32x4 *>((const char *)p.k_new + src);
        *reinterpret_cast<u32x4 *>((char *)p.v_pool + dst) =
            *reinterpret_cast<const u32x4 *>((const char *)p.v_new + src);
        if (c == 0 && p.k_scale) {
            p.k_scale[row] = p.k_scale_new[i * p.num_kv_heads + g];
            p.v_scale[row] = p.v_scale_new[i * p.num_kv_heads + g];
        }
    }
}

// ---- dispatch -------------------------------------------------------------------

template <int D, int PS, int G, int QT, int KVT>
int launch_one(const DecodeParams &p, hipStream_t stream)
{
    dim3 grid((unsigned)p.num_partitions, (unsigned)p.num_kv_heads, (unsigned)p.batch);
    void *args[] = {const_cast<DecodeParams *>(&p)};
    return (int)hipLaunchKernel((const void *)&paged_decode_kernel<D, PS, G, QT, KVT>, grid,
                                dim3(kWaves * 64), args, 0, stream);
}

template <int D, int PS, int G>
int launch_dtype(const DecodeParams &p, int qt, int kvt, hipStream_t s)
{
    if (qt == F16 && kvt == F16) return launch_one<D, PS, G, F16, F16>(p, s);
    if (qt == BF16 && kvt == BF16) return launch_one<D, PS, G, BF16, BF16>(p, s);
    if (qt == F16 && kvt == I8) return launch_one<D, PS, G, F16, I8>(p, s);
    if (qt == BF16 && kvt == I8) return launch_one<D, PS, G, BF16, I8>(p, s);
    return (int)hipErrorInvalidValue;
}

template <int D, int PS>
int launch_group(const DecodeParams &p, int G, int qt, int kvt, hipStream_t s)
{
    switch (G) {
    case 1: return launch_dtype<D, PS, 1>(p, qt, kvt, s);
    case 2: return launch_dtype<D, PS, 2>(p, qt, kvt, s);
    case 4: return launch_dtype<D, PS, 4>(p, qt, kvt, s);
    case 8: return launch_dtype<D, PS, 8>(p, qt, kvt, s);
    }
    return (int)hipErrorInvalidValue;
}

}  // namespace

bool decode_instantiated(int D, int PS, int G, int qt, int kvt)
{
    bool pair = (qt == F16 && kvt == F16) || (qt == BF16 && kvt == BF16) ||
                ((qt == F16 || qt == BF16) && kvt == I8);
    return (D == 64 || D == 128) && (PS == 16 || PS == 64) && (G == 1 || G == 2 || G == 4 || G == 8) &&
           pair;
}

int launch_decode_partitions(const DecodeParams &p, int D, int PS, int G, int qt, int kvt, void *stream)
{
    hipStream_t s = (hipStream_t)stream;
    if (D == 64 && PS == 16) return launch_group<64, 16>(p, G, qt, kvt, s);
    if (D == 64 && PS == 64) return launch_group<64, 64>(p, G, qt, kvt, s);
    if (D == 128 && PS == 16) return launch_group<128, 16>(p, G, qt, kvt, s);
    if (D == 128 && PS == 64) return launch_group<128, 64>(p, G, qt, kvt, s);
    return (int)hipErrorInvalidValue;
}

int launch_splitk_reduce(const DecodeParams &p, int D, int qt, void *stream)
{
    const void *fn;
    if (D == 64 && qt == F16) fn = (const void *)&splitk_reduce_kernel<64, F16>;
    else if (D == 64 && qt == BF16) fn = (const void *)&splitk_reduce_kernel<64, BF16>;
    else if (D == 128 && qt == F16) fn = (const void *)&splitk_reduce_kernel<128, F16>;
    else if (D == 128 && qt == BF16) fn = (const void *)&splitk_reduce_kernel<128, BF16>;
    else return (int)hipErrorInvalidValue;
    void *args[] = {const_cast<DecodeParams *>(&p)};
    return (int)hipLaunchKernel(fn, dim3((unsigned)p.num_q_heads, (unsigned)p.batch), dim3(256), args, 0,
                                (hipStream_t)stream);
}

int launch_write_kv(const WriteParams &p, void *stream)
{
    const size_t total = (size_t)p.n * p.num_kv_heads * (p.row_bytes / 16);
    size_t blocks = (total + 255) / 256;
    if (blocks > 65535)
        blocks = 65535;
    void *args[] = {const_cast<WriteParams *>(&p)};
    return (int)hipLaunchKernel((const void *)&write_kv_kernel, dim3((unsigned)blocks), dim3(256), args, 0,
                                (hipStream_t)stream);
}

}  // namespace pkv
