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
// Design.  One workgroup of eight waves per (block of query tokens, KV head,
// sequence), head_dim 64 or 128, placed so that the blocks of one (sequence,
// KV head) run on one XCD and the XCDs get an even mix of sequences.  Its 256
// rows are (token, head of the group) pairs, token-major: 256 / G query
// tokens of the G heads sharing the KV head, 32 rows per wave.
// Both contractions run on the matrix cores as 32 x 32 products
// (v_mfma_f32_32x32x16_{bf16,f16}: D[32][32] += A[32][16] . B[16][32]; lane
// l = (h, c) = (l/32, l%32) supplies A[c][8h + i] and B[8h + i][c], i < 8,
// and holds D[8(j/4) + 4h + j%4][c], j < 16), written transposed so that
// everything a lane needs for its softmax and output stays in its registers:
//
//  * S^T = K . q^T per 32-key block: K (LDS, row-major) is the A operand,
//    q (registers, the wave's 32 rows) the B operand.  Lane (h, c) ends with
//    the scores of ONE query row (c) against 16 of the block's keys; the
//    other 16 are in lane (1 - h, c).
//  * Online softmax per row in the exp2 domain: one lane exchange per tile
//    for the max, the sum combined at the end.  The causal mask is applied
//    only on tiles that reach past a valid row's position, and the
//    reference max is raised only when a tile's max passes it by more than
//    2^8, so O is rarely rescaled.
//  * O^T += V^T . P^T per 16-key step: transposed V (LDS) is the A operand
//    and the row's probabilities, rounded to q's type, are the B operand
//    straight from the score registers -- the keys of a step are taken in
//    the order the score layout holds them (4h .. 4h+3, 8 + 4h .. 8 + 4h + 3),
//    and transposed V is stored with the middle quarters of every 16 keys
//    swapped so that this order is one 16-byte read.  O^T[dim][row] lands in
//    the lane of its row: no cross-lane work until the output.
//  * K and V of a 64-key tile are loaded by the whole workgroup, 16 bytes per
//    thread per piece, through the block table (one page per tile for
//    64-token pages, four for 16-token pages, read as scalar loads a tile
//    early).  The loads are issued one tile before their LDS store (one
//    register set) and the stores one tile before the arithmetic (two LDS
//    buffers, one barrier per tile), with no branch around a load or a
//    store, so the waits before the stores cover only the loads they need.
//    V of keys past the block's last position is cleared at the store.  K is
//    stored row-major; each thread holds consecutive keys of eight dims of V
//    (two keys at head_dim 128, four at 64) and writes them transposed, 4 or
//    8 bytes per dim.
//  * int8 / E4M3 caches: 8-byte pieces of codes, widened exactly at the LDS
//    store (every int8 and E4M3 value is a bf16 and an f16 value) -- K to
//    q's type, V to f16, the type of the p.V product for these caches;
//    the tile's per-token K and V scales go to LDS beside it, the K scale
//    multiplies each score and the V scale each probability that weights V
//    (the running sum takes the probabilities without it).  The
//    exponentials carry 2^-e, with 2^e above every V scale seen so far, so
//    the f16 products stay in range and normal for any scale magnitude; O
//    and the sum carry the same factor (both rescaled by a power of two when
//    e grows), which O / sum cancels.
//
// Key tiles after the block's last position are not visited.  A sequence
// whose context length is invalid (negative, above the bound, shorter than
// its chunk, or a chunk longer than max_q_len) gets NaN rows, as does a
// block that needs a page outside the pool.

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

constexpr int kKeyTile = 64;          // keys per tile
constexpr int kRows = 256;            // query rows per workgroup (8 waves x 32)
constexpr int kThreads = 512;        // threads per workgroup
constexpr int kVStride = kKeyTile + 8;  // LDS row of transposed V (16-bit elements), padded
constexpr unsigned kXcds = 8;         // XCDs of MI355X

typedef __attribute__((ext_vector_type(2))) u32 u32x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;

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
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c)
{
    if constexpr (QT == BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
}

template <int N, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    [&]<int... I>(std::integer_sequence<int, I...>) { (f(std::integral_constant<int, I>{}), ...); }
        (std::make_integer_sequence<int, N>{});
}

// Eight int8 or OCP E4M3 codes (w.x bytes 0..3, w.y bytes 0..3) widened to
// eight values of q's 16-bit type, exactly (every int8 and every E4M3 value
// is a bf16 and an f16 value); 16-bit K/V pass through.
template <int QT, int KVT, class Raw>
__device__ __forceinline__ u32x4 widen(const Raw &w)
{
    if constexpr (KVT == FP8) {
        auto pair = [](u32 x, auto HIc) -> u32 {
            constexpr bool HI = decltype(HIc)::value;
            if constexpr (QT == BF16)
                return __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, HI));
            else
                return __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, HI));
        };
        const std::false_type lo{};
        const std::true_type hi{};
        return u32x4{pair(w.x, lo), pair(w.x, hi), pair(w.y, lo), pair(w.y, hi)};
    } else if constexpr (KVT == I8) {
        auto pair = [](u32 x, int sh) -> u32 {
            const float a = (float)(int8_t)(x >> sh), b = (float)(int8_t)(x >> (sh + 8));
            return pack2<QT>(a, b);
        };
        return u32x4{pair(w.x, 0), pair(w.x, 16), pair(w.y, 0), pair(w.y, 16)};
    } else {
        return w;
    }
}

// Column of key k (0..63 in the tile) in a row of transposed V: the middle
// quarters of every 16 keys are swapped, so that keys 4h .. 4h+3 and
// 8 + 4h .. 8 + 4h + 3 of a 16-key step sit at columns 8h .. 8h+7.
__device__ __forceinline__ int vt_column(int k)
{
    const int q = (k / 4) % 4;
    const int sq = q == 1 ? 2 : q == 2 ? 1 : q;
    return 16 * (k / 16) + 4 * sq + k % 4;
}

// Lane j of each 16-lane row reads lane (j + N) mod 16 of its row (DPP
// row_ror; no LDS round trip).
template <int N>
__device__ __forceinline__ float row_ror(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x120 + N, 0xF,
                                                                 0xF, false));
}

template <int D, int PS, int G, int QT, int KVT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void paged_prefill_kernel(PrefillParams p)
{
    constexpr int kD = D;                     // head_dim: 64 or 128
    constexpr int kKStride = kD + 8;          // LDS row of K (16-bit elements), padded
    constexpr int NQS = kD / 16;              // q.k steps of 16 dims
    constexpr int NDB = kD / 32;              // 32-dim blocks of the output
    constexpr int CPR = kD / 8;               // 16-bit 8-element chunks per K/V row
    constexpr int NKP = kKeyTile * CPR / kThreads; // K pieces per thread
    constexpr int QPB = kRows / G;            // query tokens per block
    constexpr int PPT = kKeyTile / PS;        // pages per key tile
    // byte K/V (int8 or E4M3 codes with one fp32 scale per token and KV head):
    // 8-byte pieces, widened to q's type at the LDS store
    constexpr bool kByte = KVT == I8 || KVT == FP8;
    constexpr int EB = kByte ? 1 : 2;         // bytes per K/V element
    using Raw = std::conditional_t<kByte, u32x2, u32x4>;
    // type of the p.V product: q's type for 16-bit K/V; f16 for byte K/V,
    // whose codes are exact in f16, so that the probabilities (times the V
    // scale) round to 11 bits instead of bf16's 8
    constexpr int PT = kByte ? F16 : QT;
    // two buffers: tile t is read from buffer t % 2 while tile t + 1 is stored
    // into the other one
    __shared__ __attribute__((aligned(16))) uint16_t s_k[2][kKeyTile * kKStride];
    __shared__ __attribute__((aligned(16))) uint16_t s_vt[2][kD * kVStride];
    // byte K/V: the tile's K scales (row 0) and V scales (row 1), per key,
    // and the largest V scale magnitude of the tile
    __shared__ __attribute__((aligned(16))) float s_sc[2][2][kByte ? kKeyTile : 4];
    __shared__ float s_vmax[2];

    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    const int h = lane / 32, c = lane % 32;
    const int Hq = p.num_q_heads, Hkv = p.num_kv_heads;
    // Work item of this workgroup.  The dispatcher deals workgroup L to XCD
    // L mod 8.  The (sequence, KV head) pairs are dealt to the XCDs in turn
    // (pair P to XCD P mod 8), and all query blocks of a pair go to its XCD,
    // one after another: the blocks that re-read a pair's K/V share one L2,
    // and every XCD gets an even mix of sequences.  Workgroups past the last
    // pair have no work.
    int qblk, g, b;
    {
        const unsigned L = blockIdx.x, x = L % kXcds, slot = L / kXcds;
        const unsigned nqb = (unsigned)((p.max_q_len + QPB - 1) / QPB);
        const unsigned pair = slot / nqb * kXcds + x;
        if (pair >= (unsigned)p.batch * (unsigned)Hkv)
            return;
        qblk = (int)(slot % nqb);
        g = (int)(pair % (unsigned)Hkv);
        b = (int)(pair / (unsigned)Hkv);
    }

    const int qs0 = p.q_start[b], qs1 = p.q_start[b + 1];
    if (qs0 < 0 || qs1 < qs0 || qs1 > p.n_q)
        return;   // no rows that can be written safely
    const int nq = qs1 - qs0;
    const int i0 = qblk * QPB;
    if (i0 >= nq)
        return;
    const int n = p.context_lens[b];
    // a chunk longer than max_q_len has rows no launched block covers: the
    // blocks that do run write NaN, so the sequence is visibly invalid
    const bool bad_len = n < 0 || n > p.max_context_len || nq > n || nq > p.max_q_len;
    const int tok_hi = min(nq, i0 + QPB);   // this block's query tokens: [i0, tok_hi)

    // this lane's query row: column c of the wave's 32 rows
    const int row = 32 * wave + c;
    const int tok = i0 + row / G, head = g * G + row % G;
    const bool valid_row = tok < tok_hi;
    const int pos = valid_row && !bad_len ? n - nq + tok : -1;   // -1: masks every key
    // A negative scale is applied as |scale| to -q (a sign flip, exact), so
    // that the row maximum of the raw scores is the maximum of the scaled
    // ones.  A zero scale is taken as 1e-30: 2^(1e-30 s) rounds to exactly 1
    // for any finite score s below 1e22, and a masked key (-inf) still gives 0.
    const float scale = fmaxf(fabsf(p.scale_log2), 1.0e-30f);
    const u32 qsign = p.scale_log2 < 0.0f ? 0x80008000u : 0u;
    u32x4 qb[NQS];   // B operand of step s: q[row][16s + 8h .. +8]
    {
        const char *qrow = (const char *)p.q + (((size_t)(qs0 + (valid_row ? tok : i0)) * Hq + head) * kD) * 2;
#pragma unroll
        for (int s = 0; s < NQS; ++s) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(qrow + (16 * s + 8 * h) * 2) ^ qsign;
            qb[s] = valid_row ? v : u32x4{0u, 0u, 0u, 0u};
        }
    }
    const int last_pos = bad_len ? -1 : n - nq + tok_hi - 1;
    const int n_tiles = last_pos < 0 ? 0 : last_pos / kKeyTile + 1;

    // ---- key-tile loads.  K: thread tid moves dims 8 (tid % CPR) .. +8 of
    // keys tid / CPR + (512 / CPR) j (j < NKP).  V: see KPT below.
    const size_t page_stride = (size_t)Hkv * PS * kD;   // elements
    // The block table is only read here: through the constant address space
    // its (wave-uniform) entries are scalar loads, which are counted apart
    // from the K/V loads in flight.
    typedef const __attribute__((address_space(4))) int32_t *const_i32p;
    const const_i32p bt = (const_i32p)(uintptr_t)(p.block_tables + (size_t)b * p.max_blocks);
    // V: KPT consecutive keys of 8 dims per thread -- two at head_dim 128,
    // where the 512 threads cover the tile exactly; four at head_dim 64, where
    // threads 0..127 do (the others load a duplicate and store nothing).
    constexpr int KPT = CPR == 16 ? 2 : 4;
    const int kg = KPT == 2 ? tid % 32 : tid % 16;          // key group: keys KPT kg .. +KPT
    const int dv = KPT == 2 ? tid / 32 : (tid / 16) % CPR;  // dims 8 dv .. +8
    const bool vstore = KPT == 2 || tid / 16 < CPR;
    const int kc = tid % CPR;
    bool bad = false;
    // Physical pages of a tile, one per 16 or 64 keys, -1 for none.  They are
    // read one iteration before the tile's loads are issued, so that the wait
    // for them never drains the loads in flight.
    auto fetch_pages = [&](int tile, int (&pg)[PPT]) {
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int blk = tile * PPT + i;
            pg[i] = bt[min(blk, p.max_blocks - 1)];
            pg[i] = blk < p.max_blocks ? pg[i] : -1;
        }
    };
    // Every load is issued, from page 0 when the key's page is outside the
    // pool, with no branch around it and no use of its value until the LDS
    // store, so the compiler can keep two tiles in flight.  K of keys past the
    // block's last position needs no clearing: their scores are masked (the
    // tile then reaches past every valid row's position) and the mask replaces
    // the value.  V of those keys is cleared at the store (vm: one bit per
    // key this thread holds), since a zero probability times a NaN would
    // still be NaN.
    // Byte K/V: threads 0..63 also load the K scale, 64..127 the V scale, of
    // key tid % 64 (cleared at the store past the last position: bit 4 of vm).
    auto load_tile = [&](int tile, const int (&pg)[PPT], Raw (&kr)[NKP], Raw (&vr)[4], float &sr, unsigned &vm) {
        const int key0 = tile * kKeyTile;
#pragma unroll
        for (int j = 0; j < NKP; ++j) {
            const int kk = tid / CPR + (kThreads / CPR) * j;
            int page = pg[0];
            if constexpr (PPT > 1) {
                const int pi = __builtin_amdgcn_readfirstlane(kk / PS);
#pragma unroll
                for (int i = 1; i < PPT; ++i)
                    page = pi == i ? pg[i] : page;
            }
            const bool want = key0 + kk <= last_pos;
            const bool inside = (unsigned)page < (unsigned)p.num_pages;
            bad = bad || (want && !inside);
            kr[j] = *reinterpret_cast<const Raw *>((const char *)p.k_pool +
                                                   ((size_t)(inside ? page : 0) * page_stride +
                                                    ((size_t)g * PS + kk % PS) * kD + 8 * kc) * EB);
        }
        int vpage = pg[0];
        if constexpr (PPT > 1) {
#pragma unroll
            for (int i = 1; i < PPT; ++i)
                vpage = kg / (PS / KPT) == i ? pg[i] : vpage;
        }
        const bool vinside = (unsigned)vpage < (unsigned)p.num_pages;
        vm = 0;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int kk = KPT * kg + j;
            const bool want = key0 + kk <= last_pos;
            bad = bad || (want && !vinside);
            vm |= want && vinside ? 1u << j : 0u;
            vr[j] = *reinterpret_cast<const Raw *>((const char *)p.v_pool +
                                                   ((size_t)(vinside ? vpage : 0) * page_stride +
                                                    ((size_t)g * PS + kk % PS) * kD + 8 * dv) * EB);
        }
        if constexpr (kByte) {
            const int kk = tid % 64;
            int spage = pg[0];
            if constexpr (PPT > 1) {
#pragma unroll
                for (int i = 1; i < PPT; ++i)
                    spage = kk / PS == i ? pg[i] : spage;
            }
            const bool sinside = (unsigned)spage < (unsigned)p.num_pages;
            const bool want = key0 + kk <= last_pos && sinside;
            vm |= want ? 16u : 0u;
            const float *src = tid < 64 ? p.k_scale : p.v_scale;
            sr = src[((size_t)(sinside ? spage : 0) * Hkv + g) * PS + kk % PS];
        }
    };
    const int vcol = vt_column(KPT * kg);
    auto store_tile = [&](int buf, const Raw (&kraw)[NKP], const Raw (&vraw)[4], float sr, unsigned vm) {
        u32x4 vr[KPT];
#pragma unroll
        for (int j = 0; j < KPT; ++j)
            vr[j] = (vm >> j) & 1u ? widen<PT, KVT>(vraw[j]) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < NKP; ++j)
            *reinterpret_cast<u32x4 *>(&s_k[buf][(tid / CPR + (kThreads / CPR) * j) * kKStride + 8 * kc]) =
                widen<QT, KVT>(kraw[j]);
        if constexpr (kByte) {
            const float sv = (vm & 16u) ? sr : 0.0f;
            if (tid < 128)
                s_sc[buf][tid / 64][tid % 64] = sv;
            if (wave == 1) {
                // threads 64..127 (one wave) hold the tile's V scales: the max
                // over each 16-lane row by DPP rotations, then over the rows
                float m = fabsf(sv);
                m = fmaxf(m, row_ror<8>(m));
                m = fmaxf(m, row_ror<4>(m));
                m = fmaxf(m, row_ror<2>(m));
                m = fmaxf(m, row_ror<1>(m));
                auto at = [&](int l) {
                    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m), l));
                };
                m = fmaxf(fmaxf(at(0), at(16)), fmaxf(at(32), at(48)));
                if (lane == 0)
                    s_vmax[buf] = m;
            }
        }
        // the KPT keys of dims 8 dv + 2 w (low halves) and 8 dv + 2 w + 1 (high
        // halves): consecutive keys stay consecutive in a transposed row
        if (vstore)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const u32 lo01 = (vr[0][w] & 0xFFFFu) | (vr[1][w] << 16);
            const u32 hi01 = (vr[0][w] >> 16) | (vr[1][w] & 0xFFFF0000u);
            if constexpr (KPT == 2) {
                *reinterpret_cast<u32 *>(&s_vt[buf][(8 * dv + 2 * w) * kVStride + vcol]) = lo01;
                *reinterpret_cast<u32 *>(&s_vt[buf][(8 * dv + 2 * w + 1) * kVStride + vcol]) = hi01;
            } else {
                const u32 lo23 = (vr[2][w] & 0xFFFFu) | (vr[3][w] << 16);
                const u32 hi23 = (vr[2][w] >> 16) | (vr[3][w] & 0xFFFF0000u);
                *reinterpret_cast<u32x2 *>(&s_vt[buf][(8 * dv + 2 * w) * kVStride + vcol]) = u32x2{lo01, lo23};
                *reinterpret_cast<u32x2 *>(&s_vt[buf][(8 * dv + 2 * w + 1) * kVStride + vcol]) = u32x2{hi01, hi23};
            }
        }
    };

    f32x16 oacc[NDB];   // O^T[dim 32 db + 8 (j/4) + 4 h + j%4][row c] in oacc[db][j]
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j)
            oacc[db][j] = 0.0f;
    // Reference max of the row's exponentials, in log2 units.  It starts
    // finite (a row with no visible key yet gets probabilities 0, never
    // (-inf) - (-inf)) and is raised only when a tile's max exceeds it by more
    // than kSlack: the probabilities then stay below 2^kSlack, and O and the
    // sum, scaled by the same stale reference, still give O / sum exactly.
    constexpr float kSlack = 8.0f;
    float m_run = -3.0e38f, l_run = 0.0f;
    // Byte K/V: the probabilities that weight V are multiplied by the key's V
    // scale and rounded to f16 for the p.V product.  To keep that product in
    // f16's normal range whatever the scales' magnitude, the exponentials
    // carry 2^-e_run, with 2^e_run above every V scale seen so far (e_run only
    // grows, tile by tile; O and the sum are rescaled by a power of two, an
    // exact step, when it does), so O and the sum share the factor and O /
    // sum is the output.  The V scales of a tile are the same for every row,
    // so e_run is uniform over the workgroup.  kNoExp: no nonzero V scale
    // seen yet (O is zero; the sum is kept in units of 2^0 until then).
    constexpr int kNoExp = -1000;
    int e_run = kNoExp;

    // One register set carries tile t + 1 from its loads (issued while tile
    // t - 1 is computed) to its LDS store (before tile t is computed); the
    // pages of a tile are read one iteration before its loads.  Loads are
    // issued for every tile index, clamped to the last tile (whose extra copies
    // are never read), so that no branch surrounds a load or a store and the
    // waits before the stores cover exactly the loads they need.
    Raw kreg[NKP], vreg[4];
    float sreg = 0.0f;
    unsigned vmask = 0;
    int pgn[PPT];   // pages of the next tile to load
    const int last_tile = n_tiles - 1;
    if (n_tiles > 0) {
        fetch_pages(0, pgn);
        load_tile(0, pgn, kreg, vreg, sreg, vmask);
        store_tile(0, kreg, vreg, sreg, vmask);
        fetch_pages(min(1, last_tile), pgn);
        load_tile(min(1, last_tile), pgn, kreg, vreg, sreg, vmask);
        fetch_pages(min(2, last_tile), pgn);
    }
    // tile `tile` is in LDS buffer BUF; kreg / vreg hold tile + 1
    auto tile_body = [&](int tile, auto BUFc) {
        constexpr int BUF = decltype(BUFc)::value;
        // every wave is done with tile - 1 (buffer 1 - BUF), and tile's
        // stores (buffer BUF) are complete
        __syncthreads();
        store_tile(1 - BUF, kreg, vreg, sreg, vmask);   // unread when tile + 1 is the pad tile or past it
        {
            int pg[PPT];
#pragma unroll
            for (int i = 0; i < PPT; ++i)
                pg[i] = pgn[i];
            fetch_pages(min(tile + 3, last_tile), pgn);   // before this tile's loads
            load_tile(min(tile + 2, last_tile), pg, kreg, vreg, sreg, vmask);
        }

        // ---- scores S^T[key 32 kb + 8 (j/4) + 4 h + j%4][row c] in sc[kb][j]
        f32x16 sc[2];
        static_for<2>([&](auto KBc) {
            constexpr int KB = decltype(KBc)::value;
            f32x16 x;
#pragma unroll
            for (int j = 0; j < 16; ++j)
                x[j] = 0.0f;
#pragma unroll
            for (int s = 0; s < NQS; ++s) {
                const u32x4 kop =
                    *reinterpret_cast<const u32x4 *>(&s_k[BUF][(32 * KB + c) * kKStride + 16 * s + 8 * h]);
                x = mfma32<QT>(kop, qb[s], x);
            }
            sc[KB] = x;
        });

        // byte K/V: each score times its key's K scale (lane (h, c) holds keys
        // 32 kb + 8 j4 + 4 h .. +3 in registers 4 j4 .. 4 j4 + 3)
        if constexpr (kByte) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j4 = 0; j4 < 4; ++j4) {
                    const float4 ks = *reinterpret_cast<const float4 *>(&s_sc[BUF][0][32 * kb + 8 * j4 + 4 * h]);
                    sc[kb][4 * j4] *= ks.x;
                    sc[kb][4 * j4 + 1] *= ks.y;
                    sc[kb][4 * j4 + 2] *= ks.z;
                    sc[kb][4 * j4 + 3] *= ks.w;
                }
        }

        // ---- online softmax of row c (log2 domain).  The causal mask is
        // needed only in tiles that reach past some valid row's position.
        const int key0 = tile * kKeyTile + 4 * h;
        const bool masked = __builtin_amdgcn_ballot_w64(valid_row && tile * kKeyTile + kKeyTile - 1 > pos) != 0;
        if (masked) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int key = key0 + 32 * kb + 8 * (j / 4) + j % 4;
                    sc[kb][j] = key <= pos ? sc[kb][j] : -INFINITY;
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                mx = fmaxf(mx, sc[kb][j]);
        mx = fmaxf(mx, __shfl_xor(mx, 32)) * scale;
        const bool grow = mx > m_run + kSlack;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            const float m_new = grow ? mx : m_run;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
            m_run = m_new;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    oacc[db][j] *= alpha;
        }
        // byte K/V: O and the sum are kept in units of 2^-e_run (e_run
        // raised, never lowered, to the exponent bound of the largest V
        // scale seen; O and the sum then scaled by the same power of two, an
        // exact step), so the exponentials below carry 2^-e_run and O / sum
        // needs no correction at the end
        float m_eff = m_run;
        if constexpr (kByte) {
            const float vmax = s_vmax[BUF];
            // 2^e_tile > vmax: the biased exponent of vmax minus 126
            // (clamped to [-64, 64], which keeps the sum's terms, at most
            // 2^(8 - e_run), inside fp32 for scales of any magnitude)
            const int e_tile = vmax > 0.0f
                                   ? min(max((int)((__builtin_bit_cast(u32, vmax) >> 23) & 0xFFu) - 126, -64), 64)
                                   : kNoExp;
            if (e_tile > e_run) {
                const int d = (e_run == kNoExp ? 0 : e_run) - e_tile;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int j = 0; j < 16; ++j)
                        oacc[db][j] = ldexpf(oacc[db][j], d);
                l_run = ldexpf(l_run, d);
                e_run = e_tile;
            }
            m_eff = m_run + (float)(e_run == kNoExp ? 0 : e_run);
        }
        float ls = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                // a masked key (-inf) gives 0
                const float e = __builtin_amdgcn_exp2f(fmaf(sc[kb][j], scale, -m_eff));
                sc[kb][j] = e;
                ls += e;
            }
        l_run += ls;
        // byte K/V: the probabilities that weight V carry its V scale (the
        // sum above does not)
        if constexpr (kByte) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j4 = 0; j4 < 4; ++j4) {
                    const float4 vs = *reinterpret_cast<const float4 *>(&s_sc[BUF][1][32 * kb + 8 * j4 + 4 * h]);
                    sc[kb][4 * j4] *= vs.x;
                    sc[kb][4 * j4 + 1] *= vs.y;
                    sc[kb][4 * j4 + 2] *= vs.z;
                    sc[kb][4 * j4 + 3] *= vs.w;
                }
        }

        // ---- P^T operand of 16-key step ks: keys 16 ks + 4h .. +3, 16 ks + 8 + 4h .. +3
        u32x4 pb[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int kb = ks / 2, j0 = 8 * (ks % 2);
            pb[ks] = u32x4{pack2<PT>(sc[kb][j0], sc[kb][j0 + 1]), pack2<PT>(sc[kb][j0 + 2], sc[kb][j0 + 3]),
                           pack2<PT>(sc[kb][j0 + 4], sc[kb][j0 + 5]), pack2<PT>(sc[kb][j0 + 6], sc[kb][j0 + 7])};
        }
        // ---- O^T[dim][row] += V^T[dim][key] . P^T[key][row]
        static_for<NDB>([&](auto DBc) {
            constexpr int DB = decltype(DBc)::value;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const u32x4 vop =
                    *reinterpret_cast<const u32x4 *>(&s_vt[BUF][(32 * DB + c) * kVStride + 16 * ks + 8 * h]);
                oacc[DB] = mfma32<PT>(vop, pb[ks], oacc[DB]);
            }
        });
    };
    // An odd tile count gets one pad tile: its keys lie past every row's
    // position, so its probabilities (and its cleared V) are zero.  Both
    // halves of the unrolled loop then always run, with no branch around a
    // load or store, which keeps the waits before the stores partial.
    for (int tile = 0; tile < n_tiles; tile += 2) {
        tile_body(tile, std::integral_constant<int, 0>{});
        tile_body(tile + 1, std::integral_constant<int, 1>{});
    }

    // ---- finalize: O / l, written in q's type
    const bool any_bad = __syncthreads_or(bad ? 1 : 0) != 0 || bad_len;
    const float l = l_run + __shfl_xor(l_run, 32);
    if (!valid_row)
        return;
    const float inv = any_bad ? __builtin_nanf("") : 1.0f / l;
    auto fin = [&](float x) { return x * inv; };
    u32x2 *orow = reinterpret_cast<u32x2 *>((uint16_t *)p.out + ((size_t)(qs0 + tok) * Hq + head) * kD);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
            // dims 32 db + 8 j4 + 4 h .. +3
            const int j = 4 * j4;
            orow[(32 * db + 8 * j4 + 4 * h) / 4] = u32x2{pack2<QT>(fin(oacc[db][j]), fin(oacc[db][j + 1])),
                                                        pack2<QT>(fin(oacc[db][j + 2]), fin(oacc[db][j + 3]))};
        }
}

template <int D, int PS, int G, int QT>
const void *kernel_for(int kv_dtype)
{
    if (kv_dtype == I8)
        return (const void *)&paged_prefill_kernel<D, PS, G, QT, I8>;
    if (kv_dtype == FP8)
        return (const void *)&paged_prefill_kernel<D, PS, G, QT, FP8>;
    return (const void *)&paged_prefill_kernel<D, PS, G, QT, QT>;
}

template <int D, int PS, int G>
const void *kernel_for_q(const PrefillParams &p)
{
    return p.q_dtype == BF16 ? kernel_for<D, PS, G, BF16>(p.kv_dtype) : kernel_for<D, PS, G, F16>(p.kv_dtype);
}

template <int PS, int G>
int launch_g(const PrefillParams &p, int head_dim, dim3 grid, hipStream_t s)
{
    void *args[] = {const_cast<PrefillParams *>(&p)};
    const void *fn = head_dim == 64 ? kernel_for_q<64, PS, G>(p) : kernel_for_q<128, PS, G>(p);
    return (int)hipLaunchKernel(fn, grid, dim3(kThreads), args, 0, s);
}

template <int PS>
int launch_ps(const PrefillParams &p, int G, dim3 grid, hipStream_t s)
{
    switch (G) {
    case 1: return launch_g<PS, 1>(p, p.head_dim, grid, s);
    case 2: return launch_g<PS, 2>(p, p.head_dim, grid, s);
    case 4: return launch_g<PS, 4>(p, p.head_dim, grid, s);
    case 8: return launch_g<PS, 8>(p, p.head_dim, grid, s);
    }
    return (int)hipErrorInvalidValue;
}

}  // namespace

bool prefill_instantiated(int head_dim, int page_size, int group, int q_dtype, int kv_dtype)
{
    return (head_dim == 64 || head_dim == 128) && (page_size == 16 || page_size == 64) &&
           (group == 1 || group == 2 || group == 4 || group == 8) && (q_dtype == F16 || q_dtype == BF16) &&
           (kv_dtype == q_dtype || kv_dtype == I8 || kv_dtype == FP8);
}

int launch_prefill(const PrefillParams &p, int page_size, int group, void *stream)
{
    const int qpb = kRows / group;
    const size_t pairs = (size_t)p.batch * p.num_kv_heads;
    const size_t items = (pairs + kXcds - 1) / kXcds * kXcds * (size_t)((p.max_q_len + qpb - 1) / qpb);
    if (items > 0x7FFFFFFFu)
        return (int)hipErrorInvalidValue;
    const dim3 grid((unsigned)items);
    hipStream_t s = (hipStream_t)stream;
    if (p.head_dim != 64 && p.head_dim != 128)
        return (int)hipErrorInvalidValue;
    if (page_size == 16)
        return launch_ps<16>(p, group, grid, s);
    if (page_size == 64)
        return launch_ps<64>(p, group, grid, s);
    return (int)hipErrorInvalidValue;
}

}  // namespace pkv
