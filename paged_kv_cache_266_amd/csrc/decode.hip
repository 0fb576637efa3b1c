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
// Design.  The batch's work is the flat list of 64-token tiles of all
// (sequence, KV head) segments; a persistent grid of single-wave workgroups
// splits it into equal contiguous shares, whatever the length mix, so every
// wave streams the same number of tiles (the split-K of long contexts and the
// load balance of ragged batches are one mechanism).  Per wave:
//
//  * Loads.  A (page, KV head) tile is one contiguous run of page_size rows.
//    Each lane loads 16 bytes per instruction through a buffer descriptor
//    whose base is the page and whose size is the tile, so one instruction
//    reads 1 KiB of consecutive rows (R = row_bytes/16 lanes per token row,
//    64/R tokens per instruction), non-temporal.  Slots past the context
//    length get an out-of-range offset and read as zero without touching
//    memory: no garbage (or NaN) from a partly filled last page ever enters a
//    product.
//  * Pipelining.  One ring of R 16-byte registers per lane holds K of tile t,
//    then V of tile t, then K of tile t+1: each chunk's V load is issued as
//    soon as its K has been used and the next tile's K as soon as its V has
//    been used, so a tile of K/V is always in flight behind the arithmetic,
//    across segment boundaries too (the next segment's q is fetched behind
//    the next tile's K loads).
//  * q.k.  Lane (row r, column j) holds 16 bytes of one token row and the
//    matching slice of each of the G query heads of the group; dot2
//    instructions (f16/bf16) or byte conversions + FMAs (int8) give partial
//    dots, folded into a DPP reduce-scatter tree over the R lanes of a row
//    chunk by chunk.  Each lane ends with the full scores of ONE token (token
//    r + (64/R) j of the tile) for all G heads -- no redundant softmax work.
//  * Online softmax.  Tile max per head by DPP row rotations and a
//    wave-uniform combine of the four rows; running max, per-lane running
//    sums, exp2 with log2(e) folded into the scale.  For int8, the V scale of
//    the token is folded into its probability and the K scale into its score.
//  * p.V.  Probabilities go to a per-wave LDS slot; each lane then reads, per
//    chunk, the G probabilities of the token whose V bytes it holds
//    (broadcast reads) and accumulates G x (elements per lane) fp32 sums.
//  * Combine.  Token rows are summed across lanes.  A segment a wave covers
//    whole is written directly; the pieces of a segment shared by waves go to
//    the workspace as (max, sum, unnormalised output) and are merged, after
//    the main loop, by the last wave to finish each group of them (or, in the
//    two-launch form, by the merge kernel).
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
typedef __attribute__((ext_vector_type(2))) u32 u32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;

// Cache policy of the K/V loads: non-temporal.  Every K/V byte is read once
// per step, so keeping it out of the caches' normal replacement raises the
// sustained read rate (measured on gfx950: ~6.8 vs ~6.05 TB/s for a pure
// page-tile stream).
#ifndef PKV_KV_CPOL
#define PKV_KV_CPOL 2
#endif
constexpr int kStreamingLoad = PKV_KV_CPOL;

constexpr u32 kBufferFlags = 0x00020000u;  // gfx9 raw buffer: 32-bit data format
constexpr int kOutOfRange = 0x7FFFFFF0;    // voffset that fails the range check

// ---- lane exchange ---------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                                 0xF, 0xF, false));
}

// DPP controls (lane j of a 16-lane row reads lane ...):
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]: j ^ 1
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]: j ^ 2
constexpr int kRowRor4 = 0x124;       // row_ror 4: j - 4 (mod 16)
constexpr int kRowRor8 = 0x128;       // row_ror 8: j ^ 8

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

// Reduce-scatter of per-chunk partial dots over the R lanes of a token row,
// built as a binary tree from the lowest column bit up so that chunks can be
// folded in as soon as they are computed.  At level b, lanes whose column has
// bit b clear keep the lower of two values (chunk range with that bit 0) and
// add their partner's copy of it; lanes with the bit set keep the upper one.
// After log2(R) levels, column j holds the full dot of chunk j.
//
// Partner lane at level b is j ^ 2^b: quad permutations for b < 2; for b = 2
// the lower lane reads j + 4 (row_ror 12) and the upper lane j - 4
// (row_ror 4); for b = 3, row_ror 8.
template <int B>
struct Level;
template <> struct Level<0> { static constexpr int lo = kQuadXor1, up = kQuadXor1; };
template <> struct Level<1> { static constexpr int lo = kQuadXor2, up = kQuadXor2; };
template <> struct Level<2> { static constexpr int lo = 0x12C, up = kRowRor4; };
template <> struct Level<3> { static constexpr int lo = kRowRor8, up = kRowRor8; };

template <int B, int G>
__device__ __forceinline__ void tree_combine(float (&lo)[G], const float (&up)[G], int j)
{
    const bool upper = (j >> B) & 1;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float a = lo[h] + dpp<Level<B>::lo>(lo[h]);
        const float c = up[h] + dpp<Level<B>::up>(up[h]);
        lo[h] = upper ? c : a;
    }
}

// Fold chunk I's partials v into the pending-value stack (binary counter on I).
template <int I, int B, int LEVELS, int G>
__device__ __forceinline__ void tree_push(float (&stack)[LEVELS + 1][G], float (&v)[G], int j)
{
    if constexpr (B < LEVELS && ((I >> B) & 1)) {
        tree_combine<B, G>(stack[B], v, j);
#pragma unroll
        for (int h = 0; h < G; ++h)
            v[h] = stack[B][h];
        tree_push<I, B + 1, LEVELS, G>(stack, v, j);
    } else {
#pragma unroll
        for (int h = 0; h < G; ++h)
            stack[B][h] = v[h];
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

// Two OCP E4M3 values (bytes 0, 1, or bytes 2, 3 of w) as floats; the
// gfx950 converter decodes exactly this format (checked on the hardware
// against the format definition for all 256 codes).
template <bool HI>
__device__ __forceinline__ float2 fp8_pair(u32 w)
{
    const auto v = __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
    return make_float2(v[0], v[1]);
}

// Two E4M3 codes of w (bytes 2*HI and 2*HI + 1) widened to a packed pair of
// q's 16-bit type (v_cvt_scalef32_pk_{bf16,f16}_fp8 with scale 1): exact, as
// every E4M3 value is a bf16 and an f16 value.
template <int QT, bool HI>
__device__ __forceinline__ u32 fp8_pair16(u32 w)
{
    if constexpr (QT == BF16)
        return __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
    else
        return __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}

// Unsigned byte e of w as float (v_cvt_f32_ubyteN).
template <int E>
__device__ __forceinline__ float ubyte(u32 w) { return (float)((w >> (8 * E)) & 0xFFu); }

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t rsrc, int voff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, 0, 0);
}

// The tile cursor is the same on every lane, but the compiler cannot prove
// it; a buffer descriptor built from a per-lane value costs a loop over the
// distinct values around every load.  Reading the address from the first
// active lane puts it in scalar registers.
__device__ __forceinline__ const char *uniform_ptr(const char *ptr)
{
    const uint64_t u = reinterpret_cast<uint64_t>(ptr);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return reinterpret_cast<const char *>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ float *uniform_fptr(float *ptr)
{
    return const_cast<float *>(reinterpret_cast<const float *>(uniform_ptr(reinterpret_cast<const char *>(ptr))));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char *base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), (short)0, bytes, kBufferFlags);
}

// Pieces of shared segments travel between waves that may run on different
// XCDs (each with its own L2).  They are written and read with system-
// coherent accesses (sc0 sc1: written through to memory, read from memory),
// so no device-wide cache write-back or invalidate is needed; a writer waits
// for its stores to complete before it counts its arrival.
constexpr int kCoherent = 1 | 16;

__device__ __forceinline__ void store_coherent4(float *base, int bytes, int voff, float4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), tile_rsrc((const char *)base, bytes),
                                           voff, 0, kCoherent);
}

__device__ __forceinline__ void store_coherent2(float *base, int bytes, int voff, float2 v)
{
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), tile_rsrc((const char *)base, bytes),
                                          voff, 0, kCoherent);
}

__device__ __forceinline__ float4 load_coherent4(const float *base, int bytes, int voff)
{
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(tile_rsrc((const char *)base, bytes),
                                                                            voff, 0, kCoherent));
}

__device__ __forceinline__ float2 load_coherent2(const float *base, int bytes, int voff)
{
    return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(tile_rsrc((const char *)base, bytes),
                                                                           voff, 0, kCoherent));
}

__device__ __forceinline__ float load_coherent1(const float *base, int bytes, int voff)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(tile_rsrc((const char *)base, bytes),
                                                                          voff, 0, kCoherent));
}

__device__ __forceinline__ void store_coherent1(float *base, int bytes, int voff, float v)
{
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(u32, v), tile_rsrc((const char *)base, bytes), voff,
                                          0, kCoherent);
}

// ---- the partition kernel ---------------------------------------------------

template <int D, int PS, int G, int QT, int KVT>
struct Shape {
    static constexpr int PAGE = PS;                // tokens per page
    static constexpr int EB = KVT == I8 || KVT == FP8 ? 1 : 2;   // bytes per KV element
    static constexpr int ROW = D * EB;             // bytes per token row
    // a lane's chunk of a row: 8 elements (16 bytes of 16-bit KV, 8 of byte KV)
    static constexpr int CB = 8 * EB;              // bytes per lane chunk
    using Chunk = std::conditional_t<CB == 16, u32x4, u32x2>;
    static constexpr int R = ROW / CB;             // lanes per token row
    static constexpr int LEVELS = R == 16 ? 4 : R == 8 ? 3 : 2;
    static constexpr int TPI = 64 / R;             // tokens per load instruction
    static constexpr int EPL = CB / EB;            // elements per lane chunk
    static constexpr int TILE_BYTES = PS * ROW;    // one (page, KV head) tile
    static constexpr int PPT = kTileTokens / PS;   // pages per 64-token tile
    static constexpr int PSTRIDE = 64 * G + (64 / R) * 4;  // floats in the p buffer
    static_assert(R >= 4 && R <= 16, "row split");
    static_assert(PS % TPI == 0, "a load instruction must not straddle pages");
    static_assert(kTileTokens % PS == 0, "tiles hold whole pages");
};

// Where the bytes of chunk i of a 64-token tile come from, for this lane.
// base[] is the (page, KV head) tile of each page of the tile (page 0 stands
// in for a page that does not exist; nothing is read from it).  The lane's
// byte offset within a page is the same for every chunk; the chunk's own
// offset within the page is a compile-time scalar.  A lane whose token of
// chunk i is at or past the end of the tile (chunk index >= nvalid) gets an
// out-of-range offset and reads zero without touching memory, so loads are
// issued unconditionally, also for a tile that is not there (nvalid = 0).
template <class S>
struct TileAddr {
    const char *base[S::PPT];
    int nvalid;   // chunks of this tile that hold a token for this lane's row

    __device__ __forceinline__ void set(const char *head, size_t page_stride, const int (&ph)[S::PPT],
                                        int rem, int r)
    {
#pragma unroll
        for (int pg = 0; pg < S::PPT; ++pg)
            base[pg] = uniform_ptr(head + (size_t)(ph[pg] >= 0 ? ph[pg] : 0) * page_stride);
        // token i*TPI + r exists iff i*TPI + r < rem
        nvalid = rem > r ? (rem - r + S::TPI - 1) / S::TPI : 0;
    }

    template <int I>
    __device__ __forceinline__ typename S::Chunk load(int lane_off) const
    {
        constexpr int pg = (I * S::TPI) / S::PAGE;
        constexpr int chunk_off = ((I * S::TPI) % S::PAGE) * S::ROW;
        const int voff = I < nvalid ? lane_off : kOutOfRange;
        if constexpr (S::CB == 16)
            return __builtin_amdgcn_raw_buffer_load_b128(tile_rsrc(base[pg], S::TILE_BYTES), voff, chunk_off,
                                                         kStreamingLoad);
        else
            return __builtin_amdgcn_raw_buffer_load_b64(tile_rsrc(base[pg], S::TILE_BYTES), voff, chunk_off,
                                                        kStreamingLoad);
    }
};

// ---- batch geometry ---------------------------------------------------------
//
// The work of a decode step is the flat list of 64-token tiles of every
// (sequence b, KV head g) "segment", in the order b, then g, then tile index
// k.  Sequence b contributes tiles_b = ceil(n_b / 64) tiles to each of its Hkv
// segments (0 for an empty or invalid sequence), so segment s = b*Hkv + g
// starts at global tile Hkv * sum_{b'<b} tiles_b' + g * tiles_b.  Wave w of a
// grid of NW waves streams the global tiles [w*T/NW, (w+1)*T/NW) where T is
// the total (waves beyond T idle, so no range is empty); a segment it covers
// completely is finished by that wave, the pieces of a segment shared by
// several waves are merged by the second kernel.  Piece (s, w) is stored at
// index s + w, which is unique.

__device__ __forceinline__ int tiles_of(int n, int max_len)
{
    return n >= 0 && n <= max_len ? (n + kTileTokens - 1) / kTileTokens : 0;
}

// Integer sum and inclusive prefix sum over the 64 lanes, by DPP within each
// 16-lane row and wave-uniform reads of the row totals (no LDS round trips:
// both sit on the dependent chain before a wave's first load).
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x)
{
    return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ int wave_sum_int(int x)
{
    x += dpp_i<0x128>(x);   // row_ror 8
    x += dpp_i<0x124>(x);   // row_ror 4
    x += dpp_i<0x122>(x);   // row_ror 2
    x += dpp_i<0x121>(x);   // row_ror 1: every lane holds its row's total
    return __builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16) + __builtin_amdgcn_readlane(x, 32) +
           __builtin_amdgcn_readlane(x, 48);
}

__device__ __forceinline__ int wave_incl_scan(int x, int lane)
{
    // row_shr n: lane j reads lane j - n of its row, 0 for j < n
    x += dpp_i<0x111>(x);
    x += dpp_i<0x112>(x);
    x += dpp_i<0x114>(x);
    x += dpp_i<0x118>(x);   // scan within the row
    const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
              r2 = __builtin_amdgcn_readlane(x, 47);
    const int row = lane / 16;
    return x + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// Context lengths of the first kLensRegs * 64 sequences, held in registers
// (lane l of register i: sequence 64 i + l; 0 past the batch), all loaded
// at once at the start of a wave: the wave's location in the batch, its
// first tile and every later segment change then need no further load of
// context_lens (one round trip to memory instead of a dependent chain of
// them, also spared by every wave at once on the same two cache lines).
// Sequences beyond them are read from memory.
constexpr int kLensRegs = 4;

struct Lens {
    // four named registers (not an array: an array captured by the kernels'
    // lambdas can be left in scratch memory instead of registers)
    int v0, v1, v2, v3;

    __device__ __forceinline__ void load(const DecodeParams &p, int lane)
    {
        auto at = [&](int b) { return b < p.batch ? p.context_lens[b] : 0; };
        v0 = at(lane);
        v1 = at(64 + lane);
        v2 = at(128 + lane);
        v3 = at(192 + lane);
    }

    // this lane's register of chunk i (i < kLensRegs, wave-uniform)
    __device__ __forceinline__ int reg(int i) const { return i == 0 ? v0 : i == 1 ? v1 : i == 2 ? v2 : v3; }

    // context length of sequence b (wave-uniform b, 0 <= b < batch)
    __device__ __forceinline__ int of(const DecodeParams &p, int b) const
    {
        if (b >= 64 * kLensRegs)
            return p.context_lens[b];
        return __builtin_amdgcn_readlane(reg(b / 64), b & 63);
    }

    // context lengths of sequences c .. c+63 (c a multiple of 64), lane l
    // holding sequence c + l (0 past the batch)
    __device__ __forceinline__ int chunk(const DecodeParams &p, int c, int lane) const
    {
        if (c >= 64 * kLensRegs) {
            const int b = c + lane;
            return b < p.batch ? p.context_lens[b] : 0;
        }
        return reg(c / 64);
    }
};

// Tiles of one KV head over the whole batch.
__device__ __forceinline__ int batch_tiles(const DecodeParams &p, const Lens &lens, int lane)
{
    int total = 0;
    for (int c = 0; c < p.batch; c += 64) {
        const int b = c + lane;
        total += wave_sum_int(b < p.batch ? tiles_of(lens.chunk(p, c, lane), p.max_context_len) : 0);
    }
    return total;
}

// Shares of the tile list.  With two waves on a SIMD, the one dispatched
// first (wave w < H, H the waves that are first on their SIMD) wins the
// issue arbitration and streams faster -- a third faster, measured with
// per-wave timestamps on the fp8 kernel -- so those waves take WA shares of
// the list and the others WB; with one wave per SIMD (H = NW) every wave
// takes the same share.  Every share is non-empty when T >= 2 NW and
// WA <= 2 WB (the kernels use H = NW otherwise).

// a / b for wave-uniform non-negative operands: a 32-bit division when both
// fit (always, in practice), else the 64-bit one.
__device__ __forceinline__ long long div_nonneg(long long a, long long b)
{
    if (((unsigned long long)a | (unsigned long long)b) >> 32 == 0)
        return (long long)((unsigned)a / (unsigned)b);
    return a / b;
}

// First global tile of wave w's range.
template <int WA, int WB>
__device__ __forceinline__ long long range_start(long long w, long long T, long long NW, long long H)
{
    static_assert(WB <= WA && WA <= 2 * WB, "share weights");
    const long long ws = w < H ? WA * w : WA * H + WB * (w - H);
    return div_nonneg(ws * T, WA * H + WB * (NW - H));
}

// The wave that owns global tile t (largest w with range_start(w) <= t).
template <int WA, int WB>
__device__ __forceinline__ long long owner_of(long long t, long long T, long long NW, long long H)
{
    const long long x = div_nonneg((t + 1) * (WA * H + WB * (NW - H)) - 1, T);   // largest share start <= t
    return x < WA * H ? x / WA : min(NW - 1, H + (x - WA * H) / WB);
}

// Sequence containing global tile t (t < total) and the first global tile of
// that sequence: walks the batch 64 sequences at a time.
__device__ __forceinline__ void locate(const DecodeParams &p, const Lens &lens, long long t, int lane, int &b_out,
                                       long long &start_out)
{
    int carry = 0;
    const int Hkv = p.num_kv_heads;
    for (int c = 0; c < p.batch; c += 64) {
        const int b = c + lane;
        const int nt = b < p.batch ? tiles_of(lens.chunk(p, c, lane), p.max_context_len) : 0;
        const int incl = wave_incl_scan(nt, lane);
        const bool past = b < p.batch && (long long)(carry + incl) * Hkv > t;
        const unsigned long long mask = __ballot(past);
        if (mask) {
            const int first = __builtin_ctzll(mask);
            b_out = c + first;
            start_out = (long long)(carry + __builtin_amdgcn_readlane(incl - nt, first)) * Hkv;
            return;
        }
        carry += __builtin_amdgcn_readlane(incl, 63);
    }
    b_out = p.batch;
    start_out = 0;
}

// ---- merging the pieces of a shared segment, inside the decode kernel -------
//
// The n waves w0 .. w0+n-1 that share a segment each leave a piece
// (m, l, o) -- running max in log2 units, sum of exponentials, unnormalised
// output -- in piece slot (segment + wave).  They are merged up a tree of
// fan-in 8 without any wave waiting for another: at level L the pieces form
// blocks of 8 children, a per-block counter counts arrivals, and the wave
// whose arrival completes a block merges its children (in slot order, so
// the result does not depend on which wave arrived last) into the block's
// first slot, then arrives at the next level.  The merge of the top block
// writes the normalised output.  Counters wrap to zero on the arrival that
// completes them (atomic increment modulo the child count), so a zeroed
// workspace is zero again after every call.
//
// Ordering: pieces are written and read with system-coherent accesses, a
// wave's stores have completed before its arrival is counted (a system-scope
// atomic), and the merging wave reads only after its own count returned.

template <int D, int G, int QT>
__device__ __forceinline__ void settle_piece(const DecodeParams &p, int seg, int w0, int n, int w, int lane,
                                             bool arrived0 = false)
{
    // arrived0: the piece's arrival at level 0 has been counted already (by
    // settle_pending, for all of a wave's pieces at once) and completed its
    // block
    constexpr int LPH = 64 / G;     // lanes per query head
    constexpr int DPL = D / LPH;    // output dims per lane
    constexpr int FAN = 8;
    const int h = lane / LPH, d0 = (lane % LPH) * DPL;
    const size_t slot0 = (size_t)seg + (size_t)w0;
    const size_t level_stride = (size_t)p.batch * p.num_kv_heads + (size_t)p.num_splits;
    int k = w - w0;
    int span = 1;
    for (int level = 0; span < n; ++level, span *= FAN) {
        const int parent = k - k % (span * FAN);
        const int children = min(FAN, (n - parent + span - 1) / span);
        if (children > 1) {
            if (!(arrived0 && level == 0)) {
                // this wave's stores (the piece, or the block it merged)
                // complete before its arrival is counted
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_s_waitcnt(0);
                uint32_t old = 0;
                if (lane == 0)
                    old = __builtin_amdgcn_atomic_inc32(p.counters + level * level_stride + slot0 + parent,
                                                        (uint32_t)(children - 1), __ATOMIC_RELAXED, "");
                old = __builtin_amdgcn_readfirstlane(old);
                if (old != (uint32_t)(children - 1))
                    return;               // a later arrival completes this block
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

            float mc[FAN], lc[FAN], oc[FAN][DPL];
#pragma unroll
            for (int c = 0; c < FAN; ++c) {
                const size_t slot = slot0 + parent + (size_t)(c < children ? c : 0) * span;
                const float2 ml = load_coherent2(uniform_fptr(p.part_ml + slot * G * 2), G * 8, h * 8);
                mc[c] = c < children ? ml.x : -INFINITY;
                lc[c] = ml.y;
                const float *src = uniform_fptr(p.part_o + slot * G * D);
                if constexpr (DPL % 4 == 0) {
#pragma unroll
                    for (int v = 0; v < DPL / 4; ++v) {
                        const float4 x = load_coherent4(src, G * D * 4, (h * D + d0 + 4 * v) * 4);
                        oc[c][4 * v] = x.x;
                        oc[c][4 * v + 1] = x.y;
                        oc[c][4 * v + 2] = x.z;
                        oc[c][4 * v + 3] = x.w;
                    }
                } else if constexpr (DPL == 2) {
                    const float2 x = load_coherent2(src, G * D * 4, (h * D + d0) * 4);
                    oc[c][0] = x.x;
                    oc[c][1] = x.y;
                } else {
                    oc[c][0] = load_coherent1(src, G * D * 4, (h * D + d0) * 4);
                }
            }
            float M = mc[0];
#pragma unroll
            for (int c = 1; c < FAN; ++c)
                M = fmaxf(M, mc[c]);
            float L = 0.0f, acc[DPL];
#pragma unroll
            for (int x = 0; x < DPL; ++x)
                acc[x] = 0.0f;
#pragma unroll
            for (int c = 0; c < FAN; ++c) {
                if (c < children) {
                    const float f = __builtin_amdgcn_exp2f(mc[c] - M);
                    L = fmaf(f, lc[c], L);
#pragma unroll
                    for (int x = 0; x < DPL; ++x)
                        acc[x] = fmaf(f, oc[c][x], acc[x]);
                }
            }
            if (span * FAN >= n) {
                // top of the tree: the normalised output of query head g*G + h
                const int b = seg / p.num_kv_heads, g = seg % p.num_kv_heads;
                const size_t unit = (size_t)b * p.num_q_heads + (size_t)g * G + h;
                const float inv = 1.0f / L;
                u32 *dst = reinterpret_cast<u32 *>(p.out) + (unit * D + d0) / 2;
                if constexpr (DPL >= 2) {
#pragma unroll
                    for (int x = 0; x < DPL / 2; ++x)
                        dst[x] = pack_out<QT>(acc[2 * x] * inv, acc[2 * x + 1] * inv);
                } else {
                    const float other = __shfl_xor(acc[0], 1);
                    if ((lane & 1) == 0)
                        dst[0] = pack_out<QT>(acc[0] * inv, other * inv);
                }
                return;
            }
            // the block's result replaces its first child
            const size_t slot = slot0 + parent;
            float *dst = uniform_fptr(p.part_o + slot * G * D);
            if constexpr (DPL % 4 == 0) {
#pragma unroll
                for (int v = 0; v < DPL / 4; ++v)
                    store_coherent4(dst, G * D * 4, (h * D + d0 + 4 * v) * 4,
                                    make_float4(acc[4 * v], acc[4 * v + 1], acc[4 * v + 2], acc[4 * v + 3]));
            } else if constexpr (DPL == 2) {
                store_coherent2(dst, G * D * 4, (h * D + d0) * 4, make_float2(acc[0], acc[1]));
            } else {
                store_coherent1(dst, G * D * 4, (h * D + d0) * 4, acc[0]);
            }
            if (lane % LPH == 0)
                store_coherent2(uniform_fptr(p.part_ml + slot * G * 2), G * 8, h * 8, make_float2(M, L));
        }
        k = parent;
    }
}

// ---- the first piece of a wave's range ----------------------------------------
//
// A wave's range can start inside a segment that began in an earlier wave's
// range; that segment ends inside the range, and its piece is the only one a
// wave finishes before the end of its range.  Pieces are written with
// system-coherent stores, which complete only once they have reached memory,
// and vector memory operations complete in issue order: a coherent store in
// the middle of the stream would hold up every later wait for the next
// tiles' loads.  So the first piece is kept in LDS and written after the
// wave's last tile, where the merge waits for the stores anyway.

template <int D, int G>
__device__ __forceinline__ void flush_first_piece(const DecodeParams &p, int slot, const float *so,
                                                  const float2 *sml, int lane)
{
    float *po = uniform_fptr(p.part_o + (size_t)slot * G * D);
    for (int i = lane; i < G * D / 4; i += 64)
        store_coherent4(po, G * D * 4, i * 16, reinterpret_cast<const float4 *>(so)[i]);
    if (lane < G)
        store_coherent2(uniform_fptr(p.part_ml + (size_t)slot * G * 2), G * 8, lane * 8, sml[lane]);
}

// A wave's pieces waiting for the merge (at most two: the segments its range
// starts and ends inside), once their stores have been issued: the level-0
// arrivals of all of them at once (lane i for piece i), so that their round
// trips overlap, then, one piece at a time, the merge of each block an
// arrival completed and the climb above it.
template <int D, int G, int QT>
__device__ __forceinline__ void settle_pending(const DecodeParams &p, const int (*pend)[3], int npend, int w,
                                               int lane)
{
    constexpr int FAN = 8;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_waitcnt(0);   // the pieces' stores have completed
    int mode = 0;                    // 1: arrived and completed its block, 2: arrived, 3: no level-0 arrival
    if (lane < npend) {
        const int seg = pend[lane][0], w0 = pend[lane][1], n = pend[lane][2];
        const int k = w - w0, parent = k - k % FAN, children = min(FAN, n - parent);
        if (children > 1) {
            const size_t slot0 = (size_t)seg + (size_t)w0;
            const uint32_t old =
                __builtin_amdgcn_atomic_inc32(p.counters + slot0 + parent, (uint32_t)(children - 1), __ATOMIC_RELAXED, "");
            mode = old == (uint32_t)(children - 1) ? 1 : 2;
        } else {
            mode = 3;
        }
    }
    for (int i = 0; i < npend; ++i) {
        const int m = __builtin_amdgcn_readlane(mode, i);
        if (m != 2)
            settle_piece<D, G, QT>(p, __builtin_amdgcn_readfirstlane(pend[i][0]),
                                   __builtin_amdgcn_readfirstlane(pend[i][1]),
                                   __builtin_amdgcn_readfirstlane(pend[i][2]), w, lane, m == 1);
    }
}

// ---- the partition kernel ---------------------------------------------------

template <int D, int PS, int G, int QT, int KVT>
__global__ __launch_bounds__(kWavesPerGroup * 64) void paged_decode_kernel(DecodeParams p)
{
    using S = Shape<D, PS, G, QT, KVT>;
    constexpr int R = S::R, TPI = S::TPI, EPL = S::EPL, PPT = S::PPT, LEVELS = S::LEVELS;
    // byte KV (int8 or fp8): one fp32 scale per token, q kept as fp32
    constexpr bool kByte = KVT == I8 || KVT == FP8;
    constexpr bool kI8 = KVT == I8;
    constexpr int QW = EPL / 2;         // dwords of q per head per lane
    using Chunk = typename S::Chunk;
    constexpr int CW = S::CB / 4;       // dwords per chunk

    // per-wave LDS: this wave's slot of the workgroup's arrays
    const int slot = threadIdx.x / 64;
    __shared__ float s_p_all[kWavesPerGroup][S::PSTRIDE];
    float *const s_p = s_p_all[slot];

    const int lane = threadIdx.x % 64;
    const int r = lane / R, j = lane % R;
    const int Hq = p.num_q_heads, Hkv = p.num_kv_heads;
    const long long NW = p.num_splits, w = (long long)blockIdx.x * kWavesPerGroup + slot;
    if (w >= NW)
        return;

    Lens lens;
    lens.load(p, lane);
    const long long T = (long long)batch_tiles(p, lens, lane) * Hkv;
    // a sequence without tiles (empty, or an invalid length) has no wave
    // streaming it: its outputs are written here, zeros (NaN if invalid)
    for (long long b = w; b < p.batch; b += NW) {
        const int n = lens.of(p, (int)b);
        if (tiles_of(n, p.max_context_len) == 0) {
            const float fill = (n < 0 || n > p.max_context_len) ? __builtin_nanf("") : 0.0f;
            u32 *o = reinterpret_cast<u32 *>(p.out) + (size_t)b * Hq * D / 2;
            for (int i = lane; i < Hq * D / 2; i += 64)
                o[i] = pack_out<QT>(fill, fill);
        }
    }
    // waves beyond the tile count idle, so every working wave's range is non-empty
    const long long NWe = NW < T ? NW : T;
    if (w >= NWe)
        return;
    const long long H = p.first_round < NWe && T >= 2 * NWe ? p.first_round : NWe;
    const long long lo = range_start<kShareA, kShareB>(w, T, NWe, H);
    const long long hi = range_start<kShareA, kShareB>(w + 1, T, NWe, H);
    if (w == 0 && lane == 0)
        *p.ws_tag = p.tag;               // the merge kernel reads which call it follows

    // ---- the tile cursor: sequence b (length n, tiles nt), KV head g, tile k
    struct Cursor {
        int b, n, nt, g, k;
        // the cursor is the same on every lane; keep it in scalar registers
        __device__ __forceinline__ void make_uniform()
        {
            b = __builtin_amdgcn_readfirstlane(b);
            n = __builtin_amdgcn_readfirstlane(n);
            nt = __builtin_amdgcn_readfirstlane(nt);
            g = __builtin_amdgcn_readfirstlane(g);
            k = __builtin_amdgcn_readfirstlane(k);
        }
    };
    Cursor cur;
    {
        long long start;
        locate(p, lens, lo, lane, cur.b, start);
        cur.n = lens.of(p, cur.b);
        cur.nt = tiles_of(cur.n, p.max_context_len);
        const long long off = lo - start;
        cur.g = (int)div_nonneg(off, cur.nt);
        cur.k = (int)(off - (long long)cur.g * cur.nt);
        cur.make_uniform();
    }
    auto advance = [&](const Cursor &c) {
        Cursor x = c;
        if (++x.k == x.nt) {
            x.k = 0;
            if (++x.g == Hkv) {
                x.g = 0;
                // next sequence with at least one tile (one exists: this wave
                // only advances while tiles of its range remain)
                do {
                    ++x.b;
                    x.n = x.b < p.batch ? lens.of(p, x.b) : 0;
                    x.nt = tiles_of(x.n, p.max_context_len);
                } while (x.nt == 0 && x.b < p.batch);
            }
        }
        x.make_uniform();
        return x;
    };

    bool any_bad = false;
    const size_t page_stride = (size_t)Hkv * S::TILE_BYTES;
    // Physical pages of the cursor's tile (-1: none / outside the pool); the
    // table is read at a clamped index so the lookup needs no branch.  True
    // if a page the tile needs lies outside the pool (its segment's output
    // becomes NaN once the tile is the current one).
    auto pages_of = [&](const Cursor &c, int (&ph)[PPT]) {
        const int32_t *bt = p.block_tables + (size_t)min(c.b, p.batch - 1) * p.max_blocks;
        bool bad = false;
#pragma unroll
        for (int pg = 0; pg < PPT; ++pg) {
            const int v = bt[min(c.k * PPT + pg, p.max_blocks - 1)];
            const bool exists = c.k * kTileTokens + pg * PS < c.n;
            const bool inside = (unsigned)v < (unsigned)p.num_pages;
            bad = bad || (exists && !inside);
            ph[pg] = exists && inside ? v : -1;
        }
        return bad;
    };
    auto tile_rem = [&](const Cursor &c) { return min(kTileTokens, c.n - c.k * kTileTokens); };
    auto own_page = [&](const int (&ph)[PPT]) {
        int my_phys = -1;
#pragma unroll
        for (int pg = 0; pg < PPT; ++pg)
            if (pg == (TPI * j) / PS)
                my_phys = ph[pg];
        return my_phys;
    };
    // K and V scales of this lane's own token of the cursor's tile (byte KV).
    auto own_scales = [&](const Cursor &c, const int (&ph)[PPT], float &ks, float &vs) {
        ks = 1.0f;
        vs = 1.0f;
        if constexpr (kByte) {
            const int my_phys = own_page(ph);
            const bool ok = my_phys >= 0 && c.k * kTileTokens + TPI * j + r < c.n;
            const size_t si = ok ? ((size_t)my_phys * Hkv + c.g) * PS + (TPI * j) % PS + r : 0;
            const float a = p.k_scale[si], b = p.v_scale[si];
            ks = ok ? a : 0.0f;
            vs = ok ? b : 0.0f;
        }
    };
    // Raw q dwords of this lane's slice of the G query heads of segment (b, g).
    auto load_q = [&](const Cursor &c, u32 (&raw)[G][QW]) {
        const char *base = (const char *)p.q + (((size_t)c.b * Hq + (size_t)c.g * G) * D) * 2;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const u32x4 *src = reinterpret_cast<const u32x4 *>(base + ((size_t)h * D + EPL * j) * 2);
#pragma unroll
            for (int v = 0; v < QW / 4; ++v) {
                const u32x4 x = src[v];
                raw[h][4 * v] = x.x;
                raw[h][4 * v + 1] = x.y;
                raw[h][4 * v + 2] = x.z;
                raw[h][4 * v + 3] = x.w;
            }
        }
    };

    // q in the form the dot products use: packed pairs (16-bit and fp8 KV,
    // fp8 codes being widened to q's type) or fp32 values (int8 KV, with the
    // -128 * sum(q) bias of the unsigned-byte trick).
    u32 qw[G][QW];
    float qf[kI8 ? G : 1][kI8 ? EPL : 1];
    float qbias[G];
    auto set_q = [&](const u32 (&raw)[G][QW]) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            if constexpr (!kI8) {
#pragma unroll
                for (int v = 0; v < QW; ++v)
                    qw[h][v] = raw[h][v];
                qbias[h] = 0.0f;
            } else {
                float s = 0.0f;
#pragma unroll
                for (int e = 0; e < QW; ++e) {
                    qf[h][2 * e] = q_lo<QT>(raw[h][e]);
                    qf[h][2 * e + 1] = q_hi<QT>(raw[h][e]);
                    s += qf[h][2 * e] + qf[h][2 * e + 1];
                }
                qbias[h] = kI8 ? -128.0f * s : 0.0f;
            }
        }
    };

    float m_run[G], l_run[G], acc[G][EPL], psum[G];
    auto reset_state = [&]() {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            m_run[h] = -INFINITY;
            l_run[h] = 0.0f;
            psum[h] = 0.0f;
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                acc[h][e] = 0.0f;
        }
    };

    // ---- prologue.  One register ring of R chunks carries, in turn, K of
    // tile t, V of tile t, K of tile t+1, ...: each chunk's V load is issued
    // as soon as its K has been used, and the next tile's K as soon as its V
    // has been used -- across segment boundaries too.
    const int lane_off = r * S::ROW + S::CB * j;
    int ph_cur[PPT], ph_nxt[PPT];
    bool bad_cur = pages_of(cur, ph_cur), bad_nxt = false;
    TileAddr<S> ka, va;
    ka.set((const char *)p.k_pool + (size_t)cur.g * S::TILE_BYTES, page_stride, ph_cur, tile_rem(cur), r);
    va.set((const char *)p.v_pool + (size_t)cur.g * S::TILE_BYTES, page_stride, ph_cur, tile_rem(cur), r);
    Chunk ring[R];
    [&]<int... I>(std::integer_sequence<int, I...>) { ((ring[I] = ka.template load<I>(lane_off)), ...); }
        (std::make_integer_sequence<int, R>{});
    // int8 KV: the next segment's raw q is fetched a tile ahead (its fp32
    // form takes longer to set up)
    u32 qraw[kByte ? G : 1][QW];
    {
        u32 q0[G][QW];
        load_q(cur, q0);
        set_q(q0);
    }
    reset_state();
    float ks_cur, vs_cur, ks_nxt = 1.0f, vs_nxt = 1.0f;
    own_scales(cur, ph_cur, ks_cur, vs_cur);
    bool piece_from_start = cur.k == 0;
    // Pieces of shared segments this wave wrote (at most two: the segment its
    // range starts in and the one it ends in) are settled after the loop; the
    // records (segment, first wave, wave count) wait in LDS, not registers.
    __shared__ int s_pend_all[kWavesPerGroup][2][3];
    __shared__ int s_npend_all[kWavesPerGroup];
    // the range's first piece, written after the last tile
    __shared__ __align__(16) float s_first_all[kWavesPerGroup][G * D];
    __shared__ float2 s_first_ml_all[kWavesPerGroup][G];
    int (*const s_pend)[3] = s_pend_all[slot];
    int &s_npend = s_npend_all[slot];
    float *const s_first = s_first_all[slot];
    float2 *const s_first_ml = s_first_ml_all[slot];
    int first_slot = -1;
    if (lane == 0)
        s_npend = 0;

    for (long long t = lo; t < hi; ++t) {
        // the wave holding a segment's first tile records which waves share
        // it (read by the merge kernel of the two-launch form only)
        if (!p.fused && cur.k == 0 && lane == 0)
            p.seg_geo[cur.b * Hkv + cur.g] =
                make_int4((int)p.tag, (int)w, (int)owner_of<kShareA, kShareB>(t + cur.nt - 1, T, NWe, H), 0);
        const bool last_in_range = t + 1 == hi;
        const Cursor nxt = last_in_range ? cur : advance(cur);
        const bool seg_end = last_in_range || nxt.k == 0;
        any_bad = any_bad || bad_cur;
        bad_nxt = false;
        if (!last_in_range)
            bad_nxt = pages_of(nxt, ph_nxt);
        else
#pragma unroll
            for (int pg = 0; pg < PPT; ++pg)
                ph_nxt[pg] = -1;
        if constexpr (kByte) {
            if (seg_end && !last_in_range)
                load_q(nxt, qraw);
        }

        // ---- q.k: partial dots of chunk i, folded into the reduce-scatter
        // tree as they come; chunk i's registers then take V of this tile
        float stack[LEVELS + 1][G];
        [&]<int... I>(std::integer_sequence<int, I...>) {
            (([&] {
                 float v[G];
                 const Chunk kc = ring[I];
                 u32 kw[CW];
#pragma unroll
                 for (int c = 0; c < CW; ++c)
                     kw[c] = kc[c];
                 u32 k16[KVT == FP8 ? QW : 1];
                 if constexpr (KVT == FP8) {
#pragma unroll
                     for (int c = 0; c < CW; ++c) {
                         k16[2 * c] = fp8_pair16<QT, false>(kw[c]);
                         k16[2 * c + 1] = fp8_pair16<QT, true>(kw[c]);
                     }
                 }
#pragma unroll
                 for (int h = 0; h < G; ++h) {
                     float a;
                     if constexpr (!kByte) {
                         a = 0.0f;
#pragma unroll
                         for (int c = 0; c < CW; ++c)
                             a = dot2<KVT>(kw[c], qw[h][c], a);
                     } else if constexpr (KVT == FP8) {
                         // widened E4M3 pairs against q's packed pairs
                         a = 0.0f;
#pragma unroll
                         for (int v2 = 0; v2 < QW; ++v2)
                             a = dot2<QT>(k16[v2], qw[h][v2], a);
                     } else {
                         // code + 128 as unsigned bytes; the -128 * sum(q) bias restores the sign
                         a = qbias[h];
#pragma unroll
                         for (int q4 = 0; q4 < CW; ++q4) {
                             const u32 wd = kw[q4] ^ 0x80808080u;
                             a = fmaf(qf[h][4 * q4 + 0], ubyte<0>(wd), a);
                             a = fmaf(qf[h][4 * q4 + 1], ubyte<1>(wd), a);
                             a = fmaf(qf[h][4 * q4 + 2], ubyte<2>(wd), a);
                             a = fmaf(qf[h][4 * q4 + 3], ubyte<3>(wd), a);
                         }
                     }
                     v[h] = a;
                 }
                 ring[I] = va.template load<I>(lane_off);
                 tree_push<I, 0, LEVELS, G>(stack, v, j);
             }()), ...);
        }(std::make_integer_sequence<int, R>{});

        // ---- online softmax (log2 domain); this lane's token is TPI*j + r
        const int t0 = cur.k * kTileTokens;
        const int my_phys = own_page(ph_cur);
        const bool my_valid = my_phys >= 0 && t0 + TPI * j + r < cur.n;
        own_scales(nxt, ph_nxt, ks_nxt, vs_nxt);
        float pe[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float s = my_valid ? stack[LEVELS][h] * ks_cur * p.scale_log2 : -INFINITY;
            const float m_new = fmaxf(m_run[h], wave_max(s));
            const float alpha = __builtin_amdgcn_exp2f(m_run[h] - m_new);
            const float e = __builtin_amdgcn_exp2f(s - m_new);
            l_run[h] = l_run[h] * alpha + e;
            m_run[h] = m_new;
            psum[h] *= alpha;
#pragma unroll
            for (int x = 0; x < EPL; ++x)
                acc[h][x] *= alpha;
            pe[h] = e * vs_cur;
        }

        // ---- hand each probability to the lanes holding that token's V bytes
        float *mine = s_p + lane * G + r * 4;
#pragma unroll
        for (int h = 0; h < G; ++h)
            mine[h] = pe[h];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // the next tile's K goes into each chunk's registers once its V is used
        ka.set((const char *)p.k_pool + (size_t)nxt.g * S::TILE_BYTES, page_stride, ph_nxt,
               last_in_range ? 0 : tile_rem(nxt), r);

        // ---- p.V
        [&]<int... I>(std::integer_sequence<int, I...>) {
            (([&] {
                 const float *src = s_p + (r * R + I) * G + r * 4;
                 float pv[G];
#pragma unroll
                 for (int h = 0; h < G; ++h)
                     pv[h] = src[h];
                 const Chunk vc = ring[I];
                 ring[I] = ka.template load<I>(lane_off);
                 float vf[EPL];
                 u32 wv[CW];
#pragma unroll
                 for (int c = 0; c < CW; ++c)
                     wv[c] = vc[c];
                 if constexpr (KVT == FP8) {
#pragma unroll
                     for (int q4 = 0; q4 < CW; ++q4) {
                         const float2 lo = fp8_pair<false>(wv[q4]), hi = fp8_pair<true>(wv[q4]);
                         vf[4 * q4 + 0] = lo.x;
                         vf[4 * q4 + 1] = lo.y;
                         vf[4 * q4 + 2] = hi.x;
                         vf[4 * q4 + 3] = hi.y;
                     }
                 } else if constexpr (kI8) {
#pragma unroll
                     for (int q4 = 0; q4 < CW; ++q4) {
                         const u32 u = wv[q4] ^ 0x80808080u;
                         vf[4 * q4 + 0] = ubyte<0>(u);
                         vf[4 * q4 + 1] = ubyte<1>(u);
                         vf[4 * q4 + 2] = ubyte<2>(u);
                         vf[4 * q4 + 3] = ubyte<3>(u);
                     }
                 } else {
#pragma unroll
                     for (int q2 = 0; q2 < 4; ++q2) {
                         vf[2 * q2] = KVT == BF16 ? bf16_lo(wv[q2]) : f16_lo(wv[q2]);
                         vf[2 * q2 + 1] = KVT == BF16 ? bf16_hi(wv[q2]) : f16_hi(wv[q2]);
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
             }()), ...);
        }(std::make_integer_sequence<int, R>{});
        __builtin_amdgcn_wave_barrier();
        va.set((const char *)p.v_pool + (size_t)nxt.g * S::TILE_BYTES, page_stride, ph_nxt,
               last_in_range ? 0 : tile_rem(nxt), r);

        // ---- end of a piece: this wave's share of segment (cur.b, cur.g)
        if (seg_end) {
            const bool whole = piece_from_start && cur.k == cur.nt - 1;
            const int seg = cur.b * Hkv + cur.g;
            const float nan = __builtin_nanf("");
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
                if (r == 0) {
                    if (whole) {
                        const size_t unit = (size_t)cur.b * Hq + (size_t)cur.g * G + h;
                        const float inv = any_bad ? nan : 1.0f / lt;
                        u32 packed[EPL / 2];
#pragma unroll
                        for (int x = 0; x < EPL / 2; ++x)
                            packed[x] = pack_out<QT>(acc[h][2 * x] * inv, acc[h][2 * x + 1] * inv);
                        u32x4 *o = reinterpret_cast<u32x4 *>(reinterpret_cast<u32 *>(p.out) + (unit * D + EPL * j) / 2);
#pragma unroll
                        for (int v = 0; v < EPL / 8; ++v)
                            o[v] = u32x4{packed[4 * v], packed[4 * v + 1], packed[4 * v + 2], packed[4 * v + 3]};
                    } else if (!piece_from_start && !last_in_range) {
                        // the range's first piece: to LDS, written after the last tile
#pragma unroll
                        for (int v = 0; v < EPL / 4; ++v)
                            *reinterpret_cast<float4 *>(s_first + h * D + EPL * j + 4 * v) =
                                any_bad ? make_float4(nan, nan, nan, nan)
                                        : make_float4(acc[h][4 * v], acc[h][4 * v + 1], acc[h][4 * v + 2],
                                                      acc[h][4 * v + 3]);
                        if (j == 0)
                            s_first_ml[h] = make_float2(m_run[h], any_bad ? nan : lt);
                    } else {
                        // piece group of slot (seg + w): G heads x D values, G (m, l) pairs
                        const size_t slot = (size_t)seg + (size_t)w;
                        float *po = uniform_fptr(p.part_o + slot * G * D);
#pragma unroll
                        for (int v = 0; v < EPL / 4; ++v)
                            store_coherent4(po, G * D * 4, (h * D + EPL * j + 4 * v) * 4,
                                            any_bad ? make_float4(nan, nan, nan, nan)
                                                    : make_float4(acc[h][4 * v], acc[h][4 * v + 1],
                                                                  acc[h][4 * v + 2], acc[h][4 * v + 3]));
                        if (j == 0)
                            store_coherent2(uniform_fptr(p.part_ml + slot * G * 2), G * 8, h * 8,
                                            make_float2(m_run[h], any_bad ? nan : lt));
                    }
                }
            }
            if (!whole && !piece_from_start && !last_in_range)
                first_slot = seg + (int)w;
            if (!whole) {
                const long long first = t - cur.k;   // the segment's first global tile
                const int w0 = (int)owner_of<kShareA, kShareB>(first, T, NWe, H);
                const int w1 = (int)owner_of<kShareA, kShareB>(first + cur.nt - 1, T, NWe, H);
                if (lane == 0) {
                    const int i = s_npend;
                    s_pend[i][0] = seg;
                    s_pend[i][1] = w0;
                    s_pend[i][2] = w1 - w0 + 1;
                    s_npend = i + 1;
                }
            }
            reset_state();
            any_bad = false;
            piece_from_start = true;
            if (!last_in_range) {
                if constexpr (kByte) {
                    set_q(qraw);   // loaded a tile ahead
                } else {
                    // the next segment's q: loaded now, behind the next
                    // tile's K loads already in flight, so it arrives with them
                    u32 qn[G][QW];
                    load_q(nxt, qn);
                    set_q(qn);
                }
            }
        }

        // ---- roll the window forward
#pragma unroll
        for (int pg = 0; pg < PPT; ++pg)
            ph_cur[pg] = ph_nxt[pg];
        ks_cur = ks_nxt;
        vs_cur = vs_nxt;
        bad_cur = bad_nxt;
        cur = nxt;
    }

    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (first_slot >= 0)
        flush_first_piece<D, G>(p, first_slot, s_first, s_first_ml, lane);
    if (p.fused)
        settle_pending<D, G, QT>(p, s_pend, __builtin_amdgcn_readfirstlane(s_npend), (int)w, lane);
}

// ---- fp8 KV on the matrix cores (head_dim 128) ---------------------------------
//
// The same walk over the batch's tiles as paged_decode_kernel, for E4M3 K/V,
// with both contractions of a tile on the matrix cores
// (v_mfma_f32_16x16x32_{bf16,f16}: D[16][16] += A[16][32] . B[32][16]; lane
// l supplies A[l%16][8(l/16) + i] and B[8(l/16) + i][l%16], i < 8, and holds
// D[4(l/16) + v][l%16], v < 4).  Lane l is (a, c) = (l/16, l%16).  With G
// query heads per KV head only G of the 16 rows (or columns) carry data; the
// vector unit, which in the vector kernel spends most of an fp8 tile on the
// products and their reductions, is left with the E4M3 widening and the
// softmax.
//
//  * q.k.  Lane (a, c) loads 16 bytes of K: dims 64s + 16a .. +16 of token
//    16tb + c (chunk 2tb + s).  Each half (dims 64s + 16a + 8h .. +8) is
//    widened exactly to q's type and is the B operand of dim step 2s + h; q
//    (rows = heads) is the A operand, lane (a, c) holding
//    q[head c][64s + 16a + 8h .. +8] -- the same dims at the same k index,
//    so the contraction runs over all 128 dims in a permuted order.  Scores
//    land in lane (a, c), register v: head 4a + v, token 16tb + c; the K
//    scale of that token multiplies them.
//  * p.V.  V keeps the row layout of the vector kernel's byte path: lane
//    (a, c) holds dims 8c .. 8c+7 of token 4J + a (chunk J, 8 bytes).  For
//    dim offset e and half H of the tile, A[m = c][k = 8a + i] =
//    V[token 4(8H + i) + a][dim 8c + e] comes from byte e of chunks 8H .. 8H+7:
//    one byte permute per two chunks and two dims, then one widening to a
//    bf16 pair.  B[k][n] = p[head n][that token] times the token's V scale,
//    rounded to bf16, comes from LDS; O^T[dim 8m + e][head n] accumulates in
//    8 x 4 registers.  (p in bf16 carries a relative error of at most 2^-9
//    per term, below the output's own rounding; an f16 q would need p times
//    the V scale in f16, whose range that product can leave.)
//  * The register ring, masking, online softmax and piece / merge handling
//    are those of the vector kernel.

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

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

// Calls f(std::integral_constant<int, I>) for I = 0 .. N-1.
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    [&]<int... I>(std::integer_sequence<int, I...>) { (f(std::integral_constant<int, I>{}), ...); }
        (std::make_integer_sequence<int, N>{});
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

// Eight E4M3 codes (bytes of w0, w1) widened exactly to 8 values of q's type.
template <int QT>
__device__ __forceinline__ u32x4 widen8(u32 w0, u32 w1)
{
    return u32x4{fp8_pair16<QT, false>(w0), fp8_pair16<QT, true>(w0), fp8_pair16<QT, false>(w1),
                 fp8_pair16<QT, true>(w1)};
}

// K of one 64-token fp8 tile in the q.k operand layout: chunk I = 2tb + s
// holds, for lane (a, c), the 16 bytes of dims 64s + 16a .. of token 16tb + c.
template <int PS>
struct Fp8KOperandTile {
    static constexpr int ROW = 128, TILE_BYTES = PS * ROW, PPT = kTileTokens / PS;
    const char *base[PPT];
    int nblocks;   // token blocks (of 16) that hold this lane's token

    __device__ __forceinline__ void set(const char *head, size_t page_stride, const int (&ph)[PPT], int rem, int c)
    {
#pragma unroll
        for (int pg = 0; pg < PPT; ++pg)
            base[pg] = uniform_ptr(head + (size_t)(ph[pg] >= 0 ? ph[pg] : 0) * page_stride);
        nblocks = rem > c ? (rem - c + 15) / 16 : 0;
    }

    template <int I>
    __device__ __forceinline__ u32x4 load(int lane_off) const
    {
        constexpr int tb = I / 2, st = I % 2;
        constexpr int pg = (16 * tb) / PS;
        constexpr int chunk_off = ((16 * tb) % PS) * ROW + 64 * st;
        const int voff = tb < nblocks ? lane_off : kOutOfRange;
        return __builtin_amdgcn_raw_buffer_load_b128(tile_rsrc(base[pg], TILE_BYTES), voff, chunk_off,
                                                     kStreamingLoad);
    }
};

template <int PS, int G, int QT>
__global__ __launch_bounds__(kWavesPerGroup * 64) __attribute__((amdgpu_waves_per_eu(2))) void paged_decode_fp8_mfma_kernel(DecodeParams p)
{
    constexpr int D = 128;
    using S = Shape<D, PS, G, QT, FP8>;
    constexpr int PPT = S::PPT;
    static_assert(S::R == 16 && S::TPI == 4 && S::EPL == 8 && S::CB == 8, "layout of the 128-dim fp8 tile");
    static_assert(G <= 16, "one head per matrix row");

    // per-wave LDS: this wave's slot of the workgroup's arrays
    const int slot = threadIdx.x / 64;
    __shared__ float s_p_all[kWavesPerGroup][16 * 64];   // probabilities times V scales: [head][token % 4][token / 4]
    __shared__ int s_pend_all[kWavesPerGroup][2][3];
    __shared__ int s_npend_all[kWavesPerGroup];
    // the range's first piece, written after the last tile
    __shared__ __align__(16) float s_first_all[kWavesPerGroup][G * D];
    __shared__ float2 s_first_ml_all[kWavesPerGroup][G];
    float *const s_p = s_p_all[slot];
    int (*const s_pend)[3] = s_pend_all[slot];
    int &s_npend = s_npend_all[slot];
    float *const s_first = s_first_all[slot];
    float2 *const s_first_ml = s_first_ml_all[slot];
    int first_slot = -1;

    const int lane = threadIdx.x % 64;
    const int a = lane / 16, c = lane % 16;
    const int Hq = p.num_q_heads, Hkv = p.num_kv_heads;
    const long long NW = p.num_splits, w = (long long)blockIdx.x * kWavesPerGroup + slot;
    if (w >= NW)
        return;

    Lens lens;
    lens.load(p, lane);
    const long long T = (long long)batch_tiles(p, lens, lane) * Hkv;
    for (long long b = w; b < p.batch; b += NW) {
        const int n = lens.of(p, (int)b);
        if (tiles_of(n, p.max_context_len) == 0) {
            const float fill = (n < 0 || n > p.max_context_len) ? __builtin_nanf("") : 0.0f;
            u32 *o = reinterpret_cast<u32 *>(p.out) + (size_t)b * Hq * D / 2;
            for (int i = lane; i < Hq * D / 2; i += 64)
                o[i] = pack_out<QT>(fill, fill);
        }
    }
    const long long NWe = NW < T ? NW : T;
    if (w >= NWe)
        return;
    const long long H = p.first_round < NWe && T >= 2 * NWe ? p.first_round : NWe;
    const long long lo = range_start<kShareFp8A, kShareFp8B>(w, T, NWe, H);
    const long long hi = range_start<kShareFp8A, kShareFp8B>(w + 1, T, NWe, H);
    if (w == 0 && lane == 0)
        *p.ws_tag = p.tag;

    struct Cursor {
        int b, n, nt, g, k;
        __device__ __forceinline__ void make_uniform()
        {
            b = __builtin_amdgcn_readfirstlane(b);
            n = __builtin_amdgcn_readfirstlane(n);
            nt = __builtin_amdgcn_readfirstlane(nt);
            g = __builtin_amdgcn_readfirstlane(g);
            k = __builtin_amdgcn_readfirstlane(k);
        }
    };
    Cursor cur;
    {
        long long start;
        locate(p, lens, lo, lane, cur.b, start);
        cur.n = lens.of(p, cur.b);
        cur.nt = tiles_of(cur.n, p.max_context_len);
        const long long off = lo - start;
        cur.g = (int)div_nonneg(off, cur.nt);
        cur.k = (int)(off - (long long)cur.g * cur.nt);
        cur.make_uniform();
    }
    auto advance = [&](const Cursor &x0) {
        Cursor x = x0;
        if (++x.k == x.nt) {
            x.k = 0;
            if (++x.g == Hkv) {
                x.g = 0;
                do {
                    ++x.b;
                    x.n = x.b < p.batch ? lens.of(p, x.b) : 0;
                    x.nt = tiles_of(x.n, p.max_context_len);
                } while (x.nt == 0 && x.b < p.batch);
            }
        }
        x.make_uniform();
        return x;
    };

    bool any_bad = false;
    const size_t page_stride = (size_t)Hkv * S::TILE_BYTES;
    auto pages_of = [&](const Cursor &x, int (&ph)[PPT]) {
        const int32_t *bt = p.block_tables + (size_t)min(x.b, p.batch - 1) * p.max_blocks;
        bool bad = false;
#pragma unroll
        for (int pg = 0; pg < PPT; ++pg) {
            const int v = bt[min(x.k * PPT + pg, p.max_blocks - 1)];
            const bool exists = x.k * kTileTokens + pg * PS < x.n;
            const bool inside = (unsigned)v < (unsigned)p.num_pages;
            bad = bad || (exists && !inside);
            ph[pg] = exists && inside ? v : -1;
        }
        return bad;
    };
    auto tile_rem = [&](const Cursor &x) { return min(kTileTokens, x.n - x.k * kTileTokens); };
    // K and V scales of tokens 16tb + c of the cursor's tile (0 for a token
    // that is not there)
    auto scales_of = [&](const Cursor &x, const int (&ph)[PPT], float (&ks)[4], float (&vs)[4]) {
        const int rem = x.n - x.k * kTileTokens;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            const int pg = (16 * tb) / PS;
            const bool ok = ph[pg] >= 0 && 16 * tb + c < rem;
            const size_t si = ok ? ((size_t)ph[pg] * Hkv + x.g) * PS + (16 * tb) % PS + c : 0;
            const float kv = p.k_scale[si], vv = p.v_scale[si];
            ks[tb] = ok ? kv : 0.0f;
            vs[tb] = ok ? vv : 0.0f;
        }
    };

    // q of the segment as the A operand of the four dim steps: lane (a, c)
    // holds q[head c][64s + 16a + 8h .. +8] in qa[2s + h] (zero for c >= G)
    u32x4 qa[4];
    auto load_q = [&](const Cursor &x) {
        const char *base = (const char *)p.q + (((size_t)x.b * Hq + (size_t)x.g * G + (c < G ? c : 0)) * D) * 2;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(base + (64 * (st / 2) + 16 * a + 8 * (st % 2)) * 2);
            qa[st] = c < G ? v : u32x4{0u, 0u, 0u, 0u};
        }
    };

    f32x4 acc[8];               // O^T[dim 8(4a + v) + e][head c] in acc[e][v]
    float m_row[4], l_row[4];   // running max / this lane's sum for head 4a + v
    auto reset_state = [&]() {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[e] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            m_row[v] = -INFINITY;
            l_row[v] = 0.0f;
        }
    };
    // value of a per-head quantity held row-wise (head 4a + v in register v of
    // row a) for the head of this lane's column, c
    auto head_of_column = [&](const float (&row)[4]) {
        float r = 1.0f;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float x = lane_value(row[h % 4], 16 * (h / 4));
            r = c == h ? x : r;
        }
        return r;
    };

    const int lane_off_k = c * S::ROW + 16 * a;
    const int lane_off_v = a * S::ROW + 8 * c;
    // Pages two tiles deep: the tile being computed, the next one (whose K
    // and V are in flight) and the one after it (whose block-table entries
    // are being read).
    const char *k_head = (const char *)p.k_pool, *v_head = (const char *)p.v_pool;
    int ph_cur[PPT], ph_nxt[PPT], ph_nx2[PPT];
    bool bad_cur = pages_of(cur, ph_cur), bad_nxt = false, bad_nx2 = false;
    Fp8KOperandTile<PS> ka;
    TileAddr<S> va;
    ka.set(k_head + (size_t)cur.g * S::TILE_BYTES, page_stride, ph_cur, tile_rem(cur), c);
    va.set(v_head + (size_t)cur.g * S::TILE_BYTES, page_stride, ph_cur, tile_rem(cur), a);
    // K chunk I (16 bytes) in rk[I]; V chunks 2I, 2I + 1 (8 bytes each) in
    // rv[I].  Each is refilled with the next tile's chunk as soon as it has
    // been used, so both K and V are a whole tile ahead of the arithmetic.
    u32x4 rk[8], rv[8];
    static_for<8>([&](auto Ic) {
        constexpr int I = decltype(Ic)::value;
        rk[I] = ka.template load<I>(lane_off_k);
    });
    static_for<8>([&](auto Ic) {
        constexpr int I = decltype(Ic)::value;
        const u32x2 v0 = va.template load<2 * I>(lane_off_v);
        const u32x2 v1 = va.template load<2 * I + 1>(lane_off_v);
        rv[I] = u32x4{v0[0], v0[1], v1[0], v1[1]};
    });
    load_q(cur);
    reset_state();
    float ks_cur[4], vs_cur[4], ks_nxt[4], vs_nxt[4];
    scales_of(cur, ph_cur, ks_cur, vs_cur);
    bool piece_from_start = cur.k == 0;
    if (lane == 0)
        s_npend = 0;
    Cursor nxt = lo + 1 < hi ? advance(cur) : cur;
    if (lo + 1 < hi)
        bad_nxt = pages_of(nxt, ph_nxt);
    else
#pragma unroll
        for (int pg = 0; pg < PPT; ++pg)
            ph_nxt[pg] = -1;

    for (long long t = lo; t < hi; ++t) {
        if (!p.fused && cur.k == 0 && lane == 0)
            p.seg_geo[cur.b * Hkv + cur.g] =
                make_int4((int)p.tag, (int)w, (int)owner_of<kShareFp8A, kShareFp8B>(t + cur.nt - 1, T, NWe, H), 0);
        const bool last_in_range = t + 1 == hi;
        const bool has_nx2 = t + 2 < hi;
        const Cursor nx2 = has_nx2 ? advance(nxt) : nxt;
        const bool seg_end = last_in_range || nxt.k == 0;
        any_bad = any_bad || bad_cur;
        bad_nx2 = false;
        if (has_nx2)
            bad_nx2 = pages_of(nx2, ph_nx2);
        else
#pragma unroll
            for (int pg = 0; pg < PPT; ++pg)
                ph_nx2[pg] = -1;
        // the next tile's addresses (nothing is read for a tile past the range)
        ka.set(k_head + (size_t)nxt.g * S::TILE_BYTES, page_stride, ph_nxt, last_in_range ? 0 : tile_rem(nxt), c);
        va.set(v_head + (size_t)nxt.g * S::TILE_BYTES, page_stride, ph_nxt, last_in_range ? 0 : tile_rem(nxt), a);
        scales_of(nxt, ph_nxt, ks_nxt, vs_nxt);

        // ---- q.k on the matrix cores; each K chunk's registers then take
        // the next tile's K chunk
        f32x4 sc[4];
        static_for<4>([&](auto TBc) {
            constexpr int TB = decltype(TBc)::value;
            f32x4 x = {0.0f, 0.0f, 0.0f, 0.0f};
            static_for<2>([&](auto Sc) {
                constexpr int ST = decltype(Sc)::value;
                constexpr int I = 2 * TB + ST;
                const u32x4 kc = rk[I];
                x = mfma32<QT>(qa[2 * ST], widen8<QT>(kc[0], kc[1]), x);
                x = mfma32<QT>(qa[2 * ST + 1], widen8<QT>(kc[2], kc[3]), x);
                rk[I] = ka.template load<I>(lane_off_k);
            });
            sc[TB] = x;
        });

        // ---- online softmax (log2 domain): lane (a, c), register v holds
        // head 4a + v, token 16tb + c
        const int rem = cur.n - cur.k * kTileTokens;
        float alpha_row[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float mx = -INFINITY;
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const float x = 16 * tb + c < rem ? sc[tb][v] * ks_cur[tb] * p.scale_log2 : -INFINITY;
                sc[tb][v] = x;
                mx = fmaxf(mx, x);
            }
            const float m_new = fmaxf(m_row[v], row_max16(mx));
            alpha_row[v] = __builtin_amdgcn_exp2f(m_row[v] - m_new);
            float ls = 0.0f;
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const float e = __builtin_amdgcn_exp2f(sc[tb][v] - m_new);
                sc[tb][v] = e;
                ls += e;
            }
            l_row[v] = l_row[v] * alpha_row[v] + ls;
            m_row[v] = m_new;
        }
        // probabilities times the V scale to LDS, [head][token % 4][token / 4]
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                s_p[(4 * a + v) * 64 + (c % 4) * 16 + 4 * tb + c / 4] = sc[tb][v] * vs_cur[tb];
        const float alpha_c = head_of_column(alpha_row);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[e] *= alpha_c;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- p.V on the matrix cores, one half of the tile (32 tokens) at a time
        static_for<2>([&](auto Hc) {
            constexpr int H = decltype(Hc)::value;
            const float *src = s_p + (c < G ? c : 0) * 64 + a * 16 + 8 * H;
            const float4 p0 = *reinterpret_cast<const float4 *>(src);
            const float4 p1 = *reinterpret_cast<const float4 *>(src + 4);
            u32x4 bop = {pack_out<BF16>(p0.x, p0.y), pack_out<BF16>(p0.z, p0.w), pack_out<BF16>(p1.x, p1.y),
                         pack_out<BF16>(p1.z, p1.w)};
            if (c >= G)
                bop = u32x4{0u, 0u, 0u, 0u};
            // A operand of dim offset e: bf16 pairs (chunk 8H + 2q, chunk 8H + 2q + 1), q < 4
            static_for<2>([&](auto Dc) {
                constexpr int DW = decltype(Dc)::value;   // dword of the 8-byte chunks: dims 4DW .. 4DW+3
                u32x4 aop[4];
                static_for<4>([&](auto Qc) {
                    constexpr int Q = decltype(Qc)::value;
                    const u32x4 pr = rv[4 * H + Q];        // chunks 8H + 2Q (x, y), 8H + 2Q + 1 (z, w)
                    // bytes (c0.k, c1.k, c0.k+1, c1.k+1) for k = 0 and k = 2
                    const u32 b01 = __builtin_amdgcn_perm(pr[2 + DW], pr[DW], 0x05010400u);
                    const u32 b23 = __builtin_amdgcn_perm(pr[2 + DW], pr[DW], 0x07030602u);
                    aop[0][Q] = fp8_pair16<BF16, false>(b01);
                    aop[1][Q] = fp8_pair16<BF16, true>(b01);
                    aop[2][Q] = fp8_pair16<BF16, false>(b23);
                    aop[3][Q] = fp8_pair16<BF16, true>(b23);
                });
                static_for<4>([&](auto Kc) {
                    constexpr int K = decltype(Kc)::value;
                    acc[4 * DW + K] = mfma32<BF16>(aop[K], bop, acc[4 * DW + K]);
                });
            });
            static_for<4>([&](auto Jc) {
                constexpr int I = 4 * H + decltype(Jc)::value;
                const u32x2 v0 = va.template load<2 * I>(lane_off_v);
                const u32x2 v1 = va.template load<2 * I + 1>(lane_off_v);
                rv[I] = u32x4{v0[0], v0[1], v1[0], v1[1]};
            });
        });
        __builtin_amdgcn_wave_barrier();

        // ---- end of a piece
        if (seg_end) {
            const bool whole = piece_from_start && cur.k == cur.nt - 1;
            const int seg = cur.b * Hkv + cur.g;
            const float nan = __builtin_nanf("");
            float l_tot[4];
#pragma unroll
            for (int v = 0; v < 4; ++v)
                l_tot[v] = row_sum16(l_row[v]);
            const float l_c = head_of_column(l_tot);
            const float m_c = head_of_column(m_row);
            if (c < G) {
                if (whole) {
                    const size_t unit = (size_t)cur.b * Hq + (size_t)cur.g * G + c;
                    const float inv = any_bad ? nan : 1.0f / l_c;
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const u32x4 o = {pack_out<QT>(acc[0][v] * inv, acc[1][v] * inv),
                                         pack_out<QT>(acc[2][v] * inv, acc[3][v] * inv),
                                         pack_out<QT>(acc[4][v] * inv, acc[5][v] * inv),
                                         pack_out<QT>(acc[6][v] * inv, acc[7][v] * inv)};
                        *reinterpret_cast<u32x4 *>(reinterpret_cast<u32 *>(p.out) + (unit * D + 8 * (4 * a + v)) / 2) = o;
                    }
                } else if (!piece_from_start && !last_in_range) {
                    // the range's first piece: to LDS, written after the last tile
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        float *dst = s_first + c * D + 8 * (4 * a + v);
                        *reinterpret_cast<float4 *>(dst) =
                            any_bad ? make_float4(nan, nan, nan, nan)
                                    : make_float4(acc[0][v], acc[1][v], acc[2][v], acc[3][v]);
                        *reinterpret_cast<float4 *>(dst + 4) =
                            any_bad ? make_float4(nan, nan, nan, nan)
                                    : make_float4(acc[4][v], acc[5][v], acc[6][v], acc[7][v]);
                    }
                    if (a == 0)
                        s_first_ml[c] = make_float2(m_c, any_bad ? nan : l_c);
                } else {
                    const size_t slot = (size_t)seg + (size_t)w;
                    float *po = uniform_fptr(p.part_o + slot * G * D);
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int off = (c * D + 8 * (4 * a + v)) * 4;
                        store_coherent4(po, G * D * 4, off,
                                        any_bad ? make_float4(nan, nan, nan, nan)
                                                : make_float4(acc[0][v], acc[1][v], acc[2][v], acc[3][v]));
                        store_coherent4(po, G * D * 4, off + 16,
                                        any_bad ? make_float4(nan, nan, nan, nan)
                                                : make_float4(acc[4][v], acc[5][v], acc[6][v], acc[7][v]));
                    }
                    if (a == 0)
                        store_coherent2(uniform_fptr(p.part_ml + slot * G * 2), G * 8, c * 8,
                                        make_float2(m_c, any_bad ? nan : l_c));
                }
            }
            if (!whole && !piece_from_start && !last_in_range)
                first_slot = seg + (int)w;
            if (!whole) {
                const long long first = t - cur.k;
                const int w0 = (int)owner_of<kShareFp8A, kShareFp8B>(first, T, NWe, H);
                const int w1 = (int)owner_of<kShareFp8A, kShareFp8B>(first + cur.nt - 1, T, NWe, H);
                if (lane == 0) {
                    const int i = s_npend;
                    s_pend[i][0] = seg;
                    s_pend[i][1] = w0;
                    s_pend[i][2] = w1 - w0 + 1;
                    s_npend = i + 1;
                }
            }
            reset_state();
            any_bad = false;
            piece_from_start = true;
            if (!last_in_range)
                load_q(nxt);   // behind the next tile's K loads already in flight
        }

#pragma unroll
        for (int pg = 0; pg < PPT; ++pg) {
            ph_cur[pg] = ph_nxt[pg];
            ph_nxt[pg] = ph_nx2[pg];
        }
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            ks_cur[tb] = ks_nxt[tb];
            vs_cur[tb] = vs_nxt[tb];
        }
        bad_cur = bad_nxt;
        bad_nxt = bad_nx2;
        cur = nxt;
        nxt = nx2;
    }

    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (first_slot >= 0)
        flush_first_piece<D, G>(p, first_slot, s_first, s_first_ml, lane);
    if (p.fused)
        settle_pending<D, G, QT>(p, s_pend, __builtin_amdgcn_readfirstlane(s_npend), (int)w, lane);
}

// ---- the merge kernel --------------------------------------------------------
//
// For a segment whose tiles were shared by waves w0..w1, with pieces
// (m_k, l_k, o_k) (m in log2 units): M = max m_k, L = sum l_k 2^(m_k - M),
// out = sum o_k 2^(m_k - M) / L.  One workgroup per (query head, sequence).  The
// decode kernel recorded (tag, w0, w1) for every segment it started; a
// segment one wave covered whole (w0 == w1) is already written.  An empty
// sequence gets zeros (NaN for an invalid length).  Four waves take every
// fourth piece each, merging online with several pieces' loads in flight,
// and combine through LDS.

template <int D, int QT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(DecodeParams p)
{
    constexpr int DPL = D / 64;          // output dims per lane
    constexpr int WAVES = 4, UNROLL = 4;
    __shared__ float s_m[WAVES], s_l[WAVES];
    __shared__ float s_acc[WAVES][D];

    const int h = blockIdx.x, b = blockIdx.y;
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int Hkv = p.num_kv_heads, G = p.num_q_heads / p.num_kv_heads;
    const int g = h / G, hh = h % G;
    const size_t unit = (size_t)b * p.num_q_heads + h;
    const int n = p.context_lens[b];
    const int nt = tiles_of(n, p.max_context_len);
    if (nt == 0) {
        const float fill = (n < 0 || n > p.max_context_len) ? __builtin_nanf("") : 0.0f;
        if (threadIdx.x < D / 2)
            reinterpret_cast<u32 *>(p.out)[(unit * D) / 2 + threadIdx.x] = pack_out<QT>(fill, fill);
        return;
    }
    const size_t seg = (size_t)b * Hkv + g;
    const int4 geo = p.seg_geo[seg];
    if ((uint32_t)geo.x != *p.ws_tag || geo.y >= geo.z)
        return;                          // covered whole by one wave: already written
    const int np_ = geo.z - geo.y + 1;
    const size_t first = (seg + (size_t)geo.y) * G + hh;   // wave w0's piece; + G per wave

    // online merge of this wave's pieces (k = wave, wave + 4, ...), UNROLL
    // pieces' loads in flight at a time
    float m = -INFINITY, L = 0.0f, acc[DPL];
#pragma unroll
    for (int d = 0; d < DPL; ++d)
        acc[d] = 0.0f;
    for (int k0 = wave; k0 < np_; k0 += WAVES * UNROLL) {
        float2 ml[UNROLL];
        float ov[UNROLL][DPL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int k = k0 + u * WAVES;
            const size_t pc = first + (size_t)(k < np_ ? k : 0) * G;
            ml[u] = *reinterpret_cast<const float2 *>(p.part_ml + pc * 2);
#pragma unroll
            for (int d = 0; d < DPL; ++d)
                ov[u][d] = p.part_o[pc * D + DPL * lane + d];
            if (k >= np_)
                ml[u].x = -INFINITY;
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            if (ml[u].x == -INFINITY)
                continue;
            const float m_new = fmaxf(m, ml[u].x);
            const float a = __builtin_amdgcn_exp2f(m - m_new), c = __builtin_amdgcn_exp2f(ml[u].x - m_new);
            L = L * a + ml[u].y * c;
#pragma unroll
            for (int d = 0; d < DPL; ++d)
                acc[d] = acc[d] * a + ov[u][d] * c;
            m = m_new;
        }
    }
    if (lane == 0) {
        s_m[wave] = m;
        s_l[wave] = L;
    }
#pragma unroll
    for (int d = 0; d < DPL; ++d)
        s_acc[wave][DPL * lane + d] = acc[d];
    __syncthreads();
    if (wave == 0) {
        float M = s_m[0];
#pragma unroll
        for (int q = 1; q < WAVES; ++q)
            M = fmaxf(M, s_m[q]);
        float Lt = 0.0f, o[DPL];
#pragma unroll
        for (int d = 0; d < DPL; ++d)
            o[d] = 0.0f;
#pragma unroll
        for (int q = 0; q < WAVES; ++q) {
            const float f = __builtin_amdgcn_exp2f(s_m[q] - M);   // 0 for a wave without pieces
            Lt = fmaf(f, s_l[q], Lt);
#pragma unroll
            for (int d = 0; d < DPL; ++d)
                o[d] = fmaf(f, s_acc[q][DPL * lane + d], o[d]);
        }
        const float inv = 1.0f / Lt;
        if constexpr (DPL == 2) {
            reinterpret_cast<u32 *>(p.out)[(unit * D) / 2 + lane] = pack_out<QT>(o[0] * inv, o[1] * inv);
        } else {
            const float other = __shfl_xor(o[0], 1);
            if ((lane & 1) == 0)
                reinterpret_cast<u32 *>(p.out)[(unit * D) / 2 + lane / 2] = pack_out<QT>(o[0] * inv, other * inv);
        }
    }
}

// ---- K/V scatter for appended tokens -----------------------------------------
//
// A token row (one token, one KV head) is handled by the lanes of one group,
// each lane owning 16 bytes of it, so that a wave reads whole consecutive rows
// of the caller's [n][Hkv][D] arrays.  Row indices are 32-bit (the host
// rejects n * Hkv >= 2^31); a slot's page and offset use a 32-bit division
// whenever the slot fits in 32 bits.

// Pool row of `slot` (page-major: [page][Hkv][page_size]) for KV head g;
// false for a slot outside the pool, which is skipped.
__device__ __forceinline__ bool pool_row(int64_t slot, u32 g, int32_t page_size, int32_t num_pages,
                                         int32_t num_kv_heads, size_t &row)
{
    if (slot < 0 || slot >= (int64_t)num_pages * page_size)
        return false;
    u32 page, off;
    if (slot <= (int64_t)0xFFFFFFFF) {
        page = (u32)slot / (u32)page_size;
        off = (u32)slot - page * (u32)page_size;
    } else {
        const int64_t pg = slot / page_size;
        page = (u32)pg;
        off = (u32)(slot - pg * page_size);
    }
    row = ((size_t)page * (u32)num_kv_heads + g) * (u32)page_size + off;
    return true;
}

// Copy form: rows already in the pool's type (with their scales for int8 /
// fp8).  CPR = 16-byte chunks per row.
template <int CPR>
__global__ __launch_bounds__(256) void write_kv_kernel(WriteParams p)
{
    constexpr u32 RPB = 256 / CPR;   // rows per block and pass
    const u32 c = threadIdx.x % CPR;
    const u32 rows = (u32)p.n * (u32)p.num_kv_heads;
    const u32x4 *kn = reinterpret_cast<const u32x4 *>(p.k_new);
    const u32x4 *vn = reinterpret_cast<const u32x4 *>(p.v_new);
    u32x4 *kp = reinterpret_cast<u32x4 *>(p.k_pool);
    u32x4 *vp = reinterpret_cast<u32x4 *>(p.v_pool);
    for (u32 row = blockIdx.x * RPB + threadIdx.x / CPR; row < rows; row += gridDim.x * RPB) {
        const u32x4 kx = kn[(size_t)row * CPR + c];
        const u32x4 vx = vn[(size_t)row * CPR + c];
        const u32 i = row / (u32)p.num_kv_heads, g = row - i * (u32)p.num_kv_heads;
        size_t dst;
        if (!pool_row(p.slots[i], g, p.page_size, p.num_pages, p.num_kv_heads, dst))
            continue;
        kp[dst * CPR + c] = kx;
        vp[dst * CPR + c] = vx;
        if (c == 0 && p.k_scale) {
            p.k_scale[dst] = p.k_scale_new[row];
            p.v_scale[dst] = p.v_scale_new[row];
        }
    }
}

// ---- quantise-on-append ------------------------------------------------------
//
// f16 / bf16 rows into an int8 or fp8 pool.  Each row of D values is held by
// D / 8 lanes, 8 values each; the row's exact max magnitude is reduced over
// those lanes, s = max(amax, 1e-5) / Q in fp32 (Q = 127 for int8, 448 for
// E4M3, correctly rounded division), then each value's code is
// round-half-to-even of x / s (int8 clipped to +-127; fp8 through the
// hardware converter, which rounds to nearest even; |x / s| never exceeds 448
// by more than the rounding of s, which still rounds to 448).  The scale goes
// to the pool's scale array at the row's slot.

constexpr int kRowHalfMirror = 0x141;   // row_half_mirror: j -> 7 - j within 8 lanes

// max over aligned groups of L lanes (L = 8 or 16); every lane gets its group's
template <int L>
__device__ __forceinline__ float group_max(float x)
{
    x = fmaxf(x, dpp<kQuadXor1>(x));
    x = fmaxf(x, dpp<kQuadXor2>(x));
    x = fmaxf(x, dpp<kRowHalfMirror>(x));
    if constexpr (L == 16)
        x = fmaxf(x, dpp<kRowRor8>(x));
    return x;
}

template <int L, int SRC, int KVT>
__device__ __forceinline__ void quantise8(u32x4 w, u32 &lo, u32 &hi, float &s)
{
    constexpr float kQ = KVT == I8 ? 127.0f : 448.0f;
    float x[8];
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const u32 bits = (w[e / 2] >> (16 * (e % 2))) & 0xFFFFu;
        x[e] = SRC == BF16 ? __builtin_bit_cast(float, bits << 16)
                           : (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
        amax = fmaxf(amax, fabsf(x[e]));
    }
    amax = group_max<L>(amax);
    s = fmaxf(amax, 1e-5f) / kQ;
    // x / s, correctly rounded, with one division per row instead of one per
    // value: y = RN(1 / s), then two of Markstein's corrections of x y (each
    // q' = RN(q + (x - s q) y), the remainder exact through an fma).  x y is
    // within two ulps of x / s, the first step brings it within one, and the
    // second gives the correctly rounded quotient (P. Markstein, "Computation
    // of elementary functions on the IBM RISC System/6000 processor", IBM J.
    // Res. Dev. 34(1), 1990).  Quotients small enough for underflow to matter
    // map to code 0 either way.  The quotient takes x's sign (s > 0): a -0
    // stays -0, whose code differs from +0's.
    const float y = 1.0f / s;
    auto quot = [&](float v) {
        float q = v * y;
        q = fmaf(fmaf(-s, q, v), y, q);
        return copysignf(fmaf(fmaf(-s, q, v), y, q), v);
    };
    u32 word[2];
    if constexpr (KVT == I8) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            u32 v = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float r = fminf(fmaxf(rintf(quot(x[4 * h + e])), -127.0f), 127.0f);
                v |= ((u32)(int)r & 0xFFu) << (8 * e);
            }
            word[h] = v;
        }
    } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            int v = __builtin_amdgcn_cvt_pk_fp8_f32(quot(x[4 * h]), quot(x[4 * h + 1]), 0, false);
            v = __builtin_amdgcn_cvt_pk_fp8_f32(quot(x[4 * h + 2]), quot(x[4 * h + 3]), v, true);
            word[h] = (u32)v;
        }
    }
    lo = word[0];
    hi = word[1];
}

template <int D, int SRC, int KVT>
__global__ __launch_bounds__(256) void write_kv_quant_kernel(WriteParams p)
{
    constexpr u32 L = D / 8;         // lanes per row
    constexpr u32 RPB = 256 / L;     // rows per block and pass
    const u32 sub = threadIdx.x % L;
    const u32 rows = (u32)p.n * (u32)p.num_kv_heads;
    const u32x4 *kn = reinterpret_cast<const u32x4 *>(p.k_new);
    const u32x4 *vn = reinterpret_cast<const u32x4 *>(p.v_new);
    u32x2 *kp = reinterpret_cast<u32x2 *>(p.k_pool);
    u32x2 *vp = reinterpret_cast<u32x2 *>(p.v_pool);
    for (u32 row = blockIdx.x * RPB + threadIdx.x / L; row < rows; row += gridDim.x * RPB) {
        const u32x4 kx = kn[(size_t)row * L + sub];
        const u32x4 vx = vn[(size_t)row * L + sub];
        const u32 i = row / (u32)p.num_kv_heads, g = row - i * (u32)p.num_kv_heads;
        size_t dst;
        if (!pool_row(p.slots[i], g, p.page_size, p.num_pages, p.num_kv_heads, dst))
            continue;   // the whole group skips: its lanes share the row
        u32 lo, hi;
        float s;
        quantise8<L, SRC, KVT>(kx, lo, hi, s);
        kp[dst * L + sub] = u32x2{lo, hi};
        if (sub == 0)
            p.k_scale[dst] = s;
        quantise8<L, SRC, KVT>(vx, lo, hi, s);
        vp[dst * L + sub] = u32x2{lo, hi};
        if (sub == 0)
            p.v_scale[dst] = s;
    }
}

// ---- page copies (copy-on-write of shared pages) -------------------------------
//
// Block b copies tile b % tiles_per_page of pair b / tiles_per_page: kCopyUnroll
// 16-byte chunks per thread of K and of V (all loads issued before the
// stores), plus the same index range of the page's scales.

constexpr int kCopyUnroll = kCopyTileChunks / 256;
constexpr int kCopyTile = kCopyTileChunks;
static_assert(kCopyUnroll * 256 == kCopyTile, "a tile is kCopyUnroll chunks per thread");

__global__ __launch_bounds__(256) void copy_pages_kernel(CopyParams p)
{
    const u32 tiles = (u32)p.tiles_per_page;
    const u32 total = (u32)p.n * tiles;
    for (u32 b = blockIdx.x; b < total; b += gridDim.x) {
        const u32 pair = b / tiles, tile = b - pair * tiles;
        const int32_t src = p.pairs[2 * pair], dst = p.pairs[2 * pair + 1];
        if (src < 0 || src >= p.num_pages || dst < 0 || dst >= p.num_pages)
            continue;
        const int64_t chunks = p.page_bytes / 16;
        const int64_t c0 = (int64_t)tile * kCopyTile + threadIdx.x;
        const u32x4 *ks = reinterpret_cast<const u32x4 *>((const char *)p.k_pool + (size_t)src * p.page_bytes);
        const u32x4 *vs = reinterpret_cast<const u32x4 *>((const char *)p.v_pool + (size_t)src * p.page_bytes);
        u32x4 *kd = reinterpret_cast<u32x4 *>((char *)p.k_pool + (size_t)dst * p.page_bytes);
        u32x4 *vd = reinterpret_cast<u32x4 *>((char *)p.v_pool + (size_t)dst * p.page_bytes);
        u32x4 kv[kCopyUnroll], vv[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const int64_t c = c0 + 256 * u;
            if (c < chunks) {
                kv[u] = ks[c];
                vv[u] = vs[c];
            }
        }
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const int64_t c = c0 + 256 * u;
            if (c < chunks) {
                kd[c] = kv[u];
                vd[c] = vv[u];
            }
        }
        if (p.k_scale) {
#pragma unroll
            for (int u = 0; u < kCopyUnroll; ++u) {
                const int64_t j = c0 + 256 * u;
                if (j < p.page_scales) {
                    p.k_scale[(size_t)dst * p.page_scales + j] = p.k_scale[(size_t)src * p.page_scales + j];
                    p.v_scale[(size_t)dst * p.page_scales + j] = p.v_scale[(size_t)src * p.page_scales + j];
                }
            }
        }
    }
}

// ---- dispatch -------------------------------------------------------------------

template <int D, int PS, int G, int QT, int KVT>
int launch_one(const DecodeParams &p, hipStream_t stream)
{
    // kWavesPerGroup independent waves per workgroup (fewer workgroups to
    // dispatch); wave w is wave w % kWavesPerGroup of workgroup w / kWavesPerGroup
    dim3 grid((unsigned)((p.num_splits + kWavesPerGroup - 1) / kWavesPerGroup));
    void *args[] = {const_cast<DecodeParams *>(&p)};
    const void *fn = (const void *)&paged_decode_kernel<D, PS, G, QT, KVT>;
    if constexpr (KVT == FP8 && D == 128)
        fn = (const void *)&paged_decode_fp8_mfma_kernel<PS, G, QT>;   // fp8 at head_dim 128: matrix cores
    return (int)hipLaunchKernel(fn, grid, dim3(kWavesPerGroup * 64), args, 0, stream);
}

template <int D, int PS, int G>
int launch_dtype(const DecodeParams &p, int qt, int kvt, hipStream_t s)
{
    if (qt == F16 && kvt == F16) return launch_one<D, PS, G, F16, F16>(p, s);
    if (qt == BF16 && kvt == BF16) return launch_one<D, PS, G, BF16, BF16>(p, s);
    if (qt == F16 && kvt == I8) return launch_one<D, PS, G, F16, I8>(p, s);
    if (qt == BF16 && kvt == I8) return launch_one<D, PS, G, BF16, I8>(p, s);
    if (qt == F16 && kvt == FP8) return launch_one<D, PS, G, F16, FP8>(p, s);
    if (qt == BF16 && kvt == FP8) return launch_one<D, PS, G, BF16, FP8>(p, s);
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
                ((qt == F16 || qt == BF16) && (kvt == I8 || kvt == FP8));
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

static unsigned grid_for(size_t work, size_t per_block)
{
    const size_t blocks = (work + per_block - 1) / per_block;
    return (unsigned)(blocks < 65535 ? blocks : 65535);
}

template <int D, int SRC>
static int launch_quant(const WriteParams &p, hipStream_t s)
{
    const size_t rows = (size_t)p.n * p.num_kv_heads;
    void *args[] = {const_cast<WriteParams *>(&p)};
    const void *fn = p.kv_dtype == I8 ? (const void *)&write_kv_quant_kernel<D, SRC, I8>
                                      : (const void *)&write_kv_quant_kernel<D, SRC, FP8>;
    return (int)hipLaunchKernel(fn, dim3(grid_for(rows, 256 / (D / 8))), dim3(256), args, 0, s);
}

int launch_copy_pages(const CopyParams &p, void *stream)
{
    // chunks per page cover its scales too (a row has at least 16 bytes)
    const int64_t chunks = p.page_bytes / 16;
    CopyParams q = p;
    q.tiles_per_page = (int32_t)((chunks + kCopyTile - 1) / kCopyTile);
    if (q.tiles_per_page < 1 || p.page_scales > (int64_t)q.tiles_per_page * kCopyTile ||
        (int64_t)p.n * q.tiles_per_page > (int64_t)0xFFFFFFFF)
        return (int)hipErrorInvalidValue;
    void *args[] = {&q};
    return (int)hipLaunchKernel((const void *)&copy_pages_kernel,
                                dim3(grid_for((size_t)p.n * q.tiles_per_page, 1)), dim3(256), args, 0,
                                (hipStream_t)stream);
}

int launch_write_kv(const WriteParams &p, void *stream)
{
    hipStream_t s = (hipStream_t)stream;
    if (p.src_dtype != p.kv_dtype) {   // f16 / bf16 rows into an int8 / fp8 pool
        if (p.head_dim == 64)
            return p.src_dtype == BF16 ? launch_quant<64, BF16>(p, s) : launch_quant<64, F16>(p, s);
        return p.src_dtype == BF16 ? launch_quant<128, BF16>(p, s) : launch_quant<128, F16>(p, s);
    }
    const size_t rows = (size_t)p.n * p.num_kv_heads;
    void *args[] = {const_cast<WriteParams *>(&p)};
    const void *fn;
    switch (p.row_bytes) {
    case 64: fn = (const void *)&write_kv_kernel<4>; break;
    case 128: fn = (const void *)&write_kv_kernel<8>; break;
    case 256: fn = (const void *)&write_kv_kernel<16>; break;
    default: return (int)hipErrorInvalidValue;
    }
    return (int)hipLaunchKernel(fn, dim3(grid_for(rows, 256 / (p.row_bytes / 16))), dim3(256), args, 0, s);
}

}  // namespace pkv
