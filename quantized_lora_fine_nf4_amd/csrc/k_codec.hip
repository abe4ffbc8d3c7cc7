// k_codec.hip -- NF4 codec kernels for gfx950 (CDNA4, wave64).
//
// One tile = one double-quantisation group = 256 blocks of 64 weights
// (16384 weights, 32 KB of bf16).  The tiles of all layers form one flat
// index, so one grouped launch covers the whole stack.  The fused kernel is a
// one-shot grid of one 256-thread workgroup (4 waves) per tile; lane layout:
// wave w, load j (j = 0..7), lane L reads weights
// w*4096 + j*512 + 8L .. +8 with one 128-bit load, so each load instruction of
// a wave covers 1 KB contiguously and the 8 lanes 8m..8m+7 hold the 64 weights
// of one block.  The standalone double quantisation takes one wave per tile,
// the standalone dequantisation one small workgroup per eighth of a tile
// reading a per-tile record (see there); both are one-shot grids.
//
// What is computed (see nf4.h for the full format):
//   absmax      -- "quantisation constants" per block ("QLoRA" paper summary
//                  page, How It Works; "QLoRA Explained", Double Quantization)
//   NF4 codes   -- nearest of the 16 quantile levels (QLoRA page, NF4 item)
//   int8 DQ     -- the constants quantised again (QLoRA page, Double
//                  Quantization item)
//   dequant     -- back to 16-bit (QLoRA page, How It Works; AQLoRA listing,
//                  English abstract)
//   error       -- AQLoRA's per-layer NF4 reconstruction error (AQLoRA
//                  listing, English abstract)
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "nf4_format.h"
#include "nf4_internal.h"
#include "nf4_launch.h"

namespace nf4k {
namespace {

constexpr int kWaves = kThreads / 64;                    // 4 waves, each owning 64 blocks of a tile
constexpr int kLoads = kTileElems / (kThreads * 8);      // 8 x 128-bit loads per lane
constexpr int kCThreads = kThreads;                      // fused kernel workgroup
constexpr int kCWaves = kWaves;
constexpr int kCLoads = kLoads;
static_assert(kPartsPerTile == kCWaves, "one fp64 error partial per wave and tile");
constexpr int kCells = 129;                              // encode cells, trunc(64 s) in [-64, 64]
// Lane-indexed copies of the cell table (fewer bank conflicts on its 64-bit
// reads).  Eight copies keep the fused kernel's LDS at 28.8 KB, 5 workgroups
// per CU; measured on the 14B stack in one process: 16 copies (4 per CU)
// 5.84 ms, 8 copies 5.53, 4 copies (6 per CU, registers spilled) 5.63,
// 2 copies (7 per CU, spilled) 5.75.
constexpr int kRepl = 8;
constexpr int kYStride = 256 + 17;     // per-block dequant table, code-major, padded against bank conflicts
constexpr int kCodecWavesPerEu = 4;    // register cap of the fused pass (5 fit: 91 VGPRs; LDS allows 5)
constexpr int kQuantWavesPerEu = 3;    // the pass without the error (nf4_quantize): at 4 it spilled

typedef unsigned short us2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // 128-bit load / store unit
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

// Pointers read from the layer table are generic; marking them global lets the
// loads and stores use a scalar base plus 32-bit lane offsets.
#define GLOBAL __attribute__((address_space(1)))
typedef const GLOBAL uint16_t* g_cu16;
typedef const GLOBAL u32x4* g_cu4;
typedef const GLOBAL uint8_t* g_cu8;
typedef const GLOBAL uint32_t* g_cu32;
typedef const GLOBAL int8_t* g_ci8;
typedef const GLOBAL float* g_cf32;
typedef GLOBAL uint8_t* g_u8;
typedef GLOBAL uint32_t* g_u32;
typedef GLOBAL uint16_t* g_u16;
typedef GLOBAL u32x4* g_u4;
typedef GLOBAL int8_t* g_i8;
typedef GLOBAL float* g_f32;

// Stores of streams written once and not read back by the same kernel (codes,
// dequantised weights): non-temporal, so they do not displace cached lines
// (measured: dequantisation 5.03 -> 4.87 ms, fused pass 6.79 -> 6.74 ms on the
// 14B stack).
template <typename T>
__device__ __forceinline__ void store_stream(const T& v, GLOBAL T* p)
{
    __builtin_nontemporal_store(v, p);
}

// The fused pass reads each weight once: non-temporal loads (6.86 -> 6.74 ms
// on the 14B stack).  The dequantisation's code loads measured slower so.
template <typename T>
__device__ __forceinline__ T load_stream(const GLOBAL T* p)
{
    return __builtin_nontemporal_load(p);
}

__device__ __forceinline__ float as_f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __builtin_bit_cast(uint32_t, f); }

// One encode cell.  u = 64*s is cut into cells by truncation toward zero:
// cell k > 0 holds u in [k, k+1), k < 0 holds (k-1, k], k = 0 holds (-1, 1).
// The level gap (>= 0.0796, i.e. >= 5.09 in u) is wider than any cell's
// closure, so at most one threshold lies in it:
//   code = base + (u > thr),  thr = that threshold * 64 (or +inf),
//   base = number of thresholds strictly below the cell.
// u and thr are exact scalings by 64 of s and the fp32 threshold, so the
// comparison is exactly "threshold < s".
struct alignas(8) EncCell {
    float thr;
    uint32_t base;
};

__device__ void build_cells(EncCell* cells)
{
    for (int idx = threadIdx.x; idx < kCells * kRepl; idx += kCThreads) {
        const int k = idx / kRepl - 64;
        const float lo = (k > 0) ? (float)k : (k < 0 ? (float)(k - 1) : -1.0f);
        const float hi = (k > 0) ? (float)(k + 1) : (k < 0 ? (float)k : 1.0f);
        uint32_t base = 0;
        float thr = __builtin_inff();
        for (int i = 0; i < 15; ++i) {
            const float t64 = as_f(nf4fmt::kThresholdBits[i]) * 64.0f;
            if (t64 < lo) ++base;
            else if (t64 <= hi) thr = t64;
        }
        cells[idx] = EncCell{thr, base};
    }
}

// The tables of the fused pass as one constant in device memory, computed at
// compile time: the one-shot fused kernel copies it into LDS with 16-byte
// loads instead of rebuilding it for every tile.
//   cells  the encode cells (every replica, as build_cells writes them);
//   rcp    bf16 input: fl32(1 / (1 + m/128)) for the 7 mantissa bits m, so
//          that fl32(1/a) = 2^-e rcp[m] for every normal a = 2^e (1 + m/128)
//          (scaling by a power of two is exact);
//   d127   fl32((1 + m/128) / 127), so that fl32(G/127) = 2^e d127[m] for the
//          double-quant group maximum G = 2^e (1 + m/128), G >= 2^-100.
struct CodecTables {
    EncCell cells[kCells * kRepl];
    uint32_t rcp[128];
    uint32_t d127[128];
};

constexpr CodecTables make_tables()
{
    CodecTables t{};
    for (int m = 0; m < 128; ++m) {
        const float mant = 1.0f + (float)m / 128.0f;
        t.rcp[m] = __builtin_bit_cast(uint32_t, 1.0f / mant);
        t.d127[m] = __builtin_bit_cast(uint32_t, mant / 127.0f);
    }
    for (int idx = 0; idx < kCells * kRepl; ++idx) {
        const int k = idx / kRepl - 64;
        const float lo = (k > 0) ? (float)k : (k < 0 ? (float)(k - 1) : -1.0f);
        const float hi = (k > 0) ? (float)(k + 1) : (k < 0 ? (float)k : 1.0f);
        uint32_t base = 0;
        float thr = __builtin_inff();
        for (int i = 0; i < 15; ++i) {
            const float t64 = __builtin_bit_cast(float, nf4fmt::kThresholdBits[i]) * 64.0f;
            if (t64 < lo) ++base;
            else if (t64 <= hi) thr = t64;
        }
        t.cells[idx] = EncCell{thr, base};
    }
    return t;
}

// Padded to whole rounds of 256 lanes x 16 bytes, so the copy into LDS has no
// guarded remainder (the padding is zeros and lands at the start of the
// dequant table, which is cleared anyway).
constexpr int kCopyRound = 256 * 16;
constexpr int kCopyRounds = (int)((sizeof(CodecTables) + kCopyRound - 1) / kCopyRound);
struct PaddedTables {
    CodecTables t;
    uint8_t pad[kCopyRounds * kCopyRound - sizeof(CodecTables)];
};
constexpr PaddedTables make_padded_tables()
{
    PaddedTables p{};
    p.t = make_tables();
    return p;
}
__device__ const PaddedTables kTables = make_padded_tables();
static_assert(sizeof(PaddedTables) == kCopyRounds * kCopyRound, "whole copy rounds");

// ---- 16-bit helpers ------------------------------------------------------

// largest |x| bit pattern of 8 packed 16-bit values (sign-magnitude formats:
// for non-negative values the integer order is the numeric order)
__device__ __forceinline__ uint32_t absmax_bits8(const u32x4 v)
{
    const uint32_t m = 0x7fff7fffu;
    us2 a = __builtin_bit_cast(us2, v.x & m), b = __builtin_bit_cast(us2, v.y & m);
    us2 c = __builtin_bit_cast(us2, v.z & m), d = __builtin_bit_cast(us2, v.w & m);
    us2 r = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                      __builtin_elementwise_max(c, d));
    return r.x > r.y ? (uint32_t)r.x : (uint32_t)r.y;
}

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// The same through the packed fp16 maximum / minimum instructions, which take
// three operands (two values each): the largest magnitude is max(max x, -min x).
// For fp16 input that is the IEEE order of the values.  A bf16 bit pattern
// read as fp16 orders the same way while it is not an fp16 NaN: the order of
// IEEE values, infinities included, is the integer order of their 15
// magnitude bits with the sign on top, as for bf16.  A bf16 |x| >= 2^121 reads
// as an fp16 infinity or NaN, and a NaN would propagate, so a result at or
// above the infinity pattern 0x7c00 is not trusted (the caller recomputes the
// wave's maxima with absmax_bits8).
// (A value, not a vector element: this compiler's __builtin_bit_cast of an
// element access such as v.y was seen to read element 0 instead.)
__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }

__device__ __forceinline__ uint32_t absmax_bits8_f16ops(const u32x4 v)
{
    const h2 a = as_h2(v.x), b = as_h2(v.y), c = as_h2(v.z), d = as_h2(v.w);
    // chained so that each step is one three-operand instruction: max of
    // a, b, c; min of a, b, c, then of d; then max(that max, d, -min)
    const h2 mx3 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
    const h2 mn4 = __builtin_elementwise_minimum(__builtin_elementwise_minimum(__builtin_elementwise_minimum(a, b), c), d);
    const uint32_t r = __builtin_bit_cast(uint32_t, __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx3, d), -mn4));
    const uint32_t lo = r & 0xffffu, hi = r >> 16;
    return lo > hi ? lo : hi;
}

template <int DT>
__device__ __forceinline__ float f16bits_to_f32(uint32_t h)
{
    if constexpr (DT == 0) return as_f(h << 16);
    else return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

template <int DT>
__device__ __forceinline__ void unpack2(uint32_t d, float& lo, float& hi)
{
    if constexpr (DT == 0) {
        lo = as_f(d << 16);
        hi = as_f(d & 0xffff0000u);
    } else {
        lo = (float)__builtin_bit_cast(_Float16, (uint16_t)(d & 0xffffu));
        hi = (float)__builtin_bit_cast(_Float16, (uint16_t)(d >> 16));
    }
}

// Keeps the compiler from fusing a product with the following conversion to
// fp16 (v_fma_mix* rounds the exact product once; the format rounds to fp32
// first and then to the 16-bit type).
__device__ __forceinline__ float opaque(float x)
{
    __asm__ volatile("" : "+v"(x));
    return x;
}

// Element offset of this lane's first weight within a tile (wave w of W,
// lane L: (16384 / W) w + 8 L); load j adds 512 j.
template <int THREADS = kThreads>
__device__ __forceinline__ uint32_t lane_base()
{
    return (threadIdx.x >> 6) * (uint32_t)(kTileElems / (THREADS / 64)) + (threadIdx.x & 63u) * 8u;
}

// Round two fp32 values to the 16-bit type (nearest, ties to even) and return
// the packed pair; also the rounded values back in fp32.
template <int DT>
__device__ __forceinline__ uint32_t round_pair(float y0, float y1, float& r0, float& r1)
{
    if constexpr (DT == 0) {
        f2 in = {y0, y1};
        const uint32_t p = __builtin_bit_cast(uint32_t, __builtin_convertvector(in, bf2));
        r0 = as_f(p << 16);
        r1 = as_f(p & 0xffff0000u);
        return p;
    } else {
        const _Float16 h0 = (_Float16)opaque(y0), h1 = (_Float16)opaque(y1);
        r0 = (float)h0;
        r1 = (float)h1;
        return (uint32_t)__builtin_bit_cast(uint16_t, h0) |
               ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
    }
}

// ---- cross-lane reductions -----------------------------------------------

// Reduce over the 8 lanes of a block (lanes 8m..8m+7): pairs (i, 7-i), then
// xor 1, then xor 2.  Every lane of the 8 ends with the same value, and the
// order of the additions is fixed.
__device__ __forceinline__ uint32_t max8_u32(uint32_t v)
{
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, true));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true));
    return v;
}

__device__ __forceinline__ float sum8_f32(float v)
{
    v += as_f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u(v), 0x141, 0xF, 0xF, true));
    v += as_f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u(v), 0xB1, 0xF, 0xF, true));
    v += as_f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u(v), 0x4E, 0xF, 0xF, true));
    return v;
}

// fp64 sum over the 64 lanes of a wave, fixed order: within each row of 16
// lanes by DPP (xor 1, xor 2, half-row mirror, row mirror; every lane of a
// row ends with the same value), then the four row sums in order.  Valid in
// every lane.
template <int CTRL>
__device__ __forceinline__ double dpp_mov_f64(double v)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, true);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, true);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double wave_sum_f64(double v)
{
    v += dpp_mov_f64<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp_mov_f64<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp_mov_f64<0x141>(v);   // row_half_mirror
    v += dpp_mov_f64<0x140>(v);   // row_mirror
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    double r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 16 * i);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 16 * i);
        r[i] = __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
    }
    return (r[0] + r[1]) + (r[2] + r[3]);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, true));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, true));
    const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)v, 0),
                           (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
    const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)v, 32),
                           (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
    return max(a, b);
}

// ---- tile walk ---------------------------------------------------------

// A tile's place in its matrix, with the matrix's buffers.  The buffers are
// read from the layer table when the tile is chosen, with a wave-uniform
// layer index, so they are scalar loads; read later, inside the tile's
// processing, they were vector loads queued behind the next tile's weight
// loads, and waiting for them drained that prefetch.
struct TileRef {
    const void* w;
    uint8_t* codes;
    float* absmax;
    int8_t* qabsmax;
    float* scale2;
    int64_t local;   // tile index within the layer
    int64_t e0;      // first element of the tile within the layer
    int valid;       // elements of the tile inside the layer (1..16384)
};

__device__ __forceinline__ int first_layer(const LayerDesc* tab, int nl, int64_t tile)
{
    int lo = 0, hi = nl - 1;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (tab[mid].tile_end > tile) hi = mid; else lo = mid + 1;
    }
    return lo;
}

__device__ __forceinline__ TileRef buffers_of(const LayerDesc& d)
{
    TileRef r;
    r.w = d.w;
    r.codes = d.codes;
    r.absmax = d.absmax;
    r.qabsmax = d.qabsmax;
    r.scale2 = d.scale2;
    return r;
}

__device__ __forceinline__ TileRef tile_ref(const LayerDesc* tab, int& l, int64_t tile)
{
    while (tab[l].tile_end <= tile) ++l;
    l = __builtin_amdgcn_readfirstlane(l);
    const LayerDesc& d = tab[l];
    TileRef r = buffers_of(d);
    const int64_t n = d.n;
    r.local = tile - (d.tile_end - tiles_of(n));
    r.e0 = r.local << kTileShift;
    const int64_t rem = n - r.e0;
    r.valid = rem < kTileElems ? (int)rem : kTileElems;
    return r;
}

// ---- fused quantise / double-quantise / dequantise / error --------------

// LDS of the fused kernel.  Everything per block is private to the wave that
// owns the block (wave w: blocks 64 w .. 64 w + 63 of the tile), so a wave
// reads back only what it wrote itself; the one cross-wave value is each
// wave's largest absmax for the double-quant group maximum, double-buffered by
// tile parity so that a wave one tile ahead never overwrites a value another
// wave still reads.
struct CodecShared {
    CodecTables tab;            // copied from kTables (one-shot kernel) or built (tail kernel)
    float ytab[16 * kYStride];  // ytab[c * kYStride + b] = RNE16(level[c] * dequantised absmax of block b)
    uint32_t amax[256];         // block absmax bits (16-bit pattern)
    float r64[256];             // per block: 64 / absmax (of the 2^64-scaled absmax when tiny)
    uint32_t wmax[2][kCWaves];  // per tile parity, per wave: largest absmax bits of the wave's blocks
};

// 16-bit view of LDS words written as halves and read whole
typedef uint16_t __attribute__((may_alias)) u16_alias;

// Per-launch LDS set-up of the fused kernels: the encode cells, and the bf16
// dequant table's lower halves (zero; the tiles write only the upper halves).
__device__ void init_shared(CodecShared& sh)
{
    build_cells(sh.tab.cells);
    if (threadIdx.x < 128) {
        const float mant = 1.0f + (float)threadIdx.x / 128.0f;
        sh.tab.rcp[threadIdx.x] = __builtin_bit_cast(uint32_t, 1.0f / mant);
        sh.tab.d127[threadIdx.x] = __builtin_bit_cast(uint32_t, mant / 127.0f);
    }
    for (int i = threadIdx.x; i < 16 * kYStride; i += kCThreads) sh.ytab[i] = 0.0f;
}

// Step 4 of a tile for one lane: encode, pack and store the codes of its 64
// weights; with ERR also look up each weight's dequantised value in the
// block's table and add up the squared differences in fp32 over the lane's 64
// weights (the caller adds the lanes in fp64).
// SPEC is the rare wave-uniform path for blocks with extreme absmax: the
// weights are scaled by 2^64 before normalising (absmax < 2^-100, keeps 64/a
// finite and leaves the codes unchanged), and each difference is scaled by
// 2^k before squaring so that the fp32 squares neither underflow nor
// overflow (exact; undone in fp64 per block, counted once per 8-lane group).
// FULL: a whole tile (the one-shot kernel); otherwise a matrix's ragged
// last tile (the tail kernel), whose codes past the end are 0 (an odd tail's
// high nibble) and whose bytes past the end are not written.
// NORM (with ERR): also the sum of x^2 over the lane's weights, in the same
// precision and with the same 2^k scaling as the error.
struct LaneSums {
    double err;
    double sq;
};

template <int DT, bool ERR, bool NORM, bool FULL, bool SPEC>
__device__ __forceinline__ LaneSums encode_lane(const CodecShared& sh,
                                                const u32x4 (&v)[kCLoads], g_u8 cp, int valid)
{
    const int lane = threadIdx.x & 63;
    const EncCell* cells = sh.tab.cells + (lane & (kRepl - 1));
    const uint32_t lb = lane_base<kCThreads>();
    // load j covers elements lb + 512 j ..: block (lb >> 6) + 8 j, code bytes
    // (lb >> 1) + 256 j; written as base + constant so that the constants
    // become immediate offsets of the memory instructions
    const uint32_t b0 = lb >> 6, c0 = lb >> 1;
    float e = 0.0f, q = 0.0f;
    double acc64 = 0.0, sq64 = 0.0;
#pragma unroll
    for (int j = 0; j < kCLoads; ++j) {
        const uint32_t o = lb + j * 512u;
        const int bidx = (int)(b0 + 8u * j);
        const float r64 = sh.r64[bidx];
        float scale = 1.0f;
        int ek = 0;
        if constexpr (SPEC) {
            // the rare path recomputes the block's prescale and error scaling
            // from its absmax (the same rule as codec_compute)
            const float a = f16bits_to_f32<DT>(sh.amax[bidx]);
            scale = (a > 0.0f && a < 0x1p-100f) ? 0x1p64f : 1.0f;
            ek = (ERR && a > 0.0f && (a < 0x1p-40f || a >= 0x1p40f)) ? 1 - __builtin_amdgcn_frexp_expf(a) : 0;
        }
        const uint32_t dw[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
        uint32_t cd[8];
        float eb = 0.0f, qb = 0.0f;
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2) {
            float x[2];
            unpack2<DT>(dw[k2], x[0], x[1]);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float u = (SPEC ? x[h] * scale : x[h]) * r64;
                const EncCell c = cells[((int)u + 64) * kRepl];
                uint32_t code = c.base + (u > c.thr ? 1u : 0u);
                if constexpr (ERR) {
                    float dd = x[h] - sh.ytab[__umul24(code, (uint32_t)kYStride) + (uint32_t)bidx];
                    if constexpr (SPEC) {
                        dd = __builtin_amdgcn_ldexpf(dd, ek);
                        eb = __builtin_fmaf(dd, dd, eb);
                    } else {
                        e = __builtin_fmaf(dd, dd, e);
                    }
                }
                if constexpr (NORM) {
                    if constexpr (SPEC) {
                        const float xs = __builtin_amdgcn_ldexpf(x[h], ek);
                        qb = __builtin_fmaf(xs, xs, qb);
                    } else {
                        q = __builtin_fmaf(x[h], x[h], q);
                    }
                }
                cd[2 * k2 + h] = code;
            }
        }
        // element 2m in the low nibble of byte m: a shift-and-or per pair, then
        // byte permutes (7 instructions per 8 codes)
        const uint32_t b0 = cd[0] | (cd[1] << 4), b1 = cd[2] | (cd[3] << 4);
        const uint32_t b2 = cd[4] | (cd[5] << 4), b3 = cd[6] | (cd[7] << 4);
        const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);   // b0, b1, 0, 0
        const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);   // b2, b3, 0, 0
        uint32_t pk = __builtin_amdgcn_perm(hi, lo, 0x05040100u);   // b0, b1, b2, b3
        if constexpr (FULL) {
            store_stream(pk, (g_u32)(cp + (c0 + 256u * j)));
        } else {
            const int rem = valid - (int)o;
            if (rem >= 8) {
                *(g_u32)(cp + (o >> 1)) = pk;
            } else if (rem > 0) {
                pk &= (1u << (4 * rem)) - 1u;
#pragma unroll
                for (int bb = 0; bb < 4; ++bb)
                    if (2 * bb < rem) cp[(o >> 1) + bb] = (uint8_t)(pk >> (8 * bb));
            }
        }
        if constexpr (ERR && SPEC) {
            const double blk_sse = __builtin_ldexp((double)sum8_f32(eb), -2 * ek);
            if ((lane & 7) == 0) acc64 += blk_sse;
        }
        if constexpr (NORM && SPEC) {
            const double blk_sq = __builtin_ldexp((double)sum8_f32(qb), -2 * ek);
            if ((lane & 7) == 0) sq64 += blk_sq;
        }
        // keep the scheduler from hoisting the next group's lookups (register pressure)
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (ERR && !SPEC) acc64 = (double)e;
    if constexpr (NORM && !SPEC) sq64 = (double)q;
    return LaneSums{acc64, sq64};
}

// 1. the tile's weights into registers: 8 x 128-bit loads per lane.  In a
// ragged last tile a lane loads only chunks that start inside the matrix and
// zeroes the elements past its end.  Such a chunk is 16-byte aligned (the
// weights are) and holds a valid element, so it lies within one mapped page;
// the bytes past the end are read and discarded.  Padding with zeros leaves
// every block maximum unchanged and adds nothing to the error (0 encodes to
// level 0, which dequantises to 0).
template <bool FULL>
__device__ __forceinline__ void load_tile(u32x4 (&v)[kCLoads], const TileRef& tr)
{
    const g_cu16 w = (g_cu16)tr.w + tr.e0;
    const int valid = tr.valid;
    const uint32_t lb = lane_base<kCThreads>();
    if constexpr (FULL) {
        // a uniform base plus a 32-bit lane offset plus an immediate: no 64-bit
        // address arithmetic per load
        const GLOBAL uint8_t* wb = (const GLOBAL uint8_t*)w;
#pragma unroll
        for (int j = 0; j < kCLoads; ++j) v[j] = load_stream((g_cu4)(wb + (2u * lb + 1024u * j)));
    } else {
#pragma unroll
        for (int j = 0; j < kCLoads; ++j) {
            const uint32_t o = lb + j * 512u;
            const int rem = valid - (int)o;
            u32x4 c = {0u, 0u, 0u, 0u};
            if (rem > 0) {
                c = *(g_cu4)(w + o);
                if (rem < 8) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const uint32_t keep = rem >= 2 * k + 2 ? ~0u : (rem == 2 * k + 1 ? 0xffffu : 0u);
                        c[k] &= keep;
                    }
                }
            }
            v[j] = c;
        }
    }
}

template <int DT, bool DQ, bool ERR, bool NORM, bool FULL>
__device__ __forceinline__ void codec_compute(CodecShared& sh, const u32x4 (&v)[kCLoads],
                                              const TileRef& tr, int64_t tile, int parity,
                                              double* __restrict__ partial,
                                              double* __restrict__ partial_sq)
{
    // the wave index as a scalar (wave-uniform): no vector register held for it
    const int t = threadIdx.x, lane = t & 63, wv = __builtin_amdgcn_readfirstlane(t >> 6);
    const TileRef& d = tr;
    const int valid = tr.valid;

    // 2. block absmax (exact: a max of representable values), and the wave's
    //    largest for the double-quant group maximum
    const uint32_t b0 = lane_base<kCThreads>() >> 6;   // block of load j: b0 + 8 j
    uint32_t m[kCLoads], wm = 0;
#pragma unroll
    for (int j = 0; j < kCLoads; ++j) {
        m[j] = max8_u32(absmax_bits8_f16ops(v[j]));
        wm = max(wm, m[j]);
    }
    if (DQ || DT == 0) wm = wave_max_u32(wm);
    if (DT == 0 && wm >= 0x7c00u) {   // a bf16 |x| >= 2^121 somewhere in the wave's blocks
        wm = 0;
#pragma unroll
        for (int j = 0; j < kCLoads; ++j) {
            m[j] = max8_u32(absmax_bits8(v[j]));
            wm = max(wm, m[j]);
        }
        wm = wave_max_u32(wm);
    }
#pragma unroll
    for (int j = 0; j < kCLoads; ++j)
        if ((lane & 7) == 0) sh.amax[b0 + 8u * j] = m[j];
    if constexpr (DQ) {
        if (lane == 0) sh.wmax[parity][wv] = wm;
        __syncthreads();   // the only workgroup barrier of a tile
    }

    // 3. constants of the wave's 64 blocks: lane L owns block b = 64 w + L = t
    const uint32_t a16 = sh.amax[t];
    const float a = f16bits_to_f32<DT>(a16);
    float adq = a;
    float qk = 0.0f;
    float s2 = 0.0f;
    if constexpr (DQ) {
        uint32_t g = sh.wmax[parity][0];
#pragma unroll
        for (int i = 1; i < kCWaves; ++i) g = max(g, sh.wmax[parity][i]);
        g = __builtin_amdgcn_readfirstlane(g);
        const float G = f16bits_to_f32<DT>(g);
        if (G > 0.0f) {
            if (DT == 0 && G >= 0x1p-100f) {
                // scale2 = fl32(G/127) from the mantissa table; q = rint(fl32(a /
                // scale2)): z = a * rcp(scale2) is within 2^-14 of fl32(a / scale2)
                // (both within a few ulp of a / scale2 <= 127.5), so unless z lies
                // within 2^-10 of a half-integer both round to the same integer;
                // the lanes that do divide exactly.
                s2 = __builtin_amdgcn_ldexpf(as_f(sh.tab.d127[g & 127u]), (int)(g >> 7) - 127);
                const float z = a * __builtin_amdgcn_rcpf(s2);
                qk = rintf(z);
                const bool near = __builtin_fabsf(z - qk) > 0.5f - 0x1p-10f;
                if (__builtin_amdgcn_ballot_w64(near) != 0 && near) qk = rintf(a / s2);
            } else {
                s2 = G / 127.0f;
                qk = rintf(a / s2);
            }
            // a <= G, so fl32(a / scale2) < 127.5: the int8 clamp to +-127 never applies
            adq = qk * s2;
        } else {
            adq = 0.0f;
        }
    }
    // normalisation s = fl32(x * fl32(1/a)); carried as u = 64 s = x * (64/a).
    // bf16 a in [2^-40, 2^40): fl32(1/a) = 2^-e rcp[m] exactly (a = 2^e (1 + m/128));
    // the rest (rare) divides, with the prescale and error scaling below.
    float r64 = 0.0f, pre = 1.0f;
    int ek = 0;
    const bool usual = DT == 0 ? (a16 - 0x2b80u < 0x2800u) : true;   // bf16 exponent field 87..166
    if (usual) {
        if constexpr (DT == 0)
            r64 = __builtin_amdgcn_ldexpf(as_f(sh.tab.rcp[a16 & 127u]), 133 - (int)(a16 >> 7));
        else
            r64 = a > 0.0f ? (1.0f / a) * 64.0f : 0.0f;
    } else if (a > 0.0f) {
        if (a < 0x1p-100f) {   // keeps 64/a finite; for normal a the codes are unchanged
            pre = 0x1p64f;
            r64 = (1.0f / (a * 0x1p64f)) * 64.0f;
        } else {
            r64 = (1.0f / a) * 64.0f;
        }
        if (ERR && (a < 0x1p-40f || a >= 0x1p40f)) ek = 1 - __builtin_amdgcn_frexp_expf(a);
    }
    sh.r64[t] = r64;
    if constexpr (ERR) {
        // the block's 16 dequantised values, rounded to the 16-bit type, back in
        // fp32.  A bf16 value is the upper half of its fp32 pattern, so for bf16
        // only the upper halves are written (the lower halves stay zero from
        // init_shared) and no conversion back is needed.
#pragma unroll
        for (int c = 0; c < 16; c += 2) {
            float y0, y1;
            // level 7 is 0 (its entries stay zero for bf16), levels 0 and 15 are -1 and +1
            const float p1 = c + 1 == 7 ? 0.0f : as_f(nf4fmt::kLevelBits[c + 1]) * adq;
            const uint32_t p = round_pair<DT>(as_f(nf4fmt::kLevelBits[c]) * adq, p1, y0, y1);
            if constexpr (DT == 0) {
                u16_alias* yt = reinterpret_cast<u16_alias*>(sh.ytab);
                yt[2 * (c * kYStride + t) + 1] = (uint16_t)p;
                if (c + 1 != 7) yt[2 * ((c + 1) * kYStride + t) + 1] = (uint16_t)(p >> 16);
            } else {
                sh.ytab[c * kYStride + t] = y0;
                sh.ytab[(c + 1) * kYStride + t] = y1;
            }
        }
    }
    {
        const int nbv = (valid + 63) >> 6;
        const int64_t b = (tr.e0 >> 6) + t;
        if (t < nbv) {
            if (d.absmax) ((g_f32)d.absmax)[b] = a;
            if constexpr (DQ) ((g_i8)d.qabsmax)[b] = (int8_t)(int)qk;
        }
        if constexpr (DQ) {
            if (t == 0) ((g_f32)d.scale2)[tr.local] = s2;
        }
    }
    // the wave reads back only its own blocks' constants: LDS keeps a wave's
    // accesses in order, no barrier needed
    const bool any_spec = __builtin_amdgcn_ballot_w64(pre != 1.0f || ek != 0) != 0;

    // 4. encode, pack, store codes; look up the dequantised values and square the error
    const g_u8 cp = (g_u8)d.codes + (tr.e0 >> 1);
    const LaneSums acc = any_spec ? encode_lane<DT, ERR, NORM, FULL, true>(sh, v, cp, valid)
                                  : encode_lane<DT, ERR, NORM, FULL, false>(sh, v, cp, valid);

    // 5. the wave's fp64 partial (64 lanes in a fixed order); tiles and waves
    //    are added per layer by k_reduce
    if constexpr (ERR) {
        const double acc64 = wave_sum_f64(acc.err);
        if (lane == 0) partial[tile * kPartsPerTile + wv] = acc64;
    }
    if constexpr (NORM) {
        const double sq64 = wave_sum_f64(acc.sq);
        if (lane == 0) partial_sq[tile * kPartsPerTile + wv] = sq64;
    }
}

// Where a tile of the one-shot fused kernel lies: its matrix and its index in
// it.  Written by k_codec_prep, one thread per tile (binary search over the
// layer table), and read by the tile's workgroup with scalar loads.
struct alignas(8) CodecTile {
    int32_t layer;
    int32_t local;
};

__global__ __launch_bounds__(kThreads) void k_codec_prep(const LayerDesc* __restrict__ tab, int nl,
                                                         int64_t ntiles, CodecTile* __restrict__ rec)
{
    const int64_t tile = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (tile >= ntiles) return;
    const int l = first_layer(tab, nl, tile);
    const LayerDesc& d = tab[l];
    rec[tile] = CodecTile{l, (int32_t)(tile - (d.tile_end - tiles_of(d.n)))};
}

// LDS set-up of a one-shot workgroup: the encode cells copied from the
// constant table (16 bytes per lane and load), and for bf16 the dequant
// table's lower halves cleared (the tile writes only the upper halves).
// The copy's loads are issued before the tile's weight loads, so that their
// LDS writes wait only for them (memory operations complete in order).
__device__ __forceinline__ void load_tables(u32x4 (&c)[kCopyRounds])
{
    const GLOBAL u32x4* src = (const GLOBAL u32x4*)(const void*)&kTables;
#pragma unroll
    for (int r = 0; r < kCopyRounds; ++r) c[r] = src[threadIdx.x + r * kCThreads];
}

// The tables into LDS, and for bf16 the dequant table's lower halves cleared
// (the tile writes only the upper halves).  The copy's last round writes the
// constant's zero padding over the start of the dequant table; the clearing
// covers the rest of it.
template <int DT>
__device__ __forceinline__ void store_tables(CodecShared& sh, const u32x4 (&c)[kCopyRounds])
{
    constexpr int kCleared = kCopyRounds * kCopyRound - (int)sizeof(CodecTables);
    static_assert(offsetof(CodecShared, ytab) == sizeof(CodecTables), "the dequant table follows the tables");
    static_assert(kCleared % 16 == 0 && kCleared <= (int)sizeof(float) * 16 * kYStride,
                  "the copy's padding lands inside the dequant table");
    const uint32_t t = threadIdx.x;
    u32x4* dst = reinterpret_cast<u32x4*>(&sh.tab);
#pragma unroll
    for (int r = 0; r < kCopyRounds; ++r) dst[t + r * kCThreads] = c[r];
    if constexpr (DT == 0) {
        constexpr int kChunks = ((int)sizeof(float) * 16 * kYStride - kCleared) / 16;
        constexpr int kZr = kChunks / kCThreads;
        static_assert(((int)sizeof(float) * 16 * kYStride - kCleared) % 16 == 0, "16-byte units");
        u32x4* y = reinterpret_cast<u32x4*>(reinterpret_cast<char*>(sh.ytab) + kCleared);
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int r = 0; r < kZr; ++r) y[t + r * kCThreads] = z;
        if (t < (uint32_t)(kChunks - kZr * kCThreads)) y[t + kZr * kCThreads] = z;
    }
}

// The fused pass, one workgroup per tile (a one-shot grid): the dispatcher
// hands tiles out in index order, so the tiles in flight stay one compact run
// of memory, and a CU's resident workgroups overlap one another's loads with
// their arithmetic.  Measured against the persistent walk it replaced (one
// tile prefetched in registers) with the same per-weight arithmetic: a stream
// of 32 KB read and 8 KB written per tile with 14 fp32 operations per weight
// took 6.47 ms persistent and 5.35 ms one-shot over the 14B stack's 774,400
// tiles.  A matrix's ragged last tile is left to k_codec_tail.
template <int DT, bool DQ, bool ERR, bool NORM>
__global__ __launch_bounds__(kCThreads, ERR ? kCodecWavesPerEu : kQuantWavesPerEu) void k_codec(
    const LayerDesc* __restrict__ tab, const CodecTile* __restrict__ rec, int64_t first_tile,
    double* __restrict__ partial, double* __restrict__ partial_sq)
{
    __shared__ CodecShared sh;
    const int64_t tile = first_tile + blockIdx.x;
    const CodecTile r = rec[tile];
    const LayerDesc d = tab[r.layer];   // every field at once: one round of scalar loads
    const int64_t e0 = (int64_t)r.local << kTileShift;
    if (d.n - e0 < kTileElems) return;   // uniform: the workgroup leaves together
    TileRef tr = buffers_of(d);
    tr.local = r.local;
    tr.e0 = e0;
    tr.valid = kTileElems;
    u32x4 c[kCopyRounds], v[kCLoads];
    load_tables(c);
    load_tile<true>(v, tr);
    store_tables<DT>(sh, c);
    __syncthreads();
    codec_compute<DT, DQ, ERR, NORM, true>(sh, v, tr, tile, 0, partial, partial_sq);
}

// The ragged last tile of matrix blockIdx.x (n not a multiple of 16384),
// launched after k_codec on the same stream; other workgroups exit at once.
template <int DT, bool DQ, bool ERR, bool NORM>
__global__ __launch_bounds__(kCThreads) void k_codec_tail(const LayerDesc* __restrict__ tab,
                                                          double* __restrict__ partial,
                                                          double* __restrict__ partial_sq)
{
    const int64_t n = tab[blockIdx.x].n;
    if ((n & (kTileElems - 1)) == 0) return;
    __shared__ CodecShared sh;
    init_shared(sh);
    __syncthreads();
    int l = blockIdx.x;
    const int64_t tile = tab[l].tile_end - 1;
    const TileRef tr = tile_ref(tab, l, tile);
    u32x4 v[kCLoads];
    load_tile<false>(v, tr);
    codec_compute<DT, DQ, ERR, NORM, false>(sh, v, tr, tile, 0, partial, partial_sq);
}

// ---- standalone dequantisation -------------------------------------------

constexpr int kDqSplit = 8;          // workgroups per tile in the standalone dequantisation
constexpr int kDqThreads = 64;       // threads per dequantisation workgroup (4 stores each)
constexpr int kDqElems = kTileElems / kDqSplit;       // weights per workgroup
constexpr int kDqSteps = kDqElems / (kDqThreads * 8); // 16-byte stores per thread
static_assert(kDqSteps >= 1 && kDqSteps * kDqThreads * 8 * kDqSplit == kTileElems, "dequant split");


// Per-tile descriptor, built by k_dq_prep in the workspace before the
// dequantisation: everything a workgroup needs about its tile in one 32-byte
// record, read with scalar loads (no layer search in the hot kernel).
struct alignas(32) DqTile {
    const uint8_t* codes;   // the tile's first code byte
    uint16_t* out;          // the tile's first output element
    const void* cst;        // the tile's first int8 qabsmax, or fp32 absmax
    float s2;               // the tile's scale2 (double quant), else unused
    int32_t valid;          // elements of the tile inside the layer (1..16384)
};
static_assert(sizeof(DqTile) == kPartsPerTile * sizeof(double), "a record fits a tile's partials");

// One thread per tile: find the layer (binary search over tile_end), write the
// record.  skip (device, one byte per layer, may be null): a layer with a
// nonzero byte gets valid = 0 in every record, so its units do nothing and its
// output is not touched.
template <bool DQ>
__global__ __launch_bounds__(kThreads) void k_dq_prep(const LayerDesc* __restrict__ tab, int nl,
                                                      int64_t ntiles, const uint8_t* __restrict__ skip,
                                                      DqTile* __restrict__ desc)
{
    const int64_t tile = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (tile >= ntiles) return;
    const int l = first_layer(tab, nl, tile);
    const LayerDesc& d = tab[l];
    const int64_t local = tile - (d.tile_end - tiles_of(d.n));
    const int64_t e0 = local << kTileShift;
    const int64_t rem = d.n - e0;
    DqTile r;
    r.codes = d.codes + (e0 >> 1);
    r.out = (uint16_t*)d.out + e0;
    if constexpr (DQ) {
        r.cst = d.qabsmax + (e0 >> 6);
        r.s2 = ((g_cf32)d.scale2)[local];
    } else {
        r.cst = d.absmax + (e0 >> 6);
        r.s2 = 0.0f;
    }
    r.valid = rem < kTileElems ? (int32_t)rem : kTileElems;
    if (skip && skip[l]) r.valid = 0;
    desc[tile] = r;
}

// A unit = 1/kDqSplit of a tile, one workgroup of T = kDqThreads threads.
// Step j of thread t covers the 8 weights at 8 (T j + t) of the unit, so at
// every step the workgroup writes one contiguous 16 T-byte run of output; the
// 8 lanes 8m..8m+7 of a step share a block, whose constant each lane loads
// itself (the same byte or word for the 8 lanes).  Measured on the 14B-shaped
// stack in one process (bitwise equal outputs): one 256-thread workgroup per
// tile with 8 stores per thread and a layer search 5.92 ms; from a tile
// record, 256 threads: quarter tiles 5.35 ms, half 5.59, eighth 7.92; quarter
// tiles from a tile-to-layer map and the layer table 5.60 ms; 128 threads:
// quarter tiles (4 stores per thread) 5.07 ms, half 5.99, whole 6.00; 64
// threads: eighth tiles (4 stores) 5.07, quarter 5.97, sixteenth 5.67; 512
// threads: half 5.41, quarter 7.70; an XCD-contiguous unit order changed
// nothing.  With non-temporal output stores: 64 threads over eighth tiles
// 4.855 ms, 128 over quarters 4.885, 128 over eighths 5.29, 256 over halves
// 5.36, 128 over halves 5.96.  What made the small workgroups pay off at all was issuing every
// load of a whole unit at once: with the constant load behind a bounds guard
// each load was waited for in its own branch, and quarter tiles took 7.2 ms.
template <int DT, bool DQ>
__device__ __forceinline__ void dequant_unit(const float* s_lv, const DqTile& r, int sub)
{
    const int valid = r.valid - sub * kDqElems;
    if (valid <= 0) return;   // past the end of a ragged last tile (the whole workgroup)
    const g_cu8 cp = (g_cu8)r.codes + sub * (kDqElems / 2);
    const g_u16 outp = (g_u16)r.out + (int64_t)sub * kDqElems;
    const int b0 = sub * (kDqElems / 64);
    const uint32_t t = threadIdx.x;
    const bool full = valid >= kDqElems;
    uint32_t c32[kDqSteps];
    float k[kDqSteps];
    if (full) {
        // unconditional loads, all in flight at once (a guarded load would be
        // waited for inside its branch)
        int32_t qi[kDqSteps];
#pragma unroll
        for (int j = 0; j < kDqSteps; ++j) {
            const uint32_t o = 8u * (j * (uint32_t)kDqThreads + t);
            c32[j] = *(g_cu32)(cp + (o >> 1));
            if constexpr (DQ) qi[j] = ((g_ci8)r.cst)[b0 + (o >> 6)];
            else              k[j] = ((g_cf32)r.cst)[b0 + (o >> 6)];
        }
        if constexpr (DQ) {
#pragma unroll
            for (int j = 0; j < kDqSteps; ++j) k[j] = (float)qi[j];
        }
    } else {
#pragma unroll
        for (int j = 0; j < kDqSteps; ++j) {
            const uint32_t o = 8u * (j * (uint32_t)kDqThreads + t);
            uint32_t c = 0;
#pragma unroll
            for (int bb = 0; bb < 4; ++bb)
                if (o + 2 * bb < (uint32_t)valid) c |= (uint32_t)cp[(o >> 1) + bb] << (8 * bb);
            c32[j] = c;
            const bool in = o < (uint32_t)valid;
            if constexpr (DQ) k[j] = in ? (float)((g_ci8)r.cst)[b0 + (o >> 6)] : 0.0f;
            else              k[j] = in ? ((g_cf32)r.cst)[b0 + (o >> 6)] : 0.0f;
        }
    }
    __builtin_amdgcn_wave_barrier();   // the wave's table writes precede its reads (LDS keeps a wave's order)
#pragma unroll
    for (int j = 0; j < kDqSteps; ++j) {
        const uint32_t o = 8u * (j * (uint32_t)kDqThreads + t);
        const float adq = DQ ? k[j] * r.s2 : k[j];
        uint32_t p[4];
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2) {
            const float y0 = s_lv[(c32[j] >> (8 * k2)) & 15] * adq;
            const float y1 = s_lv[(c32[j] >> (8 * k2 + 4)) & 15] * adq;
            float r0, r1;
            p[k2] = round_pair<DT>(y0, y1, r0, r1);
        }
        if (full) {
            u32x4 pv = {p[0], p[1], p[2], p[3]};
            store_stream(pv, (g_u4)(outp + o));
        } else {
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
                if (o + kk < (uint32_t)valid) outp[o + kk] = (uint16_t)(p[kk >> 1] >> (16 * (kk & 1)));
        }
    }
}

// One workgroup per unit, a one-shot grid: the dispatcher hands out units in
// index order, so the units in flight stay one compact run of memory for the
// whole launch (persistent workgroups drift apart and spread their stores).
// Each wave keeps its own copy of the level table, so the waves never wait
// for each other.
template <int DT, bool DQ>
__global__ __launch_bounds__(kDqThreads) void k_dequant(const DqTile* __restrict__ desc, int64_t first_unit)
{
    __shared__ float s_lv[kDqThreads / 64][16];
    const int lane = threadIdx.x & 63;
    float* lv = s_lv[threadIdx.x >> 6];
    if (lane < 16) {
        // from immediates: a load of the table would be waited for before the first data load
        float v = as_f(nf4fmt::kLevelBits[0]);
#pragma unroll
        for (int i = 1; i < 16; ++i) v = lane == i ? as_f(nf4fmt::kLevelBits[i]) : v;
        lv[lane] = v;
    }
    const int64_t unit = first_unit + blockIdx.x;
    const int64_t tile = unit / kDqSplit;
    const DqTile r = desc[tile];   // uniform: scalar loads
    dequant_unit<DT, DQ>(lv, r, (int)(unit - tile * kDqSplit));
}

// ---- standalone double quantisation --------------------------------------

// One wave per double-quant group (256 blocks, a tile), four groups per
// workgroup, a one-shot grid: lane L takes blocks L + 64 k (k = 0..3), so each
// load and store instruction of the wave covers one contiguous run; the group
// maximum is a wave maximum, with no workgroup barrier.  The arithmetic is
// that of the fused pass's exact-division path: s2 = fl32(G / 127), q =
// rint(fl32(a / s2)) clamped to +-127 (a <= G, so the clamp never applies).
constexpr int kDqGroupsPerWg = kThreads / 64;

__global__ __launch_bounds__(kThreads) void k_double_quant(const LayerDesc* __restrict__ tab,
                                                           int nl, int64_t ntiles)
{
    const int64_t tile = (int64_t)blockIdx.x * kDqGroupsPerWg + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (tile >= ntiles) return;   // the whole wave
    const int lane = threadIdx.x & 63;
    int l = first_layer(tab, nl, tile);
    const TileRef tr = tile_ref(tab, l, tile);
    const int nbv = (tr.valid + 63) >> 6;
    const int64_t b0 = tr.e0 >> 6;
    float a[4];
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int b = lane + 64 * k;
        a[k] = b < nbv ? ((g_cf32)tr.absmax)[b0 + b] : 0.0f;
        m = max(m, as_u(a[k]));   // absmax >= 0: the integer order is the numeric order
    }
    const float G = as_f(wave_max_u32(m));
    const float s2 = G > 0.0f ? G / 127.0f : 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int b = lane + 64 * k;
        int8_t q = 0;
        if (G > 0.0f) {
            float qf = rintf(a[k] / s2);
            qf = fminf(fmaxf(qf, -127.0f), 127.0f);
            q = (int8_t)qf;
        }
        if (b < nbv) ((g_i8)tr.qabsmax)[b0 + b] = q;
    }
    if (lane == 0) ((g_f32)tr.scale2)[tr.local] = s2;
}

// ---- per-layer reduction of the tile partials -----------------------------

__global__ __launch_bounds__(kThreads) void k_reduce(const LayerDesc* __restrict__ tab,
                                                     const double* __restrict__ partial,
                                                     double* __restrict__ err)
{
    __shared__ double s[kThreads];
    const int l = blockIdx.x, t = threadIdx.x;
    const int64_t end = tab[l].tile_end * kPartsPerTile;
    const int64_t begin = end - tiles_of(tab[l].n) * kPartsPerTile;
    double acc = 0.0;
    for (int64_t i = begin + t; i < end; i += kThreads) acc += partial[i];
    s[t] = acc;
    __syncthreads();
    for (int h = kThreads / 2; h >= 1; h >>= 1) {
        if (t < h) s[t] = s[t] + s[t + h];
        __syncthreads();
    }
    if (t == 0) err[l] = s[0];
}

// ---- launch helpers -------------------------------------------------------

// One-shot launches of at most kMaxGrid workgroups (the dispatch packet counts
// work-items in 32 bits).
constexpr int64_t kMaxGrid = (int64_t(1) << 32) / kThreads - 1;

template <int DT, bool DQ, bool ERR, bool NORM>
hipError_t codec_go(const LayerDesc* tab, int nl, int64_t ntiles, bool ragged, void* rec_ws,
                    double* partial, double* partial_sq, hipStream_t s)
{
    CodecTile* rec = static_cast<CodecTile*>(rec_ws);
    if (ntiles > kMaxGrid * kThreads) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_codec_prep, dim3((unsigned)((ntiles + kThreads - 1) / kThreads)), dim3(kThreads),
                       0, s, tab, nl, ntiles, rec);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    for (int64_t t0 = 0; t0 < ntiles; t0 += kMaxGrid) {
        const int64_t g = ntiles - t0 < kMaxGrid ? ntiles - t0 : kMaxGrid;
        hipLaunchKernelGGL((k_codec<DT, DQ, ERR, NORM>), dim3((unsigned)g), dim3(kCThreads), 0, s, tab,
                           (const CodecTile*)rec, t0, partial, partial_sq);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (!ragged) return hipSuccess;
    hipLaunchKernelGGL((k_codec_tail<DT, DQ, ERR, NORM>), dim3((unsigned)nl), dim3(kCThreads), 0, s,
                       tab, partial, partial_sq);
    return hipGetLastError();
}

template <int DT, bool DQ>
hipError_t dequant_go(const LayerDesc* tab, int nl, int64_t ntiles, const uint8_t* skip, void* desc_ws,
                      hipStream_t s)
{
    DqTile* desc = static_cast<DqTile*>(desc_ws);
    if (ntiles > kMaxGrid * kThreads) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_dq_prep<DQ>), dim3((unsigned)((ntiles + kThreads - 1) / kThreads)), dim3(kThreads),
                       0, s, tab, nl, ntiles, skip, desc);
    hipError_t e0 = hipGetLastError();
    if (e0 != hipSuccess) return e0;
    const int64_t nunits = ntiles * kDqSplit;
    constexpr int64_t kMaxDqGrid = (int64_t(1) << 32) / kDqThreads - 1;
    for (int64_t t0 = 0; t0 < nunits; t0 += kMaxDqGrid) {
        const int64_t g = nunits - t0 < kMaxDqGrid ? nunits - t0 : kMaxDqGrid;
        hipLaunchKernelGGL((k_dequant<DT, DQ>), dim3((unsigned)g), dim3(kDqThreads), 0, s,
                           (const DqTile*)desc, t0);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_codec(const LayerDesc* tab, int nl, int64_t ntiles, bool ragged, int dtype,
                        bool dq, void* rec_ws, double* err_partial, double* sq_partial, hipStream_t s)
{
    // err_partial: the error; sq_partial (only with err_partial): also the sum of squares
    const int mode = !err_partial ? 0 : (!sq_partial ? 1 : 2);
#define NF4_CODEC_GO(DT, DQ)                                                                           \
    (mode == 0 ? codec_go<DT, DQ, false, false>(tab, nl, ntiles, ragged, rec_ws, nullptr, nullptr, s)   \
     : mode == 1 ? codec_go<DT, DQ, true, false>(tab, nl, ntiles, ragged, rec_ws, err_partial, nullptr, s) \
                 : codec_go<DT, DQ, true, true>(tab, nl, ntiles, ragged, rec_ws, err_partial, sq_partial, s))
    if (dtype == 0) return dq ? NF4_CODEC_GO(0, true) : NF4_CODEC_GO(0, false);
    return dq ? NF4_CODEC_GO(1, true) : NF4_CODEC_GO(1, false);
#undef NF4_CODEC_GO
}

hipError_t launch_reduce(const LayerDesc* tab, int nl, const double* partial, double* err,
                         hipStream_t s)
{
    hipLaunchKernelGGL(k_reduce, dim3((unsigned)nl), dim3(kThreads), 0, s, tab, partial, err);
    return hipGetLastError();
}

hipError_t launch_dequant(const LayerDesc* tab, int nl, int64_t ntiles, int dtype, bool dq,
                          const uint8_t* skip, void* desc_ws, hipStream_t s)
{
    if (dtype == 0) return dq ? dequant_go<0, true>(tab, nl, ntiles, skip, desc_ws, s)
                              : dequant_go<0, false>(tab, nl, ntiles, skip, desc_ws, s);
    return dq ? dequant_go<1, true>(tab, nl, ntiles, skip, desc_ws, s)
              : dequant_go<1, false>(tab, nl, ntiles, skip, desc_ws, s);
}

hipError_t launch_double_quant(const LayerDesc* tab, int nl, int64_t ntiles, hipStream_t s)
{
    const int64_t grid = (ntiles + kDqGroupsPerWg - 1) / kDqGroupsPerWg;
    if (grid > kMaxGrid) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_double_quant, dim3((unsigned)grid), dim3(kThreads), 0, s, tab, nl, ntiles);
    return hipGetLastError();
}

}  // namespace nf4k
