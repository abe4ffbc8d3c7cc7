// k_gemm.hip -- NF4 dequantisation fused into the 16-bit matmul that consumes
// the weight, on gfx950 matrix cores (MFMA).
//
// QLoRA keeps the frozen weight in 4 bits and dequantises it on the fly for
// the forward and the backward pass ("QLoRA" paper summary page, How It
// Works); AQLoRA names that per-step dequantisation as where quantised
// fine-tuning loses its time (AQLoRA arXiv listing, English abstract).  Here
// every weight is dequantised on chip, to the value the codec defines
// (y = RNE16(fl32(level[code] * dequantised absmax)), bitwise what
// nf4_dequantize writes), and multiplied there: the 16-bit weight never goes
// to HBM.
//
//   forward   out[m, n] = sum_k x[m, k] * W[n, k]      (x: m x cols, out: m x rows)
//   backward  out[m, k] = sum_n x[m, n] * W[n, k]      (x: m x rows, out: m x cols)
//
// Products of two bf16 (or fp16) values are exact in fp32; only the fp32
// accumulation rounds.  Four kernels, chosen by m and direction:
//   * m > 128: 256 x 256 output tiles, one workgroup of four waves per CU
//     (k_nf4_mm_fwd: the weight fragments dequantised straight into MFMA
//     registers; k_nf4_mm_bwd: each wave's weight piece transposed through LDS
//     with the transposing read).  Tiles left over after the last whole round
//     run as 64-row quarters, or 128-row halves, when those fit one round;
//     with a workspace their reduction is split instead (fp32 partial blocks
//     added in split order by k_tail_sum), and with few tiles and a workspace
//     every tile's reduction is split (k_splitk_sum adds the splits).
//   * m <= 128 (and any split reduction): k_nf4_matmul, 128 x 128 tiles, three
//     workgroups per CU, the weight tile dequantised into LDS (transposed on
//     the way backward).
//   * forward with m <= 32 and a workspace: k_nf4_gemv16, one wave per 16
//     weight rows on the 16 x 16 x 32 MFMA.
//
// k_nf4_matmul: the first operand A is row-major with the reduction index
// contiguous (x, or the output gradient); the W tile is stored in LDS with the
// reduction index contiguous too -- in W's own order forward, transposed
// backward -- so the MFMA fragment reads are the same.  A 256-thread
// workgroup computes a 128 x 128 output tile in k-steps of 64 (one
// quantisation block of a W row forward); waves in a 2 x 2 grid, each
// 64 x 64 = 2 x 2 tiles of v_mfma_f32_32x32x16_bf16.  The next step's A rows
// and W codes are loaded into registers (raw: no wait) while the current step
// multiplies; after a barrier they are dequantised into the single LDS
// buffer.  39 KB of LDS per workgroup lets 3 workgroups share a CU.  Level
// lookups read a 256-entry table of level pairs (one 8-byte read per code
// byte).  Tiles are handed out in groups of 4 row tiles, each XCD taking a
// contiguous run of that order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "nf4_format.h"
#include "nf4_internal.h"
#include "nf4_launch.h"

namespace nf4k {
namespace {

constexpr int kGThreads = 256;
constexpr int kWM = 64, kWN = 64;  // output rows and columns per wave
constexpr int kTM = kWM / 32, kTN = kWN / 32;   // 32 x 32 MFMA tiles per wave
constexpr int kBM = 2 * kWM;      // output rows (of x) per workgroup
constexpr int kBN = 2 * kWN;      // output columns per workgroup
constexpr int kBK = 64;           // reduction step
constexpr int kAChunks = kBM / 32;   // 16-byte A chunks per thread and step
constexpr int kWPass = kBN / 128;    // W passes per thread and step
static_assert(kBN % 128 == 0 && kBM % 32 == 0, "tile shape");
constexpr int kLdp = kBK + 8;     // LDS row pitch in 16-bit elements (144 B: conflict-free 16-B reads)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define GLOBAL __attribute__((address_space(1)))

__device__ __forceinline__ float as_f(uint32_t u) { return __builtin_bit_cast(float, u); }

// Keeps a product from being fused with its conversion to fp16 (v_fma_mix*
// rounds the exact product once; the format rounds to fp32 first).
__device__ __forceinline__ float opaque(float x)
{
    __asm__ volatile("" : "+v"(x));
    return x;
}

// Two fp32 values rounded to the 16-bit type DT (0 bf16, 1 fp16; nearest,
// ties to even), packed low first.
template <int DT>
__device__ __forceinline__ uint32_t pack16(float y0, float y1)
{
    if constexpr (DT == 0) {
        f2 in = {y0, y1};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(in, bf2));
    } else {
        const _Float16 h0 = (_Float16)opaque(y0), h1 = (_Float16)opaque(y1);
        return (uint32_t)__builtin_bit_cast(uint16_t, h0) |
               ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
    }
}

// MFMA fragment of eight 16-bit values of type DT, and the 32x32x16 product.
template <int DT> struct Frag8 { typedef bf16x8 T; };
template <> struct Frag8<1> { typedef f16x8 T; };

template <int DT>
__device__ __forceinline__ f32x16 mfma32(const typename Frag8<DT>::T& a, const typename Frag8<DT>::T& b,
                                         const f32x16& c)
{
    if constexpr (DT == 0) return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    else return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

struct GemmArgs {
    const uint16_t* a;      // [M x kred] bf16 bits, row pitch lda
    int64_t lda;
    const uint8_t* codes;   // W codes, W row-major [rows x cols]
    const int8_t* qabsmax;  // per 64-block (double quant) ...
    const float* scale2;    // ... and per 256 blocks
    const float* absmax;    // per 64-block (no double quant)
    int64_t cols;           // W row length
    void* out;              // [M x ncol], row pitch ldo
    int64_t ldo;
    int64_t M, kred, ncol;
    int64_t ntn;            // output column tiles
    int64_t tile0;          // first (tile, split) index of this launch
    int64_t ntiles;         // output tiles (row tiles x column tiles)
    int nsplit;             // splits of the reduction (1: none)
    int64_t nfull, nhalf;   // 256 x 256 tiles: whole tiles, then nhalf tiles split into row pieces (0: none)
    int pieces;             // row pieces of each of those tiles: 2 (128 rows) or 4 (64 rows, backward)
    int split_steps;        // k-steps per split
    float* part;            // nsplit > 1: fp32 partials [nsplit][M x ncol]; tail_split > 0: see there
    int tail_split;         // 256 x 256 kernels with a workspace: the nhalf tiles from nfull on, each cut
                            // into tail_split splits of the reduction; partial (split, tile) is one
                            // 256 x 256 fp32 block at part + (split * nhalf + tile - nfull) * 65536
};

// Raw constant of W block b as loaded: the int8 and its group scale with
// double quant, else the fp32 absmax.  Kept raw until the dequantisation so
// that the loads stay in flight while the previous step multiplies.
struct RawConst {
    int32_t q;
    float s;
};

template <bool DQ>
__device__ __forceinline__ RawConst load_const(const GemmArgs& g, int64_t b)
{
    if constexpr (DQ) return RawConst{((const GLOBAL int8_t*)g.qabsmax)[b], ((const GLOBAL float*)g.scale2)[b >> 8]};
    else return RawConst{0, ((const GLOBAL float*)g.absmax)[b]};
}

// Level c (0..15) by a select chain over immediates (no memory access).
__device__ __forceinline__ float level_imm(int c)
{
    float v = as_f(nf4fmt::kLevelBits[0]);
#pragma unroll
    for (int i = 1; i < 16; ++i) v = c == i ? as_f(nf4fmt::kLevelBits[i]) : v;
    return v;
}

// The dequantised constant (fl32 product with double quant).
template <bool DQ>
__device__ __forceinline__ float block_const(const RawConst& c)
{
    if constexpr (DQ) return (float)c.q * c.s;
    else return c.s;
}

// Eight codes (one dword, element 2j in the low nibble of byte j) to eight
// 16-bit values, packed in four dwords.
template <int DT>
__device__ __forceinline__ u32x4 deq8(uint32_t c, float adq, const float* lv)
{
    u32x4 r;
    // lv: 256 (level[b & 15], level[b >> 4]) pairs
    const f2* lp = (const f2*)lv;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const f2 p = lp[(c >> (8 * j)) & 255];
        r[j] = pack16<DT>(p.x * adq, p.y * adq);
    }
    return r;
}

// Per-step loads held in registers while the previous step multiplies.
struct StepRegs {
    u32x4 a[kAChunks];        // 16-byte chunks of A rows
    uint32_t w[kWPass][4];    // codes: forward 4 dwords of one W row; backward 1 dword of 4 W rows
    RawConst k[kWPass][4];    // forward: [p][0]; backward: one per W row
};

template <bool FWD, bool DQ>
__device__ __forceinline__ void load_step(StepRegs& r, const GemmArgs& g, int64_t m0, int64_t c0,
                                          int64_t k0)
{
    const int t = threadIdx.x;
    // A: kBM rows x 64 elements; thread t: rows (t >> 3) + 32 i, 16-byte chunk t & 7.
    // Rows past M load row M-1 instead: they only feed output rows that are
    // not stored, and an unconditional load never waits for the one before.
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
        int64_t row = m0 + (t >> 3) + 32 * i;
        row = row < g.M ? row : g.M - 1;
        r.a[i] = *(const GLOBAL u32x4*)(g.a + row * g.lda + k0 + 8 * (t & 7));
    }
#pragma unroll
    for (int p = 0; p < kWPass; ++p) {
        if constexpr (FWD) {
            // W rows c0 .. c0+kBN-1 (output columns), cols k0 .. k0+63: thread t takes
            // 32 codes of row c0 + 128 p + (t >> 1), half t & 1; one block per row
            const int64_t n = c0 + 128 * p + (t >> 1);
            const int64_t e = n * g.cols + k0 + 32 * (t & 1);
            const u32x4 c = *(const GLOBAL u32x4*)(g.codes + (e >> 1));
            r.w[p][0] = c.x; r.w[p][1] = c.y; r.w[p][2] = c.z; r.w[p][3] = c.w;
            r.k[p][0] = load_const<DQ>(g, e >> 6);
        } else {
            // W rows k0 .. k0+63 (the reduction), cols c0 .. c0+kBN-1 (output columns):
            // thread t takes rows k0 + 4 (t & 15) + i, cols c0 + 128 p + 8 (t >> 4) .. + 8
            // (16 consecutive lanes: 64 consecutive rows of one 8-column group, so
            // that their transposed LDS writes form one contiguous 128-byte row)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t n = k0 + 4 * (t & 15) + i;
                const int64_t e = n * g.cols + c0 + 128 * p + 8 * (t >> 4);
                r.w[p][i] = *(const GLOBAL uint32_t*)(g.codes + (e >> 1));
                r.k[p][i] = load_const<DQ>(g, e >> 6);
            }
        }
    }
}

template <int DT, bool FWD, bool DQ>
__device__ __forceinline__ void store_step(const StepRegs& r, uint16_t* As, uint16_t* Ws,
                                           const float* lv)
{
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kAChunks; ++i)
        *(u32x4*)(As + ((t >> 3) + 32 * i) * kLdp + 8 * (t & 7)) = r.a[i];
#pragma unroll
    for (int p = 0; p < kWPass; ++p) {
        if constexpr (FWD) {
            // W tile in W's order: Ws[n][k]
            uint16_t* dst = Ws + (128 * p + (t >> 1)) * kLdp + 32 * (t & 1);
            const float adq = block_const<DQ>(r.k[p][0]);
#pragma unroll
            for (int j = 0; j < 4; ++j) *(u32x4*)(dst + 8 * j) = deq8<DT>(r.w[p][j], adq, lv);
        } else {
            // transposed: Ws[k][n] with the reduction index n contiguous; this thread's
            // four rows n0..n0+3 are consecutive, so each column gets one 8-byte write
            u32x4 y[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] = deq8<DT>(r.w[p][i], block_const<DQ>(r.k[p][i]), lv);
            const int n0 = 4 * (t & 15), cc = 128 * p + 8 * (t >> 4);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                // the 16-bit value of column c from rows (0, 1) and (2, 3): one byte
                // permute each (low halves: bytes 1:0 of each source, high: 3:2)
                const int j = c >> 1;
                const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
                const uint32_t v0 = __builtin_amdgcn_perm(y[1][j], y[0][j], sel);
                const uint32_t v1 = __builtin_amdgcn_perm(y[3][j], y[2][j], sel);
                *(u32x2*)(Ws + (cc + c) * kLdp + n0) = u32x2{v0, v1};
            }
        }
    }
}


// Tile t of a launch of n workgroups in an order where each XCD (workgroups
// are dealt to the eight XCDs in turn) takes a contiguous run of tiles.
__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t n)
{
    const int64_t per = n >> 3, rem = n & 7, x = b & 7, i = b >> 3;
    return x < rem ? x * (per + 1) + i : rem * (per + 1) + (x - rem) * per + i;
}

// Output tile coordinates in groups of four row tiles, column tiles outer.
__device__ __forceinline__ void group_coords(int64_t tile, int64_t mtiles, int64_t ntn, int64_t& mt, int64_t& nt)
{
    constexpr int kG = 4;
    const int64_t per = kG * ntn, first = (tile / per) * kG;
    const int64_t gsz = mtiles - first < kG ? mtiles - first : kG;
    const int64_t in = tile % per;
    mt = first + in % gsz;
    nt = in / gsz;
}

// PART: this workgroup sums one split of the reduction and stores it as an
// fp32 partial (k_splitk_sum adds the splits in order); otherwise the whole
// reduction, stored as fp32 or the 16-bit type.
template <int DT, bool FWD, bool DQ, bool OUT_F32, bool PART>
__global__ __launch_bounds__(kGThreads, 3) void k_nf4_matmul(GemmArgs g)
{
    // one LDS buffer (two barriers per step) leaves room for 3 workgroups per CU
    __shared__ __attribute__((aligned(16))) uint16_t s_a[kBM * kLdp];
    __shared__ __attribute__((aligned(16))) uint16_t s_w[kBN * kLdp];
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    // level tables from immediates: an indexed constant table would be a
    // memory load, waited for before the first tile's loads are issued
    __shared__ __attribute__((aligned(16))) float s_lv[2 * 256];
    for (int i = t; i < 256; i += kGThreads) {
        s_lv[2 * i] = level_imm(i & 15);
        s_lv[2 * i + 1] = level_imm(i >> 4);
    }

    int64_t tile = g.tile0 + xcd_tile(blockIdx.x, gridDim.x);
    // splits are the outer index: each split covers every output tile
    const int split = PART ? (int)(tile / g.ntiles) : 0;
    if (PART) tile -= (int64_t)split * g.ntiles;
    int64_t mt, nt;
    group_coords(tile, (g.M + kBM - 1) / kBM, g.ntn, mt, nt);
    const int64_t m0 = mt * kBM;
    const int64_t c0 = nt * kBN;
    const int wm = wv >> 1, wn = wv & 1;   // this wave's kWM x kWN quarter
    const int ksteps = (int)(g.kred / kBK);
    const int step0 = PART ? split * g.split_steps : 0;
    const int nsteps = PART ? min(g.split_steps, ksteps - step0) : ksteps;
    const int64_t kb = (int64_t)step0 * kBK;   // first reduction index of this split

    f32x16 acc[kTM][kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    StepRegs regs;
    load_step<FWD, DQ>(regs, g, m0, c0, kb);
    __syncthreads();   // level table
    store_step<DT, FWD, DQ>(regs, s_a, s_w, s_lv);
    __syncthreads();

    for (int s = 0; s < nsteps; ++s) {
        const bool more = s + 1 < nsteps;
        if (more) load_step<FWD, DQ>(regs, g, m0, c0, kb + (int64_t)(s + 1) * kBK);
        const uint16_t* As = s_a;
        const uint16_t* Ws = s_w;
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            const int kof = 16 * kk + 8 * (lane >> 5);
            typedef typename Frag8<DT>::T F;
            F fa[kTM], fb[kTN];
#pragma unroll
            for (int i = 0; i < kTM; ++i)
                fa[i] = *(const F*)(As + (kWM * wm + 32 * i + (lane & 31)) * kLdp + kof);
#pragma unroll
            for (int j = 0; j < kTN; ++j)
                fb[j] = *(const F*)(Ws + (kWN * wn + 32 * j + (lane & 31)) * kLdp + kof);
#pragma unroll
            for (int i = 0; i < kTM; ++i)
#pragma unroll
                for (int j = 0; j < kTN; ++j)
                    acc[i][j] = mfma32<DT>(fa[i], fb[j], acc[i][j]);
        }
        __syncthreads();   // every wave done reading the one buffer
        if (more) store_step<DT, FWD, DQ>(regs, s_a, s_w, s_lv);
        __syncthreads();
    }

    // D layout of a 32 x 32 tile: lane l, value r -> row 8 (r / 4) + 4 (l / 32) + r % 4,
    // column l % 32
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + kWM * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const int64_t col = c0 + kWN * wn + 32 * j + (lane & 31);
                if (row < g.M) {
                    if constexpr (PART)
                        ((GLOBAL float*)g.part)[(int64_t)split * g.M * g.ldo + row * g.ldo + col] = acc[i][j][r];
                    else if constexpr (OUT_F32)
                        ((GLOBAL float*)g.out)[row * g.ldo + col] = acc[i][j][r];
                    else
                        ((GLOBAL uint16_t*)g.out)[row * g.ldo + col] =
                            (uint16_t)pack16<DT>(acc[i][j][r], 0.0f);
                }
            }
}

// ---- large m, forward: 256 x 256 output tiles, the weight operand
// dequantised straight into matrix-core registers
//
// Four waves side by side: wave w owns output columns (W rows) c0 + 64 w ..
// c0 + 64 w + 63 (two 32-column MFMA tiles) over all 256 rows of the x tile
// (eight 32-row tiles), so each weight is dequantised once per workgroup and
// never stored anywhere.  A 64-wide k-step is one quantisation block of every
// W row: lane (q, h) = (l % 32, l / 32) loads the 32 codes of W row
// c0 + 64 w + 32 j + q at k 32 h .. 32 h + 31 (one 16-byte load) and MFMA kk of
// the step takes k 32 h + 8 kk .. + 7 of them; the x fragment reads the same k
// from LDS, so the two operands agree (the order of the reduction inside a
// step is not W's storage order, which only reorders the fp32 sum).  x is
// staged through two LDS buffers, one barrier per step; the next step's x rows
// and codes are loaded while this one multiplies.  Levels come from a table of
// level pairs per code byte in 32 interleaved copies, lane l reading copy
// l % 32 so that any codes hit distinct banks: entry e of copy c sits at byte
// 256 e + 8 c, an address one byte permute builds from the code byte.
constexpr int kXM = 256, kXN = 256;           // output tile: x rows, output columns
constexpr int kXPitch = 72;                   // staged x row, 16-bit elements (144 B: conflict-free 16-B reads)
constexpr int kLutCopies = 32;
constexpr int kLutBytes = 256 * kLutCopies * 8;
constexpr int kXBuf = kXM * kXPitch * 2;      // bytes per x buffer
constexpr int kXLds = kLutBytes + 2 * kXBuf;  // 139,264 B of LDS: one workgroup per CU

// Eight codes (one dword, element 2j in the low nibble of byte j) to eight
// 16-bit values through the level-pair table; lb = this lane's copy offset.
template <int DT>
__device__ __forceinline__ u32x4 deq8_pairs(uint32_t c, float adq, const uint8_t* lut, uint32_t lb)
{
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        // byte 1 <- code byte j, byte 0 <- lb, bytes 3:2 <- lb's zero byte 2
        const uint32_t addr = __builtin_amdgcn_perm(c, lb, 0x02020000u | ((4u + j) << 8));
        const f2 p = *(const f2*)(lut + addr);
        r[j] = pack16<DT>(p.x * adq, p.y * adq);
    }
    return r;
}

// One output tile of MT * 32 x rows (MT = 8: a whole 256-row tile; 4: one
// half of it) and 256 output columns, over k-steps step0 .. step0 + nsteps - 1,
// into out (or the fp32 partials of split `split`).  s_mem holds the level
// table; the x buffers follow it.
template <int DT, bool DQ, bool OUT_F32, bool PART, int MT>
__device__ __forceinline__ void mm_fwd_tile(const GemmArgs& g, uint8_t* s_mem, int64_t m0, int64_t c0, int split,
                                            int64_t poff, int64_t ldp)
{
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6, q = lane & 31, h = lane >> 5;
    const uint8_t* lut = s_mem;
    const uint32_t lb = (uint32_t)q << 3;
    const bool live = c0 + 64 * wv < g.ncol;   // wave-uniform: a 128-column tail leaves waves 2, 3 idle
    const int ksteps = (int)(g.kred / 64);
    const int step0 = PART ? split * g.split_steps : 0;
    const int nsteps = PART ? min(g.split_steps, ksteps - step0) : ksteps;

    // Loads address a uniform base (scalar registers, advanced per step) plus
    // a 32-bit lane offset; the launcher keeps 256 rows of x and of the codes
    // under 2 GiB.  x: thread t stages rows (t >> 3) + 32 i, 16-byte chunk
    // t & 7; rows past M repeat row M - 1 (they feed only output rows that are
    // not stored).
    const GLOBAL uint8_t* xb = (const GLOBAL uint8_t*)((const GLOBAL uint16_t*)g.a + m0 * g.lda + (int64_t)step0 * 64);
    uint32_t xo[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        int64_t row = m0 + (t >> 3) + 32 * i;
        row = row < g.M ? row : g.M - 1;
        xo[i] = (uint32_t)(((row - m0) * g.lda + 8 * (t & 7)) * 2);
    }
    // W rows of this lane: n_j = c0 + 64 wv + 32 j + q (in bounds when live)
    const int64_t nrow0 = c0 + 64 * wv + q;
    const int64_t bpr = g.cols / 64;   // blocks per W row
    const int64_t wrow = c0 + 64 * (int64_t)__builtin_amdgcn_readfirstlane(wv);   // wave-uniform
    const GLOBAL uint8_t* cb = (const GLOBAL uint8_t*)g.codes + ((wrow * g.cols + (int64_t)step0 * 64) >> 1);
    const int64_t kb = wrow * bpr + step0;   // block of W row wrow at the first step
    uint32_t co[2], ko[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        co[j] = (uint32_t)((((32 * j + q) * g.cols) >> 1) + 16 * h);
        ko[j] = (uint32_t)((32 * j + q) * bpr);
    }
    // buffer resources over the uniform bases: the step offset goes in the
    // scalar offset, the lane offset in the vector offset (no per-step vector
    // address arithmetic); 0x00020000 selects raw 32-bit data
    const __amdgpu_buffer_rsrc_t xs = __builtin_amdgcn_make_buffer_rsrc((void*)xb, 0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t cs = __builtin_amdgcn_make_buffer_rsrc((void*)cb, 0, 0x7fffffff, 0x00020000);
    const void* kbase = DQ ? (const void*)((const int8_t*)g.qabsmax + kb) : (const void*)((const float*)g.absmax + kb);
    const __amdgpu_buffer_rsrc_t ks = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, 0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t ss =
        __builtin_amdgcn_make_buffer_rsrc((void*)(DQ ? g.scale2 : g.absmax), 0, 0x7fffffff, 0x00020000);
    auto ld_x = [&](int i, int s) { return __builtin_amdgcn_raw_buffer_load_b128(xs, xo[i], 128 * s, 0); };
    auto ld_c = [&](int j, int s) { return __builtin_amdgcn_raw_buffer_load_b128(cs, co[j], 32 * s, 0); };
    // constants of this lane's rows at step s (relative to step0); the scale
    // of block b is scale2[b >> 8], b = kb + s + ko[j] = 256 A + (B + ko[j])
    auto ld_k = [&](int j, int s) -> RawConst {
        if constexpr (DQ) {
            const int8_t qv = (int8_t)__builtin_amdgcn_raw_buffer_load_b8(ks, ko[j], s, 0);
            const int64_t kbs = kb + s;
            const uint32_t grp = (uint32_t)(kbs & 255) + ko[j];
            const float sv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                 ss, (grp >> 8) << 2, (int)((kbs >> 8) << 2), 0));
            return RawConst{qv, sv};
        } else {
            return RawConst{0, __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ks, ko[j] << 2, 4 * s, 0))};
        }
    };

    f32x16 acc[MT][2];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    u32x4 xr[MT], cw[2], cn[2];
    RawConst kc[2], kn[2];
#pragma unroll
    for (int i = 0; i < MT; ++i) xr[i] = ld_x(i, 0);
    if (live) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            cw[j] = ld_c(j, 0);
            kc[j] = ld_k(j, 0);
        }
    }
    uint16_t* xs0 = (uint16_t*)(s_mem + kLutBytes);
    const int wofs = ((t >> 3)) * kXPitch + 8 * (t & 7);   // this thread's staging slot, row (t >> 3)
#pragma unroll
    for (int i = 0; i < MT; ++i) *(u32x4*)(xs0 + wofs + 32 * i * kXPitch) = xr[i];
    __syncthreads();   // level table and the first x tile

    typedef typename Frag8<DT>::T F;
    if (!live) {
        // idle columns: stage x as the live waves do, barrier for barrier
        for (int s = 0; s < nsteps; ++s) {
#pragma unroll
            for (int i = 0; i < MT; ++i) xr[i] = ld_x(i, s + 1 < nsteps ? s + 1 : s);
            uint16_t* Xn = (uint16_t*)(s_mem + kLutBytes + ((s + 1) & 1) * kXBuf);
#pragma unroll
            for (int i = 0; i < MT; ++i) *(u32x4*)(Xn + wofs + 32 * i * kXPitch) = xr[i];
            __syncthreads();
        }
        return;
    }
    // Software pipeline over sub-steps kk of 16 MFMAs: while kk multiplies, the
    // x fragments of kk + 1 are read, the level pairs of kk + 2 are looked up
    // and the weight fragments of kk + 1 are finished from the pairs looked up
    // one sub-step earlier (across the step boundary for the next step's
    // codes).  Each sub-step is one scheduling region whose reads and ALU work
    // are spread between its MFMAs.
    F fa[2][MT], fb[2][2];
    f2 lv[2][2][4];   // level pairs [slot][W tile j][code byte]
    auto rd_x = [&](const uint16_t* X, int kk, F (&d)[MT]) {
#pragma unroll
        for (int i = 0; i < MT; ++i) d[i] = *(const F*)(X + (32 * i + q) * kXPitch + 32 * h + 8 * kk);
    };
    auto rd_lv = [&](const u32x4 (&c)[2], int kk, f2 (&d)[2][4]) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int b = 0; b < 4; ++b)   // byte 1 <- code byte b, byte 0 <- lb, bytes 3:2 <- lb's zero byte 2
                d[j][b] = *(const f2*)(lut + __builtin_amdgcn_perm(c[j][kk], lb, 0x02020000u | ((4u + b) << 8)));
    };
    auto mk_w = [&](const f2 (&p)[2][4], float a0, float a1, F (&d)[2]) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float a = j ? a1 : a0;
            u32x4 r;
#pragma unroll
            for (int b = 0; b < 4; ++b) r[b] = pack16<DT>(p[j][b].x * a, p[j][b].y * a);
            d[j] = __builtin_bit_cast(F, r);
        }
    };
    auto mm = [&](const F (&a)[MT], const F (&b)[2]) {
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            acc[i][0] = mfma32<DT>(a[i], b[0], acc[i][0]);
            acc[i][1] = mfma32<DT>(a[i], b[1], acc[i][1]);
        }
    };
    auto interleave = [&]() {
#pragma unroll
        for (int i = 0; i < 2 * MT; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 8 / MT, 0);   // LDS reads
            __builtin_amdgcn_sched_group_barrier(0x002, 16 / MT, 0);  // VALU
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    float a0 = block_const<DQ>(kc[0]), a1 = block_const<DQ>(kc[1]);
    rd_lv(cw, 0, lv[0]);
    mk_w(lv[0], a0, a1, fb[0]);
    rd_lv(cw, 1, lv[1]);
    for (int s = 0; s < nsteps; ++s) {
        // the next step's codes, constants and x rows; the last step loads its
        // own again (in bounds, and what the look-ahead computes from them is
        // not used), which keeps the loop free of branches
        const int sn = s + 1 < nsteps ? s + 1 : s;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            cn[j] = ld_c(j, sn);
            kn[j] = ld_k(j, sn);
        }
#pragma unroll
        for (int i = 0; i < MT; ++i) xr[i] = ld_x(i, sn);
        __builtin_amdgcn_sched_barrier(0);
        const uint16_t* X = (const uint16_t*)(s_mem + kLutBytes + (s & 1) * kXBuf);
        rd_x(X, 0, fa[0]);
        __builtin_amdgcn_sched_barrier(0);
        mm(fa[0], fb[0]); rd_x(X, 1, fa[1]); rd_lv(cw, 2, lv[0]); mk_w(lv[1], a0, a1, fb[1]);
        interleave();
        mm(fa[1], fb[1]); rd_x(X, 2, fa[0]); rd_lv(cw, 3, lv[1]); mk_w(lv[0], a0, a1, fb[0]);
        interleave();
        const float n0 = block_const<DQ>(kn[0]), n1 = block_const<DQ>(kn[1]);
        mm(fa[0], fb[0]); rd_x(X, 3, fa[1]); rd_lv(cn, 0, lv[0]); mk_w(lv[1], a0, a1, fb[1]);
        interleave();
        mm(fa[1], fb[1]); rd_lv(cn, 1, lv[1]); mk_w(lv[0], n0, n1, fb[0]);
        interleave();
        {   // the last step writes the other buffer too: nothing reads it again
            uint16_t* Xn = (uint16_t*)(s_mem + kLutBytes + ((s + 1) & 1) * kXBuf);
#pragma unroll
            for (int i = 0; i < MT; ++i) *(u32x4*)(Xn + wofs + 32 * i * kXPitch) = xr[i];
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) { cw[j] = cn[j]; kc[j] = kn[j]; }
        a0 = n0;
        a1 = n1;
        __syncthreads();
    }

    // D layout of a 32 x 32 tile: lane l, value r -> row 8 (r / 4) + 4 (l / 32) + r % 4,
    // column l % 32
    const bool full = m0 + 32 * MT <= g.M;
    const int64_t rbase = m0 + 4 * h;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = rbase + 32 * i + 8 * (r >> 2) + (r & 3);
                const int64_t col = nrow0 + 32 * j;
                if (full || row < g.M) {
                    if constexpr (PART)
                        ((GLOBAL float*)g.part)[poff + row * ldp + col] = acc[i][j][r];
                    else if constexpr (OUT_F32)
                        ((GLOBAL float*)g.out)[row * g.ldo + col] = acc[i][j][r];
                    else
                        ((GLOBAL uint16_t*)g.out)[row * g.ldo + col] = (uint16_t)pack16<DT>(acc[i][j][r], 0.0f);
                }
            }
}


// The launch order of both large-m kernels: with nhalf > 0 it holds nfull
// whole tiles, then nhalf tiles cut into g.pieces row pieces of 128 or 64 rows
// (the tiles left over after the whole rounds of one workgroup per CU: cutting
// them shortens the last round); every XCD takes its share of whole tiles
// first and then its share of pieces, both contiguous in the tile order.
// piece = -1 for a whole tile.
__device__ __forceinline__ int64_t launch_tile(const GemmArgs& g, int& piece)
{
    piece = -1;
    if (g.nhalf == 0) return g.tile0 + xcd_tile(blockIdx.x, gridDim.x);
    const int64_t x = blockIdx.x & 7, i = blockIdx.x >> 3, fpx = g.nfull >> 3;
    const int64_t ppx = g.nhalf * g.pieces >> 3;
    if (i < fpx) return x * fpx + i;
    const int64_t pp = x * ppx + (i - fpx);
    piece = (int)(pp % g.pieces);
    return g.nfull + pp / g.pieces;
}

// What a workgroup of the large-m kernels computes: output tile (mt, nt), row
// piece (-1: the whole tile), split of the reduction, and with PART where its
// fp32 partial goes: element (row, col) at part[poff + row * ldp + col].
struct BigWork {
    int64_t mt, nt, poff, ldp;
    int piece, split;
};

template <bool PART>
__device__ __forceinline__ BigWork big_work(const GemmArgs& g)
{
    BigWork w;
    int64_t tile;
    w.piece = -1;
    w.split = 0;
    if (PART && g.tail_split > 0) {
        // the leftover tiles' splits, split outer: each XCD takes a run of
        // neighbouring tiles of one split (they share rows of x)
        const int64_t local = xcd_tile(blockIdx.x, gridDim.x);
        w.split = (int)(local / g.nhalf);
        tile = g.nfull + (local - (int64_t)w.split * g.nhalf);
    } else {
        tile = launch_tile(g, w.piece);
        if (PART) {
            w.split = (int)(tile / g.ntiles);
            tile -= (int64_t)w.split * g.ntiles;
        }
    }
    group_coords(tile, (g.M + kXM - 1) / kXM, g.ntn, w.mt, w.nt);
    w.ldp = g.ldo;
    w.poff = PART ? (int64_t)w.split * g.M * g.ldo : 0;
    if (PART && g.tail_split > 0) {
        // one 256 x 256 block per (split, tile), rows of 256
        w.ldp = kXN;
        w.poff = ((int64_t)w.split * g.nhalf + (tile - g.nfull)) * (kXM * kXN) - w.mt * kXM * kXN - w.nt * kXN;
    }
    return w;
}

template <int DT, bool DQ, bool OUT_F32, bool PART>
__global__ __launch_bounds__(256, 1) void k_nf4_mm_fwd(GemmArgs g)
{
    __shared__ __attribute__((aligned(16))) uint8_t s_mem[kXLds];
    const int t = threadIdx.x;
    {
        // thread t builds entry t; the copy pairs are written in a rotated
        // order so that the lanes of one write hit distinct banks
        const uint32_t lo = __builtin_bit_cast(uint32_t, level_imm(t & 15));
        const uint32_t hi = __builtin_bit_cast(uint32_t, level_imm(t >> 4));
        u32x4* row = (u32x4*)(s_mem + 256 * t);
#pragma unroll
        for (int c = 0; c < kLutCopies / 2; ++c) row[(c + t) & (kLutCopies / 2 - 1)] = u32x4{lo, hi, lo, hi};
    }
    const BigWork w = big_work<PART>(g);
    const int64_t m0 = w.mt * kXM, c0 = w.nt * kXN;
    if (w.piece < 0) mm_fwd_tile<DT, DQ, OUT_F32, PART, 8>(g, s_mem, m0, c0, w.split, w.poff, w.ldp);
    else if (g.pieces == 2)
        mm_fwd_tile<DT, DQ, OUT_F32, PART, 4>(g, s_mem, m0 + 128 * w.piece, c0, w.split, w.poff, w.ldp);
    else mm_fwd_tile<DT, DQ, OUT_F32, PART, 2>(g, s_mem, m0 + 64 * w.piece, c0, w.split, w.poff, w.ldp);
}

// ---- large m, backward (input gradient): 256 x 256 output tiles, the weight
// transposed through LDS
//
// out[m, c] = sum_n x[m, n] W[n, c]: the reduction runs over W's rows, across
// its quantisation blocks, so an MFMA weight fragment (eight consecutive n of
// one column) is not contiguous in W.  Wave w owns output columns
// c0 + 64 w .. + 63 over all 256 rows of the x tile.  For each 64-row k-step
// it dequantises its own 64 x 64 piece of W, lane l taking W row n0 + l
// (exactly one block: 32 code bytes and one constant), writes it to a private
// LDS region in W's order, and reads its weight fragments back with the
// transposing 64-bit LDS read: in each group of 16 lanes, lane i receives
// element i % 4 of the 4-element pieces read by lanes 4 k + i / 4 (k = 0..3),
// so the 16 lanes reading rows r .. r + 3 at columns C + 4 (i % 4) come back
// as column C + i, rows r .. r + 3.  The step's dequantisation runs one step
// ahead of its MFMAs, spread over the four sub-steps; x is double-buffered as
// in the forward kernel.  Region rows are 128 B with chunk c of row r at slot
// c ^ (4 ((r / 2) % 2) + (r / 4) % 4), conflict-free for both the row writes and
// the transposing reads; x rows are 128 B with chunk c of row r at
// c ^ ((r / 2) % 8).  (LDS serves 256 B per cycle: two consecutive 128-byte
// rows fall in different bank halves, so the swizzles separate rows of equal
// parity.)
constexpr int kBXBuf = 256 * 128;                   // x buffer: 256 rows x 64 16-bit values
constexpr int kBWReg = 64 * 128;                    // per-wave W region: 64 rows x 64 16-bit values
constexpr int kBLds = kLutBytes + 2 * kBXBuf + 4 * kBWReg;   // 163,840 B
static_assert(kBLds <= 163840, "LDS of one CU");

__device__ __forceinline__ int wslot(int r, int c) { return c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3)); }

template <int DT, bool DQ, bool OUT_F32, bool PART, int MT>
__device__ __forceinline__ void mm_bwd_tile(const GemmArgs& g, uint8_t* s_mem, int64_t m0, int64_t c0, int split,
                                            int64_t poff, int64_t ldp)
{
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6, q = lane & 31, h = lane >> 5;
    const uint8_t* lut = s_mem;
    const uint32_t lb = (uint32_t)q << 3;
    const bool live = c0 + 64 * wv < g.ncol;   // wave-uniform
    const int ksteps = (int)(g.kred / 64);
    const int step0 = PART ? split * g.split_steps : 0;
    const int nsteps = PART ? min(g.split_steps, ksteps - step0) : ksteps;

    // x (the output gradient, M x rows): thread t stages rows (t >> 3) + 32 i,
    // chunk t & 7; rows past M repeat row M - 1.  Loads: uniform base, step in
    // the scalar offset, 32-bit lane offset (the launcher keeps them in range).
    const GLOBAL uint8_t* xb = (const GLOBAL uint8_t*)((const GLOBAL uint16_t*)g.a + m0 * g.lda + (int64_t)step0 * 64);
    uint32_t xo[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        int64_t row = m0 + (t >> 3) + 32 * i;
        row = row < g.M ? row : g.M - 1;
        xo[i] = (uint32_t)(((row - m0) * g.lda + 8 * (t & 7)) * 2);
    }
    const __amdgpu_buffer_rsrc_t xs = __builtin_amdgcn_make_buffer_rsrc((void*)xb, 0, 0x7fffffff, 0x00020000);
    // W: lane l dequantises row n0 + l, columns cw .. cw + 63 (block cw / 64)
    const int64_t cw = c0 + 64 * (int64_t)__builtin_amdgcn_readfirstlane(wv);   // wave-uniform
    const int64_t bpr = g.cols / 64;
    const GLOBAL uint8_t* cb = (const GLOBAL uint8_t*)g.codes + (((int64_t)step0 * 64 * g.cols + cw) >> 1);
    const __amdgpu_buffer_rsrc_t cs = __builtin_amdgcn_make_buffer_rsrc((void*)cb, 0, 0x7fffffff, 0x00020000);
    const uint32_t co = (uint32_t)(lane * (g.cols >> 1));
    const int64_t kb = (int64_t)step0 * 64 * bpr + (cw >> 6);   // block of row n0, columns cw.. at the first step
    const uint32_t ko = (uint32_t)(lane * bpr);
    const void* kbase = DQ ? (const void*)((const int8_t*)g.qabsmax + kb) : (const void*)((const float*)g.absmax + kb);
    const __amdgpu_buffer_rsrc_t ks = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, 0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t ss =
        __builtin_amdgcn_make_buffer_rsrc((void*)(DQ ? g.scale2 : g.absmax), 0, 0x7fffffff, 0x00020000);
    const int32_t cstep = (int32_t)(32 * g.cols);   // code bytes per k-step
    const int32_t kstep = (int32_t)(64 * bpr);      // blocks per k-step
    auto ld_x = [&](int i, int s) { return __builtin_amdgcn_raw_buffer_load_b128(xs, xo[i], 128 * s, 0); };
    auto ld_c = [&](int half, int s) { return __builtin_amdgcn_raw_buffer_load_b128(cs, co + 16 * half, cstep * s, 0); };
    auto ld_k = [&](int s) -> RawConst {
        if constexpr (DQ) {
            const int8_t qv = (int8_t)__builtin_amdgcn_raw_buffer_load_b8(ks, ko, kstep * s, 0);
            const int64_t kbs = kb + (int64_t)kstep * s;
            const uint32_t grp = (uint32_t)(kbs & 255) + ko;
            const float sv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                 ss, (grp >> 8) << 2, (int)((kbs >> 8) << 2), 0));
            return RawConst{qv, sv};
        } else {
            return RawConst{0, __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ks, ko << 2, 4 * kstep * s, 0))};
        }
    };

    auto xbuf = [&](int b) { return (uint16_t*)(s_mem + kLutBytes + b * kBXBuf); };
    uint16_t* wreg = (uint16_t*)(s_mem + kLutBytes + 2 * kBXBuf + wv * kBWReg);
    const int xw = (t >> 3) * 64 + 8 * ((t & 7) ^ ((t >> 4) & 7));   // staging slot of row t >> 3
    int xrd[4];   // x fragment reads: row 32 i + q, chunk 2 kk + h
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) xrd[kk] = q * 64 + 8 * ((2 * kk + h) ^ ((q >> 1) & 7));
    int wrd[2][4][2];   // transposing reads [j][kk][t]: row 16 kk + 8 h + 4 t + (l % 16) / 4,
                        // columns 32 j + 16 ((l / 16) % 2) + 4 (l % 4) .. + 3
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int r = 16 * kk + 8 * h + 4 * u + ((lane & 15) >> 2);
                const int col = 32 * j + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
                wrd[j][kk][u] = r * 64 + 8 * wslot(r, col >> 3) + (col & 7);
            }

    u32x4 xr[MT];
    auto st_x = [&](uint16_t* X) {
#pragma unroll
        for (int i = 0; i < MT; ++i) *(u32x4*)(X + xw + 32 * i * 64) = xr[i];
    };
#pragma unroll
    for (int i = 0; i < MT; ++i) xr[i] = ld_x(i, 0);
    st_x(xbuf(0));
    if (!live) {
        // idle columns: stage x as the live waves do, barrier for barrier
        __syncthreads();
        for (int s = 0; s < nsteps; ++s) {
#pragma unroll
            for (int i = 0; i < MT; ++i) xr[i] = ld_x(i, s + 1 < nsteps ? s + 1 : s);
            st_x(xbuf((s + 1) & 1));
            __syncthreads();
        }
        return;
    }

    // dequantisation of one row block: 32 code bytes (two 16-byte halves) with
    // constant a, as 8 chunks of eight 16-bit values, written to the region
    u32x4 cw_[2], cq_[2], y[8];
    RawConst kw, kq;
    f2 lv[2][8];   // level pairs of eight code bytes, two groups in flight
    auto lut_rd = [&](int grp, f2 (&d)[8]) {   // code bytes 8 grp .. 8 grp + 7
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const uint32_t c = cw_[grp >> 1][2 * (grp & 1) + (b >> 2)];
            d[b] = *(const f2*)(lut + __builtin_amdgcn_perm(c, lb, 0x02020000u | ((4u + (b & 3)) << 8)));
        }
    };
    auto mulcvt = [&](int grp, const f2 (&p)[8], float a) {   // chunks 2 grp, 2 grp + 1
#pragma unroll
        for (int b = 0; b < 8; ++b) y[2 * grp + (b >> 2)][b & 3] = pack16<DT>(p[b].x * a, p[b].y * a);
    };
    auto st_w = [&]() {
#pragma unroll
        for (int c = 0; c < 8; ++c) *(u32x4*)(wreg + lane * 64 + 8 * wslot(lane, c)) = y[c];
    };
    // first step's W piece, synchronously
    cw_[0] = ld_c(0, 0); cw_[1] = ld_c(1, 0); kw = ld_k(0);
    {
        const float a = block_const<DQ>(kw);
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) { lut_rd(grp, lv[0]); mulcvt(grp, lv[0], a); }
        st_w();
    }
    // codes of step 1 (dequantised during step 0)
    const int s1 = nsteps > 1 ? 1 : 0;
    cw_[0] = ld_c(0, s1); cw_[1] = ld_c(1, s1); kw = ld_k(s1);
    __syncthreads();   // level table and the first x tile

    f32x16 acc[MT][2];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    typedef typename Frag8<DT>::T F;
    F fa[2][MT], fb[2][4];
    auto rd_x = [&](const uint16_t* X, int kk, F (&d)[MT]) {
#pragma unroll
        for (int i = 0; i < MT; ++i) d[i] = *(const F*)(X + xrd[kk] + 32 * i * 64);
    };
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    auto rd_w = [&]() {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4*)(wreg + wrd[j][kk][0])));
                const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4*)(wreg + wrd[j][kk][1])));
                fb[j][kk] = __builtin_bit_cast(F, u32x4{lo.x, lo.y, hi.x, hi.y});
            }
    };
    auto mm = [&](int kk, const F (&a)[MT]) {
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            acc[i][0] = mfma32<DT>(a[i], fb[0][kk], acc[i][0]);
            acc[i][1] = mfma32<DT>(a[i], fb[1][kk], acc[i][1]);
        }
    };
    auto interleave = [&]() {
#pragma unroll
        for (int i = 0; i < 2 * MT; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 8 / MT, 0);   // LDS reads
            __builtin_amdgcn_sched_group_barrier(0x002, 16 / MT, 0);  // VALU
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    for (int s = 0; s < nsteps; ++s) {
        // loads: x rows of step s + 1, codes and constant of step s + 2 (past
        // the end the last step again: in bounds, unused)
        const int sx = s + 1 < nsteps ? s + 1 : s;
        const int sc = s + 2 < nsteps ? s + 2 : nsteps - 1;
#pragma unroll
        for (int i = 0; i < MT; ++i) xr[i] = ld_x(i, sx);
        cq_[0] = ld_c(0, sc); cq_[1] = ld_c(1, sc); kq = ld_k(sc);
        __builtin_amdgcn_sched_barrier(0);
        const uint16_t* X = xbuf(s & 1);
        rd_w();              // this step's weight fragments (region written last step)
        rd_x(X, 0, fa[0]);
        __builtin_amdgcn_sched_barrier(0);
        const float a = block_const<DQ>(kw);
        mm(0, fa[0]); rd_x(X, 1, fa[1]); lut_rd(0, lv[0]);
        interleave();
        mm(1, fa[1]); rd_x(X, 2, fa[0]); lut_rd(1, lv[1]); mulcvt(0, lv[0], a);
        interleave();
        mm(2, fa[0]); rd_x(X, 3, fa[1]); lut_rd(2, lv[0]); mulcvt(1, lv[1], a);
        interleave();
        mm(3, fa[1]); lut_rd(3, lv[1]); mulcvt(2, lv[0], a);
        interleave();
        mulcvt(3, lv[1], a);
        st_w();              // next step's piece: after this step's transposing reads (in order)
        st_x(xbuf((s + 1) & 1));
        cw_[0] = cq_[0]; cw_[1] = cq_[1]; kw = kq;
        __syncthreads();
    }

    const bool full = m0 + 32 * MT <= g.M;
    const int64_t rbase = m0 + 4 * h;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = rbase + 32 * i + 8 * (r >> 2) + (r & 3);
                const int64_t col = cw + 32 * j + q;
                if (full || row < g.M) {
                    if constexpr (PART)
                        ((GLOBAL float*)g.part)[poff + row * ldp + col] = acc[i][j][r];
                    else if constexpr (OUT_F32)
                        ((GLOBAL float*)g.out)[row * g.ldo + col] = acc[i][j][r];
                    else
                        ((GLOBAL uint16_t*)g.out)[row * g.ldo + col] = (uint16_t)pack16<DT>(acc[i][j][r], 0.0f);
                }
            }
}

template <int DT, bool DQ, bool OUT_F32, bool PART>
__global__ __launch_bounds__(256, 1) void k_nf4_mm_bwd(GemmArgs g)
{
    __shared__ __attribute__((aligned(16))) uint8_t s_mem[kBLds];
    const int t = threadIdx.x;
    {
        const uint32_t lo = __builtin_bit_cast(uint32_t, level_imm(t & 15));
        const uint32_t hi = __builtin_bit_cast(uint32_t, level_imm(t >> 4));
        u32x4* row = (u32x4*)(s_mem + 256 * t);
#pragma unroll
        for (int c = 0; c < kLutCopies / 2; ++c) row[(c + t) & (kLutCopies / 2 - 1)] = u32x4{lo, hi, lo, hi};
    }
    // Each wave dequantises its weight piece whatever the rows, so a 64-row
    // quarter costs more than a quarter of a tile, but the pieces of the last
    // tiles fill one short round.
    const BigWork w = big_work<PART>(g);
    const int64_t m0 = w.mt * kXM, c0 = w.nt * kXN;
    if (w.piece < 0) mm_bwd_tile<DT, DQ, OUT_F32, PART, 8>(g, s_mem, m0, c0, w.split, w.poff, w.ldp);
    else if (g.pieces == 2)
        mm_bwd_tile<DT, DQ, OUT_F32, PART, 4>(g, s_mem, m0 + 128 * w.piece, c0, w.split, w.poff, w.ldp);
    else mm_bwd_tile<DT, DQ, OUT_F32, PART, 2>(g, s_mem, m0 + 64 * w.piece, c0, w.split, w.poff, w.ldp);
}

// ---- few tokens, forward: one wave per 16 W rows and one part of the reduction
//
// out[m x rows] = x[m x cols] W^T for m <= 32 on v_mfma_f32_16x16x32 (x rows
// padded with zeros to 16 or 32).  The reduction is cut into 128-wide super-chunks;
// in each, lane l takes W row n0 + l % 16 and x row l % 16 over the 32
// consecutive k at 32 (l / 16), four MFMA steps of 8 k (any assignment of k
// to steps gives the same dot product as long as x and W agree), so its
// weight operand for a super-chunk is one 16-byte load of 32 codes from one
// 64-weight block with one block constant.  A part is at most 8 super-chunks:
// every wave issues its share of the part's x slice and then all of its code
// and constant loads, the workgroup (four waves, one part, four row groups)
// stages the x slice in LDS, and after one barrier the MFMAs run from
// registers and LDS, each super-chunk as soon as its codes have arrived.  Lane l ends
// with output rows 4 (l / 16) + r of its W row; each part stores fp32
// partials, added in part order by k_splitk_sum.
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int DT>
__device__ __forceinline__ f32x4 mfma16(const typename Frag8<DT>::T& a, const typename Frag8<DT>::T& b,
                                        const f32x4& c)
{
    if constexpr (DT == 0) return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    else return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

struct GemvArgs {
    const uint16_t* x;      // [m x cols] 16-bit
    const uint8_t* codes;   // W [rows x cols]
    const int8_t* qabsmax;
    const float* scale2;
    const float* absmax;
    int64_t rows, cols, m;
    int64_t groups;         // rows / 16
    int part_sc;            // 128-wide super-chunks per part (1..kGvMaxSc)
    float* part;            // [parts][m x rows]
};

constexpr int kGvMaxSc = 8;   // super-chunks per part with one 16-row x block (MB = 1); 8 / MB with MB blocks

// MB: 16-row blocks of x (m <= 16 MB); each dequantised weight fragment feeds
// MB MFMAs.  The staged x slice is always 16 MB rows x (8 / MB) super-chunks
// (33 KB of LDS, rows padded by 16 B so the 16 lanes of a row group read
// distinct banks).
template <int DT, bool DQ, int MB>
__global__ __launch_bounds__(256, 4) void k_nf4_gemv16(GemvArgs g)
{
    constexpr int kSc = kGvMaxSc / MB;          // super-chunks per part at most
    constexpr int kRow = kSc * 128 + 8;         // staged x row, 16-bit values
    constexpr int kRowUnits = kSc * 16;         // 16-byte units of a staged row
    __shared__ float s_lv[16];
    __shared__ __attribute__((aligned(16))) uint16_t s_x[16 * MB * kRow];
    const int t = threadIdx.x, lane = t & 63;
    const int part = blockIdx.y;
    const int64_t grp = (int64_t)blockIdx.x * 4 + (t >> 6);   // < groups: groups is a multiple of 4
    const int nsc = (int)(g.cols / 128);
    const int s0 = part * g.part_sc;
    const int ns = min(g.part_sc, nsc - s0);    // >= 1: the part count is ceil(nsc / part_sc)
    const int64_t n = grp * 16 + (lane & 15);   // this lane's W row
    const int kg = lane >> 4, xr = lane & 15;
    // Every load below is unconditional and in bounds (a unit past the x slice
    // or past row m - 1, or a super-chunk past the part, repeats the last valid
    // one and is not used), so the compiler can wait for each super-chunk's
    // loads alone and the MFMAs of the first super-chunks overlap the arrival
    // of the later ones.  The x slice (cache-resident) goes first: waiting for
    // it leaves the code loads in flight.
    const int units = ns * 16;
    const int64_t rmax = g.m - 1;
    u32x4 xv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int u = t + 256 * i;
        const int64_t r = min((int64_t)(u / kRowUnits), rmax);
        const int c8 = min(u % kRowUnits, units - 1);
        xv[i] = *(const GLOBAL u32x4*)((const GLOBAL uint16_t*)g.x + r * g.cols + (int64_t)s0 * 128 + 8 * c8);
    }
    u32x4 cw[kSc];
    RawConst kc[kSc];
    const int64_t e0 = n * g.cols + (int64_t)s0 * 128 + 32 * kg;
#pragma unroll
    for (int sc = 0; sc < kSc; ++sc) {
        const int64_t e = e0 + 128 * min(sc, ns - 1);
        cw[sc] = *(const GLOBAL u32x4*)(g.codes + (e >> 1));
        const int64_t b = e >> 6;
        if constexpr (DQ) kc[sc] = RawConst{((const GLOBAL int8_t*)g.qabsmax)[b], ((const GLOBAL float*)g.scale2)[b >> 8]};
        else kc[sc] = RawConst{0, ((const GLOBAL float*)g.absmax)[b]};
    }
    if (t == 0) {   // immediates: an indexed table would be one more memory load to wait for
#pragma unroll
        for (int i = 0; i < 16; ++i) s_lv[i] = as_f(nf4fmt::kLevelBits[i]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int u = t + 256 * i, r = u / kRowUnits, c8 = u % kRowUnits;
        if (r < g.m && c8 < units) *(u32x4*)(s_x + r * kRow + 8 * c8) = xv[i];
    }
    __syncthreads();
    typedef typename Frag8<DT>::T F;
    f32x4 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int sc = 0; sc < kSc; ++sc) {
        if (sc >= ns) break;
        const float adq = block_const<DQ>(kc[sc]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u32x4 w;
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const uint32_t b = (cw[sc][j] >> (8 * h)) & 255u;
                w[h] = pack16<DT>(s_lv[b & 15] * adq, s_lv[b >> 4] * adq);
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int xrow = 16 * mb + xr;
                const u32x4 a = xrow < g.m ? *(const u32x4*)(s_x + xrow * kRow + 32 * kg + 128 * sc + 8 * j)
                                           : u32x4{0u, 0u, 0u, 0u};
                acc[mb] = mfma16<DT>(__builtin_bit_cast(F, a), __builtin_bit_cast(F, w), acc[mb]);
            }
        }
    }
    // lane l: output rows 16 mb + 4 (l / 16) + r of W row n
    GLOBAL float* dst = (GLOBAL float*)g.part + (int64_t)part * g.m * g.rows;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * mb + 4 * kg + r;
            if (row < g.m) dst[(int64_t)row * g.rows + n] = acc[mb][r];
        }
}

// The fp32 partials of the splits added in split order (fixed, so the result
// does not depend on timing), stored as fp32 or rounded to the 16-bit type.
// Four outputs per thread; n is a multiple of 4 (ncol is a multiple of 128).
template <int DT, bool OUT_F32>
__global__ __launch_bounds__(256) void k_splitk_sum(const float* __restrict__ part, int nsplit,
                                                    int64_t n, void* __restrict__ out)
{
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= n) return;
    typedef float f4 __attribute__((ext_vector_type(4)));
    f4 acc = *(const GLOBAL f4*)(part + i);
    for (int sp = 1; sp < nsplit; ++sp) acc += *(const GLOBAL f4*)(part + (int64_t)sp * n + i);
    if constexpr (OUT_F32) {
        *(GLOBAL f4*)((float*)out + i) = acc;
    } else {
        const u32x2 v = {pack16<DT>(acc.x, acc.y), pack16<DT>(acc.z, acc.w)};
        *(GLOBAL u32x2*)((uint16_t*)out + i) = v;
    }
}

// The tail splits' fp32 partials of each leftover tile added in split order
// and stored into out (rows below M, columns below ncol), as fp32 or rounded to
// the 16-bit type.  Workgroup b covers 1,024 consecutive elements (four per
// thread, within one row) of the 256 x 256 block of leftover tile b / 64.
template <int DT, bool OUT_F32>
__global__ __launch_bounds__(256) void k_tail_sum(GemmArgs g)
{
    const int64_t lt = blockIdx.x >> 6;
    const int e = ((int)(blockIdx.x & 63) << 10) + 4 * (int)threadIdx.x;
    int64_t mt, nt;
    group_coords(g.nfull + lt, (g.M + kXM - 1) / kXM, g.ntn, mt, nt);
    const int64_t row = mt * kXM + (e >> 8), col = nt * kXN + (e & 255);
    if (row >= g.M || col >= g.ncol) return;   // ncol is a multiple of 128: all four in or all out
    typedef float f4 __attribute__((ext_vector_type(4)));
    const GLOBAL float* p = (const GLOBAL float*)g.part + lt * (kXM * kXN) + e;
    f4 acc = *(const GLOBAL f4*)p;
    for (int sp = 1; sp < g.tail_split; ++sp) acc += *(const GLOBAL f4*)(p + (int64_t)sp * g.nhalf * (kXM * kXN));
    const int64_t i = row * g.ldo + col;
    if constexpr (OUT_F32) {
        *(GLOBAL f4*)((float*)g.out + i) = acc;
    } else {
        const u32x2 v = {pack16<DT>(acc.x, acc.y), pack16<DT>(acc.z, acc.w)};
        *(GLOBAL u32x2*)((uint16_t*)g.out + i) = v;
    }
}

// One-shot launches of at most 2^32 / 256 - 1 workgroups each.
constexpr int64_t kMaxGemmGrid = (int64_t(1) << 32) / kGThreads - 1;

// Compute units of the current device (cached per device; 0 if unknown).
int cu_count()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Which kernel takes a call.  The choices are functions of the shape only
// (the workspace a caller allocates depends on them), planned for the 256
// CUs of an MI355X.
constexpr int64_t kPlanCus = 256;

// The 256 x 256 kernels keep 256 rows of x (and of the codes, backward the
// whole weight) under 32-bit buffer offsets.
bool big_eligible(bool forward, int64_t M, int64_t ncol, int64_t kred)
{
    if (M <= 128 || kred >= (int64_t(1) << 22)) return false;
    return forward || kred * ncol < (int64_t(1) << 32);
}

// Without a split, the 256 x 256 kernels take a call when their tiles fill at
// least half a round (forward) or when the 128 x 128 tiles would need more
// than one (backward); below that the 128 x 128 kernel's more, shorter
// workgroups finish first.  Measured on the 13824 x 5120 weight: forward
// m = 512 (108 tiles) 0.117 ms on 128 x 128 tiles against 0.144, m = 768
// (162) 0.145 against 0.160; backward m = 768 0.336 against 0.392, m = 1024
// 0.393 against 0.483.
bool use_big(bool forward, int64_t M, int64_t ncol, int64_t kred)
{
    if (!big_eligible(forward, M, ncol, kred)) return false;
    if (forward) return ((M + kXM - 1) / kXM) * ((ncol + kXN - 1) / kXN) >= kPlanCus / 2;
    return ((M + kBM - 1) / kBM) * (ncol / kBN) > kPlanCus;
}

// With a workspace, when the 256 x 256 tiles do not fill a round, their
// reduction (80 k-steps forward and 216 backward on the FFN weight) is split
// across workgroups (fp32 partials added in split order).  The split count
// minimises rounds x k-steps per split plus the partials' traffic (about 0.05
// k-step per (tile, split) workgroup: 512 KB written and read back at ~5 TB/s
// against ~2 us per k-step), at least 16 k-steps per split and at most 16
// splits, and is taken when it saves at least 15%.  0: no split.
int big_splits(bool forward, int64_t M, int64_t ncol, int64_t kred)
{
    if (!big_eligible(forward, M, ncol, kred)) return 0;
    const int64_t tiles = ((M + kXM - 1) / kXM) * ((ncol + kXN - 1) / kXN), ksteps = kred / 64;
    if (tiles >= kPlanCus) return 0;
    int64_t best = 1;
    double best_cost = 0.85 * (double)ksteps;   // one round, unsplit, less the margin a split must win by
    for (int64_t sp = 2; sp <= 16 && sp <= ksteps / 16; ++sp) {
        const int64_t rounds = (tiles * sp + kPlanCus - 1) / kPlanCus, per = (ksteps + sp - 1) / sp;
        const double cost = (double)(rounds * per) + 0.05 * (double)(tiles * sp);
        if (cost < best_cost) {
            best_cost = cost;
            best = sp;
        }
    }
    if (best < 2) return 0;
    const int64_t per = (ksteps + best - 1) / best;
    return (int)((ksteps + per - 1) / per);
}

// With a workspace, the tiles left over after the last whole round of the
// 256 x 256 kernels (rem of them) run with their reduction split instead of as
// row pieces: floor(kPlanCus / rem) splits (at most 16, each of at least 16
// k-steps), so that all their (split, tile) workgroups make one round.  A row
// piece still dequantises the tile's whole weight slab for fewer MFMAs; a split
// is a whole tile's work over a part of the reduction, plus its fp32 partial
// (256 KB written and read back).  0: not taken (no leftover, or more than
// half a round of it).
int big_tail_splits(bool forward, int64_t M, int64_t ncol, int64_t kred, int64_t& full, int64_t& rem)
{
    if (!use_big(forward, M, ncol, kred)) return 0;
    const int64_t tiles = ((M + kXM - 1) / kXM) * ((ncol + kXN - 1) / kXN), ksteps = kred / 64;
    if (tiles <= kPlanCus) return 0;
    rem = tiles % kPlanCus;
    full = tiles - rem;
    if (rem == 0) return 0;
    int64_t sp = kPlanCus / rem;
    if (sp > 16) sp = 16;
    while (sp >= 2 && ksteps / sp < 16) --sp;
    if (sp < 2) return 0;
    const int64_t per = (ksteps + sp - 1) / sp;   // whole k-steps per split
    return (int)((ksteps + per - 1) / per);
}

// Row pieces for the tiles left over after the last whole round of one
// workgroup per CU (full whole tiles, rem left over): 64-row quarters when
// four per tile fit one round, else 128-row halves when two do, each split
// evenly across the 8 XCDs; 0 when neither applies.
int tail_pieces(int64_t total, int64_t ncu, int64_t& full, int64_t& rem)
{
    if (ncu <= 0 || total <= ncu) return 0;
    rem = total % ncu;
    full = total - rem;
    if (rem == 0 || full % 8 != 0) return 0;
    if (4 * rem <= ncu && rem % 2 == 0) return 4;
    if (2 * rem <= ncu && rem % 4 == 0) return 2;
    return 0;
}

// The whole tiles unsplit, then the leftover tiles' splits (one launch, one
// round), then k_tail_sum; all on the caller's stream, in order.
template <int DT, bool DQ, bool OUT_F32, bool FWD>
hipError_t big_tail_go(GemmArgs g, hipStream_t s)
{
    int64_t full = 0, rem = 0;
    if (big_tail_splits(FWD, g.M, g.ncol, g.kred, full, rem) != g.tail_split) return hipErrorInvalidValue;
    const int ksteps = (int)(g.kred / 64);
    g.nsplit = 1;
    g.nhalf = 0;
    g.pieces = 2;
    for (int64_t t0 = 0; t0 < full; t0 += kMaxGemmGrid) {
        const int64_t n = full - t0 < kMaxGemmGrid ? full - t0 : kMaxGemmGrid;
        g.tile0 = t0;
        if constexpr (FWD)
            hipLaunchKernelGGL((k_nf4_mm_fwd<DT, DQ, OUT_F32, false>), dim3((unsigned)n), dim3(256), 0, s, g);
        else
            hipLaunchKernelGGL((k_nf4_mm_bwd<DT, DQ, OUT_F32, false>), dim3((unsigned)n), dim3(256), 0, s, g);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    g.tile0 = 0;
    g.nfull = full;
    g.nhalf = rem;
    g.split_steps = (ksteps + g.tail_split - 1) / g.tail_split;
    const unsigned grid = (unsigned)(rem * g.tail_split);
    if constexpr (FWD)
        hipLaunchKernelGGL((k_nf4_mm_fwd<DT, DQ, OUT_F32, true>), dim3(grid), dim3(256), 0, s, g);
    else
        hipLaunchKernelGGL((k_nf4_mm_bwd<DT, DQ, OUT_F32, true>), dim3(grid), dim3(256), 0, s, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_tail_sum<DT, OUT_F32>), dim3((unsigned)(rem * 64)), dim3(256), 0, s, g);
    return hipGetLastError();
}

template <int DT, bool DQ, bool OUT_F32>
hipError_t mm_fwd_go(GemmArgs g, hipStream_t s)
{
    g.ntn = (g.ncol + kXN - 1) / kXN;
    g.ntiles = ((g.M + kXM - 1) / kXM) * g.ntn;
    if (g.tail_split > 0) return big_tail_go<DT, DQ, OUT_F32, true>(g, s);
    const int64_t total = g.ntiles * g.nsplit;
    // With one workgroup per CU, the tiles past the last whole round run in
    // row pieces when those fit one round.
    g.nfull = total;
    g.nhalf = 0;
    g.pieces = 2;
    int64_t full = 0, rem = 0;
    const int pieces = g.nsplit == 1 ? tail_pieces(total, cu_count(), full, rem) : 0;
    if (pieces > 0 && full + pieces * rem < kMaxGemmGrid) {
        g.nfull = full;
        g.nhalf = rem;
        g.pieces = pieces;
        g.tile0 = 0;
        hipLaunchKernelGGL((k_nf4_mm_fwd<DT, DQ, OUT_F32, false>), dim3((unsigned)(full + pieces * rem)), dim3(256),
                           0, s, g);
        return hipGetLastError();
    }
    for (int64_t t0 = 0; t0 < total; t0 += kMaxGemmGrid) {
        const int64_t n = total - t0 < kMaxGemmGrid ? total - t0 : kMaxGemmGrid;
        g.tile0 = t0;
        if (g.nsplit > 1)
            hipLaunchKernelGGL((k_nf4_mm_fwd<DT, DQ, OUT_F32, true>), dim3((unsigned)n), dim3(256), 0, s, g);
        else
            hipLaunchKernelGGL((k_nf4_mm_fwd<DT, DQ, OUT_F32, false>), dim3((unsigned)n), dim3(256), 0, s, g);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (g.nsplit > 1) {
        const int64_t n = g.M * g.ncol;
        const int64_t blocks = (n / 4 + 255) / 256;
        if (blocks > kMaxGemmGrid) return hipErrorInvalidValue;
        hipLaunchKernelGGL((k_splitk_sum<DT, OUT_F32>), dim3((unsigned)blocks), dim3(256), 0, s,
                           (const float*)g.part, g.nsplit, n, g.out);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <int DT, bool DQ, bool OUT_F32>
hipError_t mm_bwd_go(GemmArgs g, hipStream_t s)
{
    g.ntn = (g.ncol + kXN - 1) / kXN;
    g.ntiles = ((g.M + kXM - 1) / kXM) * g.ntn;
    if (g.tail_split > 0) return big_tail_go<DT, DQ, OUT_F32, false>(g, s);
    g.nfull = g.ntiles;
    g.nhalf = 0;
    g.tile0 = 0;
    g.pieces = 2;
    if (g.nsplit > 1) {
        // (tile, split) workgroups, each summing split_steps k-steps into an
        // fp32 partial tile; k_splitk_sum adds the splits in order
        const int64_t total = g.ntiles * g.nsplit;
        for (int64_t t0 = 0; t0 < total; t0 += kMaxGemmGrid) {
            const int64_t n = total - t0 < kMaxGemmGrid ? total - t0 : kMaxGemmGrid;
            g.tile0 = t0;
            hipLaunchKernelGGL((k_nf4_mm_bwd<DT, DQ, OUT_F32, true>), dim3((unsigned)n), dim3(256), 0, s, g);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        const int64_t n = g.M * g.ncol;
        const int64_t blocks = (n / 4 + 255) / 256;
        if (blocks > kMaxGemmGrid) return hipErrorInvalidValue;
        hipLaunchKernelGGL((k_splitk_sum<DT, OUT_F32>), dim3((unsigned)blocks), dim3(256), 0, s,
                           (const float*)g.part, g.nsplit, n, g.out);
        return hipGetLastError();
    }
    int64_t full = 0, rem = 0;
    const int pieces = tail_pieces(g.ntiles, cu_count(), full, rem);
    if (pieces > 0) {
        g.nfull = full;
        g.nhalf = rem;
        g.pieces = pieces;
    }
    const int64_t blocks = g.nfull + g.pieces * g.nhalf;
    if (blocks > kMaxGemmGrid) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_nf4_mm_bwd<DT, DQ, OUT_F32, false>), dim3((unsigned)blocks), dim3(256), 0, s, g);
    return hipGetLastError();
}

template <int DT, bool FWD, bool DQ, bool OUT_F32>
hipError_t gemm_go(GemmArgs g, hipStream_t s)
{
    // the 256 x 256 kernels, split as planned by nf4_matmul_splits or whole
    const bool big = g.nsplit > 1 ? big_splits(FWD, g.M, g.ncol, g.kred) == g.nsplit
                                  : use_big(FWD, g.M, g.ncol, g.kred);
    if (big) {
        if constexpr (FWD) return mm_fwd_go<DT, DQ, OUT_F32>(g, s);
        else return mm_bwd_go<DT, DQ, OUT_F32>(g, s);
    }
    const int64_t total = g.ntiles * g.nsplit;
    for (int64_t t0 = 0; t0 < total; t0 += kMaxGemmGrid) {
        const int64_t n = total - t0 < kMaxGemmGrid ? total - t0 : kMaxGemmGrid;
        g.tile0 = t0;
        if (g.nsplit > 1)
            hipLaunchKernelGGL((k_nf4_matmul<DT, FWD, DQ, OUT_F32, true>), dim3((unsigned)n), dim3(kGThreads),
                               0, s, g);
        else
            hipLaunchKernelGGL((k_nf4_matmul<DT, FWD, DQ, OUT_F32, false>), dim3((unsigned)n), dim3(kGThreads),
                               0, s, g);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (g.nsplit > 1) {
        const int64_t n = g.M * g.ncol;
        const int64_t blocks = (n / 4 + 255) / 256;
        if (blocks > kMaxGemmGrid) return hipErrorInvalidValue;
        hipLaunchKernelGGL((k_splitk_sum<DT, OUT_F32>), dim3((unsigned)blocks), dim3(256), 0, s,
                           (const float*)g.part, g.nsplit, n, g.out);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace

int nf4_matmul_splits(int64_t rows, int64_t cols, bool forward, int64_t m)
{
    // More than 128 rows of x and too few 256 x 256 tiles for a round: the
    // large-tile kernels with their reduction split (big_splits).
    // Where the large-tile kernels take the call whole (use_big): no split.
    // Otherwise the 128 x 128 kernel: with fewer output tiles than the chip
    // has CUs, each workgroup walks the whole reduction one dependent k-step
    // after another and the call is bound by that latency (0.083 ms for any
    // m <= 256 on a 13824 x 5120 weight); then aim at about 1,024 (tile,
    // split) workgroups, at most 16 splits of whole k-steps.  Measured on
    // that weight: split at m <= 128 0.038-0.051 ms forward (dequantise +
    // library GEMM 0.060-0.075), 0.063-0.070 backward (0.087-0.131); at 432
    // output tiles and 80 k-steps (m = 512 forward) a 3-way split was slower
    // than none: shapes are split below 256 tiles, or below 512 when the
    // reduction has 128 k-steps or more.
    const int64_t kred = forward ? cols : rows, ncol = forward ? rows : cols;
    const int bsp = big_splits(forward, m, ncol, kred);
    if (bsp > 0) return bsp;   // the 256 x 256 kernels, split
    if (use_big(forward, m, ncol, kred)) return 1;   // the 256 x 256 kernels, whole
    const int64_t tiles = ((m + kBM - 1) / kBM) * (ncol / kBN);
    const int64_t ksteps = kred / kBK;
    if (ksteps < 2 || tiles >= 512 || (tiles >= 256 && ksteps < 128)) return 1;
    int64_t sp = (1024 + tiles - 1) / tiles;
    if (sp > 16) sp = 16;
    if (sp > ksteps) sp = ksteps;
    const int64_t per = (ksteps + sp - 1) / sp;
    return (int)((ksteps + per - 1) / per);
}

int nf4_matmul_tail_splits(int64_t rows, int64_t cols, bool forward, int64_t m, int64_t* rem_out)
{
    // only where the 256 x 256 kernels take the call whole (no split planned)
    const int64_t kred = forward ? cols : rows, ncol = forward ? rows : cols;
    if (nf4_matmul_splits(rows, cols, forward, m) != 1) return 0;
    int64_t full = 0, rem = 0;
    const int sp = big_tail_splits(forward, m, ncol, kred, full, rem);
    if (sp > 0 && rem_out) *rem_out = rem;
    return sp;
}

namespace {

// Super-chunks per part: about 2,048 (row group, part) waves, at most
// kGvMaxSc / mb super-chunks each (mb: 16-row blocks of x).
int gemv_part_sc(int64_t rows, int64_t cols, int mb)
{
    const int64_t groups = rows / 16, nsc = cols / 128, cap = kGvMaxSc / mb;
    int64_t sc = nsc * groups / 2048;
    return (int)(sc < 1 ? 1 : sc > cap ? cap : sc);
}

int gemv_blocks(int64_t m) { return m <= 16 ? 1 : 2; }

}  // namespace

int nf4_gemv_parts(int64_t rows, int64_t cols, bool forward, int64_t m)
{
    if (!forward || m > 32) return 0;
    const int64_t sc = gemv_part_sc(rows, cols, gemv_blocks(m)), nsc = cols / 128;
    return (int)((nsc + sc - 1) / sc);
}

namespace {

template <int DT, bool DQ, bool OUT_F32>
hipError_t gemv_go(const GemvArgs& g, int parts, void* out, hipStream_t s)
{
    const int64_t blocks = (g.groups + 3) / 4;
    if (blocks > kMaxGemmGrid || parts > 65535) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks, (unsigned)parts);
    if (g.m <= 16) hipLaunchKernelGGL((k_nf4_gemv16<DT, DQ, 1>), grid, dim3(256), 0, s, g);
    else hipLaunchKernelGGL((k_nf4_gemv16<DT, DQ, 2>), grid, dim3(256), 0, s, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = g.m * g.rows;
    hipLaunchKernelGGL((k_splitk_sum<DT, OUT_F32>), dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, s,
                       (const float*)g.part, parts, n, out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_nf4_gemv(int dtype, const uint8_t* codes, const int8_t* qabsmax, const float* scale2,
                           const float* absmax, int64_t rows, int64_t cols, const void* x, int64_t m,
                           void* out, bool out_f32, float* part, int parts, hipStream_t s)
{
    GemvArgs g;
    g.x = static_cast<const uint16_t*>(x);
    g.codes = codes;
    g.qabsmax = qabsmax;
    g.scale2 = scale2;
    g.absmax = absmax;
    g.rows = rows;
    g.cols = cols;
    g.m = m;
    g.groups = rows / 16;
    if (g.groups % 4 != 0 || m < 1 || m > 32) return hipErrorInvalidValue;   // whole workgroups of live waves
    g.part_sc = gemv_part_sc(rows, cols, gemv_blocks(m));
    if ((cols / 128 + g.part_sc - 1) / g.part_sc != parts) return hipErrorInvalidValue;
    g.part = part;
    const bool dq = qabsmax != nullptr;
    if (dtype == 0) {
        if (dq) return out_f32 ? gemv_go<0, true, true>(g, parts, out, s) : gemv_go<0, true, false>(g, parts, out, s);
        return out_f32 ? gemv_go<0, false, true>(g, parts, out, s) : gemv_go<0, false, false>(g, parts, out, s);
    }
    if (dq) return out_f32 ? gemv_go<1, true, true>(g, parts, out, s) : gemv_go<1, true, false>(g, parts, out, s);
    return out_f32 ? gemv_go<1, false, true>(g, parts, out, s) : gemv_go<1, false, false>(g, parts, out, s);
}

hipError_t launch_nf4_matmul(int dtype, const uint8_t* codes, const int8_t* qabsmax, const float* scale2,
                             const float* absmax, int64_t rows, int64_t cols, bool forward,
                             const void* x, int64_t m, void* out, bool out_f32, float* part, int nsplit,
                             int tail_split, hipStream_t s)
{
    GemmArgs g;
    g.a = static_cast<const uint16_t*>(x);
    g.codes = codes;
    g.qabsmax = qabsmax;
    g.scale2 = scale2;
    g.absmax = absmax;
    g.cols = cols;
    g.out = out;
    g.M = m;
    g.kred = forward ? cols : rows;
    g.ncol = forward ? rows : cols;
    g.lda = g.kred;
    g.ldo = g.ncol;
    g.ntn = g.ncol / kBN;
    g.tile0 = 0;
    g.ntiles = ((m + kBM - 1) / kBM) * g.ntn;
    g.nfull = g.ntiles;
    g.nhalf = 0;
    g.pieces = 2;
    const int ksteps = (int)(g.kred / kBK);
    g.nsplit = (part && nsplit > 1) ? nsplit : 1;
    g.split_steps = (ksteps + g.nsplit - 1) / g.nsplit;
    g.part = part;
    g.tail_split = (part && g.nsplit == 1 && tail_split > 1) ? tail_split : 0;
    const bool dq = qabsmax != nullptr;
#define NF4_GEMM(T, F, D, O) return gemm_go<T, F, D, O>(g, s)
#define NF4_GEMM_DT(T)                                                                             \
    if (forward) {                                                                               \
        if (dq) { if (out_f32) NF4_GEMM(T, true, true, true); else NF4_GEMM(T, true, true, false); }     \
        else    { if (out_f32) NF4_GEMM(T, true, false, true); else NF4_GEMM(T, true, false, false); }   \
    } else {                                                                                     \
        if (dq) { if (out_f32) NF4_GEMM(T, false, true, true); else NF4_GEMM(T, false, true, false); }   \
        else    { if (out_f32) NF4_GEMM(T, false, false, true); else NF4_GEMM(T, false, false, false); } \
    }
    if (dtype == 0) { NF4_GEMM_DT(0) }
    NF4_GEMM_DT(1)
#undef NF4_GEMM_DT
#undef NF4_GEMM
}

}  // namespace nf4k
