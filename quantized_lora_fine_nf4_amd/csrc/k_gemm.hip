// k_gemm.hip -- NF4 dequantisation fused into the 16-bit matmul that consumes
// the weight, on gfx950 matrix cores (MFMA).
//
// QLoRA keeps the frozen weight in 4 bits and dequantises it on the fly for
// the forward and the backward pass ("QLoRA" paper summary page, How It
// Works); AQLoRA names that per-step dequantisation as where quantised
// fine-tuning loses its time (AQLoRA arXiv listing, English abstract).  Here
// the weight tile is dequantised straight into LDS, in the value the codec
// defines (y = RNE16(fl32(level[code] * dequantised absmax)), bitwise what
// nf4_dequantize writes), and multiplied there: the 16-bit weight never goes
// to HBM.
//
//   forward   out[m, n] = sum_k x[m, k] * W[n, k]      (x: m x cols, out: m x rows)
//   backward  out[m, k] = sum_n x[m, n] * W[n, k]      (x: m x rows, out: m x cols)
//
// One kernel serves both: the first operand A is always row-major with the
// reduction index contiguous (x, or the output gradient); the W tile is
// stored in LDS with the reduction index contiguous too -- in W's own order
// forward, transposed backward -- so the MFMA fragment reads are the same.
//
// Tiling: a 256-thread workgroup computes a 128 x 128 output tile in k-steps
// of 64 (one quantisation block of a W row forward); waves in a 2 x 2 grid,
// each 64 x 64 = 2 x 2 tiles of v_mfma_f32_32x32x16_bf16 with fp32
// accumulation.  The next step's A rows and W codes are loaded into registers
// (raw: no wait) while the current step multiplies; after a barrier they are
// dequantised into the single LDS buffer.  39 KB of LDS per workgroup lets 3
// workgroups share a CU, which measured faster than double buffering at 2.
// Level lookups read a 256-entry table of level pairs (one 8-byte read per
// code byte).  Tiles are handed out in groups of 4 row tiles, each XCD taking
// a contiguous run of that order.  Products of two bf16 values are exact in
// fp32; only the fp32 accumulation rounds.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nf4_format.h"
#include "nf4_internal.h"
#include "nf4_launch.h"

namespace nf4k {
namespace {

#ifndef NF4_GEMM_STAGES
#define NF4_GEMM_STAGES 1         // LDS buffers; one (two barriers per step) leaves room for 3 workgroups per CU
#endif
#ifndef NF4_GEMM_GROUP_M
#define NF4_GEMM_GROUP_M 4        // output row tiles per group of the tile order (0: row-major order)
#endif
#ifndef NF4_GEMM_XCD
#define NF4_GEMM_XCD 1            // give each XCD a contiguous run of the tile order
#endif
#ifndef NF4_GEMM_LUT2
#define NF4_GEMM_LUT2 1           // copies of a 256-entry table of level pairs (0: 16-entry level table)
#endif
#ifndef NF4_GEMM_WM
#define NF4_GEMM_WM 64            // output rows per wave
#endif
#ifndef NF4_GEMM_WN
#define NF4_GEMM_WN 64            // output columns per wave
#endif
constexpr int kGThreads = 256;
constexpr int kWM = NF4_GEMM_WM, kWN = NF4_GEMM_WN;
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
    int split_steps;        // k-steps per split
    float* part;            // nsplit > 1: fp32 partials [nsplit][M x ncol]
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
#if NF4_GEMM_LUT2
    // lv: 256 (level[b & 15], level[b >> 4]) pairs per copy, copy chosen by lane
    const f2* lp = (const f2*)lv + 256 * ((threadIdx.x & 63) % NF4_GEMM_LUT2);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const f2 p = lp[(c >> (8 * j)) & 255];
        r[j] = pack16<DT>(p.x * adq, p.y * adq);
    }
#else
#pragma unroll
    for (int j = 0; j < 4; ++j)
        r[j] = pack16<DT>(lv[(c >> (8 * j)) & 15] * adq, lv[(c >> (8 * j + 4)) & 15] * adq);
#endif
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

#ifndef NF4_GEMM_MIN_WG
#define NF4_GEMM_MIN_WG 3         // workgroups per CU the register allocation must allow
#endif

// PART: this workgroup sums one split of the reduction and stores it as an
// fp32 partial (k_splitk_sum adds the splits in order); otherwise the whole
// reduction, stored as fp32 or the 16-bit type.
template <int DT, bool FWD, bool DQ, bool OUT_F32, bool PART>
__global__ __launch_bounds__(kGThreads, NF4_GEMM_MIN_WG) void k_nf4_matmul(GemmArgs g)
{
    __shared__ __attribute__((aligned(16))) uint16_t s_a[NF4_GEMM_STAGES][kBM * kLdp];
    __shared__ __attribute__((aligned(16))) uint16_t s_w[NF4_GEMM_STAGES][kBN * kLdp];
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    // level tables from immediates: an indexed constant table would be a
    // memory load, waited for before the first tile's loads are issued
#if NF4_GEMM_LUT2
    __shared__ __attribute__((aligned(16))) float s_lv[2 * 256 * NF4_GEMM_LUT2];
    for (int i = t; i < 256 * NF4_GEMM_LUT2; i += kGThreads) {
        const int b = i & 255;
        s_lv[2 * i] = level_imm(b & 15);
        s_lv[2 * i + 1] = level_imm(b >> 4);
    }
#else
    __shared__ float s_lv[16];
    if (t < 16) s_lv[t] = level_imm(t);
#endif

    int64_t tile = g.tile0 + blockIdx.x;
    if (NF4_GEMM_XCD && (gridDim.x & 7) == 0)
        tile = g.tile0 + (int64_t)(blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    // splits are the outer index: each split covers every output tile
    const int split = PART ? (int)(tile / g.ntiles) : 0;
    if (PART) tile -= (int64_t)split * g.ntiles;
    int64_t mt, nt;
    if (NF4_GEMM_GROUP_M > 0) {
        const int64_t per = (int64_t)NF4_GEMM_GROUP_M * g.ntn;
        const int64_t first = (tile / per) * NF4_GEMM_GROUP_M;
        const int64_t mtiles = (g.M + kBM - 1) / kBM;
        const int64_t gsz = mtiles - first < NF4_GEMM_GROUP_M ? mtiles - first : NF4_GEMM_GROUP_M;
        const int64_t in = tile % per;
        mt = first + in % gsz;
        nt = in / gsz;
    } else {
        mt = tile / g.ntn;
        nt = tile % g.ntn;
    }
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
    store_step<DT, FWD, DQ>(regs, s_a[0], s_w[0], s_lv);
    __syncthreads();

    for (int s = 0; s < nsteps; ++s) {
        const int cur = NF4_GEMM_STAGES == 2 ? (s & 1) : 0;
        const bool more = s + 1 < nsteps;
        if (more) load_step<FWD, DQ>(regs, g, m0, c0, kb + (int64_t)(s + 1) * kBK);
        const uint16_t* As = s_a[cur];
        const uint16_t* Ws = s_w[cur];
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
        if (NF4_GEMM_STAGES == 1) __syncthreads();   // every wave done reading the one buffer
        if (more) store_step<DT, FWD, DQ>(regs, s_a[cur ^ (NF4_GEMM_STAGES - 1)],
                                      s_w[cur ^ (NF4_GEMM_STAGES - 1)], s_lv);
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

// One-shot launches of at most 2^32 / 256 - 1 workgroups each.
constexpr int64_t kMaxGemmGrid = (int64_t(1) << 32) / kGThreads - 1;

template <int DT, bool FWD, bool DQ, bool OUT_F32>
hipError_t gemm_go(GemmArgs g, hipStream_t s)
{
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
    // With fewer output tiles than the chip has CUs, each workgroup walks the
    // whole reduction one dependent k-step after another and the call is bound
    // by that latency (0.083 ms for any m <= 256 on a 13824 x 5120 weight);
    // then aim at about 1,024 (tile, split) workgroups, at most 16 splits of
    // whole k-steps.  Measured on that weight: split at m <= 128 0.038-0.051 ms
    // forward (dequantise + library GEMM 0.060-0.075), 0.063-0.070 backward
    // (0.087-0.131); at 432 output tiles and 80 k-steps (m = 512 forward) a
    // 3-way split was slower than none, at 320 tiles and 216 k-steps (m = 1024
    // backward) a 4-way split faster (0.327 against 0.477 ms): shapes are split
    // below 256 tiles, or below 512 when the reduction has 128 k-steps or more.
    const int64_t kred = forward ? cols : rows, ncol = forward ? rows : cols;
    const int64_t tiles = ((m + kBM - 1) / kBM) * (ncol / kBN);
    const int64_t ksteps = kred / kBK;
    if (ksteps < 2 || tiles >= 512 || (tiles >= 256 && ksteps < 128)) return 1;
    int64_t sp = (1024 + tiles - 1) / tiles;
    if (sp > 16) sp = 16;
    if (sp > ksteps) sp = ksteps;
    const int64_t per = (ksteps + sp - 1) / sp;
    return (int)((ksteps + per - 1) / per);
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
                             hipStream_t s)
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
    const int ksteps = (int)(g.kred / kBK);
    g.nsplit = (part && nsplit > 1) ? nsplit : 1;
    g.split_steps = (ksteps + g.nsplit - 1) / g.nsplit;
    g.part = part;
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
