// Backward of starting-node triangle attention on gfx950 matrix cores: bf16 inputs, D = 32
// (the gradients of the definition; see kernel_backward.hip for the formulas and the
// plain fp32 version used for every other case).
//
// The bias reaches the kernels in two forms.  dq and dk/dv read it as fp16 relative to
// each query's reference r_j (the forward's prepass, and bias_imageT16_kernel for its
// transpose): x = (q.k + (r_j - lse) sqrt(D)) log2(e)/sqrt(D) + (bias + mask - r_j) log2(e)
// is the score minus lse in log2 units, with (r_j - lse) sqrt(D) seeding the matrix
// accumulator and the image taken by one v_fma_mix_f32.  dbias takes the bias out of its
// loop over rows: it sums 2^x' (dP - delta) with x' the score without the image term and
// multiplies the sums by 2^((bias + mask - r_j) log2(e)) once, from the raw bias.
//
// Kernels, each owning the sums it produces (no atomics, deterministic):
//   bwd_prep_kernel   dout -> bf16 copy, head-major [B, H, I, N, D] (the operand of the dP
//                     and dV products), delta = dout . out per query from that rounded
//                     dout, and -delta and nb' = (r_j - lse) sqrt(D)
//                     transposed to [b, i, h, j] (rows padded to whole 256-query tiles).
//   bwd_headmajor_kernel
//                     q, k, v -> head-major copies [B, H, I, N, D], which the three
//                     streaming kernels below copy into LDS (each head's rows contiguous).
//   bwd_dq_lds        2 lines x 128 queries per workgroup, 32-key blocks streamed through
//                     an LDS ring (the forward's shape):
//                       S^T = K Q^T + nb',  dP^T = V dO^T - delta,  dS^T = P^T dP^T,
//                       dQ^T += K^T dS^T
//   bwd_dkdv_lds      2 lines x 128 keys per workgroup, 32-query blocks streamed, in the
//                     orientation in which P and dS leave the accumulator as B operands:
//                       S = Q K^T + nb',  dP = dO V^T - delta,  dV^T += dO^T P,  dK^T += Q^T dS
//   bwd_dbias_lds     256 queries x 128 keys of one (b, h) per workgroup, rows i streamed:
//                       S^T = K Q^T,  dP^T = V dO^T - delta,  acc += 2^x'^T dP^T,
//                       dbias^T = E^T acc at the end (the bias is shared by all rows)
// Every streaming kernel copies its operands straight from global memory into a ring of
// LDS stages (global_load_lds_dwordx4, one barrier per block) and reads them from there;
// transposed operands come from ds_read_b64_tr_b16 on the natural [row][d] tiles.
// Operand layouts are those of v_mfma_f32_32x32x16_bf16 (see kernel_bf16_mfma.hip): A and
// B hold one row / column per lane with 8 consecutive k-values per half-wave; the
// 32x32 fp32 result gives lane l column l % 32 and, in register r, row
// 8*(r/4) + 4*(l/32) + r%4.  A result used as the B operand of the next product keeps
// that row order, and the A operand read transposed from LDS follows it.
#include "launch.h"

#include <cmath>
#include <cstddef>

namespace tri_attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int D = 32;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSqrtD = 5.656854249492381f;
constexpr float kScale = kLog2e / kSqrtD;        // S units (q.k + sqrt(D) bias) -> log2 units
constexpr float kInvSqrtD = 0.17677669529663687f;

#define LDS_ADDR(p) static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)(p)))

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 8 bf16 at element offset `off` (16-byte aligned), or zeros
__device__ __forceinline__ bf16x8 frag(const __bf16* base, int64_t off, bool ok) {
    bf16x8 z = {};
    if (ok) z = *reinterpret_cast<const bf16x8*>(base + off);
    return z;
}

// 16-byte chunk `part` (d = 8*part .. +7) of tile row `row` sits at chunk kv_chunk(row, part)
__host__ __device__ constexpr int kv_chunk(int row, int part) { return part ^ ((row >> 1) & 3); }

// fp16 bias tiles (64-byte rows of 32 columns): the 32 columns of a row are stored in the
// order of the 32x32 MFMA result registers, so a lane's 16 values are the two 16-byte parts
// 2*h2 and 2*h2 + 1 of its row; position 8*part + t of a row holds column part_col(part, t)
__host__ __device__ constexpr int part_col(int part, int t) {
    return 8 * (2 * (part & 1) + (t >> 2)) + 4 * (part >> 1) + (t & 3);
}
// fp16 value of register r (0..15) of a lane from its two parts h0 (registers 0..7) and h1
__device__ __forceinline__ float half_of(const u32x4& h0, const u32x4& h1, int r) {
    const uint32_t word = (r < 8 ? h0 : h1)[(r & 7) >> 1];
    return static_cast<float>(__builtin_bit_cast(f16x2, word)[r & 1]);
}

__device__ __forceinline__ void to_bf16(const f32x16& x, bf16x8& lo, bf16x8& hi) {
    lo = __builtin_convertvector(__builtin_shufflevector(x, x, 0, 1, 2, 3, 4, 5, 6, 7), bf16x8);
    hi = __builtin_convertvector(__builtin_shufflevector(x, x, 8, 9, 10, 11, 12, 13, 14, 15), bf16x8);
}

// ---------------------------------------------------------------------------------------
// One thread per (b, i, h, j) with j padded to NP: dout of query (b, i, j, h) rounded to
// bf16, delta = dout . out, and, transposed to [b, i, h, j] so that the row-streaming
// kernels copy whole rows, -delta (the seed of their dP accumulators, which then hold
// dP - delta) and nb' = (r_j - lse) sqrt(D) (the shift of the score against the query's
// reference; -inf for a query without any finite score, and for the padded j, whose delta
// is 0).
// Eight lanes per query: lane `part` reads elements 4 part .. 4 part + 3 of dout and out,
// so a wave reads 1 KB of contiguous rows per load; the partial dot products meet in three
// shuffle steps.  Threads run over (line, query padded to NP, head, part); the padded
// queries only write the padding of the transposed rows.
constexpr int PREP_PARTS = D / 4;
__global__ void __launch_bounds__(256) bwd_prep_kernel(BwdProblem p, __bf16* g16, float* delta, float* deltaT,
                                                       int64_t NP, const float* ref16, int64_t nqp16, float* nbT2) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t total = p.B * p.I * NP * p.H * PREP_PARTS;   // whole groups of 8 lanes
    if (t >= total) return;
    const int part = static_cast<int>(t % PREP_PARTS);
    const int64_t qh = t / PREP_PARTS, h = qh % p.H, lj = qh / p.H, j = lj % NP, line = lj / NP;
    const bool real = j < p.N;
    const int64_t q = (line * p.N + (real ? j : 0)) * p.H + h;
    const int64_t qhm = ((line / p.I * p.H + h) * p.I + line % p.I) * p.N + j;   // head-major position of g16
    float dl = 0.0f;
    if (real) {
        // delta from the same bf16-rounded dout that the dP products use: dS = P (dP - delta)
        // is then the gradient for that rounded dout, and its rows still sum to zero
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        const f32x4 g = *reinterpret_cast<const f32x4*>(p.dout + q * D + 4 * part);
        const f32x4 o = *reinterpret_cast<const f32x4*>(p.out + q * D + 4 * part);
        const bf16x4 gb = __builtin_convertvector(g, bf16x4);
        const f32x4 gr = __builtin_convertvector(gb, f32x4);
#pragma unroll
        for (int e = 0; e < 4; ++e) dl = fmaf(gr[e], o[e], dl);
        *reinterpret_cast<bf16x4*>(g16 + qhm * D + 4 * part) = gb;
    }
    static_assert(PREP_PARTS == 8, "three shuffle steps");
    dl += __shfl_xor(dl, 1);
    dl += __shfl_xor(dl, 2);
    dl += __shfl_xor(dl, 4);
    if (part == 0) {
        const int64_t tt = (line * p.H + h) * NP + j;   // [b, i, h, j]
        if (real) delta[q] = dl;
        deltaT[tt] = -dl;                               // seeds the dP accumulators
        const float lse = real ? p.lse[q] : -INFINITY;
        // (r_j - lse) sqrt(D): with the fp16 image relative to r_j, the score in log2 units is
        // (q.k + this) * log2(e)/sqrt(D) + image
        const int64_t b = line / p.I;
        nbT2[tt] = lse == -INFINITY ? -INFINITY : (ref16[(b * p.H + h) * nqp16 + j] - lse) * kSqrtD;
    }
}

// q, k, v copied head-major, [B, H, I, N, D]: the streaming kernels then copy each head's
// rows as contiguous 64-byte runs instead of 64 bytes out of every 256 (the other heads'
// bytes share their lines).  Thread t moves 16 bytes: part t % 4 of head (t / 4) % H of
// position t / (4 H), so a wave reads 1 KB of contiguous positions and writes 256
// contiguous bytes per head; grid.y picks q, k or v.  (5.6 GB moved at N = 2700, about
// 1.9 ms: near the bandwidth the other streaming kernels see.)
__global__ void __launch_bounds__(256) bwd_headmajor_kernel(BwdProblem p, __bf16* qh, __bf16* kh, __bf16* vh) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t total = p.B * p.I * p.N * p.H * 4;
    if (t >= total) return;
    const int part = static_cast<int>(t & 3);
    const int64_t h = (t >> 2) % p.H, pos = (t >> 2) / p.H;   // pos = (b * I + i) * N + j
    const int64_t IN = p.I * p.N, b = pos / IN, rem = pos - b * IN;
    const __bf16* src = blockIdx.y == 0 ? static_cast<const __bf16*>(p.q) : blockIdx.y == 1 ? static_cast<const __bf16*>(p.k)
                                                                                             : static_cast<const __bf16*>(p.v);
    __bf16* dst = blockIdx.y == 0 ? qh : blockIdx.y == 1 ? kh : vh;
    *reinterpret_cast<u32x4*>(dst + ((b * p.H + h) * IN + rem) * D + 8 * part) =
        *reinterpret_cast<const u32x4*>(src + (pos * p.H + h) * D + 8 * part);
}

#define GPTR(p) ((const __attribute__((address_space(1))) void*)(p))
#define LPTR(p) ((__attribute__((address_space(3))) void*)(p))
__device__ __forceinline__ void db_barrier_drain() { asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---------------------------------------------------------------------------------------
// dq, in the forward's shape: a workgroup of 4 waves owns DQ_R = 2 lines (rows i) x 128
// query columns of one (b, h) and streams 32-key blocks through a ring of 4 LDS stages of
// 16 KB (K, V of its lines and its 128 rows of the forward's fp16 image tile, copied by
// global_load_lds); two workgroups share a compute unit.  Wave w owns line w / 2 and query
// tiles 2 (w % 2), +1; Q and dO of its queries stay in registers.  Per unit and block:
//   S^T = K Q^T + nb',  dP^T = V dO^T - delta,  dS^T = P^T dP^T,  dQ^T += K^T dS^T
// with K^T read transposed from the staged [key][d] tile (ds_read_b64_tr_b16).
#ifndef TRI_ATTN_DQ_WAVES
#define TRI_ATTN_DQ_WAVES 4
#endif
#ifndef TRI_ATTN_DQ_STAGES
#define TRI_ATTN_DQ_STAGES 4
#endif
#ifndef TRI_ATTN_DQ_TILE_RG
#define TRI_ATTN_DQ_TILE_RG 16
#endif
constexpr int DQ_WAVES = TRI_ATTN_DQ_WAVES;
constexpr int DQ_R = DQ_WAVES / 2;          // lines per workgroup: two waves per line
constexpr int DQ_THR = 64 * DQ_WAVES;
constexpr int DQ_STAGES = TRI_ATTN_DQ_STAGES;
constexpr int DQ_TILE_RG = TRI_ATTN_DQ_TILE_RG;   // line groups x column blocks one XCD works on together
constexpr int DQ_TILE_JB = 4;
struct DqStage {
    __bf16 k[DQ_R][32][D];     // 64-byte rows, 16-byte chunks swizzled by kv_chunk()
    __bf16 v[DQ_R][32][D];
    _Float16 bias[IMG_BJ][32];    // 128 queries of the fp16 image tile (relative to r_j) as stored
};
constexpr int DQ_STAGE_BYTES = static_cast<int>(sizeof(DqStage));
constexpr int DQ_K_OFF = static_cast<int>(offsetof(DqStage, k));
constexpr int DQ_V_OFF = static_cast<int>(offsetof(DqStage, v));
constexpr int DQ_B_OFF = static_cast<int>(offsetof(DqStage, bias));
constexpr int DQ_LINE_BYTES = 32 * D * 2;
constexpr int DQ_CTILE_BYTES = 32 * 32 * 2;           // 32 query rows of the fp16 tile
constexpr int DQ_BIAS_PER_WAVE = IMG_BJ * 32 * 2 / 1024 / DQ_WAVES;
constexpr int DQ_COPIES = 2 + DQ_BIAS_PER_WAVE;   // global_load_lds per wave per block
static_assert(DQ_LINE_BYTES == 2048 && DQ_CTILE_BYTES == 2048, "offsets below");
static_assert(DQ_R * 2 * 2 == 2 * DQ_WAVES && DQ_BIAS_PER_WAVE * DQ_WAVES * 1024 == IMG_BJ * 32 * 2,
              "two K/V pieces and whole bias pieces per wave");
__shared__ DqStage g_dq[DQ_STAGES];

struct DqCtx {
    const char* kv_row[2];     // K or V of the staged line at key 0
    uint32_t kv_lds[2];
    int key_local[2];
    int part_bytes[2];
    uint32_t lane_off[2];      // key_local * key_bytes + part_bytes: the lane's source offset in a block
    const _Float16* img_wg;    // this workgroup's 128 rows of the fp16 image tile of key block 0
    int64_t img_blk;           // halves between the tiles of consecutive key blocks
    int64_t key_bytes;
    int last_key;
};

// Copy sources are a wave-uniform base (the block's first key, the block's image tile) plus
// a 32-bit lane offset fixed for the loop, so the copies take the scalar-base address form;
// only the last, partial block clamps its padded keys to the last real one.  The empty asm
// statements keep the compiler from folding the offsets into 64-bit vector pointers.
__device__ __forceinline__ void dq_stage(const DqCtx& cx, int n, int wave, int lane) {
    char* lds = reinterpret_cast<char*>(&g_dq[n % DQ_STAGES]);
    const int kb = 32 * n;
    const int lim = cx.last_key - kb;   // last real key of the block, block-relative
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        uint32_t off = cx.lane_off[t];
        if (lim < 31)
            off = static_cast<uint32_t>(min(cx.key_local[t], lim) * static_cast<int>(cx.key_bytes) + cx.part_bytes[t]);
        asm volatile("" : "+v"(off));
        const char* base = cx.kv_row[t] + static_cast<int64_t>(kb) * cx.key_bytes;
        __builtin_amdgcn_global_load_lds(GPTR(base + off), LPTR(lds + cx.kv_lds[t]), 16, 0, 0);
    }
    const char* tile = reinterpret_cast<const char*>(cx.img_wg + n * cx.img_blk);
#pragma unroll
    for (int t = 0; t < DQ_BIAS_PER_WAVE; ++t) {
        const int base = (DQ_BIAS_PER_WAVE * wave + t) * 1024;
        uint32_t off = static_cast<uint32_t>(lane * 16 + base);
        asm volatile("" : "+v"(off));
        __builtin_amdgcn_global_load_lds(GPTR(tile + off), LPTR(lds + DQ_B_OFF + base), 16, 0, 0);
    }
}

// barrier after which every wave's copies except those of the DQ_STAGES - 2 newest blocks are complete
__device__ __forceinline__ void dq_barrier_keep() {
    constexpr int keep = DQ_COPIES * (DQ_STAGES - 2);
    static_assert(keep >= 1 && keep <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%c0)\n\ts_barrier" ::"i"(keep) : "memory");
}

// True when any column block of (b, h) holds bias beyond the fp16 image's span (the
// prepass's flags): dq and dk/dv of that (b, h) are then left to the fp32 kernels.
__device__ __forceinline__ bool any_wide(const int* wide, int64_t bh, int n) {
    int any = 0;
    for (int t = 0; t < n; ++t) any |= wide[bh * n + t];
    return any != 0;
}

__global__ void __launch_bounds__(DQ_THR, 2) bwd_dq_lds(BwdProblem p, const _Float16* img16, const float* ref16,
                                                     Prepass16 pre, const int* wide, const __bf16* g16,
                                                     const __bf16* kh, const __bf16* vh,
                                                     const float* delta, int n_jb, int n_rg, int nblk, int total) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 31, h2 = lane >> 5;
    // XCD-aware remap (as in the forward): strips of DQ_TILE_RG line groups cut into tiles
    // of DQ_TILE_RG x DQ_TILE_JB, column block fastest
    const int w = blockIdx.x;
    const int xcd = w % 8, slot = w / 8;
    const int base = total / 8, extra = total % 8;
    const int logical = xcd * base + (xcd < extra ? xcd : extra) + slot;
    const int bh = logical / (n_jb * n_rg);
    const int rem = logical - bh * n_jb * n_rg;
    const int strip = rem / (DQ_TILE_RG * n_jb);
    const int nr = min(DQ_TILE_RG, n_rg - strip * DQ_TILE_RG);
    const int o = rem - strip * DQ_TILE_RG * n_jb;
    const int tile = o / (nr * DQ_TILE_JB);
    const int nj = min(DQ_TILE_JB, n_jb - tile * DQ_TILE_JB);
    const int o2 = o - tile * nr * DQ_TILE_JB;
    const int rg = strip * DQ_TILE_RG + o2 / nj;
    const int jb = tile * DQ_TILE_JB + o2 % nj;
    const int64_t N = p.N, H = p.H, HD = H * D, I = p.I;
    const int64_t b = bh / H, h = bh % H;
    const int64_t i0 = static_cast<int64_t>(rg) * DQ_R, j0 = static_cast<int64_t>(jb) * IMG_BJ;
    if (any_wide(wide, bh, static_cast<int>(pre.n_jb))) return;

    DqCtx cx;
    {
        cx.key_bytes = D * 2;   // head-major copies: one head's keys 64 bytes apart
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            // piece 2 w + t: line w / 2, K (w even) or V (w odd), keys 16 t .. +15
            const int line = wave >> 1, kv = wave & 1;
            int64_t i = i0 + line;
            i = i < I ? i : I - 1;                       // padded lines read a real line (never stored)
            cx.kv_row[t] = reinterpret_cast<const char*>((kv ? vh : kh) + (((b * H + h) * I + i) * N) * D);
            cx.kv_lds[t] = (kv ? DQ_V_OFF : DQ_K_OFF) + line * DQ_LINE_BYTES + t * 1024;
            cx.key_local[t] = 16 * t + (lane >> 2);
            cx.part_bytes[t] = kv_chunk(cx.key_local[t], lane & 3) * 16;
            cx.lane_off[t] = static_cast<uint32_t>(cx.key_local[t] * cx.key_bytes + cx.part_bytes[t]);
        }
        // the prepass tiles hold pre.cols queries; this block's 128 are rows (jb % sub) * 128 on
        const int sub = pre.cols / IMG_BJ;
        cx.img_blk = static_cast<int64_t>(pre.cols) * 32;
        cx.img_wg = img16 + (static_cast<int64_t>(bh) * pre.n_jb + jb / sub) * pre.nblk * cx.img_blk +
                    (jb % sub) * IMG_BJ * 32;
        cx.last_key = static_cast<int>(N - 1);
    }

    const int line = wave >> 1, t0 = 2 * (wave & 1);
    const int64_t i = i0 + line;
    const bool iok = i < I;
    const __bf16* q = static_cast<const __bf16*>(p.q);
    bf16x8 qB[2][2], gB[2][2];
    float nb[2], dl[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int64_t j = j0 + 32 * (t0 + u) + c;
        const bool ok = iok && j < N;
        const int64_t qo = ((b * I + i) * N + j) * HD + h * D;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            qB[u][m] = frag(q, qo + 16 * m + 8 * h2, ok);
            gB[u][m] = frag(g16, (((b * H + h) * I + i) * N + j) * D + 16 * m + 8 * h2, ok);
        }
        const int64_t qi = ((b * I + i) * N + j) * H + h;
        const float lse = ok ? p.lse[qi] : -INFINITY;
        // (r_j - lse) sqrt(D) seeds the score accumulator: see bwd_prep_kernel
        nb[u] = lse == -INFINITY ? -INFINITY : (ref16[bh * pre.nqp + j] - lse) * kSqrtD;
        dl[u] = ok ? delta[qi] : 0.0f;
    }
    // LDS byte offsets (stage 0) of this lane's reads: K and V rows (A of S and dP), the
    // transposed K reads (A of dQ), the bias chunks of its first tile (second tile +2048)
    uint32_t ak[2], at[4], ac[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) ak[m] = DQ_K_OFF + line * DQ_LINE_BYTES + c * 64 + kv_chunk(c, 2 * m + h2) * 16;
    {
        const int ii = lane & 15, d0 = 16 * ((lane >> 4) & 1) + 4 * (ii & 3);
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int sub = 0; sub < 2; ++sub) {
                const int key = 16 * m + 8 * sub + 4 * h2 + (ii >> 2);
                at[2 * m + sub] = DQ_K_OFF + line * DQ_LINE_BYTES + key * 64 + kv_chunk(key, d0 >> 3) * 16 + (d0 & 7) * 2;
            }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) ac[h] = DQ_B_OFF + t0 * DQ_CTILE_BYTES + c * 64 + kv_chunk(c, 2 * h2 + h) * 16;
    const uint32_t st0 = LDS_ADDR(&g_dq[0]);
    f32x16 nbs[2], ndl[2];            // accumulator seeds: (r_j - lse) sqrt(D) for S, -delta for dP
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            nbs[u][r] = nb[u];
            ndl[u][r] = -dl[u];
        }

    f32x16 dQ[2] = {};
    for (int n = 0; n < DQ_STAGES - 1 && n < nblk; ++n) dq_stage(cx, n, wave, lane);
    if (nblk >= DQ_STAGES - 1)
        dq_barrier_keep();
    else
        db_barrier_drain();
    for (int n = 0; n < nblk; ++n) {
        const uint32_t st = st0 + static_cast<uint32_t>(n % DQ_STAGES) * DQ_STAGE_BYTES;
        const bool issue = n + DQ_STAGES - 1 < nblk;
        if (issue) dq_stage(cx, n + DQ_STAGES - 1, wave, lane);
        u32x4 kk[2], vv[2], cc[4];
        u32x2 tt[4];
        asm volatile(
            "ds_read_b128 %0, %12\n\t"
            "ds_read_b128 %1, %13\n\t"
            "ds_read_b128 %2, %12 offset:%c20\n\t"
            "ds_read_b128 %3, %13 offset:%c20\n\t"
            "ds_read_b64_tr_b16 %4, %14\n\t"
            "ds_read_b64_tr_b16 %5, %15\n\t"
            "ds_read_b64_tr_b16 %6, %16\n\t"
            "ds_read_b64_tr_b16 %7, %17\n\t"
            "ds_read_b128 %8, %18\n\t"
            "ds_read_b128 %9, %19\n\t"
            "ds_read_b128 %10, %18 offset:%c21\n\t"
            "ds_read_b128 %11, %19 offset:%c21\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(kk[0]), "=&v"(kk[1]), "=&v"(vv[0]), "=&v"(vv[1]), "=&v"(tt[0]), "=&v"(tt[1]), "=&v"(tt[2]),
              "=&v"(tt[3]), "=&v"(cc[0]), "=&v"(cc[1]), "=&v"(cc[2]), "=&v"(cc[3])
            : "v"(st + ak[0]), "v"(st + ak[1]), "v"(st + at[0]), "v"(st + at[1]), "v"(st + at[2]), "v"(st + at[3]),
              "v"(st + ac[0]), "v"(st + ac[1]), "i"(DQ_V_OFF - DQ_K_OFF), "i"(DQ_CTILE_BYTES));
        bf16x8 kT[2];
#pragma unroll
        for (int m = 0; m < 2; ++m)
            kT[m] = __builtin_bit_cast(bf16x8, u32x4{tt[2 * m][0], tt[2 * m][1], tt[2 * m + 1][0], tt[2 * m + 1][1]});
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            f32x16 S = mfma(__builtin_bit_cast(bf16x8, kk[0]), qB[u][0], nbs[u]);
            S = mfma(__builtin_bit_cast(bf16x8, kk[1]), qB[u][1], S);
            f32x16 dP = mfma(__builtin_bit_cast(bf16x8, vv[0]), gB[u][0], ndl[u]);   // dP - delta
            dP = mfma(__builtin_bit_cast(bf16x8, vv[1]), gB[u][1], dP);
            f32x16 dS;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                dS[r] = __builtin_amdgcn_exp2f(fmaf(S[r], kScale, half_of(cc[2 * u], cc[2 * u + 1], r))) * dP[r];
            bf16x8 s0, s1;
            to_bf16(dS, s0, s1);
            dQ[u] = mfma(kT[0], s0, dQ[u]);
            dQ[u] = mfma(kT[1], s1, dQ[u]);
        }
        if (issue)
            dq_barrier_keep();
        else
            db_barrier_drain();
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int64_t j = j0 + 32 * (t0 + u) + c;
        if (iok && j < N) {
            float* o = p.dq + ((b * I + i) * N + j) * HD + h * D;
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                f32x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = dQ[u][4 * a + e] * kInvSqrtD;
                *reinterpret_cast<f32x4*>(o + 8 * a + 4 * h2) = x;
            }
        }
    }
}

// ---------------------------------------------------------------------------------------
// dk, dv: a workgroup of 4 waves owns DK_R = 2 lines x 128 keys of one (b, h) and streams
// 32-query blocks through a ring of 4 LDS stages (two workgroups per compute unit): Q and
// dO of its lines, the 128 x 32 fp16 transposed tile (bias_imageT16_kernel: row = key, 32
// queries, relative to each query's r_q) and nb' = (r_q - lse) sqrt(D), -delta of the
// block's queries.  Wave w owns line w / 2 and key tiles 2 (w % 2), +1 (lane = key; K and
// V of its keys stay in registers).  Per unit and block, in the orientation in which P and
// dS leave the accumulator as the B operands of the next products:
//   S = Q K^T + nb',  dP = dO V^T - delta,  dS = P dP,  dV^T += dO^T P,  dK^T += Q^T dS
// with Q^T, dO^T read transposed from the staged [query][d] tiles.  A dropped key
// (masked, or past the end) gets zero gradients.
#ifndef TRI_ATTN_DK_WAVES
#define TRI_ATTN_DK_WAVES 4
#endif
#ifndef TRI_ATTN_DK_STAGES
#define TRI_ATTN_DK_STAGES 4
#endif
#ifndef TRI_ATTN_DK_TILE_RG
#define TRI_ATTN_DK_TILE_RG 16
#endif
constexpr int DK_WAVES = TRI_ATTN_DK_WAVES;
constexpr int DK_R = DK_WAVES / 2;          // lines per workgroup: two waves per line
constexpr int DK_THR = 64 * DK_WAVES;
constexpr int DK_STAGES = TRI_ATTN_DK_STAGES;
constexpr int DK_TILE_RG = TRI_ATTN_DK_TILE_RG;
constexpr int DK_TILE_KB = 4;
struct DkStage {
    __bf16 q[DK_R][32][D];        // 64-byte rows, 16-byte chunks swizzled by kv_chunk()
    __bf16 g[DK_R][32][D];        // dO rounded to bf16
    _Float16 bias[IMG_BJ][32];    // the fp16 transposed tile: row = key, 32 queries (part_col order)
    float nb[DK_R][32];
    float dl[DK_R][32];
};
constexpr int DK_STAGE_BYTES = static_cast<int>(sizeof(DkStage));
constexpr int DK_Q_OFF = static_cast<int>(offsetof(DkStage, q));
constexpr int DK_G_OFF = static_cast<int>(offsetof(DkStage, g));
constexpr int DK_B_OFF = static_cast<int>(offsetof(DkStage, bias));
constexpr int DK_N_OFF = static_cast<int>(offsetof(DkStage, nb));
constexpr int DK_GQ = DK_G_OFF - DK_Q_OFF;                                     // dO tile after the Q tile
constexpr int DK_DN = static_cast<int>(offsetof(DkStage, dl) - offsetof(DkStage, nb));   // delta rows after nb rows
constexpr int DK_BIAS_PER_WAVE = IMG_BJ * 32 * 2 / 1024 / DK_WAVES;
constexpr int DK_COPIES = 2 + DK_BIAS_PER_WAVE + 1;   // Q/dO pieces, bias pieces, the nb or delta piece
static_assert(DK_BIAS_PER_WAVE * DK_WAVES * 1024 == IMG_BJ * 32 * 2 && 2 * DK_R == DK_WAVES, "pieces per wave");
__shared__ DkStage g_dk[DK_STAGES];

// barrier after which every wave's copies except those of the DK_STAGES - 2 newest blocks are complete
__device__ __forceinline__ void dk_barrier_keep() {
    constexpr int keep = DK_COPIES * (DK_STAGES - 2);
    static_assert(keep >= 1 && keep <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%c0)\n\ts_barrier" ::"i"(keep) : "memory");
}

struct DkCtx {
    const char* qg_row[2];     // Q or dO of the staged line at query 0
    uint32_t qg_lds[2];
    int q_local[2];
    int part_bytes[2];
    uint32_t lane_off[2];      // q_local * q_bytes + part_bytes: the lane's source offset in a block
    const _Float16* img_wg;    // this workgroup's fp16 transposed tiles, nqblk consecutive 128 x 32 tiles
    const char* ls_src;        // nb or delta row of the line at query 0 (wave-uniform)
    uint32_t ls_off;           // this lane's byte offset from it (lanes 0 .. 7)
    uint32_t ls_dst;
    int64_t q_bytes;
    int last_q;
};

// Copy sources in the scalar-base form, as dq_stage's; only the last, partial block clamps
// its padded queries to the last real one.
__device__ __forceinline__ void dk_stage(const DkCtx& cx, int n, int wave, int lane) {
    char* lds = reinterpret_cast<char*>(&g_dk[n % DK_STAGES]);
    const int qb = 32 * n;
    const int lim = cx.last_q - qb;   // last real query of the block, block-relative
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        uint32_t off = cx.lane_off[t];
        if (lim < 31)
            off = static_cast<uint32_t>(min(cx.q_local[t], lim) * static_cast<int>(cx.q_bytes) + cx.part_bytes[t]);
        asm volatile("" : "+v"(off));
        const char* base = cx.qg_row[t] + static_cast<int64_t>(qb) * cx.q_bytes;
        __builtin_amdgcn_global_load_lds(GPTR(base + off), LPTR(lds + cx.qg_lds[t]), 16, 0, 0);
    }
    const char* tile = reinterpret_cast<const char*>(cx.img_wg + static_cast<int64_t>(n) * IMG_BJ * 32);
#pragma unroll
    for (int t = 0; t < DK_BIAS_PER_WAVE; ++t) {
        const int base = (DK_BIAS_PER_WAVE * wave + t) * 1024;
        uint32_t off = static_cast<uint32_t>(lane * 16 + base);
        asm volatile("" : "+v"(off));
        __builtin_amdgcn_global_load_lds(GPTR(tile + off), LPTR(lds + DK_B_OFF + base), 16, 0, 0);
    }
    if (lane < 8) {
        uint32_t off = cx.ls_off;
        asm volatile("" : "+v"(off));
        __builtin_amdgcn_global_load_lds(GPTR(cx.ls_src + qb * 4 + off), LPTR(lds + cx.ls_dst), 16, 0, 0);
    }
}

__global__ void __launch_bounds__(DK_THR, 2) bwd_dkdv_lds(BwdProblem p, const _Float16* imgT16, const int* wide,
                                                       int n_wide, const __bf16* g16, const __bf16* qh,
                                                       const float* nbT2,
                                                       const float* deltaT, int n_kb, int n_rg, int nqblk, int64_t NP,
                                                       int total) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 31, h2 = lane >> 5;
    const int w = blockIdx.x;
    const int xcd = w % 8, slot = w / 8;
    const int base = total / 8, extra = total % 8;
    const int logical = xcd * base + (xcd < extra ? xcd : extra) + slot;
    const int bh = logical / (n_kb * n_rg);
    const int rem = logical - bh * n_kb * n_rg;
    const int strip = rem / (DK_TILE_RG * n_kb);
    const int nr = min(DK_TILE_RG, n_rg - strip * DK_TILE_RG);
    const int o = rem - strip * DK_TILE_RG * n_kb;
    const int tile = o / (nr * DK_TILE_KB);
    const int nk = min(DK_TILE_KB, n_kb - tile * DK_TILE_KB);
    const int o2 = o - tile * nr * DK_TILE_KB;
    const int rg = strip * DK_TILE_RG + o2 / nk;
    const int kb = tile * DK_TILE_KB + o2 % nk;
    const int64_t N = p.N, H = p.H, HD = H * D, I = p.I;
    const int64_t b = bh / H, h = bh % H;
    const int64_t i0 = static_cast<int64_t>(rg) * DK_R, k0 = static_cast<int64_t>(kb) * IMG_BJ;
    if (any_wide(wide, bh, n_wide)) return;

    DkCtx cx;
    {
        cx.q_bytes = D * 2;   // head-major copies: one head's queries 64 bytes apart
        const int sline = wave >> 1, qg = wave & 1;   // pieces of wave w: line w / 2, Q (w even) or dO, both halves
        int64_t i = i0 + sline;
        i = i < I ? i : I - 1;                         // padded lines read a real line (never stored)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            cx.qg_row[t] = reinterpret_cast<const char*>((qg ? g16 : qh) + (((b * H + h) * I + i) * N) * D);
            cx.qg_lds[t] = (qg ? DK_G_OFF : DK_Q_OFF) + sline * 2048 + t * 1024;
            cx.q_local[t] = 16 * t + (lane >> 2);
            cx.part_bytes[t] = kv_chunk(cx.q_local[t], lane & 3) * 16;
            cx.lane_off[t] = static_cast<uint32_t>(cx.q_local[t] * cx.q_bytes + cx.part_bytes[t]);
        }
        cx.img_wg = imgT16 + (static_cast<int64_t>(bh) * n_kb + kb) * nqblk * static_cast<int64_t>(IMG_BJ * 32);
        // nb' of line w (w < DK_R) or -delta of line w - DK_R, 32 floats of the block in lanes 0 .. 7
        int64_t il = i0 + wave % DK_R;
        il = il < I ? il : I - 1;
        cx.ls_src = reinterpret_cast<const char*>((wave < DK_R ? nbT2 : deltaT) + ((b * I + il) * H + h) * NP);
        cx.ls_off = static_cast<uint32_t>(16 * (lane & 7));
        cx.ls_dst = DK_N_OFF + 128 * wave;
        cx.last_q = static_cast<int>(N - 1);
    }

    const int line = wave >> 1, t0 = 2 * (wave & 1);
    const int64_t i = i0 + line;
    const bool iok = i < I;
    const __bf16* kp = static_cast<const __bf16*>(p.k);
    const __bf16* vp = static_cast<const __bf16*>(p.v);
    bf16x8 kB[2][2], vB[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int64_t key = k0 + 32 * (t0 + u) + c;
        const int64_t ko = ((b * I + i) * N + key) * HD + h * D;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            kB[u][m] = frag(kp, ko + 16 * m + 8 * h2, iok && key < N);
            vB[u][m] = frag(vp, ko + 16 * m + 8 * h2, iok && key < N);
        }
    }
    // LDS byte offsets (stage 0) of this lane's reads: Q and dO rows (A of S and dP), the
    // transposed reads of Q and dO (A of dK, dV), the bias chunks of its first key tile
    // (second tile +2048), and nb' / -delta of its 16 query rows 8a + 4 h2 + e
    uint32_t aq[2], at[4], ac[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) aq[m] = DK_Q_OFF + line * 2048 + c * 64 + kv_chunk(c, 2 * m + h2) * 16;
    {
        const int ii = lane & 15, d0 = 16 * ((lane >> 4) & 1) + 4 * (ii & 3);
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int sub = 0; sub < 2; ++sub) {
                const int row = 16 * m + 8 * sub + 4 * h2 + (ii >> 2);
                at[2 * m + sub] = DK_Q_OFF + line * 2048 + row * 64 + kv_chunk(row, d0 >> 3) * 16 + (d0 & 7) * 2;
            }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) ac[h] = DK_B_OFF + t0 * 2048 + c * 64 + kv_chunk(c, 2 * h2 + h) * 16;
    const uint32_t an = DK_N_OFF + line * 128 + 16 * h2;
    const uint32_t st0 = LDS_ADDR(&g_dk[0]);

    f32x16 dK[2] = {}, dV[2] = {};
    for (int n = 0; n < DK_STAGES - 1 && n < nqblk; ++n) dk_stage(cx, n, wave, lane);
    if (nqblk >= DK_STAGES - 1)
        dk_barrier_keep();
    else
        db_barrier_drain();
    for (int n = 0; n < nqblk; ++n) {
        const uint32_t st = st0 + static_cast<uint32_t>(n % DK_STAGES) * DK_STAGE_BYTES;
        const bool issue = n + DK_STAGES - 1 < nqblk;
        if (issue) dk_stage(cx, n + DK_STAGES - 1, wave, lane);
        u32x4 qq[2], gg[2], nn[4], dd[4], cc[2][2];
        u32x2 tq[4], tg[4];
        asm volatile(
            "ds_read_b128 %0, %24\n\t"
            "ds_read_b128 %1, %25\n\t"
            "ds_read_b128 %2, %24 offset:%c33\n\t"
            "ds_read_b128 %3, %25 offset:%c33\n\t"
            "ds_read_b64_tr_b16 %4, %26\n\t"
            "ds_read_b64_tr_b16 %5, %27\n\t"
            "ds_read_b64_tr_b16 %6, %28\n\t"
            "ds_read_b64_tr_b16 %7, %29\n\t"
            "ds_read_b64_tr_b16 %8, %26 offset:%c33\n\t"
            "ds_read_b64_tr_b16 %9, %27 offset:%c33\n\t"
            "ds_read_b64_tr_b16 %10, %28 offset:%c33\n\t"
            "ds_read_b64_tr_b16 %11, %29 offset:%c33\n\t"
            "ds_read_b128 %12, %30\n\t"
            "ds_read_b128 %13, %30 offset:32\n\t"
            "ds_read_b128 %14, %30 offset:64\n\t"
            "ds_read_b128 %15, %30 offset:96\n\t"
            "ds_read_b128 %16, %30 offset:%c34\n\t"
            "ds_read_b128 %17, %30 offset:%c35\n\t"
            "ds_read_b128 %18, %30 offset:%c36\n\t"
            "ds_read_b128 %19, %30 offset:%c37\n\t"
            "ds_read_b128 %20, %31\n\t"
            "ds_read_b128 %21, %32\n\t"
            "ds_read_b128 %22, %31 offset:2048\n\t"
            "ds_read_b128 %23, %32 offset:2048\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(qq[0]), "=&v"(qq[1]), "=&v"(gg[0]), "=&v"(gg[1]), "=&v"(tq[0]), "=&v"(tq[1]), "=&v"(tq[2]),
              "=&v"(tq[3]), "=&v"(tg[0]), "=&v"(tg[1]), "=&v"(tg[2]), "=&v"(tg[3]), "=&v"(nn[0]), "=&v"(nn[1]),
              "=&v"(nn[2]), "=&v"(nn[3]), "=&v"(dd[0]), "=&v"(dd[1]), "=&v"(dd[2]), "=&v"(dd[3]), "=&v"(cc[0][0]),
              "=&v"(cc[0][1]), "=&v"(cc[1][0]), "=&v"(cc[1][1])
            : "v"(st + aq[0]), "v"(st + aq[1]), "v"(st + at[0]), "v"(st + at[1]), "v"(st + at[2]), "v"(st + at[3]),
              "v"(st + an), "v"(st + ac[0]), "v"(st + ac[1]), "i"(DK_GQ), "i"(DK_DN), "i"(DK_DN + 32), "i"(DK_DN + 64),
              "i"(DK_DN + 96));
        bf16x8 qT[2], gT[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            qT[m] = __builtin_bit_cast(bf16x8, u32x4{tq[2 * m][0], tq[2 * m][1], tq[2 * m + 1][0], tq[2 * m + 1][1]});
            gT[m] = __builtin_bit_cast(bf16x8, u32x4{tg[2 * m][0], tg[2 * m][1], tg[2 * m + 1][0], tg[2 * m + 1][1]});
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            // the score accumulator starts from (r_q - lse) sqrt(D) of each query row
            f32x16 S;
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int e = 0; e < 4; ++e) S[4 * a + e] = __uint_as_float(nn[a][e]);
            S = mfma(__builtin_bit_cast(bf16x8, qq[0]), kB[u][0], S);
            S = mfma(__builtin_bit_cast(bf16x8, qq[1]), kB[u][1], S);
            // register r = 4a + e holds query row 8a + 4 h2 + e: nb' and -delta from nn[a][e],
            // dd[a][e] seed the two accumulators
            f32x16 dP;
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int e = 0; e < 4; ++e) dP[4 * a + e] = __uint_as_float(dd[a][e]);
            dP = mfma(__builtin_bit_cast(bf16x8, gg[0]), vB[u][0], dP);
            dP = mfma(__builtin_bit_cast(bf16x8, gg[1]), vB[u][1], dP);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                S[r] = __builtin_amdgcn_exp2f(fmaf(S[r], kScale, half_of(cc[u][0], cc[u][1], r)));
                dP[r] = S[r] * dP[r];
            }
            bf16x8 p0, p1, s0, s1;
            to_bf16(S, p0, p1);
            to_bf16(dP, s0, s1);
            dV[u] = mfma(gT[0], p0, dV[u]);
            dV[u] = mfma(gT[1], p1, dV[u]);
            dK[u] = mfma(qT[0], s0, dK[u]);
            dK[u] = mfma(qT[1], s1, dK[u]);
        }
        if (issue)
            dk_barrier_keep();
        else
            db_barrier_drain();
    }
    if (iok) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int64_t key = k0 + 32 * (t0 + u) + c;
            if (key >= N) continue;
            const bool dropped = p.mask && p.mask[b * N + key] == -INFINITY;
            const int64_t ko = ((b * I + i) * N + key) * HD + h * D;
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                f32x4 xk, xv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    xk[e] = dropped ? 0.0f : dK[u][4 * a + e] * kInvSqrtD;
                    xv[e] = dropped ? 0.0f : dV[u][4 * a + e];
                }
                *reinterpret_cast<f32x4*>(p.dk + ko + 8 * a + 4 * h2) = xk;
                *reinterpret_cast<f32x4*>(p.dv + ko + 8 * a + 4 * h2) = xv;
            }
        }
    }
}

// ---------------------------------------------------------------------------------------
// dbias[b, h, j, k] = sum over the rows i held of dS[i, j, k].  A workgroup of 8 waves owns
// DB_Q = 256 queries x DB_K = 128 keys of one (b, h) and streams the rows i through a ring
// of LDS stages: per row the waves copy Q, dO (its queries), K, V (its keys), nb' and -delta
// straight from global memory into a stage (global_load_lds_dwordx4), and wave w computes
// queries 64 (w % 4) .. +63 against keys 64 (w / 4) .. +63 (four 32 x 32 units) from LDS.
// The bias is the same in every row, so it leaves the loop: with r_j the query's reference
// (the forward prepass's) and E[j, k] = 2^((bias + mask - r_j) log2(e)),
//   p = 2^x' E,   x' = (q.k + (r_j - lse) sqrt(D)) log2(e) / sqrt(D),
// and the loop sums acc = sum_i 2^x' (dP - delta) from S^T = K Q^T and dP^T = V dO^T alone;
// dbias = E acc at the end (0 where E is 0: keys dropped by the mask).  Inside the image's
// span (every finite (bias + mask - r_j) log2(e) >= -32, or the (b, h) is left to the fp32
// kernel) a kept key has x' <= 32, so 2^x' stays finite.  Without bias registers a wave
// issues the next unit's four products under the current unit's exponentials.  Every sum
// over i runs in one lane in row order: deterministic.
#ifndef TRI_ATTN_DB_Q
#define TRI_ATTN_DB_Q 256
#endif
#ifndef TRI_ATTN_DB_WAVES
#define TRI_ATTN_DB_WAVES 8
#endif
#ifndef TRI_ATTN_DB_WG_PER_CU
#define TRI_ATTN_DB_WG_PER_CU 1
#endif
constexpr int DB_Q = TRI_ATTN_DB_Q;
constexpr int DB_K = 128;
constexpr int DB_WAVES = TRI_ATTN_DB_WAVES;
constexpr int DB_THR = 64 * DB_WAVES;
constexpr int DB_NQP = DB_Q / 64;               // 64-query pairs of tiles; wave = (query pair, key pair)
static_assert(DB_NQP * (DB_K / 64) == DB_WAVES, "one 64 x 64 block of four units per wave");
#ifndef TRI_ATTN_DB_STAGES
#define TRI_ATTN_DB_STAGES 3
#endif
constexpr int DB_STAGES = TRI_ATTN_DB_STAGES;
#ifndef TRI_ATTN_DB_TILE_J
#define TRI_ATTN_DB_TILE_J 4
#endif
#ifndef TRI_ATTN_DB_TILE_K
#define TRI_ATTN_DB_TILE_K 8
#endif
constexpr int DB_TILE_J = TRI_ATTN_DB_TILE_J;   // query tiles x key tiles one XCD works on together
constexpr int DB_TILE_K = TRI_ATTN_DB_TILE_K;
constexpr int NP_ALIGN = 256;                   // lse / delta rows padded to whole query tiles
static_assert(NP_ALIGN % DB_Q == 0 && NP_ALIGN % 128 == 0, "a query tile never crosses the padding");

struct DbStage {
    __bf16 q[DB_Q][D];     // 64-byte rows, 16-byte chunks swizzled by kv_chunk()
    __bf16 g[DB_Q][D];     // dO rounded to bf16
    __bf16 k[DB_K][D];
    __bf16 v[DB_K][D];
    float lse[DB_Q];       // nb' = (r_j - lse) sqrt(D)
    float dl[DB_Q];        // -delta
};
constexpr int DB_STAGE_BYTES = static_cast<int>(sizeof(DbStage));
constexpr int DB_Q_OFF = static_cast<int>(offsetof(DbStage, q));
constexpr int DB_G_OFF = static_cast<int>(offsetof(DbStage, g));
constexpr int DB_K_OFF = static_cast<int>(offsetof(DbStage, k));
constexpr int DB_V_OFF = static_cast<int>(offsetof(DbStage, v));
constexpr int DB_L_OFF = static_cast<int>(offsetof(DbStage, lse));
constexpr int DB_DL_OFF = static_cast<int>(offsetof(DbStage, dl));
constexpr int DB_PQ = DB_Q * D * 2 / 1024;      // 1 KB pieces of Q (and of dO)
constexpr int DB_PK = DB_K * D * 2 / 1024;      // 1 KB pieces of K (and of V)
constexpr int DB_PIECES = (2 * DB_PQ + 2 * DB_PK) / DB_WAVES;   // per wave and row
constexpr int DB_COPIES = DB_PIECES + 1;                        // + 256 bytes of lse or delta
static_assert(DB_PIECES * DB_WAVES == 2 * DB_PQ + 2 * DB_PK, "whole pieces per wave");
static_assert(DB_WAVES * 256 == 2 * DB_Q * 4, "lse / delta: 256 bytes per wave");
static_assert(DB_STAGES >= 2 && DB_STAGES * sizeof(DbStage) * TRI_ATTN_DB_WG_PER_CU <= 160 * 1024, "LDS ring");
static_assert(DB_COPIES * (DB_STAGES - 2) <= 63, "vmcnt range");
// offset written into the operand reads below
static_assert(DB_V_OFF - DB_K_OFF == 8192, "stage layout of the dbias operand reads");
__shared__ DbStage g_db[DB_STAGES];

// Copy sources are a wave-uniform base (the piece's first row at row i = 0) plus a 32-bit
// lane offset, the same for every piece (row lane / 4 of the piece, its swizzled part), so
// the copies take the scalar-base address form; a piece that runs past the last position
// (the last tile) takes per-lane offsets clamped to it.
struct DbCtx {
    const char* src[DB_PIECES];   // this wave's pieces: (b, i = 0, first row of the piece, h)
    int64_t first[DB_PIECES];     // position of the piece's first row
    uint32_t dst[DB_PIECES];      // byte offset of each piece inside a stage
    uint32_t off;                 // this lane's offset inside a piece
    int64_t N, pos_bytes;         // positions, bytes between consecutive positions
    int64_t row_step;             // bytes between rows i of one tensor
    const char* ls_src;           // nb' / delta piece of row 0 (lanes 0 .. 15)
    int64_t ls_step;              // bytes between rows i of nbT2
    uint32_t ls_dst;
};

__device__ __forceinline__ void db_stage(const DbCtx& cx, int64_t i, int slot, int lane) {
    char* base = reinterpret_cast<char*>(&g_db[slot]);
#pragma unroll
    for (int t = 0; t < DB_PIECES; ++t) {
        const char* row = cx.src[t] + i * cx.row_step;
        if (cx.first[t] + 15 < cx.N) {
            uint32_t off = cx.off;
            asm volatile("" : "+v"(off));
            __builtin_amdgcn_global_load_lds(GPTR(row + off), LPTR(base + cx.dst[t]), 16, 0, 0);
        } else {                             // padded rows read the last real one (a 64-bit address:
            const int64_t pos = min(cx.first[t] + (lane >> 2), cx.N - 1);   // the piece may start past it)
            __builtin_amdgcn_global_load_lds(GPTR(row + (pos - cx.first[t]) * cx.pos_bytes + (cx.off % 64)),
                                             LPTR(base + cx.dst[t]), 16, 0, 0);
        }
    }
    if (lane < 16) {
        uint32_t off = static_cast<uint32_t>(lane * 16);
        asm volatile("" : "+v"(off));
        __builtin_amdgcn_global_load_lds(GPTR(cx.ls_src + i * cx.ls_step + off), LPTR(base + cx.ls_dst), 16, 0, 0);
    }
}

// Barrier after which every wave's copies except those of the DB_STAGES - 2 newest rows
// are complete; with `drain`, all of them.
__device__ __forceinline__ void db_barrier_keep() {
    if constexpr (DB_STAGES == 2)
        db_barrier_drain();
    else
        asm volatile("s_waitcnt vmcnt(%c0)\n\ts_barrier" ::"i"(DB_COPIES * (DB_STAGES - 2)) : "memory");
}

// One row's operands of a wave: [tile][d-half] K of key tile ki, V, Q of query tile qi, dO;
// nb' and -delta per query tile.
struct DbOps {
    u32x4 kk[2][2], vv[2][2], qq[2][2], gg[2][2];
    float nb[2], dl[2];
};

// Reads a row's operands from its stage at `st` (LDS byte address) and waits for them.
__device__ __forceinline__ void db_read(uint32_t st, const uint32_t (&ok)[2], const uint32_t (&oq)[2], uint32_t ol,
                                        DbOps& o) {
    asm volatile(
        "ds_read_b128 %0, %20\n\t"
        "ds_read_b128 %1, %21\n\t"
        "ds_read_b128 %2, %20 offset:2048\n\t"
        "ds_read_b128 %3, %21 offset:2048\n\t"
        "ds_read_b128 %4, %22\n\t"
        "ds_read_b128 %5, %23\n\t"
        "ds_read_b128 %6, %22 offset:2048\n\t"
        "ds_read_b128 %7, %23 offset:2048\n\t"
        "ds_read_b128 %8, %20 offset:8192\n\t"
        "ds_read_b128 %9, %21 offset:8192\n\t"
        "ds_read_b128 %10, %20 offset:10240\n\t"
        "ds_read_b128 %11, %21 offset:10240\n\t"
        "ds_read_b128 %12, %22 offset:%c25\n\t"
        "ds_read_b128 %13, %23 offset:%c25\n\t"
        "ds_read_b128 %14, %22 offset:%c26\n\t"
        "ds_read_b128 %15, %23 offset:%c26\n\t"
        "ds_read_b32 %16, %24\n\t"
        "ds_read_b32 %17, %24 offset:128\n\t"
        "ds_read_b32 %18, %24 offset:%c27\n\t"
        "ds_read_b32 %19, %24 offset:%c28\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o.kk[0][0]), "=&v"(o.kk[0][1]), "=&v"(o.kk[1][0]), "=&v"(o.kk[1][1]), "=&v"(o.qq[0][0]),
          "=&v"(o.qq[0][1]), "=&v"(o.qq[1][0]), "=&v"(o.qq[1][1]), "=&v"(o.vv[0][0]), "=&v"(o.vv[0][1]),
          "=&v"(o.vv[1][0]), "=&v"(o.vv[1][1]), "=&v"(o.gg[0][0]), "=&v"(o.gg[0][1]), "=&v"(o.gg[1][0]),
          "=&v"(o.gg[1][1]), "=&v"(o.nb[0]), "=&v"(o.nb[1]), "=&v"(o.dl[0]), "=&v"(o.dl[1])
        : "v"(st + ok[0]), "v"(st + ok[1]), "v"(st + oq[0]), "v"(st + oq[1]), "v"(st + ol),
          "i"(DB_G_OFF - DB_Q_OFF), "i"(DB_G_OFF - DB_Q_OFF + 2048), "i"(DB_DL_OFF - DB_L_OFF),
          "i"(DB_DL_OFF - DB_L_OFF + 128));
}

// One row's four units u = 2 qi + ki: acc[u] += 2^x' (dP - delta).  Each unit's products are
// issued one per chunk of four scores of the unit before it, so the matrix unit runs under
// that unit's exponentials.
__device__ __forceinline__ void db_row(const DbOps& o, f32x16 (&acc)[4]) {
    const float nbs[2] = {o.nb[0] * kScale, o.nb[1] * kScale};   // (r_j - lse) log2(e); -inf stays -inf
    const f32x16 zero = {};
    f32x16 ndl[2];                                                // -delta: seeds dP, which then holds dP - delta
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        ndl[0][r] = o.dl[0];
        ndl[1][r] = o.dl[1];
    }
    f32x16 S = mfma(__builtin_bit_cast(bf16x8, o.kk[0][0]), __builtin_bit_cast(bf16x8, o.qq[0][0]), zero);
    f32x16 dP = mfma(__builtin_bit_cast(bf16x8, o.vv[0][0]), __builtin_bit_cast(bf16x8, o.gg[0][0]), ndl[0]);
    S = mfma(__builtin_bit_cast(bf16x8, o.kk[0][1]), __builtin_bit_cast(bf16x8, o.qq[0][1]), S);
    dP = mfma(__builtin_bit_cast(bf16x8, o.vv[0][1]), __builtin_bit_cast(bf16x8, o.gg[0][1]), dP);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int qi = u >> 1;
        const int nq = (u + 1) >> 1, nk = (u + 1) & 1;   // the next unit's tiles
        f32x16 Sn = zero, dPn = zero;
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) {
            if (u + 1 < 4) {
                if (ch == 0) Sn = mfma(__builtin_bit_cast(bf16x8, o.kk[nk][0]), __builtin_bit_cast(bf16x8, o.qq[nq][0]), zero);
                if (ch == 1) dPn = mfma(__builtin_bit_cast(bf16x8, o.vv[nk][0]), __builtin_bit_cast(bf16x8, o.gg[nq][0]), ndl[nq]);
                if (ch == 2) Sn = mfma(__builtin_bit_cast(bf16x8, o.kk[nk][1]), __builtin_bit_cast(bf16x8, o.qq[nq][1]), Sn);
                if (ch == 3) dPn = mfma(__builtin_bit_cast(bf16x8, o.vv[nk][1]), __builtin_bit_cast(bf16x8, o.gg[nq][1]), dPn);
            }
#pragma unroll
            for (int r = 4 * ch; r < 4 * ch + 4; ++r)
                acc[u][r] = fmaf(__builtin_amdgcn_exp2f(fmaf(S[r], kScale, nbs[qi])), dP[r], acc[u][r]);
            asm volatile("" : "+v"(acc[u]));   // the sums are used only next row: keep them in this chunk
            __builtin_amdgcn_sched_barrier(0);
        }
        S = Sn;
        dP = dPn;
    }
}

__global__ void __launch_bounds__(DB_THR, TRI_ATTN_DB_WG_PER_CU) bwd_dbias_lds(BwdProblem p, const float* ref16, int64_t nqp16,
                                                        const int* wide, int n_wide, const __bf16* g16,
                                                        const __bf16* qh, const __bf16* kh, const __bf16* vh,
                                                        const float* nbT2, const float* deltaT, int64_t NP, int n_tq,
                                                        int n_tk, int total) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 31, h2 = lane >> 5;
    // XCD-aware remap: XCD x walks a contiguous range of logical ids; inside one (b, h)
    // strips of DB_TILE_J query tiles, cut into tiles of DB_TILE_J x DB_TILE_K, key tile fastest
    const int w = blockIdx.x;
    const int xcd = w % 8, slot = w / 8;
    const int base = total / 8, extra = total % 8;
    const int logical = xcd * base + (xcd < extra ? xcd : extra) + slot;
    const int bh = logical / (n_tq * n_tk);
    const int rem = logical - bh * n_tq * n_tk;
    const int strip = rem / (DB_TILE_J * n_tk);
    const int nr = min(DB_TILE_J, n_tq - strip * DB_TILE_J);
    const int o = rem - strip * DB_TILE_J * n_tk;
    const int tile = o / (nr * DB_TILE_K);
    const int nk = min(DB_TILE_K, n_tk - tile * DB_TILE_K);
    const int o2 = o - tile * nr * DB_TILE_K;
    const int jt = strip * DB_TILE_J + o2 / nk;
    const int kt = tile * DB_TILE_K + o2 % nk;
    const int64_t N = p.N, H = p.H;
    const int64_t b = bh / H, h = bh % H;
    const int64_t j0 = static_cast<int64_t>(jt) * DB_Q, k0 = static_cast<int64_t>(kt) * DB_K;
    if (any_wide(wide, bh, n_wide)) return;   // left to the fp32 kernel (whole workgroup)

    DbCtx cx;
    {
        // piece pi = DB_PIECES w + t: Q pieces first, then dO, K, V; piece rows 16 (local) ..
        // +15; lane l carries row l / 4, 16-byte slot l % 4, which holds logical part
        // kv_chunk(row, slot)
        const __bf16* tens[4] = {qh, g16, kh, vh};   // head-major copies
        const uint32_t offs[4] = {DB_Q_OFF, DB_G_OFF, DB_K_OFF, DB_V_OFF};
#pragma unroll
        for (int t = 0; t < DB_PIECES; ++t) {
            const int pi = DB_PIECES * wave + t;
            const int ten = pi < DB_PQ ? 0 : pi < 2 * DB_PQ ? 1 : pi < 2 * DB_PQ + DB_PK ? 2 : 3;
            const int local = pi - (ten < 2 ? ten * DB_PQ : 2 * DB_PQ + (ten - 2) * DB_PK);
            cx.first[t] = (ten < 2 ? j0 : k0) + 16 * local;
            cx.src[t] = reinterpret_cast<const char*>(tens[ten] + ((b * H + h) * p.I * N + cx.first[t]) * D);
            cx.dst[t] = offs[ten] + local * 1024;
        }
        // the swizzle depends on bits 1, 2 of the row only, so it is the same in every piece
        cx.off = static_cast<uint32_t>((lane >> 2) * D * 2 + kv_chunk(lane >> 2, lane & 3) * 16);
        cx.N = N;
        cx.pos_bytes = D * 2;
        cx.row_step = N * D * 2;
        // nb' / -delta: wave w < DB_NQP copies nb' of queries 64 w .. +63, the others -delta
        const float* ls = wave < DB_NQP ? nbT2 : deltaT;
        cx.ls_src = reinterpret_cast<const char*>(ls + (b * p.I * H + h) * NP + j0 + 64 * (wave % DB_NQP));
        cx.ls_step = H * NP * 4;
        cx.ls_dst = DB_L_OFF + 256 * wave;
    }

    const int qp = wave % DB_NQP, kp = wave / DB_NQP;
    // LDS byte offsets of this lane's operand reads (stage 0, tile 0 of each pair); the
    // second tile of a pair is 32 rows (+2048) on
    const int kr = 64 * kp + c, qr = 64 * qp + c;
    uint32_t ok[2], oq[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        ok[m] = DB_K_OFF + kr * 64 + kv_chunk(kr, 2 * m + h2) * 16;
        oq[m] = DB_Q_OFF + qr * 64 + kv_chunk(qr, 2 * m + h2) * 16;
    }
    const uint32_t ol = DB_L_OFF + qr * 4;
    const uint32_t st0 = LDS_ADDR(&g_db[0]);

    f32x16 acc[4] = {};
    DbOps ops;
    const int64_t I = p.I;
    // prologue: rows 0 .. DB_STAGES - 2 in flight, row 0 complete everywhere
    for (int64_t r = 0; r < DB_STAGES - 1 && r < I; ++r) db_stage(cx, r, static_cast<int>(r), lane);
    if (I >= DB_STAGES - 1)
        db_barrier_keep();
    else
        db_barrier_drain();
    for (int64_t i = 0; i < I; ++i) {
        const uint32_t st = st0 + static_cast<uint32_t>(i % DB_STAGES) * DB_STAGE_BYTES;
        const bool issue = i + DB_STAGES - 1 < I;
        if (issue) db_stage(cx, i + DB_STAGES - 1, static_cast<int>((i + DB_STAGES - 1) % DB_STAGES), lane);
        db_read(st, ok, oq, ol, ops);
        db_row(ops, acc);
        if (issue)
            db_barrier_keep();
        else
            db_barrier_drain();
    }
    // dbias = E acc, E = 2^((bias + mask - r_j) log2(e)) from the raw bias; a key that E
    // drops (the mask, or a query without any kept key) gets exactly 0
    const uint16_t* braw = static_cast<const uint16_t*>(p.bias);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int qi = u >> 1, ki = u & 1;
        const int64_t j = j0 + 64 * qp + 32 * qi + c;
        if (j >= N) continue;
        const float rj = ref16[bh * nqp16 + j];
        float* out = p.dbias + (bh * N + j) * N;
        const uint16_t* brow = braw + (bh * N + j) * N;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t kk = k0 + 64 * kp + 32 * ki + 8 * (r / 4) + 4 * h2 + (r % 4);
            if (kk >= N) continue;
            const float bv = __uint_as_float(static_cast<uint32_t>(brow[kk]) << 16);
            const float mk = p.mask ? p.mask[b * N + kk] : 0.0f;
            const float e = __builtin_amdgcn_exp2f((bv + mk - rj) * kLog2e);
            out[kk] = e > 0.0f ? e * acc[u][r] : 0.0f;
        }
    }
}

}  // namespace

namespace {
// fp16 transposed bias tile of dk/dv: per (b, h, key tile kt of 128 keys, query block n of
// 32 queries) a 128 x 32 tile at ((b*H + h) * n_kt + kt) * nqb + n; row kk is key
// 128 kt + kk, its 32 queries q in part_col order with 16-byte parts swizzled by kv_chunk,
// each value (bias[b, h, q, key] + mask[b, key] - r_q) log2(e) relative to the query's r_q
// (the forward prepass's reference), -inf past the last key or query.  A thread owns one
// key and two parts; the 128 threads of a part read 128 consecutive keys of one bias row.
__global__ void __launch_bounds__(256) bias_imageT16_kernel(BwdProblem p, const float* ref16, int64_t nqp16,
                                                            _Float16* out, int n_kt, int nqb) {
    const int tile = blockIdx.x, n = tile % nqb, kt = tile / nqb;
    const int64_t bh = blockIdx.y, b = bh / p.H;
    const int t = threadIdx.x, kk = t & 127;
    const int64_t key = static_cast<int64_t>(kt) * IMG_BJ + kk;
    const bool kok = key < p.N;
    const uint16_t* bias = static_cast<const uint16_t*>(p.bias);
    const float mk = (kok && p.mask) ? p.mask[b * p.N + key] : 0.0f;
    _Float16* dst = out + ((bh * n_kt + kt) * nqb + n) * static_cast<int64_t>(IMG_BJ * 32) + kk * 32;
#pragma unroll
    for (int pi = 0; pi < 2; ++pi) {
        const int part = (t >> 7) + 2 * pi;
        f16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t q = static_cast<int64_t>(n) * 32 + part_col(part, e);
            float x = -INFINITY;
            if (kok && q < p.N) {
                const float bv = __uint_as_float(static_cast<uint32_t>(bias[(bh * p.N + q) * p.N + key]) << 16);
                x = (bv + mk - ref16[bh * nqp16 + q]) * kLog2e;
            }
            v[e] = static_cast<_Float16>(x);
        }
        *reinterpret_cast<f16x8*>(dst + kv_chunk(kk, part) * 8) = v;
    }
}

struct BwdLayout {
    Problem fwd;            // the image problem: the bias and mask over all keys
    Prepass16 pre;          // the forward's prepass: fp16 image and r_j (dq, dk/dv)
    int64_t NP, nq;
    size_t pre16, imgT16, g16, qh, kh, vh, delta, nbT2, deltaT, total;   // byte offsets / total
};

BwdLayout bwd_layout(const BwdProblem& p) {
    BwdLayout L;
    L.fwd = Problem{p.q, p.k, p.v, p.bias, p.mask, nullptr, p.B, p.H, p.I, p.N, p.D, 1};
    L.pre = prepass16_layout(L.fwd);
    L.NP = (p.N + NP_ALIGN - 1) / NP_ALIGN * NP_ALIGN;
    L.nq = p.B * p.I * p.N * p.H;
    const size_t per_line = static_cast<size_t>(p.B * p.I * p.H * L.NP) * 4;
    const int64_t n_kt = (p.N + IMG_BJ - 1) / IMG_BJ, nqb = (p.N + 31) / 32;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    L.pre16 = 0;
    L.imgT16 = up(L.pre16 + L.pre.bytes);
    L.g16 = up(L.imgT16 + static_cast<size_t>(p.B * p.H * n_kt * nqb) * IMG_BJ * 32 * 2);
    L.qh = up(L.g16 + static_cast<size_t>(L.nq) * D * 2);
    L.kh = up(L.qh + static_cast<size_t>(L.nq) * D * 2);
    L.vh = up(L.kh + static_cast<size_t>(L.nq) * D * 2);
    L.delta = up(L.vh + static_cast<size_t>(L.nq) * D * 2);
    L.nbT2 = up(L.delta + static_cast<size_t>(L.nq) * 4);
    L.deltaT = L.nbT2 + per_line;
    L.total = L.deltaT + per_line;
    return L;
}
}  // namespace

size_t bwd_mfma_workspace_bytes(const BwdProblem& p) { return bwd_layout(p).total; }

hipError_t launch_backward_mfma(const BwdProblem& p, void* workspace, hipStream_t stream) {
    const BwdLayout Ly = bwd_layout(p);
    const int64_t n_jb = (p.N + IMG_BJ - 1) / IMG_BJ;
    const int64_t nblk = bias_image_blocks(Ly.fwd);      // 32-key blocks
    char* ws = static_cast<char*>(workspace);
    _Float16* img16 = reinterpret_cast<_Float16*>(ws + Ly.pre16);
    const float* ref16 = reinterpret_cast<const float*>(ws + Ly.pre16 + Ly.pre.ref_off);
    const int* wide = reinterpret_cast<const int*>(ws + Ly.pre16 + Ly.pre.wide_off);
    _Float16* imgT16 = reinterpret_cast<_Float16*>(ws + Ly.imgT16);
    __bf16* g16 = reinterpret_cast<__bf16*>(ws + Ly.g16);
    __bf16* qh = reinterpret_cast<__bf16*>(ws + Ly.qh);
    __bf16* kh = reinterpret_cast<__bf16*>(ws + Ly.kh);
    __bf16* vh = reinterpret_cast<__bf16*>(ws + Ly.vh);
    float* delta = reinterpret_cast<float*>(ws + Ly.delta);
    float* nbT2 = reinterpret_cast<float*>(ws + Ly.nbT2);
    float* deltaT = reinterpret_cast<float*>(ws + Ly.deltaT);
    const int64_t n_prep = p.B * p.I * p.H * Ly.NP * PREP_PARTS;
    const int64_t n_kt = (p.N + IMG_BJ - 1) / IMG_BJ, nqb = (p.N + 31) / 32;
    if (p.D != D || (n_prep + 255) / 256 > 0x7FFFFFFF || (p.N + 63) / 64 > 65535 || n_kt * nqb > 0x7FFFFFFF ||
        p.B * p.H > 65535 || Ly.pre.cols % IMG_BJ != 0)
        return hipErrorInvalidConfiguration;
    hipError_t e = launch_prepass16(Ly.fwd, ws + Ly.pre16, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bias_imageT16_kernel, dim3(static_cast<unsigned>(n_kt * nqb), static_cast<unsigned>(p.B * p.H)),
                       dim3(256), 0, stream, p, ref16, Ly.pre.nqp, imgT16, static_cast<int>(n_kt),
                       static_cast<int>(nqb));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_prep_kernel, dim3(static_cast<unsigned>((n_prep + 255) / 256)), dim3(256), 0, stream, p, g16,
                       delta, deltaT, Ly.NP, ref16, Ly.pre.nqp, nbT2);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t n_hm = (p.B * p.I * p.N * p.H * 4 + 255) / 256;   // within n_prep's bound checked above
    hipLaunchKernelGGL(bwd_headmajor_kernel, dim3(static_cast<unsigned>(n_hm), 3), dim3(256), 0, stream, p, qh, kh, vh);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    {
        const int64_t n_rg = (p.I + DQ_R - 1) / DQ_R;
        const int64_t total = n_jb * n_rg * p.B * p.H;
        if (total > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(bwd_dq_lds, dim3(static_cast<unsigned>(total)), dim3(DQ_THR), 0, stream, p, img16, ref16,
                           Ly.pre, wide, g16, kh, vh, delta, static_cast<int>(n_jb), static_cast<int>(n_rg),
                           static_cast<int>(nblk), static_cast<int>(total));
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    {
        const int64_t n_rg = (p.I + DK_R - 1) / DK_R;
        const int64_t total = n_jb * n_rg * p.B * p.H;
        if (total > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(bwd_dkdv_lds, dim3(static_cast<unsigned>(total)), dim3(DK_THR), 0, stream, p, imgT16, wide,
                           static_cast<int>(Ly.pre.n_jb), g16, qh, nbT2, deltaT, static_cast<int>(n_jb),
                           static_cast<int>(n_rg), static_cast<int>(nblk), Ly.NP, static_cast<int>(total));
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // dq, dk/dv and dbias of every (b, h) whose bias spans more than the fp16 image keeps
    if ((e = launch_backward_wide(p, wide, static_cast<int>(Ly.pre.n_jb), stream)) != hipSuccess) return e;
    const int64_t n_tq = (p.N + DB_Q - 1) / DB_Q, n_tk = (p.N + DB_K - 1) / DB_K;
    const int64_t total = n_tq * n_tk * p.B * p.H;
    if (total > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(bwd_dbias_lds, dim3(static_cast<unsigned>(total)), dim3(DB_THR), 0, stream, p, ref16, Ly.pre.nqp,
                       wide, static_cast<int>(Ly.pre.n_jb), g16, qh, kh, vh, nbT2, deltaT, Ly.NP, static_cast<int>(n_tq),
                       static_cast<int>(n_tk), static_cast<int>(total));
    return hipGetLastError();
}

}  // namespace tri_attn
