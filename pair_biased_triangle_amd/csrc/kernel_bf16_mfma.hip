// bf16 triangle attention on gfx950 matrix cores (head size D = 32).
//
// Per batch b and head h the rows i are independent attention problems that share one
// N x N "triangular" bias bias[b,h,j,k] ("Fold-CP", Table 1 "Triangle Attention" and
// Figure 2(a)).  A workgroup owns R lines (rows i) and BJ query columns j of one (b, h)
// and streams the call's keys in contiguous blocks of 32 in ascending order.  The ring
// steps (Table 1's caption, Figure 2) fold the key tiles into the running softmax state
// with an associative merge, so folding the 32-key blocks in the same order gives the same
// state: blocks run across tile boundaries and only the last block is partial.
//
// Three kernels run per call:
//   1. bias_ref_kernel, bias_image16_kernel: per query j the reference r_j, the largest
//      bias + mask over the call's keys, then the fp16 image the main kernel stages
//      verbatim: per (b, h, column block, key block) a BJ x 32 tile of
//      (bias + mask - r_j) * log2(e), -inf for keys past the last one.  Softmax does not
//      change when every score of a query moves by the same amount, and relative to r_j
//      every value is <= 0, so fp16 keeps 11 bits where the weights are large and a value
//      too negative for fp16 becomes -inf, whose weight is 0 anyway.
//   2. bf16_mfma_kernel: per key block the workgroup copies K and V of its R lines
//      ([key][d], natural layout) and the bias tile straight from global memory into
//      LDS (global_load_lds_dwordx4, a ring of stages, no registers on the way).  Each
//      wave owns 2 lines x 2 query tiles of 32 and runs, per (line, tile):
//        S^T = K Q^T           two v_mfma_f32_32x32x16_bf16
//        x   = S * log2(e)/sqrt(D) + c      one v_fma_mix_f32 per score: c is the fp16
//                              image value, taken from its half register as it is
//        p   = 2^x             (x is the score minus r_j, in log2 units)
//        O^T += V^T P^T        two v_mfma_f32_32x32x16_bf16 on the bf16-rounded p;
//                              V^T comes from ds_read_b64_tr_b16 on the [key][d] tile
//      The row sum is taken per lane with v_dot2_f32_bf16 on the rounded p.  The four
//      units run as a software pipeline in which every group of four exponentials carries
//      one matrix instruction of the neighbouring units (compute_block_pipe).
//
// Softmax reference.  r_j is the reference of the fast pass: the scores are not shifted
// by their running maximum -- O and l share the reference, so the result is exact
// whatever it is -- so no block needs a maximum, a cross-lane step or a branch.  At the
// end every lane checks that its normaliser lies in [2^-64, 2^64] and its accumulator is
// finite; if any lane of the workgroup fails (q.k far from 0, or rows whose keys are all
// masked), the workgroup recomputes its whole key loop with the exact running maximum m
// (log2 units) refreshed on every block.  The natural log of the normaliser adds the
// reference back: lse = r_j + m ln 2 + ln l (m = 0 in the fast pass).
//
// Shape: 4 waves own 2 lines x 256 query columns, with a ring of 3 stages of 24 KB, so
// two workgroups (72 KB of LDS each) share a compute unit.  Each waits only at its own
// barrier, so one workgroup's burst of operand reads after its barrier overlaps the
// other's arithmetic (with 8 waves and one workgroup per unit, every wave waits on the
// same burst).  Workgroup ids are remapped so that each XCD walks a contiguous range of
// (b, h, line group, column block) tiles: the workgroups an XCD runs together share each
// line group's K/V stream and each bias tile in its L2.
#include "launch.h"

#include <cmath>
#include <cstddef>

namespace tri_attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))
#define GLOBAL_PTR(T, p) ((const __attribute__((address_space(1))) T*)(p))

constexpr int D = 32;
constexpr int BK = 32;                      // keys per block
#ifndef TRI_ATTN_ROWS
#define TRI_ATTN_ROWS 2
#endif
constexpr int R = TRI_ATTN_ROWS;            // lines per workgroup
#ifndef TRI_ATTN_WAVES
#define TRI_ATTN_WAVES 4
#endif
constexpr int NWAVE = TRI_ATTN_WAVES;       // waves per workgroup
constexpr int NTHR = 64 * NWAVE;
constexpr int RW = 2;                       // lines per wave
constexpr int TW = 2;                       // query tiles per wave
constexpr int QT = NWAVE * RW * TW / R;     // 32-wide query tiles per workgroup
constexpr int BJ = 32 * QT;                 // query columns per workgroup
constexpr int NXCD = 8;
static_assert(R == 2 || R == 4 || R == 8, "2, 4 or 8 lines per workgroup");
static_assert((R / RW) * (QT / TW) == NWAVE, "every wave owns RW x TW units");
#ifndef TRI_ATTN_STAGES
#define TRI_ATTN_STAGES 3
#endif
#ifndef TRI_ATTN_TILE_RG
#define TRI_ATTN_TILE_RG (32 / TRI_ATTN_ROWS)
#endif
#ifndef TRI_ATTN_TILE_JB
#define TRI_ATTN_TILE_JB 8
#endif
constexpr int NSTAGE = TRI_ATTN_STAGES;     // key blocks in flight (LDS ring of stages)
constexpr int TILE_RG = TRI_ATTN_TILE_RG;   // line groups x column blocks that one XCD
constexpr int TILE_JB = TRI_ATTN_TILE_JB;   //   works on together (L2 reuse of K/V and bias)
constexpr int IMG_HALVES = BJ * BK;         // one fp16 bias tile of the image

// Every staged piece is 1 KB: 16 keys of one line's K or V (64-byte rows), or 16 query
// rows of the bias tile (64-byte rows of 32 fp16).  Wave w stages KV_PER_WAVE K/V pieces
// and BIAS_PER_WAVE bias pieces.
constexpr int KV_PER_WAVE = 4 * R / NWAVE;
constexpr int BIAS_PER_WAVE = BJ * BK * 2 / 1024 / NWAVE;
constexpr int COPIES_PER_BLOCK = KV_PER_WAVE + BIAS_PER_WAVE;   // global_load_lds per wave per block
static_assert(KV_PER_WAVE * NWAVE == 4 * R && BIAS_PER_WAVE * NWAVE * 1024 == BJ * BK * 2, "whole pieces");

struct Stage {
    __bf16 k[R][BK][D];      // 64-byte rows, 16-byte chunks swizzled by kv_chunk()
    __bf16 v[R][BK][D];
    _Float16 bias[BJ][BK];   // 64-byte rows (one query), 16-byte chunks swizzled by kv_chunk()
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSqrtD = 5.656854249492381f;   // sqrt(32), the scale of the backward's fp32 image
constexpr float kScale = 1.4426950408889634f / 5.656854249492381f;   // log2(e) / sqrt(32): q.k -> log2 units
// Widest span the fp16 image keeps below a query's reference: a stored value in
// (-kImageSpan, 0] is rounded by at most 2^-7 log2 units.  A column block with any finite
// value below it is handled by the fp32 kernel instead (see bias_image16_kernel).
constexpr float kImageSpan = 32.0f;
constexpr float kLo = 5.421010862427522e-20f;  // 2^-64
constexpr float kHi = 1.8446744073709552e19f;  // 2^64

// Position of a 16-byte chunk inside a 64-byte LDS row (K, V: row = key; bias: row = query).
__host__ __device__ constexpr int kv_chunk(int row, int part) { return part ^ ((row >> 1) & 3); }

// Order of the 32 keys of a block inside a bias row: lane (c, h2) of the 32x32 MFMA
// output holds keys 8a + 4*h2 + e (a, e = 0..3) of query c in registers 4a + e, so the
// row stores key 8a + 4*h2 + e at position 16*h2 + 4a + e and the lane's 16 values are
// the contiguous 16-byte parts 2*h2 and 2*h2 + 1.  Position 8*part + t holds this key:
__host__ __device__ constexpr int part_key(int part, int t) {
    return 8 * (2 * (part & 1) + (t >> 2)) + 4 * (part >> 1) + (t & 3);
}

// Key block n of the call's key range: keys 32n .. 32n + 31, the last block partial.  The
// method's T key tiles are folded into the running state in ascending key order, and the
// merge rule is associative, so folding 32-key blocks in the same order computes the same
// state: blocks run across tile boundaries and no tile's end pads a block.
struct KeyBlock {
    int64_t kb;
    int nk;
};
struct BlockPlan {
    int64_t N;
    BlockPlan() = default;
    __host__ __device__ explicit BlockPlan(int64_t n) : N(n) {}
    __host__ __device__ int64_t count() const { return (N + BK - 1) / BK; }
    __host__ __device__ KeyBlock block(int n) const {
        const int64_t kb = static_cast<int64_t>(n) * BK, rest = N - kb;
        return {kb, static_cast<int>(rest < BK ? rest : BK)};
    }
};

// ---------------------------------------------------------------------------------------
// 1a. fp32 bias image of the backward kernels (layout in launch.h)
// ---------------------------------------------------------------------------------------
constexpr int IMG_THR = 256;
constexpr int IMG_FLOATS = IMG_BJ * IMG_BK;

__global__ void __launch_bounds__(IMG_THR) bias_image_kernel(Problem p, float* img, int n_jb, int nblk) {
    const int n = blockIdx.x, jb = blockIdx.y, bh = blockIdx.z;
    const int64_t b = bh / p.H;
    const KeyBlock kbk = BlockPlan(p.nkeys()).block(n);
    const int64_t key0 = p.k0 + kbk.kb;        // absolute index of the block's first key
    const uint16_t* bg = static_cast<const uint16_t*>(p.bias);
    float* dst = img + ((static_cast<int64_t>(bh) * n_jb + jb) * nblk + n) * IMG_FLOATS;
    const int kk = threadIdx.x % IMG_BK;
    const bool key_ok = kk < kbk.nk;
    const float mk = (p.mask && key_ok) ? p.mask[b * p.N + key0 + kk] : 0.0f;
#pragma unroll
    for (int s = 0; s < IMG_FLOATS / IMG_THR; ++s) {
        const int jj = (threadIdx.x + s * IMG_THR) / IMG_BK;
        const int64_t j = static_cast<int64_t>(jb) * IMG_BJ + jj;
        float val = -INFINITY;
        if (key_ok) {
            // starting node bias[b, h, j, key]; ending node the transpose, bias[b, h, key, j]
            const int64_t bi = p.ending ? (bh * p.N + key0 + kk) * p.N + j : (bh * p.N + j) * p.N + key0 + kk;
            const float bv = j < p.N ? __uint_as_float(static_cast<uint32_t>(bg[bi]) << 16) : 0.0f;
            val = (bv + mk) * kSqrtD;
        }
        dst[jj * IMG_BK + img_chunk(jj, kk / 4) * 4 + kk % 4] = val;
    }
}

// ---------------------------------------------------------------------------------------
// 1b. fp16 bias image of the forward kernel, relative to each query's largest bias
// ---------------------------------------------------------------------------------------
constexpr int IMG16_Q = 64;                 // queries per workgroup of the image kernel
static_assert(BJ % IMG16_Q == 0, "an image workgroup fills part of one column block");

// r_j = max over the call's keys of bias + mask, written as REF_KS partial maxima per query
// (padding queries and queries whose keys are all masked give -inf).  Starting node: a
// query's biases are a contiguous row, so one wave walks it with coalesced reads (one
// partial).  Ending node: they are a column, so a wave holds 64 consecutive queries and the
// keys are split into REF_KS chunks, each a partial maximum, over 4 waves of a workgroup.
// The same launch clears the wide-span flag of every column block (one int per (b, h,
// column block)), which bias_image16_kernel sets afterwards.
constexpr int REF_KS = 16;
__global__ void __launch_bounds__(256) bias_ref_kernel(Problem p, float* part, int64_t nqp, int* wide, int n_jb) {
    const int64_t bh = blockIdx.z, b = bh / p.H, BH = gridDim.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t NK = p.nkeys();
    const uint16_t* bg = static_cast<const uint16_t*>(p.bias);
    if (!p.ending) {
        const int64_t j = static_cast<int64_t>(blockIdx.x) * 4 + wave;
        if (j >= nqp) return;
        if (j % BJ == 0 && lane == 0) wide[bh * n_jb + j / BJ] = 0;
        float mx = -INFINITY;
        if (j < p.N) {
            const uint16_t* row = bg + (bh * p.N + j) * p.N + p.k0;
            const float* mrow = p.mask ? p.mask + b * p.N + p.k0 : nullptr;
            int64_t k0 = 0;
            if ((reinterpret_cast<uintptr_t>(row) & 7) == 0 && (!mrow || (reinterpret_cast<uintptr_t>(mrow) & 15) == 0)) {
                // aligned row: 4 keys per lane and load, 256 keys per wave step
                const int64_t n4 = NK / 256 * 256;
#pragma unroll 4
                for (int64_t k = 4 * lane; k < n4; k += 256) {
                    const uint2 w2 = *reinterpret_cast<const uint2*>(row + k);
                    float x[4] = {__uint_as_float(w2.x << 16), __uint_as_float(w2.x & 0xFFFF0000u),
                                  __uint_as_float(w2.y << 16), __uint_as_float(w2.y & 0xFFFF0000u)};
                    if (mrow) {
                        const float4 m4 = *reinterpret_cast<const float4*>(mrow + k);
                        x[0] += m4.x;
                        x[1] += m4.y;
                        x[2] += m4.z;
                        x[3] += m4.w;
                    }
                    mx = fmaxf(mx, fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
                }
                k0 = n4;
            }
#pragma unroll 8
            for (int64_t k = k0 + lane; k < NK; k += 64) {
                const float bv = __uint_as_float(static_cast<uint32_t>(row[k]) << 16);
                mx = fmaxf(mx, mrow ? bv + mrow[k] : bv);
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
        if (lane == 0) part[bh * nqp + j] = mx;
        return;
    }
    __shared__ float red[4][64];
    const int64_t j = static_cast<int64_t>(blockIdx.x) * 64 + lane;
    if (blockIdx.y == 0 && threadIdx.x == 0 && j % BJ == 0) wide[bh * n_jb + j / BJ] = 0;
    const int64_t chunk = (NK + REF_KS - 1) / REF_KS;
    const int64_t lo = blockIdx.y * chunk, hi = min(NK, lo + chunk);
    float mx = -INFINITY;
    if (j < p.N) {
#pragma unroll 8
        for (int64_t k = lo + wave; k < hi; k += 4) {
            const int64_t key = p.k0 + k;
            const float bv = __uint_as_float(static_cast<uint32_t>(bg[(bh * p.N + key) * p.N + j]) << 16);
            mx = fmaxf(mx, p.mask ? bv + p.mask[b * p.N + key] : bv);
        }
    }
    red[wave][lane] = mx;
    __syncthreads();
    if (wave == 0)
        part[(static_cast<int64_t>(blockIdx.y) * BH + bh) * nqp + j] =
            fmaxf(fmaxf(red[0][lane], red[1][lane]), fmaxf(red[2][lane], red[3][lane]));
}

// One workgroup per (64 queries, IMG16_NB key blocks, (b, h)); thread t handles query jj of
// the 64 and the 8 keys of part pt of each block.  Starting node: the 4 threads of a query
// are neighbours, so a query row's 32 keys are read as 64 contiguous bytes; ending node: a
// wave holds 64 consecutive queries, which for one key are 128 contiguous bytes.  r_j is
// the largest of the n_part partial maxima (0 if every key is masked); with several
// partials the workgroups of the first blocks also store r_j for the epilogue.
//
// Span guard.  fp16 rounds a value in (-2^e, -2^(e-1)] by up to 2^(e-12), so the image error
// of a score grows with how far its bias lies below r_j.  The output error stays within
// that of the bf16 probabilities only while every kept value lies within kImageSpan of
// r_j.  A workgroup that writes a finite image value below -kImageSpan sets its column
// block's flag in `wide`; the attention kernel then leaves that block to the fp32 kernel,
// which adds the bias unrounded.  Values beyond fp16's range become -inf: keys more than
// 65520 log2 units (about 45,400 nats) below the query's largest bias get weight 0.
constexpr int IMG16_NB = 4;
__device__ __forceinline__ bool beyond_span(_Float16 h) {
    const float f = static_cast<float>(h);
    return f < -kImageSpan && f > -INFINITY;
}

__global__ void __launch_bounds__(256) bias_image16_kernel(Problem p, const float* part, int n_part, _Float16* img,
                                                           float* ref, int n_jb, int nblk, int* wide) {
    const int g = blockIdx.x, n0 = blockIdx.y * IMG16_NB;
    const int64_t bh = blockIdx.z, b = bh / p.H, BH = gridDim.z;
    const int t = threadIdx.x;
    const int jj = p.ending ? (t & 63) : (t >> 2);
    const int pt = p.ending ? (t >> 6) : (t & 3);
    const int64_t j = static_cast<int64_t>(g) * IMG16_Q + jj;   // query (columns past N are padding)
    const bool real = j < p.N;
    const int64_t nqp = static_cast<int64_t>(n_jb) * BJ;
    const uint16_t* bg = static_cast<const uint16_t*>(p.bias);

    float r = -INFINITY;
    for (int ks = 0; ks < n_part; ++ks) r = fmaxf(r, part[(ks * BH + bh) * nqp + j]);
    if (!(r > -INFINITY)) r = 0.0f;
    if (n_part > 1 && n0 == 0 && pt == 0) ref[bh * nqp + j] = r;

    const BlockPlan plan(p.nkeys());
    const int jb = static_cast<int>(j / BJ), jl = static_cast<int>(j % BJ);   // jb is the workgroup's
    bool spread = false;                                                     // (IMG16_Q divides BJ)
    _Float16* dst = img + (bh * n_jb + jb) * nblk * static_cast<int64_t>(IMG_HALVES) + jl * BK + kv_chunk(jl, pt) * 8;
    if (!p.ending) {
        // Starting node: the workgroup's blocks cover the contiguous keys k0 + kbeg .. + span
        // of 64 query rows.  Wave w copies rows w, w + 4, ... into LDS with each lane taking
        // keys 2l, 2l + 1 (256 contiguous bytes of a row per step), already relative to r_j,
        // then every thread gathers its 16-byte parts from LDS.
        __shared__ _Float16 rowbuf[IMG16_Q][IMG16_NB * BK + 2];
        __shared__ float rref[IMG16_Q];
        const int lane = t & 63, wv = t >> 6;
        if (pt == 0) rref[jj] = r;
        const KeyBlock first = plan.block(n0);
        const int nlast = min(n0 + IMG16_NB, nblk) - 1;
        const KeyBlock last = plan.block(nlast);
        const int64_t kbeg = first.kb;
        const int span = static_cast<int>(last.kb + last.nk - kbeg);   // <= IMG16_NB * BK
        float mk[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int kk = 2 * lane + h;
            mk[h] = (p.mask && kk < span) ? p.mask[b * p.N + p.k0 + kbeg + kk] : 0.0f;
        }
        __syncthreads();
        const int64_t jq0 = static_cast<int64_t>(g) * IMG16_Q;
        for (int rr = wv; rr < IMG16_Q; rr += 4) {
            const int64_t jr = jq0 + rr;
            const uint16_t* rowp = bg + (bh * p.N + (jr < p.N ? jr : 0)) * p.N + p.k0 + kbeg;
            const float rj = rref[rr];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int kk = 2 * lane + h;
                float x = 0.0f;
                if (jr < p.N && kk < span) x = (__uint_as_float(static_cast<uint32_t>(rowp[kk]) << 16) + mk[h] - rj) * kLog2e;
                const _Float16 hx = static_cast<_Float16>(x);
                spread = spread || beyond_span(hx);
                if (kk < IMG16_NB * BK) rowbuf[rr][kk] = hx;
            }
        }
        __syncthreads();
        for (int u = 0; u < IMG16_NB; ++u) {
            const int n = n0 + u;
            if (n >= nblk) break;
            const KeyBlock kbk = plan.block(n);
            const int off = static_cast<int>(kbk.kb - kbeg);
            f16x8 x;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int kk = part_key(pt, e);
                x[e] = kk < kbk.nk ? rowbuf[jj][off + kk] : static_cast<_Float16>(-INFINITY);
            }
            *reinterpret_cast<f16x8*>(dst + static_cast<int64_t>(n) * IMG_HALVES) = x;
        }
        if (__syncthreads_or(spread) && t == 0) atomicOr(wide + bh * n_jb + jb, 1);
        return;
    }
    // the query's biases at key k0 + k: base[k * kstride] (a row, or a column for the ending node)
    const int64_t kstride = p.ending ? p.N : 1;
    const uint16_t* base = bg + (p.ending ? (bh * p.N + p.k0) * p.N + (real ? j : 0) : (bh * p.N + (real ? j : 0)) * p.N + p.k0);
    const float* mbase = p.mask ? p.mask + b * p.N + p.k0 : nullptr;
    int64_t koff[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) koff[e] = part_key(pt, e) * kstride;
    float val[IMG16_NB][8];
#pragma unroll
    for (int u = 0; u < IMG16_NB; ++u) {
        const int n = n0 + u;
        const KeyBlock kbk = plan.block(n < nblk ? n : nblk - 1);
        const uint16_t* bp = base + kbk.kb * kstride;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int kk = part_key(pt, e);
            float x = -INFINITY;
            if (n < nblk && kk < kbk.nk) {
                x = 0.0f;
                if (real) {
                    x = __uint_as_float(static_cast<uint32_t>(bp[koff[e]]) << 16);
                    if (mbase) x += mbase[kbk.kb + kk];
                    x = (x - r) * kLog2e;
                }
            }
            val[u][e] = x;
        }
    }
#pragma unroll
    for (int u = 0; u < IMG16_NB; ++u) {
        if (n0 + u >= nblk) break;
        f16x8 x;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            x[e] = static_cast<_Float16>(val[u][e]);
            spread = spread || beyond_span(x[e]);
        }
        *reinterpret_cast<f16x8*>(dst + static_cast<int64_t>(n0 + u) * IMG_HALVES) = x;
    }
    if (__syncthreads_or(spread) && t == 0) atomicOr(wide + bh * n_jb + jb, 1);
}

// ---------------------------------------------------------------------------------------
// 2. attention
// ---------------------------------------------------------------------------------------
struct Ctx {
    const char* kv_row[KV_PER_WAVE];   // K or V of a staged line at the first key of the range
    uint32_t kv_lds[KV_PER_WAVE];      // LDS byte offset of the piece inside a stage
    int key_local[KV_PER_WAVE];        // key of this lane's 16-byte slot in the piece
    int part_bytes[KV_PER_WAVE];       // byte offset of the slot's logical 16-byte part inside the key
    uint32_t lane_off[KV_PER_WAVE];    // key_local * key_bytes + part_bytes: the slot's source offset in a block
    const _Float16* img_wg;            // this workgroup's bias tiles, nblk consecutive BJ x 32 tiles
    int64_t key_bytes;                 // bytes between consecutive keys of a line
    int last_key;                      // index of the last key of the range
    BlockPlan plan;
};

constexpr int ROW_BYTES = BK * D * 2;       // one staged line of K or V
constexpr int TILE_BYTES = 32 * BK * 2;     // 32 query rows of the staged bias tile
constexpr int STAGE_BYTES = static_cast<int>(sizeof(Stage));
constexpr int K_OFF = static_cast<int>(offsetof(Stage, k));
constexpr int V_OFF = static_cast<int>(offsetof(Stage, v));
constexpr int B_OFF = static_cast<int>(offsetof(Stage, bias));
static_assert(RW == 2 && TW == 2, "the operand reads below address lines +ROW_BYTES and tiles +TILE_BYTES");

__shared__ Stage g_stage[NSTAGE];
__shared__ int g_redo;

__device__ __forceinline__ uint32_t stage_addr(int n) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(LDS_PTR(char, &g_stage[0]))) +
           static_cast<uint32_t>(n % NSTAGE) * STAGE_BYTES;
}

// Wave w copies its K/V pieces and its bias pieces of block n; lane l of a piece carries
// 16 bytes into bytes 16 l .. 16 l + 15 of the piece.
__device__ __forceinline__ void stage_block(const Ctx& cx, int n, int wave, int lane) {
    const KeyBlock kbk = cx.plan.block(n);
    const int lim = cx.last_key - static_cast<int>(kbk.kb);      // last real key of the block, block-relative
    char* lds = reinterpret_cast<char*>(&g_stage[n % NSTAGE]);
    // Sources are a wave-uniform base (the piece's line at the block's first key) plus a
    // 32-bit lane offset, so the copies take the scalar-base address form.  The empty asm
    // statements keep the compiler from folding the loop-invariant lane offsets into
    // 64-bit vector pointers, which costs 64-bit vector arithmetic per block.
#pragma unroll
    for (int t = 0; t < KV_PER_WAVE; ++t) {
        uint32_t off = cx.lane_off[t];
        if (lim < BK - 1)        // the last, partial block: padded keys read the last real key (bias -inf)
            off = static_cast<uint32_t>(min(cx.key_local[t], lim) * static_cast<int>(cx.key_bytes) + cx.part_bytes[t]);
        asm volatile("" : "+v"(off));
        const char* base = cx.kv_row[t] + kbk.kb * cx.key_bytes;
        __builtin_amdgcn_global_load_lds(GLOBAL_PTR(void, base + off), LDS_PTR(void, lds + cx.kv_lds[t]), 16, 0, 0);
    }
    const char* tile = reinterpret_cast<const char*>(cx.img_wg + static_cast<int64_t>(n) * IMG_HALVES);
#pragma unroll
    for (int t = 0; t < BIAS_PER_WAVE; ++t) {
        const int base = (BIAS_PER_WAVE * wave + t) * 1024;
        uint32_t off = static_cast<uint32_t>(lane * 16 + base);
        asm volatile("" : "+v"(off));
        __builtin_amdgcn_global_load_lds(GLOBAL_PTR(void, tile + off), LDS_PTR(void, lds + B_OFF + base), 16, 0, 0);
    }
}

// LDS byte offsets (inside stage 0) of this lane's operand reads for its first line / tile.
struct Lane {
    int c, h2;
    uint32_t k[2];        // K operand of S^T = K Q^T, d-half m
    uint32_t v[2][2];     // ds_read_b64_tr_b16 sources of the V^T operand, [key half m][sub]
    uint32_t b[2];        // bias operand, 16-byte part 2*h2 + h
};

__device__ __forceinline__ Lane lane_layout(int lane, int row0, int tile0) {
    Lane L;
    L.c = lane & 31;
    L.h2 = lane >> 5;
#pragma unroll
    for (int m = 0; m < 2; ++m) L.k[m] = K_OFF + row0 * ROW_BYTES + L.c * 64 + kv_chunk(L.c, 2 * m + L.h2) * 16;
    // transpose read: lane i of a 16-lane group reads keys kbase + i/4, d = dbase + 4*(i%4) .. +3
    // and receives d = dbase + i for keys kbase .. kbase + 3
    const int i = lane & 15, dbase = 16 * ((lane >> 4) & 1);
    const int d0 = dbase + 4 * (i & 3);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int key = 16 * m + 8 * sub + 4 * L.h2 + (i >> 2);
            L.v[m][sub] = V_OFF + row0 * ROW_BYTES + key * 64 + kv_chunk(key, d0 >> 3) * 16 + (d0 & 7) * 2;
        }
#pragma unroll
    for (int h = 0; h < 2; ++h) L.b[h] = B_OFF + tile0 * TILE_BYTES + L.c * 64 + kv_chunk(L.c, 2 * L.h2 + h) * 16;
    return L;
}

// Operands of one staged block.  The reads are inline assembly that waits for its own
// results (lgkmcnt) before returning: the compiler then sees no LDS read it would have to
// order against the global->LDS copies still in flight into the other stages (ordinary
// LDS loads get a full vmcnt(0) wait in front of them, which would drain the ring).
struct VFrags {
    bf16x8 vA[RW][2];
};
struct KCFrags {
    bf16x8 kA[RW][2];
    u32x4 c16[TW][2];     // bias tile of query tile ti: fp16 registers 8h .. 8h+7 in c16[ti][h]
};

// Both operand sets of a block in one assembly block: sixteen reads and a single wait, so
// the block pays one LDS round trip instead of two.
__device__ __forceinline__ void load_vkc(uint32_t stage, const Lane& L, VFrags& fv, KCFrags& fk) {
    u32x2 t[8];
    u32x4 k[4];
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16\n\t"
        "ds_read_b64_tr_b16 %1, %17\n\t"
        "ds_read_b64_tr_b16 %2, %18\n\t"
        "ds_read_b64_tr_b16 %3, %19\n\t"
        "ds_read_b64_tr_b16 %4, %16 offset:2048\n\t"
        "ds_read_b64_tr_b16 %5, %17 offset:2048\n\t"
        "ds_read_b64_tr_b16 %6, %18 offset:2048\n\t"
        "ds_read_b64_tr_b16 %7, %19 offset:2048\n\t"
        "ds_read_b128 %8, %20\n\t"
        "ds_read_b128 %9, %21\n\t"
        "ds_read_b128 %10, %20 offset:2048\n\t"
        "ds_read_b128 %11, %21 offset:2048\n\t"
        "ds_read_b128 %12, %22\n\t"
        "ds_read_b128 %13, %23\n\t"
        "ds_read_b128 %14, %22 offset:2048\n\t"
        "ds_read_b128 %15, %23 offset:2048\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5]), "=&v"(t[6]), "=&v"(t[7]),
          "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(fk.c16[0][0]), "=&v"(fk.c16[0][1]),
          "=&v"(fk.c16[1][0]), "=&v"(fk.c16[1][1])
        : "v"(stage + L.v[0][0]), "v"(stage + L.v[0][1]), "v"(stage + L.v[1][0]), "v"(stage + L.v[1][1]),
          "v"(stage + L.k[0]), "v"(stage + L.k[1]), "v"(stage + L.b[0]), "v"(stage + L.b[1]));
    static_assert(ROW_BYTES == 2048 && TILE_BYTES == 2048, "line and tile offsets in the assembly above");
#pragma unroll
    for (int ri = 0; ri < RW; ++ri)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const u32x2 lo = t[4 * ri + 2 * m], hi = t[4 * ri + 2 * m + 1];
            const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
            fv.vA[ri][m] = __builtin_bit_cast(bf16x8, w);
            fk.kA[ri][m] = __builtin_bit_cast(bf16x8, k[2 * ri + m]);
        }
}

// Score register r of query tile ti in log2 units relative to r_j: the image value for
// register r is half r % 2 of word (r % 8) / 2 of c16[ti][r / 8]; the conversion from
// fp16 folds into v_fma_mix_f32.
__device__ __forceinline__ float score_log2(const KCFrags& kc, int ti, const f32x16& S, int r) {
    const uint32_t word = kc.c16[ti][r >> 3][(r & 7) >> 1];   // a scalar copy: bit_cast of a vector element reads element 0
    const f16x2 h = __builtin_bit_cast(f16x2, word);
    return fmaf(S[r], kScale, static_cast<float>(h[r & 1]));
}

struct State {
    f32x16 O[RW][TW];
    float mref[RW][TW];    // reference of O and l, log2 units relative to r_j
    float lsum[RW][TW];
    __device__ void reset(float m0) {
#pragma unroll
        for (int ri = 0; ri < RW; ++ri)
#pragma unroll
            for (int ti = 0; ti < TW; ++ti) {
                O[ri][ti] = f32x16{};
                mref[ri][ti] = m0;
                lsum[ri][ti] = 0.0f;
            }
    }
};

// The wave's two units (lines ri = 0, 1) of query tile TI for one key block, with the
// exact running maximum.
template <int TI>
__device__ __forceinline__ void compute_tile_exact(const KCFrags& kc, const VFrags& vf, const bf16x8 (&qB)[RW][TW][2],
                                                   State& s) {
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    constexpr int ti = TI;
#pragma unroll
    for (int ri = 0; ri < RW; ++ri) {
        f32x16 S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kc.kA[ri][0], qB[ri][ti][0], f32x16{}, 0, 0, 0);
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kc.kA[ri][1], qB[ri][ti][1], S, 0, 0, 0);
        f32x16 x;
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = score_log2(kc, ti, S, r);
        float mx = x[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, x[r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mold = s.mref[ri][ti];
        const float mnew = fmaxf(mold, mx);
        const float alpha = mold == -INFINITY ? 0.0f : exp2f(mold - mnew);
        s.lsum[ri][ti] *= alpha;
#pragma unroll
        for (int r = 0; r < 16; ++r) s.O[ri][ti][r] *= alpha;
        s.mref[ri][ti] = mnew;
        const float sh = mnew == -INFINITY ? 0.0f : mnew;
        f32x16 P;
#pragma unroll
        for (int r = 0; r < 16; ++r) P[r] = __builtin_amdgcn_exp2f(x[r] - sh);
        const bf16x8 pb0 = __builtin_convertvector(__builtin_shufflevector(P, P, 0, 1, 2, 3, 4, 5, 6, 7), bf16x8);
        const bf16x8 pb1 = __builtin_convertvector(__builtin_shufflevector(P, P, 8, 9, 10, 11, 12, 13, 14, 15), bf16x8);
        float ls = s.lsum[ri][ti];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bf16x2 a0 = {pb0[2 * e], pb0[2 * e + 1]};
            const bf16x2 a1 = {pb1[2 * e], pb1[2 * e + 1]};
            ls = __builtin_amdgcn_fdot2_f32_bf16(a0, ones, ls, false);
            ls = __builtin_amdgcn_fdot2_f32_bf16(a1, ones, ls, false);
        }
        s.lsum[ri][ti] = ls;
        s.O[ri][ti] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf.vA[ri][0], pb0, s.O[ri][ti], 0, 0, 0);
        s.O[ri][ti] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf.vA[ri][1], pb1, s.O[ri][ti], 0, 0, 0);
    }
}

__device__ __forceinline__ void compute_block_exact(const KCFrags& kc, const VFrags& vf, const bf16x8 (&qB)[RW][TW][2],
                                                    State& s) {
    static_assert(TW == 2, "two query tiles per wave");
    compute_tile_exact<0>(kc, vf, qB, s);
    compute_tile_exact<1>(kc, vf, qB, s);
}

// Fast-pass block (reference r_j) as an explicit software pipeline over the wave's four
// units u = (tile u / 2, line u % 2).  Unit u's softmax runs in four chunks of 4 scores
// (4 v_fma_mix_f32 + 4 v_exp_f32, the bf16 conversion and row sum after every second
// chunk), and each chunk carries exactly one matrix instruction: the two halves of S for
// unit u + 1 during chunks 0 and 1, the two halves of P.V for unit u - 1 during chunks 2
// and 3.  On gfx950 a matrix instruction issued among transcendental instructions runs
// almost entirely in their shadow, while one issued among plain VALU instructions mostly
// does not, so the order is pinned with scheduling barriers.
template <int U>
__device__ __forceinline__ f32x16 s_half(const KCFrags& kc, const bf16x8 (&qB)[RW][TW][2], int m, const f32x16& acc) {
    constexpr int ti = U / RW, ri = U % RW;
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(kc.kA[ri][m], qB[ri][ti][m], acc, 0, 0, 0);
}

// `between` runs after the first unit's score instructions are issued (the block's copies:
// their address work then overlaps the matrix latency).
template <typename Between>
__device__ __forceinline__ void compute_block_pipe(const KCFrags& kc, const VFrags& vf, const bf16x8 (&qB)[RW][TW][2],
                                                   State& s, Between between) {
    static_assert(RW == 2 && TW == 2, "four units per wave");
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    f32x16 S[4];
    bf16x8 P[4][2];
    const f32x16 zero = {};
    S[0] = s_half<0>(kc, qB, 0, zero);
    S[0] = s_half<0>(kc, qB, 1, S[0]);
    __builtin_amdgcn_sched_barrier(0);
    between();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int ti = u / RW, ri = u % RW;
        float ls = s.lsum[ri][ti];
        f32x16 p;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (q == 0 && u + 1 < 4) {
                if (u + 1 == 1) S[1] = s_half<1>(kc, qB, 0, zero);
                if (u + 1 == 2) S[2] = s_half<2>(kc, qB, 0, zero);
                if (u + 1 == 3) S[3] = s_half<3>(kc, qB, 0, zero);
            }
            if (q == 1 && u + 1 < 4) {
                if (u + 1 == 1) S[1] = s_half<1>(kc, qB, 1, S[1]);
                if (u + 1 == 2) S[2] = s_half<2>(kc, qB, 1, S[2]);
                if (u + 1 == 3) S[3] = s_half<3>(kc, qB, 1, S[3]);
            }
            if (q >= 2 && u > 0) {
                const int pu = u - 1, pt = pu / RW, pr = pu % RW;
                s.O[pr][pt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf.vA[pr][q - 2], P[pu][q - 2], s.O[pr][pt], 0, 0, 0);
            }
#pragma unroll
            for (int r = 4 * q; r < 4 * q + 4; ++r) p[r] = __builtin_amdgcn_exp2f(score_log2(kc, ti, S[u], r));
            if (q == 1 || q == 3) {
                const int h = q / 2;
                const f32x8 ph = h == 0 ? __builtin_shufflevector(p, p, 0, 1, 2, 3, 4, 5, 6, 7)
                                        : __builtin_shufflevector(p, p, 8, 9, 10, 11, 12, 13, 14, 15);
                P[u][h] = __builtin_convertvector(ph, bf16x8);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bf16x2 a = {P[u][h][2 * e], P[u][h][2 * e + 1]};
                    ls = __builtin_amdgcn_fdot2_f32_bf16(a, ones, ls, false);
                }
                asm volatile("" : "+v"(ls));   // keep the row sums in this chunk
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        s.lsum[ri][ti] = ls;
    }
    s.O[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf.vA[1][0], P[3][0], s.O[1][1], 0, 0, 0);
    s.O[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf.vA[1][1], P[3][1], s.O[1][1], 0, 0, 0);
}

static_assert(NSTAGE == 3 || NSTAGE == 4, "ring of three or four stages");

// Barrier after which every wave's copies except those of the NSTAGE - 2 most recent
// blocks are complete (those are needed later, the one before them next).
__device__ __forceinline__ void barrier_keep_newest() {
    constexpr int keep = COPIES_PER_BLOCK * (NSTAGE - 2);
    static_assert(keep >= 1 && keep <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%c0)\n\ts_barrier" ::"i"(keep) : "memory");
}
// Barrier after which every copy issued so far is complete.
__device__ __forceinline__ void barrier_drain() { asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory"); }

// Prologue: copies of blocks nb0 .. nb0 + NSTAGE-2 in flight, block nb0 complete everywhere.
__device__ __forceinline__ void key_prologue(const Ctx& cx, int wave, int lane, int nb0, int nb1) {
    for (int n = nb0; n < nb0 + NSTAGE - 1 && n < nb1; ++n) stage_block(cx, n, wave, lane);
    if (nb1 - nb0 >= NSTAGE - 1)
        barrier_keep_newest();
    else
        barrier_drain();
}

// One step of the key loop: read block n's operands, issue the copy of block
// n + NSTAGE - 1 into the stage block n - 1 used, compute block n, and leave block n + 1
// complete for every wave.
template <bool EXACT_MAX>
__device__ __forceinline__ void key_step(const Ctx& cx, const Lane& L, int wave, int lane,
                                         const bf16x8 (&qB)[RW][TW][2], State& s, int n, int nblk) {
    const uint32_t st = stage_addr(n);
    VFrags vf;
    KCFrags kc;
    load_vkc(st, L, vf, kc);
    const bool issue = n + NSTAGE - 1 < nblk;
    if constexpr (!EXACT_MAX) {
        compute_block_pipe(kc, vf, qB, s, [&] {
            if (issue) stage_block(cx, n + NSTAGE - 1, wave, lane);
        });
    } else {
        if (issue) stage_block(cx, n + NSTAGE - 1, wave, lane);
        compute_block_exact(kc, vf, qB, s);
    }
    if (issue)
        barrier_keep_newest();
    else
        barrier_drain();
}

// Fast pass over key blocks nb0 .. nb1-1: every block with the reference r_j.  Each loop
// has a single compute path, so the accumulators stay in place across blocks.
__device__ __forceinline__ void key_loop_fast(const Ctx& cx, const Lane& L, int wave, int lane,
                                              const bf16x8 (&qB)[RW][TW][2], State& s, int nb0, int nb1) {
    key_prologue(cx, wave, lane, nb0, nb1);
    for (int n = nb0; n < nb1; ++n) key_step<false>(cx, L, wave, lane, qB, s, n, nb1);
}

// Exact pass: the running maximum is refreshed on every block.
__device__ __forceinline__ void key_loop_exact(const Ctx& cx, const Lane& L, int wave, int lane,
                                               const bf16x8 (&qB)[RW][TW][2], State& s, int nb0, int nb1) {
    key_prologue(cx, wave, lane, nb0, nb1);
    for (int n = nb0; n < nb1; ++n) key_step<true>(cx, L, wave, lane, qB, s, n, nb1);
}

// A column block whose flag in `wide` is set (bias spread beyond kImageSpan) is left to the
// fp32 kernel that runs after this one: nothing is written for it, except that in split-key
// mode every split stores the empty state (the fp32 kernel then stores split 0's).
__global__ void __launch_bounds__(NTHR, 2) bf16_mfma_kernel(Problem p, Strides sd, const _Float16* img, const float* ref,
                                                         const int* wide, int n_jb, int n_rg, int nblk, int total) {
    // XCD-aware remap: XCD x (= hardware id mod 8) walks a contiguous range of logical ids.
    const int w = blockIdx.x;
    const int xcd = w % NXCD, slot = w / NXCD;
    const int base = total / NXCD, extra = total % NXCD;
    const int logical = xcd * base + (xcd < extra ? xcd : extra) + slot;
    // within one (b, h): strips of TILE_RG line groups, each cut into tiles of TILE_RG x
    // TILE_JB (line group, column block) pairs, column block fastest inside a tile; the last
    // strip and the last tile of a strip may be narrower
    const int bh = logical / (n_jb * n_rg);
    const int rem = logical - bh * n_jb * n_rg;
    const int strip = rem / (TILE_RG * n_jb);
    const int nr = min(TILE_RG, n_rg - strip * TILE_RG);
    const int o = rem - strip * TILE_RG * n_jb;
    const int tile = o / (nr * TILE_JB);
    const int nj = min(TILE_JB, n_jb - tile * TILE_JB);
    const int o2 = o - tile * nr * TILE_JB;
    const int rg = strip * TILE_RG + o2 / nj;
    const int jb = tile * TILE_JB + o2 % nj;
    const int64_t b = bh / p.H, h = bh % p.H;
    const int64_t i0 = static_cast<int64_t>(rg) * R, j0 = static_cast<int64_t>(jb) * BJ;
    const int64_t lines = p.ending ? p.N : p.I;      // rows i, or columns j for the ending node
    const int64_t bh_off = b * sd.batch + h * D;      // element offset of (b, line 0, query 0, h)

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;   // wave is uniform
    const int row0 = (wave / (QT / TW)) * RW;       // first of this wave's lines in the group
    const int tile0 = (wave % (QT / TW)) * TW;      // first of this wave's query tiles
    const Lane L = lane_layout(lane, row0, tile0);

    Ctx cx;
    {
        cx.key_bytes = sd.key * 2;
#pragma unroll
        for (int t = 0; t < KV_PER_WAVE; ++t) {
            // piece pi: line pi / 4, K (0) or V (1) = (pi / 2) % 2, keys 16 * (pi % 2) .. +15
            const int pi = KV_PER_WAVE * wave + t;
            const int line = pi >> 2, kv = (pi >> 1) & 1, half = pi & 1;
            int64_t i = i0 + line;
            i = i < lines ? i : lines - 1;           // padded lines read a real line (never stored)
            const int64_t row_off = (bh_off + i * sd.line + p.k0 * sd.key) * 2;
            cx.kv_row[t] = static_cast<const char*>(kv ? p.v : p.k) + row_off;
            cx.kv_lds[t] = (kv ? V_OFF : K_OFF) + line * ROW_BYTES + half * 1024;
            cx.key_local[t] = 16 * half + (lane >> 2);
            cx.part_bytes[t] = kv_chunk(cx.key_local[t], lane & 3) * 16;   // logical part at this slot
            cx.lane_off[t] = static_cast<uint32_t>(cx.key_local[t] * cx.key_bytes + cx.part_bytes[t]);
        }
        cx.img_wg = img + (static_cast<int64_t>(bh) * n_jb + jb) * nblk * static_cast<int64_t>(IMG_HALVES);
        cx.last_key = static_cast<int>(p.nkeys() - 1);
        cx.plan = BlockPlan(p.nkeys());
    }

    // Q^T operands (B of S^T = K Q^T): query j = tile*32 + c, d = 16m + 8*h2 .. +7.
    bf16x8 qB[RW][TW][2];
#pragma unroll
    for (int ri = 0; ri < RW; ++ri)
#pragma unroll
        for (int ti = 0; ti < TW; ++ti) {
            const int64_t i = i0 + row0 + ri, j = j0 + (tile0 + ti) * 32 + L.c;
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                bf16x8 z = {};
                if (i < lines && j < p.N)
                    z = *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(p.q) + bh_off + i * sd.line +
                                                         j * sd.query + 16 * m + 8 * L.h2);
                qB[ri][ti][m] = z;
            }
        }

    // let the Q loads land before the key loop starts its copies, so that their first use
    // does not wait for the copies as well (vmcnt(0); expcnt, lgkmcnt unconstrained)
    __builtin_amdgcn_s_waitcnt(0x0F70);

    // split-key mode (gridDim.y > 1): this workgroup folds key blocks nb0 .. nb1-1 into a
    // partial state; the launch points out, st_m, st_l at split 0's partials
    const int split = blockIdx.y, n_split = gridDim.y;
    const int nb0 = static_cast<int>(static_cast<int64_t>(split) * nblk / n_split);
    const int nb1 = static_cast<int>(static_cast<int64_t>(split + 1) * nblk / n_split);
    if (n_split > 1) {
        const int64_t rows = p.B * p.I * p.N * p.H;
        p.out += split * rows * D;
        p.st_m += split * rows;
        p.st_l += split * rows;
    }

    if (wide[static_cast<int64_t>(bh) * n_jb + jb]) {   // the fp32 kernel's block
        if (n_split > 1) {
#pragma unroll
            for (int ri = 0; ri < RW; ++ri)
#pragma unroll
                for (int ti = 0; ti < TW; ++ti) {
                    const int64_t i = i0 + row0 + ri, j = j0 + (tile0 + ti) * 32 + L.c;
                    if (!(i < lines && j < p.N)) continue;
                    const int64_t qo = bh_off + i * sd.line + j * sd.query;
#pragma unroll
                    for (int a = 0; a < 4; ++a) *reinterpret_cast<f32x4*>(p.out + qo + 8 * a + 4 * L.h2) = f32x4{};
                    if (L.h2 == 0) {
                        p.st_m[qo / D] = -INFINITY;
                        p.st_l[qo / D] = 0.0f;
                    }
                }
        }
        return;
    }

    State s;
    s.reset(0.0f);
    if (tid == 0) g_redo = 0;
    key_loop_fast(cx, L, wave, lane, qB, s, nb0, nb1);

    // accept the pass only if every normaliser is in range and every accumulator finite
    bool bad = false;
#pragma unroll
    for (int ri = 0; ri < RW; ++ri)
#pragma unroll
        for (int ti = 0; ti < TW; ++ti) {
            const float lt = s.lsum[ri][ti] + __shfl_xor(s.lsum[ri][ti], 32);
            bool ok = lt >= kLo && lt <= kHi;
#pragma unroll
            for (int r = 0; r < 16; ++r) ok = ok && __builtin_isfinite(s.O[ri][ti][r]);
            bad = bad || !ok;
        }
    if (__any(bad) && lane == 0) g_redo = 1;
    __syncthreads();
    if (g_redo) {
        s.reset(-INFINITY);
        key_loop_exact(cx, L, wave, lane, qB, s, nb0, nb1);
    }

    // out = O / l; lanes l and l^32 hold disjoint keys of the same query.  In state mode
    // out receives O itself, with the reference in natural-log units (r_j + m ln 2) and l;
    // the log-sum-exp is that reference plus ln l.
    const bool state = p.st_m != nullptr;
    float lt[RW][TW];
#pragma unroll
    for (int ri = 0; ri < RW; ++ri)
#pragma unroll
        for (int ti = 0; ti < TW; ++ti) lt[ri][ti] = s.lsum[ri][ti] + __shfl_xor(s.lsum[ri][ti], 32);
    if (state && p.update) {
        // fold this range's state into the running one (merge rule, natural-log units).  Every
        // old value is loaded before anything is stored, so all of them are in flight at once
        // (loads after stores to the same array would each wait for the one before).
        f32x4 old[RW][TW][4];
        float m0[RW][TW], l0[RW][TW];
#pragma unroll
        for (int ri = 0; ri < RW; ++ri)
#pragma unroll
            for (int ti = 0; ti < TW; ++ti) {
                const int64_t i = i0 + row0 + ri, j = j0 + (tile0 + ti) * 32 + L.c;
                const bool ok = i < lines && j < p.N;
                const int64_t qo = bh_off + (ok ? i * sd.line + j * sd.query : 0);
                m0[ri][ti] = ok ? p.st_m[qo / D] : -INFINITY;
                l0[ri][ti] = ok ? p.st_l[qo / D] : 0.0f;
#pragma unroll
                for (int a = 0; a < 4; ++a)
                    old[ri][ti][a] = ok ? *reinterpret_cast<const f32x4*>(p.out + qo + 8 * a + 4 * L.h2) : f32x4{};
            }
        const bool fin = p.fin != nullptr;      // final step: write the folded result as out and lse
#pragma unroll
        for (int ri = 0; ri < RW; ++ri)
#pragma unroll
            for (int ti = 0; ti < TW; ++ti) {
                const int64_t i = i0 + row0 + ri, j = j0 + (tile0 + ti) * 32 + L.c;
                if (!(i < lines && j < p.N)) continue;
                const bool some = lt[ri][ti] > 0.0f;
                if (!some && !fin) continue;    // an empty range leaves the state as it is
                const int64_t qo = bh_off + i * sd.line + j * sd.query;
                const float m1 = s.mref[ri][ti] * kLn2 + ref[static_cast<int64_t>(bh) * n_jb * BJ + j];
                float a0 = 1.0f, a1 = 0.0f, mm = m0[ri][ti];   // empty range: the old state as it is
                if (some) {
                    a0 = 0.0f;
                    a1 = 1.0f;
                    mm = m1;
                    if (l0[ri][ti] > 0.0f) {
                        mm = fmaxf(m0[ri][ti], m1);
                        a0 = expf(m0[ri][ti] - mm);
                        a1 = expf(m1 - mm);
                    }
                }
                const float ln = a0 * l0[ri][ti] + a1 * lt[ri][ti];
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const f32x4 o0 = a0 != 0.0f ? old[ri][ti][a] : f32x4{};
                    f32x4 x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        x[e] = fmaf(a0, o0[e], a1 * s.O[ri][ti][4 * a + e]);
                        if (fin) x[e] = ln > 0.0f ? x[e] / ln : 0.0f;
                    }
                    *reinterpret_cast<f32x4*>((fin ? p.fin : p.out) + qo + 8 * a + 4 * L.h2) = x;
                }
                if (L.h2 == 0) {
                    if (!fin) {
                        p.st_m[qo / D] = mm;
                        p.st_l[qo / D] = ln;
                    } else if (p.lse) {
                        p.lse[qo / D] = ln > 0.0f ? mm + logf(ln) : -INFINITY;
                    }
                }
            }
        return;
    }
    // the references r_j of this lane's two queries, loaded before any store
    float rj[TW];
#pragma unroll
    for (int ti = 0; ti < TW; ++ti) {
        const int64_t j = j0 + (tile0 + ti) * 32 + L.c;
        rj[ti] = ((state || p.lse) && j < p.N) ? ref[static_cast<int64_t>(bh) * n_jb * BJ + j] : 0.0f;
    }
#pragma unroll
    for (int ri = 0; ri < RW; ++ri)
#pragma unroll
        for (int ti = 0; ti < TW; ++ti) {
            const int64_t i = i0 + row0 + ri, j = j0 + (tile0 + ti) * 32 + L.c;
            if (!(i < lines && j < p.N)) continue;
            const float lq = lt[ri][ti];
            const int64_t qo = bh_off + i * sd.line + j * sd.query;
            float* o = p.out + qo;
            // correctly rounded O / l: a single surviving key returns its v exactly
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                f32x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float acc = s.O[ri][ti][4 * a + e];
                    x[e] = state ? acc : (lq > 0.0f ? acc / lq : 0.0f);
                }
                *reinterpret_cast<f32x4*>(o + 8 * a + 4 * L.h2) = x;
            }
            if (L.h2 == 0 && (state || p.lse)) {
                const float mnat = s.mref[ri][ti] * kLn2 + rj[ti];
                if (state) {
                    p.st_m[qo / D] = lq > 0.0f ? mnat : -INFINITY;
                    p.st_l[qo / D] = lq;
                }
                if (p.lse) p.lse[qo / D] = lq > 0.0f ? mnat + logf(lq) : -INFINITY;
            }
        }
}

// Workspace of the forward: the fp16 image, then the references r_j (fp32, padded to
// whole column blocks), the wide-span flag of every (b, h, column block) (int), then for
// the ending node REF_KS partial maxima per query, then in split-key mode the partial
// states (acc, m, l of every query, per split); each part 256-byte aligned.  The starting
// node's single partial maximum is r_j itself.
//
// Split-key mode: a call whose grid would leave most of the chip idle (attention with
// pair bias is one line; small N) cuts the key blocks into up to MAX_SPLIT ranges run side
// by side, each of at least MIN_SPLIT_BLOCKS blocks, and joins them with the merge rule.
constexpr int MAX_SPLIT = 16;
constexpr int MIN_SPLIT_BLOCKS = 8;
constexpr int64_t FILL_WGS = 512;           // two workgroups per compute unit
struct FwdLayout {
    int64_t n_jb, nblk, nqp, n_rg, wgs, rows;
    int n_part, n_split;
    size_t img_bytes, ref_off, wide_off, part_off, split_off, total;
};
FwdLayout fwd_layout(const Problem& p) {
    FwdLayout L;
    L.n_jb = (p.N + BJ - 1) / BJ;
    L.nqp = L.n_jb * BJ;
    L.nblk = BlockPlan(p.nkeys()).count();
    L.n_part = p.ending ? REF_KS : 1;
    L.n_rg = ((p.ending ? p.N : p.I) + R - 1) / R;
    L.wgs = L.n_jb * L.n_rg * p.B * p.H;
    L.rows = p.B * p.I * p.N * p.H;
    L.n_split = 1;
    if (p.st_m == nullptr && L.wgs < FILL_WGS) {
        const int64_t want = (FILL_WGS + L.wgs - 1) / L.wgs, most = L.nblk / MIN_SPLIT_BLOCKS;
        L.n_split = static_cast<int>(min(min(want, most), static_cast<int64_t>(MAX_SPLIT)));
        if (L.n_split < 2) L.n_split = 1;
    }
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    L.img_bytes = static_cast<size_t>(p.B * p.H * L.n_jb * L.nblk) * IMG_HALVES * 2;
    L.ref_off = up(L.img_bytes);
    const size_t ref_bytes = static_cast<size_t>(p.B * p.H * L.nqp) * 4;
    L.wide_off = up(L.ref_off + ref_bytes);
    const size_t wide_bytes = static_cast<size_t>(p.B * p.H * L.n_jb) * 4;
    L.part_off = up(L.wide_off + wide_bytes);
    L.split_off = p.ending ? up(L.part_off + ref_bytes * REF_KS) : L.part_off;
    L.total = L.n_split > 1 ? L.split_off + static_cast<size_t>(L.n_split * L.rows) * (D + 2) * 4
                            : (p.ending ? L.part_off + ref_bytes * REF_KS : L.wide_off + wide_bytes);
    return L;
}

}  // namespace

size_t bf16_workspace_bytes(const Problem& p) { return fwd_layout(p).total; }

size_t bias_image_bytes(const Problem& p) {
    const int64_t n_jb = (p.N + IMG_BJ - 1) / IMG_BJ;
    const int64_t nblk = BlockPlan(p.nkeys()).count();
    return static_cast<size_t>(p.B * p.H * n_jb * nblk) * IMG_FLOATS * sizeof(float);
}

int64_t bias_image_blocks(const Problem& p) { return BlockPlan(p.nkeys()).count(); }

hipError_t launch_bias_image(const Problem& p, float* img, hipStream_t stream) {
    const int64_t n_jb = (p.N + IMG_BJ - 1) / IMG_BJ;
    const int64_t nblk = BlockPlan(p.nkeys()).count();
    if (nblk > 0x7FFFFFFF || n_jb > 65535 || p.B * p.H > 65535) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(bias_image_kernel, dim3(static_cast<unsigned>(nblk), static_cast<unsigned>(n_jb),
                                               static_cast<unsigned>(p.B * p.H)),
                       dim3(IMG_THR), 0, stream, p, img, static_cast<int>(n_jb), static_cast<int>(nblk));
    return hipGetLastError();
}

namespace {
// The bias prepass: r_j (bias_ref_kernel), then the fp16 image (bias_image16_kernel).
hipError_t launch_prepass(const Problem& p, const FwdLayout& Ly, void* workspace, int64_t n_qg, hipStream_t stream) {
    _Float16* img = static_cast<_Float16*>(workspace);
    float* ref = reinterpret_cast<float*>(static_cast<char*>(workspace) + Ly.ref_off);
    int* wide = reinterpret_cast<int*>(static_cast<char*>(workspace) + Ly.wide_off);
    float* part = Ly.n_part > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + Ly.part_off) : ref;
    const unsigned bhs = static_cast<unsigned>(p.B * p.H);
    const dim3 ref_grid = p.ending ? dim3(static_cast<unsigned>(Ly.nqp / 64), REF_KS, bhs)
                                   : dim3(static_cast<unsigned>(Ly.nqp / 4), 1, bhs);
    hipLaunchKernelGGL(bias_ref_kernel, ref_grid, dim3(256), 0, stream, p, part, Ly.nqp, wide,
                       static_cast<int>(Ly.n_jb));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bias_image16_kernel,
                       dim3(static_cast<unsigned>(n_qg), static_cast<unsigned>((Ly.nblk + IMG16_NB - 1) / IMG16_NB), bhs),
                       dim3(256), 0, stream, p, part, Ly.n_part, img, ref, static_cast<int>(Ly.n_jb),
                       static_cast<int>(Ly.nblk), wide);
    return hipGetLastError();
}
}  // namespace

Prepass16 prepass16_layout(const Problem& p) {
    const FwdLayout L = fwd_layout(p);
    Prepass16 q;
    q.cols = BJ;
    q.n_jb = L.n_jb;
    q.nqp = L.nqp;
    q.nblk = L.nblk;
    q.ref_off = L.ref_off;
    q.wide_off = L.wide_off;
    q.bytes = L.wide_off + static_cast<size_t>(p.B * p.H * L.n_jb) * 4;
    return q;
}

hipError_t launch_prepass16(const Problem& p, void* workspace, hipStream_t stream) {
    if (p.ending || p.B * p.H > 65535 || fwd_layout(p).nblk > 65535) return hipErrorInvalidConfiguration;
    const FwdLayout Ly = fwd_layout(p);
    return launch_prepass(p, Ly, workspace, Ly.n_jb * (BJ / IMG16_Q), stream);
}

hipError_t launch_bf16_mfma(const Problem& p, void* workspace, hipStream_t stream) {
    const FwdLayout Ly = fwd_layout(p);
    const int64_t n_rg = Ly.n_rg;
    const Strides sd = strides_of(p);
    const int64_t total = Ly.wgs;
    const int64_t n_qg = Ly.n_jb * (BJ / IMG16_Q);
    // the 32 keys of a block are addressed with 32-bit byte offsets from the block's first key
    if (total > 0x7FFFFFFF || Ly.nblk > 65535 || Ly.nqp / 4 > 0x7FFFFFFF || p.B * p.H > 65535 ||
        BK * sd.key * 2 > 0x7FFFFFFF)
        return hipErrorInvalidConfiguration;
    _Float16* img = static_cast<_Float16*>(workspace);
    float* ref = reinterpret_cast<float*>(static_cast<char*>(workspace) + Ly.ref_off);
    const int* wide = reinterpret_cast<const int*>(static_cast<char*>(workspace) + Ly.wide_off);
    hipError_t e = launch_prepass(p, Ly, workspace, n_qg, stream);
    if (e != hipSuccess) return e;
    if (Ly.n_split == 1) {
        hipLaunchKernelGGL(bf16_mfma_kernel, dim3(static_cast<unsigned>(total)), dim3(NTHR), 0, stream, p, sd, img, ref,
                           wide, static_cast<int>(Ly.n_jb), static_cast<int>(n_rg), static_cast<int>(Ly.nblk),
                           static_cast<int>(total));
        if ((e = hipGetLastError()) != hipSuccess) return e;
        return launch_general_wide(p, wide, BJ, stream);     // the column blocks beyond the span
    }
    // split-key mode: partial states of every split, then one join into out (and lse)
    float* acc = reinterpret_cast<float*>(static_cast<char*>(workspace) + Ly.split_off);
    float* sm = acc + Ly.n_split * Ly.rows * D;
    float* sl = sm + Ly.n_split * Ly.rows;
    Problem q = p;
    q.out = acc;
    q.st_m = sm;
    q.st_l = sl;
    q.lse = nullptr;
    hipLaunchKernelGGL(bf16_mfma_kernel, dim3(static_cast<unsigned>(total), static_cast<unsigned>(Ly.n_split)),
                       dim3(NTHR), 0, stream, q, sd, img, ref, wide, static_cast<int>(Ly.n_jb), static_cast<int>(n_rg),
                       static_cast<int>(Ly.nblk), static_cast<int>(total));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = launch_general_wide(q, wide, BJ, stream)) != hipSuccess) return e;   // split 0's state
    return launch_state_combine(acc, sm, sl, Ly.n_split, Ly.rows, D, p.out, p.lse, stream);
}

}  // namespace tri_attn
