// bf16 triangle attention on gfx950 matrix cores (head size D = 32).
//
// Per batch b and head h the rows i are independent attention problems that share one
// N x N "triangular" bias bias[b,h,j,k] ("Fold-CP", Table 1 "Triangle Attention" and
// Figure 2(a)).  A workgroup owns R = 8 rows i and BJ = 128 query columns j of one
// (b, h) and streams the key axis in blocks of 32 keys.  Key blocks follow the ring-step
// tiles (Table 1's caption): they start at every tile start and are cut short at every
// tile end, so each tile is folded into the running softmax state as one ring step
// (the running state is the merged state of the tiles seen so far).
//
// Two kernels run per call:
//   1. bias_image_kernel: converts the bias once into the fp32 image the main kernel
//      stages verbatim: per (b, h, column block, key block) a 128 x 32 tile holding
//      (bias + mask) * sqrt(D), -inf for keys past the tile end, 16-byte chunks swizzled
//      against LDS bank conflicts.  Every row i of the workgroup reuses it from LDS.
//   2. bf16_mfma_kernel: per key block the workgroup copies K and V of its 8 rows
//      ([key][d], natural layout) and the bias tile straight from global memory into
//      LDS (global_load_lds_dwordx4, double buffered, no registers on the way).  Each
//      of the 8 waves owns 2 rows x 2 query tiles of 32 and runs, per (row, tile):
//        S^T = K Q^T + C       two v_mfma_f32_32x32x16_bf16, C = the bias tile, so
//                              S = sqrt(D) * (q.k / sqrt(D) + bias + mask) in fp32
//        p   = 2^(S * log2(e)/sqrt(D) + nb),  nb = -m_ref * log2(e)/sqrt(D)
//        O^T += V^T P^T        two v_mfma_f32_32x32x16_bf16 on the bf16-rounded p;
//                              V^T comes from ds_read_b64_tr_b16 on the [key][d] tile
//      The row sum is taken per lane with v_dot2_f32_bf16 on the rounded p.  In the
//      fixed-reference blocks the four units run as a software pipeline in which every
//      group of four exponentials carries one matrix instruction of the neighbouring
//      units (compute_block_pipe).
//
// Softmax reference.  The first key block sets m_ref to its exact row maximum (one
// cross-lane step: in the 32x32 output layout lanes l and l^32 hold the 16 + 16 keys of
// one query).  Later blocks keep that reference -- O and l share it, so the result is
// exact whatever it is -- and need no maximum, no cross-lane step and no branch.  At the
// end every lane checks that its normaliser lies in [2^-64, 2^64] and its accumulator is
// finite; if any lane of the workgroup fails (scores that jump far above the first
// block's maximum, or rows whose keys are all masked), the workgroup recomputes its
// whole key loop with the exact running maximum refreshed on every block.
//
// Workgroup ids are remapped so that each XCD walks a contiguous range of (b, h, row
// group, column block) tiles of 4 row groups x 8 column blocks: the workgroups an XCD runs
// together share each row group's K/V stream 8 ways and each bias tile 4 ways in its L2.
#include "launch.h"

#include <cmath>
#include <cstddef>

namespace tri_attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))
#define GLOBAL_PTR(T, p) ((const __attribute__((address_space(1))) T*)(p))

constexpr int D = 32;
constexpr int BK = 32;                      // keys per block
constexpr int R = 8;                        // rows i per workgroup
constexpr int QT = 4;                       // 32-wide query tiles per workgroup
constexpr int BJ = 32 * QT;                 // query columns per workgroup
constexpr int RW = 2;                       // rows per wave
constexpr int TW = 2;                       // query tiles per wave
constexpr int NWAVE = (R / RW) * (QT / TW);
constexpr int NTHR = 64 * NWAVE;
constexpr int NXCD = 8;
#ifndef TRI_ATTN_STAGES
#define TRI_ATTN_STAGES 3
#endif
#ifndef TRI_ATTN_TILE_RG
#define TRI_ATTN_TILE_RG 4
#endif
#ifndef TRI_ATTN_TILE_JB
#define TRI_ATTN_TILE_JB 8
#endif
constexpr int NSTAGE = TRI_ATTN_STAGES;     // key blocks in flight (LDS ring of stages)
constexpr int TILE_RG = TRI_ATTN_TILE_RG;   // row groups x column blocks that one XCD
constexpr int TILE_JB = TRI_ATTN_TILE_JB;   //   works on together (L2 reuse of K/V and bias)
constexpr int IMG_FLOATS = BJ * BK;         // one bias tile of the image
static_assert(NWAVE == R, "wave w stages K and V of row w");
static_assert(IMG_FLOATS * 4 == 2 * NWAVE * 1024, "each wave stages two 1 KB pieces of the bias tile");

struct Stage {
    __bf16 k[R][BK][D];    // 64-byte rows, 16-byte chunks swizzled by kv_chunk()
    __bf16 v[R][BK][D];
    float bias[BJ][BK];    // 128-byte rows, 16-byte chunks swizzled by bias_chunk()
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSqrtD = 5.656854249492381f;   // sqrt(32)
constexpr float kScale = kLog2e / kSqrtD;      // S units -> log2 units
constexpr float kLo = 5.421010862427522e-20f;  // 2^-64
constexpr float kHi = 1.8446744073709552e19f;  // 2^64

__host__ __device__ constexpr int kv_chunk(int key, int part) { return part ^ ((key >> 1) & 3); }
__host__ __device__ constexpr int bias_chunk(int j, int part) { return img_chunk(j, part); }
static_assert(IMG_BJ == BJ && IMG_BK == BK, "the image layout published in launch.h");

// Key block n of the tile-ordered sequence: tiles ascending, 32-key blocks inside each.
struct KeyBlock {
    int64_t kb;
    int nk;
};
struct BlockPlan {
    int64_t N;
    int T, extra, nb_big, nb_small;
    int64_t big, small;
    BlockPlan() = default;
    __host__ __device__ BlockPlan(int64_t n, int t) : N(n), T(t) {
        small = N / T;
        big = small + 1;
        extra = static_cast<int>(N % T);
        nb_big = static_cast<int>((big + BK - 1) / BK);
        nb_small = static_cast<int>((small + BK - 1) / BK);
    }
    __host__ __device__ int64_t count() const {
        return static_cast<int64_t>(extra) * nb_big + static_cast<int64_t>(T - extra) * nb_small;
    }
    __host__ __device__ KeyBlock block(int n) const {
        int64_t t, loc, len;
        if (n < extra * nb_big) {
            t = n / nb_big; loc = n % nb_big; len = big;
        } else {
            const int n2 = n - extra * nb_big;
            t = extra + n2 / nb_small; loc = n2 % nb_small; len = small;
        }
        const int64_t rest = len - loc * BK;
        return {tile_start(t, N, T) + loc * BK, static_cast<int>(rest < BK ? rest : BK)};
    }
};

// ---------------------------------------------------------------------------------------
// 1. bias image
// ---------------------------------------------------------------------------------------
constexpr int IMG_THR = 256;

__global__ void __launch_bounds__(IMG_THR) bias_image_kernel(Problem p, float* img, int n_jb, int nblk) {
    const int n = blockIdx.x, jb = blockIdx.y, bh = blockIdx.z;
    const int64_t b = bh / p.H;
    const KeyBlock kbk = BlockPlan(p.nkeys(), p.T).block(n);
    const int64_t key0 = p.k0 + kbk.kb;        // absolute index of the block's first key
    const uint16_t* bg = static_cast<const uint16_t*>(p.bias);
    float* dst = img + ((static_cast<int64_t>(bh) * n_jb + jb) * nblk + n) * IMG_FLOATS;
    const int kk = threadIdx.x % BK;
    const bool key_ok = kk < kbk.nk;
    const float mk = (p.mask && key_ok) ? p.mask[b * p.N + key0 + kk] : 0.0f;
#pragma unroll
    for (int s = 0; s < IMG_FLOATS / IMG_THR; ++s) {
        const int jj = (threadIdx.x + s * IMG_THR) / BK;
        const int64_t j = static_cast<int64_t>(jb) * BJ + jj;
        float val = -INFINITY;
        if (key_ok) {
            // starting node bias[b, h, j, key]; ending node the transpose, bias[b, h, key, j]
            const int64_t bi = p.ending ? (bh * p.N + key0 + kk) * p.N + j : (bh * p.N + j) * p.N + key0 + kk;
            const float bv = j < p.N ? __uint_as_float(static_cast<uint32_t>(bg[bi]) << 16) : 0.0f;
            val = (bv + mk) * kSqrtD;
        }
        dst[jj * BK + bias_chunk(jj, kk / 4) * 4 + kk % 4] = val;
    }
}

// ---------------------------------------------------------------------------------------
// 2. attention
// ---------------------------------------------------------------------------------------
struct Ctx {
    const char* k_row;      // K of this wave's staged line at the first key of the range
    const char* v_row;
    const float* img_wg;    // this workgroup's bias tiles, nblk consecutive 128 x 32 tiles
    int64_t key_bytes;      // bytes between consecutive keys of a line
    int key_local[2];       // key of this lane's 16-byte slot in the two 1 KB pieces
    int part_bytes[2];      // byte offset of the slot's logical 16-byte part inside the key
    int last_key;           // index of the last key of the range
    BlockPlan plan;
};

// Wave w copies K and V of staged row w (two 1 KB pieces each) and two 1 KB pieces of the
// bias tile; lane l of a piece carries 16 bytes.
__device__ __forceinline__ void stage_block(const Ctx& cx, int n, Stage& st, int wave, int lane) {
    const KeyBlock kbk = cx.plan.block(n);
    const int kb = static_cast<int>(kbk.kb);
    const char* kbase = cx.k_row + kbk.kb * cx.key_bytes;
    const char* vbase = cx.v_row + kbk.kb * cx.key_bytes;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        // padded keys read a real key (their bias is -inf); offsets from the block's first key
        const int rel = min(kb + cx.key_local[half], cx.last_key) - kb;
        const int off = rel * static_cast<int>(cx.key_bytes) + cx.part_bytes[half];
        __builtin_amdgcn_global_load_lds(GLOBAL_PTR(void, kbase + off), LDS_PTR(void, &st.k[wave][16 * half][0]), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(GLOBAL_PTR(void, vbase + off), LDS_PTR(void, &st.v[wave][16 * half][0]), 16, 0, 0);
    }
    const float* src = cx.img_wg + static_cast<int64_t>(n) * IMG_FLOATS + lane * 4;
    float* flat = &st.bias[0][0];
#pragma unroll
    for (int piece = 0; piece < 2; ++piece) {
        const int base = (2 * wave + piece) * 256;              // 256 floats = 1 KB
        __builtin_amdgcn_global_load_lds(GLOBAL_PTR(void, src + base), LDS_PTR(void, flat + base), 16, 0, 0);
    }
}

constexpr int ROW_BYTES = BK * D * 2;       // one staged row of K or V
constexpr int TILE_BYTES = 32 * BK * 4;     // 32 rows of the staged bias tile
constexpr int STAGE_BYTES = static_cast<int>(sizeof(Stage));
constexpr int K_OFF = static_cast<int>(offsetof(Stage, k));
constexpr int V_OFF = static_cast<int>(offsetof(Stage, v));
constexpr int B_OFF = static_cast<int>(offsetof(Stage, bias));
static_assert(RW == 2 && TW == 2, "the operand reads below address rows +ROW_BYTES and tiles +TILE_BYTES");

// LDS byte offsets (inside stage 0) of this lane's operand reads for its first row / tile.
struct Lane {
    int c, h2;
    uint32_t k[2];        // K operand of S^T = K Q^T, d-half m
    uint32_t v[2][2];     // ds_read_b64_tr_b16 sources of the V^T operand, [key half m][sub]
    uint32_t b[4];        // bias operand, 16-byte chunk a
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
    for (int a = 0; a < 4; ++a)
        L.b[a] = B_OFF + tile0 * TILE_BYTES + L.c * 128 + bias_chunk(L.c, 2 * a + L.h2) * 16;
    return L;
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Operands of one staged block.  The reads are inline assembly that waits for its own
// results (lgkmcnt) before returning: the compiler then sees no LDS read it would have to
// order against the global->LDS copies still in flight into the other stages.
struct VFrags {
    bf16x8 vA[RW][2];
};
struct KCFrags {
    bf16x8 kA[RW][2];
    f32x16 C[TW];
};

__device__ __forceinline__ void load_v(uint32_t stage, const Lane& L, VFrags& f) {
    u32x2 t[8];
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %9\n\t"
        "ds_read_b64_tr_b16 %2, %10\n\t"
        "ds_read_b64_tr_b16 %3, %11\n\t"
        "ds_read_b64_tr_b16 %4, %8 offset:2048\n\t"
        "ds_read_b64_tr_b16 %5, %9 offset:2048\n\t"
        "ds_read_b64_tr_b16 %6, %10 offset:2048\n\t"
        "ds_read_b64_tr_b16 %7, %11 offset:2048\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5]), "=&v"(t[6]), "=&v"(t[7])
        : "v"(stage + L.v[0][0]), "v"(stage + L.v[0][1]), "v"(stage + L.v[1][0]), "v"(stage + L.v[1][1]));
    static_assert(ROW_BYTES == 2048, "row offset in the assembly above");
#pragma unroll
    for (int ri = 0; ri < RW; ++ri)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const u32x2 lo = t[4 * ri + 2 * m], hi = t[4 * ri + 2 * m + 1];
            const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
            f.vA[ri][m] = __builtin_bit_cast(bf16x8, w);
        }
}

__device__ __forceinline__ void load_kc(uint32_t stage, const Lane& L, KCFrags& f) {
    u32x4 k[4], b[8];
    asm volatile(
        "ds_read_b128 %0, %12\n\t"
        "ds_read_b128 %1, %13\n\t"
        "ds_read_b128 %2, %12 offset:2048\n\t"
        "ds_read_b128 %3, %13 offset:2048\n\t"
        "ds_read_b128 %4, %14\n\t"
        "ds_read_b128 %5, %15\n\t"
        "ds_read_b128 %6, %16\n\t"
        "ds_read_b128 %7, %17\n\t"
        "ds_read_b128 %8, %14 offset:4096\n\t"
        "ds_read_b128 %9, %15 offset:4096\n\t"
        "ds_read_b128 %10, %16 offset:4096\n\t"
        "ds_read_b128 %11, %17 offset:4096\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(b[0]), "=&v"(b[1]), "=&v"(b[2]), "=&v"(b[3]),
          "=&v"(b[4]), "=&v"(b[5]), "=&v"(b[6]), "=&v"(b[7])
        : "v"(stage + L.k[0]), "v"(stage + L.k[1]), "v"(stage + L.b[0]), "v"(stage + L.b[1]), "v"(stage + L.b[2]),
          "v"(stage + L.b[3]));
    static_assert(TILE_BYTES == 4096, "tile offset in the assembly above");
#pragma unroll
    for (int ri = 0; ri < RW; ++ri)
#pragma unroll
        for (int m = 0; m < 2; ++m) f.kA[ri][m] = __builtin_bit_cast(bf16x8, k[2 * ri + m]);
#pragma unroll
    for (int ti = 0; ti < TW; ++ti)
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int e = 0; e < 4; ++e) f.C[ti][4 * a + e] = __uint_as_float(b[4 * ti + a][e]);
}

struct State {
    f32x16 O[RW][TW];
    float mref[RW][TW];
    float nb[RW][TW];
    float lsum[RW][TW];
    __device__ void reset() {
#pragma unroll
        for (int ri = 0; ri < RW; ++ri)
#pragma unroll
            for (int ti = 0; ti < TW; ++ti) {
                O[ri][ti] = f32x16{};
                mref[ri][ti] = -INFINITY;
                nb[ri][ti] = 0.0f;
                lsum[ri][ti] = 0.0f;
            }
    }
};

// The wave's two units (rows ri = 0, 1) of query tile TI for one key block.
template <bool EXACT_MAX, int TI>
__device__ __forceinline__ void compute_tile(const KCFrags& kc, const VFrags& vf, const bf16x8 (&qB)[RW][TW][2],
                                             State& s) {
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    constexpr int ti = TI;
    {
#pragma unroll
        for (int ri = 0; ri < RW; ++ri) {
            f32x16 S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kc.kA[ri][0], qB[ri][ti][0], kc.C[ti], 0, 0, 0);
            S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kc.kA[ri][1], qB[ri][ti][1], S, 0, 0, 0);
            if constexpr (EXACT_MAX) {
                float mx = S[0];
#pragma unroll
                for (int r = 1; r < 16; ++r) mx = fmaxf(mx, S[r]);
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                const float mold = s.mref[ri][ti];
                const float mnew = fmaxf(mold, mx);
                const float alpha = mold == -INFINITY ? 0.0f : exp2f((mold - mnew) * kScale);
                s.lsum[ri][ti] *= alpha;
#pragma unroll
                for (int r = 0; r < 16; ++r) s.O[ri][ti][r] *= alpha;
                s.mref[ri][ti] = mnew;
                s.nb[ri][ti] = mnew == -INFINITY ? 0.0f : -mnew * kScale;
            }
            const float nb = s.nb[ri][ti];
            f32x16 P;
#pragma unroll
            for (int r = 0; r < 16; ++r) P[r] = __builtin_amdgcn_exp2f(fmaf(S[r], kScale, nb));
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
}

template <bool EXACT_MAX>
__device__ __forceinline__ void compute_block(const KCFrags& kc, const VFrags& vf, const bf16x8 (&qB)[RW][TW][2],
                                              State& s) {
    static_assert(TW == 2, "two query tiles per wave");
    compute_tile<EXACT_MAX, 0>(kc, vf, qB, s);
    compute_tile<EXACT_MAX, 1>(kc, vf, qB, s);
}

// Fixed-reference block as an explicit software pipeline over the wave's four units
// u = (tile u / 2, row u % 2).  Unit u's softmax runs in four chunks of 4 scores (4 FMA +
// 4 v_exp_f32, the bf16 conversion and row sum after every second chunk), and each chunk
// carries exactly one matrix instruction: the two halves of S for unit u + 1 during
// chunks 0 and 1, the two halves of P.V for unit u - 1 during chunks 2 and 3.  On gfx950
// a matrix instruction issued among transcendental instructions runs almost entirely in
// their shadow, while one issued among plain VALU instructions mostly does not, so the
// order is pinned with scheduling barriers.
template <int U>
__device__ __forceinline__ f32x16 s_half(const KCFrags& kc, const bf16x8 (&qB)[RW][TW][2], int m, const f32x16& acc) {
    constexpr int ti = U / RW, ri = U % RW;
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(kc.kA[ri][m], qB[ri][ti][m], acc, 0, 0, 0);
}

__device__ __forceinline__ void compute_block_pipe(const KCFrags& kc, const VFrags& vf, const bf16x8 (&qB)[RW][TW][2],
                                                   State& s) {
    static_assert(RW == 2 && TW == 2, "four units per wave");
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    f32x16 S[4];
    bf16x8 P[4][2];
    S[0] = s_half<0>(kc, qB, 0, kc.C[0]);
    S[0] = s_half<0>(kc, qB, 1, S[0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int ti = u / RW, ri = u % RW;
        const float nb = s.nb[ri][ti];
        float ls = s.lsum[ri][ti];
        f32x16 p;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (q == 0 && u + 1 < 4) {
                if (u + 1 == 1) S[1] = s_half<1>(kc, qB, 0, kc.C[0]);
                if (u + 1 == 2) S[2] = s_half<2>(kc, qB, 0, kc.C[1]);
                if (u + 1 == 3) S[3] = s_half<3>(kc, qB, 0, kc.C[1]);
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
            for (int r = 4 * q; r < 4 * q + 4; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(S[u][r], kScale, nb));
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

__shared__ Stage g_stage[NSTAGE];
__shared__ int g_redo;

constexpr int COPIES_PER_BLOCK = 6;         // global_load_lds issued per wave per staged block
static_assert(NSTAGE == 3, "the barrier below keeps exactly one block of copies in flight");

// Barrier after which every wave's copies except the most recent block's are complete
// (the most recent block is still needed later, the one before it next).
__device__ __forceinline__ void barrier_keep_newest() {
    static_assert(COPIES_PER_BLOCK == 6, "vmcnt below");
    asm volatile("s_waitcnt vmcnt(6)\n\ts_barrier" ::: "memory");
}
// Barrier after which every copy issued so far is complete.
__device__ __forceinline__ void barrier_drain() { asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ uint32_t stage_addr(int n) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(LDS_PTR(char, &g_stage[0]))) +
           static_cast<uint32_t>(n % NSTAGE) * STAGE_BYTES;
}

// Prologue: copies of blocks 0 .. NSTAGE-2 in flight, block 0 complete everywhere.
__device__ __forceinline__ void key_prologue(const Ctx& cx, int wave, int lane, int nblk) {
    stage_block(cx, 0, g_stage[0], wave, lane);
    if (nblk > 1) {
        stage_block(cx, 1, g_stage[1], wave, lane);
        barrier_keep_newest();
    } else {
        barrier_drain();
    }
}

// One step of the key loop: read block n's operands, issue the copy of block
// n + NSTAGE - 1 into the stage block n - 1 used, compute block n, and leave block n + 1
// complete for every wave.
template <bool EXACT_MAX>
__device__ __forceinline__ void key_step(const Ctx& cx, const Lane& L, int wave, int lane,
                                         const bf16x8 (&qB)[RW][TW][2], State& s, int n, int nblk) {
    const uint32_t st = stage_addr(n);
    VFrags vf;
    load_v(st, L, vf);
    const bool issue = n + NSTAGE - 1 < nblk;
    if (issue) stage_block(cx, n + NSTAGE - 1, g_stage[(n + NSTAGE - 1) % NSTAGE], wave, lane);
    KCFrags kc;
    load_kc(st, L, kc);
    if constexpr (!EXACT_MAX)
        compute_block_pipe(kc, vf, qB, s);
    else
        compute_block<EXACT_MAX>(kc, vf, qB, s);
    if (issue)
        barrier_keep_newest();
    else
        barrier_drain();
}

// Fast pass: block 0 fixes the reference at its exact maximum, the other blocks reuse it.
// Each loop has a single compute path, so the accumulators stay in place across blocks.
__device__ __forceinline__ void key_loop_fast(const Ctx& cx, const Lane& L, int wave, int lane,
                                              const bf16x8 (&qB)[RW][TW][2], State& s, int nblk) {
    key_prologue(cx, wave, lane, nblk);
    key_step<true>(cx, L, wave, lane, qB, s, 0, nblk);
    for (int n = 1; n < nblk; ++n) key_step<false>(cx, L, wave, lane, qB, s, n, nblk);
}

// Exact pass: the running maximum is refreshed on every block.
__device__ __forceinline__ void key_loop_exact(const Ctx& cx, const Lane& L, int wave, int lane,
                                               const bf16x8 (&qB)[RW][TW][2], State& s, int nblk) {
    key_prologue(cx, wave, lane, nblk);
    for (int n = 0; n < nblk; ++n) key_step<true>(cx, L, wave, lane, qB, s, n, nblk);
}

__global__ void __launch_bounds__(NTHR) bf16_mfma_kernel(Problem p, Strides sd, const float* img, int n_jb, int n_rg,
                                                         int nblk, int total) {
    // XCD-aware remap: XCD x (= hardware id mod 8) walks a contiguous range of logical ids.
    const int w = blockIdx.x;
    const int xcd = w % NXCD, slot = w / NXCD;
    const int base = total / NXCD, extra = total % NXCD;
    const int logical = xcd * base + (xcd < extra ? xcd : extra) + slot;
    // within one (b, h): strips of TILE_RG row groups, each cut into tiles of TILE_RG x
    // TILE_JB (row group, column block) pairs, column block fastest inside a tile; the last
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
    const int row0 = (wave / (QT / TW)) * RW;       // first of this wave's rows in the group
    const int tile0 = (wave % (QT / TW)) * TW;      // first of this wave's query tiles
    const Lane L = lane_layout(lane, row0, tile0);

    Ctx cx;
    {
        int64_t i = i0 + wave;                       // the line this wave stages
        i = i < lines ? i : lines - 1;               // padded lines read a real line (never stored)
        const int64_t row_off = (bh_off + i * sd.line + p.k0 * sd.key) * 2;
        cx.k_row = static_cast<const char*>(p.k) + row_off;
        cx.v_row = static_cast<const char*>(p.v) + row_off;
        cx.img_wg = img + (static_cast<int64_t>(bh) * n_jb + jb) * nblk * IMG_FLOATS;
        cx.key_bytes = sd.key * 2;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            cx.key_local[half] = 16 * half + (lane >> 2);
            cx.part_bytes[half] = kv_chunk(cx.key_local[half], lane & 3) * 16;   // logical part at this slot
        }
        cx.last_key = static_cast<int>(p.nkeys() - 1);
        cx.plan = BlockPlan(p.nkeys(), p.T);
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

    State s;
    s.reset();
    if (tid == 0) g_redo = 0;
    key_loop_fast(cx, L, wave, lane, qB, s, nblk);

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
        s.reset();
        key_loop_exact(cx, L, wave, lane, qB, s, nblk);
    }

    // out = O / l; lanes l and l^32 hold disjoint keys of the same query.  In state mode
    // out receives O itself, with the reference (m_ref / sqrt(D): S carries a factor
    // sqrt(D)) and l; the log-sum-exp is m_ref / sqrt(D) + ln l.
    const bool state = p.st_m != nullptr;
#pragma unroll
    for (int ri = 0; ri < RW; ++ri)
#pragma unroll
        for (int ti = 0; ti < TW; ++ti) {
            const float lt = s.lsum[ri][ti] + __shfl_xor(s.lsum[ri][ti], 32);
            const int64_t i = i0 + row0 + ri, j = j0 + (tile0 + ti) * 32 + L.c;
            if (i < lines && j < p.N) {
                const int64_t qo = bh_off + i * sd.line + j * sd.query;
                float* o = p.out + qo;
                // correctly rounded O / l: a single surviving key returns its v exactly
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    f32x4 x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float acc = s.O[ri][ti][4 * a + e];
                        x[e] = state ? acc : (lt > 0.0f ? acc / lt : 0.0f);
                    }
                    *reinterpret_cast<f32x4*>(o + 8 * a + 4 * L.h2) = x;
                }
                const float mnat = s.mref[ri][ti] * (1.0f / kSqrtD);
                if (L.h2 == 0) {
                    if (state) {
                        p.st_m[qo / D] = lt > 0.0f ? mnat : -INFINITY;
                        p.st_l[qo / D] = lt;
                    }
                    if (p.lse) p.lse[qo / D] = lt > 0.0f ? mnat + logf(lt) : -INFINITY;
                }
            }
        }
}

}  // namespace

size_t bf16_workspace_bytes(const Problem& p) {
    const int64_t n_jb = (p.N + BJ - 1) / BJ;
    const int64_t nblk = BlockPlan(p.nkeys(), p.T).count();
    return static_cast<size_t>(p.B * p.H * n_jb * nblk) * IMG_FLOATS * sizeof(float);
}

int64_t bias_image_blocks(const Problem& p) { return BlockPlan(p.nkeys(), p.T).count(); }

hipError_t launch_bias_image(const Problem& p, float* img, hipStream_t stream) {
    const int64_t n_jb = (p.N + BJ - 1) / BJ;
    const int64_t nblk = BlockPlan(p.nkeys(), p.T).count();
    if (nblk > 0x7FFFFFFF || n_jb > 65535 || p.B * p.H > 65535) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(bias_image_kernel, dim3(static_cast<unsigned>(nblk), static_cast<unsigned>(n_jb),
                                               static_cast<unsigned>(p.B * p.H)),
                       dim3(IMG_THR), 0, stream, p, img, static_cast<int>(n_jb), static_cast<int>(nblk));
    return hipGetLastError();
}

hipError_t launch_bf16_mfma(const Problem& p, void* workspace, hipStream_t stream) {
    const int64_t n_jb = (p.N + BJ - 1) / BJ;
    const int64_t n_rg = ((p.ending ? p.N : p.I) + R - 1) / R;
    const int64_t nblk = BlockPlan(p.nkeys(), p.T).count();
    const Strides sd = strides_of(p);
    const int64_t total = n_jb * n_rg * p.B * p.H;
    // the 32 keys of a block are addressed with 32-bit byte offsets from the block's first key
    if (total > 0x7FFFFFFF || nblk > 0x7FFFFFFF || n_jb > 65535 || p.B * p.H > 65535 ||
        BK * sd.key * 2 > 0x7FFFFFFF)
        return hipErrorInvalidConfiguration;
    float* img = static_cast<float*>(workspace);
    hipLaunchKernelGGL(bias_image_kernel, dim3(static_cast<unsigned>(nblk), static_cast<unsigned>(n_jb),
                                               static_cast<unsigned>(p.B * p.H)),
                       dim3(IMG_THR), 0, stream, p, img, static_cast<int>(n_jb), static_cast<int>(nblk));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bf16_mfma_kernel, dim3(static_cast<unsigned>(total)), dim3(NTHR), 0, stream, p, sd, img,
                       static_cast<int>(n_jb), static_cast<int>(n_rg), static_cast<int>(nblk), static_cast<int>(total));
    return hipGetLastError();
}

}  // namespace tri_attn
