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
//      The row sum is taken per lane with v_dot2_f32_bf16 on the rounded p.
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
// group, column block) with the column block fastest: a row group's K/V stream and the
// bias strips stay hot in that XCD's L2.
#include "launch.h"

#include <cmath>

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
__host__ __device__ constexpr int bias_chunk(int j, int part) { return part ^ (j & 7); }

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
    const KeyBlock kbk = BlockPlan(p.N, p.T).block(n);
    const uint16_t* bg = static_cast<const uint16_t*>(p.bias);
    float* dst = img + ((static_cast<int64_t>(bh) * n_jb + jb) * nblk + n) * IMG_FLOATS;
    const int kk = threadIdx.x % BK;
    const bool key_ok = kk < kbk.nk;
    const float mk = (p.mask && key_ok) ? p.mask[b * p.N + kbk.kb + kk] : 0.0f;
#pragma unroll
    for (int s = 0; s < IMG_FLOATS / IMG_THR; ++s) {
        const int jj = (threadIdx.x + s * IMG_THR) / BK;
        const int64_t j = static_cast<int64_t>(jb) * BJ + jj;
        float val = -INFINITY;
        if (key_ok) {
            const float bv = j < p.N ? __uint_as_float(static_cast<uint32_t>(bg[(bh * p.N + j) * p.N + kbk.kb + kk]) << 16)
                                     : 0.0f;
            val = (bv + mk) * kSqrtD;
        }
        dst[jj * BK + bias_chunk(jj, kk / 4) * 4 + kk % 4] = val;
    }
}

// ---------------------------------------------------------------------------------------
// 2. attention
// ---------------------------------------------------------------------------------------
struct Ctx {
    const char* k_row;      // K of this wave's staged row: &k[b, i, 0, h, 0]
    const char* v_row;
    const float* img_wg;    // this workgroup's bias tiles, nblk consecutive 128 x 32 tiles
    int row_bytes;          // bytes between consecutive keys (H * D * 2)
    int key_local[2];       // key of this lane's 16-byte slot in the two 1 KB pieces
    int part_bytes[2];      // byte offset of the slot's logical 16-byte part inside the key
    int last_key;           // N - 1
    BlockPlan plan;
};

// Wave w copies K and V of staged row w (two 1 KB pieces each) and two 1 KB pieces of the
// bias tile; lane l of a piece carries 16 bytes.
__device__ __forceinline__ void stage_block(const Ctx& cx, int n, Stage& st, int wave, int lane) {
    const KeyBlock kbk = cx.plan.block(n);
    const int kb = static_cast<int>(kbk.kb);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const int key = min(kb + cx.key_local[half], cx.last_key);   // padded keys read a real key (bias -inf)
        const int off = key * cx.row_bytes + cx.part_bytes[half];
        __builtin_amdgcn_global_load_lds(GLOBAL_PTR(void, cx.k_row + off), LDS_PTR(void, &st.k[wave][16 * half][0]), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(GLOBAL_PTR(void, cx.v_row + off), LDS_PTR(void, &st.v[wave][16 * half][0]), 16, 0, 0);
    }
    const float* src = cx.img_wg + static_cast<int64_t>(n) * IMG_FLOATS + lane * 4;
    float* flat = &st.bias[0][0];
#pragma unroll
    for (int piece = 0; piece < 2; ++piece) {
        const int base = (2 * wave + piece) * 256;              // 256 floats = 1 KB
        __builtin_amdgcn_global_load_lds(GLOBAL_PTR(void, src + base), LDS_PTR(void, flat + base), 16, 0, 0);
    }
}

struct Lane {
    int c, h2;
    int k_off[2];          // byte offsets inside one staged row of K: A operand of S^T = K Q^T
    int v_off[2][2];       // byte offsets inside one staged row of V: ds_read_b64_tr_b16 sources
    int b_off[4];          // byte offsets inside a 32-row slab of the bias tile
};

__device__ __forceinline__ Lane lane_layout(int lane) {
    Lane L;
    L.c = lane & 31;
    L.h2 = lane >> 5;
#pragma unroll
    for (int m = 0; m < 2; ++m) L.k_off[m] = L.c * 64 + kv_chunk(L.c, 2 * m + L.h2) * 16;
    // transpose read: lane i of a 16-lane group reads keys kbase + i/4, d = dbase + 4*(i%4) .. +3
    // and receives d = dbase + i for keys kbase .. kbase + 3
    const int i = lane & 15, dbase = 16 * ((lane >> 4) & 1);
    const int d0 = dbase + 4 * (i & 3);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int key = 16 * m + 8 * sub + 4 * L.h2 + (i >> 2);
            L.v_off[m][sub] = key * 64 + kv_chunk(key, d0 >> 3) * 16 + (d0 & 7) * 2;
        }
#pragma unroll
    for (int a = 0; a < 4; ++a) L.b_off[a] = L.c * 128 + bias_chunk(L.c, 2 * a + L.h2) * 16;
    return L;
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

// V^T operands of the wave's rows.  ds_read_b64_tr_b16 carries no alias information, so
// these reads are issued before the next block's copy (a read after it would wait for it).
struct VFrags {
    bf16x8 vA[RW][2];
};

__device__ __forceinline__ void load_v(const Stage& st, const Lane& L, int row0, VFrags& f) {
    const char* vbase = reinterpret_cast<const char*>(&st.v[0][0][0]);
#pragma unroll
    for (int ri = 0; ri < RW; ++ri) {
        const int rowb = (row0 + ri) * BK * D * 2;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, vbase + rowb + L.v_off[m][0]));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, vbase + rowb + L.v_off[m][1]));
            f.vA[ri][m] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    }
}

template <bool EXACT_MAX>
__device__ __forceinline__ void compute_block(const Stage& st, const Lane& L, int row0, int tile0, const VFrags& vf,
                                              const bf16x8 (&qB)[RW][TW][2], State& s) {
    const char* kbase = reinterpret_cast<const char*>(&st.k[0][0][0]);
    const char* bbase = reinterpret_cast<const char*>(&st.bias[0][0]);
    bf16x8 kA[RW][2];
#pragma unroll
    for (int ri = 0; ri < RW; ++ri)
#pragma unroll
        for (int m = 0; m < 2; ++m)
            kA[ri][m] = *reinterpret_cast<const bf16x8*>(kbase + (row0 + ri) * BK * D * 2 + L.k_off[m]);
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
    for (int ti = 0; ti < TW; ++ti) {
        const char* brow = bbase + (tile0 + ti) * 32 * BK * 4;
        f32x16 C;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(brow + L.b_off[a]);
            C[4 * a + 0] = x[0];
            C[4 * a + 1] = x[1];
            C[4 * a + 2] = x[2];
            C[4 * a + 3] = x[3];
        }
#pragma unroll
        for (int ri = 0; ri < RW; ++ri) {
            f32x16 S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kA[ri][0], qB[ri][ti][0], C, 0, 0, 0);
            S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kA[ri][1], qB[ri][ti][1], S, 0, 0, 0);
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

__shared__ Stage g_stage0;
__shared__ Stage g_stage1;
__shared__ int g_redo;

// One pass over every key block; the first block (all blocks when `exact`) refreshes the
// reference maximum.
__device__ __forceinline__ void key_loop(const Ctx& cx, const Lane& L, int wave, int lane, int row0, int tile0,
                                         const bf16x8 (&qB)[RW][TW][2], State& s, int nblk, bool exact) {
    stage_block(cx, 0, g_stage0, wave, lane);
    __syncthreads();
    for (int n = 0; n < nblk; ++n) {
        const bool odd = n & 1;
        // read this block's operands before the next block's copy is issued, so that no LDS
        // read has to wait for the copy in flight
        const Stage& st = odd ? g_stage1 : g_stage0;
        VFrags vf;
        load_v(st, L, row0, vf);
        if (n + 1 < nblk) stage_block(cx, n + 1, odd ? g_stage0 : g_stage1, wave, lane);
        if (exact || n == 0)
            compute_block<true>(st, L, row0, tile0, vf, qB, s);
        else
            compute_block<false>(st, L, row0, tile0, vf, qB, s);
        __syncthreads();
    }
}

__global__ void __launch_bounds__(NTHR) bf16_mfma_kernel(Problem p, const float* img, int n_jb, int n_rg, int nblk,
                                                         int total) {
    // XCD-aware remap: XCD x (= hardware id mod 8) walks a contiguous range of logical ids.
    const int w = blockIdx.x;
    const int xcd = w % NXCD, slot = w / NXCD;
    const int base = total / NXCD, extra = total % NXCD;
    const int logical = xcd * base + (xcd < extra ? xcd : extra) + slot;
    const int jb = logical % n_jb;
    const int rg = (logical / n_jb) % n_rg;
    const int bh = logical / (n_jb * n_rg);
    const int64_t b = bh / p.H, h = bh % p.H;
    const int64_t i0 = static_cast<int64_t>(rg) * R, j0 = static_cast<int64_t>(jb) * BJ;

    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64;
    const Lane L = lane_layout(lane);
    const int row0 = (wave / (QT / TW)) * RW;       // first of this wave's rows in the group
    const int tile0 = (wave % (QT / TW)) * TW;      // first of this wave's query tiles

    Ctx cx;
    {
        int64_t i = i0 + wave;                       // the row this wave stages
        i = i < p.I ? i : p.I - 1;                   // padded rows read a real row (never stored)
        const int64_t row_off = ((b * p.I + i) * p.N * p.H + h) * D * 2;
        cx.k_row = static_cast<const char*>(p.k) + row_off;
        cx.v_row = static_cast<const char*>(p.v) + row_off;
        cx.img_wg = img + (static_cast<int64_t>(bh) * n_jb + jb) * nblk * IMG_FLOATS;
        cx.row_bytes = static_cast<int>(p.H * D * 2);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            cx.key_local[half] = 16 * half + (lane >> 2);
            cx.part_bytes[half] = kv_chunk(cx.key_local[half], lane & 3) * 16;   // logical part at this slot
        }
        cx.last_key = static_cast<int>(p.N - 1);
        cx.plan = BlockPlan(p.N, p.T);
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
                if (i < p.I && j < p.N)
                    z = *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(p.q) +
                                                         (((b * p.I + i) * p.N + j) * p.H + h) * D + 16 * m + 8 * L.h2);
                qB[ri][ti][m] = z;
            }
        }

    State s;
    s.reset();
    if (tid == 0) g_redo = 0;
    key_loop(cx, L, wave, lane, row0, tile0, qB, s, nblk, false);

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
        key_loop(cx, L, wave, lane, row0, tile0, qB, s, nblk, true);
    }

    // out = O / l; lanes l and l^32 hold disjoint keys of the same query.
#pragma unroll
    for (int ri = 0; ri < RW; ++ri)
#pragma unroll
        for (int ti = 0; ti < TW; ++ti) {
            const float lt = s.lsum[ri][ti] + __shfl_xor(s.lsum[ri][ti], 32);
            const int64_t i = i0 + row0 + ri, j = j0 + (tile0 + ti) * 32 + L.c;
            if (i < p.I && j < p.N) {
                float* o = p.out + (((b * p.I + i) * p.N + j) * p.H + h) * D;
                // correctly rounded O / l: a single surviving key returns its v exactly
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    f32x4 x;
                    x[0] = lt > 0.0f ? s.O[ri][ti][4 * a + 0] / lt : 0.0f;
                    x[1] = lt > 0.0f ? s.O[ri][ti][4 * a + 1] / lt : 0.0f;
                    x[2] = lt > 0.0f ? s.O[ri][ti][4 * a + 2] / lt : 0.0f;
                    x[3] = lt > 0.0f ? s.O[ri][ti][4 * a + 3] / lt : 0.0f;
                    *reinterpret_cast<f32x4*>(o + 8 * a + 4 * L.h2) = x;
                }
            }
        }
}

}  // namespace

size_t bf16_workspace_bytes(const Problem& p) {
    const int64_t n_jb = (p.N + BJ - 1) / BJ;
    const int64_t nblk = BlockPlan(p.N, p.T).count();
    return static_cast<size_t>(p.B * p.H * n_jb * nblk) * IMG_FLOATS * sizeof(float);
}

hipError_t launch_bf16_mfma(const Problem& p, void* workspace, hipStream_t stream) {
    const int64_t n_jb = (p.N + BJ - 1) / BJ;
    const int64_t n_rg = (p.I + R - 1) / R;
    const int64_t nblk = BlockPlan(p.N, p.T).count();
    const int64_t total = n_jb * n_rg * p.B * p.H;
    // one (b, i) row of K or V is addressed with 32-bit byte offsets
    if (total > 0x7FFFFFFF || nblk > 0x7FFFFFFF || n_jb > 65535 || p.B * p.H > 65535 ||
        p.N * p.H * D * 2 > 0x7FFFFFFF)
        return hipErrorInvalidConfiguration;
    float* img = static_cast<float*>(workspace);
    hipLaunchKernelGGL(bias_image_kernel, dim3(static_cast<unsigned>(nblk), static_cast<unsigned>(n_jb),
                                               static_cast<unsigned>(p.B * p.H)),
                       dim3(IMG_THR), 0, stream, p, img, static_cast<int>(n_jb), static_cast<int>(nblk));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bf16_mfma_kernel, dim3(static_cast<unsigned>(total)), dim3(NTHR), 0, stream, p, img,
                       static_cast<int>(n_jb), static_cast<int>(n_rg), static_cast<int>(nblk), static_cast<int>(total));
    return hipGetLastError();
}

}  // namespace tri_attn
