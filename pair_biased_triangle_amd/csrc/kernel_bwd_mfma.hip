// Backward of starting-node triangle attention on gfx950 matrix cores: bf16 inputs, D = 32
// (the gradients of the definition; see kernel_backward.hip for the formulas and the
// plain fp32 version used for every other case).
//
// Four kernels, each owning the sums it produces (no atomics, deterministic):
//   bwd_prep_kernel   dout -> bf16 copy (the operand of the dP and dV products) and
//                     delta = dout . out per query, in fp32.
//   bwd_dq_mfma       one wave per (b, i, h, 32 queries), looping over 32-key blocks in
//                     the forward's orientation (lane = query):
//                       S^T  = K Q^T + C          C = the forward's bias image tile
//                       dP^T = V dO^T
//                       dS^T = P^T (dP^T - delta),  P^T = exp(S^T - lse)
//                       dQ^T += K^T dS^T          K^T by an LDS transposed read
//   bwd_dkdv_mfma     one wave per (b, i, h, 32 keys), looping over 32-query blocks in the
//                     other orientation (lane = key), so that P and dS come out of the
//                     accumulator layout as the B operands of
//                       dV^T += dO^T P,  dK^T += Q^T dS     (dO^T, Q^T by transposed reads)
//   bwd_dbias_mfma    one wave per (b, h, 32 queries, 32 keys), looping over every row i:
//                       dbias^T += dS^T of row i (the bias is shared by all rows)
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

constexpr int D = 32;
constexpr int NWAVE = 4;
constexpr int NTHR = 64 * NWAVE;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSqrtD = 5.656854249492381f;
constexpr float kScale = kLog2e / kSqrtD;        // S units (q.k + sqrt(D) bias) -> log2 units
constexpr float kInvSqrtD = 0.17677669529663687f;
constexpr int TILE_BYTES = 32 * D * 2;           // one wave's 32 x 32 bf16 tile in LDS
#ifndef TRI_ATTN_DBIAS_AHEAD
#define TRI_ATTN_DBIAS_AHEAD 3
#endif

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

__device__ __forceinline__ float bf16_to_f32(uint16_t u) { return __uint_as_float(static_cast<uint32_t>(u) << 16); }

// 16-byte chunk `part` (d = 8*part .. +7) of tile row `row` sits at chunk kv_chunk(row, part)
__host__ __device__ constexpr int kv_chunk(int row, int part) { return part ^ ((row >> 1) & 3); }

// Per-lane LDS offsets inside one tile: the two row-major chunks this lane writes (row
// l%32, d-halves m = 0, 1) and the sources of the transposed reads.  A transposed read
// gives lane l row d = l%32 of the tile's transpose at tile rows {4h2 + b, 8 + 4h2 + b}
// + 16m (b = 0..3, h2 = l/32): the row order of the accumulator layout above.
struct TileLane {
    uint32_t wr[2];
    uint32_t tr[2][2];
};

__device__ __forceinline__ TileLane tile_lane(int lane) {
    TileLane L;
    const int c = lane & 31, h2 = lane >> 5;
#pragma unroll
    for (int m = 0; m < 2; ++m) L.wr[m] = c * 64 + kv_chunk(c, 2 * m + h2) * 16;
    const int i = lane & 15, d0 = 16 * ((lane >> 4) & 1) + 4 * (i & 3);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int row = 16 * m + 8 * sub + 4 * h2 + (i >> 2);
            L.tr[m][sub] = row * 64 + kv_chunk(row, d0 >> 3) * 16 + (d0 & 7) * 2;
        }
    return L;
}

// Write a tile held as row fragments (lane row l%32, d-halves w0, w1) to this wave's LDS
// tile at `base` and read back its transpose as A operands t0, t1.  The writes and reads
// wait for themselves, so the tile may be rewritten right after.
__device__ __forceinline__ void transpose_tile(uint32_t base, const TileLane& L, bf16x8 w0, bf16x8 w1, bf16x8& t0,
                                               bf16x8& t1) {
    u32x2 r0, r1, r2, r3;
    asm volatile(
        "ds_write_b128 %4, %6\n\t"
        "ds_write_b128 %5, %7\n\t"
        "s_waitcnt lgkmcnt(0)\n\t"
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %9\n\t"
        "ds_read_b64_tr_b16 %2, %10\n\t"
        "ds_read_b64_tr_b16 %3, %11\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
        : "v"(base + L.wr[0]), "v"(base + L.wr[1]), "v"(__builtin_bit_cast(u32x4, w0)),
          "v"(__builtin_bit_cast(u32x4, w1)), "v"(base + L.tr[0][0]), "v"(base + L.tr[0][1]),
          "v"(base + L.tr[1][0]), "v"(base + L.tr[1][1])
        : "memory");
    t0 = __builtin_bit_cast(bf16x8, u32x4{r0[0], r0[1], r1[0], r1[1]});
    t1 = __builtin_bit_cast(bf16x8, u32x4{r2[0], r2[1], r3[0], r3[1]});
}

__device__ __forceinline__ void to_bf16(const f32x16& x, bf16x8& lo, bf16x8& hi) {
    lo = __builtin_convertvector(__builtin_shufflevector(x, x, 0, 1, 2, 3, 4, 5, 6, 7), bf16x8);
    hi = __builtin_convertvector(__builtin_shufflevector(x, x, 8, 9, 10, 11, 12, 13, 14, 15), bf16x8);
}

// -inf for a query without any finite score (its p is 0 everywhere), else -lse in log2 units
__device__ __forceinline__ float neg_lse2(float lse) { return lse == -INFINITY ? -INFINITY : -lse * kLog2e; }

// ---------------------------------------------------------------------------------------
// One thread per (b, i, h, j) with j padded to NP: dout of query (b, i, j, h) rounded to
// bf16, delta = dout . out, and lse / delta also written transposed, [b, i, h, j], so that
// a lane can read 4 consecutive queries with one 16-byte load; padded j get lse = -inf
// (no probability) and delta = 0.
__global__ void __launch_bounds__(256) bwd_prep_kernel(BwdProblem p, __bf16* g16, float* delta, float* lseT,
                                                       float* deltaT, int64_t NP) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t total = p.B * p.I * p.H * NP;
    if (t >= total) return;
    const int64_t j = t % NP, lh = t / NP, h = lh % p.H, line = lh / p.H;   // line = b * I + i
    if (j >= p.N) {
        lseT[t] = -INFINITY;
        deltaT[t] = 0.0f;
        return;
    }
    const int64_t q = (line * p.N + j) * p.H + h;
    const f32x4* g = reinterpret_cast<const f32x4*>(p.dout + q * D);
    const f32x4* o = reinterpret_cast<const f32x4*>(p.out + q * D);
    float dl = 0.0f;
#pragma unroll
    for (int a = 0; a < D / 8; ++a) {
        const f32x4 g0 = g[2 * a], g1 = g[2 * a + 1], o0 = o[2 * a], o1 = o[2 * a + 1];
#pragma unroll
        for (int e = 0; e < 4; ++e) dl = fmaf(g0[e], o0[e], fmaf(g1[e], o1[e], dl));
        const f32x8 gg = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
        *reinterpret_cast<bf16x8*>(g16 + q * D + 8 * a) = __builtin_convertvector(gg, bf16x8);
    }
    delta[q] = dl;
    deltaT[t] = dl;
    lseT[t] = p.lse[q];
}

// ---------------------------------------------------------------------------------------
// imgT: the bias image of the transposed bias without the mask (built in the ending
// orientation), so that tile (key block of IMG_BJ, query block of IMG_BK) row kk holds
// bias[b, h, q, key] * sqrt(D) for 32 consecutive queries q (-inf past the last query):
// the accumulator input of S for a lane that owns a key.  Dropped keys are zeroed at the end.
__global__ void __launch_bounds__(NTHR, 2) bwd_dkdv_mfma(BwdProblem p, const float* imgT, const __bf16* g16,
                                                         const float* lseT, const float* deltaT, int n_kb,
                                                         int nqblk, int64_t NP) {
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 31, h2 = lane >> 5;
    const int64_t N = p.N, H = p.H, HD = H * D;
    const int64_t bh = blockIdx.z, b = bh / H, h = bh % H, i = blockIdx.y;
    const int kb = blockIdx.x;                            // block of IMG_BJ keys
    const int kk = wave * 32 + c;                         // key inside the block
    const int64_t key = static_cast<int64_t>(kb) * IMG_BJ + kk;
    const bool kok = key < N;
    const int64_t row = (b * p.I + i) * N;
    const __bf16* q = static_cast<const __bf16*>(p.q);
    const __bf16* k = static_cast<const __bf16*>(p.k);
    const __bf16* v = static_cast<const __bf16*>(p.v);
    const int64_t ko = (row + key) * HD + h * D;
    const float* lse_l = lseT + ((b * p.I + i) * H + h) * NP + 4 * h2;
    const float* dl_l = deltaT + ((b * p.I + i) * H + h) * NP + 4 * h2;
    const float* img_row = imgT + (bh * n_kb + kb) * static_cast<int64_t>(nqblk) * IMG_BJ * IMG_BK + kk * IMG_BK;

    bf16x8 kB[2], vB[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        kB[m] = frag(k, ko + 16 * m + 8 * h2, kok);
        vB[m] = frag(v, ko + 16 * m + 8 * h2, kok);
    }
    const bool dropped = !kok || (p.mask && p.mask[b * N + (kok ? key : 0)] == -INFINITY);
    const TileLane L = tile_lane(lane);
    __shared__ __attribute__((aligned(16))) char lds[NWAVE * 2 * TILE_BYTES];
    const uint32_t tile_g = LDS_ADDR(lds) + wave * 2 * TILE_BYTES, tile_q = tile_g + TILE_BYTES;

    // operands of query block n: Q, dO rows (lane = query), and for this lane's key the
    // accumulator input, lse and delta of the 16 query rows 8a + 4h2 + e of its registers
    struct Blk {
        bf16x8 qA[2], gA[2];
        f32x4 c[4], nl[4], dl[4];
    };
    auto fetch = [&](int n, Blk& X) {
        const int64_t qb = static_cast<int64_t>(n) * IMG_BK;
        const int64_t jq = qb + c;
        const bool jok = jq < N;
        const int64_t qo = (row + jq) * HD + h * D;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            X.qA[m] = frag(q, qo + 16 * m + 8 * h2, jok);
            X.gA[m] = frag(g16, qo + 16 * m + 8 * h2, jok);
        }
        const float* t = img_row + static_cast<int64_t>(n) * IMG_BJ * IMG_BK;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            X.c[a] = *reinterpret_cast<const f32x4*>(t + img_chunk(kk, 2 * a + h2) * 4);
            X.nl[a] = *reinterpret_cast<const f32x4*>(lse_l + qb + 8 * a);
            X.dl[a] = *reinterpret_cast<const f32x4*>(dl_l + qb + 8 * a);
        }
    };
    f32x16 dK = {}, dV = {};
    Blk cur, nxt;
    fetch(0, cur);
    for (int n = 0; n < nqblk; ++n) {
        if (n + 1 < nqblk) fetch(n + 1, nxt);             // next block's loads fly during this block
        const bf16x8 (&qA)[2] = cur.qA;
        const bf16x8 (&gA)[2] = cur.gA;
        f32x16 C, nl, dl;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                C[4 * a + e] = cur.c[a][e];
                nl[4 * a + e] = cur.nl[a][e];
                dl[4 * a + e] = cur.dl[a][e];
            }
        f32x16 S = mfma(qA[0], kB[0], C);
        S = mfma(qA[1], kB[1], S);
        f32x16 dP = mfma(gA[0], vB[0], f32x16{});
        dP = mfma(gA[1], vB[1], dP);
        // P overwrites S and dS overwrites dP
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            S[r] = __builtin_amdgcn_exp2f(fmaf(S[r], kScale, neg_lse2(nl[r])));
            dP[r] = S[r] * (dP[r] - dl[r]);
        }
        bf16x8 p0, p1, s0, s1, gT0, gT1, qT0, qT1;
        to_bf16(S, p0, p1);
        to_bf16(dP, s0, s1);
        transpose_tile(tile_g, L, gA[0], gA[1], gT0, gT1);
        transpose_tile(tile_q, L, qA[0], qA[1], qT0, qT1);
        dV = mfma(gT0, p0, dV);
        dV = mfma(gT1, p1, dV);
        dK = mfma(qT0, s0, dK);
        dK = mfma(qT1, s1, dK);
        cur = nxt;
    }
    if (kok) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            f32x4 xk, xv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xk[e] = dropped ? 0.0f : dK[4 * a + e] * kInvSqrtD;
                xv[e] = dropped ? 0.0f : dV[4 * a + e];
            }
            *reinterpret_cast<f32x4*>(p.dk + ko + 8 * a + 4 * h2) = xk;
            *reinterpret_cast<f32x4*>(p.dv + ko + 8 * a + 4 * h2) = xv;
        }
    }
}

#define GPTR(p) ((const __attribute__((address_space(1))) void*)(p))
#define LPTR(p) ((__attribute__((address_space(3))) void*)(p))
__device__ __forceinline__ void db_barrier_drain() { asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---------------------------------------------------------------------------------------
// dq, in the forward's shape: a workgroup of 8 waves owns DQ_R = 4 lines (rows i) x 128
// query columns of one (b, h) and streams 32-key blocks through a ring of LDS stages (K,
// V of its lines and the 128 x 32 tile of the fp32 bias image, copied by
// global_load_lds).  Wave w owns line w / 2 and query tiles 2 (w % 2), +1; Q and dO of its
// queries stay in registers.  Per unit and block:
//   S^T = K Q^T + C,  dP^T = V dO^T,  dS^T = P^T (dP^T - delta),  dQ^T += K^T dS^T
// with K^T read transposed from the staged [key][d] tile (ds_read_b64_tr_b16).
constexpr int DQ_R = 4;
constexpr int DQ_WAVES = 8;
constexpr int DQ_THR = 64 * DQ_WAVES;
#ifndef TRI_ATTN_DQ_STAGES
#define TRI_ATTN_DQ_STAGES 4
#endif
constexpr int DQ_STAGES = TRI_ATTN_DQ_STAGES;
constexpr int DQ_TILE_RG = 8;               // line groups x column blocks one XCD works on together
constexpr int DQ_TILE_JB = 4;
struct DqStage {
    __bf16 k[DQ_R][32][D];     // 64-byte rows, 16-byte chunks swizzled by kv_chunk()
    __bf16 v[DQ_R][32][D];
    float bias[IMG_BJ][IMG_BK];   // the image tile as stored: 128-byte rows, chunks img_chunk()
};
constexpr int DQ_STAGE_BYTES = static_cast<int>(sizeof(DqStage));
constexpr int DQ_K_OFF = static_cast<int>(offsetof(DqStage, k));
constexpr int DQ_V_OFF = static_cast<int>(offsetof(DqStage, v));
constexpr int DQ_B_OFF = static_cast<int>(offsetof(DqStage, bias));
constexpr int DQ_LINE_BYTES = 32 * D * 2;
constexpr int DQ_CTILE_BYTES = 32 * IMG_BK * 4;
static_assert(DQ_LINE_BYTES == 2048 && DQ_CTILE_BYTES == 4096 && DQ_V_OFF - DQ_K_OFF == 8192, "offsets below");
static_assert(DQ_R * 2 * 2 == 2 * DQ_WAVES && IMG_BJ * IMG_BK * 4 == 2 * DQ_WAVES * 1024, "two K/V, two bias pieces per wave");
__shared__ DqStage g_dq[DQ_STAGES];

struct DqCtx {
    const char* kv_row[2];     // K or V of the staged line at key 0
    uint32_t kv_lds[2];
    int key_local[2];
    int part_bytes[2];
    const float* img_wg;       // this workgroup's image tiles, nblk consecutive 128 x 32 tiles
    int64_t key_bytes;
    int last_key;
};

__device__ __forceinline__ void dq_stage(const DqCtx& cx, int n, int wave, int lane) {
    char* lds = reinterpret_cast<char*>(&g_dq[n % DQ_STAGES]);
    const int kb = 32 * n;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int rel = min(kb + cx.key_local[t], cx.last_key) - kb;   // padded keys read a real key
        const char* src = cx.kv_row[t] + static_cast<int64_t>(kb) * cx.key_bytes + rel * cx.key_bytes + cx.part_bytes[t];
        __builtin_amdgcn_global_load_lds(GPTR(src), LPTR(lds + cx.kv_lds[t]), 16, 0, 0);
    }
    const char* src = reinterpret_cast<const char*>(cx.img_wg + static_cast<int64_t>(n) * IMG_BJ * IMG_BK) + lane * 16;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int base = (2 * wave + t) * 1024;
        __builtin_amdgcn_global_load_lds(GPTR(src + base), LPTR(lds + DQ_B_OFF + base), 16, 0, 0);
    }
}

__device__ __forceinline__ void dq_barrier_keep() {
    static_assert(DQ_STAGES == 3 || DQ_STAGES == 4, "three or four stages");
    if constexpr (DQ_STAGES == 3) asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
    if constexpr (DQ_STAGES == 4) asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
}

__global__ void __launch_bounds__(DQ_THR) bwd_dq_lds(BwdProblem p, const float* img, const __bf16* g16,
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

    DqCtx cx;
    {
        cx.key_bytes = HD * 2;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            // piece 2 w + t: line w / 2, K (w even) or V (w odd), keys 16 t .. +15
            const int line = wave >> 1, kv = wave & 1;
            int64_t i = i0 + line;
            i = i < I ? i : I - 1;                       // padded lines read a real line (never stored)
            cx.kv_row[t] = reinterpret_cast<const char*>(static_cast<const __bf16*>(kv ? p.v : p.k) +
                                                         ((b * I + i) * N) * HD + h * D);
            cx.kv_lds[t] = (kv ? DQ_V_OFF : DQ_K_OFF) + line * DQ_LINE_BYTES + t * 1024;
            cx.key_local[t] = 16 * t + (lane >> 2);
            cx.part_bytes[t] = kv_chunk(cx.key_local[t], lane & 3) * 16;
        }
        cx.img_wg = img + (static_cast<int64_t>(bh) * n_jb + jb) * nblk * static_cast<int64_t>(IMG_BJ * IMG_BK);
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
            gB[u][m] = frag(g16, qo + 16 * m + 8 * h2, ok);
        }
        const int64_t qi = ((b * I + i) * N + j) * H + h;
        nb[u] = ok ? neg_lse2(p.lse[qi]) : -INFINITY;
        dl[u] = ok ? delta[qi] : 0.0f;
    }
    // LDS byte offsets (stage 0) of this lane's reads: K and V rows (A of S and dP), the
    // transposed K reads (A of dQ), the bias chunks of its first tile (second tile +4096)
    uint32_t ak[2], at[4], ac[4];
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
    for (int a = 0; a < 4; ++a) ac[a] = DQ_B_OFF + t0 * DQ_CTILE_BYTES + c * 128 + img_chunk(c, 2 * a + h2) * 16;
    const uint32_t st0 = LDS_ADDR(&g_dq[0]);

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
        u32x4 kk[2], vv[2], cc[8];
        u32x2 tt[4];
        asm volatile(
            "ds_read_b128 %0, %16\n\t"
            "ds_read_b128 %1, %17\n\t"
            "ds_read_b128 %2, %16 offset:8192\n\t"
            "ds_read_b128 %3, %17 offset:8192\n\t"
            "ds_read_b64_tr_b16 %4, %18\n\t"
            "ds_read_b64_tr_b16 %5, %19\n\t"
            "ds_read_b64_tr_b16 %6, %20\n\t"
            "ds_read_b64_tr_b16 %7, %21\n\t"
            "ds_read_b128 %8, %22\n\t"
            "ds_read_b128 %9, %23\n\t"
            "ds_read_b128 %10, %24\n\t"
            "ds_read_b128 %11, %25\n\t"
            "ds_read_b128 %12, %22 offset:4096\n\t"
            "ds_read_b128 %13, %23 offset:4096\n\t"
            "ds_read_b128 %14, %24 offset:4096\n\t"
            "ds_read_b128 %15, %25 offset:4096\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(kk[0]), "=&v"(kk[1]), "=&v"(vv[0]), "=&v"(vv[1]), "=&v"(tt[0]), "=&v"(tt[1]), "=&v"(tt[2]),
              "=&v"(tt[3]), "=&v"(cc[0]), "=&v"(cc[1]), "=&v"(cc[2]), "=&v"(cc[3]), "=&v"(cc[4]), "=&v"(cc[5]),
              "=&v"(cc[6]), "=&v"(cc[7])
            : "v"(st + ak[0]), "v"(st + ak[1]), "v"(st + at[0]), "v"(st + at[1]), "v"(st + at[2]), "v"(st + at[3]),
              "v"(st + ac[0]), "v"(st + ac[1]), "v"(st + ac[2]), "v"(st + ac[3]));
        bf16x8 kT[2];
#pragma unroll
        for (int m = 0; m < 2; ++m)
            kT[m] = __builtin_bit_cast(bf16x8, u32x4{tt[2 * m][0], tt[2 * m][1], tt[2 * m + 1][0], tt[2 * m + 1][1]});
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            f32x16 C;
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int e = 0; e < 4; ++e) C[4 * a + e] = __uint_as_float(cc[4 * u + a][e]);
            f32x16 S = mfma(__builtin_bit_cast(bf16x8, kk[0]), qB[u][0], C);
            S = mfma(__builtin_bit_cast(bf16x8, kk[1]), qB[u][1], S);
            f32x16 dP = mfma(__builtin_bit_cast(bf16x8, vv[0]), gB[u][0], f32x16{});
            dP = mfma(__builtin_bit_cast(bf16x8, vv[1]), gB[u][1], dP);
            f32x16 dS;
#pragma unroll
            for (int r = 0; r < 16; ++r) dS[r] = __builtin_amdgcn_exp2f(fmaf(S[r], kScale, nb[u])) * (dP[r] - dl[u]);
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
// dbias[b, h, j, k] = sum over the rows i held of dS[i, j, k].  A workgroup of 8 waves owns
// DB_Q = 128 queries x DB_K = 128 keys of one (b, h) and streams the rows i through a ring
// of LDS stages: per row the waves copy Q, dO (its queries), K, V (its keys), lse and delta
// straight from global memory into a stage (global_load_lds_dwordx4), and wave w computes
// queries 32 (w % 4) .. +31 against keys 64 (w / 4) .. +63 (two 32 x 32 units) from LDS:
//   S^T = K Q^T + C,  dP^T = V dO^T,  acc += P^T (dP^T - delta)
// The bias tile C stays in registers for the whole loop.  Every sum over i runs in one
// lane in row order: deterministic.
constexpr int DB_Q = 128;
constexpr int DB_K = 128;
constexpr int DB_WAVES = 8;
constexpr int DB_THR = 64 * DB_WAVES;
#ifndef TRI_ATTN_DB_STAGES
#define TRI_ATTN_DB_STAGES 4
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
constexpr int NP_ALIGN = 128;                   // lse / delta rows padded to whole query tiles
static_assert(DB_Q % NP_ALIGN == 0 || NP_ALIGN % DB_Q == 0, "a query tile never crosses the padding");

struct DbStage {
    __bf16 q[DB_Q][D];     // 64-byte rows, 16-byte chunks swizzled by kv_chunk()
    __bf16 g[DB_Q][D];     // dO rounded to bf16
    __bf16 k[DB_K][D];
    __bf16 v[DB_K][D];
    float lse[DB_Q];
    float dl[DB_Q];
};
constexpr int DB_STAGE_BYTES = static_cast<int>(sizeof(DbStage));
constexpr int DB_Q_OFF = static_cast<int>(offsetof(DbStage, q));
constexpr int DB_G_OFF = static_cast<int>(offsetof(DbStage, g));
constexpr int DB_K_OFF = static_cast<int>(offsetof(DbStage, k));
constexpr int DB_V_OFF = static_cast<int>(offsetof(DbStage, v));
constexpr int DB_L_OFF = static_cast<int>(offsetof(DbStage, lse));
// per wave and row: 4 pieces of 1 KB (16 rows of Q, dO, K or V) and 128 bytes of lse / delta
constexpr int DB_COPIES = 5;
static_assert(4 * DB_WAVES * 1024 == 4 * DB_Q * D * 2 && DB_Q == DB_K, "pieces of the four tensors");
static_assert(DB_WAVES * 128 == 2 * DB_Q * 4, "lse / delta pieces");
__shared__ DbStage g_db[DB_STAGES];


struct DbCtx {
    const char* src[4];        // this wave's four pieces: row base of (b, i = 0, pos, h), part applied
    uint32_t dst[4];           // byte offset of each piece inside a stage
    int64_t row_step;          // bytes between rows i of one tensor
    const char* ls_src;        // lse / delta piece of row 0 (lanes 0 .. 7), or null
    int64_t ls_step;           // bytes between rows i of lseT
    uint32_t ls_dst;
};

__device__ __forceinline__ void db_stage(const DbCtx& cx, int64_t i, int slot, int lane) {
    char* base = reinterpret_cast<char*>(&g_db[slot]);
#pragma unroll
    for (int t = 0; t < 4; ++t)
        __builtin_amdgcn_global_load_lds(GPTR(cx.src[t] + i * cx.row_step), LPTR(base + cx.dst[t]), 16, 0, 0);
    if (lane < 8) __builtin_amdgcn_global_load_lds(GPTR(cx.ls_src + i * cx.ls_step), LPTR(base + cx.ls_dst), 16, 0, 0);
}

__device__ __forceinline__ void db_barrier_keep() {
    static_assert(DB_STAGES == 3 || DB_STAGES == 4, "three or four stages");
    if constexpr (DB_STAGES == 3) asm volatile("s_waitcnt vmcnt(5)\n\ts_barrier" ::: "memory");
    if constexpr (DB_STAGES == 4) asm volatile("s_waitcnt vmcnt(10)\n\ts_barrier" ::: "memory");
}

__global__ void __launch_bounds__(DB_THR) bwd_dbias_lds(BwdProblem p, const float* img, const __bf16* g16,
                                                        const float* lseT, const float* deltaT, int n_jb, int nblk,
                                                        int64_t NP, int n_t, int total) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 31, h2 = lane >> 5;
    // XCD-aware remap: XCD x walks a contiguous range of logical ids; inside one (b, h)
    // strips of DB_TILE_J query tiles, cut into tiles of DB_TILE_J x DB_TILE_K, key tile fastest
    const int w = blockIdx.x;
    const int xcd = w % 8, slot = w / 8;
    const int base = total / 8, extra = total % 8;
    const int logical = xcd * base + (xcd < extra ? xcd : extra) + slot;
    const int bh = logical / (n_t * n_t);
    const int rem = logical - bh * n_t * n_t;
    const int strip = rem / (DB_TILE_J * n_t);
    const int nr = min(DB_TILE_J, n_t - strip * DB_TILE_J);
    const int o = rem - strip * DB_TILE_J * n_t;
    const int tile = o / (nr * DB_TILE_K);
    const int nk = min(DB_TILE_K, n_t - tile * DB_TILE_K);
    const int o2 = o - tile * nr * DB_TILE_K;
    const int jt = strip * DB_TILE_J + o2 / nk;
    const int kt = tile * DB_TILE_K + o2 % nk;
    const int64_t N = p.N, H = p.H, HD = H * D;
    const int64_t b = bh / H, h = bh % H;
    const int64_t j0 = static_cast<int64_t>(jt) * DB_Q, k0 = static_cast<int64_t>(kt) * DB_K;

    DbCtx cx;
    {
        // piece pi = 4 w + t: tensor pi / 8 (Q, dO, K, V), rows 16 (pi % 8) .. +15; lane l
        // carries row l / 4, 16-byte slot l % 4, which holds logical part kv_chunk(row, slot)
        const __bf16* tens[4] = {static_cast<const __bf16*>(p.q), g16, static_cast<const __bf16*>(p.k),
                                 static_cast<const __bf16*>(p.v)};
        const uint32_t offs[4] = {DB_Q_OFF, DB_G_OFF, DB_K_OFF, DB_V_OFF};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int pi = 4 * wave + t, ten = pi >> 3, r = 16 * (pi & 7) + (lane >> 2);
            int64_t pos = (ten < 2 ? j0 : k0) + r;
            pos = pos < N ? pos : N - 1;                      // padded rows read a real one
            const int part = kv_chunk(r, lane & 3);
            cx.src[t] = reinterpret_cast<const char*>(tens[ten] + (b * p.I * N + pos) * HD + h * D + 8 * part);
            cx.dst[t] = offs[ten] + (pi & 7) * 1024;
        }
        cx.row_step = N * HD * 2;
        // lse / delta: wave w < 4 copies lse of queries 32 w .. +31, wave w >= 4 delta of 32 (w - 4)
        const float* ls = wave < 4 ? lseT : deltaT;
        cx.ls_src = reinterpret_cast<const char*>(ls + (b * p.I * H + h) * NP + j0 + 32 * (wave & 3) + 4 * (lane & 7));
        cx.ls_step = H * NP * 4;
        cx.ls_dst = DB_L_OFF + 128 * wave;
    }

    const int qt = wave & 3, kp = wave >> 2;
    const int64_t j = j0 + 32 * qt + c;
    const bool jok = j < N;
    // bias (+ mask) * sqrt(D) of this lane's query for the 16 keys of each unit's registers
    f32x16 C[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int64_t kb = k0 + 64 * kp + 32 * u;             // a multiple of 32: one image key block
        if (kb >= N) {
            C[u] = f32x16{} - INFINITY;
            continue;
        }
        const int jb = static_cast<int>((jok ? j : 0) / IMG_BJ), jj = static_cast<int>((jok ? j : 0) % IMG_BJ);
        const float* t = img + ((bh * n_jb + jb) * static_cast<int64_t>(nblk) + kb / IMG_BK) * IMG_BJ * IMG_BK + jj * IMG_BK;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(t + img_chunk(jj, 2 * a + h2) * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) C[u][4 * a + e] = x[e];
        }
    }
    // LDS byte offsets of this lane's operand reads (stage 0); unit 1 is 32 rows (+2048) on
    const int kr = 64 * kp + c, qr = 32 * qt + c;
    uint32_t ok[2], oq[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        ok[m] = kr * 64 + kv_chunk(kr, 2 * m + h2) * 16;
        oq[m] = qr * 64 + kv_chunk(qr, 2 * m + h2) * 16;
    }
    const uint32_t ol = DB_L_OFF + qr * 4;
    const uint32_t st0 = LDS_ADDR(&g_db[0]);

    f32x16 acc[2] = {};
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
        u32x4 kk[4], vv[4], qq[2], gg[2];
        float lse, dl;
        asm volatile(
            "ds_read_b128 %0, %14 offset:%c18\n\t"
            "ds_read_b128 %1, %15 offset:%c18\n\t"
            "ds_read_b128 %2, %14 offset:%c19\n\t"
            "ds_read_b128 %3, %15 offset:%c19\n\t"
            "ds_read_b128 %4, %14 offset:%c20\n\t"
            "ds_read_b128 %5, %15 offset:%c20\n\t"
            "ds_read_b128 %6, %14 offset:%c21\n\t"
            "ds_read_b128 %7, %15 offset:%c21\n\t"
            "ds_read_b128 %8, %16 offset:%c22\n\t"
            "ds_read_b128 %9, %17 offset:%c22\n\t"
            "ds_read_b128 %10, %16 offset:%c23\n\t"
            "ds_read_b128 %11, %17 offset:%c23\n\t"
            "ds_read_b32 %12, %24\n\t"
            "ds_read_b32 %13, %24 offset:%c25\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(kk[0]), "=&v"(kk[1]), "=&v"(kk[2]), "=&v"(kk[3]), "=&v"(vv[0]), "=&v"(vv[1]), "=&v"(vv[2]),
              "=&v"(vv[3]), "=&v"(qq[0]), "=&v"(qq[1]), "=&v"(gg[0]), "=&v"(gg[1]), "=&v"(lse), "=&v"(dl)
            : "v"(st + ok[0]), "v"(st + ok[1]), "v"(st + oq[0]), "v"(st + oq[1]), "i"(DB_K_OFF), "i"(DB_K_OFF + 2048),
              "i"(DB_V_OFF), "i"(DB_V_OFF + 2048), "i"(DB_Q_OFF), "i"(DB_G_OFF), "v"(st + ol), "i"(DB_Q * 4));
        const float nb = neg_lse2(lse);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            f32x16 S = mfma(__builtin_bit_cast(bf16x8, kk[2 * u]), __builtin_bit_cast(bf16x8, qq[0]), C[u]);
            S = mfma(__builtin_bit_cast(bf16x8, kk[2 * u + 1]), __builtin_bit_cast(bf16x8, qq[1]), S);
            f32x16 dP = mfma(__builtin_bit_cast(bf16x8, vv[2 * u]), __builtin_bit_cast(bf16x8, gg[0]), f32x16{});
            dP = mfma(__builtin_bit_cast(bf16x8, vv[2 * u + 1]), __builtin_bit_cast(bf16x8, gg[1]), dP);
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[u][r] = fmaf(__builtin_amdgcn_exp2f(fmaf(S[r], kScale, nb)), dP[r] - dl, acc[u][r]);
        }
        if (issue)
            db_barrier_keep();
        else
            db_barrier_drain();
    }
    if (jok) {
        float* out = p.dbias + (bh * N + j) * N;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t kk = k0 + 64 * kp + 32 * u + 8 * (r / 4) + 4 * h2 + (r % 4);
                if (kk < N) out[kk] = acc[u][r];
            }
    }
}

}  // namespace

namespace {
struct BwdLayout {
    Problem fwd, tr;        // image problems: the bias, and its transpose without the mask
    int64_t NP, nq;
    size_t img, imgT, g16, delta, lseT, deltaT, total;   // byte offsets / total
};

BwdLayout bwd_layout(const BwdProblem& p) {
    BwdLayout L;
    L.fwd = Problem{p.q, p.k, p.v, p.bias, p.mask, nullptr, p.B, p.H, p.I, p.N, p.D, 1};
    L.tr = Problem{p.q, p.k, p.v, p.bias, nullptr, nullptr, p.B, p.H, p.N, p.N, p.D, 1};
    L.tr.ending = true;
    L.NP = (p.N + NP_ALIGN - 1) / NP_ALIGN * NP_ALIGN;
    L.nq = p.B * p.I * p.N * p.H;
    const size_t per_line = static_cast<size_t>(p.B * p.I * p.H * L.NP) * 4;
    L.img = 0;
    L.imgT = L.img + bias_image_bytes(L.fwd);
    L.g16 = L.imgT + bias_image_bytes(L.tr);
    L.delta = L.g16 + static_cast<size_t>(L.nq) * D * 2;
    L.lseT = L.delta + (static_cast<size_t>(L.nq) * 4 + 15) / 16 * 16;
    L.deltaT = L.lseT + per_line;
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
    float* img = reinterpret_cast<float*>(ws + Ly.img);
    float* imgT = reinterpret_cast<float*>(ws + Ly.imgT);
    __bf16* g16 = reinterpret_cast<__bf16*>(ws + Ly.g16);
    float* delta = reinterpret_cast<float*>(ws + Ly.delta);
    float* lseT = reinterpret_cast<float*>(ws + Ly.lseT);
    float* deltaT = reinterpret_cast<float*>(ws + Ly.deltaT);
    const int64_t n_prep = p.B * p.I * p.H * Ly.NP;
    if (p.D != D || (n_prep + 255) / 256 > 0x7FFFFFFF || (p.N + 63) / 64 > 65535) return hipErrorInvalidConfiguration;
    hipError_t e = launch_bias_image(Ly.fwd, img, stream);
    if (e != hipSuccess) return e;
    if ((e = launch_bias_image(Ly.tr, imgT, stream)) != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_prep_kernel, dim3(static_cast<unsigned>((n_prep + 255) / 256)), dim3(256), 0, stream, p, g16,
                       delta, lseT, deltaT, Ly.NP);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const dim3 lines(static_cast<unsigned>(n_jb), static_cast<unsigned>(p.I), static_cast<unsigned>(p.B * p.H));
    {
        const int64_t n_rg = (p.I + DQ_R - 1) / DQ_R;
        const int64_t total = n_jb * n_rg * p.B * p.H;
        if (total > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(bwd_dq_lds, dim3(static_cast<unsigned>(total)), dim3(DQ_THR), 0, stream, p, img, g16, delta,
                           static_cast<int>(n_jb), static_cast<int>(n_rg), static_cast<int>(nblk),
                           static_cast<int>(total));
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(bwd_dkdv_mfma, lines, dim3(NTHR), 0, stream, p, imgT, g16, lseT, deltaT,
                       static_cast<int>(n_jb), static_cast<int>(nblk), Ly.NP);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t n_t = (p.N + DB_Q - 1) / DB_Q;
    const int64_t total = n_t * n_t * p.B * p.H;
    if (total > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(bwd_dbias_lds, dim3(static_cast<unsigned>(total)), dim3(DB_THR), 0, stream, p, img, g16, lseT,
                       deltaT, static_cast<int>(n_jb), static_cast<int>(nblk), Ly.NP, static_cast<int>(n_t),
                       static_cast<int>(total));
    return hipGetLastError();
}

}  // namespace tri_attn
