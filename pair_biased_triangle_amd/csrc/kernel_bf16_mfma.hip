// bf16 triangle attention on gfx950 matrix cores (head size D = 32).
//
// Per batch b and head h the rows i are independent attention problems that share one
// N x N "triangular" bias bias[b,h,j,k] ("Fold-CP", Table 1 "Triangle Attention" and
// Figure 2(a)).  A workgroup owns R = 8 rows i and BJ = 128 query columns j of one
// (b, h) and streams the key axis in blocks of 32 keys.  Key blocks follow the ring-step
// tiles (Table 1's caption): they start at every tile start and are cut short at every
// tile end, so each tile is folded into the running softmax state as one ring step.
//
// Per key block the workgroup stages, in LDS:
//   * K of its 8 rows   [row][key][d]        (bf16, as stored)
//   * V of its 8 rows   [row][d][key]        (bf16, transposed while staging)
//   * the bias block    [j][key], fp32, already (bias + mask) * sqrt(D): converted once
//     per workgroup and reused by all 8 rows -- the triangular bias is shared across i.
// Each of the 8 waves owns 2 rows x 2 query tiles of 32.  For each (row, tile) it runs
//   S^T = K Q^T + C         two v_mfma_f32_32x32x16_bf16, C = the staged bias block,
//                           so S = sqrt(D) * (q.k / sqrt(D) + bias + mask) in fp32
//   p   = 2^(S * log2(e)/sqrt(D) - m_ref * log2(e)/sqrt(D))    (one FMA + v_exp_f32)
//   O^T += V^T P^T          two v_mfma_f32_32x32x16_bf16 on the bf16-rounded p
// In the 32x32 output layout each lane holds 16 keys of one query, so the row maximum
// needs one cross-lane step (lanes l and l^32) per block and the row sum is taken per
// lane with v_dot2_f32_bf16 on the rounded p (the weights the P.V product uses).
// The reference m_ref is refreshed only when a block's maximum exceeds it by more than
// 8 (in log2 units), so the O and l rescales are rare; p stays below 2^8, exact either
// way because O and l share one reference (online normaliser rule).
// Workgroup ids are remapped so that each XCD walks a contiguous range of (b, h, row
// group, column block) with the column block fastest: the K/V stream of a row group and
// the bias strips stay hot in that XCD's L2.
#include "launch.h"

#include <cmath>

namespace tri_attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

constexpr int KS_LD = 40;                   // bf16 per staged key row (32 + pad)
constexpr int VT_LD = 40;                   // bf16 per staged d row of V^T (32 keys + pad)
constexpr int BS_LD = 36;                   // fp32 per staged bias row (32 keys + pad)

struct Stage {
    __bf16 k[R][BK][KS_LD];
    __bf16 vt[R][D][VT_LD];
    float bias[BJ][BS_LD];
};
constexpr size_t kSmemBytes = 2 * sizeof(Stage);

constexpr int KV_CHUNKS = R * BK * (D / 8);         // 16-byte chunks of K (and of V) per block
constexpr int KV_PER_THR = KV_CHUNKS / NTHR;
constexpr int BIAS_PER_THR = BJ * BK / NTHR;
static_assert(KV_CHUNKS % NTHR == 0 && (BJ * BK) % NTHR == 0, "staging split");
static_assert(NTHR % BK == 0, "each thread stages one key column of the bias");

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSqrtD = 5.656854249492381f;        // sqrt(32)
constexpr float kScale = kLog2e / kSqrtD;           // S units -> log2 units
constexpr float kTau = 8.0f / kScale;               // refresh threshold in S units

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t u) {
    return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

// Walks the key blocks: tiles in ascending order, 32-key blocks inside each tile.
struct BlockCursor {
    int64_t N;
    int T;
    int t;
    int64_t kb, ke;
    __device__ void init(int64_t n, int tiles) {
        N = n; T = tiles; t = 0;
        kb = 0;
        ke = tile_start(1, N, T);
    }
    __device__ int nk() const { return static_cast<int>(ke - kb < BK ? ke - kb : BK); }
    __device__ bool valid() const { return t < T; }
    __device__ void next() {
        kb += BK;
        if (kb >= ke) {
            ++t;
            kb = ke;
            if (t < T) ke = tile_start(t + 1, N, T);
        }
    }
};

struct Prefetch {
    u32x4 k[KV_PER_THR];
    u32x4 v[KV_PER_THR];
    uint16_t bias[BIAS_PER_THR];
    float mask;
};

__device__ __forceinline__ void prefetch(Prefetch& pf, const Problem& p, int64_t b, int64_t h,
                                         int64_t i0, int64_t j0, int64_t kb, int nk, int tid) {
    const uint16_t* kg = static_cast<const uint16_t*>(p.k);
    const uint16_t* vg = static_cast<const uint16_t*>(p.v);
    const uint16_t* bg = static_cast<const uint16_t*>(p.bias);
#pragma unroll
    for (int n = 0; n < KV_PER_THR; ++n) {
        const int c = tid + n * NTHR;
        const int r = c / (BK * 4), kk = (c / 4) % BK, part = c % 4;
        const int64_t i = i0 + r;
        u32x4 zk = {0, 0, 0, 0}, zv = zk;
        if (i < p.I && kk < nk) {
            const int64_t off = (((b * p.I + i) * p.N + kb + kk) * p.H + h) * D + part * 8;
            zk = *reinterpret_cast<const u32x4*>(kg + off);
            zv = *reinterpret_cast<const u32x4*>(vg + off);
        }
        pf.k[n] = zk;
        pf.v[n] = zv;
    }
    const int kk = tid % BK;
    pf.mask = (p.mask && kk < nk) ? p.mask[b * p.N + kb + kk] : 0.0f;
#pragma unroll
    for (int n = 0; n < BIAS_PER_THR; ++n) {
        const int jj = (tid + n * NTHR) / BK;
        const int64_t j = j0 + jj;
        pf.bias[n] = (j < p.N && kk < nk) ? bg[((b * p.H + h) * p.N + j) * p.N + kb + kk] : 0;
    }
}

__device__ __forceinline__ void commit(Stage& st, const Prefetch& pf, int nk, int tid) {
#pragma unroll
    for (int n = 0; n < KV_PER_THR; ++n) {
        const int c = tid + n * NTHR;
        const int r = c / (BK * 4), kk = (c / 4) % BK, part = c % 4;
        *reinterpret_cast<u32x4*>(&st.k[r][kk][part * 8]) = pf.k[n];
        const u32x4 v = pf.v[n];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t w = v[e];
            reinterpret_cast<uint16_t*>(&st.vt[r][part * 8 + 2 * e][0])[kk] = static_cast<uint16_t>(w & 0xFFFFu);
            reinterpret_cast<uint16_t*>(&st.vt[r][part * 8 + 2 * e + 1][0])[kk] = static_cast<uint16_t>(w >> 16);
        }
    }
    const int kk = tid % BK;
    const bool key_ok = kk < nk;
#pragma unroll
    for (int n = 0; n < BIAS_PER_THR; ++n) {
        const int jj = (tid + n * NTHR) / BK;
        st.bias[jj][kk] = key_ok ? (bf16_bits_to_f32(pf.bias[n]) + pf.mask) * kSqrtD : -INFINITY;
    }
}

__global__ void __launch_bounds__(NTHR) bf16_mfma_kernel(Problem p, int n_jb, int n_rg, int total) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Stage* stages = reinterpret_cast<Stage*>(smem_raw);

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
    const int c = lane % 32, h2 = lane / 32;
    const int row0 = (wave / (QT / TW)) * RW;       // first of this wave's rows in the group
    const int tile0 = (wave % (QT / TW)) * TW;      // first of this wave's query tiles

    // Q^T operands (B of S^T = K Q^T): query j = tile*32 + c, d = 16m + 8*h2 .. +7.
    bf16x8 qB[RW][TW][2];
#pragma unroll
    for (int ri = 0; ri < RW; ++ri) {
#pragma unroll
        for (int ti = 0; ti < TW; ++ti) {
            const int64_t i = i0 + row0 + ri, j = j0 + (tile0 + ti) * 32 + c;
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                u32x4 z = {0, 0, 0, 0};
                if (i < p.I && j < p.N) {
                    const int64_t off = (((b * p.I + i) * p.N + j) * p.H + h) * D + 16 * m + 8 * h2;
                    z = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.q) + off);
                }
                qB[ri][ti][m] = __builtin_bit_cast(bf16x8, z);
            }
        }
    }

    f32x16 O[RW][TW];
    float mref[RW][TW], lsum[RW][TW];
#pragma unroll
    for (int ri = 0; ri < RW; ++ri)
#pragma unroll
        for (int ti = 0; ti < TW; ++ti) {
            O[ri][ti] = f32x16{};
            mref[ri][ti] = -INFINITY;
            lsum[ri][ti] = 0.0f;
        }

    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};

    BlockCursor cur;
    cur.init(p.N, p.T);
    Prefetch pf;
    prefetch(pf, p, b, h, i0, j0, cur.kb, cur.nk(), tid);
    commit(stages[0], pf, cur.nk(), tid);
    __syncthreads();

    int buf = 0;
    while (cur.valid()) {
        BlockCursor nxt = cur;
        nxt.next();
        if (nxt.valid()) prefetch(pf, p, b, h, i0, j0, nxt.kb, nxt.nk(), tid);

        const Stage& st = stages[buf];
        bf16x8 kA[RW][2], vA[RW][2];
#pragma unroll
        for (int ri = 0; ri < RW; ++ri) {
            const int r = row0 + ri;
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                kA[ri][m] = *reinterpret_cast<const bf16x8*>(&st.k[r][c][16 * m + 8 * h2]);
                const bf16x4 lo = *reinterpret_cast<const bf16x4*>(&st.vt[r][c][16 * m + 4 * h2]);
                const bf16x4 hi = *reinterpret_cast<const bf16x4*>(&st.vt[r][c][16 * m + 8 + 4 * h2]);
                vA[ri][m] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        }
#pragma unroll
        for (int ti = 0; ti < TW; ++ti) {
            const float* brow = &st.bias[(tile0 + ti) * 32 + c][0];
            f32x16 C;
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(brow + 8 * a + 4 * h2);
                C[4 * a + 0] = x[0];
                C[4 * a + 1] = x[1];
                C[4 * a + 2] = x[2];
                C[4 * a + 3] = x[3];
            }
#pragma unroll
            for (int ri = 0; ri < RW; ++ri) {
                f32x16 S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kA[ri][0], qB[ri][ti][0], C, 0, 0, 0);
                S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kA[ri][1], qB[ri][ti][1], S, 0, 0, 0);

                float mx = S[0];
#pragma unroll
                for (int r = 1; r < 16; ++r) mx = fmaxf(mx, S[r]);
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                const bool need = mx > mref[ri][ti] + kTau;
                if (__any(need)) {
                    const float mnew = need ? mx : mref[ri][ti];
                    const float alpha = need ? exp2f((mref[ri][ti] - mnew) * kScale) : 1.0f;
                    lsum[ri][ti] *= alpha;
#pragma unroll
                    for (int r = 0; r < 16; ++r) O[ri][ti][r] *= alpha;
                    mref[ri][ti] = mnew;
                }
                const float nb = mref[ri][ti] == -INFINITY ? 0.0f : -mref[ri][ti] * kScale;
                f32x16 P;
#pragma unroll
                for (int r = 0; r < 16; ++r) P[r] = __builtin_amdgcn_exp2f(fmaf(S[r], kScale, nb));
                const f32x8 p0 = __builtin_shufflevector(P, P, 0, 1, 2, 3, 4, 5, 6, 7);
                const f32x8 p1 = __builtin_shufflevector(P, P, 8, 9, 10, 11, 12, 13, 14, 15);
                const bf16x8 pb0 = __builtin_convertvector(p0, bf16x8);
                const bf16x8 pb1 = __builtin_convertvector(p1, bf16x8);
                float ls = lsum[ri][ti];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bf16x2 a0 = {pb0[2 * e], pb0[2 * e + 1]};
                    const bf16x2 a1 = {pb1[2 * e], pb1[2 * e + 1]};
                    ls = __builtin_amdgcn_fdot2_f32_bf16(a0, ones, ls, false);
                    ls = __builtin_amdgcn_fdot2_f32_bf16(a1, ones, ls, false);
                }
                lsum[ri][ti] = ls;
                O[ri][ti] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vA[ri][0], pb0, O[ri][ti], 0, 0, 0);
                O[ri][ti] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vA[ri][1], pb1, O[ri][ti], 0, 0, 0);
            }
        }

        if (nxt.valid()) commit(stages[buf ^ 1], pf, nxt.nk(), tid);
        __syncthreads();
        buf ^= 1;
        cur = nxt;
    }

    // out = O / l; lanes l and l^32 hold disjoint keys of the same query.
#pragma unroll
    for (int ri = 0; ri < RW; ++ri) {
#pragma unroll
        for (int ti = 0; ti < TW; ++ti) {
            const float lt = lsum[ri][ti] + __shfl_xor(lsum[ri][ti], 32);
            const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
            const int64_t i = i0 + row0 + ri, j = j0 + (tile0 + ti) * 32 + c;
            if (i < p.I && j < p.N) {
                float* o = p.out + (((b * p.I + i) * p.N + j) * p.H + h) * D;
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    f32x4 x;
                    x[0] = O[ri][ti][4 * a + 0] * inv;
                    x[1] = O[ri][ti][4 * a + 1] * inv;
                    x[2] = O[ri][ti][4 * a + 2] * inv;
                    x[3] = O[ri][ti][4 * a + 3] * inv;
                    *reinterpret_cast<f32x4*>(o + 8 * a + 4 * h2) = x;
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_bf16_mfma(const Problem& p, hipStream_t stream) {
    static bool attr_set = false;
    if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bf16_mfma_kernel),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 static_cast<int>(kSmemBytes));
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int64_t n_jb = (p.N + BJ - 1) / BJ;
    const int64_t n_rg = (p.I + R - 1) / R;
    const int64_t total = n_jb * n_rg * p.B * p.H;
    if (total > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(bf16_mfma_kernel, dim3(static_cast<unsigned>(total)), dim3(NTHR), kSmemBytes, stream,
                       p, static_cast<int>(n_jb), static_cast<int>(n_rg), static_cast<int>(total));
    return hipGetLastError();
}

}  // namespace tri_attn
