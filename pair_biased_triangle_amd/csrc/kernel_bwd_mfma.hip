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
__global__ void __launch_bounds__(256) bwd_prep_kernel(const float* dout, const float* out, __bf16* g16, float* delta,
                                                       int64_t nq) {
    const int64_t q = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (q >= nq) return;
    const f32x4* g = reinterpret_cast<const f32x4*>(dout + q * D);
    const f32x4* o = reinterpret_cast<const f32x4*>(out + q * D);
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
}

// ---------------------------------------------------------------------------------------
__global__ void __launch_bounds__(NTHR) bwd_dq_mfma(BwdProblem p, const float* img, const __bf16* g16,
                                                    const float* delta, int n_jb, int nblk) {
    __shared__ __attribute__((aligned(16))) char lds[NWAVE * TILE_BYTES];
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 31, h2 = lane >> 5;
    const int64_t N = p.N, H = p.H, HD = H * D;
    const int64_t bh = blockIdx.z, b = bh / H, h = bh % H, i = blockIdx.y;
    const int jb = blockIdx.x;
    const int jj = wave * 32 + c;                         // query inside the 128-query block
    const int64_t j = static_cast<int64_t>(jb) * IMG_BJ + jj;
    const bool jok = j < N;
    const int64_t row = (b * p.I + i) * N;                // flat (b, i, 0)
    const __bf16* q = static_cast<const __bf16*>(p.q);
    const __bf16* k = static_cast<const __bf16*>(p.k);
    const __bf16* v = static_cast<const __bf16*>(p.v);
    const int64_t qo = (row + j) * HD + h * D;

    bf16x8 qB[2], gB[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        qB[m] = frag(q, qo + 16 * m + 8 * h2, jok);
        gB[m] = frag(g16, qo + 16 * m + 8 * h2, jok);
    }
    const float nb = jok ? neg_lse2(p.lse[(row + j) * H + h]) : -INFINITY;
    const float dl = jok ? delta[(row + j) * H + h] : 0.0f;
    const TileLane L = tile_lane(lane);
    const uint32_t tile = LDS_ADDR(lds) + wave * TILE_BYTES;
    const float* img_row = img + (bh * n_jb + jb) * static_cast<int64_t>(nblk) * IMG_BJ * IMG_BK + jj * IMG_BK;

    f32x16 dQ = {};
    for (int n = 0; n < nblk; ++n) {
        const int64_t key = static_cast<int64_t>(n) * IMG_BK + c;
        const int64_t ko = (row + (key < N ? key : N - 1)) * HD + h * D;   // padded keys: bias -inf
        bf16x8 kA[2], vA[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            kA[m] = frag(k, ko + 16 * m + 8 * h2, true);
            vA[m] = frag(v, ko + 16 * m + 8 * h2, true);
        }
        f32x16 C;
        const float* t = img_row + static_cast<int64_t>(n) * IMG_BJ * IMG_BK;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(t + img_chunk(jj, 2 * a + h2) * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) C[4 * a + e] = x[e];
        }
        f32x16 S = mfma(kA[0], qB[0], C);
        S = mfma(kA[1], qB[1], S);
        f32x16 dP = mfma(vA[0], gB[0], f32x16{});
        dP = mfma(vA[1], gB[1], dP);
        f32x16 dS;
#pragma unroll
        for (int r = 0; r < 16; ++r) dS[r] = __builtin_amdgcn_exp2f(fmaf(S[r], kScale, nb)) * (dP[r] - dl);
        bf16x8 s0, s1, kT0, kT1;
        to_bf16(dS, s0, s1);
        transpose_tile(tile, L, kA[0], kA[1], kT0, kT1);
        dQ = mfma(kT0, s0, dQ);
        dQ = mfma(kT1, s1, dQ);
    }
    if (jok) {
        float* o = p.dq + qo;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            f32x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = dQ[4 * a + e] * kInvSqrtD;
            *reinterpret_cast<f32x4*>(o + 8 * a + 4 * h2) = x;
        }
    }
}

// ---------------------------------------------------------------------------------------
__global__ void __launch_bounds__(NTHR, 2) bwd_dkdv_mfma(BwdProblem p, const __bf16* g16, const float* delta) {
    __shared__ __attribute__((aligned(16))) char lds[NWAVE * 2 * TILE_BYTES];
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 31, h2 = lane >> 5;
    const int64_t N = p.N, H = p.H, HD = H * D;
    const int64_t bh = blockIdx.z, b = bh / H, h = bh % H, i = blockIdx.y;
    const int64_t key = static_cast<int64_t>(blockIdx.x) * (NWAVE * 32) + wave * 32 + c;
    const bool kok = key < N;
    const int64_t row = (b * p.I + i) * N;
    const __bf16* q = static_cast<const __bf16*>(p.q);
    const __bf16* k = static_cast<const __bf16*>(p.k);
    const __bf16* v = static_cast<const __bf16*>(p.v);
    const uint16_t* bias = static_cast<const uint16_t*>(p.bias);
    const int64_t ko = (row + key) * HD + h * D;

    bf16x8 kB[2], vB[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        kB[m] = frag(k, ko + 16 * m + 8 * h2, kok);
        vB[m] = frag(v, ko + 16 * m + 8 * h2, kok);
    }
    const float mk = !kok ? -INFINITY : (p.mask ? p.mask[b * N + key] : 0.0f);
    const TileLane L = tile_lane(lane);
    const uint32_t tile_g = LDS_ADDR(lds) + wave * 2 * TILE_BYTES, tile_q = tile_g + TILE_BYTES;

    f32x16 dK = {}, dV = {};
    for (int64_t qb = 0; qb < N; qb += 32) {
        const int64_t jq = qb + c;                        // this lane's row of the A operands
        const bool jok = jq < N;
        const int64_t qo = (row + jq) * HD + h * D;
        bf16x8 qA[2], gA[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            qA[m] = frag(q, qo + 16 * m + 8 * h2, jok);
            gA[m] = frag(g16, qo + 16 * m + 8 * h2, jok);
        }
        // C for the 16 query rows of this lane's accumulator registers
        f32x16 C;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t jr = qb + 8 * (r / 4) + 4 * h2 + (r % 4);
            const float bv = jr < N ? bf16_to_f32(bias[(bh * N + jr) * N + (kok ? key : 0)]) : 0.0f;
            C[r] = jr < N ? (bv + mk) * kSqrtD : -INFINITY;
        }
        f32x16 S = mfma(qA[0], kB[0], C);
        S = mfma(qA[1], kB[1], S);
        f32x16 dP = mfma(gA[0], vB[0], f32x16{});
        dP = mfma(gA[1], vB[1], dP);
        // P overwrites S and dS overwrites dP, row by row with that row's lse and delta
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t jr = qb + 8 * (r / 4) + 4 * h2 + (r % 4);
            const bool ok = jr < N;
            const float nb = ok ? neg_lse2(p.lse[(row + jr) * H + h]) : -INFINITY;
            const float dl = ok ? delta[(row + jr) * H + h] : 0.0f;
            S[r] = __builtin_amdgcn_exp2f(fmaf(S[r], kScale, nb));
            dP[r] = S[r] * (dP[r] - dl);
        }
        const f32x16& P = S;
        const f32x16& dS = dP;
        bf16x8 p0, p1, s0, s1, gT0, gT1, qT0, qT1;
        to_bf16(P, p0, p1);
        to_bf16(dS, s0, s1);
        transpose_tile(tile_g, L, gA[0], gA[1], gT0, gT1);
        transpose_tile(tile_q, L, qA[0], qA[1], qT0, qT1);
        dV = mfma(gT0, p0, dV);
        dV = mfma(gT1, p1, dV);
        dK = mfma(qT0, s0, dK);
        dK = mfma(qT1, s1, dK);
    }
    if (kok) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            f32x4 xk, xv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xk[e] = dK[4 * a + e] * kInvSqrtD;
                xv[e] = dV[4 * a + e];
            }
            *reinterpret_cast<f32x4*>(p.dk + ko + 8 * a + 4 * h2) = xk;
            *reinterpret_cast<f32x4*>(p.dv + ko + 8 * a + 4 * h2) = xv;
        }
    }
}

// ---------------------------------------------------------------------------------------
// Workgroup: 64 queries x 64 keys of one (b, h); wave w takes queries (w & 1) * 32 and
// keys (w >> 1) * 32 of it.
__global__ void __launch_bounds__(NTHR) bwd_dbias_mfma(BwdProblem p, const float* img, const __bf16* g16,
                                                       const float* delta, int n_jb, int nblk) {
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 31, h2 = lane >> 5;
    const int64_t N = p.N, H = p.H, HD = H * D;
    const int64_t bh = blockIdx.z, b = bh / H, h = bh % H;
    const int64_t j = static_cast<int64_t>(blockIdx.y) * 64 + (wave & 1) * 32 + c;
    const int64_t k0 = static_cast<int64_t>(blockIdx.x) * 64 + (wave >> 1) * 32;
    if (k0 >= N) return;                                  // a wave past the last key (no barriers here)
    const bool jok = j < N;
    const int64_t kc = k0 + c < N ? k0 + c : N - 1;       // padded keys read a real key (bias -inf)
    const __bf16* q = static_cast<const __bf16*>(p.q);
    const __bf16* k = static_cast<const __bf16*>(p.k);
    const __bf16* v = static_cast<const __bf16*>(p.v);

    // bias (+ mask) * sqrt(D) of this lane's query for the 16 keys of its registers
    f32x16 C;
    {
        const int jb = static_cast<int>(j / IMG_BJ), jj = static_cast<int>(j % IMG_BJ);
        const int n = static_cast<int>(k0 / IMG_BK);
        const float* t = img + ((bh * n_jb + (jok ? jb : 0)) * static_cast<int64_t>(nblk) + n) * IMG_BJ * IMG_BK +
                         jj * IMG_BK;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(t + img_chunk(jj, 2 * a + h2) * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) C[4 * a + e] = x[e];
        }
    }
    f32x16 acc = {};
    for (int64_t i = 0; i < p.I; ++i) {
        const int64_t row = (b * p.I + i) * N;
        const int64_t ko = (row + kc) * HD + h * D, qo = (row + j) * HD + h * D;
        bf16x8 kA[2], vA[2], qB[2], gB[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            kA[m] = frag(k, ko + 16 * m + 8 * h2, true);
            vA[m] = frag(v, ko + 16 * m + 8 * h2, true);
            qB[m] = frag(q, qo + 16 * m + 8 * h2, jok);
            gB[m] = frag(g16, qo + 16 * m + 8 * h2, jok);
        }
        const float nb = jok ? neg_lse2(p.lse[(row + j) * H + h]) : -INFINITY;
        const float dl = jok ? delta[(row + j) * H + h] : 0.0f;
        f32x16 S = mfma(kA[0], qB[0], C);
        S = mfma(kA[1], qB[1], S);
        f32x16 dP = mfma(vA[0], gB[0], f32x16{});
        dP = mfma(vA[1], gB[1], dP);
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = fmaf(__builtin_amdgcn_exp2f(fmaf(S[r], kScale, nb)), dP[r] - dl, acc[r]);
    }
    if (jok) {
        float* o = p.dbias + (bh * N + j) * N;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t kk = k0 + 8 * (r / 4) + 4 * h2 + (r % 4);
            if (kk < N) o[kk] = acc[r];
        }
    }
}

}  // namespace

size_t bwd_mfma_workspace_bytes(const BwdProblem& p) {
    Problem f{p.q, p.k, p.v, p.bias, p.mask, nullptr, p.B, p.H, p.I, p.N, p.D, 1};
    const size_t img = bf16_workspace_bytes(f);
    const size_t nq = static_cast<size_t>(p.B * p.I * p.N * p.H);
    return img + nq * D * 2 + nq * 4;
}

hipError_t launch_backward_mfma(const BwdProblem& p, void* workspace, hipStream_t stream) {
    Problem f{p.q, p.k, p.v, p.bias, p.mask, nullptr, p.B, p.H, p.I, p.N, p.D, 1};
    const int64_t n_jb = (p.N + IMG_BJ - 1) / IMG_BJ;
    const int64_t nblk = bias_image_blocks(f);
    const int64_t nq = p.B * p.I * p.N * p.H;
    char* ws = static_cast<char*>(workspace);
    float* img = reinterpret_cast<float*>(ws);
    __bf16* g16 = reinterpret_cast<__bf16*>(ws + bf16_workspace_bytes(f));
    float* delta = reinterpret_cast<float*>(ws + bf16_workspace_bytes(f) + static_cast<size_t>(nq) * D * 2);
    if (p.D != D || (nq + 255) / 256 > 0x7FFFFFFF || (p.N + 63) / 64 > 65535) return hipErrorInvalidConfiguration;
    hipError_t e = launch_bias_image(f, img, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_prep_kernel, dim3(static_cast<unsigned>((nq + 255) / 256)), dim3(256), 0, stream, p.dout,
                       p.out, g16, delta, nq);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const dim3 lines(static_cast<unsigned>(n_jb), static_cast<unsigned>(p.I), static_cast<unsigned>(p.B * p.H));
    hipLaunchKernelGGL(bwd_dq_mfma, lines, dim3(NTHR), 0, stream, p, img, g16, delta, static_cast<int>(n_jb),
                       static_cast<int>(nblk));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_dkdv_mfma, lines, dim3(NTHR), 0, stream, p, g16, delta);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const unsigned nt = static_cast<unsigned>((p.N + 63) / 64);
    hipLaunchKernelGGL(bwd_dbias_mfma, dim3(nt, nt, static_cast<unsigned>(p.B * p.H)), dim3(NTHR), 0, stream, p, img,
                       g16, delta, static_cast<int>(n_jb), static_cast<int>(nblk));
    return hipGetLastError();
}

}  // namespace tri_attn
