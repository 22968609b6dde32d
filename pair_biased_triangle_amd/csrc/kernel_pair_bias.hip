// Attention with pair bias in one pass over the bias ("Fold-CP", Table 1 "Attention with
// pair bias" and Figure 2(c)): token attention over one sequence (one line, I == 1) with
// an additive [B, H, N, N] bias,
//     out[b, j, h, :] = sum_k softmax_k(q_j . k_k / sqrt(D) + bias[b, h, j, k] + mask[b, k]) v_k.
// With a single line every bias value is used once, so the triangle kernel's prepass (a
// reference maximum and an fp16 image: two reads of the bias, a write and a read of the
// image) costs several times the attention itself.  Here the raw bf16 bias is copied
// straight into LDS, once, and each query keeps a running reference of its scores
// (the online-normaliser form of the tiled-softmax merge, the reference moved only when a
// score passes it by more than 8 in log2 units).  The keys are cut into ranges
// that run side by side; their partial states are joined by state_combine_kernel.
//
// A workgroup of 4 waves owns 128 queries of one (b, h) and one key range; wave w owns
// queries 32 w .. 32 w + 31.  Per 32-key block the waves copy K and V (16-byte copies of
// 64-byte rows), the 128 x 32 bias tile (4-byte copies: a bias row starts at an offset of
// N * 2 bytes, which is 4-byte aligned for even N but not 16-byte aligned in general) and
// the block's 32 mask values into a ring of LDS stages, then per wave:
//     S^T = K Q^T                   two v_mfma_f32_32x32x16_bf16 (Q in registers)
//     z   = S / sqrt(D) + bias + mask                    the score, natural units
//     m'  = max_k z if it exceeds m by more than 8 ln 2, else m;  alpha = e^(m - m'),
//     p   = 2^((z - m') log2(e))
//     O^T = alpha O^T + V^T P^T     two v_mfma_f32_32x32x16_bf16 on the bf16-rounded p
//     l   = alpha l + sum_k p       over the rounded p
// The copies of a whole block take a wave-uniform base (the block's first key) plus a
// per-lane offset fixed for the whole loop; only a block that runs past the last key
// clamps its sources (and drops its extra keys from the scores).
// Operand layouts are those of the triangle kernel (kernel_bf16_mfma.hip).
#include "pair_bias.h"

#include <cmath>
#include <cstddef>
#include <type_traits>

namespace tri_attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define PB_GPTR(p) ((const __attribute__((address_space(1))) void*)(p))
#define PB_LPTR(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int D = 32;
constexpr int BK = 32;                // keys per block
constexpr int PQ = 128;               // queries per workgroup
constexpr int PW = 4;                 // waves per workgroup, one 32-query tile each
constexpr int PTHR = 64 * PW;
#ifndef TRI_ATTN_PB_STAGES
#define TRI_ATTN_PB_STAGES 3
#endif
#ifndef TRI_ATTN_PB_FILL
#define TRI_ATTN_PB_FILL 768
#endif
#ifndef TRI_ATTN_PB_OCC
#define TRI_ATTN_PB_OCC 3
#endif
constexpr int PSTAGE = TRI_ATTN_PB_STAGES;      // LDS ring: blocks in flight
constexpr int MAX_SPLIT = 16;                   // key ranges per (b, h, query block), at most
constexpr int MIN_SPLIT_BLOCKS = 4;             //   each of at least this many blocks
constexpr int64_t FILL_WGS = TRI_ATTN_PB_FILL;  // workgroups resident at once (256 CUs x TRI_ATTN_PB_OCC): the
                                                //   key ranges stop where another would need a second round
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kInvSqrtD = 0.17677669529663687f;   // 1 / sqrt(32)
constexpr float RESCALE_SLACK = 8.0f * 0.6931471805599453f;   // a score may exceed the reference by 8 log2 units

// 16-byte chunk `part` of a 64-byte LDS row is stored at chunk kv_chunk(row, part)
__host__ __device__ constexpr int kv_chunk(int row, int part) { return part ^ ((row >> 1) & 3); }

struct PbStage {
    __bf16 k[BK][D];       // [key][d]
    __bf16 v[BK][D];
    __bf16 bias[PQ][BK];   // [query][key], natural key order inside each 16-byte chunk
    float mask[BK];        // raw mask values of the block's keys (ignored without a mask)
};
constexpr int PB_STAGE_BYTES = static_cast<int>(sizeof(PbStage));
constexpr int PB_K = static_cast<int>(offsetof(PbStage, k));
constexpr int PB_V = static_cast<int>(offsetof(PbStage, v));
constexpr int PB_B = static_cast<int>(offsetof(PbStage, bias));
constexpr int PB_M = static_cast<int>(offsetof(PbStage, mask));
// per wave and block: one 1 KB K/V piece (16-byte copies), 8 bias pieces of 256 bytes
// (4 rows, 4-byte copies) and 8 mask values (4-byte copies, lanes 0 .. 7)
constexpr int PB_BIAS_PER_WAVE = PQ * BK * 2 / 256 / PW;
constexpr int PB_COPIES = 1 + PB_BIAS_PER_WAVE + 1;
static_assert(PB_BIAS_PER_WAVE == 8 && 4 * 1024 == 2 * BK * D * 2, "pieces per wave");
__shared__ PbStage g_pb[PSTAGE];

struct PbCtx {
    const char* kv;        // this wave's K/V piece source at key 0 (wave-uniform)
    uint32_t kv_off;       // this lane's byte offset from it: key kv_key, 16-byte part kv_part
    uint32_t kv_lds;       // its place in a stage
    int kv_key;            // key of this lane's 16-byte slot inside the block
    int kv_part;           // logical 16-byte part of the key held by this lane's slot
    int64_t key_bytes;     // bytes between consecutive keys of K or V
    const char* bias;      // the (b, h) bias slab at query 0, key 0 (wave-uniform)
    uint32_t boff[PB_BIAS_PER_WAVE];   // this lane's byte offset in the slab per piece (block 0)
    const char* mrow;      // mask of this batch element at key 0 (or a valid dummy source)
    int N;
};

// Copies of block n when all its keys exist: wave-uniform sources plus fixed lane offsets.
__device__ __forceinline__ void pb_stage_full(const PbCtx& cx, int n, int wave, int lane) {
    char* st = reinterpret_cast<char*>(&g_pb[n % PSTAGE]);
    const int k0 = BK * n;
    {
        uint32_t off = cx.kv_off;
        asm volatile("" : "+v"(off));
        __builtin_amdgcn_global_load_lds(PB_GPTR(cx.kv + k0 * cx.key_bytes + off), PB_LPTR(st + cx.kv_lds), 16, 0, 0);
    }
    const char* bbase = cx.bias + k0 * 2;
#pragma unroll
    for (int t = 0; t < PB_BIAS_PER_WAVE; ++t) {
        uint32_t off = cx.boff[t];
        asm volatile("" : "+v"(off));
        __builtin_amdgcn_global_load_lds(PB_GPTR(bbase + off), PB_LPTR(st + PB_B + (PB_BIAS_PER_WAVE * wave + t) * 256), 4,
                                         0, 0);
    }
    if (lane < 8) {
        uint32_t off = static_cast<uint32_t>((8 * wave + lane) * 4);
        asm volatile("" : "+v"(off));
        __builtin_amdgcn_global_load_lds(PB_GPTR(cx.mrow + k0 * 4 + off), PB_LPTR(st + PB_M + 32 * wave), 4, 0, 0);
    }
}

// Copies of a block that runs past the last key: every source clamped to a real key.
// Bias piece t of wave w: rows 4 g .. 4 g + 3 of the tile (g = 8 w + t); lane l writes the
// 4-byte word l % 16 of row 4 g + l / 16, i.e. word w4 = l % 4 of 16-byte slot (l % 16) / 4,
// which holds keys 8 kv_chunk(row, slot) + 2 w4, +1: the first of them, inside the block.
__device__ __forceinline__ int pb_bias_key(int wave, int t, int lane) {
    const int row = 4 * (PB_BIAS_PER_WAVE * wave + t) + (lane >> 4);
    return 8 * kv_chunk(row, (lane >> 2) & 3) + 2 * (lane & 3);
}

__device__ __forceinline__ void pb_stage_tail(const PbCtx& cx, int n, int wave, int lane) {
    char* st = reinterpret_cast<char*>(&g_pb[n % PSTAGE]);
    const int k0 = BK * n;
    {
        const int key = min(k0 + cx.kv_key, cx.N - 1);                 // keys past the end read the last key
        const char* src = cx.kv + key * cx.key_bytes + cx.kv_part * 16;
        __builtin_amdgcn_global_load_lds(PB_GPTR(src), PB_LPTR(st + cx.kv_lds), 16, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < PB_BIAS_PER_WAVE; ++t) {
        const int bkey = pb_bias_key(wave, t, lane);
        const int key = min(k0 + bkey, cx.N - 2);                       // an even key: 4-byte aligned pair
        const char* src = cx.bias + cx.boff[t] + (key - bkey) * 2;
        __builtin_amdgcn_global_load_lds(PB_GPTR(src), PB_LPTR(st + PB_B + (PB_BIAS_PER_WAVE * wave + t) * 256), 4, 0,
                                         0);
    }
    if (lane < 8) {
        const int key = min(k0 + 8 * wave + lane, cx.N - 1);
        __builtin_amdgcn_global_load_lds(PB_GPTR(cx.mrow + key * 4), PB_LPTR(st + PB_M + 32 * wave), 4, 0, 0);
    }
}

__device__ __forceinline__ void pb_stage(const PbCtx& cx, int n, int wave, int lane) {
    if (BK * (n + 1) <= cx.N)
        pb_stage_full(cx, n, wave, lane);
    else
        pb_stage_tail(cx, n, wave, lane);
}

__device__ __forceinline__ void pb_barrier_keep() {
    constexpr int keep = PB_COPIES * (PSTAGE - 2);
    static_assert(keep >= 1 && keep <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%c0)\n\ts_barrier" ::"i"(keep) : "memory");
}
__device__ __forceinline__ void pb_barrier_drain() { asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory"); }

// Value of lane l ^ 32 (the other half of the wave), by a swap of the two halves.
__device__ __forceinline__ float xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    // lanes 0..31 find their partner in the second result, lanes 32..63 in the first
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// One 32-key block's operands of a wave, read from its stage.
struct PbOps {
    u32x4 kk[2], mk[4];
    u32x2 vt[4], bb[4];
};

template <bool MASK>
__device__ __forceinline__ void pb_read(uint32_t st, const uint32_t (&ak)[2], const uint32_t (&av)[4],
                                        const uint32_t (&ab)[4], const uint32_t (&am)[4], PbOps& o) {
    if constexpr (MASK) {
        asm volatile(
            "ds_read_b128 %0, %14\n\t"
            "ds_read_b128 %1, %15\n\t"
            "ds_read_b64_tr_b16 %2, %16\n\t"
            "ds_read_b64_tr_b16 %3, %17\n\t"
            "ds_read_b64_tr_b16 %4, %18\n\t"
            "ds_read_b64_tr_b16 %5, %19\n\t"
            "ds_read_b64 %6, %20\n\t"
            "ds_read_b64 %7, %21\n\t"
            "ds_read_b64 %8, %22\n\t"
            "ds_read_b64 %9, %23\n\t"
            "ds_read_b128 %10, %24\n\t"
            "ds_read_b128 %11, %25\n\t"
            "ds_read_b128 %12, %26\n\t"
            "ds_read_b128 %13, %27\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(o.kk[0]), "=&v"(o.kk[1]), "=&v"(o.vt[0]), "=&v"(o.vt[1]), "=&v"(o.vt[2]), "=&v"(o.vt[3]),
              "=&v"(o.bb[0]), "=&v"(o.bb[1]), "=&v"(o.bb[2]), "=&v"(o.bb[3]), "=&v"(o.mk[0]), "=&v"(o.mk[1]),
              "=&v"(o.mk[2]), "=&v"(o.mk[3])
            : "v"(st + ak[0]), "v"(st + ak[1]), "v"(st + av[0]), "v"(st + av[1]), "v"(st + av[2]), "v"(st + av[3]),
              "v"(st + ab[0]), "v"(st + ab[1]), "v"(st + ab[2]), "v"(st + ab[3]), "v"(st + am[0]), "v"(st + am[1]),
              "v"(st + am[2]), "v"(st + am[3]));
    } else {
        asm volatile(
            "ds_read_b128 %0, %10\n\t"
            "ds_read_b128 %1, %11\n\t"
            "ds_read_b64_tr_b16 %2, %12\n\t"
            "ds_read_b64_tr_b16 %3, %13\n\t"
            "ds_read_b64_tr_b16 %4, %14\n\t"
            "ds_read_b64_tr_b16 %5, %15\n\t"
            "ds_read_b64 %6, %16\n\t"
            "ds_read_b64 %7, %17\n\t"
            "ds_read_b64 %8, %18\n\t"
            "ds_read_b64 %9, %19\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(o.kk[0]), "=&v"(o.kk[1]), "=&v"(o.vt[0]), "=&v"(o.vt[1]), "=&v"(o.vt[2]), "=&v"(o.vt[3]),
              "=&v"(o.bb[0]), "=&v"(o.bb[1]), "=&v"(o.bb[2]), "=&v"(o.bb[3])
            : "v"(st + ak[0]), "v"(st + ak[1]), "v"(st + av[0]), "v"(st + av[1]), "v"(st + av[2]), "v"(st + av[3]),
              "v"(st + ab[0]), "v"(st + ab[1]), "v"(st + ab[2]), "v"(st + ab[3]));
    }
}

// S^T = K Q^T of a block (two products on the matrix cores).
__device__ __forceinline__ f32x16 pb_scores(const PbOps& o, const bf16x8 (&qB)[2]) {
    f32x16 S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, o.kk[0]), qB[0], f32x16{}, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, o.kk[1]), qB[1], S, 0, 0, 0);
}

// The rest of a block from its operands and S: scores, the running reference, p, the row
// sum and O^T += V^T P^T.  TAIL: the block runs past the last key (nk keys exist).
template <bool MASK, bool TAIL>
__device__ __forceinline__ void pb_soft(const PbOps& o, const f32x16& S, int h2, int nk, f32x16& O, float& mref,
                                        float& lsum) {
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    // register r holds key 8 (r / 4) + 4 h2 + r % 4 of the block; z = S / sqrt(D) + bias + mask
    f32x16 x;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int a = r >> 2, e = r & 3;
        const uint32_t word = o.bb[a][e >> 1];
        const float bv = __uint_as_float((e & 1) ? (word & 0xffff0000u) : (word << 16));
        x[r] = fmaf(S[r], kInvSqrtD, bv);
        if constexpr (MASK) x[r] += __uint_as_float(o.mk[a][e]);
    }
    if constexpr (TAIL) {   // the block past the last key: its extra keys drop out
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (8 * (r >> 2) + 4 * h2 + (r & 3) >= nk) x[r] = -INFINITY;
    }
    float mx = x[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, x[r]);
    mx = fmaxf(mx, xor32(mx));
    // The reference moves only when a score exceeds it by more than RESCALE_SLACK:
    // p then stays below 2^8, and the rescale of O and l (and its exponential) is
    // skipped for the whole wave in the usual case.  Sums and the final normalisation
    // use the same reference, so the result is unchanged up to rounding.
    if (__any(mx > mref + RESCALE_SLACK)) {
        const bool grow = mx > mref + RESCALE_SLACK;
        const float mnew = grow ? mx : mref;
        const float alpha = !grow ? 1.0f : (mref == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((mref - mnew) * kLog2e));
        mref = mnew;
        lsum *= alpha;
#pragma unroll
        for (int r = 0; r < 16; ++r) O[r] *= alpha;
    }
    const float sh = mref == -INFINITY ? 0.0f : -mref * kLog2e;
    f32x16 P;
#pragma unroll
    for (int r = 0; r < 16; ++r) P[r] = __builtin_amdgcn_exp2f(fmaf(x[r], kLog2e, sh));
    const bf16x8 pb0 = __builtin_convertvector(__builtin_shufflevector(P, P, 0, 1, 2, 3, 4, 5, 6, 7), bf16x8);
    const bf16x8 pb1 = __builtin_convertvector(__builtin_shufflevector(P, P, 8, 9, 10, 11, 12, 13, 14, 15), bf16x8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const bf16x2 a0 = {pb0[2 * e], pb0[2 * e + 1]};
        const bf16x2 a1 = {pb1[2 * e], pb1[2 * e + 1]};
        lsum = __builtin_amdgcn_fdot2_f32_bf16(a0, ones, lsum, false);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(a1, ones, lsum, false);
    }
    bf16x8 vA[2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
        vA[m] = __builtin_bit_cast(bf16x8, u32x4{o.vt[2 * m][0], o.vt[2 * m][1], o.vt[2 * m + 1][0], o.vt[2 * m + 1][1]});
    O = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vA[0], pb0, O, 0, 0, 0);
    O = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vA[1], pb1, O, 0, 0, 0);
}

template <bool MASK>
__global__ void __launch_bounds__(PTHR, TRI_ATTN_PB_OCC) pair_bias_direct_kernel(Problem p, float* acc_ws, float* m_ws, float* l_ws,
                                                                int n_qb, int n_split, int nblk) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 31, h2 = lane >> 5;
    const int wg = blockIdx.x;
    const int split = wg % n_split, rest = wg / n_split;
    const int qb = rest % n_qb;
    const int64_t bh = rest / n_qb, b = bh / p.H, h = bh % p.H;
    const int N = static_cast<int>(p.N);
    const int64_t HD = p.H * D;
    const int64_t j0 = static_cast<int64_t>(qb) * PQ;
    const int nb0 = static_cast<int>(static_cast<int64_t>(split) * nblk / n_split);
    const int nb1 = static_cast<int>(static_cast<int64_t>(split + 1) * nblk / n_split);

    PbCtx cx;
    {
        cx.N = N;
        cx.key_bytes = HD * 2;
        // K/V piece of wave w: K (w < 2) or V, keys 16 (w % 2) .. +15; lane l carries key
        // 16 (w % 2) + l / 4 and 16-byte slot l % 4, which holds part kv_chunk(key, slot)
        const bool isv = wave >= 2;
        const int half = wave & 1;
        cx.kv = reinterpret_cast<const char*>(static_cast<const __bf16*>(isv ? p.v : p.k) + b * p.N * HD + h * D);
        cx.kv_lds = (isv ? PB_V : PB_K) + half * 1024;
        cx.kv_key = 16 * half + (lane >> 2);
        cx.kv_part = kv_chunk(cx.kv_key, lane & 3);
        cx.kv_off = static_cast<uint32_t>(cx.kv_key * cx.key_bytes + cx.kv_part * 16);
        // bias piece t (pb_bias_key): query row 4 (8 w + t) + l / 16, padded queries reading
        // the last real row
        const uint16_t* bias = static_cast<const uint16_t*>(p.bias);
        cx.bias = reinterpret_cast<const char*>(bias + bh * p.N * p.N);
#pragma unroll
        for (int t = 0; t < PB_BIAS_PER_WAVE; ++t) {
            const int row = 4 * (PB_BIAS_PER_WAVE * wave + t) + (lane >> 4);
            int64_t j = j0 + row;
            j = j < p.N ? j : p.N - 1;
            cx.boff[t] = static_cast<uint32_t>((j * p.N + pb_bias_key(wave, t, lane)) * 2);   // < 2^32: see pair_bias_direct_applies
        }
        cx.mrow = p.mask ? reinterpret_cast<const char*>(p.mask + b * p.N)
                         : reinterpret_cast<const char*>(static_cast<const __bf16*>(p.k) + b * p.N * HD);
    }

    // Q^T operand (B of S^T = K Q^T): query j = j0 + 32 w + c, d = 16 m + 8 h2 .. +7
    const int64_t j = j0 + 32 * wave + c;
    const bool jok = j < p.N;
    const int64_t row = (b * p.N + (jok ? j : 0)) * p.H + h;           // query index of out, lse, states
    bf16x8 qB[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        bf16x8 z = {};
        if (jok) z = *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(p.q) + row * D + 16 * m + 8 * h2);
        qB[m] = z;
    }
    // LDS byte offsets (stage 0) of this lane's reads: K rows (A of S^T), the transposed V
    // reads (A of O^T), its query's bias words and the mask values of its 16 keys
    uint32_t ak[2], av[4], ab[4], am[4];
#pragma unroll
    for (int m = 0; m < 2; ++m) ak[m] = PB_K + c * 64 + kv_chunk(c, 2 * m + h2) * 16;
    {
        const int i = lane & 15, d0 = 16 * ((lane >> 4) & 1) + 4 * (i & 3);
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int sub = 0; sub < 2; ++sub) {
                const int key = 16 * m + 8 * sub + 4 * h2 + (i >> 2);
                av[2 * m + sub] = PB_V + key * 64 + kv_chunk(key, d0 >> 3) * 16 + (d0 & 7) * 2;
            }
    }
    const int brow = 32 * wave + c;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        ab[a] = PB_B + brow * 64 + kv_chunk(brow, a) * 16 + 8 * h2;      // keys 8 a + 4 h2 .. +3
        am[a] = PB_M + (8 * a + 4 * h2) * 4;
    }
    const uint32_t st0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(PB_LPTR(&g_pb[0])));

    f32x16 O = {};
    float mref = -INFINITY, lsum = 0.0f;
    // the Q loads land before the copies start, so that vmcnt counts copies only
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    for (int n = nb0; n < nb0 + PSTAGE - 1 && n < nb1; ++n) pb_stage(cx, n, wave, lane);
    if (nb1 - nb0 >= PSTAGE - 1)
        pb_barrier_keep();
    else
        pb_barrier_drain();
    auto step = [&](int n, auto tail) {
        constexpr bool TAIL = decltype(tail)::value;
        const uint32_t st = st0 + static_cast<uint32_t>(n % PSTAGE) * PB_STAGE_BYTES;
        const bool issue = n + PSTAGE - 1 < nb1;
        if (issue) pb_stage(cx, n + PSTAGE - 1, wave, lane);
        PbOps o;
        pb_read<MASK>(st, ak, av, ab, am, o);
        const f32x16 S = pb_scores(o, qB);
        pb_soft<MASK, TAIL>(o, S, h2, TAIL ? N - BK * n : BK, O, mref, lsum);
        if (issue)
            pb_barrier_keep();
        else
            pb_barrier_drain();
    };
    // only the last block of the call can run past the last key: it leaves the loop, so the
    // loop body has one code path for O
    const int nfull = min(nb1, N / BK);
    for (int n = nb0; n < nfull; ++n) step(n, std::false_type{});
    for (int n = max(nb0, nfull); n < nb1; ++n) step(n, std::true_type{});

    // lanes l and l ^ 32 hold disjoint keys of the same query; register r holds
    // d = 8 (r / 4) + 4 h2 + r % 4
    const float lt = lsum + xor32(lsum);
    if (!jok) return;
    const float mnat = lt > 0.0f ? mref : -INFINITY;
    if (n_split > 1) {
        float* o = acc_ws + (static_cast<int64_t>(split) * p.B * p.N * p.H + row) * D;
#pragma unroll
        for (int a = 0; a < 4; ++a)
            *reinterpret_cast<f32x4*>(o + 8 * a + 4 * h2) = f32x4{O[4 * a], O[4 * a + 1], O[4 * a + 2], O[4 * a + 3]};
        if (h2 == 0) {
            m_ws[static_cast<int64_t>(split) * p.B * p.N * p.H + row] = mnat;
            l_ws[static_cast<int64_t>(split) * p.B * p.N * p.H + row] = lt;
        }
        return;
    }
    float* o = p.out + row * D;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        f32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = lt > 0.0f ? O[4 * a + e] / lt : 0.0f;
        *reinterpret_cast<f32x4*>(o + 8 * a + 4 * h2) = y;
    }
    if (h2 == 0 && p.lse) p.lse[row] = lt > 0.0f ? mnat + logf(lt) : -INFINITY;
}

struct PbLayout {
    int64_t n_qb, nblk, rows;
    int n_split;
    size_t acc, m, l, total;
};
PbLayout pb_layout(const Problem& p) {
    PbLayout L;
    L.n_qb = (p.N + PQ - 1) / PQ;
    L.nblk = (p.N + BK - 1) / BK;
    L.rows = p.B * p.N * p.H;
    const int64_t wgs = p.B * p.H * L.n_qb;
    const int64_t want = FILL_WGS / wgs, most = L.nblk / MIN_SPLIT_BLOCKS;   // one round of resident workgroups
    int64_t s = want < most ? want : most;
    s = s < MAX_SPLIT ? s : MAX_SPLIT;
    L.n_split = s < 2 ? 1 : static_cast<int>(s);
    L.acc = 0;
    L.m = L.acc + static_cast<size_t>(L.n_split * L.rows * D) * 4;
    L.l = L.m + (static_cast<size_t>(L.n_split * L.rows) * 4 + 255) / 256 * 256;
    L.total = L.n_split > 1 ? L.l + static_cast<size_t>(L.n_split * L.rows) * 4 : 0;
    return L;
}

}  // namespace

bool pair_bias_direct_applies(const Problem& p) {
    // the copies address one (b, h) bias slab with 32-bit byte offsets: N * N * 2 < 2^32
    return p.I == 1 && !p.ending && p.st_m == nullptr && p.k0 == 0 && (p.NK == 0 || p.NK == p.N) && p.D == D &&
           p.N % 2 == 0 && p.N <= 46340 && reinterpret_cast<uintptr_t>(p.bias) % 16 == 0;
}

size_t pair_bias_direct_workspace_bytes(const Problem& p) { return pb_layout(p).total; }

hipError_t launch_pair_bias_direct(const Problem& p, void* workspace, hipStream_t stream) {
    const PbLayout L = pb_layout(p);
    const int64_t grid = p.B * p.H * L.n_qb * L.n_split;
    if (grid > 0x7FFFFFFF || p.N > 0x3FFFFFFF || (L.n_split > 1 && workspace == nullptr))
        return hipErrorInvalidConfiguration;
    char* ws = static_cast<char*>(workspace);
    float* acc = L.n_split > 1 ? reinterpret_cast<float*>(ws + L.acc) : nullptr;
    float* m = L.n_split > 1 ? reinterpret_cast<float*>(ws + L.m) : nullptr;
    float* l = L.n_split > 1 ? reinterpret_cast<float*>(ws + L.l) : nullptr;
    if (p.mask)
        hipLaunchKernelGGL(pair_bias_direct_kernel<true>, dim3(static_cast<unsigned>(grid)), dim3(PTHR), 0, stream, p, acc,
                           m, l, static_cast<int>(L.n_qb), L.n_split, static_cast<int>(L.nblk));
    else
        hipLaunchKernelGGL(pair_bias_direct_kernel<false>, dim3(static_cast<unsigned>(grid)), dim3(PTHR), 0, stream, p, acc,
                           m, l, static_cast<int>(L.n_qb), L.n_split, static_cast<int>(L.nblk));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || L.n_split == 1) return e;
    return launch_state_combine(acc, m, l, L.n_split, L.rows, D, p.out, p.lse, stream);
}

}  // namespace tri_attn
