// Backward of starting-node triangle attention (gradients of the definition), fp32
// arithmetic for fp32 or bf16 inputs and any head size D <= 64.
//
// With p_k = exp(s_k - lse) recomputed from the forward's log-sum-exp, per (b, i, j, h):
//     delta = dout . out,   dp_k = dout . v_k,   ds_k = p_k (dp_k - delta)
//     dq_j  = sum_k ds_k k_k / sqrt(D)          (over the keys of the row)
//     dk_k  = sum_j ds_k q_j / sqrt(D),  dv_k = sum_j p_k dout_j   (over the queries)
//     dbias[b,h,j,k] = sum_i ds_k               (over the rows: the bias is shared)
// Three kernels, each owning the sum it produces, so nothing is accumulated with
// atomics and every result is deterministic:
//   1. bwd_dq_kernel:    one thread per query, K, V and the bias block staged in LDS
//   2. bwd_dkdv_kernel:  one thread per key, queries (q, dout, lse, delta) staged in LDS
//   3. bwd_dbias_kernel: one workgroup per 64 x 64 (j, k) tile of one (b, h); each thread
//      holds a 4 x 4 block of pairs and walks the rows i in order, the row's q, dout, k,
//      v, lse and delta staged in LDS.
// A query whose keys are all dropped has lse = -inf and no gradient (p = 0 for it).
#include "launch.h"

#include <cmath>

namespace tri_attn {
namespace {

constexpr int BT = 64;   // threads of the per-query and per-key kernels
constexpr int BKB = 32;  // keys (kernel 1) or queries (kernel 2) per staged block

template <bool BF16>
__device__ __forceinline__ float ld(const void* base, int64_t idx) {
    if constexpr (BF16) {
        return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(base)[idx]) << 16);
    } else {
        return static_cast<const float*>(base)[idx];
    }
}

// probability of a score against the query's log-sum-exp (0 for a query with no key)
__device__ __forceinline__ float prob(float s, float lse) { return lse == -INFINITY ? 0.0f : expf(s - lse); }

// With `wide` set (the bf16 backward's span flags, n_wide per (b, h)), a workgroup works
// only if its (b, h) (blockIdx.z) has a flag set; in dq and dk/dv rows i then run
// blockIdx.y, blockIdx.y + gridDim.y, ...
__device__ __forceinline__ bool skip_bh(const int* wide, int n_wide) {
    if (!wide) return false;
    int any = 0;
    for (int t = 0; t < n_wide; ++t) any |= wide[static_cast<int64_t>(blockIdx.z) * n_wide + t];
    return any == 0;
}

template <bool BF16, int DP>
__global__ void __launch_bounds__(BT) bwd_dq_kernel(BwdProblem p, const int* wide, int n_wide) {
    if (skip_bh(wide, n_wide)) return;
    const int64_t N = p.N, H = p.H, D = p.D, I = p.I;
    const int64_t b = blockIdx.z / H, h = blockIdx.z % H;
    const int64_t j = static_cast<int64_t>(blockIdx.x) * BT + threadIdx.x;
    const int tid = threadIdx.x;
    __shared__ float Ks[BKB][DP + 1];
    __shared__ float Vs[BKB][DP + 1];
    __shared__ float Bs[BT][BKB + 1];
    for (int64_t i = blockIdx.y; i < I; i += gridDim.y) {
        const int64_t row = (b * I + i) * N;      // flat (b, i, 0)

        const bool live = j < N;
        float q[DP], g[DP], dq[DP];
        float delta = 0.0f;
        const float lse = live ? p.lse[(row + j) * H + h] : -INFINITY;
#pragma unroll
        for (int d = 0; d < DP; ++d) {
            const bool ok = live && d < D;
            const int64_t e = ((row + j) * H + h) * D + d;
            q[d] = ok ? ld<BF16>(p.q, e) : 0.0f;
            g[d] = ok ? p.dout[e] : 0.0f;
            delta = fmaf(g[d], ok ? p.out[e] : 0.0f, delta);
            dq[d] = 0.0f;
        }
        const float scale = 1.0f / sqrtf(static_cast<float>(D));
        for (int64_t kb = 0; kb < N; kb += BKB) {
            const int nk = static_cast<int>(N - kb < BKB ? N - kb : BKB);
            __syncthreads();
            for (int e = tid; e < BKB * DP; e += BT) {
                const int kk = e / DP, d = e % DP;
                const bool ok = kk < nk && d < D;
                const int64_t off = ((row + kb + kk) * H + h) * D + d;
                Ks[kk][d] = ok ? ld<BF16>(p.k, off) : 0.0f;
                Vs[kk][d] = ok ? ld<BF16>(p.v, off) : 0.0f;
            }
            const int64_t j0 = static_cast<int64_t>(blockIdx.x) * BT;
            for (int e = tid; e < BT * BKB; e += BT) {
                const int jj = e / BKB, kk = e % BKB;
                float bv = -INFINITY;
                if (kk < nk && j0 + jj < N) {
                    bv = ld<BF16>(p.bias, ((b * H + h) * N + j0 + jj) * N + kb + kk);
                    if (p.mask) bv += p.mask[b * N + kb + kk];
                }
                Bs[jj][kk] = bv;
            }
            __syncthreads();
            for (int kk = 0; kk < nk; ++kk) {
                float s = 0.0f, dp = 0.0f;
#pragma unroll
                for (int d = 0; d < DP; ++d) {
                    s = fmaf(q[d], Ks[kk][d], s);
                    dp = fmaf(g[d], Vs[kk][d], dp);
                }
                const float pk = prob(s * scale + Bs[tid][kk], lse);
                const float ds = pk * (dp - delta);
#pragma unroll
                for (int d = 0; d < DP; ++d) dq[d] = fmaf(ds, Ks[kk][d], dq[d]);
            }
        }
        if (live) {
#pragma unroll
            for (int d = 0; d < DP; ++d)
                if (d < D) p.dq[((row + j) * H + h) * D + d] = dq[d] * scale;
        }
    }   // rows i
}

template <bool BF16, int DP>
__global__ void __launch_bounds__(BT) bwd_dkdv_kernel(BwdProblem p, const int* wide, int n_wide) {
    if (skip_bh(wide, n_wide)) return;
    const int64_t N = p.N, H = p.H, D = p.D, I = p.I;
    const int64_t b = blockIdx.z / H, h = blockIdx.z % H;
    const int64_t k0 = static_cast<int64_t>(blockIdx.x) * BT;
    const int64_t key = k0 + threadIdx.x;
    const int tid = threadIdx.x;
    __shared__ float Qs[BKB][DP + 1];
    __shared__ float Gs[BKB][DP + 1];
    __shared__ float Ls[BKB], Ds[BKB];
    __shared__ float Bs[BKB][BT + 1];
    for (int64_t i = blockIdx.y; i < I; i += gridDim.y) {
        const int64_t row = (b * I + i) * N;

        const bool live = key < N;
        float kv[DP], vv[DP], dk[DP], dv[DP];
#pragma unroll
        for (int d = 0; d < DP; ++d) {
            const bool ok = live && d < D;
            const int64_t e = ((row + key) * H + h) * D + d;
            kv[d] = ok ? ld<BF16>(p.k, e) : 0.0f;
            vv[d] = ok ? ld<BF16>(p.v, e) : 0.0f;
            dk[d] = dv[d] = 0.0f;
        }
        const float mk = (live && p.mask) ? p.mask[b * N + key] : 0.0f;
        const float scale = 1.0f / sqrtf(static_cast<float>(D));
        for (int64_t jb = 0; jb < N; jb += BKB) {
            const int nq = static_cast<int>(N - jb < BKB ? N - jb : BKB);
            __syncthreads();
            for (int e = tid; e < BKB * DP; e += BT) {
                const int jj = e / DP, d = e % DP;
                const bool ok = jj < nq && d < D;
                const int64_t off = ((row + jb + jj) * H + h) * D + d;
                Qs[jj][d] = ok ? ld<BF16>(p.q, off) : 0.0f;
                Gs[jj][d] = ok ? p.dout[off] : 0.0f;
            }
            if (tid < BKB) {
                float lse = -INFINITY, delta = 0.0f;
                if (tid < nq) {
                    const int64_t qi = (row + jb + tid) * H + h;
                    lse = p.lse[qi];
                    for (int d = 0; d < D; ++d) delta = fmaf(p.dout[qi * D + d], p.out[qi * D + d], delta);
                }
                Ls[tid] = lse;
                Ds[tid] = delta;
            }
            for (int e = tid; e < BKB * BT; e += BT) {
                const int jj = e / BT, kk = e % BT;
                Bs[jj][kk] = (jj < nq && k0 + kk < N) ? ld<BF16>(p.bias, ((b * H + h) * N + jb + jj) * N + k0 + kk) : 0.0f;
            }
            __syncthreads();
            for (int jj = 0; jj < nq; ++jj) {
                float s = 0.0f, dp = 0.0f;
#pragma unroll
                for (int d = 0; d < DP; ++d) {
                    s = fmaf(Qs[jj][d], kv[d], s);
                    dp = fmaf(Gs[jj][d], vv[d], dp);
                }
                const float pk = prob(s * scale + Bs[jj][tid] + mk, Ls[jj]);
                const float ds = pk * (dp - Ds[jj]);
#pragma unroll
                for (int d = 0; d < DP; ++d) {
                    dk[d] = fmaf(ds, Qs[jj][d], dk[d]);
                    dv[d] = fmaf(pk, Gs[jj][d], dv[d]);
                }
            }
        }
        if (live) {
#pragma unroll
            for (int d = 0; d < DP; ++d)
                if (d < D) {
                    const int64_t e = ((row + key) * H + h) * D + d;
                    p.dk[e] = dk[d] * scale;
                    p.dv[e] = dv[d];
                }
        }
    }   // rows i
}

constexpr int TB = 64;            // (j, k) tile edge of the dbias kernel
constexpr int TT = 4;             // pairs per thread along j and along k
constexpr int TBT = (TB / TT) * (TB / TT);   // 256 threads

template <bool BF16, int DP>
__global__ void __launch_bounds__(TBT) bwd_dbias_kernel(BwdProblem p, const int* wide, int n_wide) {
    if (skip_bh(wide, n_wide)) return;
    const int64_t N = p.N, H = p.H, D = p.D, I = p.I;
    const int64_t b = blockIdx.z / H, h = blockIdx.z % H;
    const int64_t j0 = static_cast<int64_t>(blockIdx.y) * TB, k0 = static_cast<int64_t>(blockIdx.x) * TB;
    const int tid = threadIdx.x;
    const int tj = tid / (TB / TT), tk = tid % (TB / TT);
    __shared__ float Qs[TB][DP + 1];
    __shared__ float Gs[TB][DP + 1];
    __shared__ float Ks[TB][DP + 1];
    __shared__ float Vs[TB][DP + 1];
    __shared__ float Ls[TB], Ds[TB];

    float bias[TT][TT], acc[TT][TT];
#pragma unroll
    for (int a = 0; a < TT; ++a)
#pragma unroll
        for (int c = 0; c < TT; ++c) {
            const int64_t j = j0 + tj * TT + a, k = k0 + tk * TT + c;
            float bv = -INFINITY;
            if (j < N && k < N) {
                bv = ld<BF16>(p.bias, ((b * H + h) * N + j) * N + k);
                if (p.mask) bv += p.mask[b * N + k];
            }
            bias[a][c] = bv;
            acc[a][c] = 0.0f;
        }
    const float scale = 1.0f / sqrtf(static_cast<float>(D));
    for (int64_t i = 0; i < I; ++i) {
        const int64_t row = (b * I + i) * N;
        __syncthreads();
        for (int e = tid; e < TB * DP; e += TBT) {
            const int r = e / DP, d = e % DP;
            const bool okj = j0 + r < N && d < D, okk = k0 + r < N && d < D;
            const int64_t oj = ((row + j0 + r) * H + h) * D + d, ok = ((row + k0 + r) * H + h) * D + d;
            Qs[r][d] = okj ? ld<BF16>(p.q, oj) : 0.0f;
            Gs[r][d] = okj ? p.dout[oj] : 0.0f;
            Ks[r][d] = okk ? ld<BF16>(p.k, ok) : 0.0f;
            Vs[r][d] = okk ? ld<BF16>(p.v, ok) : 0.0f;
        }
        if (tid < TB) {
            float lse = -INFINITY, delta = 0.0f;
            if (j0 + tid < N) {
                const int64_t qi = (row + j0 + tid) * H + h;
                lse = p.lse[qi];
                for (int d = 0; d < D; ++d) delta = fmaf(p.dout[qi * D + d], p.out[qi * D + d], delta);
            }
            Ls[tid] = lse;
            Ds[tid] = delta;
        }
        __syncthreads();
        float s[TT][TT], dp[TT][TT];
#pragma unroll
        for (int a = 0; a < TT; ++a)
#pragma unroll
            for (int c = 0; c < TT; ++c) s[a][c] = dp[a][c] = 0.0f;
#pragma unroll 4
        for (int d = 0; d < DP; ++d) {
            float qa[TT], ga[TT], kc[TT], vc[TT];
#pragma unroll
            for (int a = 0; a < TT; ++a) {
                qa[a] = Qs[tj * TT + a][d];
                ga[a] = Gs[tj * TT + a][d];
                kc[a] = Ks[tk * TT + a][d];
                vc[a] = Vs[tk * TT + a][d];
            }
#pragma unroll
            for (int a = 0; a < TT; ++a)
#pragma unroll
                for (int c = 0; c < TT; ++c) {
                    s[a][c] = fmaf(qa[a], kc[c], s[a][c]);
                    dp[a][c] = fmaf(ga[a], vc[c], dp[a][c]);
                }
        }
#pragma unroll
        for (int a = 0; a < TT; ++a) {
            const float lse = Ls[tj * TT + a], delta = Ds[tj * TT + a];
#pragma unroll
            for (int c = 0; c < TT; ++c) {
                const float pk = prob(s[a][c] * scale + bias[a][c], lse);
                acc[a][c] = fmaf(pk, dp[a][c] - delta, acc[a][c]);
            }
        }
    }
#pragma unroll
    for (int a = 0; a < TT; ++a)
#pragma unroll
        for (int c = 0; c < TT; ++c) {
            const int64_t j = j0 + tj * TT + a, k = k0 + tk * TT + c;
            if (j < N && k < N) p.dbias[((b * H + h) * N + j) * N + k] = acc[a][c];
        }
}

template <bool BF16, int DP>
hipError_t launch_dp(const BwdProblem& p, hipStream_t stream) {
    const unsigned nb = static_cast<unsigned>((p.N + BT - 1) / BT);
    const dim3 grid(nb, static_cast<unsigned>(p.I), static_cast<unsigned>(p.B * p.H));
    hipLaunchKernelGGL((bwd_dq_kernel<BF16, DP>), grid, dim3(BT), 0, stream, p, nullptr, 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv_kernel<BF16, DP>), grid, dim3(BT), 0, stream, p, nullptr, 0);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned nt = static_cast<unsigned>((p.N + TB - 1) / TB);
    hipLaunchKernelGGL((bwd_dbias_kernel<BF16, DP>), dim3(nt, nt, static_cast<unsigned>(p.B * p.H)), dim3(TBT), 0,
                       stream, p, nullptr, 0);
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_bf(const BwdProblem& p, hipStream_t stream) {
    if (p.D <= 16) return launch_dp<BF16, 16>(p, stream);
    if (p.D <= 32) return launch_dp<BF16, 32>(p, stream);
    return launch_dp<BF16, 64>(p, stream);
}

}  // namespace

hipError_t launch_backward(const BwdProblem& p, bool bf16, hipStream_t stream) {
    if ((p.N + TB - 1) / TB > 65535) return hipErrorInvalidConfiguration;
    return bf16 ? launch_bf<true>(p, stream) : launch_bf<false>(p, stream);
}

hipError_t launch_backward_wide(const BwdProblem& p, const int* wide, int n_wide, hipStream_t stream) {
    if (p.D > 32) return hipErrorInvalidValue;
    // usually no (b, h) is flagged: a small grid (rows walked in up to 64 slots) keeps the
    // launch cheap when every workgroup returns
    const unsigned nb = static_cast<unsigned>((p.N + BT - 1) / BT);
    const dim3 grid(nb, static_cast<unsigned>(p.I < 64 ? p.I : 64), static_cast<unsigned>(p.B * p.H));
    hipLaunchKernelGGL((bwd_dq_kernel<true, 32>), grid, dim3(BT), 0, stream, p, wide, n_wide);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv_kernel<true, 32>), grid, dim3(BT), 0, stream, p, wide, n_wide);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const unsigned nt = static_cast<unsigned>((p.N + TB - 1) / TB);
    hipLaunchKernelGGL((bwd_dbias_kernel<true, 32>), dim3(nt, nt, static_cast<unsigned>(p.B * p.H)), dim3(TBT), 0,
                       stream, p, wide, n_wide);
    return hipGetLastError();
}

}  // namespace tri_attn
