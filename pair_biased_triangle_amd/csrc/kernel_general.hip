// Plain fp32 triangle-attention kernel for any head size D <= 64 and fp32 or bf16 inputs.
//
// One workgroup covers 64 queries of one (b, line, h) -- a line is a row i for the
// starting node and a column j for the ending node; each thread owns one query
// and keeps its q vector, running maximum, normaliser and fp32 accumulator in registers
// (online softmax over key blocks; "Fold-CP", Figure 2(a): tiled-softmax merge).  Key
// blocks of 32 never straddle a ring-step tile, so each tile is folded into the running
// state exactly as one ring step would be.  K, V and the bias block (with the additive
// key mask folded in) are staged through LDS.  The same kernel writes the log-sum-exp of
// each query, or a key range's unnormalised partial state (accumulator, running maximum,
// normaliser) for the split-tile entry points.
#include "launch.h"

#include <cmath>

namespace tri_attn {
namespace {

constexpr int GJ = 64;  // queries per workgroup, one per thread
constexpr int GK = 32;  // keys per block

template <bool BF16>
__device__ __forceinline__ float load_elem(const void* base, int64_t idx) {
    if constexpr (BF16) {
        const uint32_t u = static_cast<uint32_t>(static_cast<const uint16_t*>(base)[idx]) << 16;
        return __uint_as_float(u);
    } else {
        return static_cast<const float*>(base)[idx];
    }
}

template <int DP>
struct Tiles {
    float K[GK][DP + 1];
    float V[GK][DP + 1];
    float B[GJ][GK + 1];
};

// One line r of the workgroup's 64 queries.
template <bool BF16, int DP>
__device__ void general_line(const Problem& p, const Strides& st, int64_t r, Tiles<DP>& sh) {
    const int64_t N = p.N, H = p.H, D = p.D, NK = p.nkeys();
    const int64_t b = blockIdx.z / H, h = blockIdx.z % H;
    const int64_t j0 = static_cast<int64_t>(blockIdx.x) * GJ;
    const int tid = threadIdx.x;
    const int64_t j = j0 + tid;                   // this thread's query
    const int64_t line = b * st.batch + r * st.line + h * D;   // element offset of (b, line r, head h)
    float (&Ks)[GK][DP + 1] = sh.K;
    float (&Vs)[GK][DP + 1] = sh.V;
    float (&Bs)[GJ][GK + 1] = sh.B;

    float q[DP], acc[DP];
#pragma unroll
    for (int d = 0; d < DP; ++d) {
        q[d] = (j < N && d < D) ? load_elem<BF16>(p.q, line + j * st.query + d) : 0.0f;
        acc[d] = 0.0f;
    }
    const float scale = 1.0f / sqrtf(static_cast<float>(D));
    float m = -INFINITY, l = 0.0f;

    for (int t = 0; t < p.T; ++t) {
        const int64_t ks = p.k0 + tile_start(t, NK, p.T), ke = p.k0 + tile_start(t + 1, NK, p.T);
        for (int64_t kb = ks; kb < ke; kb += GK) {
            const int nk = static_cast<int>(ke - kb < GK ? ke - kb : GK);
            __syncthreads();
            for (int e = tid; e < GK * DP; e += GJ) {
                const int kk = e / DP, d = e % DP;
                const bool ok = kk < nk && d < D;
                const int64_t off = line + (kb + kk) * st.key + d;
                Ks[kk][d] = ok ? load_elem<BF16>(p.k, off) : 0.0f;
                Vs[kk][d] = ok ? load_elem<BF16>(p.v, off) : 0.0f;
            }
            for (int e = tid; e < GJ * GK; e += GJ) {
                const int jj = e / GK, kk = e % GK;
                const int64_t jg = j0 + jj, key = kb + kk;
                float bv = -INFINITY;
                if (kk < nk && jg < N) {
                    const int64_t bi = p.ending ? ((b * H + h) * N + key) * N + jg : ((b * H + h) * N + jg) * N + key;
                    bv = load_elem<BF16>(p.bias, bi);
                    if (p.mask) bv += p.mask[b * N + key];
                }
                Bs[jj][kk] = bv;
            }
            __syncthreads();

            float s[GK];
            float mx = -INFINITY;
#pragma unroll
            for (int kk = 0; kk < GK; ++kk) {
                float dot = 0.0f;
#pragma unroll
                for (int d = 0; d < DP; ++d) dot = fmaf(q[d], Ks[kk][d], dot);
                s[kk] = dot * scale + Bs[tid][kk];
                mx = fmaxf(mx, s[kk]);
            }
            if (mx == -INFINITY) continue;  // every key of the block dropped for this query
            const float mnew = fmaxf(m, mx);
            const float alpha = expf(m - mnew);  // 0 while m is still -inf
            l *= alpha;
#pragma unroll
            for (int d = 0; d < DP; ++d) acc[d] *= alpha;
#pragma unroll
            for (int kk = 0; kk < GK; ++kk) {
                const float pk = expf(s[kk] - mnew);
                l += pk;
#pragma unroll
                for (int d = 0; d < DP; ++d) acc[d] = fmaf(pk, Vs[kk][d], acc[d]);
            }
            m = mnew;
        }
    }
    if (j < N) {
        const int64_t qo = line + j * st.query;   // element offset of this query's D values
        const int64_t so = qo / D;                // offset in the [B, I, N, H] per-query arrays
        float* o = p.out + qo;
        if (p.st_m && p.update && p.fin) {        // final step: the folded state, normalised
            const float m0 = p.st_m[so], l0 = p.st_l[so];
            float a0 = 1.0f, a1 = 0.0f, mm = m0;   // empty range: the old state as it is
            if (l > 0.0f) {
                a0 = 0.0f;
                a1 = 1.0f;
                mm = m;
                if (l0 > 0.0f) {
                    mm = fmaxf(m0, m);
                    a0 = expf(m0 - mm);
                    a1 = expf(m - mm);
                }
            }
            const float ln = a0 * l0 + a1 * l;
            float* f = p.fin + qo;
#pragma unroll
            for (int d = 0; d < DP; ++d)
                if (d < D) {
                    const float x = a0 == 0.0f ? a1 * acc[d] : fmaf(a0, o[d], a1 * acc[d]);
                    f[d] = ln > 0.0f ? x / ln : 0.0f;
                }
            if (p.lse) p.lse[so] = ln > 0.0f ? mm + logf(ln) : -INFINITY;
            return;
        }
        if (p.st_m && p.update) {                 // fold into the running state (merge rule)
            const float m0 = p.st_m[so], l0 = p.st_l[so];
            if (l > 0.0f) {
                float a0 = 0.0f, a1 = 1.0f, mm = m;
                if (l0 > 0.0f) {
                    mm = fmaxf(m0, m);
                    a0 = expf(m0 - mm);
                    a1 = expf(m - mm);
                }
#pragma unroll
                for (int d = 0; d < DP; ++d)
                    if (d < D) o[d] = a0 == 0.0f ? a1 * acc[d] : fmaf(a0, o[d], a1 * acc[d]);
                p.st_m[so] = mm;
                p.st_l[so] = a0 * l0 + a1 * l;
            }
        } else if (p.st_m) {                      // partial state: unnormalised accumulator
#pragma unroll
            for (int d = 0; d < DP; ++d)
                if (d < D) o[d] = acc[d];
            p.st_m[so] = m;
            p.st_l[so] = l;
        } else {
            const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
            for (int d = 0; d < DP; ++d)
                if (d < D) o[d] = acc[d] * inv;
        }
        if (p.lse) p.lse[so] = l > 0.0f ? m + logf(l) : -INFINITY;
    }
}

// Lines blockIdx.y, blockIdx.y + gridDim.y, ...  With `wide` set, only workgroups whose
// query column block (of wide_cols columns) is flagged do any work.
template <bool BF16, int DP>
__global__ void __launch_bounds__(GJ) general_kernel(Problem p, Strides st, const int* wide, int wide_cols) {
    if (wide) {
        const int64_t n_jb = (p.N + wide_cols - 1) / wide_cols;
        const int64_t jb = static_cast<int64_t>(blockIdx.x) * GJ / wide_cols;
        if (!wide[static_cast<int64_t>(blockIdx.z) * n_jb + jb]) return;
    }
    __shared__ Tiles<DP> sh;
    const int64_t lines = p.ending ? p.N : p.I;   // rows i, or columns j for the ending node (I == N)
    for (int64_t r = blockIdx.y; r < lines; r += gridDim.y) {
        __syncthreads();                          // the previous line's last reads of the tiles
        general_line<BF16, DP>(p, st, r, sh);
    }
}

template <bool BF16>
hipError_t launch_dp(const Problem& p, const int* wide, int wide_cols, unsigned line_slots, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>((p.N + GJ - 1) / GJ), line_slots, static_cast<unsigned>(p.B * p.H));
    const Strides st = strides_of(p);
    if (p.D <= 16)
        hipLaunchKernelGGL((general_kernel<BF16, 16>), grid, dim3(GJ), 0, stream, p, st, wide, wide_cols);
    else if (p.D <= 32)
        hipLaunchKernelGGL((general_kernel<BF16, 32>), grid, dim3(GJ), 0, stream, p, st, wide, wide_cols);
    else
        hipLaunchKernelGGL((general_kernel<BF16, 64>), grid, dim3(GJ), 0, stream, p, st, wide, wide_cols);
    return hipGetLastError();
}

int64_t lines_of(const Problem& p) { return p.ending ? p.N : p.I; }

}  // namespace

hipError_t launch_general(const Problem& p, bool bf16, hipStream_t stream) {
    // one workgroup per (64 queries, line, (b, h))
    const unsigned slots = static_cast<unsigned>(lines_of(p));
    return bf16 ? launch_dp<true>(p, nullptr, GJ, slots, stream) : launch_dp<false>(p, nullptr, GJ, slots, stream);
}

hipError_t launch_general_wide(const Problem& p, const int* wide, int cols, hipStream_t stream) {
    if (cols % GJ != 0) return hipErrorInvalidValue;
    // Usually no block is flagged, so the grid is kept small (each workgroup walks up to
    // 64 line slots' worth of lines) to make the launch cheap when every workgroup returns.
    constexpr int64_t kLineSlots = 64;
    const int64_t lines = lines_of(p);
    return launch_dp<true>(p, wide, cols, static_cast<unsigned>(lines < kLineSlots ? lines : kLineSlots), stream);
}

}  // namespace tri_attn
