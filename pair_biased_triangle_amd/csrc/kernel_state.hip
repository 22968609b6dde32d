// Merge and finalisation of partial softmax states, the step that joins ring steps
// ("Fold-CP", Figure 2(a) and (c): key tiles computed separately are combined by the
// tiled-softmax merge).  A state of one query is (acc[D], m, l): the accumulator
// sum_k e^(s_k - m) v_k, a reference m in natural-log units and the normaliser
// sum_k e^(s_k - m).  Any finite reference gives the same merged result; a state with
// l == 0 (no finite score) is the identity of the merge.
//
// Both kernels are HBM-bound: they read and write every state once, with coalesced
// accesses (see below).
#include "launch.h"

#include <cmath>

namespace tri_attn {
namespace {

constexpr int ST_THR = 256;   // threads per workgroup
constexpr int ST_Q = 64;      // queries per workgroup
typedef float f32x4 __attribute__((ext_vector_type(4)));

// VEC: D % 4 == 0 and the accumulators 16-byte aligned, so four consecutive floats belong
// to one query and each lane moves 16 bytes per access (a wave 1 KB); else one float.

// A workgroup owns ST_Q consecutive queries.  Their per-query factors are formed once in
// LDS; then every thread walks the workgroup's ST_Q * D contiguous floats with a stride
// of ST_THR, so each wave reads and writes 256 consecutive bytes per access.  The per-query
// values m and l are read and rewritten by the same thread, on either side of the barriers.
template <bool VEC>
__global__ void __launch_bounds__(ST_THR) state_merge_kernel(float* acc, float* m, float* l, const float* acc_t,
                                                             const float* m_t, const float* l_t, int64_t rows,
                                                             int D) {
    __shared__ float fa[ST_Q], fb[ST_Q];
    const int64_t q0 = static_cast<int64_t>(blockIdx.x) * ST_Q;
    const int nq = static_cast<int>(rows - q0 < ST_Q ? rows - q0 : ST_Q);
    const int tid = threadIdx.x;
    float mm = 0.0f, ll = 0.0f;
    if (tid < nq) {
        const int64_t q = q0 + tid;
        const float la = l[q], lb = l_t[q];
        float alpha, beta;
        if (!(lb > 0.0f)) {                   // incoming tile holds no finite score: keep the state
            alpha = 1.0f;
            beta = 0.0f;
            mm = m[q];
            ll = la;
        } else if (!(la > 0.0f)) {            // running state empty: take the tile's state
            alpha = 0.0f;
            beta = 1.0f;
            mm = m_t[q];
            ll = lb;
        } else {
            const float ma = m[q], mb = m_t[q];
            mm = fmaxf(ma, mb);
            alpha = expf(ma - mm);
            beta = expf(mb - mm);
            ll = alpha * la + beta * lb;
        }
        fa[tid] = alpha;
        fb[tid] = beta;
    }
    __syncthreads();
    const int64_t e0 = q0 * D;
    const int ne = nq * D;
    if constexpr (VEC) {
        f32x4* a4 = reinterpret_cast<f32x4*>(acc + e0);
        const f32x4* t4 = reinterpret_cast<const f32x4*>(acc_t + e0);
        for (int e = tid; e < ne / 4; e += ST_THR) {
            const int qq = 4 * e / D;
            const float a = fa[qq], b = fb[qq];
            if (b == 0.0f) continue;          // an empty tile leaves the accumulator as it is
            const f32x4 t = t4[e];
            f32x4 x = a == 0.0f ? f32x4{} : a4[e];
#pragma unroll
            for (int c = 0; c < 4; ++c) x[c] = a == 0.0f ? b * t[c] : a * x[c] + b * t[c];
            a4[e] = x;
        }
    } else {
        for (int e = tid; e < ne; e += ST_THR) {
            const int qq = e / D;
            const float a = fa[qq], b = fb[qq];
            if (b == 0.0f) continue;          // an empty tile leaves the accumulator as it is
            const float bt = b * acc_t[e0 + e];
            acc[e0 + e] = a == 0.0f ? bt : a * acc[e0 + e] + bt;
        }
    }
    if (tid < nq) {
        m[q0 + tid] = mm;
        l[q0 + tid] = ll;
    }
}

template <bool VEC>
__global__ void __launch_bounds__(ST_THR) state_finalize_kernel(const float* acc, const float* m, const float* l,
                                                                float* out, float* lse, int64_t rows, int D) {
    __shared__ float inv[ST_Q];
    const int64_t q0 = static_cast<int64_t>(blockIdx.x) * ST_Q;
    const int nq = static_cast<int>(rows - q0 < ST_Q ? rows - q0 : ST_Q);
    const int tid = threadIdx.x;
    if (tid < nq) {
        const float lq = l[q0 + tid];
        const bool some = lq > 0.0f;
        inv[tid] = lq;
        if (lse) lse[q0 + tid] = some ? m[q0 + tid] + logf(lq) : -INFINITY;
    }
    __syncthreads();
    const int64_t e0 = q0 * D;
    const int ne = nq * D;
    if constexpr (VEC) {
        const f32x4* a4 = reinterpret_cast<const f32x4*>(acc + e0);
        f32x4* o4 = reinterpret_cast<f32x4*>(out + e0);
        for (int e = tid; e < ne / 4; e += ST_THR) {
            const float lq = inv[4 * e / D];
            const f32x4 x = a4[e];
            f32x4 y;
#pragma unroll
            for (int c = 0; c < 4; ++c) y[c] = lq > 0.0f ? x[c] / lq : 0.0f;
            o4[e] = y;
        }
    } else {
        for (int e = tid; e < ne; e += ST_THR) {
            const float lq = inv[e / D];
            out[e0 + e] = lq > 0.0f ? acc[e0 + e] / lq : 0.0f;
        }
    }
}

// Join n_split partial states stored split after split (acc [n_split][rows][D], m and l
// [n_split][rows]) into out = acc / l and lse = m + ln l of the merged state, in one pass:
// the merge rule applied to all splits at once, m* = max m_s, l = sum e^(m_s - m*) l_s.
// A thread owns 4 (VEC) or 1 consecutive elements of one query and issues every load it
// needs (each split's m, l and acc elements) before using any, so the join costs one
// memory round trip; the threads of a query repeat its m and l loads (cache hits).
constexpr int MAX_COMBINE = 16;
constexpr int CB_THR = 256;
template <bool VEC>
__global__ void __launch_bounds__(CB_THR) state_combine_kernel(const float* acc, const float* m, const float* l,
                                                               int n_split, int64_t rows, int D, float* out,
                                                               float* lse) {
    constexpr int W = VEC ? 4 : 1;
    const int per_q = D / W;                          // threads per query (D % W == 0)
    const int64_t t = static_cast<int64_t>(blockIdx.x) * CB_THR + threadIdx.x;
    if (t >= rows * per_q) return;
    const int64_t q = t / per_q;
    const int part = static_cast<int>(t - q * per_q);
    float ms[MAX_COMBINE], ls[MAX_COMBINE];
    float a[MAX_COMBINE][W];
#pragma unroll
    for (int s = 0; s < MAX_COMBINE; ++s) {
        if (s < n_split) {
            ms[s] = m[s * rows + q];
            ls[s] = l[s * rows + q];
            const float* src = acc + (s * rows + q) * D + part * W;
            if constexpr (VEC) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(src);
#pragma unroll
                for (int c = 0; c < W; ++c) a[s][c] = v[c];
            } else {
                a[s][0] = *src;
            }
        } else {
            ms[s] = -INFINITY;
            ls[s] = 0.0f;
#pragma unroll
            for (int c = 0; c < W; ++c) a[s][c] = 0.0f;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int s = 0; s < MAX_COMBINE; ++s)
        if (ls[s] > 0.0f) mx = fmaxf(mx, ms[s]);
    float lt = 0.0f, x[W] = {};
#pragma unroll
    for (int s = 0; s < MAX_COMBINE; ++s) {
        const float f = ls[s] > 0.0f ? expf(ms[s] - mx) : 0.0f;
        lt += f * ls[s];
#pragma unroll
        for (int c = 0; c < W; ++c) x[c] = fmaf(f, a[s][c], x[c]);
    }
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    float* dst = out + q * D + part * W;
    if constexpr (VEC) {
        *reinterpret_cast<f32x4*>(dst) = f32x4{x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv};
    } else {
        *dst = x[0] * inv;
    }
    if (lse && part == 0) lse[q] = lt > 0.0f ? mx + logf(lt) : -INFINITY;
}

}  // namespace

namespace {
bool vec_ok(int64_t D, const void* a, const void* b) {
    return D % 4 == 0 && reinterpret_cast<uintptr_t>(a) % 16 == 0 && reinterpret_cast<uintptr_t>(b) % 16 == 0;
}
}  // namespace

hipError_t launch_state_merge(float* acc, float* m, float* l, const float* acc_t, const float* m_t,
                              const float* l_t, int64_t rows, int64_t D, hipStream_t stream) {
    const int64_t blocks = (rows + ST_Q - 1) / ST_Q;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    if (vec_ok(D, acc, acc_t))
        hipLaunchKernelGGL(state_merge_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(ST_THR), 0, stream, acc,
                           m, l, acc_t, m_t, l_t, rows, static_cast<int>(D));
    else
        hipLaunchKernelGGL(state_merge_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(ST_THR), 0, stream, acc,
                           m, l, acc_t, m_t, l_t, rows, static_cast<int>(D));
    return hipGetLastError();
}

hipError_t launch_state_finalize(const float* acc, const float* m, const float* l, float* out, float* lse,
                                 int64_t rows, int64_t D, hipStream_t stream) {
    const int64_t blocks = (rows + ST_Q - 1) / ST_Q;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    if (vec_ok(D, acc, out))
        hipLaunchKernelGGL(state_finalize_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(ST_THR), 0, stream,
                           acc, m, l, out, lse, rows, static_cast<int>(D));
    else
        hipLaunchKernelGGL(state_finalize_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(ST_THR), 0, stream,
                           acc, m, l, out, lse, rows, static_cast<int>(D));
    return hipGetLastError();
}

hipError_t launch_state_combine(const float* acc, const float* m, const float* l, int n_split, int64_t rows,
                                int64_t D, float* out, float* lse, hipStream_t stream) {
    if (D < 1 || n_split < 1 || n_split > MAX_COMBINE) return hipErrorInvalidConfiguration;
    const int64_t threads = rows * (vec_ok(D, acc, out) ? D / 4 : D);
    const int64_t blocks = (threads + CB_THR - 1) / CB_THR;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    if (blocks == 0) return hipSuccess;
    // every split's accumulator block is rows * D floats: 16-byte aligned when D % 4 == 0
    if (vec_ok(D, acc, out))
        hipLaunchKernelGGL(state_combine_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(CB_THR), 0, stream,
                           acc, m, l, n_split, rows, static_cast<int>(D), out, lse);
    else
        hipLaunchKernelGGL(state_combine_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(CB_THR), 0, stream,
                           acc, m, l, n_split, rows, static_cast<int>(D), out, lse);
    return hipGetLastError();
}

}  // namespace tri_attn
