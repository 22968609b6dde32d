// Merge and finalisation of partial softmax states, the step that joins ring steps
// ("Fold-CP", Figure 2(a) and (c): key tiles computed separately are combined by the
// tiled-softmax merge).  A state of one query is (acc[D], m, l): the accumulator
// sum_k e^(s_k - m) v_k, a reference m in natural-log units and the normaliser
// sum_k e^(s_k - m).  Any finite reference gives the same merged result; a state with
// l == 0 (no finite score) is the identity of the merge.
//
// One thread per query; D consecutive floats per query, so a wave covers 64 * D * 4
// contiguous bytes.  Both kernels are HBM-bound (they read and write every state once).
#include "launch.h"

#include <cmath>

namespace tri_attn {
namespace {

constexpr int ST_THR = 256;

__global__ void __launch_bounds__(ST_THR) state_merge_kernel(float* acc, float* m, float* l, const float* acc_t,
                                                             const float* m_t, const float* l_t, int64_t rows,
                                                             int D) {
    const int64_t q = static_cast<int64_t>(blockIdx.x) * ST_THR + threadIdx.x;
    if (q >= rows) return;
    const float la = l[q], lb = l_t[q];
    if (!(lb > 0.0f)) return;                 // incoming tile holds no finite score
    float* a = acc + q * D;
    const float* at = acc_t + q * D;
    if (!(la > 0.0f)) {                       // running state empty: take the tile's state
        for (int d = 0; d < D; ++d) a[d] = at[d];
        m[q] = m_t[q];
        l[q] = lb;
        return;
    }
    const float ma = m[q], mb = m_t[q];
    const float mm = fmaxf(ma, mb);
    const float alpha = expf(ma - mm), beta = expf(mb - mm);
    for (int d = 0; d < D; ++d) a[d] = alpha * a[d] + beta * at[d];
    m[q] = mm;
    l[q] = alpha * la + beta * lb;
}

__global__ void __launch_bounds__(ST_THR) state_finalize_kernel(const float* acc, const float* m, const float* l,
                                                                float* out, float* lse, int64_t rows, int D) {
    const int64_t q = static_cast<int64_t>(blockIdx.x) * ST_THR + threadIdx.x;
    if (q >= rows) return;
    const float lq = l[q];
    const bool some = lq > 0.0f;
    for (int d = 0; d < D; ++d) out[q * D + d] = some ? acc[q * D + d] / lq : 0.0f;
    if (lse) lse[q] = some ? m[q] + logf(lq) : -INFINITY;
}

}  // namespace

hipError_t launch_state_merge(float* acc, float* m, float* l, const float* acc_t, const float* m_t,
                              const float* l_t, int64_t rows, int64_t D, hipStream_t stream) {
    const int64_t blocks = (rows + ST_THR - 1) / ST_THR;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(state_merge_kernel, dim3(static_cast<unsigned>(blocks)), dim3(ST_THR), 0, stream, acc, m, l,
                       acc_t, m_t, l_t, rows, static_cast<int>(D));
    return hipGetLastError();
}

hipError_t launch_state_finalize(const float* acc, const float* m, const float* l, float* out, float* lse,
                                 int64_t rows, int64_t D, hipStream_t stream) {
    const int64_t blocks = (rows + ST_THR - 1) / ST_THR;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(state_finalize_kernel, dim3(static_cast<unsigned>(blocks)), dim3(ST_THR), 0, stream, acc, m,
                       l, out, lse, rows, static_cast<int>(D));
    return hipGetLastError();
}

}  // namespace tri_attn
