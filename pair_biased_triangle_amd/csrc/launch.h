// Internal declarations shared by the host entry points and the kernel translation units
// of libtri_attn.so.  Not part of the public C ABI (that is include/tri_attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace tri_attn {

// One call's problem, already validated by the entry point.
//
// Orientation.  The kernels work on "lines": attention problems that share the key axis
// with their queries.  Starting node: line r is row i, queries are columns j, keys the
// entries (i, k) of the same row, bias[b, h, j, k].  Ending node: line r is column j,
// queries are rows i, keys the entries (k, j) of the same column, bias[b, h, k, i] (the
// bias transposed: "Fold-CP", Figure 2(a), cross-axis transpose).  Both use the same
// kernels with different strides (Strides below); the ending node needs I == N.
struct Problem {
    const void* q;
    const void* k;
    const void* v;
    const void* bias;
    const float* mask;   // may be null
    float* out;          // normalised output, or the unnormalised accumulator (state mode)
    int64_t B, H, I, N, D;
    int32_t T;           // key tiles (ring steps) over the key range
    int64_t k0 = 0;      // key range [k0, k0 + NK) (one ring step's keys in state mode)
    int64_t NK = 0;      //   NK == 0 means all N keys
    bool ending = false; // ending-node orientation
    float* lse = nullptr;   // optional [B, I, N, H]: natural-log normaliser of each query
    float* st_m = nullptr;  // state mode when non-null: reference (natural-log units) ...
    float* st_l = nullptr;  //   ... and normaliser of each query; out gets the accumulator
    bool update = false;    // state mode: fold into the state already in out, st_m, st_l
    float* fin = nullptr;   // with update: write the folded result here as the final output
                            // (fin = acc / l, lse = m + ln l) and leave the state untouched
    __host__ __device__ int64_t nkeys() const { return NK > 0 ? NK : N; }
};

// Element strides of q, k, v and out ([B, I, N, H, D] storage) for a line r, a query
// and a key; lse, st_m and st_l use the same offsets divided by D.
struct Strides {
    int64_t batch, line, query, key;
};
__host__ __device__ inline Strides strides_of(const Problem& p) {
    const int64_t HD = p.H * p.D;
    if (p.ending) return Strides{p.N * p.N * HD, HD, p.N * HD, p.N * HD};
    return Strides{p.I * p.N * HD, p.N * HD, HD, HD};
}

// Backward (starting node): gradients for the upstream gradient dout, from the forward's
// out and lse.  dq, dk, dv like q; dbias [B, H, N, N] summed over the I rows held.
struct BwdProblem {
    const void* q;
    const void* k;
    const void* v;
    const void* bias;
    const float* mask;   // may be null
    const float* out;
    const float* lse;
    const float* dout;
    float* dq;
    float* dk;
    float* dv;
    float* dbias;
    int64_t B, H, I, N, D;
};
hipError_t launch_backward(const BwdProblem& p, bool bf16, hipStream_t stream);
// dq, dk, dv and dbias of the fp32 kernels (bf16 inputs), only for the (b, h) whose n_wide
// flags wide[(b*H + h) * n_wide + t] include a nonzero one; every other workgroup returns
// at once.
hipError_t launch_backward_wide(const BwdProblem& p, const int* wide, int n_wide, hipStream_t stream);

// bf16 inputs, D == 32: matrix-core forward.  `workspace` (16-byte aligned, at least
// bf16_workspace_bytes(p) bytes) receives its fp16 bias image and per-query references.
size_t bf16_workspace_bytes(const Problem& p);
hipError_t launch_bf16_mfma(const Problem& p, void* workspace, hipStream_t stream);

// The forward's bias prepass on its own (starting orientation, the call's whole key range),
// for the backward: into `workspace` (bytes long, 256-byte aligned) the fp16 image of
// (bias + mask - r_j) * log2(e), one cols x 32 tile per (b, h, column block jb, key block n)
// at ((b*H + h) * n_jb + jb) * nblk + n (row jj = query jb*cols + jj, its 32 keys in the
// matrix-core register order, 16-byte parts swizzled by row), then r_j as fp32 at
// ref_off + ((b*H + h) * nqp + j) * 4 (nqp = n_jb * cols), then one int per (b, h, jb) at
// wide_off + ((b*H + h) * n_jb + jb) * 4, nonzero when the column block holds a finite
// image value more than the image's span below r_j (its fp16 rounding would exceed the
// bound the matrix-core kernels assume; such blocks go to the fp32 kernels).
struct Prepass16 {
    size_t ref_off, wide_off, bytes;
    int64_t n_jb, nqp, nblk;
    int cols;
};
Prepass16 prepass16_layout(const Problem& p);
hipError_t launch_prepass16(const Problem& p, void* workspace, hipStream_t stream);

// The fp32 bias image of the backward kernels.  Layout: per (b, h), column block jb of IMG_BJ query columns
// and key block n (keys 32n .. 32n + 31 of the call's range), one IMG_BJ x IMG_BK
// fp32 tile at img + ((b*H + h) * n_jb + jb) * nblk + n) * IMG_BJ * IMG_BK holding
// (bias + mask) * sqrt(D), -inf past the block's last key; row jj (a query column) has its
// 16-byte chunk `part` (keys 4*part .. 4*part+3) at position img_chunk(jj, part).
constexpr int IMG_BJ = 128;
constexpr int IMG_BK = 32;
__host__ __device__ constexpr int img_chunk(int jj, int part) { return part ^ (jj & 7); }
int64_t bias_image_blocks(const Problem& p);   // nblk
size_t bias_image_bytes(const Problem& p);
hipError_t launch_bias_image(const Problem& p, float* img, hipStream_t stream);

// Backward on matrix cores (bf16, D == 32).  Workspace: the forward's prepass (fp16 image,
// references, span flags), the transposed fp16 image, dout rounded to bf16, delta = dout .
// out per query and the per-row statistics; bwd_mfma_workspace_bytes() bytes.
size_t bwd_mfma_workspace_bytes(const BwdProblem& p);
hipError_t launch_backward_mfma(const BwdProblem& p, void* workspace, hipStream_t stream);

// Any D <= 64, fp32 or bf16 inputs: plain fp32 kernel.
hipError_t launch_general(const Problem& p, bool bf16, hipStream_t stream);
// The same kernel (bf16 inputs) restricted to the query column blocks of `cols` columns
// whose flag wide[(b*H + h) * n_jb + jb] is nonzero (n_jb = ceil(N / cols)); every other
// workgroup returns at once.  cols is a multiple of 64.
hipError_t launch_general_wide(const Problem& p, const int* wide, int cols, hipStream_t stream);

// Partial softmax states (state mode above), rows = B * I * N * H queries of D values:
// (acc, m, l) <- merge((acc, m, l), (acc_t, m_t, l_t)), and out = acc / l, lse = m + ln l.
hipError_t launch_state_merge(float* acc, float* m, float* l, const float* acc_t, const float* m_t,
                              const float* l_t, int64_t rows, int64_t D, hipStream_t stream);
hipError_t launch_state_finalize(const float* acc, const float* m, const float* l, float* out, float* lse,
                                 int64_t rows, int64_t D, hipStream_t stream);
// n_split partial states stored one after another ([n_split][rows][D], [n_split][rows])
// joined into out = acc / l and lse = m + ln l of their merge (n_split <= 16).
hipError_t launch_state_combine(const float* acc, const float* m, const float* l, int n_split, int64_t rows,
                                int64_t D, float* out, float* lse, hipStream_t stream);


// The allocation-free entry point's workspace: a static device array of
// static_scratch_bytes() bytes; static_scratch() returns its address on the current device
// (looked up once per device).
size_t static_scratch_bytes();
hipError_t static_scratch(void** out);

// Start of key tile t when N keys are cut into T near-equal contiguous tiles
// (the first N mod T tiles hold one key more).
__host__ __device__ inline int64_t tile_start(int64_t t, int64_t N, int64_t T) {
    const int64_t base = N / T, extra = N % T;
    return t * base + (t < extra ? t : extra);
}

}  // namespace tri_attn
