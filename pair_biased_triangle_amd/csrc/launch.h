// Internal declarations shared by the host entry points and the kernel translation units
// of libtri_attn.so.  Not part of the public C ABI (that is include/tri_attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace tri_attn {

// One call's problem, already validated by the entry point.
struct Problem {
    const void* q;
    const void* k;
    const void* v;
    const void* bias;
    const float* mask;   // may be null
    float* out;
    int64_t B, H, I, N, D;
    int32_t T;           // key tiles (ring steps)
};

// bf16 inputs, D == 32: matrix-core kernels.  `workspace` (16-byte aligned, at least
// bf16_workspace_bytes(p) bytes) receives the converted bias image.
size_t bf16_workspace_bytes(const Problem& p);
hipError_t launch_bf16_mfma(const Problem& p, void* workspace, hipStream_t stream);

// Any D <= 64, fp32 or bf16 inputs: plain fp32 kernel.
hipError_t launch_general(const Problem& p, bool bf16, hipStream_t stream);

// Start of key tile t when N keys are cut into T near-equal contiguous tiles
// (the first N mod T tiles hold one key more).
__host__ __device__ inline int64_t tile_start(int64_t t, int64_t N, int64_t T) {
    const int64_t base = N / T, extra = N % T;
    return t * base + (t < extra ? t : extra);
}

}  // namespace tri_attn
