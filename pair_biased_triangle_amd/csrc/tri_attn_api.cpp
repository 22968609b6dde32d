// C ABI of libtri_attn.so (declared in include/tri_attn.h): argument checks, kernel choice,
// launch.  Nothing here allocates device memory or synchronises.
#include "tri_attn.h"

#include <hip/hip_runtime.h>

#include <cstdint>

#include "launch.h"

namespace {

thread_local int g_last_hip_error = 0;

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    *out = a * b;
    return true;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlaps(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + static_cast<uintptr_t>(b_bytes) && b0 < a0 + static_cast<uintptr_t>(a_bytes);
}

int run(const void* q, const void* k, const void* v, const void* bias, const float* mask, float* out,
        int64_t B, int64_t H, int64_t I, int64_t N, int64_t D, int32_t n_key_tiles, int32_t dtype,
        void* stream) {
    if (!q || !k || !v || !bias || !out) return TRI_ATTN_ERR_NULL;
    if (B < 1 || H < 1 || I < 1 || N < 1 || D < 1 || I > N) return TRI_ATTN_ERR_SHAPE;
    int64_t rows, qkv_elems, bias_elems, t;
    if (!mul_ok(B, I, &rows) || !mul_ok(rows, N, &t) || !mul_ok(t, H, &t) || !mul_ok(t, D, &qkv_elems) ||
        !mul_ok(qkv_elems, 4, &t))
        return TRI_ATTN_ERR_SHAPE;
    if (!mul_ok(B, H, &t) || !mul_ok(t, N, &t) || !mul_ok(t, N, &bias_elems) || !mul_ok(bias_elems, 4, &t))
        return TRI_ATTN_ERR_SHAPE;
    if (dtype != TRI_ATTN_FP32 && dtype != TRI_ATTN_BF16) return TRI_ATTN_ERR_DTYPE;
    if (D > 64) return TRI_ATTN_ERR_UNSUPPORTED;
    // the general kernel puts the rows i and the (b, h) pairs on grid dimensions y and z
    if (!(dtype == TRI_ATTN_BF16 && D == 32) && (I > 65535 || B * H > 65535)) return TRI_ATTN_ERR_UNSUPPORTED;
    if (n_key_tiles < 1 || n_key_tiles > N) return TRI_ATTN_ERR_TILES;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(bias, 16) || !aligned(out, 16) ||
        (mask && !aligned(mask, 4)))
        return TRI_ATTN_ERR_ALIGN;
    const int64_t esz = dtype == TRI_ATTN_BF16 ? 2 : 4;
    const int64_t out_bytes = qkv_elems * 4;
    if (overlaps(out, out_bytes, q, qkv_elems * esz) || overlaps(out, out_bytes, k, qkv_elems * esz) ||
        overlaps(out, out_bytes, v, qkv_elems * esz) || overlaps(out, out_bytes, bias, bias_elems * esz) ||
        (mask && overlaps(out, out_bytes, mask, B * N * 4)))
        return TRI_ATTN_ERR_ALIAS;

    tri_attn::Problem p{q, k, v, bias, mask, out, B, H, I, N, D, n_key_tiles};
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (dtype == TRI_ATTN_BF16 && D == 32)
        e = tri_attn::launch_bf16_mfma(p, s);
    else
        e = tri_attn::launch_general(p, dtype == TRI_ATTN_BF16, s);
    if (e != hipSuccess) {
        g_last_hip_error = static_cast<int>(e);
        return TRI_ATTN_ERR_HIP;
    }
    return TRI_ATTN_OK;
}

}  // namespace

extern "C" {

int tri_attn_fwd(const void* q, const void* k, const void* v, const void* bias, const float* mask, float* out,
                 int64_t B, int64_t H, int64_t N, int64_t D, int32_t n_key_tiles, int32_t dtype, void* stream) {
    return run(q, k, v, bias, mask, out, B, H, N, N, D, n_key_tiles, dtype, stream);
}

int tri_attn_fwd_rows(const void* q, const void* k, const void* v, const void* bias, const float* mask, float* out,
                      int64_t B, int64_t H, int64_t I, int64_t N, int64_t D, int32_t n_key_tiles, int32_t dtype,
                      void* stream) {
    return run(q, k, v, bias, mask, out, B, H, I, N, D, n_key_tiles, dtype, stream);
}

const char* tri_attn_status_string(int status) {
    switch (status) {
        case TRI_ATTN_OK: return "ok";
        case TRI_ATTN_ERR_NULL: return "a required pointer is NULL";
        case TRI_ATTN_ERR_SHAPE: return "invalid sizes (each >= 1, I <= N, element counts within int64)";
        case TRI_ATTN_ERR_DTYPE: return "unknown dtype (expected TRI_ATTN_FP32 or TRI_ATTN_BF16)";
        case TRI_ATTN_ERR_UNSUPPORTED: return "unsupported problem (head size D > 64, or grid limits)";
        case TRI_ATTN_ERR_ALIGN: return "misaligned pointer (16 bytes for q, k, v, bias, out; 4 for mask)";
        case TRI_ATTN_ERR_TILES: return "n_key_tiles outside [1, N]";
        case TRI_ATTN_ERR_HIP: return "the HIP runtime refused the launch (see tri_attn_last_hip_error)";
        case TRI_ATTN_ERR_ALIAS: return "out overlaps an input";
        default: return "unknown status";
    }
}

int tri_attn_last_hip_error(void) { return g_last_hip_error; }

int tri_attn_version(void) { return 10000; }

}  // extern "C"
