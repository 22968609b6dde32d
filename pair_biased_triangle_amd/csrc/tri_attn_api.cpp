// C ABI of libtri_attn.so (declared in include/tri_attn.h): argument checks, kernel choice,
// workspace handling, launch.  Nothing here synchronises.
#include "tri_attn.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "launch.h"

namespace {

thread_local int g_last_hip_error = 0;

bool uses_matrix_cores(int32_t dtype, int64_t D) { return dtype == TRI_ATTN_BF16 && D == 32; }

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

int hip_fail(hipError_t e) {
    g_last_hip_error = static_cast<int>(e);
    return TRI_ATTN_ERR_HIP;
}

// Checks that need no pointers; fills `p` sizes.  Returns a tri_attn_status.
int check_sizes(int64_t B, int64_t H, int64_t I, int64_t N, int64_t D, int32_t n_key_tiles, int32_t dtype,
                int64_t* qkv_elems, int64_t* bias_elems) {
    if (B < 1 || H < 1 || I < 1 || N < 1 || D < 1 || I > N) return TRI_ATTN_ERR_SHAPE;
    int64_t rows, t;
    if (!mul_ok(B, I, &rows) || !mul_ok(rows, N, &t) || !mul_ok(t, H, &t) || !mul_ok(t, D, qkv_elems) ||
        !mul_ok(*qkv_elems, 4, &t))
        return TRI_ATTN_ERR_SHAPE;
    if (!mul_ok(B, H, &t) || !mul_ok(t, N, &t) || !mul_ok(t, N, bias_elems) || !mul_ok(*bias_elems, 4, &t))
        return TRI_ATTN_ERR_SHAPE;
    if (dtype != TRI_ATTN_FP32 && dtype != TRI_ATTN_BF16) return TRI_ATTN_ERR_DTYPE;
    if (D > 64) return TRI_ATTN_ERR_UNSUPPORTED;
    // grid limits: the general kernel puts rows i and (b, h) on grid y and z, the matrix-core
    // kernels put column blocks and (b, h) on grid y and z of the bias conversion
    if (I > 65535 || B * H > 65535) return TRI_ATTN_ERR_UNSUPPORTED;
    // the matrix-core kernels address one (b, i) row of K or V with 32-bit byte offsets
    if (uses_matrix_cores(dtype, D) && N * H * D * 2 > INT32_MAX) return TRI_ATTN_ERR_UNSUPPORTED;
    if (n_key_tiles < 1 || n_key_tiles > N) return TRI_ATTN_ERR_TILES;
    return TRI_ATTN_OK;
}

int check_pointers(const void* q, const void* k, const void* v, const void* bias, const float* mask, float* out,
                   int64_t B, int64_t N, int64_t qkv_elems, int64_t bias_elems, int32_t dtype) {
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(bias, 16) || !aligned(out, 16) ||
        (mask && !aligned(mask, 4)))
        return TRI_ATTN_ERR_ALIGN;
    const int64_t esz = dtype == TRI_ATTN_BF16 ? 2 : 4;
    const int64_t out_bytes = qkv_elems * 4;
    if (overlaps(out, out_bytes, q, qkv_elems * esz) || overlaps(out, out_bytes, k, qkv_elems * esz) ||
        overlaps(out, out_bytes, v, qkv_elems * esz) || overlaps(out, out_bytes, bias, bias_elems * esz) ||
        (mask && overlaps(out, out_bytes, mask, B * N * 4)))
        return TRI_ATTN_ERR_ALIAS;
    return TRI_ATTN_OK;
}

tri_attn::Problem make_problem(const void* q, const void* k, const void* v, const void* bias, const float* mask,
                               float* out, int64_t B, int64_t H, int64_t I, int64_t N, int64_t D, int32_t T) {
    return tri_attn::Problem{q, k, v, bias, mask, out, B, H, I, N, D, T};
}

// Stream-ordered memory pool of the library, one per device, created on first use.  Its
// release threshold is unlimited, so memory freed at the end of a call stays reserved for
// the next one instead of going back to the driver at every synchronisation.
hipError_t workspace_pool(hipMemPool_t* out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static hipMemPool_t pools[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!pools[dev]) {
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t pool = nullptr;
        e = hipMemPoolCreate(&pool, &props);
        if (e != hipSuccess) return e;
        uint64_t keep = UINT64_MAX;
        e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
        if (e != hipSuccess) {
            (void)hipMemPoolDestroy(pool);
            return e;
        }
        pools[dev] = pool;
    }
    *out = pools[dev];
    return hipSuccess;
}

// ws == nullptr && ws_bytes < 0: allocate the workspace stream-ordered on `stream`.
int run(const void* q, const void* k, const void* v, const void* bias, const float* mask, float* out, int64_t B,
        int64_t H, int64_t I, int64_t N, int64_t D, int32_t n_key_tiles, int32_t dtype, void* ws, int64_t ws_bytes,
        void* stream) {
    if (!q || !k || !v || !bias || !out) return TRI_ATTN_ERR_NULL;
    int64_t qkv_elems = 0, bias_elems = 0;
    int st = check_sizes(B, H, I, N, D, n_key_tiles, dtype, &qkv_elems, &bias_elems);
    if (st != TRI_ATTN_OK) return st;
    st = check_pointers(q, k, v, bias, mask, out, B, N, qkv_elems, bias_elems, dtype);
    if (st != TRI_ATTN_OK) return st;

    const tri_attn::Problem p = make_problem(q, k, v, bias, mask, out, B, H, I, N, D, n_key_tiles);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (!uses_matrix_cores(dtype, D)) {
        const hipError_t e = tri_attn::launch_general(p, dtype == TRI_ATTN_BF16, s);
        return e == hipSuccess ? TRI_ATTN_OK : hip_fail(e);
    }
    const int64_t need = static_cast<int64_t>(tri_attn::bf16_workspace_bytes(p));
    if (ws_bytes >= 0) {  // caller-provided workspace
        if (!ws) return TRI_ATTN_ERR_NULL;
        if (!aligned(ws, 16)) return TRI_ATTN_ERR_ALIGN;
        if (ws_bytes < need) return TRI_ATTN_ERR_WORKSPACE;
        if (overlaps(ws, need, out, qkv_elems * 4) || overlaps(ws, need, q, qkv_elems * 2) ||
            overlaps(ws, need, k, qkv_elems * 2) || overlaps(ws, need, v, qkv_elems * 2) ||
            overlaps(ws, need, bias, bias_elems * 2) || (mask && overlaps(ws, need, mask, B * N * 4)))
            return TRI_ATTN_ERR_ALIAS;
        const hipError_t e = tri_attn::launch_bf16_mfma(p, ws, s);
        return e == hipSuccess ? TRI_ATTN_OK : hip_fail(e);
    }
    hipMemPool_t pool = nullptr;
    hipError_t e = workspace_pool(&pool);
    if (e != hipSuccess) return hip_fail(e);
    void* own = nullptr;
    e = hipMallocFromPoolAsync(&own, static_cast<size_t>(need), pool, s);
    if (e != hipSuccess) return hip_fail(e);
    e = tri_attn::launch_bf16_mfma(p, own, s);
    const hipError_t ef = hipFreeAsync(own, s);
    if (e != hipSuccess) return hip_fail(e);
    if (ef != hipSuccess) return hip_fail(ef);
    return TRI_ATTN_OK;
}

}  // namespace

extern "C" {

int tri_attn_fwd(const void* q, const void* k, const void* v, const void* bias, const float* mask, float* out,
                 int64_t B, int64_t H, int64_t N, int64_t D, int32_t n_key_tiles, int32_t dtype, void* stream) {
    return run(q, k, v, bias, mask, out, B, H, N, N, D, n_key_tiles, dtype, nullptr, -1, stream);
}

int tri_attn_fwd_rows(const void* q, const void* k, const void* v, const void* bias, const float* mask, float* out,
                      int64_t B, int64_t H, int64_t I, int64_t N, int64_t D, int32_t n_key_tiles, int32_t dtype,
                      void* stream) {
    return run(q, k, v, bias, mask, out, B, H, I, N, D, n_key_tiles, dtype, nullptr, -1, stream);
}

int64_t tri_attn_workspace_bytes(int64_t B, int64_t H, int64_t I, int64_t N, int64_t D, int32_t n_key_tiles,
                                 int32_t dtype) {
    int64_t qkv_elems = 0, bias_elems = 0;
    const int st = check_sizes(B, H, I, N, D, n_key_tiles, dtype, &qkv_elems, &bias_elems);
    if (st != TRI_ATTN_OK) return st;
    if (!uses_matrix_cores(dtype, D)) return 0;
    const tri_attn::Problem p = make_problem(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, B, H, I, N, D,
                                             n_key_tiles);
    return static_cast<int64_t>(tri_attn::bf16_workspace_bytes(p));
}

int tri_attn_fwd_rows_ws(const void* q, const void* k, const void* v, const void* bias, const float* mask,
                         float* out, int64_t B, int64_t H, int64_t I, int64_t N, int64_t D, int32_t n_key_tiles,
                         int32_t dtype, void* workspace, int64_t workspace_bytes, void* stream) {
    if (workspace_bytes < 0) return TRI_ATTN_ERR_WORKSPACE;
    return run(q, k, v, bias, mask, out, B, H, I, N, D, n_key_tiles, dtype, workspace, workspace_bytes, stream);
}

const char* tri_attn_status_string(int status) {
    switch (status) {
        case TRI_ATTN_OK: return "ok";
        case TRI_ATTN_ERR_NULL: return "a required pointer is NULL";
        case TRI_ATTN_ERR_SHAPE: return "invalid sizes (each >= 1, I <= N, element counts within int64)";
        case TRI_ATTN_ERR_DTYPE: return "unknown dtype (expected TRI_ATTN_FP32 or TRI_ATTN_BF16)";
        case TRI_ATTN_ERR_UNSUPPORTED: return "unsupported problem (head size D > 64, I or B*H above 65535, or a bf16 row of K/V over 2 GiB)";
        case TRI_ATTN_ERR_ALIGN: return "misaligned pointer (16 bytes for q, k, v, bias, out, workspace; 4 for mask)";
        case TRI_ATTN_ERR_TILES: return "n_key_tiles outside [1, N]";
        case TRI_ATTN_ERR_HIP: return "the HIP runtime refused an allocation or launch (see tri_attn_last_hip_error)";
        case TRI_ATTN_ERR_ALIAS: return "out or the workspace overlaps an input";
        case TRI_ATTN_ERR_WORKSPACE: return "workspace smaller than tri_attn_workspace_bytes()";
        default: return "unknown status";
    }
}

int tri_attn_last_hip_error(void) { return g_last_hip_error; }

int tri_attn_version(void) { return 10100; }

}  // extern "C"
