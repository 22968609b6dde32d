// C ABI of libtri_attn.so (declared in include/tri_attn.h): argument checks, kernel choice,
// workspace handling, launch.  Nothing here synchronises.
#include "tri_attn.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "launch.h"
#include "pair_bias.h"

namespace {

thread_local int g_last_hip_error = 0;

bool uses_matrix_cores(int32_t dtype, int64_t D) { return dtype == TRI_ATTN_BF16 && D == 32; }

// Matrix-core forward: one line without state output (attention with pair bias) reads the
// raw bias once in the single-pass kernel; everything else goes through the fp16 image.
size_t mfma_workspace_bytes(const tri_attn::Problem& p) {
    return tri_attn::pair_bias_direct_applies(p) ? tri_attn::pair_bias_direct_workspace_bytes(p)
                                                 : tri_attn::bf16_workspace_bytes(p);
}
hipError_t launch_mfma(const tri_attn::Problem& p, void* ws, hipStream_t s) {
    return tri_attn::pair_bias_direct_applies(p) ? tri_attn::launch_pair_bias_direct(p, ws, s)
                                                 : tri_attn::launch_bf16_mfma(p, ws, s);
}

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
    if (n_key_tiles < 1 || n_key_tiles > N) return TRI_ATTN_ERR_TILES;
    return TRI_ATTN_OK;
}

// Everything one entry point asks for.
struct Call {
    const void* q;
    const void* k;
    const void* v;
    const void* bias;
    const float* mask;
    float* out;
    int64_t B, H, I, N, D;
    int32_t T, dtype;
    int64_t key_begin = 0, key_end = -1;   // key range (state mode); -1: all keys
    bool ending = false;
    float* lse = nullptr;
    float* st_m = nullptr;
    float* st_l = nullptr;
    bool update = false;                   // state mode: fold into the given state
    float* fin = nullptr;                  // with update: final output (state only read)
    void* ws = nullptr;                    // caller workspace when ws_bytes >= 0
    int64_t ws_bytes = -1;
    bool static_ws = false;                // workspace: the library's static device scratch
};

struct Span {
    const void* p;
    int64_t bytes;
};

int check_pointers(const Call& c, int64_t qkv_elems, int64_t bias_elems) {
    if (!aligned(c.q, 16) || !aligned(c.k, 16) || !aligned(c.v, 16) || !aligned(c.bias, 16) || !aligned(c.out, 16) ||
        (c.mask && !aligned(c.mask, 4)) || (c.lse && !aligned(c.lse, 4)) || (c.st_m && !aligned(c.st_m, 4)) ||
        (c.st_l && !aligned(c.st_l, 4)) || (c.fin && !aligned(c.fin, 16)))
        return TRI_ATTN_ERR_ALIGN;
    const int64_t esz = c.dtype == TRI_ATTN_BF16 ? 2 : 4;
    const int64_t per_query = qkv_elems / c.D * 4;   // bytes of one fp32 value per query
    const Span inputs[] = {{c.q, qkv_elems * esz}, {c.k, qkv_elems * esz}, {c.v, qkv_elems * esz},
                           {c.bias, bias_elems * esz}, {c.mask, c.B * c.N * 4}};
    const Span outputs[] = {{c.out, qkv_elems * 4}, {c.lse, per_query}, {c.st_m, per_query}, {c.st_l, per_query},
                            {c.fin, qkv_elems * 4}};
    constexpr int n_out = 5;
    for (int a = 0; a < n_out; ++a) {
        if (!outputs[a].p) continue;
        for (const Span& in : inputs)
            if (in.p && overlaps(outputs[a].p, outputs[a].bytes, in.p, in.bytes)) return TRI_ATTN_ERR_ALIAS;
        for (int o = a + 1; o < n_out; ++o)
            if (outputs[o].p && overlaps(outputs[a].p, outputs[a].bytes, outputs[o].p, outputs[o].bytes))
                return TRI_ATTN_ERR_ALIAS;
    }
    return TRI_ATTN_OK;
}

tri_attn::Problem make_problem(const Call& c) {
    tri_attn::Problem p{c.q, c.k, c.v, c.bias, c.mask, c.out, c.B, c.H, c.I, c.N, c.D, c.T};
    p.k0 = c.key_begin;
    p.NK = c.key_end >= 0 ? c.key_end - c.key_begin : 0;
    p.ending = c.ending;
    p.lse = c.lse;
    p.st_m = c.st_m;
    p.st_l = c.st_l;
    p.update = c.update;
    p.fin = c.fin;
    return p;
}

// Stream-ordered memory pool of the library, one per device, created on first use.  Its
// release threshold is unlimited, so memory freed at the end of a call stays reserved for
// the next one instead of going back to the driver at every synchronisation.
constexpr int kMaxDevices = 64;
std::mutex g_pool_mu;
hipMemPool_t g_pools[kMaxDevices] = {};

hipError_t workspace_pool(hipMemPool_t* out, bool create = true) {
    hipMemPool_t* pools = g_pools;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_pool_mu);
    if (!pools[dev] && !create) {
        *out = nullptr;
        return hipSuccess;
    }
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

int run(const Call& c, void* stream) {
    if (!c.q || !c.k || !c.v || !c.bias || !c.out) return TRI_ATTN_ERR_NULL;
    if ((c.st_m == nullptr) != (c.st_l == nullptr)) return TRI_ATTN_ERR_NULL;
    int64_t qkv_elems = 0, bias_elems = 0;
    int st = check_sizes(c.B, c.H, c.I, c.N, c.D, c.T, c.dtype, &qkv_elems, &bias_elems);
    if (st != TRI_ATTN_OK) return st;
    if (c.ending && c.I != c.N) return TRI_ATTN_ERR_SHAPE;
    if (c.key_end >= 0 && !(0 <= c.key_begin && c.key_begin < c.key_end && c.key_end <= c.N))
        return TRI_ATTN_ERR_RANGE;
    // the matrix-core kernel addresses the 32 keys of a block with 32-bit byte offsets; in
    // the ending orientation consecutive keys are N * H * D elements apart
    if (uses_matrix_cores(c.dtype, c.D) && c.ending && 32 * c.N * c.H * c.D * 2 > INT32_MAX)
        return TRI_ATTN_ERR_UNSUPPORTED;
    st = check_pointers(c, qkv_elems, bias_elems);
    if (st != TRI_ATTN_OK) return st;

    const tri_attn::Problem p = make_problem(c);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (!uses_matrix_cores(c.dtype, c.D)) {
        const hipError_t e = tri_attn::launch_general(p, c.dtype == TRI_ATTN_BF16, s);
        return e == hipSuccess ? TRI_ATTN_OK : hip_fail(e);
    }
    const int64_t need = static_cast<int64_t>(mfma_workspace_bytes(p));
    if (c.static_ws) {      // the static scratch: no allocation, bounded size
        if (need > static_cast<int64_t>(tri_attn::static_scratch_bytes())) return TRI_ATTN_ERR_SCRATCH;
        void* scratch = nullptr;
        if (need > 0) {
            const hipError_t e = tri_attn::static_scratch(&scratch);
            if (e != hipSuccess) return hip_fail(e);
        }
        const hipError_t e = launch_mfma(p, scratch, s);
        return e == hipSuccess ? TRI_ATTN_OK : hip_fail(e);
    }
    if (c.ws_bytes >= 0) {  // caller-provided workspace
        if (!c.ws && need > 0) return TRI_ATTN_ERR_NULL;
        if (!aligned(c.ws, 16)) return TRI_ATTN_ERR_ALIGN;
        if (c.ws_bytes < need) return TRI_ATTN_ERR_WORKSPACE;
        const Span others[] = {{c.out, qkv_elems * 4}, {c.q, qkv_elems * 2},  {c.k, qkv_elems * 2},
                               {c.v, qkv_elems * 2},   {c.bias, bias_elems * 2}, {c.mask, c.B * c.N * 4},
                               {c.lse, qkv_elems / c.D * 4}, {c.st_m, qkv_elems / c.D * 4},
                               {c.st_l, qkv_elems / c.D * 4}};
        for (const Span& o : others)
            if (o.p && overlaps(c.ws, need, o.p, o.bytes)) return TRI_ATTN_ERR_ALIAS;
        const hipError_t e = launch_mfma(p, c.ws, s);
        return e == hipSuccess ? TRI_ATTN_OK : hip_fail(e);
    }
    if (need == 0) {  // nothing to allocate
        const hipError_t e = launch_mfma(p, nullptr, s);
        return e == hipSuccess ? TRI_ATTN_OK : hip_fail(e);
    }
    hipMemPool_t pool = nullptr;
    hipError_t e = workspace_pool(&pool);
    if (e != hipSuccess) return hip_fail(e);
    void* own = nullptr;
    e = hipMallocFromPoolAsync(&own, static_cast<size_t>(need), pool, s);
    if (e != hipSuccess) return hip_fail(e);
    e = launch_mfma(p, own, s);
    const hipError_t ef = hipFreeAsync(own, s);
    if (e != hipSuccess) return hip_fail(e);
    if (ef != hipSuccess) return hip_fail(ef);
    return TRI_ATTN_OK;
}

Call make_call(const void* q, const void* k, const void* v, const void* bias, const float* mask, float* out, int64_t B,
               int64_t H, int64_t I, int64_t N, int64_t D, int32_t T, int32_t dtype) {
    Call c{q, k, v, bias, mask, out, B, H, I, N, D, T, dtype};
    return c;
}

int check_state_args(const float* a, const float* b, const float* c, int64_t rows, int64_t D) {
    if (!a || !b || !c) return TRI_ATTN_ERR_NULL;
    int64_t t;
    if (rows < 1 || D < 1 || D > 64 || !mul_ok(rows, D, &t) || !mul_ok(t, 4, &t)) return TRI_ATTN_ERR_SHAPE;
    if (!aligned(a, 4) || !aligned(b, 4) || !aligned(c, 4)) return TRI_ATTN_ERR_ALIGN;
    return TRI_ATTN_OK;
}

}  // namespace

extern "C" {

int tri_attn_fwd(const void* q, const void* k, const void* v, const void* bias, const float* mask, float* out,
                 int64_t B, int64_t H, int64_t N, int64_t D, int32_t n_key_tiles, int32_t dtype, void* stream) {
    return run(make_call(q, k, v, bias, mask, out, B, H, N, N, D, n_key_tiles, dtype), stream);
}

int tri_attn_fwd_rows(const void* q, const void* k, const void* v, const void* bias, const float* mask, float* out,
                      int64_t B, int64_t H, int64_t I, int64_t N, int64_t D, int32_t n_key_tiles, int32_t dtype,
                      void* stream) {
    return run(make_call(q, k, v, bias, mask, out, B, H, I, N, D, n_key_tiles, dtype), stream);
}

int64_t tri_attn_workspace_bytes(int64_t B, int64_t H, int64_t I, int64_t N, int64_t D, int32_t n_key_tiles,
                                 int32_t dtype) {
    int64_t qkv_elems = 0, bias_elems = 0;
    const int st = check_sizes(B, H, I, N, D, n_key_tiles, dtype, &qkv_elems, &bias_elems);
    if (st != TRI_ATTN_OK) return st;
    if (!uses_matrix_cores(dtype, D)) return 0;
    const tri_attn::Problem p =
        make_problem(make_call(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, B, H, I, N, D, n_key_tiles, dtype));
    return static_cast<int64_t>(mfma_workspace_bytes(p));
}

int tri_attn_fwd_rows_ws(const void* q, const void* k, const void* v, const void* bias, const float* mask,
                         float* out, int64_t B, int64_t H, int64_t I, int64_t N, int64_t D, int32_t n_key_tiles,
                         int32_t dtype, void* workspace, int64_t workspace_bytes, void* stream) {
    if (workspace_bytes < 0) return TRI_ATTN_ERR_WORKSPACE;
    Call c = make_call(q, k, v, bias, mask, out, B, H, I, N, D, n_key_tiles, dtype);
    c.ws = workspace;
    c.ws_bytes = workspace_bytes;
    return run(c, stream);
}

int tri_attn_fwd_rows_noalloc(const void* q, const void* k, const void* v, const void* bias, const float* mask,
                              float* out, int64_t B, int64_t H, int64_t I, int64_t N, int64_t D, int32_t n_key_tiles,
                              int32_t dtype, void* stream) {
    Call c = make_call(q, k, v, bias, mask, out, B, H, I, N, D, n_key_tiles, dtype);
    c.static_ws = true;
    return run(c, stream);
}

int64_t tri_attn_noalloc_scratch_bytes(void) { return static_cast<int64_t>(tri_attn::static_scratch_bytes()); }

}  // extern "C"

namespace {

// The forward-family calls with an optional caller workspace (ws_bytes < 0: the pool).
int fwd_lse(const void* q, const void* k, const void* v, const void* bias, const float* mask, float* out, float* lse,
            int64_t B, int64_t H, int64_t I, int64_t N, int64_t D, int32_t T, int32_t dtype, void* ws,
            int64_t ws_bytes, void* stream) {
    if (!lse) return TRI_ATTN_ERR_NULL;
    Call c = make_call(q, k, v, bias, mask, out, B, H, I, N, D, T, dtype);
    c.lse = lse;
    c.ws = ws;
    c.ws_bytes = ws_bytes;
    return run(c, stream);
}

int fwd_ending(const void* q, const void* k, const void* v, const void* bias, const float* mask, float* out, float* lse,
               int64_t B, int64_t H, int64_t N, int64_t D, int32_t T, int32_t dtype, void* ws, int64_t ws_bytes,
               void* stream) {
    Call c = make_call(q, k, v, bias, mask, out, B, H, N, N, D, T, dtype);
    c.ending = true;
    c.lse = lse;
    c.ws = ws;
    c.ws_bytes = ws_bytes;
    return run(c, stream);
}

// One ring step: `update` folds it into the state (acc, m, l); `fin`, with update, writes the
// folded result there (and lse) and only reads the state.
int ring_step(const void* q, const void* k, const void* v, const void* bias, const float* mask, float* acc, float* m,
              float* l, float* fin, float* lse, bool update, int64_t B, int64_t H, int64_t I, int64_t N, int64_t D,
              int64_t key_begin, int64_t key_end, int32_t ending, int32_t dtype, void* ws, int64_t ws_bytes,
              void* stream) {
    Call c = make_call(q, k, v, bias, mask, acc, B, H, I, N, D, 1, dtype);
    c.key_begin = key_begin;
    c.key_end = key_end < 0 ? 0 : key_end;   // a negative end is an empty (invalid) range
    c.ending = ending != 0;
    c.st_m = m;
    c.st_l = l;
    c.update = update;
    c.fin = fin;
    c.lse = lse;
    c.ws = ws;
    c.ws_bytes = ws_bytes;
    return run(c, stream);
}

int pair_bias(const void* q, const void* k, const void* v, const void* bias, const float* mask, float* out, float* lse,
              int64_t B, int64_t H, int64_t N, int64_t D, int32_t T, int32_t dtype, void* ws, int64_t ws_bytes,
              void* stream) {
    // one sequence per batch element: the [B, N, H, D] tensors are [B, 1, N, H, D]
    Call c = make_call(q, k, v, bias, mask, out, B, H, 1, N, D, T, dtype);
    c.lse = lse;
    c.ws = ws;
    c.ws_bytes = ws_bytes;
    return run(c, stream);
}

int bwd(const void* q, const void* k, const void* v, const void* bias, const float* mask, const float* out,
        const float* lse, const float* dout, float* dq, float* dk, float* dv, float* dbias, int64_t B, int64_t H,
        int64_t I, int64_t N, int64_t D, int32_t dtype, void* ws, int64_t ws_bytes, void* stream) {
    if (!q || !k || !v || !bias || !out || !lse || !dout || !dq || !dk || !dv || !dbias) return TRI_ATTN_ERR_NULL;
    int64_t qkv_elems = 0, bias_elems = 0;
    const int st = check_sizes(B, H, I, N, D, 1, dtype, &qkv_elems, &bias_elems);
    if (st != TRI_ATTN_OK) return st;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(bias, 16) || (mask && !aligned(mask, 4)) ||
        !aligned(out, 4) || !aligned(lse, 4) || !aligned(dout, 4) || !aligned(dq, 4) || !aligned(dk, 4) ||
        !aligned(dv, 4) || !aligned(dbias, 4))
        return TRI_ATTN_ERR_ALIGN;
    const int64_t esz = dtype == TRI_ATTN_BF16 ? 2 : 4;
    const Span inputs[] = {{q, qkv_elems * esz},   {k, qkv_elems * esz},  {v, qkv_elems * esz},
                           {bias, bias_elems * esz}, {mask, B * N * 4},     {out, qkv_elems * 4},
                           {lse, qkv_elems / D * 4}, {dout, qkv_elems * 4}};
    const Span outputs[] = {{dq, qkv_elems * 4}, {dk, qkv_elems * 4}, {dv, qkv_elems * 4}, {dbias, bias_elems * 4}};
    for (int a = 0; a < 4; ++a) {
        for (const Span& in : inputs)
            if (in.p && overlaps(outputs[a].p, outputs[a].bytes, in.p, in.bytes)) return TRI_ATTN_ERR_ALIAS;
        for (int o = a + 1; o < 4; ++o)
            if (overlaps(outputs[a].p, outputs[a].bytes, outputs[o].p, outputs[o].bytes)) return TRI_ATTN_ERR_ALIAS;
    }
    const tri_attn::BwdProblem p{q, k, v, bias, mask, out, lse, dout, dq, dk, dv, dbias, B, H, I, N, D};
    const hipStream_t s = static_cast<hipStream_t>(stream);
    // matrix cores for bf16 with D == 32 when the fp32 tensors allow 16-byte accesses
    const bool mfma = uses_matrix_cores(dtype, D) && aligned(out, 16) && aligned(dout, 16) && aligned(dq, 16) &&
                      aligned(dk, 16) && aligned(dv, 16);
    if (!mfma) {
        const hipError_t e = tri_attn::launch_backward(p, dtype == TRI_ATTN_BF16, s);
        return e == hipSuccess ? TRI_ATTN_OK : hip_fail(e);
    }
    const int64_t need = static_cast<int64_t>(tri_attn::bwd_mfma_workspace_bytes(p));
    if (ws_bytes >= 0) {   // caller-provided workspace
        if (!ws) return TRI_ATTN_ERR_NULL;
        if (!aligned(ws, 16)) return TRI_ATTN_ERR_ALIGN;
        if (ws_bytes < need) return TRI_ATTN_ERR_WORKSPACE;
        for (const Span& o : inputs)
            if (o.p && overlaps(ws, need, o.p, o.bytes)) return TRI_ATTN_ERR_ALIAS;
        for (const Span& o : outputs)
            if (overlaps(ws, need, o.p, o.bytes)) return TRI_ATTN_ERR_ALIAS;
        const hipError_t e = tri_attn::launch_backward_mfma(p, ws, s);
        return e == hipSuccess ? TRI_ATTN_OK : hip_fail(e);
    }
    hipMemPool_t pool = nullptr;
    hipError_t e = workspace_pool(&pool);
    if (e != hipSuccess) return hip_fail(e);
    void* own = nullptr;
    e = hipMallocFromPoolAsync(&own, static_cast<size_t>(need), pool, s);
    if (e != hipSuccess) return hip_fail(e);
    e = tri_attn::launch_backward_mfma(p, own, s);
    const hipError_t ef = hipFreeAsync(own, s);
    if (e != hipSuccess) return hip_fail(e);
    if (ef != hipSuccess) return hip_fail(ef);
    return TRI_ATTN_OK;
}

}  // namespace

extern "C" {

int tri_attn_fwd_lse(const void* q, const void* k, const void* v, const void* bias, const float* mask, float* out,
                     float* lse, int64_t B, int64_t H, int64_t I, int64_t N, int64_t D, int32_t n_key_tiles,
                     int32_t dtype, void* stream) {
    return fwd_lse(q, k, v, bias, mask, out, lse, B, H, I, N, D, n_key_tiles, dtype, nullptr, -1, stream);
}

int tri_attn_fwd_lse_ws(const void* q, const void* k, const void* v, const void* bias, const float* mask, float* out,
                        float* lse, int64_t B, int64_t H, int64_t I, int64_t N, int64_t D, int32_t n_key_tiles,
                        int32_t dtype, void* workspace, int64_t workspace_bytes, void* stream) {
    if (workspace_bytes < 0) return TRI_ATTN_ERR_WORKSPACE;
    return fwd_lse(q, k, v, bias, mask, out, lse, B, H, I, N, D, n_key_tiles, dtype, workspace, workspace_bytes,
                   stream);
}

int tri_attn_fwd_ending(const void* q, const void* k, const void* v, const void* bias, const float* mask,
                        float* out, float* lse, int64_t B, int64_t H, int64_t N, int64_t D, int32_t n_key_tiles,
                        int32_t dtype, void* stream) {
    return fwd_ending(q, k, v, bias, mask, out, lse, B, H, N, D, n_key_tiles, dtype, nullptr, -1, stream);
}

int tri_attn_fwd_ending_ws(const void* q, const void* k, const void* v, const void* bias, const float* mask,
                           float* out, float* lse, int64_t B, int64_t H, int64_t N, int64_t D, int32_t n_key_tiles,
                           int32_t dtype, void* workspace, int64_t workspace_bytes, void* stream) {
    if (workspace_bytes < 0) return TRI_ATTN_ERR_WORKSPACE;
    return fwd_ending(q, k, v, bias, mask, out, lse, B, H, N, D, n_key_tiles, dtype, workspace, workspace_bytes,
                      stream);
}

int tri_attn_tile_state(const void* q, const void* k, const void* v, const void* bias, const float* mask, float* acc,
                        float* m, float* l, int64_t B, int64_t H, int64_t I, int64_t N, int64_t D, int64_t key_begin,
                        int64_t key_end, int32_t ending, int32_t dtype, void* stream) {
    if (!m || !l) return TRI_ATTN_ERR_NULL;
    return ring_step(q, k, v, bias, mask, acc, m, l, nullptr, nullptr, false, B, H, I, N, D, key_begin, key_end, ending,
                     dtype, nullptr, -1, stream);
}

int tri_attn_tile_state_ws(const void* q, const void* k, const void* v, const void* bias, const float* mask,
                           float* acc, float* m, float* l, int64_t B, int64_t H, int64_t I, int64_t N, int64_t D,
                           int64_t key_begin, int64_t key_end, int32_t ending, int32_t dtype, void* workspace,
                           int64_t workspace_bytes, void* stream) {
    if (!m || !l) return TRI_ATTN_ERR_NULL;
    if (workspace_bytes < 0) return TRI_ATTN_ERR_WORKSPACE;
    return ring_step(q, k, v, bias, mask, acc, m, l, nullptr, nullptr, false, B, H, I, N, D, key_begin, key_end, ending,
                     dtype, workspace, workspace_bytes, stream);
}

int tri_attn_tile_state_update(const void* q, const void* k, const void* v, const void* bias, const float* mask,
                               float* acc, float* m, float* l, int64_t B, int64_t H, int64_t I, int64_t N, int64_t D,
                               int64_t key_begin, int64_t key_end, int32_t ending, int32_t dtype, void* stream) {
    if (!m || !l) return TRI_ATTN_ERR_NULL;
    return ring_step(q, k, v, bias, mask, acc, m, l, nullptr, nullptr, true, B, H, I, N, D, key_begin, key_end, ending,
                     dtype, nullptr, -1, stream);
}

int tri_attn_tile_state_update_ws(const void* q, const void* k, const void* v, const void* bias, const float* mask,
                                  float* acc, float* m, float* l, int64_t B, int64_t H, int64_t I, int64_t N,
                                  int64_t D, int64_t key_begin, int64_t key_end, int32_t ending, int32_t dtype,
                                  void* workspace, int64_t workspace_bytes, void* stream) {
    if (!m || !l) return TRI_ATTN_ERR_NULL;
    if (workspace_bytes < 0) return TRI_ATTN_ERR_WORKSPACE;
    return ring_step(q, k, v, bias, mask, acc, m, l, nullptr, nullptr, true, B, H, I, N, D, key_begin, key_end, ending,
                     dtype, workspace, workspace_bytes, stream);
}

int tri_attn_tile_state_final(const void* q, const void* k, const void* v, const void* bias, const float* mask,
                              const float* acc, const float* m, const float* l, float* out, float* lse, int64_t B,
                              int64_t H, int64_t I, int64_t N, int64_t D, int64_t key_begin, int64_t key_end,
                              int32_t ending, int32_t dtype, void* stream) {
    if (!m || !l || !out) return TRI_ATTN_ERR_NULL;
    // the state is only read here; the kernels take it through the state pointers
    return ring_step(q, k, v, bias, mask, const_cast<float*>(acc), const_cast<float*>(m), const_cast<float*>(l), out,
                     lse, true, B, H, I, N, D, key_begin, key_end, ending, dtype, nullptr, -1, stream);
}

int tri_attn_tile_state_final_ws(const void* q, const void* k, const void* v, const void* bias, const float* mask,
                                 const float* acc, const float* m, const float* l, float* out, float* lse, int64_t B,
                                 int64_t H, int64_t I, int64_t N, int64_t D, int64_t key_begin, int64_t key_end,
                                 int32_t ending, int32_t dtype, void* workspace, int64_t workspace_bytes,
                                 void* stream) {
    if (!m || !l || !out) return TRI_ATTN_ERR_NULL;
    if (workspace_bytes < 0) return TRI_ATTN_ERR_WORKSPACE;
    return ring_step(q, k, v, bias, mask, const_cast<float*>(acc), const_cast<float*>(m), const_cast<float*>(l), out,
                     lse, true, B, H, I, N, D, key_begin, key_end, ending, dtype, workspace, workspace_bytes, stream);
}

int tri_attn_state_merge(float* acc, float* m, float* l, const float* acc_t, const float* m_t, const float* l_t,
                         int64_t rows, int64_t D, void* stream) {
    int st = check_state_args(acc, m, l, rows, D);
    if (st != TRI_ATTN_OK) return st;
    st = check_state_args(acc_t, m_t, l_t, rows, D);
    if (st != TRI_ATTN_OK) return st;
    const Span mine[] = {{acc, rows * D * 4}, {m, rows * 4}, {l, rows * 4}};
    const Span theirs[] = {{acc_t, rows * D * 4}, {m_t, rows * 4}, {l_t, rows * 4}};
    for (const Span& a : mine)
        for (const Span& b : theirs)
            if (overlaps(a.p, a.bytes, b.p, b.bytes)) return TRI_ATTN_ERR_ALIAS;
    const hipError_t e =
        tri_attn::launch_state_merge(acc, m, l, acc_t, m_t, l_t, rows, D, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TRI_ATTN_OK : hip_fail(e);
}

int tri_attn_state_finalize(const float* acc, const float* m, const float* l, float* out, float* lse, int64_t rows,
                            int64_t D, void* stream) {
    int st = check_state_args(acc, m, l, rows, D);
    if (st != TRI_ATTN_OK) return st;
    if (!out) return TRI_ATTN_ERR_NULL;
    if (!aligned(out, 4) || (lse && !aligned(lse, 4))) return TRI_ATTN_ERR_ALIGN;
    const Span ins[] = {{acc, rows * D * 4}, {m, rows * 4}, {l, rows * 4}};
    for (const Span& a : ins)
        if (overlaps(out, rows * D * 4, a.p, a.bytes) || (lse && overlaps(lse, rows * 4, a.p, a.bytes)))
            return TRI_ATTN_ERR_ALIAS;
    if (lse && overlaps(out, rows * D * 4, lse, rows * 4)) return TRI_ATTN_ERR_ALIAS;
    const hipError_t e = tri_attn::launch_state_finalize(acc, m, l, out, lse, rows, D, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TRI_ATTN_OK : hip_fail(e);
}

int tri_attn_bwd(const void* q, const void* k, const void* v, const void* bias, const float* mask, const float* out,
                 const float* lse, const float* dout, float* dq, float* dk, float* dv, float* dbias, int64_t B,
                 int64_t H, int64_t I, int64_t N, int64_t D, int32_t dtype, void* stream) {
    return bwd(q, k, v, bias, mask, out, lse, dout, dq, dk, dv, dbias, B, H, I, N, D, dtype, nullptr, -1, stream);
}

int tri_attn_bwd_ws(const void* q, const void* k, const void* v, const void* bias, const float* mask, const float* out,
                    const float* lse, const float* dout, float* dq, float* dk, float* dv, float* dbias, int64_t B,
                    int64_t H, int64_t I, int64_t N, int64_t D, int32_t dtype, void* workspace,
                    int64_t workspace_bytes, void* stream) {
    if (workspace_bytes < 0) return TRI_ATTN_ERR_WORKSPACE;
    return bwd(q, k, v, bias, mask, out, lse, dout, dq, dk, dv, dbias, B, H, I, N, D, dtype, workspace,
               workspace_bytes, stream);
}

int pair_bias_attn_fwd(const void* q, const void* k, const void* v, const void* bias, const float* mask, float* out,
                       float* lse, int64_t B, int64_t H, int64_t N, int64_t D, int32_t n_key_tiles, int32_t dtype,
                       void* stream) {
    return pair_bias(q, k, v, bias, mask, out, lse, B, H, N, D, n_key_tiles, dtype, nullptr, -1, stream);
}

int pair_bias_attn_fwd_ws(const void* q, const void* k, const void* v, const void* bias, const float* mask, float* out,
                          float* lse, int64_t B, int64_t H, int64_t N, int64_t D, int32_t n_key_tiles, int32_t dtype,
                          void* workspace, int64_t workspace_bytes, void* stream) {
    if (workspace_bytes < 0) return TRI_ATTN_ERR_WORKSPACE;
    return pair_bias(q, k, v, bias, mask, out, lse, B, H, N, D, n_key_tiles, dtype, workspace, workspace_bytes, stream);
}

int64_t tri_attn_call_workspace_bytes(int32_t call, int64_t B, int64_t H, int64_t I, int64_t N, int64_t D,
                                      int64_t key_count, int32_t dtype) {
    if (call < TRI_ATTN_CALL_FWD || call > TRI_ATTN_CALL_BWD) return TRI_ATTN_ERR_SHAPE;
    int64_t qkv_elems = 0, bias_elems = 0;
    const int st = check_sizes(B, H, I, N, D, 1, dtype, &qkv_elems, &bias_elems);
    if (st != TRI_ATTN_OK) return st;
    const bool ending = call == TRI_ATTN_CALL_ENDING || call == TRI_ATTN_CALL_STATE_ENDING;
    const bool state = call == TRI_ATTN_CALL_STATE || call == TRI_ATTN_CALL_STATE_ENDING;
    if ((ending && I != N) || (call == TRI_ATTN_CALL_PAIR_BIAS && I != 1)) return TRI_ATTN_ERR_SHAPE;
    if (state && (key_count < 1 || key_count > N)) return TRI_ATTN_ERR_RANGE;
    if (!uses_matrix_cores(dtype, D)) return 0;
    if (call == TRI_ATTN_CALL_BWD) {
        const tri_attn::BwdProblem p{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                     nullptr, nullptr, nullptr, B, H, I, N, D};
        return static_cast<int64_t>(tri_attn::bwd_mfma_workspace_bytes(p));
    }
    Call c = make_call(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, B, H, I, N, D, 1, dtype);
    c.ending = ending;
    if (state) {   // a state call's layout depends on how many keys its range holds, not where it starts
        static float placeholder;
        c.key_begin = 0;
        c.key_end = key_count;
        c.st_m = c.st_l = &placeholder;
    }
    return static_cast<int64_t>(mfma_workspace_bytes(make_problem(c)));
}

int64_t tri_attn_pool_reserved_bytes(void) {
    hipMemPool_t pool = nullptr;
    const hipError_t e = workspace_pool(&pool, false);
    if (e != hipSuccess) return hip_fail(e);
    if (!pool) return 0;
    uint64_t reserved = 0;
    const hipError_t ea = hipMemPoolGetAttribute(pool, hipMemPoolAttrReservedMemCurrent, &reserved);
    if (ea != hipSuccess) return hip_fail(ea);
    return static_cast<int64_t>(reserved);
}

int tri_attn_pool_release(void) {
    std::lock_guard<std::mutex> lock(g_pool_mu);
    for (hipMemPool_t pool : g_pools) {
        if (!pool) continue;
        const hipError_t e = hipMemPoolTrimTo(pool, 0);
        if (e != hipSuccess) return hip_fail(e);
    }
    return TRI_ATTN_OK;
}

const char* tri_attn_status_string(int status) {
    switch (status) {
        case TRI_ATTN_OK: return "ok";
        case TRI_ATTN_ERR_NULL: return "a required pointer is NULL";
        case TRI_ATTN_ERR_SHAPE: return "invalid sizes (each >= 1, I <= N, element counts within int64)";
        case TRI_ATTN_ERR_DTYPE: return "unknown dtype (expected TRI_ATTN_FP32 or TRI_ATTN_BF16)";
        case TRI_ATTN_ERR_UNSUPPORTED: return "unsupported problem (head size D > 64, I or B*H above 65535, or an ending-node bf16 key block beyond 32-bit offsets)";
        case TRI_ATTN_ERR_ALIGN: return "misaligned pointer (16 bytes for q, k, v, bias, out, workspace; 4 for mask)";
        case TRI_ATTN_ERR_TILES: return "n_key_tiles outside [1, N]";
        case TRI_ATTN_ERR_HIP: return "the HIP runtime refused an allocation or launch (see tri_attn_last_hip_error)";
        case TRI_ATTN_ERR_ALIAS: return "an output or the workspace overlaps an input or another output";
        case TRI_ATTN_ERR_WORKSPACE: return "workspace smaller than tri_attn_workspace_bytes()";
        case TRI_ATTN_ERR_RANGE: return "key range outside 0 <= key_begin < key_end <= N";
        case TRI_ATTN_ERR_SCRATCH: return "the problem needs more workspace than the static scratch of tri_attn_fwd_rows_noalloc (tri_attn_noalloc_scratch_bytes())";
        default: return "unknown status";
    }
}

int tri_attn_last_hip_error(void) { return g_last_hip_error; }

int tri_attn_version(void) { return 10500; }

}  // extern "C"
