/*
 * tri_attn.h -- C ABI of the MI355X (gfx950) pair-biased triangle-attention library
 * (libtri_attn.so).
 *
 * The operation (starting-node triangle attention; "Fold-CP: A Context Parallelism
 * Framework for Biomolecular Modeling", Table 1 row "Triangle Attention", and
 * Figure 2(a)): for every batch b, query row i, query column j and head h,
 *
 *     s_k               = q[b,i,j,h,:] . k[b,i,k,h,:] / sqrt(D) + bias[b,h,j,k] + mask[b,k]
 *     out[b,i,j,h,:]    = sum_k softmax_k(s)_k * v[b,i,k,h,:]
 *
 * The bias is the "triangular" one: indexed by the third edge (j,k), it is shared by
 * every row i.  The key axis is cut into n_key_tiles contiguous tiles -- one per ring
 * step of the context-parallel schedule (Table 1's caption: every ring pattern takes
 * P steps) -- and the tiles are joined, in ascending order, by the tiled online-softmax
 * merge (running maximum, normaliser and accumulator; Figure 2(a) and (c)).  Tile t
 * holds keys [t*(N/T) + min(t, N%T), (t+1)*(N/T) + min(t+1, N%T)): the first N mod T
 * tiles take ceil(N/T) keys, the rest floor(N/T).  The tiling changes only rounding:
 * the merge is associative, so the bf16 matrix-core path folds 32-key blocks in the same
 * ascending order across tile boundaries and its result does not depend on T at all; the
 * fp32 path folds tile by tile.
 *
 * Layouts: every tensor is dense and C-contiguous, elements as listed (last fastest):
 *     q, k, v   [B, I, N, H, D]   dtype (see tri_attn_dtype)
 *     bias      [B, H, N, N]      dtype, k innermost
 *     mask      [B, N]            binary32, additive over the key index (0 keeps a key,
 *                                 -inf drops it); may be NULL (no mask)
 *     out       [B, I, N, H, D]   binary32 for both dtypes
 * I is the number of query rows held by this call (I == N in tri_attn_fwd; 1 <= I <= N
 * in tri_attn_fwd_rows, which serves one rank's row share: rows i in [0, I) of q, k, v,
 * with the full j and k axes and the full bias).
 *
 * Results: a row whose keys are all -inf yields out = 0 (never NaN).  The bf16 path
 * computes q.k and P.V on bf16 matrix cores with fp32 accumulation; softmax statistics
 * are fp32 and the probabilities are rounded to bf16 (nearest even) only as the P.V
 * operand.  It takes bias + mask relative to each query's largest bias + mask over the
 * call's keys (softmax does not change when all scores of a query move together), in
 * log2 units, rounded to fp16: every such value is <= 0 and keeps 11 significant bits.
 * The fp32 path computes in fp32 throughout.
 *
 * Accuracy envelope of the bf16 path.  The fp16 rounding of a bias value x log2 units
 * below its query's largest is up to |x| 2^-11, so it is bounded by a span: every
 * (b, h, block of 256 query columns) whose finite bias + mask values all lie within 32
 * log2 units (about 22.2 nats) of their query's largest runs on the matrix cores, with
 * at most 2^-7 log2 units of image rounding per score (max |error| against fp64 about
 * 1e-3 to 5e-3 on N(0,1)-N(0,4) biases, about 4e-3 at the edge of the span when q.k
 * puts the weight on the farthest keys); every other block is computed on the fp32 path
 * with the bias unrounded, so the 1e-2 bf16 bar holds whatever the bias spread.
 * Finite values more than 65520 log2 units (about 45,400 nats) below the largest are
 * beyond fp16 and count as dropped keys (weight 0): such a key could only matter if its
 * q.k / sqrt(D) made up that distance.  Hence a mask written into the bias or mask as
 * a large finite negative number sends its blocks to the fp32 path when it lies within
 * that range (e.g. -1e4) and not when it lies beyond it (e.g. -1e9); -inf is always free.
 * The same envelope and routing apply to the matrix-core backward's dq, dk and dv (per
 * (b, h)); its dbias kernel always adds the fp32 bias.
 *
 * Ownership and memory: every pointer is a device pointer owned by the caller; the
 * library keeps none of them after returning.  q, k, v, bias and mask are only read and
 * may alias one another; outputs must not overlap any input.  q, k, v, bias and out must be
 * 16-byte aligned, mask 4-byte aligned.  The bf16 matrix-core path (D == 32; one-row calls
 * with even N aside, see pair_bias_attn_fwd) first
 * converts the bias into an fp16 image plus one fp32 reference per query, together
 * tri_attn_workspace_bytes() bytes: roughly 2 * B * H * N * N bytes (queries padded to a
 * multiple of 256, keys to a multiple of 32), plus,
 * for calls too small to fill the GPU (fewer than 512 workgroups of 2 rows x 256 columns
 * and at least 16 key blocks), the partial softmax states of up to 16 key ranges that run
 * side by side and are then joined (16 * 34 * B * I * N * H bytes at most).  Three ways
 * to provide it:
 *   - the caller: every entry point that needs a workspace has a *_ws form that takes one
 *     (sized by tri_attn_call_workspace_bytes) and allocates nothing;
 *   - a static 64 MiB device array inside the library: tri_attn_fwd_rows_noalloc;
 *   - the library's pool: the entry points without a workspace argument (the operator's
 *     own signature has none) obtain it stream-ordered on `stream`
 *     (hipMallocFromPoolAsync / hipFreeAsync) from a memory pool the library creates once
 *     per device; the pool keeps freed memory reserved for later calls, at most the
 *     largest workspace in use at once, until tri_attn_pool_release() or the end of the
 *     process (tri_attn_pool_reserved_bytes() reports it).
 * The fp32 paths need no workspace.
 *
 * Streams: calls only enqueue work on `stream` (a hipStream_t; NULL is the null
 * stream) and return without synchronising.  A kernel fault surfaces at the caller's
 * next synchronisation on that stream.
 *
 * Errors: every entry point returns a tri_attn_status and never throws, aborts or
 * prints.  Arguments are checked in this order, before any device work: NULL
 * pointers; sizes (all >= 1, I <= N, element counts fit int64); dtype; head size
 * (D <= 64; the matrix-core path serves bf16 with D == 32, every other case runs on
 * the general fp32 path); I and B*H at most 65535; n_key_tiles in [1, N]; I == N for
 * the ending orientation; the key range of tri_attn_tile_state; alignment; an output
 * overlapping an input or another output.  A failed allocation or launch returns
 * TRI_ATTN_ERR_HIP and records the HIP error code for tri_attn_last_hip_error() (per
 * calling thread).
 */
#ifndef TRI_ATTN_H
#define TRI_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element type of q, k, v and bias */
typedef enum {
    TRI_ATTN_FP32 = 0,   /* IEEE binary32 */
    TRI_ATTN_BF16 = 1    /* bfloat16 (upper half of a binary32) */
} tri_attn_dtype;

typedef enum {
    TRI_ATTN_OK = 0,
    TRI_ATTN_ERR_NULL = -1,         /* a required pointer is NULL */
    TRI_ATTN_ERR_SHAPE = -2,        /* a size < 1, I > N, or a size overflows int64 */
    TRI_ATTN_ERR_DTYPE = -3,        /* dtype is not a tri_attn_dtype */
    TRI_ATTN_ERR_UNSUPPORTED = -4,  /* D > 64, I or B*H above 65535, or (ending node, bf16,
                                       D == 32) 32 * N * H * D * 2 above 2^31 - 1 */
    TRI_ATTN_ERR_ALIGN = -5,        /* a pointer is not aligned as required */
    TRI_ATTN_ERR_TILES = -6,        /* n_key_tiles outside [1, N] */
    TRI_ATTN_ERR_HIP = -7,          /* the HIP runtime refused an allocation or launch */
    TRI_ATTN_ERR_ALIAS = -8,        /* an output (or the workspace) overlaps an input or another output */
    TRI_ATTN_ERR_WORKSPACE = -9,    /* caller workspace smaller than tri_attn_workspace_bytes() */
    TRI_ATTN_ERR_RANGE = -10,       /* key range not within 0 <= key_begin < key_end <= N */
    TRI_ATTN_ERR_SCRATCH = -11      /* workspace need above tri_attn_noalloc_scratch_bytes() */
} tri_attn_status;

/*
 * Triangle attention over all N query rows (I == N).
 *   q, k, v   [B, N, N, H, D] device, dtype      bias [B, H, N, N] device, dtype
 *   mask      [B, N] device binary32 or NULL      out  [B, N, N, H, D] device binary32
 *   n_key_tiles  number of ring-step key tiles, 1 <= n_key_tiles <= N
 *   dtype        a tri_attn_dtype
 *   stream       hipStream_t to enqueue on (NULL: null stream)
 * Returns TRI_ATTN_OK or a negative tri_attn_status.
 */
int tri_attn_fwd(const void *q, const void *k, const void *v, const void *bias,
                 const float *mask, float *out,
                 int64_t B, int64_t H, int64_t N, int64_t D,
                 int32_t n_key_tiles, int32_t dtype, void *stream);

/*
 * The same operation for one rank's share of query rows: q, k, v and out hold rows
 * i in [0, I) ([B, I, N, H, D]); bias and mask keep their full [B, H, N, N] / [B, N]
 * shapes ("Design-CP: Context Parallelism for Design of Protein Nanoparticles",
 * abstract: 1D row-sharding of the pair representation).  1 <= I <= N.
 */
int tri_attn_fwd_rows(const void *q, const void *k, const void *v, const void *bias,
                      const float *mask, float *out,
                      int64_t B, int64_t H, int64_t I, int64_t N, int64_t D,
                      int32_t n_key_tiles, int32_t dtype, void *stream);

/*
 * Device workspace, in bytes, that the call with these sizes needs (0 when its path needs
 * none), or a negative tri_attn_status for sizes the entry points would reject (same
 * checks and order as they apply, minus the pointer checks).
 */
int64_t tri_attn_workspace_bytes(int64_t B, int64_t H, int64_t I, int64_t N, int64_t D,
                                 int32_t n_key_tiles, int32_t dtype);

/*
 * tri_attn_fwd_rows with a caller-owned device workspace of workspace_bytes bytes
 * (16-byte aligned, at least tri_attn_workspace_bytes(); it must not overlap any input
 * or out).  The library allocates nothing in this call.  The workspace is overwritten and
 * must not be touched by other work until the call's kernels have finished on `stream`.
 * Extra errors: TRI_ATTN_ERR_WORKSPACE (too small or negative size), TRI_ATTN_ERR_NULL
 * (NULL workspace where one is needed), TRI_ATTN_ERR_ALIGN, TRI_ATTN_ERR_ALIAS.
 */
int tri_attn_fwd_rows_ws(const void *q, const void *k, const void *v, const void *bias,
                         const float *mask, float *out,
                         int64_t B, int64_t H, int64_t I, int64_t N, int64_t D,
                         int32_t n_key_tiles, int32_t dtype,
                         void *workspace, int64_t workspace_bytes, void *stream);

/*
 * tri_attn_fwd_rows for callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the workspace is a static device array
 * of tri_attn_noalloc_scratch_bytes() bytes (64 MiB) inside the library, one per GPU, held
 * from the loading of the library's code until the process ends.  This call allocates
 * nothing and frees nothing.  Problems whose workspace (tri_attn_workspace_bytes()) exceeds
 * the array are rejected with TRI_ATTN_ERR_SCRATCH before any device work; B = 1, H = 4
 * fits up to N = I = 2816.  Every call on one GPU uses the same array and leaves its
 * contents there (each call writes all it reads): calls that overlap in time on one GPU,
 * from several streams or threads, race on it and must be serialised by the caller.
 * Arguments, results and other errors as tri_attn_fwd_rows.
 */
int tri_attn_fwd_rows_noalloc(const void *q, const void *k, const void *v, const void *bias,
                              const float *mask, float *out,
                              int64_t B, int64_t H, int64_t I, int64_t N, int64_t D,
                              int32_t n_key_tiles, int32_t dtype, void *stream);

/* Size in bytes of the static scratch of tri_attn_fwd_rows_noalloc. */
int64_t tri_attn_noalloc_scratch_bytes(void);

/*
 * Forward that also returns the natural-log normaliser of every query,
 *     lse[b,i,j,h] = ln sum_k exp(s_k)       (-inf for a query with no finite score),
 * the statistic a backward pass recomputes the probabilities from (p_k = exp(s_k - lse)).
 * Arguments as tri_attn_fwd_rows; lse is device binary32 [B, I, N, H], 4-byte aligned,
 * and must not overlap any input or out.
 */
int tri_attn_fwd_lse(const void *q, const void *k, const void *v, const void *bias,
                     const float *mask, float *out, float *lse,
                     int64_t B, int64_t H, int64_t I, int64_t N, int64_t D,
                     int32_t n_key_tiles, int32_t dtype, void *stream);

/*
 * Ending-node orientation: attention along the columns of the pair tensor, with the
 * triangular bias transposed ("Fold-CP", Figure 2(a): the bias is transposed across
 * axes before the ring).  For every b, i, j, h:
 *     s_k            = q[b,i,j,h,:] . k[b,k,j,h,:] / sqrt(D) + bias[b,h,k,i] + mask[b,k]
 *     out[b,i,j,h,:] = sum_k softmax_k(s)_k * v[b,k,j,h,:]
 * i.e. the starting-node operation on the tensors with their first two pair axes
 * swapped (and the bias's last two), without moving any data.  Same layouts, tiling,
 * numerics and rules as tri_attn_fwd (I == N); lse is optional ([B, N, N, H] or NULL).
 */
int tri_attn_fwd_ending(const void *q, const void *k, const void *v, const void *bias,
                        const float *mask, float *out, float *lse,
                        int64_t B, int64_t H, int64_t N, int64_t D,
                        int32_t n_key_tiles, int32_t dtype, void *stream);

/*
 * Split-tile primitive: the partial softmax state of one ring step, the keys
 * [key_begin, key_end) taken as a single tile ("Fold-CP", Table 1's caption and
 * Figure 2(a)/(c): each ring step's tile is computed on its own and joined by the
 * tiled-softmax merge).  For every query (b, i, j, h) of the orientation chosen by
 * `ending` (0: starting node, rows i in [0, I); 1: ending node, I == N):
 *     m   = a reference in natural-log units (any value; the matrix-core path takes the
 *           query's largest bias + mask over the range, plus the range's exact running
 *           maximum of the scores where that reference leaves l out of range; the fp32
 *           path takes the running maximum)
 *     l   = sum_k exp(s_k - m)                          over the key range
 *     acc = sum_k exp(s_k - m) * v_k                    [D] values, unnormalised
 * A query with no finite score in the range gets m = -inf, l = 0, acc = 0 (the
 * identity of the merge).  acc is device binary32 [B, I, N, H, D] (16-byte aligned),
 * m and l device binary32 [B, I, N, H] (4-byte aligned); none may overlap an input or
 * each other.  Other arguments and rules as tri_attn_fwd_rows.  Extra error:
 * TRI_ATTN_ERR_RANGE.  States are joined with tri_attn_state_merge and turned into the
 * output with tri_attn_state_finalize; merging every tile of a partition of [0, N) in
 * any order gives tri_attn_fwd's result up to rounding.
 */
int tri_attn_tile_state(const void *q, const void *k, const void *v, const void *bias,
                        const float *mask, float *acc, float *m, float *l,
                        int64_t B, int64_t H, int64_t I, int64_t N, int64_t D,
                        int64_t key_begin, int64_t key_end, int32_t ending,
                        int32_t dtype, void *stream);

/*
 * One ring step folded into a running state: the partial state of the keys
 * [key_begin, key_end) (as tri_attn_tile_state computes it) merged in place into the
 * state (acc, m, l) the caller passes, with the rule of tri_attn_state_merge.  The state
 * must hold a valid partial state, for instance the previous step's, or l = 0 (the
 * identity: acc and m are then not read).  Same arguments, layouts and errors as
 * tri_attn_tile_state; acc, m and l are read and written.  Equivalent to
 * tri_attn_tile_state into a scratch state followed by tri_attn_state_merge, without the
 * scratch state's round trip through memory.
 */
int tri_attn_tile_state_update(const void *q, const void *k, const void *v, const void *bias,
                               const float *mask, float *acc, float *m, float *l,
                               int64_t B, int64_t H, int64_t I, int64_t N, int64_t D,
                               int64_t key_begin, int64_t key_end, int32_t ending,
                               int32_t dtype, void *stream);

/*
 * The last ring step: the keys [key_begin, key_end) folded into the state (acc, m, l) as
 * tri_attn_tile_state_update does, and the result finalised straight into out
 * (out = acc / l, 0 where l == 0) and, when lse is not NULL, lse = m + ln l (-inf where
 * l == 0), as tri_attn_state_finalize would.  acc, m and l are only read.  Equivalent to
 * tri_attn_tile_state_update followed by tri_attn_state_finalize, without writing the
 * state back and reading it again.  out [B, I, N, H, D] fp32, 16-byte aligned; lse
 * [B, I, N, H] or NULL; neither may overlap an input or the state.  Other arguments,
 * layouts and errors as tri_attn_tile_state.
 */
int tri_attn_tile_state_final(const void *q, const void *k, const void *v, const void *bias,
                              const float *mask, const float *acc, const float *m, const float *l,
                              float *out, float *lse,
                              int64_t B, int64_t H, int64_t I, int64_t N, int64_t D,
                              int64_t key_begin, int64_t key_end, int32_t ending,
                              int32_t dtype, void *stream);

/*
 * The merge of two partial states, in place into the first, for `rows` queries of D
 * values (rows = B * I * N * H for the states above; 1 <= D <= 64):
 *     M = max(m, m_t);  a = exp(m - M), b = exp(m_t - M)
 *     acc = a * acc + b * acc_t;  l = a * l + b * l_t;  m = M
 * where a state with l == 0 contributes nothing.  All pointers are device binary32,
 * 4-byte aligned; acc, m, l must not overlap acc_t, m_t, l_t.
 */
int tri_attn_state_merge(float *acc, float *m, float *l,
                         const float *acc_t, const float *m_t, const float *l_t,
                         int64_t rows, int64_t D, void *stream);

/*
 * out = acc / l (0 where l == 0) and, when lse is not NULL, lse = m + ln l (-inf where
 * l == 0), for `rows` queries of D values.  out [rows, D] and lse [rows] are device
 * binary32, 4-byte aligned, and must not overlap the state or each other.
 */
int tri_attn_state_finalize(const float *acc, const float *m, const float *l,
                            float *out, float *lse, int64_t rows, int64_t D, void *stream);

/*
 * Backward of the starting-node operation: the gradients of the definition for an
 * upstream gradient dout (Fold-CP trains through its context-parallel modules; the
 * pages give no formula, so these are the plain derivatives).  With
 * p_k = exp(s_k - lse[b,i,j,h]), delta = dout[b,i,j,h,:] . out[b,i,j,h,:],
 * dp_k = dout[b,i,j,h,:] . v[b,i,k,h,:] and ds_k = p_k (dp_k - delta):
 *     dq[b,i,j,h,:] = sum_k ds_k k[b,i,k,h,:] / sqrt(D)
 *     dk[b,i,k,h,:] = sum_j ds_k q[b,i,j,h,:] / sqrt(D)
 *     dv[b,i,k,h,:] = sum_j p_k dout[b,i,j,h,:]
 *     dbias[b,h,j,k] = sum_i ds_k            (summed over the I rows held by the call; the
 *                                             row shares of several calls add up)
 *   q, k, v [B, I, N, H, D], bias [B, H, N, N] (dtype), mask [B, N] or NULL: the forward's
 *   inputs;  out [B, I, N, H, D] and lse [B, I, N, H]: the forward's results
 *   (tri_attn_fwd_lse);  dout [B, I, N, H, D] binary32;
 *   dq, dk, dv [B, I, N, H, D] and dbias [B, H, N, N]: binary32 results, overwritten.
 * bf16 inputs with D == 32 and out, dout, dq, dk, dv 16-byte aligned run on matrix
 * cores: dout, p and ds are rounded to bf16 as product operands (delta from the same
 * rounded dout), sums are fp32, and a workspace (bias images, bf16 dout and head-major
 * copies of q, k, v, [B, H, I, N, D], per-query statistics: about 4 B H N^2 + 8 B I N H D
 * bytes; tri_attn_call_workspace_bytes with TRI_ATTN_CALL_BWD)
 * comes from the library pool as described above, or from the caller through
 * tri_attn_bwd_ws.  Every other case computes in fp32, any D <= 64, with no workspace.
 * Both are deterministic (every sum is taken by one thread in a fixed order, no atomics).
 * A query with lse = -inf contributes nothing.  q, k, v, bias 16-byte aligned, the other
 * pointers 4-byte aligned; no result may overlap an input or another result.  Same error
 * rules as the forward.
 */
int tri_attn_bwd(const void *q, const void *k, const void *v, const void *bias,
                 const float *mask, const float *out, const float *lse, const float *dout,
                 float *dq, float *dk, float *dv, float *dbias,
                 int64_t B, int64_t H, int64_t I, int64_t N, int64_t D,
                 int32_t dtype, void *stream);

/*
 * Attention with pair bias ("Fold-CP", Table 1 row "Attention with Pair Bias", and
 * Figure 2(c)): one sequence of N tokens per batch element, biased by the pair
 * representation,
 *     s_k            = q[b,j,h,:] . k[b,k,h,:] / sqrt(D) + bias[b,h,j,k] + mask[b,k]
 *     out[b,j,h,:]   = sum_k softmax_k(s)_k * v[b,k,h,:]
 * q, k, v, out [B, N, H, D]; bias [B, H, N, N]; mask [B, N] or NULL; lse [B, N, H] or
 * NULL.  It is the triangle operation with a single row (I == 1), with the same tiling
 * and rules.  With one row every bias value is used once, so for bf16, D == 32, even N up
 * to 46340 and a 16-byte aligned bias the call (like any one-row tri_attn_fwd_rows call)
 * runs a single-pass kernel that reads the raw bias once with a running reference per
 * query instead of the fp16 image; its workspace holds only the partial states of key
 * ranges run side by side (none when one range suffices).  Other one-row calls take the
 * image path.
 */
int pair_bias_attn_fwd(const void *q, const void *k, const void *v, const void *bias,
                       const float *mask, float *out, float *lse,
                       int64_t B, int64_t H, int64_t N, int64_t D,
                       int32_t n_key_tiles, int32_t dtype, void *stream);

/*
 * Caller-workspace forms.  Each *_ws entry point is its namesake with a caller-owned
 * device workspace appended (workspace, workspace_bytes): 16-byte aligned, at least
 * tri_attn_call_workspace_bytes() bytes for that call (NULL with 0 bytes when that is 0),
 * not overlapping any input or result, overwritten by the call and not to be touched by
 * other work until the call's kernels have finished on `stream`.  The library allocates
 * nothing in these calls.  Extra errors as tri_attn_fwd_rows_ws: TRI_ATTN_ERR_WORKSPACE
 * (too small or negative size), TRI_ATTN_ERR_NULL (NULL where bytes are needed),
 * TRI_ATTN_ERR_ALIGN, TRI_ATTN_ERR_ALIAS.  Everything else as the namesake.
 */
int tri_attn_fwd_lse_ws(const void *q, const void *k, const void *v, const void *bias,
                        const float *mask, float *out, float *lse,
                        int64_t B, int64_t H, int64_t I, int64_t N, int64_t D,
                        int32_t n_key_tiles, int32_t dtype,
                        void *workspace, int64_t workspace_bytes, void *stream);
int tri_attn_fwd_ending_ws(const void *q, const void *k, const void *v, const void *bias,
                           const float *mask, float *out, float *lse,
                           int64_t B, int64_t H, int64_t N, int64_t D,
                           int32_t n_key_tiles, int32_t dtype,
                           void *workspace, int64_t workspace_bytes, void *stream);
int tri_attn_tile_state_ws(const void *q, const void *k, const void *v, const void *bias,
                           const float *mask, float *acc, float *m, float *l,
                           int64_t B, int64_t H, int64_t I, int64_t N, int64_t D,
                           int64_t key_begin, int64_t key_end, int32_t ending, int32_t dtype,
                           void *workspace, int64_t workspace_bytes, void *stream);
int tri_attn_tile_state_update_ws(const void *q, const void *k, const void *v, const void *bias,
                                  const float *mask, float *acc, float *m, float *l,
                                  int64_t B, int64_t H, int64_t I, int64_t N, int64_t D,
                                  int64_t key_begin, int64_t key_end, int32_t ending, int32_t dtype,
                                  void *workspace, int64_t workspace_bytes, void *stream);
int tri_attn_tile_state_final_ws(const void *q, const void *k, const void *v, const void *bias,
                                 const float *mask, const float *acc, const float *m, const float *l,
                                 float *out, float *lse,
                                 int64_t B, int64_t H, int64_t I, int64_t N, int64_t D,
                                 int64_t key_begin, int64_t key_end, int32_t ending, int32_t dtype,
                                 void *workspace, int64_t workspace_bytes, void *stream);
int pair_bias_attn_fwd_ws(const void *q, const void *k, const void *v, const void *bias,
                          const float *mask, float *out, float *lse,
                          int64_t B, int64_t H, int64_t N, int64_t D,
                          int32_t n_key_tiles, int32_t dtype,
                          void *workspace, int64_t workspace_bytes, void *stream);
int tri_attn_bwd_ws(const void *q, const void *k, const void *v, const void *bias,
                    const float *mask, const float *out, const float *lse, const float *dout,
                    float *dq, float *dk, float *dv, float *dbias,
                    int64_t B, int64_t H, int64_t I, int64_t N, int64_t D, int32_t dtype,
                    void *workspace, int64_t workspace_bytes, void *stream);

/* which call tri_attn_call_workspace_bytes sizes */
typedef enum {
    TRI_ATTN_CALL_FWD = 0,            /* tri_attn_fwd, _rows, _lse (and their _ws forms) */
    TRI_ATTN_CALL_ENDING = 1,         /* tri_attn_fwd_ending (I == N) */
    TRI_ATTN_CALL_STATE = 2,          /* tri_attn_tile_state, _update, _final, starting node */
    TRI_ATTN_CALL_STATE_ENDING = 3,   /* the same, ending node (I == N) */
    TRI_ATTN_CALL_PAIR_BIAS = 4,      /* pair_bias_attn_fwd (I == 1) */
    TRI_ATTN_CALL_BWD = 5             /* tri_attn_bwd */
} tri_attn_call;

/*
 * Workspace bytes (0 if none) of one call of kind `call` (a tri_attn_call) at these
 * sizes; key_count is the number of keys of a ring step's range (state calls only, 1 to
 * N; pass N otherwise).  For the backward it assumes the matrix-core path (16-byte
 * aligned fp32 tensors).  Negative tri_attn_status on invalid sizes (the checks of the
 * call itself that need no pointers).
 */
int64_t tri_attn_call_workspace_bytes(int32_t call, int64_t B, int64_t H, int64_t I, int64_t N,
                                      int64_t D, int64_t key_count, int32_t dtype);

/*
 * The library's memory pool (used by the entry points that take no workspace argument):
 * bytes it holds reserved on the current device (0 before its first use), and a release of
 * every device pool's unused memory back to the driver (memory of calls still in flight on
 * a stream stays until they finish).  TRI_ATTN_ERR_HIP on a HIP error.
 */
int64_t tri_attn_pool_reserved_bytes(void);
int tri_attn_pool_release(void);

/* Static, NUL-terminated description of a tri_attn_status (unknown codes included). */
const char *tri_attn_status_string(int status);

/* HIP error code (hipError_t value) of this thread's last TRI_ATTN_ERR_HIP; 0 if none. */
int tri_attn_last_hip_error(void);

/* Library ABI version: major * 10000 + minor * 100 + patch. */
int tri_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TRI_ATTN_H */
