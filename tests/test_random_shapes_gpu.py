"""GPU parity on seeded random shapes: a fixed list of problems drawn from a seeded
generator (batch, rows, tokens, heads, head size, dtype, key tiles, bias scale and a
random mask with some keys dropped and, now and then, every key of a batch element),
each run through the forward, the log-sum-exp, the allocation-free forward (when its
scratch suffices), the ring of T steps, the ending node (square ones), attention with pair
bias (one row) and the backward, and compared element by element with the fp64 oracle on
the same inputs.  Bars as everywhere: 1e-5 (fp32) and 1e-2 (bf16) on
outputs and lse; the backward's as in test_backward_gpu.py (exact statistics).
"""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.test_parity_gpu import TOL, compare, say, to_dev

pytestmark = pytest.mark.gpu

N_CASES = 24


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import pair_biased_triangle_amd as P
    P.load_library()
    return torch


def draw(case):
    """Problem `case` of the list: sizes from a generator seeded by the case number."""
    rng = np.random.default_rng(9000 + case)
    dtype = "bf16" if rng.random() < 0.75 else "fp32"
    if dtype == "bf16":
        D = 32 if rng.random() < 0.6 else int(rng.choice([8, 16, 24, 48, 64]))   # 32: the matrix-core path
    else:
        D = int(rng.choice([8, 16, 32, 64]))
    N = int(rng.integers(1, 180))
    square = rng.random() < 0.4
    I = N if square else int(rng.integers(1, min(N, 40) + 1))
    B = int(rng.integers(1, 3))
    H = int(rng.integers(1, 5))
    T = int(rng.integers(1, min(N, 12) + 1))
    sigma = float(rng.choice([0.5, 2.0, 6.0]))
    w = W.make_inputs(W.custom_config(B=B, I=I, N=N, H=H, D=D, dtype=dtype, n_key_tiles=T, seed=300 + case,
                                      sigma_bias=sigma, mask_last=0))
    mask = np.zeros((B, N), dtype=np.float32)
    mask[rng.random((B, N)) < 0.15] = -np.inf
    if B > 1 and rng.random() < 0.25:
        mask[1, :] = -np.inf                       # a batch element without any key
    soft = rng.random((B, N)) < 0.2
    mask[soft & np.isfinite(mask)] = -2.0 * rng.random(int((soft & np.isfinite(mask)).sum()))
    return w, mask, T


def compare_lse(got, expect, tol, what):
    fin = np.isfinite(expect)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: -inf pattern differs"
    err = float(np.max(np.abs(got[fin] - expect[fin]))) if fin.any() else 0.0
    say(f"  {what}: max|err| = {err:.3e} (bar {tol:g})")
    assert err <= tol, f"{what}: {err:.3e} > {tol:g}"


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_shape(torch_dev, case):
    import pair_biased_triangle_amd as P
    t = torch_dev
    w, mask, T = draw(case)
    c = w.cfg
    say(f"[random {case}] B={c.B} I={c.I} N={c.N} H={c.H} D={c.D} {c.dtype} T={T}")
    tol = TOL[c.dtype]
    q, k, v, bias = (to_dev(t, x) for x in (w.q, w.k, w.v, w.bias))
    m = to_dev(t, mask)
    fn = P.tri_attn_fwd if c.I == c.N else P.tri_attn_fwd_rows
    out = fn(q, k, v, bias, m, n_key_tiles=T)
    out2, lse = P.tri_attn_fwd_lse(q, k, v, bias, m, n_key_tiles=T)
    t.cuda.synchronize()
    ref, ref_lse = oracle.tri_attn(w.q, w.k, w.v, w.bias, mask, n_key_tiles=T)
    compare(out.cpu().numpy(), ref, tol, "forward")
    compare(out2.cpu().numpy(), ref, tol, "forward with lse")
    compare_lse(lse.cpu().numpy(), ref_lse, tol, "lse")
    if P.workspace_bytes(c.B, c.H, c.I, c.N, c.D, T, P.TRI_ATTN_BF16 if c.dtype == "bf16" else P.TRI_ATTN_FP32) <= \
            P.noalloc_scratch_bytes():
        on = P.tri_attn_fwd_rows_noalloc(q, k, v, bias, m, n_key_tiles=T)
        t.cuda.synchronize()
        compare(on.cpu().numpy(), ref, tol, "forward without allocation")
    # the ring: T tile states folded by updates, the last step finalising
    bounds = [s * (c.N // T) + min(s, c.N % T) for s in range(T + 1)]
    if T == 1:
        acc, ms, ls = P.tri_attn_tile_state(q, k, v, bias, m, key_begin=0, key_end=c.N)
        orng, lrng = P.tri_attn_state_finalize(acc, ms, ls)
    else:
        acc, ms, ls = P.tri_attn_tile_state(q, k, v, bias, m, key_begin=bounds[0], key_end=bounds[1])
        for s in range(1, T - 1):
            P.tri_attn_tile_state_update(q, k, v, bias, m, key_begin=bounds[s], key_end=bounds[s + 1], acc=acc, m=ms,
                                         l=ls)
        orng, lrng = P.tri_attn_tile_state_final(q, k, v, bias, m, key_begin=bounds[T - 1], key_end=bounds[T],
                                                 acc=acc, m=ms, l=ls, want_lse=True)
    t.cuda.synchronize()
    compare(orng.cpu().numpy(), ref, tol, "ring")
    compare_lse(lrng.cpu().numpy(), ref_lse, tol, "ring lse")
    if c.I == c.N:
        oe = P.tri_attn_fwd_ending(q, k, v, bias, m, n_key_tiles=T)
        t.cuda.synchronize()
        re_, _ = oracle.tri_attn(w.q, w.k, w.v, w.bias, mask, n_key_tiles=T, ending=True)
        compare(oe.cpu().numpy(), re_, tol, "ending node")
    # attention with pair bias: the first row of the problem as the token sequence
    shp = (c.B, c.N, c.H, c.D)
    q1, k1, v1 = (x[:, 0].contiguous().view(shp) for x in (q, k, v))
    op, lp = P.pair_bias_attn_fwd(q1, k1, v1, bias, m, n_key_tiles=T, want_lse=True)
    t.cuda.synchronize()
    sl = lambda a: np.ascontiguousarray(a[:, :1])
    rp, rlp = oracle.tri_attn(sl(w.q), sl(w.k), sl(w.v), w.bias, mask, n_key_tiles=T)
    compare(op.cpu().numpy(), rp[:, 0], tol, "pair bias")
    compare_lse(lp.cpu().numpy(), rlp[:, 0], tol, "pair bias lse")
    # backward from the oracle's statistics
    dout = np.random.default_rng(700 + case).standard_normal(w.q.shape).astype(np.float32)
    g = P.tri_attn_bwd(q, k, v, bias, m, t.from_numpy(ref.astype(np.float32)).cuda(),
                       t.from_numpy(ref_lse.astype(np.float32)).cuda(), t.from_numpy(dout).cuda())
    t.cuda.synchronize()
    gref = oracle.tri_attn_bwd(w.q, w.k, w.v, w.bias, mask, dout)
    bar = 1e-2 if (c.dtype == "bf16" and c.D == 32) else 1e-4
    for name, a, r in zip(("dq", "dk", "dv", "dbias"), (x.cpu().numpy() for x in g), gref):
        compare(a, r, bar * max(1.0, float(np.max(np.abs(r)))), f"backward {name}")
