"""GPU parity of the backward (tri_attn_bwd) against the fp64 oracle's gradients.

Bars, stated relative to the largest reference gradient of the tensor (gradients of
the bias are sums over every row i and grow with I):
  * the kernels alone, fed the oracle's exact forward statistics (out, lse rounded to
    fp32): the fp32 path (fp32 inputs, or bf16 with D != 32) computes in fp32 throughout,
    max |gpu - oracle| <= 1e-4 * max(1, max|oracle|) over sums of up to N*I terms; the
    matrix-core path (bf16, D == 32) rounds dout, P and dS to bf16 as product operands
    (relative 2^-9 each), so its bar is the bf16 one, 1e-2 * max(1, max|oracle|);
  * end to end, from the GPU's own forward (tri_attn_fwd_lse): the fp32 path keeps 1e-4;
    the bf16 path also inherits the forward's error (|out| and |lse| errors up to
    ~5e-3), so its bar is 2e-2 * max(1, max|oracle|).
"""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.test_parity_gpu import say, to_dev

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dbias")


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import pair_biased_triangle_amd as P
    P.load_library()
    return torch


def case(dtype, I, N, D, seed=51, mask_last=5, B=1, H=4):
    w = W.make_inputs(W.custom_config(B=B, I=I, N=N, H=H, D=D, dtype=dtype, n_key_tiles=1, seed=seed,
                                      sigma_bias=2.0, mask_last=mask_last))
    dout = np.random.default_rng(seed + 1).standard_normal(w.q.shape).astype(np.float32)
    return w, dout


def compare_rel(got, ref, rel, what):
    scale = max(1.0, float(np.max(np.abs(ref))))
    err = float(np.max(np.abs(got.astype(np.float64) - ref)))
    say(f"  {what}: max|err| = {err:.3e}, bar {rel:g} * {scale:.3g}")
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    assert err <= rel * scale, f"{what}: {err:.3e} > {rel * scale:.3e}"


def gpu_bwd(torch, w, dout, out, lse):
    import pair_biased_triangle_amd as P
    q, k, v, bias, mask = (to_dev(torch, x) for x in (w.q, w.k, w.v, w.bias, w.mask))
    g = P.tri_attn_bwd(q, k, v, bias, mask, out, lse, torch.from_numpy(dout).cuda())
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in g]


@pytest.mark.parametrize("dtype,I,N,D,bar", [("bf16", 20, 130, 32, 1e-2), ("bf16", 7, 33, 32, 1e-2),
                                             ("bf16", 2, 300, 32, 1e-2), ("fp32", 9, 70, 16, 1e-4),
                                             ("fp32", 5, 33, 64, 1e-4), ("bf16", 3, 200, 48, 1e-4),
                                             ("fp32", 4, 40, 32, 1e-4)])
def test_kernels_with_exact_statistics(torch_dev, dtype, I, N, D, bar):
    w, dout = case(dtype, I, N, D)
    say(f"[bwd] exact statistics {dtype} I={I} N={N} D={D}")
    out, lse = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask)
    got = gpu_bwd(torch_dev, w, dout, torch_dev.from_numpy(out.astype(np.float32)).cuda(),
                  torch_dev.from_numpy(lse.astype(np.float32)).cuda())
    ref = oracle.tri_attn_bwd(w.q, w.k, w.v, w.bias, w.mask, dout)
    for n, g, r in zip(NAMES, got, ref):
        compare_rel(g, r, bar, f"{n} {dtype} D={D}")


def test_several_batches_heads_and_tiles(torch_dev):
    """B = 2, H = 3 and N = 520: three 256-query dbias tiles (the last one ragged), five
    128-key tiles, and rows of the second batch element, with exact statistics."""
    w, dout = case("bf16", 3, 520, 32, seed=77, mask_last=9, B=2, H=3)
    say("[bwd] exact statistics bf16 B=2 H=3 I=3 N=520")
    out, lse = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask)
    got = gpu_bwd(torch_dev, w, dout, torch_dev.from_numpy(out.astype(np.float32)).cuda(),
                  torch_dev.from_numpy(lse.astype(np.float32)).cuda())
    ref = oracle.tri_attn_bwd(w.q, w.k, w.v, w.bias, w.mask, dout)
    for n, g, r in zip(NAMES, got, ref):
        compare_rel(g, r, 1e-2, f"{n} bf16 B=2 H=3 N=520")


@pytest.mark.parametrize("dtype,I,N,D,bar", [("bf16", 24, 160, 32, 2e-2), ("fp32", 12, 96, 32, 1e-4)])
def test_end_to_end(torch_dev, dtype, I, N, D, bar):
    import pair_biased_triangle_amd as P
    w, dout = case(dtype, I, N, D, seed=61)
    say(f"[bwd] end to end {dtype} I={I} N={N}")
    q, k, v, bias, mask = (to_dev(torch_dev, x) for x in (w.q, w.k, w.v, w.bias, w.mask))
    out, lse = P.tri_attn_fwd_lse(q, k, v, bias, mask, n_key_tiles=3)
    got = gpu_bwd(torch_dev, w, dout, out, lse)
    ref = oracle.tri_attn_bwd(w.q, w.k, w.v, w.bias, w.mask, dout)
    for n, g, r in zip(NAMES, got, ref):
        compare_rel(g, r, bar, f"{n} {dtype}")


@pytest.mark.parametrize("dtype,bar", [("fp32", 1e-4), ("bf16", 1e-2)])
def test_masked_rows_and_keys(torch_dev, dtype, bar):
    """Dropped keys get no gradient; a batch element whose keys are all dropped gets none."""
    w, dout = case(dtype, 6, 40, 32, B=2, mask_last=0)
    mask = np.zeros((2, 40), dtype=np.float32)
    mask[0, [3, 17, 39]] = -np.inf
    mask[1, :] = -np.inf
    out, lse = oracle.tri_attn(w.q, w.k, w.v, w.bias, mask)
    import pair_biased_triangle_amd as P
    t = torch_dev
    q, k, v, bias = (to_dev(t, x) for x in (w.q, w.k, w.v, w.bias))
    g = P.tri_attn_bwd(q, k, v, bias, to_dev(t, mask), t.from_numpy(out.astype(np.float32)).cuda(),
                       t.from_numpy(lse.astype(np.float32)).cuda(), t.from_numpy(dout).cuda())
    t.cuda.synchronize()
    dq, dk, dv, dbias = (x.cpu().numpy() for x in g)
    for x in (dq[1], dk[1], dv[1], dbias[1]):
        assert np.all(x == 0)
    assert np.all(dk[0][:, [3, 17, 39]] == 0) and np.all(dv[0][:, [3, 17, 39]] == 0)
    assert np.all(dbias[0][..., [3, 17, 39]] == 0)
    ref = oracle.tri_attn_bwd(w.q, w.k, w.v, w.bias, mask, dout)
    for n, a, r in zip(NAMES, (dq, dk, dv, dbias), ref):
        compare_rel(a, r, bar, f"masked {n} {dtype}")


@pytest.mark.parametrize("dtype,bar", [("fp32", 1e-4), ("bf16", 1e-2)])
def test_row_shares_add_up(torch_dev, dtype, bar):
    """dbias of a row share is that share's sum: two halves add to the whole."""
    import pair_biased_triangle_amd as P
    w, dout = case(dtype, 16, 64, 32, seed=71)
    out, lse = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask)
    t = torch_dev
    parts = []
    for lo, hi in ((0, 7), (7, 16)):
        sl = lambda x: np.ascontiguousarray(x[:, lo:hi])
        q, k, v = (to_dev(t, sl(x)) for x in (w.q, w.k, w.v))
        g = P.tri_attn_bwd(q, k, v, to_dev(t, w.bias), to_dev(t, w.mask),
                           t.from_numpy(sl(out).astype(np.float32)).cuda(),
                           t.from_numpy(sl(lse).astype(np.float32)).cuda(), t.from_numpy(sl(dout)).cuda())
        parts.append(g[3].cpu().numpy().astype(np.float64))
    ref = oracle.tri_attn_bwd(w.q, w.k, w.v, w.bias, w.mask, dout)[3]
    compare_rel(parts[0] + parts[1], ref, bar, f"dbias of two row shares {dtype}")


def test_autograd_function(torch_dev):
    """triangle_attention() differentiates through the same kernels."""
    import pair_biased_triangle_amd as P
    t = torch_dev
    w, dout = case("fp32", 8, 48, 32, seed=81)
    q, k, v, bias = (to_dev(t, x).requires_grad_(True) for x in (w.q, w.k, w.v, w.bias))
    out = P.triangle_attention(q, k, v, bias, to_dev(t, w.mask), n_key_tiles=2)
    out.backward(t.from_numpy(dout).cuda())
    t.cuda.synchronize()
    ref = oracle.tri_attn_bwd(w.q, w.k, w.v, w.bias, w.mask, dout)
    for n, x, r in zip(NAMES, (q, k, v, bias), ref):
        compare_rel(x.grad.cpu().numpy(), r, 1e-4, f"autograd {n}")


@pytest.mark.parametrize("deep", [False, True])
def test_soft_mask_and_shifted_bias(torch_dev, deep):
    """A mask of finite values (keys in [-4, 0], none dropped) and one head's bias shifted
    by +50: the matrix-core dbias multiplies its row sums by 2^((bias + mask - r_j) log2 e)
    at the end, so a mask that is neither 0 nor -inf and a bias far from 0 both pass
    through that factor.  With `deep`, every seventh key's mask is -30 instead: finite
    values further below the row's reference than the fp16 bias image spans, which sends
    those columns to the fp32 kernels.  Exact statistics, bf16 bar."""
    import pair_biased_triangle_amd as P
    t = torch_dev
    w = W.make_inputs(W.custom_config(B=1, I=8, N=300, H=4, D=32, dtype="bf16", n_key_tiles=1, seed=91,
                                      sigma_bias=1.0, mask_last=0))
    bias = W.bf16_bits_to_f32(w.bias)
    bias[0, 2] += 50.0
    w.bias = W.f32_to_bf16_bits(bias)
    mask = (-4.0 * np.random.default_rng(92).random((1, 300))).astype(np.float32)
    if deep:
        mask[0, ::7] = -30.0
    dout = np.random.default_rng(93).standard_normal(w.q.shape).astype(np.float32)
    say(f"[bwd] soft mask{' with deep keys' if deep else ''}, head 2 shifted by +50, bf16 I=8 N=300")
    out, lse = oracle.tri_attn(w.q, w.k, w.v, w.bias, mask)
    q, k, v, b = (to_dev(t, x) for x in (w.q, w.k, w.v, w.bias))
    g = P.tri_attn_bwd(q, k, v, b, to_dev(t, mask), t.from_numpy(out.astype(np.float32)).cuda(),
                       t.from_numpy(lse.astype(np.float32)).cuda(), t.from_numpy(dout).cuda())
    t.cuda.synchronize()
    ref = oracle.tri_attn_bwd(w.q, w.k, w.v, w.bias, mask, dout)
    for n, a, r in zip(NAMES, (x.cpu().numpy() for x in g), ref):
        compare_rel(a, r, 1e-2, f"soft mask{' deep' if deep else ''} {n} bf16")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_dbias_rows_sum_to_zero(torch_dev, dtype):
    """sum_k ds_k = sum_k p_k (dp_k - delta) = 0 when delta = dout . out and out = sum_k p_k v_k.
    Fed the oracle's exact statistics, the matrix-core path forms delta from the same
    bf16-rounded dout as its dP products, so each dbias row sums to zero up to fp32
    rounding, far inside the gradient's own bar: |row sum| <= 1e-4 of the row's sum of
    magnitudes (the fp32 path likewise)."""
    import pair_biased_triangle_amd as P
    t = torch_dev
    w, dout = case(dtype, 8, 300, 32, seed=95, mask_last=7)
    out, lse = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask)
    say(f"[bwd] dbias row sums, {dtype}")
    q, k, v, b, m = (to_dev(t, x) for x in (w.q, w.k, w.v, w.bias, w.mask))
    g = P.tri_attn_bwd(q, k, v, b, m, t.from_numpy(out.astype(np.float32)).cuda(),
                       t.from_numpy(lse.astype(np.float32)).cuda(), t.from_numpy(dout).cuda())
    t.cuda.synchronize()
    db = g[3].cpu().numpy().astype(np.float64)
    worst = float(np.max(np.abs(db.sum(axis=-1)) / np.maximum(np.abs(db).sum(axis=-1), 1e-30)))
    say(f"  max |row sum| / sum |.| = {worst:.3e} (bar 1e-4)")
    assert worst <= 1e-4
