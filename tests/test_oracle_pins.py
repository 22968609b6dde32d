"""Pins of the fp64 oracle to things other than itself.

Each pin comes from the mathematics of the definition (Fold-CP, Table 1 'Triangle
Attention'; Figure 2(a): triangular bias shared across rows, ring steps joined by a
tiled-softmax merge), not from re-running the oracle's own formula:

  * a special case that reduces to a library routine: with the rows i and heads h
    batched, triangle attention IS scaled dot-product attention with an additive
    mask bias[b,h] + mask[b] -> torch's SDPA in float64 on the CPU;
  * the merge identity: the result does not depend on how the key axis is cut into
    ring steps, nor on which step runs first;
  * invariances: permuting the keys (k, v, bias columns and mask together) changes
    nothing, permuting the queries j permutes the output;
  * closed forms: uniform attention gives the mean of v, a single kept key copies its
    v, a constant added to a bias row changes nothing, outputs lie in the convex hull
    of the values, rows with no kept key give 0;
  * brute force at 60 significant digits (mpmath) on tiny inputs, over every
    contiguous tiling of the key axis;
  * the hand-derived worked examples in tests/golden/worked_examples.json.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def rand_case(rng, B=1, I=4, N=13, H=2, D=8, masked=(), sigma_b=1.0):
    q = rng.standard_normal((B, I, N, H, D)).astype(np.float32)
    k = rng.standard_normal((B, I, N, H, D)).astype(np.float32)
    v = rng.standard_normal((B, I, N, H, D)).astype(np.float32)
    bias = (sigma_b * rng.standard_normal((B, H, N, N))).astype(np.float32)
    mask = None
    if masked:
        mask = np.zeros((B, N), dtype=np.float32)
        mask[:, list(masked)] = -np.inf
    return q, k, v, bias, mask


def sdpa_reference(q, k, v, bias, mask):
    """torch.nn.functional.scaled_dot_product_attention (float64, CPU) with the rows i and
    heads h folded into the batch; the additive attention mask is bias[b,h] + mask[b]."""
    import torch
    B, I, N, H, D = q.shape
    def f64(x):
        from workloads import bf16_bits_to_f32
        x = bf16_bits_to_f32(x) if x.dtype == np.uint16 else x
        return torch.from_numpy(np.asarray(x, dtype=np.float64))
    Q = f64(q).permute(0, 1, 3, 2, 4)          # [B, I, H, N, D]
    K = f64(k).permute(0, 1, 3, 2, 4)
    V = f64(v).permute(0, 1, 3, 2, 4)
    M = f64(bias)[:, None]                      # [B, 1, H, N(j), N(k)]
    if mask is not None:
        M = M + torch.from_numpy(mask.astype(np.float64))[:, None, None, None, :]
    M = M.expand(B, I, H, N, N)
    out = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=M)
    return out.permute(0, 1, 3, 2, 4).numpy()   # [B, I, N, H, D]


# ---------------------------------------------------------------------------
# library special case
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("shape,masked,T", [
    (dict(B=1, I=5, N=37, H=3, D=16), (), 1),
    (dict(B=2, I=4, N=37, H=3, D=16), (0, 5, 36), 5),
    (dict(B=1, I=3, N=64, H=4, D=32), tuple(range(48, 64)), 4),
    (dict(B=1, I=7, N=20, H=1, D=1), (3,), 20),
])
def test_matches_library_sdpa(oracle_mod, shape, masked, T):
    rng = np.random.default_rng(11)
    q, k, v, bias, mask = rand_case(rng, masked=masked, sigma_b=2.0, **shape)
    out, _ = oracle_mod.tri_attn(q, k, v, bias, mask, n_key_tiles=T)
    ref = sdpa_reference(q, k, v, bias, mask)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_matches_library_sdpa_bf16_row_share(oracle_mod, wl):
    """bfloat16 inputs (widened exactly) and fewer query rows I than tokens N."""
    cfg = wl.custom_config(B=1, I=6, N=40, H=4, D=32, dtype="bf16", n_key_tiles=3, seed=7,
                           sigma_bias=2.0, mask_last=5)
    w = wl.make_inputs(cfg)
    out, _ = oracle_mod.tri_attn(w.q, w.k, w.v, w.bias, w.mask, n_key_tiles=3)
    ref = sdpa_reference(w.q, w.k, w.v, w.bias, w.mask)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_lse_matches_logsumexp(oracle_mod):
    from scipy.special import logsumexp
    rng = np.random.default_rng(3)
    q, k, v, bias, mask = rand_case(rng, B=1, I=3, N=21, H=2, D=8, masked=(2, 20))
    _, lse = oracle_mod.tri_attn(q, k, v, bias, mask, n_key_tiles=4)
    qd, kd = q.astype(np.float64), k.astype(np.float64)
    s = np.einsum("bijhd,bikhd->bijhk", qd, kd) / math.sqrt(8)
    s = s + np.transpose(bias.astype(np.float64), (0, 2, 1, 3))[:, None] + mask[:, None, None, None, :]
    np.testing.assert_allclose(lse, logsumexp(s, axis=-1), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# the merge identity: ring steps
# ---------------------------------------------------------------------------
def test_tile_count_invariance(oracle_mod):
    rng = np.random.default_rng(5)
    N = 29
    q, k, v, bias, mask = rand_case(rng, B=1, I=3, N=N, H=2, D=8, masked=(0, 1, 2, 28), sigma_b=3.0)
    base, base_lse = oracle_mod.tri_attn(q, k, v, bias, mask, n_key_tiles=1)
    for T in (2, 3, 5, 8, N):
        for first in sorted({0, T // 2, T - 1}):
            out, lse = oracle_mod.tri_attn(q, k, v, bias, mask, n_key_tiles=T, first_tile=first)
            np.testing.assert_allclose(out, base, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse, base_lse, rtol=0, atol=1e-12)


def test_uneven_partitions(oracle_mod):
    rng = np.random.default_rng(6)
    N = 31
    q, k, v, bias, mask = rand_case(rng, B=1, I=2, N=N, H=2, D=4, masked=(10, 11, 12))
    base, _ = oracle_mod.tri_attn(q, k, v, bias, mask, n_key_tiles=1)
    for _ in range(20):
        T = int(rng.integers(2, 12))
        cuts = np.sort(rng.choice(np.arange(1, N), size=T - 1, replace=False))
        starts = np.concatenate([[0], cuts, [N]])
        out, _ = oracle_mod.tri_attn(q, k, v, bias, mask, tile_starts=starts,
                                     first_tile=int(rng.integers(0, T)))
        np.testing.assert_allclose(out, base, rtol=0, atol=1e-12)


def test_even_tiles_rule(oracle_mod):
    """Near-equal contiguous tiles: first N mod T tiles hold ceil(N/T) keys."""
    s = oracle_mod.even_tiles(2700, 8)
    assert s.tolist() == [0, 338, 676, 1014, 1352, 1689, 2026, 2363, 2700]
    for N in (1, 7, 64, 255, 1000):
        for T in range(1, min(N, 17) + 1):
            s = oracle_mod.even_tiles(N, T)
            sizes = np.diff(s)
            assert s[0] == 0 and s[-1] == N and len(sizes) == T
            assert sizes.max() - sizes.min() <= 1 and np.all(sizes[:-1] >= sizes[1:])
            assert np.array_equal(sizes, [len(c) for c in np.array_split(np.arange(N), T)])


# ---------------------------------------------------------------------------
# invariances
# ---------------------------------------------------------------------------
def test_key_permutation_invariance(oracle_mod):
    rng = np.random.default_rng(8)
    N = 23
    q, k, v, bias, mask = rand_case(rng, B=2, I=3, N=N, H=2, D=8, masked=(4, 9))
    base, base_lse = oracle_mod.tri_attn(q, k, v, bias, mask, n_key_tiles=3)
    perm = rng.permutation(N)
    out, lse = oracle_mod.tri_attn(q, k[:, :, perm], v[:, :, perm], bias[..., perm],
                                   mask[:, perm], n_key_tiles=4)
    np.testing.assert_allclose(out, base, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, base_lse, rtol=0, atol=1e-12)


def test_query_permutation_equivariance(oracle_mod):
    rng = np.random.default_rng(9)
    N = 19
    q, k, v, bias, mask = rand_case(rng, B=1, I=2, N=N, H=3, D=8)
    base, _ = oracle_mod.tri_attn(q, k, v, bias, mask, n_key_tiles=2)
    perm = rng.permutation(N)
    out, _ = oracle_mod.tri_attn(q[:, :, perm], k, v, bias[:, :, perm, :], mask, n_key_tiles=2)
    np.testing.assert_allclose(out, base[:, :, perm], rtol=0, atol=1e-12)


def test_row_and_head_independence(oracle_mod):
    """Changing row i' or head h' leaves every other (i, h) untouched; the bias is
    shared by all rows, so it may only change when the bias itself changes."""
    rng = np.random.default_rng(10)
    q, k, v, bias, mask = rand_case(rng, B=1, I=4, N=11, H=3, D=4)
    base, _ = oracle_mod.tri_attn(q, k, v, bias, mask)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[:, 1] += 1.0; k2[:, 1] *= -1.0; v2[:, 1] += 5.0
    out, _ = oracle_mod.tri_attn(q2, k2, v2, bias, mask)
    assert not np.allclose(out[:, 1], base[:, 1])
    np.testing.assert_array_equal(np.delete(out, 1, axis=1), np.delete(base, 1, axis=1))
    k3, v3, b3 = k.copy(), v.copy(), bias.copy()
    k3[..., 2, :] *= 3.0; v3[..., 2, :] -= 1.0; b3[:, 2] += rng.standard_normal((11, 11)).astype(np.float32)
    out, _ = oracle_mod.tri_attn(q, k3, v3, b3, mask)
    assert not np.allclose(out[..., 2, :], base[..., 2, :])
    np.testing.assert_array_equal(out[..., :2, :], base[..., :2, :])


def test_bias_is_shared_across_rows(oracle_mod):
    """Rows i with identical q, k, v produce identical outputs: the bias carries no i."""
    rng = np.random.default_rng(12)
    q, k, v, bias, mask = rand_case(rng, B=1, I=1, N=15, H=2, D=8)
    rep = lambda x: np.repeat(x, 5, axis=1)
    out, _ = oracle_mod.tri_attn(rep(q), rep(k), rep(v), bias, mask, n_key_tiles=3)
    for i in range(1, 5):
        np.testing.assert_array_equal(out[:, i], out[:, 0])


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------
def test_uniform_attention_is_mean_of_v(oracle_mod):
    rng = np.random.default_rng(13)
    B, I, N, H, D = 2, 3, 17, 2, 8
    z = np.zeros((B, I, N, H, D), np.float32)
    v = rng.standard_normal((B, I, N, H, D)).astype(np.float32)
    bias = np.zeros((B, H, N, N), np.float32)
    out, lse = oracle_mod.tri_attn(z, z, v, bias, None, n_key_tiles=4)
    mean = v.astype(np.float64).mean(axis=2, keepdims=True)
    np.testing.assert_allclose(out, np.broadcast_to(mean, out.shape), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, math.log(N), rtol=0, atol=1e-14)
    keep = np.ones(N, bool); keep[[0, 3, 16]] = False
    mask = np.where(keep, 0.0, -np.inf).astype(np.float32)[None].repeat(B, 0)
    out, lse = oracle_mod.tri_attn(z, z, v, bias, mask, n_key_tiles=5)
    mean = v.astype(np.float64)[:, :, keep].mean(axis=2, keepdims=True)
    np.testing.assert_allclose(out, np.broadcast_to(mean, out.shape), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, math.log(keep.sum()), rtol=0, atol=1e-14)


def test_single_kept_key_copies_value(oracle_mod):
    rng = np.random.default_rng(14)
    q, k, v, bias, _ = rand_case(rng, B=1, I=3, N=9, H=2, D=4, sigma_b=5.0)
    mask = np.full((1, 9), -np.inf, np.float32)
    mask[0, 6] = 0.0
    for T in (1, 3, 9):
        out, _ = oracle_mod.tri_attn(q, k, v, bias, mask, n_key_tiles=T)
        np.testing.assert_array_equal(out, np.broadcast_to(v[:, :, 6:7].astype(np.float64), out.shape))


def test_bias_row_shift_invariance(oracle_mod):
    """softmax over k ignores a constant per (h, j): huge shifts (+-800) must not
    overflow or underflow, which also pins the subtraction of the running maximum."""
    rng = np.random.default_rng(15)
    q, k, v, bias, mask = rand_case(rng, B=1, I=3, N=14, H=2, D=8, masked=(13,))
    bias = np.round(bias * 256) / 256          # on a 2^-8 grid, so bias + 800 stays exact in fp32
    base, base_lse = oracle_mod.tri_attn(q, k, v, bias, mask, n_key_tiles=3)
    shift = rng.choice([-800.0, 800.0, 37.0], size=(1, 2, 14, 1)).astype(np.float32)
    out, lse = oracle_mod.tri_attn(q, k, v, bias + shift, mask, n_key_tiles=3)
    np.testing.assert_allclose(out, base, rtol=0, atol=1e-10)
    np.testing.assert_allclose(lse, base_lse + shift[0].transpose(1, 0, 2)[None, None, :, :, 0],
                               rtol=0, atol=1e-10)


def test_output_in_convex_hull_of_values(oracle_mod):
    rng = np.random.default_rng(16)
    q, k, v, bias, mask = rand_case(rng, B=1, I=4, N=25, H=2, D=8, sigma_b=4.0, masked=(7,))
    out, _ = oracle_mod.tri_attn(q, k, v, bias, mask, n_key_tiles=6)
    vk = np.delete(v.astype(np.float64), 7, axis=2)
    lo, hi = vk.min(axis=2, keepdims=True), vk.max(axis=2, keepdims=True)
    assert np.all(out >= lo - 1e-13) and np.all(out <= hi + 1e-13)


def test_fully_masked_row_gives_zero(oracle_mod):
    rng = np.random.default_rng(17)
    q, k, v, bias, _ = rand_case(rng, B=2, I=2, N=6, H=2, D=4)
    mask = np.zeros((2, 6), np.float32)
    mask[1, :] = -np.inf
    for T in (1, 2, 6):
        out, lse = oracle_mod.tri_attn(q, k, v, bias, mask, n_key_tiles=T)
        assert np.all(out[1] == 0.0) and np.all(np.isneginf(lse[1]))
        assert np.all(np.isfinite(out[0])) and np.all(np.isfinite(lse[0]))


def test_row_subset_matches_full(oracle_mod):
    rng = np.random.default_rng(18)
    B, I, N = 2, 3, 10
    q, k, v, bias, mask = rand_case(rng, B=B, I=I, N=N, H=2, D=4, masked=(9,))
    full, full_lse = oracle_mod.tri_attn(q, k, v, bias, mask, n_key_tiles=2)
    rows = rng.choice(B * I * N, size=17, replace=False)
    out, lse = oracle_mod.tri_attn(q, k, v, bias, mask, n_key_tiles=2, rows=rows)
    np.testing.assert_array_equal(out, full.reshape(B * I * N, 2, 4)[rows])
    np.testing.assert_array_equal(lse, full_lse.reshape(B * I * N, 2)[rows])


# ---------------------------------------------------------------------------
# brute force at high precision
# ---------------------------------------------------------------------------
def mp_direct(q, k, v, bias, mask, digits=60):
    """The definition, term by term, in mpmath at `digits` significant digits."""
    import mpmath
    mpmath.mp.dps = digits
    B, I, N, H, D = q.shape
    out = np.empty(q.shape, dtype=object)
    lse = np.empty((B, I, N, H), dtype=object)
    for b, i, j, h in itertools.product(range(B), range(I), range(N), range(H)):
        s = []
        for kk in range(N):
            dot = mpmath.fsum(mpmath.mpf(float(q[b, i, j, h, d])) * mpmath.mpf(float(k[b, i, kk, h, d]))
                              for d in range(D))
            sc = dot / mpmath.sqrt(D) + mpmath.mpf(float(bias[b, h, j, kk]))
            if mask is not None and mask[b, kk] == -np.inf:
                continue
            if mask is not None:
                sc += mpmath.mpf(float(mask[b, kk]))
            s.append((kk, sc))
        w = [(kk, mpmath.exp(sc)) for kk, sc in s]
        l = mpmath.fsum(x for _, x in w)
        for d in range(D):
            out[b, i, j, h, d] = mpmath.fsum(x * mpmath.mpf(float(v[b, i, kk, h, d])) for kk, x in w) / l
        lse[b, i, j, h] = mpmath.log(l)
    return out, lse


@pytest.mark.parametrize("N", [1, 2, 3, 5, 6])
def test_brute_force_every_tiling(oracle_mod, N):
    rng = np.random.default_rng(100 + N)
    masked = (N - 1,) if N >= 3 else ()
    q, k, v, bias, mask = rand_case(rng, B=1, I=min(2, N), N=N, H=2, D=3, masked=masked, sigma_b=3.0)
    ref, ref_lse = mp_direct(q, k, v, bias, mask)
    ref = ref.astype(np.float64)
    ref_lse = ref_lse.astype(np.float64)
    for cut_bits in range(2 ** (N - 1)):   # every contiguous tiling of N keys
        cuts = [c for c in range(1, N) if cut_bits >> (c - 1) & 1]
        starts = np.array([0] + cuts + [N])
        for first in range(len(starts) - 1):
            out, lse = oracle_mod.tri_attn(q, k, v, bias, mask, tile_starts=starts, first_tile=first)
            np.testing.assert_allclose(out, ref, rtol=0, atol=1e-13)
            np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# hand-derived worked examples
# ---------------------------------------------------------------------------
def _num(x):
    if isinstance(x, (int, float)):
        return float(x)
    table = {"-inf": -math.inf, "ln2": math.log(2), "ln3": math.log(3), "2+ln3": 2 + math.log(3),
             "5+ln2": 5 + math.log(2), "2+ln2": 2 + math.log(2), "1": 1.0, "-3": -3.0,
             "2": 2.0, "2^-133": 2.0 ** -133, "255*2^120": 255.0 * 2.0 ** 120}
    return table[x]


def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_worked_examples(oracle_mod, case):
    B, I, N, H, D = (case[x] for x in "BINHD")
    mask = None
    if case.get("mask") is not None:
        mask = np.array([[_num(x) for x in case["mask"]]], dtype=np.float32)
    if case["name"] == "single_kept_key_copies_its_value_bf16":
        bits = lambda s: int(s, 16)
        q = np.full((B, I, N, H, D), bits(case["q_bits"]), np.uint16)
        k = np.full((B, I, N, H, D), bits(case["k_bits"]), np.uint16)
        v = np.full((B, I, N, H, D), bits(case["v_other_bits"]), np.uint16)
        for h in range(H):
            v[0, 0, 2, h] = [bits(s) for s in case["v_key2_bits"][h]]
        bias = np.full((B, H, N, N), bits(case["bias_bits"]), np.uint16)
        expect = np.array([[_num(x) for x in row] for row in case["out_per_head"]])
        expect = np.broadcast_to(expect, (B, I, N, H, D))
        expect_lse = np.full((B, I, N, H), _num(case["lse"]))
    elif case["name"] == "fully_masked_ring_step_is_merge_identity":
        z = np.zeros((B, I, N, H, D), np.float32)
        q = k = z
        v = np.array(case["v"], np.float32).reshape(B, I, N, H, D)
        bias = np.zeros((B, H, N, N), np.float32)
        expect = np.broadcast_to(np.array(case["out"], np.float64), (B, I, N, H, D))
        expect_lse = np.full((B, I, N, H), _num(case["lse"]))
    else:
        q = np.array(case["q"], np.float32).reshape(B, I, N, H, D)
        k = np.array(case["k"], np.float32).reshape(B, I, N, H, D)
        v = np.array(case["v"], np.float32).reshape(B, I, N, H, D)
        # v is given per key; every row j sees the same keys
        bias = np.array(case["bias"], np.float32).reshape(B, H, N, N)
        expect = np.array(case["out"], np.float64).reshape(B, I, N, H, D)
        expect_lse = np.array([_num(x) for x in case["lse"]]).reshape(B, I, N, H)
    for T in case["n_key_tiles"]:
        for first in range(T):
            out, lse = oracle_mod.tri_attn(q, k, v, bias, mask, n_key_tiles=T, first_tile=first)
            np.testing.assert_allclose(out, expect, rtol=1e-15, atol=1e-15)
            np.testing.assert_allclose(lse, expect_lse, rtol=0, atol=1e-14)
