"""Pins of the oracle's ending-node orientation, its ring-step states and the merge.

  * ending node ("Fold-CP", Figure 2(a): the pair tensor is transposed across its axes
    before the ring): with the columns j and heads h batched it IS scaled dot-product
    attention over the rows, with the transposed bias -> torch's SDPA in float64; and
    it equals the starting-node result on the swapped tensors; and an mpmath brute
    force of its own formula agrees;
  * ring-step states (Figure 2(a)/(c), Table 1's caption): the state of the whole key
    axis, finalised, is the forward; the states of any partition merged in any order
    give the same result; a range with no finite score is the identity of the merge;
    the range's maximum weight is exactly 1;
  * the merge rule itself, on two states, against mpmath;
  * attention with pair bias (Table 1, Figure 2(c)) is the single-row case, pinned to
    SDPA on [B, H, N, D].
"""
import itertools
import math

import numpy as np
import pytest

from tests.test_oracle_pins import rand_case, sdpa_reference


def swap(x):
    """Swap the two pair axes of a [B, N, N, ...] tensor."""
    return np.ascontiguousarray(np.swapaxes(x, 1, 2))


def sdpa_ending(q, k, v, bias, mask):
    """Ending node through the library routine: per (b, column j, h) the queries are the
    rows i, the keys the rows k of the same column, the additive mask bias[b,h,k,i]."""
    return swap(sdpa_reference(swap(q), swap(k), swap(v), np.ascontiguousarray(np.swapaxes(bias, 2, 3)), mask))


# ---------------------------------------------------------------------------
# ending node
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("N,masked,T,dtype", [(11, (), 1, "f32"), (17, (0, 16), 4, "f32"), (13, (3,), 13, "bf16")])
def test_ending_matches_library_sdpa(oracle_mod, N, masked, T, dtype):
    from workloads import bf16_bits_to_f32, f32_to_bf16_bits
    rng = np.random.default_rng(40 + N)
    q, k, v, bias, mask = rand_case(rng, B=2, I=N, N=N, H=3, D=8, masked=masked, sigma_b=2.0)
    if dtype == "bf16":
        q, k, v, bias = (f32_to_bf16_bits(x) for x in (q, k, v, bias))
    out, _ = oracle_mod.tri_attn(q, k, v, bias, mask, n_key_tiles=T, ending=True)
    if dtype == "bf16":
        q, k, v, bias = (bf16_bits_to_f32(x) for x in (q, k, v, bias))
    np.testing.assert_allclose(out, sdpa_ending(q, k, v, bias, mask), rtol=0, atol=1e-12)


def test_ending_is_starting_on_swapped_axes(oracle_mod):
    rng = np.random.default_rng(4)
    q, k, v, bias, mask = rand_case(rng, B=1, I=10, N=10, H=2, D=4, masked=(9,), sigma_b=1.5)
    out, lse = oracle_mod.tri_attn(q, k, v, bias, mask, n_key_tiles=3, ending=True)
    ref, ref_lse = oracle_mod.tri_attn(swap(q), swap(k), swap(v), np.ascontiguousarray(np.swapaxes(bias, 2, 3)),
                                       mask, n_key_tiles=3)
    np.testing.assert_allclose(out, swap(ref), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, swap(ref_lse), rtol=0, atol=1e-13)


def test_ending_differs_from_starting(oracle_mod):
    """The orientation matters: a pin that both orientations passed would pin neither."""
    rng = np.random.default_rng(6)
    q, k, v, bias, mask = rand_case(rng, B=1, I=6, N=6, H=1, D=4)
    a, _ = oracle_mod.tri_attn(q, k, v, bias, mask, ending=True)
    b, _ = oracle_mod.tri_attn(q, k, v, bias, mask)
    assert np.max(np.abs(a - b)) > 0.1


def mp_ending(q, k, v, bias, mask, digits=50):
    """The ending-node definition, term by term, in mpmath."""
    import mpmath
    mpmath.mp.dps = digits
    B, N, _, H, D = q.shape
    out = np.empty(q.shape, dtype=object)
    for b, i, j, h in itertools.product(range(B), range(N), range(N), range(H)):
        w = []
        for kk in range(N):
            if mask is not None and mask[b, kk] == -np.inf:
                continue
            dot = mpmath.fsum(mpmath.mpf(float(q[b, i, j, h, d])) * mpmath.mpf(float(k[b, kk, j, h, d]))
                              for d in range(D))
            sc = dot / mpmath.sqrt(D) + mpmath.mpf(float(bias[b, h, kk, i]))
            if mask is not None:
                sc += mpmath.mpf(float(mask[b, kk]))
            w.append((kk, mpmath.exp(sc)))
        l = mpmath.fsum(x for _, x in w)
        for d in range(D):
            out[b, i, j, h, d] = mpmath.fsum(x * mpmath.mpf(float(v[b, kk, j, h, d])) for kk, x in w) / l
    return out.astype(np.float64)


@pytest.mark.parametrize("N", [1, 3, 4])
def test_ending_brute_force(oracle_mod, N):
    rng = np.random.default_rng(70 + N)
    q, k, v, bias, mask = rand_case(rng, B=1, I=N, N=N, H=2, D=3, masked=(N - 1,) if N > 2 else (), sigma_b=3.0)
    ref = mp_ending(q, k, v, bias, mask)
    for T in range(1, N + 1):
        out, _ = oracle_mod.tri_attn(q, k, v, bias, mask, n_key_tiles=T, ending=True)
        np.testing.assert_allclose(out, ref, rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# ring-step states and the merge
# ---------------------------------------------------------------------------
def test_whole_range_state_is_the_forward(oracle_mod):
    rng = np.random.default_rng(8)
    q, k, v, bias, mask = rand_case(rng, B=2, I=3, N=19, H=2, D=8, masked=(0, 18), sigma_b=2.0)
    acc, m, l = oracle_mod.tile_state(q, k, v, bias, mask, key_begin=0, key_end=19)
    out, lse = oracle_mod.finalize_states(acc, m, l)
    ref, ref_lse = oracle_mod.tri_attn(q, k, v, bias, mask)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-13)


def test_state_reference_is_the_range_maximum(oracle_mod):
    """m is the largest score of the range, so the largest weight is exactly 1 and l >= 1."""
    rng = np.random.default_rng(9)
    q, k, v, bias, mask = rand_case(rng, B=1, I=2, N=15, H=2, D=4, sigma_b=2.0)
    acc, m, l = oracle_mod.tile_state(q, k, v, bias, mask, key_begin=4, key_end=11)
    qd, kd = q.astype(np.float64), k.astype(np.float64)
    s = np.einsum("bijhd,bikhd->bijhk", qd, kd)[..., 4:11] / 2.0
    s = s + np.transpose(bias.astype(np.float64), (0, 2, 1, 3))[:, None, ..., 4:11]
    np.testing.assert_allclose(m, s.max(axis=-1), rtol=0, atol=1e-13)
    assert np.all(l >= 1.0)


@pytest.mark.parametrize("seed", range(4))
def test_states_of_any_partition_merge_to_the_forward(oracle_mod, seed):
    rng = np.random.default_rng(200 + seed)
    N = 23
    ending = seed % 2 == 1
    I = N if ending else 4
    q, k, v, bias, mask = rand_case(rng, B=1, I=I, N=N, H=2, D=8, masked=(1, 2, 3), sigma_b=2.5)
    cuts = np.sort(rng.choice(np.arange(1, N), size=rng.integers(1, 6), replace=False))
    bounds = [0, *cuts.tolist(), N]
    parts = list(zip(bounds[:-1], bounds[1:]))
    rng.shuffle(parts)                       # a ring may start anywhere
    st = None
    for lo, hi in parts:
        s = oracle_mod.tile_state(q, k, v, bias, mask, key_begin=lo, key_end=hi, ending=ending)
        st = s if st is None else oracle_mod.merge_states(*st, *s)
    out, lse = oracle_mod.finalize_states(*st)
    ref, ref_lse = oracle_mod.tri_attn(q, k, v, bias, mask, ending=ending)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


def test_masked_range_is_the_identity(oracle_mod):
    rng = np.random.default_rng(10)
    q, k, v, bias, mask = rand_case(rng, B=1, I=2, N=12, H=2, D=4, masked=(5, 6, 7))
    acc, m, l = oracle_mod.tile_state(q, k, v, bias, mask, key_begin=5, key_end=8)
    assert np.all(acc == 0) and np.all(m == -np.inf) and np.all(l == 0)
    a2, m2, l2 = oracle_mod.tile_state(q, k, v, bias, mask, key_begin=0, key_end=5)
    for merged in (oracle_mod.merge_states(a2, m2, l2, acc, m, l), oracle_mod.merge_states(acc, m, l, a2, m2, l2)):
        np.testing.assert_array_equal(merged[0], a2)
        np.testing.assert_array_equal(merged[1], m2)
        np.testing.assert_array_equal(merged[2], l2)


def test_merge_rule_against_mpmath(oracle_mod):
    """Two hand-made states of one query: the merged (acc, l) relative to the merged m
    equals the exact sum of the two ranges' weights."""
    import mpmath
    mpmath.mp.dps = 40
    a1, m1, l1 = np.array([[0.5, -2.0]]), np.array([3.0]), np.array([1.75])
    a2, m2, l2 = np.array([[1.25, 4.0]]), np.array([-1.5]), np.array([2.5])
    acc, m, l = oracle_mod.merge_states(a1, m1, l1, a2, m2, l2)
    assert m[0] == 3.0
    e = mpmath.exp(mpmath.mpf(-1.5) - 3)
    assert abs(l[0] - float(mpmath.mpf(1.75) + e * mpmath.mpf(2.5))) < 1e-15
    for d, (x1, x2) in enumerate(zip(a1[0], a2[0])):
        assert abs(acc[0, d] - float(mpmath.mpf(x1) + e * mpmath.mpf(x2))) < 1e-15
    out, lse = oracle_mod.finalize_states(acc, m, l)
    assert abs(lse[0] - float(3 + mpmath.log(mpmath.mpf(1.75) + e * mpmath.mpf(2.5)))) < 1e-14


# ---------------------------------------------------------------------------
# attention with pair bias: one row
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("masked,T", [((), 1), ((0, 30), 6)])
def test_pair_bias_attention_is_the_single_row_case(oracle_mod, masked, T):
    import torch
    rng = np.random.default_rng(12)
    B, N, H, D = 2, 31, 3, 16
    q, k, v, bias, mask = rand_case(rng, B=B, I=1, N=N, H=H, D=D, masked=masked, sigma_b=2.0)
    out, lse = oracle_mod.tri_attn(q, k, v, bias, mask, n_key_tiles=T)
    Q, K, V = (torch.from_numpy(x[:, 0].astype(np.float64)).permute(0, 2, 1, 3) for x in (q, k, v))   # [B,H,N,D]
    M = torch.from_numpy(bias.astype(np.float64))
    if mask is not None:
        M = M + torch.from_numpy(mask.astype(np.float64))[:, None, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=M).permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(out[:, 0], ref, rtol=0, atol=1e-12)
    assert lse.shape == (B, 1, N, H) and np.all(np.isfinite(lse))
