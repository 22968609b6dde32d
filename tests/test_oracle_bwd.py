"""Pins of the oracle's backward (gradients of the definition) to things other than itself:

  * the library special case: torch autograd through scaled_dot_product_attention in
    float64 on the CPU, with the rows i and heads h batched and the shared bias
    broadcast over the rows (so autograd sums its gradient over i);
  * central finite differences of <dout, out> on tiny inputs (out from the oracle's
    forward, which is pinned on its own);
  * closed forms: every row of dbias sums to zero (adding a constant to a bias row
    changes nothing), dropped keys receive no gradient, and the value gradients of a
    line sum to the line's upstream gradients (the weights of each query sum to one).
"""
import numpy as np
import pytest

from tests.test_oracle_pins import rand_case


def autograd_reference(q, k, v, bias, mask, dout):
    import torch
    t = lambda x: torch.tensor(np.asarray(x, dtype=np.float64), requires_grad=True)
    Q, K, V, Bi = t(q), t(k), t(v), t(bias)
    B, I, N, H, D = q.shape
    M = Bi[:, None].expand(B, I, H, N, N)
    if mask is not None:
        M = M + torch.from_numpy(mask.astype(np.float64))[:, None, None, None, :]
    out = torch.nn.functional.scaled_dot_product_attention(
        Q.permute(0, 1, 3, 2, 4), K.permute(0, 1, 3, 2, 4), V.permute(0, 1, 3, 2, 4), attn_mask=M)
    out = out.permute(0, 1, 3, 2, 4)
    out.backward(torch.from_numpy(dout.astype(np.float64)))
    return (Q.grad.numpy(), K.grad.numpy(), V.grad.numpy(), Bi.grad.numpy())


@pytest.mark.parametrize("shape,masked", [(dict(B=1, I=3, N=11, H=2, D=8), ()),
                                          (dict(B=2, I=4, N=17, H=3, D=16), (0, 9, 16)),
                                          (dict(B=1, I=2, N=33, H=1, D=32), tuple(range(20, 33)))])
def test_matches_autograd(oracle_mod, shape, masked):
    rng = np.random.default_rng(90)
    q, k, v, bias, mask = rand_case(rng, masked=masked, sigma_b=2.0, **shape)
    dout = rng.standard_normal(q.shape).astype(np.float32)
    got = oracle_mod.tri_attn_bwd(q, k, v, bias, mask, dout)
    ref = autograd_reference(q, k, v, bias, mask, dout)
    for name, g, r in zip(("dq", "dk", "dv", "dbias"), got, ref):
        np.testing.assert_allclose(g, r, rtol=0, atol=1e-12, err_msg=name)


def test_bf16_inputs_match_autograd_on_widened_values(oracle_mod, wl):
    from workloads import bf16_bits_to_f32
    cfg = wl.custom_config(B=1, I=5, N=24, H=2, D=32, dtype="bf16", n_key_tiles=1, seed=4, sigma_bias=2.0,
                           mask_last=3)
    w = wl.make_inputs(cfg)
    dout = np.random.default_rng(1).standard_normal(w.q.shape).astype(np.float32)
    got = oracle_mod.tri_attn_bwd(w.q, w.k, w.v, w.bias, w.mask, dout)
    ref = autograd_reference(*(bf16_bits_to_f32(x) for x in (w.q, w.k, w.v, w.bias)), w.mask, dout)
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, rtol=0, atol=1e-12)


def test_central_finite_differences(oracle_mod):
    rng = np.random.default_rng(91)
    q, k, v, bias, mask = rand_case(rng, B=1, I=2, N=5, H=1, D=3, masked=(4,), sigma_b=1.0)
    dout = rng.standard_normal(q.shape).astype(np.float32)
    grads = oracle_mod.tri_attn_bwd(q, k, v, bias, mask, dout)
    loss = lambda *x: float(np.sum(oracle_mod.tri_attn(*x, mask)[0] * dout.astype(np.float64)))
    h = np.float32(2.0 ** -9)
    inputs = [q, k, v, bias]
    for which, g in enumerate(grads):
        x = inputs[which]
        for idx in np.ndindex(x.shape):
            plus, minus = [a.copy() for a in inputs], [a.copy() for a in inputs]
            plus[which][idx] += h
            minus[which][idx] -= h
            step = float(plus[which][idx]) - float(minus[which][idx])
            fd = (loss(*plus) - loss(*minus)) / step
            assert abs(fd - g[idx]) < 2e-5 * max(1.0, abs(g[idx])), (which, idx, fd, g[idx])


def test_closed_forms(oracle_mod):
    rng = np.random.default_rng(92)
    masked = (1, 6, 12)
    q, k, v, bias, mask = rand_case(rng, B=2, I=3, N=13, H=2, D=8, masked=masked, sigma_b=2.0)
    dout = rng.standard_normal(q.shape).astype(np.float32)
    dq, dk, dv, dbias = oracle_mod.tri_attn_bwd(q, k, v, bias, mask, dout)
    np.testing.assert_allclose(dbias.sum(axis=-1), 0.0, rtol=0, atol=1e-13)     # bias-row shift invariance
    assert np.all(dbias[..., list(masked)] == 0)
    assert np.all(dk[:, :, list(masked)] == 0) and np.all(dv[:, :, list(masked)] == 0)
    np.testing.assert_allclose(dv.sum(axis=2), dout.astype(np.float64).sum(axis=2), rtol=0, atol=1e-12)


def test_dbias_sums_the_rows(oracle_mod):
    """dbias of I rows is the sum of the per-row dbias: a rank's share adds up."""
    rng = np.random.default_rng(93)
    q, k, v, bias, mask = rand_case(rng, B=1, I=4, N=9, H=2, D=4)
    dout = rng.standard_normal(q.shape).astype(np.float32)
    total = oracle_mod.tri_attn_bwd(q, k, v, bias, mask, dout)[3]
    parts = sum(oracle_mod.tri_attn_bwd(q[:, i:i + 1], k[:, i:i + 1], v[:, i:i + 1], bias, mask,
                                        dout[:, i:i + 1])[3] for i in range(4))
    np.testing.assert_allclose(total, parts, rtol=0, atol=1e-13)


def test_fully_masked_row_has_no_gradient(oracle_mod):
    rng = np.random.default_rng(94)
    q, k, v, bias, _ = rand_case(rng, B=1, I=2, N=6, H=1, D=4)
    mask = np.full((1, 6), -np.inf, dtype=np.float32)
    dout = rng.standard_normal(q.shape).astype(np.float32)
    for g in oracle_mod.tri_attn_bwd(q, k, v, bias, mask, dout):
        assert np.all(g == 0)


@pytest.mark.parametrize("shape,masked,cols", [(dict(B=1, I=4, N=11, H=2, D=8), (), (0, 5, 10)),
                                               (dict(B=2, I=5, N=17, H=3, D=16), (0, 9, 16), (16, 3, 3, 8))])
def test_dbias_columns_match_autograd(oracle_mod, shape, masked, cols):
    """The column form of dbias (summed over every row) against torch autograd, and a
    batch element whose keys are all masked contributes nothing."""
    rng = np.random.default_rng(93)
    q, k, v, bias, mask = rand_case(rng, masked=masked, sigma_b=2.0, **shape)
    if shape["B"] > 1:
        mask = np.zeros((shape["B"], shape["N"]), dtype=np.float32) if mask is None else mask.copy()
        mask[1, :] = -np.inf
    dout = rng.standard_normal(q.shape).astype(np.float32)
    got = oracle_mod.tri_attn_dbias_cols(q, k, v, bias, mask, dout, list(cols))
    if shape["B"] > 1:
        assert np.all(got[1] == 0)
        ref = autograd_reference(q[:1], k[:1], v[:1], bias[:1], mask[:1], dout[:1])[3]
        got = got[:1]
    else:
        ref = autograd_reference(q, k, v, bias, mask, dout)[3]
    np.testing.assert_allclose(got, ref[:, :, list(cols)], rtol=0, atol=1e-12)
