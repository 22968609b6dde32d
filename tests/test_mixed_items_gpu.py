"""GPU parity of launches whose workgroups take different paths side by side.

A forward of thousands of (b, h, line group, column block) workgroups in which some leave
the fast pass (their exact running maximum restages the ring), a whole batch element has no
kept key (every one of its workgroups takes the exact pass), and one column block's bias
spans beyond the fp16 image (that block is the fp32 kernel's); and the ring-step entry
points on such a launch with a q.k jump in the middle tile, so that state-update
workgroups take the exact pass.  Bars as the forward: 1e-2 for bf16 inputs with fp32
accumulation.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.test_parity_gpu import TOL, compare, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import pair_biased_triangle_amd as P
    P.load_library()
    return torch


def rows_of(B, I, N, pairs):
    return np.unique(np.array([oracle.flat_rows(B, I, N, b, i, j)[0] for b, i, j in pairs], dtype=np.int64))


def test_mixed_workgroups(torch_dev):
    """B = 2, I = N = 520, H = 4: 6,240 workgroups, many rounds of those resident at once.  Batch element 0: q.k of key 300 about 90 nats above the rest for queries 5..40
    and 300..330 of a few lines (those workgroups take the exact pass), and a bias 40 nats below
    the rest on one key of head 1's second column block (that block goes to the fp32
    kernel).  Batch element 1: every key masked (out 0, lse -inf, every item exact)."""
    import pair_biased_triangle_amd as P
    torch = torch_dev
    B, I, N, H = 2, 520, 520, 4
    cfg = W.custom_config(B=B, I=I, N=N, H=H, D=32, dtype="bf16", n_key_tiles=3, seed=53, mask_last=9)
    w = W.make_inputs(cfg)
    q, k, b = (W.bf16_bits_to_f32(x) for x in (w.q, w.k, w.bias))
    jump_lines = [3, 4, 130, 131, 257, 400, 519]
    for i in jump_lines:
        q[0, i, 5:41, 0, :] = 4.0
        q[0, i, 300:331, 2, :] = 4.0
        k[0, i, 300, 0, :] = 4.0
        k[0, i, 300, 2, :] = 4.0
    b[0, 1, 256:512, 17] -= 40.0                      # head 1, column block 1: span beyond the image
    w.q, w.k, w.bias = (W.f32_to_bf16_bits(x) for x in (q, k, b))
    mask = w.mask.copy()
    mask[1, :] = -np.inf
    w.mask = mask

    qd, kd, vd, bd, md = (to_dev(torch, x) for x in (w.q, w.k, w.v, w.bias, w.mask))
    say("[mixed] B=2 N=520: q.k jumps, a wide column block, a fully masked batch element")
    out, lse = P.tri_attn_fwd_lse(qd, kd, vd, bd, md, n_key_tiles=3)
    plain = P.tri_attn_fwd(qd, kd, vd, bd, md, n_key_tiles=3)
    torch.cuda.synchronize()
    assert torch.equal(out, plain), "the lse entry point changed the output"
    out, lse = out.cpu().numpy(), lse.cpu().numpy()

    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1])), "fully masked batch element"
    rng = np.random.default_rng(5)
    pairs = [(0, i, j) for i in jump_lines for j in list(range(0, 48)) + list(range(250, 340)) + [511, 512, 519]]
    pairs += [(0, i, j) for i in (0, 1, 2, 5, 128, 129, 255, 256, 258, 518) for j in range(0, N, 3)]
    pairs += [(0, int(i), int(j)) for i, j in zip(rng.integers(0, I, 1500), rng.integers(0, N, 1500))]
    rows = rows_of(B, I, N, pairs)
    ref, ref_lse = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, n_key_tiles=3, rows=rows)
    got = out.reshape(-1, H, 32)[rows]
    compare(got, ref, TOL["bf16"], "out, mixed workgroups")
    got_lse = lse.reshape(-1, H)[rows].astype(np.float64)
    err = float(np.max(np.abs(got_lse - ref_lse)))
    say(f"  lse, mixed workgroups: max|err| = {err:.3e} over {got_lse.size} values")
    assert err <= TOL["bf16"]
    # the jump rows return key 300's value (weight 1 up to e^-90)
    v = W.bf16_bits_to_f32(w.v)
    for i in jump_lines:
        np.testing.assert_allclose(out[0, i, 5:41, 0], np.broadcast_to(v[0, i, 300, 0], (36, 32)), atol=1e-6)
        np.testing.assert_allclose(out[0, i, 300:331, 2], np.broadcast_to(v[0, i, 300, 2], (31, 32)), atol=1e-6)


def test_ring_steps_with_exact_updates(torch_dev):
    """The ring-step entry points on the same kind of launch (I = N = 520, 3,120
    workgroups): a first step, an update folded into it and a final step equal the
    forward's result within the bar, where state-update workgroups whose fast pass fails
    (a q.k jump in the middle tile) keep the merge exact."""
    import pair_biased_triangle_amd as P
    torch = torch_dev
    B, I, N, H = 1, 520, 520, 4
    cfg = W.custom_config(B=B, I=I, N=N, H=H, D=32, dtype="bf16", n_key_tiles=3, seed=54, mask_last=11)
    w = W.make_inputs(cfg)
    q, k = W.bf16_bits_to_f32(w.q), W.bf16_bits_to_f32(w.k)
    for i in (10, 11, 300):
        q[0, i, 100:160, 3, :] = 4.0
        k[0, i, 250, 3, :] = 4.0                      # in the middle key tile
    w.q, w.k = W.f32_to_bf16_bits(q), W.f32_to_bf16_bits(k)
    qd, kd, vd, bd, md = (to_dev(torch, x) for x in (w.q, w.k, w.v, w.bias, w.mask))
    bounds = [0, 174, 347, 520]                      # array_split of 520 keys into 3 tiles
    acc = torch.empty((B, I, N, H, 32), dtype=torch.float32, device="cuda")
    m = torch.empty((B, I, N, H), dtype=torch.float32, device="cuda")
    l = torch.empty_like(m)
    out = torch.empty_like(acc)
    say("[mixed] ring steps N=520 with a q.k jump in the middle tile")
    P.tri_attn_tile_state(qd, kd, vd, bd, md, key_begin=bounds[0], key_end=bounds[1], acc=acc, m=m, l=l)
    P.tri_attn_tile_state_update(qd, kd, vd, bd, md, key_begin=bounds[1], key_end=bounds[2], acc=acc, m=m, l=l)
    P.tri_attn_tile_state_final(qd, kd, vd, bd, md, key_begin=bounds[2], key_end=bounds[3], acc=acc, m=m, l=l, out=out)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    pairs = [(0, i, j) for i in (10, 11, 300) for j in range(90, 170)]
    pairs += [(0, int(i), int(j)) for i, j in zip(rng.integers(0, I, 2000), rng.integers(0, N, 2000))]
    rows = rows_of(B, I, N, pairs)
    ref, _ = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, n_key_tiles=3, rows=rows)
    compare(out.cpu().numpy().reshape(-1, H, 32)[rows], ref, TOL["bf16"], "ring out, mixed workgroups")
