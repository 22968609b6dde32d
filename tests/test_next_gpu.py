"""GPU parity of the entry points beyond the forward: the log-sum-exp output, the
ending-node orientation, the split-tile primitive (ring-step states, their merge and
finalisation) and attention with pair bias -- each through the C ABI against the fp64
oracle on the same seeded inputs.

Bars (absolute, every compared element): outputs as the forward (1e-5 fp32, 1e-2 bf16
with fp32 accumulation); log-sum-exps and partial log-sum-exps the same bars.  States
are compared through what does not depend on the reference m each side picked: the
normalised partial output acc / l and the partial log-sum-exp m + ln l.
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


def dev_inputs(torch, w):
    return tuple(to_dev(torch, x) for x in (w.q, w.k, w.v, w.bias, w.mask))


def small(dtype, B=1, I=64, N=64, H=4, D=32, T=3, seed=31, mask_last=5, sigma_bias=2.0):
    return W.make_inputs(W.custom_config(B=B, I=I, N=N, H=H, D=D, dtype=dtype, n_key_tiles=T, seed=seed,
                                         sigma_bias=sigma_bias, mask_last=mask_last))


def compare_lse(got, expect, tol, what):
    got = got.astype(np.float64)
    fin = np.isfinite(expect)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: -inf pattern differs"
    err = np.abs(got[fin] - expect[fin])
    worst = float(err.max()) if err.size else 0.0
    say(f"  {what}: max|err| = {worst:.3e} (bar {tol:g}) over {err.size} finite values")
    assert worst <= tol, f"{what}: {worst:.3e} > {tol:g}"


# ---------------------------------------------------------------------------
# log-sum-exp
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,D", [("bf16", 32), ("fp32", 32), ("bf16", 16)])
def test_forward_lse(torch_dev, dtype, D):
    import pair_biased_triangle_amd as P
    w = small(dtype, I=40, N=130, D=D, T=4)
    say(f"[next] lse {dtype} D={D}")
    q, k, v, bias, mask = dev_inputs(torch_dev, w)
    out, lse = P.tri_attn_fwd_lse(q, k, v, bias, mask, n_key_tiles=4)
    plain = P.tri_attn_fwd_rows(q, k, v, bias, mask, n_key_tiles=4)
    torch_dev.cuda.synchronize()
    assert torch_dev.equal(out, plain), "the lse entry point changed the output"
    ref, ref_lse = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, n_key_tiles=4)
    compare(out.cpu().numpy(), ref, TOL[dtype], f"out {dtype}")
    compare_lse(lse.cpu().numpy(), ref_lse, TOL[dtype], f"lse {dtype}")


@pytest.mark.parametrize("jump", [False, True])
def test_split_key_mode(torch_dev, jump):
    """A grid of a few workgroups (8 lines of N = 1024, two heads) runs in split-key mode:
    the key blocks are cut into ranges folded side by side, whose states the merge rule
    joins.  With q.k of one key far above the rest, the range holding that key takes the
    exact pass while the others keep the fast one."""
    import pair_biased_triangle_amd as P
    w = small("bf16", B=2, I=8, N=1024, H=2, T=3, seed=41, mask_last=70)
    w.mask[1, :] = -np.inf                           # batch element 1: every key masked (out 0, lse -inf)
    if jump:
        q, k = W.bf16_bits_to_f32(w.q), W.bf16_bits_to_f32(w.k)
        q[0, :, 100:140, 1, :] = 4.0
        k[0, :, 700, 1, :] = 4.0
        w.q, w.k = W.f32_to_bf16_bits(q), W.f32_to_bf16_bits(k)
    # the workspace holds the partial states only in split-key mode
    blocks = 3 * -(-342 // 32)
    image_and_refs = 4 * 4 * blocks * 256 * 32 * 2 + 4 * 4 * 256 * 4
    assert P.workspace_bytes(2, 2, 8, 1024, 32, 3, 1) > image_and_refs
    say(f"[next] split-key mode, jump={jump}")
    qd, kd, vd, bias, mask = dev_inputs(torch_dev, w)
    out, lse = P.tri_attn_fwd_lse(qd, kd, vd, bias, mask, n_key_tiles=3)
    torch_dev.cuda.synchronize()
    ref, ref_lse = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, n_key_tiles=3)
    compare(out.cpu().numpy(), ref, TOL["bf16"], "out, split-key mode")
    compare_lse(lse.cpu().numpy(), ref_lse, TOL["bf16"], "lse, split-key mode")
    assert np.all(out.cpu().numpy()[1] == 0) and np.all(np.isneginf(lse.cpu().numpy()[1]))
    # the caller-workspace entry point runs the same split-key launch
    ws = torch_dev.empty(P.workspace_bytes(2, 2, 8, 1024, 32, 3, 1), dtype=torch_dev.uint8, device="cuda")
    a = P.tri_attn_fwd_rows(qd, kd, vd, bias, mask, n_key_tiles=3)
    b = P.tri_attn_fwd_rows_ws(qd, kd, vd, bias, mask, workspace=ws, n_key_tiles=3)
    torch_dev.cuda.synchronize()
    assert torch_dev.equal(a, b) and torch_dev.equal(a, out)
    if jump:
        np.testing.assert_allclose(out.cpu().numpy()[0, :, 100:140, 1],
                                   W.bf16_bits_to_f32(w.v)[0, :, 700:701, 1].repeat(40, axis=1), atol=1e-6)


def test_lse_of_fully_masked_rows(torch_dev):
    import pair_biased_triangle_amd as P
    for dtype in ("bf16", "fp32"):
        w = small(dtype, I=8, N=40, T=2, mask_last=0)
        mask = np.zeros((1, 40), dtype=np.float32)
        mask[0, :] = -np.inf
        q, k, v, bias, _ = dev_inputs(torch_dev, w)
        out, lse = P.tri_attn_fwd_lse(q, k, v, bias, to_dev(torch_dev, mask), n_key_tiles=2)
        torch_dev.cuda.synchronize()
        assert torch_dev.all(out == 0) and torch_dev.all(lse == -float("inf"))


# ---------------------------------------------------------------------------
# ending node
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,N,D,T", [("bf16", 64, 32, 1), ("bf16", 150, 32, 5), ("fp32", 70, 32, 3),
                                         ("fp32", 33, 48, 2), ("bf16", 9, 16, 9)])
def test_ending_small_full(torch_dev, dtype, N, D, T):
    import pair_biased_triangle_amd as P
    w = small(dtype, B=2 if N < 100 else 1, I=N, N=N, D=D, T=T, mask_last=3)
    say(f"[next] ending {dtype} N={N} D={D} T={T}")
    q, k, v, bias, mask = dev_inputs(torch_dev, w)
    out, lse = P.tri_attn_fwd_ending(q, k, v, bias, mask, n_key_tiles=T, want_lse=True)
    torch_dev.cuda.synchronize()
    ref, ref_lse = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, n_key_tiles=T, ending=True)
    compare(out.cpu().numpy(), ref, TOL[dtype], f"ending out {dtype}")
    compare_lse(lse.cpu().numpy(), ref_lse, TOL[dtype], f"ending lse {dtype}")


def test_ending_large_sampled(torch_dev):
    """N = 1024, bf16, the four-chain workload's inputs in the ending orientation."""
    import pair_biased_triangle_amd as P
    w = W.make_inputs("complex_n1024")
    cfg = w.cfg
    say("[next] ending complex_n1024 sampled")
    q, k, v, bias, mask = dev_inputs(torch_dev, w)
    out = P.tri_attn_fwd_ending(q, k, v, bias, mask, n_key_tiles=cfg.n_key_tiles)
    torch_dev.cuda.synchronize()
    rng = np.random.default_rng(5)
    N = cfg.N
    edges = [0, 1, 31, 32, 127, 128, N // 2, N - 2, N - 1]
    rows = [oracle.flat_rows(1, N, N, 0, i, j)[0] for i in edges for j in edges]
    rows = np.unique(np.array(rows + list(rng.integers(0, N * N, size=300)), dtype=np.int64))
    ref, _ = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, n_key_tiles=cfg.n_key_tiles, ending=True, rows=rows)
    got = out.view(-1, cfg.H, cfg.D)[torch_dev.from_numpy(rows).cuda()].cpu().numpy()
    compare(got, ref, TOL["bf16"], "ending complex_n1024")


# ---------------------------------------------------------------------------
# split-tile primitive
# ---------------------------------------------------------------------------
def normalised(acc, m, l):
    l = l.astype(np.float64)
    some = l > 0
    safe = np.where(some, l, 1.0)
    out = np.where(some[..., None], acc.astype(np.float64) / safe[..., None], 0.0)
    lse = np.where(some, m.astype(np.float64) + np.log(safe), -np.inf)
    return out, lse


@pytest.mark.parametrize("dtype,ending", [("bf16", False), ("fp32", False), ("bf16", True), ("fp32", True)])
def test_tile_states_and_ring_merge(torch_dev, dtype, ending):
    import pair_biased_triangle_amd as P
    N = 97
    w = small(dtype, I=N if ending else 20, N=N, T=1, mask_last=4)
    say(f"[next] ring-step states {dtype} ending={ending}")
    q, k, v, bias, mask = dev_inputs(torch_dev, w)
    bounds = [0, 13, 45, 46, 93, N]                 # ragged tiles, one of a single key, one fully masked
    order = [2, 4, 0, 3, 1]                          # a ring that starts mid-axis
    run = None
    for t in order:
        lo, hi = bounds[t], bounds[t + 1]
        acc, m, l = P.tri_attn_tile_state(q, k, v, bias, mask, key_begin=lo, key_end=hi, ending=ending)
        torch_dev.cuda.synchronize()
        racc, rm, rl = oracle.tile_state(w.q, w.k, w.v, w.bias, w.mask, key_begin=lo, key_end=hi, ending=ending)
        g_out, g_lse = normalised(acc.cpu().numpy(), m.cpu().numpy(), l.cpu().numpy())
        r_out, r_lse = normalised(racc, rm, rl)
        compare(g_out, r_out, TOL[dtype], f"tile [{lo},{hi}) partial output")
        compare_lse(g_lse, r_lse, TOL[dtype], f"tile [{lo},{hi}) partial lse")
        if run is None:
            run = (acc.clone(), m.clone(), l.clone())
        else:
            P.tri_attn_state_merge(*run, acc, m, l)
    out, lse = P.tri_attn_state_finalize(*run)
    torch_dev.cuda.synchronize()
    ref, ref_lse = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, ending=ending)
    compare(out.cpu().numpy(), ref, TOL[dtype], "merged ring")
    compare_lse(lse.cpu().numpy(), ref_lse, TOL[dtype], "merged ring lse")


@pytest.mark.parametrize("dtype,ending,N,I", [("bf16", False, 97, 20), ("fp32", False, 97, 20), ("bf16", True, 97, 97),
                                              ("fp32", True, 97, 97), ("bf16", False, 600, 12)])
def test_ring_by_state_updates(torch_dev, dtype, ending, N, I):
    """The ring folded step by step into one running state with tri_attn_tile_state_update,
    starting from the empty state (l = 0), then finalised: tri_attn_fwd's result."""
    import pair_biased_triangle_amd as P
    w = small(dtype, I=I, N=N, T=1, mask_last=4)
    say(f"[next] ring by state updates {dtype} ending={ending} N={N}")
    q, k, v, bias, mask = dev_inputs(torch_dev, w)
    t = torch_dev
    acc = t.full((1, I, N, 4, 32), 7.0, dtype=t.float32, device="cuda")    # not read while l = 0
    m = t.full((1, I, N, 4), 3.0, dtype=t.float32, device="cuda")
    l = t.zeros((1, I, N, 4), dtype=t.float32, device="cuda")
    bounds = [0, 13, 45, 46, 93, N] if N == 97 else [0, 150, 151, 420, N]
    order = [2, 4, 0, 3, 1] if N == 97 else [3, 1, 0, 2]
    for tt in order:
        P.tri_attn_tile_state_update(q, k, v, bias, mask, key_begin=bounds[tt], key_end=bounds[tt + 1],
                                     ending=ending, acc=acc, m=m, l=l)
    out, lse = P.tri_attn_state_finalize(acc, m, l)
    t.cuda.synchronize()
    ref, ref_lse = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, ending=ending)
    compare(out.cpu().numpy(), ref, TOL[dtype], "ring by updates")
    compare_lse(lse.cpu().numpy(), ref_lse, TOL[dtype], "ring by updates lse")


@pytest.mark.parametrize("dtype,ending,N,I", [("bf16", False, 97, 20), ("fp32", False, 97, 20), ("bf16", True, 97, 97),
                                              ("fp32", True, 97, 97), ("bf16", False, 600, 12)])
def test_ring_with_final_step(torch_dev, dtype, ending, N, I):
    """The ring folded by updates except its last step, which tri_attn_tile_state_final
    folds and finalises in one call: tri_attn_fwd's result and lse, with the state left
    as it was.  The first range's keys are all masked for N = 97 (an empty step)."""
    import pair_biased_triangle_amd as P
    w = small(dtype, I=I, N=N, T=1, mask_last=4)
    if N == 97:
        w.mask[0, 0:13] = -np.inf
    say(f"[next] ring with a final step {dtype} ending={ending} N={N}")
    q, k, v, bias, mask = dev_inputs(torch_dev, w)
    t = torch_dev
    acc = t.full((1, I, N, 4, 32), 7.0, dtype=t.float32, device="cuda")    # not read while l = 0
    m = t.full((1, I, N, 4), 3.0, dtype=t.float32, device="cuda")
    l = t.zeros((1, I, N, 4), dtype=t.float32, device="cuda")
    bounds = [0, 13, 45, 46, 93, N] if N == 97 else [0, 150, 151, 420, N]
    order = [2, 4, 3, 1, 0] if N == 97 else [3, 1, 0, 2]
    for tt in order[:-1]:
        P.tri_attn_tile_state_update(q, k, v, bias, mask, key_begin=bounds[tt], key_end=bounds[tt + 1],
                                     ending=ending, acc=acc, m=m, l=l)
    state = [x.clone() for x in (acc, m, l)]
    last = order[-1]
    out, lse = P.tri_attn_tile_state_final(q, k, v, bias, mask, key_begin=bounds[last], key_end=bounds[last + 1],
                                           ending=ending, acc=acc, m=m, l=l, want_lse=True)
    t.cuda.synchronize()
    assert all(t.equal(a, b) for a, b in zip(state, (acc, m, l))), "the final step wrote the state"
    ref, ref_lse = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, ending=ending)
    compare(out.cpu().numpy(), ref, TOL[dtype], "ring with a final step")
    compare_lse(lse.cpu().numpy(), ref_lse, TOL[dtype], "ring with a final step, lse")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_final_step_from_empty_state(torch_dev, dtype):
    """tri_attn_tile_state_final on the empty state (l = 0) over the whole key range is the
    forward itself; over a fully masked range it gives out 0 and lse -inf."""
    import pair_biased_triangle_amd as P
    w = small(dtype, I=9, N=70, T=1, mask_last=10)
    say(f"[next] final step from the empty state {dtype}")
    q, k, v, bias, mask = dev_inputs(torch_dev, w)
    t = torch_dev
    acc = t.full((1, 9, 70, 4, 32), float("nan"), dtype=t.float32, device="cuda")   # never read while l = 0
    m = t.full((1, 9, 70, 4), float("nan"), dtype=t.float32, device="cuda")
    l = t.zeros((1, 9, 70, 4), dtype=t.float32, device="cuda")
    out, lse = P.tri_attn_tile_state_final(q, k, v, bias, mask, key_begin=0, key_end=70, acc=acc, m=m, l=l,
                                           want_lse=True)
    o2, l2 = P.tri_attn_tile_state_final(q, k, v, bias, mask, key_begin=60, key_end=70, acc=acc, m=m, l=l,
                                         want_lse=True)
    t.cuda.synchronize()
    ref, ref_lse = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask)
    compare(out.cpu().numpy(), ref, TOL[dtype], "final step from the empty state")
    compare_lse(lse.cpu().numpy(), ref_lse, TOL[dtype], "final step from the empty state, lse")
    assert t.all(o2 == 0) and t.all(t.isneginf(l2))


@pytest.mark.parametrize("D,shift", [(24, 0), (6, 0), (24, 1)], ids=["vector", "D6_scalar", "offset_scalar"])
def test_state_merge_and_finalize_kernels(torch_dev, D, shift):
    """The merge and finalisation kernels on random fp32 states (empty states mixed in)
    against the oracle module's merge rule in fp64 on the same values.  D % 4 == 0 with
    16-byte aligned accumulators takes the 16-byte path; D = 6, or accumulators that start
    4 bytes past a 16-byte boundary (shift), take the one-float path."""
    import pair_biased_triangle_amd as P
    rng = np.random.default_rng(17)
    rows = 5000
    def state(empty_frac):
        acc = rng.standard_normal((rows, D)).astype(np.float32)
        m = (3 * rng.standard_normal(rows)).astype(np.float32)
        l = rng.uniform(1.0, 50.0, rows).astype(np.float32)
        empty = rng.random(rows) < empty_frac
        acc[empty], m[empty], l[empty] = 0.0, -np.inf, 0.0
        return acc, m, l
    a, b = state(0.1), state(0.1)
    for st in (a, b):                                # rows 0..9: both states present ...
        st[1][:10] = np.float32(1.5)
        st[2][:10] = np.float32(3.0)
    b[1][:5] = np.float32(-2.0)                      # ... with equal references in 5..9
    say("[next] state merge/finalize kernels")
    def dev(x):
        if x.ndim == 1 or shift == 0:
            return torch_dev.from_numpy(x.copy()).cuda()
        buf = torch_dev.empty(x.size + shift, dtype=torch_dev.float32, device="cuda")
        t = buf[shift:].view(x.shape)
        t.copy_(torch_dev.from_numpy(x))
        assert t.data_ptr() % 16 == 4 * shift
        return t
    ga = tuple(dev(x) for x in a)
    gb = tuple(dev(x) for x in b)
    P.tri_attn_state_merge(*ga, *gb)
    out, lse = P.tri_attn_state_finalize(*ga)
    torch_dev.cuda.synchronize()
    e_acc, e_m, e_l = oracle.merge_states(*a, *b)
    e_out, e_lse = oracle.finalize_states(e_acc, e_m, e_l)
    np.testing.assert_allclose(ga[2].cpu().numpy(), e_l, rtol=2e-6, atol=0)
    fin = np.isfinite(e_m)
    np.testing.assert_array_equal(np.isfinite(ga[1].cpu().numpy()), fin)
    np.testing.assert_allclose(ga[1].cpu().numpy()[fin], e_m[fin], rtol=0, atol=0)
    np.testing.assert_allclose(out.cpu().numpy(), e_out, rtol=5e-6, atol=1e-6)
    compare_lse(lse.cpu().numpy(), e_lse, 1e-5, "finalize lse")


def test_tile_state_of_masked_range_is_empty(torch_dev):
    import pair_biased_triangle_amd as P
    for dtype in ("bf16", "fp32"):
        w = small(dtype, I=16, N=70, T=1, mask_last=20)       # keys 50..69 dropped
        q, k, v, bias, mask = dev_inputs(torch_dev, w)
        acc, m, l = P.tri_attn_tile_state(q, k, v, bias, mask, key_begin=52, key_end=70)
        torch_dev.cuda.synchronize()
        assert torch_dev.all(acc == 0) and torch_dev.all(l == 0) and torch_dev.all(m == -float("inf"))


# ---------------------------------------------------------------------------
# attention with pair bias
# ---------------------------------------------------------------------------
# bf16 with D = 32 and even N: the single-pass kernel (N = 100: one key range, N = 300 and
# 2700: ranges joined by the combine); odd N goes through the fp16 image; fp32 the general path
@pytest.mark.parametrize("dtype,N,D,T,B", [("bf16", 300, 32, 4, 2), ("fp32", 130, 16, 1, 3), ("bf16", 2700, 32, 8, 1),
                                           ("bf16", 100, 32, 3, 3), ("bf16", 301, 32, 2, 1)])
def test_pair_bias_attention(torch_dev, dtype, N, D, T, B):
    import pair_biased_triangle_amd as P
    w = small(dtype, B=B, I=1, N=N, D=D, T=T, mask_last=7)
    say(f"[next] pair-bias attention {dtype} B={B} N={N} D={D} T={T}")
    q, k, v, bias, mask = dev_inputs(torch_dev, w)
    shp = (B, N, 4, D)
    out, lse = P.pair_bias_attn_fwd(q.view(shp), k.view(shp), v.view(shp), bias, mask, n_key_tiles=T, want_lse=True)
    torch_dev.cuda.synchronize()
    ref, ref_lse = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, n_key_tiles=T)
    compare(out.cpu().numpy(), ref[:, 0], TOL[dtype], f"pair-bias out {dtype}")
    compare_lse(lse.cpu().numpy(), ref_lse[:, 0], TOL[dtype], f"pair-bias lse {dtype}")


@pytest.mark.parametrize("N", [100, 640])
def test_pair_bias_single_pass_extremes(torch_dev, N):
    """The single-pass kernel keeps a running reference: a bias jump of +60 on one key
    of some queries makes that key take all the weight, a batch element with every key
    masked gives out 0 and lse -inf, and the rest still matches the oracle."""
    import pair_biased_triangle_amd as P
    w = small("bf16", B=2, I=1, N=N, D=32, T=1, mask_last=5)
    w.mask[1, :] = -np.inf
    bias = W.bf16_bits_to_f32(w.bias)
    bias[0, 2, 10:40, N // 3] += 60.0
    w.bias = W.f32_to_bf16_bits(bias)
    say(f"[next] pair-bias single pass, extremes, N={N}")
    q, k, v, b, mask = dev_inputs(torch_dev, w)
    shp = (2, N, 4, 32)
    out, lse = P.pair_bias_attn_fwd(q.view(shp), k.view(shp), v.view(shp), b, mask, want_lse=True)
    torch_dev.cuda.synchronize()
    ref, ref_lse = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, n_key_tiles=1)
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    compare(o, ref[:, 0], TOL["bf16"], "pair-bias single pass out")
    compare_lse(l, ref_lse[:, 0], TOL["bf16"], "pair-bias single pass lse")
    assert np.all(o[1] == 0) and np.all(np.isneginf(l[1]))
    vv = W.bf16_bits_to_f32(w.v)[0, 0, N // 3, 2]                     # the value row of the dominant key
    np.testing.assert_allclose(o[0, 10:40, 2], np.broadcast_to(vv, (30, 32)), atol=1e-6)


@pytest.mark.parametrize("N", [640, 2700])
def test_pair_bias_single_pass_moving_reference(torch_dev, N):
    """Bias ramps rising along the keys with a slope that differs per query (0 to 1.2 per
    key block, in natural-log units, some falling instead), so that the single-pass kernel
    moves its reference many times, at different blocks for different queries of a wave
    (queries whose reference stays keep a factor of 1 inside the rescale branch); the
    result matches the oracle."""
    import pair_biased_triangle_amd as P
    w = small("bf16", B=1, I=1, N=N, D=32, T=1, mask_last=3)
    bias = W.bf16_bits_to_f32(w.bias)
    keys = np.arange(N, dtype=np.float32) / 32.0                       # key blocks
    slope = np.random.default_rng(5).uniform(-0.4, 1.2, size=(4, N)).astype(np.float32)
    bias[0] += slope[:, :, None] * keys[None, None, :]
    w.bias = W.f32_to_bf16_bits(bias)
    say(f"[next] pair-bias single pass, moving reference, N={N}")
    q, k, v, b, mask = dev_inputs(torch_dev, w)
    shp = (1, N, 4, 32)
    out, lse = P.pair_bias_attn_fwd(q.view(shp), k.view(shp), v.view(shp), b, mask, want_lse=True)
    torch_dev.cuda.synchronize()
    ref, ref_lse = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, n_key_tiles=1)
    compare(out.cpu().numpy(), ref[:, 0], TOL["bf16"], "pair-bias moving reference out")
    compare_lse(lse.cpu().numpy(), ref_lse[:, 0], TOL["bf16"], "pair-bias moving reference lse")


@pytest.mark.parametrize("N", [100, 640, 2700])
def test_pair_bias_without_mask(torch_dev, N):
    """The single-pass kernel's maskless form (mask = None): one key range at N = 100, whole
    32-key blocks only at N = 640, ranges joined by the combine and a last block past the
    last key at N = 2700."""
    import pair_biased_triangle_amd as P
    w = small("bf16", B=1, I=1, N=N, D=32, T=1, mask_last=0)
    assert w.mask is None
    say(f"[next] pair-bias without a mask, N={N}")
    q, k, v, bias, _ = dev_inputs(torch_dev, w)
    shp = (1, N, 4, 32)
    out, lse = P.pair_bias_attn_fwd(q.view(shp), k.view(shp), v.view(shp), bias, None, want_lse=True)
    torch_dev.cuda.synchronize()
    ref, ref_lse = oracle.tri_attn(w.q, w.k, w.v, w.bias, None, n_key_tiles=1)
    compare(out.cpu().numpy(), ref[:, 0], TOL["bf16"], "pair-bias without mask out")
    compare_lse(lse.cpu().numpy(), ref_lse[:, 0], TOL["bf16"], "pair-bias without mask lse")


@pytest.mark.timeout(600)
def test_pair_bias_largest_single_pass_size(torch_dev):
    """The largest N the single-pass kernel takes (46340: its copies address one (b, h)
    bias slab of N * N * 2 bytes with 32-bit offsets, so rows past j = 23170 lie more than
    2^31 bytes into it).  Each sampled query gets +30 on one key spread over the whole
    range, so its output is essentially that key's value and any misaddressed bias row or
    key shows; compared with the oracle on those queries."""
    import pair_biased_triangle_amd as P
    N = 46340
    w = W.make_inputs(W.custom_config(B=1, I=1, N=N, H=1, D=32, dtype="bf16", n_key_tiles=1, seed=97,
                                      sigma_bias=2.0, mask_last=6))
    rows = np.array([0, 1, 127, 128, 23170, 23171, 33000, 40000, 46211, 46338, 46339])
    keys = (rows * 7919 + 11) % (N - 6)
    bias = w.bias.reshape(N, N)
    sel = W.bf16_bits_to_f32(bias[rows, keys]) + 30.0
    bias[rows, keys] = W.f32_to_bf16_bits(sel)
    ws = P.call_workspace_bytes(P.CALL_PAIR_BIAS, 1, 1, 1, N, 32, N, P.TRI_ATTN_BF16)
    assert ws < 64 << 20, f"{ws} bytes of workspace: not the single-pass kernel's partial states"
    say(f"[next] pair-bias at N={N} (single pass, {ws} bytes of workspace)")
    q, k, v, b, mask = dev_inputs(torch_dev, w)
    shp = (1, N, 1, 32)
    out, lse = P.pair_bias_attn_fwd(q.view(shp), k.view(shp), v.view(shp), b, mask, want_lse=True)
    torch_dev.cuda.synchronize()
    del b
    ref, ref_lse = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, n_key_tiles=1, rows=rows)
    got = out.view(N, 1, 32)[torch_dev.from_numpy(rows).cuda()].cpu().numpy()
    got_lse = lse.view(N, 1)[torch_dev.from_numpy(rows).cuda()].cpu().numpy()
    compare(got, ref, TOL["bf16"], f"pair-bias N={N}, {len(rows)} queries")
    compare_lse(got_lse, ref_lse, TOL["bf16"], f"pair-bias lse N={N}")
    vk = W.bf16_bits_to_f32(w.v.reshape(N, 32)[keys])
    assert np.max(np.abs(got[:, 0] - vk)) < 0.1, "a query's output is not its heavy key's value"


@pytest.mark.parametrize("N", [1, 2])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_degenerate_sizes(torch_dev, dtype, N):
    """One or two tokens through the entry points beyond the forward: attention with pair
    bias (N = 2 is the smallest the single pass takes, N = 1 goes through the image), the
    ending node, the ring with one key per step and the backward (with a single key every
    probability is 1, so the oracle's dq, dk and dbias vanish and dv is dout)."""
    import pair_biased_triangle_amd as P
    t = torch_dev
    say(f"[next] degenerate sizes {dtype} N={N}")
    w = small(dtype, B=2, I=N, N=N, H=2, D=32, T=N, mask_last=0)
    q, k, v, bias, mask = dev_inputs(t, w)
    ref, ref_lse = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, n_key_tiles=N, ending=True)
    out = P.tri_attn_fwd_ending(q, k, v, bias, mask, n_key_tiles=N)
    t.cuda.synchronize()
    compare(out.cpu().numpy(), ref, TOL[dtype], f"ending N={N}")
    ref, ref_lse = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, n_key_tiles=N)
    acc, m, l = P.tri_attn_tile_state(q, k, v, bias, mask, key_begin=0, key_end=1)
    if N == 2:
        out, lse = P.tri_attn_tile_state_final(q, k, v, bias, mask, key_begin=1, key_end=2, acc=acc, m=m, l=l,
                                               want_lse=True)
    else:
        out, lse = P.tri_attn_state_finalize(acc, m, l)
    t.cuda.synchronize()
    compare(out.cpu().numpy(), ref, TOL[dtype], f"ring N={N}")
    compare_lse(lse.cpu().numpy(), ref_lse, TOL[dtype], f"ring lse N={N}")
    pb = small(dtype, B=2, I=1, N=N, H=2, D=32, T=1, mask_last=0)
    q1, k1, v1, b1, _ = dev_inputs(t, pb)
    shp = (2, N, 2, 32)
    out, lse = P.pair_bias_attn_fwd(q1.view(shp), k1.view(shp), v1.view(shp), b1, None, want_lse=True)
    t.cuda.synchronize()
    pref, pref_lse = oracle.tri_attn(pb.q, pb.k, pb.v, pb.bias, None)
    compare(out.cpu().numpy(), pref[:, 0], TOL[dtype], f"pair bias N={N}")
    compare_lse(lse.cpu().numpy(), pref_lse[:, 0], TOL[dtype], f"pair bias lse N={N}")
    dout = np.random.default_rng(5).standard_normal(w.q.shape).astype(np.float32)
    fo, fl = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask)
    g = P.tri_attn_bwd(q, k, v, bias, mask, t.from_numpy(fo.astype(np.float32)).cuda(),
                       t.from_numpy(fl.astype(np.float32)).cuda(), t.from_numpy(dout).cuda())
    t.cuda.synchronize()
    gref = oracle.tri_attn_bwd(w.q, w.k, w.v, w.bias, w.mask, dout)
    bar = 1e-2 if dtype == "bf16" else 1e-4
    for name, a, r in zip(("dq", "dk", "dv", "dbias"), (x.cpu().numpy() for x in g), gref):
        compare(a, r, bar * max(1.0, float(np.max(np.abs(r)))), f"backward {name} N={N}")
