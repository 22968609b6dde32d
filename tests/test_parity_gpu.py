"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the same
seeded inputs, element by element.

Bars (absolute, on every compared element):
  * fp32 inputs:               max |gpu - oracle| <= 1e-5
  * bf16 inputs, fp32 accum.:  max |gpu - oracle| <= 1e-2
Small workloads are compared in full; the full-size ones run in exactly the launch
configuration the benchmark times and are compared on sampled query rows (all heads
and d of each row) chosen to cover workgroup, tile and ragged edges.
"""
import math
import sys

import numpy as np
import pytest

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-5, "bf16": 1e-2}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import pair_biased_triangle_amd as P
    P.load_library()
    return torch


def to_dev(torch, a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def run_gpu(torch, w, n_key_tiles, rows_entry=False):
    import pair_biased_triangle_amd as P
    q, k, v, bias, mask = (to_dev(torch, x) for x in (w.q, w.k, w.v, w.bias, w.mask))
    fn = P.tri_attn_fwd_rows if (rows_entry or w.cfg.I != w.cfg.N) else P.tri_attn_fwd
    out = fn(q, k, v, bias, mask, n_key_tiles=n_key_tiles)
    torch.cuda.synchronize()
    return out


def edge_rows(cfg, rng, n_random=256):
    """Flat (b, i, j) rows: workgroup/row-group edges, ragged tails, mask edge, random."""
    B, I, N = cfg.B, cfg.I, cfg.N
    ii = sorted({0, 1, 7, 8, 9, 15, 16, I // 2, I - 9, I - 8, I - 1} & set(range(I)))
    jj = sorted({0, 1, 31, 32, 63, 64, 127, 128, 129, N // 2, N - cfg.mask_last - 1, N - cfg.mask_last,
                 N - 33, N - 32, N - 2, N - 1} & set(range(N)))
    rows = [oracle.flat_rows(B, I, N, b, i, j)[0] for b in range(B) for i in ii for j in jj]
    rows += list(rng.integers(0, B * I * N, size=n_random))
    return np.unique(np.array(rows, dtype=np.int64))


def compare(out_gpu, expect, tol, what):
    got = out_gpu.astype(np.float64)
    err = np.abs(got - expect)
    worst = float(np.nanmax(err)) if err.size else 0.0
    say(f"  {what}: max|err| = {worst:.3e} (bar {tol:g}) over {err.size} elements")
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert worst <= tol, f"{what}: max abs error {worst:.3e} > {tol:g}"


# ---------------------------------------------------------------------------
# the workloads
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny_n32_fp32", "crop_n256"])
def test_small_workloads_full(torch_dev, name):
    w = W.make_inputs(name)
    cfg = w.cfg
    say(f"[parity] {name}: full tensor, T={cfg.n_key_tiles}")
    out = run_gpu(torch_dev, w, cfg.n_key_tiles).cpu().numpy()
    ref, _ = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, n_key_tiles=cfg.n_key_tiles)
    compare(out, ref, TOL[cfg.dtype], name)


@pytest.mark.parametrize("name", ["single_gpu_n2700", "ring_share_n4096_i1024"])
def test_large_workloads_sampled(torch_dev, name):
    torch = torch_dev
    w = W.make_inputs(name)
    cfg = w.cfg
    rng = np.random.default_rng(cfg.seed)
    rows = edge_rows(cfg, rng)
    say(f"[parity] {name}: bench launch, T={cfg.n_key_tiles}, {len(rows)} sampled rows")
    out = run_gpu(torch, w, cfg.n_key_tiles)
    got = out.view(-1, cfg.H, cfg.D)[torch.from_numpy(rows).cuda()].cpu().numpy()
    del out
    ref, _ = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, n_key_tiles=cfg.n_key_tiles, rows=rows)
    compare(got, ref, TOL[cfg.dtype], name)


# ---------------------------------------------------------------------------
# edge shapes, through both entry points and both kernels
# ---------------------------------------------------------------------------
SHAPES = [
    # B, I, N, H, D, dtype, T, mask_last
    (1, 1, 1, 1, 32, "bf16", 1, 0),
    (1, 7, 7, 2, 32, "bf16", 3, 2),
    (2, 33, 33, 3, 32, "bf16", 5, 1),
    (1, 65, 65, 4, 32, "bf16", 65, 0),
    (1, 130, 130, 4, 32, "bf16", 7, 10),
    (1, 9, 300, 4, 32, "bf16", 8, 17),
    (1, 17, 17, 2, 16, "bf16", 2, 0),
    (1, 20, 20, 2, 64, "bf16", 3, 4),
    (1, 20, 20, 2, 48, "fp32", 4, 3),
    (2, 40, 40, 3, 32, "fp32", 6, 5),
    (1, 5, 70, 1, 8, "fp32", 70, 0),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}_I{}_N{}_H{}_D{}_{}_T{}_m{}".format(*s))
def test_edge_shapes_full(torch_dev, shape):
    B, I, N, H, D, dt, T, ml = shape
    cfg = W.custom_config(B=B, I=I, N=N, H=H, D=D, dtype=dt, n_key_tiles=T, seed=1000 + N + D,
                          sigma_bias=2.0, mask_last=ml)
    w = W.make_inputs(cfg)
    say(f"[parity] edge shape {shape}")
    out = run_gpu(torch_dev, w, T).cpu().numpy()
    ref, _ = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, n_key_tiles=T)
    compare(out, ref, TOL[dt], str(shape))


def test_both_entry_points_agree(torch_dev):
    w = W.make_inputs(W.custom_config(B=1, I=40, N=40, H=4, D=32, dtype="bf16", n_key_tiles=3, seed=77))
    say("[parity] tri_attn_fwd vs tri_attn_fwd_rows")
    a = run_gpu(torch_dev, w, 3, rows_entry=False)
    b = run_gpu(torch_dev, w, 3, rows_entry=True)
    assert torch_dev.equal(a, b)


# ---------------------------------------------------------------------------
# properties
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_ring_step_count_invariance(torch_dev, dtype):
    """T key tiles joined by the merge give the result of T = 1.  The fp32 path folds tile
    by tile, so T changes only its rounding.  The matrix-core forward folds contiguous
    32-key blocks in the same ascending order whatever T is (the merge is associative), so
    for bf16 the tiles are also run as separate ring steps -- one state per tile, merged in
    ring order by tri_attn_state_merge -- which is the per-tile merge made explicit."""
    import pair_biased_triangle_amd as P
    torch = torch_dev
    w = W.make_inputs(W.custom_config(B=1, I=64, N=200, H=4, D=32, dtype=dtype, seed=31, sigma_bias=2.0,
                                      mask_last=9))
    say(f"[parity] T sweep on N=200, {dtype}")
    ref, _ = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, n_key_tiles=1)
    base = run_gpu(torch, w, 1).cpu().numpy()
    q, k, v, bias, mask = (to_dev(torch, x) for x in (w.q, w.k, w.v, w.bias, w.mask))
    for T in (2, 3, 8, 13, 200):
        out = run_gpu(torch, w, T).cpu().numpy()
        compare(out, ref, TOL[dtype], f"T={T} vs oracle")
        compare(out, base, TOL[dtype] if dtype == "bf16" else 1e-5, f"T={T} vs T=1")
        if dtype == "bf16" and T <= 13:
            bounds = [t * (200 // T) + min(t, 200 % T) for t in range(T + 1)]
            run = P.tri_attn_tile_state(q, k, v, bias, mask, key_begin=bounds[0], key_end=bounds[1])
            for t in range(1, T):
                P.tri_attn_state_merge(*run, *P.tri_attn_tile_state(q, k, v, bias, mask, key_begin=bounds[t],
                                                                    key_end=bounds[t + 1]))
            merged, _ = P.tri_attn_state_finalize(*run)
            tref, _ = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, n_key_tiles=T)
            compare(merged.cpu().numpy(), tref, TOL[dtype], f"T={T} tile states merged in ring order vs oracle")


def test_fully_masked_rows_give_zero(torch_dev):
    torch = torch_dev
    for dt in ("bf16", "fp32"):
        cfg = W.custom_config(B=2, I=12, N=40, H=2, D=32, dtype=dt, n_key_tiles=4, seed=5)
        w = W.make_inputs(cfg)
        w.mask = np.zeros((2, 40), np.float32)
        w.mask[1, :] = -np.inf
        say(f"[parity] fully masked batch, {dt}")
        out = run_gpu(torch, w, 4).cpu().numpy()
        assert np.all(out[1] == 0.0)
        ref, _ = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, n_key_tiles=4)
        compare(out, ref, TOL[dt], f"masked batch {dt}")


def test_single_kept_key_copies_value(torch_dev):
    torch = torch_dev
    cfg = W.custom_config(B=1, I=16, N=100, H=4, D=32, dtype="bf16", n_key_tiles=5, seed=8, sigma_bias=4.0)
    w = W.make_inputs(cfg)
    w.mask = np.full((1, 100), -np.inf, np.float32)
    w.mask[0, 77] = 0.0
    say("[parity] one kept key")
    out = run_gpu(torch, w, 5).cpu().numpy()
    v = W.bf16_bits_to_f32(w.v)[:, :, 77:78]
    np.testing.assert_array_equal(out, np.broadcast_to(v, out.shape))


def test_uniform_attention_is_mean_of_v(torch_dev):
    torch = torch_dev
    cfg = W.custom_config(B=1, I=8, N=96, H=4, D=32, dtype="bf16", n_key_tiles=3, seed=9)
    w = W.make_inputs(cfg)
    w.q[:] = 0
    w.k[:] = 0
    w.bias[:] = 0
    say("[parity] uniform attention")
    out = run_gpu(torch, w, 3).cpu().numpy()
    mean = W.bf16_bits_to_f32(w.v).astype(np.float64).mean(axis=2, keepdims=True)
    compare(out, np.broadcast_to(mean, out.shape), 1e-5, "mean of v")


def test_huge_bias_shift_is_stable(torch_dev):
    """A +-1000 shift of bias rows (bias + 1000 rounds in bf16, so compare to the oracle on
    the rounded inputs): no overflow, no NaN."""
    torch = torch_dev
    cfg = W.custom_config(B=1, I=16, N=80, H=2, D=32, dtype="bf16", n_key_tiles=4, seed=10)
    w = W.make_inputs(cfg)
    b = W.bf16_bits_to_f32(w.bias)
    b[:, :, ::2, :] += 1000.0
    b[:, :, 1::2, :] -= 1000.0
    w.bias = W.f32_to_bf16_bits(b)
    say("[parity] +-1000 bias shift")
    out = run_gpu(torch, w, 4).cpu().numpy()
    ref, _ = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, n_key_tiles=4)
    compare(out, ref, TOL["bf16"], "shifted bias")


def test_repeatable_bitwise(torch_dev):
    torch = torch_dev
    w = W.make_inputs("crop_n256")
    say("[parity] two runs bitwise equal")
    a = run_gpu(torch, w, 4)
    b = run_gpu(torch, w, 4)
    assert torch.equal(a, b)


def test_guard_regions_untouched(torch_dev):
    import pair_biased_triangle_amd as P
    torch = torch_dev
    cfg = W.custom_config(B=1, I=19, N=45, H=4, D=32, dtype="bf16", n_key_tiles=2, seed=12)
    w = W.make_inputs(cfg)
    q, k, v, bias = (to_dev(torch, x) for x in (w.q, w.k, w.v, w.bias))
    n = q.numel()
    guard = 4096
    buf = torch.full((n + 2 * guard,), 7.25, dtype=torch.float32, device="cuda")
    out = buf[guard:guard + n].view(q.shape)
    say("[parity] guard canaries around out")
    P.tri_attn_fwd_rows(q, k, v, bias, None, n_key_tiles=2, out=out)
    torch.cuda.synchronize()
    assert torch.all(buf[:guard] == 7.25) and torch.all(buf[guard + n:] == 7.25)
    ref, _ = oracle.tri_attn(w.q, w.k, w.v, w.bias, None, n_key_tiles=2)
    compare(out.cpu().numpy(), ref, TOL["bf16"], "guarded out")


def test_non_default_stream(torch_dev):
    import pair_biased_triangle_amd as P
    torch = torch_dev
    w = W.make_inputs(W.custom_config(B=1, I=64, N=64, H=4, D=32, dtype="bf16", n_key_tiles=2, seed=13))
    q, k, v, bias = (to_dev(torch, x) for x in (w.q, w.k, w.v, w.bias))
    s = torch.cuda.Stream()
    say("[parity] side stream")
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out = P.tri_attn_fwd(q, k, v, bias, None, n_key_tiles=2, stream=s)
    s.synchronize()
    ref, _ = oracle.tri_attn(w.q, w.k, w.v, w.bias, None, n_key_tiles=2)
    compare(out.cpu().numpy(), ref, TOL["bf16"], "side stream")


def test_binding_rejects_bad_tensors(torch_dev):
    import pair_biased_triangle_amd as P
    torch = torch_dev
    q = torch.zeros((1, 8, 8, 2, 32), dtype=torch.bfloat16, device="cuda")
    bias = torch.zeros((1, 2, 8, 8), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(P.TriAttnError) as e:
        P.tri_attn_fwd(q, q, q, bias, n_key_tiles=9)
    assert e.value.status == -6
    with pytest.raises(TypeError):
        P.tri_attn_fwd(q, q, q, bias.float())
    with pytest.raises(ValueError):
        P.tri_attn_fwd(q, q, q, bias[:, :, :, :4])


def test_caller_workspace_matches_pool_workspace(torch_dev):
    import pair_biased_triangle_amd as P
    torch = torch_dev
    cfg = W.custom_config(B=2, I=21, N=150, H=3, D=32, dtype="bf16", n_key_tiles=6, seed=14, mask_last=7)
    w = W.make_inputs(cfg)
    q, k, v, bias, mask = (to_dev(torch, x) for x in (w.q, w.k, w.v, w.bias, w.mask))
    need = P.workspace_bytes(2, 3, 21, 150, 32, 6, P.TRI_ATTN_BF16)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    say("[parity] caller workspace vs library pool")
    a = P.tri_attn_fwd_rows(q, k, v, bias, mask, n_key_tiles=6, workspace=P.LIBRARY)
    b = P.tri_attn_fwd_rows_ws(q, k, v, bias, mask, workspace=ws, n_key_tiles=6)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    with pytest.raises(P.TriAttnError) as e:
        P.tri_attn_fwd_rows_ws(q, k, v, bias, mask, workspace=ws[: need - 16], n_key_tiles=6)
    assert e.value.status == -9


def test_bias_jump_is_exact(torch_dev):
    """A bias far above the rest of its row (+120 nats) and one far below (-1000): both
    leave the fp16 image's span, so those column blocks are computed by the fp32 kernel;
    the large key's value is returned."""
    torch = torch_dev
    cfg = W.custom_config(B=1, I=24, N=260, H=2, D=32, dtype="bf16", n_key_tiles=3, seed=15)
    w = W.make_inputs(cfg)
    b = W.bf16_bits_to_f32(w.bias)
    b[0, 0, 5:40, 200] = 120.0
    b[0, 1, 100:101, 250] = -1000.0
    w.bias = W.f32_to_bf16_bits(b)
    say("[parity] bias jump above the rest of the row")
    out = run_gpu(torch, w, 3).cpu().numpy()
    ref, _ = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, n_key_tiles=3)
    compare(out, ref, TOL["bf16"], "score jump")
    np.testing.assert_allclose(out[0, :, 5:40, 0], np.broadcast_to(W.bf16_bits_to_f32(w.v)[0, :, 200:201, 0], (24, 35, 32)),
                               atol=1e-6)


def test_qk_jump_takes_exact_fallback(torch_dev):
    """q.k of one key about 90 nats above the rest overflows the fast pass's reference
    (the normaliser leaves [2^-64, 2^64]); the workgroup recomputes with the exact running
    maximum and returns that key's value."""
    torch = torch_dev
    cfg = W.custom_config(B=1, I=24, N=260, H=2, D=32, dtype="bf16", n_key_tiles=3, seed=25)
    w = W.make_inputs(cfg)
    q, k = W.bf16_bits_to_f32(w.q), W.bf16_bits_to_f32(w.k)
    q[0, :, 5:40, 0, :] = 4.0
    k[0, :, 200, 0, :] = 4.0
    w.q, w.k = W.f32_to_bf16_bits(q), W.f32_to_bf16_bits(k)
    say("[parity] q.k jump past the fast pass's range")
    out = run_gpu(torch, w, 3).cpu().numpy()
    ref, _ = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, n_key_tiles=3)
    compare(out, ref, TOL["bf16"], "q.k jump")
    np.testing.assert_allclose(out[0, :, 5:40, 0], W.bf16_bits_to_f32(w.v)[0, :, 200:201, 0].repeat(35, axis=1),
                               atol=1e-6)


def test_masked_first_blocks(torch_dev):
    """Keys masked at the front: the first block of every row has no finite score."""
    torch = torch_dev
    cfg = W.custom_config(B=1, I=16, N=200, H=4, D=32, dtype="bf16", n_key_tiles=4, seed=16)
    w = W.make_inputs(cfg)
    w.mask = np.zeros((1, 200), np.float32)
    w.mask[0, :70] = -np.inf
    say("[parity] masked leading keys")
    out = run_gpu(torch, w, 4).cpu().numpy()
    ref, _ = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, n_key_tiles=4)
    compare(out, ref, TOL["bf16"], "masked leading keys")
