"""GPU parity at the sizes the benchmark times, for every pass it times.

* complex_n1024 (N = 1024, four chains): the whole output tensor against the oracle.
* The backward at N = 2700 (single_gpu_n2700): one tri_attn_bwd over all 2700 rows, as
  `bench.py --pass bwd` runs it, compared on 16 sampled lines i (dq, dk, dv of a line
  depend on that line alone).  The forward statistics of those lines are the oracle's, so
  the bar is the kernels' own (1e-2 x max(1, max|oracle|)); the other lines keep the GPU
  forward's.  dbias sums over every line, so it is checked through a row-share call:
  the same 16 lines gathered into I = 16 (tri_attn_bwd on a row share returns the dbias
  of its rows), against the oracle's dbias of those lines; and the full call's dbias,
  summed over all 2700 rows, on eight query columns against the oracle's column form.
* The split-tile ring at N = 2700, T = 8 (`bench.py --pass ring`): the first step's
  state, six updates folded into it and the final step, on sampled query rows.
* One rank's share of a ring over a large assembly (ring_share_n4096_i1024: 1,024 rows of
  N = 4,096): the eight-step ring on sampled rows, and the backward (dq, dk, dv of four
  lines, dbias of the share on six query columns).
"""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.test_parity_gpu import TOL, compare, edge_rows, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import pair_biased_triangle_amd as P
    P.load_library()
    return torch


@pytest.fixture(scope="module")
def n2700(torch_dev):
    """single_gpu_n2700 inputs on the host and on the device."""
    w = W.make_inputs("single_gpu_n2700")
    dev = tuple(to_dev(torch_dev, x) for x in (w.q, w.k, w.v, w.bias, w.mask))
    return w, dev


@pytest.mark.timeout(600)
def test_complex_n1024_full(torch_dev):
    import pair_biased_triangle_amd as P
    w = W.make_inputs("complex_n1024")
    cfg = w.cfg
    say(f"[full] complex_n1024: whole tensor, T={cfg.n_key_tiles}")
    q, k, v, bias, mask = (to_dev(torch_dev, x) for x in (w.q, w.k, w.v, w.bias, w.mask))
    out = P.tri_attn_fwd(q, k, v, bias, mask, n_key_tiles=cfg.n_key_tiles)
    torch_dev.cuda.synchronize()
    got = out.cpu().numpy()
    del out
    ref, _ = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, n_key_tiles=cfg.n_key_tiles)
    compare(got, ref, TOL["bf16"], "complex_n1024 full tensor")


LINES = np.array([0, 1, 2, 127, 128, 255, 256, 1023, 1349, 1350, 2047, 2048, 2600, 2697, 2698, 2699])


def compare_rel(got, ref, rel, what):
    scale = max(1.0, float(np.max(np.abs(ref))))
    compare(got, ref, rel * scale, f"{what} (bar {rel:g} x {scale:.3g})")


@pytest.mark.timeout(900)
def test_backward_n2700_sampled_lines(torch_dev, n2700):
    import pair_biased_triangle_amd as P
    torch = torch_dev
    w, (q, k, v, bias, mask) = n2700
    cfg = w.cfg
    sel = lambda a: np.ascontiguousarray(a[:, LINES])
    say(f"[full] backward N=2700: oracle on {len(LINES)} lines")
    dout = torch.randn(q.shape, dtype=torch.float32, device="cuda", generator=torch.Generator("cuda").manual_seed(5))
    dout_l = sel(dout.cpu().numpy())
    wq, wk, wv = sel(w.q), sel(w.k), sel(w.v)
    ref_out, ref_lse = oracle.tri_attn(wq, wk, wv, w.bias, w.mask)
    ref = oracle.tri_attn_bwd(wq, wk, wv, w.bias, w.mask, dout_l)

    say("[full] backward N=2700: all 2700 lines on the GPU (the benchmark's call)")
    out, lse = P.tri_attn_fwd_lse(q, k, v, bias, mask, n_key_tiles=cfg.n_key_tiles)
    idx = torch.from_numpy(LINES).cuda()
    out[:, idx] = torch.from_numpy(ref_out.astype(np.float32)).cuda()
    lse[:, idx] = torch.from_numpy(ref_lse.astype(np.float32)).cuda()
    dq, dk, dv, dbias = P.tri_attn_bwd(q, k, v, bias, mask, out, lse, dout)
    torch.cuda.synchronize()
    del dbias, out, lse
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref[:3]):
        compare_rel(g[:, idx].cpu().numpy(), r, 1e-2, f"{name} N=2700, 16 lines of a full call")
    del dq, dk, dv

    say("[full] backward N=2700: the same 16 lines as one row share (dbias of those lines)")
    share = [to_dev(torch, x) for x in (wq, wk, wv)]
    g = P.tri_attn_bwd(*share, bias, mask, torch.from_numpy(ref_out.astype(np.float32)).cuda(),
                       torch.from_numpy(ref_lse.astype(np.float32)).cuda(), torch.from_numpy(dout_l).cuda())
    torch.cuda.synchronize()
    for name, got, r in zip(("dq", "dk", "dv", "dbias"), g, ref):
        compare_rel(got.cpu().numpy(), r, 1e-2, f"{name} N=2700 row share I=16")


@pytest.mark.timeout(600)
def test_ring_n2700_t8_sampled(torch_dev, n2700):
    import pair_biased_triangle_amd as P
    torch = torch_dev
    w, (q, k, v, bias, mask) = n2700
    cfg = w.cfg
    B, I, N, H, D, T = cfg.B, cfg.I, cfg.N, cfg.H, cfg.D, cfg.n_key_tiles
    bounds = [t * (N // T) + min(t, N % T) for t in range(T + 1)]
    say(f"[full] ring N=2700: state, {T - 2} updates, final step")
    acc, m, l = P.tri_attn_tile_state(q, k, v, bias, mask, key_begin=bounds[0], key_end=bounds[1])
    for t in range(1, T - 1):
        P.tri_attn_tile_state_update(q, k, v, bias, mask, key_begin=bounds[t], key_end=bounds[t + 1],
                                     acc=acc, m=m, l=l)
    out, lse = P.tri_attn_tile_state_final(q, k, v, bias, mask, key_begin=bounds[T - 1], key_end=bounds[T],
                                           acc=acc, m=m, l=l, want_lse=True)
    torch.cuda.synchronize()
    del acc, m, l
    rows = edge_rows(cfg, np.random.default_rng(17))
    idx = torch.from_numpy(rows).cuda()
    got = out.view(-1, H, D)[idx].cpu().numpy()
    got_lse = lse.view(-1, H)[idx].cpu().numpy()
    ref, ref_lse = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, n_key_tiles=T, rows=rows)
    compare(got, ref, TOL["bf16"], f"ring out, {len(rows)} rows")
    compare(got_lse, ref_lse, TOL["bf16"], f"ring lse, {len(rows)} rows")


@pytest.mark.timeout(600)
def test_backward_n2700_dbias_of_all_rows(torch_dev, n2700):
    """dbias of the full N = 2700 call sums dS over all 2700 rows, beyond what the oracle
    can compute here; two properties that hold at any size check it.
      * Every row of dbias sums to zero: sum_k ds_k = sum_k p_k (dp_k - delta) = 0,
        because sum_k p_k dp_k = dout . out = delta and sum_k p_k = 1.  The bar is the
        rounding of the 2700-term sums: 1e-2 of the largest |dbias| row sum of |values|.
      * The dbias of the whole call is the sum of the dbias of two row shares (rows
        [0, 1350) and [1350, 2700)), each a separate call: the cross-row reduction at full
        size.  Bar: 1e-4 of max |dbias| (fp32 sums of 2700 terms, different order)."""
    import pair_biased_triangle_amd as P
    torch = torch_dev
    w, (q, k, v, bias, mask) = n2700
    cfg = w.cfg
    say("[full] backward N=2700: dbias over all rows, then over two row shares")
    out, lse = P.tri_attn_fwd_lse(q, k, v, bias, mask, n_key_tiles=cfg.n_key_tiles)
    dout = torch.randn(q.shape, dtype=torch.float32, device="cuda", generator=torch.Generator("cuda").manual_seed(9))
    full = P.tri_attn_bwd(q, k, v, bias, mask, out, lse, dout)[3]
    torch.cuda.synchronize()
    half = cfg.I // 2
    parts = []
    for lo, hi in ((0, half), (half, cfg.I)):
        sl = lambda t: t[:, lo:hi].contiguous()
        parts.append(P.tri_attn_bwd(sl(q), sl(k), sl(v), bias, mask, sl(out), sl(lse), sl(dout))[3])
        torch.cuda.synchronize()
    kept = slice(0, cfg.N - cfg.mask_last)            # masked keys get no gradient
    row_sum = full[..., kept].double().sum(dim=-1)
    row_abs = full[..., kept].double().abs().sum(dim=-1)
    worst = float((row_sum.abs() / row_abs.clamp_min(1e-30)).max())
    say(f"  dbias row sums: max |sum| / sum|.| = {worst:.3e} (bar 1e-2), max |dbias| = {float(full.abs().max()):.3g}")
    assert worst <= 1e-2
    assert torch.all(full[..., cfg.N - cfg.mask_last:] == 0), "a masked key got a bias gradient"
    scale = float(full.abs().max())
    diff = float((full.double() - parts[0].double() - parts[1].double()).abs().max())
    say(f"  dbias(all rows) - dbias(rows < 1350) - dbias(rows >= 1350): max |diff| = {diff:.3e} (bar {1e-4 * scale:.3e})")
    assert diff <= 1e-4 * scale



@pytest.mark.timeout(900)
def test_backward_n2700_dbias_columns_over_all_rows(torch_dev, n2700):
    """dbias of the benchmark's full call (every one of the 2700 rows summed, from the GPU
    forward's out and lse) against the oracle's column form (dS summed over all rows in
    fp64, pinned to autograd) on eight query columns j: the first, tile and row-share
    edges, the last kept key's column and the last one, all heads and keys.  Bar: the
    backward's own, 1e-2 x max(1, max|oracle|)."""
    import pair_biased_triangle_amd as P
    torch = torch_dev
    w, (q, k, v, bias, mask) = n2700
    cfg = w.cfg
    cols = [0, 1, 255, 256, 1350, 2047, cfg.N - cfg.mask_last - 1, cfg.N - 1]
    say(f"[full] backward N=2700: dbias over all rows on columns {cols}")
    out, lse = P.tri_attn_fwd_lse(q, k, v, bias, mask, n_key_tiles=cfg.n_key_tiles)
    dout = torch.randn(q.shape, dtype=torch.float32, device="cuda", generator=torch.Generator("cuda").manual_seed(11))
    dbias = P.tri_attn_bwd(q, k, v, bias, mask, out, lse, dout)[3]
    torch.cuda.synchronize()
    got = dbias[:, :, cols].cpu().numpy()
    del dbias, out, lse
    ref = oracle.tri_attn_dbias_cols(w.q, w.k, w.v, w.bias, w.mask, dout.cpu().numpy(), cols)
    compare_rel(got, ref, 1e-2, "dbias N=2700, 8 columns summed over 2700 rows")
    assert np.all(got[..., cfg.N - cfg.mask_last:] == 0), "a masked key got a bias gradient"


@pytest.mark.timeout(600)
def test_ending_n2700_sampled(torch_dev, n2700):
    """The ending node on the benchmark's workload, as `bench.py --pass ending` runs it:
    with the lse, on sampled (i, j) against the oracle's ending orientation."""
    import pair_biased_triangle_amd as P
    torch = torch_dev
    w, (q, k, v, bias, mask) = n2700
    cfg = w.cfg
    say("[full] ending node N=2700")
    out, lse = P.tri_attn_fwd_ending(q, k, v, bias, mask, n_key_tiles=cfg.n_key_tiles, want_lse=True)
    torch.cuda.synchronize()
    rows = edge_rows(cfg, np.random.default_rng(23))
    idx = torch.from_numpy(rows).cuda()
    got = out.view(-1, cfg.H, cfg.D)[idx].cpu().numpy()
    got_lse = lse.view(-1, cfg.H)[idx].cpu().numpy()
    ref, ref_lse = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, n_key_tiles=cfg.n_key_tiles, rows=rows,
                                   ending=True)
    compare(got, ref, TOL["bf16"], f"ending out, {len(rows)} rows")
    compare(got_lse, ref_lse, TOL["bf16"], f"ending lse, {len(rows)} rows")


@pytest.fixture(scope="module")
def share4096(torch_dev):
    """ring_share_n4096_i1024 inputs (one rank's 1,024 rows of N = 4,096) on host and device."""
    w = W.make_inputs("ring_share_n4096_i1024")
    dev = tuple(to_dev(torch_dev, x) for x in (w.q, w.k, w.v, w.bias, w.mask))
    return w, dev


@pytest.mark.timeout(600)
def test_ring_share_n4096_t8_sampled(torch_dev, share4096):
    """The rank's share of a ring as the workload describes it: its 1,024 rows against
    all 4,096 keys in 8 key tiles folded by the ring-step entry points (first step, six
    updates, final step), on sampled rows against the oracle's tiled forward."""
    import pair_biased_triangle_amd as P
    torch = torch_dev
    w, (q, k, v, bias, mask) = share4096
    cfg = w.cfg
    B, I, N, H, D, T = cfg.B, cfg.I, cfg.N, cfg.H, cfg.D, cfg.n_key_tiles
    bounds = [t * (N // T) + min(t, N % T) for t in range(T + 1)]
    say(f"[full] ring share I=1024 N=4096: state, {T - 2} updates, final step")
    acc, m, l = P.tri_attn_tile_state(q, k, v, bias, mask, key_begin=bounds[0], key_end=bounds[1])
    for t in range(1, T - 1):
        P.tri_attn_tile_state_update(q, k, v, bias, mask, key_begin=bounds[t], key_end=bounds[t + 1],
                                     acc=acc, m=m, l=l)
    out, lse = P.tri_attn_tile_state_final(q, k, v, bias, mask, key_begin=bounds[T - 1], key_end=bounds[T],
                                           acc=acc, m=m, l=l, want_lse=True)
    torch.cuda.synchronize()
    del acc, m, l
    rows = edge_rows(cfg, np.random.default_rng(19))
    idx = torch.from_numpy(rows).cuda()
    got = out.view(-1, H, D)[idx].cpu().numpy()
    got_lse = lse.view(-1, H)[idx].cpu().numpy()
    ref, ref_lse = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, n_key_tiles=T, rows=rows)
    compare(got, ref, TOL["bf16"], f"ring share out, {len(rows)} rows")
    compare(got_lse, ref_lse, TOL["bf16"], f"ring share lse, {len(rows)} rows")


@pytest.mark.timeout(900)
def test_backward_ring_share_n4096(torch_dev, share4096):
    """The backward of the rank's share (I = 1024 rows, N = 4096): dq, dk, dv of four
    lines (their forward statistics the oracle's, bar the kernels' own 1e-2 x
    max(1, max|oracle|)) and dbias, summed over the share's 1,024 rows (the share's part of
    the bias gradient), on six query columns against the oracle's column form, end to end
    from the GPU forward's out and lse."""
    import pair_biased_triangle_amd as P
    torch = torch_dev
    w, (q, k, v, bias, mask) = share4096
    cfg = w.cfg
    lines = np.array([0, 511, 1000, 1023])
    sel = lambda a: np.ascontiguousarray(a[:, lines])
    dout = torch.randn(q.shape, dtype=torch.float32, device="cuda", generator=torch.Generator("cuda").manual_seed(13))
    dout_h = dout.cpu().numpy()
    say("[full] backward ring share I=1024 N=4096: oracle on 4 lines")
    wq, wk, wv = sel(w.q), sel(w.k), sel(w.v)
    ref_out, ref_lse = oracle.tri_attn(wq, wk, wv, w.bias, w.mask)
    ref = oracle.tri_attn_bwd(wq, wk, wv, w.bias, w.mask, sel(dout_h))
    out, lse = P.tri_attn_fwd_lse(q, k, v, bias, mask, n_key_tiles=cfg.n_key_tiles)
    idx = torch.from_numpy(lines).cuda()
    out_e, lse_e = out.clone(), lse.clone()           # end to end, for dbias
    out[:, idx] = torch.from_numpy(ref_out.astype(np.float32)).cuda()
    lse[:, idx] = torch.from_numpy(ref_lse.astype(np.float32)).cuda()
    dq, dk, dv, _ = P.tri_attn_bwd(q, k, v, bias, mask, out, lse, dout)
    torch.cuda.synchronize()
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref[:3]):
        compare_rel(g[:, idx].cpu().numpy(), r, 1e-2, f"{name} I=1024 N=4096, 4 lines of a full call")
    del dq, dk, dv, out, lse
    cols = [0, 67, 68, 2048, 4079, 4095]
    dbias = P.tri_attn_bwd(q, k, v, bias, mask, out_e, lse_e, dout)[3]
    torch.cuda.synchronize()
    got = dbias[:, :, cols].cpu().numpy()
    del dbias
    refc = oracle.tri_attn_dbias_cols(w.q, w.k, w.v, w.bias, w.mask, dout_h, cols)
    compare_rel(got, refc, 1e-2, "dbias I=1024 N=4096, 6 columns summed over 1024 rows")


N4200 = (4200, 4, 32, 8)          # N = I, H, D, key tiles


@pytest.fixture(scope="module")
def n4200(torch_dev):
    """A square problem larger than any benchmarked one: N = I = 4200 (H = 4, D = 32), whose
    q, k, v, out and gradients hold 2.26e9 elements each, so lines from i = 3995 on start
    past 2^31 elements (and 2^32 bytes of bf16).  Inputs from a seeded device generator."""
    torch = torch_dev
    N, H, D, _ = N4200
    g = torch.Generator("cuda").manual_seed(4200)
    q, k, v = (torch.randn((1, N, N, H, D), dtype=torch.bfloat16, device="cuda", generator=g) for _ in range(3))
    bias = torch.randn((1, H, N, N), dtype=torch.bfloat16, device="cuda", generator=g)
    mask = torch.zeros((1, N), dtype=torch.float32, device="cuda")
    mask[:, N - 30:] = -float("inf")
    return q, k, v, bias, mask


def bf16_host(torch, t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.timeout(600)
def test_forward_square_n4200_past_2_31_elements(torch_dev, n4200):
    """The oracle on sampled queries of lines on both sides of the 2^31-element boundary;
    each line's output depends on its own q, k, v and the shared bias only."""
    import pair_biased_triangle_amd as P
    torch = torch_dev
    N, H, D, T = N4200
    q, k, v, bias, mask = n4200
    say(f"[full] forward N=I={N}: one call over {N * N * H * D:.3g} elements per tensor")
    out = P.tri_attn_fwd(q, k, v, bias, mask, n_key_tiles=T)
    torch.cuda.synchronize()
    lines = [0, 1, 2047, 3994, 3995, 3996, 4199]
    cols = np.array([0, 1, 255, 256, 2100, 4170, 4199])
    idx = torch.tensor(lines, device="cuda")
    qs, ks, vs = (bf16_host(torch, t[:, idx]) for t in (q, k, v))
    got = out[:, idx][:, :, torch.from_numpy(cols).cuda()].cpu().numpy()
    del out
    rows = np.array([i * N + j for i in range(len(lines)) for j in cols])
    ref, _ = oracle.tri_attn(qs, ks, vs, bf16_host(torch, bias), mask.cpu().numpy(), n_key_tiles=T, rows=rows)
    compare(got.reshape(-1, H, D), ref, TOL["bf16"], f"N={N} forward, {len(rows)} queries of {len(lines)} lines")


@pytest.mark.timeout(900)
def test_backward_square_n4200_past_2_31_elements(torch_dev, n4200):
    """The backward over all 4200 lines: dq, dk, dv of lines on both sides of the 2^31-element
    boundary against the oracle (the forward statistics of those lines are the oracle's, so
    the bar is the kernels' own, 1e-2 x max(1, max|oracle|)), and dbias, a sum over every
    line, through its zero row sums."""
    import pair_biased_triangle_amd as P
    torch = torch_dev
    N, H, D, T = N4200
    q, k, v, bias, mask = n4200
    lines = [1, 3994, 3995, 4199]
    idx = torch.tensor(lines, device="cuda")
    qs, ks, vs = (bf16_host(torch, t[:, idx]) for t in (q, k, v))
    bias_h, mask_h = bf16_host(torch, bias), mask.cpu().numpy()
    dout = torch.randn(q.shape, dtype=torch.float32, device="cuda", generator=torch.Generator("cuda").manual_seed(42))
    dout_s = dout[:, idx].cpu().numpy()
    say(f"[full] backward N=I={N}: oracle on {len(lines)} lines")
    ref_out, ref_lse = oracle.tri_attn(qs, ks, vs, bias_h, mask_h)
    ref = oracle.tri_attn_bwd(qs, ks, vs, bias_h, mask_h, dout_s)
    say(f"[full] backward N=I={N}: all lines on the GPU")
    out, lse = P.tri_attn_fwd_lse(q, k, v, bias, mask, n_key_tiles=T)
    out[:, idx] = torch.from_numpy(ref_out.astype(np.float32)).cuda()
    lse[:, idx] = torch.from_numpy(ref_lse.astype(np.float32)).cuda()
    dq, dk, dv, dbias = P.tri_attn_bwd(q, k, v, bias, mask, out, lse, dout)
    torch.cuda.synchronize()
    del out, lse, dout
    for name, g_, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref[:3]):
        compare_rel(g_[:, idx].cpu().numpy(), r, 1e-2, f"{name} N={N}, {len(lines)} lines of a full call")
    del dq, dk, dv
    kept = slice(0, N - 30)
    row_sum = dbias[..., kept].double().sum(dim=-1)
    row_abs = dbias[..., kept].double().abs().sum(dim=-1)
    worst = float((row_sum.abs() / row_abs.clamp_min(1e-30)).max())
    say(f"  dbias row sums: max |sum| / sum|.| = {worst:.3e} (bar 1e-2)")
    assert worst <= 1e-2
    assert torch.all(dbias[..., N - 30:] == 0), "a masked key got a bias gradient"


@pytest.mark.timeout(600)
def test_ending_square_n4200_past_2_31_elements(torch_dev, n4200):
    """The ending node on the same problem: line j is a column, its keys (k, j) lie N * H * D
    elements apart, and outputs of rows i >= 3995 lie past 2^31 elements; the oracle's
    ending orientation on sampled (i, j)."""
    import pair_biased_triangle_amd as P
    torch = torch_dev
    N, H, D, T = N4200
    q, k, v, bias, mask = n4200
    say(f"[full] ending node N={N}")
    out = P.tri_attn_fwd_ending(q, k, v, bias, mask, n_key_tiles=T)
    torch.cuda.synchronize()
    ii = np.array([0, 1, 2047, 3994, 3995, 4199])
    jj = np.array([0, 255, 256, 2100, 4199])
    rows = np.array([i * N + j for i in ii for j in jj])
    got = out.view(-1, H, D)[torch.from_numpy(rows).cuda()].cpu().numpy()
    del out
    ref, _ = oracle.tri_attn(bf16_host(torch, q), bf16_host(torch, k), bf16_host(torch, v), bf16_host(torch, bias),
                             mask.cpu().numpy(), n_key_tiles=T, rows=rows, ending=True)
    compare(got, ref, TOL["bf16"], f"N={N} ending, {len(rows)} queries")


@pytest.mark.timeout(600)
def test_ring_square_n4200_past_2_31_elements(torch_dev, n4200):
    """The split-tile ring on the same problem (first state, six updates, final step): the
    states hold 2.26e9 accumulator elements; sampled queries of lines on both sides of the
    boundary against the oracle."""
    import pair_biased_triangle_amd as P
    torch = torch_dev
    N, H, D, T = N4200
    q, k, v, bias, mask = n4200
    bounds = [t * (N // T) + min(t, N % T) for t in range(T + 1)]
    say(f"[full] ring N={N}: state, {T - 2} updates, final step")
    acc, m, l = P.tri_attn_tile_state(q, k, v, bias, mask, key_begin=bounds[0], key_end=bounds[1])
    for t in range(1, T - 1):
        P.tri_attn_tile_state_update(q, k, v, bias, mask, key_begin=bounds[t], key_end=bounds[t + 1], acc=acc, m=m, l=l)
    out, lse = P.tri_attn_tile_state_final(q, k, v, bias, mask, key_begin=bounds[T - 1], key_end=bounds[T],
                                           acc=acc, m=m, l=l, want_lse=True)
    torch.cuda.synchronize()
    del acc, m, l
    lines = [2, 3995, 4199]
    cols = np.array([0, 256, 4199])
    idx = torch.tensor(lines, device="cuda")
    cidx = torch.from_numpy(cols).cuda()
    got = out[:, idx][:, :, cidx].cpu().numpy().reshape(-1, H, D)
    got_lse = lse[:, idx][:, :, cidx].cpu().numpy().reshape(-1, H)
    del out, lse
    qs, ks, vs = (bf16_host(torch, t[:, idx]) for t in (q, k, v))
    rows = np.array([i * N + j for i in range(len(lines)) for j in cols])
    ref, ref_lse = oracle.tri_attn(qs, ks, vs, bf16_host(torch, bias), mask.cpu().numpy(), n_key_tiles=T, rows=rows)
    compare(got, ref, TOL["bf16"], f"N={N} ring out, {len(rows)} queries")
    compare(got_lse, ref_lse, TOL["bf16"], f"N={N} ring lse")
