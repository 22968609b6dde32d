"""Workspace ownership through the C ABI.

Every entry point that needs a matrix-core workspace runs two ways: its *_ws form with a
workspace the caller (here torch) allocates, in which the library allocates nothing -- the
binding's default -- and its namesake without a workspace argument, which takes one from
the library's pool.  Both run the same kernels, so the results must agree bit for bit.  The
pool's reserve must stay bounded by what calls use at once, and go back on release.
"""
import numpy as np
import pytest

import workloads as W
from tests.test_parity_gpu import say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import pair_biased_triangle_amd as P
    P.load_library()
    return torch


def inputs(torch, B=1, I=40, N=300, H=3, seed=81, mask_last=7):
    w = W.make_inputs(W.custom_config(B=B, I=I, N=N, H=H, D=32, dtype="bf16", n_key_tiles=3, seed=seed,
                                      sigma_bias=2.0, mask_last=mask_last))
    return w, tuple(to_dev(torch, x) for x in (w.q, w.k, w.v, w.bias, w.mask))


def same(torch, a, b, what):
    a = a if isinstance(a, (tuple, list)) else (a,)
    b = b if isinstance(b, (tuple, list)) else (b,)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y), f"{what}: caller workspace and pool differ"
    say(f"  {what}: bitwise equal")


def test_every_ws_form_matches_the_pool(torch_dev):
    import pair_biased_triangle_amd as P
    torch = torch_dev
    lib = P.LIBRARY
    _, (q, k, v, bias, mask) = inputs(torch)
    say("[ws] forward family, caller workspace vs pool")
    same(torch, P.tri_attn_fwd_rows(q, k, v, bias, mask, n_key_tiles=3),
         P.tri_attn_fwd_rows(q, k, v, bias, mask, n_key_tiles=3, workspace=lib), "fwd_rows")
    same(torch, P.tri_attn_fwd_lse(q, k, v, bias, mask, n_key_tiles=3),
         P.tri_attn_fwd_lse(q, k, v, bias, mask, n_key_tiles=3, workspace=lib), "fwd_lse")
    acc, m, l = P.tri_attn_tile_state(q, k, v, bias, mask, key_begin=10, key_end=200)
    acc2, m2, l2 = P.tri_attn_tile_state(q, k, v, bias, mask, key_begin=10, key_end=200, workspace=lib)
    same(torch, (acc, m, l), (acc2, m2, l2), "tile_state")
    P.tri_attn_tile_state_update(q, k, v, bias, mask, key_begin=200, key_end=260, acc=acc, m=m, l=l)
    P.tri_attn_tile_state_update(q, k, v, bias, mask, key_begin=200, key_end=260, acc=acc2, m=m2, l=l2, workspace=lib)
    same(torch, (acc, m, l), (acc2, m2, l2), "tile_state_update")
    f1 = P.tri_attn_tile_state_final(q, k, v, bias, mask, key_begin=0, key_end=10, acc=acc, m=m, l=l, want_lse=True)
    f2 = P.tri_attn_tile_state_final(q, k, v, bias, mask, key_begin=0, key_end=10, acc=acc2, m=m2, l=l2,
                                     want_lse=True, workspace=lib)
    same(torch, f1, f2, "tile_state_final")

    _, (q, k, v, bias, mask) = inputs(torch, I=150, N=150, H=2, seed=82)
    same(torch, P.tri_attn_fwd_ending(q, k, v, bias, mask, n_key_tiles=2, want_lse=True),
         P.tri_attn_fwd_ending(q, k, v, bias, mask, n_key_tiles=2, want_lse=True, workspace=lib), "fwd_ending")
    acc, m, l = P.tri_attn_tile_state(q, k, v, bias, mask, key_begin=5, key_end=99, ending=True)
    same(torch, (acc, m, l), P.tri_attn_tile_state(q, k, v, bias, mask, key_begin=5, key_end=99, ending=True,
                                                   workspace=lib), "tile_state ending")

    for N in (2700, 301):     # the single pass over the raw bias, and the image path
        _, (q, k, v, bias, mask) = inputs(torch, I=1, N=N, H=4, seed=83)
        shp = (1, N, 4, 32)
        q1, k1, v1 = (t.view(shp) for t in (q, k, v))
        same(torch, P.pair_bias_attn_fwd(q1, k1, v1, bias, mask, n_key_tiles=8, want_lse=True),
             P.pair_bias_attn_fwd(q1, k1, v1, bias, mask, n_key_tiles=8, want_lse=True, workspace=lib),
             f"pair_bias N={N}")

    say("[ws] backward, caller workspace vs pool")
    _, (q, k, v, bias, mask) = inputs(torch, I=5, N=260, H=2, seed=84)
    out, lse = P.tri_attn_fwd_lse(q, k, v, bias, mask)
    dout = torch.randn(q.shape, dtype=torch.float32, device="cuda", generator=torch.Generator("cuda").manual_seed(3))
    same(torch, P.tri_attn_bwd(q, k, v, bias, mask, out, lse, dout),
         P.tri_attn_bwd(q, k, v, bias, mask, out, lse, dout, workspace=lib), "bwd")


def test_ws_forms_refuse_short_workspaces(torch_dev):
    import pair_biased_triangle_amd as P
    torch = torch_dev
    _, (q, k, v, bias, mask) = inputs(torch, I=8, N=200, H=2, seed=85)
    need = P.call_workspace_bytes(P.CALL_FWD, 1, 2, 8, 200, 32, 200, P.TRI_ATTN_BF16)
    short = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(P.TriAttnError) as e:
        P.tri_attn_fwd_lse(q, k, v, bias, mask, workspace=short)
    assert e.value.status == -9
    need_b = P.call_workspace_bytes(P.CALL_BWD, 1, 2, 8, 200, 32, 200, P.TRI_ATTN_BF16)
    out, lse = P.tri_attn_fwd_lse(q, k, v, bias, mask)
    dout = torch.zeros(q.shape, dtype=torch.float32, device="cuda")
    with pytest.raises(P.TriAttnError) as e:
        P.tri_attn_bwd(q, k, v, bias, mask, out, lse, dout,
                       workspace=torch.empty(need_b - 256, dtype=torch.uint8, device="cuda"))
    assert e.value.status == -9


def test_pool_reserve_stays_bounded_and_is_released(torch_dev):
    """Calls without a workspace argument, repeated and of different sizes, one after the
    other on one stream: the pool holds at most what one call needs (plus the driver's
    allocation granularity), not the sum of the calls; releasing it returns the memory."""
    import pair_biased_triangle_amd as P
    torch = torch_dev
    sizes = [(40, 300), (80, 600), (40, 300), (80, 600), (20, 150), (80, 600)]
    cases = {s: inputs(torch, I=s[0], N=s[1], H=3, seed=86)[1] for s in set(sizes)}
    largest = max(P.call_workspace_bytes(P.CALL_FWD, 1, 3, I, N, 32, N, P.TRI_ATTN_BF16) for I, N in sizes)
    P.pool_release()
    torch.cuda.synchronize()
    seen = []
    for rep in range(3):
        for s in sizes:
            q, k, v, bias, mask = cases[s]
            P.tri_attn_fwd_rows(q, k, v, bias, mask, n_key_tiles=3, workspace=P.LIBRARY)
            torch.cuda.synchronize()
            seen.append(P.pool_reserved_bytes())
    say(f"[ws] pool reserve over {len(seen)} calls: max {max(seen)} bytes, largest call needs {largest}")
    # measured on the MI355X: 42,968,344 bytes reserved for a largest need of 41,979,136
    assert max(seen) <= largest + (4 << 20), f"pool reserve {max(seen)} beyond one call's {largest} + 4 MiB"
    assert seen[-1] == seen[len(sizes) - 1], "the reserve kept growing over repeated calls"
    P.pool_release()
    torch.cuda.synchronize()
    after = P.pool_reserved_bytes()
    say(f"[ws] after release: {after} bytes")
    assert after == 0
