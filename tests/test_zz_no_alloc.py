"""The allocation-free forward (tri_attn_fwd_rows_noalloc, static device scratch) against
the allocating entry point it varies (tri_attn_fwd_rows, same kernels), through the C ABI.

Two calls in a row on one GPU, the second smaller, so the second runs on what the first
left in the shared scratch: (1) the benchmark's own size, N = 2700 with 8 key tiles, with
one column block whose bias spans 64 nats (its span flag set in the scratch); (2) a small
call with a narrow bias and a different layout of the scratch, which must clear and
rewrite what it reads.  Each output must equal the allocating entry point's bit for bit
(the bf16 bar of 1e-2 against the oracle follows from that; the small call is also checked
against the oracle directly).
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


def test_noalloc_matches_allocating_entry_point_twice(torch_dev):
    import pair_biased_triangle_amd as P
    torch = torch_dev

    cfg = W.CONFIGS["single_gpu_n2700"]
    w = W.make_inputs(cfg)
    b = W.bf16_bits_to_f32(w.bias)
    b[0, 1, 512:768, 100] = 64.0                    # one column block of head 1 beyond the image's span
    w.bias = W.f32_to_bf16_bits(b)
    del b
    q, k, v, bias, mask = (to_dev(torch, x) for x in (w.q, w.k, w.v, w.bias, w.mask))
    say("[noalloc] call 1: N=2700, T=8, one wide column block")
    ref1 = P.tri_attn_fwd_rows(q, k, v, bias, mask, n_key_tiles=cfg.n_key_tiles, workspace=P.LIBRARY)
    got1 = P.tri_attn_fwd_rows_noalloc(q, k, v, bias, mask, n_key_tiles=cfg.n_key_tiles)
    torch.cuda.synchronize()
    assert torch.equal(got1, ref1), "call 1 differs from tri_attn_fwd_rows"
    del q, k, v, bias, mask, got1, ref1

    small = W.custom_config(B=2, I=40, N=300, H=3, D=32, dtype="bf16", n_key_tiles=3, seed=71, mask_last=9)
    w2 = W.make_inputs(small)
    q, k, v, bias, mask = (to_dev(torch, x) for x in (w2.q, w2.k, w2.v, w2.bias, w2.mask))
    say("[noalloc] call 2: B=2, I=40, N=300, H=3, narrow bias")
    ref2 = P.tri_attn_fwd_rows(q, k, v, bias, mask, n_key_tiles=3, workspace=P.LIBRARY)
    got2 = P.tri_attn_fwd_rows_noalloc(q, k, v, bias, mask, n_key_tiles=3)
    torch.cuda.synchronize()
    assert torch.equal(got2, ref2), "call 2 differs from tri_attn_fwd_rows"
    expect, _ = oracle.tri_attn(w2.q, w2.k, w2.v, w2.bias, w2.mask, n_key_tiles=3)
    compare(got2.cpu().numpy(), expect, TOL["bf16"], "call 2 against the oracle")


def test_noalloc_refuses_a_problem_beyond_the_scratch(torch_dev):
    import pair_biased_triangle_amd as P
    torch = torch_dev
    q = torch.zeros((1, 2, 4096, 4, 32), dtype=torch.bfloat16, device="cuda")
    bias = torch.zeros((1, 4, 4096, 4096), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(P.TriAttnError) as e:
        P.tri_attn_fwd_rows_noalloc(q, q, q, bias, n_key_tiles=8)
    assert e.value.status == -11
