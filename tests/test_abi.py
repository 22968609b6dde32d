"""The C-ABI library: it loads, exports exactly what include/tri_attn.h declares, and
rejects bad arguments before any device work (so these run without a GPU).

No call here passes validation: the pointers are placeholders and must never reach a
kernel."""
import ctypes
import os
import re
import subprocess

import pytest

import pair_biased_triangle_amd as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tri_attn.h")

FP32, BF16 = 0, 1
OK, E_NULL, E_SHAPE, E_DTYPE, E_UNSUP, E_ALIGN, E_TILES, E_HIP, E_ALIAS, E_WS = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(tri_attn_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return P.load_library()


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(P.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", P.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(tri_attn_\w+)$", out, flags=re.M))
    assert exported == set(declared_functions())
    for name in declared_functions():
        assert hasattr(lib, name)


def test_version_and_status_strings(lib):
    assert lib.tri_attn_version() == 10100
    seen = set()
    for code in (OK, E_NULL, E_SHAPE, E_DTYPE, E_UNSUP, E_ALIGN, E_TILES, E_HIP, E_ALIAS, E_WS):
        s = P.status_string(code)
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == 10
    assert P.status_string(12345) == "unknown status"
    assert lib.tri_attn_last_hip_error() == 0


def fake(addr):
    return ctypes.c_void_p(addr)


# distinct, 16-byte aligned, far apart placeholders (never dereferenced)
Q, K, V, BIAS, MASK, OUT = (fake(0x10000000 * (n + 1)) for n in range(6))


def call(lib, q=Q, k=K, v=V, bias=BIAS, mask=None, out=OUT, B=1, H=4, N=64, D=32, T=1, dtype=BF16):
    return lib.tri_attn_fwd(q, k, v, bias, mask, out, B, H, N, D, T, dtype, None)


def call_rows(lib, I, N=64, **kw):
    return lib.tri_attn_fwd_rows(Q, K, V, BIAS, None, OUT, 1, 4, I, N, 32, kw.get("T", 1), BF16, None)


@pytest.mark.parametrize("which", ["q", "k", "v", "bias", "out"])
def test_null_pointers(lib, which):
    assert call(lib, **{which: None}) == E_NULL


def test_null_checked_before_shape(lib):
    assert call(lib, q=None, B=0, dtype=7) == E_NULL


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0), dict(D=0), dict(B=-3),
                                dict(N=1 << 40), dict(B=1 << 62, N=2)])
def test_bad_sizes(lib, kw):
    assert call(lib, **kw) == E_SHAPE


def test_rows_must_not_exceed_tokens(lib):
    assert call_rows(lib, I=65, N=64) == E_SHAPE
    assert call_rows(lib, I=0, N=64) == E_SHAPE


def test_bad_dtype(lib):
    assert call(lib, dtype=2) == E_DTYPE
    assert call(lib, dtype=-1) == E_DTYPE


def test_head_size_limit(lib):
    assert call(lib, D=65) == E_UNSUP
    assert call(lib, D=65, dtype=FP32) == E_UNSUP


@pytest.mark.parametrize("T", [0, -1, 65, 1 << 30])
def test_tile_count_range(lib, T):
    assert call(lib, T=T) == E_TILES


def test_tiles_checked_before_alignment(lib):
    assert call(lib, T=0, q=fake(0x10000002)) == E_TILES


@pytest.mark.parametrize("which", ["q", "k", "v", "bias", "out"])
def test_alignment(lib, which):
    assert call(lib, **{which: fake(0x70000008)}) == E_ALIGN


def test_mask_alignment(lib):
    assert call(lib, mask=fake(0x70000002)) == E_ALIGN


def test_out_overlapping_an_input(lib):
    assert call(lib, out=Q) == E_ALIAS
    assert call(lib, out=fake(0x10000000 * 4 + 64)) == E_ALIAS   # inside bias
    assert call(lib, mask=fake(0x10000000 * 6 + 1024)) == E_ALIAS  # mask inside out


# ---------------------------------------------------------------------------
# workspace
# ---------------------------------------------------------------------------
def test_workspace_bytes(lib):
    # bf16 D=32: B*H*ceil(N/128)*(key blocks)*128*32*4; key blocks = sum over tiles of ceil(len/32)
    assert lib.tri_attn_workspace_bytes(1, 4, 2700, 2700, 32, 8, BF16) == 4 * 22 * (8 * 11) * 128 * 32 * 4
    assert lib.tri_attn_workspace_bytes(1, 4, 1024, 4096, 32, 8, BF16) == 4 * 32 * (8 * 16) * 128 * 32 * 4
    assert lib.tri_attn_workspace_bytes(2, 3, 5, 7, 32, 3, BF16) == 6 * 1 * 3 * 128 * 32 * 4
    assert lib.tri_attn_workspace_bytes(1, 4, 64, 64, 32, 1, FP32) == 0
    assert lib.tri_attn_workspace_bytes(1, 4, 64, 64, 16, 1, BF16) == 0
    assert lib.tri_attn_workspace_bytes(1, 4, 64, 64, 32, 0, BF16) == E_TILES
    assert lib.tri_attn_workspace_bytes(1, 4, 65, 64, 32, 1, BF16) == E_SHAPE
    assert P.workspace_bytes(1, 4, 2700, 2700, 32, 8, 1) == 4 * 22 * 88 * 16384


WS = fake(0x70000000)


def call_ws(lib, ws=WS, nbytes=1 << 30, **kw):
    args = dict(q=Q, k=K, v=V, bias=BIAS, mask=None, out=OUT, B=1, H=4, I=64, N=64, D=32, T=1, dtype=BF16)
    args.update(kw)
    return lib.tri_attn_fwd_rows_ws(args["q"], args["k"], args["v"], args["bias"], args["mask"], args["out"],
                                    args["B"], args["H"], args["I"], args["N"], args["D"], args["T"], args["dtype"],
                                    ws, nbytes, None)


def test_workspace_errors(lib):
    need = lib.tri_attn_workspace_bytes(1, 4, 64, 64, 32, 1, BF16)
    assert call_ws(lib, nbytes=need - 1) == E_WS
    assert call_ws(lib, nbytes=-1) == E_WS
    assert call_ws(lib, ws=None) == E_NULL
    assert call_ws(lib, ws=fake(0x70000008)) == E_ALIGN
    assert call_ws(lib, ws=fake(0x10000000 + 256)) == E_ALIAS        # inside q
    assert call_ws(lib, ws=fake(0x10000000 * 6 - 64)) == E_ALIAS      # runs into out
    assert call_ws(lib, q=None) == E_NULL                              # ordinary checks come first
    assert call_ws(lib, T=65) == E_TILES


def test_row_span_limit_of_matrix_core_path(lib):
    # one (b, i) row of K holds N*H*D bf16 values; 32-bit byte offsets cap it below 2 GiB
    assert call(lib, N=1 << 16, H=1 << 9) == E_UNSUP
