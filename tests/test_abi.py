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
OK, E_NULL, E_SHAPE, E_DTYPE, E_UNSUP, E_ALIGN, E_TILES, E_HIP, E_ALIAS, E_WS, E_RANGE, E_SCRATCH = (
    0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10, -11)
NAME = r"(?:tri_attn_\w+|pair_bias_attn_\w+)"


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(" + NAME + r")\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return P.load_library()


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(P.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", P.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(" + NAME + r")$", out, flags=re.M))
    assert exported == set(declared_functions())
    for name in declared_functions():
        assert hasattr(lib, name)


def test_version_and_status_strings(lib):
    assert lib.tri_attn_version() == 10500
    seen = set()
    codes = (OK, E_NULL, E_SHAPE, E_DTYPE, E_UNSUP, E_ALIGN, E_TILES, E_HIP, E_ALIAS, E_WS, E_RANGE, E_SCRATCH)
    for code in codes:
        s = P.status_string(code)
        assert s and s != "unknown status"
        assert P.STATUS[code]
        seen.add(s)
    assert len(seen) == len(codes)
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
    # bf16 D=32: the fp16 image, B*H*ceil(N/256)*ceil(N/32)*256*32*2 bytes (256-column
    # blocks; 32-key blocks over the whole key range, whatever T), padded to 256 bytes, then
    # one fp32 reference per (b, h, query column padded to a multiple of 256), then one int
    # span flag per (b, h, column block)
    def need(B, H, N, blocks):
        img = B * H * -(-N // 256) * blocks * 256 * 32 * 2
        return -(-img // 256) * 256 + B * H * -(-N // 256) * 256 * 4 + B * H * -(-N // 256) * 4
    assert lib.tri_attn_workspace_bytes(1, 4, 2700, 2700, 32, 8, BF16) == need(1, 4, 2700, 85)
    assert lib.tri_attn_workspace_bytes(1, 4, 2700, 2700, 32, 200, BF16) == need(1, 4, 2700, 85)
    assert lib.tri_attn_workspace_bytes(1, 4, 1024, 4096, 32, 8, BF16) == need(1, 4, 4096, 128)
    assert lib.tri_attn_workspace_bytes(2, 3, 5, 7, 32, 3, BF16) == need(2, 3, 7, 1)
    assert need(1, 4, 2700, 85) == 4 * 11 * 85 * 16384 + 4 * 11 * 1024 + 4 * 11 * 4
    assert lib.tri_attn_workspace_bytes(1, 4, 64, 64, 32, 1, FP32) == 0
    assert lib.tri_attn_workspace_bytes(1, 4, 64, 64, 16, 1, BF16) == 0
    assert lib.tri_attn_workspace_bytes(1, 4, 64, 64, 32, 0, BF16) == E_TILES
    assert lib.tri_attn_workspace_bytes(1, 4, 65, 64, 32, 1, BF16) == E_SHAPE
    assert P.workspace_bytes(1, 4, 2700, 2700, 32, 8, 1) == need(1, 4, 2700, 85)


def test_workspace_bytes_of_one_row_calls(lib):
    # one row (attention with pair bias), bf16, D=32, even N: the single-pass kernel's key-range
    # states, S splits of [rows][D] accumulators plus m and l per row (S = as many ranges of
    # the B*H*ceil(N/128) query-block workgroups as one round of 768 resident workgroups
    # holds, at most 16, each split at least 4 key blocks); none when one range suffices;
    # odd N goes through the fp16 image
    def single_pass(B, H, N):
        n_qb, nblk, rows = -(-N // 128), -(-N // 32), B * N * H
        s = min(768 // (B * H * n_qb), nblk // 4, 16)
        if s < 2:
            return 0
        return s * rows * 32 * 4 + -(-(s * rows * 4) // 256) * 256 + s * rows * 4
    assert single_pass(1, 4, 2700) == 8 * 10800 * 32 * 4 + 345600 + 8 * 10800 * 4
    assert lib.tri_attn_workspace_bytes(1, 4, 1, 2700, 32, 8, BF16) == single_pass(1, 4, 2700)
    assert lib.tri_attn_workspace_bytes(3, 4, 1, 100, 32, 3, BF16) == 0 == single_pass(3, 4, 100)
    assert lib.tri_attn_workspace_bytes(2, 4, 1, 300, 32, 4, BF16) == single_pass(2, 4, 300) > 0
    odd = lib.tri_attn_workspace_bytes(1, 4, 1, 301, 32, 2, BF16)
    assert odd == 4 * 2 * 10 * 256 * 32 * 2 + 4 * 2 * 256 * 4 + 4 * 2 * 4   # image (2 column blocks x 10 key
                                                                             # blocks) + r_j + span flags
    assert P.workspace_bytes(1, 4, 1, 2700, 32, 8, 1) == single_pass(1, 4, 2700)


WS = fake(0x70000000)


def call_noalloc(lib, I=64, N=64, **kw):
    a = dict(q=Q, k=K, v=V, bias=BIAS, mask=None, out=OUT, B=1, H=4, D=32, T=1, dtype=BF16)
    a.update(kw)
    return lib.tri_attn_fwd_rows_noalloc(a["q"], a["k"], a["v"], a["bias"], a["mask"], a["out"], a["B"], a["H"], I, N,
                                         a["D"], a["T"], a["dtype"], None)


def test_noalloc_scratch_limit(lib):
    # the static scratch is 64 MiB; a workspace need above it is refused before any device
    # work (N = 4096: the fp16 image alone is 4 * 16 * 128 * 16 KB = 128 MiB)
    assert lib.tri_attn_noalloc_scratch_bytes() == 64 << 20 == P.noalloc_scratch_bytes()
    assert lib.tri_attn_workspace_bytes(1, 4, 64, 4096, 32, 1, BF16) > 64 << 20
    assert call_noalloc(lib, I=64, N=4096) == E_SCRATCH
    assert lib.tri_attn_workspace_bytes(1, 4, 2816, 2816, 32, 8, BF16) <= 64 << 20    # the stated limit
    assert lib.tri_attn_workspace_bytes(1, 4, 2817, 2817, 32, 8, BF16) > 64 << 20
    # the ordinary checks come first
    assert call_noalloc(lib, I=64, N=4096, q=None) == E_NULL
    assert call_noalloc(lib, I=64, N=4096, T=0) == E_TILES
    assert call_noalloc(lib, I=64, N=4096, out=fake(0x60000008)) == E_ALIGN


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


def test_ending_key_span_limit_of_matrix_core_path(lib):
    # ending node: consecutive keys are N*H*D bf16 values apart; a 32-key block must stay
    # within 32-bit byte offsets
    assert lib.tri_attn_fwd_ending(Q, K, V, BIAS, None, OUT, None, 1, 128, 8192, 32, 1, BF16, None) == E_UNSUP
    # the fp32 path has no such limit: the same sizes get as far as the alias check (out == k)
    assert lib.tri_attn_fwd_ending(Q, K, V, BIAS, None, K, None, 1, 128, 8192, 32, 1, FP32, None) == E_ALIAS


# ---------------------------------------------------------------------------
# lse, ending node, ring-step states, pair-bias attention
# ---------------------------------------------------------------------------
LSE, M_, L_ = (fake(0x10000000 * (n + 8)) for n in range(3))


def call_lse(lib, lse=LSE, **kw):
    a = dict(q=Q, k=K, v=V, bias=BIAS, mask=None, out=OUT, B=1, H=4, I=64, N=64, D=32, T=1, dtype=BF16)
    a.update(kw)
    return lib.tri_attn_fwd_lse(a["q"], a["k"], a["v"], a["bias"], a["mask"], a["out"], lse,
                                a["B"], a["H"], a["I"], a["N"], a["D"], a["T"], a["dtype"], None)


def test_lse_errors(lib):
    assert call_lse(lib, lse=None) == E_NULL
    assert call_lse(lib, q=None) == E_NULL
    assert call_lse(lib, lse=fake(0x10000000 * 8 + 2)) == E_ALIGN
    assert call_lse(lib, lse=fake(0x10000000 + 4096)) == E_ALIAS           # inside q
    assert call_lse(lib, lse=fake(0x10000000 * 6 + 4096)) == E_ALIAS       # inside out
    assert call_lse(lib, T=0) == E_TILES
    assert call_lse(lib, I=65) == E_SHAPE


def test_ending_errors(lib):
    f = lambda **kw: lib.tri_attn_fwd_ending(kw.get("q", Q), K, V, BIAS, None, kw.get("out", OUT), kw.get("lse"),
                                             1, 4, kw.get("N", 64), 32, kw.get("T", 1), BF16, None)
    assert f(q=None) == E_NULL
    assert f(N=0) == E_SHAPE
    assert f(T=65) == E_TILES
    assert f(out=K) == E_ALIAS
    assert f(lse=fake(0x10000000 * 6 + 64)) == E_ALIAS


STATE_ENTRIES = ("tri_attn_tile_state", "tri_attn_tile_state_update")


def call_state(lib, kb=0, ke=64, ending=0, m=M_, l=L_, acc=OUT, I=64, entry="tri_attn_tile_state", **kw):
    return getattr(lib, entry)(kw.get("q", Q), K, V, BIAS, None, acc, m, l, 1, 4, I, 64, 32, kb, ke, ending,
                               kw.get("dtype", BF16), None)


@pytest.mark.parametrize("entry", STATE_ENTRIES)
@pytest.mark.parametrize("kb,ke", [(-1, 10), (5, 5), (10, 5), (0, 65), (64, 70), (0, -1)])
def test_tile_state_key_range(lib, kb, ke, entry):
    assert call_state(lib, kb=kb, ke=ke, entry=entry) == E_RANGE


@pytest.mark.parametrize("entry", STATE_ENTRIES)
def test_tile_state_errors(lib, entry):
    call_state = lambda lib, **kw: globals()["call_state"](lib, entry=entry, **kw)
    assert call_state(lib, m=None) == E_NULL
    assert call_state(lib, l=None) == E_NULL
    assert call_state(lib, q=None) == E_NULL
    assert call_state(lib, ending=1, I=32) == E_SHAPE                     # the ending node needs I == N
    assert call_state(lib, m=fake(0x10000000 * 9 + 2)) == E_ALIGN
    assert call_state(lib, m=L_) == E_ALIAS                               # m and l share memory
    assert call_state(lib, l=fake(0x10000000 * 6 + 128)) == E_ALIAS      # l inside acc
    assert call_state(lib, dtype=5) == E_DTYPE


FOUT, FLSE = fake(0x10000000 * 20), fake(0x10000000 * 21)


def call_final(lib, kb=0, ke=64, m=M_, l=L_, acc=OUT, out=FOUT, lse=None, I=64, ending=0, **kw):
    return lib.tri_attn_tile_state_final(kw.get("q", Q), K, V, BIAS, None, acc, m, l, out, lse, 1, 4, I, 64, 32, kb, ke,
                                         ending, kw.get("dtype", BF16), None)


@pytest.mark.parametrize("kb,ke", [(-1, 10), (5, 5), (10, 5), (0, 65), (64, 70), (0, -1)])
def test_tile_state_final_key_range(lib, kb, ke):
    assert call_final(lib, kb=kb, ke=ke) == E_RANGE


def test_tile_state_final_errors(lib):
    assert call_final(lib, m=None) == E_NULL
    assert call_final(lib, l=None) == E_NULL
    assert call_final(lib, out=None) == E_NULL
    assert call_final(lib, q=None) == E_NULL
    assert call_final(lib, ending=1, I=32) == E_SHAPE
    assert call_final(lib, out=fake(0x10000000 * 20 + 8)) == E_ALIGN        # out needs 16 bytes
    assert call_final(lib, lse=fake(0x10000000 * 21 + 2)) == E_ALIGN
    assert call_final(lib, out=fake(0x10000000 * 6 + 256)) == E_ALIAS       # out inside acc
    assert call_final(lib, out=fake(0x10000000 + 4096)) == E_ALIAS          # out inside q
    assert call_final(lib, lse=fake(0x10000000 * 9)) == E_ALIAS             # lse on m
    assert call_final(lib, lse=fake(0x10000000 * 20 + 64)) == E_ALIAS       # lse inside out
    assert call_final(lib, dtype=5) == E_DTYPE


def test_state_merge_errors(lib):
    A, M1, L1, A2, M2, L2 = (fake(0x10000000 * (n + 1)) for n in range(6))
    mg = lambda rows=100, D=32, **kw: lib.tri_attn_state_merge(kw.get("a", A), M1, L1, kw.get("a2", A2), M2, L2,
                                                               rows, D, None)
    assert mg(a=None) == E_NULL
    assert mg(a2=None) == E_NULL
    assert mg(rows=0) == E_SHAPE
    assert mg(D=0) == E_SHAPE
    assert mg(D=65) == E_SHAPE
    assert mg(a=fake(0x10000002)) == E_ALIGN
    assert mg(a2=fake(0x10000000 + 64)) == E_ALIAS
    fin = lambda out=fake(0x70000000), lse=None: lib.tri_attn_state_finalize(A, M1, L1, out, lse, 100, 32, None)
    assert fin(out=None) == E_NULL
    assert fin(out=fake(0x10000000 + 256)) == E_ALIAS                     # out inside acc
    assert fin(lse=fake(0x10000000 * 2)) == E_ALIAS                       # lse on m
    assert fin(lse=fake(0x70000000 + 64)) == E_ALIAS                      # lse inside out
    assert fin(lse=fake(0x70100002)) == E_ALIGN


def test_pair_bias_errors(lib):
    pb = lambda **kw: lib.pair_bias_attn_fwd(kw.get("q", Q), K, V, BIAS, None, kw.get("out", OUT), kw.get("lse"),
                                             kw.get("B", 1), 4, kw.get("N", 64), kw.get("D", 32), kw.get("T", 1),
                                             BF16, None)
    assert pb(q=None) == E_NULL
    assert pb(B=0) == E_SHAPE
    assert pb(D=65) == E_UNSUP
    assert pb(T=65) == E_TILES
    assert pb(out=V) == E_ALIAS


def test_backward_errors(lib):
    OUTB, LSEB, DOUT, DQ, DK, DV, DB = (fake(0x10000000 * (n + 12)) for n in range(7))
    def bw(**kw):
        a = dict(q=Q, k=K, v=V, bias=BIAS, mask=None, out=OUTB, lse=LSEB, dout=DOUT, dq=DQ, dk=DK, dv=DV, db=DB,
                 B=1, H=4, I=64, N=64, D=32, dtype=BF16)
        a.update(kw)
        return lib.tri_attn_bwd(a["q"], a["k"], a["v"], a["bias"], a["mask"], a["out"], a["lse"], a["dout"],
                                a["dq"], a["dk"], a["dv"], a["db"], a["B"], a["H"], a["I"], a["N"], a["D"],
                                a["dtype"], None)
    for name in ("q", "k", "v", "bias", "out", "lse", "dout", "dq", "dk", "dv", "db"):
        assert bw(**{name: None}) == E_NULL, name
    assert bw(I=65) == E_SHAPE
    assert bw(dtype=3) == E_DTYPE
    assert bw(D=65) == E_UNSUP
    assert bw(q=fake(0x10000004)) == E_ALIGN
    assert bw(dq=fake(0x10000000 * 15 + 2)) == E_ALIGN
    assert bw(dq=Q) == E_ALIAS                                 # a result on an input
    assert bw(dk=DQ) == E_ALIAS                                # two results share memory
    assert bw(db=fake(0x10000000 * 12 + 512)) == E_ALIAS      # dbias inside out
