"""The oracle: plain fp64 CPU reference for pair-biased triangle attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path (the
HIP library and its binding) never imports, links or calls it, and it shares no code
with that path.

The arithmetic lives in ``tri_attn_oracle.c`` (double precision loops, one OpenMP
thread per query row, no fast-math).  This module only builds that file with gcc and
marshals numpy arrays into it.

What it computes and which passages it follows is stated at the top of the C file:
triangle attention (Fold-CP, Table 1) with the triangular bias shared across rows
(Fold-CP, Figure 2(a)), over T contiguous key tiles (one per ring step, Table 1's
caption) joined by the online-normaliser merge; the ending-node orientation; one ring
step's softmax state; the backward (gradients of the definition).  ``merge_states`` and
``finalize_states`` restate the merge rule
in numpy for states kept outside the C loop.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "tri_attn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libtri_attn_oracle.so")

DTYPE_FP32, DTYPE_BF16 = 0, 1


def build(force: bool = True, source: str = SOURCE, target: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc: -O2, OpenMP, no fast-math, no FMA contraction."""
    if force or not os.path.exists(target):
        tmp = target + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-ffp-contract=off", "-fno-fast-math", "-o", tmp, source, "-lm"])
        os.replace(tmp, target)
    return target


def _bind(path: str):
    L = ctypes.CDLL(path)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    L.oracle_tri_attn.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int,
                                  i64, i64, i64, i64, i64,
                                  vp, i64, i64, vp, i64, vp, vp]
    L.oracle_tri_attn.restype = ctypes.c_int
    L.oracle_tri_attn_ending.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int,
                                         i64, i64, i64, i64,
                                         vp, i64, i64, vp, i64, vp, vp]
    L.oracle_tri_attn_ending.restype = ctypes.c_int
    L.oracle_tile_state.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int,
                                    i64, i64, i64, i64, i64,
                                    i64, i64, ctypes.c_int, vp, i64, vp, vp]
    L.oracle_tile_state.restype = ctypes.c_int
    L.oracle_tri_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_int,
                                      i64, i64, i64, i64, i64, vp, vp, vp, vp]
    L.oracle_tri_attn_bwd.restype = ctypes.c_int
    L.oracle_tri_attn_dbias_cols.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_int,
                                             i64, i64, i64, i64, i64, vp, i64, vp]
    L.oracle_tri_attn_dbias_cols.restype = ctypes.c_int
    L.oracle_even_tiles.argtypes = [i64, i64, vp]
    L.oracle_even_tiles.restype = None
    L.oracle_num_threads.argtypes = []
    L.oracle_num_threads.restype = ctypes.c_int
    return L


_libs: dict[str, ctypes.CDLL] = {}


def load(path: str = _LIB_PATH):
    if path not in _libs:
        if path == _LIB_PATH and not os.path.exists(path):
            build(force=False)
        _libs[path] = _bind(path)
    return _libs[path]


def even_tiles(N: int, T: int, lib_path: str = _LIB_PATH) -> np.ndarray:
    """T+1 tile starts: the first N mod T tiles hold ceil(N/T) keys, the rest floor(N/T)."""
    starts = np.empty(T + 1, dtype=np.int64)
    load(lib_path).oracle_even_tiles(N, T, starts.ctypes.data)
    return starts


def num_threads(lib_path: str = _LIB_PATH) -> int:
    """OpenMP threads the oracle runs on."""
    return int(load(lib_path).oracle_num_threads())


def _dtype_of(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return DTYPE_FP32
    if a.dtype == np.uint16:
        return DTYPE_BF16
    raise TypeError(f"oracle inputs are binary32 or bfloat16 bits (uint16), got {a.dtype}")


def _prepare(q, k, v, bias, mask):
    q, k, v, bias = (np.ascontiguousarray(x) for x in (q, k, v, bias))
    dt = _dtype_of(q)
    if not all(_dtype_of(x) == dt for x in (k, v, bias)):
        raise TypeError("q, k, v and bias must share one dtype")
    B, I, N, H, D = q.shape
    if k.shape != q.shape or v.shape != q.shape or bias.shape != (B, H, N, N):
        raise ValueError("shape mismatch")
    if mask is not None:
        mask = np.ascontiguousarray(mask, dtype=np.float32)
        if mask.shape != (B, N):
            raise ValueError("mask must be [B, N]")
    return q, k, v, bias, mask, dt


def tri_attn(q, k, v, bias, mask=None, *, n_key_tiles: int = 1, tile_starts=None,
             first_tile: int = 0, rows=None, ending: bool = False, lib_path: str = _LIB_PATH):
    """Triangle attention in fp64.

    q, k, v: [B, I, N, H, D] float32 or uint16 (bfloat16 bits); bias: [B, H, N, N], same
    dtype; mask: [B, N] float32 additive or None.  Tiles: ``tile_starts`` (T+1 offsets)
    if given, else ``n_key_tiles`` near-equal contiguous tiles.  ``rows``: flat indices
    (b*I + i)*N + j to compute, or None for all.  ``ending``: the ending-node orientation
    (attention along columns, bias transposed; needs I == N).

    Returns (out, lse): out is [B, I, N, H, D] float64 (or [len(rows), H, D]), lse the
    matching [.., H] log-sum-exp of the scores.
    """
    q, k, v, bias, mask, dt = _prepare(q, k, v, bias, mask)
    B, I, N, H, D = q.shape
    if tile_starts is None:
        tile_starts = even_tiles(N, n_key_tiles, lib_path)
    tile_starts = np.ascontiguousarray(tile_starts, dtype=np.int64)
    T = len(tile_starts) - 1
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n = len(rows)
        out = np.empty((n, H, D), dtype=np.float64)
        lse = np.empty((n, H), dtype=np.float64)
    else:
        n = 0
        out = np.empty((B, I, N, H, D), dtype=np.float64)
        lse = np.empty((B, I, N, H), dtype=np.float64)
    L = load(lib_path)
    common = (q.ctypes.data, k.ctypes.data, v.ctypes.data, bias.ctypes.data,
              None if mask is None else mask.ctypes.data, dt)
    tail = (tile_starts.ctypes.data, T, first_tile, None if rows is None else rows.ctypes.data, n,
            out.ctypes.data, lse.ctypes.data)
    if ending:
        if I != N:
            raise ValueError("the ending orientation needs I == N")
        rc = L.oracle_tri_attn_ending(*common, B, H, N, D, *tail)
    else:
        rc = L.oracle_tri_attn(*common, B, H, I, N, D, *tail)
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")
    return out, lse


def tile_state(q, k, v, bias, mask=None, *, key_begin: int, key_end: int, ending: bool = False,
               rows=None, lib_path: str = _LIB_PATH):
    """One ring step's softmax state over keys [key_begin, key_end), in fp64.

    Returns (acc, m, l): acc [.., H, D] = sum_k e^(s_k - m) v_k, m [.., H] the range's
    maximum score (-inf when none is finite), l [.., H] = sum_k e^(s_k - m) (0 then).
    """
    q, k, v, bias, mask, dt = _prepare(q, k, v, bias, mask)
    B, I, N, H, D = q.shape
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n = len(rows)
        acc = np.empty((n, H, D), dtype=np.float64)
        ml = np.empty((n, H, 2), dtype=np.float64)
    else:
        n = 0
        acc = np.empty((B, I, N, H, D), dtype=np.float64)
        ml = np.empty((B, I, N, H, 2), dtype=np.float64)
    rc = load(lib_path).oracle_tile_state(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, bias.ctypes.data,
        None if mask is None else mask.ctypes.data, dt, B, H, I, N, D,
        int(key_begin), int(key_end), int(bool(ending)),
        None if rows is None else rows.ctypes.data, n, acc.ctypes.data, ml.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")
    return acc, ml[..., 0].copy(), ml[..., 1].copy()


def tri_attn_bwd(q, k, v, bias, mask, dout, *, lib_path: str = _LIB_PATH):
    """Gradients of starting-node triangle attention for the upstream gradient dout
    ([B, I, N, H, D] float32), in fp64.  Returns (dq, dk, dv, dbias): dq, dk, dv
    [B, I, N, H, D], dbias [B, H, N, N] summed over the rows i held."""
    q, k, v, bias, mask, dt = _prepare(q, k, v, bias, mask)
    dout = np.ascontiguousarray(dout, dtype=np.float32)
    B, I, N, H, D = q.shape
    if dout.shape != q.shape:
        raise ValueError("dout must be shaped like q")
    dq, dk, dv = (np.empty(q.shape, dtype=np.float64) for _ in range(3))
    dbias = np.empty((B, H, N, N), dtype=np.float64)
    rc = load(lib_path).oracle_tri_attn_bwd(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, bias.ctypes.data,
        None if mask is None else mask.ctypes.data, dout.ctypes.data, dt, B, H, I, N, D,
        dq.ctypes.data, dk.ctypes.data, dv.ctypes.data, dbias.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")
    return dq, dk, dv, dbias


def tri_attn_dbias_cols(q, k, v, bias, mask, dout, cols, *, lib_path: str = _LIB_PATH):
    """dbias of the query columns `cols` summed over every row i held: [B, H, len(cols), N]
    fp64, equal to tri_attn_bwd(...)[3][:, :, cols] at a cost of O(I N D) per column."""
    q, k, v, bias, mask, dt = _prepare(q, k, v, bias, mask)
    dout = np.ascontiguousarray(dout, dtype=np.float32)
    B, I, N, H, D = q.shape
    if dout.shape != q.shape:
        raise ValueError("dout must be shaped like q")
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    out = np.empty((B, H, len(cols), N), dtype=np.float64)
    rc = load(lib_path).oracle_tri_attn_dbias_cols(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, bias.ctypes.data,
        None if mask is None else mask.ctypes.data, dout.ctypes.data, dt, B, H, I, N, D,
        cols.ctypes.data, len(cols), out.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")
    return out


def merge_states(acc, m, l, acc_t, m_t, l_t):
    """The tiled-softmax merge of two states (Fold-CP, Figure 2(a)/(c); the online-normaliser
    rule), in fp64: M = max(m, m_t), l = e^(m-M) l + e^(m_t-M) l_t, acc likewise.  A state
    with l == 0 (no finite score) is the identity.  Returns the merged (acc, m, l)."""
    acc, m, l, acc_t, m_t, l_t = (np.asarray(x, dtype=np.float64) for x in (acc, m, l, acc_t, m_t, l_t))
    empty, empty_t = ~(l > 0), ~(l_t > 0)
    M = np.where(empty, m_t, np.where(empty_t, m, np.maximum(m, m_t)))
    with np.errstate(invalid="ignore", over="ignore"):
        alpha = np.where(empty, 0.0, np.exp(np.where(empty, 0.0, m - M)))
        beta = np.where(empty_t, 0.0, np.exp(np.where(empty_t, 0.0, m_t - M)))
    return alpha[..., None] * acc + beta[..., None] * acc_t, M, alpha * l + beta * l_t


def finalize_states(acc, m, l):
    """out = acc / l and lse = m + ln l (0 and -inf where l == 0), in fp64."""
    acc, m, l = (np.asarray(x, dtype=np.float64) for x in (acc, m, l))
    some = l > 0
    safe = np.where(some, l, 1.0)
    out = np.where(some[..., None], acc / safe[..., None], 0.0)
    lse = np.where(some, m + np.log(safe), -np.inf)
    return out, lse


def flat_rows(B: int, I: int, N: int, b, i, j) -> np.ndarray:
    """Flat row indices (b*I + i)*N + j for broadcastable index arrays."""
    return ((np.asarray(b, dtype=np.int64) * I + np.asarray(i, dtype=np.int64)) * N
            + np.asarray(j, dtype=np.int64)).ravel()
