"""Pair-biased triangle attention on AMD MI355X (gfx950).

Thin Python binding of ``libtri_attn.so`` (C ABI in ``include/tri_attn.h``).  Every
step of the computation runs in the library's HIP kernels; this module only checks and
marshals torch device tensors (torch provides device memory and streams) and raises
when the library is missing -- there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libtri_attn.so")

# tri_attn_dtype
TRI_ATTN_FP32, TRI_ATTN_BF16 = 0, 1
# tri_attn_call (kinds of calls that tri_attn_call_workspace_bytes sizes)
CALL_FWD, CALL_ENDING, CALL_STATE, CALL_STATE_ENDING, CALL_PAIR_BIAS, CALL_BWD = range(6)
# tri_attn_status
STATUS = {
    0: "TRI_ATTN_OK", -1: "TRI_ATTN_ERR_NULL", -2: "TRI_ATTN_ERR_SHAPE", -3: "TRI_ATTN_ERR_DTYPE",
    -4: "TRI_ATTN_ERR_UNSUPPORTED", -5: "TRI_ATTN_ERR_ALIGN", -6: "TRI_ATTN_ERR_TILES",
    -7: "TRI_ATTN_ERR_HIP", -8: "TRI_ATTN_ERR_ALIAS", -9: "TRI_ATTN_ERR_WORKSPACE",
    -10: "TRI_ATTN_ERR_RANGE", -11: "TRI_ATTN_ERR_SCRATCH",
}
EXPORTS = ("tri_attn_fwd", "tri_attn_fwd_rows", "tri_attn_fwd_rows_ws", "tri_attn_workspace_bytes",
           "tri_attn_fwd_rows_noalloc", "tri_attn_noalloc_scratch_bytes",
           "tri_attn_fwd_lse_ws", "tri_attn_fwd_ending_ws", "tri_attn_tile_state_ws", "tri_attn_tile_state_update_ws",
           "tri_attn_tile_state_final_ws", "pair_bias_attn_fwd_ws", "tri_attn_bwd_ws",
           "tri_attn_call_workspace_bytes", "tri_attn_pool_reserved_bytes", "tri_attn_pool_release",
           "tri_attn_fwd_lse", "tri_attn_fwd_ending", "tri_attn_tile_state", "tri_attn_tile_state_update",
           "tri_attn_tile_state_final", "tri_attn_state_merge",
           "tri_attn_state_finalize", "pair_bias_attn_fwd", "tri_attn_bwd",
           "tri_attn_status_string", "tri_attn_last_hip_error", "tri_attn_version")


class TriAttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libtri_attn.so (built by pair_biased_triangle_amd.build); raise if it is absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with `python -m pair_biased_triangle_amd.build`")
        L = ctypes.CDLL(path)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        L.tri_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, vp]
        L.tri_attn_fwd.restype = ctypes.c_int
        L.tri_attn_fwd_rows.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, i32, vp]
        L.tri_attn_fwd_rows.restype = ctypes.c_int
        L.tri_attn_fwd_rows_ws.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, i32, vp, i64, vp]
        L.tri_attn_fwd_rows_ws.restype = ctypes.c_int
        L.tri_attn_fwd_rows_noalloc.argtypes = L.tri_attn_fwd_rows.argtypes
        L.tri_attn_fwd_rows_noalloc.restype = ctypes.c_int
        L.tri_attn_noalloc_scratch_bytes.argtypes = []
        L.tri_attn_noalloc_scratch_bytes.restype = ctypes.c_int64
        L.tri_attn_fwd_lse.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, i32, vp]
        L.tri_attn_fwd_lse.restype = ctypes.c_int
        L.tri_attn_fwd_ending.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, vp]
        L.tri_attn_fwd_ending.restype = ctypes.c_int
        L.tri_attn_tile_state.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64,
                                          i32, i32, vp]
        L.tri_attn_tile_state.restype = ctypes.c_int
        L.tri_attn_tile_state_update.argtypes = L.tri_attn_tile_state.argtypes
        L.tri_attn_tile_state_update.restype = ctypes.c_int
        L.tri_attn_tile_state_final.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                                i64, i32, i32, vp]
        L.tri_attn_tile_state_final.restype = ctypes.c_int
        L.tri_attn_state_merge.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, vp]
        L.tri_attn_state_merge.restype = ctypes.c_int
        L.tri_attn_state_finalize.argtypes = [vp, vp, vp, vp, vp, i64, i64, vp]
        L.tri_attn_state_finalize.restype = ctypes.c_int
        L.pair_bias_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, vp]
        L.pair_bias_attn_fwd.restype = ctypes.c_int
        L.tri_attn_bwd.argtypes = [vp] * 12 + [i64, i64, i64, i64, i64, i32, vp]
        L.tri_attn_bwd.restype = ctypes.c_int
        W = [vp, i64]   # workspace, workspace_bytes
        L.tri_attn_fwd_lse_ws.argtypes = list(L.tri_attn_fwd_lse.argtypes)[:-1] + W + [vp]
        L.tri_attn_fwd_ending_ws.argtypes = list(L.tri_attn_fwd_ending.argtypes)[:-1] + W + [vp]
        L.tri_attn_tile_state_ws.argtypes = list(L.tri_attn_tile_state.argtypes)[:-1] + W + [vp]
        L.tri_attn_tile_state_update_ws.argtypes = list(L.tri_attn_tile_state_update.argtypes)[:-1] + W + [vp]
        L.tri_attn_tile_state_final_ws.argtypes = list(L.tri_attn_tile_state_final.argtypes)[:-1] + W + [vp]
        L.pair_bias_attn_fwd_ws.argtypes = list(L.pair_bias_attn_fwd.argtypes)[:-1] + W + [vp]
        L.tri_attn_bwd_ws.argtypes = list(L.tri_attn_bwd.argtypes)[:-1] + W + [vp]
        for name in ("tri_attn_fwd_lse_ws", "tri_attn_fwd_ending_ws", "tri_attn_tile_state_ws",
                     "tri_attn_tile_state_update_ws", "tri_attn_tile_state_final_ws", "pair_bias_attn_fwd_ws",
                     "tri_attn_bwd_ws", "tri_attn_pool_release"):
            getattr(L, name).restype = ctypes.c_int
        L.tri_attn_pool_release.argtypes = []
        L.tri_attn_pool_reserved_bytes.argtypes = []
        L.tri_attn_pool_reserved_bytes.restype = ctypes.c_int64
        L.tri_attn_call_workspace_bytes.argtypes = [i32, i64, i64, i64, i64, i64, i64, i32]
        L.tri_attn_call_workspace_bytes.restype = ctypes.c_int64
        L.tri_attn_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i32, i32]
        L.tri_attn_workspace_bytes.restype = ctypes.c_int64
        L.tri_attn_status_string.argtypes = [ctypes.c_int]
        L.tri_attn_status_string.restype = ctypes.c_char_p
        L.tri_attn_last_hip_error.argtypes = []
        L.tri_attn_last_hip_error.restype = ctypes.c_int
        L.tri_attn_version.argtypes = []
        L.tri_attn_version.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return load_library().tri_attn_status_string(status).decode()


def _check(rc: int):
    if rc != 0:
        msg = status_string(rc)
        if rc == -7:
            msg += f" (hipError {load_library().tri_attn_last_hip_error()})"
        raise TriAttnError(rc, msg)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return TRI_ATTN_BF16
    if t.dtype == torch.float32:
        return TRI_ATTN_FP32
    raise TypeError(f"q, k, v and bias must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _validate(q, k, v, bias, mask, out):
    import torch
    dt = _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("bias", bias)):
        if t.dtype != q.dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, q has {q.dtype}")
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if q.dim() != 5 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, I, N, H, D] shape")
    B, I, N, H, D = q.shape
    if tuple(bias.shape) != (B, H, N, N):
        raise ValueError(f"bias must be [B, H, N, N] = {(B, H, N, N)}, got {tuple(bias.shape)}")
    if mask is not None:
        if (mask.dtype != torch.float32 or tuple(mask.shape) != (B, N) or not mask.is_cuda
                or not mask.is_contiguous()):
            raise ValueError("mask must be a contiguous float32 device tensor of shape [B, N]")
    if out is None:
        out = torch.empty((B, I, N, H, D), dtype=torch.float32, device=q.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (B, I, N, H, D) or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor shaped like q")
    return dt, out


def call_workspace_bytes(kind: int, B: int, H: int, I: int, N: int, D: int, key_count: int, dtype_code: int) -> int:
    """Device workspace (bytes, 0 if none) of one call of kind ``kind`` (CALL_FWD, ...) at
    these sizes; ``key_count`` is the number of keys of a ring step's range (state calls).
    Calls tri_attn_call_workspace_bytes."""
    n = load_library().tri_attn_call_workspace_bytes(int(kind), B, H, I, N, D, int(key_count), dtype_code)
    if n < 0:
        raise TriAttnError(int(n), status_string(int(n)))
    return int(n)


def workspace_bytes(B: int, H: int, I: int, N: int, D: int, n_key_tiles: int, dtype_code: int) -> int:
    """Device workspace (bytes) tri_attn_fwd_rows_ws needs for these sizes (0 if none)."""
    n = load_library().tri_attn_workspace_bytes(B, H, I, N, D, int(n_key_tiles), dtype_code)
    if n < 0:
        raise TriAttnError(int(n), status_string(int(n)))
    return int(n)


def pool_reserved_bytes() -> int:
    """Bytes the library's memory pool holds on the current device (tri_attn_pool_reserved_bytes)."""
    n = load_library().tri_attn_pool_reserved_bytes()
    if n < 0:
        _check(int(n))
    return int(n)


def pool_release() -> None:
    """Return the unused memory of the library's pools to the driver (tri_attn_pool_release)."""
    _check(load_library().tri_attn_pool_release())


LIBRARY = "library"   # workspace=LIBRARY: call the entry point without a workspace argument (library pool)


def _workspace(workspace, kind, sizes, key_count, dt, device, stream):
    """The (pointer, bytes) pair a *_ws entry point takes, plus the tensor to keep alive, or
    None when the call should go to the entry point without a workspace (its pool).

    workspace=None: a uint8 tensor of exactly the call's need from torch's allocator (the
    library then allocates nothing); a tensor: used as given; LIBRARY: the pool."""
    import torch
    if isinstance(workspace, str):
        if workspace != LIBRARY:
            raise ValueError(f"workspace must be None, a device tensor or {LIBRARY!r}")
        return None
    B, H, I, N, D = sizes
    if workspace is None:
        need = call_workspace_bytes(kind, B, H, I, N, D, key_count, dt)
        if need == 0:
            return (None, 0), None
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
        if stream is not None and stream != torch.cuda.current_stream(device):
            workspace.record_stream(stream)   # torch must not hand it out again before the call's kernels end
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    return (_ptr(workspace), workspace.numel() * workspace.element_size()), workspace


def tri_attn_fwd_rows(q, k, v, bias, mask=None, *, n_key_tiles: int = 1, out=None, workspace=None, stream=None):
    """Triangle attention for the query rows i held in q, k, v (one rank's row share).

    q, k, v: [B, I, N, H, D] (bfloat16 or float32, device, contiguous); bias: [B, H, N, N]
    of the same dtype; mask: [B, N] float32 additive or None.  Returns out [B, I, N, H, D]
    float32 (written into ``out`` when given).  Enqueued on ``stream`` (default: torch's
    current stream); nothing is synchronised.  The workspace comes from torch (``workspace``
    None: the C entry point tri_attn_fwd_rows_ws, so the library allocates nothing), from
    the caller (a uint8 device tensor), or from the library's pool (``workspace=LIBRARY``:
    the C entry point tri_attn_fwd_rows).
    """
    L = load_library()
    dt, out = _validate(q, k, v, bias, mask, out)
    B, I, N, H, D = q.shape
    ws = _workspace(workspace, CALL_FWD, (B, H, I, N, D), N, dt, q.device, stream)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(mask), _ptr(out), B, H, I, N, D, int(n_key_tiles), dt)
    if ws is None:
        _check(L.tri_attn_fwd_rows(*args, _stream_handle(stream)))
    else:
        _check(L.tri_attn_fwd_rows_ws(*args, *ws[0], _stream_handle(stream)))
    return out


def tri_attn_fwd(q, k, v, bias, mask=None, *, n_key_tiles: int = 1, out=None, workspace=None, stream=None):
    """Triangle attention over all N query rows: q, k, v are [B, N, N, H, D].  With
    ``workspace=LIBRARY`` it calls the C entry point tri_attn_fwd; otherwise as
    tri_attn_fwd_rows (with I == N)."""
    L = load_library()
    if q.dim() != 5 or q.shape[1] != q.shape[2]:
        raise ValueError("tri_attn_fwd needs q of shape [B, N, N, H, D]; use tri_attn_fwd_rows for a row share")
    if isinstance(workspace, str) and workspace == LIBRARY:
        dt, out = _validate(q, k, v, bias, mask, out)
        B, _, N, H, D = q.shape
        _check(L.tri_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(mask), _ptr(out),
                              B, H, N, D, int(n_key_tiles), dt, _stream_handle(stream)))
        return out
    return tri_attn_fwd_rows(q, k, v, bias, mask, n_key_tiles=n_key_tiles, out=out, workspace=workspace, stream=stream)


def tri_attn_fwd_rows_ws(q, k, v, bias, mask=None, *, workspace, n_key_tiles: int = 1, out=None, stream=None):
    """tri_attn_fwd_rows with a caller-owned device workspace (a uint8 tensor of at least
    workspace_bytes(...) bytes); the library allocates nothing.  Calls tri_attn_fwd_rows_ws."""
    if workspace is None or isinstance(workspace, str):
        raise ValueError("workspace must be a contiguous device tensor")
    return tri_attn_fwd_rows(q, k, v, bias, mask, n_key_tiles=n_key_tiles, out=out, workspace=workspace,
                             stream=stream)


def tri_attn_fwd_rows_noalloc(q, k, v, bias, mask=None, *, n_key_tiles: int = 1, out=None, stream=None):
    """tri_attn_fwd_rows on the library's static device scratch: the library allocates
    nothing (for callers that cannot).  Calls on one GPU must not overlap in time.  Raises
    TRI_ATTN_ERR_SCRATCH when the problem needs more than noalloc_scratch_bytes().  Calls
    tri_attn_fwd_rows_noalloc."""
    L = load_library()
    dt, out = _validate(q, k, v, bias, mask, out)
    B, I, N, H, D = q.shape
    _check(L.tri_attn_fwd_rows_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(mask), _ptr(out),
                                       B, H, I, N, D, int(n_key_tiles), dt, _stream_handle(stream)))
    return out


def noalloc_scratch_bytes() -> int:
    """Size of the static scratch behind tri_attn_fwd_rows_noalloc."""
    return int(load_library().tri_attn_noalloc_scratch_bytes())


def _per_query(out, shape, name, t):
    """Check or allocate a float32 per-query array (one value per (b, ..., h))."""
    import torch
    if t is None:
        return torch.empty(shape, dtype=torch.float32, device=out.device)
    if t.dtype != torch.float32 or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name} must be a contiguous float32 device tensor of shape {tuple(shape)}")
    return t


def tri_attn_fwd_lse(q, k, v, bias, mask=None, *, n_key_tiles: int = 1, out=None, lse=None, workspace=None,
                     stream=None):
    """tri_attn_fwd_rows that also returns lse [B, I, N, H] (natural-log normaliser of every
    query; -inf where no key survives).  Returns (out, lse).  Calls tri_attn_fwd_lse_ws (or
    tri_attn_fwd_lse with workspace=LIBRARY)."""
    L = load_library()
    dt, out = _validate(q, k, v, bias, mask, out)
    B, I, N, H, D = q.shape
    lse = _per_query(out, (B, I, N, H), "lse", lse)
    ws = _workspace(workspace, CALL_FWD, (B, H, I, N, D), N, dt, q.device, stream)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(mask), _ptr(out), _ptr(lse), B, H, I, N, D,
            int(n_key_tiles), dt)
    if ws is None:
        _check(L.tri_attn_fwd_lse(*args, _stream_handle(stream)))
    else:
        _check(L.tri_attn_fwd_lse_ws(*args, *ws[0], _stream_handle(stream)))
    return out, lse


def tri_attn_fwd_ending(q, k, v, bias, mask=None, *, n_key_tiles: int = 1, out=None, lse=None,
                        want_lse: bool = False, workspace=None, stream=None):
    """Ending-node triangle attention (attention along columns, bias transposed):
    out[b,i,j] = sum_k softmax_k(q[b,i,j].k[b,k,j]/sqrt(D) + bias[b,h,k,i] + mask[b,k]) v[b,k,j].
    q, k, v: [B, N, N, H, D].  Returns out, or (out, lse) when want_lse or lse is given.
    Calls tri_attn_fwd_ending_ws (or tri_attn_fwd_ending with workspace=LIBRARY)."""
    L = load_library()
    if q.dim() != 5 or q.shape[1] != q.shape[2]:
        raise ValueError("tri_attn_fwd_ending needs q of shape [B, N, N, H, D]")
    dt, out = _validate(q, k, v, bias, mask, out)
    B, _, N, H, D = q.shape
    if want_lse or lse is not None:
        lse = _per_query(out, (B, N, N, H), "lse", lse)
    ws = _workspace(workspace, CALL_ENDING, (B, H, N, N, D), N, dt, q.device, stream)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(mask), _ptr(out), _ptr(lse), B, H, N, D, int(n_key_tiles), dt)
    if ws is None:
        _check(L.tri_attn_fwd_ending(*args, _stream_handle(stream)))
    else:
        _check(L.tri_attn_fwd_ending_ws(*args, *ws[0], _stream_handle(stream)))
    return (out, lse) if lse is not None else out


def _ring_step(name, q, k, v, bias, mask, key_begin, key_end, ending, acc, m, l, extra, dt, workspace, stream):
    L = load_library()
    B, I, N, H, D = q.shape
    kind = CALL_STATE_ENDING if ending else CALL_STATE
    count = max(1, min(int(key_end), N) - max(int(key_begin), 0))   # invalid ranges are refused by the call itself
    ws = _workspace(workspace, kind, (B, H, I, N, D), count, dt, q.device, stream)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(mask), _ptr(acc), _ptr(m), _ptr(l), *extra,
            B, H, I, N, D, int(key_begin), int(key_end), int(bool(ending)), dt)
    if ws is None:
        _check(getattr(L, name)(*args, _stream_handle(stream)))
    else:
        _check(getattr(L, name + "_ws")(*args, *ws[0], _stream_handle(stream)))


def tri_attn_tile_state(q, k, v, bias, mask=None, *, key_begin: int, key_end: int, ending: bool = False,
                        acc=None, m=None, l=None, workspace=None, stream=None):
    """Partial softmax state of the keys [key_begin, key_end) as one ring step: returns
    (acc [B, I, N, H, D] unnormalised, m [B, I, N, H] reference, l [B, I, N, H] normaliser).
    Calls tri_attn_tile_state_ws (or tri_attn_tile_state with workspace=LIBRARY)."""
    dt, acc = _validate(q, k, v, bias, mask, acc)
    B, I, N, H, D = q.shape
    m = _per_query(acc, (B, I, N, H), "m", m)
    l = _per_query(acc, (B, I, N, H), "l", l)
    _ring_step("tri_attn_tile_state", q, k, v, bias, mask, key_begin, key_end, ending, acc, m, l, (), dt,
               workspace, stream)
    return acc, m, l


def tri_attn_tile_state_update(q, k, v, bias, mask=None, *, key_begin: int, key_end: int, acc, m, l,
                               ending: bool = False, workspace=None, stream=None):
    """Fold the keys [key_begin, key_end), as one ring step, into the running state
    (acc, m, l) in place (l = 0 is the empty state).  Calls tri_attn_tile_state_update_ws
    (or tri_attn_tile_state_update with workspace=LIBRARY)."""
    dt, acc = _validate(q, k, v, bias, mask, acc)
    B, I, N, H, D = q.shape
    m = _per_query(acc, (B, I, N, H), "m", m)
    l = _per_query(acc, (B, I, N, H), "l", l)
    _ring_step("tri_attn_tile_state_update", q, k, v, bias, mask, key_begin, key_end, ending, acc, m, l, (), dt,
               workspace, stream)
    return acc, m, l


def tri_attn_tile_state_final(q, k, v, bias, mask=None, *, key_begin: int, key_end: int, acc, m, l,
                              ending: bool = False, out=None, lse=None, want_lse: bool = False, workspace=None,
                              stream=None):
    """The last ring step: fold the keys [key_begin, key_end) into the state (acc, m, l),
    which is only read, and return the finalised out [B, I, N, H, D] (and lse [B, I, N, H]
    when asked).  Calls tri_attn_tile_state_final_ws (or tri_attn_tile_state_final with
    workspace=LIBRARY)."""
    dt, acc = _validate(q, k, v, bias, mask, acc)
    _, out = _validate(q, k, v, bias, mask, out)
    B, I, N, H, D = q.shape
    m = _per_query(acc, (B, I, N, H), "m", m)
    l = _per_query(acc, (B, I, N, H), "l", l)
    if want_lse or lse is not None:
        lse = _per_query(acc, (B, I, N, H), "lse", lse)
    _ring_step("tri_attn_tile_state_final", q, k, v, bias, mask, key_begin, key_end, ending, acc, m, l,
               (_ptr(out), _ptr(lse)), dt, workspace, stream)
    return (out, lse) if lse is not None else out


def _state_shape(acc, m, l):
    import torch
    for name, t in (("acc", acc), ("m", m), ("l", l)):
        if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 device tensor")
    if tuple(m.shape) != tuple(acc.shape[:-1]) or tuple(l.shape) != tuple(m.shape):
        raise ValueError("m and l must have acc's shape without its last axis")
    return m.numel(), acc.shape[-1]


def tri_attn_state_merge(acc, m, l, acc_t, m_t, l_t, *, stream=None):
    """Merge the state (acc_t, m_t, l_t) into (acc, m, l) in place.  Calls tri_attn_state_merge."""
    L = load_library()
    rows, D = _state_shape(acc, m, l)
    if _state_shape(acc_t, m_t, l_t) != (rows, D) or acc_t.shape != acc.shape:
        raise ValueError("both states must have the same shapes")
    _check(L.tri_attn_state_merge(_ptr(acc), _ptr(m), _ptr(l), _ptr(acc_t), _ptr(m_t), _ptr(l_t), rows, D,
                                  _stream_handle(stream)))
    return acc, m, l


def tri_attn_state_finalize(acc, m, l, *, out=None, lse=None, stream=None):
    """out = acc / l (0 where l == 0) and lse = m + ln l.  Returns (out, lse).
    Calls tri_attn_state_finalize."""
    import torch
    L = load_library()
    rows, D = _state_shape(acc, m, l)
    if out is None:
        out = torch.empty_like(acc)
    if lse is None:
        lse = torch.empty_like(m)
    _check(L.tri_attn_state_finalize(_ptr(acc), _ptr(m), _ptr(l), _ptr(out), _ptr(lse), rows, D,
                                     _stream_handle(stream)))
    return out, lse


def pair_bias_attn_fwd(q, k, v, bias, mask=None, *, n_key_tiles: int = 1, out=None, lse=None,
                       want_lse: bool = False, workspace=None, stream=None):
    """Attention with pair bias: q, k, v [B, N, H, D], bias [B, H, N, N], mask [B, N] or None.
    Returns out [B, N, H, D] float32, or (out, lse [B, N, H]).  Calls pair_bias_attn_fwd_ws
    (or pair_bias_attn_fwd with workspace=LIBRARY)."""
    L = load_library()
    if q.dim() != 4:
        raise ValueError("pair_bias_attn_fwd needs q, k, v of shape [B, N, H, D]")
    B, N, H, D = q.shape
    q5, k5, v5 = (t.view(B, 1, N, H, D) for t in (q, k, v))
    out5 = None if out is None else out.view(B, 1, N, H, D)
    dt, out5 = _validate(q5, k5, v5, bias, mask, out5)
    if want_lse or lse is not None:
        lse = _per_query(out5, (B, N, H), "lse", lse)
    ws = _workspace(workspace, CALL_PAIR_BIAS, (B, H, 1, N, D), N, dt, q.device, stream)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(mask), _ptr(out5), _ptr(lse), B, H, N, D, int(n_key_tiles), dt)
    if ws is None:
        _check(L.pair_bias_attn_fwd(*args, _stream_handle(stream)))
    else:
        _check(L.pair_bias_attn_fwd_ws(*args, *ws[0], _stream_handle(stream)))
    out = out5.view(B, N, H, D)
    return (out, lse) if lse is not None else out


def tri_attn_bwd(q, k, v, bias, mask, out, lse, dout, *, workspace=None, stream=None):
    """Gradients of the starting-node operation for the upstream gradient dout.

    q, k, v, bias, mask: the forward's inputs; out, lse: its results (tri_attn_fwd_lse);
    dout: float32 shaped like q.  Returns (dq, dk, dv, dbias), float32; dbias [B, H, N, N]
    is summed over the rows i held.  Calls tri_attn_bwd_ws (or tri_attn_bwd with
    workspace=LIBRARY).
    """
    import torch
    L = load_library()
    dt, out = _validate(q, k, v, bias, mask, out)
    B, I, N, H, D = q.shape
    lse = _per_query(out, (B, I, N, H), "lse", lse)
    if dout.dtype != torch.float32 or tuple(dout.shape) != tuple(q.shape) or not dout.is_contiguous():
        raise ValueError("dout must be a contiguous float32 tensor shaped like q")
    dq, dk, dv = (torch.empty(q.shape, dtype=torch.float32, device=q.device) for _ in range(3))
    dbias = torch.empty((B, H, N, N), dtype=torch.float32, device=q.device)
    ws = _workspace(workspace, CALL_BWD, (B, H, I, N, D), N, dt, q.device, stream)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(mask), _ptr(out), _ptr(lse), _ptr(dout),
            _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbias), B, H, I, N, D, dt)
    if ws is None:
        _check(L.tri_attn_bwd(*args, _stream_handle(stream)))
    else:
        _check(L.tri_attn_bwd_ws(*args, *ws[0], _stream_handle(stream)))
    return dq, dk, dv, dbias


def _autograd_function():
    import torch

    class TriangleAttention(torch.autograd.Function):
        """Starting-node triangle attention as a differentiable torch op: forward through
        tri_attn_fwd_lse, backward through tri_attn_bwd (the mask is a constant)."""

        @staticmethod
        def forward(ctx, q, k, v, bias, mask, n_key_tiles):
            out, lse = tri_attn_fwd_lse(q, k, v, bias, mask, n_key_tiles=n_key_tiles)
            ctx.save_for_backward(q, k, v, bias, out, lse)
            ctx.mask = mask
            return out

        @staticmethod
        def backward(ctx, dout):
            q, k, v, bias, out, lse = ctx.saved_tensors
            dq, dk, dv, dbias = tri_attn_bwd(q, k, v, bias, ctx.mask, out, lse,
                                             dout.to(torch.float32).contiguous())
            return dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), dbias.to(bias.dtype), None, None

    return TriangleAttention


_TRI_FN = None


def triangle_attention(q, k, v, bias, mask=None, *, n_key_tiles: int = 1):
    """Differentiable starting-node triangle attention ([B, I, N, H, D] inputs; returns
    float32 out).  Gradients flow to q, k, v and bias."""
    global _TRI_FN
    if _TRI_FN is None:
        _TRI_FN = _autograd_function()
    return _TRI_FN.apply(q, k, v, bias, mask, int(n_key_tiles))
