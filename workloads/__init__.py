"""Seeded synthetic workloads for pair-biased triangle attention.

This module is shared by both sides of every parity check (the CPU oracle and the
HIP path) and by the benchmark.  It holds no attention arithmetic: it only draws the
inputs (q, k, v, the pair bias and the key padding mask) with the shapes, value
distributions and structure of the workloads the Fold-CP and Design-CP pages run,
from the counter-based generator in ``gen.c``.

Tensor layouts (all C-contiguous):
  q, k, v  [B, I, N, H, D]   bfloat16 bits (uint16) or binary32
  bias     [B, H, N, N]      same dtype as q
  mask     [B, N]            binary32, additive (0 keeps a key, -inf drops it), or None
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB_PATH = os.path.join(_HERE, "libworkloads.so")

# stream ids of the counter-based generator
TID_Q, TID_K, TID_V, TID_BIAS, TID_CHAIN, TID_PATTERN = 0, 1, 2, 3, 10, 11


def build(force: bool = True) -> str:
    """Compile gen.c into libworkloads.so next to it (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-ffp-contract=off", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        u64, i64, dbl = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double
        vp = ctypes.c_void_p
        L.wl_stream_key.argtypes = [u64, u64]
        L.wl_stream_key.restype = u64
        L.wl_word.argtypes = [u64, u64]
        L.wl_word.restype = u64
        L.wl_normal.argtypes = [u64, u64]
        L.wl_normal.restype = dbl
        L.wl_uniform.argtypes = [u64, u64]
        L.wl_uniform.restype = dbl
        L.wl_f32_to_bf16.argtypes = [vp, vp, i64]
        L.wl_f32_to_bf16.restype = None
        L.wl_normal_f32.argtypes = [u64, u64, i64, i64, dbl, vp]
        L.wl_normal_f32.restype = None
        L.wl_normal_bf16.argtypes = [u64, u64, i64, i64, dbl, vp]
        L.wl_normal_bf16.restype = None
        L.wl_bias.argtypes = [u64, u64, i64, i64, i64, dbl, vp, dbl, i64, i64, u64, vp, vp]
        L.wl_bias.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


# ---------------------------------------------------------------------------
# workload table
# ---------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    B: int
    I: int            # query rows i (I == N except for one rank's row share)
    N: int            # tokens (j and k axes)
    H: int
    D: int
    dtype: str        # "fp32" or "bf16": dtype of q, k, v and bias
    n_key_tiles: int  # ring steps of the context-parallel schedule, as key tiles
    seed: int
    sigma_qk: float = 1.0
    sigma_v: float = 1.0
    sigma_bias: float = 1.0
    mask_last: int = 0          # last M keys masked with -inf
    n_chains: int = 0           # block-diagonal chain term in the bias
    chain_add: float = 0.0
    pattern_L: int = 0          # repeated subunit block of size L on the diagonal
    pattern_blocks: int = 0
    stands_for: str = ""

    @property
    def flops(self) -> float:
        """Nominal FLOPs of the two contractions: 4*B*H*I*N*N*D (masked keys included)."""
        return 4.0 * self.B * self.H * self.I * self.N * self.N * self.D

    @property
    def in_bytes(self) -> int:
        return 4 if self.dtype == "fp32" else 2

    @property
    def algorithmic_bytes(self) -> int:
        """q, k, v and bias read once, mask read once, fp32 out written once."""
        s = self.in_bytes
        qkv = 3 * self.B * self.I * self.N * self.H * self.D * s
        bias = self.B * self.H * self.N * self.N * s
        mask = 4 * self.B * self.N if self.mask_last else 0
        out = 4 * self.B * self.I * self.N * self.H * self.D
        return qkv + bias + mask + out


CONFIGS: dict[str, Config] = {c.name: c for c in [
    Config("tiny_n32_fp32", B=1, I=32, N=32, H=4, D=32, dtype="fp32", n_key_tiles=2, seed=1,
           stands_for="smallest case, every element checked"),
    Config("crop_n256", B=1, I=256, N=256, H=4, D=32, dtype="bf16", n_key_tiles=4, seed=2,
           sigma_bias=2.0, mask_last=16,
           stands_for="the 256-token training crop (Fold-CP, Figure 5)"),
    Config("complex_n1024", B=1, I=1024, N=1024, H=4, D=32, dtype="bf16", n_key_tiles=8, seed=3,
           sigma_qk=32.0 ** -0.25, n_chains=4, chain_add=3.0,
           stands_for="a mid-size four-chain complex (Fold-CP, Figures 6 and 7)"),
    Config("single_gpu_n2700", B=1, I=2700, N=2700, H=4, D=32, dtype="bf16", n_key_tiles=8,
           seed=4, mask_last=60,
           stands_for="the single-GPU maximum of 2,700 tokens (Fold-CP, Table 2, 1x1 row)"),
    Config("ring_share_n4096_i1024", B=1, I=1024, N=4096, H=4, D=32, dtype="bf16",
           n_key_tiles=8, seed=5, pattern_L=68, pattern_blocks=60,
           stands_for="one rank's row share of a 60-subunit icosahedral assembly "
                      "(Design-CP, abstract)"),
]}


def custom_config(name="custom", *, B, I, N, H, D, dtype="bf16", n_key_tiles=1, seed=0, **kw):
    return Config(name, B=B, I=I, N=N, H=H, D=D, dtype=dtype, n_key_tiles=n_key_tiles,
                  seed=seed, **kw)


def chain_of(cfg: Config, seed: int | None = None) -> np.ndarray | None:
    """Chain id per token: n_chains contiguous chains with cut points drawn uniformly
    (without repetition) from {1, ..., N-1}."""
    if cfg.n_chains <= 1:
        return None
    seed = cfg.seed if seed is None else seed
    L = lib()
    key = L.wl_stream_key(seed, TID_CHAIN)
    cuts: list[int] = []
    c = 0
    while len(cuts) < cfg.n_chains - 1:
        cut = 1 + int(L.wl_uniform(key, c) * (cfg.N - 1))
        c += 1
        if cut not in cuts:
            cuts.append(cut)
    cuts.sort()
    chain = np.zeros(cfg.N, dtype=np.int32)
    for cut in cuts:
        chain[cut:] += 1
    return chain


@dataclasses.dataclass
class Workload:
    cfg: Config
    seed: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    bias: np.ndarray
    mask: np.ndarray | None

    @property
    def is_bf16(self) -> bool:
        return self.cfg.dtype == "bf16"


def normal_tensor(seed: int, tid: int, shape, sigma: float, dtype: str,
                  start: int = 0) -> np.ndarray:
    """sigma * N(0,1) from stream (seed, tid), elements start .. start + prod(shape) - 1."""
    n = int(np.prod(shape))
    if dtype == "bf16":
        a = np.empty(shape, dtype=np.uint16)
        lib().wl_normal_bf16(seed, tid, start, n, float(sigma), _ptr(a))
    else:
        a = np.empty(shape, dtype=np.float32)
        lib().wl_normal_f32(seed, tid, start, n, float(sigma), _ptr(a))
    return a


def make_bias(cfg: Config, seed: int | None = None) -> np.ndarray:
    seed = cfg.seed if seed is None else seed
    shape = (cfg.B, cfg.H, cfg.N, cfg.N)
    chain = chain_of(cfg, seed)
    f32 = b16 = None
    if cfg.dtype == "bf16":
        out = b16 = np.empty(shape, dtype=np.uint16)
    else:
        out = f32 = np.empty(shape, dtype=np.float32)
    lib().wl_bias(seed, TID_BIAS, cfg.B, cfg.H, cfg.N, float(cfg.sigma_bias),
                  _ptr(chain), float(cfg.chain_add), cfg.pattern_L, cfg.pattern_blocks,
                  TID_PATTERN, _ptr(f32), _ptr(b16))
    return out


def make_mask(cfg: Config) -> np.ndarray | None:
    if not cfg.mask_last:
        return None
    m = np.zeros((cfg.B, cfg.N), dtype=np.float32)
    m[:, cfg.N - cfg.mask_last:] = -np.inf
    return m


def make_inputs(cfg: Config | str, seed: int | None = None) -> Workload:
    """Draw every input of a workload.  q, k (sigma_qk), v (sigma_v) and the bias are
    i.i.d. normal plus the bias structure terms; the mask drops the last mask_last keys."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    seed = cfg.seed if seed is None else seed
    shape = (cfg.B, cfg.I, cfg.N, cfg.H, cfg.D)
    q = normal_tensor(seed, TID_Q, shape, cfg.sigma_qk, cfg.dtype)
    k = normal_tensor(seed, TID_K, shape, cfg.sigma_qk, cfg.dtype)
    v = normal_tensor(seed, TID_V, shape, cfg.sigma_v, cfg.dtype)
    bias = make_bias(cfg, seed)
    return Workload(cfg, seed, q, k, v, bias, make_mask(cfg))


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to binary32 values."""
    return (a.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().wl_f32_to_bf16(_ptr(a), _ptr(out), a.size)
    return out
