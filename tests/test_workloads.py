"""The seeded input generator: definition, determinism, distributions, structure."""
import hashlib
import json
import math
import os

import numpy as np
import pytest

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "workload_sha256.json")
MASK64 = (1 << 64) - 1


def py_mix64(z):
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def py_normal(seed, tid, e):
    """The generator's published definition, written out in Python integers."""
    key = py_mix64(py_mix64(seed) ^ ((tid * 0xD1B54A32D192ED03) & MASK64))
    w = py_mix64((key + ((e >> 1) + 1) * 0x9E3779B97F4A7C15) & MASK64)
    u1 = ((w >> 32) + 0.5) / 2 ** 32
    u2 = ((w & 0xFFFFFFFF) + 0.5) / 2 ** 32
    r = math.sqrt(-2.0 * math.log(u1))
    return r * (math.sin if e & 1 else math.cos)(2 * math.pi * u2)


def test_splitmix64_known_values():
    # SplitMix64 seeded with 0: the first outputs of the reference generator
    # (state += 0x9E3779B97F4A7C15, then the mix) are well known.
    assert py_mix64(0x9E3779B97F4A7C15) == 0xE220A8397B1DCDAF
    assert py_mix64((2 * 0x9E3779B97F4A7C15) & MASK64) == 0x6E789E6AA1B965F4
    L = W.lib()
    assert L.wl_word(0, 0) == 0xE220A8397B1DCDAF
    assert L.wl_word(0, 1) == 0x6E789E6AA1B965F4


def test_c_generator_matches_definition():
    a = W.normal_tensor(7, 3, (64,), 1.0, "fp32", start=1000)
    b = np.array([py_normal(7, 3, 1000 + e) for e in range(64)], dtype=np.float32)
    np.testing.assert_array_equal(a, b)
    s = W.normal_tensor(7, 3, (64,), 2.5, "fp32", start=1000)
    np.testing.assert_array_equal(s, (2.5 * np.array([py_normal(7, 3, 1000 + e) for e in range(64)])).astype(np.float32))


def test_bf16_rounding_is_nearest_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5,
                  3.3895313892515355e38, np.inf, -np.inf, 0.0, -0.0], dtype=np.float32)
    bits = W.f32_to_bf16_bits(f)
    assert bits.tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x7F7F, 0x7F80, 0xFF80, 0x0000, 0x8000]
    nan = W.f32_to_bf16_bits(np.array([np.nan], np.float32))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    back = W.bf16_bits_to_f32(W.f32_to_bf16_bits(x))
    assert np.all(np.abs(back - x) <= np.abs(x) * 2.0 ** -8)   # unit roundoff of bf16


def test_slices_are_consistent():
    full = W.normal_tensor(3, 1, (10, 7), 1.0, "bf16")
    part = W.normal_tensor(3, 1, (3, 7), 1.0, "bf16", start=4 * 7)
    np.testing.assert_array_equal(full[4:7], part)


def test_distribution_moments():
    x = W.normal_tensor(11, 0, (1 << 20,), 2.0, "fp32").astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 2.0) < 0.01
    assert abs(((x / 2) ** 4).mean() - 3.0) < 0.05


def test_streams_differ():
    a = W.normal_tensor(1, 0, (256,), 1.0, "fp32")
    b = W.normal_tensor(1, 1, (256,), 1.0, "fp32")
    c = W.normal_tensor(2, 0, (256,), 1.0, "fp32")
    assert abs(np.corrcoef(a, b)[0, 1]) < 0.2 and abs(np.corrcoef(a, c)[0, 1]) < 0.2


def test_chain_structure():
    cfg = W.CONFIGS["complex_n1024"]
    chain = W.chain_of(cfg)
    assert chain[0] == 0 and chain[-1] == 3 and np.all(np.diff(chain) >= 0)
    assert sorted(set(chain.tolist())) == [0, 1, 2, 3]
    small = W.custom_config(B=1, I=40, N=40, H=2, D=4, dtype="fp32", seed=9, sigma_bias=0.0,
                            n_chains=4, chain_add=3.0)
    bias = W.make_bias(small)
    ch = W.chain_of(small)
    same = ch[:, None] == ch[None, :]
    np.testing.assert_array_equal(bias[0, 0], np.where(same, 3.0, 0.0).astype(np.float32))


def test_repeated_block_pattern():
    cfg = W.custom_config(B=1, I=20, N=20, H=2, D=4, dtype="fp32", seed=5, sigma_bias=0.0,
                          pattern_L=6, pattern_blocks=3)
    bias = W.make_bias(cfg)
    for h in range(2):
        blocks = [bias[0, h, 6 * u:6 * u + 6, 6 * u:6 * u + 6] for u in range(3)]
        assert np.all(blocks[0] != 0)
        np.testing.assert_array_equal(blocks[0], blocks[1])
        np.testing.assert_array_equal(blocks[0], blocks[2])
        off = bias[0, h].copy()
        for u in range(3):
            off[6 * u:6 * u + 6, 6 * u:6 * u + 6] = 0
        assert np.all(off == 0)        # tokens 18, 19 and every off-diagonal block get nothing
    assert not np.array_equal(bias[0, 0, :6, :6], bias[0, 1, :6, :6])


def test_masks():
    m = W.make_mask(W.CONFIGS["single_gpu_n2700"])
    assert m.shape == (1, 2700) and np.all(np.isneginf(m[0, 2640:])) and np.all(m[0, :2640] == 0)
    assert W.make_mask(W.CONFIGS["complex_n1024"]) is None


def _digest(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def test_recorded_hashes():
    """Bytes of the small workloads are fixed by their seeds (recorded by
    tests/golden/make_workload_hashes.py, which calls only the generator)."""
    with open(GOLDEN) as f:
        rec = json.load(f)
    for name in ("tiny_n32_fp32", "crop_n256"):
        w = W.make_inputs(name)
        got = {t: _digest(getattr(w, t)) for t in ("q", "k", "v", "bias")}
        assert got == rec[name]


def test_config_table_accounting():
    c = W.CONFIGS["single_gpu_n2700"]
    assert c.flops == 4 * 4 * 2700 ** 3 * 32
    assert abs(c.flops / 1e12 - 10.0777) < 1e-3
    assert c.algorithmic_bytes == 3 * 2700 * 2700 * 128 * 2 + 4 * 2700 * 2700 * 2 + 4 * 2700 + 2700 * 2700 * 128 * 4
    r = W.CONFIGS["ring_share_n4096_i1024"]
    assert r.flops == 4 * 4 * 1024 * 4096 * 4096 * 32
