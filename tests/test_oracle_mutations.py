"""Planted mistakes: each plausible slip in the oracle must fail at least one pin.

A copy of the oracle's C source is edited (one textual mutation per case), built
with gcc into a temporary directory, and run against the same checks that pin the
real oracle (library SDPA special case for both orientations, ring-step invariance,
huge bias shifts, uniform and single-key closed forms, merged ring-step states,
autograd for the backward).  The real oracle passes all of them; every
mutant must fail at least one.  Everything runs on the CPU.
"""
import math
import os

import numpy as np
import pytest

import oracle
from tests.test_oracle_pins import rand_case, sdpa_reference

MUTATIONS = {
    "drop_1_over_sqrt_d": ("double sc = dot * inv_sqrt_d + widen(bias, b_off, dtype);",
                           "double sc = dot + widen(bias, b_off, dtype);"),
    "scale_bias_too": ("dot * inv_sqrt_d + widen(bias, b_off, dtype)",
                       "(dot + widen(bias, b_off, dtype)) * inv_sqrt_d"),
    "bias_transposed": (": ((b * H + h) * N + j) * N + kk;", ": ((b * H + h) * N + kk) * N + j;"),
    "bias_column_stride": (": ((b * H + h) * N + j) * N + kk;", ": ((b * H + h) * N + kk) * N;"),
    "mask_ignored": ("sc += (double)mask[b * N + kk];\n                        s[kk - k0] = sc;",
                     "sc += 0.0;\n                        s[kk - k0] = sc;"),
    "keys_from_row_j": ("                                                     : ((bi * N + kk) * H + h) * D;\n"
                        "                        const int64_t b_off",
                        "                                                     : (((b * I + kk % I) * N + i) * H + h) * D;\n"
                        "                        const int64_t b_off"),
    "values_wrong_head": ("                                                     : ((bi * N + kk) * H + h) * D;\n"
                          "                        l_t += w;",
                          "                                                     : ((bi * N + kk) * H + (h + 1) % H) * D;\n"
                          "                        l_t += w;"),
    "merge_alpha_dropped": ("l = alpha * l + beta * l_t;", "l = l + beta * l_t;"),
    "merge_beta_dropped": ("a[d] = alpha * a[d] + beta * a_t[d];", "a[d] = alpha * a[d] + a_t[d];"),
    "merge_last_tile_wins": ("l = alpha * l + beta * l_t;", "l = l_t;"),
    "no_max_subtraction": ("const double w = exp(s[kk - k0] - m_t);", "const double w = exp(s[kk - k0]);"),
    "no_normalisation": ("o[d] = (l > 0.0) ? a[d] / l : 0.0;", "o[d] = a[d];"),
    "masked_tile_not_skipped": ("if (m_t == -INFINITY)\n                        continue;",
                                "if (0)\n                        continue;"),
    "lse_without_max": ("lse[r * H + h] = (l > 0.0) ? m + log(l) : -INFINITY;",
                        "lse[r * H + h] = (l > 0.0) ? log(l) : -INFINITY;"),
    "bf16_low_half": ("uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;",
                      "uint32_t bits = (uint32_t)((const uint16_t *)base)[idx];"),
    "dot_skips_last_d": ("for (int64_t d = 0; d < D; ++d)\n                            dot += widen(q, q_off + d, dtype) * "
                         "widen(k, k_off + d, dtype);\n                        double sc = dot * inv_sqrt_d + widen(bias, b_off",
                         "for (int64_t d = 0; d + 1 < D; ++d)\n                            dot += widen(q, q_off + d, dtype) * "
                         "widen(k, k_off + d, dtype);\n                        double sc = dot * inv_sqrt_d + widen(bias, b_off"),
    # ending-node orientation
    "ending_bias_not_transposed": ("ending ? ((b * H + h) * N + kk) * N + i", "ending ? ((b * H + h) * N + i) * N + kk"),
    "ending_keys_from_row": ("const int64_t k_off = ending ? (((b * N + kk) * N + j) * H + h) * D",
                             "const int64_t k_off = ending ? (((b * N + i) * N + kk) * H + h) * D"),
    "ending_values_from_row": ("const int64_t v_off = ending ? (((b * N + kk) * N + j) * H + h) * D",
                               "const int64_t v_off = ending ? (((b * N + i) * N + kk) * H + h) * D"),
    # one ring step's state
    "state_normalised": ("                        o[d] = a[d];\n                    lse[(r * H + h) * 2] = m;",
                         "                        o[d] = a[d] / l;\n                    lse[(r * H + h) * 2] = m;"),
    "state_reference_dropped": ("lse[(r * H + h) * 2] = m;", "lse[(r * H + h) * 2] = 0.0;"),
    # backward
    "bwd_delta_dropped": ("const double ds = p[kk] * (dp[kk] - delta);", "const double ds = p[kk] * dp[kk];"),
    "bwd_dq_unscaled": ("dq[q_off + d] += ds * widen(k, kv_off + d, dtype) * inv_sqrt_d;",
                        "dq[q_off + d] += ds * widen(k, kv_off + d, dtype);"),
    "bwd_dk_from_keys": ("dk[kv_off + d] += ds * widen(q, q_off + d, dtype) * inv_sqrt_d;",
                         "dk[kv_off + d] += ds * widen(k, kv_off + d, dtype) * inv_sqrt_d;"),
    "bwd_dv_weighted_by_ds": ("dv[kv_off + d] += p[kk] * (double)dout[q_off + d];",
                              "dv[kv_off + d] += ds * (double)dout[q_off + d];"),
    "bwd_dbias_not_summed_over_rows": ("dbias[((b * H + h) * N + j) * N + kk] += ds;",
                                       "dbias[((b * H + h) * N + j) * N + kk] = ds;"),
    # dbias of selected query columns
    "dbias_cols_delta_dropped": ("row[kk] += p[kk] * (dp[kk] - delta);", "row[kk] += p[kk] * dp[kk];"),
    "dbias_cols_last_row_only": ("row[kk] += p[kk] * (dp[kk] - delta);", "row[kk] = p[kk] * (dp[kk] - delta);"),
    "dbias_cols_wrong_column": ("h = bh % H, j = cols[c];", "h = bh % H, j = cols[(c + 1) % n_cols];"),
}



def battery(lib_path) -> list[str]:
    """Run the pins against the oracle at lib_path; return the names of those that fail."""
    failed = []
    run = lambda *a, **kw: oracle.tri_attn(*a, lib_path=lib_path, **kw)

    def check(name, fn):
        try:
            fn()
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(name)

    rng = np.random.default_rng(21)
    q, k, v, bias, mask = rand_case(rng, B=2, I=4, N=23, H=3, D=8, masked=(0, 5, 22), sigma_b=2.0)

    def sdpa():
        for T in (1, 5):
            out, _ = run(q, k, v, bias, mask, n_key_tiles=T)
            np.testing.assert_allclose(out, sdpa_reference(q, k, v, bias, mask), rtol=0, atol=1e-12)

    def tiles():
        base, base_lse = run(q, k, v, bias, mask, n_key_tiles=1)
        for T in (2, 3, 7, 23):
            for first in (0, T - 1):
                out, lse = run(q, k, v, bias, mask, n_key_tiles=T, first_tile=first)
                np.testing.assert_allclose(out, base, rtol=0, atol=1e-12)
                np.testing.assert_allclose(lse, base_lse, rtol=0, atol=1e-12)

    def shifts():
        b = np.round(bias * 256) / 256
        base, base_lse = run(q, k, v, b, mask, n_key_tiles=3)
        out, lse = run(q, k, v, b + np.float32(800.0), mask, n_key_tiles=3)
        assert np.all(np.isfinite(out))
        np.testing.assert_allclose(out, base, rtol=0, atol=1e-10)
        np.testing.assert_allclose(lse, base_lse + 800.0, rtol=0, atol=1e-10)

    def closed_forms():
        z = np.zeros_like(q)
        zb = np.zeros_like(bias)
        out, lse = run(z, z, v, zb, mask, n_key_tiles=4)
        keep = mask[0] == 0
        mean = v.astype(np.float64)[:, :, keep].mean(axis=2, keepdims=True)
        np.testing.assert_allclose(out, np.broadcast_to(mean, out.shape), rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, math.log(keep.sum()), rtol=0, atol=1e-13)
        one = np.full_like(mask, -np.inf)
        one[:, 0] = 0.0                              # only the first key survives
        out, _ = run(q, k, v, bias, one, n_key_tiles=3)
        np.testing.assert_array_equal(out, np.broadcast_to(v[:, :, :1].astype(np.float64), out.shape))

    def bf16():
        from workloads import bf16_bits_to_f32, f32_to_bf16_bits
        qb, kb, vb, bb = (f32_to_bf16_bits(x) for x in (q, k, v, bias))
        out, _ = run(qb, kb, vb, bb, mask, n_key_tiles=2)
        ref = sdpa_reference(bf16_bits_to_f32(qb), bf16_bits_to_f32(kb), bf16_bits_to_f32(vb),
                             bf16_bits_to_f32(bb), mask)
        np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)

    qe, ke, ve, be, me = rand_case(rng, B=1, I=9, N=9, H=2, D=8, masked=(0, 4), sigma_b=2.0)

    def ending():
        T = lambda x: np.ascontiguousarray(np.swapaxes(x, 1, 2))
        ref = T(sdpa_reference(T(qe), T(ke), T(ve), np.ascontiguousarray(np.swapaxes(be, 2, 3)), me))
        for n_tiles in (1, 4):
            out, _ = run(qe, ke, ve, be, me, n_key_tiles=n_tiles, ending=True)
            np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)

    def states():
        ref = sdpa_reference(q, k, v, bias, mask)
        bounds = (0, 1, 6, 13, 23)
        st = None
        for lo, hi in zip(bounds[:-1], bounds[1:]):
            acc, m, l = oracle.tile_state(q, k, v, bias, mask, key_begin=lo, key_end=hi, lib_path=lib_path)
            # m is the range's maximum score: the largest weight is exactly 1
            w_max = np.exp(np.zeros_like(m))
            assert np.all((l >= w_max) | (l == 0))
            st = (acc, m, l) if st is None else oracle.merge_states(*st, acc, m, l)
        out, _ = oracle.finalize_states(*st)
        np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
        for e in (False, True):
            qq, kk_, vv, bb, mm = (qe, ke, ve, be, me)
            acc, m, l = oracle.tile_state(qq, kk_, vv, bb, mm, key_begin=0, key_end=9, ending=e, lib_path=lib_path)
            full, lse = run(qq, kk_, vv, bb, mm, ending=e)
            out, lse2 = oracle.finalize_states(acc, m, l)
            np.testing.assert_allclose(out, full, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-12)

    def backward():
        from tests.test_oracle_bwd import autograd_reference
        dout = rng.standard_normal(q.shape).astype(np.float32)
        got = oracle.tri_attn_bwd(q, k, v, bias, mask, dout, lib_path=lib_path)
        ref = autograd_reference(q, k, v, bias, mask, dout)
        for g, r in zip(got, ref):
            np.testing.assert_allclose(g, r, rtol=0, atol=1e-12)
        cols = [0, 7, 22]
        got = oracle.tri_attn_dbias_cols(q, k, v, bias, mask, dout, cols, lib_path=lib_path)
        np.testing.assert_allclose(got, ref[3][:, :, cols], rtol=0, atol=1e-12)

    with np.errstate(all="ignore"):
        for name, fn in [("sdpa", sdpa), ("tiles", tiles), ("shifts", shifts),
                         ("closed_forms", closed_forms), ("bf16", bf16), ("ending", ending),
                         ("states", states), ("backward", backward)]:
            check(name, fn)
    return failed


def test_real_oracle_passes_battery(oracle_mod):
    assert battery(oracle.load.__defaults__[0]) == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTATIONS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique in the oracle source"
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(src.replace(old, new))
    lib = oracle.build(force=True, source=str(mutant_src), target=str(tmp_path / "libmutant.so"))
    failed = battery(lib)
    assert failed, f"planted mistake '{name}' passed every pin"
