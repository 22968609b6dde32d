"""The error model behind the span guard of the matrix-core path (CPU only).

The bf16 kernels fold the bias into each score as fp16 values relative to the query's
largest bias r_j, in log2 units: c = fp16((bias + mask - r_j) log2 e).  fp16 keeps 11
significant bits, so c carries an absolute error up to |c| 2^-11, which grows with how far
a key's bias lies below r_j.  It matters when such a key still carries weight, i.e. when
its q.k makes up the distance.  The prepass therefore flags every (b, h, column block)
with a finite c below -kImageSpan (32 log2 units, about 22.2 nats), and those blocks run in
the fp32 kernels.

This file emulates the kernel's arithmetic in numpy (fp16 image, fp32 scores in log2
units, probabilities rounded to bf16, row sums over the rounded probabilities, an exact
running maximum) on the worst construction for the image: one key per query at r_j = +G
whose q.k puts its score 3 nats below zero, so that every other key, whose bias sits G
below r_j, carries the weight.  It checks that
  * inside the span (G <= 22 nats) the fp16 image keeps the result within half the bf16
    bar of 1e-2;
  * beyond it the error passes the bar (G = 64, 256), so the guard is needed;
  * an unrounded (fp32) bias stays at the bf16-probability level for every G;
and that the kernel source uses that span.
"""
import os
import re

import numpy as np
import pytest

L2E = 1.4426950408889634
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL = os.path.join(ROOT, "pair_biased_triangle_amd", "csrc", "kernel_bf16_mfma.hip")
SPAN_LOG2 = 32.0


def bf16_round(x):
    """Round binary32 values to bfloat16 (nearest even), returned as binary32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def inputs(G, seed, N=256, D=32):
    rng = np.random.default_rng(seed)
    k = bf16_round(rng.standard_normal((N, D)))
    q = bf16_round(rng.standard_normal((N, D)))
    v = bf16_round(rng.standard_normal((N, D))).astype(np.float64)
    bias = bf16_round(rng.standard_normal((N, N))).astype(np.float64)
    s = (q.astype(np.float64) @ k.T.astype(np.float64)) / np.sqrt(D)   # q.k / sqrt(D), exact products
    bias[:, 0] = G                                   # key 0: the largest bias of every query ...
    s[:, 0] = -(G + 3.0)                             # ... and a q.k that takes it back below zero
    return s, bias, v


def reference(s, bias, v):
    x = s + bias
    p = np.exp(x - x.max(axis=1, keepdims=True))
    return (p @ v) / p.sum(axis=1, keepdims=True)


def emulate(s, bias, v, image):
    """The matrix-core path's arithmetic with the bias image in `image` precision."""
    r = bias.max(axis=1, keepdims=True)
    c = ((bias - r) * L2E).astype(np.float32)
    if image == "fp16":
        c = c.astype(np.float16)
    x = (s.astype(np.float32) * np.float32(L2E)).astype(np.float64) + c.astype(np.float64)
    x = x - x.max(axis=1, keepdims=True)             # exact running maximum
    p = bf16_round(np.exp2(x).astype(np.float32)).astype(np.float64)
    return (p @ v) / p.sum(axis=1, keepdims=True)


def worst_error(G, image, seeds=(0, 1, 2)):
    err = 0.0
    for seed in seeds:
        s, bias, v = inputs(G, seed)
        err = max(err, float(np.max(np.abs(emulate(s, bias, v, image) - reference(s, bias, v)))))
    return err


@pytest.mark.parametrize("G", [0.0, 8.0, 16.0, SPAN_LOG2 / L2E - 0.05])
def test_fp16_image_inside_the_span_keeps_half_the_bar(G):
    assert (G * L2E) < SPAN_LOG2
    err = worst_error(G, "fp16")
    assert err <= 5e-3, f"G={G}: {err:.2e}"


@pytest.mark.parametrize("G", [64.0, 256.0])
def test_fp16_image_beyond_the_span_breaks_the_bar(G):
    err = worst_error(G, "fp16")
    assert err > 1e-2, f"G={G}: {err:.2e} (the guard would not be needed)"


@pytest.mark.parametrize("G", [0.0, 32.0, 64.0, 256.0])
def test_unrounded_bias_stays_at_the_probability_rounding_level(G):
    err = worst_error(G, "fp32")
    assert err <= 2e-3, f"G={G}: {err:.2e}"


def test_error_grows_with_the_span():
    errs = [worst_error(G, "fp16") for G in (8.0, 32.0, 128.0)]
    assert errs[0] < errs[1] < errs[2], errs


def test_kernel_uses_this_span():
    src = open(KERNEL).read()
    m = re.search(r"constexpr float kImageSpan = ([0-9.]+)f;", src)
    assert m, "kImageSpan not found in the kernel source"
    assert float(m.group(1)) == SPAN_LOG2
