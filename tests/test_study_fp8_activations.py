"""Accuracy leg of the FP8-activation experiment on the latent-MoE layer.

The pages' engine quantizes the layer input to 8 bits before the D product
(TEARDOWN "A latent in front of the experts", the kernel excerpt: the input
rows are quantized, then multiplied with the 8-bit D codes). On gfx950 the
analogous fast path feeds every activation operand to the scaled
f8f6f4 matrix instructions as OCP E4M3 with one power-of-two (E8M0) scale per
32 consecutive values along the contraction. This module measures what that
rounding costs on the layer output, at the 145B and 120B layer shapes, with
every weight exact.

Variant, as the hardware would consume it (OCP Microscaling Formats v1.0:
shared scale 2^(floor(log2 max|v|) - 8), 8 being E4M3's largest exponent;
elements rounded to nearest even, saturated at 448): the operand of D (x),
of the expert gate/up (the latent), of the expert down (the SwiGLU product)
and of U (the per-group weighted sums). Routing stays exact (the router
reads x in fp32). "all" also rounds the shared expert's operands.

The exact forward is the oracle's; the variant reuses the oracle's decoded
weights, routing and SwiGLU and differs only in the rounding calls, so the
difference between the two is the rounding's effect alone.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as fm
from oracle import layer as ol
from latent_mixture_experts_amd import workloads as wl

import cases


def mx_e4m3(v, block=32):
    """Round the last axis of ``v`` to E4M3 with a power-of-two scale per
    ``block`` values (OCP MX, E8M0 shared scale)."""
    v = np.asarray(v, np.float64)
    b = v.reshape(-1, block)
    amax = np.abs(b).max(axis=1, keepdims=True)
    _, ex = np.frexp(np.where(amax == 0, 1.0, amax))
    scale = np.ldexp(1.0, (ex - 1) - 8)
    q = np.minimum(fm.round_pos(np.abs(b) / scale, 3, -6), 448.0) * np.sign(b)
    return (q * scale).reshape(v.shape)


def _forward(c, rnd, shared_too):
    """The layer with ``rnd`` applied to each routed GEMM's activation operand
    (and the shared expert's, if ``shared_too``)."""
    d, dec = c.d, c.dec
    lab = np.asarray(c.blobs["labels"], np.int64)
    x = c.x.astype(np.float64)
    lg = oracle.router_logits(c.x, c.blobs["router_bf16"], c.blobs.get("router_bias"))
    idx, w = oracle.select_topk(lg, d.top_k)
    xq = rnd(x)
    y = np.zeros((x.shape[0], d.hidden))
    for t in range(x.shape[0]):
        sums = {}
        for k in range(d.top_k):
            e = int(idx[t, k])
            g = int(lab[e])
            z = rnd(dec["D"][g] @ xq[t])
            wg, wu, wd = d.unpack_record(c.blobs["experts"][e])
            h = rnd(ol.silu(wg @ z) * (wu @ z))
            sums[g] = sums.get(g, 0.0) + w[t, k] * (wd @ h)
        for g in sorted(sums):
            y[t] += dec["U"][g] @ rnd(sums[g])
        sg, su, sd = dec["shared"]
        xs = xq[t] if shared_too else x[t]
        hs = ol.silu(sg @ xs) * (su @ xs)
        y[t] += sd @ (rnd(hs) if shared_too else hs)
    return y


def test_mx_e4m3_matches_torch_e4m3fn():
    """The rounding helper against torch's float8_e4m3fn cast (values inside
    the format's range, where the cast does not saturate), and its block
    scale: every block's largest magnitude lands in [256, 448]."""
    rng = np.random.default_rng(5)
    v = rng.standard_normal((64, 32)) * np.exp(rng.uniform(-12, 12, (64, 1)))
    got = mx_e4m3(v)
    amax = np.abs(v).max(axis=1, keepdims=True)
    _, ex = np.frexp(amax)
    scale = np.ldexp(1.0, (ex - 1) - 8)
    inside = np.abs(v) / scale <= 448.0
    ref = torch.from_numpy(v / scale).to(torch.float8_e4m3fn).to(torch.float64).numpy() * scale
    assert np.array_equal(got[np.broadcast_to(inside, v.shape)], ref[inside])
    top = np.abs(got).max(axis=1, keepdims=True) / scale
    assert np.all((top >= 256.0) & (top <= 448.0))
    assert np.array_equal(mx_e4m3(np.zeros((2, 32))), np.zeros((2, 32)))


@pytest.mark.slow
@pytest.mark.parametrize("name", ["145b_decode", "120b_decode"])
def test_fp8_activations_miss_the_output_bar(name):
    """Measured (seed 3, 4 tokens): E4M3 activations put the routed part of y
    7.5 % off (145B and 120B) and y itself 1.5 % / 1.0 % off, against the
    1e-3 bar that every path here meets; rounding the shared expert too
    raises y's error to 5.7 %. The variant is therefore not built."""
    c = cases.Case(wl.WORKLOADS[name], seed=3, tokens=4)
    ex = c.expect()
    y, yr = ex["y"], ex["y_routed"]
    same = _forward(c, lambda v: v, False)
    assert np.linalg.norm(same - y) <= 1e-12 * np.linalg.norm(y)
    for shared_too, lo_y in ((False, 5e-3), (True, 3e-2)):
        yy = _forward(c, mx_e4m3, shared_too)
        rel_y = np.linalg.norm(yy - y) / np.linalg.norm(y)
        rel_routed = np.linalg.norm(yy - y) / np.linalg.norm(yr)
        print("%s shared_too=%s: rel y %.3e, rel routed part %.3e" % (name, shared_too, rel_y,
                                                                       rel_routed))
        assert rel_y > lo_y > cases.REL_L2
        assert rel_routed > 3e-2
