"""Pins of the oracle's layer, routing, permutation and stack.

The pages print no worked example of a layer output, so the layer is pinned
by: a pure-Python brute force written from the layer equation as printed
(U applied per expert, explicit index loops, no grouping); the linearity
identity; special cases that reduce to a plain top-K MoE or to the shared
expert alone; library routines (scipy softmax, torch silu); and invariants
that define the stable permutation uniquely."""

import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import formats as fm
from oracle import layer as ol
from oracle import kquants as kq
from oracle.layer import LayerDims, layer_forward, pack_layer, decode_layer

# Tiny, deliberately non-square shapes: H != ell != F != Fs, K < G < E.
SMALL = LayerDims(hidden=96, latent=64, n_experts=7, top_k=3, n_groups=3,
                  expert_ffn=32, shared_ffn=48, du_bits=8)


def _masters(d, seed=0, std=0.05, labels=None, expert_scale=1.0):
    rng = np.random.default_rng(seed)
    n = lambda *s: (rng.standard_normal(s) * std).astype(np.float32)
    ex = {e: (n(d.expert_ffn, d.latent) * expert_scale, n(d.expert_ffn, d.latent) * expert_scale,
              n(d.latent, d.expert_ffn) * expert_scale) for e in range(d.n_experts)}
    if labels is None:
        labels = rng.integers(0, d.n_groups, d.n_experts)
    return {
        "router": (rng.standard_normal((d.n_experts, d.hidden)) / math.sqrt(d.hidden)).astype(np.float32),
        "router_bias": None,
        "labels": np.asarray(labels, dtype=np.uint8),
        "D": np.stack([n(d.latent, d.hidden) * 4 for _ in range(d.n_groups)]),
        "U": np.stack([n(d.hidden, d.latent) for _ in range(d.n_groups)]),
        "experts": lambda e: ex[e],
        "shared": (n(d.shared_ffn, d.hidden), n(d.shared_ffn, d.hidden), n(d.hidden, d.shared_ffn)),
    }


def _x(d, t, seed=1):
    return np.random.default_rng(seed).standard_normal((t, d.hidden)).astype(np.float32)


# ---------------------------------------------------------------------------
# Brute force, pure Python


def _matvec(m, v):
    rows, cols = len(m), len(m[0])
    assert cols == len(v)
    return [sum(m[r][c] * v[c] for c in range(cols)) for r in range(rows)]


def _silu(z):
    return z / (1.0 + math.exp(-z))


def _brute_layer(d, blobs, x):
    """y[t] = sum_k w_k U_{g(e_k)} E_{e_k}(D_{g(e_k)} x[t]) + shared(x[t]),
    every product an explicit loop; U is applied per expert, not per group."""
    wr = fm.bf16_bits_to_f64(blobs["router_bf16"]).tolist()
    gb = fm.du_group_bytes(d.latent, d.hidden, d.du_bits)
    D = [fm.unpack_du(blobs["d_blob"][g * gb:(g + 1) * gb], d.latent, d.hidden, d.du_bits).tolist()
         for g in range(d.n_groups)]
    gb = fm.du_group_bytes(d.hidden, d.latent, d.du_bits)
    U = [fm.unpack_du(blobs["u_blob"][g * gb:(g + 1) * gb], d.hidden, d.latent, d.du_bits).tolist()
         for g in range(d.n_groups)]
    sg, su, sd = (fm.bf16_bits_to_f64(a).tolist() for a in blobs["shared"])
    labels = [int(v) for v in blobs["labels"]]
    bias = blobs.get("router_bias")
    ys, idxs = [], []
    for xt in np.asarray(x, np.float32).astype(np.float64).tolist():
        logits = [sum(xt[i] * wr[e][i] for i in range(d.hidden)) + (0.0 if bias is None else float(bias[e]))
                  for e in range(d.n_experts)]
        top = sorted(range(d.n_experts), key=lambda e: (-logits[e], e))[:d.top_k]
        m = max(logits[e] for e in top)
        z = [math.exp(logits[e] - m) for e in top]
        w = [v / sum(z) for v in z]
        y = [0.0] * d.hidden
        for wk, e in zip(w, top):
            g = labels[e]
            unpack = kq.unpack_q3k_record if d.expert_format == 1 else fm.unpack_expert_record
            gate, up, down = (a.tolist() for a in unpack(blobs["experts"][e], d.latent, d.expert_ffn))
            xl = _matvec(D[g], xt)
            hid = [_silu(a) * b for a, b in zip(_matvec(gate, xl), _matvec(up, xl))]
            out = _matvec(U[g], _matvec(down, hid))
            y = [yi + wk * oi for yi, oi in zip(y, out)]
        sh = _matvec(sd, [_silu(a) * b for a, b in zip(_matvec(sg, xt), _matvec(su, xt))])
        ys.append([a + b for a, b in zip(y, sh)])
        idxs.append(top)
    return np.array(ys), np.array(idxs)


@pytest.mark.parametrize("bits,bias", [(8, False), (4, True)])
def test_layer_matches_brute_force(bits, bias):
    d = LayerDims(**{**SMALL.__dict__, "du_bits": bits})
    m = _masters(d, seed=bits)
    if bias:
        m["router_bias"] = np.random.default_rng(3).standard_normal(d.n_experts).astype(np.float32)
    blobs = pack_layer(d, m)
    x = _x(d, 3)
    got = layer_forward(d, blobs, x, intermediates=True)
    want, idx = _brute_layer(d, blobs, x)
    assert np.array_equal(got["idx"], idx)
    assert np.max(np.abs(got["y"] - want)) <= 1e-12 * np.max(np.abs(want))


def test_q3k_layer_matches_brute_force():
    """The layer with Q3_K gate/up and IQ4_NL down expert records (latent
    256, one Q3_K super-block per row) against the brute force."""
    d = LayerDims(hidden=96, latent=256, n_experts=5, top_k=2, n_groups=2, expert_ffn=32,
                  shared_ffn=48, du_bits=8, expert_format=1)
    blobs = pack_layer(d, _masters(d, seed=5))
    assert blobs["experts"].shape == (5, kq.q3k_record_bytes(256, 32))
    x = _x(d, 2)
    got = layer_forward(d, blobs, x, intermediates=True)
    want, idx = _brute_layer(d, blobs, x)
    assert np.array_equal(got["idx"], idx)
    assert np.max(np.abs(got["y"] - want)) <= 1e-12 * np.max(np.abs(want))


def test_linearity_identity():
    """sum over experts of w U_{g(e)} E_e(...) == sum over groups of U_g sum_e."""
    d = SMALL
    blobs = pack_layer(d, _masters(d))
    x = _x(d, 4)
    r = layer_forward(d, blobs, x, intermediates=True)
    dec = decode_layer(d, blobs)
    lab = np.asarray(blobs["labels"], np.int64)
    per_expert = np.zeros_like(r["y_routed"])
    for t in range(x.shape[0]):
        for k in range(d.top_k):
            per_expert[t] += dec["U"][lab[r["idx"][t, k]]] @ r["o"][t * d.top_k + k]
    assert np.max(np.abs(per_expert - r["y_routed"])) <= 1e-12 * np.max(np.abs(per_expert))


def test_single_group_is_plain_topk_moe():
    """G = 1: a textbook top-K MoE whose experts are U . E_e . D."""
    d = LayerDims(**{**SMALL.__dict__, "n_groups": 1})
    blobs = pack_layer(d, _masters(d, labels=np.zeros(SMALL.n_experts)))
    x = _x(d, 3)
    got = layer_forward(d, blobs, x)
    dec = decode_layer(d, blobs)
    D, U = dec["D"][0], dec["U"][0]
    logits = x.astype(np.float64) @ dec["Wr"].T
    probs = scipy.special.softmax(logits, axis=1)
    for t in range(x.shape[0]):
        top = np.argsort(-logits[t], kind="stable")[:d.top_k]
        wts = probs[t, top] / probs[t, top].sum()       # softmax, top-k, renormalize
        y = np.zeros(d.hidden)
        for wk, e in zip(wts, top):
            g_, u_, dn = fm.unpack_expert_record(blobs["experts"][e], d.latent, d.expert_ffn)
            z = D @ x[t]
            hid = torch.nn.functional.silu(torch.from_numpy(g_ @ z)).numpy() * (u_ @ z)
            y += wk * (U @ (dn @ hid))
        sg, su, sd = dec["shared"]
        y += sd @ (torch.nn.functional.silu(torch.from_numpy(sg @ x[t])).numpy() * (su @ x[t]))
        assert np.max(np.abs(got[t] - y)) <= 1e-12 * np.max(np.abs(y))


def test_top1_weight_is_one_and_zero_experts_leave_shared():
    d = LayerDims(**{**SMALL.__dict__, "top_k": 1})
    blobs = pack_layer(d, _masters(d, expert_scale=0.0))
    x = _x(d, 3)
    r = layer_forward(d, blobs, x, intermediates=True)
    assert np.all(r["w"] == 1.0)
    assert np.all(r["y_routed"] == 0.0)
    assert np.array_equal(r["y"], r["y_shared"])


def test_identity_projections_reduce_to_full_width_moe():
    """ell = H with D = U = (127/128) I held exactly in Q8: the layer is a
    plain MoE whose experts work at full width, scaled by (127/128)."""
    d = LayerDims(hidden=64, latent=64, n_experts=5, top_k=2, n_groups=2, expert_ffn=32,
                  shared_ffn=32, du_bits=8)
    m = _masters(d, seed=11)
    eye = np.eye(64, dtype=np.float32) * np.float32(127 / 128)
    m["D"] = np.stack([eye, eye])
    m["U"] = np.stack([eye, eye])
    blobs = pack_layer(d, m)
    x = _x(d, 3, seed=12)
    r = layer_forward(d, blobs, x, intermediates=True)
    c = 127 / 128
    for t in range(3):
        y = np.zeros(64)
        for k in range(2):
            e = r["idx"][t, k]
            g_, u_, dn = fm.unpack_expert_record(blobs["experts"][e], 64, 32)
            z = c * x[t].astype(np.float64)
            y += r["w"][t, k] * c * (dn @ (oracle.layer.silu(g_ @ z) * (u_ @ z)))
        assert np.max(np.abs(r["y_routed"][t] - y)) <= 1e-12 * np.max(np.abs(y))


# ---------------------------------------------------------------------------
# Routing


def test_topk_order_ties_and_weights():
    lg = np.array([[0.5, 2.0, 2.0, -1.0, 2.0, 0.5],
                   [0.0, 0.0, 0.0, 0.0, 0.0, 0.0]])
    idx, w = oracle.select_topk(lg, 4)
    assert idx.tolist() == [[1, 2, 4, 0], [0, 1, 2, 3]]
    full = scipy.special.softmax(lg, axis=1)
    for t in range(2):
        sel = full[t, idx[t]]
        assert np.allclose(w[t], sel / sel.sum(), rtol=1e-15, atol=0)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=1e-15)


def test_topk_random_against_full_sort():
    rng = np.random.default_rng(20)
    lg = rng.standard_normal((50, 64)).round(1)           # many exact ties
    idx, _ = oracle.select_topk(lg, 10)
    for t in range(50):
        want = sorted(range(64), key=lambda e: (-lg[t, e], e))[:10]
        assert idx[t].tolist() == want


def test_router_logits_exact_products():
    """bf16 x fp32 products are exact in fp64; with small integer-valued
    inputs the whole dot product is exact and equals integer arithmetic."""
    rng = np.random.default_rng(21)
    xi = rng.integers(-8, 8, (3, 64))
    wi = rng.integers(-8, 8, (5, 64))
    bits = fm.f32_to_bf16_bits(wi.astype(np.float32))
    lg = oracle.router_logits(xi.astype(np.float32), bits, np.arange(5, dtype=np.float32))
    assert np.array_equal(lg, (xi @ wi.T + np.arange(5)).astype(np.float64))


# ---------------------------------------------------------------------------
# Permutation


def _perm_by_counting(idx, labels, n_experts, n_groups):
    """Counting sort written out: groups in order, experts in index order
    inside a group, assignments in ascending a inside an expert."""
    flat = np.asarray(idx).ravel().tolist()
    perm = []
    for g in range(n_groups):
        for e in range(n_experts):
            if labels[e] != g:
                continue
            perm += [a for a, ea in enumerate(flat) if ea == e]
    return perm


def test_permute_matches_counting_sort_and_invariants():
    rng = np.random.default_rng(22)
    e_n, g_n, t_n, k = 40, 5, 30, 6
    labels = rng.integers(0, g_n, e_n)
    idx = np.stack([rng.choice(e_n, k, replace=False) for _ in range(t_n)])
    perm, count, goff = oracle.permute(idx, labels, e_n, g_n)
    assert perm.tolist() == _perm_by_counting(idx, labels, e_n, g_n)
    assert sorted(perm.tolist()) == list(range(t_n * k))
    flat = idx.ravel()
    key = labels[flat[perm]] * e_n + flat[perm]
    assert np.all(np.diff(key) >= 0)
    same = np.diff(key) == 0
    assert np.all(np.diff(perm)[same] > 0)
    assert count.sum() == t_n * k and np.array_equal(count, np.bincount(flat, minlength=e_n))
    assert goff[0] == 0 and goff[-1] == t_n * k
    for g in range(g_n):
        seg = perm[goff[g]:goff[g + 1]]
        assert np.all(labels[flat[seg]] == g)


def test_expert_offsets_count_lower_experts():
    rng = np.random.default_rng(41)
    idx = rng.integers(0, 9, size=(6, 3)).astype(np.int32)
    _, count, _ = oracle.permute(idx, rng.integers(0, 2, 9).astype(np.uint8), 9, 2)
    off = oracle.expert_offsets(count)
    assert off.shape == (10,) and off.dtype == np.int32
    for e in range(10):      # brute force: assignments to experts below e
        assert off[e] == sum(1 for v in idx.ravel().tolist() if v < e)


def test_permute_empty():
    perm, count, goff = oracle.permute(np.zeros((0, 3), np.int32), np.zeros(4, np.uint8), 4, 2)
    assert perm.size == 0 and count.sum() == 0 and goff.tolist() == [0, 0, 0]


# ---------------------------------------------------------------------------
# Stack


def test_rmsnorm_closed_form():
    v = np.full((2, 8), 3.0)
    assert np.allclose(oracle.rmsnorm(v), 3.0 / np.sqrt(9.0 + 1e-6), rtol=1e-15)
    r = np.random.default_rng(23).standard_normal((4, 256))
    n = oracle.rmsnorm(r, eps=0.0)
    assert np.allclose(np.mean(n * n, axis=1), 1.0, rtol=1e-14)


def test_stack_is_residual_of_layers():
    d = SMALL
    layers = [pack_layer(d, _masters(d, seed=30 + i)) for i in range(3)]
    x = _x(d, 2, seed=31)
    out = oracle.stack_forward(d, layers, x)
    xd = x.astype(np.float64)
    for blobs in layers:
        xn = xd / np.sqrt((xd ** 2).mean(axis=1, keepdims=True) + 1e-6)
        xd = xd + layer_forward(d, blobs, xn)
    assert np.array_equal(out, xd)


def _identity_layer(dims, blobs, x, dec=None, intermediates=False):
    return np.asarray(x, dtype=np.float64)


def stack_closed_form_holds():
    """Pins stack_forward by hand-computed closed forms, with every layer
    replaced by the identity map (pre-norm residual: x + x / rms(x)):
    a constant row of 3s over two layers, and a ragged row over one."""
    x0 = np.full((1, 8), 3.0, dtype=np.float32)
    x1 = 3.0 + 3.0 / math.sqrt(9.0 + 1e-6)
    x2 = x1 + x1 / math.sqrt(x1 * x1 + 1e-6)
    got = ol.stack_forward(SMALL, [None, None], x0)
    ok = got.shape == (1, 8) and np.allclose(got, x2, rtol=1e-15, atol=0)
    v = np.array([[1.0, -2.0, 4.0, 0.5]], dtype=np.float32)
    ms = (1.0 + 4.0 + 16.0 + 0.25) / 4.0
    want = v.astype(np.float64) * (1.0 + 1.0 / math.sqrt(ms + 1e-6))
    got1 = ol.stack_forward(SMALL, [None], v)
    return ok and np.allclose(got1, want, rtol=1e-15, atol=0)


def test_stack_closed_form(monkeypatch):
    monkeypatch.setattr(ol, "layer_forward", _identity_layer)
    assert stack_closed_form_holds()
    # zero layers leave x as it is
    x = _x(SMALL, 2, seed=5)
    assert np.array_equal(oracle.stack_forward(SMALL, [], x), x.astype(np.float64))


def test_normalized_input_scales_logits():
    """A layer fed c * x routes like x: its logits are c times x's (no bias)."""
    blobs = pack_layer(SMALL, _masters(SMALL))
    x = _x(SMALL, 3)
    a = layer_forward(SMALL, blobs, x, intermediates=True)
    b = layer_forward(SMALL, blobs, x.astype(np.float64) * 0.25, intermediates=True)
    assert np.array_equal(a["idx"], b["idx"])
    assert np.array_equal(b["logits"], 0.25 * a["logits"])     # power of two: exact


def test_empty_token_batch():
    blobs = pack_layer(SMALL, _masters(SMALL))
    r = layer_forward(SMALL, blobs, np.zeros((0, SMALL.hidden), np.float32), intermediates=True)
    assert r["y"].shape == (0, SMALL.hidden) and r["perm"].size == 0
