"""Builds layer cases for the GPU tests: masters from the seeded generator,
packed by the oracle's quantizers, expected outputs from the oracle. The
packed bytes are the only thing both sides share."""

import numpy as np

import oracle
from latent_mixture_experts_amd import workloads as wl

# Parity bar on the layer output.
REL_L2 = 1e-3
MAX_ABS_OF_RMS = 1e-2


def dims_of(w):
    return oracle.LayerDims(w.hidden, w.latent, w.n_experts, w.top_k, w.n_groups, w.expert_ffn,
                            w.shared_ffn, w.du_bits, getattr(w, "expert_format", 0))


class Case:
    """Packed blobs of one layer plus x for up to `tokens` tokens. Only the
    experts some token routes to are quantized; other records stay zero (they
    are never read by a correct forward)."""

    def __init__(self, w, seed=0, tokens=None, layer=0, x=None, masters=None, pack_tokens=None):
        self.w = w
        self.d = dims_of(w)
        t = w.tokens if tokens is None else tokens
        self.x = wl.x(w, seed, layer, tokens=t) if x is None else np.asarray(x, np.float32)
        m = wl.masters(w, seed, layer) if masters is None else masters
        bits = oracle.f32_to_bf16_bits(m["router"])
        lg = oracle.router_logits(self.x, bits, m["router_bias"])
        idx, _ = oracle.select_topk(lg, w.top_k)
        # pack_tokens: quantize only the experts these tokens route to (the
        # other tokens' outputs are then not meaningful; their routing is)
        sel = idx if pack_tokens is None else idx[np.asarray(pack_tokens)]
        m["expert_ids"] = sorted(set(sel.ravel().tolist()))
        self.logits, self.idx = lg, idx
        self.blobs = oracle.pack_layer(self.d, m)
        self.dec = oracle.decode_layer(self.d, self.blobs)

    def expect(self, T=None):
        x = self.x if T is None else self.x[:T]
        return oracle.layer_forward(self.d, self.blobs, x, dec=self.dec, intermediates=True)


def rel_errors(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    rms = np.sqrt(np.mean(want ** 2))
    rel = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300)
    mx = np.max(np.abs(got - want)) / max(rms, 1e-300) if want.size else 0.0
    return rel, mx


def assert_close(got, want, what):
    rel, mx = rel_errors(got, want)
    assert rel <= REL_L2 and mx <= MAX_ABS_OF_RMS, \
        "%s: relative L2 %.3g (bar %.0e), max-abs/rms %.3g (bar %.0e)" % (what, rel, REL_L2, mx,
                                                                          MAX_ABS_OF_RMS)
    return rel, mx
