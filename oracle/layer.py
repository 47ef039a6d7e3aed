"""The latent-MoE layer, its routing and the 48-layer stack, in plain fp64.

Test infrastructure only (see the package docstring).

The layer (TEARDOWN "A latent in front of the experts", layer equation; LAYER
"Edge0-145B architecture" text):

    y = U_g( sum_{e in top-K} w_e E_e(D_g x) ) + shared(x)

with D_g in R^{ell x H}, E_e : R^ell -> R^F -> R^ell a SwiGLU, and g the group
label of each expert (LAYER "Model profile", row "Latent compression": each
layer has G groups of D/U, chosen by each expert's group label). Readings:

* g is g(e) per expert; U is applied once per group a token routed into,
  to the w-weighted sum of that group's expert outputs (TEARDOWN states U
  runs once per group the window's tokens routed into). By linearity this
  equals applying U_{g(e)} per expert.
* w_e: softmax over all E router logits, keep the top K, renormalize. The
  E-way denominator cancels, so w is the softmax of the K kept logits.
  Ordering of the kept experts: descending logit, ties to the lower index.
* The router reads the full-width x, not the latent (TEARDOWN, "A latent in
  front of the experts"); logits are exact dot products of the fp32
  x with the bf16 weights, plus an optional per-expert bias.
* SwiGLU: h = silu(W_gate z) * (W_up z), out = W_down h, silu(v) = v/(1+e^-v).
* The shared expert is a full-width SwiGLU on x (LAYER: only the 512 experts
  work at ell; everything outside the expert pool stays at full width), not
  gated, added after U.
* Group permutation: the stable sort of assignments a = t*K + k by the key
  (g(e), e) -- group-major, expert-minor, ascending a within an expert.
* Stack: pre-norm residual x_{l+1} = x_l + layer_l(RMSNorm(x_l)), RMSNorm
  with unit gain and eps 1e-6, no final norm.
"""

from dataclasses import dataclass

import numpy as np

from . import formats as fm
from . import kquants as kq


@dataclass(frozen=True)
class LayerDims:
    hidden: int       # H
    latent: int       # ell
    n_experts: int    # E
    top_k: int        # K
    n_groups: int     # G
    expert_ffn: int   # F
    shared_ffn: int   # F_s
    du_bits: int      # 8 (Q8) or 4 (Q4)
    expert_format: int = 0   # 0 NVFP4; 1 Q3_K gate/up + IQ4_NL down (oracle/kquants.py)

    @property
    def record_bytes(self):
        if self.expert_format == 1:
            return kq.q3k_record_bytes(self.latent, self.expert_ffn)
        return fm.expert_record_bytes(self.latent, self.expert_ffn)

    def pack_record(self, gate, up, down):
        if self.expert_format == 1:
            return kq.pack_q3k_record(gate, up, down)
        return fm.pack_expert_record(gate, up, down)

    def unpack_record(self, rec):
        if self.expert_format == 1:
            return kq.unpack_q3k_record(rec, self.latent, self.expert_ffn)
        return fm.unpack_expert_record(rec, self.latent, self.expert_ffn)


# ---------------------------------------------------------------------------
# Packing master fp32 weights into the blobs both sides consume.


def pack_layer(dims, m):
    """m: dict of fp32 masters: router [E,H], router_bias [E] or None,
    labels uint8 [E], D [G,ell,H], U [G,H,ell], experts: callable e ->
    (gate [F,ell], up [F,ell], down [ell,F]) or list, shared (gate [Fs,H],
    up [Fs,H], down [H,Fs]). ``expert_ids`` (optional) limits which expert
    records are quantized; the others are left as zero bytes."""
    d = dims
    out = {}
    out["router_bf16"] = fm.f32_to_bf16_bits(m["router"])
    out["router_bias"] = None if m.get("router_bias") is None else \
        np.asarray(m["router_bias"], dtype=np.float32)
    out["labels"] = np.asarray(m["labels"], dtype=np.uint8)
    out["d_blob"] = np.concatenate([fm.pack_du(m["D"][g], d.du_bits) for g in range(d.n_groups)])
    out["u_blob"] = np.concatenate([fm.pack_du(m["U"][g], d.du_bits) for g in range(d.n_groups)])
    rb = d.record_bytes
    experts = np.zeros((d.n_experts, rb), dtype=np.uint8)
    ids = m.get("expert_ids")
    ids = range(d.n_experts) if ids is None else ids
    for e in ids:
        g_, u_, w_ = m["experts"](e)
        experts[e] = d.pack_record(g_, u_, w_)
    out["experts"] = experts
    out["shared"] = tuple(fm.f32_to_bf16_bits(a) for a in m["shared"])
    return out


def decode_layer(dims, blobs, expert_ids=None):
    """Dequantize every tensor the forward needs to fp64 (experts: only
    ``expert_ids``, decoded lazily by ``layer_forward`` otherwise)."""
    d = dims
    dec = {}
    dec["Wr"] = fm.bf16_bits_to_f64(blobs["router_bf16"])
    dec["bias"] = None if blobs.get("router_bias") is None else \
        np.asarray(blobs["router_bias"], dtype=np.float64)
    gb = fm.du_group_bytes(d.latent, d.hidden, d.du_bits)
    dec["D"] = [fm.unpack_du(blobs["d_blob"][g * gb:(g + 1) * gb], d.latent, d.hidden, d.du_bits)
                for g in range(d.n_groups)]
    gb = fm.du_group_bytes(d.hidden, d.latent, d.du_bits)
    dec["U"] = [fm.unpack_du(blobs["u_blob"][g * gb:(g + 1) * gb], d.hidden, d.latent, d.du_bits)
                for g in range(d.n_groups)]
    dec["shared"] = tuple(fm.bf16_bits_to_f64(a) for a in blobs["shared"])
    return dec


# ---------------------------------------------------------------------------
# Routing.


def _exact_input(x):
    """The layer input at its own precision: fp32 arrays are widened exactly;
    fp64 arrays (a normalized input inside the stack) are used as they are."""
    x = np.asarray(x)
    return x.astype(np.float64) if x.dtype == np.float64 else \
        x.astype(np.float32).astype(np.float64)


def router_logits(x, wr_bf16_bits, bias=None):
    """l[t, e] = sum_i x[t, i] * Wr[e, i] (+ b[e]), fp64."""
    wr = fm.bf16_bits_to_f64(wr_bf16_bits)
    lg = _exact_input(x) @ wr.T
    if bias is not None:
        lg = lg + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    return lg


def select_topk(logits, k):
    """Top-k per row ordered by (-logit, expert index); renormalized softmax
    weights over the kept logits. Returns (idx int32 [T,k], w fp64 [T,k])."""
    t_n, e_n = logits.shape
    idx = np.empty((t_n, k), dtype=np.int32)
    for t in range(t_n):
        order = np.lexsort((np.arange(e_n), -logits[t]))
        idx[t] = order[:k]
    sel = np.take_along_axis(logits, idx.astype(np.int64), axis=1)
    m = sel.max(axis=1, keepdims=True)
    ex = np.exp(sel - m)
    w = ex / ex.sum(axis=1, keepdims=True)
    return idx, w


def permute(idx, labels, n_experts, n_groups):
    """Stable sort of the assignments a = t*K + k by (g(e), e).

    Returns perm int32 [T*K] (perm[j] = the a at sorted position j),
    expert_count int32 [E], group_off int32 [G+1] (start of each group's
    segment in perm)."""
    lab = np.asarray(labels, dtype=np.int64)
    flat = np.asarray(idx, dtype=np.int64).ravel()
    key = lab[flat] * n_experts + flat
    perm = np.argsort(key, kind="stable").astype(np.int32)
    count = np.bincount(flat, minlength=n_experts).astype(np.int32)
    gcount = np.bincount(lab[flat], minlength=n_groups)
    group_off = np.concatenate([[0], np.cumsum(gcount)]).astype(np.int32)
    return perm, count, group_off


def expert_offsets(count):
    """Exclusive scan of the per-expert counts in expert-id order: off[e] is
    the number of assignments to experts below e, off[E] = T*K."""
    return np.concatenate([[0], np.cumsum(np.asarray(count, dtype=np.int64))]).astype(np.int32)


# ---------------------------------------------------------------------------
# Forward.


def silu(v):
    return v / (1.0 + np.exp(-v))


def swiglu(gate, up, down, z):
    """down @ (silu(gate @ z) * (up @ z)) for a vector z."""
    return down @ (silu(gate @ z) * (up @ z))


def layer_forward(dims, blobs, x, dec=None, intermediates=False):
    """Forward of one layer for x [T, H] (fp32, or fp64 for a normalized
    input inside the stack). Returns y fp64 [T, H], or a dict with every
    intermediate when ``intermediates`` is set."""
    d = dims
    xd = _exact_input(x)
    t_n = xd.shape[0]
    if dec is None:
        dec = decode_layer(d, blobs)
    labels = np.asarray(blobs["labels"], dtype=np.int64)

    logits = router_logits(xd, blobs["router_bf16"], blobs.get("router_bias"))
    idx, w = select_topk(logits, d.top_k)
    perm, count, group_off = permute(idx, labels, d.n_experts, d.n_groups)

    # D for the (t, g) pairs used (the reference engine computes all groups;
    # unused pairs never reach y).
    xl = np.full((t_n, d.n_groups, d.latent), np.nan)
    for t in range(t_n):
        for g in sorted(set(labels[idx[t]].tolist())):
            xl[t, g] = dec["D"][g] @ xd[t]

    # Experts, one assignment a = t*K + k at a time.
    cache = {}
    h = np.zeros((t_n * d.top_k, d.expert_ffn))
    o = np.zeros((t_n * d.top_k, d.latent))
    for t in range(t_n):
        for k in range(d.top_k):
            e = int(idx[t, k])
            if e not in cache:
                cache[e] = d.unpack_record(blobs["experts"][e])
            wg, wu, wd = cache[e]
            z = xl[t, labels[e]]
            a = t * d.top_k + k
            h[a] = silu(wg @ z) * (wu @ z)
            o[a] = w[t, k] * (wd @ h[a])

    # Per-group sums in ascending k, then U once per used group.
    s = np.zeros((t_n, d.n_groups, d.latent))
    used = np.zeros((t_n, d.n_groups), dtype=bool)
    for t in range(t_n):
        for k in range(d.top_k):
            g = labels[idx[t, k]]
            s[t, g] += o[t * d.top_k + k]
            used[t, g] = True
    y_routed = np.zeros((t_n, d.hidden))
    for t in range(t_n):
        for g in range(d.n_groups):
            if used[t, g]:
                y_routed[t] += dec["U"][g] @ s[t, g]

    sg, su, sd = dec["shared"]
    y_shared = np.stack([swiglu(sg, su, sd, xd[t]) for t in range(t_n)]) if t_n else \
        np.zeros((0, d.hidden))
    y = y_routed + y_shared
    if not intermediates:
        return y
    return dict(y=y, logits=logits, idx=idx, w=w, perm=perm, expert_count=count,
                expert_off=expert_offsets(count), group_off=group_off, xl=xl, h=h, o=o, s=s, used=used,
                y_routed=y_routed, y_shared=y_shared)


def rmsnorm(x, eps=1e-6):
    """v / sqrt(mean(v^2) + eps) per row, unit gain, fp64."""
    xd = np.asarray(x, dtype=np.float64)
    return xd / np.sqrt(np.mean(xd * xd, axis=-1, keepdims=True) + eps)


def stack_forward(dims, layers, x, eps=1e-6):
    """x_{l+1} = x_l + layer_l(RMSNorm(x_l)); ``layers`` yields blob dicts.
    Reading: the normalized input reaches the layer at full precision (not
    rounded), so the router sees 1/rms(x) times the logits of x."""
    xd = np.asarray(x, dtype=np.float64)
    for blobs in layers:
        xd = xd + layer_forward(dims, blobs, rmsnorm(xd, eps))
    return xd
