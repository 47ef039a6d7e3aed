"""Seeded synthetic inputs for the latent-MoE layer.

This module only draws random numbers: fp32 master weights, activations,
router biases and group labels. It holds none of the layer's arithmetic and
no quantizer; packing the masters into NVFP4 / Q8 / Q4 / bf16 blobs is done
by whoever consumes them. Both the CPU oracle (through the tests) and the
HIP path (through the tests and the benchmark) take their inputs from here.

Workloads (shapes of the Edge0 145B / 120B layer, "Edge0 145B and Edge0 120B"
model page, "Model profile" and architecture tables):

* ``tiny``: H 256, ell 128, 16 experts, top-2, 2 groups with label e mod 2,
  F 64, shared 64, Q8 D/U, router weights N(0, 1/16), T 4.
* ``145b_decode``: H 2560, ell 1792, 512 experts, top-10, 8 groups with
  uniform random labels, F 640 NVFP4, shared 640 bf16, Q8 D/U, T 4.
* ``120b_decode``: as above with ell 1280, Q4 D/U, T 5.
* ``145b_prefill``: as 145b_decode with T 4096 and a per-expert router bias
  N(0, 1) that skews expert loads.
* ``145b_stack``: 48 independently seeded 145b_decode layers, T 4.
* ``145b_q3k_decode``: 145b_decode with the Q3_K build's expert records (Q3_K
  gate/up, IQ4_NL down: 1,630,720 bytes an expert).
* ``mtp_draft``: the MoE of the multi-token-prediction draft layer ("MTP
  head" row of the architecture tables: 1.26B parameters in 512 experts,
  i.e. 2,457,600 = 3 x 1280 x 640 per expert): ell 1280, F 640 NVFP4, top-10,
  8 groups, Q8 D/U, shared 640 bf16, H 2560, T 1 (one drafted token).

Every non-router weight is N(0, 0.02); router weights N(0, 1/sqrt(H));
activations N(0, 1). Each tensor (and each expert, each group's D and U) has
its own counter-free stream keyed by (seed, layer, tensor, index), so any
subset of experts can be drawn alone.
"""

from dataclasses import dataclass, replace

import numpy as np

WEIGHT_STD = 0.02


@dataclass(frozen=True)
class Workload:
    name: str
    hidden: int
    latent: int
    n_experts: int
    top_k: int
    n_groups: int
    expert_ffn: int
    shared_ffn: int
    du_bits: int
    tokens: int
    router_bias: bool = False
    labels_mod: bool = False     # label = e mod G instead of uniform random
    n_layers: int = 1
    expert_format: int = 0       # 0 NVFP4 records, 1 Q3_K gate/up + IQ4_NL down

    @property
    def router_std(self):
        return 1.0 / np.sqrt(self.hidden)

    def with_tokens(self, t):
        return replace(self, tokens=t)


WORKLOADS = {
    "tiny": Workload("tiny", 256, 128, 16, 2, 2, 64, 64, 8, 4, labels_mod=True),
    "145b_decode": Workload("145b_decode", 2560, 1792, 512, 10, 8, 640, 640, 8, 4),
    "120b_decode": Workload("120b_decode", 2560, 1280, 512, 10, 8, 640, 640, 4, 5),
    "145b_prefill": Workload("145b_prefill", 2560, 1792, 512, 10, 8, 640, 640, 8, 4096,
                             router_bias=True),
    "145b_stack": Workload("145b_stack", 2560, 1792, 512, 10, 8, 640, 640, 8, 4, n_layers=48),
    "mtp_draft": Workload("mtp_draft", 2560, 1280, 512, 10, 8, 640, 640, 8, 1),
    "145b_q3k_decode": Workload("145b_q3k_decode", 2560, 1792, 512, 10, 8, 640, 640, 8, 4,
                                expert_format=1),
}

# stream identifiers
_X, _ROUTER, _BIAS, _LABELS, _D, _U, _EXPERT, _SHARED = range(8)


def _rng(seed, layer, tensor, index=0):
    ss = np.random.SeedSequence(int(seed), spawn_key=(int(layer), int(tensor), int(index)))
    return np.random.Generator(np.random.PCG64(ss))


def _normal(rng, shape, std):
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def x(w, seed=0, layer=0, tokens=None):
    t = w.tokens if tokens is None else tokens
    return _normal(_rng(seed, layer, _X), (t, w.hidden), 1.0)


def router(w, seed=0, layer=0):
    return _normal(_rng(seed, layer, _ROUTER), (w.n_experts, w.hidden), w.router_std)


def router_bias(w, seed=0, layer=0):
    if not w.router_bias:
        return None
    return _normal(_rng(seed, layer, _BIAS), (w.n_experts,), 1.0)


def labels(w, seed=0, layer=0):
    if w.labels_mod:
        return (np.arange(w.n_experts) % w.n_groups).astype(np.uint8)
    return _rng(seed, layer, _LABELS).integers(0, w.n_groups, w.n_experts).astype(np.uint8)


def d_master(w, g, seed=0, layer=0):
    """D_g, fp32 [ell, H]."""
    return _normal(_rng(seed, layer, _D, g), (w.latent, w.hidden), WEIGHT_STD)


def u_master(w, g, seed=0, layer=0):
    """U_g, fp32 [H, ell]."""
    return _normal(_rng(seed, layer, _U, g), (w.hidden, w.latent), WEIGHT_STD)


def expert_master(w, e, seed=0, layer=0):
    """(gate [F, ell], up [F, ell], down [ell, F]) fp32 for expert e."""
    r = _rng(seed, layer, _EXPERT, e)
    f, ell = w.expert_ffn, w.latent
    return (_normal(r, (f, ell), WEIGHT_STD), _normal(r, (f, ell), WEIGHT_STD),
            _normal(r, (ell, f), WEIGHT_STD))


def shared_master(w, seed=0, layer=0):
    """(gate [Fs, H], up [Fs, H], down [H, Fs]) fp32."""
    r = _rng(seed, layer, _SHARED)
    fs, h = w.shared_ffn, w.hidden
    return (_normal(r, (fs, h), WEIGHT_STD), _normal(r, (fs, h), WEIGHT_STD),
            _normal(r, (h, fs), WEIGHT_STD))


def masters(w, seed=0, layer=0, expert_ids=None):
    """All masters of one layer as a dict; experts are drawn lazily."""
    return {
        "router": router(w, seed, layer),
        "router_bias": router_bias(w, seed, layer),
        "labels": labels(w, seed, layer),
        "D": np.stack([d_master(w, g, seed, layer) for g in range(w.n_groups)]),
        "U": np.stack([u_master(w, g, seed, layer) for g in range(w.n_groups)]),
        "experts": lambda e: expert_master(w, e, seed, layer),
        "expert_ids": expert_ids,
        "shared": shared_master(w, seed, layer),
    }


def torch_expert_masters(w, seed, layer, first, count, device):
    """Bulk GPU draw of ``count`` experts' masters starting at ``first`` as
    three fp32 tensors [count, F, ell], [count, F, ell], [count, ell, F].
    Used where drawing every expert on the host would be too slow; the values
    differ from ``expert_master`` (another generator)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1000003 + int(layer) * 7919 + int(first)) & 0x7FFFFFFFFFFFFFFF)
    f, ell = w.expert_ffn, w.latent
    mk = lambda *s: torch.randn(*s, generator=g, device=device, dtype=torch.float32) * WEIGHT_STD
    return mk(count, f, ell), mk(count, f, ell), mk(count, ell, f)
