"""Parity of lmoe_forward_block (x += layer(RMSNorm(x))) with the oracle,
layer by layer with teacher forcing: layer l of the oracle reads the GPU's
own fp32 x_l, so rounding upstream cannot legitimately flip a near-tie
downstream. Each layer's update x_{l+1} - x_l is held to the parity bar
and its routed part to 1e-4; the end-to-end drift against the oracle's own
stack is printed, not gated."""

import numpy as np
import pytest

import oracle
from cases import assert_close, dims_of, rel_errors
from latent_mixture_experts_amd import workloads as wl

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _layer_blobs(w, d, seed, layer, xn):
    m = wl.masters(w, seed, layer)
    lg = oracle.router_logits(xn, oracle.f32_to_bf16_bits(m["router"]), m["router_bias"])
    idx, _ = oracle.select_topk(lg, w.top_k)
    m["expert_ids"] = sorted(set(idx.ravel().tolist()))
    return oracle.pack_layer(d, m)


def run_stack(w, n_layers, T, seed=0, eps=1e-6):
    from latent_mixture_experts_amd import lmoe
    d = dims_of(w)
    x0 = wl.x(w, seed, 0, tokens=T)
    xg = torch.from_numpy(x0).cuda()
    oracle_blobs = []
    for layer_idx in range(n_layers):
        print("stack layer", layer_idx, "T", T, flush=True)
        xin = xg.cpu().numpy().astype(np.float64)
        xn = oracle.rmsnorm(xin, eps)
        blobs = _layer_blobs(w, d, seed, layer_idx, xn)
        oracle_blobs.append(blobs)
        r = oracle.layer_forward(d, blobs, xn, intermediates=True)
        layer = lmoe.Layer(w.hidden, w.latent, w.n_experts, w.top_k, w.n_groups, w.expert_ffn,
                           w.shared_ffn, w.du_bits, T, has_router_bias=w.router_bias)
        layer.load(blobs)
        layer.forward_block(xg, eps)
        torch.cuda.synchronize()
        layer.close()
        xout = xg.cpu().numpy().astype(np.float64)
        delta = xout - xin
        rel, mx = assert_close(delta, r["y"], "layer %d update" % layer_idx)
        # the routed part, through the fp32 residual add: allow 1e-4 of its
        # norm plus the rounding of x + y to fp32, half an ulp per element for
        # each of the two additions onto x the prefill path makes (the shared
        # expert, then U; the decode path adds once)
        err = np.linalg.norm(delta - r["y_shared"] - r["y_routed"])
        ulp_noise = 2 * np.linalg.norm(np.abs(xout) * 2.0 ** -24)
        bound = 1e-4 * np.linalg.norm(r["y_routed"]) + ulp_noise
        print("  update rel L2 %.3g max/rms %.3g; routed-part error %.3g (bound %.3g)" % (
            rel, mx, err, bound), flush=True)
        assert err <= bound
    want = oracle.stack_forward(d, oracle_blobs, x0, eps)
    drift, _ = rel_errors(xg.cpu().numpy(), want)
    print("end-to-end relative drift after %d layers: %.3g" % (n_layers, drift), flush=True)
    return drift


def test_tiny_stack_8_layers():
    w = wl.WORKLOADS["tiny"]
    for T in (4, 3):
        run_stack(w, 8, T)


@pytest.mark.parametrize("T", [1, 2, 5, 8])
def test_tiny_stack_block_t(T):
    """Three block forwards at the other decode token counts (the 1/rms is
    formed inside the decode kernels for every T)."""
    run_stack(wl.WORKLOADS["tiny"], 3, T, seed=T)


def test_145b_stack_2_layers():
    w = wl.WORKLOADS["145b_stack"]
    run_stack(w, 2, w.tokens)


@pytest.mark.parametrize("T", [4, 24])
def test_tiny_stack_router_bias(T):
    """Block forwards of a layer with a router bias: the logits of the
    normalized row (exact 1/rms) plus the bias decide the top K on both the
    decode (T = 4) and prefill (T = 24) paths."""
    w = wl.Workload("tiny_bias", 256, 128, 16, 2, 2, 64, 64, 8, T, router_bias=True,
                    labels_mod=True)
    run_stack(w, 3, T)


def _device_layer(w, seed, layer_idx):
    """A layer drawn and packed on the device (the library's packers, torch's
    generator): it only carries the stack between the checked layers."""
    from latent_mixture_experts_amd import lmoe
    dev = "cuda"
    E, H, L, G, F, Fs = w.n_experts, w.hidden, w.latent, w.n_groups, w.expert_ffn, w.shared_ffn
    layer = lmoe.Layer(H, L, E, w.top_k, G, F, Fs, w.du_bits, w.tokens)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed * 7919 + layer_idx * 104729 + 3)
    rnd = lambda *sh: torch.randn(*sh, generator=gen, device=dev) * wl.WEIGHT_STD
    router = torch.empty(E, H, dtype=torch.int16, device=dev)
    lmoe.pack_bf16(torch.from_numpy(wl.router(w, seed, layer_idx)).to(dev), router)
    dg, ug = lmoe.du_matrix_bytes(L, H, w.du_bits), lmoe.du_matrix_bytes(H, L, w.du_bits)
    d_blob = torch.empty(G * dg, dtype=torch.uint8, device=dev)
    u_blob = torch.empty(G * ug, dtype=torch.uint8, device=dev)
    for g in range(G):
        lmoe.pack_blocks(rnd(L, H), w.du_bits, d_blob[g * dg:(g + 1) * dg])
        lmoe.pack_blocks(rnd(H, L), w.du_bits, u_blob[g * ug:(g + 1) * ug])
    shared = []
    for shp in ((Fs, H), (Fs, H), (H, Fs)):
        t = torch.empty(*shp, dtype=torch.int16, device=dev)
        lmoe.pack_bf16(rnd(*shp), t)
        shared.append(t)
    experts = torch.empty(E, lmoe.expert_record_bytes(L, F), dtype=torch.uint8, device=dev)
    for e0 in range(0, E, 64):
        g_, u_, d_ = wl.torch_expert_masters(w, seed, layer_idx, e0, min(64, E - e0), dev)
        lmoe.pack_expert_records(g_, u_, d_, experts[e0:e0 + g_.shape[0]])
    layer.load(dict(router_bf16=router, router_bias=None,
                    labels=torch.from_numpy(wl.labels(w, seed, layer_idx)).to(dev),
                    d_blob=d_blob, u_blob=u_blob, experts=experts, shared=tuple(shared)))
    torch.cuda.synchronize()
    return layer


def test_145b_stack_48_layers_sampled():
    """The 48-layer stack of 145B-shaped layers at T = 4, run block by block
    on the device. A seeded sample of layers is built from the oracle's
    packing and checked by teacher forcing (the oracle reads the device's
    x_l); the layers between them are drawn on the device and only carry
    the stack forward."""
    from latent_mixture_experts_amd import lmoe
    w = wl.WORKLOADS["145b_stack"]
    d = dims_of(w)
    T, eps = w.tokens, 1e-6
    checked = sorted(np.random.default_rng(48).choice(w.n_layers, 4, replace=False).tolist())
    print("checked layers", checked, flush=True)
    xg = torch.from_numpy(wl.x(w, 0, 0, tokens=T)).cuda()
    for layer_idx in range(w.n_layers):
        if layer_idx not in checked:
            layer = _device_layer(w, 0, layer_idx)
            layer.forward_block(xg, eps)
            torch.cuda.synchronize()
            layer.close()
            continue
        print("stack layer", layer_idx, "checked", flush=True)
        xin = xg.cpu().numpy().astype(np.float64)
        xn = oracle.rmsnorm(xin, eps)
        blobs = _layer_blobs(w, d, 0, layer_idx, xn)
        r = oracle.layer_forward(d, blobs, xn, intermediates=True)
        layer = lmoe.Layer(w.hidden, w.latent, w.n_experts, w.top_k, w.n_groups, w.expert_ffn,
                           w.shared_ffn, w.du_bits, T)
        layer.load(blobs)
        layer.forward_block(xg, eps)
        torch.cuda.synchronize()
        layer.close()
        xout = xg.cpu().numpy().astype(np.float64)
        delta = xout - xin
        rel, mx = assert_close(delta, r["y"], "layer %d update" % layer_idx)
        err = np.linalg.norm(delta - r["y_shared"] - r["y_routed"])
        bound = 1e-4 * np.linalg.norm(r["y_routed"]) + np.linalg.norm(np.abs(xout) * 2.0 ** -24)
        print("  update rel L2 %.3g max/rms %.3g; routed-part error %.3g (bound %.3g)" % (
            rel, mx, err, bound), flush=True)
        assert err <= bound
    assert np.isfinite(xg.cpu().numpy()).all()


def test_block_rejects_bad_eps():
    from latent_mixture_experts_amd import lmoe
    w = wl.WORKLOADS["tiny"]
    layer = lmoe.Layer(w.hidden, w.latent, w.n_experts, w.top_k, w.n_groups, w.expert_ffn,
                       w.shared_ffn, w.du_bits, 4)
    d = dims_of(w)
    layer.load(_layer_blobs(w, d, 0, 0, np.ones((1, w.hidden))))
    x = torch.zeros(4, w.hidden, device="cuda")
    with pytest.raises(lmoe.LmoeError):
        layer.forward_block(x, eps=-1.0)
