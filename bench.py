#!/usr/bin/env python3
"""Throughput of the latent-MoE layer on one MI355X.

A step is one lmoe_forward over one batch of T tokens (router, top-K,
permutation, D, routed experts, combine + U, shared expert). The default
workload is the Edge0-145B-shaped decode / speculative-verify layer: H 2560,
latent 1792, 512 NVFP4 experts, top-10, 8 Q8 D/U groups, shared expert 640,
T = 4. Weights are synthetic (seeded N(0, 0.02) masters quantized on the GPU
by the library's packers; router N(0, 1/sqrt(H)) and x ~ N(0, 1) from the
same seeded generator as the tests). Steps rotate over --copies independently
seeded layers so that the 256 MB Infinity Cache cannot hold the weights a
step reads; inputs are resident in HBM before the timed region.

The default line also carries a "prefill" object: the Edge0-145B-shaped
prefill layer (T = 4096, router bias N(0, 1) skewing expert loads) on the
prefill path, with its per-kernel MFMA roofline. --workload 145b_prefill makes
that the primary line.

Prints one JSON line (rank 0). --gpus above 1 is refused: the library runs
on one GPU.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense fp16 / bf16 matrix peak, published
PREFILL_PHASES = ["route", "permute", "d", "shared_gate_up", "expert_gate_up", "expert_down",
                  "combine", "u_shared_down"]
PREFILL_KERNELS = ["k_prep + k_dense_dma<BF16,Logits> + k_select", "k_perm_*",
                   "k_dense16<F16> (D; 128 x 128 wave tiles, LDS DMA)",
                   "k_dense_dma<BF16,SwigluB2> (shared gate/up)",
                   "k_grouped_dma<GateUp> (LDS DMA) + k_grouped_short<GateUp> (64- and 32-token pieces)",
                   "k_down_res (activations resident in LDS; 64- and 32-token blocks)", "k_combine",
                   "k_dense_dma<F16,Y> (U + shared down, split along k; LDS DMA) + k_ytiles (split sums)"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_145b_t4_traffic.json")
PREFILL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_145b_t4096_traffic.json")
# kernel of each prefill phase as rocprofv3 names it (D and U on fp16 weights)
PREFILL_KERNEL_IDS = [["k_prep", "k_dense_dma<3, 0>", "k_select<5, 8>"],
                      ["k_perm_mask", "k_perm_scan", "k_perm_scatter"], "k_dense16<1>",
                      "k_dense_dma<3, 2>",
                      ["k_grouped_dma<0>", "k_grouped_short<0, 2, 8>", "k_grouped_short<0, 1, 8>"],
                      ["k_down_res<8, 2>", "k_down_res<8, 1>"], "k_combine",
                      ["k_dense_dma<5, 3>", "k_ytiles<4>"]]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_layer(lm, wl, w, seed, layer_idx, torch):
    """One layer's weights, drawn and packed on the device."""
    dev = "cuda"
    E, H, L, G, F, Fs = w.n_experts, w.hidden, w.latent, w.n_groups, w.expert_ffn, w.shared_ffn
    layer = lm.Layer(H, L, E, w.top_k, G, F, Fs, w.du_bits, max(w.tokens, 1),
                     has_router_bias=w.router_bias)
    router = torch.from_numpy(wl.router(w, seed, layer_idx)).to(dev)
    router_bf16 = torch.empty(E, H, dtype=torch.int16, device=dev)
    lm.pack_bf16(router, router_bf16)
    bias = wl.router_bias(w, seed, layer_idx)
    labels = wl.labels(w, seed, layer_idx)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed * 1000003 + layer_idx * 7919 + 17)
    rnd = lambda *s: torch.randn(*s, generator=gen, device=dev) * wl.WEIGHT_STD
    dg = lm.du_matrix_bytes(L, H, w.du_bits)
    ug = lm.du_matrix_bytes(H, L, w.du_bits)
    d_blob = torch.empty(G * dg, dtype=torch.uint8, device=dev)
    u_blob = torch.empty(G * ug, dtype=torch.uint8, device=dev)
    for g in range(G):
        lm.pack_blocks(rnd(L, H), w.du_bits, d_blob[g * dg:(g + 1) * dg])
        lm.pack_blocks(rnd(H, L), w.du_bits, u_blob[g * ug:(g + 1) * ug])
    shared = []
    for shp in ((Fs, H), (Fs, H), (H, Fs)):
        t = torch.empty(*shp, dtype=torch.int16, device=dev)
        lm.pack_bf16(rnd(*shp), t)
        shared.append(t)
    rec = lm.expert_record_bytes(L, F)
    experts = torch.empty(E, rec, dtype=torch.uint8, device=dev)
    chunk = 64
    for e0 in range(0, E, chunk):
        n = min(chunk, E - e0)
        g_, u_, d_ = wl.torch_expert_masters(w, seed, layer_idx, e0, n, dev)
        lm.pack_expert_records(g_, u_, d_, experts[e0:e0 + n])
        del g_, u_, d_
    layer.load(dict(router_bf16=router_bf16,
                    router_bias=None if bias is None else torch.from_numpy(bias).to(dev),
                    labels=torch.from_numpy(labels).to(dev), d_blob=d_blob, u_blob=u_blob,
                    experts=experts, shared=tuple(shared)))
    torch.cuda.synchronize()
    return layer, labels


def phase_bytes(w, idx, labels):
    """Algorithmic HBM bytes of each of the four decode kernels for one
    forward with routing idx [T][K]: every weight the step must read once,
    plus the activations it must read and write."""
    T, H, L, E, K, G, F, Fs = (w.tokens, w.hidden, w.latent, w.n_experts, w.top_k, w.n_groups,
                               w.expert_ffn, w.shared_ffn)
    du = (w.du_bits / 8.0) * (34.0 / 32.0 if w.du_bits == 8 else 18.0 / 16.0)  # bytes / weight
    distinct = len(set(idx.ravel().tolist()))
    used_groups = len(set(labels[idx.ravel()].tolist()))
    fp4 = 0.5 + 1.0 / 16.0
    p1 = E * H * 2 + G * L * H * du + 2 * Fs * H * 2 + T * H * 4 + T * G * L * 4 + T * Fs * 4
    p2 = distinct * 2 * F * L * fp4 + T * K * (L + F) * 4
    p3 = distinct * L * F * fp4 + T * K * (F + L) * 4
    p4 = used_groups * H * L * du + H * Fs * 2 + T * (G * L + Fs + H) * 4
    return [p1, p2, p3, p4], distinct, used_groups


def measured_traffic(kernel, workload, path=TRAFFIC_FILE):
    """HBM bytes per launch of `kernel` (a name, or a list of names whose
    launches make up one phase: their bytes add) from the committed rocprofv3
    counter summary, or None when there is none or the kernel source has
    changed since the counters were taken."""
    import hashlib
    try:
        with open(path) as f:
            t = json.load(f)
        src = open(os.path.join(ROOT, t["source"]), "rb").read()
    except (OSError, ValueError, KeyError):
        return None
    if t.get("workload") != workload or hashlib.sha256(src).hexdigest() != t["source_sha256"]:
        return None
    names = kernel if isinstance(kernel, list) else [kernel]
    ks = [t["kernels"].get(n) for n in names]
    return None if any(k is None for k in ks) else sum(k["traffic_bytes"] for k in ks)


def prefill_flops(w, idx, labels):
    """Algorithmic flops of each prefill phase for routing idx [T][K]: D and
    U count the (token, group) pairs the tokens route into (the kernels run
    all G groups; that figure is reported beside it), the router one pass of
    bf16 products (the kernel runs two)."""
    T, H, L, E, K, G, F, Fs = (idx.shape[0], w.hidden, w.latent, w.n_experts, w.top_k,
                               w.n_groups, w.expert_ffn, w.shared_ffn)
    lab = labels[idx]
    pairs = int(sum(len(set(r.tolist())) for r in lab))
    fl = [2.0 * T * E * H, 0.0, 2.0 * pairs * L * H, 2.0 * T * 2 * Fs * H,
          2.0 * T * K * 2 * F * L, 2.0 * T * K * L * F, 0.0,
          2.0 * pairs * H * L + 2.0 * T * H * Fs]
    executed = [4.0 * T * E * H, 0.0, 2.0 * T * G * L * H, 4.0 * T * 2 * Fs * H, None, None, 0.0,
                2.0 * T * G * H * L + 4.0 * T * H * Fs]
    return fl, executed, pairs


def bench_prefill(lm, wl, w, args, torch):
    """Times lmoe_forward on the prefill path; returns the result dict."""
    layers = []
    t_build = time.time()
    for r in range(args.prefill_copies):
        L_, lab = build_layer(lm, wl, w, args.seed, r, torch)
        layers.append((L_, lab))
    log("prefill: built %d layers in %.1f s" % (len(layers), time.time() - t_build))
    T = w.tokens
    x = torch.from_numpy(wl.x(w, args.seed, 0)).cuda()
    y = torch.empty(T, w.hidden, device="cuda")
    fl, ex, pairs, counts = [], [], [], []
    for L_, lab in layers:
        idx = torch.empty(T, w.top_k, dtype=torch.int32, device="cuda")
        cnt = torch.empty(w.n_experts, dtype=torch.int32, device="cuda")
        L_.forward(x, y, debug=dict(topk_idx=idx, expert_count=cnt))
        torch.cuda.synchronize()
        f_, e_, p_ = prefill_flops(w, idx.cpu().numpy(), lab)
        fl.append(f_); ex.append(e_); pairs.append(p_); counts.append(cnt.cpu().numpy())
    flops = np.mean(np.array(fl), axis=0)
    n = len(layers)
    for i in range(args.prefill_warmup):
        layers[i % n][0].forward(x, y)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.prefill_steps):
        layers[i % n][0].forward(x, y)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.prefill_steps

    nph = lm.lib().lmoe_phase_count(T)
    assert nph == len(PREFILL_PHASES)
    nprof = max(2 * n, 8)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nph + 1)] for _ in range(nprof)]
    for row in evs:          # torch creates the HIP event at its first record
        for e in row:
            e.record()
    torch.cuda.synchronize()
    for i in range(nprof):
        L_ = layers[i % n][0]
        L_.set_phase_events([e.cuda_event for e in evs[i]])
        L_.forward(x, y)
    for L_, _ in layers:
        L_.set_phase_events(None)
    torch.cuda.synchronize()
    phase_ms = np.array([[row[k].elapsed_time(row[k + 1]) for k in range(nph)] for row in evs])
    phase_avg = phase_ms.mean(axis=0)
    tflops = [f / (p * 1e-3) / 1e12 if f else 0.0 for f, p in zip(flops, phase_avg)]
    dom = int(np.argmax(phase_avg))
    log("prefill step %.3f ms (%.0f tokens/s); phases (us): %s" % (
        ms, T / (ms * 1e-3), " ".join("%s %.1f" % (nm, p * 1e3)
                                       for nm, p in zip(PREFILL_PHASES, phase_avg))))
    log("prefill phase TFLOP/s (algorithmic): %s" % " ".join(
        "%s %.0f" % (nm, t) for nm, t in zip(PREFILL_PHASES, tflops) if t))
    c = np.concatenate(counts)
    gemm = [2, 3, 4, 5, 7]
    gemm_fl = float(sum(flops[i] for i in gemm))
    gemm_ms = float(sum(phase_avg[i] for i in gemm))
    grouped_fl = float(flops[4] + flops[5])
    grouped_ms = float(phase_avg[4] + phase_avg[5])
    out = {
        "workload": w.name,
        "tokens": T,
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "ms_per_step": ms,
        "steps": args.prefill_steps,
        "warmup": args.prefill_warmup,
        "weight_copies": n,
        "step_algorithmic_tflop": float(np.sum(flops)) / 1e12,
        "step_tflops": float(np.sum(flops)) / (ms * 1e-3) / 1e12,
        "token_group_pairs": float(np.mean(pairs)),
        "expert_tokens": {"max": int(c.max()), "median": float(np.median(c)),
                          "zero": int((c == 0).sum()) // n},
        "phases_us": {nm: float(p * 1e3) for nm, p in zip(PREFILL_PHASES, phase_avg)},
        "phase_tflops": {nm: t for nm, t in zip(PREFILL_PHASES, tflops) if t},
        "grouped_gemm": {"achieved": grouped_fl / (grouped_ms * 1e-3) / 1e12,
                         "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": grouped_fl / (grouped_ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS},
        "all_gemms": {"achieved": gemm_fl / (gemm_ms * 1e-3) / 1e12,
                      "frac": gemm_fl / (gemm_ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS},
        "roofline": {"bound": "mfma", "achieved": tflops[dom], "peak": MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops[dom] / MFMA_PEAK_TFLOPS,
                     "traffic": measured_traffic(PREFILL_KERNEL_IDS[dom], w.name, PREFILL_TRAFFIC_FILE),
                     "kernel": PREFILL_KERNELS[dom],
                     "phase": PREFILL_PHASES[dom], "kernel_us": float(phase_avg[dom] * 1e3),
                     "kernel_algorithmic_flop": float(flops[dom]),
                     "kernel_executed_flop": ex[0][dom]},
    }
    for L_, _ in layers:
        L_.close()
    return out


def cpu_baseline(w, seed, tokens):
    """The fp64 oracle timed on the host on a bounded sample: one forward of
    `tokens` tokens of layer 0 (including its on-the-fly dequantization of
    D, U and the experts it touches; excluding weight drawing and packing)."""
    import oracle
    from latent_mixture_experts_amd import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = 1
    d = oracle.LayerDims(w.hidden, w.latent, w.n_experts, w.top_k, w.n_groups, w.expert_ffn,
                         w.shared_ffn, w.du_bits)
    x = wl.x(w, seed, 0, tokens=tokens)
    m = wl.masters(w, seed, 0)
    lg = oracle.router_logits(x, oracle.f32_to_bf16_bits(m["router"]), m["router_bias"])
    idx, _ = oracle.select_topk(lg, w.top_k)
    m["expert_ids"] = sorted(set(idx.ravel().tolist()))
    blobs = oracle.pack_layer(d, m)
    t0 = time.perf_counter()
    oracle.layer_forward(d, blobs, x)
    dt = time.perf_counter() - t0
    return {"value": tokens / dt, "unit": "tokens/s", "cores": int(blas), "kind": "oracle",
            "sample": "one fp64 NumPy forward of %d tokens of the %s layer (seed %d), including "
                      "dequantization of D, U and the %d experts it touches; %.1f s" % (
                          tokens, w.name, seed, len(m["expert_ids"]), dt)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="145b_decode")
    ap.add_argument("--copies", type=int, default=8)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-workload", default="145b_prefill")
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--prefill-warmup", type=int, default=3)
    ap.add_argument("--prefill-copies", type=int, default=2)
    ap.add_argument("--no-prefill", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(--gpus %d refused)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from latent_mixture_experts_amd import lmoe as lm
    from latent_mixture_experts_amd import workloads as wl

    w = wl.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    if w.tokens > 8:
        pre = bench_prefill(lm, wl, w, args, torch)
        out = {
            "metric": "latent-MoE layer tokens/s (prefill; MFMA roofline)",
            "value": pre["value"], "unit": "tokens/s", "n_gpus": 1,
            "steps": args.prefill_steps, "warmup": args.prefill_warmup,
            "ms_per_step": pre["ms_per_step"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f16", "data": "synthetic",
            "config": {"workload": w.name, "tokens": w.tokens, "hidden": w.hidden,
                       "latent": w.latent, "experts": w.n_experts, "top_k": w.top_k,
                       "groups": w.n_groups, "expert_ffn": w.expert_ffn,
                       "shared_ffn": w.shared_ffn, "du_format": "Q%d" % w.du_bits,
                       "expert_format": "NVFP4", "router_bias": w.router_bias,
                       "weight_copies": args.prefill_copies},
            "roofline": pre["roofline"],
            "prefill": pre,
        }
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline(w, args.seed, 16)
        print(json.dumps(out), flush=True)
        return
    stack = w.n_layers > 1
    n_handles = w.n_layers if stack else args.copies
    t_build = time.time()
    layers, labels = [], []
    for r in range(n_handles):
        L_, lab = build_layer(lm, wl, w, args.seed, r, torch)
        layers.append(L_)
        labels.append(lab)
    log("built %d layers in %.1f s" % (n_handles, time.time() - t_build))

    T = w.tokens
    x0 = torch.from_numpy(wl.x(w, args.seed, 0)).cuda()
    x = x0.clone()
    y = torch.empty(T, w.hidden, device="cuda")

    def step(i):
        if stack:
            for L_ in layers:
                L_.forward_block(x)
        else:
            layers[i % n_handles].forward(x, y)

    # routing of each layer, for the algorithmic byte counts
    bytes_per_layer, distinct, groups = [], [], []
    xr = x0.clone()
    for r, L_ in enumerate(layers):
        idx = torch.empty(T, w.top_k, dtype=torch.int32, device="cuda")
        if stack:
            # the routing a block sees is that of its normalized input
            xn = xr / torch.sqrt((xr.double() ** 2).mean(dim=1, keepdim=True) + 1e-6).float()
            L_.forward(xn, y, debug=dict(topk_idx=idx))
            xr = xr + y
        else:
            L_.forward(x, y, debug=dict(topk_idx=idx))
        torch.cuda.synchronize()
        pb, dn, ug = phase_bytes(w, idx.cpu().numpy(), labels[r])
        bytes_per_layer.append(pb)
        distinct.append(dn)
        groups.append(ug)
    pbytes = np.mean(np.array(bytes_per_layer), axis=0)
    layer_bytes = float(np.sum(pbytes))

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        step(i)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps

    # per-kernel durations, with HIP events on the stream the kernels run on.
    # Single layer: each phase is launched alone, back to back over the weight
    # copies (cold, as in the forward), one event pair around the run, so a
    # figure is one kernel's launch-to-launch time. Stack (block forwards):
    # events between the phases of each forward, which add their own gaps.
    nph = lm.lib().lmoe_phase_count(T)
    if not stack:
        for L_ in layers:
            L_.forward(x, y)               # the workspace state each phase reads
        nrep = max(n_handles * 8, 64)
        phase_avg = []
        for k in range(1, nph + 1):
            for i in range(n_handles):
                layers[i].run_phase(x, y, k)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(nrep):
                layers[i % n_handles].run_phase(x, y, k)
            e1.record()
            torch.cuda.synchronize()
            phase_avg.append(e0.elapsed_time(e1) / nrep)
        phase_avg = np.array(phase_avg)
    else:
        nprof = max(n_handles * 2, 32)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nph + 1)] for _ in range(nprof)]
        for row in evs:
            for e in row:
                e.record()
        torch.cuda.synchronize()
        for i in range(nprof):
            L_ = layers[i % n_handles]
            L_.set_phase_events([e.cuda_event for e in evs[i]])
            L_.forward_block(x)
        for L_ in layers:
            L_.set_phase_events(None)
        torch.cuda.synchronize()
        phase_ms = np.array([[row[k].elapsed_time(row[k + 1]) for k in range(nph)] for row in evs])
        phase_avg = phase_ms.mean(axis=0)
    dom = int(np.argmax(phase_avg))
    achieved = pbytes[dom] / (phase_avg[dom] * 1e-3) / 1e9
    step_bytes = layer_bytes * (w.n_layers if stack else 1)
    log("step %.2f us; phases (us): %s; phase GB/s: %s; whole-step %.0f GB/s over %.1f MB" % (
        ms * 1e3, " ".join("%.2f" % (p * 1e3) for p in phase_avg),
        " ".join("%.0f" % (b / (p * 1e-3) / 1e9) for b, p in zip(pbytes, phase_avg)),
        step_bytes / (ms * 1e-3) / 1e9, step_bytes / 1e6))
    log("distinct experts per layer %.1f, groups used %.1f" % (np.mean(distinct), np.mean(groups)))

    out = {
        "metric": ("latent-MoE %d-layer stack tokens/s (decode; HBM roofline)" % w.n_layers) if stack
                  else "latent-MoE layer tokens/s (decode; HBM roofline)",
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": T, "hidden": w.hidden, "latent": w.latent,
                   "experts": w.n_experts, "top_k": w.top_k, "groups": w.n_groups,
                   "expert_ffn": w.expert_ffn, "shared_ffn": w.shared_ffn,
                   "du_format": "Q%d" % w.du_bits, "expert_format": "NVFP4",
                   "layers": w.n_layers,
                   "weight_copies": None if stack else args.copies,
                   "step_algorithmic_bytes": step_bytes,
                   "step_GBps": step_bytes / (ms * 1e-3) / 1e9},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic("k_phase%d" % (dom + 1), w.name),
                     "kernel": "k_phase%d" % (dom + 1),
                     "kernel_us": phase_avg[dom] * 1e3,
                     "kernel_algorithmic_bytes": pbytes[dom]},
    }
    for L_ in layers:
        L_.close()
    del layers
    if not args.no_prefill and not stack:
        out["prefill"] = bench_prefill(lm, wl, wl.WORKLOADS[args.prefill_workload], args, torch)
    if not args.no_cpu_baseline and not stack:
        out["cpu_baseline"] = cpu_baseline(w, args.seed, T)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
