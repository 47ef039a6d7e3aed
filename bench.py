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

The default line also carries nested objects, each with its own roofline and
oracle CPU baseline: "decode_t1" (the same layers at T = 1, with the byte
counts of reading D and U for used groups only and for all groups),
"decode_120b" (the Edge0-120B-shaped layer, Q4 D/U, latent 1280, T = 5),
"mtp_draft" (the draft layer's MoE: 512 experts of 3 x 1280 x 640, Q8 D/U,
T = 1, one drafted token), "decode_q3k" (the 145B layer at T = 4 with the
Q3_K build's expert records: Q3_K gate/up, IQ4_NL down),
"ple_gather" (the n-gram embedding gather on the full 51.2 GB table at
T = 4096 and T = 4), "stack_145b" (48 independently seeded 145B-shaped layers as pre-norm
residual blocks, T = 4: whole-stack tokens/s and sustained HBM bandwidth) and
"prefill" (the 145B-shaped layer at T = 4096 with a router bias skewing expert
loads, on the prefill path, with its per-kernel MFMA roofline).
--workload picks another primary line.

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
PREFILL_KERNELS = ["k_prep + k_dense_dma<BF16,Logits> + k_select", "k_perm_* (with the routed D's group lists)",
                   "k_dense16<F16, gather> (D over the routed (t, g) pairs; 128 x 128 wave tiles, LDS DMA)",
                   "k_dense_dma<BF16,SwigluB2> (shared gate/up)",
                   "k_grouped_dma<GateUp> (LDS DMA) + k_grouped_short<GateUp> (64- and 32-token pieces)",
                   "k_down_res (activations resident in LDS; 64- and 32-token blocks)", "k_combine",
                   "k_dense_dma<BF16,Y> (shared down into y) + k_dense16<Y> (U, split along k) + k_ytiles (split sums onto y)"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
PREFILL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_145b_t4096_traffic.json")
# kernel of each prefill phase as rocprofv3 names it (D and U on fp16 weights)
PREFILL_KERNEL_IDS = [["k_prep", "k_dense_dma<3, 0>", "k_select<5, 8>"],
                      ["k_perm_mask", "k_perm_scan", "k_perm_scatter"], ["k_dense16<1, true>"],
                      "k_dense_dma<3, 2>",
                      ["k_grouped_dma<0>", "k_grouped_short<0, 2, 8>", "k_grouped_short<0, 1, 8>"],
                      ["k_down_res<8, 2>", "k_down_res<8, 1>"], "k_combine",
                      ["k_dense_dma<3, 3>", "k_dense16<3, false>", "k_ytiles<3>"]]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_layer(lm, wl, w, seed, layer_idx, torch):
    """One layer's weights, drawn and packed on the device."""
    dev = "cuda"
    E, H, L, G, F, Fs = w.n_experts, w.hidden, w.latent, w.n_groups, w.expert_ffn, w.shared_ffn
    layer = lm.Layer(H, L, E, w.top_k, G, F, Fs, w.du_bits, max(w.tokens, 1),
                     has_router_bias=w.router_bias, expert_format=w.expert_format)
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
    rec = lm.expert_record_bytes(L, F, w.expert_format)
    experts = torch.empty(E, rec, dtype=torch.uint8, device=dev)
    if w.expert_format == 1:
        # Q3_K / IQ4_NL records of random codes and scales (the library has no
        # device packer for them): every fp16 d set to a value of the size a
        # quantizer gives N(0, 0.02) weights
        experts.copy_(torch.randint(0, 256, (E, rec), generator=gen, device=dev, dtype=torch.uint8))
        n1 = F * (L // 256) * 110
        def set_d(view, off):
            d = (torch.rand(view.shape[:-1], generator=gen, device=dev) * 3e-4 + 3e-4).to(torch.float16)
            view[..., off:off + 2] = d.view(torch.uint8).view(*view.shape[:-1], 2)
        set_d(experts[:, :2 * n1].reshape(E, 2 * F * (L // 256), 110), 108)
        set_d(experts[:, 2 * n1:].reshape(E, L * (F // 32), 18), 0)
    else:
        for e0 in range(0, E, 64):
            n = min(64, E - e0)
            g_, u_, d_ = wl.torch_expert_masters(w, seed, layer_idx, e0, n, dev)
            lm.pack_expert_records(g_, u_, d_, experts[e0:e0 + n])
            del g_, u_, d_
    layer.load(dict(router_bf16=router_bf16,
                    router_bias=None if bias is None else torch.from_numpy(bias).to(dev),
                    labels=torch.from_numpy(labels).to(dev), d_blob=d_blob, u_blob=u_blob,
                    experts=experts, shared=tuple(shared)))
    torch.cuda.synchronize()
    return layer, labels


def decode_bytes(w, idx, labels):
    """Algorithmic HBM bytes of one decode forward with routing idx [T][K]:
    every weight the forward must read once (router, D of every group as the
    layer computes it, U of the groups the tokens use, each distinct expert's
    record, the shared expert) plus the activations read and written. Also
    the two variants of the T = 1 accounting: D and U of the used groups
    only, and of all groups."""
    T, H, L, E, K, G, F, Fs = (idx.shape[0], w.hidden, w.latent, w.n_experts, w.top_k,
                               w.n_groups, w.expert_ffn, w.shared_ffn)
    du = (w.du_bits / 8.0) * (34.0 / 32.0 if w.du_bits == 8 else 18.0 / 16.0)  # bytes / weight
    distinct = len(set(idx.ravel().tolist()))
    used = len(set(labels[idx.ravel()].tolist()))
    if getattr(w, "expert_format", 0) == 1:
        gu_w, dn_w = 110.0 / 256.0, 18.0 / 32.0      # Q3_K gate/up, IQ4_NL down: bytes / weight
    else:
        gu_w = dn_w = 0.5 + 1.0 / 16.0              # NVFP4
    common = E * H * 2 + distinct * F * L * (2 * gu_w + dn_w) + 3 * Fs * H * 2 + 2 * T * H * 4
    phases = [E * H * 2 + G * L * H * du + 2 * Fs * H * 2 + T * H * 4 + T * G * L * 4 + T * Fs * 4,
              distinct * 2 * F * L * gu_w + T * K * (L + F) * 4,
              distinct * L * F * dn_w + T * K * (F + L) * 4,
              used * H * L * du + H * Fs * 2 + T * (G * L + Fs + H) * 4]
    out = {
        "phases": phases,
        "bytes": common + (G + used) * L * H * du,
        "bytes_used_groups": common + 2 * used * L * H * du,
        "bytes_all_groups": common + 2 * G * L * H * du,
        "distinct_experts": distinct,
        "used_groups": used,
    }
    return out


def measured_traffic(kernel, workload, path=TRAFFIC_FILE):
    """HBM bytes per launch of `kernel` (a name, or a list of names whose
    launches make up one phase: their bytes add) from the committed rocprofv3
    counter summary for `workload`, or None when there is none or the kernel
    source has changed since the counters were taken."""
    import hashlib
    try:
        with open(path) as f:
            t = json.load(f)
        src = open(os.path.join(ROOT, t["source"]), "rb").read()
    except (OSError, ValueError, KeyError):
        return None
    if hashlib.sha256(src).hexdigest() != t["source_sha256"]:
        return None
    entry = t.get("workloads", {}).get(workload) if "workloads" in t else \
        (t if t.get("workload") == workload else None)
    if entry is None:
        return None
    names = kernel if isinstance(kernel, list) else [kernel]
    ks = [entry["kernels"].get(n) for n in names]
    return None if any(k is None for k in ks) else sum(k["traffic_bytes"] for k in ks)


def prefill_flops(w, idx, labels):
    """Algorithmic flops of each prefill phase for routing idx [T][K]: D and
    U count the (token, group) pairs the tokens route into (D runs over
    those pairs; U, and D in its all-groups form, over all G groups: that
    figure is reported beside it), the router one pass of bf16 products (the
    kernel runs two)."""
    T, H, L, E, K, G, F, Fs = (idx.shape[0], w.hidden, w.latent, w.n_experts, w.top_k,
                               w.n_groups, w.expert_ffn, w.shared_ffn)
    lab = labels[idx]
    pairs = int(sum(len(set(r.tolist())) for r in lab))
    fl = [2.0 * T * E * H, 0.0, 2.0 * pairs * L * H, 2.0 * T * 2 * Fs * H,
          2.0 * T * K * 2 * F * L, 2.0 * T * K * L * F, 0.0,
          2.0 * pairs * H * L + 2.0 * T * H * Fs]
    executed = [4.0 * T * E * H, 0.0, 2.0 * pairs * L * H, 4.0 * T * 2 * Fs * H, None, None, 0.0,
                2.0 * T * G * H * L + 4.0 * T * H * Fs]
    return fl, executed, pairs


PLE_ROW_BYTES = 160


def ple_head_rows():
    """Rows per hash head of the n-gram table: 20,000,003 for the first (as
    printed) and the rest of the 320,001,536 rows split evenly, the first
    three of the others taking one row more."""
    total, first, n = 320001536, 20000003, 15
    base, extra = divmod(total - first, n)
    return [first] + [base + (1 if h <= extra else 0) for h in range(1, 16)]


def bench_ple(lm, args, torch, cpu):
    """The PLE n-gram gather on the full table (51.2 GB of E4M3 rows, drawn
    on the device) at T = 4096 (a prefill batch) and T = 4 (a verify window).
    Each step gathers one of 8 pre-drawn token batches; HIP events on the
    stream the kernel runs on time the steps."""
    dev = "cuda"
    sizes = ple_head_rows()
    n = sum(sizes)
    table = torch.empty(n, PLE_ROW_BYTES, dtype=torch.uint8, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(args.seed * 7919 + 11)
    for r0 in range(0, n, 1 << 22):
        r1 = min(n, r0 + (1 << 22))
        table[r0:r1] = torch.randint(0, 256, (r1 - r0, PLE_ROW_BYTES), generator=g, device=dev,
                                     dtype=torch.uint8)
    res = {"table_bytes": n * PLE_ROW_BYTES, "head_rows": sizes}
    per_tok = 16 * PLE_ROW_BYTES * 3           # E4M3 rows read, bf16 rows written
    for T, steps in ((4096, 200), (4, 400)):
        toks = [torch.randint(-1, 248000, (T + 2,), generator=g, device=dev, dtype=torch.int32)
                for _ in range(8)]
        out = torch.empty(T, 16, PLE_ROW_BYTES, dtype=torch.int16, device=dev)
        for i in range(20):
            lm.ple_gather(toks[i % 8], table, sizes, out)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            lm.ple_gather(toks[i % 8], table, sizes, out)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        algo = T * (per_tok + 4) + 8
        gbs = algo / (us * 1e-6) / 1e9
        res["t%d" % T] = {
            "tokens": T, "us_per_step": us, "value": T / (us * 1e-6), "unit": "tokens/s",
            "steps": steps, "algorithmic_bytes": algo,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": None, "kernel": "k_ple",
                         "kernel_us": us, "kernel_algorithmic_bytes": algo},
        }
        log("ple gather T=%d: %.2f us/step, %.0f GB/s algorithmic" % (T, us, gbs))
    del table
    torch.cuda.empty_cache()
    if cpu:
        import oracle.ple as ople
        rng = np.random.default_rng(args.seed)
        small = [100003] * 16
        tab = rng.integers(0, 256, (sum(small), PLE_ROW_BYTES), dtype=np.uint8)
        T = 2048
        toks = rng.integers(-1, 248000, T + 2)
        t0 = time.perf_counter()
        ople.ple_gather(toks, tab, small)
        dt = time.perf_counter() - t0
        cores = host_cores()
        res["cpu_baseline"] = {
            "value": T / dt, "unit": "tokens/s", "cores": 1, "cpu_count": cores["cpu_count"],
            "affinity": cores["affinity"], "kind": "oracle",
            "sample": "the oracle's hash and gather of %d tokens over a table of 16 x 100,003 rows "
                      "(Python integer hashing, one core); %.2f s" % (T, dt)}
    return res


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
    nph = lm.lib().lmoe_phase_count(T)
    assert nph == len(PREFILL_PHASES)

    def timed():
        """Step time over the timed steps, then per-phase times (events)."""
        for i in range(args.prefill_warmup):
            layers[i % n][0].forward(x, y)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(args.prefill_steps):
            layers[i % n][0].forward(x, y)
        end.record()
        torch.cuda.synchronize()
        step_ms = start.elapsed_time(end) / args.prefill_steps
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
        pm = np.array([[row[k].elapsed_time(row[k + 1]) for k in range(nph)] for row in evs])
        return step_ms, pm.mean(axis=0)

    ms, phase_avg = timed()
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
        "dtype": "f16",
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
    # the variant with D over all G groups of every token (the reference
    # engine's form), on the second stream beside the routing
    for L_, _ in layers:
        L_.set_prefill_d(0)
    ms_a, phase_a = timed()
    for L_, _ in layers:
        L_.set_prefill_d(1)
    d_all = 2.0 * T * w.n_groups * w.latent * w.hidden
    log("prefill, D over all groups: step %.3f ms; D %.1f us (routed pairs: %.1f us)" % (
        ms_a, phase_a[2] * 1e3, phase_avg[2] * 1e3))
    out["d_all_groups"] = {
        "ms_per_step": ms_a, "value": T / (ms_a * 1e-3), "unit": "tokens/s",
        "phases_us": {nm: float(p * 1e3) for nm, p in zip(PREFILL_PHASES, phase_a)},
        "d_executed_tflop": d_all / 1e12,
        "d_tflops_executed": d_all / (phase_a[2] * 1e-3) / 1e12,
        "routed_d_executed_tflop": flops[2] / 1e12,
        "routed_d_tflops": flops[2] / (phase_avg[2] * 1e-3) / 1e12,
    }
    for L_, _ in layers:
        L_.close()
    return out


def calibrate_hbm(torch, copy_bytes=256 << 20, reps=4, read_bytes=1 << 30):
    """Reference runs for the profiler's HBM counters (--calibrate-hbm):
    a device-to-device copy of exactly 256 MiB, repeated (each copy reads
    and writes 268,435,456 bytes: the scale for FETCH_SIZE / WRITE_SIZE), and
    the read bandwidth of a plain streaming reduction over 1 GiB (the
    achievable-bandwidth reference beside the published peak)."""
    src = torch.ones(copy_bytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    big = torch.ones(read_bytes // 4, dtype=torch.float32, device="cuda")
    for _ in range(3):
        big.sum()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 20
    start.record()
    for _ in range(n):
        big.sum()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / n
    print(json.dumps({"copy_bytes_per_launch": copy_bytes, "copies": reps,
                      "sum_read_bytes": read_bytes, "sum_ms": ms,
                      "sum_read_GBps": read_bytes / (ms * 1e-3) / 1e9}), flush=True)


def host_cores():
    """Threads the oracle can use on this host: os.cpu_count(), the
    affinity-mask size and the BLAS thread count."""
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = 1
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = os.cpu_count()
    return {"cpu_count": os.cpu_count(), "affinity": aff, "blas_threads": int(blas)}


def cpu_baseline(w, seed, tokens, layers=1, min_seconds=0.0):
    """The fp64 oracle timed on the host on a bounded sample: one forward of
    `tokens` tokens of layer 0 (including its on-the-fly dequantization of
    D, U and the experts it touches; excluding weight drawing and packing).
    For a stack of `layers` layers the sample is one layer, and the rate is
    scaled by the layer count."""
    import oracle
    from latent_mixture_experts_amd import workloads as wl
    cores = host_cores()
    d = oracle.LayerDims(w.hidden, w.latent, w.n_experts, w.top_k, w.n_groups, w.expert_ffn,
                         w.shared_ffn, w.du_bits)
    x = wl.x(w, seed, 0, tokens=tokens)
    if layers > 1:
        x = oracle.rmsnorm(x)
    m = wl.masters(w, seed, 0)
    lg = oracle.router_logits(x, oracle.f32_to_bf16_bits(m["router"]), m["router_bias"])
    idx, _ = oracle.select_topk(lg, w.top_k)
    m["expert_ids"] = sorted(set(idx.ravel().tolist()))
    blobs = oracle.pack_layer(d, m)
    t0 = time.perf_counter()
    reps = 0
    while True:
        oracle.layer_forward(d, blobs, x)
        reps += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = (time.perf_counter() - t0) / reps
    what = ("%d fp64 NumPy forward%s of %d tokens of the %s layer (seed %d), each including "
            "dequantization of D, U and the %d experts it touches; %.1f s each" % (
                reps, "s" if reps > 1 else "", tokens, w.name, seed, len(m["expert_ids"]), dt))
    if layers > 1:
        what = ("layer 0 of the %d-layer stack: " % layers) + what + \
               "; the stack's rate is this layer's divided by %d" % layers
    return {"value": tokens / (dt * layers), "unit": "tokens/s", "cores": cores["blas_threads"],
            "cpu_count": cores["cpu_count"], "affinity": cores["affinity"], "kind": "oracle",
            "sample": what}


def phase_times(lm, layers, x, y, T, torch, stack):
    """Per-kernel durations in ms with HIP events on the stream the kernels
    run on. Single layer: each phase is launched alone, back to back over the
    weight copies (cold, as in the forward), one event pair around the run,
    so a figure is one kernel's launch-to-launch time. Stack (block
    forwards): events between the phases of each forward, which add their
    own gaps."""
    nph = lm.lib().lmoe_phase_count(T)
    n = len(layers)
    if not stack:
        for L_, _ in layers:
            L_.forward(x, y)               # the workspace state each phase reads
        nrep = max(n * 8, 64)
        out = []
        for k in range(1, nph + 1):
            for i in range(n):
                layers[i][0].run_phase(x, y, k)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(nrep):
                layers[i % n][0].run_phase(x, y, k)
            e1.record()
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) / nrep)
        return np.array(out)
    nprof = max(n * 2, 32)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nph + 1)] for _ in range(nprof)]
    for row in evs:
        for e in row:
            e.record()
    torch.cuda.synchronize()
    for i in range(nprof):
        L_ = layers[i % n][0]
        L_.set_phase_events([e.cuda_event for e in evs[i]])
        L_.forward_block(x)
    for L_, _ in layers:
        L_.set_phase_events(None)
    torch.cuda.synchronize()
    ms = np.array([[row[k].elapsed_time(row[k + 1]) for k in range(nph)] for row in evs])
    return ms.mean(axis=0)


def bench_decode(lm, wl, w, args, torch, T=None, layers=None, steps=None, warmup=None):
    """Times decode forwards (block forwards through a stack for a workload
    with n_layers > 1); returns the result dict (value, timing percentiles,
    bytes, roofline, stage spans) and the layers for reuse."""
    T = w.tokens if T is None else T
    stack = w.n_layers > 1
    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    if layers is None:
        n_handles = w.n_layers if stack else args.copies
        t_build = time.time()
        layers = [build_layer(lm, wl, w, args.seed, r, torch) for r in range(n_handles)]
        log("%s: built %d layers in %.1f s" % (w.name, n_handles, time.time() - t_build))
    n_handles = len(layers)
    x0 = torch.from_numpy(wl.x(w, args.seed, 0, tokens=T)).cuda()
    x = x0.clone()
    y = torch.empty(T, w.hidden, device="cuda")

    def step(i):
        if stack:
            for L_, _ in layers:
                L_.forward_block(x)
        else:
            layers[i % n_handles][0].forward(x, y)

    # routing of each layer, for the algorithmic byte counts
    per = []
    xr = x0.clone()
    for L_, lab in layers:
        idx = torch.empty(T, w.top_k, dtype=torch.int32, device="cuda")
        if stack:
            # the routing a block sees is that of its normalized input
            xn = xr / torch.sqrt((xr.double() ** 2).mean(dim=1, keepdim=True) + 1e-6).float()
            L_.forward(xn, y, debug=dict(topk_idx=idx))
            xr = xr + y
        else:
            L_.forward(x, y, debug=dict(topk_idx=idx))
        torch.cuda.synchronize()
        per.append(decode_bytes(w, idx.cpu().numpy(), lab))
    keys = ["bytes", "bytes_used_groups", "bytes_all_groups", "distinct_experts", "used_groups"]
    mean = {k: float(np.mean([p[k] for p in per])) for k in keys}
    layer_bytes = mean["bytes"]
    step_bytes = layer_bytes * (len(layers) if stack else 1)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        step(i)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    # per-step distribution: an event pair around each step
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i, (a, b) in enumerate(ev):
        a.record()
        step(i)
        b.record()
    torch.cuda.synchronize()
    per_step = np.array([a.elapsed_time(b) for a, b in ev])
    p10, p50, p90 = (float(v) for v in np.percentile(per_step, [10, 50, 90]))
    x.copy_(x0)
    pt = phase_times(lm, layers, x, y, T, torch, stack)
    x.copy_(x0)
    pbytes = np.mean(np.array([p["phases"] for p in per]), axis=0)
    gbps = step_bytes / (ms * 1e-3) / 1e9
    dom = int(np.argmax(pt))
    kern_us = float(pt[dom] * 1e3)
    # phase 4 is two launches from four tokens on (its partials' ordered sum
    # is a kernel of its own): its time and traffic are those of both
    ysum = T >= 4
    phase_names = ["k_phase1", "k_phase2", "k_phase3", "k_phase4 + k_ysum" if ysum else "k_phase4"]
    phase_ids = ["k_phase1", "k_phase2", "k_phase3", ["k_phase4", "k_ysum"] if ysum else "k_phase4"]
    kbytes = float(pbytes[dom])
    log("%s T=%d: %.2f us/step (p10 %.2f, median %.2f, p90 %.2f us); %.0f GB/s over %.1f MB; "
        "%.1f distinct experts, %.1f groups used; kernels (us): %s; kernel GB/s: %s" % (
            w.name, T, ms * 1e3, p10 * 1e3, p50 * 1e3, p90 * 1e3, gbps, step_bytes / 1e6,
            mean["distinct_experts"], mean["used_groups"],
            " ".join("%.2f" % (v * 1e3) for v in pt),
            " ".join("%.0f" % (b / (v * 1e-3) / 1e9) for b, v in zip(pbytes, pt))))
    out = {
        "workload": w.name,
        "tokens": T,
        "layers": len(layers) if stack else 1,
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "ms_per_step": ms,
        "step_us_p10": p10 * 1e3, "step_us_median": p50 * 1e3, "step_us_p90": p90 * 1e3,
        "steps": steps, "warmup": warmup,
        "weight_copies": None if stack else n_handles,
        "step_algorithmic_bytes": step_bytes,
        "step_GBps": gbps,
        "hbm_frac": gbps / HBM_PEAK_GBS,
        "distinct_experts": mean["distinct_experts"],
        "used_groups": mean["used_groups"],
        "roofline": {"bound": "hbm", "achieved": kbytes / (kern_us * 1e-6) / 1e9, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": kbytes / (kern_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                     "traffic": measured_traffic(phase_ids[dom], "%s_t%d" % (w.name, T)),
                     "kernel": phase_names[dom], "kernel_us": kern_us,
                     "kernel_algorithmic_bytes": kbytes},
        "kernels_us": {"k_phase%d" % (k + 1): float(v * 1e3) for k, v in enumerate(pt)},
        "kernels_GBps": {"k_phase%d" % (k + 1): float(b / (v * 1e-3) / 1e9)
                         for k, (b, v) in enumerate(zip(pbytes, pt))},
        "kernels_algorithmic_bytes": {"k_phase%d" % (k + 1): float(b) for k, b in enumerate(pbytes)},
    }
    if T == 1 and not stack:
        out["t1_bytes"] = {"used_groups_only": mean["bytes_used_groups"],
                           "all_groups": mean["bytes_all_groups"],
                           "read_by_kernel": mean["bytes"],
                           "GBps_used_groups_only": mean["bytes_used_groups"] / (ms * 1e-3) / 1e9,
                           "GBps_all_groups": mean["bytes_all_groups"] / (ms * 1e-3) / 1e9}
    return out, layers


def close_layers(layers):
    for L_, _ in layers:
        L_.close()


def config_of(w, T, copies):
    return {"workload": w.name, "tokens": T, "hidden": w.hidden, "latent": w.latent,
            "experts": w.n_experts, "top_k": w.top_k, "groups": w.n_groups,
            "expert_ffn": w.expert_ffn, "shared_ffn": w.shared_ffn,
            "du_format": "Q%d" % w.du_bits,
            "expert_format": "Q3_K+IQ4_NL" if w.expert_format == 1 else "NVFP4",
            "router_bias": w.router_bias, "layers": w.n_layers, "weight_copies": copies}


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
    ap.add_argument("--stack-steps", type=int, default=20)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="only the primary line: no T = 1, 120B, stack or prefill objects")
    ap.add_argument("--calibrate-hbm", action="store_true",
                    help="only run the reference copy and read for the HBM counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(--gpus %d refused)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_hbm:
        calibrate_hbm(torch)
        return
    from latent_mixture_experts_amd import lmoe as lm
    from latent_mixture_experts_amd import workloads as wl

    torch.cuda.set_device(0)
    cpu = not args.no_cpu_baseline
    if args.workload == "ple_gather":
        res = bench_ple(lm, args, torch, cpu)
        r = res["t4096"]
        out = {
            "metric": "PLE n-gram embedding gather tokens/s (HBM roofline)",
            "value": r["value"], "unit": "tokens/s", "n_gpus": 1, "steps": r["steps"], "warmup": 20,
            "ms_per_step": r["us_per_step"] * 1e-3, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "e4m3->bf16", "data": "synthetic",
            "config": {"workload": "ple_gather", "tokens": 4096, "table_bytes": res["table_bytes"]},
            "roofline": r["roofline"], "ple_gather": res,
        }
        if cpu:
            out["cpu_baseline"] = res["cpu_baseline"]
        print(json.dumps(out), flush=True)
        return
    w = wl.WORKLOADS[args.workload]
    if w.tokens > 8:
        pre = bench_prefill(lm, wl, w, args, torch)
        out = {
            "metric": "latent-MoE layer tokens/s (prefill; MFMA roofline)",
            "value": pre["value"], "unit": "tokens/s", "n_gpus": 1,
            "steps": args.prefill_steps, "warmup": args.prefill_warmup,
            "ms_per_step": pre["ms_per_step"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f16", "data": "synthetic",
            "config": config_of(w, w.tokens, args.prefill_copies),
            "roofline": pre["roofline"],
            "prefill": pre,
        }
        if cpu:
            out["cpu_baseline"] = pre.get("cpu_baseline") or cpu_baseline(w, args.seed, 8)
        print(json.dumps(out), flush=True)
        return

    stack = w.n_layers > 1
    res, layers = bench_decode(lm, wl, w, args, torch,
                               steps=args.stack_steps if stack else args.steps)
    out = {
        "metric": ("latent-MoE %d-layer stack tokens/s (decode; HBM roofline)" % w.n_layers) if stack
                  else "latent-MoE layer tokens/s (decode; HBM roofline)",
        "value": res["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": res["steps"],
        "warmup": res["warmup"],
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": dict(config_of(w, w.tokens, None if stack else args.copies),
                       step_algorithmic_bytes=res["step_algorithmic_bytes"],
                       step_GBps=res["step_GBps"]),
        "roofline": res["roofline"],
        "decode": res,
    }
    if cpu:
        out["cpu_baseline"] = cpu_baseline(w, args.seed, w.tokens, layers=w.n_layers, min_seconds=10.0)
    if not stack and not args.no_extra:
        r1, _ = bench_decode(lm, wl, w, args, torch, T=1, layers=layers)
        if cpu:
            r1["cpu_baseline"] = cpu_baseline(w, args.seed, 1)
        out["decode_t1"] = r1
    close_layers(layers)
    del layers
    if not stack and not args.no_extra:
        w120 = wl.WORKLOADS["120b_decode"]
        r120, l120 = bench_decode(lm, wl, w120, args, torch)
        close_layers(l120)
        del l120
        if cpu:
            r120["cpu_baseline"] = cpu_baseline(w120, args.seed, w120.tokens)
        out["decode_120b"] = r120
        wm = wl.WORKLOADS["mtp_draft"]
        rm, lmm = bench_decode(lm, wl, wm, args, torch)
        close_layers(lmm)
        del lmm
        if cpu:
            rm["cpu_baseline"] = cpu_baseline(wm, args.seed, wm.tokens)
        out["mtp_draft"] = rm
        wq = wl.WORKLOADS["145b_q3k_decode"]
        rq, lq = bench_decode(lm, wl, wq, args, torch)
        close_layers(lq)
        del lq
        if cpu:
            rq["cpu_baseline"] = cpu_baseline(wq, args.seed, wq.tokens)
        out["decode_q3k"] = rq
        ws = wl.WORKLOADS["145b_stack"]
        rs, ls = bench_decode(lm, wl, ws, args, torch, steps=args.stack_steps,
                              warmup=min(args.warmup, 3))
        close_layers(ls)
        del ls
        if cpu:
            rs["cpu_baseline"] = cpu_baseline(ws, args.seed, ws.tokens, layers=ws.n_layers)
        out["stack_145b"] = rs
    if not stack and not args.no_extra:
        out["ple_gather"] = bench_ple(lm, args, torch, cpu)
    if not stack and not args.no_extra and not args.no_prefill:
        pre = bench_prefill(lm, wl, wl.WORKLOADS[args.prefill_workload], args, torch)
        if cpu:
            pre["cpu_baseline"] = cpu_baseline(wl.WORKLOADS[args.prefill_workload], args.seed, 8)
        out["prefill"] = pre
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
