"""Parity of the prefill path (T > 8 tokens: MFMA GEMMs over the sorted
assignments) with the fp64 oracle, through the C ABI.

Bit-exact: top-K indices, the group permutation, expert counts and group
offsets, for every token. Within the parity bar: y (relative L2 <= 1e-3,
max-abs <= 1e-2 * rms(y)). The path rounds its activations to fp16 five
times (x, D x, h, the weighted expert outputs, the per-group sums) and the
D/U weights q * d once; each rounding adds about 2e-4 relative error to the
routed part of y (measured 6.4e-4 at the 145B shape, up to 1.2e-3 at the
tiny one), so the routed part is held to 2e-3 and the latent D x (two
roundings) to 1e-3. Softmax weights come from fp64 logits: 1e-6.

At the 145B/120B shapes the oracle routes all tokens (cheap) but runs the
experts only for a sample of tokens: only the experts those tokens route to
are quantized, and y is compared on those tokens."""

import numpy as np
import pytest

import oracle
from cases import Case, assert_close, rel_errors
from latent_mixture_experts_amd import workloads as wl

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

ROUTED_BAR = 2e-3
LATENT_BAR = 1e-3


def make_layer(case, max_tokens):
    from latent_mixture_experts_amd import lmoe
    w = case.w
    layer = lmoe.Layer(w.hidden, w.latent, w.n_experts, w.top_k, w.n_groups, w.expert_ffn,
                       w.shared_ffn, w.du_bits, max_tokens, has_router_bias=w.router_bias)
    layer.load(case.blobs)
    return layer


def run(layer, w, x):
    T = x.shape[0]
    dev = "cuda"
    xg = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    y = torch.empty(T, w.hidden, device=dev, dtype=torch.float32)
    dbg = dict(
        topk_idx=torch.empty(T, w.top_k, dtype=torch.int32, device=dev),
        topk_w=torch.empty(T, w.top_k, dtype=torch.float32, device=dev),
        perm=torch.empty(T * w.top_k, dtype=torch.int32, device=dev),
        expert_count=torch.empty(w.n_experts, dtype=torch.int32, device=dev),
        expert_off=torch.empty(w.n_experts + 1, dtype=torch.int32, device=dev),
        group_off=torch.empty(w.n_groups + 1, dtype=torch.int32, device=dev),
        latent=torch.full((T, w.n_groups, w.latent), float("nan"), device=dev),
    )
    layer.forward(xg, y, debug=dbg)
    torch.cuda.synchronize()
    return y.cpu().numpy(), {k: v.cpu().numpy() for k, v in dbg.items()}


def check_routing(case, dbg, T):
    """idx, w, perm, counts, group offsets of all T tokens against the oracle."""
    lg = case.logits[:T]
    idx, w = oracle.select_topk(lg, case.w.top_k)
    perm, count, goff = oracle.permute(idx, case.blobs["labels"], case.w.n_experts, case.w.n_groups)
    srt = -np.sort(-lg, axis=1)
    gap = srt[:, case.w.top_k - 1] - srt[:, case.w.top_k]
    print("  smallest K-th/K+1-th logit gap %.3g" % gap.min(), flush=True)
    assert np.array_equal(dbg["topk_idx"], idx), "top-K indices differ"
    assert np.array_equal(dbg["perm"], perm), "permutation differs"
    assert np.array_equal(dbg["expert_count"], count)
    assert np.array_equal(dbg["expert_off"], oracle.expert_offsets(count))
    assert np.array_equal(dbg["group_off"], goff)
    assert np.max(np.abs(dbg["topk_w"] - w)) <= 1e-6


def check_outputs(case, got, dbg, tokens):
    r = oracle.layer_forward(case.d, case.blobs, case.x[tokens], dec=case.dec, intermediates=True)
    used = r["used"]
    lat = dbg["latent"][tokens]
    rel_l, _ = rel_errors(lat[used], r["xl"][used])
    rel, mx = assert_close(got[tokens], r["y"], "y")
    rel_r, _ = rel_errors(got[tokens] - r["y_shared"], r["y_routed"])
    print("  %d tokens: y rel L2 %.3g max/rms %.3g; routed part %.3g; latent %.3g" % (
        len(tokens), rel, mx, rel_r, rel_l), flush=True)
    assert rel_l <= LATENT_BAR, "latent relative error %.3g" % rel_l
    assert rel_r <= ROUTED_BAR, "routed part relative error %.3g" % rel_r


# ---------------------------------------------------------------------------
# tiny layer, all tokens checked

@pytest.fixture(scope="module")
def tiny():
    c = Case(wl.WORKLOADS["tiny"], tokens=300)
    return c, make_layer(c, 300)


@pytest.mark.parametrize("T", [9, 64, 130, 300])
def test_tiny_prefill(tiny, T):
    c, layer = tiny
    print("case tiny prefill T", T, flush=True)
    got, dbg = run(layer, c.w, c.x[:T])
    check_routing(c, dbg, T)
    check_outputs(c, got, dbg, np.arange(T))


def test_tiny_prefill_repeatable(tiny):
    c, layer = tiny
    print("case tiny prefill repeat", flush=True)
    a, _ = run(layer, c.w, c.x[:200])
    b, _ = run(layer, c.w, c.x[:200])
    assert np.array_equal(a, b)


def test_tiny_decode_and_prefill_share_a_handle(tiny):
    c, layer = tiny
    for T in (4, 300, 5, 17):
        print("case tiny shared handle T", T, flush=True)
        got, dbg = run(layer, c.w, c.x[:T])
        check_routing(c, dbg, T)
        r = oracle.layer_forward(c.d, c.blobs, c.x[:T], dec=c.dec)
        assert_close(got, r, "y")


def test_tiny_prefill_repeated_token():
    """Every token the same: one expert set takes all T assignments (several
    128-row pieces per expert)."""
    w = wl.WORKLOADS["tiny"]
    x = np.repeat(wl.x(w, 0, 0, tokens=1), 300, axis=0)
    c = Case(w, x=x)
    layer = make_layer(c, 300)
    print("case tiny repeated token T 300", flush=True)
    got, dbg = run(layer, w, x)
    check_routing(c, dbg, 300)
    assert np.sort(dbg["expert_count"])[-w.top_k:].tolist() == [300] * w.top_k
    check_outputs(c, got, dbg, np.array([0, 150, 299]))


def test_tiny_prefill_zero_rows_tie():
    """Zero rows: every logit is exactly 0, the kept experts are 0..K-1."""
    w = wl.WORKLOADS["tiny"]
    x = wl.x(w, 0, 0, tokens=40)
    x[::3] = 0.0
    c = Case(w, x=x)
    layer = make_layer(c, 40)
    print("case tiny zero rows T 40", flush=True)
    got, dbg = run(layer, w, x)
    check_routing(c, dbg, 40)
    assert (dbg["topk_idx"][::3] == np.arange(w.top_k)).all()
    check_outputs(c, got, dbg, np.arange(40))


def test_tiny_prefill_nonfinite_rows():
    """Rows of NaN, +inf and -inf: their logits are not finite, so the
    selection has fewer than K finite values and its threshold falls to
    -inf. Every token must still get K distinct experts in [0, E) (only real
    experts are candidates: the padded logit slots past E are never rescored,
    so no router row past the table is read), and the finite rows keep the
    oracle's routing and outputs."""
    w = wl.WORKLOADS["tiny"]
    T = 40
    x = wl.x(w, 0, 0, tokens=T)
    bad = [3, 7, 11]
    x[3] = np.nan
    x[7] = np.inf
    x[11] = -np.inf
    good = np.setdiff1d(np.arange(T), bad)
    with np.errstate(invalid="ignore"):          # the oracle's logits of the bad rows
        c = Case(w, x=x, pack_tokens=good)
    layer = make_layer(c, T)
    print("case tiny non-finite rows T 40", flush=True)
    got, dbg = run(layer, w, x)
    idx = dbg["topk_idx"]
    for t in range(T):
        row = idx[t].tolist()
        assert len(set(row)) == w.top_k and min(row) >= 0 and max(row) < w.n_experts, (t, row)
    oidx, ow = oracle.select_topk(c.logits[good], w.top_k)
    assert np.array_equal(idx[good], oidx)
    assert np.max(np.abs(dbg["topk_w"][good] - ow)) <= 1e-6
    check_outputs(c, got, dbg, good)


def test_tiny_prefill_block():
    """x += layer(RMSNorm(x)) for T > 8."""
    w = wl.WORKLOADS["tiny"]
    T, eps = 77, 1e-6
    x = wl.x(w, 0, 0, tokens=T) * np.float32(3.0)
    xn = oracle.rmsnorm(x.astype(np.float64), eps)
    c = Case(w, x=xn.astype(np.float32))
    m = wl.masters(w, 0, 0)
    m["expert_ids"] = None
    blobs = oracle.pack_layer(c.d, m)
    c.blobs = blobs
    c.dec = oracle.decode_layer(c.d, blobs)
    layer = make_layer(c, T)
    print("case tiny prefill block T", T, flush=True)
    xg = torch.from_numpy(x.copy()).cuda()
    layer.forward_block(xg, eps)
    torch.cuda.synchronize()
    got = xg.cpu().numpy().astype(np.float64) - x
    want = oracle.layer_forward(c.d, blobs, xn)
    rel, mx = assert_close(got, want, "block update")
    print("  update rel L2 %.3g max/rms %.3g" % (rel, mx), flush=True)


def test_prefill_u_split_along_k():
    """latent 256 and top-8: U has one 256-token tile (far less than a round
    of the chip) and room for 6 partial sums per 128-token half, so it splits
    k four ways (8 of its 32 stages each, across group boundaries), the
    partials added onto the shared down projection already in y; T = 137
    leaves the tile's second half mostly empty. Every token is checked."""
    w = wl.Workload("u_split", 256, 256, 32, 8, 4, 128, 192, 8, 200)
    c = Case(w, seed=11, tokens=200)
    layer = make_layer(c, 200)
    for T in (200, 137):
        print("case u_split prefill T", T, flush=True)
        got, dbg = run(layer, w, c.x[:T])
        check_routing(c, dbg, T)
        check_outputs(c, got, dbg, np.arange(T))


def test_prefill_expert_piece_classes():
    """A skewed router (per-expert bias) over 32 experts: expert loads from 0
    to 596 tokens, so the expert GEMMs get full 128-token pieces, partial
    pieces of more than 64 tokens, of 33 to 64 and of at most 32 tokens, each
    class on its own kernel path. Latent 512 and expert ffn 160 give 8 down
    tiles and 5 gate/up tiles (the 8-wave narrow-piece workgroup with three
    waves past the last tile) and a K-ragged second FP4 stage (32 of 128
    columns) in the resident down projection. Every token is checked."""
    w = wl.Workload("classes", 256, 512, 32, 4, 4, 160, 64, 8, 700, router_bias=True)
    c = Case(w, seed=3, tokens=700)
    layer = make_layer(c, 700)
    for T in (700, 333):
        print("case classes prefill T", T, flush=True)
        got, dbg = run(layer, w, c.x[:T])
        check_routing(c, dbg, T)
        cnt = dbg["expert_count"]
        rem = cnt % 128
        assert (cnt >= 128).any() and (rem > 64).any()
        assert ((rem > 32) & (rem <= 64)).any() and ((rem > 0) & (rem <= 32)).any()
        check_outputs(c, got, dbg, np.arange(T))


def test_prefill_wide_expert_ffn():
    """Expert ffn 1056: the down projection's K is past what the LDS holds
    resident, so it runs on the staged 128-token and narrow-piece kernels; K
    ends 32 columns into its ninth FP4 stage. Skewed router, every piece
    class present, every token checked."""
    w = wl.Workload("wide_ffn", 256, 256, 16, 4, 2, 1056, 64, 8, 400, router_bias=True)
    c = Case(w, seed=4, tokens=400)
    layer = make_layer(c, 400)
    print("case wide_ffn prefill T 400", flush=True)
    got, dbg = run(layer, w, c.x)
    check_routing(c, dbg, 400)
    cnt = dbg["expert_count"]
    rem = cnt % 128
    assert (cnt >= 128).any() and (rem > 64).any()
    assert ((rem > 32) & (rem <= 64)).any() and ((rem > 0) & (rem <= 32)).any()
    check_outputs(c, got, dbg, np.arange(400))


def test_prefill_latent_not_multiple_of_128():
    """Latent 192 (Q8 D/U): the expert gate/up's K is not a multiple of the
    128-column FP4 stage, so its pieces of more than 64 tokens run on the
    register-staged k_grouped (the DMA-fed kernel needs whole stages) and its
    last stage is half real columns; the down projection (K = 96) is ragged
    in the resident kernel. Skewed router, every piece class present, every
    token checked."""
    w = wl.Workload("latent192", 256, 192, 16, 4, 2, 96, 64, 8, 300, router_bias=True)
    c = Case(w, seed=4, tokens=300)
    layer = make_layer(c, 300)
    print("case latent192 prefill T 300", flush=True)
    got, dbg = run(layer, w, c.x)
    check_routing(c, dbg, 300)
    cnt = dbg["expert_count"]
    rem = cnt % 128
    assert (cnt >= 128).any() and (rem > 64).any()
    assert ((rem > 32) & (rem <= 64)).any() and ((rem > 0) & (rem <= 32)).any()
    check_outputs(c, got, dbg, np.arange(300))


def test_prefill_shared_ffn_not_multiple_of_64():
    """Shared ffn 96: the shared down projection's K is not a multiple of the
    64-column unit the DMA-fed dense GEMM splits by, so U + shared down runs
    on the register-staged k_dense (its other users always qualify). Every
    token checked."""
    w = wl.Workload("shared96", 256, 128, 16, 2, 2, 64, 96, 8, 200)
    c = Case(w, seed=5, tokens=200)
    layer = make_layer(c, 200)
    for T in (200, 77):
        print("case shared96 prefill T", T, flush=True)
        got, dbg = run(layer, w, c.x[:T])
        check_routing(c, dbg, T)
        check_outputs(c, got, dbg, np.arange(T))


# expert loads on both sides of every piece-class boundary (pieces of 32 /
# 33, 64 / 65 tokens; a whole 128-token piece; 128 + 1) plus idle experts
BOUNDARY_COUNTS = [32, 33, 64, 65, 128, 129, 1, 0, 127, 96, 31, 63, 0, 2, 97, 30]


@pytest.mark.parametrize("latent,ffn", [(128, 64), (512, 160)])
def test_prefill_piece_class_boundaries(latent, ffn):
    """Exact expert loads by construction: the router is the identity on the
    first 16 hidden dimensions and token t's row carries 4 and 3.9 on its two
    experts (small noise elsewhere), so top-2 picks them with a wide margin;
    the sorted assignment list, split in halves, gives every token two
    distinct experts. Latent 128 / ffn 64 runs the narrow-piece kernels with
    4 waves, latent 512 / ffn 160 with 8 (three of them past the last gate/up
    tile). Every token checked."""
    T = sum(BOUNDARY_COUNTS) // 2
    w = wl.Workload("bounds", 256, latent, 16, 2, 2, ffn, 64, 8, T)
    m = wl.masters(w, seed=6)
    r = np.zeros((16, 256), np.float32)
    r[np.arange(16), np.arange(16)] = 1.0
    m["router"] = r
    lst = np.repeat(np.arange(16), BOUNDARY_COUNTS)
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((T, 256)) * 0.05).astype(np.float32)
    x[np.arange(T), lst[:T]] += 4.0
    x[np.arange(T), lst[T:]] += 3.9
    c = Case(w, x=x, masters=m, tokens=T)
    layer = make_layer(c, T)
    print("case bounds latent %d ffn %d prefill T %d" % (latent, ffn, T), flush=True)
    got, dbg = run(layer, w, c.x)
    check_routing(c, dbg, T)
    assert dbg["expert_count"].tolist() == BOUNDARY_COUNTS
    check_outputs(c, got, dbg, np.arange(T))


# ---------------------------------------------------------------------------
# 145B / 120B shapes, routing over all tokens, outputs on a sample

def piece_class_tokens(idx, labels, E, G, T, n_total, seed=1234):
    """Tokens whose assignments land on every piece class of the grouped
    GEMMs (an expert's assignments are cut into pieces of 128 in sorted
    order; the last piece has 1..128): the last and the first assignment of
    the largest expert, the last assignment of an expert whose last piece
    holds 65..127, 33..64 and 1..32, the last token of the batch and one in
    its last 64-token chunk; then seeded random tokens up to n_total."""
    perm, count, goff = oracle.permute(idx, labels, E, G)
    K = idx.shape[1]
    lab = np.asarray(labels, np.int64)
    order = np.lexsort((np.arange(E), lab))           # (label, expert) order of the segments
    start = np.concatenate([[0], np.cumsum(count[order])])[:-1]
    seg = {int(e): int(s0) for e, s0 in zip(order, start)}
    picks = []
    big = int(np.argmax(count))
    picks += [int(perm[seg[big] + count[big] - 1]) // K, int(perm[seg[big]]) // K]
    last = np.where(count > 0, count - 128 * ((count - 1) // 128), 0)
    for lo, hi in ((65, 127), (33, 64), (1, 32)):
        es = np.where((last >= lo) & (last <= hi))[0]
        if len(es):
            e = int(es[0])
            picks.append(int(perm[seg[e] + count[e] - 1]) // K)
    picks += [T - 1, T - 1 - int(np.random.default_rng(seed).integers(1, min(64, T)))]
    rng = np.random.default_rng(seed)
    tokens = set(picks)
    while len(tokens) < n_total:
        tokens.add(int(rng.integers(0, T)))
    return np.array(sorted(tokens))


def _sampled(name, T, n_sample, seed=0, all_groups_d=False):
    w = wl.WORKLOADS[name]
    pre = Case(w, seed=seed, tokens=T, pack_tokens=[0])          # routing of every token
    labels = np.asarray(pre.blobs["labels"])
    tokens = piece_class_tokens(pre.idx, labels, w.n_experts, w.n_groups, T, n_sample)
    print("case %s prefill T %d, packing experts of tokens %s" % (name, T, tokens.tolist()),
          flush=True)
    c = Case(w, seed=seed, tokens=T, pack_tokens=tokens)
    layer = make_layer(c, T)
    if all_groups_d:
        layer.set_prefill_d(0)
    got, dbg = run(layer, w, c.x)
    check_routing(c, dbg, T)
    check_outputs(c, got, dbg, tokens)
    layer.close()


def test_145b_prefill_4096():
    _sampled("145b_prefill", 4096, 16)


def test_120b_prefill_q4():
    _sampled("120b_decode", 600, 16)


# ---------------------------------------------------------------------------
# D over all groups of every token (lmoe_set_prefill_d(h, 0)); the default,
# D over the routed (token, group) pairs, runs in every other prefill test

def test_145b_prefill_4096_all_groups_d():
    _sampled("145b_prefill", 4096, 16, all_groups_d=True)


@pytest.mark.parametrize("T", [9, 64, 300])
def test_tiny_prefill_all_groups_d(tiny, T):
    c, layer = tiny
    layer.set_prefill_d(0)
    try:
        print("case tiny prefill all-groups D T", T, flush=True)
        got, dbg = run(layer, c.w, c.x[:T])
        check_routing(c, dbg, T)
        check_outputs(c, got, dbg, np.arange(T))
    finally:
        layer.set_prefill_d(1)


def test_prefill_routed_d_skewed_groups():
    """A skewed router over 32 experts in 4 groups (some groups draw most of
    the 700 tokens, their lists span several 256-token tiles; others few):
    every token checked, the routed and the all-groups D agree on y."""
    w = wl.Workload("classes", 256, 512, 32, 4, 4, 160, 64, 8, 700, router_bias=True)
    c = Case(w, seed=3, tokens=700)
    layer = make_layer(c, 700)
    print("case skewed groups prefill routed D T 700", flush=True)
    layer.set_prefill_d(0)
    dense, _ = run(layer, w, c.x)
    layer.set_prefill_d(1)
    got, dbg = run(layer, w, c.x)
    check_routing(c, dbg, 700)
    check_outputs(c, got, dbg, np.arange(700))
    rel, _ = rel_errors(got, dense)
    assert rel <= 1e-6, rel


def test_set_prefill_d_rejects_bad_values(tiny):
    from latent_mixture_experts_amd import lmoe
    c, layer = tiny
    with pytest.raises(lmoe.LmoeError):
        layer.set_prefill_d(2)


@pytest.mark.parametrize("name", ["tiny", "145b_decode"])
def test_prefill_activation_range(name):
    """Prefill rows far from unit scale: x scaled by 1e-3, 1e2, 3e3, 1e-9 and
    1e4, and a row of elements around 1e-6 with every seventh element near
    1e5 (fp16 alone would lose the first rows to subnormals and overflow on
    the last ones). Each token's fp16 activations carry an exact power-of-two
    scale, so each token meets the bar on its own, and its latent D x too."""
    w = wl.WORKLOADS[name]
    T = 16
    x = wl.x(w, 12, tokens=T)
    for t, f in ((0, 1e-3), (1, 1e2), (2, 1e-6), (3, 3e3), (4, 1e-9), (5, 1e4),
                 (8, 1e-3), (9, 1e2), (10, 1e-6), (11, 3e3), (12, 1e-9), (13, 1e4)):
        x[t] *= np.float32(f)
    x[2, ::7] *= np.float32(1e11)
    x[10, ::7] *= np.float32(1e11)
    c = Case(w, seed=12, x=x)
    layer = make_layer(c, T)
    print("case %s prefill activation range T %d" % (name, T), flush=True)
    got, dbg = run(layer, w, x)
    check_routing(c, dbg, T)
    r = oracle.layer_forward(c.d, c.blobs, x, dec=c.dec, intermediates=True)
    for t in range(T):
        rel, mx = assert_close(got[t], r["y"][t], "token %d" % t)
        rel_r, _ = rel_errors(got[t] - r["y_shared"][t], r["y_routed"][t])
        u = r["used"][t]
        rel_l, _ = rel_errors(dbg["latent"][t][u], r["xl"][t][u])
        print("  token %d (max |x| %.3g): y rel L2 %.3g max/rms %.3g; routed part %.3g; latent %.3g" % (
            t, float(np.max(np.abs(x[t]))), rel, mx, rel_r, rel_l), flush=True)
        assert rel_r <= ROUTED_BAR, "token %d routed part relative error %.3g" % (t, rel_r)
        assert rel_l <= LATENT_BAR, "token %d latent relative error %.3g" % (t, rel_l)
