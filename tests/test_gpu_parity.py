"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Bit-exact: top-K indices, the group permutation, expert counts and group
offsets. Within the parity bar: y (relative L2 <= 1e-3 and max-abs <=
1e-2 * rms(y)); routing weights and latents are held to a far tighter bound
because the path computes in fp32 / fp64 throughout."""

import sys

import numpy as np
import pytest

from cases import Case, assert_close, rel_errors
from latent_mixture_experts_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _lmoe():
    from latent_mixture_experts_amd import lmoe
    return lmoe


def make_layer(case, max_tokens=8):
    lm = _lmoe()
    w = case.w
    layer = lm.Layer(w.hidden, w.latent, w.n_experts, w.top_k, w.n_groups, w.expert_ffn,
                     w.shared_ffn, w.du_bits, max_tokens, has_router_bias=w.router_bias,
                     expert_format=w.expert_format)
    layer.load(case.blobs)
    return layer


def run(layer, case, T):
    w = case.w
    dev = "cuda"
    x = torch.from_numpy(np.ascontiguousarray(case.x[:T])).to(dev)
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
    layer.forward(x, y, debug=dbg)
    torch.cuda.synchronize()
    return y.cpu().numpy(), {k: v.cpu().numpy() for k, v in dbg.items()}


def check(case, layer, T, label):
    print("case", label, "T", T, flush=True)
    got, dbg = run(layer, case, T)
    r = case.expect(T)
    assert np.array_equal(dbg["topk_idx"], r["idx"]), "top-K indices differ"
    assert np.array_equal(dbg["perm"], r["perm"]), "permutation differs"
    assert np.array_equal(dbg["expert_count"], r["expert_count"])
    assert np.array_equal(dbg["expert_off"], r["expert_off"])
    assert np.array_equal(dbg["group_off"], r["group_off"])
    assert np.max(np.abs(dbg["topk_w"] - r["w"])) <= 1e-6
    used = r["used"]
    rel, _ = rel_errors(dbg["latent"][used], r["xl"][used])
    assert rel <= 1e-5, "latent D x relative error %.3g" % rel
    rel, mx = assert_close(got, r["y"], "y")
    rel_r, _ = rel_errors(got - r["y_shared"], r["y_routed"])
    print("  y rel L2 %.3g max/rms %.3g; routed part rel L2 %.3g" % (rel, mx, rel_r), flush=True)
    assert rel_r <= 1e-4, "routed part relative error %.3g" % rel_r
    return got


# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def tiny():
    c = Case(wl.WORKLOADS["tiny"], tokens=8)
    return c, make_layer(c)


@pytest.mark.parametrize("T", range(1, 9))
def test_tiny_all_token_counts(tiny, T):
    case, layer = tiny
    check(case, layer, T, "tiny")


def test_tiny_repeatable_bitwise(tiny):
    case, layer = tiny
    a, da = run(layer, case, 4)
    b, db = run(layer, case, 4)
    assert np.array_equal(a, b) and all(np.array_equal(da[k], db[k]) for k in da if k != "latent")


@pytest.fixture(scope="module")
def l145():
    c = Case(wl.WORKLOADS["145b_decode"], tokens=8)
    return c, make_layer(c)


@pytest.mark.parametrize("T", [4, 1, 5, 8])
def test_145b_decode(l145, T):
    case, layer = l145
    check(case, layer, T, "145b_decode")


@pytest.fixture(scope="module")
def l120():
    c = Case(wl.WORKLOADS["120b_decode"], tokens=8)
    return c, make_layer(c)


@pytest.mark.parametrize("T", [5, 2, 7])
def test_120b_decode(l120, T):
    case, layer = l120
    check(case, layer, T, "120b_decode")


@pytest.fixture(scope="module")
def lmtp():
    c = Case(wl.WORKLOADS["mtp_draft"], tokens=4)
    return c, make_layer(c, 4)


@pytest.mark.parametrize("T", [1, 4])
def test_mtp_draft_layer(lmtp, T):
    """The draft layer's MoE (512 experts of 3 x 1280 x 640, Q8 D/U): one
    drafted token, and the four tokens of a verify window."""
    case, layer = lmtp
    check(case, layer, T, "mtp_draft")


# ---------------------------------------------------------------------------
# Q3_K gate/up + IQ4_NL down expert records (decode path)

Q3K_TINY = wl.Workload("q3k_tiny", 256, 256, 16, 2, 2, 64, 64, 8, 8, labels_mod=True,
                       expert_format=1)


@pytest.fixture(scope="module")
def q3k_tiny():
    c = Case(Q3K_TINY, tokens=8)
    return c, make_layer(c)


@pytest.mark.parametrize("T", range(1, 9))
def test_q3k_tiny_all_token_counts(q3k_tiny, T):
    case, layer = q3k_tiny
    check(case, layer, T, "q3k tiny")


@pytest.fixture(scope="module")
def l145q3k():
    c = Case(wl.WORKLOADS["145b_q3k_decode"], tokens=8)
    return c, make_layer(c)


@pytest.mark.parametrize("T", [4, 1, 8])
def test_145b_q3k_decode(l145q3k, T):
    case, layer = l145q3k
    check(case, layer, T, "145b q3k")


def test_120b_q3k_decode():
    """The 120B shapes (latent 1280, Q4 D/U) with Q3_K records: 1,164,800
    bytes an expert, as the model page prints."""
    w = wl.Workload("120b_q3k", 2560, 1280, 512, 10, 8, 640, 640, 4, 5, expert_format=1)
    c = Case(w, tokens=5)
    assert c.blobs["experts"].shape[1] == 1164800
    layer = make_layer(c, 5)
    check(c, layer, 5, "120b q3k")


def test_q3k_batches_above_8_tokens():
    """Q3_K records, T = 20 and 12: the batch runs as decode forwards of 8
    tokens each; every token's routing, weights, latent and output against
    the oracle, and the whole-batch debug outputs refused."""
    from latent_mixture_experts_amd import lmoe
    c = Case(Q3K_TINY, seed=5, tokens=20)
    layer = make_layer(c, 20)
    for T in (20, 12):
        print("case q3k tiny chunked T", T, flush=True)
        dev = "cuda"
        x = torch.from_numpy(np.ascontiguousarray(c.x[:T])).to(dev)
        y = torch.empty(T, c.w.hidden, device=dev)
        dbg = dict(topk_idx=torch.empty(T, c.w.top_k, dtype=torch.int32, device=dev),
                   topk_w=torch.empty(T, c.w.top_k, dtype=torch.float32, device=dev),
                   latent=torch.full((T, c.w.n_groups, c.w.latent), float("nan"), device=dev))
        layer.forward(x, y, debug=dbg)
        torch.cuda.synchronize()
        r = c.expect(T)
        assert np.array_equal(dbg["topk_idx"].cpu().numpy(), r["idx"])
        assert np.max(np.abs(dbg["topk_w"].cpu().numpy() - r["w"])) <= 1e-6
        used = r["used"]
        rel, _ = rel_errors(dbg["latent"].cpu().numpy()[used], r["xl"][used])
        assert rel <= 1e-5, rel
        got = y.cpu().numpy()
        assert_close(got, r["y"], "y")
        rel_r, _ = rel_errors(got - r["y_shared"], r["y_routed"])
        assert rel_r <= 1e-4, rel_r
    with pytest.raises(lmoe.LmoeError):
        layer.forward(x, y, debug=dict(perm=torch.empty(12 * c.w.top_k, dtype=torch.int32, device="cuda")))
    layer.close()


def test_q3k_decode_activation_range():
    """Rows at 1e-3, 1e2, 1e-6 with every seventh element near 1e5, and 3e3
    through the Q3_K / IQ4_NL decoders (the token scales are undone on the
    super-step's chain and on each 32-column block)."""
    x = wl.x(Q3K_TINY, 11, tokens=5)
    x[0] *= 1e-3
    x[1] *= 1e2
    x[2] *= 1e-6
    x[2, ::7] = x[2, ::7] * 1e11
    x[4] *= 3e3
    c = Case(Q3K_TINY, seed=11, x=x)
    layer = make_layer(c)
    got, dbg = run(layer, c, 5)
    r = c.expect(5)
    r["x"] = x
    assert np.array_equal(dbg["topk_idx"], r["idx"])
    _per_token_close(got, r, "q3k tiny")


def test_same_token_repeated_shares_experts():
    """All tokens identical: every routed expert serves T tokens at once."""
    w = wl.WORKLOADS["tiny"]
    x = np.repeat(wl.x(w, 3, tokens=1), 8, axis=0)
    c = Case(w, seed=3, x=x)
    layer = make_layer(c)
    check(c, layer, 8, "tiny repeated token")


def test_exact_ties_break_to_lower_index():
    """Integer-valued x and router rows make every logit an exact integer, so
    ties are exact on both sides; the lower expert index must win."""
    w = wl.WORKLOADS["tiny"]
    m = wl.masters(w, seed=5)
    rng = np.random.default_rng(5)
    m["router"] = rng.integers(-1, 2, (w.n_experts, w.hidden)).astype(np.float32)
    m["router"][8:] = m["router"][:8]                  # duplicate rows: exact ties
    x = rng.integers(-1, 2, (6, w.hidden)).astype(np.float32)
    x[5] = 0.0                                         # all logits tie at zero
    c = Case(w, seed=5, x=x, masters=m)
    layer = make_layer(c)
    check(c, layer, 6, "tiny exact ties")


def test_145b_zero_rows_all_logits_tie():
    """Zero token rows at the 145B shape: all 512 logits are exactly 0, more
    candidates than one wavefront ranks at once; experts 0..K-1 must win."""
    w = wl.WORKLOADS["145b_decode"]
    x = wl.x(w, 0, tokens=4)
    x[1] = 0.0
    x[3] = 0.0
    c = Case(w, x=x)
    layer = make_layer(c, max_tokens=4)
    _, dbg = run(layer, c, 4)
    assert (dbg["topk_idx"][1] == np.arange(w.top_k)).all()
    assert (dbg["topk_idx"][3] == np.arange(w.top_k)).all()
    check(c, layer, 4, "145b zero rows")


def test_wide_ffn_many_picks():
    """expert_ffn 4096 and top-16 at T = 8: 128 assignments (ranked, not the
    one-wavefront sort), sixteen down super-steps per slot, and a group's
    weighted outputs that leave the down phase too little LDS for one
    wavefront per super-step, so some wavefronts take two in turn."""
    w = wl.Workload("wide_ffn", 256, 128, 32, 16, 2, 4096, 64, 8, 8)
    c = Case(w, seed=7)
    layer = make_layer(c)
    for T in (8, 3):
        check(c, layer, T, "wide ffn T=%d" % T)


def test_argument_errors_on_device():
    lm = _lmoe()
    c = Case(wl.WORKLOADS["tiny"], tokens=4)
    layer = make_layer(c, max_tokens=4)
    x = torch.zeros(8, 256, device="cuda")
    y = torch.zeros(8, 256, device="cuda")
    with pytest.raises(lm.LmoeError) as e:
        layer.forward(x, y, T=5)
    assert e.value.code == lm.EINVAL
    with pytest.raises(lm.LmoeError) as e:
        layer.forward(x, y, T=0)
    assert e.value.code == lm.EINVAL
    with pytest.raises(lm.LmoeError) as e:
        layer.forward(x, x, T=2)
    assert e.value.code == lm.EINVAL
    fresh = lm.Layer(256, 128, 16, 2, 2, 64, 64, 8, 4)
    with pytest.raises(lm.LmoeError) as e:
        fresh.forward(x, y, T=1)
    assert e.value.code == lm.ESTATE
    bad = dict(c.blobs)
    bad["labels"] = np.full(16, 2, np.uint8)
    with pytest.raises(lm.LmoeError) as e:
        fresh.load(bad)
    assert e.value.code == lm.EINVAL


def test_run_phase_repeats_the_forward():
    """Each decode phase run alone after a forward (the profiling hook) reads
    and writes the same workspace state: rerunning phases 1..4 in order gives
    y bit for bit; a phase before any forward of that T is refused."""
    lm = _lmoe()
    w = wl.WORKLOADS["145b_decode"]
    c = Case(w, tokens=4)
    layer = make_layer(c, max_tokens=8)
    x = torch.from_numpy(np.ascontiguousarray(c.x[:4])).cuda()
    y = torch.empty(4, w.hidden, device="cuda")
    with pytest.raises(lm.LmoeError) as e:
        layer.run_phase(x, y, 1)
    assert e.value.code == lm.ESTATE
    layer.forward(x, y)
    torch.cuda.synchronize()
    want = y.cpu().numpy().copy()
    for _ in range(2):
        y.zero_()
        for k in (1, 2, 3, 4):
            layer.run_phase(x, y, k)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy(), want)
    for k in (0, 5):
        with pytest.raises(lm.LmoeError) as e:
            layer.run_phase(x, y, k)
        assert e.value.code == lm.EINVAL
    with pytest.raises(lm.LmoeError) as e:
        layer.run_phase(x[:2], y[:2], 1)               # last forward was of 4 tokens
    assert e.value.code == lm.ESTATE


def _per_token_close(got, r, what):
    """The bar per token: rows of very different magnitude each meet it."""
    for t in range(got.shape[0]):
        rel, mx = assert_close(got[t], r["y"][t], "%s token %d" % (what, t))
        rel_r, _ = rel_errors(got[t] - r["y_shared"][t], r["y_routed"][t])
        print("  token %d (max |x| %.3g): y rel L2 %.3g max/rms %.3g; routed part %.3g" % (
            t, float(np.max(np.abs(r["x"][t]))), rel, mx, rel_r), flush=True)
        assert rel_r <= 1e-4, "token %d routed part relative error %.3g" % (t, rel_r)


@pytest.mark.parametrize("name", ["tiny", "145b_decode"])
def test_decode_activation_range(name):
    """Token rows far from unit scale: x scaled by 1e-3 and by 1e2, a row of
    elements around 1e-6 with every seventh element near 1e5, and a row at
    3e3. The fp16 staging of every activation is scaled per token by a power
    of two, so each token meets the bar on its own."""
    w = wl.WORKLOADS[name]
    x = wl.x(w, 11, tokens=5)
    x[0] *= 1e-3
    x[1] *= 1e2
    x[2] *= 1e-6
    x[2, ::7] = x[2, ::7] * 1e11
    x[4] *= 3e3
    c = Case(w, seed=11, x=x)
    layer = make_layer(c)
    got, dbg = run(layer, c, 5)
    r = c.expect(5)
    r["x"] = x
    assert np.array_equal(dbg["topk_idx"], r["idx"])
    assert np.array_equal(dbg["perm"], r["perm"])
    _per_token_close(got, r, name)
