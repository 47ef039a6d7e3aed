"""Plant plausible mistakes in the oracle (CPU only) and check that the pins
catch each one: a pin that passes a broken oracle pins nothing."""

import numpy as np
import pytest
import torch

from oracle import formats as fm
from oracle import layer as ol

from test_oracle_layer import (SMALL, _brute_layer, _identity_layer, _masters, _x,
                               stack_closed_form_holds)

_ORIG = {"select_topk": ol.select_topk, "unpack_expert_record": fm.unpack_expert_record,
         "e4m3_decode": fm.e4m3_decode, "unpack_nibbles": fm.unpack_nibbles}


def _swap_gate_up(rec, ell, ff):
    g, u, dn = _ORIG["unpack_expert_record"](rec, ell, ff)
    return u, g, dn


def _transpose_down(rec, ell, ff):
    g, u, dn = _ORIG["unpack_expert_record"](rec, ell, ff)
    return g, u, dn * 0 + dn[::-1]          # rows reversed: a wrong index map


def _unrenormalized_topk(lg, k):
    idx, _ = _ORIG["select_topk"](lg, k)
    full = np.exp(lg - lg.max(axis=1, keepdims=True))
    full /= full.sum(axis=1, keepdims=True)
    return idx, np.take_along_axis(full, idx.astype(np.int64), axis=1)


def _reversed_topk(lg, k):
    idx, w = _ORIG["select_topk"](lg, k)
    return idx[:, ::-1].copy(), w[:, ::-1].copy()


def _lowest_topk(lg, k):
    return _ORIG["select_topk"](-lg, k)


LAYER_MUTATIONS = {
    "silu sign": (ol, "silu", lambda v: v / (1.0 + np.exp(v))),
    "gate/up swapped": (fm, "unpack_expert_record", _swap_gate_up),
    "down rows permuted": (fm, "unpack_expert_record", _transpose_down),
    "softmax over all experts, not renormalized": (ol, "select_topk", _unrenormalized_topk),
    "top-k order reversed": (ol, "select_topk", _reversed_topk),
    "lowest logits kept": (ol, "select_topk", _lowest_topk),
}


def _case(seed=0):
    blobs = ol.pack_layer(SMALL, _masters(SMALL, seed=seed))
    x = _x(SMALL, 3)
    want, idx = _brute_layer(SMALL, blobs, x)
    return blobs, x, want, idx


def _agrees(blobs, x, want, idx):
    got = ol.layer_forward(SMALL, blobs, x, intermediates=True)
    return np.array_equal(got["idx"], idx) and \
        np.max(np.abs(got["y"] - want)) <= 1e-12 * np.max(np.abs(want))


def test_unmutated_oracle_agrees():
    assert _agrees(*_case())


@pytest.mark.parametrize("name", sorted(LAYER_MUTATIONS))
def test_layer_mutation_is_caught(name, monkeypatch):
    case = _case()                       # brute force taken before the plant
    mod, attr, repl = LAYER_MUTATIONS[name]
    monkeypatch.setattr(mod, attr, repl)
    assert not _agrees(*case)


def test_group_label_mistake_is_caught(monkeypatch):
    blobs, x, want, idx = _case()
    wrong = dict(blobs)
    wrong["labels"] = (np.asarray(blobs["labels"]) + 1) % SMALL.n_groups
    got = ol.layer_forward(SMALL, wrong, x)
    assert np.max(np.abs(got - want)) > 1e-6 * np.max(np.abs(want))


def test_dropped_shared_expert_is_caught():
    blobs, x, want, idx = _case()
    r = ol.layer_forward(SMALL, blobs, x, intermediates=True)
    assert np.max(np.abs(r["y_routed"] - want)) > 1e-6 * np.max(np.abs(want))


def test_e4m3_mistake_caught_by_library_pin(monkeypatch):
    monkeypatch.setattr(fm, "e4m3_decode", lambda b: _ORIG["e4m3_decode"](b) * 2.0)
    b = np.arange(0x7F, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).double().numpy()
    assert not np.array_equal(fm.e4m3_decode(b), ref)


def test_nibble_order_mistake_caught_by_byte_pin(monkeypatch):
    """A swap applied on both pack and unpack survives a round trip; the pin
    that byte 0 holds element 0 in its low nibble must catch it."""
    def swapped_pack(c):
        c = np.asarray(c, dtype=np.uint8)
        return (c[..., 1::2] & 0xF) | ((c[..., 0::2] & 0xF) << 4)
    monkeypatch.setattr(fm, "pack_nibbles", swapped_pack)
    w = (np.arange(64, dtype=np.float32).reshape(2, 32) - 31.5) / 32.0
    w[0, 1] = 0.5                       # distinct codes in the first byte
    blob = fm.pack_du(w, 4)
    codes, _ = fm.quantize_blocks(w, 4)
    assert blob[0] != (codes[0, 0] | (codes[0, 1] << 4))


def _post_norm_stack(dims, layers, x, eps=1e-6):
    xd = np.asarray(x, dtype=np.float64)
    for blobs in layers:
        xd = ol.rmsnorm(xd + ol.layer_forward(dims, blobs, xd), eps)
    return xd


def _no_residual_stack(dims, layers, x, eps=1e-6):
    xd = np.asarray(x, dtype=np.float64)
    for blobs in layers:
        xd = ol.layer_forward(dims, blobs, ol.rmsnorm(xd, eps))
    return xd


STACK_MUTATIONS = {
    "post-norm instead of pre-norm": (ol, "stack_forward", _post_norm_stack),
    "residual dropped": (ol, "stack_forward", _no_residual_stack),
    "rmsnorm without eps": (ol, "rmsnorm", lambda v, eps=1e-6: np.asarray(v, np.float64) / np.sqrt(
        np.mean(np.asarray(v, np.float64) ** 2, axis=-1, keepdims=True))),
    "rmsnorm without the square root": (ol, "rmsnorm", lambda v, eps=1e-6: np.asarray(v, np.float64) / (
        np.mean(np.asarray(v, np.float64) ** 2, axis=-1, keepdims=True) + eps)),
    "rmsnorm over the sum, not the mean": (ol, "rmsnorm", lambda v, eps=1e-6: np.asarray(v, np.float64) / np.sqrt(
        np.sum(np.asarray(v, np.float64) ** 2, axis=-1, keepdims=True) + eps)),
}


def test_unmutated_stack_pin_holds(monkeypatch):
    monkeypatch.setattr(ol, "layer_forward", _identity_layer)
    assert stack_closed_form_holds()


@pytest.mark.parametrize("name", sorted(STACK_MUTATIONS))
def test_stack_mutation_is_caught(name, monkeypatch):
    monkeypatch.setattr(ol, "layer_forward", _identity_layer)
    mod, attr, repl = STACK_MUTATIONS[name]
    monkeypatch.setattr(mod, attr, repl)
    assert not stack_closed_form_holds()
