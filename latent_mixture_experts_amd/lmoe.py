"""ctypes binding of liblmoe.so (C ABI in include/lmoe.h).

Argument marshalling only: every step of the layer runs in the HIP library.
Tensors are torch tensors (device memory and streams come from PyTorch);
host-side packed weights may be numpy arrays or CPU tensors. There is no
fallback: if the library is missing, importing this module raises.
"""

import ctypes
import os

import numpy as np

# PyTorch ships its own copy of the HIP runtime under the same soname as
# /opt/rocm's. Importing it first makes liblmoe.so bind to that copy, so the
# library and PyTorch share one runtime (one device context, one set of
# streams and allocations).
import torch  # noqa: F401

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblmoe.so")

OK, EINVAL, ENOMEM, EHIP, ESTATE, EUNSUPPORTED = 0, -1, -2, -3, -4, -5


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "hidden", "latent", "n_experts", "top_k", "n_groups", "expert_ffn", "shared_ffn",
        "du_bits", "max_tokens", "has_router_bias", "expert_format")]

EXPERTS_NVFP4, EXPERTS_Q3K = 0, 1


class Weights(ctypes.Structure):
    _fields_ = [
        ("router_bf16", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
        ("group_labels", ctypes.c_void_p),
        ("d_blob", ctypes.c_void_p), ("d_bytes", ctypes.c_size_t),
        ("u_blob", ctypes.c_void_p), ("u_bytes", ctypes.c_size_t),
        ("experts", ctypes.c_void_p), ("expert_record_bytes", ctypes.c_size_t),
        ("shared_gate_bf16", ctypes.c_void_p), ("shared_up_bf16", ctypes.c_void_p),
        ("shared_down_bf16", ctypes.c_void_p),
    ]


class Debug(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "topk_idx", "topk_w", "perm", "expert_count", "expert_off", "group_off", "latent")]


class LmoeError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        super().__init__("%s failed: %s (%d): %s" % (where, _lib.lmoe_strerror(code).decode(), code,
                                                     _lib.lmoe_last_error().decode()))


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("liblmoe.so is not built (run __graft_entry__.build() or "
                          "python latent_mixture_experts_amd/build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "lmoe_create": (ctypes.c_int, [ctypes.POINTER(Dims), ctypes.c_int, ctypes.POINTER(vp)]),
        "lmoe_load_weights": (ctypes.c_int, [vp, ctypes.POINTER(Weights), vp]),
        "lmoe_forward": (ctypes.c_int, [vp, vp, i32, vp, ctypes.POINTER(Debug), vp]),
        "lmoe_forward_block": (ctypes.c_int, [vp, vp, i32, ctypes.c_float, vp]),
        "lmoe_forward_noalloc": (ctypes.c_int, [vp, vp, i32, vp, vp]),
        "lmoe_destroy": (None, [vp]),
        "lmoe_set_phase_events": (ctypes.c_int, [vp, ctypes.POINTER(vp), i32]),
        "lmoe_phase_count": (i32, [i32]),
        "lmoe_run_phase": (ctypes.c_int, [vp, vp, i32, i32, vp, vp]),
        "lmoe_strerror": (ctypes.c_char_p, [ctypes.c_int]),
        "lmoe_last_error": (ctypes.c_char_p, []),
        "lmoe_expert_record_bytes": (sz, [i32, i32]),
        "lmoe_du_matrix_bytes": (sz, [i32, i32, i32]),
        "lmoe_pack_bf16": (ctypes.c_int, [vp, sz, vp, vp]),
        "lmoe_pack_blocks": (ctypes.c_int, [vp, i32, i32, i32, vp, vp]),
        "lmoe_pack_expert_records": (ctypes.c_int, [vp, vp, vp, i32, i32, i32, vp, vp]),
        "lmoe_ple_gather": (ctypes.c_int, [vp, i32, vp, vp, i32, vp, vp]),
        "lmoe_expert_record_bytes_fmt": (sz, [i32, i32, i32]),
        "lmoe_set_prefill_d": (ctypes.c_int, [vp, i32]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()


def lib():
    return _lib


def _check(rc, where):
    if rc != OK:
        raise LmoeError(rc, where)


def _ptr(a):
    """Address of a torch tensor or numpy array (None -> NULL)."""
    if a is None:
        return None
    if isinstance(a, np.ndarray):
        if not a.flags["C_CONTIGUOUS"]:
            raise ValueError("array must be C-contiguous")
        return a.ctypes.data
    if not a.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return a.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def expert_record_bytes(latent, ffn, expert_format=0):
    return _lib.lmoe_expert_record_bytes_fmt(latent, ffn, expert_format)


def du_matrix_bytes(rows, cols, bits):
    return _lib.lmoe_du_matrix_bytes(rows, cols, bits)


class Layer:
    """One latent-MoE layer on one GPU."""

    def __init__(self, hidden, latent, n_experts, top_k, n_groups, expert_ffn, shared_ffn,
                 du_bits, max_tokens, has_router_bias=False, device=0, expert_format=0):
        self.dims = Dims(hidden, latent, n_experts, top_k, n_groups, expert_ffn, shared_ffn,
                         du_bits, max_tokens, int(bool(has_router_bias)), int(expert_format))
        h = ctypes.c_void_p()
        _check(_lib.lmoe_create(ctypes.byref(self.dims), device, ctypes.byref(h)), "lmoe_create")
        self._h = h
        self.device = device

    def set_prefill_d(self, routed_only):
        """1: prefill D over the routed (token, group) pairs only (default); 0: over all groups."""
        _check(_lib.lmoe_set_prefill_d(self._h, int(routed_only)), "lmoe_set_prefill_d")

    def load(self, blobs, stream=None):
        """blobs: router_bf16, router_bias (or None), labels, d_blob, u_blob,
        experts ([E, record] or flat), shared (gate, up, down); numpy arrays
        or torch tensors (host or device)."""
        def nbytes(a):
            return a.nbytes if isinstance(a, np.ndarray) else a.numel() * a.element_size()
        ex = blobs["experts"]
        rec = expert_record_bytes(self.dims.latent, self.dims.expert_ffn, self.dims.expert_format)
        sg, su, sd = blobs["shared"]
        w = Weights(_ptr(blobs["router_bf16"]), _ptr(blobs.get("router_bias")),
                    _ptr(blobs["labels"]),
                    _ptr(blobs["d_blob"]), nbytes(blobs["d_blob"]),
                    _ptr(blobs["u_blob"]), nbytes(blobs["u_blob"]),
                    _ptr(ex), rec if nbytes(ex) == rec * self.dims.n_experts else nbytes(ex),
                    _ptr(sg), _ptr(su), _ptr(sd))
        self._keep = blobs
        _check(_lib.lmoe_load_weights(self._h, ctypes.byref(w), _stream(stream)),
               "lmoe_load_weights")
        self._keep = None

    def forward(self, x, y, T=None, debug=None, stream=None):
        T = x.shape[0] if T is None else T
        dbg = None
        if debug is not None:
            dbg = Debug(*[_ptr(debug.get(k)) for k in (
                "topk_idx", "topk_w", "perm", "expert_count", "expert_off", "group_off", "latent")])
        _check(_lib.lmoe_forward(self._h, _ptr(x), T, _ptr(y),
                                 ctypes.byref(dbg) if dbg is not None else None, _stream(stream)),
               "lmoe_forward")
        return y

    def forward_noalloc(self, x, y, T=None, stream=None):
        """lmoe_forward_noalloc: the decode forward on the static scratch."""
        T = x.shape[0] if T is None else T
        _check(_lib.lmoe_forward_noalloc(self._h, _ptr(x), T, _ptr(y), _stream(stream)),
               "lmoe_forward_noalloc")
        return y

    def forward_block(self, x, eps=1e-6, T=None, stream=None):
        T = x.shape[0] if T is None else T
        _check(_lib.lmoe_forward_block(self._h, _ptr(x), T, eps, _stream(stream)),
               "lmoe_forward_block")
        return x

    def run_phase(self, x, y, phase, T=None, stream=None):
        """Decode phase `phase` (1..4) alone, on what the last forward of the
        same T left in the workspace (profiling)."""
        T = x.shape[0] if T is None else T
        _check(_lib.lmoe_run_phase(self._h, _ptr(x), T, phase, _ptr(y), _stream(stream)),
               "lmoe_run_phase")
        return y

    def set_phase_events(self, events):
        """events: sequence of hipEvent_t handles (ints), or None."""
        if events is None:
            _check(_lib.lmoe_set_phase_events(self._h, None, 0), "lmoe_set_phase_events")
            return
        arr = (ctypes.c_void_p * len(events))(*events)
        _check(_lib.lmoe_set_phase_events(self._h, arr, len(events)), "lmoe_set_phase_events")

    def close(self):
        if getattr(self, "_h", None):
            _lib.lmoe_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def pack_bf16(src, dst, stream=None):
    _check(_lib.lmoe_pack_bf16(_ptr(src), src.numel(), _ptr(dst), _stream(stream)), "lmoe_pack_bf16")
    return dst


def pack_blocks(src, bits, dst, stream=None):
    rows, cols = src.shape
    _check(_lib.lmoe_pack_blocks(_ptr(src), rows, cols, bits, _ptr(dst), _stream(stream)),
           "lmoe_pack_blocks")
    return dst


def pack_expert_records(gate, up, down, dst, stream=None):
    n, f, ell = gate.shape
    _check(_lib.lmoe_pack_expert_records(_ptr(gate), _ptr(up), _ptr(down), n, ell, f, _ptr(dst),
                                         _stream(stream)), "lmoe_pack_expert_records")
    return dst


def ple_gather(tokens, table, head_rows, out, row_bytes=160, stream=None):
    """lmoe_ple_gather: tokens int32 [T + 2] (the two ids before the batch
    first), table uint8 [rows][row_bytes], head_rows 16 ints, out [T][16][row_bytes]
    in a 2-byte dtype (bf16 bit patterns), all device tensors but head_rows."""
    T = tokens.numel() - 2
    hr = (ctypes.c_int64 * 16)(*[int(v) for v in head_rows])
    _check(_lib.lmoe_ple_gather(_ptr(tokens), T, _ptr(table), hr, row_bytes, _ptr(out), _stream(stream)),
           "lmoe_ple_gather")
    return out
