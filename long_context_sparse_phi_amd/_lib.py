"""ctypes mirror of include/nsa.h and loader of the in-tree libnsa.so.

Argument marshalling only: every computation happens in the HIP library.
The library is never built or replaced here; a missing library is an error.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnsa.so")

(NSA_OK, NSA_ERR_INVALID_ARG, NSA_ERR_UNSUPPORTED, NSA_ERR_WORKSPACE, NSA_ERR_HIP,
 NSA_ERR_INTERNAL) = range(6)
NSA_ERR_SCRATCH = 7
NSA_BF16, NSA_FP32 = 0, 1
NSA_PHI_MEANPOOL, NSA_PHI_MLP = 0, 1
(NSA_OP_FWD_PREFILL, NSA_OP_FWD_DECODE, NSA_OP_BWD, NSA_OP_COMPRESS, NSA_OP_DENSE, NSA_OP_APPEND,
 NSA_OP_DENSE_BWD, NSA_OP_LAYER_FWD, NSA_OP_LAYER_BWD) = range(9)
ABI_VERSION = 5

_vp = ctypes.c_void_p


class nsa_params(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "seqlen", "n_kv_heads", "group_size", "d_k", "d_v",
        "cmp_block", "cmp_stride", "sel_block", "n_select", "window",
        "gate_dim", "phi_hidden", "phi", "io_dtype")] + [("scale", ctypes.c_float),
                                                        ("gate_hidden", ctypes.c_int32)]


class nsa_phi_weights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("pe", "w1", "b1", "w2", "b2")]


class nsa_phi_grads(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("pe", "w1", "b1", "w2", "b2")]


class nsa_gate_mlp(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("w1", "b1", "b2")]


class nsa_gate_grads(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("w1", "b1", "b2")]


class nsa_prefill_args(ctypes.Structure):
    _fields_ = ([(n, _vp) for n in ("q", "k", "v", "x", "w_gate")] +
                [("phi_k", nsa_phi_weights), ("phi_v", nsa_phi_weights)] +
                [(n, _vp) for n in ("o", "k_cmp", "v_cmp", "lse", "idx", "o_branch", "p_slc", "gates",
                                    "k_slc", "v_slc", "k_win", "v_win")] +
                [("gate_mlp", nsa_gate_mlp)] +
                [(n, _vp) for n in ("k_cmp_in", "v_cmp_in")])


class nsa_decode_args(ctypes.Structure):
    _fields_ = ([(n, _vp) for n in ("q", "k_cache", "v_cache", "k_cmp_cache", "v_cmp_cache", "x", "w_gate")] +
                [("cmp_cache_cap", ctypes.c_int32)] +
                [(n, _vp) for n in ("o", "idx", "p_slc", "lse", "o_branch", "seq_lens",
                                    "k_win_cache", "v_win_cache")] +
                [("gate_mlp", nsa_gate_mlp)])


class nsa_append_args(ctypes.Structure):
    _fields_ = ([(n, _vp) for n in ("k_new", "v_new", "seq_lens", "k_cache", "v_cache",
                                    "k_cmp_cache", "v_cmp_cache")] +
                [("cmp_cache_cap", ctypes.c_int32)] +
                [("phi_k", nsa_phi_weights), ("phi_v", nsa_phi_weights)] +
                [(n, _vp) for n in ("k_slc_new", "v_slc_new", "k_slc_cache", "v_slc_cache",
                                    "k_win_new", "v_win_new", "k_win_cache", "v_win_cache")])


class nsa_bwd_args(ctypes.Structure):
    _fields_ = ([(n, _vp) for n in ("q", "k", "v", "x", "w_gate")] +
                [("phi_k", nsa_phi_weights), ("phi_v", nsa_phi_weights)] +
                [(n, _vp) for n in ("k_cmp", "v_cmp", "lse", "idx", "o_branch", "d_o",
                                    "dq", "dk", "dv", "dw_gate")] +
                [("d_phi_k", nsa_phi_grads), ("d_phi_v", nsa_phi_grads)] +
                [(n, _vp) for n in ("k_slc", "v_slc", "k_win", "v_win",
                                    "dk_slc", "dv_slc", "dk_win", "dv_win")] +
                [("gate_mlp", nsa_gate_mlp), ("d_gate_mlp", nsa_gate_grads), ("dx", _vp)])


class nsa_dense_args(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("q", "k", "v", "o", "lse")]


class nsa_dense_bwd_args(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("q", "k", "v", "o", "lse", "d_o", "dq", "dk", "dv")]


class nsa_layer_args(ctypes.Structure):
    _fields_ = ([(n, _vp) for n in ("h", "w_q", "w_k", "w_v", "w_o", "w_gate")] +
                [("gate_mlp", nsa_gate_mlp), ("phi_k", nsa_phi_weights), ("phi_v", nsa_phi_weights)] +
                [(n, _vp) for n in ("y", "q", "k", "v", "o", "k_cmp", "v_cmp", "lse", "idx", "o_branch")])


class nsa_layer_bwd_args(ctypes.Structure):
    _fields_ = ([(n, _vp) for n in ("h", "w_q", "w_k", "w_v", "w_o", "w_gate")] +
                [("gate_mlp", nsa_gate_mlp), ("phi_k", nsa_phi_weights), ("phi_v", nsa_phi_weights)] +
                [(n, _vp) for n in ("q", "k", "v", "o", "k_cmp", "v_cmp", "lse", "idx", "o_branch", "dy",
                                    "dh", "dw_q", "dw_k", "dw_v", "dw_o", "dw_gate")] +
                [("d_gate_mlp", nsa_gate_grads), ("d_phi_k", nsa_phi_grads), ("d_phi_v", nsa_phi_grads)])


EXPORTS = ("nsa_abi_version", "nsa_status_str", "nsa_workspace_size", "nsa_compress",
           "nsa_fwd_prefill", "nsa_fwd_decode", "nsa_bwd", "nsa_dense_fwd",
           "nsa_decode_append", "nsa_dense_bwd", "nsa_layer_fwd", "nsa_layer_bwd", "nsa_fwd_decode_noalloc")

_LIB = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libnsa.so (once) and declare the signatures of its exports."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(f"NSA HIP library not built: {path} is missing "
                           "(run python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.nsa_abi_version.restype = ctypes.c_int
    lib.nsa_abi_version.argtypes = []
    lib.nsa_status_str.restype = ctypes.c_char_p
    lib.nsa_status_str.argtypes = [ctypes.c_int]
    lib.nsa_workspace_size.restype = ctypes.c_int
    lib.nsa_workspace_size.argtypes = [P(nsa_params), ctypes.c_int, P(ctypes.c_size_t)]
    lib.nsa_compress.restype = ctypes.c_int
    lib.nsa_compress.argtypes = [P(nsa_params), ctypes.c_int, _vp, P(nsa_phi_weights), _vp, _vp,
                                 ctypes.c_size_t, _vp]
    for name, argt in (("nsa_fwd_prefill", nsa_prefill_args), ("nsa_fwd_decode", nsa_decode_args),
                       ("nsa_bwd", nsa_bwd_args), ("nsa_dense_fwd", nsa_dense_args),
                       ("nsa_decode_append", nsa_append_args), ("nsa_dense_bwd", nsa_dense_bwd_args),
                       ("nsa_layer_fwd", nsa_layer_args), ("nsa_layer_bwd", nsa_layer_bwd_args)):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [P(nsa_params), P(argt), _vp, ctypes.c_size_t, _vp]
    lib.nsa_fwd_decode_noalloc.restype = ctypes.c_int
    lib.nsa_fwd_decode_noalloc.argtypes = [P(nsa_params), P(nsa_decode_args), _vp]
    if lib.nsa_abi_version() != ABI_VERSION:
        raise RuntimeError("libnsa.so ABI version mismatch")
    _LIB = lib
    return lib


def status_str(code: int) -> str:
    return load().nsa_status_str(code).decode()


class NSAError(RuntimeError):
    def __init__(self, where: str, code: int):
        super().__init__(f"{where}: {status_str(code)} (status {code})")
        self.code = code
