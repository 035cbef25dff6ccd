"""MI355X (gfx950) Native Sparse Attention: Python binding of libnsa.so.

The functions here take torch tensors that already live on the GPU, check
their dtypes and shapes, and pass raw pointers and the current HIP stream to
the C ABI (include/nsa.h).  torch provides device memory and streams only;
every step of the operator runs in the library's HIP kernels.  Output tensors
are allocated with torch when the caller does not pass them.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
from typing import Dict, Optional

import torch

from . import _lib
from ._lib import (NSA_BF16, NSA_FP32, NSA_OP_APPEND, NSA_OP_BWD, NSA_OP_COMPRESS, NSA_OP_DENSE,
                   NSA_OP_DENSE_BWD, NSA_OP_FWD_DECODE, NSA_OP_FWD_PREFILL, NSA_OP_LAYER_BWD,
                   NSA_OP_LAYER_FWD, NSA_PHI_MEANPOOL, NSA_PHI_MLP, NSAError)

__all__ = ["Config", "workspace_size", "nsa_compress", "nsa_fwd_prefill", "nsa_fwd_decode",
           "nsa_decode_append", "nsa_bwd", "nsa_dense_fwd", "nsa_dense_bwd", "nsa_layer_fwd", "nsa_layer_bwd",
           "load_library", "NSAError"]

load_library = _lib.load


@dataclasses.dataclass(frozen=True)
class Config:
    """Shapes and hyper-parameters (mirrors nsa_params)."""
    B: int
    T: int
    H_kv: int
    G: int
    d_k: int
    d_v: int
    l: int = 32
    d: int = 16
    l_sel: int = 64
    n: int = 16
    w: int = 512
    gate_dim: int = 256
    hidden: int = 256
    phi: str = "mlp"          # "mlp" | "mean"
    dtype: str = "bf16"       # "bf16" | "fp32"
    scale: float = 0.0        # 0 => 1/sqrt(d_k)
    gate_hidden: int = 0      # 0: one linear gate layer; else the gate MLP's hidden width

    @property
    def H_q(self) -> int:
        return self.H_kv * self.G

    @property
    def n_cmp(self) -> int:
        return 0 if self.T < self.l else (self.T - self.l) // self.d + 1

    @property
    def n_sel(self) -> int:
        return -(-self.T // self.l_sel)

    @property
    def gate_in(self) -> int:
        """Input width of the gate layer that w_gate holds."""
        return self.gate_hidden if self.gate_hidden else self.gate_dim

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def params(self) -> _lib.nsa_params:
        return _lib.nsa_params(
            batch=self.B, seqlen=self.T, n_kv_heads=self.H_kv, group_size=self.G,
            d_k=self.d_k, d_v=self.d_v, cmp_block=self.l, cmp_stride=self.d,
            sel_block=self.l_sel, n_select=self.n, window=self.w, gate_dim=self.gate_dim,
            phi_hidden=self.hidden if self.phi == "mlp" else 0,
            phi=NSA_PHI_MLP if self.phi == "mlp" else NSA_PHI_MEANPOOL,
            io_dtype=NSA_BF16 if self.dtype == "bf16" else NSA_FP32, scale=self.scale,
            gate_hidden=self.gate_hidden)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check(t: torch.Tensor, name: str, shape, dtype: torch.dtype, dev: torch.device):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or t.device != dev:
        raise ValueError(f"{name} must live on {dev}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def workspace_size(cfg: Config, op: int) -> int:
    n = ctypes.c_size_t(0)
    p = cfg.params()
    st = _lib.load().nsa_workspace_size(ctypes.byref(p), op, ctypes.byref(n))
    if st != 0:
        raise NSAError("nsa_workspace_size", st)
    return int(n.value)


def _workspace(cfg: Config, op: int, dev, ws: Optional[torch.Tensor]) -> torch.Tensor:
    need = workspace_size(cfg, op)
    if ws is None:
        return torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace of {need} bytes needed")
    return ws


def _phi_struct(cfg: Config, phi: Optional[Dict[str, torch.Tensor]], D: int, dev) -> _lib.nsa_phi_weights:
    w = _lib.nsa_phi_weights()
    if cfg.phi != "mlp":
        return w
    shapes = {"pe": (cfg.l, D), "w1": (cfg.l * D, cfg.hidden), "b1": (cfg.hidden,),
              "w2": (cfg.hidden, D), "b2": (D,)}
    for k, shp in shapes.items():
        _check(phi[k], f"phi.{k}", shp, cfg.torch_dtype, dev)
        setattr(w, k, phi[k].data_ptr())
    return w


def _gate_struct(cfg: Config, gate_mlp: Optional[Dict[str, torch.Tensor]], dev) -> _lib.nsa_gate_mlp:
    """First layer and biases of the gate MLP ({"w1", "b1", "b2"}), required
    exactly when cfg.gate_hidden > 0."""
    g = _lib.nsa_gate_mlp()
    if not cfg.gate_hidden:
        if gate_mlp is not None:
            raise ValueError("gate_mlp given but cfg.gate_hidden is 0")
        return g
    if gate_mlp is None:
        raise ValueError("cfg.gate_hidden > 0 needs gate_mlp = {w1, b1, b2}")
    shapes = {"w1": (cfg.gate_dim, cfg.gate_hidden), "b1": (cfg.gate_hidden,), "b2": (cfg.H_q, 3)}
    for k, shp in shapes.items():
        _check(gate_mlp[k], f"gate_mlp.{k}", shp, cfg.torch_dtype, dev)
        setattr(g, k, gate_mlp[k].data_ptr())
    return g


def nsa_compress(cfg: Config, x: torch.Tensor, phi: Optional[Dict[str, torch.Tensor]], is_value: bool,
                 out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Compressed keys (is_value=False) or values of x [B,T,Hkv,D] -> [B,Ncmp,Hkv,D]."""
    dev = x.device
    D = cfg.d_v if is_value else cfg.d_k
    _check(x, "x", (cfg.B, cfg.T, cfg.H_kv, D), cfg.torch_dtype, dev)
    if out is None:
        out = torch.empty(cfg.B, cfg.n_cmp, cfg.H_kv, D, dtype=cfg.torch_dtype, device=dev)
    _check(out, "out", (cfg.B, cfg.n_cmp, cfg.H_kv, D), cfg.torch_dtype, dev)
    ws = _workspace(cfg, NSA_OP_COMPRESS, dev, workspace)
    p = cfg.params()
    w = _phi_struct(cfg, phi, D, dev)
    st = _lib.load().nsa_compress(ctypes.byref(p), int(is_value), x.data_ptr(), ctypes.byref(w),
                                  out.data_ptr() if out.numel() else x.data_ptr(), ws.data_ptr(),
                                  ws.numel(), _stream(dev))
    if st != 0:
        raise NSAError("nsa_compress", st)
    return out


def _branch_kv(cfg: Config, kv, tag: str, dev):
    """Pointers of a branch's own (k, v) pair, or (None, None)."""
    if kv is None:
        return None, None
    k, v = kv
    _check(k, f"k_{tag}", (cfg.B, cfg.T, cfg.H_kv, cfg.d_k), cfg.torch_dtype, dev)
    _check(v, f"v_{tag}", (cfg.B, cfg.T, cfg.H_kv, cfg.d_v), cfg.torch_dtype, dev)
    return k.data_ptr(), v.data_ptr()


def nsa_fwd_prefill(cfg: Config, q, k, v, x, w_gate, phi_k=None, phi_v=None, *, out=None,
                    save_for_backward: bool = False, debug: bool = False, kv_slc=None, kv_win=None,
                    gate_mlp=None, kv_cmp=None, workspace: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """NSA prefill forward.  Returns {"o": ...} plus, when save_for_backward,
    k_cmp, v_cmp, lse, idx, o_branch, and, when debug, also p_slc and gates.
    kv_slc, kv_win: (k, v) pairs of the selected and window branches when each
    branch has its own keys and values (both or neither); k, v then feed the
    compressed branch only.  With cfg.gate_hidden > 0, gate_mlp holds the gate
    MLP's first layer and biases and w_gate its output layer [Hg, Hq, 3].
    kv_cmp: precomputed compressed (k_cmp [B,Ncmp,Hkv,dk], v_cmp [B,Ncmp,Hkv,dv])
    used instead of running phi (phi_k, phi_v are then not needed)."""
    dev = q.device
    dt = cfg.torch_dtype
    B, T, Hq, Hkv = cfg.B, cfg.T, cfg.H_q, cfg.H_kv
    _check(q, "q", (B, T, Hq, cfg.d_k), dt, dev)
    _check(k, "k", (B, T, Hkv, cfg.d_k), dt, dev)
    _check(v, "v", (B, T, Hkv, cfg.d_v), dt, dev)
    _check(x, "x", (B, T, cfg.gate_dim), dt, dev)
    _check(w_gate, "w_gate", (cfg.gate_in, Hq, 3), dt, dev)
    res = {"o": out if out is not None else torch.empty(B, T, Hq, cfg.d_v, dtype=dt, device=dev)}
    _check(res["o"], "o", (B, T, Hq, cfg.d_v), dt, dev)
    if save_for_backward or debug:
        res["k_cmp"] = torch.empty(B, cfg.n_cmp, Hkv, cfg.d_k, dtype=dt, device=dev)
        res["v_cmp"] = torch.empty(B, cfg.n_cmp, Hkv, cfg.d_v, dtype=dt, device=dev)
        res["lse"] = torch.empty(3, B, T, Hq, dtype=torch.float32, device=dev)
        res["idx"] = torch.empty(B, T, Hkv, cfg.n, dtype=torch.int32, device=dev)
        res["o_branch"] = torch.empty(3, B, T, Hq, cfg.d_v, dtype=torch.float32, device=dev)
    if debug:
        res["p_slc"] = torch.empty(B, T, Hkv, cfg.n_sel, dtype=torch.float32, device=dev)
        res["gates"] = torch.empty(B, T, Hq, 3, dtype=torch.float32, device=dev)
    a = _lib.nsa_prefill_args()
    for name, t in (("q", q), ("k", k), ("v", v), ("x", x), ("w_gate", w_gate)):
        setattr(a, name, t.data_ptr())
    if kv_cmp is None:
        a.phi_k = _phi_struct(cfg, phi_k, cfg.d_k, dev)
        a.phi_v = _phi_struct(cfg, phi_v, cfg.d_v, dev)
    else:
        kc, vc = kv_cmp
        _check(kc, "k_cmp_in", (B, cfg.n_cmp, Hkv, cfg.d_k), dt, dev)
        _check(vc, "v_cmp_in", (B, cfg.n_cmp, Hkv, cfg.d_v), dt, dev)
        a.k_cmp_in = kc.data_ptr() if kc.numel() else None
        a.v_cmp_in = vc.data_ptr() if vc.numel() else None
    for name in ("o", "k_cmp", "v_cmp", "lse", "idx", "o_branch", "p_slc", "gates"):
        t = res.get(name)
        setattr(a, name, t.data_ptr() if (t is not None and t.numel()) else None)
    if (kv_slc is None) != (kv_win is None):
        raise ValueError("kv_slc and kv_win go together")
    a.k_slc, a.v_slc = _branch_kv(cfg, kv_slc, "slc", dev)
    a.k_win, a.v_win = _branch_kv(cfg, kv_win, "win", dev)
    a.gate_mlp = _gate_struct(cfg, gate_mlp, dev)
    ws = _workspace(cfg, NSA_OP_FWD_PREFILL, dev, workspace)
    p = cfg.params()
    st = _lib.load().nsa_fwd_prefill(ctypes.byref(p), ctypes.byref(a), ws.data_ptr(), ws.numel(), _stream(dev))
    if st != 0:
        raise NSAError("nsa_fwd_prefill", st)
    res["_workspace"] = ws
    return res


def nsa_fwd_decode(cfg: Config, q, k_cache, v_cache, k_cmp_cache, v_cmp_cache, x, w_gate, *,
                   out=None, debug: bool = False, seq_lens: Optional[torch.Tensor] = None,
                   kv_win_cache=None, gate_mlp=None, workspace: Optional[torch.Tensor] = None,
                   no_alloc: bool = False):
    """One decode step; cfg.T is the cache length S (query at position S-1).
    With seq_lens (int32 [B] on the device), cfg.T is the cache capacity and
    sequence b holds seq_lens[b] tokens, its query at position seq_lens[b]-1.
    kv_win_cache: the window branch's own (k, v) caches when each branch has
    independent keys and values (k_cache, v_cache then serve the selected one).
    no_alloc: call nsa_fwd_decode_noalloc, which takes no workspace (the
    library's static per-GPU scratch buffer; calls on one GPU must not
    overlap)."""
    dev = q.device
    dt = cfg.torch_dtype
    B, S, Hq, Hkv = cfg.B, cfg.T, cfg.H_q, cfg.H_kv
    _check(q, "q", (B, Hq, cfg.d_k), dt, dev)
    _check(k_cache, "k_cache", (B, S, Hkv, cfg.d_k), dt, dev)
    _check(v_cache, "v_cache", (B, S, Hkv, cfg.d_v), dt, dev)
    cap = k_cmp_cache.shape[1]
    _check(k_cmp_cache, "k_cmp_cache", (B, cap, Hkv, cfg.d_k), dt, dev)
    _check(v_cmp_cache, "v_cmp_cache", (B, cap, Hkv, cfg.d_v), dt, dev)
    _check(x, "x", (B, cfg.gate_dim), dt, dev)
    _check(w_gate, "w_gate", (cfg.gate_in, Hq, 3), dt, dev)
    res = {"o": out if out is not None else torch.empty(B, Hq, cfg.d_v, dtype=dt, device=dev)}
    if debug:
        res["idx"] = torch.empty(B, Hkv, cfg.n, dtype=torch.int32, device=dev)
        res["p_slc"] = torch.empty(B, Hkv, cfg.n_sel, dtype=torch.float32, device=dev)
        res["lse"] = torch.empty(3, B, Hq, dtype=torch.float32, device=dev)
        res["o_branch"] = torch.empty(3, B, Hq, cfg.d_v, dtype=torch.float32, device=dev)
    a = _lib.nsa_decode_args()
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("x", x), ("w_gate", w_gate)):
        setattr(a, name, t.data_ptr())
    a.k_cmp_cache = k_cmp_cache.data_ptr() if k_cmp_cache.numel() else None
    a.v_cmp_cache = v_cmp_cache.data_ptr() if v_cmp_cache.numel() else None
    a.cmp_cache_cap = cap
    for name in ("o", "idx", "p_slc", "lse", "o_branch"):
        t = res.get(name)
        setattr(a, name, t.data_ptr() if t is not None else None)
    if seq_lens is not None:
        _check(seq_lens, "seq_lens", (B,), torch.int32, dev)
        a.seq_lens = seq_lens.data_ptr()
    if kv_win_cache is not None:
        _check(kv_win_cache[0], "k_win_cache", (B, S, Hkv, cfg.d_k), dt, dev)
        _check(kv_win_cache[1], "v_win_cache", (B, S, Hkv, cfg.d_v), dt, dev)
        a.k_win_cache, a.v_win_cache = kv_win_cache[0].data_ptr(), kv_win_cache[1].data_ptr()
    a.gate_mlp = _gate_struct(cfg, gate_mlp, dev)
    p = cfg.params()
    if no_alloc:
        st = _lib.load().nsa_fwd_decode_noalloc(ctypes.byref(p), ctypes.byref(a), _stream(dev))
        if st != 0:
            raise NSAError("nsa_fwd_decode_noalloc", st)
        return res
    ws = _workspace(cfg, NSA_OP_FWD_DECODE, dev, workspace)
    st = _lib.load().nsa_fwd_decode(ctypes.byref(p), ctypes.byref(a), ws.data_ptr(), ws.numel(), _stream(dev))
    if st != 0:
        raise NSAError("nsa_fwd_decode", st)
    res["_workspace"] = ws
    return res


def nsa_decode_append(cfg: Config, k_new, v_new, seq_lens, k_cache, v_cache, k_cmp_cache, v_cmp_cache,
                      phi_k=None, phi_v=None, *, kv_slc=None, kv_win=None,
                      workspace: Optional[torch.Tensor] = None) -> None:
    """Append one token per sequence at slot seq_lens[b] of the raw caches
    (cfg.T = their capacity) and write the compressed block it completes, if
    any.  seq_lens (int32 [B], device) is read only; advance it afterwards.
    With independent keys/values per branch, kv_slc and kv_win are each
    (k_new, v_new, k_cache, v_cache) of the selected and window branches,
    appended at the same slot; k_cache, v_cache are then the compressed
    branch's (the rows phi reads)."""
    dev = k_cache.device
    dt = cfg.torch_dtype
    B, S, Hkv = cfg.B, cfg.T, cfg.H_kv
    _check(k_new, "k_new", (B, Hkv, cfg.d_k), dt, dev)
    _check(v_new, "v_new", (B, Hkv, cfg.d_v), dt, dev)
    _check(seq_lens, "seq_lens", (B,), torch.int32, dev)
    _check(k_cache, "k_cache", (B, S, Hkv, cfg.d_k), dt, dev)
    _check(v_cache, "v_cache", (B, S, Hkv, cfg.d_v), dt, dev)
    cap = k_cmp_cache.shape[1]
    _check(k_cmp_cache, "k_cmp_cache", (B, cap, Hkv, cfg.d_k), dt, dev)
    _check(v_cmp_cache, "v_cmp_cache", (B, cap, Hkv, cfg.d_v), dt, dev)
    a = _lib.nsa_append_args()
    for name, t in (("k_new", k_new), ("v_new", v_new), ("seq_lens", seq_lens), ("k_cache", k_cache),
                    ("v_cache", v_cache)):
        setattr(a, name, t.data_ptr())
    a.k_cmp_cache = k_cmp_cache.data_ptr() if k_cmp_cache.numel() else None
    a.v_cmp_cache = v_cmp_cache.data_ptr() if v_cmp_cache.numel() else None
    a.cmp_cache_cap = cap
    a.phi_k = _phi_struct(cfg, phi_k, cfg.d_k, dev)
    a.phi_v = _phi_struct(cfg, phi_v, cfg.d_v, dev)
    for tag, quad in (("slc", kv_slc), ("win", kv_win)):
        if quad is None:
            continue
        kn, vn, kc, vc = quad
        _check(kn, f"k_{tag}_new", (B, Hkv, cfg.d_k), dt, dev)
        _check(vn, f"v_{tag}_new", (B, Hkv, cfg.d_v), dt, dev)
        _check(kc, f"k_{tag}_cache", (B, S, Hkv, cfg.d_k), dt, dev)
        _check(vc, f"v_{tag}_cache", (B, S, Hkv, cfg.d_v), dt, dev)
        for n, t in ((f"k_{tag}_new", kn), (f"v_{tag}_new", vn), (f"k_{tag}_cache", kc), (f"v_{tag}_cache", vc)):
            setattr(a, n, t.data_ptr())
    ws = _workspace(cfg, NSA_OP_APPEND, dev, workspace)
    p = cfg.params()
    st = _lib.load().nsa_decode_append(ctypes.byref(p), ctypes.byref(a), ws.data_ptr(), ws.numel(),
                                       _stream(dev))
    if st != 0:
        raise NSAError("nsa_decode_append", st)


def nsa_bwd(cfg: Config, q, k, v, x, w_gate, phi_k, phi_v, saved: Dict[str, torch.Tensor], d_o, *,
            kv_slc=None, kv_win=None, recompute_row_terms: bool = False, gate_mlp=None,
            want_dx: bool = False, workspace: Optional[torch.Tensor] = None) -> Dict[str, object]:
    """Backward with the forward's selected blocks fixed.  `saved` is the dict
    nsa_fwd_prefill returned with save_for_backward=True.  Gradients are fp32.
    With kv_slc, kv_win (as passed to the forward) the result also holds
    dk_slc, dv_slc, dk_win, dv_win, and dk, dv are the compressed branch's part.
    The softmax row terms <dO, O_c> are read from saved["o_branch"] when it is
    there, unless recompute_row_terms asks for them to be recomputed.
    With cfg.gate_hidden > 0 the result holds d_gate_mlp {w1, b1, b2}, and
    dw_gate is the output layer's gradient; want_dx adds dx, the gradient
    with respect to the gate input x."""
    dev = q.device
    dt = cfg.torch_dtype
    B, T, Hq, Hkv = cfg.B, cfg.T, cfg.H_q, cfg.H_kv
    _check(d_o, "d_o", (B, T, Hq, cfg.d_v), dt, dev)
    f32 = torch.float32
    res = {"dq": torch.empty(B, T, Hq, cfg.d_k, dtype=f32, device=dev),
           "dk": torch.empty(B, T, Hkv, cfg.d_k, dtype=f32, device=dev),
           "dv": torch.empty(B, T, Hkv, cfg.d_v, dtype=f32, device=dev),
           "dw_gate": torch.empty(cfg.gate_in, Hq, 3, dtype=f32, device=dev)}
    a = _lib.nsa_bwd_args()
    for name, t in (("q", q), ("k", k), ("v", v), ("x", x), ("w_gate", w_gate), ("d_o", d_o)):
        setattr(a, name, t.data_ptr())
    for name in ("k_cmp", "v_cmp", "lse", "idx"):
        t = saved[name]
        setattr(a, name, t.data_ptr() if t.numel() else None)
    if saved.get("o_branch") is not None and not recompute_row_terms:
        _check(saved["o_branch"], "o_branch", (3, B, T, Hq, cfg.d_v), torch.float32, dev)
        a.o_branch = saved["o_branch"].data_ptr()
    a.phi_k = _phi_struct(cfg, phi_k, cfg.d_k, dev)
    a.phi_v = _phi_struct(cfg, phi_v, cfg.d_v, dev)
    for name in ("dq", "dk", "dv", "dw_gate"):
        setattr(a, name, res[name].data_ptr())
    if (kv_slc is None) != (kv_win is None):
        raise ValueError("kv_slc and kv_win go together")
    if kv_slc is not None:
        a.k_slc, a.v_slc = _branch_kv(cfg, kv_slc, "slc", dev)
        a.k_win, a.v_win = _branch_kv(cfg, kv_win, "win", dev)
        for tag in ("slc", "win"):
            res["dk_" + tag] = torch.empty(B, T, Hkv, cfg.d_k, dtype=f32, device=dev)
            res["dv_" + tag] = torch.empty(B, T, Hkv, cfg.d_v, dtype=f32, device=dev)
            setattr(a, "dk_" + tag, res["dk_" + tag].data_ptr())
            setattr(a, "dv_" + tag, res["dv_" + tag].data_ptr())
    if cfg.phi == "mlp":
        for tag, D in (("d_phi_k", cfg.d_k), ("d_phi_v", cfg.d_v)):
            g = {"pe": torch.empty(cfg.l, D, dtype=f32, device=dev),
                 "w1": torch.empty(cfg.l * D, cfg.hidden, dtype=f32, device=dev),
                 "b1": torch.empty(cfg.hidden, dtype=f32, device=dev),
                 "w2": torch.empty(cfg.hidden, D, dtype=f32, device=dev),
                 "b2": torch.empty(D, dtype=f32, device=dev)}
            gs = _lib.nsa_phi_grads(**{kk: vv.data_ptr() for kk, vv in g.items()})
            setattr(a, tag, gs)
            res[tag] = g
    a.gate_mlp = _gate_struct(cfg, gate_mlp, dev)
    if cfg.gate_hidden:
        gg = {"w1": torch.empty(cfg.gate_dim, cfg.gate_hidden, dtype=f32, device=dev),
              "b1": torch.empty(cfg.gate_hidden, dtype=f32, device=dev),
              "b2": torch.empty(Hq, 3, dtype=f32, device=dev)}
        a.d_gate_mlp = _lib.nsa_gate_grads(**{kk: vv.data_ptr() for kk, vv in gg.items()})
        res["d_gate_mlp"] = gg
    if want_dx:
        res["dx"] = torch.empty(B, T, cfg.gate_dim, dtype=f32, device=dev)
        a.dx = res["dx"].data_ptr()
    ws = _workspace(cfg, NSA_OP_BWD, dev, workspace)
    p = cfg.params()
    st = _lib.load().nsa_bwd(ctypes.byref(p), ctypes.byref(a), ws.data_ptr(), ws.numel(), _stream(dev))
    if st != 0:
        raise NSAError("nsa_bwd", st)
    res["_workspace"] = ws
    return res


def nsa_dense_fwd(cfg: Config, q, k, v, *, out=None, want_lse: bool = False,
                  workspace: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """Dense causal attention (the baseline NSA is measured against): every query
    attends to all keys at or before its position.  Uses cfg's shapes only."""
    dev = q.device
    dt = cfg.torch_dtype
    B, T, Hq, Hkv = cfg.B, cfg.T, cfg.H_q, cfg.H_kv
    _check(q, "q", (B, T, Hq, cfg.d_k), dt, dev)
    _check(k, "k", (B, T, Hkv, cfg.d_k), dt, dev)
    _check(v, "v", (B, T, Hkv, cfg.d_v), dt, dev)
    res = {"o": out if out is not None else torch.empty(B, T, Hq, cfg.d_v, dtype=dt, device=dev)}
    if want_lse:
        res["lse"] = torch.empty(B, T, Hq, dtype=torch.float32, device=dev)
    a = _lib.nsa_dense_args(q=q.data_ptr(), k=k.data_ptr(), v=v.data_ptr(), o=res["o"].data_ptr(),
                            lse=res["lse"].data_ptr() if want_lse else None)
    ws = _workspace(cfg, NSA_OP_DENSE, dev, workspace)
    p = cfg.params()
    st = _lib.load().nsa_dense_fwd(ctypes.byref(p), ctypes.byref(a), ws.data_ptr(), ws.numel(), _stream(dev))
    if st != 0:
        raise NSAError("nsa_dense_fwd", st)
    res["_workspace"] = ws
    return res


def nsa_dense_bwd(cfg: Config, q, k, v, o, lse, d_o, *,
                  workspace: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """Backward of nsa_dense_fwd (o and lse as it returned them); fp32 gradients."""
    dev = q.device
    dt = cfg.torch_dtype
    B, T, Hq, Hkv = cfg.B, cfg.T, cfg.H_q, cfg.H_kv
    _check(q, "q", (B, T, Hq, cfg.d_k), dt, dev)
    _check(k, "k", (B, T, Hkv, cfg.d_k), dt, dev)
    _check(v, "v", (B, T, Hkv, cfg.d_v), dt, dev)
    _check(o, "o", (B, T, Hq, cfg.d_v), dt, dev)
    _check(lse, "lse", (B, T, Hq), torch.float32, dev)
    _check(d_o, "d_o", (B, T, Hq, cfg.d_v), dt, dev)
    f32 = torch.float32
    res = {"dq": torch.empty(B, T, Hq, cfg.d_k, dtype=f32, device=dev),
           "dk": torch.empty(B, T, Hkv, cfg.d_k, dtype=f32, device=dev),
           "dv": torch.empty(B, T, Hkv, cfg.d_v, dtype=f32, device=dev)}
    a = _lib.nsa_dense_bwd_args(q=q.data_ptr(), k=k.data_ptr(), v=v.data_ptr(), o=o.data_ptr(),
                                lse=lse.data_ptr(), d_o=d_o.data_ptr(), dq=res["dq"].data_ptr(),
                                dk=res["dk"].data_ptr(), dv=res["dv"].data_ptr())
    ws = _workspace(cfg, NSA_OP_DENSE_BWD, dev, workspace)
    p = cfg.params()
    st = _lib.load().nsa_dense_bwd(ctypes.byref(p), ctypes.byref(a), ws.data_ptr(), ws.numel(), _stream(dev))
    if st != 0:
        raise NSAError("nsa_dense_bwd", st)
    res["_workspace"] = ws
    return res


def _layer_weights(cfg: Config, proj: Dict[str, torch.Tensor], dev):
    C, dt = cfg.gate_dim, cfg.torch_dtype
    shapes = {"w_q": (C, cfg.H_q * cfg.d_k), "w_k": (C, cfg.H_kv * cfg.d_k), "w_v": (C, cfg.H_kv * cfg.d_v),
              "w_o": (cfg.H_q * cfg.d_v, C)}
    for k, shp in shapes.items():
        _check(proj[k], f"proj.{k}", shp, dt, dev)
    return {k: proj[k].data_ptr() for k in shapes}


def nsa_layer_fwd(cfg: Config, h, proj: Dict[str, torch.Tensor], w_gate, phi_k=None, phi_v=None, *,
                  gate_mlp=None, workspace: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """Attention layer around the operator: q, k, v = h w_q, h w_k, h w_v;
    o = NSA(q, k, v) with h as the gate input; y = o w_o.  h [B,T,C] with
    C = cfg.gate_dim; proj = {w_q [C,Hq*dk], w_k [C,Hkv*dk], w_v [C,Hkv*dv],
    w_o [Hq*dv,C]}.  Returns y and what nsa_layer_bwd needs (q, k, v, o,
    k_cmp, v_cmp, lse, idx, o_branch)."""
    dev = h.device
    dt = cfg.torch_dtype
    B, T, Hq, Hkv = cfg.B, cfg.T, cfg.H_q, cfg.H_kv
    _check(h, "h", (B, T, cfg.gate_dim), dt, dev)
    _check(w_gate, "w_gate", (cfg.gate_in, Hq, 3), dt, dev)
    a = _lib.nsa_layer_args(h=h.data_ptr(), w_gate=w_gate.data_ptr(), **_layer_weights(cfg, proj, dev))
    res = {"y": torch.empty(B, T, cfg.gate_dim, dtype=dt, device=dev),
           "q": torch.empty(B, T, Hq, cfg.d_k, dtype=dt, device=dev),
           "k": torch.empty(B, T, Hkv, cfg.d_k, dtype=dt, device=dev),
           "v": torch.empty(B, T, Hkv, cfg.d_v, dtype=dt, device=dev),
           "o": torch.empty(B, T, Hq, cfg.d_v, dtype=dt, device=dev),
           "k_cmp": torch.empty(B, cfg.n_cmp, Hkv, cfg.d_k, dtype=dt, device=dev),
           "v_cmp": torch.empty(B, cfg.n_cmp, Hkv, cfg.d_v, dtype=dt, device=dev),
           "lse": torch.empty(3, B, T, Hq, dtype=torch.float32, device=dev),
           "idx": torch.empty(B, T, Hkv, cfg.n, dtype=torch.int32, device=dev),
           "o_branch": torch.empty(3, B, T, Hq, cfg.d_v, dtype=torch.float32, device=dev)}
    for name, t in res.items():
        setattr(a, name, t.data_ptr() if t.numel() else None)
    a.phi_k = _phi_struct(cfg, phi_k, cfg.d_k, dev)
    a.phi_v = _phi_struct(cfg, phi_v, cfg.d_v, dev)
    a.gate_mlp = _gate_struct(cfg, gate_mlp, dev)
    ws = _workspace(cfg, NSA_OP_LAYER_FWD, dev, workspace)
    p = cfg.params()
    st = _lib.load().nsa_layer_fwd(ctypes.byref(p), ctypes.byref(a), ws.data_ptr(), ws.numel(), _stream(dev))
    if st != 0:
        raise NSAError("nsa_layer_fwd", st)
    res["_workspace"] = ws
    return res


def nsa_layer_bwd(cfg: Config, h, proj: Dict[str, torch.Tensor], w_gate, phi_k, phi_v,
                  saved: Dict[str, torch.Tensor], dy, *, gate_mlp=None,
                  workspace: Optional[torch.Tensor] = None) -> Dict[str, object]:
    """Backward of nsa_layer_fwd (saved = its result) for dy [B,T,C]: dh,
    dw_q, dw_k, dw_v, dw_o, dw_gate, and d_gate_mlp / d_phi_k / d_phi_v where
    those weights exist; all fp32."""
    dev = h.device
    dt = cfg.torch_dtype
    B, T, Hq = cfg.B, cfg.T, cfg.H_q
    C = cfg.gate_dim
    _check(h, "h", (B, T, C), dt, dev)
    _check(dy, "dy", (B, T, C), dt, dev)
    _check(w_gate, "w_gate", (cfg.gate_in, Hq, 3), dt, dev)
    f32 = torch.float32
    a = _lib.nsa_layer_bwd_args(h=h.data_ptr(), w_gate=w_gate.data_ptr(), dy=dy.data_ptr(),
                                **_layer_weights(cfg, proj, dev))
    for name in ("q", "k", "v", "o", "k_cmp", "v_cmp", "lse", "idx", "o_branch"):
        t = saved[name]
        setattr(a, name, t.data_ptr() if t.numel() else None)
    res = {"dh": torch.empty(B, T, C, dtype=f32, device=dev),
           "dw_gate": torch.empty(cfg.gate_in, Hq, 3, dtype=f32, device=dev)}
    for k, t in proj.items():
        res["d" + k] = torch.empty(t.shape, dtype=f32, device=dev)
    for name in ("dh", "dw_gate", "dw_q", "dw_k", "dw_v", "dw_o"):
        setattr(a, name, res[name].data_ptr())
    a.phi_k = _phi_struct(cfg, phi_k, cfg.d_k, dev)
    a.phi_v = _phi_struct(cfg, phi_v, cfg.d_v, dev)
    a.gate_mlp = _gate_struct(cfg, gate_mlp, dev)
    if cfg.gate_hidden:
        gg = {"w1": torch.empty(C, cfg.gate_hidden, dtype=f32, device=dev),
              "b1": torch.empty(cfg.gate_hidden, dtype=f32, device=dev),
              "b2": torch.empty(Hq, 3, dtype=f32, device=dev)}
        a.d_gate_mlp = _lib.nsa_gate_grads(**{kk: vv.data_ptr() for kk, vv in gg.items()})
        res["d_gate_mlp"] = gg
    if cfg.phi == "mlp":
        for tag, D in (("d_phi_k", cfg.d_k), ("d_phi_v", cfg.d_v)):
            g = {"pe": torch.empty(cfg.l, D, dtype=f32, device=dev),
                 "w1": torch.empty(cfg.l * D, cfg.hidden, dtype=f32, device=dev),
                 "b1": torch.empty(cfg.hidden, dtype=f32, device=dev),
                 "w2": torch.empty(cfg.hidden, D, dtype=f32, device=dev),
                 "b2": torch.empty(D, dtype=f32, device=dev)}
            setattr(a, tag, _lib.nsa_phi_grads(**{kk: vv.data_ptr() for kk, vv in g.items()}))
            res[tag] = g
    ws = _workspace(cfg, NSA_OP_LAYER_BWD, dev, workspace)
    p = cfg.params()
    st = _lib.load().nsa_layer_bwd(ctypes.byref(p), ctypes.byref(a), ws.data_ptr(), ws.numel(), _stream(dev))
    if st != 0:
        raise NSAError("nsa_layer_bwd", st)
    res["_workspace"] = ws
    return res


def config_from_workload(w, **over) -> Config:
    """Config for a workload description of the shared input generator."""
    c = Config(B=w.B, T=w.T, H_kv=w.H_kv, G=w.G, d_k=w.d_k, d_v=w.d_v, l=w.l, d=w.d, l_sel=w.l_sel,
               n=w.n, w=w.w, gate_dim=w.gate_dim, hidden=w.hidden, phi=w.phi, dtype=w.dtype,
               gate_hidden=getattr(w, "gate_hidden", 0),
               scale=0.0 if getattr(w, "scale_mult", 1.0) == 1.0 else w.scale_mult / math.sqrt(w.d_k))
    return dataclasses.replace(c, **over) if over else c
