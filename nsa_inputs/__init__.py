"""Seeded synthetic inputs for the Native Sparse Attention (NSA) operator.

This module is shared by the fp64 oracle's tests, the GPU parity tests and the
benchmark.  It holds workload shapes and the random-number recipe only: none of
the operator's arithmetic lives here.

Every tensor is drawn from its own torch CPU generator whose seed is derived
from ``(seed, tensor name)``, so adding a tensor never shifts another one's
values, and the values are independent of the device that later consumes them.
Values are drawn in float32 and rounded once (round-to-nearest-even) to the
workload's I/O dtype; both the GPU path and the oracle consume exactly those
rounded values.
"""
from __future__ import annotations

import dataclasses
import zlib
from typing import Dict, Optional

import torch

__all__ = ["Workload", "WORKLOADS", "workload", "make_prefill_inputs",
           "make_decode_inputs", "make_grad_output", "make_layer_inputs", "tensor_seed"]


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shapes, NSA hyper-parameters and the input distribution of one workload.

    ``T`` is the sequence length for prefill/backward and the KV-cache length
    for decode.  ``l``/``d`` are the compression block length and stride,
    ``l_sel`` the selection block length, ``n`` the number of selected blocks
    (forced ones included) and ``w`` the sliding-window size.
    """
    name: str
    mode: str                   # "prefill" | "decode" | "train"
    B: int
    T: int
    H_kv: int
    G: int
    d_k: int
    d_v: int
    phi: str                    # "mean" | "mlp"
    l: int = 32
    d: int = 16
    l_sel: int = 64
    n: int = 16
    w: int = 512
    gate_dim: int = 256
    hidden: int = 256
    dtype: str = "bf16"         # I/O dtype: "bf16" | "fp32"
    kv_offset_std: float = 0.0  # std of per-selection-block mean offsets added to K and V
    phi_std: float = 0.02       # std of phi weights and the position embedding
    bias_std: float = 0.0       # std of phi biases (0: biases start at zero)
    gate_std: float = 0.02      # std of the gate projection weights
    gate_hidden: int = 0        # 0: linear gate; else hidden width of a two-layer gate MLP
    q_group_corr: float = 0.0   # correlation between the query heads of one KV group (each stays N(0,1))
    scale_mult: float = 1.0     # softmax scale = scale_mult / sqrt(d_k)

    @property
    def H_q(self) -> int:
        return self.H_kv * self.G

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def torch_dtype(self) -> torch.dtype:
        return {"bf16": torch.bfloat16, "fp32": torch.float32}[self.dtype]


# The five workloads NSA is measured and checked on.
WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload("tiny_fp32", "prefill", B=1, T=1024, H_kv=1, G=4, d_k=64, d_v=64,
                 phi="mean", n=4, w=128, dtype="fp32"),
        Workload("prefill_8k", "prefill", B=1, T=8192, H_kv=4, G=16, d_k=128, d_v=128,
                 phi="mlp"),
        Workload("prefill_64k", "prefill", B=1, T=65536, H_kv=4, G=16, d_k=192, d_v=128,
                 phi="mlp", kv_offset_std=0.5),
        Workload("decode_64k", "decode", B=32, T=65536, H_kv=4, G=16, d_k=192, d_v=128,
                 phi="mlp", kv_offset_std=0.5),
        Workload("train_16k", "train", B=2, T=16384, H_kv=4, G=16, d_k=128, d_v=128,
                 phi="mlp"),
    ]
}


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return w.replace(**overrides) if overrides else w


def tensor_seed(seed: int, name: str) -> int:
    """Stable 63-bit seed for tensor ``name`` under master ``seed``."""
    h = zlib.crc32(f"nsa:{seed}:{name}".encode())
    return (int(seed) * 0x9E3779B1 + h) & 0x7FFFFFFFFFFFFFFF


def _normal(seed: int, name: str, shape, std: float = 1.0) -> torch.Tensor:
    g = torch.Generator(device="cpu")
    g.manual_seed(tensor_seed(seed, name))
    t = torch.randn(*shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def _kv(seed: int, name: str, w: Workload, B: int, T: int, dim: int) -> torch.Tensor:
    """N(0,1) keys/values plus, optionally, a mean-offset vector per selection block."""
    t = _normal(seed, name, (B, T, w.H_kv, dim))
    if w.kv_offset_std > 0:
        nblk = -(-T // w.l_sel)
        mu = _normal(seed, "mu_" + name, (B, nblk, w.H_kv, dim), w.kv_offset_std)
        mu = mu.repeat_interleave(w.l_sel, dim=1)[:, :T]
        t.add_(mu)
    return t


def _queries(seed: int, name: str, w: Workload, lead) -> torch.Tensor:
    """Query heads [*lead, Hq, dk], each N(0,1).  With q_group_corr = c > 0 the
    G heads of a KV group share a component: q = sqrt(c) * s_group + sqrt(1-c) * z_head,
    so heads of one group favour the same keys (peaked group-shared scores)."""
    q = _normal(seed, name, (*lead, w.H_q, w.d_k))
    c = w.q_group_corr
    if c > 0:
        s = _normal(seed, name + "_group", (*lead, w.H_kv, w.d_k))
        q.mul_((1.0 - c) ** 0.5).add_(s.repeat_interleave(w.G, dim=-2), alpha=c ** 0.5)
    return q


def _phi(seed: int, tag: str, w: Workload, dim: int) -> Dict[str, torch.Tensor]:
    """Random-init parameters of the compression MLP phi for K (dim=d_k) or V (dim=d_v).

    Layouts: pe [l, dim]; w1 [l*dim, hidden] (input index = j*dim + e for token j of
    the block and feature e); b1 [hidden]; w2 [hidden, dim]; b2 [dim].
    """
    if w.phi != "mlp":
        return {}
    out = {
        "pe": _normal(seed, tag + ".pe", (w.l, dim), w.phi_std),
        "w1": _normal(seed, tag + ".w1", (w.l * dim, w.hidden), w.phi_std),
        "w2": _normal(seed, tag + ".w2", (w.hidden, dim), w.phi_std),
    }
    if w.bias_std > 0:
        out["b1"] = _normal(seed, tag + ".b1", (w.hidden,), w.bias_std)
        out["b2"] = _normal(seed, tag + ".b2", (dim,), w.bias_std)
    else:
        out["b1"] = torch.zeros(w.hidden)
        out["b2"] = torch.zeros(dim)
    return out


def _gate(seed: int, w: Workload) -> Dict[str, object]:
    """Gate weights.  Linear gate: w_gate [gate_dim,Hq,3] ~ N(0, gate_std^2).
    Two-layer gate MLP (gate_hidden = Hg > 0): w1 [gate_dim,Hg] ~ N(0, 1/gate_dim)
    (unit-variance pre-activations for unit-variance x), b1 [Hg] and b2 [Hq,3]
    ~ N(0, 0.1^2), output layer w_gate [Hg,Hq,3] ~ N(0, 1/Hg)."""
    if not w.gate_hidden:
        return {"w_gate": _normal(seed, "w_gate", (w.gate_dim, w.H_q, 3), w.gate_std)}
    Hg = w.gate_hidden
    return {"w_gate": _normal(seed, "gate.w2", (Hg, w.H_q, 3), Hg ** -0.5),
            "gate_mlp": {"w1": _normal(seed, "gate.w1", (w.gate_dim, Hg), w.gate_dim ** -0.5),
                         "b1": _normal(seed, "gate.b1", (Hg,), 0.1),
                         "b2": _normal(seed, "gate.b2", (w.H_q, 3), 0.1)}}


def _cast(d: Dict, dt: torch.dtype) -> Dict:
    res = {}
    for k, v in d.items():
        res[k] = _cast(v, dt) if isinstance(v, dict) else v.to(dt).contiguous()
    return res


def make_prefill_inputs(w: Workload, seed: int = 0) -> Dict[str, object]:
    """Inputs of one prefill / training forward call (CPU tensors in the I/O dtype).

    q [B,T,Hq,dk], k [B,T,Hkv,dk], v [B,T,Hkv,dv], x [B,T,gate_dim],
    w_gate [gate_dim,Hq,3], phi_k / phi_v dicts (empty for mean-pool); with a
    gate MLP, w_gate [Hg,Hq,3] and gate_mlp {w1, b1, b2}.
    """
    B, T = w.B, w.T
    d = {
        "q": _queries(seed, "q", w, (B, T)),
        "k": _kv(seed, "k", w, B, T, w.d_k),
        "v": _kv(seed, "v", w, B, T, w.d_v),
        "x": _normal(seed, "x", (B, T, w.gate_dim)),
        "phi_k": _phi(seed, "phi_k", w, w.d_k),
        "phi_v": _phi(seed, "phi_v", w, w.d_v),
    }
    d.update(_gate(seed, w))
    return _cast(d, w.torch_dtype)


def make_decode_inputs(w: Workload, seed: int = 0) -> Dict[str, object]:
    """Inputs of one decode step: the query token sits at cache position T-1.

    q [B,Hq,dk], k_cache [B,T,Hkv,dk], v_cache [B,T,Hkv,dv], x [B,gate_dim],
    w_gate, phi_k / phi_v (used only to build the compressed cache).  The compressed
    caches themselves are not drawn here: they are the compression of the raw cache
    and are produced by whoever builds the cache.
    """
    B, T = w.B, w.T
    d = {
        "q": _queries(seed, "dec.q", w, (B,)),
        "k_cache": _kv(seed, "k", w, B, T, w.d_k),
        "v_cache": _kv(seed, "v", w, B, T, w.d_v),
        "x": _normal(seed, "dec.x", (B, w.gate_dim)),
        "phi_k": _phi(seed, "phi_k", w, w.d_k),
        "phi_v": _phi(seed, "phi_v", w, w.d_v),
    }
    d.update(_gate(seed, w))
    return _cast(d, w.torch_dtype)


def make_layer_inputs(w: Workload, seed: int = 0) -> Dict[str, object]:
    """Inputs of the projection layer around the operator (layer width
    C = gate_dim): h [B,T,C] ~ N(0,1); proj = {w_q [C,Hq*dk], w_k [C,Hkv*dk],
    w_v [C,Hkv*dv]} ~ N(0, 1/C), so that q, k, v have unit variance like the
    operator's own inputs, and w_o [Hq*dv,C] ~ N(0, 1/(Hq*dv)); gate and phi
    weights as for the operator; dy [B,T,C] ~ N(0,1)."""
    B, T, C = w.B, w.T, w.gate_dim
    d = {
        "h": _normal(seed, "layer.h", (B, T, C)),
        "proj": {"w_q": _normal(seed, "layer.w_q", (C, w.H_q * w.d_k), C ** -0.5),
                 "w_k": _normal(seed, "layer.w_k", (C, w.H_kv * w.d_k), C ** -0.5),
                 "w_v": _normal(seed, "layer.w_v", (C, w.H_kv * w.d_v), C ** -0.5),
                 "w_o": _normal(seed, "layer.w_o", (w.H_q * w.d_v, C), (w.H_q * w.d_v) ** -0.5)},
        "phi_k": _phi(seed, "phi_k", w, w.d_k),
        "phi_v": _phi(seed, "phi_v", w, w.d_v),
        "dy": _normal(seed, "layer.dy", (B, T, C)),
    }
    d.update(_gate(seed, w))
    return _cast(d, w.torch_dtype)


def make_grad_output(w: Workload, seed: int = 0) -> torch.Tensor:
    """Upstream gradient dO ~ N(0,1) of shape [B,T,Hq,dv] in the I/O dtype."""
    return _normal(seed, "d_o", (w.B, w.T, w.H_q, w.d_v)).to(w.torch_dtype).contiguous()


def to_numpy64(d):
    """Convert a (nested) dict of tensors to float64 numpy arrays (exact)."""
    import numpy as np
    if isinstance(d, dict):
        return {k: to_numpy64(v) for k, v in d.items()}
    return d.detach().to(torch.float64).cpu().numpy().astype(np.float64)
