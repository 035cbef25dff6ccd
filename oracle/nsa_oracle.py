"""Plain fp64 CPU oracle of Native Sparse Attention (NSA).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or run this module; the GPU library
never routes through it and shares no code with it.

It writes out, step by step and in float64 numpy, what the NSA operator
computes: the gate, token compression phi, compressed attention, the remap of
its probabilities onto selection blocks, the GQA head reduction, top-n block
selection, selected-block attention, sliding-window attention, the gated sum,
the single-token decode step and the backward pass with the selected blocks
held fixed.  Nothing is blocked, fused or reordered beyond the definitions, so
each function can be checked against the pages by eye.

Sources (web pages about the NSA paper "Native Sparse Attention:
Hardware-Aligned and Natively Trainable Sparse Attention"):

* [YLY] m.youleyou.com, "硬件对齐+原生训练！DeepSeek NSA打造高效稀疏Attention",
  section 二 (NSA核心工作): 整体框架, 令牌压缩, 重要性分数计算, Top-n块选择,
  滑动窗口, 最终输出计算; and 效率分析/解码速度.
* [XK] xookee.cn, "NSA（Natively Sparse Attention）论文原理解析" and its
  follow-on explainers: 压缩注意力机制解析 §2.1-2.4 (mean-pool / MLP
  compression, softmax(QK^T/sqrt(d_k))V), 滑动窗口注意力 §2 (window key set,
  gated sum), 三种注意力如何组合 §2 (gates g = sigmoid(MLP(X))).

Where the pages leave a step open the reading taken is stated at the step
("Reading:").  Pins: every function here is checked by tests against brute
force, closed forms or library routines (tests/test_oracle_*.py), except the
two conventions marked "parity unpinned" below: the exact architecture of the
MLP compressor phi and the remap weights for l != l' (the pages strip both
formulas; the readings are pinned only by their invariants).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np
from scipy.special import erf

__all__ = [
    "Params", "gate", "gate_logits", "compress", "remap_matrix", "attend", "n_cmp_visible",
    "candidate_blocks", "forced_blocks", "top_n", "is_near_tie", "SCORE_FLOOR", "forward",
    "decode", "append_token", "backward", "layer_forward", "layer_backward", "dq_rows", "dense_causal", "dense_causal_bwd", "round_io", "gelu", "gelu_grad", "sigmoid",
    "cmp_keys", "slc_keys", "win_keys", "decode_token_count", "dkv_keys",
]


@dataclasses.dataclass(frozen=True)
class Params:
    """NSA hyper-parameters as the oracle reads them.

    l: compression block length; d: compression stride; l_sel: selection block
    length; n: number of selected blocks, the forced ones included; w: window;
    phi: "mean" (mean-pool) or "mlp"; io: rounding applied to the stored
    compressed keys/values ("bf16", "fp32" or None for exact fp64);
    scale: softmax scale (None means 1/sqrt(d_k)).
    """
    l: int = 32
    d: int = 16
    l_sel: int = 64
    n: int = 16
    w: int = 512
    phi: str = "mlp"
    io: Optional[str] = "bf16"
    scale: Optional[float] = None


# ---------------------------------------------------------------------------
# Elementary functions
# ---------------------------------------------------------------------------

def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def gelu(a):
    """Exact (erf) GELU: a * Phi(a)."""
    return 0.5 * a * (1.0 + erf(a / math.sqrt(2.0)))


def gelu_grad(a):
    """d/da [a Phi(a)] = Phi(a) + a * phi(a)."""
    return 0.5 * (1.0 + erf(a / math.sqrt(2.0))) + a * np.exp(-0.5 * a * a) / math.sqrt(2.0 * math.pi)


def round_io(x, io: Optional[str]):
    """Round float64 values once, to nearest-even, to the I/O dtype.

    bf16 keeps 8 significant bits; fp32 keeps 24.  Reading: the compressed keys
    and values are stored tensors (the decode cache holds them), so they are
    rounded to the I/O dtype like every other stored tensor.
    """
    x = np.asarray(x, dtype=np.float64)
    if io is None:
        return x.copy()
    if io == "fp32":
        return x.astype(np.float32).astype(np.float64)
    if io == "bf16":
        m, e = np.frexp(x)                  # x = m * 2**e, 0.5 <= |m| < 1
        return np.ldexp(np.rint(m * 256.0) / 256.0, e)
    raise ValueError(io)


def _scale(p: Params, d_k: int) -> float:
    return p.scale if p.scale is not None else 1.0 / math.sqrt(d_k)


# ---------------------------------------------------------------------------
# Gate  [YLY 整体框架: gate scores from the input features through an MLP and a
# sigmoid; XK 三种注意力如何组合 §2: g = sigmoid(MLP(X))]
# Reading: one gate per (token, query head, branch), c = (cmp, slc, win).  The
# pages leave the MLP's depth open; two forms are computed:
#   linear (default): g[b,t,h,c] = sigmoid(x[b,t,:] . W_g[:,h,c]), no bias;
#   two-layer MLP:    a = x W1 + b1, u = gelu(a) (erf form, as the compression
#                     MLP), g = sigmoid(u W_g + b2), W_g [Hg,Hq,3].
# ---------------------------------------------------------------------------

def gate_logits(x, w_gate, mlp: Optional[Dict[str, np.ndarray]] = None):
    """Pre-sigmoid gate logits z [...,Hq,3] of x [...,C], and the MLP's hidden
    pre-activation a [...,Hg] and activation u (None for the linear gate)."""
    if mlp is None:
        return np.einsum("...c,chk->...hk", x, w_gate), None, None
    a = np.einsum("...c,cj->...j", x, mlp["w1"]) + mlp["b1"]
    u = gelu(a)
    z = np.einsum("...j,jhk->...hk", u, w_gate) + mlp["b2"]
    return z, a, u


def gate(x, w_gate, mlp: Optional[Dict[str, np.ndarray]] = None):
    """x [B,T,C], w_gate [C,Hq,3] (linear) or [Hg,Hq,3] with mlp = {w1 [C,Hg],
    b1 [Hg], b2 [Hq,3]} -> g [B,T,Hq,3]."""
    return sigmoid(gate_logits(x, w_gate, mlp)[0])


# ---------------------------------------------------------------------------
# Token compression  [YLY 令牌压缩: blocks of length l slid with stride d, each
# mapped by a learnable MLP with intra-block position encoding to one
# compressed key; likewise values.  XK 压缩注意力 §2.2-2.3: mean pooling or MLP]
# Reading: block i covers tokens [i*d, i*d + l); only complete blocks exist.
# ---------------------------------------------------------------------------

def n_cmp_visible(t: int, l: int, d: int) -> int:
    """Number of complete compression blocks whose last token is <= t."""
    s = t + 1
    return 0 if s < l else (s - l) // d + 1


def compress(kv, phi: Dict[str, np.ndarray], p: Params):
    """kv [B,T,H,D] -> [B,N,H,D] with N = n_cmp_visible(T-1).

    mean: (1/l) * sum_j kv[i*d + j].
    mlp (parity unpinned as an architecture: the pages name only "MLP with
    intra-block position encoding"): u = concat_j (kv[i*d+j] + pe[j]) (token j
    major, feature minor), out = W2^T gelu(W1^T u + b1) + b2 with w1 [l*D, hidden],
    w2 [hidden, D].  The same phi serves every KV head.
    The result is rounded to the I/O dtype.
    """
    B, T, H, D = kv.shape
    N = n_cmp_visible(T - 1, p.l, p.d)
    out = np.zeros((B, N, H, D))
    for i in range(N):
        blk = kv[:, i * p.d: i * p.d + p.l]           # [B,l,H,D]
        if p.phi == "mean":
            out[:, i] = blk.mean(axis=1)
        else:
            u = (blk + phi["pe"][None, :, None, :])    # [B,l,H,D]
            u = np.transpose(u, (0, 2, 1, 3)).reshape(B, H, p.l * D)
            a = u @ phi["w1"] + phi["b1"]
            out[:, i] = gelu(a) @ phi["w2"] + phi["b2"]
    return round_io(out, p.io)


# ---------------------------------------------------------------------------
# Attention over one key set  [XK 压缩注意力 §2.4, 滑动窗口 §2: softmax(q K^T /
# sqrt(d_k)) V].  An empty key set yields O = 0 and lse = -inf.
# ---------------------------------------------------------------------------

def attend(qh, K, V, scale: float):
    """qh [H,dk], K [N,dk], V [N,dv] -> (O [H,dv], lse [H], P [H,N])."""
    H = qh.shape[0]
    if K.shape[0] == 0:
        return np.zeros((H, V.shape[1])), np.full(H, -np.inf), np.zeros((H, 0))
    z = scale * (qh @ K.T)
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    s = e.sum(axis=1, keepdims=True)
    P = e / s
    return P @ V, (m + np.log(s))[:, 0], P


# ---------------------------------------------------------------------------
# Key sets of the three branches at query position t.
# ---------------------------------------------------------------------------

def cmp_keys(t: int, p: Params) -> np.ndarray:
    """Compressed blocks visible at t: those complete at or before t."""
    return np.arange(n_cmp_visible(t, p.l, p.d))


def slc_keys(t: int, blocks: Sequence[int], p: Params) -> np.ndarray:
    """Tokens of the selected blocks, concatenated, with a token-level causal mask.

    [YLY Top-n块选择: the selected keys are the concatenation of the chosen
    blocks' tokens].  Reading: tokens after t are masked.
    """
    toks = [np.arange(j * p.l_sel, min((j + 1) * p.l_sel, t + 1)) for j in sorted(blocks)]
    return np.concatenate(toks) if toks else np.zeros(0, dtype=np.int64)


def win_keys(t: int, p: Params) -> np.ndarray:
    """[YLY 滑动窗口; XK 滑动窗口 §2: only the most recent w tokens].

    Reading: w keys, positions [max(0, t-w+1), t].
    """
    return np.arange(max(0, t - p.w + 1), t + 1)


# ---------------------------------------------------------------------------
# Importance scores  [YLY 重要性分数计算]: the compressed branch's softmax
# probabilities are reused.  When compression and selection blocking differ
# (l <= l', d | l, d | l') they are remapped onto selection blocks.
# Reading (remap weights parity unpinned: the formula is stripped from the
# page): selection block j receives from compression block i the overlap of
# their token ranges in units of d,
#     W[i, j] = |[i*d, i*d+l) ∩ [j*l', (j+1)*l')| / d,
# which is the double sum over m < l'/d and r < l/d of p_cmp[(l'/d) j + m - r],
# and the identity when l = l' = d.
# ---------------------------------------------------------------------------

def remap_matrix(n_cmp: int, n_sel: int, p: Params) -> np.ndarray:
    i = np.arange(n_cmp)[:, None]
    j = np.arange(n_sel)[None, :]
    a0, a1 = i * p.d, i * p.d + p.l                 # compression block token range
    b0, b1 = j * p.l_sel, (j + 1) * p.l_sel         # selection block token range
    ov = np.maximum(0, np.minimum(a1, b1) - np.maximum(a0, b0))
    return ov / p.d


# ---------------------------------------------------------------------------
# Top-n block selection  [YLY Top-n块选择: keep the blocks ranked highest by
# the group-shared importance score; the n selected blocks include 1 initial
# block and 2 local blocks that are always active (实验设置)].
# Readings: candidates are the causal blocks j <= floor(t/l'); the forced set is
# {0, floor(t/l'), floor(t/l') - 1} among the candidates; the remaining slots
# go to the best other candidates ranked by (-score, j), so the lower block
# index wins a tie; when there are at most n candidates all are selected.
# ---------------------------------------------------------------------------

def candidate_blocks(t: int, p: Params) -> List[int]:
    return list(range(t // p.l_sel + 1))


def forced_blocks(t: int, p: Params) -> List[int]:
    jc = t // p.l_sel
    return sorted({j for j in (0, jc, jc - 1) if 0 <= j <= jc})


def _ranked_rest(scores, t: int, p: Params) -> List[int]:
    F = set(forced_blocks(t, p))
    rest = [j for j in candidate_blocks(t, p) if j not in F]
    return sorted(rest, key=lambda j: (-scores[j], j))


def top_n(scores, t: int, p: Params) -> List[int]:
    """Selected block set at position t (ascending) from one group's score row."""
    J = candidate_blocks(t, p)
    if len(J) <= p.n:
        return J
    F = forced_blocks(t, p)
    r = p.n - len(F)
    return sorted(F + _ranked_rest(scores, t, p)[:r])


# Smallest score an fp32 kernel still resolves to 1e-3: scores are sums of
# probabilities (each head's row sums to 1); below 2^-100 a score's terms sit
# at or under fp32's normal range, so two such scores count as a tie.
SCORE_FLOOR = 2.0 ** -100


def is_near_tie(scores, t: int, p: Params, rel: float = 1e-3, floor: float = SCORE_FLOOR) -> bool:
    """True when the last selected and first unselected ranked scores are within
    ``rel`` of the larger one, so that rounding may legitimately swap them, or
    when both lie below ``floor`` (indistinguishable from 0 in fp32 arithmetic)."""
    J = candidate_blocks(t, p)
    if len(J) <= p.n:
        return False
    r = p.n - len(forced_blocks(t, p))
    rest = _ranked_rest(scores, t, p)
    if r <= 0 or len(rest) <= r:
        return False
    a, b = scores[rest[r - 1]], scores[rest[r]]
    big = max(abs(a), abs(b))
    return abs(a - b) <= rel * big or big < floor


def decode_token_count(s: int, p: Params) -> int:
    """Tokens one decode step loads per KV group in the pages' memory model
    [YLY 效率分析/解码速度]: floor((s-l)/d) compressed + n*l' selected + w window."""
    return (s - p.l) // p.d + p.n * p.l_sel + p.w


# ---------------------------------------------------------------------------
# One query position, all heads  [YLY 整体框架 and 最终输出计算:
# o_t = sum over c in {cmp, slc, win} of g_t^c * Attn(q_t, K_t^c, V_t^c)]
# ---------------------------------------------------------------------------

def _row(p: Params, t: int, q_t, k, v, kc, vc, g_t, n_sel: int,
         sel: Optional[List[List[int]]] = None, tie_scores=None, W_full=None, kv_win=None):
    """All NSA quantities at position t of one sequence.

    q_t [Hq,dk]; k [*,Hkv,dk], v [*,Hkv,dv] raw keys/values of the selected
    branch (positions <= t used); kv_win: the window branch's own (k, v), by
    default the same; kc, vc compressed keys/values [*,Hkv,*]; g_t [Hq,3] gates.
    sel: optional fixed block sets per KV head.  tie_scores: optional [Hkv,n_sel]
    score rows used for selection instead of the oracle's own where the oracle's
    own row is a near tie.
    """
    Hq, dk = q_t.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    dv = v.shape[2]
    sc = _scale(p, dk)
    ic = cmp_keys(t, p)
    W = (W_full if W_full is not None else remap_matrix(len(ic), n_sel, p))[:len(ic)]
    o_br = np.zeros((3, Hq, dv))
    lse = np.zeros((3, Hq))
    p_slc = np.zeros((Hkv, n_sel))
    sets, retied = [], []
    for g in range(Hkv):
        hs = slice(g * G, (g + 1) * G)
        # compressed branch; its probabilities are the importance scores
        o_br[0, hs], lse[0, hs], P = attend(q_t[hs], kc[ic, g], vc[ic, g], sc)
        # remap onto selection blocks, then sum over the group's query heads
        p_slc[g] = (P @ W).sum(axis=0)
        if sel is not None:
            S = [j for j in sel[g] if j >= 0]
            retied.append(False)
        elif tie_scores is not None and is_near_tie(p_slc[g], t, p):
            S = top_n(tie_scores[g], t, p)
            retied.append(True)
        else:
            S = top_n(p_slc[g], t, p)
            retied.append(False)
        sets.append(S)
        ks = slc_keys(t, S, p)
        o_br[1, hs], lse[1, hs], _ = attend(q_t[hs], k[ks, g], v[ks, g], sc)
        kw = win_keys(t, p)
        k_w, v_w = (k, v) if kv_win is None else kv_win
        o_br[2, hs], lse[2, hs], _ = attend(q_t[hs], k_w[kw, g], v_w[kw, g], sc)
    o = (g_t[:, :, None] * np.transpose(o_br, (1, 0, 2))).sum(axis=1)
    return o, o_br, lse, p_slc, sets, retied


def _sets_to_idx(sets: List[List[int]], n: int) -> np.ndarray:
    out = np.full((len(sets), n), -1, dtype=np.int64)
    for g, S in enumerate(sets):
        out[g, :len(S)] = sorted(S)
    return out


def forward(p: Params, q, k, v, x, w_gate, phi_k=None, phi_v=None, rows=None,
            idx=None, tie_scores=None, kc=None, vc=None, kv_slc=None, kv_win=None,
            gate_mlp=None) -> Dict[str, np.ndarray]:
    """NSA prefill forward.

    q [B,T,Hq,dk], k [B,T,Hkv,dk], v [B,T,Hkv,dv], x [B,T,C], w_gate [C,Hq,3].
    kv_slc, kv_win: optional (k, v) pairs of the selected and window branches
    [YLY 滑动窗口: each branch may have its own keys and values so that the
    branches' gradients do not interfere]; k, v then feed the compressed branch
    only.  Default: one k, v for all three.
    rows: query positions to evaluate (default all).  idx: optional fixed block
    indices [B,T,Hkv,n] (-1 padded), used instead of top-n.  tie_scores: optional
    [B,T,Hkv,N_sel] score rows consulted only where the oracle's own row is a near
    tie.  kc, vc: optional precomputed compressed keys/values.  gate_mlp:
    optional {w1, b1, b2} of a two-layer gate MLP (w_gate is then its output
    layer [Hg,Hq,3]).

    Returns o [B,R,Hq,dv], o_branch [3,B,R,Hq,dv], lse [3,B,R,Hq],
    p_slc [B,R,Hkv,N_sel], idx [B,R,Hkv,n], retied [B,R,Hkv], gates [B,R,Hq,3],
    k_cmp, v_cmp, rows.
    """
    B, T, Hq, dk = q.shape
    Hkv, dv = k.shape[2], v.shape[3]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    R = len(rows)
    n_sel = -(-T // p.l_sel)
    if kc is None:
        kc = compress(k, phi_k, p)
    if vc is None:
        vc = compress(v, phi_v, p)
    g_all = gate(x[:, rows], w_gate, gate_mlp)
    W_full = remap_matrix(kc.shape[1], n_sel, p)
    out = {
        "o": np.zeros((B, R, Hq, dv)), "o_branch": np.zeros((3, B, R, Hq, dv)),
        "lse": np.zeros((3, B, R, Hq)), "p_slc": np.zeros((B, R, Hkv, n_sel)),
        "idx": np.full((B, R, Hkv, p.n), -1, dtype=np.int64),
        "retied": np.zeros((B, R, Hkv), dtype=bool), "gates": g_all,
        "k_cmp": kc, "v_cmp": vc, "rows": rows,
    }
    for b in range(B):
        for r, t in enumerate(rows):
            sel = None if idx is None else [list(idx[b, t, g]) for g in range(Hkv)]
            ts = None if tie_scores is None else tie_scores[b, t]
            k_s, v_s = (k, v) if kv_slc is None else kv_slc
            kvw = None if kv_win is None else (kv_win[0][b], kv_win[1][b])
            o, o_br, lse, ps, sets, ret = _row(p, int(t), q[b, t], k_s[b], v_s[b], kc[b], vc[b],
                                               g_all[b, r], n_sel, sel, ts, W_full, kvw)
            out["o"][b, r] = o
            out["o_branch"][:, b, r] = o_br
            out["lse"][:, b, r] = lse
            out["p_slc"][b, r] = ps
            out["idx"][b, r] = _sets_to_idx(sets, p.n)
            out["retied"][b, r] = ret
    return out


def decode(p: Params, q, k_cache, v_cache, kc_cache, vc_cache, x, w_gate,
           tie_scores=None, seq_lens=None, kv_win_cache=None, gate_mlp=None) -> Dict[str, np.ndarray]:
    """One decode step: the query token sits at position S-1 of a length-S cache,
    its own key/value already stored there; compressed blocks come from the
    given compressed cache (complete blocks only), not from phi.

    q [B,Hq,dk], k_cache [B,S,Hkv,dk], v_cache [B,S,Hkv,dv], kc_cache [B,>=N,Hkv,dk],
    vc_cache [B,>=N,Hkv,dv], x [B,C].  Returns o [B,Hq,dv], o_branch [3,B,Hq,dv],
    lse [3,B,Hq], p_slc [B,Hkv,N_sel], idx [B,Hkv,n], retied [B,Hkv].
    seq_lens [B] (optional): sequence b holds only its first seq_lens[b] cache
    rows, and its query sits at seq_lens[b]-1; p_slc keeps the width of the full
    cache, zero beyond the sequence's own blocks.  kv_win_cache: optional
    (k, v) caches of the window branch when it has its own keys and values
    (k_cache, v_cache then serve the selected branch only).  gate_mlp: as in
    forward.
    """
    B, S = k_cache.shape[:2]
    Hq, dv = q.shape[1], v_cache.shape[3]
    Hkv = k_cache.shape[2]
    n_sel = -(-S // p.l_sel)
    g_all = gate(x[:, None], w_gate, gate_mlp)[:, 0]
    out = {"o": np.zeros((B, Hq, dv)), "o_branch": np.zeros((3, B, Hq, dv)),
           "lse": np.zeros((3, B, Hq)), "p_slc": np.zeros((B, Hkv, n_sel)),
           "idx": np.full((B, Hkv, p.n), -1, dtype=np.int64),
           "retied": np.zeros((B, Hkv), dtype=bool), "gates": g_all}
    for b in range(B):
        Sb = S if seq_lens is None else int(seq_lens[b])
        nb = -(-Sb // p.l_sel)
        ts = None if tie_scores is None else tie_scores[b]
        kvw = None if kv_win_cache is None else (kv_win_cache[0][b, :Sb], kv_win_cache[1][b, :Sb])
        o, o_br, lse, ps, sets, ret = _row(p, Sb - 1, q[b], k_cache[b, :Sb], v_cache[b, :Sb], kc_cache[b],
                                           vc_cache[b], g_all[b], nb, None, ts, None, kvw)
        out["o"][b], out["o_branch"][:, b], out["lse"][:, b] = o, o_br, lse
        out["p_slc"][b, :, :nb], out["idx"][b], out["retied"][b] = ps, _sets_to_idx(sets, p.n), ret
    return out


def append_token(p: Params, k_cache, v_cache, kc_cache, vc_cache, k_new, v_new, seq_lens,
                 phi_k=None, phi_v=None):
    """Decode-time cache maintenance [YLY 令牌压缩: block i covers tokens
    i*d .. i*d+l-1 and exists once its last token does].

    For every sequence b with L = seq_lens[b] < capacity: the new token's key and
    value go to cache row L; if that token completes block i (L+1 >= l and
    (L+1-l) % d == 0, i = (L+1-l)/d), row i of the compressed caches becomes
    phi of that block, computed by compress() on the block's l tokens.
    Returns updated copies of the four caches; seq_lens is not advanced.
    """
    k_cache, v_cache = k_cache.copy(), v_cache.copy()
    kc_cache, vc_cache = kc_cache.copy(), vc_cache.copy()
    S = k_cache.shape[1]
    for b in range(k_cache.shape[0]):
        L = int(seq_lens[b])
        if not 0 <= L < S:
            continue
        k_cache[b, L], v_cache[b, L] = k_new[b], v_new[b]
        n = L + 1 - p.l
        if n < 0 or n % p.d:
            continue
        i = n // p.d
        blk = slice(i * p.d, i * p.d + p.l)
        kc_cache[b, i] = compress(k_cache[b:b + 1, blk], phi_k, p)[0, 0]
        vc_cache[b, i] = compress(v_cache[b:b + 1, blk], phi_v, p)[0, 0]
    return k_cache, v_cache, kc_cache, vc_cache


# ---------------------------------------------------------------------------
# Backward with the selected blocks held fixed (no gradient flows through the
# scores or the discrete selection).  Per branch c, with dO_c = g_c * dO:
#   dV += P^T dO_c;  dP = dO_c V^T;  D = rowsum(dO_c * O_c);  dS = P * (dP - D)
#   dq += scale * dS K;  dK += scale * dS^T q
# Gate: dg_c = <dO, O_c>, dz = dg * g * (1 - g); linear gate: dW_g = x^T dz,
# dx = dz W_g^T; gate MLP: dW_g = u^T dz, db2 = sum dz, du = dz W_g^T,
# da = du * gelu'(a), dW1 = x^T da, db1 = sum da, dx = da W1^T.
# Compressed-branch dK_cmp / dV_cmp flow back through phi to k / v and to the
# phi parameters.  Rounding of the stored compressed tensors is not
# differentiated (use io=None when comparing with finite differences).
# ---------------------------------------------------------------------------

def _attend_bwd(qh, K, V, P, O, dOc, scale):
    dV = P.T @ dOc
    dP = dOc @ V.T
    D = (dOc * O).sum(axis=1, keepdims=True)
    dS = P * (dP - D)
    return scale * dS @ K, scale * dS.T @ qh, dV


def _phi_bwd(kv, phi, dout, p: Params):
    """Gradients of compress() w.r.t. its input and parameters (no rounding)."""
    B, T, H, D = kv.shape
    N = dout.shape[1]
    dkv = np.zeros_like(kv)
    grads = {}
    if p.phi == "mean":
        for i in range(N):
            dkv[:, i * p.d: i * p.d + p.l] += dout[:, i][:, None] / p.l
        return dkv, grads
    for key in ("pe", "w1", "b1", "w2", "b2"):
        grads[key] = np.zeros_like(phi[key])
    for i in range(N):
        blk = kv[:, i * p.d: i * p.d + p.l] + phi["pe"][None, :, None, :]
        u = np.transpose(blk, (0, 2, 1, 3)).reshape(B * H, p.l * D)
        a = u @ phi["w1"] + phi["b1"]
        hh = gelu(a)
        do = dout[:, i].reshape(B * H, D)
        grads["b2"] += do.sum(axis=0)
        grads["w2"] += hh.T @ do
        da = (do @ phi["w2"].T) * gelu_grad(a)
        grads["w1"] += u.T @ da
        grads["b1"] += da.sum(axis=0)
        du = (da @ phi["w1"].T).reshape(B, H, p.l, D)
        du = np.transpose(du, (0, 2, 1, 3))           # [B,l,H,D]
        dkv[:, i * p.d: i * p.d + p.l] += du
        grads["pe"] += du.sum(axis=(0, 2))
    return dkv, grads


# ---------------------------------------------------------------------------
# Projection layer around the operator [XK 三种注意力如何组合 §2: the module
# projects its input to queries, keys and values, runs the three branches,
# gates them from the same input and projects the result; YLY 整体框架].
# Reading: q = h W_q, k = h W_k, v = h W_v and the attention output o are
# stored tensors, rounded to the I/O dtype (R16); the gate input is h;
# y = o W_o, rounded likewise.  Backward: dO = dy W_o^T rounded to the I/O
# dtype (the operator takes dO as a stored tensor), dW_o = o^T dy, then the
# operator's backward, dW_p = h^T d_p and dh = dx + sum_p d_p W_p^T for
# p in (q, k, v).
# ---------------------------------------------------------------------------

def layer_forward(p: Params, h, proj: Dict[str, np.ndarray], w_gate, n_heads, phi_k=None, phi_v=None,
                  gate_mlp=None, tie_scores=None, idx=None) -> Dict[str, np.ndarray]:
    """h [B,T,C]; proj = {w_q [C,Hq*dk], w_k [C,Hkv*dk], w_v [C,Hkv*dv],
    w_o [Hq*dv,C]}; n_heads = (Hq, Hkv).  idx: optional fixed block indices
    (as in forward).  Returns y [B,T,C], q, k, v, o (as stored) and the
    operator's forward result under "nsa"."""
    B, T, C = h.shape
    Hq, Hkv = n_heads
    dk = proj["w_q"].shape[1] // Hq
    dv = proj["w_o"].shape[0] // Hq
    q = round_io(h @ proj["w_q"], p.io).reshape(B, T, Hq, dk)
    k = round_io(h @ proj["w_k"], p.io).reshape(B, T, Hkv, dk)
    v = round_io(h @ proj["w_v"], p.io).reshape(B, T, Hkv, dv)
    f = forward(p, q, k, v, h, w_gate, phi_k, phi_v, idx=idx, tie_scores=tie_scores, gate_mlp=gate_mlp)
    o = round_io(f["o"], p.io)
    y = round_io(o.reshape(B, T, Hq * dv) @ proj["w_o"], p.io)
    return {"y": y, "q": q, "k": k, "v": v, "o": o, "nsa": f}


def layer_backward(p: Params, h, proj: Dict[str, np.ndarray], w_gate, n_heads, phi_k, phi_v, dy, idx,
                   gate_mlp=None) -> Dict[str, object]:
    """Gradients of L = sum(dy * y) with the block indices idx fixed: dh,
    dw_q, dw_k, dw_v, dw_o, and the operator's own (dw_gate, dgate_mlp,
    dphi_k, dphi_v).  The forward that gives o for dw_o runs with the same
    fixed idx, the selection the whole backward holds fixed."""
    B, T, C = h.shape
    f = layer_forward(p, h, proj, w_gate, n_heads, phi_k, phi_v, gate_mlp, idx=idx)
    Hq = n_heads[0]
    dv = proj["w_o"].shape[0] // Hq
    o2 = f["o"].reshape(B * T, -1)
    dy2 = dy.reshape(B * T, C)
    d_o = round_io(dy2 @ proj["w_o"].T, p.io).reshape(B, T, Hq, dv)
    g = backward(p, f["q"], f["k"], f["v"], h, w_gate, phi_k, phi_v, d_o, idx, gate_mlp=gate_mlp)
    h2 = h.reshape(B * T, C)
    out = {"dw_o": o2.T @ dy2, "dw_gate": g["dw_gate"], "dgate_mlp": g["dgate_mlp"],
           "dphi_k": g["dphi_k"], "dphi_v": g["dphi_v"]}
    dh = g["dx"].reshape(B * T, C).copy()
    for name, d in (("q", g["dq"]), ("k", g["dk"]), ("v", g["dv"])):
        d2 = d.reshape(B * T, -1)
        out["dw_" + name] = h2.T @ d2
        dh += d2 @ proj["w_" + name].T
    out["dh"] = dh.reshape(B, T, C)
    return out


def dense_causal(q, k, v, scale=None):
    """Dense causal attention, the baseline NSA's speed is measured against
    [YLY 效率分析]: query head h of KV head h // G attends to every key j <= t.

    q [B,T,Hq,dk], k [B,T,Hkv,dk], v [B,T,Hkv,dv] -> o [B,T,Hq,dv], lse [B,T,Hq]
    (natural log).
    """
    B, T, Hq, dk = q.shape
    Hkv, dv = k.shape[2], v.shape[3]
    G = Hq // Hkv
    sc = 1.0 / np.sqrt(dk) if scale is None else scale
    o = np.zeros((B, T, Hq, dv))
    lse = np.zeros((B, T, Hq))
    causal = np.tril(np.ones((T, T), dtype=bool))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            s = sc * (q[b, :, h] @ k[b, :, g].T)
            s = np.where(causal, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            l_ = e.sum(axis=1, keepdims=True)
            o[b, :, h] = (e @ v[b, :, g]) / l_
            lse[b, :, h] = (m + np.log(l_))[:, 0]
    return o, lse


def dense_causal_bwd(q, k, v, d_o, scale=None, o=None):
    """Gradients of L = sum(d_o * O) for O = dense_causal(q, k, v): the
    textbook attention backward per head, dV = P^T dO, dP = dO V^T,
    D = rowsum(dO * O), dS = P (dP - D), dq = scale dS K, dK = scale dS^T q,
    key/value gradients summed over the query heads of each KV head.
    o: the forward output to form D from (default: the exact one).
    Returns dq, dk, dv.
    """
    B, T, Hq, dk = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    sc = 1.0 / np.sqrt(dk) if scale is None else scale
    if o is None:
        o, _ = dense_causal(q, k, v, sc)
    dq, dkk, dvv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    causal = np.tril(np.ones((T, T), dtype=bool))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            s = np.where(causal, sc * (q[b, :, h] @ k[b, :, g].T), -np.inf)
            P = np.exp(s - s.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            dO = d_o[b, :, h]
            dvv[b, :, g] += P.T @ dO
            D = (dO * o[b, :, h]).sum(axis=1, keepdims=True)
            dS = P * (dO @ v[b, :, g].T - D)
            dq[b, :, h] = sc * dS @ k[b, :, g]
            dkk[b, :, g] += sc * dS.T @ q[b, :, h]
    return dq, dkk, dvv


def dq_rows(p: Params, q_rows, k, v, kc, vc, g_rows, d_o_rows, idx_rows, rows, kv_win=None) -> np.ndarray:
    """dq of the given query positions only (the same per-row arithmetic as
    backward(): dq_t depends on row t and the keys/values it attends).

    q_rows [B,R,Hq,dk], d_o_rows [B,R,Hq,dv], g_rows [B,R,Hq,3] gates, idx_rows
    [B,R,Hkv,n]; k, v raw and kc, vc compressed keys/values of whole sequences;
    kv_win: optional own (k, v) of the window branch (k, v then serve the
    selected branch).
    """
    B, R, Hq, dk_ = q_rows.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    sc = _scale(p, dk_)
    dq = np.zeros_like(q_rows)
    for b in range(B):
        for r, t in enumerate(rows):
            t = int(t)
            for g in range(Hkv):
                hs = slice(g * G, (g + 1) * G)
                qh, dO, gg = q_rows[b, r, hs], d_o_rows[b, r, hs], g_rows[b, r, hs]
                branches = [
                    (kc[b, :, g], vc[b, :, g], cmp_keys(t, p)),
                    (k[b, :, g], v[b, :, g], slc_keys(t, [j for j in idx_rows[b, r, g] if j >= 0], p)),
                    ((k if kv_win is None else kv_win[0])[b, :, g], (v if kv_win is None else kv_win[1])[b, :, g],
                     win_keys(t, p)),
                ]
                for c, (KK, VV, keys) in enumerate(branches):
                    if len(keys) == 0:
                        continue
                    K, V = KK[keys], VV[keys]
                    O, _, P = attend(qh, K, V, sc)
                    dqh, _, _ = _attend_bwd(qh, K, V, P, O, gg[:, c:c + 1] * dO, sc)
                    dq[b, r, hs] += dqh
    return dq


def dkv_keys(p: Params, q, k, v, g_all, d_o, idx, keys, phi_k=None, phi_v=None, pairs=None, tie_scores=None):
    """Key/value gradients at the sampled token positions ``keys`` of the
    (sequence, KV head) pairs ``pairs`` (None: every pair), plus phi's
    parameter gradients: the same per-row arithmetic as backward(), restricted
    to the rows that reach those tokens.

    Every row contributes its compressed branch: every block's dK_cmp, dV_cmp
    is needed, since phi's gradients sum over all blocks and a token's gradient
    through phi comes from the blocks that contain it.  Rows that see the same
    compressed blocks (the d consecutive positions between two block ends) are
    stacked into one product; each row's softmax is still its own.  The
    selected branch is evaluated for the rows that selected a block holding a
    sampled token at or before the row; the window branch for the rows whose
    window holds one.

    q [B,T,Hq,dk], k, v [B,T,Hkv,*], g_all [B,T,Hq,3] gates, d_o [B,T,Hq,dv],
    idx [B,T,Hkv,n] the selected blocks, or None: then every row's selection is
    made here from the compressed branch's probabilities, as forward() does
    (tie_scores [B,T,Hkv,N_sel] consulted on near ties only), and returned.
    Returns dk, dv [B,len(keys),Hkv,*] (the sum over the three branches, as
    backward()'s dk, dv at those tokens; NaN for pairs not asked for), dk_cmp,
    dv_cmp [B,Ncmp,Hkv,*], dphi_k, dphi_v and idx (-1 rows for pairs not asked
    for when the selection was made here).
    """
    B, T, Hq, dk_ = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    sc = _scale(p, dk_)
    keys = [int(s) for s in keys]
    pairs = {(b, g) for b in range(B) for g in range(Hkv)} if pairs is None else {tuple(x) for x in pairs}
    pos = {s: r for r, s in enumerate(keys)}
    kc = compress(k, phi_k, p)
    vc = compress(v, phi_v, p)
    dkc, dvc = np.zeros_like(kc), np.zeros_like(vc)
    dk_s = np.zeros((B, len(keys), Hkv, k.shape[3]))
    dv_s = np.zeros((B, len(keys), Hkv, v.shape[3]))
    blocks_of = {}
    for s in keys:
        blocks_of.setdefault(s // p.l_sel, []).append(s)
    own_sel = idx is None
    if own_sel:
        idx = np.full((B, T, Hkv, p.n), -1, dtype=np.int64)
        for b, g in pairs:
            for t in range(T):
                if n_cmp_visible(t, p.l, p.d) == 0:
                    # no complete compressed block: every causal block (at most
                    # one, so fewer than n candidates)
                    idx[b, t, g] = _sets_to_idx([top_n(np.zeros(t // p.l_sel + 1), t, p)], p.n)[0]
    # compressed branch: runs of rows with the same visible blocks
    runs = {}
    for t in range(T):
        runs.setdefault(n_cmp_visible(t, p.l, p.d), []).append(t)
    for b in range(B):
        for g in range(Hkv):
            hs = slice(g * G, (g + 1) * G)
            for nv, ts in runs.items():
                if nv == 0:
                    continue
                K, V = kc[b, :nv, g], vc[b, :nv, g]
                qh = q[b, ts, hs].reshape(-1, dk_)
                dOc = (g_all[b, ts, hs, 0:1] * d_o[b, ts, hs]).reshape(len(ts) * G, -1)
                O, _, P = attend(qh, K, V, sc)
                _, dK, dV = _attend_bwd(qh, K, V, P, O, dOc, sc)
                dkc[b, :nv, g] += dK
                dvc[b, :nv, g] += dV
                if own_sel and (b, g) in pairs:
                    # importance scores and top-n of each row, as in forward()
                    W = remap_matrix(nv, ts[-1] // p.l_sel + 1, p)
                    for r, t in enumerate(ts):
                        ns = t // p.l_sel + 1
                        scores = (P[r * G:(r + 1) * G] @ W[:, :ns]).sum(axis=0)
                        if tie_scores is not None and is_near_tie(scores, t, p):
                            S = top_n(tie_scores[b, t, g], t, p)
                        else:
                            S = top_n(scores, t, p)
                        idx[b, t, g] = _sets_to_idx([S], p.n)[0]
    # selected and window branches of the asked pairs
    for b, g in sorted(pairs):
        hs = slice(g * G, (g + 1) * G)
        for t in range(T):
            qh, dO, gg = q[b, t, hs], d_o[b, t, hs], g_all[b, t, hs]
            sel = [j for j in idx[b, t, g] if j >= 0]
            in_slc = [s for j in sel for s in blocks_of.get(j, []) if s <= t]
            in_win = [s for s in keys if t - p.w + 1 <= s <= t]
            for c, kidx, wanted in ((1, slc_keys(t, sel, p), in_slc), (2, win_keys(t, p), in_win)):
                if not wanted:
                    continue
                K, V = k[b, kidx, g], v[b, kidx, g]
                O, _, P = attend(qh, K, V, sc)
                _, dK, dV = _attend_bwd(qh, K, V, P, O, gg[:, c:c + 1] * dO, sc)
                at = np.searchsorted(kidx, wanted)     # key lists are ascending
                for s, i in zip(wanted, at):
                    dk_s[b, pos[s], g] += dK[i]
                    dv_s[b, pos[s], g] += dV[i]
    dk_phi, dphi_k = _phi_bwd(k, phi_k, dkc, p)
    dv_phi, dphi_v = _phi_bwd(v, phi_v, dvc, p)
    dk_s += dk_phi[:, keys]
    dv_s += dv_phi[:, keys]
    for b in range(B):
        for g in range(Hkv):
            if (b, g) not in pairs:
                dk_s[b, :, g] = np.nan
                dv_s[b, :, g] = np.nan
    return {"dk": dk_s, "dv": dv_s, "dk_cmp": dkc, "dv_cmp": dvc, "dphi_k": dphi_k, "dphi_v": dphi_v,
            "idx": idx}


def backward(p: Params, q, k, v, x, w_gate, phi_k, phi_v, d_o, idx, kv_slc=None, kv_win=None,
             gate_mlp=None) -> Dict[str, object]:
    """Gradients of L = sum(d_o * O) with block indices idx [B,T,Hkv,n] fixed.

    Returns dq, dk, dv, dw_gate, dphi_k, dphi_v (dicts keyed like phi), and the
    per-branch parts of the key/value gradients: dk_phi, dv_phi (through phi,
    the compressed branch), dk_slc, dv_slc, dk_win, dv_win.  With one k, v for
    all branches dk = dk_phi + dk_slc + dk_win (dv alike).  With kv_slc, kv_win
    (independent keys/values per branch, as in forward) dk, dv are the
    compressed branch's part only and the others are the gradients of the
    branches' own tensors.  Gate: dw_gate (the output layer's gradient when
    gate_mlp is given, which adds dgate_mlp = {w1, b1, b2}) and dx, the
    gradient with respect to the gate input x.
    """
    B, T, Hq, dk_ = q.shape
    Hkv, dv_ = k.shape[2], v.shape[3]
    G = Hq // Hkv
    sc = _scale(p, dk_)
    kc = compress(k, phi_k, p)
    vc = compress(v, phi_v, p)
    z_all, a_gate, u_gate = gate_logits(x, w_gate, gate_mlp)
    g_all = sigmoid(z_all)
    k_s, v_s = (k, v) if kv_slc is None else kv_slc
    k_w, v_w = (k, v) if kv_win is None else kv_win
    dq = np.zeros_like(q)
    dks, dvs = np.zeros_like(k_s), np.zeros_like(v_s)
    dkw, dvw = np.zeros_like(k_w), np.zeros_like(v_w)
    dkc = np.zeros_like(kc)
    dvc = np.zeros_like(vc)
    dz = np.zeros_like(g_all)
    for b in range(B):
        for t in range(T):
            for g in range(Hkv):
                hs = slice(g * G, (g + 1) * G)
                qh = q[b, t, hs]
                dO = d_o[b, t, hs]
                gg = g_all[b, t, hs]
                branches = [
                    ("cmp", cmp_keys(t, p)),
                    ("slc", slc_keys(t, [j for j in idx[b, t, g] if j >= 0], p)),
                    ("win", win_keys(t, p)),
                ]
                for c, (name, keys) in enumerate(branches):
                    if len(keys) == 0:
                        continue
                    if name == "cmp":
                        K, V = kc[b, keys, g], vc[b, keys, g]
                    elif name == "slc":
                        K, V = k_s[b, keys, g], v_s[b, keys, g]
                    else:
                        K, V = k_w[b, keys, g], v_w[b, keys, g]
                    O, _, P = attend(qh, K, V, sc)
                    dg = (dO * O).sum(axis=1)
                    dz[b, t, hs, c] = dg * gg[:, c] * (1.0 - gg[:, c])
                    dOc = gg[:, c:c + 1] * dO
                    dqh, dK, dV = _attend_bwd(qh, K, V, P, O, dOc, sc)
                    dq[b, t, hs] += dqh
                    if name == "cmp":
                        dkc[b, keys, g] += dK
                        dvc[b, keys, g] += dV
                    elif name == "slc":
                        np.add.at(dks[b, :, g], keys, dK)
                        np.add.at(dvs[b, :, g], keys, dV)
                    else:
                        np.add.at(dkw[b, :, g], keys, dK)
                        np.add.at(dvw[b, :, g], keys, dV)
    dk_phi, dphi_k = _phi_bwd(k, phi_k, dkc, p)
    dv_phi, dphi_v = _phi_bwd(v, phi_v, dvc, p)
    if gate_mlp is None:
        dw_gate = np.einsum("btc,bthk->chk", x, dz)
        dx = np.einsum("bthk,chk->btc", dz, w_gate)
        dgate_mlp = None
    else:
        dw_gate = np.einsum("btj,bthk->jhk", u_gate, dz)
        du = np.einsum("bthk,jhk->btj", dz, w_gate)
        da = du * gelu_grad(a_gate)
        dgate_mlp = {"w1": np.einsum("btc,btj->cj", x, da), "b1": da.sum(axis=(0, 1)),
                     "b2": dz.sum(axis=(0, 1))}
        dx = np.einsum("btj,cj->btc", da, gate_mlp["w1"])
    split = kv_slc is not None or kv_win is not None
    return {"dq": dq, "dk": dk_phi if split else dk_phi + dks + dkw,
            "dv": dv_phi if split else dv_phi + dvs + dvw, "dw_gate": dw_gate,
            "dx": dx, "dgate_mlp": dgate_mlp,
            "dphi_k": dphi_k, "dphi_v": dphi_v, "dk_cmp": dkc, "dv_cmp": dvc,
            "dk_phi": dk_phi, "dv_phi": dv_phi, "dk_slc": dks, "dv_slc": dvs, "dk_win": dkw, "dv_win": dvw}
