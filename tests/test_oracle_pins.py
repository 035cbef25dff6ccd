"""Pins of the fp64 oracle against facts that do not come from the oracle itself:
brute force on tiny inputs, closed forms, invariants, library routines
(torch fp64 attention / autograd, scipy) and the numbers the pages print.

CPU only.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(12345)


def rand(*shape, rng=None):
    return (rng or RNG).standard_normal(shape)


def small_problem(B=2, T=150, Hkv=2, G=3, dk=16, dv=8, C=12, phi="mean", l=8, d=4,
                  l_sel=16, n=5, w=24, hidden=10, seed=0, scale_kv=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, Hkv * G, dk))
    k = scale_kv * rng.standard_normal((B, T, Hkv, dk))
    v = rng.standard_normal((B, T, Hkv, dv))
    x = rng.standard_normal((B, T, C))
    wg = 0.3 * rng.standard_normal((C, Hkv * G, 3))

    def mk(D):
        if phi == "mean":
            return {}
        return {"pe": 0.2 * rng.standard_normal((l, D)),
                "w1": 0.2 * rng.standard_normal((l * D, hidden)),
                "b1": 0.2 * rng.standard_normal(hidden),
                "w2": 0.2 * rng.standard_normal((hidden, D)),
                "b2": 0.2 * rng.standard_normal(D)}
    p = O.Params(l=l, d=d, l_sel=l_sel, n=n, w=w, phi=phi, io=None)
    return p, dict(q=q, k=k, v=v, x=x, w_gate=wg, phi_k=mk(dk), phi_v=mk(dv))


def torch_dense_causal(q, k, v):
    """Library reference: torch fp64 causal SDPA with GQA heads repeated.
    q [B,T,Hq,dk], k [B,T,Hkv,dk] -> O [B,T,Hq,dv], lse [B,T,Hq]."""
    Hq, Hkv = q.shape[2], k.shape[2]
    G = Hq // Hkv
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    s = (tq @ tk.transpose(-1, -2)) / math.sqrt(q.shape[-1])
    T = q.shape[1]
    mask = torch.triu(torch.ones(T, T, dtype=torch.bool), 1)
    lse = torch.logsumexp(s.masked_fill(mask, -float("inf")), dim=-1)
    return o.permute(0, 2, 1, 3).numpy(), lse.permute(0, 2, 1).numpy()


# ---------------------------------------------------------------- elementary

def test_round_io_bf16_matches_torch_rne():
    x = torch.randn(20000, dtype=torch.float32) * 10.0 ** torch.randint(-6, 6, (20000,)).float()
    ref = x.to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_io(x.to(torch.float64).numpy(), "bf16")
    np.testing.assert_array_equal(got, ref)
    # exact halfway cases round to even
    assert O.round_io(np.array([1.0 + 2 ** -8]), "bf16")[0] == 1.0
    assert O.round_io(np.array([1.0 + 3 * 2 ** -8]), "bf16")[0] == 1.0 + 2 ** -6


def test_gelu_matches_scipy_and_grad_matches_fd():
    a = np.linspace(-6, 6, 241)
    np.testing.assert_allclose(O.gelu(a), a * scipy.special.ndtr(a), rtol=1e-14, atol=1e-15)
    eps = 1e-6
    fd = (O.gelu(a + eps) - O.gelu(a - eps)) / (2 * eps)
    np.testing.assert_allclose(O.gelu_grad(a), fd, rtol=1e-7, atol=1e-8)


# ---------------------------------------------------------------- gate

def test_gate_zero_weights_is_half_and_matches_loops():
    x = rand(2, 5, 7)
    np.testing.assert_array_equal(O.gate(x, np.zeros((7, 4, 3))), 0.5)
    w = rand(7, 4, 3)
    g = O.gate(x, w)
    for b, t, h, c in itertools.product(range(2), range(5), range(4), range(3)):
        z = sum(x[b, t, i] * w[i, h, c] for i in range(7))
        assert abs(g[b, t, h, c] - scipy.special.expit(z)) < 1e-14
    assert np.all((g > 0) & (g < 1))


def gate_mlp_weights(C, Hg, Hq, seed):
    rng = np.random.default_rng(seed)
    mlp = {"w1": rng.standard_normal((C, Hg)) / math.sqrt(C), "b1": 0.3 * rng.standard_normal(Hg),
           "b2": 0.3 * rng.standard_normal((Hq, 3))}
    return mlp, rng.standard_normal((Hg, Hq, 3)) / math.sqrt(Hg)


def test_gate_mlp_matches_torch_gelu_sigmoid():
    """Two-layer gate against torch's fp64 erf-GELU, linear and sigmoid."""
    x = rand(2, 7, 9)
    mlp, w2 = gate_mlp_weights(9, 11, 4, seed=3)
    t = lambda a: torch.from_numpy(a)
    h = torch.nn.functional.gelu(t(x) @ t(mlp["w1"]) + t(mlp["b1"]), approximate="none")
    ref = torch.sigmoid(torch.einsum("btj,jhk->bthk", h, t(w2)) + t(mlp["b2"])).numpy()
    np.testing.assert_allclose(O.gate(x, w2, mlp), ref, rtol=1e-13, atol=1e-15)


def test_gate_mlp_reduces_to_linear_gate_on_the_gelu_identity_range():
    """With the hidden pre-activations shifted far positive (gelu(a) = a to
    double precision there) and the shift cancelled by b2, the MLP gate is the
    linear gate with weights W1 W_g."""
    x = rand(3, 5, 6)
    mlp, w2 = gate_mlp_weights(6, 8, 4, seed=4)
    c = 60.0
    mlp["b1"] = np.full(8, c)
    mlp["b2"] = -c * w2.sum(axis=0)
    lin = O.gate(x, np.einsum("cj,jhk->chk", mlp["w1"], w2))
    np.testing.assert_allclose(O.gate(x, w2, mlp), lin, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- compression

def test_n_cmp_visible_closed_form():
    l, d = 32, 16
    for t in range(0, 400):
        # brute force: count blocks [i*d, i*d+l) fully inside [0, t]
        cnt = sum(1 for i in range(100) if i * d + l - 1 <= t)
        assert O.n_cmp_visible(t, l, d) == cnt
    assert O.n_cmp_visible(65535, 32, 16) == 4095


def test_meanpool_identity_when_l_eq_d_eq_1():
    k = rand(2, 9, 3, 5)
    p = O.Params(l=1, d=1, phi="mean", io=None)
    np.testing.assert_array_equal(O.compress(k, {}, p), k)


def test_meanpool_matches_loops():
    k = rand(1, 40, 2, 3)
    p = O.Params(l=8, d=4, phi="mean", io=None)
    kc = O.compress(k, {}, p)
    assert kc.shape == (1, 9, 2, 3)
    for i in range(9):
        for h in range(2):
            for e in range(3):
                s = 0.0
                for j in range(8):
                    s += k[0, i * 4 + j, h, e]
                assert abs(kc[0, i, h, e] - s / 8) < 1e-14


def test_mlp_phi_matches_explicit_loops():
    p, inp = small_problem(B=1, T=20, Hkv=2, G=1, dk=3, dv=2, phi="mlp", l=4, d=2, hidden=5)
    k, ph = inp["k"], inp["phi_k"]
    kc = O.compress(k, ph, p)
    N = (20 - 4) // 2 + 1
    assert kc.shape == (1, N, 2, 3)
    for i in range(N):
        for h in range(2):
            u = []
            for j in range(4):
                for e in range(3):
                    u.append(k[0, i * 2 + j, h, e] + ph["pe"][j, e])
            hid = []
            for o in range(5):
                a = ph["b1"][o] + sum(u[m] * ph["w1"][m, o] for m in range(12))
                hid.append(0.5 * a * (1 + math.erf(a / math.sqrt(2))))
            for e in range(3):
                ref = ph["b2"][e] + sum(hid[o] * ph["w2"][o, e] for o in range(5))
                assert abs(kc[0, i, h, e] - ref) < 1e-12


def test_compress_rounds_to_io_dtype():
    k = rand(1, 64, 1, 8)
    kc = O.compress(k, {}, O.Params(l=32, d=16, phi="mean", io="bf16"))
    np.testing.assert_array_equal(kc, torch.from_numpy(kc).float().bfloat16().double().numpy())


# ---------------------------------------------------------------- attention core

def test_attend_rows_sum_to_one_and_empty_set():
    q, K, V = rand(4, 6), rand(9, 6), rand(9, 3)
    o, lse, P = O.attend(q, K, V, 0.4)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    z = 0.4 * q @ K.T
    np.testing.assert_allclose(lse, scipy.special.logsumexp(z, axis=1), rtol=1e-14)
    np.testing.assert_allclose(o, scipy.special.softmax(z, axis=1) @ V, rtol=1e-13, atol=1e-14)
    o, lse, P = O.attend(q, K[:0], V[:0], 0.4)
    assert np.all(o == 0) and np.all(np.isneginf(lse)) and P.shape == (4, 0)


def test_compressed_branch_is_dense_causal_when_l_eq_d_eq_1():
    p, inp = small_problem(T=40, phi="mean", l=1, d=1, l_sel=4, n=3, w=5)
    out = O.forward(p, **inp)
    ref_o, ref_lse = torch_dense_causal(inp["q"], inp["k"], inp["v"])
    np.testing.assert_allclose(out["o_branch"][0], ref_o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out["lse"][0], ref_lse, rtol=1e-12, atol=1e-12)


def test_compressed_branch_empty_rows():
    p, inp = small_problem(T=30, l=8, d=4)
    out = O.forward(p, **inp)
    # rows t < l-1 see no complete compressed block
    assert np.all(out["o_branch"][0][:, :7] == 0)
    assert np.all(np.isneginf(out["lse"][0][:, :7]))
    assert np.all(out["p_slc"][:, :7] == 0)
    assert np.all(np.isfinite(out["lse"][0][:, 7:]))


# ---------------------------------------------------------------- remap

def test_remap_identity_when_l_eq_lsel_eq_d():
    p = O.Params(l=16, d=16, l_sel=16)
    np.testing.assert_array_equal(O.remap_matrix(7, 7, p), np.eye(7))


def test_remap_matches_double_sum_index_formula():
    """Overlap geometry == index form sum_{m<l'/d} sum_{r<l/d} p[(l'/d) j + m - r]."""
    for (l, d, ls) in [(32, 16, 64), (8, 4, 16), (12, 4, 24), (16, 16, 64), (16, 8, 16)]:
        p = O.Params(l=l, d=d, l_sel=ls)
        ncmp, nsel = 40, 12
        W = O.remap_matrix(ncmp, nsel, p)
        W2 = np.zeros_like(W)
        for j in range(nsel):
            for m in range(ls // d):
                for r in range(l // d):
                    i = (ls // d) * j + m - r
                    if 0 <= i < ncmp:
                        W2[i, j] += 1
        np.testing.assert_array_equal(W, W2)


def test_remap_weights_32_16_64_and_row_sums():
    p = O.Params(l=32, d=16, l_sel=64)
    W = O.remap_matrix(40, 11, p)
    j = 5
    np.testing.assert_array_equal(W[4 * j - 1: 4 * j + 4, j], [1, 2, 2, 2, 1])
    assert W[:, j].sum() == 8
    np.testing.assert_array_equal(W.sum(axis=1), 2.0)   # each block spreads l/d


def test_p_slc_sum_invariant():
    p, inp = small_problem(T=150, phi="mlp")
    out = O.forward(p, **inp)
    G = 3
    for t in range(150):
        s = out["p_slc"][:, t].sum(axis=-1)
        want = 0.0 if O.n_cmp_visible(t, p.l, p.d) == 0 else G * p.l / p.d
        np.testing.assert_allclose(s, want, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- head reduce / selection

def test_head_reduce_g1_is_per_head_and_permutation_invariant():
    p, inp = small_problem(T=120, G=1, phi="mean")
    out = O.forward(p, **inp)
    # G=1: p_slc equals each head's own remapped probabilities
    t = 100
    for h in range(2):
        ic = O.cmp_keys(t, p)
        _, _, P = O.attend(inp["q"][0, t, h:h + 1], O.compress(inp["k"], {}, p)[0][ic, h],
                           O.compress(inp["v"], {}, p)[0][ic, h], 1 / 4)
        ref = P @ O.remap_matrix(len(ic), out["p_slc"].shape[-1], p)
        np.testing.assert_allclose(out["p_slc"][0, t, h], ref[0], rtol=1e-12, atol=1e-15)
    # permuting query heads inside a group leaves scores and selection unchanged
    p, inp = small_problem(T=120, G=3, phi="mean", seed=3)
    perm = np.array([2, 0, 1, 4, 5, 3])
    inp2 = dict(inp)
    inp2["q"] = inp["q"][:, :, perm]
    inp2["w_gate"] = inp["w_gate"][:, perm]
    a, b = O.forward(p, **inp), O.forward(p, **inp2)
    np.testing.assert_allclose(a["p_slc"], b["p_slc"], rtol=1e-12, atol=1e-15)
    np.testing.assert_array_equal(a["idx"], b["idx"])
    np.testing.assert_allclose(a["o"][:, :, perm], b["o"], rtol=1e-12, atol=1e-12)


def test_top_n_brute_force():
    rng = np.random.default_rng(7)
    p = O.Params(l_sel=16, n=5)
    for t in range(0, 16 * 11, 3):
        J = O.candidate_blocks(t, p)
        s = rng.random(len(J))
        got = O.top_n(s, t, p)
        F = O.forced_blocks(t, p)
        assert set(F) <= set(got)
        assert len(got) == min(p.n, len(J))
        assert got == sorted(got)
        if len(J) > p.n:
            rest = [j for j in J if j not in F]
            best = max(itertools.combinations(rest, p.n - len(F)),
                       key=lambda c: sum(s[j] for j in c))
            assert got == sorted(F + list(best))
        else:
            assert got == J


def test_top_n_ties_prefer_lower_index_and_forced_blocks():
    p = O.Params(l_sel=64, n=4)
    t = 64 * 9 + 5                      # candidates 0..9, forced {0, 8, 9}
    s = np.zeros(10)
    s[[3, 5, 6]] = 0.7                   # three-way tie for one free slot
    assert O.top_n(s, t, p) == [0, 3, 8, 9]
    assert O.forced_blocks(t, p) == [0, 8, 9]
    assert O.forced_blocks(10, p) == [0]
    assert O.forced_blocks(70, p) == [0, 1]
    s[6] = 0.1
    s[3] = 0.7 * (1 - 5e-4)
    assert O.is_near_tie(s, t, p)
    s[3] = 0.7 * (1 - 5e-3)
    assert not O.is_near_tie(s, t, p)
    # below the fp32 score floor two scores tie whatever their ratio; above it
    # the relative rule alone decides
    s[:] = 0.0
    s[3], s[5] = 2.0 ** -101, 2.0 ** -130
    assert O.is_near_tie(s, t, p)
    s[3], s[5] = 2.0 ** -90, 2.0 ** -95
    assert not O.is_near_tie(s, t, p)


# ---------------------------------------------------------------- selected / window branches

def masked_dense(q, k, v, mask_fn, scale):
    """Independent formulation: full score row, masked to allowed keys."""
    T = k.shape[0]
    o = np.zeros((q.shape[0], v.shape[1]))
    for t in range(T):
        allowed = np.array([mask_fn(t, s) for s in range(T)])
        z = scale * q[t] @ k.T
        z = np.where(allowed, z, -np.inf)
        z -= z.max()
        e = np.exp(z)
        o[t] = (e / e.sum()) @ v
    return o


def test_selected_branch_dense_when_n_covers_all_blocks():
    T, ls = 130, 16
    p, inp = small_problem(T=T, l_sel=ls, n=-(-T // ls), phi="mlp")
    out = O.forward(p, **inp)
    ref, ref_lse = torch_dense_causal(inp["q"], inp["k"], inp["v"])
    np.testing.assert_allclose(out["o_branch"][1], ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out["lse"][1], ref_lse, rtol=1e-12, atol=1e-12)


def test_selected_branch_gathered_equals_masked_dense():
    p, inp = small_problem(B=1, T=120, Hkv=1, G=1, phi="mean", l_sel=16, n=3)
    out = O.forward(p, **inp)
    idx = out["idx"][0, :, 0]

    def allowed(t, s):
        return s <= t and (s // p.l_sel) in set(int(j) for j in idx[t] if j >= 0)
    ref = masked_dense(inp["q"][0, :, 0], inp["k"][0, :, 0], inp["v"][0, :, 0], allowed, 1 / 4)
    np.testing.assert_allclose(out["o_branch"][1][0, :, 0], ref, rtol=1e-12, atol=1e-12)


def test_window_branch_dense_and_unit_window():
    p, inp = small_problem(T=60, w=60)
    out = O.forward(p, **inp)
    ref, _ = torch_dense_causal(inp["q"], inp["k"], inp["v"])
    np.testing.assert_allclose(out["o_branch"][2], ref, rtol=1e-12, atol=1e-12)
    p, inp = small_problem(T=60, w=1)
    out = O.forward(p, **inp)
    G = 3
    np.testing.assert_allclose(out["o_branch"][2], np.repeat(inp["v"], G, axis=2), rtol=0, atol=1e-15)


def test_window_branch_matches_masked_band():
    p, inp = small_problem(B=1, T=90, Hkv=1, G=1, w=17)
    out = O.forward(p, **inp)
    ref = masked_dense(inp["q"][0, :, 0], inp["k"][0, :, 0], inp["v"][0, :, 0],
                       lambda t, s: t - 17 < s <= t, 1 / 4)
    np.testing.assert_allclose(out["o_branch"][2][0, :, 0], ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- combine / full forward

def test_full_forward_all_branches_dense():
    T = 48
    p, inp = small_problem(T=T, l=1, d=1, l_sel=8, n=6, w=T, phi="mean")
    out = O.forward(p, **inp)
    ref, _ = torch_dense_causal(inp["q"], inp["k"], inp["v"])
    gsum = O.gate(inp["x"], inp["w_gate"]).sum(axis=-1)
    np.testing.assert_allclose(out["o"], gsum[..., None] * ref, rtol=1e-12, atol=1e-12)


def test_combine_is_gated_sum_of_branches():
    p, inp = small_problem(T=70, phi="mlp")
    out = O.forward(p, **inp)
    g = out["gates"]
    ref = sum(g[..., c, None] * out["o_branch"][c] for c in range(3))
    np.testing.assert_allclose(out["o"], ref, rtol=1e-14, atol=1e-14)


def test_rows_subset_matches_full():
    p, inp = small_problem(T=100, phi="mlp")
    full = O.forward(p, **inp)
    rows = [0, 7, 33, 64, 99]
    sub = O.forward(p, **inp, rows=rows)
    for key in ("o", "p_slc", "idx"):
        np.testing.assert_array_equal(sub[key], full[key][:, rows])


def test_tie_scores_only_used_on_near_ties():
    p, inp = small_problem(T=150, phi="mean", n=4)
    a = O.forward(p, **inp)
    # adversarial alternative scores: only near-tie rows may change
    alt = -a["p_slc"]
    b = O.forward(p, **inp, tie_scores=alt)
    changed = np.any(a["idx"] != b["idx"], axis=-1)
    assert np.all(changed <= b["retied"])


# ---------------------------------------------------------------- decode

def test_decode_equals_prefill_last_row():
    for S in (37, 150):
        p, inp = small_problem(T=S, phi="mlp", seed=S)
        full = O.forward(p, **inp, rows=[S - 1])
        kc = O.compress(inp["k"], inp["phi_k"], p)
        vc = O.compress(inp["v"], inp["phi_v"], p)
        dec = O.decode(p, inp["q"][:, S - 1], inp["k"], inp["v"], kc, vc, inp["x"][:, S - 1],
                       inp["w_gate"])
        np.testing.assert_allclose(dec["o"], full["o"][:, 0], rtol=1e-14, atol=1e-14)
        np.testing.assert_array_equal(dec["idx"], full["idx"][:, 0])


def test_decode_seq_lens_equals_prefill_rows_of_each_prefix():
    # sequence b holds only its first S_b tokens: its decode row must be the
    # prefill forward's row S_b-1 over that prefix alone; rows beyond it are
    # NaN and must never be read
    S, lens = 150, [150, 61, 9]
    p, inp = small_problem(B=3, T=S, phi="mlp", seed=21)
    kc = O.compress(inp["k"], inp["phi_k"], p)
    vc = O.compress(inp["v"], inp["phi_v"], p)
    kcache, vcache = inp["k"].copy(), inp["v"].copy()
    q = np.stack([inp["q"][b, L - 1] for b, L in enumerate(lens)])
    x = np.stack([inp["x"][b, L - 1] for b, L in enumerate(lens)])
    for b, L in enumerate(lens):
        kcache[b, L:] = vcache[b, L:] = np.nan
        kc[b, O.n_cmp_visible(L - 1, p.l, p.d):] = np.nan
        vc[b, O.n_cmp_visible(L - 1, p.l, p.d):] = np.nan
    dec = O.decode(p, q, kcache, vcache, kc, vc, x, inp["w_gate"], seq_lens=lens)
    for b, L in enumerate(lens):
        sub = {k: (v[b:b + 1, :L] if k in ("q", "k", "v", "x") else v) for k, v in inp.items()}
        full = O.forward(p, **sub, rows=[L - 1])
        np.testing.assert_allclose(dec["o"][b], full["o"][0, 0], rtol=1e-13, atol=1e-13)
        np.testing.assert_array_equal(dec["idx"][b], full["idx"][0, 0])
        nb = -(-L // p.l_sel)
        np.testing.assert_allclose(dec["p_slc"][b, :, :nb], full["p_slc"][0, 0], rtol=1e-13, atol=1e-15)
        assert not dec["p_slc"][b, :, nb:].any()


@pytest.mark.parametrize("phi", ["mean", "mlp"])
def test_append_token_maintains_the_one_shot_compression(phi):
    # appending tokens one at a time from ragged starting lengths must rebuild
    # exactly the compressed cache that compress() gives for the whole sequence
    S, B = 64, 3
    p, inp = small_problem(B=B, T=S, phi=phi, seed=5)
    k, v = inp["k"], inp["v"]
    ncap = O.n_cmp_visible(S - 1, p.l, p.d)
    kcache, vcache = np.full_like(k, np.nan), np.full_like(v, np.nan)
    kc = np.full((B, ncap) + k.shape[2:], np.nan)
    vc = np.full((B, ncap) + v.shape[2:], np.nan)
    lens = np.array([0, 13, 61])
    for b, L in enumerate(lens):
        kcache[b, :L], vcache[b, :L] = k[b, :L], v[b, :L]
        n = O.n_cmp_visible(L - 1, p.l, p.d)
        if n:
            kc[b, :n] = O.compress(k[b:b + 1, :L], inp["phi_k"], p)[0]
            vc[b, :n] = O.compress(v[b:b + 1, :L], inp["phi_v"], p)[0]
    for _ in range(S + 2):   # the last sequences reach the capacity and stay there
        kn = np.stack([k[b, min(L, S - 1)] for b, L in enumerate(lens)])
        vn = np.stack([v[b, min(L, S - 1)] for b, L in enumerate(lens)])
        before = kc.copy()
        kcache, vcache, kc, vc = O.append_token(p, kcache, vcache, kc, vc, kn, vn, lens,
                                                inp["phi_k"], inp["phi_v"])
        for b, L in enumerate(lens):
            done = L < S and L + 1 >= p.l and (L + 1 - p.l) % p.d == 0
            changed = ~np.all((kc[b] == before[b]) | (np.isnan(kc[b]) & np.isnan(before[b])), axis=(1, 2))
            assert changed.sum() == (1 if done else 0)
        lens = np.minimum(lens + 1, S)
    np.testing.assert_array_equal(kcache, k)
    np.testing.assert_array_equal(vcache, v)
    np.testing.assert_allclose(kc, O.compress(k, inp["phi_k"], p), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(vc, O.compress(v, inp["phi_v"], p), rtol=1e-12, atol=1e-12)


def test_decode_token_model_reproduces_pages():
    with open(os.path.join(GOLDEN, "decode_token_model.json")) as f:
        g = json.load(f)
    p = O.Params(l=g["l"], d=g["d"], l_sel=g["l_sel"], n=g["n"], w=g["w"])
    s = g["context"]
    tokens = O.decode_token_count(s, p)
    assert tokens == g["tokens_per_step"]
    assert round(s / tokens, 1) == g["speedup_printed"]
    assert round(100 * (1 - tokens / s), 1) == g["sparsity_pct_printed"]


# ---------------------------------------------------------------- backward

def _loss(p, inp, d_o, idx):
    out = O.forward(p, **inp, idx=idx)
    return float((out["o"] * d_o).sum())


@pytest.mark.parametrize("phi", ["mean", "mlp"])
def test_backward_matches_finite_differences(phi):
    p, inp = small_problem(B=1, T=26, Hkv=2, G=2, dk=3, dv=2, C=4, phi=phi, l=4, d=2,
                           l_sel=8, n=2, w=5, hidden=4, seed=11)
    # n=2 < candidates for t>=16: exercises real selection, forced blocks only
    p = O.Params(l=4, d=2, l_sel=8, n=3, w=5, phi=phi, io=None)
    rng = np.random.default_rng(5)
    d_o = rng.standard_normal((1, 26, 4, 2))
    idx = O.forward(p, **inp)["idx"]
    gr = O.backward(p, d_o=d_o, idx=idx, **inp)
    eps = 1e-6

    def check(arr, grad, n_pick=12):
        flat = arr.reshape(-1)
        picks = rng.choice(flat.size, size=min(n_pick, flat.size), replace=False)
        for i in picks:
            old = flat[i]
            flat[i] = old + eps
            lp = _loss(p, inp, d_o, idx)
            flat[i] = old - eps
            lm = _loss(p, inp, d_o, idx)
            flat[i] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad.reshape(-1)[i]) < 1e-6 + 1e-6 * abs(fd), (i, fd, grad.reshape(-1)[i])

    check(inp["q"], gr["dq"])
    check(inp["k"], gr["dk"])
    check(inp["v"], gr["dv"])
    check(inp["w_gate"], gr["dw_gate"])
    if phi == "mlp":
        for key in ("pe", "w1", "b1", "w2", "b2"):
            check(inp["phi_k"][key], gr["dphi_k"][key])
            check(inp["phi_v"][key], gr["dphi_v"][key])


def test_independent_kv_per_branch_reduces_to_shared():
    # the same tensors passed as every branch's own keys/values: forward is
    # unchanged and the per-branch gradients add up to the shared ones
    p, inp = small_problem(T=70, phi="mlp", seed=4)
    base = O.forward(p, **inp)
    kv = (inp["k"], inp["v"])
    split = O.forward(p, **inp, kv_slc=kv, kv_win=kv)
    np.testing.assert_array_equal(split["o"], base["o"])
    np.testing.assert_array_equal(split["idx"], base["idx"])
    rng = np.random.default_rng(2)
    d_o = rng.standard_normal(base["o"].shape)
    g0 = O.backward(p, d_o=d_o, idx=base["idx"], **inp)
    g1 = O.backward(p, d_o=d_o, idx=base["idx"], **inp, kv_slc=kv, kv_win=kv)
    np.testing.assert_allclose(g1["dk"] + g1["dk_slc"] + g1["dk_win"], g0["dk"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g1["dv"] + g1["dv_slc"] + g1["dv_win"], g0["dv"], rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(g1["dq"], g0["dq"])


def test_independent_kv_backward_matches_finite_differences():
    p, inp = small_problem(B=1, T=26, Hkv=2, G=2, dk=3, dv=2, C=4, phi="mlp", l=4, d=2,
                           l_sel=8, n=3, w=5, hidden=4, seed=13)
    p = O.Params(l=4, d=2, l_sel=8, n=3, w=5, phi="mlp", io=None)
    rng = np.random.default_rng(6)
    kv_s = (rng.standard_normal(inp["k"].shape), rng.standard_normal(inp["v"].shape))
    kv_w = (rng.standard_normal(inp["k"].shape), rng.standard_normal(inp["v"].shape))
    d_o = rng.standard_normal((1, 26, 4, 2))
    idx = O.forward(p, **inp, kv_slc=kv_s, kv_win=kv_w)["idx"]
    gr = O.backward(p, d_o=d_o, idx=idx, **inp, kv_slc=kv_s, kv_win=kv_w)
    eps = 1e-6

    def loss():
        return float((O.forward(p, **inp, idx=idx, kv_slc=kv_s, kv_win=kv_w)["o"] * d_o).sum())

    def check(arr, grad, n_pick=10):
        flat = arr.reshape(-1)
        for i in rng.choice(flat.size, size=min(n_pick, flat.size), replace=False):
            old = flat[i]
            flat[i] = old + eps
            lp = loss()
            flat[i] = old - eps
            lm = loss()
            flat[i] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad.reshape(-1)[i]) < 1e-6 + 1e-6 * abs(fd), (i, fd, grad.reshape(-1)[i])

    check(inp["k"], gr["dk"])
    check(inp["v"], gr["dv"])
    check(kv_s[0], gr["dk_slc"])
    check(kv_s[1], gr["dv_slc"])
    check(kv_w[0], gr["dk_win"])
    check(kv_w[1], gr["dv_win"])
    check(inp["q"], gr["dq"])


def test_dq_rows_matches_finite_differences():
    """Per-row dq (used where the whole backward is too large for the oracle)
    against central differences of the loss in q at those rows."""
    p, inp = small_problem(B=1, T=26, Hkv=2, G=2, dk=3, dv=2, C=4, phi="mlp", l=4, d=2,
                           l_sel=8, n=2, w=5, hidden=4, seed=13)
    p = O.Params(l=4, d=2, l_sel=8, n=3, w=5, phi="mlp", io=None)
    rng = np.random.default_rng(17)
    d_o = rng.standard_normal((1, 26, 4, 2))
    idx = O.forward(p, **inp)["idx"]
    rows = np.array([3, 17, 25])
    kc = O.compress(inp["k"], inp["phi_k"], p)
    vc = O.compress(inp["v"], inp["phi_v"], p)
    g_rows = O.gate(inp["x"][:, rows], inp["w_gate"])
    dq = O.dq_rows(p, inp["q"][:, rows], inp["k"], inp["v"], kc, vc, g_rows, d_o[:, rows], idx[:, rows], rows)
    eps = 1e-6
    for r, t in enumerate(rows):
        for h in range(4):
            for e in range(3):
                old = inp["q"][0, t, h, e]
                inp["q"][0, t, h, e] = old + eps
                lp = _loss(p, inp, d_o, idx)
                inp["q"][0, t, h, e] = old - eps
                lm = _loss(p, inp, d_o, idx)
                inp["q"][0, t, h, e] = old
                fd = (lp - lm) / (2 * eps)
                assert abs(fd - dq[0, r, h, e]) < 1e-6 + 1e-6 * abs(fd), (t, h, e, fd, dq[0, r, h, e])


def test_dkv_keys_matches_finite_differences():
    """Key/value gradients at sampled tokens (used where the whole backward is
    too large for the oracle) against central differences of the loss in k
    and v at those tokens, through all three branches and phi, and phi's
    parameter gradients against the same differences in its parameters."""
    for phi in ("mlp", "mean"):
        p, inp = small_problem(B=2, T=30, Hkv=2, G=2, dk=3, dv=2, C=4, phi=phi, l=4, d=2,
                               l_sel=8, n=3, w=5, hidden=4, seed=21)
        p = O.Params(l=4, d=2, l_sel=8, n=3, w=5, phi=phi, io=None)
        rng = np.random.default_rng(23)
        d_o = rng.standard_normal((2, 30, 4, 2))
        idx = O.forward(p, **inp)["idx"]
        keys = [0, 1, 7, 8, 13, 24, 29]
        g_all = O.gate(inp["x"], inp["w_gate"])
        got = O.dkv_keys(p, inp["q"], inp["k"], inp["v"], g_all, d_o, idx, keys, inp["phi_k"], inp["phi_v"])
        eps = 1e-6

        def fd(arr, i):
            old = arr[i]
            arr[i] = old + eps
            lp = _loss(p, inp, d_o, idx)
            arr[i] = old - eps
            lm = _loss(p, inp, d_o, idx)
            arr[i] = old
            return (lp - lm) / (2 * eps)

        for name, g_name in (("k", "dk"), ("v", "dv")):
            for b in range(2):
                for r, s in enumerate(keys):
                    for g in range(2):
                        for e in range(inp[name].shape[3]):
                            want = fd(inp[name], (b, s, g, e))
                            have = got[g_name][b, r, g, e]
                            assert abs(want - have) < 1e-6 + 1e-6 * abs(want), (phi, name, b, s, g, e, want, have)
        if phi == "mlp":
            for tag, gk in (("phi_k", "dphi_k"), ("phi_v", "dphi_v")):
                for key in ("pe", "w1", "b1", "w2", "b2"):
                    flat = inp[tag][key].reshape(-1)
                    for i in rng.choice(flat.size, size=min(4, flat.size), replace=False):
                        want = fd(flat, i)
                        have = got[gk][key].reshape(-1)[i]
                        assert abs(want - have) < 1e-6 + 1e-6 * abs(want), (tag, key, i, want, have)


def test_dkv_keys_equals_the_full_backward_at_every_token():
    p, inp = small_problem(B=1, T=70, Hkv=2, G=3, dk=5, dv=4, C=4, phi="mlp", l=8, d=4,
                           l_sel=16, n=3, w=9, hidden=6, seed=4)
    rng = np.random.default_rng(2)
    d_o = rng.standard_normal((1, 70, 6, 4))
    idx = O.forward(p, **inp)["idx"]
    full = O.backward(p, d_o=d_o, idx=idx, **inp)
    got = O.dkv_keys(p, inp["q"], inp["k"], inp["v"], O.gate(inp["x"], inp["w_gate"]), d_o, idx, range(70),
                     inp["phi_k"], inp["phi_v"])
    np.testing.assert_allclose(got["dk"], full["dk"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got["dv"], full["dv"], rtol=1e-12, atol=1e-12)
    for key in ("pe", "w1", "b1", "w2", "b2"):
        np.testing.assert_allclose(got["dphi_k"][key], full["dphi_k"][key], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(got["dphi_v"][key], full["dphi_v"][key], rtol=1e-12, atol=1e-12)
    # selecting the blocks itself from its own scores gives forward()'s indices
    # and the same gradients; pairs not asked for are left out
    own = O.dkv_keys(p, inp["q"], inp["k"], inp["v"], O.gate(inp["x"], inp["w_gate"]), d_o, None, range(70),
                     inp["phi_k"], inp["phi_v"], pairs=[(0, 1)])
    np.testing.assert_array_equal(own["idx"][:, :, 1], idx[:, :, 1])
    np.testing.assert_allclose(own["dk"][:, :, 1], full["dk"][:, :, 1], rtol=1e-12, atol=1e-12)
    assert np.isnan(own["dk"][:, :, 0]).all()


def test_backward_dense_case_matches_torch_autograd():
    T = 40
    p, inp = small_problem(B=1, T=T, Hkv=2, G=2, dk=6, dv=5, C=5, l=1, d=1, l_sel=8,
                           n=5, w=T, phi="mean", seed=2)
    rng = np.random.default_rng(9)
    d_o = rng.standard_normal((1, T, 4, 5))
    idx = O.forward(p, **inp)["idx"]
    gr = O.backward(p, d_o=d_o, idx=idx, **inp)
    tq, tk, tv, tx, tw = (torch.tensor(inp[n], requires_grad=True)
                          for n in ("q", "k", "v", "x", "w_gate"))
    dense = lambda: torch.nn.functional.scaled_dot_product_attention(
        tq.permute(0, 2, 1, 3), tk.permute(0, 2, 1, 3).repeat_interleave(2, 1),
        tv.permute(0, 2, 1, 3).repeat_interleave(2, 1), is_causal=True).permute(0, 2, 1, 3)
    g = torch.sigmoid(torch.einsum("btc,chk->bthk", tx, tw))
    out = g.sum(-1, keepdim=True) * dense()
    (out * torch.from_numpy(d_o)).sum().backward()
    np.testing.assert_allclose(gr["dq"], tq.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(gr["dk"], tk.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(gr["dv"], tv.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(gr["dw_gate"], tw.grad.numpy(), rtol=1e-10, atol=1e-11)


@pytest.mark.parametrize("mlp_gate", [False, True])
def test_backward_gate_and_gate_input_match_torch_autograd(mlp_gate):
    """Dense case (every branch attends all past keys) with torch fp64 autograd
    through a linear or two-layer gate: dw_gate, the gate MLP's weights and
    dx, the gradient with respect to the gate input."""
    T, C, Hg, Hq = 36, 5, 7, 4
    p, inp = small_problem(B=2, T=T, Hkv=2, G=2, dk=6, dv=5, C=C, l=1, d=1, l_sel=8,
                           n=5, w=T, phi="mean", seed=21)
    mlp = None
    if mlp_gate:
        mlp, inp["w_gate"] = gate_mlp_weights(C, Hg, Hq, seed=22)
    rng = np.random.default_rng(23)
    d_o = rng.standard_normal((2, T, Hq, 5))
    idx = O.forward(p, **inp, gate_mlp=mlp)["idx"]
    gr = O.backward(p, d_o=d_o, idx=idx, **inp, gate_mlp=mlp)
    tq, tk, tv, tx, tw = (torch.tensor(inp[n], requires_grad=True) for n in ("q", "k", "v", "x", "w_gate"))
    dense = torch.nn.functional.scaled_dot_product_attention(
        tq.permute(0, 2, 1, 3), tk.permute(0, 2, 1, 3).repeat_interleave(2, 1),
        tv.permute(0, 2, 1, 3).repeat_interleave(2, 1), is_causal=True).permute(0, 2, 1, 3)
    if mlp_gate:
        tm = {k: torch.tensor(v, requires_grad=True) for k, v in mlp.items()}
        h = torch.nn.functional.gelu(tx @ tm["w1"] + tm["b1"], approximate="none")
        z = torch.einsum("btj,jhk->bthk", h, tw) + tm["b2"]
    else:
        z = torch.einsum("btc,chk->bthk", tx, tw)
    out = torch.sigmoid(z).sum(-1, keepdim=True) * dense
    (out * torch.from_numpy(d_o)).sum().backward()
    tol = dict(rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(gr["dq"], tq.grad.numpy(), **tol)
    np.testing.assert_allclose(gr["dk"], tk.grad.numpy(), **tol)
    np.testing.assert_allclose(gr["dw_gate"], tw.grad.numpy(), **tol)
    np.testing.assert_allclose(gr["dx"], tx.grad.numpy(), **tol)
    if mlp_gate:
        for key in ("w1", "b1", "b2"):
            np.testing.assert_allclose(gr["dgate_mlp"][key], tm[key].grad.numpy(), **tol)
    else:
        assert gr["dgate_mlp"] is None


def test_gate_mlp_backward_matches_finite_differences_with_real_selection():
    p, inp = small_problem(B=1, T=26, Hkv=2, G=2, dk=3, dv=2, C=4, phi="mlp", l=4, d=2,
                           l_sel=8, n=3, w=5, hidden=4, seed=31)
    p = O.Params(l=4, d=2, l_sel=8, n=3, w=5, phi="mlp", io=None)
    mlp, inp["w_gate"] = gate_mlp_weights(4, 6, 4, seed=32)
    rng = np.random.default_rng(33)
    d_o = rng.standard_normal((1, 26, 4, 2))
    idx = O.forward(p, **inp, gate_mlp=mlp)["idx"]
    gr = O.backward(p, d_o=d_o, idx=idx, **inp, gate_mlp=mlp)
    eps = 1e-6

    def loss():
        return float((O.forward(p, **inp, idx=idx, gate_mlp=mlp)["o"] * d_o).sum())

    def check(arr, grad, n_pick=10):
        flat = arr.reshape(-1)
        for i in rng.choice(flat.size, size=min(n_pick, flat.size), replace=False):
            old = flat[i]
            flat[i] = old + eps
            lp = loss()
            flat[i] = old - eps
            lm = loss()
            flat[i] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad.reshape(-1)[i]) < 1e-6 + 1e-6 * abs(fd), (i, fd, grad.reshape(-1)[i])

    check(inp["x"], gr["dx"])
    check(inp["w_gate"], gr["dw_gate"])
    for key in ("w1", "b1", "b2"):
        check(mlp[key], gr["dgate_mlp"][key])
    check(inp["q"], gr["dq"])


def layer_problem(T, C, Hkv, G, dk, dv, seed, phi="mean", **kw):
    rng = np.random.default_rng(seed)
    Hq = Hkv * G
    h = rng.standard_normal((1, T, C))
    proj = {"w_q": rng.standard_normal((C, Hq * dk)) / math.sqrt(C),
            "w_k": rng.standard_normal((C, Hkv * dk)) / math.sqrt(C),
            "w_v": rng.standard_normal((C, Hkv * dv)) / math.sqrt(C),
            "w_o": rng.standard_normal((Hq * dv, C)) / math.sqrt(Hq * dv)}
    w_gate = 0.3 * rng.standard_normal((C, Hq, 3))
    return h, proj, w_gate, rng


def test_layer_matches_torch_autograd_in_the_dense_case():
    """Projections + operator + output projection against torch fp64 autograd
    where all three branches are dense causal attention (l = d = 1, mean phi,
    n covering all blocks, w >= T)."""
    T, C, Hkv, G, dk, dv = 30, 6, 2, 2, 4, 3
    h, proj, w_gate, rng = layer_problem(T, C, Hkv, G, dk, dv, seed=41)
    p = O.Params(l=1, d=1, l_sel=8, n=4, w=T, phi="mean", io=None)
    dy = rng.standard_normal((1, T, C))
    f = O.layer_forward(p, h, proj, w_gate, (Hkv * G, Hkv))
    g = O.layer_backward(p, h, proj, w_gate, (Hkv * G, Hkv), None, None, dy, f["nsa"]["idx"])
    th = torch.tensor(h, requires_grad=True)
    tw = {k: torch.tensor(v, requires_grad=True) for k, v in proj.items()}
    tg = torch.tensor(w_gate, requires_grad=True)
    q = (th @ tw["w_q"]).reshape(1, T, Hkv * G, dk).permute(0, 2, 1, 3)
    k = (th @ tw["w_k"]).reshape(1, T, Hkv, dk).permute(0, 2, 1, 3).repeat_interleave(G, 1)
    v = (th @ tw["w_v"]).reshape(1, T, Hkv, dv).permute(0, 2, 1, 3).repeat_interleave(G, 1)
    dense = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True).permute(0, 2, 1, 3)
    gates = torch.sigmoid(torch.einsum("btc,chk->bthk", th, tg))
    o = gates.sum(-1, keepdim=True) * dense
    y = o.reshape(1, T, -1) @ tw["w_o"]
    np.testing.assert_allclose(f["y"], y.detach().numpy(), rtol=1e-11, atol=1e-12)
    (y * torch.from_numpy(dy)).sum().backward()
    tol = dict(rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(g["dh"], th.grad.numpy(), **tol)
    np.testing.assert_allclose(g["dw_gate"], tg.grad.numpy(), **tol)
    for key in proj:
        np.testing.assert_allclose(g["d" + key], tw[key].grad.numpy(), **tol)


def test_layer_backward_matches_finite_differences_with_real_selection():
    T, C, Hkv, G, dk, dv = 26, 4, 2, 2, 3, 2
    h, proj, w_gate, rng = layer_problem(T, C, Hkv, G, dk, dv, seed=43)
    p = O.Params(l=4, d=2, l_sel=8, n=3, w=5, phi="mlp", io=None)
    hid = 4
    phi = {D: {"pe": 0.2 * rng.standard_normal((4, D)), "w1": 0.2 * rng.standard_normal((4 * D, hid)),
               "b1": 0.2 * rng.standard_normal(hid), "w2": 0.2 * rng.standard_normal((hid, D)),
               "b2": 0.2 * rng.standard_normal(D)} for D in (dk, dv)}
    mlp, w_gate = gate_mlp_weights(C, 5, Hkv * G, seed=44)
    heads = (Hkv * G, Hkv)
    dy = rng.standard_normal((1, T, C))
    idx = O.layer_forward(p, h, proj, w_gate, heads, phi[dk], phi[dv], mlp)["nsa"]["idx"]
    g = O.layer_backward(p, h, proj, w_gate, heads, phi[dk], phi[dv], dy, idx, gate_mlp=mlp)
    eps = 1e-6

    def loss():
        B = 1
        q = (h @ proj["w_q"]).reshape(B, T, heads[0], dk)
        k = (h @ proj["w_k"]).reshape(B, T, Hkv, dk)
        v = (h @ proj["w_v"]).reshape(B, T, Hkv, dv)
        o = O.forward(p, q, k, v, h, w_gate, phi[dk], phi[dv], idx=idx, gate_mlp=mlp)["o"]
        return float(((o.reshape(B, T, -1) @ proj["w_o"]) * dy).sum())

    def check(arr, grad, n_pick=8):
        flat = arr.reshape(-1)
        for i in rng.choice(flat.size, size=min(n_pick, flat.size), replace=False):
            old = flat[i]
            flat[i] = old + eps
            lp = loss()
            flat[i] = old - eps
            lm = loss()
            flat[i] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad.reshape(-1)[i]) < 1e-6 + 1e-6 * abs(fd), (i, fd, grad.reshape(-1)[i])

    check(h, g["dh"])
    for key in proj:
        check(proj[key], g["d" + key])
    check(mlp["w1"], g["dgate_mlp"]["w1"])
    check(phi[dk]["w1"], g["dphi_k"]["w1"])


def test_dense_causal_matches_torch_sdpa():
    """The dense baseline against torch's fp64 scaled-dot-product attention
    (causal, GQA by repeating the KV heads)."""
    rng = np.random.default_rng(23)
    B, T, Hkv, G, dk, dv = 2, 37, 2, 3, 5, 4
    q = rng.standard_normal((B, T, Hkv * G, dk))
    k = rng.standard_normal((B, T, Hkv, dk))
    v = rng.standard_normal((B, T, Hkv, dv))
    o, lse = O.dense_causal(q, k, v)
    tq, tk, tv = (torch.from_numpy(a).permute(0, 2, 1, 3) for a in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(G, 1), tv.repeat_interleave(G, 1), is_causal=True).permute(0, 2, 1, 3)
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-12)
    s = np.einsum("bthd,bjhd->bhtj", q, np.repeat(k, G, axis=2)) / np.sqrt(dk)
    s = np.where(np.tril(np.ones((T, T), dtype=bool)), s, -np.inf)
    np.testing.assert_allclose(lse, np.transpose(np.log(np.exp(s).sum(-1)), (0, 2, 1)), rtol=1e-12)


def test_dense_causal_bwd_matches_torch_autograd():
    """The dense baseline's backward against torch fp64 autograd through
    scaled_dot_product_attention (causal, GQA by repeating the KV heads)."""
    rng = np.random.default_rng(29)
    B, T, Hkv, G, dk, dv = 2, 33, 2, 3, 5, 4
    q = rng.standard_normal((B, T, Hkv * G, dk))
    k = rng.standard_normal((B, T, Hkv, dk))
    v = rng.standard_normal((B, T, Hkv, dv))
    d_o = rng.standard_normal((B, T, Hkv * G, dv))
    dq, dk_, dv_ = O.dense_causal_bwd(q, k, v, d_o)
    tq, tk, tv = (torch.from_numpy(a).permute(0, 2, 1, 3).clone().requires_grad_(True) for a in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(G, 1), tv.repeat_interleave(G, 1), is_causal=True)
    (out * torch.from_numpy(d_o).permute(0, 2, 1, 3)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.permute(0, 2, 1, 3).numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk_, tk.grad.permute(0, 2, 1, 3).numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv_, tv.grad.permute(0, 2, 1, 3).numpy(), rtol=1e-10, atol=1e-12)
