"""GPU parity with independent keys/values per branch (the compressed branch
compresses k, v; the selected and window branches attend their own pairs),
against the fp64 oracle: prefill forward, backward (per-branch key/value
gradients), decode (a separate window cache) and decode-time cache maintenance
of all three pairs.  Same bars as the shared
case: indices bit-exact outside near ties, floats within 2e-2 absolute +
1e-2 relative."""
import numpy as np
import pytest
import torch

import nsa_inputs as NI
from tests.nsa_testutil import assert_close, np64, oracle_params, to_dev

pytestmark = pytest.mark.gpu

W = NI.workload
DEV = "cuda:0"

CASES = {
    "mlp_d192_offsets": W("prefill_64k", T=900, H_kv=2, n=6, w=100, bias_std=0.02),
    "mean_fp32_g4": W("tiny_fp32", T=520),
}


def branch_inputs(w):
    """Own keys/values of the selected and window branches: the k, v draws of
    other seeds of the same workload."""
    s = NI.make_prefill_inputs(w, 11)
    v = NI.make_prefill_inputs(w, 12)
    return (s["k"], s["v"]), (v["k"], v["v"])


@pytest.mark.parametrize("case", list(CASES))
def test_split_kv_prefill_and_backward(case):
    import long_context_sparse_phi_amd as nsa
    import oracle as O
    w = CASES[case]
    cfg = nsa.config_from_workload(w)
    inp = NI.make_prefill_inputs(w, 0)
    kv_s, kv_w = branch_inputs(w)
    d_o = NI.make_grad_output(w, 0)
    d = to_dev(inp)
    ks, kw = tuple(t.to(DEV) for t in kv_s), tuple(t.to(DEV) for t in kv_w)
    print(f"[gpu] split-kv prefill+backward {case} T={w.T}", flush=True)
    fwd = nsa.nsa_fwd_prefill(cfg, d["q"], d["k"], d["v"], d["x"], d["w_gate"], d["phi_k"], d["phi_v"],
                              debug=True, kv_slc=ks, kv_win=kw)
    g = nsa.nsa_bwd(cfg, d["q"], d["k"], d["v"], d["x"], d["w_gate"], d["phi_k"], d["phi_v"], fwd, d_o.to(DEV),
                    kv_slc=ks, kv_win=kw)
    torch.cuda.synchronize()
    a = NI.to_numpy64(inp)
    s64 = tuple(np64(t) for t in kv_s)
    w64 = tuple(np64(t) for t in kv_w)
    p = oracle_params(w)
    ref = O.forward(p, a["q"], a["k"], a["v"], a["x"], a["w_gate"], a["phi_k"], a["phi_v"],
                    tie_scores=np64(fwd["p_slc"]), kv_slc=s64, kv_win=w64)
    gi = fwd["idx"].cpu().numpy().astype(np.int64)
    assert np.array_equal(gi, ref["idx"])
    for c, name in enumerate(("cmp", "slc", "win")):
        assert_close(np64(fwd["lse"][c]), ref["lse"][c], f"lse_{name}")
        assert_close(np64(fwd["o_branch"][c]), ref["o_branch"][c], f"o_{name}")
    assert_close(np64(fwd["o"]), ref["o"], "o")
    rg = O.backward(p, a["q"], a["k"], a["v"], a["x"], a["w_gate"], a["phi_k"], a["phi_v"], np64(d_o),
                    ref["idx"], kv_slc=s64, kv_win=w64)
    for name in ("dq", "dk", "dv", "dk_slc", "dv_slc", "dk_win", "dv_win", "dw_gate"):
        err = assert_close(np64(g[name]), rg[name], name)
        print(f"[gpu] {case} {name}: max abs err {err:.3e}, max |ref| {np.abs(rg[name]).max():.3e}")
    if w.phi == "mlp":
        for key in ("pe", "w1", "b1", "w2", "b2"):
            assert_close(np64(g["d_phi_k"][key]), rg["dphi_k"][key], f"dphi_k.{key}")
            assert_close(np64(g["d_phi_v"][key]), rg["dphi_v"][key], f"dphi_v.{key}")


def test_split_kv_with_shared_tensors_equals_shared_call():
    # passing k, v as every branch's own pair gives the shared forward exactly,
    # and per-branch gradients that add up to the shared ones
    import long_context_sparse_phi_amd as nsa
    w = CASES["mlp_d192_offsets"]
    cfg = nsa.config_from_workload(w)
    d = to_dev(NI.make_prefill_inputs(w, 1))
    d_o = NI.make_grad_output(w, 1).to(DEV)
    args = (cfg, d["q"], d["k"], d["v"], d["x"], d["w_gate"], d["phi_k"], d["phi_v"])
    kv = (d["k"], d["v"])
    print("[gpu] split-kv with shared tensors", flush=True)
    f0 = nsa.nsa_fwd_prefill(*args, debug=True)
    f1 = nsa.nsa_fwd_prefill(*args, debug=True, kv_slc=kv, kv_win=kv)
    g0 = nsa.nsa_bwd(*args, f0, d_o)
    g1 = nsa.nsa_bwd(*args, f1, d_o, kv_slc=kv, kv_win=kv)
    torch.cuda.synchronize()
    for key in ("o", "idx", "p_slc", "lse", "o_branch"):
        assert torch.equal(f0[key], f1[key]), key
    assert torch.equal(g0["dq"], g1["dq"])
    for x in ("k", "v"):
        tot = g1["d" + x] + g1[f"d{x}_slc"] + g1[f"d{x}_win"]
        assert_close(np64(tot), np64(g0["d" + x]), "d" + x, atol=1e-4, rtol=1e-5)


def test_split_kv_decode_window_cache():
    import long_context_sparse_phi_amd as nsa
    import oracle as O
    w = W("decode_64k", B=3, T=1300, H_kv=2, bias_std=0.02)
    p = oracle_params(w)
    cfg = nsa.config_from_workload(w)
    inp = NI.make_decode_inputs(w, 4)
    other = NI.make_decode_inputs(w, 5)
    a = NI.to_numpy64(inp)
    kc = O.compress(a["k_cache"], a["phi_k"], p)
    vc = O.compress(a["v_cache"], a["phi_v"], p)
    dt = cfg.torch_dtype
    lens = [1300, 700, 90]
    print("[gpu] split-kv decode", flush=True)
    res = nsa.nsa_fwd_decode(cfg, inp["q"].to(DEV), inp["k_cache"].to(DEV), inp["v_cache"].to(DEV),
                             torch.from_numpy(kc).to(dt).to(DEV), torch.from_numpy(vc).to(dt).to(DEV),
                             inp["x"].to(DEV), inp["w_gate"].to(DEV), debug=True,
                             seq_lens=torch.tensor(lens, dtype=torch.int32, device=DEV),
                             kv_win_cache=(other["k_cache"].to(DEV), other["v_cache"].to(DEV)))
    torch.cuda.synchronize()
    ref = O.decode(p, a["q"], a["k_cache"], a["v_cache"], kc, vc, a["x"], a["w_gate"],
                   tie_scores=np64(res["p_slc"]), seq_lens=lens,
                   kv_win_cache=(np64(other["k_cache"]), np64(other["v_cache"])))
    assert np.array_equal(res["idx"].cpu().numpy().astype(np.int64), ref["idx"])
    for c, name in enumerate(("cmp", "slc", "win")):
        assert_close(np64(res["lse"][c]), ref["lse"][c], f"lse_{name}")
        assert_close(np64(res["o_branch"][c]), ref["o_branch"][c], f"o_{name}")
    assert_close(np64(res["o"]), ref["o"], "o")


def test_split_kv_append_then_decode():
    """nsa_decode_append with the selected and window branches' own pairs:
    all three raw caches hold exactly the appended tokens, the compressed
    caches the oracle's phi over the compressed branch's rows, and a decode
    over the maintained caches matches the oracle with three pairs."""
    import long_context_sparse_phi_amd as nsa
    import oracle as O
    w = W("decode_64k", B=3, T=700, H_kv=2, bias_std=0.02)
    S, B = w.T, w.B
    p = oracle_params(w)
    cfg = nsa.config_from_workload(w)
    dt = cfg.torch_dtype
    src = NI.make_decode_inputs(w, 6)                      # compressed branch's rows, q, x, weights
    sel = NI.make_decode_inputs(w, 7)                      # selected branch's rows
    win = NI.make_decode_inputs(w, 8)                      # window branch's rows
    a = NI.to_numpy64(src)
    ncmp = lambda L: O.n_cmp_visible(L - 1, w.l, w.d)
    kc_ref = O.compress(a["k_cache"], a["phi_k"], p)
    vc_ref = O.compress(a["v_cache"], a["phi_v"], p)
    start, steps = [0, 45, S - 3], 40

    def nan_beyond(t, n_of):
        t = t.clone()
        for b, L in enumerate(start):
            t[b, n_of(L):] = float("nan")
        return t.to(DEV)

    full = {n: (d["k_cache"].to(DEV), d["v_cache"].to(DEV)) for n, d in (("cmp", src), ("slc", sel), ("win", win))}
    caches = {n: (nan_beyond(d["k_cache"], lambda L: L), nan_beyond(d["v_cache"], lambda L: L))
              for n, d in (("cmp", src), ("slc", sel), ("win", win))}
    kcmp = nan_beyond(torch.from_numpy(kc_ref).to(dt), ncmp)
    vcmp = nan_beyond(torch.from_numpy(vc_ref).to(dt), ncmp)
    phi_k, phi_v = to_dev(src["phi_k"]), to_dev(src["phi_v"])
    lens = torch.tensor(start, dtype=torch.int32, device=DEV)
    rows = torch.arange(B, device=DEV)
    print(f"[gpu] split-kv append: {steps} steps from {start}", flush=True)
    for _ in range(steps):
        slot = lens.clamp(max=S - 1).long()
        new = {n: (full[n][0][rows, slot].contiguous(), full[n][1][rows, slot].contiguous()) for n in full}
        nsa.nsa_decode_append(cfg, *new["cmp"], lens, *caches["cmp"], kcmp, vcmp, phi_k, phi_v,
                              kv_slc=(*new["slc"], *caches["slc"]), kv_win=(*new["win"], *caches["win"]))
        lens += 1
    torch.cuda.synchronize()
    final = [min(L + steps, S) for L in start]
    for n in caches:
        for b, L in enumerate(final):
            for c in (0, 1):
                assert torch.equal(caches[n][c][b, :L], full[n][c][b, :L]), (n, b, c)
                assert torch.isnan(caches[n][c][b, L:]).all(), (n, b, c)
    for b, L in enumerate(final):
        m = ncmp(L)
        assert_close(np64(kcmp[b, :m]), kc_ref[b, :m], f"k_cmp[{b}]")
        assert_close(np64(vcmp[b, :m]), vc_ref[b, :m], f"v_cmp[{b}]")
        assert torch.isnan(kcmp[b, m:].float()).all() and torch.isnan(vcmp[b, m:].float()).all()
    res = nsa.nsa_fwd_decode(cfg, src["q"].to(DEV), *caches["slc"], kcmp, vcmp, src["x"].to(DEV),
                             src["w_gate"].to(DEV), debug=True, seq_lens=lens, kv_win_cache=caches["win"])
    torch.cuda.synchronize()
    ks, vs = np64(sel["k_cache"]), np64(sel["v_cache"])
    kw, vw = np64(win["k_cache"]), np64(win["v_cache"])
    kcr, vcr = kc_ref.copy(), vc_ref.copy()
    for b, L in enumerate(final):
        ks[b, L:] = vs[b, L:] = kw[b, L:] = vw[b, L:] = np.nan
        kcr[b, ncmp(L):] = vcr[b, ncmp(L):] = np.nan
    ref = O.decode(p, a["q"], ks, vs, kcr, vcr, a["x"], a["w_gate"], tie_scores=np64(res["p_slc"]),
                   seq_lens=final, kv_win_cache=(kw, vw))
    assert np.array_equal(res["idx"].cpu().numpy().astype(np.int64), ref["idx"])
    for c, name in enumerate(("cmp", "slc", "win")):
        assert_close(np64(res["lse"][c]), ref["lse"][c], f"lse_{name}")
        assert_close(np64(res["o_branch"][c]), ref["o_branch"][c], f"o_{name}")
    assert_close(np64(res["o"]), ref["o"], "o")

