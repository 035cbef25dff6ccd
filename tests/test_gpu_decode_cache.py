"""GPU parity of decode with per-sequence cache lengths and of decode-time
cache maintenance (nsa_decode_append), against the fp64 oracle.

Cache rows beyond a sequence's own length hold NaN on both sides, so a kernel
that reads one fails the comparison.  Indices are bit-exact outside near ties
(the oracle re-selects from the GPU's exported scores only there); floats
within 2e-2 absolute + 1e-2 relative."""
import numpy as np
import pytest
import torch

import nsa_inputs as NI
from tests.nsa_testutil import assert_close, np64, oracle_params, to_dev

pytestmark = pytest.mark.gpu

W = NI.workload
DEV = "cuda:0"

RAGGED = {
    "d192_mlp": (W("decode_64k", B=4, T=1500, H_kv=2, bias_std=0.02), [1500, 1031, 517, 20]),
    "d128_g8": (W("decode_64k", B=3, T=900, H_kv=2, G=8, d_k=128, d_v=128, kv_offset_std=0.0), [64, 899, 333]),
    "fp32_mean": (W("tiny_fp32", mode="decode", B=3, T=1024), [1024, 129, 31]),
}


def nan_beyond(t, lens, n_of):
    t = t.clone()
    for b, L in enumerate(lens):
        t[b, n_of(L):] = float("nan")
    return t


def compare(res, ref):
    assert_close(np64(res["p_slc"]), ref["p_slc"], "p_slc", atol=1e-5, rtol=2e-3)
    gi = res["idx"].cpu().numpy().astype(np.int64)
    assert np.array_equal(gi, ref["idx"]), (gi, ref["idx"])
    for c, name in enumerate(("cmp", "slc", "win")):
        assert_close(np64(res["lse"][c]), ref["lse"][c], f"lse_{name}")
        assert_close(np64(res["o_branch"][c]), ref["o_branch"][c], f"o_{name}")
    assert_close(np64(res["o"]), ref["o"], "o")


@pytest.mark.parametrize("case", list(RAGGED))
def test_decode_per_sequence_lengths(case):
    import long_context_sparse_phi_amd as nsa
    import oracle as O
    w, lens = RAGGED[case]
    p = oracle_params(w)
    cfg = nsa.config_from_workload(w)
    inp = NI.make_decode_inputs(w, 1)
    a = NI.to_numpy64(inp)
    ncmp = lambda L: O.n_cmp_visible(L - 1, w.l, w.d)
    kc = O.compress(a["k_cache"], a["phi_k"], p)
    vc = O.compress(a["v_cache"], a["phi_v"], p)
    dt = cfg.torch_dtype
    kcache = nan_beyond(inp["k_cache"], lens, lambda L: L)
    vcache = nan_beyond(inp["v_cache"], lens, lambda L: L)
    kct = nan_beyond(torch.from_numpy(kc).to(dt), lens, ncmp)
    vct = nan_beyond(torch.from_numpy(vc).to(dt), lens, ncmp)
    print(f"[gpu] ragged decode {case} lens={lens}", flush=True)
    res = nsa.nsa_fwd_decode(cfg, inp["q"].to(DEV), kcache.to(DEV), vcache.to(DEV), kct.to(DEV), vct.to(DEV),
                             inp["x"].to(DEV), inp["w_gate"].to(DEV), debug=True,
                             seq_lens=torch.tensor(lens, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    ref = O.decode(p, a["q"], np64(kcache), np64(vcache), np64(kct), np64(vct), a["x"], a["w_gate"],
                   tie_scores=np64(res["p_slc"]), seq_lens=lens)
    compare(res, ref)


def test_decode_seq_lens_equal_to_capacity_matches_plain_decode():
    import long_context_sparse_phi_amd as nsa
    w = W("decode_64k", B=2, T=700, H_kv=1)
    cfg = nsa.config_from_workload(w)
    inp = to_dev(NI.make_decode_inputs(w, 2))
    kc = nsa.nsa_compress(cfg, inp["k_cache"], inp["phi_k"], False)
    vc = nsa.nsa_compress(cfg, inp["v_cache"], inp["phi_v"], True)
    args = (cfg, inp["q"], inp["k_cache"], inp["v_cache"], kc, vc, inp["x"], inp["w_gate"])
    print("[gpu] seq_lens == capacity", flush=True)
    a = nsa.nsa_fwd_decode(*args, debug=True)
    b = nsa.nsa_fwd_decode(*args, debug=True, seq_lens=torch.full((2,), 700, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    for k in ("o", "idx", "p_slc", "lse", "o_branch"):
        assert torch.equal(a[k], b[k]), k


APPEND = {
    "d192_mlp": W("decode_64k", B=4, T=700, H_kv=2, bias_std=0.02),
    "d128_mlp_g4": W("decode_64k", B=4, T=700, H_kv=2, G=4, d_k=128, d_v=128, kv_offset_std=0.0,
                     bias_std=0.02),
    "fp32_mean": W("tiny_fp32", mode="decode", B=4, T=700),
}


@pytest.mark.parametrize("case", list(APPEND))
def test_append_maintains_caches_then_decodes(case):
    import long_context_sparse_phi_amd as nsa
    import oracle as O
    w = APPEND[case]
    S, B = w.T, w.B
    p = oracle_params(w)
    cfg = nsa.config_from_workload(w)
    src = NI.make_decode_inputs(w, 3)          # raw caches: the tokens to be appended
    a = NI.to_numpy64(src)
    ncmp = lambda L: O.n_cmp_visible(L - 1, w.l, w.d)
    kc_ref = O.compress(a["k_cache"], a["phi_k"], p)
    vc_ref = O.compress(a["v_cache"], a["phi_v"], p)
    dt = cfg.torch_dtype
    start = [0, 45, 600, S - 3]
    steps = 80
    # starting state: each sequence's prefix in the raw caches, its complete
    # blocks in the compressed caches, NaN everywhere else
    kcache = nan_beyond(src["k_cache"], start, lambda L: L).to(DEV)
    vcache = nan_beyond(src["v_cache"], start, lambda L: L).to(DEV)
    kcmp = nan_beyond(torch.from_numpy(kc_ref).to(dt), start, ncmp).to(DEV)
    vcmp = nan_beyond(torch.from_numpy(vc_ref).to(dt), start, ncmp).to(DEV)
    ks, vs = src["k_cache"].to(DEV), src["v_cache"].to(DEV)
    phi_k, phi_v = to_dev(src["phi_k"]), to_dev(src["phi_v"])
    lens = torch.tensor(start, dtype=torch.int32, device=DEV)
    rows = torch.arange(B, device=DEV)
    print(f"[gpu] append {case}: {steps} steps from {start}", flush=True)
    for _ in range(steps):
        slot = lens.clamp(max=S - 1).long()
        nsa.nsa_decode_append(cfg, ks[rows, slot].contiguous(), vs[rows, slot].contiguous(), lens,
                              kcache, vcache, kcmp, vcmp, phi_k, phi_v)
        lens += 1
    torch.cuda.synchronize()
    final = [min(L + steps, S) for L in start]
    # raw caches: exactly the appended tokens, NaN beyond
    for b, L in enumerate(final):
        assert torch.equal(kcache[b, :L], ks[b, :L]) and torch.equal(vcache[b, :L], vs[b, :L])
        assert torch.isnan(kcache[b, L:]).all() and torch.isnan(vcache[b, L:]).all()
    # compressed caches: the oracle's compression of each prefix, NaN beyond
    for b, L in enumerate(final):
        n = ncmp(L)
        assert_close(np64(kcmp[b, :n]), kc_ref[b, :n], f"k_cmp[{b}]")
        assert_close(np64(vcmp[b, :n]), vc_ref[b, :n], f"v_cmp[{b}]")
        assert torch.isnan(kcmp[b, n:].float()).all() and torch.isnan(vcmp[b, n:].float()).all()
    # a decode step over the maintained caches (lengths past the capacity clamp to it)
    res = nsa.nsa_fwd_decode(cfg, src["q"].to(DEV), kcache, vcache, kcmp, vcmp, src["x"].to(DEV),
                             src["w_gate"].to(DEV), debug=True, seq_lens=lens)
    torch.cuda.synchronize()
    kr = a["k_cache"].copy()
    vr = a["v_cache"].copy()
    kcr, vcr = kc_ref.copy(), vc_ref.copy()
    for b, L in enumerate(final):
        kr[b, L:] = vr[b, L:] = np.nan
        kcr[b, ncmp(L):] = vcr[b, ncmp(L):] = np.nan
    ref = O.decode(p, a["q"], kr, vr, kcr, vcr, a["x"], a["w_gate"], tie_scores=np64(res["p_slc"]),
                   seq_lens=final)
    compare(res, ref)
