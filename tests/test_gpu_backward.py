"""GPU parity of nsa_bwd against the fp64 oracle's backward.

Both sides hold the selected blocks fixed at the forward's selection: the GPU
uses the indices its forward saved, the oracle the ones its own forward chose
(re-selecting from the GPU's exported scores only on near ties); the test
first checks that the two index sets are identical.  Gradients agree within
2e-2 absolute + 1e-2 relative of the oracle."""
import numpy as np
import pytest
import torch

import nsa_inputs as NI
from tests.nsa_testutil import assert_close, np64, oracle_params, to_dev

pytestmark = pytest.mark.gpu

W = NI.workload
CASES = {
    "mlp_d128_selection": W("train_16k", B=1, T=700, H_kv=1, n=6, w=128, bias_std=0.02),
    "mean_fp32_g4": W("tiny_fp32", mode="train", T=520),
    "mlp_d192_offsets": W("prefill_64k", mode="train", T=600, H_kv=1, n=6, w=100, bias_std=0.02),
    "small_blocks_g4_b2": W("tiny_fp32", mode="train", dtype="bf16", B=2, T=300, l=8, d=4, l_sel=16, n=5, w=24),
    "g8_mlp_d64": W("train_16k", T=400, G=8, H_kv=2, d_k=64, d_v=64, hidden=64, n=5, w=60, bias_std=0.05),
    "short_no_cmp_block": W("train_16k", T=20, H_kv=1),
    # thousands of query positions per key: the dK/dV partials span several
    # 512-position segments (block 0 is selected by every position; the first
    # compressed keys are seen by all later ones), so the ordered segment sums run
    "multi_segment_bf16_d64": W("tiny_fp32", mode="train", dtype="bf16", T=2200),
    "multi_segment_mlp_d128": W("train_16k", B=1, T=2100, H_kv=1, n=6, w=128, bias_std=0.02),
    # several segments per key for each of four (sequence, KV head) pairs
    "multi_segment_b2_hkv2": W("tiny_fp32", mode="train", dtype="bf16", B=2, T=1500, H_kv=2),
    # more than 1024 selection blocks (l = l' = d = 16): the reverse index over
    # 1025 blocks, 33 segments for block 0 (the oracle takes about 30 s)
    "long_score_rows_t16400": W("tiny_fp32", mode="train", dtype="bf16", T=16400, l=16, d=16, l_sel=16, n=8,
                                w=128),
}


def run_case(w, seed=0, recompute_row_terms=False):
    import long_context_sparse_phi_amd as nsa
    import oracle as O
    cfg = nsa.config_from_workload(w)
    inp = NI.make_prefill_inputs(w, seed)
    d_o = NI.make_grad_output(w, seed)
    d = to_dev(inp)
    print(f"[gpu] backward case B={w.B} T={w.T} Hkv={w.H_kv} G={w.G} dk={w.d_k} phi={w.phi} dtype={w.dtype}",
          flush=True)
    fwd = nsa.nsa_fwd_prefill(cfg, d["q"], d["k"], d["v"], d["x"], d["w_gate"], d["phi_k"], d["phi_v"], debug=True)
    grads = nsa.nsa_bwd(cfg, d["q"], d["k"], d["v"], d["x"], d["w_gate"], d["phi_k"], d["phi_v"], fwd,
                        d_o.to("cuda:0"), recompute_row_terms=recompute_row_terms)
    torch.cuda.synchronize()
    a = NI.to_numpy64(inp)
    p = oracle_params(w)
    ref_f = O.forward(p, a["q"], a["k"], a["v"], a["x"], a["w_gate"], a["phi_k"], a["phi_v"],
                      tie_scores=np64(fwd["p_slc"]))
    assert np.array_equal(ref_f["idx"], fwd["idx"].cpu().numpy().astype(np.int64))
    ref = O.backward(p, a["q"], a["k"], a["v"], a["x"], a["w_gate"], a["phi_k"], a["phi_v"],
                     np64(d_o), ref_f["idx"])
    return grads, ref


@pytest.mark.parametrize("case", list(CASES) + ["mlp_d128_selection/recompute", "mean_fp32_g4/recompute"])
def test_backward_matches_oracle(case):
    # "/recompute": the softmax row terms are recomputed from the probabilities
    # instead of read from the forward's saved branch outputs
    name, _, mode = case.partition("/")
    w = CASES[name]
    g, ref = run_case(w, recompute_row_terms=mode == "recompute")
    for name in ("dq", "dk", "dv", "dw_gate"):
        err = assert_close(np64(g[name]), ref[name], name)
        print(f"[gpu] {case} {name}: max abs err {err:.3e}, max |ref| {np.abs(ref[name]).max():.3e}")
    if w.phi == "mlp":
        for tag in ("dphi_k", "dphi_v"):
            gk = "d_phi_k" if tag == "dphi_k" else "d_phi_v"
            for key in ("pe", "w1", "b1", "w2", "b2"):
                err = assert_close(np64(g[gk][key]), ref[tag][key], f"{tag}.{key}")
                print(f"[gpu] {case} {tag}.{key}: max abs err {err:.3e}, "
                      f"max |ref| {np.abs(ref[tag][key]).max():.3e}")


def test_backward_is_deterministic():
    import long_context_sparse_phi_amd as nsa
    w = CASES["mlp_d128_selection"]
    cfg = nsa.config_from_workload(w)
    d = to_dev(NI.make_prefill_inputs(w, 0))
    d_o = NI.make_grad_output(w, 0).to("cuda:0")
    fwd = nsa.nsa_fwd_prefill(cfg, d["q"], d["k"], d["v"], d["x"], d["w_gate"], d["phi_k"], d["phi_v"],
                              save_for_backward=True)
    g1 = nsa.nsa_bwd(cfg, d["q"], d["k"], d["v"], d["x"], d["w_gate"], d["phi_k"], d["phi_v"], fwd, d_o)
    g2 = nsa.nsa_bwd(cfg, d["q"], d["k"], d["v"], d["x"], d["w_gate"], d["phi_k"], d["phi_v"], fwd, d_o)
    torch.cuda.synchronize()
    for key in ("dq", "dk", "dv", "dw_gate"):
        assert torch.equal(g1[key], g2[key]), key
    for key in ("pe", "w1", "b1", "w2", "b2"):
        assert torch.equal(g1["d_phi_k"][key], g2["d_phi_k"][key]), key
