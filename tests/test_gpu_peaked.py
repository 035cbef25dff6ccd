"""GPU parity on peaked importance scores.

NSA's selection is meant for score rows on which a few blocks dominate (youleyou
NSA page, 令牌选择: 块级选择, 重要性分数计算 and Top-n块选择).  The workload
recipes give nearly flat rows, so these cases use the peaked recipes (the query
heads of a group share a component and the softmax scale is a multiple of
1/sqrt(d_k)), whose compressed logits span about 60, 130 and 200 nats.  Top-n decisions are then
taken on block scores many orders of magnitude below the row maximum.  The GPU
must still match the oracle bit-exactly on the selected indices outside near
ties (rows whose last kept and first dropped scores are within 1e-3 relative,
or both below 2^-100), and every output within 2e-2 absolute + 1e-2 relative.
Each case prints its near-tie fraction.
"""
import numpy as np
import pytest
import torch

import nsa_inputs as NI
from tests.nsa_testutil import PEAKED, assert_close, np64, oracle_params, to_dev
from tests import test_gpu_decode as DEC
from tests import test_gpu_prefill as PRE
from tests.test_gpu_fullsize import check_decode_sequences, check_prefill_sampled_rows

pytestmark = pytest.mark.gpu

W = NI.workload

PREFILL = {
    "peaked_d128": W("prefill_8k", T=4096, H_kv=2, **PEAKED["peaked"]),
    "steep_d128_ragged": W("prefill_8k", T=4001, H_kv=2, **PEAKED["steep"]),
    "extreme_d192": W("prefill_64k", T=3000, H_kv=2, **PEAKED["extreme"]),
    "steep_mean_g4": W("tiny_fp32", dtype="bf16", T=3000, H_kv=2, q_group_corr=0.95, kv_offset_std=2.0,
                       scale_mult=8.0),
    "steep_g8_d64": W("prefill_8k", T=2500, G=8, H_kv=2, d_k=64, d_v=64, hidden=64, **PEAKED["steep"]),
    "extreme_fp32_mean": W("tiny_fp32", T=2000, q_group_corr=0.95, kv_offset_std=2.0, scale_mult=12.0),
}


def oracle_cmp(w, a):
    """The oracle's compressed keys and values (rounded to the I/O dtype)."""
    import oracle as O
    p = oracle_params(w)
    return O.compress(a["k"], a["phi_k"], p), O.compress(a["v"], a["phi_v"], p)


@pytest.mark.parametrize("case", list(PREFILL))
def test_prefill_peaked(case):
    # On rows spanning tens of nats a one-ulp difference in a bf16 compressed
    # key moves a block's probability by about a percent, and the GPU's fp32
    # phi and the fp64 oracle's round a few keys to neighbouring bf16 values.
    # The score path is therefore compared on the oracle's compressed keys,
    # given to the GPU as an input (phi's own parity is checked elsewhere).
    import long_context_sparse_phi_amd as nsa
    import oracle as O
    w = PREFILL[case]
    cfg = nsa.config_from_workload(w)
    inp = NI.make_prefill_inputs(w, 0)
    a = NI.to_numpy64(inp)
    kc, vc = oracle_cmp(w, a)
    d = to_dev(inp)
    kv_cmp = tuple(torch.from_numpy(x).to(cfg.torch_dtype).contiguous().to("cuda:0") for x in (kc, vc))
    print(f"[gpu] peaked prefill {case}: T={w.T} Hkv={w.H_kv} G={w.G} dk={w.d_k} phi={w.phi}", flush=True)
    res = nsa.nsa_fwd_prefill(cfg, d["q"], d["k"], d["v"], d["x"], d["w_gate"], d["phi_k"], d["phi_v"],
                              debug=True, kv_cmp=kv_cmp)
    torch.cuda.synchronize()
    ref = O.forward(oracle_params(w), a["q"], a["k"], a["v"], a["x"], a["w_gate"], a["phi_k"], a["phi_v"],
                    tie_scores=np64(res["p_slc"]), kc=kc, vc=vc)
    PRE.compare(w, inp, res, ref)
    z = []
    for t in range(w.T // 2, w.T, 97):
        qh = a["q"][0, t, :w.G]
        nv = O.n_cmp_visible(t, w.l, w.d)
        s = oracle_params(w).scale * (qh @ kc[0, :nv, 0].T)
        z.append(np.mean(s.max(axis=1) - s.min(axis=1)))
    print(f"[gpu] {case}: compressed logit range {np.mean(z):.1f} nats, "
          f"near-tie fraction {ref['retied'].mean():.3f}", flush=True)


def test_prefill_64k_steep_sampled_rows():
    frac = check_prefill_sampled_rows(W("prefill_64k", **PEAKED["steep"]), row_seed=5, feed_oracle_cmp=True)
    assert frac < 0.5


DECODE = {
    "steep_d128_b3": W("decode_64k", B=3, T=6000, H_kv=2, d_k=128, d_v=128, kv_offset_std=0.0, **PEAKED["steep"]),
    "extreme_d192_b2": W("decode_64k", B=2, T=9000, H_kv=1, **PEAKED["extreme"]),
}


@pytest.mark.parametrize("case", list(DECODE))
def test_decode_peaked(case):
    res, ref = DEC.run_case(DECODE[case])
    DEC.compare(res, ref)
    print(f"[gpu] {case}: near-tie fraction {ref['retied'].mean():.3f}", flush=True)


def test_decode_64k_steep_sequences():
    frac = check_decode_sequences(W("decode_64k", B=2, **PEAKED["steep"]), (0, 1), feed_oracle_cmp=True)
    print(f"[gpu] 64K decode steep: near-tie fraction {frac:.3f}")


BACKWARD = {
    "peaked_d128": W("train_16k", B=1, T=1500, H_kv=2, **PEAKED["peaked"]),
    "peaked_d192": W("prefill_64k", mode="train", T=1300, H_kv=1, **PEAKED["peaked"]),
    "steep_d192": W("prefill_64k", mode="train", T=1300, H_kv=1, **PEAKED["steep"]),
    # the same with the row terms recomputed from the probabilities instead of
    # read from the saved branch outputs
    "steep_d128/recompute": W("train_16k", B=1, T=1200, H_kv=2, **PEAKED["steep"]),
}

# Beyond about 100 nats a softmax row is nearly one-hot, so dS = P (dP - D)
# cancels and the compressed keys' gradients and phi's hidden-layer gradient
# come out as differences of large terms.  The kernels carry those factors
# with about 16 significant bits.  phi's weight gradients sum them over every
# compressed block: entries reach 1e3 while single entries of a few 1e-2 are
# left after the cancellation.  Fed the same 16-bit precision (every saved
# branch output perturbed by 2^-17), the fp64 oracle itself misses such
# entries by up to 1e-4 of the largest.  In the steep cases phi's weight
# gradients are therefore held to that precision:
#     |gpu - oracle| <= 2e-2 + 1e-2 |oracle| + 2^-13 max|oracle|,
# and every other output, and the peaked cases throughout, to the plain bound.
# (At the extreme recipe's 300 nats phi_k's bias gradient, which is exactly 0
# because every row of dS sums to 0, comes out as a cancellation of 16-bit
# terms near 1e2 and lands near 3e-2; the backward is not run there.)
STEEP_PHI_REL = 2.0 ** -13


@pytest.mark.parametrize("case", list(BACKWARD))
def test_backward_peaked(case):
    # the forward runs on the oracle's compressed keys (see test_prefill_peaked);
    # the backward then takes them as the forward's saved k_cmp, v_cmp
    import long_context_sparse_phi_amd as nsa
    import oracle as O
    w = BACKWARD[case]
    cfg = nsa.config_from_workload(w)
    inp = NI.make_prefill_inputs(w, 0)
    d_o = NI.make_grad_output(w, 0)
    a = NI.to_numpy64(inp)
    kc, vc = oracle_cmp(w, a)
    d = to_dev(inp)
    kv_cmp = tuple(torch.from_numpy(x).to(cfg.torch_dtype).contiguous().to("cuda:0") for x in (kc, vc))
    print(f"[gpu] peaked backward {case}: T={w.T} Hkv={w.H_kv} G={w.G} dk={w.d_k}", flush=True)
    fwd = nsa.nsa_fwd_prefill(cfg, d["q"], d["k"], d["v"], d["x"], d["w_gate"], d["phi_k"], d["phi_v"],
                              debug=True, kv_cmp=kv_cmp)
    g = nsa.nsa_bwd(cfg, d["q"], d["k"], d["v"], d["x"], d["w_gate"], d["phi_k"], d["phi_v"], fwd,
                    d_o.to("cuda:0"), recompute_row_terms=case.endswith("/recompute"))
    torch.cuda.synchronize()
    p = oracle_params(w)
    ref_f = O.forward(p, a["q"], a["k"], a["v"], a["x"], a["w_gate"], a["phi_k"], a["phi_v"],
                      tie_scores=np64(fwd["p_slc"]), kc=kc, vc=vc)
    assert np.array_equal(ref_f["idx"], fwd["idx"].cpu().numpy().astype(np.int64))
    ref = O.backward(p, a["q"], a["k"], a["v"], a["x"], a["w_gate"], a["phi_k"], a["phi_v"], np64(d_o),
                     ref_f["idx"])
    for name in ("dq", "dk", "dv", "dw_gate"):
        err = assert_close(np64(g[name]), ref[name], name)
        print(f"[gpu] {case} {name}: max abs err {err:.3e}, max |ref| {np.abs(ref[name]).max():.3e}")
    for tag, gk in (("dphi_k", "d_phi_k"), ("dphi_v", "d_phi_v")):
        for key in ("pe", "w1", "b1", "w2", "b2"):
            r = ref[tag][key]
            atol = 2e-2 + (0.0 if case.startswith("peaked") else STEEP_PHI_REL * np.abs(r).max())
            err = assert_close(np64(g[gk][key]), r, f"{tag}.{key}", atol=atol)
            print(f"[gpu] {case} {tag}.{key}: max abs err {err:.3e} ({err / np.abs(r).max():.1e} of max |ref| "
                  f"{np.abs(r).max():.3e})")
    print(f"[gpu] {case}: near-tie fraction {ref_f['retied'].mean():.3f}", flush=True)
