"""GPU parity of nsa_fwd_decode against the fp64 oracle's decode step.

The compressed caches are the oracle's compression of the raw caches (rounded
to the I/O dtype) and are fed to both sides.  Indices bit-exact outside near
ties; outputs within 2e-2 absolute + 1e-2 relative.  Also: decode at position
S-1 equals the GPU prefill's row S-1 on the same inputs."""
import numpy as np
import pytest
import torch

import nsa_inputs as NI
from tests.nsa_testutil import assert_close, np64, oracle_params

pytestmark = pytest.mark.gpu

W = NI.workload
CASES = {
    "d128_b3": W("decode_64k", B=3, T=1000, H_kv=2, d_k=128, d_v=128, kv_offset_std=0.0, bias_std=0.02),
    "d192_offsets_two_chunks": W("decode_64k", B=1, T=9000, H_kv=1, bias_std=0.02),
    "fp32_mean_g4": W("tiny_fp32", mode="decode", B=2, T=1024),
    "few_blocks": W("decode_64k", B=2, T=300, H_kv=1),
    "no_cmp_block": W("decode_64k", B=1, T=20, H_kv=2),
    "g8_window_larger_than_cache": W("tiny_fp32", mode="decode", dtype="bf16", B=2, T=700, G=8, H_kv=2, w=1000),
    # more than 1024 selection blocks in the score row (l = l' = d = 16)
    "long_score_row_g16": W("decode_64k", B=2, T=16400, H_kv=1, d_k=64, d_v=64, l=16, d=16, l_sel=16, n=8,
                            w=128, hidden=64, bias_std=0.02),
    "long_score_row_g4": W("tiny_fp32", mode="decode", dtype="bf16", B=2, T=16400, l=16, d=16, l_sel=16, n=8,
                           w=128),
}


def oracle_caches(w, inp):
    import oracle as O
    a = NI.to_numpy64(inp)
    p = oracle_params(w)
    return a, O.compress(a["k_cache"], a["phi_k"], p), O.compress(a["v_cache"], a["phi_v"], p)


def run_case(w, seed=0, extra_cap=0):
    import long_context_sparse_phi_amd as nsa
    import oracle as O
    cfg = nsa.config_from_workload(w)
    inp = NI.make_decode_inputs(w, seed)
    a, kc, vc = oracle_caches(w, inp)
    dt = cfg.torch_dtype
    kct = torch.from_numpy(kc).to(dt)
    vct = torch.from_numpy(vc).to(dt)
    if extra_cap:
        # a cache with room for more blocks: the rows past the valid ones hold junk
        kct = torch.cat([kct, 100 * torch.randn(w.B, extra_cap, w.H_kv, w.d_k).to(dt)], dim=1)
        vct = torch.cat([vct, 100 * torch.randn(w.B, extra_cap, w.H_kv, w.d_v).to(dt)], dim=1)
    dev = "cuda:0"
    print(f"[gpu] decode case B={w.B} S={w.T} Hkv={w.H_kv} G={w.G} dk={w.d_k} dtype={w.dtype}", flush=True)
    res = nsa.nsa_fwd_decode(cfg, inp["q"].to(dev), inp["k_cache"].to(dev), inp["v_cache"].to(dev),
                             kct.contiguous().to(dev), vct.contiguous().to(dev), inp["x"].to(dev),
                             inp["w_gate"].to(dev), debug=True)
    torch.cuda.synchronize()
    ref = O.decode(oracle_params(w), a["q"], a["k_cache"], a["v_cache"], kc, vc, a["x"], a["w_gate"],
                   tie_scores=np64(res["p_slc"]))
    return res, ref


def compare(res, ref):
    assert_close(np64(res["p_slc"]), ref["p_slc"], "p_slc", atol=1e-5, rtol=2e-3)
    gi = res["idx"].cpu().numpy().astype(np.int64)
    assert np.array_equal(gi, ref["idx"]), (gi, ref["idx"])
    for c, name in enumerate(("cmp", "slc", "win")):
        assert_close(np64(res["lse"][c]), ref["lse"][c], f"lse_{name}")
        assert_close(np64(res["o_branch"][c]), ref["o_branch"][c], f"o_{name}")
    assert_close(np64(res["o"]), ref["o"], "o")


@pytest.mark.parametrize("case", list(CASES))
def test_decode_matches_oracle(case):
    res, ref = run_case(CASES[case])
    compare(res, ref)


def test_decode_cache_with_spare_capacity():
    res, ref = run_case(W("decode_64k", B=2, T=1500, H_kv=1), extra_cap=37)
    compare(res, ref)


def test_decode_equals_prefill_last_row():
    import long_context_sparse_phi_amd as nsa
    for S in (1024, 4096):
        w = W("prefill_8k", T=S, H_kv=2, bias_std=0.02)
        cfg = nsa.config_from_workload(w)
        inp = NI.make_prefill_inputs(w, 3)
        dev = "cuda:0"
        d = {k: ({kk: vv.to(dev) for kk, vv in v.items()} if isinstance(v, dict) else v.to(dev))
             for k, v in inp.items()}
        print(f"[gpu] decode==prefill S={S}", flush=True)
        pre = nsa.nsa_fwd_prefill(cfg, d["q"], d["k"], d["v"], d["x"], d["w_gate"], d["phi_k"], d["phi_v"],
                                  save_for_backward=True)
        dec = nsa.nsa_fwd_decode(cfg, d["q"][:, S - 1].contiguous(), d["k"], d["v"], pre["k_cmp"], pre["v_cmp"],
                                 d["x"][:, S - 1].contiguous(), d["w_gate"], debug=True)
        torch.cuda.synchronize()
        assert torch.equal(dec["idx"], pre["idx"][:, S - 1])
        assert_close(np64(dec["o"]), np64(pre["o"][:, S - 1]), "o", atol=1e-2, rtol=1e-2)
