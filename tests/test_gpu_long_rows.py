"""GPU parity of the prefill forward when a position's score row holds more
than 1024 selection blocks (nsel = ceil(T / l') > 1024).

Score rows that long take other paths of the compressed branch's second pass:
the per-position top-n (instead of the two-position register form used up to
1024 blocks) and, when the rows no longer fit beside two 4-wave workgroups'
tiles, the 8-wave or one-column-tile launch shapes.  With l = l' = d = 16 the
row length passes 1024 at T = 16400; sampled positions (block and window
boundaries, the last positions, seeded random ones) are compared with the
oracle as in the full-size tests: indices bit-exact (near ties re-selected from
the GPU's exported scores), floats within 2e-2 absolute + 1e-2 relative."""
import numpy as np
import pytest
import torch

import nsa_inputs as NI
from tests.nsa_testutil import SampledRows, assert_close, np64, oracle_params, to_dev
from tests.test_gpu_fullsize import sample_rows

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]

W = NI.workload
CASES = {
    # G = 4: four positions per column tile, the score rows take the one-column-tile shape
    "g4_mean_d64": W("tiny_fp32", dtype="bf16", T=16400, l=16, d=16, l_sel=16, n=8, w=128),
    # G = 16: one position per column tile, the default shape with the per-position top-n
    "g16_mlp_d64": W("prefill_8k", T=16400, H_kv=1, G=16, d_k=64, d_v=64, l=16, d=16, l_sel=16, n=8, w=128,
                     hidden=64, bias_std=0.02),
}


@pytest.mark.parametrize("case", list(CASES))
def test_prefill_score_rows_longer_than_1024(case):
    import long_context_sparse_phi_amd as nsa
    import oracle as O
    w = CASES[case]
    assert -(-w.T // w.l_sel) > 1024
    cfg = nsa.config_from_workload(w)
    inp = NI.make_prefill_inputs(w, 3)
    d = to_dev(inp)
    print(f"[gpu] long score rows {case}: T={w.T} nsel={-(-w.T // w.l_sel)} G={w.G} dk={w.d_k} phi={w.phi}",
          flush=True)
    res = nsa.nsa_fwd_prefill(cfg, d["q"], d["k"], d["v"], d["x"], d["w_gate"], d["phi_k"], d["phi_v"], debug=True)
    torch.cuda.synchronize()
    rows = sample_rows(w.T, w.l_sel, w.w, seed=5)
    rt = torch.from_numpy(rows).to("cuda:0")
    g = {"o": np64(res["o"][:, rt]), "o_branch": np64(res["o_branch"][:, :, rt]), "lse": np64(res["lse"][:, :, rt]),
         "p_slc": np64(res["p_slc"][:, rt]), "idx": res["idx"][:, rt].cpu().numpy().astype(np.int64)}
    del res, d
    p = oracle_params(w)
    k = inp["k"].double().numpy()
    v = inp["v"].double().numpy()
    phi_k, phi_v = NI.to_numpy64(inp["phi_k"]), NI.to_numpy64(inp["phi_v"])
    kc = O.compress(k, phi_k, p)
    vc = O.compress(v, phi_v, p)
    ref = O.forward(p, SampledRows(inp["q"][:, rows].double().numpy(), rows, w.T), k, v,
                    inp["x"].double().numpy(), inp["w_gate"].double().numpy(), phi_k, phi_v, rows=rows,
                    tie_scores=SampledRows(g["p_slc"], rows, w.T), kc=kc, vc=vc)
    assert_close(g["p_slc"], ref["p_slc"], "p_slc", atol=1e-5, rtol=2e-3)
    mism = np.argwhere(np.any(g["idx"] != ref["idx"], axis=-1))
    assert len(mism) == 0, f"idx mismatch at rows {rows[mism[:, 1]].tolist()}"
    for c, name in enumerate(("cmp", "slc", "win")):
        assert_close(g["lse"][c], ref["lse"][c], f"lse_{name}")
        assert_close(g["o_branch"][c], ref["o_branch"][c], f"o_{name}")
    assert_close(g["o"], ref["o"], "o")
    print(f"[gpu] {case}: {len(rows)} rows checked, near ties re-selected: {int(ref['retied'].sum())}")
