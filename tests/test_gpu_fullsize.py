"""GPU parity at the full benchmark sizes, in the launch configurations the
benchmark times, on outputs the fp64 oracle can compute one by one:

* 64K prefill (B=1, T=65536, 4 KV x 16 query heads, d_k=192, d_v=128, MLP phi):
  every compressed key and value, and all outputs, scores and selected indices
  of sampled query positions (block and window boundaries, the last position,
  seeded random ones);
* 64K decode (32 sequences): the compressed caches and the decode outputs of
  sampled sequences;
* 16K training shape (B=2, T=16384, d=128): dq of sampled positions, with the
  selected indices checked first.

Tolerances as in the small-size tests: indices bit-exact (near ties re-selected
from the GPU's exported scores), floating outputs within 2e-2 absolute + 1e-2
relative."""
import numpy as np
import pytest
import torch

import nsa_inputs as NI
from tests.nsa_testutil import SampledRows, assert_close, np64, oracle_params, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


def sample_rows(T, ls, w, seed, n_random=6):
    base = [0, 1, 31, 32, 47, ls - 1, ls, 2 * ls - 1, w - 1, w, w + 1, T // 4, T // 2 - 1, T // 2,
            (3 * T) // 4 + 17, T - ls - 1, T - ls, T - 2, T - 1]
    rng = np.random.default_rng(seed)
    extra = rng.integers(0, T, size=n_random).tolist()
    return np.array(sorted({int(t) for t in base + extra if 0 <= t < T}), dtype=np.int64)


def test_prefill_64k_sampled_rows():
    import long_context_sparse_phi_amd as nsa
    import oracle as O
    w = NI.workload("prefill_64k")
    cfg = nsa.config_from_workload(w)
    inp = NI.make_prefill_inputs(w, 0)
    d = to_dev(inp)
    print(f"[gpu] full-size prefill T={w.T} Hkv={w.H_kv} G={w.G} dk={w.d_k}", flush=True)
    res = nsa.nsa_fwd_prefill(cfg, d["q"], d["k"], d["v"], d["x"], d["w_gate"], d["phi_k"], d["phi_v"], debug=True)
    torch.cuda.synchronize()
    del d
    rows = sample_rows(w.T, w.l_sel, w.w, seed=1)
    rt = torch.from_numpy(rows).to("cuda:0")
    g = {"o": np64(res["o"][:, rt]), "o_branch": np64(res["o_branch"][:, :, rt]), "lse": np64(res["lse"][:, :, rt]),
         "p_slc": np64(res["p_slc"][:, rt]), "idx": res["idx"][:, rt].cpu().numpy().astype(np.int64),
         "gates": np64(res["gates"][:, rt]), "k_cmp": np64(res["k_cmp"]), "v_cmp": np64(res["v_cmp"])}
    del res
    torch.cuda.empty_cache()
    p = oracle_params(w)
    k = inp["k"].double().numpy()
    v = inp["v"].double().numpy()
    phi_k, phi_v = NI.to_numpy64(inp["phi_k"]), NI.to_numpy64(inp["phi_v"])
    kc = O.compress(k, phi_k, p)
    vc = O.compress(v, phi_v, p)
    assert_close(g["k_cmp"], kc, "k_cmp")
    assert_close(g["v_cmp"], vc, "v_cmp")
    ref = O.forward(p, SampledRows(inp["q"][:, rows].double().numpy(), rows, w.T), k, v,
                    inp["x"].double().numpy(), inp["w_gate"].double().numpy(), phi_k, phi_v, rows=rows,
                    tie_scores=SampledRows(g["p_slc"], rows, w.T), kc=kc, vc=vc)
    assert_close(g["gates"], ref["gates"], "gates", atol=1e-5, rtol=1e-5)
    assert_close(g["p_slc"], ref["p_slc"], "p_slc", atol=1e-5, rtol=2e-3)
    mism = np.argwhere(np.any(g["idx"] != ref["idx"], axis=-1))
    assert len(mism) == 0, f"idx mismatch at rows {rows[mism[:, 1]].tolist()}"
    for c, name in enumerate(("cmp", "slc", "win")):
        assert_close(g["lse"][c], ref["lse"][c], f"lse_{name}")
        assert_close(g["o_branch"][c], ref["o_branch"][c], f"o_{name}")
    assert_close(g["o"], ref["o"], "o")
    print(f"[gpu] 64K prefill: {len(rows)} rows checked, near ties re-selected: {int(ref['retied'].sum())}")


def test_decode_64k_sampled_sequences():
    import long_context_sparse_phi_amd as nsa
    import oracle as O
    w = NI.workload("decode_64k")
    cfg = nsa.config_from_workload(w)
    inp = NI.make_decode_inputs(w, 0)
    d = to_dev(inp)
    print(f"[gpu] full-size decode B={w.B} S={w.T} Hkv={w.H_kv} G={w.G} dk={w.d_k}", flush=True)
    kct = nsa.nsa_compress(cfg, d["k_cache"], d["phi_k"], False)
    vct = nsa.nsa_compress(cfg, d["v_cache"], d["phi_v"], True)
    res = nsa.nsa_fwd_decode(cfg, d["q"], d["k_cache"], d["v_cache"], kct, vct, d["x"], d["w_gate"], debug=True)
    torch.cuda.synchronize()
    p = oracle_params(w)
    phi_k, phi_v = NI.to_numpy64(inp["phi_k"]), NI.to_numpy64(inp["phi_v"])
    for b in (0, 13, w.B - 1):
        sl = slice(b, b + 1)
        kcache = inp["k_cache"][sl].double().numpy()
        vcache = inp["v_cache"][sl].double().numpy()
        kc = O.compress(kcache, phi_k, p)
        vc = O.compress(vcache, phi_v, p)
        assert_close(np64(kct[sl, :kc.shape[1]]), kc, f"k_cmp_cache[{b}]")
        assert_close(np64(vct[sl, :vc.shape[1]]), vc, f"v_cmp_cache[{b}]")
        ref = O.decode(p, inp["q"][sl].double().numpy(), kcache, vcache, kc, vc, inp["x"][sl].double().numpy(),
                       inp["w_gate"].double().numpy(), tie_scores=np64(res["p_slc"][sl]))
        assert_close(np64(res["p_slc"][sl]), ref["p_slc"], f"p_slc[{b}]", atol=1e-5, rtol=2e-3)
        gi = res["idx"][sl].cpu().numpy().astype(np.int64)
        assert np.array_equal(gi, ref["idx"]), (b, gi, ref["idx"])
        for c, name in enumerate(("cmp", "slc", "win")):
            assert_close(np64(res["lse"][c][sl]), ref["lse"][c], f"lse_{name}[{b}]")
            assert_close(np64(res["o_branch"][c][sl]), ref["o_branch"][c], f"o_{name}[{b}]")
        assert_close(np64(res["o"][sl]), ref["o"], f"o[{b}]")
        print(f"[gpu] 64K decode sequence {b} checked", flush=True)


def test_train_16k_sampled_dq():
    import long_context_sparse_phi_amd as nsa
    import oracle as O
    w = NI.workload("train_16k")
    cfg = nsa.config_from_workload(w)
    inp = NI.make_prefill_inputs(w, 0)
    d_o = NI.make_grad_output(w, 0)
    d = to_dev(inp)
    print(f"[gpu] full-size backward B={w.B} T={w.T} Hkv={w.H_kv} G={w.G} dk={w.d_k}", flush=True)
    fwd = nsa.nsa_fwd_prefill(cfg, d["q"], d["k"], d["v"], d["x"], d["w_gate"], d["phi_k"], d["phi_v"], debug=True)
    grads = nsa.nsa_bwd(cfg, d["q"], d["k"], d["v"], d["x"], d["w_gate"], d["phi_k"], d["phi_v"], fwd,
                        d_o.to("cuda:0"))
    torch.cuda.synchronize()
    rows = sample_rows(w.T, w.l_sel, w.w, seed=2, n_random=4)
    rt = torch.from_numpy(rows).to("cuda:0")
    g_dq = np64(grads["dq"][:, rt])
    g_idx = fwd["idx"][:, rt].cpu().numpy().astype(np.int64)
    g_ps = np64(fwd["p_slc"][:, rt])
    del grads, fwd, d
    torch.cuda.empty_cache()
    p = oracle_params(w)
    k = inp["k"].double().numpy()
    v = inp["v"].double().numpy()
    phi_k, phi_v = NI.to_numpy64(inp["phi_k"]), NI.to_numpy64(inp["phi_v"])
    kc = O.compress(k, phi_k, p)
    vc = O.compress(v, phi_v, p)
    q_rows = inp["q"][:, rows].double().numpy()
    x = inp["x"].double().numpy()
    wg = inp["w_gate"].double().numpy()
    ref_f = O.forward(p, SampledRows(q_rows, rows, w.T), k, v, x, wg, phi_k, phi_v, rows=rows,
                      tie_scores=SampledRows(g_ps, rows, w.T), kc=kc, vc=vc)
    assert np.array_equal(ref_f["idx"], g_idx)
    dq = O.dq_rows(p, q_rows, k, v, kc, vc, ref_f["gates"], d_o[:, rows].double().numpy(), ref_f["idx"], rows)
    assert_close(g_dq, dq, "dq")
    print(f"[gpu] 16K backward: dq of {len(rows)} rows x {w.B} sequences checked", flush=True)
