"""GPU parity of the two-layer gate MLP (g = sigmoid(gelu(x W1 + b1) W_g + b2))
and of the gate input's gradient dx, against the fp64 oracle: prefill forward,
backward (dW_g, dW1, db1, db2, dx and the attention gradients) and decode.
Indices bit-exact outside near ties; floats within 2e-2 absolute + 1e-2
relative of the oracle."""
import numpy as np
import pytest
import torch

import nsa_inputs as NI
from tests.nsa_testutil import assert_close, np64, oracle_params, to_dev

pytestmark = pytest.mark.gpu

W = NI.workload
DEV = "cuda:0"

CASES = {
    "mlp_d128_hg64": W("train_16k", B=1, T=700, H_kv=2, G=4, n=6, w=128, bias_std=0.02, gate_hidden=64),
    "mean_fp32_hg96": W("tiny_fp32", mode="train", B=2, T=300, gate_hidden=96),
    "mlp_d192_hg256": W("prefill_64k", mode="train", T=520, H_kv=1, n=6, w=100, gate_hidden=256),
    "linear_gate_dx": W("train_16k", B=1, T=600, H_kv=2, G=4, n=6, w=128),
}


@pytest.mark.parametrize("case", list(CASES))
def test_gate_mlp_prefill_and_backward(case):
    import long_context_sparse_phi_amd as nsa
    import oracle as O
    w = CASES[case]
    cfg = nsa.config_from_workload(w)
    inp = NI.make_prefill_inputs(w, 0)
    d_o = NI.make_grad_output(w, 0)
    d = to_dev(inp)
    mlp_dev = d.get("gate_mlp")
    print(f"[gpu] gate case {case} T={w.T} gate_hidden={w.gate_hidden}", flush=True)
    fwd = nsa.nsa_fwd_prefill(cfg, d["q"], d["k"], d["v"], d["x"], d["w_gate"], d["phi_k"], d["phi_v"],
                              debug=True, gate_mlp=mlp_dev)
    g = nsa.nsa_bwd(cfg, d["q"], d["k"], d["v"], d["x"], d["w_gate"], d["phi_k"], d["phi_v"], fwd,
                    d_o.to(DEV), gate_mlp=mlp_dev, want_dx=True)
    torch.cuda.synchronize()
    a = NI.to_numpy64(inp)
    mlp = a.get("gate_mlp")
    p = oracle_params(w)
    ref = O.forward(p, a["q"], a["k"], a["v"], a["x"], a["w_gate"], a["phi_k"], a["phi_v"],
                    tie_scores=np64(fwd["p_slc"]), gate_mlp=mlp)
    assert np.array_equal(fwd["idx"].cpu().numpy().astype(np.int64), ref["idx"])
    assert_close(np64(fwd["gates"]), ref["gates"], "gates", atol=2e-3, rtol=2e-3)
    assert_close(np64(fwd["o"]), ref["o"], "o")
    rg = O.backward(p, a["q"], a["k"], a["v"], a["x"], a["w_gate"], a["phi_k"], a["phi_v"], np64(d_o),
                    ref["idx"], gate_mlp=mlp)
    for name in ("dq", "dk", "dv", "dw_gate", "dx"):
        err = assert_close(np64(g[name]), rg[name], name)
        print(f"[gpu] {case} {name}: max abs err {err:.3e}, max |ref| {np.abs(rg[name]).max():.3e}")
    if mlp is not None:
        for key in ("w1", "b1", "b2"):
            err = assert_close(np64(g["d_gate_mlp"][key]), rg["dgate_mlp"][key], f"dgate_mlp.{key}")
            print(f"[gpu] {case} dgate_mlp.{key}: max abs err {err:.3e}")
    else:
        assert "d_gate_mlp" not in g


def test_gate_mlp_decode_ragged():
    import long_context_sparse_phi_amd as nsa
    import oracle as O
    w = W("decode_64k", B=3, T=1300, H_kv=2, bias_std=0.02, gate_hidden=128)
    p = oracle_params(w)
    cfg = nsa.config_from_workload(w)
    inp = NI.make_decode_inputs(w, 6)
    a = NI.to_numpy64(inp)
    kc = O.compress(a["k_cache"], a["phi_k"], p)
    vc = O.compress(a["v_cache"], a["phi_v"], p)
    dt = cfg.torch_dtype
    lens = [1300, 611, 45]
    print("[gpu] gate MLP decode", flush=True)
    res = nsa.nsa_fwd_decode(cfg, inp["q"].to(DEV), inp["k_cache"].to(DEV), inp["v_cache"].to(DEV),
                             torch.from_numpy(kc).to(dt).to(DEV), torch.from_numpy(vc).to(dt).to(DEV),
                             inp["x"].to(DEV), inp["w_gate"].to(DEV), debug=True,
                             seq_lens=torch.tensor(lens, dtype=torch.int32, device=DEV),
                             gate_mlp=to_dev(inp["gate_mlp"]))
    torch.cuda.synchronize()
    ref = O.decode(p, a["q"], a["k_cache"], a["v_cache"], kc, vc, a["x"], a["w_gate"],
                   tie_scores=np64(res["p_slc"]), seq_lens=lens, gate_mlp=a["gate_mlp"])
    assert np.array_equal(res["idx"].cpu().numpy().astype(np.int64), ref["idx"])
    for c, name in enumerate(("cmp", "slc", "win")):
        assert_close(np64(res["o_branch"][c]), ref["o_branch"][c], f"o_{name}")
    assert_close(np64(res["o"]), ref["o"], "o")
    # the gates themselves: the gated sum of the GPU's own branch outputs
    # must reproduce its output with the oracle's gates
    ob = np64(res["o_branch"])
    recon = np.einsum("bhc,cbhd->bhd", ref["gates"], ob)
    assert_close(np64(res["o"]), recon, "o from oracle gates", atol=1e-2, rtol=1e-2)


def test_gate_mlp_rejects_missing_weights():
    import long_context_sparse_phi_amd as nsa
    from long_context_sparse_phi_amd import _lib
    w = CASES["mean_fp32_hg96"]
    cfg = nsa.config_from_workload(w)
    d = to_dev(NI.make_prefill_inputs(w, 1))
    with pytest.raises(ValueError):
        nsa.nsa_fwd_prefill(cfg, d["q"], d["k"], d["v"], d["x"], d["w_gate"])
    # through the C ABI with a null w1: invalid argument, nothing launched
    a = _lib.nsa_prefill_args()
    for name in ("q", "k", "v", "x", "w_gate"):
        setattr(a, name, d[name].data_ptr())
    o = torch.empty(w.B, w.T, w.H_q, w.d_v, device=DEV)
    a.o = o.data_ptr()
    a.gate_mlp = _lib.nsa_gate_mlp(w1=None, b1=d["gate_mlp"]["b1"].data_ptr(), b2=d["gate_mlp"]["b2"].data_ptr())
    p = cfg.params()
    ws = torch.empty(nsa.workspace_size(cfg, _lib.NSA_OP_FWD_PREFILL), dtype=torch.uint8, device=DEV)
    st = _lib.load().nsa_fwd_prefill(p, a, ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert st == _lib.NSA_ERR_INVALID_ARG
