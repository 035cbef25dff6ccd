"""GPU test of nsa_fwd_decode_noalloc, the decode entry point that takes no
workspace and allocates nothing (for callers that cannot allocate: code under
HIP graph capture, allocation-free serving loops).

Called raw through the C ABI (ctypes), it must reproduce nsa_fwd_decode, the
entry point with a caller workspace, on the same inputs, on two calls in a row
(the second smaller, so it runs over what the first left in the shared static
buffer), and must reject a problem larger than that buffer before launching
anything."""
import ctypes

import numpy as np
import pytest
import torch

import nsa_inputs as NI
from tests.nsa_testutil import assert_close, np64, oracle_params

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _decode_args(cfg, d, kct, vct, res):
    from long_context_sparse_phi_amd import _lib
    a = _lib.nsa_decode_args()
    for name in ("q", "k_cache", "v_cache", "x", "w_gate"):
        setattr(a, name, d[name].data_ptr())
    a.k_cmp_cache, a.v_cmp_cache = kct.data_ptr(), vct.data_ptr()
    a.cmp_cache_cap = kct.shape[1]
    for name in ("o", "idx", "p_slc", "lse", "o_branch"):
        setattr(a, name, res[name].data_ptr())
    return a


def _outputs(cfg, w):
    f32 = torch.float32
    return {"o": torch.full((w.B, w.H_q, w.d_v), float("nan"), dtype=cfg.torch_dtype, device=DEV),
            "idx": torch.full((w.B, w.H_kv, w.n), -7, dtype=torch.int32, device=DEV),
            "p_slc": torch.full((w.B, w.H_kv, cfg.n_sel), float("nan"), dtype=f32, device=DEV),
            "lse": torch.full((3, w.B, w.H_q), float("nan"), dtype=f32, device=DEV),
            "o_branch": torch.full((3, w.B, w.H_q, w.d_v), float("nan"), dtype=f32, device=DEV)}


def _run_pair(w, seed):
    """nsa_fwd_decode_noalloc through ctypes, then nsa_fwd_decode on the same inputs."""
    import long_context_sparse_phi_amd as nsa
    from long_context_sparse_phi_amd import _lib
    cfg = nsa.config_from_workload(w)
    inp = NI.make_decode_inputs(w, seed)
    d = {k: (v.to(DEV) if torch.is_tensor(v) else {kk: vv.to(DEV) for kk, vv in v.items()})
         for k, v in inp.items()}
    kct = nsa.nsa_compress(cfg, d["k_cache"], d["phi_k"], False)
    vct = nsa.nsa_compress(cfg, d["v_cache"], d["phi_v"], True)
    res = _outputs(cfg, w)
    a = _decode_args(cfg, d, kct, vct, res)
    p = cfg.params()
    print(f"[gpu] nsa_fwd_decode_noalloc B={w.B} S={w.T} Hkv={w.H_kv} G={w.G} dk={w.d_k}", flush=True)
    st = _lib.load().nsa_fwd_decode_noalloc(ctypes.byref(p), ctypes.byref(a),
                                           torch.cuda.current_stream().cuda_stream)
    assert st == 0, _lib.status_str(st)
    torch.cuda.synchronize()
    ref = nsa.nsa_fwd_decode(cfg, d["q"], d["k_cache"], d["v_cache"], kct, vct, d["x"], d["w_gate"], debug=True)
    torch.cuda.synchronize()
    return inp, kct, vct, res, ref


def _check_same(res, ref):
    for key in ("o", "idx", "p_slc", "lse", "o_branch"):
        assert torch.equal(res[key], ref[key]), key


def test_noalloc_decode_matches_workspace_decode_twice():
    # a 16K-token cache of 8 sequences, then a smaller problem (3 sequences,
    # 5000 tokens, fewer heads) over whatever the first call left in the buffer
    big = NI.workload("decode_64k", B=8, T=16384, bias_std=0.02)
    small = NI.workload("decode_64k", B=3, T=5000, H_kv=2, d_k=128, d_v=128, bias_std=0.02)
    for w, seed in ((big, 0), (small, 1)):
        inp, kct, vct, res, ref = _run_pair(w, seed)
        _check_same(res, ref)
    # the second, smaller call also against the oracle (its compressed caches
    # as the GPU built them; these are compared with the oracle's elsewhere)
    import oracle as O
    a = NI.to_numpy64(inp)
    oref = O.decode(oracle_params(small), a["q"], a["k_cache"], a["v_cache"], np64(kct), np64(vct), a["x"],
                    a["w_gate"], tie_scores=np64(res["p_slc"]))
    assert np.array_equal(res["idx"].cpu().numpy(), oref["idx"])
    assert_close(np64(res["o"]), oref["o"], "o")


def test_noalloc_decode_rejects_problems_beyond_the_buffer():
    import long_context_sparse_phi_amd as nsa
    from long_context_sparse_phi_amd import _lib
    # 256 sequences of 64K tokens need far more than the static buffer; the
    # call must refuse before touching any pointer (none of these is read)
    w = NI.workload("decode_64k", B=256)
    cfg = nsa.config_from_workload(w)
    assert nsa.workspace_size(cfg, _lib.NSA_OP_FWD_DECODE) > 64 << 20
    dummy = torch.zeros(64, dtype=torch.float32, device=DEV)
    a = _lib.nsa_decode_args()
    for name in ("q", "k_cache", "v_cache", "x", "w_gate", "k_cmp_cache", "v_cmp_cache", "o"):
        setattr(a, name, dummy.data_ptr())
    a.cmp_cache_cap = cfg.n_cmp
    p = cfg.params()
    st = _lib.load().nsa_fwd_decode_noalloc(ctypes.byref(p), ctypes.byref(a),
                                           torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 7, _lib.status_str(st)   # NSA_ERR_SCRATCH
    assert torch.count_nonzero(dummy) == 0
