"""GPU test of the timed prefill entry point used by the benchmark.

nsa_fwd_prefill_timed does the work of nsa_fwd_prefill with HIP events
between its stages; with one more event it also runs the gather calibration
(the selected branch's walk over the same tiles without its arithmetic).
Neither may change the outputs: every output (o, the compressed keys and
values, lse, the selection, the branch outputs, the block scores and the
gates) is compared bit for bit with the untimed entry point's, and every event must have been
recorded (elapsed times are finite and non-negative).
"""
import ctypes

import numpy as np
import pytest
import torch

import nsa_inputs as NI
from tests.nsa_testutil import to_dev

pytestmark = pytest.mark.gpu


def _events(lib, n):
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventCreate.restype = ctypes.c_int
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    lib.hipEventElapsedTime.restype = ctypes.c_int
    out = []
    for _ in range(n):
        e = ctypes.c_void_p()
        assert lib.hipEventCreate(ctypes.byref(e)) == 0
        out.append(e.value)
    return out


def _elapsed(lib, a, b):
    ms = ctypes.c_float()
    assert lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
    return float(ms.value)


@pytest.mark.parametrize("calibrate", [False, True])
def test_timed_prefill_matches_untimed(calibrate):
    import long_context_sparse_phi_amd as nsa
    from long_context_sparse_phi_amd import _lib
    w = NI.workload("prefill_8k", T=1500, H_kv=2)
    cfg = nsa.config_from_workload(w)
    d = to_dev(NI.make_prefill_inputs(w, 0))
    ref = nsa.nsa_fwd_prefill(cfg, d["q"], d["k"], d["v"], d["x"], d["w_gate"], d["phi_k"], d["phi_v"], debug=True)
    torch.cuda.synchronize()
    lib = _lib.load()
    lib.nsa_fwd_prefill_timed.restype = ctypes.c_int
    lib.nsa_fwd_prefill_timed.argtypes = [ctypes.POINTER(_lib.nsa_params), ctypes.POINTER(_lib.nsa_prefill_args),
                                          ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                          ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]
    dev = torch.device("cuda:0")
    outs = ("o", "k_cmp", "v_cmp", "lse", "idx", "o_branch", "p_slc", "gates")
    got = {n: torch.empty_like(ref[n]) for n in outs}
    ws = torch.empty(nsa.workspace_size(cfg, _lib.NSA_OP_FWD_PREFILL), dtype=torch.uint8, device=dev)
    p = cfg.params()
    a = _lib.nsa_prefill_args()
    for name in ("q", "k", "v", "x", "w_gate"):
        setattr(a, name, d[name].data_ptr())
    a.phi_k = nsa._phi_struct(cfg, d["phi_k"], w.d_k, dev)
    a.phi_v = nsa._phi_struct(cfg, d["phi_v"], w.d_v, dev)
    for n in outs:
        setattr(a, n, got[n].data_ptr())
    nst = lib.nsa_prefill_stage_count()
    n_ev = nst + 2 if calibrate else nst + 1
    evs = _events(lib, n_ev)
    arr = (ctypes.c_void_p * n_ev)(*evs)
    stream = torch.cuda.current_stream(dev).cuda_stream
    print(f"[gpu] timed prefill T={w.T} calibrate={calibrate}", flush=True)
    st = lib.nsa_fwd_prefill_timed(ctypes.byref(p), ctypes.byref(a), ws.data_ptr(), ws.numel(), stream, arr, n_ev)
    assert st == 0, _lib.status_str(st)
    torch.cuda.synchronize()
    for n in outs:
        assert torch.equal(got[n], ref[n]), n
    times = [_elapsed(lib, evs[i], evs[i + 1]) for i in range(n_ev - 1)]
    assert all(np.isfinite(t) and t >= 0 for t in times), times
    # too few events for the stages is rejected before anything runs
    st = lib.nsa_fwd_prefill_timed(ctypes.byref(p), ctypes.byref(a), ws.data_ptr(), ws.numel(), stream, arr, nst)
    assert st == _lib.NSA_ERR_INVALID_ARG
