"""The C-ABI library loads and exports every entry point include/nsa.h declares.
CPU only: no compute call is made."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "long_context_sparse_phi_amd", "libnsa.so")
HEADER = os.path.join(ROOT, "include", "nsa.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nsa_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libnsa.so is not built (run __graft_entry__.build())")
    return ctypes.CDLL(LIB)


def test_header_declares_the_three_entry_points():
    fns = declared_functions()
    for f in ("nsa_fwd_prefill", "nsa_fwd_decode", "nsa_bwd", "nsa_workspace_size"):
        assert f in fns


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings(lib):
    lib.nsa_abi_version.restype = ctypes.c_int
    assert lib.nsa_abi_version() == 5
    lib.nsa_status_str.restype = ctypes.c_char_p
    lib.nsa_status_str.argtypes = [ctypes.c_int]
    assert lib.nsa_status_str(0) == b"ok"
    assert lib.nsa_status_str(3).startswith(b"workspace")


def test_ctypes_mirror_matches_header_and_validation_runs_on_host():
    import long_context_sparse_phi_amd as nsa
    from long_context_sparse_phi_amd import _lib
    # nsa_params: 15 int32 + 1 float
    assert ctypes.sizeof(_lib.nsa_params) == 68
    cfg = nsa.Config(B=1, T=1024, H_kv=1, G=4, d_k=64, d_v=64, n=4, w=128, phi="mean", dtype="fp32")
    assert nsa.workspace_size(cfg, _lib.NSA_OP_FWD_PREFILL) > 0
    bad = nsa.Config(B=1, T=1024, H_kv=1, G=3, d_k=64, d_v=64)
    with pytest.raises(nsa.NSAError) as e:
        nsa.workspace_size(bad, _lib.NSA_OP_FWD_PREFILL)
    assert e.value.code == _lib.NSA_ERR_UNSUPPORTED
    bad = nsa.Config(B=1, T=1024, H_kv=1, G=4, d_k=64, d_v=64, l=24, d=16)
    with pytest.raises(nsa.NSAError) as e:
        nsa.workspace_size(bad, _lib.NSA_OP_FWD_PREFILL)
    assert e.value.code == _lib.NSA_ERR_INVALID_ARG
    bad = nsa.Config(B=1, T=1024, H_kv=1, G=4, d_k=64, d_v=64, n=2)
    with pytest.raises(nsa.NSAError) as e:
        nsa.workspace_size(bad, _lib.NSA_OP_FWD_PREFILL)
    assert e.value.code == _lib.NSA_ERR_INVALID_ARG
    # a key row of every KV head must stay below 2^24 elements
    bad = nsa.Config(B=1, T=64, H_kv=(1 << 24) // 192 + 1, G=1, d_k=192, d_v=128)
    with pytest.raises(nsa.NSAError) as e:
        nsa.workspace_size(bad, _lib.NSA_OP_FWD_DECODE)
    assert e.value.code == _lib.NSA_ERR_UNSUPPORTED


def test_dense_bwd_rejects_fp32_wide_heads_before_touching_memory():
    # fp32 with d_k = 128: the key tiles do not fit the local memory, which is
    # reported before any pointer is used (the pointers here are never valid)
    import long_context_sparse_phi_amd as nsa
    from long_context_sparse_phi_amd import _lib
    lib = _lib.load()
    cfg = nsa.Config(B=1, T=256, H_kv=1, G=4, d_k=128, d_v=128, phi="mean", dtype="fp32")
    p = cfg.params()
    a = _lib.nsa_dense_bwd_args(**{n: 4096 for n in ("q", "k", "v", "o", "lse", "d_o", "dq", "dk", "dv")})
    st = lib.nsa_dense_bwd(ctypes.byref(p), ctypes.byref(a), None, 0, None)
    assert st == _lib.NSA_ERR_UNSUPPORTED


def test_gate_hidden_width_is_validated_on_host():
    import long_context_sparse_phi_amd as nsa
    from long_context_sparse_phi_amd import _lib
    ok = nsa.Config(B=1, T=512, H_kv=1, G=4, d_k=64, d_v=64, n=4, w=128, phi="mean", gate_hidden=64)
    assert nsa.workspace_size(ok, _lib.NSA_OP_BWD) > nsa.workspace_size(
        nsa.Config(B=1, T=512, H_kv=1, G=4, d_k=64, d_v=64, n=4, w=128, phi="mean"), _lib.NSA_OP_BWD)
    for bad_width in (-1, 1025):
        bad = nsa.Config(B=1, T=512, H_kv=1, G=4, d_k=64, d_v=64, n=4, w=128, phi="mean", gate_hidden=bad_width)
        with pytest.raises(nsa.NSAError) as e:
            nsa.workspace_size(bad, _lib.NSA_OP_FWD_PREFILL)
        assert e.value.code == _lib.NSA_ERR_INVALID_ARG


def test_append_args_mirror_and_partial_branch_pairs_rejected_on_host():
    """nsa_append_args keeps its earlier fields in place and adds the selected
    and window branches' quartets; a quartet given in part is rejected before
    any pointer is used (the pointers here are never valid)."""
    import long_context_sparse_phi_amd as nsa
    from long_context_sparse_phi_amd import _lib
    A = _lib.nsa_append_args
    ptr = ctypes.sizeof(ctypes.c_void_p)
    assert A.k_new.offset == 0 and A.cmp_cache_cap.offset == 7 * ptr
    assert A.k_slc_new.offset == A.phi_v.offset + ctypes.sizeof(_lib.nsa_phi_weights)
    assert A.v_win_cache.offset == A.k_slc_new.offset + 7 * ptr
    lib = _lib.load()
    cfg = nsa.Config(B=1, T=256, H_kv=1, G=4, d_k=64, d_v=64, n=4, w=64, phi="mean")
    p = cfg.params()
    base = {n: 4096 for n in ("k_new", "v_new", "seq_lens", "k_cache", "v_cache", "k_cmp_cache", "v_cmp_cache")}
    ws = nsa.workspace_size(cfg, _lib.NSA_OP_APPEND)
    for partial in ({"k_slc_new": 4096}, {"k_slc_new": 4096, "v_slc_new": 4096, "k_slc_cache": 4096},
                    {"v_win_cache": 4096}, {"k_win_new": 4096, "v_win_new": 4096, "k_win_cache": 4096}):
        a = A(cmp_cache_cap=64, **base, **partial)
        st = lib.nsa_decode_append(ctypes.byref(p), ctypes.byref(a), ctypes.c_void_p(4096), ws, None)
        assert st == _lib.NSA_ERR_INVALID_ARG, partial

