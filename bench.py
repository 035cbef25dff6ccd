"""Benchmark of the NSA hot path on one MI355X.

A step is one NSA prefill forward (gates, compression, compressed attention
with scores and top-n, selected attention, window attention and the gated
combine) over the 64K-token workload (B=1, T=65536, 4 KV x 16 query heads,
d_k=192, d_v=128, bf16), inputs resident in HBM.  The JSON line reports
tokens/s for that step, the per-stage times measured with HIP events on the
launch stream inside the timed region, and the roofline of the dominant
kernel.  Two further legs are measured the same way: one decode step of 32
sequences over a 64K cache (HBM GB/s, caches cold), and the backward pass of
the 16K training shape (MFMA fraction).  The fp64 CPU oracle is timed on a
bounded sample of the prefill workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NSA prefill fwd tokens/s at 64K (MFMA % peak); decode HBM GB/s at 64K KV"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E

PREFILL_STAGES = [
    ("gates", "k_gate"), ("compress_k", "k_phi_gemm1"), ("compress_v", "k_phi_gemm1"),
    ("transpose_v", "k_transpose_seq"), ("cmp_lse", "k_cmp_lse"), ("cmp_out_topn", "k_cmp_out"),
    ("selected", "k_slc"), ("window_combine", "k_win"),
]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------- work model

def key_counts(w):
    """Per-position key counts of the three branches (numpy int64 arrays)."""
    import numpy as np
    t = np.arange(w.T, dtype=np.int64)
    s = t + 1
    n_cmp = np.where(s < w.l, 0, (s - w.l) // w.d + 1)
    all_blocks = (t // w.l_sel + 1) <= w.n
    n_slc = np.where(all_blocks, s, (w.n - 1) * w.l_sel + (t % w.l_sel) + 1)
    n_win = np.minimum(s, w.w)
    return n_cmp, n_slc, n_win


def useful_flops(w):
    """Algorithmic FLOPs of the prefill forward (2 per multiply-add, unmasked
    query-key pairs only; the log-sum-exp recompute is not counted)."""
    n_cmp, n_slc, n_win = key_counts(w)
    per_pair = 2 * (w.d_k + w.d_v) * w.B * w.H_q
    ncmp_tot = 0 if w.T < w.l else (w.T - w.l) // w.d + 1
    phi = 0
    if w.phi == "mlp":
        phi = 2 * w.B * w.H_kv * ncmp_tot * (w.l * w.d_k * w.hidden + w.hidden * w.d_k +
                                             w.l * w.d_v * w.hidden + w.hidden * w.d_v)
    gate = 2 * w.B * w.T * w.gate_dim * 3 * w.H_q
    return {"cmp": per_pair * int(n_cmp.sum()), "slc": per_pair * int(n_slc.sum()),
            "win": per_pair * int(n_win.sum()), "phi": phi, "gate": gate,
            "cmp_lse": 2 * w.d_k * w.B * w.H_q * int(n_cmp.sum())}


# ---------------------------------------------------------------- HIP events

class HipEvents:
    def __init__(self, lib):
        self.lib = lib
        lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        lib.hipEventCreate.restype = ctypes.c_int
        lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        lib.hipEventElapsedTime.restype = ctypes.c_int
        lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        lib.hipEventRecord.restype = ctypes.c_int

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.lib.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        return out

    def record(self, e, stream):
        if self.lib.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


_CSRC = "long_context_sparse_phi_amd/csrc/"
_HDRS = [_CSRC + h for h in ("nsa_common.hpp", "nsa_kernels.hpp", "nsa_tiles.hpp")]
# kernels whose HBM traffic is reported: name pattern in the profiler's kernel
# names, and the sources their code comes from
TRAFFIC_KERNELS = {
    "k_slc": (r"k_slcI", [_CSRC + "nsa_attn.hip"] + _HDRS),
    "k_dec_cmp": (r"k_dec_cmpI", [_CSRC + "nsa_decode.hip"] + _HDRS),
    "k_cmp_out": (r"k_cmpI.*Lb1E", [_CSRC + "nsa_cmp.hip"] + _HDRS),
    "k_cmp_lse": (r"k_cmpI.*Lb0E", [_CSRC + "nsa_cmp.hip"] + _HDRS),
    "k_win": (r"k_winI", [_CSRC + "nsa_attn.hip"] + _HDRS),
}
COPY_BYTES = 1 << 30     # calibration: read 1 GiB, write 1 GiB


def traffic_for(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 PMC summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a copy kernel of known size), when it
    was taken from the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path) or kernel not in TRAFFIC_KERNELS:
        return None
    with open(path) as f:
        rec = json.load(f).get("kernels", {}).get(kernel)
    if not rec or rec.get("source_sha") != source_hash(TRAFFIC_KERNELS[kernel][1]):
        return None
    return rec.get("hbm_bytes_per_launch")


def calibrate_copy():
    """A plain elementwise kernel that reads and writes COPY_BYTES (the PMC
    calibration: its FETCH_SIZE / WRITE_SIZE give the counters' byte scale)."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 2.0, out=dst)
    torch.cuda.synchronize()
    log("copy calibration done")


def _pmc_per_kernel(csv_path, counter):
    """Median value of `counter` per dispatch, keyed by kernel name."""
    import csv
    import statistics
    vals = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: statistics.median(v) for k, v in vals.items()}


def write_traffic(cal_fetch, cal_write, run_fetch, run_write, out_path, command):
    """profiles/traffic.json from four rocprofv3 --pmc runs (FETCH_SIZE and
    WRITE_SIZE of the copy calibration and of the benchmark)."""
    import re
    cf, cw = _pmc_per_kernel(cal_fetch, "FETCH_SIZE"), _pmc_per_kernel(cal_write, "WRITE_SIZE")
    kf = max(cf, key=cf.get)                     # the 1 GiB elementwise kernel
    f_fetch = COPY_BYTES / (cf[kf] * 1024.0)
    f_write = COPY_BYTES / (cw[kf] * 1024.0)
    rf, rw = _pmc_per_kernel(run_fetch, "FETCH_SIZE"), _pmc_per_kernel(run_write, "WRITE_SIZE")
    kernels = {}
    for name, (pat, srcs) in TRAFFIC_KERNELS.items():
        hits = [k for k in rf if re.search(pat, k)]
        if not hits:
            continue
        k = max(hits, key=lambda x: rf[x])
        fetch = rf[k] * 1024.0 * f_fetch
        write = rw.get(k, 0.0) * 1024.0 * f_write
        kernels[name] = {"kernel_name": k, "fetch_kib_per_dispatch": rf[k], "write_kib_per_dispatch": rw.get(k),
                         "hbm_read_bytes": round(fetch), "hbm_write_bytes": round(write),
                         "hbm_bytes_per_launch": round(fetch + write), "source_sha": source_hash(srcs)}
    rec = {"command": command, "calibration": {"kernel_name": kf, "bytes_each_way": COPY_BYTES,
                                               "fetch_kib": cf[kf], "write_kib": cw[kf],
                                               "fetch_scale": f_fetch, "write_scale": f_write},
           "kernels": kernels}
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


# ---------------------------------------------------------------- prefill leg

def run_prefill(steps, warmup, wname="prefill_64k", calibrate=False):
    """Times `steps` calls of the plain entry point (wall clock, and a HIP
    event pair around each call), then `steps` calls of the timed entry
    point for the per-stage split (its events between stages are
    instrumentation, so they stay out of the step time).  With calibrate,
    three further calls carry one more event, behind which the library runs
    the selected branch's gather alone: the walk of k_slc over the same index
    rows and tiles without its arithmetic.  Returns (workload, wall s, stage
    ms, GPU ms, calibration)."""
    import torch
    import long_context_sparse_phi_amd as nsa
    from long_context_sparse_phi_amd import _lib
    import nsa_inputs as NI

    w = NI.workload(wname)
    cfg = nsa.config_from_workload(w)
    log(f"generating inputs for {wname}")
    inp = NI.make_prefill_inputs(w, 0)
    dev = torch.device("cuda:0")
    d = {k: ({kk: vv.to(dev) for kk, vv in v.items()} if isinstance(v, dict) else v.to(dev))
         for k, v in inp.items()}
    del inp
    o = torch.empty(w.B, w.T, w.H_q, w.d_v, dtype=cfg.torch_dtype, device=dev)
    ws = torch.empty(nsa.workspace_size(cfg, _lib.NSA_OP_FWD_PREFILL), dtype=torch.uint8, device=dev)
    lib = _lib.load()
    lib.nsa_fwd_prefill_timed.restype = ctypes.c_int
    lib.nsa_fwd_prefill_timed.argtypes = [ctypes.POINTER(_lib.nsa_params), ctypes.POINTER(_lib.nsa_prefill_args),
                                          ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                          ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]
    p = cfg.params()
    a = _lib.nsa_prefill_args()
    for name in ("q", "k", "v", "x", "w_gate"):
        setattr(a, name, d[name].data_ptr())
    a.phi_k = nsa._phi_struct(cfg, d["phi_k"], w.d_k, dev)
    a.phi_v = nsa._phi_struct(cfg, d["phi_v"], w.d_v, dev)
    a.o = o.data_ptr()
    stream = torch.cuda.current_stream(dev).cuda_stream
    nst = len(PREFILL_STAGES)
    ev = HipEvents(lib)
    events = [ev.create(nst + 1) for _ in range(steps)]

    def step(evs=None):
        if evs is None:
            st = lib.nsa_fwd_prefill(ctypes.byref(p), ctypes.byref(a), ws.data_ptr(), ws.numel(), stream)
        else:
            arr = (ctypes.c_void_p * len(evs))(*evs)
            st = lib.nsa_fwd_prefill_timed(ctypes.byref(p), ctypes.byref(a), ws.data_ptr(), ws.numel(), stream,
                                           arr, len(evs))
        if st != 0:
            raise RuntimeError(f"nsa_fwd_prefill failed: {_lib.status_str(st)}")

    log(f"prefill warmup {warmup}")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    log(f"prefill timed {steps}")
    pair = [ev.create(2) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev.record(pair[i][0], stream)
        step()
        ev.record(pair[i][1], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = sum(ev.elapsed_ms(e0, e1) for e0, e1 in pair) / steps
    log(f"prefill stage split {steps}")
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    stage_ms = [sum(ev.elapsed_ms(events[i][s], events[i][s + 1]) for i in range(steps)) / steps
                for s in range(nst)]
    cal = None
    if calibrate:
        ncal = 3
        cev = [ev.create(nst + 2) for _ in range(ncal)]
        for i in range(ncal):
            step(cev[i])
        torch.cuda.synchronize()
        isel = [n for n, _ in PREFILL_STAGES].index("selected")
        cal = {"selected_ms": sum(ev.elapsed_ms(e[isel], e[isel + 1]) for e in cev) / ncal,
               "gather_only_ms": sum(ev.elapsed_ms(e[nst], e[nst + 1]) for e in cev) / ncal}
    return w, wall, stage_ms, gpu_ms, cal


def prefill_roofline(w, stage_ms):
    fl = useful_flops(w)
    work = {"gates": fl["gate"], "compress_k": fl["phi"] * w.d_k / (w.d_k + w.d_v),
            "compress_v": fl["phi"] * w.d_v / (w.d_k + w.d_v), "transpose_v": 0, "cmp_lse": fl["cmp_lse"],
            "cmp_out_topn": fl["cmp"], "selected": fl["slc"], "window_combine": fl["win"]}
    i = max(range(len(stage_ms)), key=lambda s: stage_ms[s])
    name, kern = PREFILL_STAGES[i]
    achieved = work[name] / (stage_ms[i] * 1e-3) / 1e12
    return {"kernel": kern, "stage": name, "bound": "mfma", "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic_for(kern),
            "launch_ms": round(stage_ms[i], 4), "algorithmic_flops_per_launch": work[name]}


def prefill_leg(steps, warmup, wname):
    """Another prefill workload measured like the headline one (tokens/s from
    the wall clock, stage times from HIP events) with its MFMA fraction on
    useful FLOPs and the time 50 % of the bf16 peak would take."""
    w, wall, stage_ms, gpu_ms, _ = run_prefill(steps, warmup, wname)
    ms = wall * 1e3 / steps
    fl = useful_flops(w)
    useful = fl["cmp"] + fl["slc"] + fl["win"] + fl["phi"] + fl["gate"]
    return {"workload": wname, "B": w.B, "T": w.T, "H_kv": w.H_kv, "G": w.G, "d_k": w.d_k, "d_v": w.d_v,
            "steps": steps, "ms_per_step": round(ms, 4), "tokens_per_s": round(w.B * w.T / (ms * 1e-3), 1),
            "gpu_ms_per_step": round(gpu_ms, 4), "useful_tflop_per_step": round(useful / 1e12, 4),
            "mfma_frac_useful": round(useful / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "ms_at_half_peak": round(useful / (0.5 * PEAK_BF16_TFLOPS * 1e12) * 1e3, 4),
            "stages_ms": {name: round(x, 4) for (name, _), x in zip(PREFILL_STAGES, stage_ms)},
            "roofline": prefill_roofline(w, stage_ms)}


def selected_gather(w, stage_ms, cal=None):
    """The selected branch as a gather: K/V bytes of every (position, KV head)'s
    selected tokens (16 FLOP/B at G = 16, served mostly by L2 and MALL), per
    second of the selected-attention stage.  With the calibration of
    run_prefill, the same bytes per second of the gather alone (k_slc's walk
    over the same tiles without its arithmetic) are the ceiling this access
    stream reaches on the device, and frac is k_slc's rate against it."""
    _, n_slc, _ = key_counts(w)
    nbytes = int(n_slc.sum()) * w.B * w.H_kv * (w.d_k + w.d_v) * 2
    i = [n for n, _ in PREFILL_STAGES].index("selected")
    out = {"kernel": "k_slc", "block_fetch_bytes": nbytes,
           "TB_per_s": round(nbytes / (stage_ms[i] * 1e-3) / 1e12, 2)}
    if cal:
        ceil = nbytes / (cal["gather_only_ms"] * 1e-3) / 1e12
        rate = nbytes / (cal["selected_ms"] * 1e-3) / 1e12
        out["gather_ceiling"] = {"kernel": "k_slc_gather", "gather_only_ms": round(cal["gather_only_ms"], 4),
                                 "selected_ms": round(cal["selected_ms"], 4), "ceiling_TB_per_s": round(ceil, 2),
                                 "k_slc_TB_per_s": round(rate, 2), "frac": round(rate / ceil, 4)}
    return out


# ---------------------------------------------------------------- decode leg

DECODE_STAGES = [("cmp_partials", "k_dec_cmp"), ("combine_topn", "k_dec_combine"),
                 ("sel_win_merge", "k_dec_sw")]


def decode_bytes(w, idx):
    """Algorithmic HBM bytes of one decode step: the compressed cache, the union
    of selected-block and window tokens of every (sequence, KV head), q, o, x, W_g."""
    import numpy as np
    S = w.T
    t = S - 1
    ncmp = 0 if S < w.l else (S - w.l) // w.d + 1
    row = (w.d_k + w.d_v) * 2
    total = w.B * w.H_kv * ncmp * row
    win = set(range(max(0, t - w.w + 1), t + 1))
    for b in range(w.B):
        for g in range(w.H_kv):
            u = set(win)
            for j in idx[b, g]:
                if j >= 0:
                    u.update(range(j * w.l_sel, min((j + 1) * w.l_sel, S)))
            total += len(u) * row
    total += w.B * w.H_q * (w.d_k + w.d_v) * 2 + w.B * w.gate_dim * 2 + w.gate_dim * w.H_q * 3 * 2
    return int(total)


def run_decode(steps, warmup, wname="decode_64k"):
    import numpy as np
    import torch
    import long_context_sparse_phi_amd as nsa
    from long_context_sparse_phi_amd import _lib
    import nsa_inputs as NI

    w = NI.workload(wname)
    cfg = nsa.config_from_workload(w)
    log(f"generating inputs for {wname}")
    inp = NI.make_decode_inputs(w, 0)
    dev = torch.device("cuda:0")
    d = {k: ({kk: vv.to(dev) for kk, vv in v.items()} if isinstance(v, dict) else v.to(dev))
         for k, v in inp.items()}
    del inp
    # compressed caches: phi over the raw caches (cache maintenance, untimed)
    kc = nsa.nsa_compress(cfg, d["k_cache"], d["phi_k"], False)
    vc = nsa.nsa_compress(cfg, d["v_cache"], d["phi_v"], True)
    dbg = nsa.nsa_fwd_decode(cfg, d["q"], d["k_cache"], d["v_cache"], kc, vc, d["x"], d["w_gate"], debug=True)
    torch.cuda.synchronize()
    idx = dbg["idx"].cpu().numpy()
    del dbg
    o = torch.empty(w.B, w.H_q, w.d_v, dtype=cfg.torch_dtype, device=dev)
    ws = torch.empty(nsa.workspace_size(cfg, _lib.NSA_OP_FWD_DECODE), dtype=torch.uint8, device=dev)
    # Cold caches before every step: a 512 MB buffer is written (evicting L2 and
    # the 256 MB MALL) and then read, so the write-backs of its dirty lines
    # happen here and not inside the timed step.
    flush = torch.empty(128 << 20, dtype=torch.float32, device=dev)
    lib = _lib.load()
    lib.nsa_fwd_decode_timed.restype = ctypes.c_int
    lib.nsa_fwd_decode_timed.argtypes = [ctypes.POINTER(_lib.nsa_params), ctypes.POINTER(_lib.nsa_decode_args),
                                         ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                         ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]
    p = cfg.params()
    a = _lib.nsa_decode_args()
    for name in ("q", "k_cache", "v_cache", "x", "w_gate"):
        setattr(a, name, d[name].data_ptr())
    a.k_cmp_cache, a.v_cmp_cache, a.cmp_cache_cap = kc.data_ptr(), vc.data_ptr(), kc.shape[1]
    a.o = o.data_ptr()
    stream = torch.cuda.current_stream(dev).cuda_stream
    nst = len(DECODE_STAGES)
    ev = HipEvents(lib)
    events = [ev.create(nst + 1) for _ in range(steps)]

    def step(evs=None, flush_first=True):
        if flush_first:
            flush.fill_(1.0)
            flush.sum()
        if evs is None:
            st = lib.nsa_fwd_decode(ctypes.byref(p), ctypes.byref(a), ws.data_ptr(), ws.numel(), stream)
        else:
            arr = (ctypes.c_void_p * len(evs))(*evs)
            st = lib.nsa_fwd_decode_timed(ctypes.byref(p), ctypes.byref(a), ws.data_ptr(), ws.numel(), stream,
                                          arr, len(evs))
        if st != 0:
            raise RuntimeError(f"nsa_fwd_decode failed: {_lib.status_str(st)}")

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # the step time: an event pair around each call of the plain entry point
    # (after the cache flush); the stage split: further calls of the timed
    # entry point, whose events between stages add a few microseconds each
    log(f"decode timed {steps}")
    pair = [ev.create(2) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        flush.fill_(1.0)
        flush.sum()
        ev.record(pair[i][0], stream)
        step(flush_first=False)
        ev.record(pair[i][1], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = sum(ev.elapsed_ms(e0, e1) for e0, e1 in pair) / steps
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    stage_ms = [sum(ev.elapsed_ms(events[i][s], events[i][s + 1]) for i in range(steps)) / steps
                for s in range(nst)]
    staged_ms = sum(ev.elapsed_ms(events[i][0], events[i][nst]) for i in range(steps)) / steps
    append = run_append(w, cfg, d, kc, vc)
    nbytes = decode_bytes(w, idx)
    ncmp = (w.T - w.l) // w.d + 1
    cmp_bytes = w.B * w.H_kv * ncmp * (w.d_k + w.d_v) * 2 + w.B * w.H_q * w.d_k * 2
    gbs = cmp_bytes / (stage_ms[0] * 1e-3) / 1e9
    return {
        "workload": wname, "B": w.B, "cache_len": w.T, "steps": steps, "warmup": warmup,
        "us_per_step": round(step_ms * 1e3, 2), "wall_ms_incl_cache_flush": round(wall * 1e3 / steps, 3),
        "algorithmic_bytes": nbytes, "GB_per_s": round(nbytes / (step_ms * 1e-3) / 1e9, 1),
        "frac_hbm_peak": round(nbytes / (step_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "stages_us": {n: round(ms * 1e3, 2) for (n, _), ms in zip(DECODE_STAGES, stage_ms)},
        "staged_call_us": round(staged_ms * 1e3, 2),
        "roofline": {"kernel": "k_dec_cmp", "stage": "cmp_partials", "bound": "hbm", "achieved": round(gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic_for("k_dec_cmp"),
                     "algorithmic_bytes_per_launch": cmp_bytes, "launch_us": round(stage_ms[0] * 1e3, 2)},
        "cold_cache": "512 MB buffer written then read before every step (outside the timed events)",
        "append": append,
    }


def run_append(w, cfg, d, kc, vc, reps=3):
    """Decode-time cache maintenance: one nsa_decode_append per step appends a
    token to every sequence; over d = 16 consecutive steps exactly one (here the
    first) completes a compression block in every sequence and runs phi.  Each
    call is timed alone with HIP events; the lengths are set so the appended
    rows rewrite the cache's own last rows (the caches keep their contents)."""
    import torch
    from long_context_sparse_phi_amd import _lib
    dev = torch.device("cuda:0")
    lib = _lib.load()
    p = cfg.params()
    lens = torch.empty(w.B, dtype=torch.int32, device=dev)
    start = w.T - 1 - w.d
    kn = [d["k_cache"][:, start + i].contiguous() for i in range(w.d)]
    vn = [d["v_cache"][:, start + i].contiguous() for i in range(w.d)]
    a = _lib.nsa_append_args()
    a.seq_lens = lens.data_ptr()
    a.k_cache, a.v_cache = d["k_cache"].data_ptr(), d["v_cache"].data_ptr()
    a.k_cmp_cache, a.v_cmp_cache, a.cmp_cache_cap = kc.data_ptr(), vc.data_ptr(), kc.shape[1]
    for name, ph in (("phi_k", d["phi_k"]), ("phi_v", d["phi_v"])):
        st = getattr(a, name)
        for f in ("pe", "w1", "b1", "w2", "b2"):
            if f in ph:
                setattr(st, f, ph[f].data_ptr())
    ws = torch.empty(max(256, nsa_ws(cfg, _lib.NSA_OP_APPEND)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    times = [[] for _ in range(w.d)]
    for r in range(reps + 1):
        lens.fill_(start)
        for i in range(w.d):
            a.k_new, a.v_new = kn[i].data_ptr(), vn[i].data_ptr()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            st = lib.nsa_decode_append(ctypes.byref(p), ctypes.byref(a), ws.data_ptr(), ws.numel(), stream)
            e1.record()
            if st != 0:
                raise RuntimeError(f"nsa_decode_append failed: {_lib.status_str(st)}")
            lens.add_(1)
            if r > 0:
                times[i].append((e0, e1))
    torch.cuda.synchronize()
    us = [sum(x.elapsed_time(y) for x, y in t) / len(t) * 1e3 for t in times]
    return {"calls_per_stride": w.d, "us_block_completing": round(us[0], 2),
            "us_other_mean": round(sum(us[1:]) / (len(us) - 1), 2),
            "us_mean_per_token": round(sum(us) / len(us), 2)}


def nsa_ws(cfg, op):
    import long_context_sparse_phi_amd as nsa
    return nsa.workspace_size(cfg, op)


# ---------------------------------------------------------------- backward leg

BWD_STAGES = ["gates", "transposes", "rowterms_dq", "cmp_dkdv", "win_dkdv", "slc_dkdv", "phi", "dw_gate"]


def run_backward(steps, warmup, wname="train_16k"):
    import torch
    import long_context_sparse_phi_amd as nsa
    from long_context_sparse_phi_amd import _lib
    import nsa_inputs as NI

    w = NI.workload(wname)
    cfg = nsa.config_from_workload(w)
    log(f"generating inputs for {wname}")
    inp = NI.make_prefill_inputs(w, 0)
    dev = torch.device("cuda:0")
    d = {k: ({kk: vv.to(dev) for kk, vv in v.items()} if isinstance(v, dict) else v.to(dev))
         for k, v in inp.items()}
    d_o = NI.make_grad_output(w, 0).to(dev)
    fwd = nsa.nsa_fwd_prefill(cfg, d["q"], d["k"], d["v"], d["x"], d["w_gate"], d["phi_k"], d["phi_v"],
                              save_for_backward=True)
    res = nsa.nsa_bwd(cfg, d["q"], d["k"], d["v"], d["x"], d["w_gate"], d["phi_k"], d["phi_v"], fwd, d_o)
    torch.cuda.synchronize()
    lib = _lib.load()
    lib.nsa_bwd_timed.restype = ctypes.c_int
    lib.nsa_bwd_timed.argtypes = [ctypes.POINTER(_lib.nsa_params), ctypes.POINTER(_lib.nsa_bwd_args),
                                  ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                  ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]
    p = cfg.params()
    a = _lib.nsa_bwd_args()
    for name in ("q", "k", "v", "x", "w_gate"):
        setattr(a, name, d[name].data_ptr())
    a.d_o = d_o.data_ptr()
    for name in ("k_cmp", "v_cmp", "lse", "idx", "o_branch"):
        setattr(a, name, fwd[name].data_ptr())
    a.phi_k = nsa._phi_struct(cfg, d["phi_k"], w.d_k, dev)
    a.phi_v = nsa._phi_struct(cfg, d["phi_v"], w.d_v, dev)
    for name in ("dq", "dk", "dv", "dw_gate"):
        setattr(a, name, res[name].data_ptr())
    a.d_phi_k = _lib.nsa_phi_grads(**{k: v.data_ptr() for k, v in res["d_phi_k"].items()})
    a.d_phi_v = _lib.nsa_phi_grads(**{k: v.data_ptr() for k, v in res["d_phi_v"].items()})
    ws = res["_workspace"]
    stream = torch.cuda.current_stream(dev).cuda_stream
    nst = len(BWD_STAGES)
    ev = HipEvents(lib)
    events = [ev.create(nst + 1) for _ in range(steps)]

    def step(evs=None):
        if evs is None:
            st = lib.nsa_bwd(ctypes.byref(p), ctypes.byref(a), ws.data_ptr(), ws.numel(), stream)
        else:
            arr = (ctypes.c_void_p * len(evs))(*evs)
            st = lib.nsa_bwd_timed(ctypes.byref(p), ctypes.byref(a), ws.data_ptr(), ws.numel(), stream, arr,
                                   len(evs))
        if st != 0:
            raise RuntimeError(f"nsa_bwd failed: {_lib.status_str(st)}")

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    log(f"backward timed {steps}")
    t0 = time.perf_counter()
    for i in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the stage split from further calls of the timed entry point
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    stage_ms = [sum(ev.elapsed_ms(events[i][s], events[i][s + 1]) for i in range(steps)) / steps
                for s in range(nst)]
    # the training-mode forward that saves the fp32 branch outputs (and with
    # them the softmax row terms) for this backward
    fwd_ms = []
    for _ in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        nsa.nsa_fwd_prefill(cfg, d["q"], d["k"], d["v"], d["x"], d["w_gate"], d["phi_k"], d["phi_v"],
                            save_for_backward=True, workspace=fwd["_workspace"])
        e1.record()
        fwd_ms.append((e0, e1))
    torch.cuda.synchronize()
    fwd_ms = sum(x.elapsed_time(y) for x, y in fwd_ms) / steps
    fl = useful_flops(w)
    useful = 2 * (fl["cmp"] + fl["slc"] + fl["win"]) + 2 * fl["phi"] + fl["gate"]
    ms = wall * 1e3 / steps
    return {"workload": wname, "B": w.B, "T": w.T, "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 4),
            "useful_tflop_per_step": round(useful / 1e12, 4),
            "tflops": round(useful / (ms * 1e-3) / 1e12, 2),
            "mfma_frac_useful": round(useful / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "stages_ms": {n: round(x, 4) for n, x in zip(BWD_STAGES, stage_ms)},
            "row_terms": "read from the forward's saved fp32 branch outputs",
            "training_forward_ms": round(fwd_ms, 4)}


# ---------------------------------------------------------------- projection layer

def run_layer(reps=5, wname="train_16k"):
    """The projection layer around the operator (q/k/v/o projections as the
    library's MFMA GEMMs, layer width C = gate_dim) at the training shape: layer forward and
    backward against the operator's own forward and backward on the same
    projected inputs, so that the difference is the projections' cost."""
    import torch
    import long_context_sparse_phi_amd as nsa
    import nsa_inputs as NI

    w = NI.workload(wname)
    cfg = nsa.config_from_workload(w)
    log(f"generating layer inputs for {wname}")
    d = {k: ({kk: vv.to("cuda:0") for kk, vv in v.items()} if isinstance(v, dict) else v.to("cuda:0"))
         for k, v in NI.make_layer_inputs(w, 0).items()}
    args = (cfg, d["h"], d["proj"], d["w_gate"], d["phi_k"], d["phi_v"])
    f = nsa.nsa_layer_fwd(*args)
    g = nsa.nsa_layer_bwd(*args, f, d["dy"])
    d_o = NI.make_grad_output(w, 0).to("cuda:0")
    op_args = (cfg, f["q"], f["k"], f["v"], d["h"], d["w_gate"], d["phi_k"], d["phi_v"])
    torch.cuda.synchronize()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ev = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            ev.append((e0, e1))
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in ev) / reps

    fws, bws = f["_workspace"], g["_workspace"]
    layer_f = timed(lambda: nsa.nsa_layer_fwd(*args, workspace=fws))
    layer_b = timed(lambda: nsa.nsa_layer_bwd(*args, f, d["dy"], workspace=bws))
    op_f = timed(lambda: nsa.nsa_fwd_prefill(*op_args, save_for_backward=True, workspace=fws))
    op_b = timed(lambda: nsa.nsa_bwd(*op_args, f, d_o, want_dx=True))
    ntok, C = w.B * w.T, w.gate_dim
    proj_fwd = 2.0 * ntok * C * (w.H_q * w.d_k + w.H_kv * (w.d_k + w.d_v) + w.H_q * w.d_v)
    pf, pb = max(layer_f - op_f, 1e-9), max(layer_b - op_b, 1e-9)
    return {"workload": wname, "C": C, "reps": reps,
            "layer_fwd_ms": round(layer_f, 4), "layer_bwd_ms": round(layer_b, 4),
            "operator_fwd_ms": round(op_f, 4), "operator_bwd_ms": round(op_b, 4),
            "projection_tflop_fwd": round(proj_fwd / 1e12, 4), "projection_tflop_bwd": round(2 * proj_fwd / 1e12, 4),
            "projection_fwd_tflops": round(proj_fwd / (pf * 1e-3) / 1e12, 1),
            "projection_bwd_tflops": round(2 * proj_fwd / (pb * 1e-3) / 1e12, 1)}


# ---------------------------------------------------------------- dense baseline

def run_dense_comparison(lengths=(8192, 16384, 32768, 65536), wname="prefill_64k", reps=2,
                         bwd_lengths=(8192, 16384, 32768, 65536)):
    """NSA prefill forward against dense causal attention on the same inputs
    (the comparison the pages' kernel-speed figures make), per sequence length:
    milliseconds of each (HIP events around the call, after one warmup) and the
    ratio."""
    import torch
    import long_context_sparse_phi_amd as nsa
    import nsa_inputs as NI

    w = NI.workload(wname)
    log(f"generating inputs for the dense comparison ({wname})")
    inp = NI.make_prefill_inputs(w, 0)
    dev = torch.device("cuda:0")
    full = {k: ({kk: vv.to(dev) for kk, vv in v.items()} if isinstance(v, dict) else v.to(dev))
            for k, v in inp.items()}
    del inp
    out = []
    for T in lengths:
        wt = w.replace(T=T)
        cfg = nsa.config_from_workload(wt)
        d = {k: (v if isinstance(v, dict) or k == "w_gate" else v[:, :T].contiguous()) for k, v in full.items()}

        def timed(fn):
            fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        ws_n = torch.empty(nsa.workspace_size(cfg, nsa.NSA_OP_FWD_PREFILL), dtype=torch.uint8, device=dev)
        o_n = torch.empty(1, T, wt.H_q, wt.d_v, dtype=cfg.torch_dtype, device=dev)
        t_nsa = timed(lambda: nsa.nsa_fwd_prefill(cfg, d["q"], d["k"], d["v"], d["x"], d["w_gate"], d["phi_k"],
                                                  d["phi_v"], out=o_n, workspace=ws_n))
        del ws_n
        ws_d = torch.empty(nsa.workspace_size(cfg, nsa.NSA_OP_DENSE), dtype=torch.uint8, device=dev)
        t_dense = timed(lambda: nsa.nsa_dense_fwd(cfg, d["q"], d["k"], d["v"], out=o_n, workspace=ws_d))
        del ws_d
        row = {"T": T, "nsa_ms": round(t_nsa, 3), "dense_ms": round(t_dense, 3),
               "speedup": round(t_dense / t_nsa, 2)}
        log(f"T={T}: forward NSA {t_nsa:.2f} ms, dense {t_dense:.2f} ms")
        if T in bwd_lengths:
            d_o = NI.make_grad_output(wt, 0).to(dev)
            saved = nsa.nsa_fwd_prefill(cfg, d["q"], d["k"], d["v"], d["x"], d["w_gate"], d["phi_k"], d["phi_v"],
                                        save_for_backward=True)
            ws_b = torch.empty(nsa.workspace_size(cfg, nsa.NSA_OP_BWD), dtype=torch.uint8, device=dev)
            t_nsa_b = timed(lambda: nsa.nsa_bwd(cfg, d["q"], d["k"], d["v"], d["x"], d["w_gate"], d["phi_k"],
                                                d["phi_v"], saved, d_o, workspace=ws_b))
            del ws_b, saved
            dfw = nsa.nsa_dense_fwd(cfg, d["q"], d["k"], d["v"], want_lse=True)
            ws_db = torch.empty(nsa.workspace_size(cfg, nsa.NSA_OP_DENSE_BWD), dtype=torch.uint8, device=dev)
            t_dense_b = timed(lambda: nsa.nsa_dense_bwd(cfg, d["q"], d["k"], d["v"], dfw["o"], dfw["lse"], d_o,
                                                        workspace=ws_db))
            del ws_db, dfw, d_o
            row.update({"nsa_bwd_ms": round(t_nsa_b, 3), "dense_bwd_ms": round(t_dense_b, 3),
                        "bwd_speedup": round(t_dense_b / t_nsa_b, 2)})
            log(f"T={T}: backward NSA {t_nsa_b:.2f} ms, dense {t_dense_b:.2f} ms")
        del d
        torch.cuda.empty_cache()
        out.append(row)
    return {"workload": wname, "passes": "forward; backward (NSA with the forward's saved tensors)",
            "per_length": out}


# ---------------------------------------------------------------- CPU oracle leg

class _SampledRows:
    """q holding only the sampled positions, indexed by absolute position."""

    def __init__(self, data, rows, T):
        self.data = data
        self.pos = {int(t): i for i, t in enumerate(rows)}
        self.shape = (data.shape[0], T) + tuple(data.shape[2:])

    def __getitem__(self, idx):
        b, t = idx
        return self.data[b, self.pos[int(t)]]


def cpu_baseline(wname="prefill_64k", nrows=1536):
    """fp64 oracle on a bounded sample of the workload: the compression of the
    whole sequence plus `nrows` query positions spread evenly over [0, T);
    tokens/s = T / (t_compress + t_rows * T / nrows)."""
    import numpy as np
    import torch
    import nsa_inputs as NI
    import oracle as O

    w = NI.workload(wname)
    cores = len(os.sched_getaffinity(0))
    torch.set_num_threads(cores)
    inp = NI.make_prefill_inputs(w, 0)
    rows = np.linspace(0, w.T - 1, nrows).astype(np.int64)
    a = {"q": inp["q"][:, rows].double().numpy(), "k": inp["k"].double().numpy(),
         "v": inp["v"].double().numpy(), "x": inp["x"].double().numpy(), "w_gate": inp["w_gate"].double().numpy(),
         "phi_k": NI.to_numpy64(inp["phi_k"]), "phi_v": NI.to_numpy64(inp["phi_v"])}
    del inp
    p = O.Params(l=w.l, d=w.d, l_sel=w.l_sel, n=w.n, w=w.w, phi=w.phi, io="bf16")
    t0 = time.perf_counter()
    kc = O.compress(a["k"], a["phi_k"], p)
    vc = O.compress(a["v"], a["phi_v"], p)
    t_cmp = time.perf_counter() - t0
    t0 = time.perf_counter()
    O.forward(p, _SampledRows(a["q"], rows, w.T), a["k"], a["v"], a["x"], a["w_gate"], a["phi_k"], a["phi_v"],
              rows=rows, kc=kc, vc=vc)
    t_rows = time.perf_counter() - t0
    est = t_cmp + t_rows * w.T / nrows
    return {"value": round(w.B * w.T / est, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{wname}: phi compression of all {kc.shape[1]} blocks ({t_cmp:.1f} s) + {nrows} query "
                      f"rows evenly spaced over [0,{w.T}) ({t_rows:.1f} s), scaled to {w.T} rows"}


def cpu_baseline_decode(wname="decode_64k", nseq=2, reps=10):
    """fp64 oracle decode step on `nseq` of the workload's sequences, averaged
    over `reps` repetitions (their compressed caches are built first by the
    oracle's compression and are not timed: the step takes them as an input);
    scaled to all B sequences."""
    import numpy as np
    import torch
    import nsa_inputs as NI
    import oracle as O

    w = NI.workload(wname)
    cores = len(os.sched_getaffinity(0))
    torch.set_num_threads(cores)
    inp = NI.make_decode_inputs(w.replace(B=nseq), 0)
    a = NI.to_numpy64(inp)
    del inp
    p = O.Params(l=w.l, d=w.d, l_sel=w.l_sel, n=w.n, w=w.w, phi=w.phi, io="bf16")
    kc = O.compress(a["k_cache"], a["phi_k"], p)
    vc = O.compress(a["v_cache"], a["phi_v"], p)
    t0 = time.perf_counter()
    for _ in range(reps):
        O.decode(p, a["q"], a["k_cache"], a["v_cache"], kc, vc, a["x"], a["w_gate"])
    t = (time.perf_counter() - t0) / reps
    us = t * 1e6 * w.B / nseq
    return {"value": round(us, 1), "unit": "us/step", "cores": cores, "kind": "oracle",
            "sample": f"{wname}: the decode step of {nseq} of the {w.B} sequences ({t:.2f} s, mean of {reps}), "
                      f"scaled to {w.B}; compressed caches built beforehand, untimed"}


def cpu_baseline_backward(wname="train_16k", nrows=384):
    """fp64 oracle backward on a bounded sample: phi's forward and backward
    over every compressed block, plus the per-row backward arithmetic (each
    branch's softmax and its gradients, what backward() does for every row) of
    `nrows` positions spread evenly over each sequence; tokens/s = B*T /
    (t_phi + t_rows * B*T / (B*nrows))."""
    import numpy as np
    import torch
    import nsa_inputs as NI
    import oracle as O

    w = NI.workload(wname)
    cores = len(os.sched_getaffinity(0))
    torch.set_num_threads(cores)
    inp = NI.make_prefill_inputs(w, 0)
    d_o = NI.make_grad_output(w, 0)
    rows = np.linspace(0, w.T - 1, nrows).astype(np.int64)
    q_rows = inp["q"][:, rows].double().numpy()
    k, v = inp["k"].double().numpy(), inp["v"].double().numpy()
    phi_k, phi_v = NI.to_numpy64(inp["phi_k"]), NI.to_numpy64(inp["phi_v"])
    x = inp["x"].double().numpy()
    wg = inp["w_gate"].double().numpy()
    d_o_rows = d_o[:, rows].double().numpy()
    del inp, d_o
    p = O.Params(l=w.l, d=w.d, l_sel=w.l_sel, n=w.n, w=w.w, phi=w.phi, io="bf16")
    t0 = time.perf_counter()
    kc = O.compress(k, phi_k, p)
    vc = O.compress(v, phi_v, p)
    from oracle import nsa_oracle as ON
    ON._phi_bwd(k, phi_k, np.ones_like(kc), p)
    ON._phi_bwd(v, phi_v, np.ones_like(vc), p)
    t_phi = time.perf_counter() - t0
    f = O.forward(p, _SampledRows(q_rows, rows, w.T), k, v, x, wg, phi_k, phi_v, rows=rows, kc=kc, vc=vc)
    t0 = time.perf_counter()
    O.dq_rows(p, q_rows, k, v, kc, vc, f["gates"], d_o_rows, f["idx"], rows)
    t_rows = time.perf_counter() - t0
    est = t_phi + t_rows * w.T / nrows
    return {"value": round(w.B * w.T / est, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{wname}: phi forward and backward over all {kc.shape[1]} blocks of {w.B} sequences "
                      f"({t_phi:.1f} s) + the per-row backward of {nrows} positions evenly spaced over each "
                      f"sequence ({t_rows:.1f} s), scaled to {w.T} rows"}


# ---------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="prefill_64k")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=20)
    ap.add_argument("--bwd-steps", type=int, default=5)
    ap.add_argument("--no-dense", action="store_true", help="skip the NSA-vs-dense comparison")
    ap.add_argument("--no-layer", action="store_true", help="skip the projection-layer leg")
    ap.add_argument("--no-prefill-8k", action="store_true", help="skip the 8K prefill leg")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run the 1 GiB elementwise kernel used to scale the PMC byte counters")
    ap.add_argument("--traffic-from", nargs=4, metavar=("CAL_FETCH", "CAL_WRITE", "RUN_FETCH", "RUN_WRITE"),
                    help="rocprofv3 counter CSVs; writes the traffic summary and exits (no GPU use)")
    ap.add_argument("--traffic-out", default=os.path.join(ROOT, "profiles", "traffic.json"))
    ap.add_argument("--traffic-command", default="")
    args = ap.parse_args()
    if args.traffic_from:
        write_traffic(*args.traffic_from, args.traffic_out, args.traffic_command)
        return
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this NSA build runs on exactly one GPU; multi-GPU runs are not supported",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    w, wall, stage_ms, gpu_ms, cal = run_prefill(args.steps, args.warmup, args.workload, calibrate=True)
    ms_per_step = wall * 1e3 / args.steps
    fl = useful_flops(w)
    useful = fl["cmp"] + fl["slc"] + fl["win"] + fl["phi"] + fl["gate"]
    out = {
        "metric": METRIC,
        "value": round(w.B * w.T / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "B": w.B, "T": w.T, "H_kv": w.H_kv, "G": w.G, "d_k": w.d_k,
                   "d_v": w.d_v, "l": w.l, "d": w.d, "l_sel": w.l_sel, "n": w.n, "w": w.w, "phi": w.phi},
        "gpu_ms_per_step": round(gpu_ms, 4),
        "useful_tflop_per_step": round(useful / 1e12, 4),
        "mfma_frac_useful": round(useful / (ms_per_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "stages_ms": {name: round(ms, 4) for (name, _), ms in zip(PREFILL_STAGES, stage_ms)},
        "roofline": prefill_roofline(w, stage_ms),
        "selected_gather": selected_gather(w, stage_ms, cal),
    }
    if not args.no_prefill_8k:
        out["prefill_8k"] = prefill_leg(args.steps, args.warmup, "prefill_8k")
    if not args.no_decode:
        out["decode"] = run_decode(args.decode_steps, 3)
    if not args.no_backward:
        out["backward"] = run_backward(args.bwd_steps, 2)
    if not args.no_layer:
        out["layer"] = run_layer()
    if not args.no_dense:
        out["dense_baseline"] = run_dense_comparison()
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on a sample")
        out["cpu_baseline"] = cpu_baseline(args.workload)
        if "decode" in out:
            log("timing the fp64 oracle's decode step on a sample")
            out["decode"]["cpu_baseline"] = cpu_baseline_decode()
        if "backward" in out:
            log("timing the fp64 oracle's backward on a sample")
            out["backward"]["cpu_baseline"] = cpu_baseline_backward()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
