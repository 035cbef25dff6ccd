"""Helpers shared by the GPU parity tests: move seeded inputs to the GPU and
run the oracle on the same values."""
import numpy as np
import torch

import nsa_inputs as NI

ATOL, RTOL = 2e-2, 1e-2   # |gpu - oracle| <= ATOL + RTOL * |oracle|


def oracle_params(w):
    import oracle as O
    return O.Params(l=w.l, d=w.d, l_sel=w.l_sel, n=w.n, w=w.w, phi=w.phi,
                    io="bf16" if w.dtype == "bf16" else "fp32",
                    scale=None if w.scale_mult == 1.0 else w.scale_mult / np.sqrt(w.d_k))


def to_dev(d, dev="cuda:0"):
    if isinstance(d, dict):
        return {k: to_dev(v, dev) for k, v in d.items()}
    return d.to(dev)


def np64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def assert_close(gpu, ref, name, atol=ATOL, rtol=RTOL):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    both_inf = np.isinf(gpu) & np.isinf(ref) & (np.sign(gpu) == np.sign(ref))
    err = np.where(both_inf, 0.0, np.abs(gpu - ref))
    bad = ~(err <= atol + rtol * np.abs(np.where(both_inf, 0.0, ref)))
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{name}: {bad.sum()} of {bad.size} elements out of tolerance; first at "
                             f"{tuple(i)}: gpu={gpu[tuple(i)]} oracle={ref[tuple(i)]} max err={err.max():.3e}")
    return float(err.max()) if err.size else 0.0


class SampledRows:
    """Stand-in for a [B, T, ...] array of which only some positions are held
    (rows R, data [B, R, ...]); indexing [b, t] returns position t's data.
    Lets the oracle evaluate sampled rows of a full-size sequence without the
    whole query tensor in float64."""

    def __init__(self, data, rows, T):
        self.data = np.asarray(data)
        self.pos = {int(t): i for i, t in enumerate(rows)}
        self.shape = (self.data.shape[0], T) + tuple(self.data.shape[2:])

    def __getitem__(self, idx):
        b, t = idx
        return self.data[b, self.pos[int(t)]]


# Input recipes whose compressed-branch scores are peaked: the G query heads of
# a KV group share a component (so they favour the same blocks), phi's weights
# are somewhat larger than the workloads' 0.02 and the softmax scale is a
# multiple of 1/sqrt(d_k), so the logits spread over tens to hundreds of nats
# while keys, values and compressed keys keep magnitudes near 1.  The scale
# multiplies all three branches' logits, so the selected and window softmaxes
# are peaked too.  "extreme" also offsets every selection block's keys and
# values (std 1).
PEAKED = {
    "peaked": dict(phi_std=0.05, q_group_corr=0.9, scale_mult=8.0, bias_std=0.02),
    "steep": dict(phi_std=0.05, q_group_corr=0.95, scale_mult=16.0, bias_std=0.02),
    "extreme": dict(phi_std=0.05, q_group_corr=0.95, scale_mult=24.0, bias_std=0.02, kv_offset_std=1.0),
}
