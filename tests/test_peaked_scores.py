"""CPU checks of the peaked-score inputs used by the GPU parity tests.

The importance scores NSA selects on are the compressed branch's softmax
probabilities, remapped to selection blocks and summed over a GQA group's heads
(youleyou NSA page, 重要性分数计算 and Top-n块选择).  Selection is meant for rows
on which a few blocks dominate.  The workload recipe (random-init phi weights at
std 0.02, independent query heads) gives nearly flat rows, so the parity tests
add recipes in which the heads of a group share a query component and the
softmax scale is a multiple of 1/sqrt(d_k):

* peaked:  softmax scale 8/sqrt(d_k), head correlation 0.9  (about 60 nats of
  logit range)
* steep:   scale 16/sqrt(d_k), head correlation 0.95 (about 130 nats)
* extreme: scale 24/sqrt(d_k), head correlation 0.95, block offsets of std 1
  (about 200 nats)
(phi weights at std 0.05 in all three, so compressed keys and values stay
near 1 in magnitude).

These tests check, without a GPU, that the recipes really reach that regime,
and that the steep rows tell a score path of full fp32 range apart from one
that loses small probabilities: scaled by 2^14 and rounded to fp16, the
scores of blocks far below the row maximum become subnormal or zero and the
top-n then ranks them by index on rows that are not near ties.
"""
import numpy as np
import pytest
import torch

import nsa_inputs as NI
import oracle as O
from tests.nsa_testutil import PEAKED, oracle_params


def _group_rows(w, rows, seed=0):
    """Per (row, KV head): compressed logits [G, N] and head probabilities."""
    inp = NI.make_prefill_inputs(w, seed)
    a = NI.to_numpy64(inp)
    p = oracle_params(w)
    kc = O.compress(a["k"], a["phi_k"], p)
    vc = O.compress(a["v"], a["phi_v"], p)
    sc = p.scale
    out = []
    for t in rows:
        nv = O.n_cmp_visible(t, w.l, w.d)
        for g in range(w.H_kv):
            qh = a["q"][0, t, g * w.G:(g + 1) * w.G]
            z = sc * qh @ kc[0, :nv, g].T
            _, _, P = O.attend(qh, kc[0, :nv, g], vc[0, :nv, g], sc)
            out.append((t, z, P))
    return p, out


def _scores(P, t, p):
    W = O.remap_matrix(P.shape[1], t // p.l_sel + 1, p)
    return (P @ W).sum(axis=0)


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()


ROWS = list(range(1100, 2048, 61))


@pytest.mark.parametrize("name,min_range", [("peaked", 30.0), ("steep", 80.0), ("extreme", 120.0)])
def test_peaked_recipes_span_wide_logit_ranges(name, min_range):
    w = NI.workload("prefill_8k", T=2048, H_kv=2, **PEAKED[name])
    p, rows = _group_rows(w, ROWS)
    ranges = [float(np.mean(z.max(axis=1) - z.min(axis=1))) for _, z, _ in rows]
    assert np.mean(ranges) >= min_range, ranges
    # every head's probabilities still sum to one, and the remapped group row to
    # G * l / d, at these ranges
    for t, _, P in rows:
        np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=1e-12)
        np.testing.assert_allclose(_scores(P, t, p).sum(), w.G * w.l / w.d, rtol=1e-12)


def test_steep_rows_separate_full_range_scores_from_fp16():
    w = NI.workload("prefill_8k", T=2048, H_kv=2, **PEAKED["steep"])
    p, rows = _group_rows(w, ROWS)
    fp16_wrong = split_wrong = decided = 0
    for t, _, P in rows:
        ref = _scores(P, t, p)
        if O.is_near_tie(ref, t, p):
            continue
        decided += 1
        want = O.top_n(ref, t, p)
        # probabilities scaled by 2^14 and rounded to fp16 before the remap
        p16 = (P * 2.0 ** 14).astype(np.float16).astype(np.float64) / 2.0 ** 14
        fp16_wrong += O.top_n(_scores(p16, t, p), t, p) != want
        # probabilities as a bf16 hi + lo pair (fp32's exponent range)
        P32 = P.astype(np.float32).astype(np.float64)
        hi = _bf16(P32)
        lo = _bf16(P32 - hi)
        split_wrong += O.top_n(_scores(hi + lo, t, p), t, p) != want
    assert decided >= len(rows) // 2
    assert fp16_wrong > 0, "the steep recipe no longer reaches scores fp16 cannot hold"
    assert split_wrong == 0
