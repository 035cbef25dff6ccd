"""CPU test of the rule by which the kernels read a selected-block row.

The backward takes the forward's selected-block indices back from the caller,
and the reverse index (a per-block histogram, then an ordered fill of query
positions) uses each entry to address memory.  Every kernel that reads a row
therefore reads it only while each entry is non-negative, above the previous
one and causal (first token j*l' <= t).  A stale or foreign buffer can then
never address past the block count or give dq and dK/dV different entries.

The predicate is the kernels' own (nsa_common.hpp, compiled host-only); the
expected prefix lengths come from the rule written out here.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_sparse_phi_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

PROGRAM = r"""
#include "nsa_common.hpp"
#include <cstdio>
int main() {
  int n, t, ls;
  while (std::scanf("%d %d %d", &n, &t, &ls) == 3) {
    int ids[64];
    for (int i = 0; i < n; ++i) std::scanf("%d", &ids[i]);
    int prev = -1, k = 0;
    for (; k < n && nsa::sel_slot_ok(ids[k], prev, t, ls); ++k) prev = ids[k];
    std::printf("%d\n", k);
  }
  return 0;
}
"""


def expected_len(row, t, ls):
    prev = -1
    for k, j in enumerate(row):
        if not (j > prev and 0 <= j and j * ls <= t):
            return k
        prev = j
    return len(row)


@pytest.fixture(scope="module")
def rule_binary(tmp_path_factory):
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("selrule")
    src, exe = d / "rule.cpp", d / "rule"
    src.write_text(PROGRAM)
    subprocess.run([HIPCC, "-x", "hip", "--offload-host-only", "-O1", "-std=c++17", "-I", CSRC,
                    "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True,
                   capture_output=True)
    return str(exe)


def test_row_prefix_rule(rule_binary):
    rng = np.random.default_rng(7)
    cases = [
        ([0, 1, 2, 3], 200, 64),            # a valid row
        ([0, 2, 2, 3], 200, 64),            # repeated entry: stop before it
        ([0, 3, 1, 2], 300, 64),            # descending entry
        ([0, 1, 5, -1], 70, 64),            # block 5 starts after t
        ([-1, 0, 1], 10, 64),               # padding first
        ([0, 1, -1, 2], 500, 64),           # entries after padding are never read
        ([0, 10**6, 10**6 + 1], 10**5, 16),  # far past the block count
        ([-7, -3, 0], 50, 16),
        (list(range(32)), 32 * 64 - 1, 64),  # a full row of 32 causal blocks
        (list(range(32)), 31 * 64 - 1, 64),  # its last block starts after t
    ]
    for _ in range(300):
        n = int(rng.integers(1, 33))
        ls = int(rng.choice([16, 32, 64, 128]))
        t = int(rng.integers(0, 5000))
        row = np.sort(rng.integers(-2, t // ls + 3, size=n))
        if rng.random() < 0.3:
            row = rng.integers(-5, t // ls + 3, size=n)
        cases.append((row.tolist(), t, ls))
    text = "".join(f"{len(r)} {t} {ls}\n{' '.join(map(str, r))}\n" for r, t, ls in cases)
    out = subprocess.run([rule_binary], input=text, capture_output=True, text=True, check=True).stdout.split()
    got = [int(x) for x in out]
    want = [expected_len(r, t, ls) for r, t, ls in cases]
    assert got == want
    # the usable prefix never addresses a block past t, so never past the block count
    for (r, t, ls), k in zip(cases, got):
        assert all(0 <= j <= t // ls for j in r[:k])
