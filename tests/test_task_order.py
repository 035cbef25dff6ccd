"""CPU test of the workgroup -> task mappings of the dK/dV kernels and the GEMM.

Every workgroup of a launch must receive a distinct task and every task a
workgroup, or a key group's gradient segment is computed twice and another
never.  The mappings are the kernels' own (nsa_common.hpp, compiled
host-only): xcd_map for the window keys' (unit, key group) tasks,
span_task_order for the compressed keys' (unit, key group, segment) tasks and
gemm_tile_order for the MFMA GEMM's output tiles.
Beyond the bijection, the test checks the order the mapping exists for: on
each XCD (workgroup id mod 8) one unit's tasks come in nondecreasing first
query position.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_sparse_phi_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

PROGRAM = r"""
#include "nsa_common.hpp"
#include <cstdio>
int main() {
  int kind, units, ngroup, nseg, span, seglen;
  while (std::scanf("%d %d %d %d %d %d", &kind, &units, &ngroup, &nseg, &span, &seglen) == 6) {
    if (kind == 3) {
      // segmented GEMM columns: units = segment count, ngroup = N, nseg and
      // span = the second and third segments' offsets, seglen = tile width
      const int off[3] = {0, nseg, span};
      const int nt = nsa::seg_tiles(units, off, ngroup, seglen);
      for (int t = 0; t < nt; ++t) {
        int s = -1, n0 = -1;
        nsa::seg_tile(t, units, off, ngroup, seglen, s, n0);
        std::printf("%d %d %d\n", s, n0, nsa::seg_width(s, units, off, ngroup));
      }
      std::printf("end\n");
      continue;
    }
    const int n = units * ngroup * nseg;
    for (int id = 0; id < n; ++id) {
      int u = -1, kg = -1, seg = 0;
      if (kind == 0) nsa::xcd_map(id, units, ngroup, u, kg);
      else if (kind == 1) nsa::span_task_order(id, units, ngroup, nseg, span, seglen, u, kg, seg);
      else nsa::gemm_tile_order(id, ngroup, units, u, kg);   // row tile, column tile
      std::printf("%d %d %d\n", u, kg, seg);
    }
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def order_binary(tmp_path_factory):
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("taskorder")
    src, exe = d / "order.cpp", d / "order"
    src.write_text(PROGRAM)
    subprocess.run([HIPCC, "-x", "hip", "--offload-host-only", "-O1", "-std=c++17", "-I", CSRC,
                    "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True,
                   capture_output=True)
    return str(exe)


def run(binary, cases):
    text = "".join(" ".join(map(str, c)) + "\n" for c in cases)
    out = subprocess.run([binary], input=text, capture_output=True, text=True, check=True).stdout.split("\n")
    res, i = [], 0
    for kind, units, ngroup, nseg, _, _ in cases:
        n = units * ngroup * nseg
        res.append([tuple(int(x) for x in line.split()) for line in out[i:i + n]])
        i += n
    return res


# (units, key groups, segments, group span in positions, segment length)
CMP_SHAPES = [
    (8, 16, 32, 1024, 512),    # train_16k: B=2, Hkv=4, d=16
    (4, 64, 128, 1024, 512),   # 64K, B=1, Hkv=4
    (1, 3, 5, 1024, 512),
    (2, 7, 9, 512, 512),       # d=8: one segment per group step
    (3, 5, 4, 2048, 512),      # units not dividing 8
    (16, 4, 6, 1024, 512),
    (8, 5, 7, 768, 512),       # d=12: span not a multiple of the segment
    (6, 2, 3, 320, 512),
]
WIN_SHAPES = [(8, 256), (4, 1024), (1, 33), (2, 64), (3, 10), (16, 5), (12, 7), (8, 1)]


def test_compressed_task_order_is_a_bijection_in_position_order(order_binary):
    res = run(order_binary, [(1,) + s for s in CMP_SHAPES])
    for (units, ngroup, nseg, span, seglen), tasks in zip(CMP_SHAPES, res):
        assert sorted(tasks) == [(u, k, s) for u in range(units) for k in range(ngroup) for s in range(nseg)]
        if span % seglen:
            continue
        R = span // seglen
        # dispatch order on each XCD, per unit: nondecreasing a = R*kg + seg
        last = {}
        for wid, (u, kg, seg) in enumerate(tasks):
            key = (wid % 8, u)
            a = R * kg + seg
            assert a >= last.get(key, -1), (units, ngroup, nseg, wid)
            last[key] = a


def test_window_task_map_is_a_bijection(order_binary):
    res = run(order_binary, [(0, u, n, 1, 1, 1) for u, n in WIN_SHAPES])
    for (units, ntiles), tasks in zip(WIN_SHAPES, res):
        assert sorted((u, k) for u, k, _ in tasks) == [(u, k) for u in range(units) for k in range(ntiles)]


# (row tiles, column tiles) of the layer and phi GEMMs and odd shapes
GEMM_GRIDS = [(256, 64), (256, 2), (256, 4), (8, 1), (16, 3), (5, 7), (12, 2), (1, 1)]


def test_gemm_tile_order_is_a_bijection_with_rows_grouped_per_xcd(order_binary):
    res = run(order_binary, [(2, rows, cols, 1, 1, 1) for rows, cols in GEMM_GRIDS])
    for (rows, cols), tasks in zip(GEMM_GRIDS, res):
        assert sorted((m, n) for m, n, _ in tasks) == [(m, n) for m in range(rows) for n in range(cols)]
        if rows % 8 == 0:
            # every row tile is served by a single XCD (workgroup id mod 8)
            xcd = {}
            for wid, (m, n, _) in enumerate(tasks):
                assert xcd.setdefault(m, wid % 8) == wid % 8


# (segment count, N, second offset, third offset, tile width): q|k|v widths of
# the layer shapes and ragged ones
SEG_CASES = [
    (3, 9216, 8192, 8704, 128),    # train_16k: 64 x 128 | 4 x 128 | 4 x 128
    (3, 13568, 12288, 13056, 128),  # 64 query heads x 192 | 4 x 192 | 4 x 128
    (3, 448, 256, 384, 128),       # one KV head of 64: 64-wide segments
    (2, 200, 72, 0, 128),
    (3, 3, 1, 2, 128),
    (3, 640, 128, 256, 64),
]


def test_segment_tiles_cover_every_column_once(order_binary):
    text = "".join(f"3 {n} {w} {o1} {o2} {tw}\n" for n, w, o1, o2, tw in SEG_CASES)
    out = subprocess.run([order_binary], input=text, capture_output=True, text=True, check=True).stdout
    blocks = out.split("end\n")[:-1]
    assert len(blocks) == len(SEG_CASES)
    for (nsg, N, o1, o2, tw), blk in zip(SEG_CASES, blocks):
        offs = [0, o1, o2][:nsg]
        widths = [(offs[i + 1] if i + 1 < nsg else N) - offs[i] for i in range(nsg)]
        tiles = [tuple(int(x) for x in line.split()) for line in blk.strip().splitlines()]
        # segments in order, each one's tiles from its first column in steps of tw
        expect = [(s, n0, widths[s]) for s in range(nsg) for n0 in range(0, widths[s], tw)]
        assert tiles == expect, (nsg, N, o1, o2, tw)
        cols = sorted(c for s, n0, w in tiles for c in range(offs[s] + n0, offs[s] + min(n0 + tw, w)))
        assert cols == list(range(N))
