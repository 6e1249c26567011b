"""The GEMM kernels' block-to-tile mapping (csrc/tile_map.h), compiled on the host.

The header is plain integer arithmetic; here it is built with g++ into a small
driver that checks, for every grid of up to 140 x 24 tiles and both walk orders:
every block id maps to a tile inside the grid and no two ids share a tile (a
bijection, so a launch covers each output tile exactly once), and, for the
spread order, that when only a leading range of block-rows does work (a device
row count) those tiles are dealt evenly to the 8 XCDs (block id % 8): no XCD gets
more than one group of tiles (GROUP_M x tn) above an even share. The in-order
walk does not have this property: on a 63 x 12 grid (16 000 tokens, N = 3072) with
16 working block-rows it puts them on 3 of the 8 XCDs.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "flow_matching_tts_amd", "csrc")

DRIVER = r"""
#define __host__
#define __device__
#include <cstdio>
#include <vector>
#include "tile_map.h"
// tiles with block-row < live on the busiest XCD
static int max_share(int tm, int tn, int live, bool spread) {
    int per[8] = {0};
    for (int bid = 0; bid < tm * tn; ++bid) {
        int mt, nt;
        cfm::tile_of(bid, tm * tn, tm, tn, spread, mt, nt);
        if (mt < live) per[bid % 8]++;
    }
    int hi = 0;
    for (int x = 0; x < 8; ++x) hi = per[x] > hi ? per[x] : hi;
    return hi;
}

int main() {
    long bad = 0, checked = 0;
    for (int tm = 1; tm <= 140; ++tm)
        for (int tn = 1; tn <= 24; ++tn)
            for (int spread = 0; spread < 2; ++spread) {
                const int n = tm * tn;
                std::vector<int> hit(n, 0);
                for (int bid = 0; bid < n; ++bid) {
                    int mt = -1, nt = -1;
                    cfm::tile_of(bid, n, tm, tn, spread != 0, mt, nt);
                    if (mt < 0 || mt >= tm || nt < 0 || nt >= tn) { ++bad; continue; }
                    hit[mt * tn + nt]++;
                }
                for (int i = 0; i < n; ++i) bad += hit[i] != 1;
                ++checked;
                if (!spread) continue;
                for (int live = 1; live <= tm; ++live) {   // block-rows that do work
                    const int worst = max_share(tm, tn, live, true);
                    const int even = (live * tn + 7) / 8;
                    if (worst > even + cfm::GROUP_M * tn) {
                        ++bad;
                        if (bad < 5) std::printf("imbalance tm=%d tn=%d live=%d: %d > %d\n", tm, tn, live, worst, even);
                    }
                }
            }
    // the in-order walk on a 63 x 12 grid with 16 working block-rows: 3 XCDs busy
    const int in_order = max_share(63, 12, 16, false), spread = max_share(63, 12, 16, true);
    std::printf("63x12, 16 live rows: busiest XCD %d tiles in order, %d spread (even share 24)\n", in_order, spread);
    bad += !(in_order > 24 + cfm::GROUP_M * 12 && spread <= 24 + cfm::GROUP_M * 12);
    std::printf("checked %ld grids, %ld failures\n", checked, bad);
    return bad != 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_tile_map_is_a_bijection_and_spreads_leading_rows(tmp_path):
    src = tmp_path / "tile_map_check.cpp"
    src.write_text(DRIVER)
    exe = tmp_path / "tile_map_check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True)
    print(res.stdout)
    assert res.returncode == 0, res.stdout
