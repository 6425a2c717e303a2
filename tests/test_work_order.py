"""The kernels' XCD-aware work order (csrc/device_util.h, xcd_order), on the host.

Every attention launch maps workgroup b to a (head, block) unit through
xcd_order; a unit visited twice or never would compute a block of rows twice
or leave it unwritten.  This test compiles the header's function into a small
host program and checks, over a range of shapes, that the map is a bijection
onto [0, H) x [0, nblk), that each XCD (workgroups b with the same b mod 8)
runs its units by non-increasing block index, and that each XCD's units form
one contiguous head-major range of (head, position) items, where block q sits
at position 2 (nblk - 1 - q) in the upper half and 2 q + 1 in the lower.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

PROGRAM = r"""
#include "device_util.h"
#include <cstdio>
#include <vector>
int main() {
    long units = 0;
    for (int nblk = 1; nblk <= 160; ++nblk)
        for (int H = 1; H <= 40; ++H) {
            const int nwg = H * nblk;
            std::vector<int> seen(nwg, 0);
            std::vector<int> lastq(8, 1 << 30), lo(8, 1 << 30), hi(8, -1);
            for (int b = 0; b < nwg; ++b) {
                int head = -1, blk = -1;
                rtr::dev::xcd_order(b, nwg, nblk, head, blk);
                if (head < 0 || head >= H || blk < 0 || blk >= nblk) {
                    printf("out of range: nblk %d H %d b %d -> (%d, %d)\n", nblk, H, b, head, blk);
                    return 1;
                }
                ++seen[head * nblk + blk];
                const int x = b & 7;
                if (blk > lastq[x]) {
                    printf("order: nblk %d H %d b %d block %d after %d\n", nblk, H, b, blk, lastq[x]);
                    return 1;
                }
                lastq[x] = blk;
                const int half = nblk >> 1;
                const int p = blk >= half ? 2 * (nblk - 1 - blk) : 2 * blk + 1;
                const int item = head * nblk + p;
                lo[x] = item < lo[x] ? item : lo[x];
                hi[x] = item > hi[x] ? item : hi[x];
            }
            for (int u = 0; u < nwg; ++u)
                if (seen[u] != 1) {
                    printf("unit %d of nblk %d H %d visited %d times\n", u, nblk, H, seen[u]);
                    return 1;
                }
            int count = 0;
            for (int x = 0; x < 8; ++x) {
                const int n = (nwg >> 3) + (x < (nwg & 7) ? 1 : 0);
                if (n == 0) continue;
                count += n;
                if (hi[x] - lo[x] + 1 != n) {
                    printf("XCD %d of nblk %d H %d: items %d..%d for %d units\n", x, nblk, H, lo[x], hi[x], n);
                    return 1;
                }
            }
            units += count;
        }
    printf("ok %ld\n", units);
    return 0;
}
"""


@pytest.mark.skipif(not (os.path.exists(HIPCC) or shutil.which("hipcc")), reason="hipcc not available")
def test_xcd_order_is_a_bijection_in_block_order(tmp_path):
    src = tmp_path / "order.hip"
    src.write_text(PROGRAM)
    exe = tmp_path / "order"
    hipcc = HIPCC if os.path.exists(HIPCC) else shutil.which("hipcc")
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O2", "-std=c++17",
                    "-I", os.path.join(ROOT, "causal_attention_frame_amd", "csrc"),
                    "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok "), out.stdout
