"""The overflow split of the head_dim-128 forward (csrc/attn_fwd.hip), on the host.

When a launch has U units (heads x 256-row query blocks) just beyond one round
of G workgroups, plan_overflow gives the first nx query blocks of every head no
main workgroup and cuts their key tiles into pieces that every workgroup takes
after its own unit.  A unit run twice or never, a tile in no piece or in two,
or a combine that reads another piece's slot would all corrupt O silently.
This test compiles the source into a small host program that calls the
planner and the kernel's role, piece and slot functions (host-callable), and
checks, over streaming shapes of several frame lengths, head counts, chunk
and cache sizes and both workspace sizes (the full one and the 256 slots of the
static scratch), that:
  - every unit of a query block >= nx is the main of exactly one workgroup and
    no unit of a block < nx is;
  - the workgroups' piece ranges [pk[b], pk[b + 8]) (the XCD's end for the last
    workgroup of an XCD) partition [0, K) with K within the workspace slots;
  - the pieces cover every key tile of every extra unit exactly once, in unit
    order, and the combine's slot numbering (pieces of the units before it,
    head-major) names exactly the pieces of each unit.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

PROGRAM = r"""
#include "attn_fwd.hip"
#include <cstdio>
#include <vector>

namespace rtr {
int run() {
    long plans = 0;
    for (int kpf : {96, 333, 700, 1000, 1024, 1560, 2080})
        for (int H : {1, 2, 5, 12, 16, 24, 30, 35, 40})
            for (int C = 1; C <= 4; ++C)
                for (int pf : {0, 1, 3, 7, 10})
                    for (long slots : {512L, 256L}) {
                        KArgs k{};
                        k.Tq = C * kpf;
                        k.prefix = pf * kpf;
                        k.Tk = k.prefix + k.Tq;
                        k.kpf = kpf;
                        k.nqb = (k.Tq + 255) / 256;
                        const int G = 256;
                        SplitPlan plan{};
                        int32_t nx = 0;
                        if (!plan_overflow(k, H, G, slots, &plan, &nx, k.pk)) continue;
                        ++plans;
                        k.units = k.nqb * H;
                        k.nprog = G;
                        k.cut = plan.cut;
                        k.piece = plan.piece;
                        k.tail_total = plan.pieces;
                        k.nxqb = nx;
                        const int K = plan.pieces;
                        if (nx <= 0 || nx >= k.nqb || K <= 0 || K > slots) {
                            printf("bad plan kpf %d H %d C %d pf %d: nx %d K %d\n", kpf, H, C, pf, nx, K);
                            return 1;
                        }
                        // mains
                        std::vector<int> mains(k.units, 0);
                        for (int b = 0; b < G; ++b) {
                            int unit = -1, spare = -1;
                            split_role(b, k, unit, spare);
                            if (unit >= 0) ++mains[unit];
                        }
                        for (int u = 0; u < k.units; ++u)
                            if (mains[u] != (u % k.nqb >= nx ? 1 : 0)) {
                                printf("unit %d main count %d (kpf %d H %d C %d pf %d)\n", u, mains[u], kpf, H, C, pf);
                                return 1;
                            }
                        // piece ranges and prefix
                        std::vector<int> sPre(1, 0);
                        for (int pu = 0; pu < piece_units(k); ++pu)
                            sPre.push_back(sPre.back() + unit_pieces(piece_unit(pu, k), k));
                        if (sPre.back() != K) {
                            printf("prefix %d != K %d\n", sPre.back(), K);
                            return 1;
                        }
                        std::vector<int> taken(K, 0);
                        std::vector<std::vector<int>> covered(k.units);
                        std::vector<std::vector<int>> pieces_of(k.units);
                        for (int b = 0; b < G; ++b) {
                            const int k0 = k.pk[b];
                            const int k1 = b + 8 < G ? k.pk[b + 8] : (int)((long)((b & 7) + 1) * K / 8);
                            if (k0 > k1 || k0 < 0 || k1 > K) {
                                printf("workgroup %d range [%d, %d) of %d\n", b, k0, k1, K);
                                return 1;
                            }
                            for (int kk = k0; kk < k1; ++kk) {
                                ++taken[kk];
                                const int pu = find_tail_unit(sPre.data(), piece_units(k), kk);
                                const int i = kk - sPre[pu];
                                const int u = piece_unit(pu, k);
                                const int qb = u % k.nqb;
                                const int tb = i * k.piece, te = std::min(block_tiles(qb, k), tb + k.piece);
                                if (qb >= nx || tb >= te) {
                                    printf("piece %d: unit %d qb %d tiles [%d, %d)\n", kk, u, qb, tb, te);
                                    return 1;
                                }
                                for (int t = tb; t < te; ++t) covered[u].push_back(t);
                                pieces_of[u].push_back(kk);
                            }
                        }
                        for (int kk = 0; kk < K; ++kk)
                            if (taken[kk] != 1) {
                                printf("piece %d taken %d times\n", kk, taken[kk]);
                                return 1;
                            }
                        for (int u = 0; u < k.units; ++u) {
                            const int qb = u % k.nqb, head = u / k.nqb;
                            if (qb >= nx) {
                                if (!covered[u].empty()) return 1;
                                continue;
                            }
                            std::vector<int> c = covered[u];
                            std::sort(c.begin(), c.end());
                            const int nt = block_tiles(qb, k);
                            if ((int)c.size() != nt) {
                                printf("unit %d: %zu tiles covered of %d\n", u, c.size(), nt);
                                return 1;
                            }
                            for (int t = 0; t < nt; ++t)
                                if (c[t] != t) return 1;
                            // the combine's slots: pieces of the units before u, then q of its own
                            int k0 = 0;
                            for (int bq = 0; bq < k.nqb; ++bq) {
                                const int qp = unit_pieces(bq, k);
                                k0 += qp * head + (bq < qb ? qp : 0);
                            }
                            std::vector<int> p = pieces_of[u];
                            std::sort(p.begin(), p.end());
                            const int q = unit_pieces(u, k);
                            if ((int)p.size() != q) return 1;
                            for (int j = 0; j < q; ++j)
                                if (p[j] != k0 + j) {
                                    printf("unit %d: combine slot %d, piece %d\n", u, k0 + j, p[j]);
                                    return 1;
                                }
                        }
                    }
    printf("ok %ld\n", plans);
    return plans > 0 ? 0 : 1;
}
}  // namespace rtr

int main() { return rtr::run(); }
"""


@pytest.mark.skipif(not (os.path.exists(HIPCC) or shutil.which("hipcc")), reason="hipcc not available")
def test_overflow_split_plans_partition_the_work(tmp_path):
    src = tmp_path / "ovf.hip"
    src.write_text(PROGRAM)
    exe = tmp_path / "ovf"
    hipcc = HIPCC if os.path.exists(HIPCC) else shutil.which("hipcc")
    res = subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-std=c++17",
                          "-I", os.path.join(ROOT, "causal_attention_frame_amd", "csrc"),
                          "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok "), out.stdout
