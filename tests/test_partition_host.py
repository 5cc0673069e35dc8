"""Host check of the work split shared by the decode kernels (csrc/common.h).

The split kernel gives worker w the units [part_begin(w), part_begin(w + 1)).
Between one worker per SIMD and the maximum, the worker count is rounded down
to one per SIMD.
The ranges must tile [0, total), and part_of(u), their inverse, must agree
with them exactly and never return a worker without units.  part_begin
divides with div_nonneg, whose 32-bit, corrected double-precision and 64-bit
routes are each reached by the sizes below, and div_nonneg is also checked
directly against the 64-bit quotient.  The header is compiled for the host
with hipcc (no GPU needed).
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COMMON = os.path.join(ROOT, "decode_attention_int4_block_amd", "csrc", "common.h")

CHECKER = r"""
#include <hip/hip_runtime.h>
#include <cstdio>
#include "COMMON_H"
using namespace kvq;
int main() {
    const int32_t weights[3][4] = {{128, 128, 100, 100}, {131, 123, 103, 97}, {1, 1, 1, 1}};
    long checks = 0;
    // exact division on every route: 32-bit, double-precision with correction, 64-bit
    for (long long n : {0LL, 1LL, 4294967295LL, 4294967296LL, 12345678901234LL, 9007199254740991LL,
                        9007199254740992LL, 9007199254740993LL, 4611686018427387903LL})
    for (long long d : {1LL, 2LL, 3LL, 7LL, 2047LL, 285887LL, 4294967295LL, 4294967296LL, 4294967311LL}) {
        if (div_nonneg(n, d) != n / d) { printf("div_nonneg(%lld, %lld) = %lld, want %lld\n", n, d, (long long)div_nonneg(n, d), n / d); return 1; }
        for (long long k : {1LL, 2LL, 1000003LL}) {
            const long long m = n / k;
            if (div_nonneg(m, d) != m / d) { printf("div_nonneg(%lld, %lld)\n", m, d); return 1; }
            if (m >= 1 && div_nonneg(m - 1, d) != (m - 1) / d) { printf("div_nonneg(%lld, %lld)\n", m - 1, d); return 1; }
        }
    }
    // workers of [0, n) in even-numbered workgroups, against a count
    for (int l : {0, 1, 2})
    for (long long n = 0; n < 200; ++n) {
        long long c = 0;
        for (long long w = 0; w < n; ++w) c += ((w >> l) & 1) == 0;
        if (even_wg_workers(n, l) != c) { printf("even_wg_workers(%lld, %d) = %lld, want %lld\n", n, l, (long long)even_wg_workers(n, l), c); return 1; }
    }
    for (int wg : {1, 4})
    for (const auto &wt : weights)
    for (long long total : {1LL, 7LL, 8LL, 100LL, 8230LL, 12000LL, 16383LL, 16384LL, 16385LL, 96700LL, 1234567LL,
                            99999989LL, 1099511627776LL})
    for (long long maxw : {1LL, 2LL, 3LL, 5LL, 2047LL, 2048LL, 2816LL})
    for (long long simds : {0LL, 1024LL}) {
        const Partition p = make_partition(total, maxw, wt, 8, wg, simds);
        if (p.W < 1 || p.W > maxw) { printf("bad W\n"); return 1; }
        // between one worker per SIMD and the maximum, one per SIMD
        const Partition p0 = make_partition(total, maxw, wt, 8, wg, 0);
        const long long want = (simds > 0 && p0.W > simds && p0.W < maxw) ? simds : p0.W;
        if (p.W != want) { printf("W %lld, want %lld (total %lld, max %lld)\n", (long long)p.W, want, total, maxw); return 1; }
        long long prev = 0;
        for (long long w = 0; w < p.W; ++w) {
            const long long b0 = part_begin(p, w), b1 = part_begin(p, w + 1);
            if (b0 != prev || b1 < b0) { printf("ranges do not tile: total %lld W %lld w %lld\n", total, (long long)p.W, w); return 1; }
            prev = b1;
            const long long step = (b1 - b0) > 64 ? (b1 - b0) / 17 : 1;
            for (long long u = b0; u < b1; u += step, ++checks)
                if (part_of(p, u) != w) { printf("part_of(%lld) = %lld, want %lld (total %lld W %lld)\n", u, (long long)part_of(p, u), w, total, (long long)p.W); return 1; }
            if (b1 > b0 && part_of(p, b1 - 1) != w) { printf("last unit of %lld\n", w); return 1; }
        }
        if (prev != total) { printf("end %lld != total %lld\n", prev, total); return 1; }
    }
    printf("ok %ld\n", checks);
    return 0;
}
"""


def _hipcc():
    h = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    return h if os.path.exists(h) or shutil.which(h) else None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_partition_begin_and_owner_agree(tmp_path):
    src = tmp_path / "check_partition.cpp"
    src.write_text(CHECKER.replace("COMMON_H", COMMON))
    exe = tmp_path / "check_partition"
    r = subprocess.run([_hipcc(), "-O2", "-w", "-o", str(exe), str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok")
