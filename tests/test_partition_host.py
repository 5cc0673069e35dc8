"""Host check of the work split shared by the decode kernels (csrc/common.h).

The split kernel gives worker w the units [part_begin(w), part_begin(w + 1))
and the combine kernel finds the workers of a segment with part_of(u); the two
must agree exactly, the ranges must tile [0, total), and no unit may map to a
worker without units.  The header is compiled for the host with hipcc and the
properties are checked on many sizes (no GPU needed).
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
    for (const auto &wt : weights)
    for (long long total : {1LL, 7LL, 8LL, 100LL, 16383LL, 16384LL, 16385LL, 96700LL, 1234567LL, 99999989LL})
    for (long long maxw : {1LL, 2LL, 3LL, 5LL, 2047LL, 2048LL, 2816LL}) {
        const Partition p = make_partition(total, maxw, wt, 8);
        if (p.W < 1 || p.W > maxw) { printf("bad W\n"); return 1; }
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
