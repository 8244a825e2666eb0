"""Host check of the packed-sequence span clamp (csrc/jb_span.h), compiled with g++ on
the CPU: whatever cu_seqlens holds, every kernel's row span stays inside the packed
rows and the planned maximum length, and well-formed offsets pass through unchanged."""
import itertools
import os
import subprocess
import tempfile

import pytest

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "gated_delta_rule_jetblock_amd", "csrc")

PROG = r"""
#include <stdio.h>
#include "jb_span.h"
int main() {
  int c0, c1, tmax; long long total;
  while (scanf("%d %d %d %lld", &c0, &c1, &tmax, &total) == 4) {
    int64_t tok0; int T;
    jb::clamp_span(c0, c1, tmax, total, tok0, T);
    printf("%lld %d\n", (long long)tok0, T);
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def clamp_exe():
    d = tempfile.mkdtemp()
    src, exe = os.path.join(d, "span.cpp"), os.path.join(d, "span")
    open(src, "w").write(PROG)
    subprocess.check_call(["g++", "-O1", "-std=c++17", "-I", HDR, src, "-o", exe])
    return exe


def test_span_clamp(clamp_exe):
    vals = [-2147483648, -1000, -3, -1, 0, 1, 5, 64, 199, 200, 201, 299, 300, 301, 5000, 2147483647]
    cases = [(c0, c1, tmax, total) for c0, c1 in itertools.product(vals, vals)
             for tmax in (1, 200, 4096) for total in (0, 1, 300)]
    inp = "".join(f"{c0} {c1} {tm} {tot}\n" for c0, c1, tm, tot in cases)
    out = subprocess.run([clamp_exe], input=inp, capture_output=True, text=True, check=True).stdout.split("\n")
    for (c0, c1, tmax, total), line in zip(cases, out):
        tok0, T = map(int, line.split())
        assert 0 <= tok0 <= total and 0 <= T <= tmax and tok0 + T <= total, (c0, c1, tmax, total, tok0, T)
        if 0 <= c0 <= c1 <= total:
            # well-formed: the span itself, cut to the planned maximum length
            assert (tok0, T) == (c0, min(c1 - c0, tmax)), (c0, c1, tmax, total, tok0, T)
