"""Host-side launch chunking (csrc/chunks.hpp), compiled with g++ and run on
the CPU: every row and every (batch, head) pair is covered exactly once, no
launch exceeds its limit, and small problems stay one launch."""
import os
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "row_wise_online_amd", "csrc")

DRIVER = r"""
#include <stdio.h>
#include <stdlib.h>
#include <vector>
#include "chunks.hpp"

static int fail(const char *what, long long a, long long b) {
    printf("FAIL %s %lld %lld\n", what, a, b);
    return 1;
}

int main() {
    // rows: every M around the limit and its multiples, with small limits
    // standing in for 2^22 as well as the real one
    const long long limits[] = {1, 2, 3, 7, 64, 1000, 1LL << 22};
    for (long long lim : limits) {
        std::vector<long long> Ms = {0, 1, 2, lim - 1, lim, lim + 1, 2 * lim - 1,
                                     2 * lim, 2 * lim + 1, 7 * lim + 3};
        if (lim == (1LL << 22)) Ms.push_back((1LL << 31) - 1);
        for (long long M : Ms) {
            if (M < 0) continue;
            os::RowChunks rc = os::row_chunks(M, lim);
            if (M <= lim && (rc.count != 1 || rc.rows != M)) return fail("single", M, lim);
            if (rc.rows > lim) return fail("rows>lim", M, lim);
            long long covered = 0;
            for (long long c = 0; c < rc.count; ++c) {
                long long r0 = c * rc.rows;
                long long n = M - r0 < rc.rows ? M - r0 : rc.rows;
                if (r0 != covered) return fail("gap", M, c);
                if (M > 0 && n < 1) return fail("empty part", M, c);
                if (M > lim && 2 * n <= lim && c + 1 < rc.count) return fail("short", M, c);
                covered += n;
            }
            if (covered != M) return fail("cover", M, covered);
        }
    }
    // heads: (B, H, per_head, limit)
    const long long cases[][4] = {
        {1, 1, 1, 8}, {3, 5, 1, 8}, {3, 5, 2, 8}, {2, 7, 3, 8}, {4, 3, 8, 8},
        {5, 9, 7, 8}, {1, 20, 1, 8}, {6, 2, 4, 8}, {3, 1398102, 1, 1LL << 22},
        {1, (1LL << 22) + 5, 1, 1LL << 22}, {2, 3, 1LL << 22, 1LL << 22},
        {8193, 1024, 1, 1LL << 22}, {1, 1, 1, 1LL << 22}};
    for (auto &cs : cases) {
        long long B = cs[0], H = cs[1], ph = cs[2], lim = cs[3];
        std::vector<int> seen((size_t)(B * H), 0);
        long long launches = 0;
        bool bad = false;
        os::for_each_head_chunk(B, H, ph, [&](const os::HeadChunk &c) {
            ++launches;
            if (c.nb < 1 || c.nh < 1 || c.b0 < 0 || c.h0 < 0) bad = true;
            if (c.b0 + c.nb > B || c.h0 + c.nh > H) bad = true;
            if (c.nb > 1 && (c.h0 != 0 || c.nh != H)) bad = true;
            if (c.nb * c.nh * ph > lim) bad = true;
            for (long long b = c.b0; b < c.b0 + c.nb && !bad; ++b)
                for (long long h = c.h0; h < c.h0 + c.nh; ++h) seen[b * H + h]++;
        }, lim);
        if (bad) return fail("head chunk", B, H);
        for (size_t i = 0; i < seen.size(); ++i)
            if (seen[i] != 1) return fail("head cover", (long long)i, seen[i]);
        if (B * H * ph <= lim && launches != 1) return fail("one launch", B, H);
    }
    printf("OK\n");
    return 0;
}
"""


def test_chunk_plans_cover_once():
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "drv.cpp")
        exe = os.path.join(d, "drv")
        with open(src, "w") as f:
            f.write(DRIVER)
        subprocess.run(["g++", "-std=c++17", "-O1", "-I", CSRC, src, "-o", exe],
                       check=True)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0 and r.stdout.strip() == "OK", r.stdout
