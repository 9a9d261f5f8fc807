"""Host logic of the GEMM work order, on the CPU: the closed-form count of
the A and B panels a run of work items touches (walk_panels) against a
brute-force count over the same walk, and the group sizes gemm_walk_group
picks for the MLP products.  The two functions are compiled with g++ from
their text in gemm.hip (plain host C++), so the test runs without a GPU."""
import os
import random
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "causal_attention_attn_amd", "csrc", "gemm.hip")

HARNESS = r"""
#include <algorithm>
#include <cstdio>
%s
int main()
{
    long long a, b;
    int tm, tn, g;
    char op;
    while (std::scanf(" %%c", &op) == 1) {
        if (op == 'p' && std::scanf("%%lld %%lld %%d %%d %%d", &a, &b, &tm, &tn, &g) == 5)
            std::printf("%%lld\n", walk_panels(a, b, tm, tn, g));
        else if (op == 'g' && std::scanf("%%d %%d %%d", &tm, &tn, &g) == 3)
            std::printf("%%d\n", gemm_walk_group(tm, tn, g));
    }
    return 0;
}
"""


def brute_panels(a, b, tiles_m, tiles_n, g):
    """Distinct (chunk, m-tile) and (chunk, n-tile) pairs of items [a, b):
    item v is tile t = v mod tiles of chunk v / tiles; tiles are walked in
    groups of g m-tiles, m fastest (the kernel's work order)."""
    tiles = tiles_m * tiles_n
    A, B = set(), set()
    for v in range(a, b):
        s, t = divmod(v, tiles)
        gi = g * tiles_n
        first = (t // gi) * g
        gs = min(tiles_m - first, g)
        A.add((s, first + (t % gi) % gs))
        B.add((s, (t % gi) // gs))
    return len(A) + len(B)


@pytest.fixture(scope="module")
def walk_exe(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    text = open(SRC, encoding="utf-8").read()
    m = re.search(r"long long walk_panels\(.*?\n}\n.*?int gemm_walk_group\(.*?\n}\n", text, re.S)
    assert m, "walk_panels / gemm_walk_group not found in gemm.hip"
    d = tmp_path_factory.mktemp("walk")
    cpp = d / "walk.cpp"
    cpp.write_text(HARNESS % m.group(0))
    exe = d / "walk"
    subprocess.run([gxx, "-O1", "-std=c++17", str(cpp), "-o", str(exe)], check=True)
    return str(exe)


def run(exe, lines):
    p = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True, check=True)
    return [int(x) for x in p.stdout.split()]


def test_walk_panels_matches_brute_force(walk_exe):
    rng = random.Random(7)
    cases = []
    for _ in range(3000):
        tm, tn, sp = rng.randint(1, 30), rng.randint(1, 20), rng.randint(1, 4)
        g = rng.randint(1, tm)
        items = tm * tn * sp
        a = rng.randrange(items)
        b = a + 1 + rng.randrange(items - a)
        cases.append((a, b, tm, tn, g))
    got = run(walk_exe, ["p %d %d %d %d %d" % c for c in cases])
    for c, x in zip(cases, got):
        assert x == brute_panels(*c), c


def test_walk_group_choices(walk_exe):
    # X W1^T 8192 x 3072 (64 x 24 tiles of 128), dY W1 8192 x 768 (64 x 6),
    # dY^T X 3072 x 768 in three chunks (24 x 6 x 3), 4096^3 in 256-tiles (16 x 16)
    got = run(walk_exe, ["g 64 24 1", "g 64 6 1", "g 24 6 3", "g 16 16 1", "g 5 7 1", "g 3 3 1"])
    assert got[:4] == [8, 8, 1, 8]
    assert got[4] == 5  # 35 items do not split into eight equal runs: the largest group, at most tiles_m
    assert 1 <= got[5] <= 3
    # the shapes of the GPU test of the walk (tests/test_gemm_gpu.py, WALK)
    assert run(walk_exe, ["g 5 8 1", "g 7 8 1", "g 6 4 2", "g 6 6 2"]) == [2, 4, 1, 4]


def test_walk_group_is_the_cheapest_candidate(walk_exe):
    """The chosen group reads no more panels over the eight equal XCD runs
    than any other candidate (1, 2, 4, 8 up to tiles_m), by brute force."""
    rng = random.Random(11)
    shapes = [(rng.randint(1, 24), rng.randint(1, 12), rng.randint(1, 3)) for _ in range(60)]
    shapes = [s for s in shapes if (s[0] * s[1] * s[2]) % 8 == 0][:25]
    got = run(walk_exe, ["g %d %d %d" % s for s in shapes])

    def cost(tm, tn, sp, g):
        items = tm * tn * sp
        return sum(brute_panels(x * items // 8, (x + 1) * items // 8, tm, tn, g) for x in range(8))

    for (tm, tn, sp), g in zip(shapes, got):
        cands = [c for c in (1, 2, 4, 8) if c < min(8, tm)] + [min(8, tm)]
        assert g in cands
        assert cost(tm, tn, sp, g) == min(cost(tm, tn, sp, c) for c in cands), (tm, tn, sp, g)
