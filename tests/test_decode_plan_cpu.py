"""The decode kernels' split plans, checked on the CPU (nothing here runs on
a GPU): a small host program includes the library's launch header, calls
both planners over many shapes and prints what they return; the test then
forms each wave's (split kernel) or workgroup's (kernel for 2 or 4 column
groups) key range the way the kernels do and checks that the ranges cover
keys 0 .. L-1 exactly once, that every workgroup gets keys, that step starts
stay multiples of 32 (64) from the range start, and that a head's extra
steps are spread evenly over the workgroups."""
import os
import random
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "zero_shot_rope_jl_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")

PROG = r"""
#include <cstdio>
#include "internal.h"
int main() {
    long long B, Hkv, L;
    while (std::scanf("%lld %lld %lld", &B, &Hkv, &L) == 3) {
        int ns, ch, ex, sf, mns, mch, mex;
        jl::decode_split_plan(B, Hkv, L, &ns, &ch, &ex, &sf);
        jl::decode_multi_plan(B, Hkv, L, &mns, &mch, &mex);
        std::printf("%d %d %d %d %d %d %d %d %d\n", ns, ch, ex, jl::decode_heads_per_wg(Hkv), mns, mch, mex,
                    jl::kDecodeWaves, sf);
    }
    return 0;
}
"""


@pytest.fixture(scope="module")
def planner(tmp_path_factory):
    d = tmp_path_factory.mktemp("plan")
    src = d / "plan.cpp"
    src.write_text(PROG)
    exe = d / "plan"
    # host code only: the header's device helpers are not compiled
    subprocess.run([HIPCC, "-O1", "-std=c++17", "--offload-arch=gfx950", "--cuda-host-only", "-I", CSRC, "-I", os.path.join(ROOT, "include"), str(src),
                    "-o", str(exe)], check=True, capture_output=True, text=True)
    return str(exe)


def _cases():
    rng = random.Random(20261204)
    cases = [(1, 8, L) for L in (1, 31, 32, 33, 4100, 131072, 131073, 131136, 131200, 131328, 1 << 20, (1 << 20) + 1)]
    cases += [(1, 1, (1 << 20) + s) for s in (0, 1, 7, 256)]
    for _ in range(3000):
        cases.append((rng.choice([1, 2, 3, 8, 64, 300]), rng.choice([1, 2, 4, 8, 16]), rng.randint(1, 400000)))
    return cases


def test_plans_cover_every_key_once(planner):
    cases = _cases()
    r = subprocess.run([planner], input="".join(f"{b} {h} {l}\n" for b, h, l in cases), capture_output=True,
                       text=True, check=True)
    rows = [list(map(int, line.split())) for line in r.stdout.splitlines()]
    assert len(rows) == len(cases)
    for (B, Hkv, L), (ns, ch, ex, wh, mns, mch, mex, nwaves, sf) in zip(cases, rows):
        # split kernel: wave (split, sub) of a head takes the steps numbered
        # sub * ns + split (split-fastest, the dealt plan) or split * NW + sub
        # (one KV head per workgroup: whole steps rounded up, no extra steps)
        NW = nwaves // wh
        assert sf == (0 if wh == 1 else 1) and (sf or ex == 0), (B, Hkv, L)
        assert 1 <= ns <= 256 and ch % 32 == 0 and 0 <= ex < ns * NW, (B, Hkv, L)
        ranges, extra_per_wg = [], {}
        for split in range(ns):
            got = False
            for sub in range(NW):
                j = sub * ns + split if sf else split * NW + sub
                lo = j * ch + 32 * min(j, ex)
                hi = min(L, lo + ch + (32 if j < ex else 0))
                if lo < hi:
                    ranges.append((lo, hi))
                    got = True
                if j < ex:
                    extra_per_wg[split] = extra_per_wg.get(split, 0) + 1
            assert got, ("a workgroup without keys", B, Hkv, L, split)
        # the extra steps are spread over the workgroups: their counts differ
        # by at most one (at most one each while there are fewer than splits)
        per_wg = [extra_per_wg.get(s, 0) for s in range(ns)]
        assert max(per_wg) - min(per_wg) <= 1, (B, Hkv, L)
        ranges.sort()
        pos = 0
        for lo, hi in ranges:
            assert lo == pos and lo % 32 == 0, (B, Hkv, L, lo, pos)
            pos = hi
        assert pos == L, (B, Hkv, L, pos)
        # kernel for 2 or 4 column groups: workgroup s, 64-key stages
        assert 1 <= mns and mch % 64 == 0 and 0 <= mex < mns, (B, Hkv, L)
        pos = 0
        for s in range(mns):
            lo = s * mch + 64 * min(s, mex)
            hi = min(L, lo + mch + (64 if s < mex else 0))
            assert lo == pos and hi > lo, (B, Hkv, L, s)
            pos = hi
        assert pos == L, (B, Hkv, L)
        # about one workgroup per compute unit
        assert ns * B * (Hkv // wh) <= max(256, B * (Hkv // wh)), (B, Hkv, L)
