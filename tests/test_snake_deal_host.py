"""The prefill's deal of work items to the 8 XCDs for sequences of different
lengths (duo_internal.h: snake_deal_items on the host, snake_deal_item as the
kernels use it), checked on the host over seeded sequence sets: every (unit,
query tile) is dealt to exactly one work item, the work-group count is 8 x
the largest XCD's tile count, and a deal is offered only when the XCDs' work
is within 10% of even.  A mapping mistake here would silently drop or repeat
query tiles of the prefill; the GPU parity tests would see it only at sizes
with 16 or more retrieval units."""

import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_snake_deal_is_a_bijection_and_balanced(tmp_path):
    from kv_cache_duo_amd import build as b
    lib_dir = os.path.join(ROOT, "kv_cache_duo_amd")
    exe = str(tmp_path / "snake_deal_check")
    cmd = [b.hipcc(), "-x", "hip", f"--offload-arch={b.ARCH}", "-O1", "-std=c++17",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{b.CSRC}",
           os.path.join(ROOT, "tests", "native", "snake_deal_check.cpp"),
           f"-L{lib_dir}", "-lduo", f"-Wl,-rpath,{lib_dir}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert r.stdout.startswith("ok"), r.stdout


def test_planted_mistake_in_the_deal_is_caught(tmp_path):
    """The same check against a copy of the header whose kernel-side walk
    deals every round forward (the library's host count keeps the snake):
    some tiles are then dealt twice or not at all, and the check fails."""
    from kv_cache_duo_amd import build as b
    src = open(os.path.join(b.CSRC, "duo_internal.h")).read()
    good = "return kPrefillXcds * j + ((j & 1) ? kPrefillXcds - 1 - x : x);"
    assert good in src
    inc = tmp_path / "inc"
    inc.mkdir()
    (inc / "duo_internal.h").write_text(src.replace(good, "return kPrefillXcds * j + x;"))
    lib_dir = os.path.join(ROOT, "kv_cache_duo_amd")
    exe = str(tmp_path / "snake_deal_check")
    cmd = [b.hipcc(), "-x", "hip", f"--offload-arch={b.ARCH}", "-O1", "-std=c++17", f"-I{inc}",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{b.CSRC}",
           os.path.join(ROOT, "tests", "native", "snake_deal_check.cpp"),
           f"-L{lib_dir}", "-lduo", f"-Wl,-rpath,{lib_dir}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "FAIL" in r.stdout, r.stdout[-2000:]
