"""Host-side pin of the expert GEMM's tile order and of the backward's batched GEMM entries.

The kernels take both from mixture_experts_layer_group_amd/csrc/moe_tile_map.h.  Here that
header is compiled for the host with g++ (tests/tile_map_check.cpp) and checked over 10^4
layer shapes, one- and two-problem launches, both tile shapes: the block -> tile map is a
bijection, every tile and every batched entry stays inside its own problem, and every
operand block stays inside its buffer.  Planted mistakes in a copy of the header must each
make the check fail.  Two-problem launches that are not dealt by entries must also give every
XCD an eighth of each problem's tiles.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_layer_group_amd", "csrc")
HEADER = os.path.join(CSRC, "moe_tile_map.h")
CHECK = os.path.join(ROOT, "tests", "tile_map_check.cpp")


def _build(tmp_path, header_text=None, werror=True):
    inc = tmp_path / "inc"
    inc.mkdir(exist_ok=True)
    if header_text is None:
        shutil.copy(HEADER, inc / "moe_tile_map.h")
    else:
        (inc / "moe_tile_map.h").write_text(header_text)
    exe = tmp_path / "tile_map_check"
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    flags = ["-Wall", "-Werror"] if werror else []
    r = subprocess.run([cxx, "-O2", "-std=c++17"] + flags + ["-I", str(inc), CHECK, "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def _run(exe, n, seed=1):
    return subprocess.run([str(exe), str(n), str(seed)], capture_output=True, text=True,
                          timeout=600)


def test_tile_map_bijection_and_bounds(tmp_path):
    exe = _build(tmp_path)
    r = _run(exe, 10000)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok 10000 shapes"), r.stdout


PLANTED = {
    # the XCD ranges: the remainder slots given to the wrong XCDs
    "xcd_remainder": ("(xcd < r ? xcd : r)", "(xcd < r ? r : xcd)"),
    # dealt entries: bins one slot too short
    "deal_bins": ("base + ((T - b + 7) >> 3) <= sl", "base + ((T - b + 6) >> 3) <= sl"),
    # m-tile groups: the last group sized as a full one
    "group_size": ("mts - first < group_m ? mts - first : group_m", "group_m"),
    # routed dW1 entries: A offset with the wrong row pitch
    "dw1_pitch": ("return BatchEntry{o * H1, o * M, e * H1 * M, cnt, 0};",
                  "return BatchEntry{o * M, o * M, e * H1 * M, cnt, 0};"),
    # shared ranges: the last range not clipped to the token count
    "shared_clip": ("return static_cast<int>(kshared < N - n0 ? kshared : N - n0);",
                    "return static_cast<int>(kshared);"),
    # router weight-gradient partials written over each other
    "dwg_partials": ("return BatchEntry{n0 * Ep, n0 * M, q * E * M,",
                     "return BatchEntry{n0 * Ep, n0 * M, q * M,"),
    # batched tile rows: the last m-tile of an entry not clipped
    "batch_rows": ("nrows = rows - row0 < BM ? rows - row0 : BM;", "nrows = BM;"),
    # two-problem ranges: problem 1's remainder tiles given to the same XCDs as problem 0's
    "second_remainder": ("before += ((x - r0 + 8) & 7) < r1 ? 1 : 0;", "before += x < r1 ? 1 : 0;"),
    # two-problem ranges: the problems concatenated and cut into eight (unbalanced when their
    # K differ)
    "concatenated": ("if (s.tpe == 0 && tot0 > 0 && tot1 > 0) {", "if (false) {"),
}


@pytest.mark.parametrize("name", sorted(PLANTED))
def test_tile_map_planted_mistake_fails(tmp_path, name):
    old, new = PLANTED[name]
    text = open(HEADER).read()
    assert text.count(old) == 1, f"pattern of planted mistake {name} not found once"
    exe = _build(tmp_path, text.replace(old, new), werror=False)
    r = _run(exe, 3000)
    # a reported failure, or a crash of the check (a decoded slot past the last problem makes
    # the group arithmetic divide by zero)
    assert ("FAIL" in r.stdout and r.returncode == 1) or r.returncode < 0, (r.returncode,
                                                                            r.stdout)
