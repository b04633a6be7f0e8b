"""Host logic of the tile tuner: token ranges, the choice rule, and the generated table source."""

import os
import subprocess

import pytest

from mhc_hyper_connection_pre_amd import build, tune


def test_ranges_merge_and_cover():
    pts = [(16, -80), (64, -80), (256, -56), (2048, -32), (16384, -32)]
    r = tune.ranges(pts)
    assert r[0][0] == 1 and r[-1][1] == tune.T_MAX
    assert [ns for _, _, ns in r] == [-80, -56, -32]
    for (lo, hi, _), (lo2, _, _) in zip(r, r[1:]):
        assert hi + 1 == lo2                      # contiguous, no overlap
    # the boundary between 64 and 256 sits at their geometric mean
    assert r[0][1] == 128 and r[1][0] == 129
    assert tune.ranges([(2048, -32)]) == [(1, tune.T_MAX, -32)]
    # with the kernel instance: a change of instance alone starts a new range
    r2 = tune.ranges([(64, -80, 0), (256, -80, 0), (2048, -80, 1), (16384, -32, 1)])
    assert [c for _, _, *c in r2] == [[-80, 0], [-80, 1], [-32, 1]]


def test_pick_keeps_library_tiling_within_three_percent():
    assert tune.pick({-32: 47.0, -28: 46.0, 16: 70.0}, -32) == -32
    assert tune.pick({-32: 47.0, -28: 45.0, 16: 70.0}, -32) == -28
    assert tune.pick({4: 10.0, 8: 9.0}, None) == 8


def test_generated_table_compiles(tmp_path):
    entries = [{"op": "pre", "n": 4, "D": 7168, "dtype": "bf16", "dt": 0,
                "points": [{"T": 64, "best": -56, "stagger": 0}, {"T": 2048, "best": -32, "stagger": 1}]},
               {"op": "boundary", "n": 4, "D": 5120, "dtype": "bf16", "dt": 0,
                "points": [{"T": 32, "best": -80, "stagger": 0}]},
               {"op": "pre", "n": 8, "D": 4096, "dtype": "bf16", "dt": 0,
                "points": [{"T": 32, "best": 16, "stagger": -1}]}]
    src = tmp_path / "table.cpp"
    tune.write_cpp(str(src), entries, "test device", "now")
    text = src.read_text()
    assert "{0, 4, 7168, 0, 1, 362, -56, 0}," in text
    assert "{0, 4, 7168, 0, 363, 2147483647, -32, 1}," in text
    assert "{1, 4, 5120, 0, 1, 2147483647, -80, 0}," in text
    assert "{0, 8, 4096, 0, 1, 2147483647, 16, -1}," in text
    cc = build.hipcc()
    inc = os.path.join(build.PKG, "csrc")
    r = subprocess.run([cc, *build.COMMON_FLAGS, f"-I{inc}", "-c", str(src), "-o", str(tmp_path / "t.o")],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout


def test_committed_table_matches_its_record():
    """Every range in the compiled table comes from the tuner's JSON record of the same run."""
    import json
    rec = os.path.join(build.PKG, "tile_table.json")
    if not os.path.exists(rec):
        pytest.skip("no tuner record")
    d = json.load(open(rec))
    # the record covers n = 2, 3, 4 and 8, and several hidden sizes at n = 4
    assert {e["n"] for e in d["entries"]} >= {2, 3, 4, 8}
    assert {e["D"] for e in d["entries"] if e["n"] == 4} >= {4096, 5120, 6144, 7168}
    with open(os.path.join(build.CSRC, "mhc_tile_table.cpp")) as f:
        text = f.read()
    assert d["measured"] in text
    import mhc_hyper_connection_pre_amd as mhc
    L = mhc.lib()
    for e in d["entries"]:
        for lo, hi, ns, st in tune.ranges([(p["T"], p["best"], p["stagger"]) for p in e["points"]]):
            op = 0 if e["op"] == "pre" else 1
            assert f"{{{op}, {e['n']}, {e['D']}, {e['dt']}, {lo}, {hi}, {ns}, {st}}}," in text
            assert ns < 0 or st == -1   # an instance only for the single-pass kernel
        # the library's choice at every measured token count is the measured best
        for p in e["points"]:
            want = p["best"]
            if e["op"] == "pre":
                assert L.mhc_pre_splits(p["T"], e["n"], e["D"], 0, e["dt"]) == abs(want)
            else:
                assert L.mhc_post_pre_fused(p["T"], e["n"], e["D"], 0, e["dt"]) == (1 if want < 0 else 0)


def test_input_set_rotation_outruns_the_infinity_cache():
    from mhc_hyper_connection_pre_amd.tune import set_count
    for T, n, D in ((2048, 4, 7168), (1024, 4, 4096), (16384, 4, 7168), (32, 4, 5120)):
        k = set_count(T, n, D, 2)
        per_set = T * (2 * n + 2) * D * 2
        assert 2 <= k <= 8
        # the other sets move at least twice the 256 MB cache, unless the cap of 8 applies
        assert (k - 1) * per_set >= 2 * 256 * 10 ** 6 or k == 8
    assert set_count(2048, 4, 7168, 2) == 3
