"""The host planner's multi-stream split, without a GPU: the workspace query
includes the parts' layouts when a batch is split, so where the parts' tile
choices or alignment differ from the whole batch's, its size tells whether
the library splits a batch.  Each case runs in a child process, since
MUON_SPLIT is read once per process."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CASES = {
    # one launch group, 7.6e11 nominal flops: split (three parts)
    "three-parts-uneven": [(768, 3072)] * 13 + [(3072, 768)] * 5 + [(768, 768)] * 2,
    # one launch group, 1.3e12 nominal flops: split (two parts)
    "two-parts-uneven": [(2048, 2048)] * 5,
    # the GPT-2 124M set: split
    "gpt2-124m": [(768, 2304), (768, 768), (768, 3072), (3072, 768)] * 12,
    # tile-64 and tile-128 shapes: several launch groups, never split
    "several-groups": [(768, 768), (768, 2304), (3072, 768), (64, 128), (128, 64), (200, 520), (33, 17),
                       (768, 2304)] + [(768, 3072)] * 10,
    # one group but 3.6e11 nominal flops: below the split threshold
    "small": [(768, 3072)] * 9,
    # 5e11+ flops but a single matrix: nothing to split
    "one-matrix": [(4096, 4096)],
}


def _sizes(env_split):
    env = dict(os.environ)
    env.pop("MUON_SPLIT", None)
    if env_split is not None:
        env["MUON_SPLIT"] = env_split
    code = ("import json, sys; from newton_schulz_09_amd import muon; "
            "cases = json.loads(sys.argv[1]); "
            "print(json.dumps({k: muon.batched_workspace_size([tuple(s) for s in v]) for k, v in cases.items()}))")
    import json
    r = subprocess.run([sys.executable, "-c", code, json.dumps(CASES)], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    return json.loads(r.stdout.strip().splitlines()[-1])


@pytest.fixture(scope="module")
def sizes():
    return {"default": _sizes(None), "off": _sizes("0"), "two": _sizes("2"), "three": _sizes("3")}


@pytest.mark.parametrize("name", ["three-parts-uneven", "two-parts-uneven", "gpt2-124m"])
def test_large_single_group_batches_are_split(sizes, name):
    assert sizes["default"][name] != sizes["off"][name]


@pytest.mark.parametrize("name", ["several-groups", "small", "one-matrix"])
def test_other_batches_are_not_split(sizes, name):
    for mode in ("default", "two", "three"):
        assert sizes[mode][name] == sizes["off"][name], mode


def test_part_count_follows_the_elements_per_flop(sizes):
    # the 768 class takes three parts by default, the 2048 class two
    assert sizes["default"]["three-parts-uneven"] == sizes["three"]["three-parts-uneven"]
    assert sizes["default"]["gpt2-124m"] == sizes["three"]["gpt2-124m"]
    assert sizes["default"]["two-parts-uneven"] == sizes["two"]["two-parts-uneven"]
