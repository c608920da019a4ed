"""The stored workload facts against closed forms of the pages' formulas."""
import json
import math
import os

import workloads

HERE = os.path.dirname(os.path.abspath(__file__))


def _facts():
    with open(os.path.join(HERE, "golden", "workload_facts.json")) as fh:
        return json.load(fh)


def test_facts_cover_every_workload():
    assert set(_facts()) == set(workloads.WORKLOADS)


def test_facts_match_closed_forms():
    for name, f in _facts().items():
        w0, wp = f["w0"], f["w_pretrained"]
        for s in f["sequences"]:
            L = s["L"]
            assert s["G"] == max(1, math.ceil(L / wp))
            assert s["f_last"] == (L - 1) // s["G"] <= wp - 1
            assert s["causal_pairs"] == L * (L + 1) // 2
            m = min(L, w0)
            assert s["window_pairs"] == m * (m + 1) // 2 + (L - m) * w0


def test_known_values():
    f = _facts()
    big = f["qwen3_4b_128k"]["sequences"][0]
    assert (big["G"], big["f_last"]) == (4, 32767)
    assert [s["G"] for s in f["qwen3_8b_ragged"]["sequences"]] == [4, 2]
    assert f["tiny_f32"]["sequences"][0]["G"] == 4
    assert f["qwen3_1p7b_32k_g1"]["sequences"][0]["G"] == 1
    # the boundary run ends past L = 4 * w_pretrained: G = 5
    assert f["qwen3_8b_decode_boundary"]["sequences"][0]["G"] == 5
    assert f["qwen3_8b_decode_128k"]["sequences"][0]["G"] == 4
