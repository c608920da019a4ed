"""Writes tests/golden/workload_facts.json from the oracle's position functions.

Run from the repository root: python tests/golden/make_golden.py
Calls only oracle/ (group_size, alias) and plain integer counting; the
stored numbers are checked against closed forms in tests/test_golden.py.
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402
from oracle.bifocal_ref import alias, group_size  # noqa: E402


def window_pairs(L, w0):
    # number of (i, j) with 0 <= i - j < w0, j >= 0, i < L
    return sum(min(i + 1, w0) for i in range(L))


def main():
    facts = {}
    for name, w in workloads.WORKLOADS.items():
        lens = list(w.seqlens) if w.kind == "prefill" else [w.cache_len]
        seqs = []
        for L in lens:
            G = group_size(L, w.w_pretrained)
            seqs.append({
                "L": L, "G": G, "f_last": int(alias(L - 1, G)),
                "causal_pairs": L * (L + 1) // 2,
                "window_pairs": window_pairs(L, w.w0),
            })
        facts[name] = {
            "cite": "G = max(1, ceil(L / w_pretrained)) and f(x) = floor(x / G): Jet-Long "
                    "technical summary (gist.science), Methodology section 1",
            "w0": w.w0, "w_pretrained": w.w_pretrained, "Hq": w.Hq, "D": w.D,
            "sequences": seqs,
        }
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "workload_facts.json")
    with open(out, "w") as fh:
        json.dump(facts, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print("wrote", out)


if __name__ == "__main__":
    main()
