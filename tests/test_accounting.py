"""Pins for the work accounting that the benchmark uses (no GPU).

Checked against brute-force enumeration of visible pairs and against the values the
DualKV paper prints (tests/golden/paper_closed_forms.json: Appendix C.2's ideal
speedups, Table 6's byte counts and the rho values of §2.2 / Table 7).
"""
import json
import os

import pytest

from shared_prompt_exact_dkv_amd import accounting as acc

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                     "paper_closed_forms.json")))


def _brute(P, lens, wl):
    def vis(t, j):
        return j <= t and (wl < 0 or j >= t - wl)
    call1 = sum(vis(t, j) for t in range(P) for j in range(P))
    call2 = sum(vis(P + r, j) for R in lens for r in range(R) for j in range(P + R))
    ncopy = sum(vis(t, j) for R in lens for t in range(P + R) for j in range(P + R))
    return call1, call2, ncopy


@pytest.mark.parametrize("P,lens,wl", [(0, [3, 4], -1), (5, [1, 0, 7], -1), (9, [4, 6], 2),
                                      (6, [3], 0), (13, [5, 9, 2], 20), (7, [12], 5)])
def test_pair_counts_match_brute_force(P, lens, wl):
    c1, c2, nc = _brute(P, lens, wl)
    assert acc.pairs_call1(P, wl) == c1
    assert acc.pairs_call2(P, lens, wl) == c2
    assert acc.pairs_ncopy(P, lens, wl) == nc


def test_ideal_speedup_matches_printed_eq34():
    for c in GOLDEN["ideal_attention_speedup"]["cases"]:
        s = acc.ideal_speedup(c["P"], [c["R"]] * c["N"])
        assert round(s, 2) == pytest.approx(c["printed"], abs=1e-9), c


def test_token_reduction_matches_printed_rho():
    for c in GOLDEN["token_reduction_rho"]["cases"]:
        assert round(acc.token_reduction(c["P"], c["N"], c["R"]), 1) == pytest.approx(c["printed"])


def test_table6_bytes_match_printed():
    g = GOLDEN["memory_savings_table6"]
    b = acc.prompt_bytes_saved(g["N"], g["P"], g["H"], g["Hk"], g["d"], g["elem_bytes"])
    for k, mb in g["printed_MB"].items():
        # the page rounds to whole MB (1e6 B), apart from the 4-byte LSE row, which
        # matches in MiB; all within one unit of the exact byte count
        assert abs(b[k] / 1e6 - mb) <= 1.0 or abs(b[k] / 2**20 - mb) <= 1.0, (k, b[k])


def test_useful_flops():
    assert acc.useful_flops(10, 32, 128) == 14 * 128 * 32 * 10
    assert acc.useful_flops(10, 32, 128, bwd=False) == 4 * 128 * 32 * 10
