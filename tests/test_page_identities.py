"""Byte identities that pin the expert container layout to figures the pages
print (CPU only).  The fixture file names the page and section of each."""
import json
import os

import gen


def test_page_identities(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "page_identities.json")))
    H, I = g["shape"]["hidden"], g["shape"]["inter"]
    eb = gen.expert_bytes(gen.I4, H, I)
    code_bytes = eb["gate_up"] + eb["down"]
    for c in g["checks"]:
        if "expected_bytes" in c and "cold token" not in c["what"]:
            assert eb["total"] == c["expected_bytes"], c
            assert abs(eb["total"] / c["approx"] - 1) <= c["rel_tol"], c
        elif "expected_fraction" in c:
            frac = eb["scales"] / code_bytes
            assert abs(frac - c["expected_fraction"]) < 5e-6, c
            assert abs(frac - c["approx"]) <= c["abs_tol"], c
        else:
            tok = 75 * 8 * eb["total"]
            assert tok == c["expected_bytes"], c
            assert abs(tok / c["approx"] - 1) <= c["rel_tol"], c
    # the int2 variant of the same expert
    assert gen.expert_bytes(gen.I2, H, I)["total"] == 9478144
