"""Stored fixtures: the pages' LoRA arguments, and the oracle's codebook as written by
tests/golden/make_golden.py (a regression guard on the oracle itself)."""
import json
import os

import numpy as np

from oracle import nf4

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_codebook_fixture_unchanged():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "nf4_codebook_f32.txt")) if not l.startswith("#")]
    bits = np.array([int(r[1], 16) for r in rows], dtype=np.uint32)
    assert np.array_equal(bits, nf4.codebook_f32().view(np.uint32))


def test_page_lora_args_give_exact_scales():
    cases = json.load(open(os.path.join(GOLDEN, "page_lora_args.json")))["cases"]
    for c in cases:
        assert c["lora_dropout"] == 0  # the op has no dropout
        s = np.float32(c["lora_alpha"]) / np.float32(c["r"])
        assert float(s) == c["lora_alpha"] / c["r"]  # alpha/r exact in float32 for the pages' values
