"""Planted mistakes in the oracle must each be caught by at least one pin.

Each mutation is a compile-time switch in oracle.c (ORACLE_MUTATION=n) that
introduces one plausible slip: interleaved instead of contiguous GQA groups,
top-left instead of bottom-right causal alignment, RoPE rotating the wrong way,
K used in place of V, the scale dropped, a base-2 log in the LSE; in the
backward, the D term, dK's scale, the inverse rotation, or the group sum; the
additive mask scaled with the scores or read transposed; fp16 decoded with a
wrong exponent bias or rounded without its subnormal range.  The mutants
are built into a temporary directory; the product oracle is untouched.
"""
import os

import pytest

import oracle
from oracle import build as obuild
from oracle_pins import ALL_PINS

MUTATIONS = {
    1: "gqa interleaved groups",
    2: "causal top-left alignment",
    3: "rope wrong direction",
    4: "K used as V",
    5: "scale dropped",
    6: "base-2 log in LSE",
    7: "backward without the rowsum(dO o O) term",
    8: "backward without the scale on dK",
    9: "backward without the inverse rotation",
    10: "backward dK/dV from one query head of a group",
    11: "additive mask multiplied by the scale",
    12: "additive mask read transposed",
    13: "fp16 exponent bias 14",
    14: "fp16 rounding without its subnormal range",
}


@pytest.mark.parametrize("mut", sorted(MUTATIONS), ids=[MUTATIONS[m] for m in sorted(MUTATIONS)])
def test_mutation_is_caught(mut, tmp_path):
    path = obuild.build(out=os.path.join(tmp_path, f"liboracle_mut{mut}.so"),
                        defines=(f"ORACLE_MUTATION={mut}",))
    lib = oracle.load(path)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"mutation '{MUTATIONS[mut]}' passed every pin"
