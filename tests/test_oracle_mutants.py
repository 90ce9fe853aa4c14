"""Every planted mistake in the oracle must be caught by at least one pin.

Each mutant is oracle.c compiled with -DORACLE_MUTANT=n (one deliberate error:
swapped nibble order, silu on the wrong projection, scale bias off by one, one
scale for the whole row, ties to the higher index, gates normalised over all
experts, no gate in the combine, w2 read transposed, h left unrounded, last input
column dropped, wrong subnormal, sign bit ignored; for the MXFP8 mode: scale
exponent off by one, no saturation, sign of FP8 dropped, ties away from zero;
for the router logits: last input dropped, weight read transposed; for the
saliency: a row missing from the norm, the gate left out; for the shared
expert: block-scale index transposed, w2 read transposed)."""
import pytest

import oracle
import pins

MUTANTS = {1: "nibble order", 2: "silu on w3", 3: "scale bias 126", 4: "one scale per row",
           5: "ties to higher index", 6: "softmax over all experts", 7: "no gate",
           8: "w2 transposed", 9: "h not rounded", 10: "last column dropped",
           11: "subnormal = 1.0", 12: "sign ignored", 13: "mx8 scale exponent off by one",
           14: "fp8 not saturated", 15: "fp8 sign dropped", 16: "fp8 ties away from zero",
           17: "router last input dropped", 18: "router weight transposed",
           19: "saliency norm misses a row", 20: "saliency without the gate",
           21: "shared block scale transposed", 22: "shared w2 transposed"}


@pytest.mark.parametrize("n", sorted(MUTANTS), ids=lambda n: MUTANTS[n].replace(" ", "_"))
def test_mutant_is_caught(n, tmp_path):
    so = oracle.build(str(tmp_path / f"liboracle_mut{n}.so"), mutant=n)
    o = oracle.Oracle(so)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(o)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {n} ({MUTANTS[n]}) passes every pin"
