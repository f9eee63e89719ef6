"""The pins catch plausible mistakes: each planted mistake (a build of the
oracle with ORACLE_MUTANT=n, on the CPU) must make at least one pin fail."""
import os

import pytest

import oracle
import oracle_pins

MUTANTS = {
    1: "logits without the 1/sqrt(d) scale",
    2: "Mask_0 also zeroes the diagonal",
    3: "key-query conv looks at later queries",
    4: "key offset sign flipped",
    5: "kernel key axis reversed",
    6: "head-mix matrix transposed",
    7: "softmax rows not normalised",
    8: "head gate used without its sigmoid",
    9: "exact indicator taken against the input row",
    10: "3D kernel with output and source head swapped",
    11: "Mask_0 after the post-softmax convolution dropped in the layer",
}


@pytest.mark.parametrize("n", sorted(MUTANTS), ids=lambda n: f"mutant{n}")
def test_mutant_is_caught(n, tmp_path):
    so = oracle.build(out=os.path.join(str(tmp_path), f"libmta_oracle_m{n}.so"), mutant=n)
    lib = oracle.load(so)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
            break
    assert caught, f"no pin caught mutant {n}: {MUTANTS[n]}"
