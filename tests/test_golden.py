"""The oracle reproduces the hand-derived examples exactly."""
import numpy as np

from tests.golden import hand


def test_oracle_hand_examples(orc):
    for c in hand.cases():
        y, _ = orc.gemm(c["act"], c["qweight"], c["scales"], c["qzeros"], c["group"])
        assert np.array_equal(y, c["y"]), c["name"]
