"""The CPU oracle against its pins (no GPU).  See tests/pins.py for what pins each part."""
import pytest

import oracle
from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)


MUTANTS = {
    1: "forward reads X through the row index",
    2: "forward drops the last term",
    3: "input gradient has the wrong sign",
    4: "value gradient uses transposed operands",
    5: "regrow position map is off by one",
    6: "prune removes the largest magnitudes",
    7: "regrow ignores occupied positions",
    8: "gradient regrow breaks score ties towards the larger position",
    9: "gradient regrow ranks the signed sum instead of its magnitude",
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: f"mutant{m}")
def test_pins_reject_planted_mistake(tmp_path, mutant):
    """Each plausible mistake planted in the oracle (on the CPU) must fail at least one pin."""
    path = oracle.build(mutant=mutant, out_dir=str(tmp_path))
    orc = oracle.Oracle(path)
    assert orc.mutant == mutant
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {mutant}: {MUTANTS[mutant]}"
