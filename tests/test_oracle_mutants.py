"""Every planted mistake in the oracle must trip at least one pin.

Each mutant is a copy of the oracle compiled with one plausible mistake
(gate on the wrong term, erase sign, exclusive output, transposed write, gate
index shifted, write strength ignored); the pins of ``tests/oracle_pins.py``
must reject every one of them.  Runs on the CPU only.
"""
import pytest

import oracle
from oracle.build import build_oracle
from tests import oracle_pins

MUTANTS = {
    1: "gate moved from the erased state to the write",
    2: "erase sign flipped",
    3: "exclusive output (state before token t)",
    4: "write outer product transposed",
    5: "gate applied to the write too",
    6: "gate index shifted by one token",
    7: "write strength forced to one",
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: MUTANTS[m])
def test_pins_reject_mutant(mutant, tmp_path):
    path = build_oracle(mutant=mutant, out_dir=str(tmp_path))
    lib = oracle.load(path=path)
    assert lib.gdn_oracle_mutant_id() == mutant

    def orc(q, k, v, alpha, beta, S0=None, eta=None):
        return oracle.recurrent(q, k, v, alpha, beta, S0=S0, eta=eta, lib=lib)

    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {mutant} ({MUTANTS[mutant]})"
