"""Every planted mistake must trip at least one pin of the oracle.

Each mutant is a copy of ``oracle/gdn_oracle.c`` with one plausible mistake
written in by a text patch (gate on the wrong term, erase sign, exclusive
output, transposed write, gate index shifted, write strength ignored),
compiled into the test's temporary directory; the pins of
``tests/oracle_pins.py`` must reject every one of them.  The oracle's own
source carries no mistake.  Runs on the CPU only.
"""
import pytest

import oracle
from oracle.build import SRC, build_oracle
from tests import oracle_pins

UPDATE = "S[i * dk + j] = a * (s - b * u[i] * kt[j]) + e * vt[i] * kt[j];"
OUT_STORE = "            ot[i] = acc;\n"
EXCLUSIVE_OUT = """        for (int64_t i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int64_t j = 0; j < dk; ++j) acc += S[i * dk + j] * qt[j];
            O[t * dv + i] = acc;
        }
"""

# name -> list of (text in the clean source, replacement); each text must
# occur exactly once
MUTANTS = {
    "gate moved from the erased state to the write": [
        (UPDATE, "S[i * dk + j] = (s - b * u[i] * kt[j]) + a * e * vt[i] * kt[j];")],
    "erase sign flipped": [
        (UPDATE, "S[i * dk + j] = a * (s + b * u[i] * kt[j]) + e * vt[i] * kt[j];")],
    "exclusive output (state before token t)": [
        ("        /* u = S k_t */\n", EXCLUSIVE_OUT + "        /* u = S k_t */\n"),
        (OUT_STORE, "            (void)acc;\n")],
    "write outer product transposed": [
        (UPDATE, "S[i * dk + j] = a * (s - b * u[i] * kt[j]) + e * vt[j % dv] * kt[i % dk];")],
    "gate applied to the write too": [
        (UPDATE, "S[i * dk + j] = a * (s - b * u[i] * kt[j] + e * vt[i] * kt[j]);")],
    "gate index shifted by one token": [
        ("double a = alpha ? alpha[t] : 1.0;",
         "double a = alpha ? (t > 0 ? alpha[t - 1] : 1.0) : 1.0;")],
    "write strength forced to one": [
        ("double e = eta ? eta[t] : beta[t];", "double e = 1.0; (void)eta;")],
}


def mutant_source(patches) -> str:
    src = open(SRC).read()
    for old, new in patches:
        assert src.count(old) == 1, f"patch target not found once: {old!r}"
        src = src.replace(old, new)
    return src


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    src = tmp_path / "gdn_oracle_mutant.c"
    src.write_text(mutant_source(MUTANTS[name]))
    lib = oracle.load(path=build_oracle(src=str(src), out=str(tmp_path / "libmutant.so")))

    def orc(q, k, v, alpha, beta, S0=None, eta=None):
        return oracle.recurrent(q, k, v, alpha, beta, S0=S0, eta=eta, lib=lib)

    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin caught the mutant: {name}"


def test_clean_source_passes_every_pin():
    for pin in oracle_pins.ALL_PINS:
        pin(lambda *a, **kw: oracle.recurrent(*a, **kw))
