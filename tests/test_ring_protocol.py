"""Exhaustive interleaving checks of the claim / prefetch-ring protocol (CPU only).

Pins: the configurations the kernel uses (depth 3, claims-ahead 0/1/2) must be
safe for every interleaving; configurations that are unsafe by a simple
argument must be reported as unsafe (a depth-1 ring written while a slow wave
still has to read it; depth 2 with two claims ahead), and a producer that
claims after a failure (planted in the program) must be caught.
"""

import pytest

from oracle import ring_model
from oracle.ring_model import check_ring_protocol


@pytest.mark.parametrize("q", [0, 1, 2])
@pytest.mark.parametrize("W", [2, 3, 4])
@pytest.mark.parametrize("n_valid", [0, 1, 3])
@pytest.mark.parametrize("nb", [0, 1])
def test_depth3_is_safe(q, W, n_valid, nb):
    r = check_ring_protocol(W=W, D=3, q=q, n_valid=n_valid, nb=nb)
    assert r.ok, r.violation


def test_depth1_with_prefetch_is_unsafe():
    r = check_ring_protocol(W=2, D=1, q=1, n_valid=2, nb=1)
    assert not r.ok and r.violation.startswith("R1")


def test_depth1_without_prefetch_needs_a_main_loop_barrier():
    assert check_ring_protocol(W=3, D=1, q=0, n_valid=3, nb=1).ok
    r = check_ring_protocol(W=2, D=1, q=0, n_valid=2, nb=0)
    assert not r.ok and r.violation.startswith("R1")


def test_depth2_two_ahead_is_unsafe_one_ahead_is_safe():
    r = check_ring_protocol(W=2, D=2, q=2, n_valid=3, nb=1)
    assert not r.ok and r.violation.startswith("R1")
    assert check_ring_protocol(W=3, D=2, q=1, n_valid=3, nb=1).ok


def test_claim_after_failure_is_caught(monkeypatch):
    real = ring_model.wave_program

    def buggy(w, n_valid, q, nb):
        prog = real(w, n_valid, q, nb)
        if w == 0:
            # planted bug: one more claim just before exiting
            prog.insert(len(prog) - 1, ("issue", (n_valid + 1,), ("never",)))
        return prog

    monkeypatch.setattr(ring_model, "wave_program", buggy)
    r = ring_model.check_ring_protocol(W=2, D=3, q=1, n_valid=1, nb=1)
    assert not r.ok and r.violation.startswith("R2")
