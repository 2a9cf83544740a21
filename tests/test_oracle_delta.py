"""CPU tests pinning the oracle's DeltaKATA recurrence and decode step (no GPU), and
checking that the pins catch mistakes planted in a copy of the recurrence."""
import numpy as np
import pytest

from oracle import kata_oracle as O
from tests import oracle_delta_pins as pins


@pytest.mark.parametrize("name", sorted(pins.PINS))
def test_delta_pin(name):
    fn, bound = pins.PINS[name]
    r = fn(O.delta_recurrence)
    assert r <= bound, f"pin {name}: residual {r} > {bound}"


def test_unit_feature_pin():
    assert pins.pin_unit_feature() <= 1e-12


def test_delta_decode_pin():
    assert pins.pin_decode_is_recurrence_step() <= 1e-12


def _mutant(kind):
    def rec(q, k, v, P, beta, S0=None):
        B, H, T, _ = q.shape
        dv = v.shape[-1]
        pp = P.shape[1] ** 2
        y = np.zeros((B, H, T, dv))
        ST = np.zeros((B, H, pp, dv))
        for b in range(B):
            for h in range(H):
                S = np.zeros((pp, dv)) if S0 is None else np.array(S0[b, h])
                feat = O.feature_full if kind == "unnormalised" else O.feature_unit
                fq = feat(q[b, h] @ P[h].T)
                fk = feat(k[b, h] @ P[h].T)
                for t in range(T):
                    e = v[b, h, t] - (0 if kind == "no_correction" else S.T @ fk[t])
                    bt = 1.0 if kind == "beta_ignored" else beta[b, h, t]
                    Sn = S + bt * np.outer(fk[t], e)
                    y[b, h, t] = (S if kind == "readout_before" else Sn).T @ fq[t]
                    S = Sn
                ST[b, h] = S
        return y, ST
    return rec


MUTANTS = ["unnormalised", "no_correction", "beta_ignored", "readout_before"]


def test_delta_reference_mutant_is_clean():
    assert pins.failing_pins(_mutant("none")) == []


@pytest.mark.parametrize("kind", MUTANTS)
def test_delta_pins_catch_mutant(kind):
    assert pins.failing_pins(_mutant(kind)), f"no pin caught {kind}"
