"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that the
pins catch every one of them.  This guards the pins themselves: a pin set that
lets a dropped term, a wrong index or a transposed operand through is too weak.
"""
import numpy as np
import pytest

from oracle import kata_oracle as O
from tests import oracle_pins as pins


def _mutant(kind):
    def fwd(q, k, v, P, S0=None, z0=None, rows=None, block=256):
        q = np.asarray(q, dtype=np.float64)
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        P = np.asarray(P, dtype=np.float64)
        B, H, T, _ = q.shape
        y = np.zeros((B, H, T, v.shape[-1]))
        for b in range(B):
            for h in range(H):
                Ph = P[h].T if kind == "transposed_P" else P[h]
                u = q[b, h] @ Ph.T
                w = k[b, h] @ Ph.T
                dot = u @ w.T
                if kind == "no_square":
                    a = np.abs(dot)
                elif kind == "raw_dot":
                    a = dot
                elif kind == "cubed":
                    a = np.abs(dot) ** 3
                elif kind == "q_for_k":
                    a = (u @ u.T) ** 2
                else:
                    a = dot ** 2
                mask = np.tril(np.ones((T, T)), -1 if kind == "strict_causal" else 0)
                if kind == "anti_causal":
                    mask = np.triu(np.ones((T, T)))
                a = a * mask
                num = a @ v[b, h]
                den = a.sum(1)
                if kind == "unnormalised":
                    den = np.ones_like(den)
                if kind == "den_off_by_one":
                    den = den + 1.0
                if kind == "v_shift":
                    num = a[:, :] @ np.roll(v[b, h], 1, axis=0)
                safe = np.where(den == 0, 1.0, den)
                y[b, h] = np.where(den[:, None] == 0, 0.0, num / safe[:, None])
        return y
    return fwd


MUTANTS = ["transposed_P", "no_square", "raw_dot", "cubed", "q_for_k", "strict_causal",
           "anti_causal", "unnormalised", "den_off_by_one", "v_shift"]


def test_reference_mutant_is_clean():
    """The mutant harness with no mutation passes every pin (it is a correct form)."""
    assert pins.failing_pins(_mutant("none")) == []


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_catch_mutant(kind):
    assert pins.failing_pins(_mutant(kind)), f"no pin caught mutant {kind}"


def _weights_mutant(kind):
    """A copy of the oracle's weights with one planted mistake."""
    def weights(q, k, P):
        u = np.asarray(q, dtype=np.float64) @ np.asarray(P, dtype=np.float64).T
        w = np.asarray(k, dtype=np.float64) @ np.asarray(P, dtype=np.float64).T
        dot = (u @ u.T) if kind == "q_for_k" else u @ w.T
        a = {"no_square": np.abs(dot), "raw_dot": dot, "cubed": np.abs(dot) ** 3}.get(kind, dot ** 2)
        if kind == "strict_causal":
            return np.tril(a, -1)
        if kind == "anti_causal":
            return np.triu(a)
        return np.tril(a)
    return weights


WEIGHT_MUTANTS = ["no_square", "raw_dot", "cubed", "q_for_k", "strict_causal", "anti_causal"]


@pytest.mark.parametrize("kind", WEIGHT_MUTANTS)
def test_weight_pins_catch_mutant(kind, monkeypatch):
    """The golden-scalar and normalised-row pins of O.weights fail on each planted mistake."""
    from tests import test_oracle_pins as tp
    monkeypatch.setattr(O, "weights", _weights_mutant(kind))
    caught = 0
    for check in (tp.test_weights_golden_scalar, tp.test_weights_normalised_rows_are_the_forward):
        try:
            with np.errstate(all="ignore"):
                check()
        except AssertionError:
            caught += 1
    assert caught, f"no weights pin caught mutant {kind}"
