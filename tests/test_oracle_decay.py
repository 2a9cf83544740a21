"""CPU tests pinning the oracle's decay-gated forward, final state and decode step (no
GPU), and checking that the pins catch mistakes planted in a copy of the forward."""
import numpy as np
import pytest

from oracle import kata_oracle as O
from tests import oracle_decay_pins as pins


@pytest.mark.parametrize("name", sorted(pins.PINS))
def test_decay_pin(name):
    fn, bound = pins.PINS[name]
    r = fn(O.forward_decay_quadratic)
    assert r <= bound, f"pin {name}: residual {r} > {bound}"


def test_decay_final_state_pin():
    assert pins.pin_decay_final_state(O.final_state_decay) <= 1e-12


def test_decay_decode_pin():
    assert pins.pin_decay_decode_step() <= 1e-12


def _mutant(kind):
    def fwd(q, k, v, P, lam, S0=None, z0=None):
        B, H, T, _ = q.shape
        y = np.zeros((B, H, T, v.shape[-1]))
        m = np.tril(np.ones((T, T), dtype=bool))
        for b in range(B):
            for h in range(H):
                u = q[b, h] @ P[h].T
                w = k[b, h] @ P[h].T
                Lam = np.cumsum(lam[b, h])
                if kind == "exclusive_cumsum":
                    Lam = Lam - lam[b, h]
                    Lam = np.concatenate([[0.0], np.cumsum(lam[b, h])[:-1]])
                diff = Lam[:, None] - Lam[None, :]
                if kind == "current_decayed":
                    diff = diff + lam[b, h][:, None]
                if kind == "sign":
                    diff = -diff
                dec = np.exp(np.where(m, diff, 0.0)) * m
                a = (u @ w.T) ** 2
                num = (a * dec) @ v[b, h]
                den = (a * (m if kind == "numerator_only" else dec)).sum(1)
                if S0 is not None:
                    f = O.feature_full(u)
                    fs = f * (1.0 if kind == "state_undecayed" else np.exp(Lam)[:, None])
                    num = num + fs @ S0[b, h]
                    den = den + fs @ z0[b, h]
                y[b, h] = num / den[:, None]
        return y
    return fwd


MUTANTS = ["current_decayed", "sign", "numerator_only", "state_undecayed", "exclusive_cumsum"]


def test_decay_reference_mutant_is_clean():
    assert pins.failing_pins(_mutant("none")) == []


@pytest.mark.parametrize("kind", MUTANTS)
def test_decay_pins_catch_mutant(kind):
    assert pins.failing_pins(_mutant(kind)), f"no pin caught {kind}"
