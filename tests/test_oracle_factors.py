"""CPU tests pinning the oracle's KATA-Mg and KATA-Sigma-g forwards and final states,
and checking that the pins catch mistakes planted in copies of them (no GPU)."""
import numpy as np
import pytest

from oracle import kata_oracle as O
from tests import oracle_factor_pins as pins


@pytest.mark.parametrize("name", sorted(pins.PINS_MG))
def test_mg_pin(name):
    fn, bound = pins.PINS_MG[name]
    r = fn(O.forward_mg_quadratic)
    assert r <= bound, f"pin {name}: residual {r} > {bound}"


@pytest.mark.parametrize("name", sorted(pins.PINS_SG))
def test_sg_pin(name):
    fn, bound = pins.PINS_SG[name]
    r = fn(O.forward_sg_quadratic)
    assert r <= bound, f"pin {name}: residual {r} > {bound}"


def test_final_states_pin():
    assert pins.pin_final_states() <= 1e-12


def test_variants_differ():
    """The two readings are different functions once g > 1 (so neither pin set is vacuous)."""
    q, k, v, P = pins.fcase(11)
    assert pins.rel(O.forward_mg_quadratic(q, k, v, P), O.forward_sg_quadratic(q, k, v, P)) > 1e-3


def _weights_mutant(kind):
    """The O(T^2) form with the score of one variant written with a planted mistake."""
    def fwd(q, k, v, P, S0=None, z0=None):
        B, H, T, _ = q.shape
        G = P.shape[1]
        y = np.zeros(v.shape)
        mask = np.tril(np.ones((T, T)), -1 if kind == "strict" else 0) > 0
        for b in range(B):
            for h in range(H):
                U = [q[b, h] @ P[h, i].T for i in range(G)]
                W = [k[b, h] @ P[h, i].T for i in range(G)]
                if kind == "square_of_sum":
                    a = sum(U[i] @ W[i].T for i in range(G)) ** 2
                elif kind in ("cross_terms", "sg_none"):
                    a = sum((U[i] @ W[j].T) ** 2 for i in range(G) for j in range(G))
                elif kind == "sg_diag_only":
                    a = sum((U[i] @ W[i].T) ** 2 for i in range(G))
                elif kind == "first_factor_keys":
                    a = sum((U[i] @ W[0].T) ** 2 for i in range(G))
                elif kind == "sg_one_sided":
                    a = sum((U[0] @ W[j].T) ** 2 for j in range(G))
                else:   # "mg_none", "strict"
                    a = sum((U[i] @ W[i].T) ** 2 for i in range(G))
                a = np.where(mask, a, 0.0)
                num, den = a @ v[b, h], a.sum(1)
                if S0 is not None:
                    if kind.startswith("sg") or kind == "cross_terms":
                        fq = sum(O.feature_full(U[i]) for i in range(G))
                    else:
                        fq = np.concatenate([O.feature_full(U[i]) for i in range(G)], axis=1)
                    num = num + fq @ S0[b, h]
                    den = den + fq @ z0[b, h]
                y[b, h] = np.where(den[:, None] != 0, num / np.where(den[:, None] != 0, den[:, None], 1), 0)
        return y
    return fwd


MG_MUTANTS = ["square_of_sum", "cross_terms", "first_factor_keys", "strict"]
SG_MUTANTS = ["sg_diag_only", "first_factor_keys", "sg_one_sided", "strict"]


def test_mutant_baselines_clean():
    assert pins.failing(pins.PINS_MG, _weights_mutant("mg_none")) == []
    assert pins.failing(pins.PINS_SG, _weights_mutant("sg_none")) == []


@pytest.mark.parametrize("kind", MG_MUTANTS)
def test_mg_pins_catch(kind):
    assert pins.failing(pins.PINS_MG, _weights_mutant(kind)), kind


@pytest.mark.parametrize("kind", SG_MUTANTS)
def test_sg_pins_catch(kind):
    assert pins.failing(pins.PINS_SG, _weights_mutant(kind)), kind


@pytest.mark.parametrize("mode", ["concat", "sum"])
def test_decode_factors_pin(mode):
    assert pins.pin_decode_steps(mode) <= 1e-12


def test_decode_factors_mode_matters():
    """The two decode modes differ once g > 1 (and the sum mode keeps the one-factor state size)."""
    q, k, v, P = pins.fcase(13, B=1, T=5)
    Sm, zm = O.final_state_mg(k, v, P)
    Ss, zs = O.final_state_sg(k, v, P)
    assert Sm.shape[2] == 2 * Ss.shape[2]
    ym, _, _ = O.decode_factors_reference(Sm, zm, q[:, :, 0], k[:, :, 0], v[:, :, 0], P, "concat")
    ys, _, _ = O.decode_factors_reference(Ss, zs, q[:, :, 0], k[:, :, 0], v[:, :, 0], P, "sum")
    assert pins.rel(ym, ys) > 1e-3
