"""CPU tests pinning the oracle's backward (gradients of the causal KATA forward) to
finite differences of the pinned forward, closed forms and invariants, and checking
that those pins catch plausible mistakes planted in a copy of it (no GPU)."""
import numpy as np
import pytest

from oracle import kata_oracle as O
from tests import oracle_bwd_pins as pins


@pytest.mark.parametrize("name", sorted(pins.PINS))
def test_bwd_pin(name):
    fn, bound = pins.PINS[name]
    r = fn(O.backward_quadratic)
    assert r <= bound, f"pin {name}: residual {r} > {bound}"


def _mutant(kind):
    """The chain rule of the forward with one planted mistake (``none``: no mistake)."""
    def bwd(q, k, v, P, gy, S0=None, z0=None, gST=None, gzT=None):
        q = np.asarray(q, dtype=np.float64); k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64); P = np.asarray(P, dtype=np.float64)
        B, H, T, d = q.shape
        dv = v.shape[-1]
        p = P.shape[1]
        pp = p * p
        out = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros_like(P),
               np.zeros((B, H, pp, dv)), np.zeros((B, H, pp))]
        mask = np.tril(np.ones((T, T)), -1 if kind == "strict_mask" else 0) > 0
        for b in range(B):
            for h in range(H):
                s0 = np.zeros((pp, dv)) if S0 is None else S0[b, h]
                zz = np.zeros(pp) if z0 is None else z0[b, h]
                gs = np.zeros((pp, dv)) if gST is None else gST[b, h]
                gz = np.zeros(pp) if gzT is None else gzT[b, h]
                u = q[b, h] @ P[h].T
                w = k[b, h] @ P[h].T
                fu = np.einsum("ti,tj->tij", u, u).reshape(T, pp)
                fw = np.einsum("ti,tj->tij", w, w).reshape(T, pp)
                X = u @ w.T
                a = np.where(mask, X * X, 0.0)
                num = a @ v[b, h] + fu @ s0
                den = a.sum(1) + fu @ zz
                y = num / den[:, None]
                gnum = gy[b, h] / den[:, None]
                gden = -np.sum(gy[b, h] * y, axis=1) / den
                if kind == "no_gden":
                    gden = 0 * gden
                if kind == "gden_sign":
                    gden = -gden
                ga = np.where(mask, gnum @ v[b, h].T + gden[:, None], 0.0)
                gX = (1.0 if kind == "no_factor2" else 2.0) * X * ga
                du = gX @ (u if kind == "u_for_w" else w)
                dw = (gX if kind == "transposed_gX" else gX.T) @ u
                for t in range(T):
                    M = (s0 @ gnum[t] + zz * gden[t]).reshape(p, p)
                    du[t] += (M if kind == "S0_unsym" else M + M.T) @ u[t]
                    N = (gs @ v[b, h, t] + gz).reshape(p, p)
                    dw[t] += (N + N.T) @ w[t] if kind != "gST_dropped" else 0.0
                out[2][b, h] = (a @ gnum if kind == "dv_untransposed" else a.T @ gnum) + fw @ gs
                out[0][b, h] = du @ P[h]
                out[1][b, h] = dw @ P[h]
                out[3][h] += du.T @ q[b, h] + (0.0 if kind == "dP_q_only" else dw.T @ k[b, h])
                out[4][b, h] = (0.0 if kind == "dS0_no_gST" else gs) + fu.T @ gnum
                out[5][b, h] = gz + fu.T @ gden
        return tuple(out)
    return bwd


MUTANTS = ["no_gden", "gden_sign", "no_factor2", "u_for_w", "transposed_gX", "strict_mask", "S0_unsym",
           "gST_dropped", "dv_untransposed", "dP_q_only", "dS0_no_gST"]


def test_bwd_reference_mutant_is_clean():
    assert pins.failing_pins(_mutant("none")) == []


@pytest.mark.parametrize("kind", MUTANTS)
def test_bwd_pins_catch_mutant(kind):
    assert pins.failing_pins(_mutant(kind)), f"no pin caught mutant {kind}"


def test_bwd_zero_denominator_rows():
    """A query row with u_t = 0 has den_t = 0 and y_t = 0 (constant): its gradients are
    0 and it adds nothing to the others (the reading for an empty weight row)."""
    c = pins.bwd_case(9, T=8, state=False)
    c["q"][:, :, 3] = 0.0
    dq, dk, dv, dP, _, _ = O.backward_quadratic(c["q"], c["k"], c["v"], c["P"], c["gy"])
    assert np.all(dq[:, :, 3] == 0)
    c2 = dict(c)
    c2["gy"] = c["gy"].copy()
    c2["gy"][:, :, 3] = 123.0   # the gradient of a constant output is ignored
    g2 = O.backward_quadratic(c2["q"], c2["k"], c2["v"], c2["P"], c2["gy"])
    assert np.array_equal(g2[1], dk) and np.array_equal(g2[2], dv)
