"""Pins of the oracle's KATA-Mg and KATA-Sigma-g functions (several PSD factors,
concatenated or summed) against the pinned one-factor oracle, token loops, closed forms
and invariances that tell the two variants apart."""
from __future__ import annotations

import numpy as np

from oracle import kata_oracle as O


def fcase(seed, B=1, H=2, T=24, d=6, p=4, dv=3, G=2):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, H, T, d))
    k = r.standard_normal((B, H, T, d))
    v = r.standard_normal((B, H, T, dv))
    P = r.standard_normal((H, G, p, d)) / np.sqrt(d)
    return q, k, v, P


def rel(a, b):
    n = np.linalg.norm(b)
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / (n if n > 0 else 1.0))


def rand_orth(r, n):
    Q, R = np.linalg.qr(r.standard_normal((n, n)))
    return Q * np.sign(np.diag(R))


# ---- pins that take the forward under test, fwd(q, k, v, P, S0=None, z0=None) -------

def pin_one_factor_is_kata(fwd):
    """g = 1 is KATA itself (the pinned one-factor oracle)."""
    q, k, v, P = fcase(1, G=1)
    return rel(fwd(q, k, v, P), O.forward_quadratic(q, k, v, P[:, 0]))


def pin_mg_loop(fwd):
    q, k, v, P = fcase(2, G=3)
    return rel(fwd(q, k, v, P), O.recurrence_mg(q, k, v, P))


def pin_sg_loop(fwd):
    q, k, v, P = fcase(3, G=3)
    return rel(fwd(q, k, v, P), O.recurrence_sg(q, k, v, P))


def pin_mg_zero_factor(fwd):
    """Mg: a zero second factor adds nothing, y = KATA with the first factor."""
    q, k, v, P = fcase(4)
    P[:, 1] = 0.0
    return rel(fwd(q, k, v, P), O.forward_quadratic(q, k, v, P[:, 0]))


def pin_sg_zero_factor(fwd):
    """Sigma-g: a zero second factor adds nothing either."""
    q, k, v, P = fcase(5)
    P[:, 1] = 0.0
    return rel(fwd(q, k, v, P), O.forward_quadratic(q, k, v, P[:, 0]))


def pin_mg_per_factor_rotation(fwd):
    """Mg: rotating each factor's projection by its own orthogonal O_i leaves every
    (u_i . w_i), hence y, unchanged."""
    q, k, v, P = fcase(6)
    r = np.random.default_rng(60)
    P2 = P.copy()
    for h in range(P.shape[0]):
        for i in range(P.shape[1]):
            P2[h, i] = rand_orth(r, P.shape[2]) @ P[h, i]
    return rel(fwd(q, k, v, P2), fwd(q, k, v, P))


def pin_sg_factor_mixing(fwd):
    """Sigma-g: the feature sum_i u_i u_i^T = U U^T is unchanged when the factors are
    mixed by an orthogonal g x g matrix (P'_i = sum_j R_ji P_j), hence so is y."""
    q, k, v, P = fcase(7, G=3)
    r = np.random.default_rng(70)
    P2 = P.copy()
    for h in range(P.shape[0]):
        R = rand_orth(r, P.shape[1])
        P2[h] = np.einsum("ji,jab->iab", R, P[h])
    return rel(fwd(q, k, v, P2), fwd(q, k, v, P))


def pin_sg_weights_closed_form(fwd):
    """Sigma-g at p = d = 1 with two factors: u_i = c_i q, w_j = c_j k, so
    a_ts = (sum_i c_i^2)^2 (q_t k_s)^2: y = the one-factor KATA with P = 1."""
    q, k, v, _ = fcase(8, d=1, p=1)
    P = np.array([[[[0.7]], [[-1.3]]]] * 2)
    return rel(fwd(q, k, v, P), O.forward_quadratic(q, k, v, np.ones((2, 1, 1))))


def pin_mg_state_resume(fwd, final):
    """Resume: the second half from the first half's state = the whole sequence."""
    q, k, v, P = fcase(9, T=30)
    m = 13
    S0, z0 = final(k[:, :, :m], v[:, :, :m], P)
    y2 = fwd(q[:, :, m:], k[:, :, m:], v[:, :, m:], P, S0, z0)
    return rel(y2, fwd(q, k, v, P)[:, :, m:])


PINS_MG = {
    "one_factor_is_kata": (pin_one_factor_is_kata, 1e-12),
    "mg_loop": (pin_mg_loop, 1e-12),
    "mg_zero_factor": (pin_mg_zero_factor, 1e-12),
    "mg_per_factor_rotation": (pin_mg_per_factor_rotation, 1e-12),
    "mg_resume": (lambda f: pin_mg_state_resume(f, O.final_state_mg), 1e-12),
}
PINS_SG = {
    "one_factor_is_kata": (pin_one_factor_is_kata, 1e-12),
    "sg_loop": (pin_sg_loop, 1e-12),
    "sg_zero_factor": (pin_sg_zero_factor, 1e-12),
    "sg_factor_mixing": (pin_sg_factor_mixing, 1e-12),
    "sg_weights_closed_form": (pin_sg_weights_closed_form, 1e-12),
    "sg_resume": (lambda f: pin_mg_state_resume(f, O.final_state_sg), 1e-12),
}


def failing(pins, fwd):
    out = []
    for name, (fn, bound) in pins.items():
        try:
            r = fn(fwd)
        except Exception:
            out.append(name)
            continue
        if not (r <= bound):
            out.append(name)
    return out


def pin_final_states():
    """Final states against explicit per-token outer products."""
    _, k, v, P = fcase(10, G=2, T=7)
    Sm, zm = O.final_state_mg(k, v, P)
    Ss, zs = O.final_state_sg(k, v, P)
    res = []
    for b in range(k.shape[0]):
        for h in range(k.shape[1]):
            Sm_r = np.zeros_like(Sm[b, h]); Ss_r = np.zeros_like(Ss[b, h])
            zm_r = np.zeros_like(zm[b, h]); zs_r = np.zeros_like(zs[b, h])
            for t in range(k.shape[2]):
                ws = [P[h, i] @ k[b, h, t] for i in range(P.shape[1])]
                fcat = np.concatenate([np.outer(w, w).ravel() for w in ws])
                fsum = sum(np.outer(w, w) for w in ws).ravel()
                Sm_r += np.outer(fcat, v[b, h, t]); Ss_r += np.outer(fsum, v[b, h, t])
                zm_r += fcat; zs_r += fsum
            res += [rel(Sm[b, h], Sm_r), rel(Ss[b, h], Ss_r), rel(zm[b, h], zm_r), rel(zs[b, h], zs_r)]
    return max(res)


def pin_decode_steps(mode):
    """Decode steps from the final state of a prefix reproduce the forward over the whole
    sequence at the decoded tokens (the state is the whole history)."""
    q, k, v, P = fcase(12, B=2, T=12)
    m = 7
    fin = O.final_state_mg if mode == "concat" else O.final_state_sg
    fwd = O.forward_mg_quadratic if mode == "concat" else O.forward_sg_quadratic
    S, z = fin(k[:, :, :m], v[:, :, :m], P)
    yfull = fwd(q, k, v, P)
    worst = 0.0
    for t in range(m, q.shape[2]):
        yt, S, z = O.decode_factors_reference(S, z, q[:, :, t], k[:, :, t], v[:, :, t], P, mode)
        worst = max(worst, rel(yt, yfull[:, :, t]))
    Sf, zf = fin(k, v, P)
    return max(worst, rel(S, Sf), rel(z, zf))
