"""Pins of the oracle's DeltaKATA recurrence (``delta_recurrence``,
``delta_decode_reference``) against closed forms of the delta rule and an independent
chunked (WY) algorithm.  Reading: DeltaNet's delta rule with KATA's feature normalised
to unit norm, phi^(x) = vec(u u^T)/|u|^2, and the readout y_t = S_t^T phi^(q_t)."""
from __future__ import annotations

import numpy as np

from oracle import kata_oracle as O


def dcase(seed, B=1, H=2, T=20, d=6, p=4, dv=3):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, H, T, d))
    k = r.standard_normal((B, H, T, d))
    v = r.standard_normal((B, H, T, dv))
    P = r.standard_normal((H, p, d)) / np.sqrt(d)
    beta = r.uniform(0.2, 1.0, (B, H, T))
    return q, k, v, P, beta


def rel(a, b):
    n = np.linalg.norm(b)
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / (n if n > 0 else 1.0))


def pin_unit_feature():
    """|phi^(u)| = 1 and phi^(u).phi^(w) = cos^2(u, w)."""
    r = np.random.default_rng(1)
    u, w = r.standard_normal((30, 5)), r.standard_normal((30, 5))
    fu, fw = O.feature_unit(u), O.feature_unit(w)
    c2 = (np.sum(u * w, 1) ** 2) / (np.sum(u * u, 1) * np.sum(w * w, 1))
    return max(float(np.max(np.abs(np.linalg.norm(fu, axis=1) - 1))), float(np.max(np.abs(np.sum(fu * fw, 1) - c2))))


def pin_exact_overwrite(rec):
    """beta = 1, a key written twice: querying it returns the latest value (the delta rule
    replaces the binding), whatever other keys were written in between if they are
    orthogonal to it in feature space."""
    p, d, dv = 4, 4, 3
    P = np.eye(4)[None]
    e = np.eye(4)
    k = np.stack([e[0], e[1], e[0], e[2]])[None, None]          # key e0 written twice
    v = np.array([[1.0, 2, 3], [4, 5, 6], [7, 8, 9], [1, 1, 1]])[None, None]
    q = np.stack([e[0], e[1], e[0], e[0]])[None, None]
    y, _ = rec(q, k, v, P, np.ones((1, 1, 4)))
    return float(max(np.max(np.abs(y[0, 0, 2] - v[0, 0, 2])), np.max(np.abs(y[0, 0, 3] - v[0, 0, 2])),
                     np.max(np.abs(y[0, 0, 1] - v[0, 0, 1]))))


def pin_orthogonal_keys_sum(rec):
    """Keys with mutually orthogonal features (orthogonal projected keys): no correction
    acts, S_T = sum_t beta_t phi^(k_t) v_t^T (plain linear-attention sum)."""
    r = np.random.default_rng(3)
    Q, _ = np.linalg.qr(r.standard_normal((4, 4)))
    P = np.eye(4)[None]
    k = (Q.T * r.uniform(0.5, 2.0, 4)[:, None])[None, None]       # 4 orthogonal keys
    v = r.standard_normal((1, 1, 4, 3))
    q = r.standard_normal((1, 1, 4, 4))
    beta = r.uniform(0.1, 1.0, (1, 1, 4))
    _, ST = rec(q, k, v, P, beta)
    fk = O.feature_unit(k[0, 0])
    return rel(ST[0, 0], (fk * beta[0, 0, :, None]).T @ v[0, 0])


def pin_beta_zero(rec):
    """beta = 0: nothing is written; y_t = S0^T phi^(q_t)."""
    q, k, v, P, beta = dcase(4)
    S0 = np.random.default_rng(40).standard_normal((1, 2, 16, 3))
    y, ST = rec(q, k, v, P, 0 * beta, S0)
    fq = O.feature_unit(np.einsum("hpd,bhtd->bhtp", P, q))
    return max(rel(y, np.einsum("bhtf,bhfc->bhtc", fq, S0)), rel(ST, S0))


def chunked_wy(q, k, v, P, beta, C):
    """The chunked delta rule (WY form): per chunk, with the keys' unit features K (C x D),
    A = I + tril(diag(beta) K K^T, -1), W = A^{-1} diag(beta) K, U = A^{-1} diag(beta) V;
    then E = U - W S, Y = Q S + tril(Q K^T) E, S <- S + K^T E."""
    B, H, T, d = q.shape
    p = P.shape[1]
    dv = v.shape[-1]
    y = np.zeros((B, H, T, dv))
    ST = np.zeros((B, H, p * p, dv))
    for b in range(B):
        for h in range(H):
            Qf = O.feature_unit(q[b, h] @ P[h].T)
            Kf = O.feature_unit(k[b, h] @ P[h].T)
            S = np.zeros((p * p, dv))
            for s0 in range(0, T, C):
                e = min(s0 + C, T)
                K, Qc, V, bt = Kf[s0:e], Qf[s0:e], v[b, h, s0:e], beta[b, h, s0:e]
                n = e - s0
                A = np.eye(n) + np.tril(bt[:, None] * (K @ K.T), -1)
                W = np.linalg.solve(A, bt[:, None] * K)
                U = np.linalg.solve(A, bt[:, None] * V)
                E = U - W @ S
                y[b, h, s0:e] = Qc @ S + np.tril(Qc @ K.T) @ E
                S = S + K.T @ E
            ST[b, h] = S
    return y, ST


def pin_chunked_wy(rec):
    q, k, v, P, beta = dcase(5, T=30)
    y, ST = rec(q, k, v, P, beta)
    res = []
    for C in (1, 4, 7, 30):
        yc, Sc = chunked_wy(q, k, v, P, beta, C)
        res += [rel(yc, y), rel(Sc, ST)]
    return max(res)


def pin_decode_is_recurrence_step():
    q, k, v, P, beta = dcase(6, B=3, T=5)
    y, ST = O.delta_recurrence(q, k, v, P, beta)
    S = np.zeros((3, 2, 16, 3))
    worst = 0.0
    for t in range(5):
        yt, S = O.delta_decode_reference(S, q[:, :, t], k[:, :, t], v[:, :, t], P, beta[:, :, t])
        worst = max(worst, rel(yt, y[:, :, t]))
    return max(worst, rel(S, ST))


PINS = {
    "exact_overwrite": (pin_exact_overwrite, 1e-12),
    "orthogonal_keys_sum": (pin_orthogonal_keys_sum, 1e-12),
    "beta_zero": (pin_beta_zero, 1e-12),
    "chunked_wy": (pin_chunked_wy, 1e-10),
}


def failing_pins(rec):
    out = []
    for name, (fn, bound) in PINS.items():
        try:
            r = fn(rec)
        except Exception:
            out.append(name)
            continue
        if not (r <= bound):
            out.append(name)
    return out
