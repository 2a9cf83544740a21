"""Pins of the CPU oracle against facts the pages and the mathematics fix.

Each check takes the function under test (the oracle's ``forward_quadratic``,
or a deliberately broken copy of it in the mutation tests) and returns a
float residual; a check passes when the residual is below its bound.  None
of these retypes the oracle's formula: each compares against a closed form,
a brute-force alternative algorithm, an invariant, or a hand-derived value.

Citations: the method is "Kernelized Linear Attention: Breaking the Capacity
Wall with Symmetric Cones" (arXiv 2607.17419); [ABS] its abstract,
[TS-x] section x of the gist.science technical summary of that paper.
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rand_case(seed, B=1, H=1, T=48, d=8, p=4, dv=5):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, H, T, d))
    k = r.standard_normal((B, H, T, d))
    v = r.standard_normal((B, H, T, dv))
    P = r.standard_normal((H, p, d)) / np.sqrt(d)
    return q, k, v, P


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    n = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (n if n > 0 else 1.0))


# --- brute-force alternatives (independent algorithms, tiny sizes only) -------------------

def brute_recurrence(q, k, v, P):
    """Token-by-token state recurrence with explicit outer products, pure loops ([TS-1])."""
    B, H, T, d = q.shape
    p = P.shape[1]
    dv = v.shape[-1]
    y = np.zeros((B, H, T, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((p, p, dv))
            z = np.zeros((p, p))
            for t in range(T):
                w = P[h] @ k[b, h, t]
                u = P[h] @ q[b, h, t]
                for i in range(p):
                    for j in range(p):
                        S[i, j] += w[i] * w[j] * v[b, h, t]
                        z[i, j] += w[i] * w[j]
                num = np.zeros(dv)
                den = 0.0
                for i in range(p):
                    for j in range(p):
                        num += u[i] * u[j] * S[i, j]
                        den += u[i] * u[j] * z[i, j]
                y[b, h, t] = num / den if den != 0 else 0.0
    return y


def chunked_fp64(q, k, v, P, C):
    """The chunked-state decomposition ([TS-2.3]): per chunk, the prefix state read
    out through phi(q) plus the masked squared score tile of the chunk, with the
    chunk states combined by an explicit prefix sum."""
    B, H, T, d = q.shape
    p = P.shape[1]
    dv = v.shape[-1]
    y = np.zeros((B, H, T, dv))
    for b in range(B):
        for h in range(H):
            u = q[b, h] @ P[h].T
            w = k[b, h] @ P[h].T
            fk = np.einsum("ti,tj->tij", w, w).reshape(T, p * p)
            fq = np.einsum("ti,tj->tij", u, u).reshape(T, p * p)
            starts = list(range(0, T, C))
            dS = [fk[s:s + C].T @ v[b, h, s:s + C] for s in starts]
            dz = [fk[s:s + C].sum(0) for s in starts]
            pre_S = np.zeros((p * p, dv))
            pre_z = np.zeros(p * p)
            for ci, s in enumerate(starts):
                e = min(s + C, T)
                a = np.tril((u[s:e] @ w[s:e].T) ** 2)
                num = fq[s:e] @ pre_S + a @ v[b, h, s:e]
                den = fq[s:e] @ pre_z + a.sum(1)
                y[b, h, s:e] = np.where(den[:, None] != 0, num / np.where(den == 0, 1, den)[:, None], 0)
                pre_S = pre_S + dS[ci]
                pre_z = pre_z + dz[ci]
    return y


# --- pins ------------------------------------------------------------------------------

def pin_golden_scalar(fwd):
    """Hand-derived p = d = 1 example (tests/golden/scalar_p1.json)."""
    g = json.load(open(os.path.join(GOLDEN, "scalar_p1.json")))
    T = len(g["q"])
    q = np.array(g["q"]).reshape(1, 1, T, 1)
    k = np.array(g["k"]).reshape(1, 1, T, 1)
    v = np.array(g["v"]).reshape(1, 1, T, 1)
    P = np.array(g["P"]).reshape(1, 1, 1)
    y = fwd(q, k, v, P)[0, 0, :, 0]
    return float(np.max(np.abs(y - np.array(g["y"]))))


def pin_first_token(fwd):
    """y_0 = v_0: the first token only attends to itself (causal sum includes s = t)."""
    q, k, v, P = rand_case(1)
    y = fwd(q, k, v, P)
    return float(np.max(np.abs(y[..., 0, :] - v[..., 0, :])))


def pin_convex_hull(fwd):
    """Convex output gate ([TS-2.1], [ABS]): every y_t lies inside the box spanned by
    v_0..v_t, coordinate-wise.  Returns the largest violation."""
    q, k, v, P = rand_case(2, T=64)
    y = fwd(q, k, v, P)
    lo = np.minimum.accumulate(v, axis=2)
    hi = np.maximum.accumulate(v, axis=2)
    return float(max(np.max(lo - y), np.max(y - hi), 0.0))


def pin_gate_form(fwd):
    """y_t = lam_t r_t + (1 - lam_t) v_t with lam_t in [0, 1] and r_t the readout of the
    previous state at q_t ([TS-2.1]); r_t comes from the same function evaluated with v
    shifted to exclude token t (set v_t := r_t leaves y_t unchanged)."""
    q, k, v, P = rand_case(3, T=32)
    y = fwd(q, k, v, P)
    worst = 0.0
    for t in (5, 17, 31):
        # r_t: readout over s < t at query q_t -> make token t invisible by a zero key.
        k2 = k.copy()
        k2[..., t, :] = 0.0
        r = fwd(q, k2, v, P)[..., t, :]
        # lam from the residual along v_t - r_t
        dvec = (v[..., t, :] - r).ravel()
        lam = 1.0 - float(np.dot((y[..., t, :] - r).ravel(), dvec) / np.dot(dvec, dvec))
        recon = lam * r + (1.0 - lam) * v[..., t, :]
        worst = max(worst, float(np.max(np.abs(recon - y[..., t, :]))))
        if not (-1e-12 <= lam <= 1 + 1e-12):
            worst = max(worst, 1.0)
    return worst


def pin_causality(fwd):
    """Perturbing tokens after t leaves y_0..y_t bitwise unchanged."""
    q, k, v, P = rand_case(4, T=40)
    y = fwd(q, k, v, P)
    t = 23
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    r = np.random.default_rng(9)
    q2[..., t + 1:, :] = r.standard_normal(q2[..., t + 1:, :].shape)
    k2[..., t + 1:, :] = r.standard_normal(k2[..., t + 1:, :].shape)
    v2[..., t + 1:, :] = r.standard_normal(v2[..., t + 1:, :].shape)
    y2 = fwd(q2, k2, v2, P)
    return float(np.max(np.abs(y2[..., :t + 1, :] - y[..., :t + 1, :])))


def pin_brute_recurrence(fwd):
    """Quadratic form vs a pure-loop state recurrence ([TS-1]) on a tiny case."""
    q, k, v, P = rand_case(5, B=1, H=2, T=20, d=6, p=3, dv=4)
    return rel(fwd(q, k, v, P), brute_recurrence(q, k, v, P))


def pin_chunked_exact(fwd):
    """The chunked-state form is exact ([ABS], [TS-2.3]) for any chunk size."""
    q, k, v, P = rand_case(6, T=40)
    y = fwd(q, k, v, P)
    return max(rel(chunked_fp64(q, k, v, P, C), y) for C in (1, 3, 8, 16, 40))


def pin_rank_one_P(fwd):
    """Only row 0 of P nonzero: a_ts = (u0_t b_s)^2 with b_s = P_0 . k_s, so y_t is the
    running mean of v weighted by b_s^2, independent of q (a textbook weighted mean)."""
    q, k, v, P = rand_case(7, T=30)
    P = P.copy()
    P[:, 1:, :] = 0.0
    y = fwd(q, k, v, P)
    b2 = np.einsum("hd,bhtd->bht", P[:, 0, :], k) ** 2
    ref = np.cumsum(b2[..., None] * v, axis=2) / np.cumsum(b2, axis=2)[..., None]
    return rel(y, ref)


def pin_equal_keys(fwd):
    """All keys equal: every weight in row t is the same, so y_t is the plain running mean."""
    q, k, v, P = rand_case(8, T=30)
    k = np.broadcast_to(k[..., :1, :], k.shape).copy()
    y = fwd(q, k, v, P)
    ref = np.cumsum(v, axis=2) / np.arange(1, v.shape[2] + 1)[None, None, :, None]
    return rel(y, ref)


def pin_identity_projection(fwd):
    """P = I (d = p): squared dot-product (degree-2 homogeneous polynomial kernel)
    attention, evaluated by explicit double loops over query/key pairs."""
    q, k, v, _ = rand_case(10, T=16, d=4, p=4, dv=3)
    P = np.eye(4)[None]
    y = fwd(q, k, v, P)
    T = q.shape[2]
    ref = np.zeros_like(y)
    for t in range(T):
        num = np.zeros(3)
        den = 0.0
        for s in range(t + 1):
            a = float(np.dot(q[0, 0, t], k[0, 0, s])) ** 2
            num += a * v[0, 0, s]
            den += a
        ref[0, 0, t] = num / den
    return rel(y, ref)


def pin_invariances(fwd):
    """Homogeneity and isometric invariance ([TS-2.1], assumptions 2 and 3): y(alpha P) =
    y(P); y(O P) = y(P) for orthogonal O; affine equivariance in v: y(beta v + c) =
    beta y(v) + c."""
    q, k, v, P = rand_case(11, T=36)
    y = fwd(q, k, v, P)
    r = np.random.default_rng(12)
    O, _ = np.linalg.qr(r.standard_normal((P.shape[1], P.shape[1])))
    res = [rel(fwd(q, k, v, 3.7 * P), y),
           rel(fwd(q, k, v, np.einsum("ij,hjd->hid", O, P)), y),
           rel(fwd(q, k, -2.5 * v + 0.75, P), -2.5 * y + 0.75)]
    return max(res)


def pin_orthogonal_left_only(fwd):
    """Isometric invariance acts on the projected space (P -> O P), not on the input
    space: for a generic orthogonal R on the input side, y(P R) differs from y(P)."""
    q, k, v, P = rand_case(13, T=36, d=6, p=6)
    r = np.random.default_rng(14)
    R, _ = np.linalg.qr(r.standard_normal((6, 6)))
    y = fwd(q, k, v, P)
    y2 = fwd(q, k, v, np.einsum("hid,de->hie", P, R))
    # Returns a residual that is small only when y changed (as it must).
    return 1.0 / (1.0 + 1e6 * rel(y2, y))


PINS = {
    "golden_scalar": (pin_golden_scalar, 1e-12),
    "first_token": (pin_first_token, 1e-12),
    "convex_hull": (pin_convex_hull, 1e-12),
    "gate_form": (pin_gate_form, 1e-9),
    "causality": (pin_causality, 0.0),
    "brute_recurrence": (pin_brute_recurrence, 1e-12),
    "chunked_exact": (pin_chunked_exact, 1e-12),
    "rank_one_P": (pin_rank_one_P, 1e-12),
    "equal_keys": (pin_equal_keys, 1e-12),
    "identity_projection": (pin_identity_projection, 1e-12),
    "invariances": (pin_invariances, 1e-11),
    "orthogonal_left_only": (pin_orthogonal_left_only, 1e-3),
}


def failing_pins(fwd):
    out = []
    for name, (fn, bound) in PINS.items():
        try:
            r = fn(fwd)
        except Exception:  # a broken variant may also crash
            out.append(name)
            continue
        if not (r <= bound):
            out.append(name)
    return out
