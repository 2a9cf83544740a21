"""Pins of the oracle's decay-gated forward (``forward_decay_quadratic``,
``final_state_decay``, ``decode_decay_reference``) against an independent token
recurrence, special cases with closed forms, invariants and an independent chunked
(affine-scan) decomposition.

The gate reading (the abstract names decay gates but defines none): S_t = gamma_t
S_{t-1} + phi(k_t) v_t^T and z_t likewise, gamma_t = exp(lam_t) per token and head.
Each check takes the function under test and returns a residual.
"""
from __future__ import annotations

import numpy as np

from oracle import kata_oracle as O


def dcase(seed, B=1, H=2, T=24, d=6, p=4, dv=3, scale=0.4):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, H, T, d))
    k = r.standard_normal((B, H, T, d))
    v = r.standard_normal((B, H, T, dv))
    P = r.standard_normal((H, p, d)) / np.sqrt(d)
    lam = -np.abs(r.standard_normal((B, H, T))) * scale
    return q, k, v, P, lam


def rel(a, b):
    n = np.linalg.norm(b)
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / (n if n > 0 else 1.0))


def loop_recurrence(q, k, v, P, lam, S0=None, z0=None):
    """Token loop with explicit outer products and pure-Python feature sums."""
    B, H, T, d = q.shape
    p = P.shape[1]
    dv = v.shape[-1]
    y = np.zeros((B, H, T, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((p, p, dv)) if S0 is None else S0[b, h].reshape(p, p, dv).copy()
            z = np.zeros((p, p)) if z0 is None else z0[b, h].reshape(p, p).copy()
            for t in range(T):
                g = np.exp(lam[b, h, t])
                w = P[h] @ k[b, h, t]
                u = P[h] @ q[b, h, t]
                S = g * S + np.einsum("i,j,c->ijc", w, w, v[b, h, t])
                z = g * z + np.outer(w, w)
                num = np.einsum("i,j,ijc->c", u, u, S)
                den = float(u @ z @ u)
                y[b, h, t] = num / den if den != 0 else 0.0
    return y


def pin_decay_recurrence(fwd):
    q, k, v, P, lam = dcase(1)
    return rel(fwd(q, k, v, P, lam), loop_recurrence(q, k, v, P, lam))


def pin_decay_with_state(fwd):
    q, k, v, P, lam = dcase(2, T=15)
    r = np.random.default_rng(20)
    S0 = r.standard_normal((1, 2, 16, 3))
    S0 = (S0.reshape(1, 2, 4, 4, 3) + S0.reshape(1, 2, 4, 4, 3).transpose(0, 1, 3, 2, 4)).reshape(1, 2, 16, 3)
    w0 = r.standard_normal((1, 2, 4))
    z0 = (np.einsum("bhi,bhj->bhij", w0, w0) + np.eye(4)).reshape(1, 2, 16)
    return rel(fwd(q, k, v, P, lam, S0, z0), loop_recurrence(q, k, v, P, lam, S0, z0))


def pin_decay_no_gate_is_plain(fwd):
    """lam = 0 (gamma = 1) is plain KATA (the separately pinned forward)."""
    q, k, v, P, lam = dcase(3)
    return rel(fwd(q, k, v, P, 0.0 * lam), O.forward_quadratic(q, k, v, P))


def pin_decay_full_forget(fwd):
    """gamma = 0 at every token: only the current token is left, y_t = v_t."""
    q, k, v, P, lam = dcase(4)
    y = fwd(q, k, v, P, np.full_like(lam, -1e4))
    return float(np.max(np.abs(y - v)))


def pin_decay_geometric_mean(fwd):
    """All keys equal, constant gamma: y_t = sum_s gamma^(t-s) v_s / sum_s gamma^(t-s)."""
    q, k, v, P, lam = dcase(5, T=30)
    k = np.broadcast_to(k[..., :1, :], k.shape).copy()
    gam = 0.8
    y = fwd(q, k, v, P, np.full_like(lam, np.log(gam)))
    T = v.shape[2]
    ref = np.zeros_like(y)
    for t in range(T):
        wts = gam ** (t - np.arange(t + 1))
        ref[..., t, :] = np.einsum("s,bhsc->bhc", wts, v[..., :t + 1, :]) / wts.sum()
    return rel(y, ref)


def pin_decay_convex(fwd):
    """The output gate stays convex: y_t within the box of v_0..v_t."""
    q, k, v, P, lam = dcase(6, T=40, scale=1.5)
    y = fwd(q, k, v, P, lam)
    lo = np.minimum.accumulate(v, axis=2)
    hi = np.maximum.accumulate(v, axis=2)
    return float(max(np.max(lo - y), np.max(y - hi), 0.0))


def chunked_affine(q, k, v, P, lam, C):
    """Chunked form: per chunk the decayed chunk state (keys weighted exp(L_c - l_s)),
    the inter-chunk prefix by the affine recurrence H <- exp(L_c) H + state_c, and inside
    the chunk the readout exp(l_t) phi(q_t)^T H plus weights (u_t.w_s)^2 exp(l_t - l_s)."""
    B, H, T, d = q.shape
    p = P.shape[1]
    dv = v.shape[-1]
    y = np.zeros((B, H, T, dv))
    for b in range(B):
        for h in range(H):
            u = q[b, h] @ P[h].T
            w = k[b, h] @ P[h].T
            fq = np.einsum("ti,tj->tij", u, u).reshape(T, p * p)
            fk = np.einsum("ti,tj->tij", w, w).reshape(T, p * p)
            Hs = np.zeros((p * p, dv))
            Hz = np.zeros(p * p)
            for s0 in range(0, T, C):
                e = min(s0 + C, T)
                l = np.cumsum(lam[b, h, s0:e])
                Lc = l[-1]
                a = np.tril((u[s0:e] @ w[s0:e].T) ** 2 * np.exp(l[:, None] - l[None, :]))
                num = np.exp(l)[:, None] * (fq[s0:e] @ Hs) + a @ v[b, h, s0:e]
                den = np.exp(l) * (fq[s0:e] @ Hz) + a.sum(1)
                y[b, h, s0:e] = num / den[:, None]
                wk = np.exp(Lc - l)
                Hs = np.exp(Lc) * Hs + (fk[s0:e] * wk[:, None]).T @ v[b, h, s0:e]
                Hz = np.exp(Lc) * Hz + (fk[s0:e] * wk[:, None]).sum(0)
    return y


def pin_decay_chunked_exact(fwd):
    q, k, v, P, lam = dcase(7, T=40)
    y = fwd(q, k, v, P, lam)
    return max(rel(chunked_affine(q, k, v, P, lam, C), y) for C in (1, 3, 8, 16, 40))


def pin_decay_final_state(fwd_state):
    """final state = the recurrence's, and resuming from it continues the sequence."""
    q, k, v, P, lam = dcase(8, T=18)
    B, H, T, d = q.shape
    p = P.shape[1]
    S = np.zeros((B, H, p * p, v.shape[-1]))
    z = np.zeros((B, H, p * p))
    for t in range(T):
        g = np.exp(lam[:, :, t])
        fk = O.feature_full(np.einsum("hpd,bhd->bhp", P, k[:, :, t]))
        S = g[..., None, None] * S + fk[..., :, None] * v[:, :, t, None, :]
        z = g[..., None] * z + fk
    ST, zT = fwd_state(k, v, P, lam)
    return max(rel(ST, S), rel(zT, z))


def pin_decay_resume(fwd):
    q, k, v, P, lam = dcase(9, T=30)
    m = 11
    full = fwd(q, k, v, P, lam)
    S1, z1 = O.final_state_decay(k[:, :, :m], v[:, :, :m], P, lam[:, :, :m])
    part = fwd(q[:, :, m:], k[:, :, m:], v[:, :, m:], P, lam[:, :, m:], S1, z1)
    return rel(part, full[:, :, m:])


def pin_decay_decode_step():
    """The decode step equals one step of the token recurrence."""
    r = np.random.default_rng(10)
    N, H, d, p, dv = 3, 2, 5, 4, 3
    P = r.standard_normal((H, p, d))
    S = r.standard_normal((N, H, p * p, dv))
    z = np.abs(r.standard_normal((N, H, p * p))) + 1.0
    q, k = r.standard_normal((N, H, d)), r.standard_normal((N, H, d))
    v = r.standard_normal((N, H, dv))
    lam = -np.abs(r.standard_normal((N, H)))
    y, S2, z2 = O.decode_decay_reference(S, z, q, k, v, P, lam)
    g = np.exp(lam)
    fk = O.feature_full(np.einsum("hpd,nhd->nhp", P, k))
    fq = O.feature_full(np.einsum("hpd,nhd->nhp", P, q))
    Sr = g[..., None, None] * S + fk[..., :, None] * v[..., None, :]
    zr = g[..., None] * z + fk
    yr = np.einsum("nhf,nhfc->nhc", fq, Sr) / np.einsum("nhf,nhf->nh", fq, zr)[..., None]
    return max(rel(y, yr), rel(S2, Sr), rel(z2, zr))


PINS = {
    "recurrence": (pin_decay_recurrence, 1e-10),
    "with_state": (pin_decay_with_state, 1e-10),
    "no_gate_is_plain": (pin_decay_no_gate_is_plain, 1e-12),
    "full_forget": (pin_decay_full_forget, 1e-12),
    "geometric_mean": (pin_decay_geometric_mean, 1e-12),
    "convex": (pin_decay_convex, 1e-12),
    "chunked_exact": (pin_decay_chunked_exact, 1e-10),
    "resume": (pin_decay_resume, 1e-10),
}


def failing_pins(fwd):
    out = []
    for name, (fn, bound) in PINS.items():
        try:
            r = fn(fwd)
        except Exception:
            out.append(name)
            continue
        if not (r <= bound):
            out.append(name)
    return out
