"""Pins of the oracle's backward (``backward_quadratic``) against facts fixed by the
forward definition and by calculus, independently of the backward's own formulas.

Each check takes a backward function with the oracle's signature (the oracle's
own, or a deliberately broken copy in the mutation tests) and returns a float
residual; it passes below its bound.  The references are: central finite
differences of the (separately pinned) forward oracle, Euler's identity for the
homogeneities of the forward, the T = 1 closed form, and the exact split of a
sequence into two segments joined by the recurrent state.

Citations: "Kernelized Linear Attention: Breaking the Capacity Wall with Symmetric
Cones" (arXiv 2607.17419); [ABS] its abstract, [TS-x] section x of the
gist.science technical summary of it.  The pages give no backward pass: the
gradient is the derivative of the forward they define ([TS-1], [TS-2.2]).
"""
from __future__ import annotations

import numpy as np

from oracle import kata_oracle as O


def bwd_case(seed, B=1, H=2, T=9, d=6, p=4, dv=3, state=True):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, H, T, d))
    k = r.standard_normal((B, H, T, d))
    v = r.standard_normal((B, H, T, dv))
    P = r.standard_normal((H, p, d)) / np.sqrt(d)
    gy = r.standard_normal((B, H, T, dv))
    out = dict(q=q, k=k, v=v, P=P, gy=gy, S0=None, z0=None, gST=None, gzT=None)
    if state:
        out["S0"] = r.standard_normal((B, H, p * p, dv))
        out["z0"] = np.abs(r.standard_normal((B, H, p * p))) + 1.0
        out["gST"] = r.standard_normal((B, H, p * p, dv))
        out["gzT"] = r.standard_normal((B, H, p * p))
    return out


def loss(c, q=None, k=None, v=None, P=None, S0=None, z0=None):
    """L = sum gy . y + <gST, S_T> + <gzT, z_T> from the forward oracle."""
    q = c["q"] if q is None else q
    k = c["k"] if k is None else k
    v = c["v"] if v is None else v
    P = c["P"] if P is None else P
    S0 = c["S0"] if S0 is None else S0
    z0 = c["z0"] if z0 is None else z0
    y = O.forward_quadratic(q, k, v, P, S0, z0)
    L = float(np.sum(c["gy"] * y))
    if c["gST"] is not None:
        ST, zT = O.final_state(k, v, P, S0, z0)
        L += float(np.sum(c["gST"] * ST) + np.sum(c["gzT"] * zT))
    return L


def _grads(bwd, c):
    return bwd(c["q"], c["k"], c["v"], c["P"], c["gy"], c["S0"], c["z0"], c["gST"], c["gzT"])


NAMES = ("q", "k", "v", "P", "S0", "z0")


def _fd_directional(bwd, c, eps=1e-6, seed=100):
    g = _grads(bwd, c)
    r = np.random.default_rng(seed)
    worst = 0.0
    for i, name in enumerate(NAMES):
        if c[name] is None:
            continue
        e = r.standard_normal(c[name].shape)
        fp = loss(c, **{name: c[name] + eps * e})
        fm = loss(c, **{name: c[name] - eps * e})
        fd = (fp - fm) / (2 * eps)
        an = float(np.sum(g[i] * e))
        worst = max(worst, abs(fd - an) / max(abs(fd), 1e-3))
    return worst


def pin_bwd_fd_directional(bwd):
    """Directional derivative along random directions of every input (q, k, v, P, S0,
    z0) equals the central difference of the forward oracle (with an initial state
    and a final-state gradient)."""
    return _fd_directional(bwd, bwd_case(1))


def pin_bwd_fd_p16(bwd):
    """The same at the projection dimension of the kernels (p = 16), no state."""
    return _fd_directional(bwd, bwd_case(2, B=2, H=1, T=7, d=5, p=16, dv=4, state=False))


def pin_bwd_fd_entries(bwd):
    """Every single entry of every gradient against a central difference (tiny case)."""
    c = bwd_case(3, B=1, H=1, T=4, d=3, p=2, dv=2)
    g = _grads(bwd, c)
    eps = 1e-6
    worst = 0.0
    for i, name in enumerate(NAMES):
        x = c[name]
        for idx in np.ndindex(x.shape):
            e = np.zeros_like(x)
            e[idx] = 1.0
            fd = (loss(c, **{name: x + eps * e}) - loss(c, **{name: x - eps * e})) / (2 * eps)
            worst = max(worst, abs(fd - g[i][idx]) / max(abs(fd), 1e-2))
    return worst


def pin_bwd_query_scale(bwd):
    """y_t is unchanged when q_t is scaled (weights and readout are homogeneous of the
    same degree in u_t, [TS-2.1]), so by Euler <dq_t, q_t> = 0 for every token."""
    c = bwd_case(4, T=12)
    dq = _grads(bwd, c)[0]
    s = np.abs(np.einsum("bhtd,bhtd->bht", dq, c["q"]))
    return float(np.max(s) / np.max(np.abs(dq)))


def pin_bwd_value_linear(bwd):
    """With no initial state, y and S_T are linear in v, so <dv, v> = sum gy . y + <gST, S_T>."""
    c = bwd_case(5, T=11)
    c["S0"] = None
    c["z0"] = None
    dv = _grads(bwd, c)[2]
    lhs = float(np.sum(dv * c["v"]))
    y = O.forward_quadratic(c["q"], c["k"], c["v"], c["P"])
    ST, _ = O.final_state(c["k"], c["v"], c["P"])
    rhs = float(np.sum(c["gy"] * y) + np.sum(c["gST"] * ST))
    return abs(lhs - rhs) / abs(rhs)


def pin_bwd_projection_scale(bwd):
    """With no initial state, P -> alpha P leaves y unchanged and scales S_T, z_T by
    alpha^2, so <dP, P> = 2 <gST, S_T> + 2 <gzT, z_T>."""
    c = bwd_case(6, T=10)
    c["S0"] = None
    c["z0"] = None
    dP = _grads(bwd, c)[3]
    ST, zT = O.final_state(c["k"], c["v"], c["P"])
    rhs = 2.0 * float(np.sum(c["gST"] * ST) + np.sum(c["gzT"] * zT))
    return abs(float(np.sum(dP * c["P"])) - rhs) / abs(rhs)


def pin_bwd_single_token(bwd):
    """T = 1, no state: y_0 = v_0 exactly, so dv_0 = gy_0 and dq, dk, dP vanish."""
    c = bwd_case(7, T=1, state=False)
    dq, dk, dv, dP, _, _ = _grads(bwd, c)
    return float(max(np.max(np.abs(dv - c["gy"])), np.max(np.abs(dq)), np.max(np.abs(dk)),
                     np.max(np.abs(dP))))


def pin_bwd_sequence_split(bwd):
    """Splitting a sequence at token m and carrying the state ([TS-1]): the gradient of
    the whole sequence equals that of the second segment started from (S_m, z_m), whose
    dS0, dz0 are fed as the final-state gradient of the first segment."""
    c = bwd_case(8, T=14, state=False)
    m = 6
    q, k, v, P, gy = c["q"], c["k"], c["v"], c["P"], c["gy"]
    full = bwd(q, k, v, P, gy)
    Sm, zm = O.final_state(k[:, :, :m], v[:, :, :m], P)
    g2 = bwd(q[:, :, m:], k[:, :, m:], v[:, :, m:], P, gy[:, :, m:], Sm, zm)
    g1 = bwd(q[:, :, :m], k[:, :, :m], v[:, :, :m], P, gy[:, :, :m], None, None, g2[4], g2[5])
    res = [O_rel(np.concatenate([g1[i], g2[i]], axis=2), full[i]) for i in range(3)]
    res.append(O_rel(g1[3] + g2[3], full[3]))
    return max(res)


def O_rel(a, b):
    n = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (n if n > 0 else 1.0))


PINS = {
    "fd_directional": (pin_bwd_fd_directional, 1e-6),
    "fd_p16": (pin_bwd_fd_p16, 1e-6),
    "fd_entries": (pin_bwd_fd_entries, 1e-6),
    "query_scale": (pin_bwd_query_scale, 1e-12),
    "value_linear": (pin_bwd_value_linear, 1e-12),
    "projection_scale": (pin_bwd_projection_scale, 1e-11),
    "single_token": (pin_bwd_single_token, 1e-13),
    "sequence_split": (pin_bwd_sequence_split, 1e-12),
}


def failing_pins(bwd):
    out = []
    for name, (fn, bound) in PINS.items():
        try:
            r = fn(bwd)
        except Exception:
            out.append(name)
            continue
        if not (r <= bound):
            out.append(name)
    return out
