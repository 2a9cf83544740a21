"""Plain fp64 CPU oracle for the KATA causal forward pass, its gradients and the decode step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its Python binding) never imports, calls or links it, and
this module imports nothing from the product package.

Sources (pages describing "Kernelized Linear Attention: Breaking the Capacity
Wall with Symmetric Cones", arXiv 2607.17419):

* [ABS]    the paper's abstract (fugumt.com entry for arXiv 2607.17419v1).
* [TS-1]   gist.science technical summary of 2607.17419, section 1
           ("Planteamiento del Problema"): normalised linear attention with a
           fixed-size state and constant-time recurrent inference.
* [TS-2.1] same summary, section 2.1 ("Marco Teorico"): nonnegative weights
           certified by a self-dual cone; the denominator of normalised linear
           attention acts as a parameter-free convex output gate.
* [TS-2.2] same summary, section 2.2 ("Teoria de la Capacidad", item
           "Cono PSD"): rank-one PSD feature psi(u) = u u^T, which squares the
           raw inner product; capacity grows with the projection dimension p.
* [TS-2.3] same summary, section 2.3: chunked form, exact O(T) chunked state.
* [TS-4]   same summary, section 4 ("Resultados"): the delta-rule variant
           (DeltaKATA) corrects stale bindings under repeated-key overwrite.
* [TS-2.3v] same summary, section 2.3, item "Variantes": KATA-Mg (several PSD
           factors) and KATA-Sigma-g (summed PSD factors).

What is computed (plain definition, no blocking beyond bounding memory):

    u_t = P q_t,  w_s = P k_s                    (projection to dimension p)
    a_ts = <psi(u_t), psi(w_s)> = (u_t . w_s)^2   for s <= t, else 0
    y_t  = sum_s a_ts v_s / sum_s a_ts            (0 where the sum is 0)

with an optional initial state (S0, z0) that adds phi(q_t)^T S0 to the
numerator and phi(q_t) . z0 to the denominator, phi(x) = vec((Px)(Px)^T) in
the canonical row-major index i*p + j.  The final state is
S_T = S0 + sum_s phi(k_s) v_s^T, z_T = z0 + sum_s phi(k_s).

The backward (``backward_quadratic``) is the chain rule through this same
definition: the pages give no backward pass, so the gradient of the forward they
define is the only reading; it is pinned against finite differences of the
forward, not against itself.

Readings where the pages leave a step open (each also listed in the design
notes): the causal sum includes s = t (the convex gate of [TS-2.1] mixes in
the current value); there is no temperature and no epsilon; a zero
denominator gives y = 0; P is a p x d matrix per head.

All arithmetic is float64.  bf16 inputs are decoded bit-exactly from their
uint16 storage (``bf16_bits_to_f64``) so the oracle sees exactly the values
the GPU sees.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits_to_f64",
    "project",
    "feature_full",
    "feature_packed",
    "weights",
    "forward_quadratic",
    "final_state",
    "recurrence",
    "decode_reference",
    "backward_quadratic",
    "forward_decay_quadratic",
    "final_state_decay",
    "decode_decay_reference",
    "feature_unit",
    "delta_recurrence",
    "delta_decode_reference",
    "factor_projections",
    "forward_mg_quadratic",
    "final_state_mg",
    "recurrence_mg",
    "forward_sg_quadratic",
    "final_state_sg",
    "recurrence_sg",
    "decode_factors_reference",
]


def bf16_bits_to_f64(bits):
    """Decode bfloat16 values stored as uint16 bit patterns into float64.

    bfloat16 is the upper half of an IEEE float32, so shifting the 16 stored
    bits into the high half of a 32-bit word gives the float32 with the same
    value; widening to float64 is exact.
    """
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    with np.errstate(invalid="ignore"):   # NaN payloads widen to NaN
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def project(x, P):
    """u = P x for every vector of x ([..., d]) with P of shape [p, d] ([TS-2.2], [ABS]).

    Returns [..., p] in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    P = np.asarray(P, dtype=np.float64)
    return x @ P.T


def feature_full(u):
    """Rank-one PSD feature psi(u) = u u^T, flattened row-major: index i*p + j ([TS-2.2])."""
    u = np.asarray(u, dtype=np.float64)
    p = u.shape[-1]
    return (u[..., :, None] * u[..., None, :]).reshape(u.shape[:-1] + (p * p,))


def feature_packed(u):
    """Symmetric packing of psi(u): the p(p+1)/2 entries i <= j in row-major order,
    off-diagonal entries scaled by sqrt(2) so that the inner product of two
    packed features equals that of the full features ([TS-2.2]).
    """
    u = np.asarray(u, dtype=np.float64)
    p = u.shape[-1]
    iu, ju = np.triu_indices(p)
    scale = np.where(iu == ju, 1.0, np.sqrt(2.0))
    return u[..., iu] * u[..., ju] * scale


def weights(q, k, P):
    """Causal attention weights a_ts = ((P q_t) . (P k_s))^2 for s <= t, 0 otherwise.

    q: [T, d], k: [T, d], P: [p, d].  Returns [T, T] float64.  Every entry is a
    square, hence nonnegative ([TS-2.1], [ABS]).
    """
    u = project(q, P)
    w = project(k, P)
    a = (u @ w.T) ** 2
    return np.tril(a)


def _head_forward(q, k, v, P, S0, z0, rows, block):
    """y for one head at the query rows ``rows`` (sorted int array)."""
    u = project(q, P)            # [T, p]
    w = project(k, P)            # [T, p]
    v = np.asarray(v, dtype=np.float64)
    dv = v.shape[1]
    y = np.zeros((len(rows), dv))
    for r0 in range(0, len(rows), block):
        rr = rows[r0:r0 + block]
        smax = int(rr[-1]) + 1
        a = (u[rr] @ w[:smax].T) ** 2                   # [nb, smax]
        a[np.arange(smax)[None, :] > rr[:, None]] = 0.0  # causal: keep s <= t
        num = a @ v[:smax]
        den = a.sum(axis=1)
        if S0 is not None:
            f = feature_full(u[rr])
            num = num + f @ S0
            den = den + f @ z0
        ok = den != 0.0
        y[r0:r0 + block][ok] = num[ok] / den[ok, None]
    return y


def forward_quadratic(q, k, v, P, S0=None, z0=None, rows=None, block=256):
    """Causal normalised KATA attention by the O(T^2) definition.

    q, k: [B, H, T, d]; v: [B, H, T, dv]; P: [H, p, d] (one projection per head);
    S0: [B, H, p*p, dv] or None; z0: [B, H, p*p] or None; rows: optional sorted
    query indices (evaluates y only there, e.g. to sample a long sequence).
    Returns y: [B, H, len(rows) or T, dv] float64.

    Definition ([TS-1], [TS-2.1], [TS-2.2], [ABS]): y_t = (sum_{s<=t} a_ts v_s
    + phi(q_t)^T S0) / (sum_{s<=t} a_ts + phi(q_t) . z0), a_ts = ((Pq_t).(Pk_s))^2;
    y_t = 0 where the denominator is 0.
    """
    q = np.asarray(q); k = np.asarray(k); v = np.asarray(v); P = np.asarray(P)
    B, H, T, _ = q.shape
    dv = v.shape[-1]
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    y = np.zeros((B, H, len(rows), dv))
    has_init = S0 is not None or z0 is not None
    pp = P.shape[1] * P.shape[1]
    for b in range(B):
        for h in range(H):
            s0 = zz = None
            if has_init:
                s0 = np.zeros((pp, dv)) if S0 is None else np.asarray(S0[b, h], dtype=np.float64)
                zz = np.zeros(pp) if z0 is None else np.asarray(z0[b, h], dtype=np.float64)
            y[b, h] = _head_forward(q[b, h], k[b, h], v[b, h], P[h], s0, zz, rows, block)
    return y


def final_state(k, v, P, S0=None, z0=None):
    """Final recurrent state after all tokens ([TS-1]: fixed-size state).

    S_T = S0 + sum_s phi(k_s) v_s^T   ([B, H, p*p, dv])
    z_T = z0 + sum_s phi(k_s)         ([B, H, p*p])
    with phi the canonical full feature (row-major i*p + j).
    """
    k = np.asarray(k); v = np.asarray(v, dtype=np.float64); P = np.asarray(P)
    B, H, T, _ = k.shape
    p = P.shape[1]
    ST = np.zeros((B, H, p * p, v.shape[-1]))
    zT = np.zeros((B, H, p * p))
    for b in range(B):
        for h in range(H):
            f = feature_full(project(k[b, h], P[h]))     # [T, p*p]
            ST[b, h] = f.T @ v[b, h]
            zT[b, h] = f.sum(axis=0)
    if S0 is not None:
        ST = ST + np.asarray(S0, dtype=np.float64)
    if z0 is not None:
        zT = zT + np.asarray(z0, dtype=np.float64)
    return ST, zT


def recurrence(q, k, v, P, S0=None, z0=None):
    """Token-by-token recurrent form ([TS-1]: constant-time recurrent inference).

    For each token in order: S += phi(k_t) v_t^T, z += phi(k_t), then
    y_t = S^T phi(q_t) / (z . phi(q_t)) (0 when the denominator is 0).
    Returns (y [B,H,T,dv], S_T, z_T).
    """
    q = np.asarray(q); k = np.asarray(k); v = np.asarray(v, dtype=np.float64); P = np.asarray(P)
    B, H, T, _ = q.shape
    p = P.shape[1]
    dv = v.shape[-1]
    y = np.zeros((B, H, T, dv))
    ST = np.zeros((B, H, p * p, dv))
    zT = np.zeros((B, H, p * p))
    for b in range(B):
        for h in range(H):
            S = np.zeros((p * p, dv)) if S0 is None else np.array(S0[b, h], dtype=np.float64)
            z = np.zeros(p * p) if z0 is None else np.array(z0[b, h], dtype=np.float64)
            fq = feature_full(project(q[b, h], P[h]))
            fk = feature_full(project(k[b, h], P[h]))
            for t in range(T):
                S += np.outer(fk[t], v[b, h, t])
                z += fk[t]
                den = fq[t] @ z
                if den != 0.0:
                    y[b, h, t] = (fq[t] @ S) / den
            ST[b, h] = S
            zT[b, h] = z
    return y, ST, zT


def decode_reference(S, z, q, k, v, P):
    """One recurrent decode step for N independent streams ([TS-1], [ABS]).

    S: [N, H, p*p, dv], z: [N, H, p*p] (state before the step), q, k: [N, H, d],
    v: [N, H, dv], P: [H, p, d].  The step first folds the new token into the
    state, then reads it out (the current token is part of its own causal sum):

        S' = S + phi(k) v^T,  z' = z + phi(k),  y = S'^T phi(q) / (z' . phi(q)).

    Returns (y [N, H, dv], S', z').
    """
    S = np.array(S, dtype=np.float64)
    z = np.array(z, dtype=np.float64)
    q = np.asarray(q); k = np.asarray(k); v = np.asarray(v, dtype=np.float64); P = np.asarray(P)
    N, H = q.shape[:2]
    y = np.zeros(v.shape)
    for h in range(H):
        fq = feature_full(project(q[:, h], P[h]))    # [N, p*p]
        fk = feature_full(project(k[:, h], P[h]))
        S[:, h] += fk[:, :, None] * v[:, h, None, :]
        z[:, h] += fk
        den = np.einsum("nf,nf->n", fq, z[:, h])
        num = np.einsum("nf,nfj->nj", fq, S[:, h])
        ok = den != 0.0
        y[ok, h] = num[ok] / den[ok, None]
    return y, S, z


def _sym_mat(x, p):
    """The symmetric p x p matrix M + M^T of a flattened row-major p*p vector."""
    m = np.asarray(x, dtype=np.float64).reshape(p, p)
    return m + m.T


def backward_quadratic(q, k, v, P, gy, S0=None, z0=None, gST=None, gzT=None):
    """Gradients of the causal KATA forward by the chain rule through its O(T^2) definition.

    PARITY NOTE: the pages give no backward pass; the gradient is fixed by the forward
    definition alone ([TS-1], [TS-2.1], [TS-2.2], [ABS]: the same quantities as
    ``forward_quadratic`` and ``final_state``).  The scalar being differentiated is

        L = sum_t gy_t . y_t + <gST, S_T> + <gzT, z_T>

    with y, S_T, z_T as in ``forward_quadratic`` / ``final_state`` (the initial state
    enters through the full feature phi(x) = vec(u u^T), so S0 and z0 are used with
    every entry).  Inputs as for ``forward_quadratic``; gy [B, H, T, dv]; gST [B, H,
    p*p, dv] and gzT [B, H, p*p] or None (zero).

    Per head, with u = P q, w = P k, X = u w^T and a = tril(X^2):
      num_t = sum_s a_ts v_s + phi(u_t)^T S0,  den_t = sum_s a_ts + phi(u_t) . z0
      gnum_t = gy_t / den_t,  gden_t = -(gy_t . y_t) / den_t   (both 0 where den_t = 0,
                                                              where y_t is the constant 0)
      ga_ts = gnum_t . v_s + gden_t   (s <= t),  gX = 2 X o ga
      du_t = sum_s gX_ts w_s + (M_t + M_t^T) u_t,  M_t = mat(S0 gnum_t + z0 gden_t)
      dw_s = sum_t gX_ts u_t + (N_s + N_s^T) w_s,  N_s = mat(gST v_s + gzT)
      dv_s = sum_t a_ts gnum_t + gST^T phi(w_s)
      dq = du P, dk = dw P, dP = sum over batch rows and tokens of du q^T + dw k^T
      dS0 = gST + sum_t phi(u_t) gnum_t^T,  dz0 = gzT + sum_t phi(u_t) gden_t

    Returns (dq [B,H,T,d], dk [B,H,T,d], dv [B,H,T,dv], dP [H,p,d], dS0 [B,H,p*p,dv],
    dz0 [B,H,p*p]), all float64.
    """
    q = np.asarray(q, dtype=np.float64); k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64); P = np.asarray(P, dtype=np.float64)
    gy = np.asarray(gy, dtype=np.float64)
    B, H, T, d = q.shape
    dv = v.shape[-1]
    p = P.shape[1]
    pp = p * p
    dq = np.zeros_like(q); dk = np.zeros_like(k); dvv = np.zeros_like(v)
    dP = np.zeros_like(P)
    dS0 = np.zeros((B, H, pp, dv)); dz0 = np.zeros((B, H, pp))
    causal = np.tril(np.ones((T, T), dtype=bool))
    for b in range(B):
        for h in range(H):
            s0 = np.zeros((pp, dv)) if S0 is None else np.asarray(S0[b, h], dtype=np.float64)
            zz = np.zeros(pp) if z0 is None else np.asarray(z0[b, h], dtype=np.float64)
            gs = np.zeros((pp, dv)) if gST is None else np.asarray(gST[b, h], dtype=np.float64)
            gz = np.zeros(pp) if gzT is None else np.asarray(gzT[b, h], dtype=np.float64)
            u = project(q[b, h], P[h])
            w = project(k[b, h], P[h])
            fu = feature_full(u)
            fw = feature_full(w)
            X = u @ w.T
            a = np.where(causal, X * X, 0.0)
            num = a @ v[b, h] + fu @ s0
            den = a.sum(axis=1) + fu @ zz
            ok = den != 0.0
            safe = np.where(ok, den, 1.0)
            y = np.where(ok[:, None], num / safe[:, None], 0.0)
            gnum = np.where(ok[:, None], gy[b, h] / safe[:, None], 0.0)
            gden = np.where(ok, -np.einsum("tj,tj->t", gy[b, h], y) / safe, 0.0)
            ga = np.where(causal, gnum @ v[b, h].T + gden[:, None], 0.0)
            gX = 2.0 * X * ga
            du = gX @ w
            dw = gX.T @ u
            for t in range(T):
                du[t] += _sym_mat(s0 @ gnum[t] + zz * gden[t], p) @ u[t]
                dw[t] += _sym_mat(gs @ v[b, h, t] + gz, p) @ w[t]
            dvv[b, h] = a.T @ gnum + fw @ gs
            dq[b, h] = du @ P[h]
            dk[b, h] = dw @ P[h]
            dP[h] += du.T @ q[b, h] + dw.T @ k[b, h]
            dS0[b, h] = gs + fu.T @ gnum
            dz0[b, h] = gz + fu.T @ gden
    return dq, dk, dvv, dP, dS0, dz0


# ---- decay-gated KATA ------------------------------------------------------------------
#
# PARITY NOTE (reading): the abstract names "decay gates" among the mechanisms studied
# with KATA's features but defines none.  The plainest reading, the scalar forget gate of
# gated linear attention, applied to KATA's state [S | z]:
#
#     S_t = gamma_t S_{t-1} + phi(k_t) v_t^T,   z_t = gamma_t z_{t-1} + phi(k_t),
#     y_t = S_t^T phi(q_t) / (z_t . phi(q_t)),   gamma_t = exp(lam_t), lam_t <= 0,
#
# one gate per token and head, the current token undecayed.  Unrolled, the weight of key
# s in query t is a_ts = (u_t . w_s)^2 exp(Lam_t - Lam_s) with Lam_t = sum_{r<=t} lam_r;
# an initial state enters with exp(Lam_t).  Numerator and denominator decay alike, so
# y_t stays a convex combination (the output gate of [TS-2.1]).


def forward_decay_quadratic(q, k, v, P, lam, S0=None, z0=None):
    """Decay-gated causal KATA by its O(T^2) definition (see the reading above).

    q, k: [B, H, T, d]; v: [B, H, T, dv]; P: [H, p, d]; lam: [B, H, T] log-gates (<= 0);
    S0 [B, H, p*p, dv], z0 [B, H, p*p] or None.  Returns y [B, H, T, dv] float64.
    """
    q = np.asarray(q, dtype=np.float64); k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64); P = np.asarray(P, dtype=np.float64)
    lam = np.asarray(lam, dtype=np.float64)
    B, H, T, _ = q.shape
    dv = v.shape[-1]
    pp = P.shape[1] * P.shape[1]
    y = np.zeros((B, H, T, dv))
    causal = np.tril(np.ones((T, T), dtype=bool))
    for b in range(B):
        for h in range(H):
            u = project(q[b, h], P[h])
            w = project(k[b, h], P[h])
            Lam = np.cumsum(lam[b, h])
            decay = np.where(causal, np.exp(np.where(causal, Lam[:, None] - Lam[None, :], 0.0)), 0.0)
            a = (u @ w.T) ** 2 * decay
            num = a @ v[b, h]
            den = a.sum(axis=1)
            if S0 is not None:
                f = feature_full(u) * np.exp(Lam)[:, None]
                num = num + f @ np.asarray(S0[b, h], dtype=np.float64)
                den = den + f @ np.asarray(z0[b, h], dtype=np.float64)
            ok = den != 0.0
            y[b, h][ok] = num[ok] / den[ok, None]
    return y


def final_state_decay(k, v, P, lam, S0=None, z0=None):
    """Final state of the decay-gated recurrence:
    S_T = exp(Lam_T) S0 + sum_s exp(Lam_T - Lam_s) phi(k_s) v_s^T, likewise z_T."""
    k = np.asarray(k, dtype=np.float64); v = np.asarray(v, dtype=np.float64)
    P = np.asarray(P, dtype=np.float64); lam = np.asarray(lam, dtype=np.float64)
    B, H, T, _ = k.shape
    pp = P.shape[1] * P.shape[1]
    ST = np.zeros((B, H, pp, v.shape[-1]))
    zT = np.zeros((B, H, pp))
    for b in range(B):
        for h in range(H):
            Lam = np.cumsum(lam[b, h])
            tot = Lam[-1] if T > 0 else 0.0
            wgt = np.exp(tot - Lam)                       # [T]
            f = feature_full(project(k[b, h], P[h]))      # [T, pp]
            ST[b, h] = (f * wgt[:, None]).T @ v[b, h]
            zT[b, h] = (f * wgt[:, None]).sum(axis=0)
            if S0 is not None:
                ST[b, h] += np.exp(tot) * np.asarray(S0[b, h], dtype=np.float64)
                zT[b, h] += np.exp(tot) * np.asarray(z0[b, h], dtype=np.float64)
    return ST, zT


def decode_decay_reference(S, z, q, k, v, P, lam):
    """One decay-gated recurrent decode step for N streams: S' = gamma S + phi(k) v^T,
    z' = gamma z + phi(k), gamma = exp(lam) [N, H]; y = S'^T phi(q) / (z' . phi(q))."""
    g = np.exp(np.asarray(lam, dtype=np.float64))
    S = np.array(S, dtype=np.float64) * g[:, :, None, None]
    z = np.array(z, dtype=np.float64) * g[:, :, None]
    return decode_reference(S, z, q, k, v, P)


# ---- DeltaKATA -------------------------------------------------------------------------
#
# PARITY NOTE (reading): [TS-4] and [ABS] name DeltaKATA (KATA with the delta rule; it
# corrects stale bindings under repeated-key overwrite) without defining it.  The plainest
# reading: the delta rule of DeltaNet with KATA's rank-one PSD feature normalised to unit
# norm (as DeltaNet normalises its keys and queries),
#
#     phi^(x) = vec(u u^T) / |u|^2,                 u = P x   (|phi^(x)| = 1)
#     S_t = S_{t-1} + beta_t phi^(k_t) (v_t - S_{t-1}^T phi^(k_t))^T,   beta_t in [0, 1]
#     y_t = S_t^T phi^(q_t)
#
# with no denominator (the delta rule replaces the normalisation); phi^(x) = 0 where u = 0.


def feature_unit(u):
    """phi^(u) = vec(u u^T) / |u|^2 (unit Frobenius norm; 0 for u = 0)."""
    u = np.asarray(u, dtype=np.float64)
    n2 = np.sum(u * u, axis=-1, keepdims=True)
    f = feature_full(u)
    return np.where(n2 > 0, f / np.where(n2 > 0, n2, 1.0), 0.0)


def delta_recurrence(q, k, v, P, beta, S0=None):
    """DeltaKATA by its token recurrence (see the reading above).

    q, k: [B, H, T, d]; v: [B, H, T, dv]; P: [H, p, d]; beta: [B, H, T]; S0 [B, H, p*p, dv]
    or None.  Returns (y [B, H, T, dv], S_T [B, H, p*p, dv]).
    """
    q = np.asarray(q, dtype=np.float64); k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64); P = np.asarray(P, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    B, H, T, _ = q.shape
    dv = v.shape[-1]
    pp = P.shape[1] * P.shape[1]
    y = np.zeros((B, H, T, dv))
    ST = np.zeros((B, H, pp, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((pp, dv)) if S0 is None else np.array(S0[b, h], dtype=np.float64)
            fq = feature_unit(project(q[b, h], P[h]))
            fk = feature_unit(project(k[b, h], P[h]))
            for t in range(T):
                e = v[b, h, t] - S.T @ fk[t]
                S = S + beta[b, h, t] * np.outer(fk[t], e)
                y[b, h, t] = S.T @ fq[t]
            ST[b, h] = S
    return y, ST


def delta_decode_reference(S, q, k, v, P, beta):
    """One DeltaKATA decode step for N streams: S' = S + beta phi^(k) (v - S^T phi^(k))^T,
    y = S'^T phi^(q).  S [N, H, p*p, dv]; q, k [N, H, d]; v [N, H, dv]; beta [N, H].
    Returns (y, S')."""
    S = np.array(S, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64); k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64); P = np.asarray(P, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    N, H = q.shape[:2]
    y = np.zeros(v.shape)
    for h in range(H):
        fq = feature_unit(project(q[:, h], P[h]))
        fk = feature_unit(project(k[:, h], P[h]))
        e = v[:, h] - np.einsum("nf,nfc->nc", fk, S[:, h])
        S[:, h] = S[:, h] + beta[:, h, None, None] * fk[:, :, None] * e[:, None, :]
        y[:, h] = np.einsum("nf,nfc->nc", fq, S[:, h])
    return y, S


# ---- KATA-Mg and KATA-Sigma-g ----------------------------------------------------------
#
# PARITY NOTE (reading): [TS-2.3v] names two variants with g PSD factors, "several" (Mg) and
# "summed" (Sigma-g), trading state size against packing efficiency, without defining
# them.  With g projections P_1..P_g per head (P [H, g, p, d]) and u_i = P_i q, w_i = P_i k:
#
#   Mg      phi(x) = [vec(u_1 u_1^T); ...; vec(u_g u_g^T)]     state g*p*p x dv
#           a_ts = sum_i (u_i,t . w_i,s)^2
#   Sigma-g phi(x) = vec(sum_i u_i u_i^T)                      state p*p x dv
#           a_ts = sum_i sum_j (u_i,t . w_j,s)^2
#
# and y_t = sum_s a_ts v_s / sum_s a_ts over s <= t as for KATA (g = 1 is KATA itself in
# both).  Initial and final states are in the layouts above (Mg: factor-major blocks of
# p*p rows).


def factor_projections(x, P):
    """u_i = P_i x for every factor: x [..., d], P [g, p, d] -> [g, ..., p]."""
    x = np.asarray(x, dtype=np.float64)
    P = np.asarray(P, dtype=np.float64)
    return np.stack([x @ P[i].T for i in range(P.shape[0])])


def _gate(num, den):
    return np.where(den[:, None] != 0, num / np.where(den[:, None] != 0, den[:, None], 1.0), 0.0)


def forward_mg_quadratic(q, k, v, P, S0=None, z0=None):
    """KATA-Mg by its O(T^2) definition.  q, k [B,H,T,d]; v [B,H,T,dv]; P [H,g,p,d];
    S0 [B,H,g*p*p,dv], z0 [B,H,g*p*p] or None.  Returns y [B,H,T,dv]."""
    q = np.asarray(q, dtype=np.float64); k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64); P = np.asarray(P, dtype=np.float64)
    B, H, T, _ = q.shape
    G, p = P.shape[1], P.shape[2]
    y = np.zeros(v.shape)
    mask = np.tril(np.ones((T, T))) > 0
    for b in range(B):
        for h in range(H):
            U = factor_projections(q[b, h], P[h])     # [g, T, p]
            W = factor_projections(k[b, h], P[h])
            a = np.zeros((T, T))
            for i in range(G):
                a += (U[i] @ W[i].T) ** 2
            a = np.where(mask, a, 0.0)
            num = a @ v[b, h]
            den = a.sum(axis=1)
            if S0 is not None:
                fq = np.concatenate([feature_full(U[i]) for i in range(G)], axis=1)
                num = num + fq @ np.asarray(S0[b, h], dtype=np.float64)
                den = den + fq @ np.asarray(z0[b, h], dtype=np.float64)
            y[b, h] = _gate(num, den)
    return y


def final_state_mg(k, v, P, S0=None, z0=None):
    """S_T = S0 + sum_s phi(k_s) v_s^T, z_T = z0 + sum_s phi(k_s) with the concatenated
    feature of KATA-Mg; [B,H,g*p*p,dv] and [B,H,g*p*p]."""
    k = np.asarray(k, dtype=np.float64); v = np.asarray(v, dtype=np.float64)
    P = np.asarray(P, dtype=np.float64)
    B, H, T, _ = k.shape
    G, p = P.shape[1], P.shape[2]
    S = np.zeros((B, H, G * p * p, v.shape[-1]))
    z = np.zeros((B, H, G * p * p))
    for b in range(B):
        for h in range(H):
            W = factor_projections(k[b, h], P[h])
            f = np.concatenate([feature_full(W[i]) for i in range(G)], axis=1)
            S[b, h] = f.T @ v[b, h]
            z[b, h] = f.sum(axis=0)
    if S0 is not None:
        S = S + S0
        z = z + z0
    return S, z


def recurrence_mg(q, k, v, P):
    """KATA-Mg by the token loop over the concatenated state (small inputs)."""
    q = np.asarray(q, dtype=np.float64); k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64); P = np.asarray(P, dtype=np.float64)
    B, H, T, _ = q.shape
    G, p = P.shape[1], P.shape[2]
    y = np.zeros(v.shape)
    for b in range(B):
        for h in range(H):
            S = np.zeros((G * p * p, v.shape[-1]))
            z = np.zeros(G * p * p)
            for t in range(T):
                fk = np.concatenate([np.outer(P[h, i] @ k[b, h, t], P[h, i] @ k[b, h, t]).ravel() for i in range(G)])
                fq = np.concatenate([np.outer(P[h, i] @ q[b, h, t], P[h, i] @ q[b, h, t]).ravel() for i in range(G)])
                S += np.outer(fk, v[b, h, t])
                z += fk
                den = fq @ z
                y[b, h, t] = (fq @ S) / den if den != 0 else 0.0
    return y


def _feature_sum(X):
    """vec(sum_i x_i x_i^T) for X [g, n, p] -> [n, p*p]."""
    return sum(feature_full(X[i]) for i in range(X.shape[0]))


def forward_sg_quadratic(q, k, v, P, S0=None, z0=None):
    """KATA-Sigma-g by its O(T^2) definition.  P [H,g,p,d]; S0 [B,H,p*p,dv], z0 [B,H,p*p]
    or None.  Returns y [B,H,T,dv]."""
    q = np.asarray(q, dtype=np.float64); k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64); P = np.asarray(P, dtype=np.float64)
    B, H, T, _ = q.shape
    G = P.shape[1]
    y = np.zeros(v.shape)
    mask = np.tril(np.ones((T, T))) > 0
    for b in range(B):
        for h in range(H):
            U = factor_projections(q[b, h], P[h])
            W = factor_projections(k[b, h], P[h])
            a = np.zeros((T, T))
            for i in range(G):
                for j in range(G):
                    a += (U[i] @ W[j].T) ** 2
            a = np.where(mask, a, 0.0)
            num = a @ v[b, h]
            den = a.sum(axis=1)
            if S0 is not None:
                fq = _feature_sum(U)
                num = num + fq @ np.asarray(S0[b, h], dtype=np.float64)
                den = den + fq @ np.asarray(z0[b, h], dtype=np.float64)
            y[b, h] = _gate(num, den)
    return y


def final_state_sg(k, v, P, S0=None, z0=None):
    """Final state of KATA-Sigma-g: S_T = S0 + sum_s vec(sum_i w_i w_i^T) v_s^T, z_T likewise."""
    k = np.asarray(k, dtype=np.float64); v = np.asarray(v, dtype=np.float64)
    P = np.asarray(P, dtype=np.float64)
    B, H, T, _ = k.shape
    p = P.shape[2]
    S = np.zeros((B, H, p * p, v.shape[-1]))
    z = np.zeros((B, H, p * p))
    for b in range(B):
        for h in range(H):
            f = _feature_sum(factor_projections(k[b, h], P[h]))
            S[b, h] = f.T @ v[b, h]
            z[b, h] = f.sum(axis=0)
    if S0 is not None:
        S = S + S0
        z = z + z0
    return S, z


def recurrence_sg(q, k, v, P):
    """KATA-Sigma-g by the token loop over the p*p state (small inputs)."""
    q = np.asarray(q, dtype=np.float64); k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64); P = np.asarray(P, dtype=np.float64)
    B, H, T, _ = q.shape
    G, p = P.shape[1], P.shape[2]
    y = np.zeros(v.shape)
    for b in range(B):
        for h in range(H):
            S = np.zeros((p * p, v.shape[-1]))
            z = np.zeros(p * p)
            for t in range(T):
                Mk = sum(np.outer(P[h, i] @ k[b, h, t], P[h, i] @ k[b, h, t]) for i in range(G))
                Mq = sum(np.outer(P[h, i] @ q[b, h, t], P[h, i] @ q[b, h, t]) for i in range(G))
                S += np.outer(Mk.ravel(), v[b, h, t])
                z += Mk.ravel()
                den = Mq.ravel() @ z
                y[b, h, t] = (Mq.ravel() @ S) / den if den != 0 else 0.0
    return y


def decode_factors_reference(S, z, q, k, v, P, mode):
    """One decode step of KATA-Mg (mode "concat") or KATA-Sigma-g (mode "sum") for N
    streams: the token's feature is folded into the state, then read out (as the one-factor
    step).  S [N,H,R,dv], z [N,H,R] with R = g*p*p (concat, factor-major) or p*p (sum);
    q, k [N,H,d]; v [N,H,dv]; P [H,g,p,d].  Returns (y, S', z')."""
    S = np.array(S, dtype=np.float64)
    z = np.array(z, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64); k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64); P = np.asarray(P, dtype=np.float64)
    N, H = q.shape[:2]
    y = np.zeros(v.shape)
    for h in range(H):
        U = factor_projections(q[:, h], P[h])      # [g, N, p]
        W = factor_projections(k[:, h], P[h])
        if mode == "concat":
            fq = np.concatenate([feature_full(U[i]) for i in range(U.shape[0])], axis=1)
            fk = np.concatenate([feature_full(W[i]) for i in range(W.shape[0])], axis=1)
        else:
            fq = _feature_sum(U)
            fk = _feature_sum(W)
        S[:, h] += fk[:, :, None] * v[:, h, None, :]
        z[:, h] += fk
        num = np.einsum("nf,nfc->nc", fq, S[:, h])
        den = np.einsum("nf,nf->n", fq, z[:, h])
        y[:, h] = np.where(den[:, None] != 0, num / np.where(den[:, None] != 0, den[:, None], 1.0), 0.0)
    return y, S, z
