"""Ill-conditioned output gates, built on purpose, against the fp64 oracle.

The gate divides by den_t = sum_s (u_t . w_s)^2.  Where den_t is a small fraction r_t of
sum_s |u_t|^2 |w_s|^2 (the query nearly orthogonal to the keys it sees), y_t rests on
weights that are small differences of large products, and a path with 8-bit operands
loses them.  Random inputs rarely do this except with very few keys, so the inputs here
are constructed: per (batch row, head) the keys' projections w = P k lie in a random
4-dimensional subspace of R^16 and the queries' projections u = P q lie almost in its
orthogonal complement, u = u_perp + eps u_par, so every query of the sequence, however
many keys it sees (in its own chunk, in earlier chunks, in an initial state), has r_t of
about eps^2 / 16.  q and k carry random components in the null space of P as well, so
they look like ordinary 64-dim inputs; the bf16 rounding of q and k moves u and w off the
subspaces by about 2^-9, which sets a floor of a few 1e-6 on r_t.

What each compute type holds to the bf16 bar (2e-2, normwise per (batch row, head)):
  * KATA_BF16 (the default): the score tiles take u and w as hi/lo pairs, so keys in the
    query's own chunk give the right y_t at any r_t (down to the 1e-6 floor); keys read
    through a state (earlier chunks, an initial state) go through single-bf16 features and
    state, fine for the gates of random inputs and for these structured keys at eps = 1
    (r_t about 6e-2), not for much worse.  The flash forward (no state) holds at any r_t.
  * KATA_BF16_HILO (precise=True) and float32 inputs: features and state as hi/lo pairs too,
    state-carried keys down to r_t around 1e-3 (eps = 0.2 and 0.1 here).
  * The decode steps (float32 state and arithmetic) from such a state.
"""
import numpy as np
import pytest
import torch

import kernelized_linear_attention_kata_amd as kata
from oracle import kata_oracle as O

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = 2e-2


def bf16_host64(t):
    bits = t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")
    return O.bf16_bits_to_f64(bits)


def subspace_tokens(B, H, T, P, eps, rng, d=64):
    """q, k, v [B, H, T, d] float64 with P k in a 4-dim subspace and P q almost orthogonal
    to it (P [H, 16, d]); the subspace is drawn per (b, h) from rng."""
    q = np.zeros((B, H, T, d))
    k = np.zeros((B, H, T, d))
    for h in range(H):
        Pp = np.linalg.pinv(P[h])                      # d x 16
        N = np.eye(d) - Pp @ P[h]                      # projector onto the null space of P_h
        for b in range(B):
            Qr, _ = np.linalg.qr(rng.standard_normal((16, 16)))
            Ksub, Qsub = Qr[:, :4], Qr[:, 4:]
            w = (rng.standard_normal((T, 4)) / 4) @ Ksub.T
            u = (rng.standard_normal((T, 12)) / 4) @ Qsub.T + eps * (rng.standard_normal((T, 4)) / 4) @ Ksub.T
            k[b, h] = w @ Pp.T + (rng.standard_normal((T, d)) / 8) @ N.T
            q[b, h] = u @ Pp.T + (rng.standard_normal((T, d)) / 8) @ N.T
    v = rng.standard_normal((B, H, T, d)) / 8
    return q, k, v


def make_case(B, H, T, eps, seed, T0=0):
    """bf16 tokens (T0 prefix tokens first, then T) of the subspace construction, one P per
    head, as torch CPU tensors, with their exact float64 values."""
    rng = np.random.default_rng(seed)
    P = rng.standard_normal((H, 16, 64)) / 8
    q, k, v = subspace_tokens(B, H, T0 + T, P, eps, rng)
    tq, tk, tv = (torch.from_numpy(x).float().to(torch.bfloat16) for x in (q, k, v))
    Pt = torch.from_numpy(P).float()
    return tq, tk, tv, Pt


def gate_ratios(qh, kh, Ph, S0k=None):
    """r_t = den_t / sum_s |u_t|^2 |w_s|^2 per query [B, H, T] (S0k: prefix keys)."""
    B, H, T, _ = qh.shape
    r = np.zeros((B, H, T))
    for b in range(B):
        for h in range(H):
            U = qh[b, h] @ Ph[h].T
            K = kh[b, h] if S0k is None else np.concatenate([S0k[b, h], kh[b, h]])
            W = K @ Ph[h].T
            n0 = 0 if S0k is None else S0k.shape[2]
            a = (U @ W.T) ** 2
            mask = np.arange(W.shape[0])[None, :] <= n0 + np.arange(T)[:, None]
            den = (a * mask).sum(1)
            scale = (U * U).sum(1) * ((W * W).sum(1)[None, :] * mask).sum(1)
            r[b, h] = den / scale
    return r


def slice_rel(got, ref):
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    g = g.reshape(g.shape[0] * g.shape[1], -1)
    r = r.reshape(r.shape[0] * r.shape[1], -1)
    den = np.linalg.norm(r, axis=1)
    return float(np.max(np.linalg.norm(g - r, axis=1) / np.where(den == 0, 1.0, den)))


@pytest.mark.parametrize("T,eps,precise", [(40, 0.03, False), (40, 0.0, False), (200, 1.0, False),
                                            (200, 0.1, True), (333, 0.2, True)])
def test_forward_ill_conditioned(T, eps, precise):
    """No initial state: T = 40 keeps every key in the query's chunk (score tiles only);
    T = 200 and 333 carry keys across chunks (running state, readout)."""
    q, k, v, P = make_case(2, 3, T, eps, seed=int(1000 * eps) + T)
    qh, kh, vh = (bf16_host64(t) for t in (q, k, v))
    Ph = P.double().numpy()
    r = gate_ratios(qh, kh, Ph)
    y, ST, zT = kata.forward(*(t.to(DEV) for t in (q, k, v, P)), 64, return_state=True, out_dtype=torch.float32,
                             precise=precise)
    torch.cuda.synchronize()
    yr = O.forward_quadratic(qh, kh, vh, Ph)
    Sr, zr = O.final_state(kh, vh, Ph)
    ey, eS, ez = slice_rel(y.cpu().numpy(), yr), slice_rel(ST.cpu().numpy(), Sr), slice_rel(zT.cpu().numpy(), zr)
    print(f"[ill-conditioned forward T={T} eps={eps} precise={precise}] median r {np.median(r[:, :, 1:]):.1e} "
          f"min r {r[:, :, 1:].min():.1e}: y {ey:.2e} S {eS:.2e} z {ez:.2e}", flush=True)
    assert np.median(r[:, :, 1:]) < (1e-3 if eps < 0.05 else (1e-2 if eps < 0.5 else 1e-1))
    assert ey <= TOL and eS <= TOL and ez <= TOL


@pytest.mark.parametrize("source", ["oracle", "export"])
@pytest.mark.parametrize("mode,eps", [("bf16", 1.0), ("precise", 0.2), ("f32", 0.2)])
def test_forward_ill_conditioned_from_state(source, mode, eps):
    """40 tokens from an initial state built over a 100-token prefix of subspace keys, by
    the oracle (exact) or by the forward's own state export (same compute type); f32 runs
    the same values as float32 inputs (every operand hi/lo)."""
    T0, T = 100, 40
    q, k, v, P = make_case(2, 3, T, eps, seed=77, T0=T0)
    qh, kh, vh = (bf16_host64(t) for t in (q, k, v))
    Ph = P.double().numpy()
    if mode == "f32":
        q, k, v = (t.float() for t in (q, k, v))                # the same values, stored as float32
    precise = mode == "precise"
    if source == "oracle":
        S0n, z0n = O.final_state(kh[:, :, :T0], vh[:, :, :T0], Ph)
        S0, z0 = torch.from_numpy(S0n).float().to(DEV), torch.from_numpy(z0n).float().to(DEV)
    else:
        _, S0, z0 = kata.forward(*(t[:, :, :T0].contiguous().to(DEV) for t in (q, k, v)), P.to(DEV), 64,
                                 return_state=True, precise=precise)
    qs, ks, vs = (t[:, :, T0:].contiguous() for t in (q, k, v))
    y = kata.forward(qs.to(DEV), ks.to(DEV), vs.to(DEV), P.to(DEV), 64, S0=S0, z0=z0, out_dtype=torch.float32,
                     precise=precise)
    torch.cuda.synchronize()
    yr = O.forward_quadratic(qh, kh, vh, Ph)[:, :, T0:]
    r = gate_ratios(qh[:, :, T0:], kh[:, :, T0:], Ph, S0k=kh[:, :, :T0])
    ey = slice_rel(y.cpu().numpy(), yr)
    print(f"[ill-conditioned forward from {source} state, {mode}] median r {np.median(r):.1e}: y {ey:.2e}",
          flush=True)
    assert ey <= TOL


def test_flash_and_decay_ill_conditioned():
    """The flash forward (no state) at eps = 0.03 (r_t around 7e-5); the decay-gated forward
    (single-bf16 state) at eps = 1."""
    T = 200
    qd_, kd_, vd_, Pd_ = make_case(2, 3, T, 0.03, seed=78)
    qh, kh, vh = (bf16_host64(t) for t in (qd_, kd_, vd_))
    Ph = Pd_.double().numpy()
    yf = kata.flash_forward(*(t.to(DEV) for t in (qd_, kd_, vd_, Pd_)), out_dtype=torch.float32)
    qm, km, vm, Pm = make_case(2, 3, T, 1.0, seed=79)
    qmh, kmh, vmh = (bf16_host64(t) for t in (qm, km, vm))
    lam = torch.log(torch.rand((2, 3, T), generator=torch.Generator().manual_seed(78)) * 0.1 + 0.9)
    ydc = kata.forward_decay(*(t.to(DEV) for t in (qm, km, vm, Pm)), lam.to(DEV), 64, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ef = slice_rel(yf.cpu().numpy(), O.forward_quadratic(qh, kh, vh, Ph))
    ed = slice_rel(ydc.cpu().numpy(), O.forward_decay_quadratic(qmh, kmh, vmh, Pm.double().numpy(),
                                                                lam.double().numpy()))
    print(f"[ill-conditioned T={T}] flash y {ef:.2e} (eps 0.03), decay y {ed:.2e} (eps 1)", flush=True)
    assert ef <= TOL and ed <= TOL


def test_decode_steps_ill_conditioned():
    """Canonical and packed decode steps from the precise forward's export over 100
    subspace tokens (eps = 0.2), then 8 steps whose queries are nearly orthogonal to every
    key."""
    T0, T = 100, 8
    q, k, v, P = make_case(4, 3, T, 0.2, seed=80, T0=T0)
    qh, kh, vh = (bf16_host64(t) for t in (q, k, v))
    Ph = P.double().numpy()
    Pd = P.to(DEV)
    _, S, z = kata.forward(*(t[:, :, :T0].contiguous().to(DEV) for t in (q, k, v)), Pd, 64, return_state=True,
                           precise=True)
    Sp, zp = kata.state_pack(S, z)
    Sr, zr = O.final_state(kh[:, :, :T0], vh[:, :, :T0], Ph)
    worst = 0.0
    for t in range(T0, T0 + T):
        qt, kt, vt = (x[:, :, t].contiguous().to(DEV) for x in (q, k, v))
        yc = kata.decode_step(S, z, qt, kt, vt, Pd)
        yp = kata.decode_step_packed(Sp, zp, qt, kt, vt, Pd)
        torch.cuda.synchronize()
        yr, Sr, zr = O.decode_reference(Sr, zr, qh[:, :, t], kh[:, :, t], vh[:, :, t], Ph)
        for got in (yc, yp):
            worst = max(worst, slice_rel(got.cpu().numpy()[:, :, None], yr[:, :, None]))
    print(f"[ill-conditioned decode] y {worst:.2e}", flush=True)
    assert worst <= TOL


@pytest.mark.parametrize("T", [1, 63, 200, 4096])
def test_precise_mode_on_random_inputs(T):
    """KATA_BF16_HILO on the mid workload's inputs: the oracle at the bf16 bar, with an
    initial state, chunks 32, 64 and 128 (its own leaf plan at two workgroups per compute
    unit), and no worse than the default mode."""
    from kernelized_linear_attention_kata_amd import inputs as I
    case = I.make_forward("mid", B=2, H=4, T=T, seed=81)
    pre = I.make_forward("mid", B=2, H=4, T=50, seed=82)
    qh, kh, vh = (bf16_host64(t) for t in (case.q, case.k, case.v))
    Ph = case.P.double().numpy()
    S0n, z0n = O.final_state(bf16_host64(pre.k), bf16_host64(pre.v), Ph)
    S0, z0 = torch.from_numpy(S0n).float().to(DEV), torch.from_numpy(z0n).float().to(DEV)
    yr = O.forward_quadratic(qh, kh, vh, Ph, S0n, z0n)
    Sr, zr = O.final_state(kh, vh, Ph, S0n, z0n)
    q, k, v, P = (t.to(DEV) for t in (case.q, case.k, case.v, case.P))
    for chunk in (32, 64, 128):
        e = {}
        for precise in (False, True):
            y, ST, zT = kata.forward(q, k, v, P, chunk, S0=S0, z0=z0, return_state=True, out_dtype=torch.float32,
                                     precise=precise)
            torch.cuda.synchronize()
            e[precise] = (slice_rel(y.cpu().numpy(), yr), slice_rel(ST.cpu().numpy(), Sr),
                          slice_rel(zT.cpu().numpy(), zr))
        print(f"[random T={T} C={chunk}] default y {e[False][0]:.2e} S {e[False][1]:.2e}; "
              f"precise y {e[True][0]:.2e} S {e[True][1]:.2e}", flush=True)
        assert max(e[True]) <= TOL
        assert e[True][0] <= 1.5 * e[False][0] + 1e-4
