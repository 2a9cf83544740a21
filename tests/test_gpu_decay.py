"""Decay-gated forward (kata_forward_decay) and decode step (kata_decode_step_decay)
against the oracle's decay-gated definition, and against the plain path and themselves.
Tolerance as for the plain forward: normwise relative error per row of y (and per
(b, h) slice of the state) <= 2e-2 for bf16 inputs."""
import numpy as np
import pytest
import torch

import kernelized_linear_attention_kata_amd as kata
from kernelized_linear_attention_kata_amd import inputs as I
from oracle import kata_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-2


def host64(t):
    return O.bf16_bits_to_f64(I.bf16_bits(t))


def row_rel(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref, axis=-1)
    return float(np.max(np.linalg.norm(got - ref, axis=-1) / np.where(den == 0, 1.0, den)))


def slice_rel(got, ref):
    g = np.asarray(got, dtype=np.float64).reshape(got.shape[0] * got.shape[1], -1)
    r = np.asarray(ref, dtype=np.float64).reshape(ref.shape[0] * ref.shape[1], -1)
    return float(np.max(np.linalg.norm(g - r, axis=1) / np.linalg.norm(r, axis=1)))


def run(case, lam, **kw):
    q, k, v, P = (t.to(DEV) for t in (case.q, case.k, case.v, case.P))
    out = kata.forward_decay(q, k, v, P, lam.to(DEV), chunk=64, **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("T", [1, 63, 64, 65, 300, 1000])
def test_decay_against_oracle(T):
    """Ragged T (one token, under, at and over one chunk, several chunks and leaves)."""
    case = I.make_forward("mid", B=2, H=3, T=T, seed=60 + T)
    lam = I.make_log_decay(2, 3, T, seed=T)
    y = run(case, lam, out_dtype=torch.float32).double().cpu().numpy()
    ref = O.forward_decay_quadratic(host64(case.q), host64(case.k), host64(case.v), case.P.double().numpy(),
                                    lam.double().numpy())
    e = row_rel(y, ref)
    print(f"[decay mid T={T}] rel y {e:.3e}", flush=True)
    assert e <= TOL


def test_decay_strong_gates_and_state():
    """Gates down to 0.3, an initial state (decayed like the rest) and the final-state
    export against the oracle; bf16 output."""
    pre = I.make_forward("mid", B=2, H=2, T=200, seed=70)
    S0, z0 = O.final_state(host64(pre.k), host64(pre.v), pre.P.double().numpy())
    case = I.make_forward("mid", B=2, H=2, T=777, seed=71)
    lam = I.make_log_decay(2, 2, 777, seed=71, lo=0.3, hi=1.0)
    S0t, z0t = torch.from_numpy(S0).float().to(DEV), torch.from_numpy(z0).float().to(DEV)
    y, ST, zT = run(case, lam, S0=S0t, z0=z0t, return_state=True)
    args = (host64(case.q), host64(case.k), host64(case.v), case.P.double().numpy(), lam.double().numpy())
    ref = O.forward_decay_quadratic(*args, S0, z0)
    Sref, zref = O.final_state_decay(*args[1:], S0, z0)
    ey = row_rel(y.double().cpu().numpy(), ref)
    eS = slice_rel(ST.double().cpu().numpy(), Sref)
    ez = slice_rel(zT.double().cpu().numpy(), zref)
    print(f"[decay strong+state] y {ey:.3e} S_T {eS:.3e} z_T {ez:.3e}", flush=True)
    assert ey <= TOL and eS <= TOL and ez <= TOL


def test_decay_no_gate_equals_plain_forward():
    """lam = 0 reproduces the plain chunked forward."""
    case = I.make_forward("mid", B=2, H=4, T=2000, seed=72)
    lam = torch.zeros((2, 4, 2000), dtype=torch.float32)
    yd, Sd, zd = run(case, lam, out_dtype=torch.float32, return_state=True)
    q, k, v, P = (t.to(DEV) for t in (case.q, case.k, case.v, case.P))
    yp, Sp, zp = kata.forward(q, k, v, P, chunk=64, out_dtype=torch.float32, return_state=True)
    torch.cuda.synchronize()
    for a, b in ((yd, yp), (Sd, Sp), (zd, zp)):
        e = float((a.double() - b.double()).norm() / b.double().norm())
        assert e <= 1e-6, e


def test_decay_scan_modes_agree():
    """The affine scan over leaves: auto, 1 and 5 chunks per leaf and the sequential mode
    agree up to the order of fp32 sums."""
    case = I.make_forward("mid", B=1, H=2, T=3000, seed=73)
    lam = I.make_log_decay(1, 2, 3000, seed=73, lo=0.5)
    base, Sb, zb = run(case, lam, out_dtype=torch.float32, return_state=True)
    for kw in (dict(scan_leaf=1), dict(scan_leaf=5), dict(scan="sequential")):
        y, S, z = run(case, lam, out_dtype=torch.float32, return_state=True, **kw)
        for a, b in ((y, base), (S, Sb), (z, zb)):
            e = float((a.double() - b.double()).norm() / b.double().norm())
            print(f"[decay scan {kw}] {e:.2e}", flush=True)
            assert e <= 1e-4, (kw, e)


def test_decay_lm340m_workload():
    case = I.make_forward("lm340m", B=2, H=4, T=512, seed=74)
    lam = I.make_log_decay(2, 4, 512, seed=74)
    y = run(case, lam).double().cpu().numpy()
    ref = O.forward_decay_quadratic(host64(case.q), host64(case.k), host64(case.v), case.P.double().numpy(),
                                    lam.double().numpy())
    e = row_rel(y, ref)
    print(f"[decay lm340m] rel y {e:.3e}", flush=True)
    assert e <= TOL


def test_decay_long_prefix_and_final_state():
    """The long-context shape (B=1, H=16, T=131072) in the launch configuration the
    benchmark uses: y on the first 2048 tokens against the oracle on that prefix (y_t
    depends on tokens <= t only), and the final state against the oracle's O(T) form."""
    T = 131072
    case = I.make_forward("long", T=T, seed=75)
    lam = I.make_log_decay(1, 16, T, seed=75, lo=0.99, hi=1.0)
    y, ST, zT = run(case, lam, return_state=True)
    m = 2048
    ref = O.forward_decay_quadratic(host64(case.q[:, :, :m]), host64(case.k[:, :, :m]), host64(case.v[:, :, :m]),
                                    case.P.double().numpy(), lam[:, :, :m].double().numpy())
    ey = row_rel(y[:, :, :m].double().cpu().numpy(), ref)
    Sref, zref = O.final_state_decay(host64(case.k), host64(case.v), case.P.double().numpy(), lam.double().numpy())
    eS = slice_rel(ST.double().cpu().numpy(), Sref)
    ez = slice_rel(zT.double().cpu().numpy(), zref)
    print(f"[decay long] y prefix {ey:.3e} S_T {eS:.3e} z_T {ez:.3e}", flush=True)
    assert ey <= TOL and eS <= TOL and ez <= TOL
    assert torch.all(torch.isfinite(y.float()))


def test_decode_decay_against_oracle_and_forward():
    """The decay-gated decode step against the oracle's step, and a prefill by the
    chunked forward followed by decode steps against the forward over the whole sequence."""
    r = torch.Generator().manual_seed(76)
    N, H, T0, steps = 3, 2, 150, 6
    case = I.make_forward("mid", B=N, H=H, T=T0 + steps, seed=76)
    lam = I.make_log_decay(N, H, T0 + steps, seed=76, lo=0.5)
    q, k, v, P = (t.to(DEV) for t in (case.q, case.k, case.v, case.P))
    lamd = lam.to(DEV)
    yfull = kata.forward_decay(q, k, v, P, lamd, out_dtype=torch.float32)
    _, S, z = kata.forward_decay(q[:, :, :T0].contiguous(), k[:, :, :T0].contiguous(), v[:, :, :T0].contiguous(), P,
                                 lamd[:, :, :T0].contiguous(), return_state=True)
    Sh, zh = S.double().cpu().numpy(), z.double().cpu().numpy()
    for j in range(steps):
        t = T0 + j
        qs, ks, vs = (x[:, :, t].contiguous() for x in (q, k, v))
        ls = lamd[:, :, t].contiguous()
        yj = kata.decode_step_decay(S, z, qs, ks, vs, P, ls)
        torch.cuda.synchronize()
        yr, Sh, zh = O.decode_decay_reference(Sh, zh, host64(qs.cpu()), host64(ks.cpu()), host64(vs.cpu()),
                                              case.P.double().numpy(), ls.double().cpu().numpy())
        e1 = row_rel(yj.double().cpu().numpy(), yr)
        e2 = row_rel(yj.double().cpu().numpy(), yfull[:, :, t].double().cpu().numpy())
        assert e1 <= 1e-5 and e2 <= TOL, (j, e1, e2)
