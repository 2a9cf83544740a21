"""KATA-Mg (kata_forward_factors, concatenated PSD factors) against the oracle's O(T^2)
definition, its final state against the oracle's, and against the one-factor path.
Tolerance as for the one-factor forward: normwise relative error per row of y (per
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


def run(case, P, **kw):
    q, k, v = (t.to(DEV) for t in (case.q, case.k, case.v))
    out = kata.forward_factors(q, k, v, P.to(DEV), "concat", **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("g", [2, 3])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 300, 1000])
def test_mg_against_oracle(g, T):
    """Ragged T: one token, under, at and over one chunk, several chunks and leaves."""
    case = I.make_forward("mid", B=2, H=3, T=T, seed=90 + T)
    P = I.make_factor_projections(3, g, seed=T + g, per_head=True)
    y = run(case, P, out_dtype=torch.float32).double().cpu().numpy()
    ref = O.forward_mg_quadratic(host64(case.q), host64(case.k), host64(case.v), P.double().numpy())
    e = row_rel(y, ref)
    print(f"[mg g={g} T={T}] rel y {e:.3e}", flush=True)
    assert e <= TOL


def test_mg_state_in_and_out():
    """An initial state (the oracle's Mg final state of a prefix) and the final-state
    export, against the oracle; bf16 output."""
    g = 2
    P = I.make_factor_projections(2, g, seed=91, per_head=True)
    pre = I.make_forward("mid", B=2, H=2, T=150, seed=91)
    S0, z0 = O.final_state_mg(host64(pre.k), host64(pre.v), P.double().numpy())
    case = I.make_forward("mid", B=2, H=2, T=700, seed=92)
    S0t, z0t = torch.from_numpy(S0).float().to(DEV), torch.from_numpy(z0).float().to(DEV)
    y, ST, zT = run(case, P, S0=S0t, z0=z0t, return_state=True)
    args = (host64(case.q), host64(case.k), host64(case.v), P.double().numpy())
    ref = O.forward_mg_quadratic(*args, S0, z0)
    Sref, zref = O.final_state_mg(*args[1:], S0, z0)
    ey = row_rel(y.double().cpu().numpy(), ref)
    eS = slice_rel(ST.double().cpu().numpy(), Sref)
    ez = slice_rel(zT.double().cpu().numpy(), zref)
    print(f"[mg state] y {ey:.3e} S_T {eS:.3e} z_T {ez:.3e}", flush=True)
    assert ey <= TOL and eS <= TOL and ez <= TOL


def test_mg_factor_states_are_one_factor_states():
    """Factor i's block of the exported state equals the one-factor forward's state with
    P_i (the same kernels on the same data, up to the order of fp32 sums)."""
    g = 2
    case = I.make_forward("mid", B=1, H=4, T=2000, seed=93)
    P = I.make_factor_projections(4, g, seed=93, per_head=True)
    _, ST, zT = run(case, P, out_dtype=torch.float32, return_state=True)
    q, k, v = (t.to(DEV) for t in (case.q, case.k, case.v))
    for i in range(g):
        _, S1, z1 = kata.forward(q, k, v, P[:, i].contiguous().to(DEV), chunk=64, return_state=True)
        torch.cuda.synchronize()
        Si = ST[:, :, i * 256:(i + 1) * 256]
        zi = zT[:, :, i * 256:(i + 1) * 256]
        eS = float((Si.double() - S1.double()).norm() / S1.double().norm())
        ez = float((zi.double() - z1.double()).norm() / z1.double().norm())
        assert eS <= 1e-5 and ez <= 1e-5, (i, eS, ez)


def test_mg_equal_factors_is_one_factor():
    """g equal factors give weights g (u.w)^2, which the gate cancels: y equals the
    one-factor forward's."""
    case = I.make_forward("mid", B=2, H=2, T=1500, seed=94)
    P1 = I.make_factor_projections(2, 1, seed=94, per_head=True)
    P = P1.expand(2, 2, 16, 64).contiguous()
    y = run(case, P, out_dtype=torch.float32)
    q, k, v = (t.to(DEV) for t in (case.q, case.k, case.v))
    y1 = kata.forward(q, k, v, P1[:, 0].contiguous().to(DEV), chunk=64, out_dtype=torch.float32)
    torch.cuda.synchronize()
    e = float((y.double() - y1.double()).norm() / y1.double().norm())
    print(f"[mg equal factors] {e:.2e}", flush=True)
    assert e <= 1e-3


def test_mg_one_factor_runs_plain_forward():
    case = I.make_forward("mid", B=1, H=2, T=500, seed=95)
    P = I.make_factor_projections(2, 1, seed=95, per_head=True)
    y = run(case, P)
    q, k, v = (t.to(DEV) for t in (case.q, case.k, case.v))
    y1 = kata.forward(q, k, v, P[:, 0].contiguous().to(DEV), chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(y, y1)


def test_mg_lm340m_workload():
    case = I.make_forward("lm340m", B=2, H=4, T=512, seed=96)
    P = I.make_factor_projections(4, 2, seed=96, per_head=True)
    y = run(case, P).double().cpu().numpy()
    ref = O.forward_mg_quadratic(host64(case.q), host64(case.k), host64(case.v), P.double().numpy())
    e = row_rel(y, ref)
    print(f"[mg lm340m] rel y {e:.3e}", flush=True)
    assert e <= TOL


def test_mg_long_prefix_and_final_state():
    """The long-context shape (B=1, H=16, T=131072) with two factors, in the launch
    configuration the benchmark uses: y on the first 2048 tokens against the oracle on
    that prefix, and the final state of all heads against the oracle's."""
    T = 131072
    case = I.make_forward("long", T=T, seed=97)
    P = I.make_factor_projections(16, 2, seed=97)
    y, ST, zT = run(case, P, return_state=True)
    m = 2048
    ref = O.forward_mg_quadratic(host64(case.q[:, :, :m]), host64(case.k[:, :, :m]), host64(case.v[:, :, :m]),
                                 P.double().numpy())
    ey = row_rel(y[:, :, :m].double().cpu().numpy(), ref)
    Sref, zref = O.final_state_mg(host64(case.k), host64(case.v), P.double().numpy())
    eS = slice_rel(ST.double().cpu().numpy(), Sref)
    ez = slice_rel(zT.double().cpu().numpy(), zref)
    print(f"[mg long] y prefix {ey:.3e} S_T {eS:.3e} z_T {ez:.3e}", flush=True)
    assert ey <= TOL and eS <= TOL and ez <= TOL
    assert torch.all(torch.isfinite(y.float()))


# ---- KATA-Sigma-g (summed PSD factors) ----------------------------------------------------

def run_sg(case, P, **kw):
    q, k, v = (t.to(DEV) for t in (case.q, case.k, case.v))
    out = kata.forward_factors(q, k, v, P.to(DEV), "sum", **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("g", [2, 3])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 300, 1000])
def test_sg_against_oracle(g, T):
    case = I.make_forward("mid", B=2, H=3, T=T, seed=100 + T)
    P = I.make_factor_projections(3, g, seed=50 + T + g, per_head=True)
    y = run_sg(case, P, out_dtype=torch.float32).double().cpu().numpy()
    ref = O.forward_sg_quadratic(host64(case.q), host64(case.k), host64(case.v), P.double().numpy())
    e = row_rel(y, ref)
    print(f"[sg g={g} T={T}] rel y {e:.3e}", flush=True)
    assert e <= TOL


def test_sg_state_in_and_out():
    g = 2
    P = I.make_factor_projections(2, g, seed=101, per_head=True)
    pre = I.make_forward("mid", B=2, H=2, T=150, seed=101)
    S0, z0 = O.final_state_sg(host64(pre.k), host64(pre.v), P.double().numpy())
    case = I.make_forward("mid", B=2, H=2, T=700, seed=102)
    S0t, z0t = torch.from_numpy(S0).float().to(DEV), torch.from_numpy(z0).float().to(DEV)
    y, ST, zT = run_sg(case, P, S0=S0t, z0=z0t, return_state=True)
    args = (host64(case.q), host64(case.k), host64(case.v), P.double().numpy())
    ref = O.forward_sg_quadratic(*args, S0, z0)
    Sref, zref = O.final_state_sg(*args[1:], S0, z0)
    ey = row_rel(y.double().cpu().numpy(), ref)
    eS = slice_rel(ST.double().cpu().numpy(), Sref)
    ez = slice_rel(zT.double().cpu().numpy(), zref)
    print(f"[sg state] y {ey:.3e} S_T {eS:.3e} z_T {ez:.3e}", flush=True)
    assert ey <= TOL and eS <= TOL and ez <= TOL


def test_sg_state_is_sum_of_factor_states():
    """The Sigma-g state equals the sum of the g one-factor states (same data)."""
    g = 3
    case = I.make_forward("mid", B=1, H=4, T=2000, seed=103)
    P = I.make_factor_projections(4, g, seed=103, per_head=True)
    _, ST, zT = run_sg(case, P, out_dtype=torch.float32, return_state=True)
    q, k, v = (t.to(DEV) for t in (case.q, case.k, case.v))
    S_sum = torch.zeros_like(ST)
    z_sum = torch.zeros_like(zT)
    for i in range(g):
        _, S1, z1 = kata.forward(q, k, v, P[:, i].contiguous().to(DEV), chunk=64, return_state=True)
        S_sum += S1
        z_sum += z1
    torch.cuda.synchronize()
    eS = float((ST.double() - S_sum.double()).norm() / S_sum.double().norm())
    ez = float((zT.double() - z_sum.double()).norm() / z_sum.double().norm())
    assert eS <= 1e-5 and ez <= 1e-5, (eS, ez)


def test_sg_factor_mixing_invariance():
    """y depends on the factors only through sum_i P_i^T P_i-type products: mixing the
    factors by an orthogonal g x g matrix leaves y unchanged (the cross terms must be
    right for this to hold)."""
    g = 2
    case = I.make_forward("mid", B=1, H=2, T=1500, seed=104)
    P = I.make_factor_projections(2, g, seed=104, per_head=True)
    c, s_ = np.cos(0.7), np.sin(0.7)
    R = torch.tensor([[c, -s_], [s_, c]], dtype=torch.float32)
    Pm = torch.einsum("ji,hjab->hiab", R, P).contiguous()
    y = run_sg(case, P, out_dtype=torch.float32)
    ym = run_sg(case, Pm, out_dtype=torch.float32)
    e = float((y.double() - ym.double()).norm() / y.double().norm())
    print(f"[sg mixing] {e:.2e}", flush=True)
    assert e <= 5e-3


def test_sg_equal_factors_is_one_factor():
    """g equal factors give weights g^2 (u.w)^2, which the gate cancels."""
    case = I.make_forward("mid", B=2, H=2, T=1500, seed=105)
    P1 = I.make_factor_projections(2, 1, seed=105, per_head=True)
    P = P1.expand(2, 2, 16, 64).contiguous()
    y = run_sg(case, P, out_dtype=torch.float32)
    q, k, v = (t.to(DEV) for t in (case.q, case.k, case.v))
    y1 = kata.forward(q, k, v, P1[:, 0].contiguous().to(DEV), chunk=64, out_dtype=torch.float32)
    torch.cuda.synchronize()
    e = float((y.double() - y1.double()).norm() / y1.double().norm())
    print(f"[sg equal factors] {e:.2e}", flush=True)
    assert e <= 1e-3


def test_sg_lm340m_workload():
    case = I.make_forward("lm340m", B=2, H=4, T=512, seed=106)
    P = I.make_factor_projections(4, 2, seed=106, per_head=True)
    y = run_sg(case, P).double().cpu().numpy()
    ref = O.forward_sg_quadratic(host64(case.q), host64(case.k), host64(case.v), P.double().numpy())
    e = row_rel(y, ref)
    print(f"[sg lm340m] rel y {e:.3e}", flush=True)
    assert e <= TOL


def test_sg_long_prefix_and_final_state():
    T = 131072
    case = I.make_forward("long", T=T, seed=107)
    P = I.make_factor_projections(16, 2, seed=107)
    y, ST, zT = run_sg(case, P, return_state=True)
    m = 2048
    ref = O.forward_sg_quadratic(host64(case.q[:, :, :m]), host64(case.k[:, :, :m]), host64(case.v[:, :, :m]),
                                 P.double().numpy())
    ey = row_rel(y[:, :, :m].double().cpu().numpy(), ref)
    Sref, zref = O.final_state_sg(host64(case.k), host64(case.v), P.double().numpy())
    eS = slice_rel(ST.double().cpu().numpy(), Sref)
    ez = slice_rel(zT.double().cpu().numpy(), zref)
    print(f"[sg long] y prefix {ey:.3e} S_T {eS:.3e} z_T {ez:.3e}", flush=True)
    assert ey <= TOL and eS <= TOL and ez <= TOL
    assert torch.all(torch.isfinite(y.float()))


# ---- decode steps (kata_decode_step_factors) --------------------------------------------

@pytest.mark.parametrize("mode", ["concat", "sum"])
@pytest.mark.parametrize("g", [2, 3])
def test_factor_decode_against_oracle_and_forward(mode, g):
    """Prefill by the chunked factor forward (state export), then decode steps: each step
    against the oracle's step from the same state, and against the forward over the whole
    sequence."""
    N, H, T0, steps = 3, 2, 150, 5
    case = I.make_forward("mid", B=N, H=H, T=T0 + steps, seed=130 + g)
    P = I.make_factor_projections(H, g, seed=130 + g, per_head=True).to(DEV)
    q, k, v = (t.to(DEV) for t in (case.q, case.k, case.v))
    yfull = kata.forward_factors(q, k, v, P, mode, out_dtype=torch.float32)
    _, S, z = kata.forward_factors(q[:, :, :T0].contiguous(), k[:, :, :T0].contiguous(), v[:, :, :T0].contiguous(),
                                   P, mode, return_state=True)
    torch.cuda.synchronize()
    Sh, zh = S.double().cpu().numpy(), z.double().cpu().numpy()
    Ph = P.double().cpu().numpy()
    for j in range(steps):
        t = T0 + j
        qs, ks, vs = (x[:, :, t].contiguous() for x in (q, k, v))
        yj = kata.decode_step_factors(S, z, qs, ks, vs, P, mode)
        torch.cuda.synchronize()
        yr, Sh, zh = O.decode_factors_reference(Sh, zh, host64(qs.cpu()), host64(ks.cpu()), host64(vs.cpu()), Ph,
                                                mode)
        e1 = row_rel(yj.double().cpu().numpy(), yr)
        e2 = row_rel(yj.double().cpu().numpy(), yfull[:, :, t].double().cpu().numpy())
        print(f"[factor decode {mode} g={g} step {j}] vs oracle {e1:.2e} vs forward {e2:.2e}", flush=True)
        assert e1 <= 1e-5 and e2 <= TOL, (j, e1, e2)
    eS = slice_rel(S.double().cpu().numpy(), Sh)
    assert eS <= 1e-5


def test_factor_decode_workload_sampled():
    """The decode workload's shape (256 streams x 16 heads) with two concatenated factors:
    one step from a seeded state, sampled streams against the oracle's step."""
    dc = I.make_decode(T_prefill=1, steps=1, seed=131)
    N, H = dc.N, dc.H
    P = I.make_factor_projections(H, 2, seed=131).to(DEV)
    g = torch.Generator().manual_seed(131)
    S = (torch.rand((N, H, 512, 64), generator=g) / 8).to(DEV)
    z = (torch.rand((N, H, 512), generator=g) + 0.5).to(DEV)
    S0, z0 = S.double().cpu().numpy(), z.double().cpu().numpy()
    qs, ks, vs = (x[0].to(DEV) for x in (dc.q, dc.k, dc.v))
    y = kata.decode_step_factors(S, z, qs, ks, vs, P, "concat")
    torch.cuda.synchronize()
    rng = np.random.default_rng(131)
    sel = [(0, 0), (N - 1, H - 1)] + [tuple(x) for x in rng.integers(0, [N, H], size=(4, 2))]
    for n, h in sel:
        yr, Sr, zr = O.decode_factors_reference(S0[n:n + 1, h:h + 1], z0[n:n + 1, h:h + 1],
                                                host64(dc.q[0, n:n + 1, h:h + 1]), host64(dc.k[0, n:n + 1, h:h + 1]),
                                                host64(dc.v[0, n:n + 1, h:h + 1]), P[h:h + 1].double().cpu().numpy(),
                                                "concat")
        assert row_rel(y[n:n + 1, h:h + 1].double().cpu().numpy(), yr) <= 1e-5
        assert slice_rel(S[n:n + 1, h:h + 1].double().cpu().numpy(), Sr) <= 1e-6
