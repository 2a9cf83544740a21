"""Backward of the chunked forward (kata_backward) against the oracle's gradients
(``backward_quadratic``, the chain rule through the O(T^2) definition, pinned by finite
differences), and against identities that hold at any size.

Tolerance.  The bound for bf16 inputs with fp32 accumulation is 2e-2, as for the
forward.  A gradient row can vanish by cancellation: dq_0 is exactly 0, since y_0 = v_0
does not depend on q_0.  A per-row relative error is therefore meaningless for
gradients.  Each (batch row, head) slice is instead compared normwise,
||got - ref||_F / ||ref||_F <= 2e-2.  A row-wise guard backs this up: every row's
error is at most 0.1 of the slice's RMS row norm, which catches a wrong tile or mask
that the normwise figure could average away.
"""
import numpy as np
import pytest
import torch

import kernelized_linear_attention_kata_amd as kata
from kernelized_linear_attention_kata_amd import inputs as I
from oracle import kata_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-2
ROW_TOL = 0.1


def host64(t):
    if t.dtype == torch.bfloat16:
        return O.bf16_bits_to_f64(I.bf16_bits(t))
    return t.detach().double().cpu().numpy()


def grad_err(got, ref):
    """(max normwise relative error, max row error / RMS row norm) over the leading
    (batch, head) slices."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    g2 = got.reshape(-1, got.shape[-2], got.shape[-1])
    r2 = ref.reshape(-1, ref.shape[-2], ref.shape[-1])
    rel, row = 0.0, 0.0
    for g, r in zip(g2, r2):
        nr = np.linalg.norm(r)
        if nr == 0:
            rel = max(rel, float(np.linalg.norm(g)))
            continue
        rel = max(rel, float(np.linalg.norm(g - r) / nr))
        rms = np.sqrt(np.mean(np.sum(r * r, axis=-1)))
        row = max(row, float(np.max(np.linalg.norm(g - r, axis=-1)) / rms))
    return rel, row


def run_case(case, out_dtype=torch.bfloat16, seed=0, S0=None, z0=None, gST=None, gzT=None, **kw):
    q, k, v, P = (t.to(DEV) for t in (case.q, case.k, case.v, case.P))
    S0d = None if S0 is None else S0.to(DEV)
    z0d = None if z0 is None else z0.to(DEV)
    gy = I.make_output_grad(case.B, case.H, case.T, case.dv, "bf16" if out_dtype == torch.bfloat16 else "f32",
                            seed=seed).to(DEV)
    want_state = gST is not None or S0 is not None
    res = kata.backward(q, k, v, P, gy, S0=S0d, z0=z0d, gST=None if gST is None else gST.to(DEV),
                        gzT=None if gzT is None else gzT.to(DEV), return_state_grad=want_state, **kw)
    torch.cuda.synchronize()
    ref = O.backward_quadratic(host64(case.q), host64(case.k), host64(case.v), case.P.double().numpy(),
                               host64(gy), None if S0 is None else S0.double().numpy(),
                               None if z0 is None else z0.double().numpy(),
                               None if gST is None else gST.double().numpy(),
                               None if gzT is None else gzT.double().numpy())
    return res, ref, gy


def check(res, ref, label):
    names = ("dq", "dk", "dv")
    out = {}
    for i, nm in enumerate(names):
        out[nm] = grad_err(res[i].double().cpu().numpy(), ref[i])
    dP = res[3].double().cpu().numpy()
    out["dP"] = (float(np.linalg.norm(dP - ref[3]) / np.linalg.norm(ref[3])), 0.0)
    print(f"[{label}] " + " ".join(f"{k} {a:.2e}/{b:.2e}" for k, (a, b) in out.items()), flush=True)
    for nm, (a, b) in out.items():
        assert a <= TOL, f"{label} {nm}: normwise {a}"
        assert b <= ROW_TOL, f"{label} {nm}: row {b}"
    return out


def test_backward_single_token():
    """T = 1: y_0 = v_0 exactly, so dv_0 = gy_0 and dq, dk, dP vanish.  On the GPU g . v_0
    and h_0 = -g . y_0 cancel up to rounding, so dq and dk are rounding noise: they are
    bounded against the natural scale of a gradient through one score,
    2 |gy| |v| |w| ||P|| / |u . w| (and |u| for dk)."""
    case = I.make_forward("mid", B=2, H=3, T=1, seed=41)
    res, ref, gy = run_case(case, seed=1)
    gyh = host64(gy)
    u = np.einsum("hpd,bhtd->bhtp", case.P.double().numpy(), host64(case.q))
    w = np.einsum("hpd,bhtd->bhtp", case.P.double().numpy(), host64(case.k))
    X = np.abs(np.sum(u * w, axis=-1))[..., 0]
    nP = np.linalg.norm(case.P.double().numpy()[0])
    base = 2 * np.linalg.norm(gyh[..., 0, :], axis=-1) * np.linalg.norm(host64(case.v)[..., 0, :], axis=-1) * nP / X
    sq = base * np.linalg.norm(w[..., 0, :], axis=-1)
    sk = base * np.linalg.norm(u[..., 0, :], axis=-1)
    eq = float(np.max(np.linalg.norm(res[0].double().cpu().numpy()[..., 0, :], axis=-1) / sq))
    ek = float(np.max(np.linalg.norm(res[1].double().cpu().numpy()[..., 0, :], axis=-1) / sk))
    ev = grad_err(res[2].double().cpu().numpy(), ref[2])[0]
    print(f"[bwd T=1] dq/scale {eq:.2e} dk/scale {ek:.2e} dv {ev:.2e}", flush=True)
    assert eq <= 1e-2 and ek <= 1e-2 and ev <= TOL


@pytest.mark.parametrize("T", [2, 63, 64, 65, 200, 1000])
def test_backward_against_oracle(T):
    """Ragged T: two tokens, under one chunk, one chunk, one chunk plus one, several."""
    case = I.make_forward("mid", B=2, H=3, T=T, seed=40 + T)
    res, ref, _ = run_case(case, seed=T)
    check(res, ref, f"bwd mid T={T}")


def test_backward_f32_output_and_many_leaves():
    """gy in float32; T = 2048 spans several leaves and chunks per leaf."""
    case = I.make_forward("mid", B=1, H=2, T=2048, seed=47)
    res, ref, _ = run_case(case, out_dtype=torch.float32, seed=7)
    check(res, ref, "bwd mid f32 y T=2048")


def test_backward_lm340m_workload():
    """Per-head P and unit-norm keys (the 340M-layer inputs)."""
    case = I.make_forward("lm340m", B=2, H=4, T=384, seed=48)
    res, ref, _ = run_case(case, seed=8)
    check(res, ref, "bwd lm340m T=384")


def test_backward_initial_state_and_state_gradient():
    """A symmetric initial state from an earlier segment, and a (non-symmetric)
    gradient of the final state: dS0, dz0 are the symmetric part of the oracle's."""
    pre = I.make_forward("mid", B=2, H=2, T=300, seed=49)
    S0, z0 = O.final_state(host64(pre.k), host64(pre.v), pre.P.double().numpy())
    S0 = torch.from_numpy(S0).float()
    z0 = torch.from_numpy(z0).float()
    case = I.make_forward("mid", B=2, H=2, T=333, seed=50)
    gST, gzT = I.make_state_grad(2, 2, 64, seed=3)
    res, ref, _ = run_case(case, seed=9, S0=S0, z0=z0, gST=gST, gzT=gzT)
    check(res, ref, "bwd with state T=333")
    dS0 = res[4].double().cpu().numpy().reshape(2, 2, 16, 16, 64)
    dz0 = res[5].double().cpu().numpy().reshape(2, 2, 16, 16)
    rS = ref[4].reshape(2, 2, 16, 16, 64)
    rz = ref[5].reshape(2, 2, 16, 16)
    symS = 0.5 * (rS + rS.transpose(0, 1, 3, 2, 4))
    symz = 0.5 * (rz + rz.transpose(0, 1, 3, 2))
    eS = np.linalg.norm(dS0 - symS) / np.linalg.norm(symS)
    ez = np.linalg.norm(dz0 - symz) / np.linalg.norm(symz)
    print(f"[bwd state grads] dS0 {eS:.2e} dz0 {ez:.2e}", flush=True)
    assert eS <= TOL and ez <= TOL
    # S mirror entries are one packed value; the z block's (a, b) and (b, a) entries are
    # separate MFMA results, equal up to rounding
    assert np.array_equal(dS0, dS0.transpose(0, 1, 3, 2, 4))
    assert np.max(np.abs(dz0 - dz0.transpose(0, 1, 3, 2))) <= 1e-6 * np.max(np.abs(dz0))


def test_backward_scan_modes_agree():
    """Associative leaves (auto, 1 chunk, 3 chunks) and the sequential scan give the same
    gradients up to the order of fp32 sums."""
    case = I.make_forward("mid", B=1, H=2, T=1500, seed=51)
    q, k, v, P = (t.to(DEV) for t in (case.q, case.k, case.v, case.P))
    gy = I.make_output_grad(1, 2, 1500, 64, seed=11).to(DEV)
    base = kata.backward(q, k, v, P, gy)
    for kw in (dict(scan_leaf=1), dict(scan_leaf=3), dict(scan="sequential")):
        other = kata.backward(q, k, v, P, gy, **kw)
        torch.cuda.synchronize()
        for a, b, nm in zip(base, other, ("dq", "dk", "dv", "dP")):
            e = float((a.double() - b.double()).norm() / b.double().norm())
            print(f"[bwd scan {kw}] {nm} {e:.2e}", flush=True)
            assert e <= 1e-2, (kw, nm, e)


def test_backward_sequence_split():
    """The state carries the gradient across a split: the backward of the second
    segment (from the first's final state) yields dS0, dz0, which fed as gST, gzT to the
    first segment's backward reproduce the whole sequence's gradients."""
    case = I.make_forward("mid", B=1, H=2, T=640, seed=52)
    q, k, v, P = (t.to(DEV) for t in (case.q, case.k, case.v, case.P))
    m = 320
    gy = I.make_output_grad(1, 2, 640, 64, dtype="f32", seed=12).to(DEV)
    full = kata.backward(q, k, v, P, gy)
    sl1 = [t[:, :, :m].contiguous() for t in (q, k, v)]
    sl2 = [t[:, :, m:].contiguous() for t in (q, k, v)]
    _, S1, z1 = kata.forward(*sl1, P, chunk=64, out_dtype=torch.float32, return_state=True)
    g2 = kata.backward(*sl2, P, gy[:, :, m:].contiguous(), S0=S1, z0=z1, return_state_grad=True)
    g1 = kata.backward(*sl1, P, gy[:, :, :m].contiguous(), gST=g2[4], gzT=g2[5])
    torch.cuda.synchronize()
    for i, nm in enumerate(("dq", "dk", "dv")):
        cat = torch.cat([g1[i], g2[i]], dim=2).double()
        e = float((cat - full[i].double()).norm() / full[i].double().norm())
        print(f"[bwd split] {nm} {e:.2e}", flush=True)
        assert e <= TOL
    e = float(((g1[3] + g2[3]).double() - full[3].double()).norm() / full[3].double().norm())
    assert e <= TOL


def test_backward_zero_query_rows():
    """u_t = 0 gives den_t = 0 and y_t = 0 (a constant): dq_t = 0, and gy_t is ignored."""
    case = I.make_forward("mid", B=1, H=2, T=300, seed=53)
    case.q[:, :, 0] = 0
    case.q[:, :, 150] = 0
    q, k, v, P = (t.to(DEV) for t in (case.q, case.k, case.v, case.P))
    gy = I.make_output_grad(1, 2, 300, 64, seed=13).to(DEV)
    a = kata.backward(q, k, v, P, gy)
    gy2 = gy.clone()
    gy2[:, :, 150] = 7.0
    b = kata.backward(q, k, v, P, gy2)
    torch.cuda.synchronize()
    assert torch.all(a[0][:, :, 0] == 0) and torch.all(a[0][:, :, 150] == 0)
    for x, z in zip(a, b):
        assert torch.equal(x, z)
    for t in a:
        assert torch.all(torch.isfinite(t.float()))


@pytest.mark.parametrize("T", [4096, 131072])
def test_backward_identities_at_size(T):
    """Identities of the exact gradient at the long-context shape (and at the mid T),
    in the launch configuration the benchmark times (auto leaf plan):
      <dq_t, q_t> = 0 for every token (y_t is homogeneous of degree 0 in q_t), to within
      1e-2 of |q_t| max(|dq_t|, RMS |dq|);
      <dv, v> = sum gy . y  (y is linear in v without an initial state);
      <dP, P> = 0  (y is invariant under P -> alpha P)."""
    case = I.make_forward("long", T=T, seed=54)
    q, k, v, P = (t.to(DEV) for t in (case.q, case.k, case.v, case.P))
    y = kata.forward(q, k, v, P, chunk=64, out_dtype=torch.float32)
    gy = I.make_output_grad(case.B, case.H, T, 64, dtype="f32", seed=14).to(DEV)
    dq, dk, dv, dP = kata.backward(q, k, v, P, gy)
    torch.cuda.synchronize()
    # per token, relative to |q_t| times |dq_t| floored at the slice's RMS |dq| (a token
    # whose exact dq vanishes, like t = 0, carries rounding noise of any direction; the
    # first tokens' gradients are up to ~100x the RMS)
    qd, dqd = q.double(), dq.double()
    per_tok = (dqd * qd).sum(-1).abs()
    nrm = dqd.norm(dim=-1)
    rms = dqd.pow(2).sum(-1).mean(-1, keepdim=True).sqrt()
    e1 = float((per_tok / (torch.maximum(nrm, rms) * qd.norm(dim=-1)).clamp_min(1e-30)).max())
    lhs = float((dv.double() * v.double()).sum())
    rhs = float((gy.double() * y.double()).sum())
    e2 = abs(lhs - rhs) / (dv.double().norm() * v.double().norm()).item()
    e3 = abs(float((dP.double() * P.double()).sum())) / (dP.double().norm() * P.double().norm()).item()
    print(f"[bwd identities T={T}] q.dq {e1:.2e} v.dv {e2:.2e} P.dP {e3:.2e}", flush=True)
    assert e1 <= 1e-2 and e2 <= 1e-2 and e3 <= 1e-2
    for t in (dq, dk, dv, dP):
        assert torch.all(torch.isfinite(t.float()))


def test_backward_long_sampled_against_oracle():
    """The long-context shape's first head, compared with the oracle on the first 4096
    tokens: the gradient of a prefix loss (gy = 0 after 4096) equals the oracle's
    backward of that prefix, and vanishes for the later tokens."""
    T = 131072
    case = I.make_forward("long", T=T, H=1, seed=55)
    q, k, v, P = (t.to(DEV) for t in (case.q, case.k, case.v, case.P))
    m = 4096
    gy = torch.zeros((1, 1, T, 64), dtype=torch.bfloat16, device=DEV)
    gy[:, :, :m] = I.make_output_grad(1, 1, m, 64, seed=15).to(DEV)
    dq, dk, dv, dP = kata.backward(q, k, v, P, gy)
    torch.cuda.synchronize()
    ref = O.backward_quadratic(host64(case.q[:, :, :m]), host64(case.k[:, :, :m]), host64(case.v[:, :, :m]),
                               case.P.double().numpy(), host64(gy[:, :, :m].cpu()))
    out = {nm: grad_err(t[:, :, :m].double().cpu().numpy(), r) for nm, t, r in
           (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2]))}
    print("[bwd long prefix] " + " ".join(f"{k} {a:.2e}/{b:.2e}" for k, (a, b) in out.items()), flush=True)
    for nm, (a, b) in out.items():
        assert a <= TOL and b <= ROW_TOL, nm
    for t in (dq, dk, dv):
        assert torch.count_nonzero(t[:, :, m:]) == 0
    eP = float(np.linalg.norm(dP.double().cpu().numpy() - ref[3]) / np.linalg.norm(ref[3]))
    assert eP <= TOL
