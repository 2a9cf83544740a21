"""The packed symmetric state (kata_state_pack, kata_state_unpack) and the decode step on it
(kata_decode_step_packed).

The packed layout is a relabelling of the canonical state: row (delta, a) stands for the
pair {a, (a + delta) mod 16}.  The tests check the layout against a CPU transcription of
that definition, the round trip, and the packed step against the oracle's decode step on
the canonical state and against kata_decode_step, at small sizes and on the decode
workload (256 streams x 16 heads, prefilled by kata_forward) sampled over several steps."""
import numpy as np
import pytest
import torch

import kernelized_linear_attention_kata_amd as kata
from kernelized_linear_attention_kata_amd import inputs as I
from oracle import kata_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def host64(t):
    return O.bf16_bits_to_f64(I.bf16_bits(t)) if t.dtype == torch.bfloat16 else t.double().numpy()


def slice_rel(got, ref):
    g = np.asarray(got, dtype=np.float64).reshape(got.shape[0] * got.shape[1], -1)
    r = np.asarray(ref, dtype=np.float64).reshape(ref.shape[0] * ref.shape[1], -1)
    return float(np.max(np.linalg.norm(g - r, axis=1) / np.linalg.norm(r, axis=1)))


def pair_rows():
    """(row, a, b) of the packed layout, from its definition."""
    rows = [(16 * dl + a, a, (a + dl) % 16) for dl in range(8) for a in range(16)]
    rows += [(128 + a, a, a + 8) for a in range(8)]
    return rows


def symmetric_state(N, H, dv, g):
    S = torch.randn((N, H, 256, dv), generator=g)
    S = (S + S.view(N, H, 16, 16, dv).transpose(2, 3).reshape(N, H, 256, dv)) / 2
    z = torch.rand((N, H, 256), generator=g)
    z = (z + z.view(N, H, 16, 16).transpose(2, 3).reshape(N, H, 256)) / 2 + 1.0
    return S, z


def test_pack_layout_and_round_trip():
    g = torch.Generator().manual_seed(91)
    for dv in (16, 64):
        S = torch.randn((3, 2, 256, dv), generator=g)                  # not symmetric
        z = torch.randn((3, 2, 256), generator=g)
        Sp, zp = kata.state_pack(S.to(DEV), z.to(DEV))
        torch.cuda.synchronize()
        Sp, zp = Sp.cpu(), zp.cpu()
        assert Sp.shape == (3, 2, 136, dv) and kata.PACKED_ROWS == 136
        for r, a, b in pair_rows():                                     # the mean of the mirror rows
            ref = (S[:, :, 16 * a + b] + S[:, :, 16 * b + a]) / 2
            assert torch.equal(Sp[:, :, r], ref)
            assert torch.equal(zp[:, :, r], (z[:, :, 16 * a + b] + z[:, :, 16 * b + a]) / 2)
        Su, zu = kata.state_unpack(Sp.to(DEV), zp.to(DEV))
        torch.cuda.synchronize()
        Su, zu = Su.cpu(), zu.cpu()
        sym = (S + S.view(3, 2, 16, 16, dv).transpose(2, 3).reshape(3, 2, 256, dv)) / 2
        assert torch.allclose(Su, sym, rtol=0, atol=1e-6)               # unpack(pack(S)) = sym(S)
        for r, a, b in pair_rows():
            assert torch.equal(Su[:, :, 16 * a + b], Sp[:, :, r]) and torch.equal(Su[:, :, 16 * b + a], Sp[:, :, r])
        # a symmetric state survives the round trip bit for bit
        Ss, zs = symmetric_state(2, 3, dv, g)
        Sp2, zp2 = kata.state_pack(Ss.to(DEV), zs.to(DEV))
        back, zback = kata.state_unpack(Sp2, zp2)
        torch.cuda.synchronize()
        assert torch.equal(back.cpu(), Ss) and torch.equal(zback.cpu(), zs)
        # S alone (z = NULL)
        assert torch.equal(kata.state_pack(Ss.to(DEV)).cpu(), Sp2.cpu())


def test_packed_step_against_oracle():
    """One packed step from a canonical state against the oracle's decode step on it:
    y, and the unpacked updated state."""
    for dt, d in ((torch.bfloat16, 64), (torch.float32, 16)):
        g = torch.Generator().manual_seed(92)
        N, H = 5, 3
        S, z = symmetric_state(N, H, d, g)
        q = (torch.randn((N, H, d), generator=g) / 8).to(dt)
        k = (torch.randn((N, H, d), generator=g) / 8).to(dt)
        v = (torch.randn((N, H, d), generator=g) / 8).to(dt)
        P = torch.randn((H, 16, d), generator=g) / d ** 0.5
        Sp, zp = kata.state_pack(S.to(DEV), z.to(DEV))
        y = kata.decode_step_packed(Sp, zp, q.to(DEV), k.to(DEV), v.to(DEV), P.to(DEV))
        Su, zu = kata.state_unpack(Sp, zp)
        torch.cuda.synchronize()
        yr, Sr, zr = O.decode_reference(S.double().numpy(), z.double().numpy(), host64(q), host64(k), host64(v),
                                        P.double().numpy())
        ey = slice_rel(y.double().cpu().numpy()[:, :, None], yr[:, :, None])
        eS, ez = slice_rel(Su.cpu().numpy(), Sr), slice_rel(zu.cpu().numpy(), zr)
        print(f"[packed step {dt}] rel y {ey:.2e} S {eS:.2e} z {ez:.2e}", flush=True)
        assert ey <= 1e-4 and eS <= 1e-6 and ez <= 1e-6


def test_packed_steps_match_canonical_steps_from_forward():
    """Prefill with kata_forward (state export), then steps on the canonical and on the
    packed state side by side: same y and, unpacked, the same state."""
    case = I.make_forward("mid", B=2, H=3, T=90, seed=93)
    q, k, v, P = (t.to(DEV) for t in (case.q, case.k, case.v, case.P))
    _, S, z = kata.forward(q[:, :, :80].contiguous(), k[:, :, :80].contiguous(), v[:, :, :80].contiguous(), P,
                           chunk=64, return_state=True)
    Sp, zp = kata.state_pack(S, z)
    back, zback = kata.state_unpack(Sp, zp)
    torch.cuda.synchronize()
    assert torch.equal(back, S)                                         # S's mirror rows in the export are equal
    # the export's z = vec(sum w w^T) comes from hi/lo MFMA products whose cross terms pair
    # up differently for Z[a][b] and Z[b][a]: mirror entries agree to that rounding, and a
    # read sees only their sum, which packing keeps
    zs = (z + z.view(2, 3, 16, 16).transpose(2, 3).reshape(2, 3, 256)) / 2
    assert torch.allclose(zback, zs, rtol=1e-6, atol=0)
    assert slice_rel(z.cpu().numpy(), zs.cpu().numpy()) <= 1e-5       # normwise: off-diagonal sums can cancel
    for t in range(80, 90):
        qt, kt, vt = (x[:, :, t].contiguous() for x in (q, k, v))
        yc = kata.decode_step(S, z, qt, kt, vt, P)
        yp = kata.decode_step_packed(Sp, zp, qt, kt, vt, P)
        torch.cuda.synchronize()
        assert slice_rel(yp.double().cpu().numpy()[:, :, None], yc.double().cpu().numpy()[:, :, None]) <= 1e-5
    Su, zu = kata.state_unpack(Sp, zp)
    torch.cuda.synchronize()
    assert slice_rel(Su.cpu().numpy(), S.cpu().numpy()) <= 1e-6
    assert slice_rel(zu.cpu().numpy(), z.cpu().numpy()) <= 1e-6


def test_packed_decode_workload_sampled():
    """The decode workload (256 streams x 16 heads, d = dv = 64, bf16 tokens) prefilled
    with 512 tokens by kata_forward: four steps on the packed state against four steps on
    the canonical state, every stream and head."""
    dc = I.make_decode(device=DEV, T_prefill=512, steps=4)
    N, H = dc.q0.shape[:2]
    _, S, z = kata.forward(dc.q0, dc.k0, dc.v0, dc.P, chunk=64, return_state=True)
    Sp, zp = kata.state_pack(S, z)
    for t in range(4):
        yc = kata.decode_step(S, z, dc.q[t], dc.k[t], dc.v[t], dc.P)
        yp = kata.decode_step_packed(Sp, zp, dc.q[t], dc.k[t], dc.v[t], dc.P)
        torch.cuda.synchronize()
        assert slice_rel(yp.double().cpu().numpy()[:, :, None], yc.double().cpu().numpy()[:, :, None]) <= 1e-5
    Su, zu = kata.state_unpack(Sp, zp)
    torch.cuda.synchronize()
    assert slice_rel(Su.cpu().numpy(), S.cpu().numpy()) <= 1e-6
    assert slice_rel(zu.cpu().numpy(), z.cpu().numpy()) <= 1e-6


def _sym_blocks(N, H, blocks, dv, g):
    """Random canonical states with equal mirror rows: [N, H, blocks*256, dv] and z."""
    S, z = symmetric_state(N, H * blocks, dv, g)
    return S.reshape(N, H, blocks * 256, dv), z.reshape(N, H, blocks * 256)


def _tokens(N, H, d, g, dt=torch.bfloat16):
    return [(torch.randn((N, H, d), generator=g) / 8).to(dt) for _ in range(3)]


@pytest.mark.parametrize("d", [64, 16])
def test_packed_decay_step_against_oracle_and_canonical(d):
    g = torch.Generator().manual_seed(94)
    N, H = 5, 3
    S, z = symmetric_state(N, H, d, g)
    q, k, v = _tokens(N, H, d, g)
    P = torch.randn((H, 16, d), generator=g) / d ** 0.5
    lam = torch.log(torch.rand((N, H), generator=g) * 0.1 + 0.9)
    dq, dk, dvv, dP, dlam = (x.to(DEV) for x in (q, k, v, P, lam))
    Sp, zp = kata.state_pack(S.to(DEV), z.to(DEV))
    yp = kata.decode_step_decay_packed(Sp, zp, dq, dk, dvv, dP, dlam)
    Sc, zc = S.to(DEV), z.to(DEV)
    yc = kata.decode_step_decay(Sc, zc, dq, dk, dvv, dP, dlam)
    Su, zu = kata.state_unpack(Sp, zp)
    torch.cuda.synchronize()
    yr, Sr, zr = O.decode_decay_reference(S.double().numpy(), z.double().numpy(), host64(q), host64(k), host64(v),
                                          P.double().numpy(), lam.double().numpy())
    assert slice_rel(yp.double().cpu().numpy()[:, :, None], yr[:, :, None]) <= 1e-4
    assert slice_rel(Su.cpu().numpy(), Sr) <= 1e-6 and slice_rel(zu.cpu().numpy(), zr) <= 1e-6
    # the canonical step sums 256 terms, the packed one 136, of a state whose sums cancel
    # in part: the two y agree to the oracle's decode bound
    assert slice_rel(yp.double().cpu().numpy()[:, :, None], yc.double().cpu().numpy()[:, :, None]) <= 1e-4
    assert slice_rel(Su.cpu().numpy(), Sc.cpu().numpy()) <= 1e-6


@pytest.mark.parametrize("mode,G,d", [("concat", 2, 64), ("concat", 3, 64), ("sum", 2, 64), ("sum", 3, 64),
                                      ("concat", 2, 16), ("sum", 3, 16)])
def test_packed_factor_step_against_oracle_and_canonical(mode, G, d):
    g = torch.Generator().manual_seed(95 + G)
    N, H = 4, 3
    blocks = G if mode == "concat" else 1
    S, z = _sym_blocks(N, H, blocks, d, g)
    q, k, v = _tokens(N, H, d, g)
    P = torch.randn((H, G, 16, d), generator=g) / d ** 0.5
    dq, dk, dvv, dP = (x.to(DEV) for x in (q, k, v, P))
    # a concatenated state is G canonical blocks: pack them as N*H*G states
    Sp, zp = kata.state_pack(S.to(DEV).reshape(N, H * blocks, 256, d), z.to(DEV).reshape(N, H * blocks, 256))
    Sp, zp = Sp.reshape(N, H, blocks * 136, d), zp.reshape(N, H, blocks * 136)
    yp = kata.decode_step_factors_packed(Sp, zp, dq, dk, dvv, dP, mode)
    Sc, zc = S.to(DEV), z.to(DEV)
    yc = kata.decode_step_factors(Sc, zc, dq, dk, dvv, dP, mode)
    Su, zu = kata.state_unpack(Sp.reshape(N, H * blocks, 136, d), zp.reshape(N, H * blocks, 136))
    torch.cuda.synchronize()
    Su, zu = Su.reshape(N, H, blocks * 256, d), zu.reshape(N, H, blocks * 256)
    yr, Sr, zr = O.decode_factors_reference(S.double().numpy(), z.double().numpy(), host64(q), host64(k),
                                            host64(v), P.double().numpy(), mode)
    ey = slice_rel(yp.double().cpu().numpy()[:, :, None], yr[:, :, None])
    print(f"[packed factors {mode} g={G}] rel y {ey:.2e}", flush=True)
    assert ey <= 1e-4
    assert slice_rel(Su.cpu().numpy(), Sr) <= 1e-6 and slice_rel(zu.cpu().numpy(), zr) <= 1e-6
    assert slice_rel(yp.double().cpu().numpy()[:, :, None], yc.double().cpu().numpy()[:, :, None]) <= 1e-4
    assert slice_rel(Su.cpu().numpy(), Sc.cpu().numpy()) <= 1e-6


def test_packed_delta_step_against_oracle_and_canonical():
    """The DeltaKATA decode step on the packed state, from a kata_forward_delta export
    (packed exactly: its mirror rows are equal), over ten steps: against
    kata_decode_step_delta on the canonical export, and against the oracle's delta steps
    from the oracle's own recurrence over the same prefix."""
    case = I.make_forward("mid", B=3, H=2, T=60, seed=97)
    beta = I.make_beta(3, 2, 60, seed=97)
    q, k, v, P, b = (t.to(DEV) for t in (case.q, case.k, case.v, case.P, beta))
    pre = slice(0, 50)
    _, S = kata.forward_delta(q[:, :, pre].contiguous(), k[:, :, pre].contiguous(), v[:, :, pre].contiguous(), P,
                              b[:, :, pre].contiguous(), return_state=True)
    Sp = kata.state_pack(S)
    torch.cuda.synchronize()
    assert torch.equal(kata.state_unpack(Sp), S)
    q64, k64, v64, P64 = host64(case.q), host64(case.k), host64(case.v), case.P.double().numpy()
    b64 = beta.double().numpy()
    _, Sref = O.delta_recurrence(q64[:, :, pre], k64[:, :, pre], v64[:, :, pre], P64, b64[:, :, pre])
    for t in range(50, 60):
        qt, kt, vt = (x[:, :, t].contiguous() for x in (q, k, v))
        bt = b[:, :, t].contiguous()
        yc = kata.decode_step_delta(S, qt, kt, vt, P, bt)
        yp = kata.decode_step_delta_packed(Sp, qt, kt, vt, P, bt)
        torch.cuda.synchronize()
        yr, Sref = O.delta_decode_reference(Sref, q64[:, :, t], k64[:, :, t], v64[:, :, t], P64, b64[:, :, t])
        assert slice_rel(yp.double().cpu().numpy()[:, :, None], yc.double().cpu().numpy()[:, :, None]) <= 1e-4
        assert slice_rel(yp.double().cpu().numpy()[:, :, None], yr[:, :, None]) <= 1e-3
    Su = kata.state_unpack(Sp)
    torch.cuda.synchronize()
    assert slice_rel(Su.cpu().numpy(), S.cpu().numpy()) <= 1e-5
    assert slice_rel(Su.cpu().numpy(), Sref) <= 1e-3


@pytest.mark.parametrize("d", [64, 16])
def test_packed_delta_step_from_a_given_state(d):
    """One DeltaKATA step on the packed state from a symmetric fp32 state built on the
    host (for d = dv = 16 the last register quad of every thread lies past the 136 rows),
    against the oracle's delta step and against kata_decode_step_delta."""
    g = torch.Generator().manual_seed(98)
    N, H = 5, 3
    S, _ = symmetric_state(N, H, d, g)
    q, k, v = _tokens(N, H, d, g)
    P = torch.randn((H, 16, d), generator=g) / d ** 0.5
    beta = torch.rand((N, H), generator=g) * 0.5 + 0.5
    dq, dk, dvv, dP, db = (x.to(DEV) for x in (q, k, v, P, beta))
    Sp = kata.state_pack(S.to(DEV))
    yp = kata.decode_step_delta_packed(Sp, dq, dk, dvv, dP, db)
    Sc = S.to(DEV)
    yc = kata.decode_step_delta(Sc, dq, dk, dvv, dP, db)
    Su = kata.state_unpack(Sp)
    torch.cuda.synchronize()
    yr, Sr = O.delta_decode_reference(S.double().numpy(), host64(q), host64(k), host64(v), P.double().numpy(),
                                      beta.double().numpy())
    assert slice_rel(yp.double().cpu().numpy()[:, :, None], yr[:, :, None]) <= 1e-4
    assert slice_rel(Su.cpu().numpy(), Sr) <= 1e-6
    assert slice_rel(yp.double().cpu().numpy()[:, :, None], yc.double().cpu().numpy()[:, :, None]) <= 1e-4
    assert slice_rel(Su.cpu().numpy(), Sc.cpu().numpy()) <= 1e-6


def test_packed_empty_is_a_no_op():
    Sp = torch.zeros((0, 4, 136, 64), device=DEV)
    zp = torch.zeros((0, 4, 136), device=DEV)
    x = torch.zeros((0, 4, 64), device=DEV, dtype=torch.bfloat16)
    P = torch.zeros((4, 16, 64), device=DEV)
    y = kata.decode_step_packed(Sp, zp, x, x, x, P)
    torch.cuda.synchronize()
    assert y.shape == (0, 4, 64)
