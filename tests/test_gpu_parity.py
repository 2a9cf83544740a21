"""GPU parity of the HIP path (through the C ABI) against the fp64 CPU oracle.

Bars (relative error ||gpu - oracle||_2 / ||oracle||_2 per (batch, head) slice, max
over slices): 1e-4 for float32 inputs, 2e-2 for bfloat16 inputs with float32
accumulation.  Inputs are the seeded synthetic workloads of
kernelized_linear_attention_kata_amd.inputs; the oracle reads the stored tensors
back bit-exactly.
"""
import numpy as np
import pytest
import torch

import kernelized_linear_attention_kata_amd as kata
from kernelized_linear_attention_kata_amd import inputs as I
from oracle import kata_oracle as O

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TOL = {"f32": 1e-4, "bf16": 2e-2}


def host64(t):
    if t.dtype == torch.bfloat16:
        return O.bf16_bits_to_f64(I.bf16_bits(t))
    return t.detach().double().cpu().numpy()


def slice_rel(got, ref):
    """max over leading (b, h) slices of ||got - ref|| / ||ref||."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    g2 = got.reshape(got.shape[0] * got.shape[1], -1)
    r2 = ref.reshape(ref.shape[0] * ref.shape[1], -1)
    num = np.linalg.norm(g2 - r2, axis=1)
    den = np.linalg.norm(r2, axis=1)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(num / den)) if len(num) else 0.0


def run(case, chunk=None, **kw):
    q, k, v, P = (t.to(DEV) for t in (case.q, case.k, case.v, case.P))
    out = kata.forward(q, k, v, P, chunk=chunk or case.chunk, return_state=True, **kw)
    torch.cuda.synchronize()
    return out


def oracle_case(case, rows=None):
    qh, kh, vh = host64(case.q), host64(case.k), host64(case.v)
    Ph = case.P.double().cpu().numpy()
    y = O.forward_quadratic(qh, kh, vh, Ph, rows=rows)
    S, z = O.final_state(kh, vh, Ph)
    return y, S, z


def check_case(case, chunk=None, rows=None, tol=None, **kw):
    tol = TOL[case.dtype] if tol is None else tol
    y, ST, zT = run(case, chunk, out_dtype=torch.float32, **kw)
    yref, Sref, zref = oracle_case(case, rows)
    yg = y.double().cpu().numpy()
    if rows is not None:
        yg = yg[:, :, rows]
    ey, eS, ez = slice_rel(yg, yref), slice_rel(ST.cpu().numpy(), Sref), slice_rel(zT.cpu().numpy(), zref)
    print(f"[{case.name} B={case.B} H={case.H} T={case.T} C={chunk or case.chunk} {kw}] "
          f"rel y {ey:.3e} S {eS:.3e} z {ez:.3e}", flush=True)
    assert ey <= tol and eS <= tol and ez <= tol, (ey, eS, ez)
    return ey


# ---- small cases: several tiles, ragged tails, every chunk size -------------------------

@pytest.mark.parametrize("chunk", [32, 64, 128])
@pytest.mark.parametrize("T", [1, 17, 64, 200, 513])
def test_small_bf16(chunk, T):
    check_case(I.make_forward("mid", B=2, H=3, T=T, seed=100 + T), chunk)


@pytest.mark.parametrize("chunk", [32, 64, 128])
@pytest.mark.parametrize("T", [1, 33, 256, 301])
def test_small_f32(chunk, T):
    check_case(I.make_forward("tiny", B=2, H=2, T=T, seed=200 + T), chunk)


def test_bf16_output_dtype():
    case = I.make_forward("mid", B=1, H=2, T=300, seed=7)
    q, k, v, P = (t.to(DEV) for t in (case.q, case.k, case.v, case.P))
    y = kata.forward(q, k, v, P, chunk=64)
    assert y.dtype == torch.bfloat16
    yref, _, _ = oracle_case(case)
    assert slice_rel(host64(y), yref) <= 2e-2


# ---- the five workloads at their own sizes ------------------------------------------------

def test_workload_tiny():
    check_case(I.make_forward("tiny"))


def test_workload_mid():
    check_case(I.make_forward("mid", device=DEV))


def test_workload_lm340m():
    check_case(I.make_forward("lm340m", device=DEV))


def leaf_starts(B, H, T, chunk):
    """First token of every leaf after the first in the library's own leaf plan, read back
    from the workspace size (B*H*n_leaf blocks of 144*64 + 256 floats)."""
    ws = kata.forward_workspace_bytes(B, H, T, 64, 64, chunk)
    n_leaf = ws // (B * H * (144 * 64 + 256) * 4)
    n_chunks = -(-T // chunk)
    leaf = -(-n_chunks // n_leaf)
    assert -(-n_chunks // leaf) == n_leaf
    return [j * leaf * chunk for j in range(1, n_leaf)]


@pytest.mark.parametrize("chunk", [64, 128])
def test_workload_long_sampled(chunk):
    """T = 131072: y checked on sampled query rows (first/last rows, chunk boundaries, the
    last token of every leaf and the first two of the next, random rows); the final state
    in full."""
    case = I.make_forward("long", device=DEV)
    T = case.T
    r = np.random.default_rng(5)
    starts = leaf_starts(case.B, case.H, T, chunk)
    if chunk == 64:
        assert starts[:2] == [2752, 5504]          # 48 leaves of 43 chunks per head
    edges = np.concatenate([[s - 1, s, s + 1] for s in starts])
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 65, 127, 128, 4095, 4096, T // 2, T - 2, T - 1],
                                     edges, r.integers(0, T, 40)]))
    print(f"[long C={chunk}] {len(starts) + 1} leaves per head, {len(rows)} sampled rows", flush=True)
    check_case(case, chunk, rows=rows)


# ---- agreement between the GPU paths ------------------------------------------------------

def test_paths_agree():
    """Chunk 32/64/128, leaf 1 (every chunk state scanned), automatic leaves and the
    sequential inter-chunk mode agree with each other and with the oracle."""
    case = I.make_forward("mid", B=2, H=4, T=1000, seed=3)
    ys = {}
    for name, kw in {"c64": dict(chunk=64), "c32": dict(chunk=32), "c128": dict(chunk=128),
                     "leaf1": dict(chunk=64, scan_leaf=1), "leaf3": dict(chunk=64, scan_leaf=3),
                     "seq": dict(chunk=64, scan="sequential")}.items():
        chunk = kw.pop("chunk")
        y, ST, zT = run(case, chunk, out_dtype=torch.float32, **kw)
        ys[name] = (y.double().cpu().numpy(), ST.cpu().numpy(), zT.cpu().numpy())
    base = ys["c64"]
    for name, (y, S, z) in ys.items():
        assert slice_rel(y, base[0]) <= 2e-2, name
        assert slice_rel(S, base[1]) <= 1e-5, name
        assert slice_rel(z, base[2]) <= 1e-5, name
    yref, _, _ = oracle_case(case)
    assert slice_rel(base[0], yref) <= 2e-2


_SCAN_CASE = {}


def _scan_case():
    """T = 32*600 + 7 with chunk 32: 601 chunks per head, a random initial state."""
    if not _SCAN_CASE:
        case = I.make_forward("mid", B=1, H=2, T=32 * 600 + 7, seed=21)
        g = torch.Generator().manual_seed(5)
        S0 = torch.randn((1, 2, 256, 64), generator=g)
        S0 = 0.5 * (S0 + S0.view(1, 2, 16, 16, 64).transpose(2, 3).reshape(1, 2, 256, 64))   # symmetric
        z0 = torch.rand((1, 2, 16, 16), generator=g)
        z0 = (z0 + z0.transpose(2, 3)).reshape(1, 2, 256)
        Sr, zr = O.final_state(host64(case.k), host64(case.v), case.P.double().cpu().numpy())
        _SCAN_CASE.update(case=case, S0=S0, z0=z0, Sref=Sr + S0.double().numpy(), zref=zr + z0.double().numpy())
        q, k, v, P = (t.to(DEV) for t in (case.q, case.k, case.v, case.P))
        y, ST, zT = kata.forward(q, k, v, P, chunk=32, S0=S0.to(DEV), z0=z0.to(DEV), return_state=True,
                                 out_dtype=torch.float32)
        _SCAN_CASE.update(ybase=y.double().cpu().numpy(), Sbase=ST.cpu().numpy(), zbase=zT.cpu().numpy())
    return _SCAN_CASE


@pytest.mark.parametrize("leaf", [1, 3, 15, 36, 40, 601])
def test_scan_leaf_counts(leaf):
    """Leaf counts 601 (three passes of the scan), 201, 41, 17, 16 and 1 (one to sixteen
    segments per column).  Against the automatic plan, which groups the same per-token
    terms into different leaves, only the fp32 summation order differs: S, z and y
    agree to 1e-5 / 1e-5 / 1e-3.  Against the oracle's S0 + sum: z (hi/lo W) to 1e-5,
    S (bf16 features) to the bf16 bar."""
    sc = _scan_case()
    case = sc["case"]
    q, k, v, P = (t.to(DEV) for t in (case.q, case.k, case.v, case.P))
    y, ST, zT = kata.forward(q, k, v, P, chunk=32, S0=sc["S0"].to(DEV), z0=sc["z0"].to(DEV), return_state=True,
                             out_dtype=torch.float32, scan_leaf=leaf)
    torch.cuda.synchronize()
    eS = slice_rel(ST.cpu().numpy(), sc["Sbase"])
    ez = slice_rel(zT.cpu().numpy(), sc["zbase"])
    ey = slice_rel(y.double().cpu().numpy(), sc["ybase"])
    oS = slice_rel(ST.cpu().numpy(), sc["Sref"])
    oz = slice_rel(zT.cpu().numpy(), sc["zref"])
    print(f"[scan leaf={leaf}] vs auto: S {eS:.2e} z {ez:.2e} y {ey:.2e}; vs oracle: S {oS:.2e} z {oz:.2e}",
          flush=True)
    assert eS <= 1e-5 and ez <= 1e-5 and ey <= 1e-3
    assert oS <= TOL["bf16"] and oz <= 1e-5


def test_resume_from_state():
    """forward(x1 || x2) on the x2 part equals forward(x2) from the state after x1,
    which is how a sequence split across devices would be joined."""
    case = I.make_forward("mid", B=2, H=2, T=700, seed=4)
    q, k, v, P = (t.to(DEV) for t in (case.q, case.k, case.v, case.P))
    y, ST, zT = kata.forward(q, k, v, P, chunk=64, return_state=True, out_dtype=torch.float32)
    t1 = 300
    sl1 = (slice(None), slice(None), slice(0, t1))
    sl2 = (slice(None), slice(None), slice(t1, None))
    _, S1, z1 = kata.forward(q[sl1].contiguous(), k[sl1].contiguous(), v[sl1].contiguous(), P, chunk=64,
                             return_state=True, out_dtype=torch.float32)
    y2, S2, z2 = kata.forward(q[sl2].contiguous(), k[sl2].contiguous(), v[sl2].contiguous(), P, chunk=64,
                              S0=S1, z0=z1, return_state=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert slice_rel(y2.double().cpu().numpy(), y[sl2].double().cpu().numpy()) <= 2e-2
    assert slice_rel(S2.cpu().numpy(), ST.cpu().numpy()) <= 1e-5
    assert slice_rel(z2.cpu().numpy(), zT.cpu().numpy()) <= 1e-5
    # and against the oracle started from its own state after x1
    qh, kh, vh = host64(case.q), host64(case.k), host64(case.v)
    Ph = case.P.double().cpu().numpy()
    Sa, za = O.final_state(kh[:, :, :t1], vh[:, :, :t1], Ph)
    yr = O.forward_quadratic(qh[:, :, t1:], kh[:, :, t1:], vh[:, :, t1:], Ph, S0=Sa, z0=za)
    assert slice_rel(y2.double().cpu().numpy(), yr) <= 2e-2


def test_deterministic():
    case = I.make_forward("mid", B=2, H=2, T=777, seed=9)
    a = run(case, 64)
    b = run(case, 64)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# ---- the scan: workspace after the call holds the exclusive prefix of the leaf states ---

def unpack_leaf(block, dv):
    """Leaf block of the workspace -> canonical (S [256, dv], z [256]).

    S: packed slots (delta, a) in accumulator-tile order: tile delta * (dv/16) + nb,
    lane 16 g + n, element r holds S[(a, (a + delta) % 16)][16 nb + n], a = 4 g + r.
    z: the 16 x 16 matrix Z after the 144 * dv S slots, lane 16 g + b element r holding
    Z[4 g + r][b]."""
    nb = dv // 16
    S = np.zeros((256, dv))
    z = np.zeros(256)
    for delta in range(9):
        for a in range(16):
            if delta == 8 and a >= 8:
                continue
            b = (a + delta) % 16
            g, r = a // 4, a % 4
            for blk in range(nb):
                for n in range(16):
                    lane = 16 * g + n
                    val = block[((delta * nb + blk) * 64 + lane) * 4 + r]
                    S[a * 16 + b, 16 * blk + n] = val
                    S[b * 16 + a, 16 * blk + n] = val
    for lane in range(64):
        b, g = lane % 16, lane // 16
        for r in range(4):
            z[(4 * g + r) * 16 + b] = block[144 * dv + lane * 4 + r]
    return S, z


@pytest.mark.parametrize("leaf", [1, 4])
def test_scan_exclusive_prefix(leaf):
    case = I.make_forward("mid", B=1, H=2, T=64 * 11 + 5, seed=12)
    q, k, v, P = (t.to(DEV) for t in (case.q, case.k, case.v, case.P))
    nbytes = kata.forward_workspace_bytes(1, 2, case.T, 64, 64, 64, scan_leaf=leaf)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    kata.forward(q, k, v, P, chunk=64, scan_leaf=leaf, workspace=ws)
    torch.cuda.synchronize()
    E = 144 * 64 + 256
    n_leaf = -(-12 // leaf)
    W = ws.view(torch.float32).cpu().numpy().reshape(2, n_leaf, E)
    kh, vh = host64(case.k), host64(case.v)
    Ph = case.P.double().cpu().numpy()
    for h in range(2):
        for g in range(n_leaf):
            t_end = g * leaf * 64
            S, z = unpack_leaf(W[h, g], 64)
            Sr, zr = O.final_state(kh[:, h:h + 1, :t_end], vh[:, h:h + 1, :t_end], Ph[h:h + 1])
            scale = max(np.linalg.norm(Sr), 1e-30)
            assert np.linalg.norm(S - Sr[0, 0]) / scale <= 1e-2 if t_end else np.all(S == 0)
            assert np.linalg.norm(z - zr[0, 0]) / max(np.linalg.norm(zr), 1e-30) <= 1e-2 if t_end else np.all(z == 0)


@pytest.mark.parametrize("B,H,T,initial", [(8, 16, 549, False), (8, 16, 549, True), (4, 32, 2048, True),
                                             (16, 8, 40, False), (2, 3, 200, True)])
def test_prefix_in_the_intra_pass_agrees_with_the_scan(B, H, T, initial):
    """With at most 8 leaves per sequence the library's plan runs no scan: the intra pass's
    workgroup of leaf g adds the leaf sums of 0 .. g-1 (and the symmetric part of S0) and the
    last one exports S_T, z_T.  The same leaves through the scan (an explicit scan_leaf)
    give the same y and final state up to summation order, both match the oracle, and the
    workspace of the scanned call holds prefixes while the other holds the leaf sums."""
    case = I.make_forward("lm340m", B=B, H=H, T=T, seed=40 + T)
    q, k, v, P = (t.to(DEV) for t in (case.q, case.k, case.v, case.P))
    E = 144 * 64 + 256
    nbytes = kata.forward_workspace_bytes(B, H, T, 64, 64, 64)
    n_leaf = nbytes // (B * H * E * 4)
    n_chunks = -(-T // 64)
    leaf = -(-n_chunks // n_leaf)
    assert -(-n_chunks // leaf) == n_leaf and n_leaf <= 8
    kw = {}
    if initial:
        kh, vh = host64(case.k), host64(case.v)
        Ph = case.P.double().cpu().numpy()
        S0, z0 = O.final_state(kh[:, :, : T // 3], vh[:, :, : T // 3], Ph)
        g = np.random.default_rng(T)
        A = g.standard_normal(S0.shape).reshape(B, H, 16, 16, 64)
        S0 = S0 + 0.3 * (A - A.transpose(0, 1, 3, 2, 4)).reshape(S0.shape) * np.abs(S0).max()   # not symmetric
        kw = dict(S0=torch.tensor(S0, dtype=torch.float32, device=DEV),
                  z0=torch.tensor(z0, dtype=torch.float32, device=DEV))
    ws_d = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    ws_s = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    yd, Sd, zd = kata.forward(q, k, v, P, chunk=64, workspace=ws_d, return_state=True, out_dtype=torch.float32, **kw)
    ys, Ss, zs = kata.forward(q, k, v, P, chunk=64, scan_leaf=leaf, workspace=ws_s, return_state=True,
                              out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    ey = slice_rel(yd.double().cpu().numpy(), ys.double().cpu().numpy())
    eS = slice_rel(Sd.cpu().numpy(), Ss.cpu().numpy())
    ez = slice_rel(zd.cpu().numpy(), zs.cpu().numpy())
    print(f"[B={B} H={H} T={T} n_leaf={n_leaf} S0={initial}] direct vs scan: y {ey:.2e} S {eS:.2e} z {ez:.2e}")
    assert ey <= 2e-3 and eS <= 1e-5 and ez <= 1e-5, (ey, eS, ez)
    # against the oracle
    qh, kh, vh = host64(case.q), host64(case.k), host64(case.v)
    Ph = case.P.double().cpu().numpy()
    rows = np.unique(np.linspace(0, T - 1, 24).astype(int))
    o = {kk: vv.double().cpu().numpy() for kk, vv in kw.items()}
    yr = O.forward_quadratic(qh, kh, vh, Ph, rows=rows, **o)
    if initial:   # the export carries the symmetric part of S0 (the only part a read sees)
        S0h = o["S0"].reshape(B, H, 16, 16, 64)
        o["S0"] = (0.5 * (S0h + S0h.transpose(0, 1, 3, 2, 4))).reshape(B, H, 256, 64)
        z0h = o["z0"].reshape(B, H, 16, 16)
        o["z0"] = (0.5 * (z0h + z0h.transpose(0, 1, 3, 2))).reshape(B, H, 256)
    Sr, zr = O.final_state(kh, vh, Ph, **o)
    assert slice_rel(yd.double().cpu().numpy()[:, :, rows], yr) <= 2e-2
    assert slice_rel(Sd.cpu().numpy(), Sr) <= 2e-2 and slice_rel(zd.cpu().numpy(), zr) <= 2e-2
    # the scanned workspace holds exclusive prefixes (leaf 0's is the initial state, or 0),
    # the other the leaf sums: they agree on leaf 0 only when there is no initial state
    Wd = ws_d.view(torch.float32).cpu().numpy().reshape(B * H, n_leaf, E)
    Ws = ws_s.view(torch.float32).cpu().numpy().reshape(B * H, n_leaf, E)
    S1, _ = unpack_leaf(Ws[0, 1 if n_leaf > 1 else 0], 64)
    Sl, _ = unpack_leaf(Wd[0, 0], 64)
    if n_leaf > 1 and not initial:
        assert np.allclose(S1, Sl, rtol=1e-5, atol=1e-6 * np.abs(Sl).max())


# ---- edge cases ------------------------------------------------------------------------

def test_empty_sequence_copies_initial_state():
    B, H = 2, 3
    q = torch.empty((B, H, 0, 64), dtype=torch.bfloat16, device=DEV)
    P = torch.randn((H, 16, 64), device=DEV)
    S0 = torch.randn((B, H, 256, 64), device=DEV)
    z0 = torch.rand((B, H, 256), device=DEV)
    y, ST, zT = kata.forward(q, q, q, P, chunk=64, S0=S0, z0=z0, return_state=True)
    torch.cuda.synchronize()
    assert y.shape == (B, H, 0, 64)
    # the state as every entry point reads it: the mean of the mirror entries (i, j), (j, i)
    Sm = S0.view(B, H, 16, 16, 64)
    zm = z0.view(B, H, 16, 16)
    assert torch.equal(ST, (0.5 * (Sm + Sm.transpose(2, 3))).reshape(B, H, 256, 64))
    assert torch.equal(zT, (0.5 * (zm + zm.transpose(2, 3))).reshape(B, H, 256))
    y, ST, zT = kata.forward(q, q, q, P, chunk=64, return_state=True)
    torch.cuda.synchronize()
    assert torch.all(ST == 0) and torch.all(zT == 0)


def test_zero_query_rows_give_zero():
    case = I.make_forward("mid", B=1, H=2, T=130, seed=13)
    case.q[:, :, 70] = 0
    case.q[:, :, 0] = 0
    y, _, _ = run(case, 64, out_dtype=torch.float32)
    assert torch.all(y[:, :, 70] == 0) and torch.all(y[:, :, 0] == 0)
    yref, _, _ = oracle_case(case)
    assert slice_rel(y.double().cpu().numpy(), yref) <= 2e-2


def test_many_heads_and_batches():
    check_case(I.make_forward("mid", B=16, H=16, T=96, seed=14), 64)


def test_initial_state_symmetric_read():
    """A caller state is read through its symmetric part, the mean of the mirror entries:
    swapping every mirror pair of S0 and z0 leaves y bit for bit unchanged, and a state
    with an antisymmetric part added gives the oracle's y (the readout phi(q)^T S0 sees
    only the symmetric part)."""
    case = I.make_forward("mid", B=1, H=2, T=150, seed=15)
    kh, vh = host64(case.k), host64(case.v)
    Ph = case.P.double().cpu().numpy()
    S0, z0 = O.final_state(kh[:, :, :40], vh[:, :, :40], Ph)
    g = np.random.default_rng(15)
    A = g.standard_normal(S0.shape).reshape(1, 2, 16, 16, 64)
    S0 = S0 + (A - A.transpose(0, 1, 3, 2, 4)).reshape(S0.shape) * np.abs(S0).max()   # not symmetric
    a = g.standard_normal(z0.shape).reshape(1, 2, 16, 16)
    z0 = z0 + (a - a.transpose(0, 1, 3, 2)).reshape(z0.shape) * np.abs(z0).max()
    S0 = torch.tensor(S0, dtype=torch.float32, device=DEV)
    z0 = torch.tensor(z0, dtype=torch.float32, device=DEV)
    q, k, v, P = (t.to(DEV) for t in (case.q, case.k, case.v, case.P))
    y1 = kata.forward(q, k, v, P, chunk=64, S0=S0, z0=z0, out_dtype=torch.float32)
    S0t = S0.view(1, 2, 16, 16, 64).transpose(2, 3).reshape(1, 2, 256, 64).contiguous()
    z0t = z0.view(1, 2, 16, 16).transpose(2, 3).reshape(1, 2, 256).contiguous()
    y2 = kata.forward(q, k, v, P, chunk=64, S0=S0t, z0=z0t, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    qh = host64(case.q)
    yr = O.forward_quadratic(qh, kh, vh, Ph, S0=S0.double().cpu().numpy(), z0=z0.double().cpu().numpy())
    assert slice_rel(y1.double().cpu().numpy(), yr) <= 2e-2


# ---- feature map -------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_feature_map_identity(dtype):
    name = "tiny" if dtype == "f32" else "mid"
    case = I.make_forward(name, B=1, H=2, T=50, seed=16)
    q = case.q[0].transpose(0, 1).contiguous().to(DEV)      # [n, H, d]
    k = case.k[0].transpose(0, 1).contiguous().to(DEV)
    P = case.P.to(DEV)
    full_q = kata.feature_map(q, P, "full").double().cpu().numpy()
    pq = kata.feature_map(q, P, "packed_query").double().cpu().numpy()
    pk = kata.feature_map(k, P, "packed_key").double().cpu().numpy()
    torch.cuda.synchronize()
    qh = host64(case.q[0].transpose(0, 1).contiguous())
    kh = host64(case.k[0].transpose(0, 1).contiguous())
    Ph = case.P.double().cpu().numpy()
    for h in range(2):
        u = O.project(qh[:, h], Ph[h])
        w = O.project(kh[:, h], Ph[h])
        ref_full = O.feature_full(u)
        assert np.linalg.norm(full_q[:, h] - ref_full) / np.linalg.norm(ref_full) <= 1e-5
        dots = np.sum(pq[:, h] * pk[:, h], axis=1)
        ref = np.sum(u * w, axis=1) ** 2
        assert np.max(np.abs(dots - ref) / np.maximum(ref, 1e-12)) <= 1e-4 or \
            np.linalg.norm(dots - ref) / np.linalg.norm(ref) <= 1e-5
    assert np.all(pk[:, :, 8 * 16 + 8:] == 0) and np.all(pq[:, :, 8 * 16 + 8:] == 0)


# ---- decode ------------------------------------------------------------------------------

def _decode_run(dc, steps):
    P = dc.P.to(DEV)
    q0, k0, v0 = dc.q0.to(DEV), dc.k0.to(DEV), dc.v0.to(DEV)
    _, S, z = kata.forward(q0, k0, v0, P, chunk=64, return_state=True)
    ys = []
    for j in range(steps):
        ys.append(kata.decode_step(S, z, dc.q[j].to(DEV), dc.k[j].to(DEV), dc.v[j].to(DEV), P))
    torch.cuda.synchronize()
    return torch.stack(ys), S, z


def test_decode_small_against_oracle():
    dc = I.make_decode(N=4, H=3, T_prefill=100, steps=9)
    y, S, z = _decode_run(dc, 9)
    Ph = dc.P.double().numpy()
    q = np.concatenate([host64(dc.q0), host64(dc.q.permute(1, 2, 0, 3).contiguous())], axis=2)
    k = np.concatenate([host64(dc.k0), host64(dc.k.permute(1, 2, 0, 3).contiguous())], axis=2)
    v = np.concatenate([host64(dc.v0), host64(dc.v.permute(1, 2, 0, 3).contiguous())], axis=2)
    yref = O.forward_quadratic(q, k, v, Ph, rows=np.arange(100, 109))        # [N, H, 9, dv]
    yg = y.permute(1, 2, 0, 3).double().cpu().numpy()
    assert slice_rel(yg, yref) <= 2e-2
    Sref, zref = O.final_state(k, v, Ph)
    assert slice_rel(S.cpu().numpy(), Sref) <= 2e-2
    assert slice_rel(z.cpu().numpy(), zref) <= 2e-2


def test_decode_step_exact_recurrence():
    """One step from a given fp32 state against the oracle's decode step (fp32 state,
    bf16 and fp32 token inputs)."""
    for dt, d in ((torch.bfloat16, 64), (torch.float32, 16)):
        g = torch.Generator().manual_seed(17)
        N, H = 5, 3
        S = torch.randn((N, H, 256, d), generator=g)
        S = (S + S.view(N, H, 16, 16, d).transpose(2, 3).reshape(N, H, 256, d)) / 2    # symmetric
        z = torch.rand((N, H, 256), generator=g)
        z = (z + z.view(N, H, 16, 16).transpose(2, 3).reshape(N, H, 256)) / 2 + 1.0
        q = (torch.randn((N, H, d), generator=g) / 8).to(dt)
        k = (torch.randn((N, H, d), generator=g) / 8).to(dt)
        v = (torch.randn((N, H, d), generator=g) / 8).to(dt)
        P = torch.randn((H, 16, d), generator=g) / d ** 0.5
        Sd, zd = S.to(DEV), z.to(DEV)
        y = kata.decode_step(Sd, zd, q.to(DEV), k.to(DEV), v.to(DEV), P.to(DEV))
        torch.cuda.synchronize()
        yr, Sr, zr = O.decode_reference(S.double().numpy(), z.double().numpy(), host64(q), host64(k),
                                        host64(v), P.double().numpy())
        assert slice_rel(y.double().cpu().numpy()[:, :, None], yr[:, :, None]) <= 1e-4
        assert slice_rel(Sd.cpu().numpy(), Sr) <= 1e-6
        assert slice_rel(zd.cpu().numpy(), zr) <= 1e-6


def test_decode_matches_chunked_forward():
    """Recurrent path vs chunked path: T decode steps from zero state give the same y as
    one chunked forward over the T tokens."""
    case = I.make_forward("mid", B=2, H=3, T=70, seed=18)
    q, k, v, P = (t.to(DEV) for t in (case.q, case.k, case.v, case.P))
    y, ST, zT = kata.forward(q, k, v, P, chunk=32, return_state=True, out_dtype=torch.float32)
    S = torch.zeros((2, 3, 256, 64), device=DEV)
    z = torch.zeros((2, 3, 256), device=DEV)
    yd = torch.stack([kata.decode_step(S, z, q[:, :, t].contiguous(), k[:, :, t].contiguous(),
                                       v[:, :, t].contiguous(), P) for t in range(70)], dim=2)
    torch.cuda.synchronize()
    assert slice_rel(yd.double().cpu().numpy(), y.double().cpu().numpy()) <= 2e-2
    # the decode state is accumulated in fp32 from fp32 features; the chunked state
    # from bf16-rounded features (fp32 accumulation): agreement to the bf16 bar
    assert slice_rel(S.cpu().numpy(), ST.cpu().numpy()) <= 2e-2
    assert slice_rel(z.cpu().numpy(), zT.cpu().numpy()) <= 2e-2


@pytest.mark.parametrize("name,T,chunk", [("mid", 200, 64), ("mid", 333, 32), ("mid", 77, 128), ("tiny", 130, 64),
                                          ("mid", 4096, 64)])
def test_bf16_output_is_the_rounded_fp32_output(name, T, chunk):
    """y stored as bf16 is exactly the fp32 y rounded to nearest even: both leave the same
    gated tile, and the bf16 rows (written two 16-byte pieces per lane after a lane-pair
    exchange) must land every column of every token in its place, ragged tails included."""
    case = I.make_forward(name, B=2, H=3, T=T, seed=170, dtype="bf16")
    q, k, v, P = (t.to(DEV) for t in (case.q, case.k, case.v, case.P))
    y32 = kata.forward(q, k, v, P, chunk=chunk, out_dtype=torch.float32)
    y16 = kata.forward(q, k, v, P, chunk=chunk, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y16, y32.to(torch.bfloat16))
