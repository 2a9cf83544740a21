"""CPU tests pinning the fp64 oracle to the pages and to mathematics (no GPU).

Method: "Kernelized Linear Attention: Breaking the Capacity Wall with Symmetric
Cones" (arXiv 2607.17419).  [ABS] = its abstract; [TS-x] = section x of the
gist.science technical summary of it.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import kata_oracle as O
from tests import oracle_pins as pins


@pytest.mark.parametrize("name", sorted(pins.PINS))
def test_pin(name):
    fn, bound = pins.PINS[name]
    r = fn(O.forward_quadratic)
    assert r <= bound, f"pin {name}: residual {r} > {bound}"


def test_bf16_decoder_known_bits():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0x3E80, 0x0001, 0x4049], dtype=np.uint16)
    got = O.bf16_bits_to_f64(bits)
    want = [1.0, -2.0, 0.0, -0.0, np.inf, 0.25, 2.0 ** -133, 3.140625]
    assert np.array_equal(got, np.array(want))
    assert np.signbit(got[3])


def test_bf16_decoder_matches_torch_on_every_finite_pattern():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().double().numpy()
    got = O.bf16_bits_to_f64(bits)
    fin = np.isfinite(t)
    assert np.array_equal(got[fin], t[fin])
    assert np.array_equal(np.isnan(got), np.isnan(t))


def test_feature_identity_closed_form():
    """<psi(u), psi(w)> = <u, w>^2 for the full and the sqrt2-packed feature ([TS-2.2])."""
    r = np.random.default_rng(0)
    u = r.standard_normal((50, 16))
    w = r.standard_normal((50, 16))
    ref = np.sum(u * w, axis=1) ** 2
    full = np.sum(O.feature_full(u) * O.feature_full(w), axis=1)
    packed = np.sum(O.feature_packed(u) * O.feature_packed(w), axis=1)
    assert O.feature_packed(u).shape == (50, 136)
    assert np.max(np.abs(full - ref) / ref) < 1e-12
    assert np.max(np.abs(packed - ref) / ref) < 1e-12


def test_feature_is_rank_one_psd():
    """psi(u) reshaped to p x p is symmetric PSD of rank one with trace |u|^2 ([TS-2.2])."""
    u = np.random.default_rng(1).standard_normal(16)
    M = O.feature_full(u).reshape(16, 16)
    ev = np.linalg.eigvalsh(M)
    assert np.allclose(M, M.T)
    assert ev.min() > -1e-12
    assert np.sum(ev > 1e-9 * ev.max()) == 1
    assert abs(np.trace(M) - u @ u) < 1e-12


def test_weights_nonnegative_and_causal():
    q, k, v, P = pins.rand_case(20, T=30)
    a = O.weights(q[0, 0], k[0, 0], P[0])
    assert a.min() >= 0.0
    assert np.all(np.triu(a, 1) == 0.0)
    assert np.all(np.diag(a) > 0.0)


def test_weights_golden_scalar():
    """The hand-derived weights of the p = d = 1 example (tests/golden/scalar_p1.json):
    a_ts = (P q_t * P k_s)^2 row by row, so |u.w| or u.w in place of the square, a strict
    or reversed mask, or the query used for the key all fail."""
    g = json.load(open(os.path.join(pins.GOLDEN, "scalar_p1.json")))
    T = len(g["q"])
    a = O.weights(np.array(g["q"]).reshape(T, 1), np.array(g["k"]).reshape(T, 1), np.array(g["P"]))
    assert np.array_equal(a, np.array(g["a"]))


def test_weights_normalised_rows_are_the_forward():
    """Rows of the weights normalised to sum 1, times V, give the forward's y, which its own
    pins fix independently (convex gate, brute-force recurrence, hand-derived values)."""
    q, k, v, P = pins.rand_case(22, T=40, d=6, p=5, dv=3)
    a = O.weights(q[0, 0], k[0, 0], P[0])
    y = (a @ v[0, 0]) / a.sum(1, keepdims=True)
    assert pins.rel(y, O.forward_quadratic(q, k, v, P)[0, 0]) < 1e-12


def test_final_state_brute_force():
    """S_T = sum_s phi(k_s) v_s^T by explicit per-token outer products ([TS-1])."""
    q, k, v, P = pins.rand_case(21, B=2, H=2, T=9, d=5, p=3, dv=4)
    ST, zT = O.final_state(k, v, P)
    for b in range(2):
        for h in range(2):
            S = np.zeros((3, 3, 4))
            z = np.zeros((3, 3))
            for t in range(9):
                w = P[h] @ k[b, h, t]
                for i in range(3):
                    for j in range(3):
                        S[i, j] += w[i] * w[j] * v[b, h, t]
                        z[i, j] += w[i] * w[j]
            assert np.allclose(ST[b, h], S.reshape(9, 4), rtol=1e-13, atol=1e-13)
            assert np.allclose(zT[b, h], z.reshape(9), rtol=1e-13, atol=1e-13)


def test_golden_final_state():
    g = json.load(open(os.path.join(pins.GOLDEN, "scalar_p1.json")))
    T = len(g["k"])
    k = np.array(g["k"]).reshape(1, 1, T, 1)
    v = np.array(g["v"]).reshape(1, 1, T, 1)
    P = np.array(g["P"]).reshape(1, 1, 1)
    ST, zT = O.final_state(k, v, P)
    assert ST[0, 0].tolist() == g["S_T"]
    assert zT[0, 0].tolist() == g["z_T"]


def test_recurrence_matches_quadratic_and_final_state():
    q, k, v, P = pins.rand_case(22, B=2, H=2, T=33, d=8, p=4, dv=5)
    y, ST, zT = O.recurrence(q, k, v, P)
    assert pins.rel(y, O.forward_quadratic(q, k, v, P)) < 1e-12
    S2, z2 = O.final_state(k, v, P)
    assert pins.rel(ST, S2) < 1e-12 and pins.rel(zT, z2) < 1e-12


def test_resume_from_state():
    """Checkpoint/resume: forward(x1 || x2) restricted to x2 equals forward(x2) started
    from the state after x1, and the final states agree."""
    q, k, v, P = pins.rand_case(23, B=1, H=2, T=50, d=8, p=4, dv=5)
    y = O.forward_quadratic(q, k, v, P)
    t1 = 19
    S1, z1 = O.final_state(k[:, :, :t1], v[:, :, :t1], P)
    y2 = O.forward_quadratic(q[:, :, t1:], k[:, :, t1:], v[:, :, t1:], P, S0=S1, z0=z1)
    assert pins.rel(y2, y[:, :, t1:]) < 1e-12
    S2, z2 = O.final_state(k[:, :, t1:], v[:, :, t1:], P, S0=S1, z0=z1)
    Sf, zf = O.final_state(k, v, P)
    assert pins.rel(S2, Sf) < 1e-12 and pins.rel(z2, zf) < 1e-12


def test_state_additivity_over_chunks():
    """The inter-chunk combine is plain addition: the state of a sequence equals the
    sum of its chunk states, in any bracketing ([TS-2.3]: associative scan)."""
    q, k, v, P = pins.rand_case(24, T=64)
    parts = [O.final_state(k[:, :, s:s + 16], v[:, :, s:s + 16], P) for s in range(0, 64, 16)]
    full = O.final_state(k, v, P)
    left = ((parts[0][0] + parts[1][0]) + parts[2][0]) + parts[3][0]
    tree = (parts[0][0] + parts[1][0]) + (parts[2][0] + parts[3][0])
    assert pins.rel(left, full[0]) < 1e-13 and pins.rel(tree, full[0]) < 1e-13
    cum = np.cumsum(np.stack([p_[0] for p_ in parts]), axis=0)
    for c in range(4):
        pre = O.final_state(k[:, :, :16 * (c + 1)], v[:, :, :16 * (c + 1)], P)[0]
        assert pins.rel(cum[c], pre) < 1e-13


def test_decode_reference_extends_the_sequence():
    """One decode step after a prefill equals the last row of the forward pass over the
    concatenated sequence, and its state equals the final state of that sequence."""
    r = np.random.default_rng(25)
    N, H, T0, d, p, dv = 3, 2, 17, 8, 4, 5
    q = r.standard_normal((N, H, T0 + 1, d))
    k = r.standard_normal((N, H, T0 + 1, d))
    v = r.standard_normal((N, H, T0 + 1, dv))
    P = r.standard_normal((H, p, d))
    S, z = O.final_state(k[:, :, :T0], v[:, :, :T0], P)
    y, S1, z1 = O.decode_reference(S, z, q[:, :, T0], k[:, :, T0], v[:, :, T0], P)
    yref = O.forward_quadratic(q, k, v, P, rows=[T0])[:, :, 0]
    assert pins.rel(y, yref) < 1e-12
    Sf, zf = O.final_state(k, v, P)
    assert pins.rel(S1, Sf) < 1e-12 and pins.rel(z1, zf) < 1e-12


def test_zero_denominator_reading():
    """q = 0 makes every weight of that row 0; the reading adopted is y = 0."""
    q, k, v, P = pins.rand_case(26, T=10)
    q[..., 4, :] = 0.0
    y = O.forward_quadratic(q, k, v, P)
    assert np.all(y[..., 4, :] == 0.0)
    y2, _, _ = O.recurrence(q, k, v, P)
    assert np.all(y2[..., 4, :] == 0.0)


def test_sampled_rows_equal_full_rows():
    q, k, v, P = pins.rand_case(27, T=70)
    rows = [0, 1, 13, 40, 69]
    y = O.forward_quadratic(q, k, v, P)
    ys = O.forward_quadratic(q, k, v, P, rows=rows, block=2)
    assert pins.rel(ys, y[:, :, rows]) < 1e-14


def test_empty_sequence():
    q, k, v, P = pins.rand_case(28, T=0)
    assert O.forward_quadratic(q, k, v, P).shape == (1, 1, 0, 5)
    ST, zT = O.final_state(k, v, P)
    assert np.all(ST == 0) and np.all(zT == 0)
