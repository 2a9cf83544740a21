"""Flash-style O(T^2) forward (kata_flash_forward) against the oracle's O(T^2)
definition, and against the chunked path."""
import numpy as np
import pytest
import torch

import kernelized_linear_attention_kata_amd as kata
from kernelized_linear_attention_kata_amd import inputs as I
from oracle import kata_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL_BF16 = 2e-2


def host64(t):
    return O.bf16_bits_to_f64(I.bf16_bits(t))


def slice_rel(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    g2 = got.reshape(got.shape[0] * got.shape[1], -1)
    r2 = ref.reshape(ref.shape[0] * ref.shape[1], -1)
    den = np.linalg.norm(r2, axis=1)
    return float(np.max(np.linalg.norm(g2 - r2, axis=1) / np.where(den == 0, 1.0, den)))


def flash(case, out_dtype=torch.float32):
    q, k, v, P = (t.to(DEV) for t in (case.q, case.k, case.v, case.P))
    y = kata.flash_forward(q, k, v, P, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("T", [1, 100, 128, 129, 257, 1000])
def test_flash_against_oracle(T):
    """Ragged T (one token, under one 128-query block, one block plus one token, ...)."""
    case = I.make_forward("mid", B=2, H=3, T=T, seed=30 + T)
    y = flash(case).double().cpu().numpy()
    yref = O.forward_quadratic(host64(case.q), host64(case.k), host64(case.v), case.P.double().numpy())
    e = slice_rel(y, yref)
    print(f"[flash mid T={T}] rel y {e:.3e}", flush=True)
    assert e <= TOL_BF16


def test_flash_lm340m_workload():
    """Per-head P and unit-norm keys (the 340M-layer inputs)."""
    case = I.make_forward("lm340m", B=2, H=4, T=384, seed=31)
    y = flash(case).double().cpu().numpy()
    yref = O.forward_quadratic(host64(case.q), host64(case.k), host64(case.v), case.P.double().numpy())
    e = slice_rel(y, yref)
    print(f"[flash lm340m T=384] rel y {e:.3e}", flush=True)
    assert e <= TOL_BF16


def test_flash_matches_chunked_path_and_bf16_output():
    case = I.make_forward("mid", B=2, H=4, T=2048, seed=32)
    q, k, v, P = (t.to(DEV) for t in (case.q, case.k, case.v, case.P))
    yf = kata.flash_forward(q, k, v, P, out_dtype=torch.float32)
    yc = kata.forward(q, k, v, P, chunk=64, out_dtype=torch.float32)
    yb = kata.flash_forward(q, k, v, P)
    torch.cuda.synchronize()
    assert yb.dtype == torch.bfloat16
    e = slice_rel(yf.double().cpu().numpy(), yc.double().cpu().numpy())
    eb = slice_rel(yb.double().cpu().numpy(), yf.double().cpu().numpy())
    print(f"[flash vs chunked T=2048] rel {e:.3e}; bf16 output vs f32 {eb:.3e}", flush=True)
    assert e <= TOL_BF16 and eb <= 1e-2


def test_flash_long_sampled_rows():
    """T = 8192: sampled query rows (first, last, around block edges) against the oracle."""
    case = I.make_forward("mid", B=1, H=2, T=8192, seed=33)
    rows = np.array([0, 1, 63, 64, 127, 128, 129, 1000, 4095, 4096, 8000, 8190, 8191])
    y = flash(case).double().cpu().numpy()[:, :, rows]
    yref = O.forward_quadratic(host64(case.q), host64(case.k), host64(case.v), case.P.double().numpy(), rows=rows)
    e = slice_rel(y, yref)
    print(f"[flash T=8192 sampled] rel y {e:.3e}", flush=True)
    assert e <= TOL_BF16


def test_flash_zero_query_rows_give_zero():
    case = I.make_forward("mid", B=1, H=2, T=300, seed=34)
    case.q[:, :, 0] = 0
    case.q[:, :, 200] = 0
    y = flash(case)
    assert torch.all(y[:, :, 0] == 0) and torch.all(y[:, :, 200] == 0)
    assert torch.all(torch.isfinite(y))
