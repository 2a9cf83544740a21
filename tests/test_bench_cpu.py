"""Host-side parts of bench.py (no GPU): the one-GPU guard, and the algorithmic byte
counts that the roofline's achieved rate is built on, checked against the sizes of the
tensors the step reads and writes and against the library's own leaf-state buffer."""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def nbytes(*shape, dtype=torch.bfloat16):
    return torch.empty(shape, dtype=dtype, device="meta").numel() * torch.empty((), dtype=dtype).element_size()


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       timeout=120, env={**os.environ, **env}, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def lib():
    try:
        import kernelized_linear_attention_kata_amd as kata
        kata.forward_workspace_bytes(1, 1, 64, 64, 64, 64)
        return kata
    except (OSError, ImportError, RuntimeError) as e:  # library not built here
        pytest.skip(f"libkata not loadable: {e}")


@pytest.mark.parametrize("chunk", [64, 128])
def test_forward_bytes_match_tensor_and_workspace_sizes(chunk):
    """The long-context workload: the state pass reads k and v and writes the leaf
    states; the intra pass reads q, k, v and the scanned leaf states and writes y; the
    scan reads and writes the leaf states but for their 8 * dv unused packed slots
    (delta = 8, a >= 8) and writes the final state (S, z).  The leaf states are exactly
    the library's forward workspace."""
    kata = lib()
    B, H, T, d, dv = 1, 16, 131072, 64, 64
    ws = kata.forward_workspace_bytes(B, H, T, d, dv, chunk)
    E = 144 * dv + 256
    assert ws % (B * H * E * 4) == 0
    n_leaf = ws // (B * H * E * 4)
    got = bench.algorithmic_bytes(B, H, T, d, dv, n_leaf, 2, 2)
    qkv = nbytes(B, H, T, d) * 2 + nbytes(B, H, T, dv)
    y = nbytes(B, H, T, dv)
    final = nbytes(B, H, 256, dv, dtype=torch.float32) + nbytes(B, H, 256, dtype=torch.float32)
    assert got["kata_chunk_state"] == nbytes(B, H, T, d) + nbytes(B, H, T, dv) + ws
    assert got["kata_chunk_intra"] == qkv + ws + y
    unused = B * H * n_leaf * 8 * dv * 4
    assert got["kata_state_scan"] == 2 * (ws - unused) + final


def test_decay_and_factor_bytes():
    """Decay adds the fp32 log-gates (read by both token passes) and one float per leaf;
    g concatenated factors multiply the leaf states, not the token streams."""
    B, H, T, d, dv, n = 1, 16, 131072, 64, 64, 48
    base = bench.algorithmic_bytes(B, H, T, d, dv, n, 2, 2)
    dec = bench.algorithmic_bytes(B, H, T, d, dv, n, 2, 2, decay=True)
    lam = nbytes(B, H, T, dtype=torch.float32)
    per_leaf = nbytes(B, H, n, dtype=torch.float32)
    assert dec["kata_chunk_state"] - base["kata_chunk_state"] == lam + per_leaf
    assert dec["kata_chunk_intra"] - base["kata_chunk_intra"] == lam
    mg = bench.algorithmic_bytes(B, H, T, d, dv, n, 2, 2, factors=2)
    states = B * H * n * (144 * dv + 256) * 4
    assert mg["kata_chunk_intra"] - base["kata_chunk_intra"] == states
    assert mg["kata_chunk_state"] - base["kata_chunk_state"] == states


def test_backward_bytes_match_workspace():
    """The backward's leaf count recovered from its workspace as bench.py does, and the key
    walk's bytes: q, k, v, gy and the per-token (1/den, h) pair read, dk, dv written,
    plus the leaf states and the dP partials."""
    kata = lib()
    B, H, T, d, dv = 1, 16, 131072, 64, 64
    ws = kata.backward_workspace_bytes(B, H, T, d, dv, 64)
    E = 144 * dv + 256
    tok = B * H * T
    n_leaf = (ws - tok * 8) // (2 * B * H * (E + 16 * d) * 4)
    assert ws == tok * 8 + 2 * B * H * n_leaf * (E + 16 * d) * 4
    got = bench.bwd_algorithmic_bytes(B, H, T, d, dv, n_leaf, 2)
    states = B * H * n_leaf * E * 4
    parts = B * H * n_leaf * 16 * d * 4
    streams = (2 * nbytes(B, H, T, d) + nbytes(B, H, T, dv) + nbytes(B, H, T, dv)   # q, k, v, gy
               + nbytes(B, H, T, 2, dtype=torch.float32)                            # (1/den, h)
               + nbytes(B, H, T, d) + nbytes(B, H, T, dv))                          # dk, dv
    assert got["kata_bwd_key"] == streams + states + parts


def test_bytes_without_a_scan():
    """When the plan runs no scan, the intra pass reads the earlier leaves' states (leaf g
    reads g of them) and writes the final state; the scan moves nothing."""
    B, H, T, d, dv, n = 8, 16, 2048, 64, 64, 4
    got = bench.algorithmic_bytes(B, H, T, d, dv, n, 2, 2, scan=False)
    E = 144 * dv + 256
    final = nbytes(B, H, 256, dv, dtype=torch.float32) + nbytes(B, H, 256, dtype=torch.float32)
    tokens = nbytes(B, H, T, d) * 2 + nbytes(B, H, T, dv) * 2
    assert got["kata_state_scan"] == 0
    assert got["kata_chunk_intra"] == tokens + B * H * (0 + 1 + 2 + 3) * E * 4 + final
    assert got["kata_chunk_state"] == nbytes(B, H, T, d) + nbytes(B, H, T, dv) + B * H * n * E * 4
