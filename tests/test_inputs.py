"""Seeded input generators: determinism and the workload recipes (CPU only)."""
import torch

from kernelized_linear_attention_kata_amd import inputs as I


def test_same_seed_same_bytes():
    a = I.make_forward("mid", B=1, H=2, T=128)
    b = I.make_forward("mid", B=1, H=2, T=128)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v), (a.P, b.P)):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y)


def test_shapes_and_dtypes():
    t = I.make_forward("tiny")
    assert t.q.shape == (1, 1, 256, 16) and t.q.dtype == torch.float32 and t.chunk == 32
    assert t.P.shape == (1, 16, 16)
    m = I.make_forward("mid", B=2, H=3, T=64)
    assert m.q.dtype == torch.bfloat16 and m.P.shape == (3, 16, 64)
    assert torch.equal(m.P[0], m.P[2])          # one P shared by the heads


def test_lm340m_keys_unit_norm_and_per_head_P():
    c = I.make_forward("lm340m", B=1, T=32)
    n = c.k.float().norm(dim=-1)
    assert torch.all((n - 1).abs() < 2e-2)
    assert not torch.equal(c.P[0], c.P[1])


def test_decode_repeat_pattern():
    d = I.make_decode(N=3, H=2, T_prefill=10, steps=12)
    src = d.repeat_src
    for j in range(12):
        if j % 4 == 3:
            assert torch.all(src[j] >= 0) and torch.all(src[j] < 10 + j)
            for n in range(3):
                for h in range(2):
                    r = int(src[j, n, h])
                    ref = d.k0[n, h, r] if r < 10 else d.k[r - 10, n, h]
                    assert torch.equal(d.k[j, n, h].view(torch.int16), ref.view(torch.int16))
        else:
            assert torch.all(src[j] == -1)
