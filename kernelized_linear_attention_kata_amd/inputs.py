"""Seeded synthetic inputs for the KATA forward pass and decode step.

This module only draws random tensors of the shapes and distributions of the
five workloads below; it contains none of the method's arithmetic.  The GPU
path and the CPU oracle both consume what it produces (the oracle always
reads the stored tensors back, bit-exactly), so the generator never affects
parity.

Workloads (name: shapes, distributions, storage dtype, chunk):

* ``tiny``   B=1, H=1, T=256, d=dv=16, P 16x16 with entries N(0, 1/16)
             (std 1/4), q, k, v standard normal / 4, float32, chunk 32, seed 0.
* ``mid``    B=4, H=8, T=4096, d=dv=64, one P 16x64 with entries N(0, 1/64)
             (std 1/8) shared by all heads, q, k, v standard normal / 8,
             bfloat16, chunk 64, seed 1.
* ``lm340m`` B=8, T=2048, d_model=1024 as 16 heads of 64: hidden states
             X ~ N(0, 1), q/k/v = X W^T with W ~ U(-1/32, 1/32) (a random
             initialised bias-free linear layer), keys L2-normalised per head
             in float32, then all cast to bfloat16; one P per head, chunk 64,
             seed 2.
* ``long``   B=1, H=16, T=131072, d=dv=64, one P shared by all heads, q, k, v
             standard normal / 8, bfloat16, chunk 64 or 128, seed 3.
* ``decode`` 256 streams x 16 heads, d=dv=64, a prefill of 8192 bfloat16
             tokens and 1024 decode steps with q, k, v standard normal / 8;
             at decode step j with j % 4 == 3 the key repeats the key of an
             earlier position of the same stream and head, drawn uniformly
             over every earlier position (prefill included); seed 4.

Draw order within a workload: P, then q, k, v, each as one tensor in
[B, H, T, d] order (for ``lm340m``: X, W_q, W_k, W_v, then P; for ``decode``:
P, prefill q, k, v, decode q, k, v, then the repeat positions).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

P_DIM = 16

WORKLOADS = {
    "tiny": dict(B=1, H=1, T=256, d=16, dtype="f32", chunk=32, seed=0),
    "mid": dict(B=4, H=8, T=4096, d=64, dtype="bf16", chunk=64, seed=1),
    "lm340m": dict(B=8, H=16, T=2048, d=64, dtype="bf16", chunk=64, seed=2),
    "long": dict(B=1, H=16, T=131072, d=64, dtype="bf16", chunk=64, seed=3),
}

DECODE = dict(N=256, H=16, d=64, T_prefill=8192, steps=1024, dtype="bf16", chunk=64, seed=4)


@dataclasses.dataclass
class ForwardInputs:
    name: str
    B: int
    H: int
    T: int
    d: int
    dv: int
    p: int
    chunk: int
    dtype: str                 # "f32" or "bf16": storage dtype of q, k, v
    q: torch.Tensor            # [B, H, T, d]
    k: torch.Tensor            # [B, H, T, d]
    v: torch.Tensor            # [B, H, T, dv]
    P: torch.Tensor            # [H, p, d] float32


@dataclasses.dataclass
class DecodeInputs:
    N: int
    H: int
    d: int
    dv: int
    p: int
    T_prefill: int
    steps: int
    P: torch.Tensor            # [H, p, d] float32
    q0: torch.Tensor           # prefill [N, H, T_prefill, d] bf16
    k0: torch.Tensor
    v0: torch.Tensor
    q: torch.Tensor            # decode [steps, N, H, d] bf16
    k: torch.Tensor            # (repeats already substituted)
    v: torch.Tensor
    repeat_src: torch.Tensor   # [steps, N, H] int64 source position, -1 = fresh key


def _torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, std, g, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def make_forward(name: str, device="cpu", *, B: Optional[int] = None, H: Optional[int] = None,
                 T: Optional[int] = None, chunk: Optional[int] = None,
                 seed: Optional[int] = None, dtype: Optional[str] = None) -> ForwardInputs:
    """Draw one forward workload; any size may be overridden (smaller parity cases)."""
    if name not in WORKLOADS:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}")
    cfg = dict(WORKLOADS[name])
    B = cfg["B"] if B is None else B
    H = cfg["H"] if H is None else H
    T = cfg["T"] if T is None else T
    d = cfg["d"]
    chunk = cfg["chunk"] if chunk is None else chunk
    seed = cfg["seed"] if seed is None else seed
    dtype = cfg["dtype"] if dtype is None else dtype
    tdt = _torch_dtype(dtype)
    g = _gen(seed, device)
    p = P_DIM
    if name == "lm340m":
        dm = H * d
        X = _normal((B, T, dm), 1.0, g, device)
        bound = 1.0 / dm ** 0.5
        Ws = [(torch.rand((dm, dm), generator=g, device=device) * 2.0 - 1.0) * bound for _ in range(3)]
        P = _normal((H, p, d), 1.0 / d ** 0.5, g, device)
        q, k, v = [(X @ W.T).reshape(B, T, H, d).permute(0, 2, 1, 3).contiguous() for W in Ws]
        k = k / k.norm(dim=-1, keepdim=True).clamp_min(1e-30)
        q, k, v = q.to(tdt), k.to(tdt), v.to(tdt)
    else:
        std = 1.0 / d ** 0.5
        P1 = _normal((1, p, d), std, g, device)
        P = P1.expand(H, p, d).contiguous()
        q = _normal((B, H, T, d), std, g, device).to(tdt)
        k = _normal((B, H, T, d), std, g, device).to(tdt)
        v = _normal((B, H, T, d), std, g, device).to(tdt)
    return ForwardInputs(name=name, B=B, H=H, T=T, d=d, dv=d, p=p, chunk=chunk, dtype=dtype,
                         q=q, k=k, v=v, P=P.contiguous())


def make_decode(device="cpu", *, N: Optional[int] = None, H: Optional[int] = None,
                T_prefill: Optional[int] = None, steps: Optional[int] = None,
                seed: Optional[int] = None) -> DecodeInputs:
    """Draw the decode workload (prefill tokens, decode tokens, repeated keys)."""
    cfg = dict(DECODE)
    N = cfg["N"] if N is None else N
    H = cfg["H"] if H is None else H
    T0 = cfg["T_prefill"] if T_prefill is None else T_prefill
    steps = cfg["steps"] if steps is None else steps
    seed = cfg["seed"] if seed is None else seed
    d = cfg["d"]
    p = P_DIM
    std = 1.0 / d ** 0.5
    g = _gen(seed, device)
    P1 = _normal((1, p, d), std, g, device)
    P = P1.expand(H, p, d).contiguous()
    bf = torch.bfloat16
    q0 = _normal((N, H, T0, d), std, g, device).to(bf)
    k0 = _normal((N, H, T0, d), std, g, device).to(bf)
    v0 = _normal((N, H, T0, d), std, g, device).to(bf)
    q = _normal((steps, N, H, d), std, g, device).to(bf)
    k = _normal((steps, N, H, d), std, g, device).to(bf)
    v = _normal((steps, N, H, d), std, g, device).to(bf)
    src = torch.full((steps, N, H), -1, dtype=torch.int64, device=device)
    for j in range(3, steps, 4):
        earlier = T0 + j
        if earlier == 0:
            continue
        r = torch.randint(0, earlier, (N, H), generator=g, device=device)
        src[j] = r
        from_prefill = r < T0
        pre = torch.gather(k0, 2, r.clamp(max=max(T0 - 1, 0)).view(N, H, 1, 1).expand(N, H, 1, d)).squeeze(2) \
            if T0 > 0 else torch.zeros_like(k[j])
        dec_idx = (r - T0).clamp(min=0)
        kd = k.permute(1, 2, 0, 3)       # [N, H, steps, d]
        dec = torch.gather(kd, 2, dec_idx.view(N, H, 1, 1).expand(N, H, 1, d)).squeeze(2)
        k[j] = torch.where(from_prefill.unsqueeze(-1), pre, dec)
    return DecodeInputs(N=N, H=H, d=d, dv=d, p=p, T_prefill=T0, steps=steps, P=P,
                        q0=q0, k0=k0, v0=v0, q=q, k=k, v=v, repeat_src=src)


def make_output_grad(B: int, H: int, T: int, dv: int, dtype: str = "bf16", seed: int = 0,
                     device="cpu") -> torch.Tensor:
    """A seeded gradient of the loss with respect to y, [B, H, T, dv]: standard normal / 8
    (the scale of the value inputs), stored in ``dtype`` ("bf16" or "f32")."""
    g = _gen(1000 + seed, device)
    return _normal((B, H, T, dv), 1.0 / 8.0, g, device).to(_torch_dtype(dtype))


def make_state_grad(B: int, H: int, dv: int, seed: int = 0, device="cpu"):
    """A seeded gradient (gST, gzT) of the loss with respect to the final state, float32,
    standard normal / 8 (not symmetric in the feature pair)."""
    g = _gen(2000 + seed, device)
    gST = _normal((B, H, P_DIM * P_DIM, dv), 1.0 / 8.0, g, device)
    gzT = _normal((B, H, P_DIM * P_DIM), 1.0 / 8.0, g, device)
    return gST, gzT


def make_log_decay(B: int, H: int, T: int, seed: int = 0, lo: float = 0.9, hi: float = 1.0,
                   device="cpu") -> torch.Tensor:
    """Seeded log-gates lam = log(gamma) [B, H, T] float32 with gamma uniform in [lo, hi]
    (per token and head), the range of forget gates of gated linear attention."""
    g = _gen(3000 + seed, device)
    gam = lo + (hi - lo) * torch.rand((B, H, T), generator=g, device=device, dtype=torch.float32)
    return torch.log(gam)


def make_beta(*shape: int, seed: int = 0, lo: float = 0.5, hi: float = 1.0, device="cpu") -> torch.Tensor:
    """Seeded delta-rule write strengths beta, float32 uniform in [lo, hi], of the given
    shape ([B, H, T] for a forward, [N, H] or [steps, N, H] for decode steps)."""
    g = _gen(4000 + seed, device)
    return lo + (hi - lo) * torch.rand(shape, generator=g, device=device, dtype=torch.float32)


def make_factor_projections(H: int, g: int, d: int = 64, seed: int = 0, per_head: bool = False,
                            device="cpu") -> torch.Tensor:
    """Seeded projections of g PSD factors, P [H, g, 16, d] float32 with entries N(0, 1/d)
    (each factor drawn like the one projection of the one-factor workloads); one set shared
    by all heads unless per_head."""
    gen = _gen(5000 + seed, device)
    std = 1.0 / d ** 0.5
    if per_head:
        return _normal((H, g, P_DIM, d), std, gen, device)
    return _normal((1, g, P_DIM, d), std, gen, device).expand(H, g, P_DIM, d).contiguous()


def bf16_bits(t: torch.Tensor):
    """Raw uint16 bit patterns of a bfloat16 tensor, as a numpy array on the host."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")
