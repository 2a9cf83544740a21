"""The *_timed entry points (kata_forward_timed, kata_forward_decay_timed,
kata_forward_factors_timed, kata_forward_delta_chunked_timed, kata_flash_forward with
events, kata_backward_timed): the events ride on the launches and change nothing else.

For every path, a call with all events and a call with only some of them (the rest
NULL, which the library skips) give outputs bit-identical to the untimed call: the same
kernels run on the same inputs, none of them with atomics.  The stamped events mark
the launches in order, so the intervals between them are non-negative, and a launch's
start and end stamps bracket a positive duration."""
import pytest
import torch

import kernelized_linear_attention_kata_amd as kata
from kernelized_linear_attention_kata_amd import inputs as I

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def small_case(T=300, H=2, seed=11):
    c = I.make_forward("long", B=1, H=H, T=T, seed=seed)
    return tuple(t.to(DEV) for t in (c.q, c.k, c.v, c.P))


def event_sets(n):
    """No events, all n, and every other one (the first and the last always kept)."""
    full = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    part = [torch.cuda.Event(enable_timing=True) if (j % 2 == 0 or j == n - 1) else None for j in range(n)]
    return [None, full, part]


def check_events(evs):
    stamped = [e for e in evs if e is not None]
    assert len(stamped) >= 2
    for a, b in zip(stamped, stamped[1:]):
        assert a.query() and b.query()
        assert a.elapsed_time(b) >= 0.0
    assert stamped[0].elapsed_time(stamped[-1]) > 0.0


def same_outputs(run, n_events):
    ref = None
    for evs in event_sets(n_events):
        out = run(evs)
        torch.cuda.synchronize()
        out = [o.clone() for o in (out if isinstance(out, (tuple, list)) else (out,))]
        if ref is None:
            ref = out
        else:
            for a, b in zip(out, ref):
                assert torch.equal(a, b)
            check_events(evs)


def test_forward_timed():
    q, k, v, P = small_case()
    same_outputs(lambda ev: kata.forward(q, k, v, P, 64, return_state=True, events=ev), 4)


def test_forward_decay_timed():
    q, k, v, P = small_case()
    lam = I.make_log_decay(1, q.shape[1], q.shape[2], seed=3).to(DEV)
    same_outputs(lambda ev: kata.forward_decay(q, k, v, P, lam, 64, return_state=True, events=ev), 4)


@pytest.mark.parametrize("mode", ["concat", "sum"])
def test_forward_factors_timed(mode):
    q, k, v, _ = small_case()
    Pg = I.make_factor_projections(q.shape[1], 2, 64, seed=5).to(DEV)
    same_outputs(lambda ev: kata.forward_factors(q, k, v, Pg, mode, 64, return_state=True, events=ev), 4)


def test_forward_delta_chunked_timed():
    q, k, v, P = small_case()
    beta = I.make_beta(1, q.shape[1], q.shape[2], seed=4).to(DEV)
    same_outputs(lambda ev: kata.forward_delta_chunked(q, k, v, P, beta, return_state=True, events=ev), 3)


def test_flash_forward_timed():
    q, k, v, P = small_case()
    same_outputs(lambda ev: kata.flash_forward(q, k, v, P, events=ev), 3)


def test_backward_timed():
    q, k, v, P = small_case()
    gy = I.make_output_grad(1, q.shape[1], q.shape[2], v.shape[-1], seed=6).to(DEV)
    same_outputs(lambda ev: kata.backward(q, k, v, P, gy, 64, events=ev), 8)


def test_wrong_event_count_is_rejected():
    q, k, v, P = small_case(T=64, H=1)
    with pytest.raises(ValueError):
        kata.forward(q, k, v, P, 64, events=[torch.cuda.Event(enable_timing=True)] * 3)
