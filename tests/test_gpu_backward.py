"""Parity of the HIP backward pass (through the C ABI) with the CPU oracle.

The oracle's moga_backward gives the gradients of sum(O * dO) for the MoGA
output in float64; the GPU path runs moga_group_attention_train (saving the
log-sum-exp), moga_unpermute_backward, moga_group_attention_backward and
moga_route_backward.  Gradients are compared with the relative bars of
tests/parity.py (assert_grad_close); the saved log-sum-exp and the row sums
delta with absolute float32 bars.
"""

import numpy as np
import pytest
import torch

import oracle
from parity import assert_grad_close, assert_output_close
from workloads import get_workload, make_inputs
from workloads.gen import to_numpy_f32

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def moga():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_long_router_amd as m
    return m


def _np(t):
    return to_numpy_f32(t)


def _case(name, seed=None, bias=False, **over):
    inp = make_inputs(get_workload(name), device="cpu", seed=seed, **over)
    X, Wr, Q, K, V = (inp[k].to(DEV) for k in ("X", "Wr", "Q", "K", "V"))
    g = torch.Generator().manual_seed(4242 + X.shape[0])
    dO = torch.randn(Q.shape, generator=g).bfloat16().to(DEV)
    b = (torch.randn(Wr.shape[0], generator=g) * 0.5).to(DEV) if bias else None
    return X, Wr, Q, K, V, dO, b


def _check(moga, X, Wr, Q, K, V, dO, bias=None, label=""):
    N, H, D = Q.shape
    M, d = Wr.shape
    print(f"[backward] {label} N={N} H={H} D={D} M={M} d={d}", flush=True)
    tr = moga.MogaTraining(N, d, H, D, M, DEV)
    tr.forward(X, Wr, Q, K, V, bias)
    grads = tr.backward(dO)
    torch.cuda.synchronize()
    ref = oracle.moga_backward(_np(X), _np(Wr), _np(Q), _np(K), _np(V), M, _np(dO),
                               bias=None if bias is None else bias.cpu().numpy())
    np.testing.assert_array_equal(tr.group_id.cpu().numpy(), ref["group_id"])
    np.testing.assert_array_equal(tr.perm.cpu().numpy(), ref["perm"])
    assert_output_close(_np(tr.Op), ref["Op"], "Op")
    np.testing.assert_allclose(tr.lse.cpu().numpy(), ref["lse"], atol=2e-4, rtol=0)
    assert_grad_close(tr.delta.cpu().numpy(), ref["delta"], "delta")
    errs = {}
    for k in ("dgate", "dQ", "dK", "dV", "dX", "dWr", "dbias"):
        got = grads[k].float().cpu().numpy()
        if k == "dbias" and np.abs(ref[k]).max() == 0:
            assert np.abs(got).max() == 0
            continue
        errs[k] = round(assert_grad_close(got, ref[k], k)["rel_fro"], 5)
    print(f"[backward] {label} rel_fro {errs}", flush=True)
    return tr, grads


def test_backward_tiny(moga):
    _check(moga, *_case("tiny"), label="tiny")


@pytest.mark.parametrize("N,H,D,M,d", [
    (3001, 2, 128, 5, 256),   # ragged groups, several tiles
    (777, 3, 64, 3, 128),
    (1, 2, 128, 4, 128),      # one token: one group of one
    (5, 2, 64, 3, 64),
    (2500, 2, 128, 1, 128),   # M = 1: the router gradient vanishes
    (2000, 1, 64, 64, 128),   # many (and empty) groups
])
def test_backward_shapes(moga, N, H, D, M, d):
    _check(moga, *_case("wan13b_21f", seed=77, N=N, H=H, D=D, M=M, d_model=d), label=f"shape {N, H, D, M, d}")


def test_backward_with_bias(moga):
    X, Wr, Q, K, V, dO, b = _case("wan13b_21f", seed=78, bias=True, N=1500, H=2, D=128, M=6, d_model=128)
    _check(moga, X, Wr, Q, K, V, dO, b, label="bias")


def test_backward_mid_size(moga):
    """Groups of thousands of rows: many key and query tiles per item."""
    _check(moga, *_case("clip30s_122f", N=12000, H=4, D=128, M=6, d_model=256), label="mid size")


def test_backward_deterministic(moga):
    X, Wr, Q, K, V, dO, _ = _case("wan13b_21f", seed=79, N=4000, H=2, D=128, M=4, d_model=128)
    tr = moga.MogaTraining(4000, 128, 2, 128, 4, DEV)
    tr.forward(X, Wr, Q, K, V)
    a = {k: v.clone() for k, v in tr.backward(dO).items()}
    b = tr.backward(dO)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k
