"""The parity bar must reject plausible wrong results (negative controls).

On the tiny workload, the oracle's own output rounded to bf16 passes the bar,
while each planted error must fail it: zero output, gate left out, softmax
scale 1/sqrt(d_model) instead of 1/sqrt(D), one token sent to a wrong group,
and a group boundary moved by one row.
"""

import math

import numpy as np
import pytest

import oracle
from parity import bf16_round, output_errors, output_ok
from workloads import get_workload, make_inputs
from workloads.gen import to_numpy_f32


@pytest.fixture(scope="module")
def case():
    wl = get_workload("tiny")
    inp = make_inputs(wl, device="cpu")
    X, Wr, Q, K, V = (to_numpy_f32(inp[k]) for k in ("X", "Wr", "Q", "K", "V"))
    out = oracle.moga_forward(X, Wr, Q, K, V, wl.M)
    return wl, X, Wr, Q, K, V, out


def test_rounded_oracle_passes(case):
    *_, out = case
    e = output_errors(bf16_round(out["O"]), out["O"])
    assert output_ok(e), e


def _fails(got, want):
    e = output_errors(got, want)
    assert not output_ok(e), f"negative control passed the bar: {e}"


def test_zero_output_fails(case):
    *_, out = case
    _fails(np.zeros_like(out["O"]), out["O"])


def test_missing_gate_fails(case):
    *_, out = case
    _fails(out["O"] / out["gate"].astype(np.float64)[:, None, None], out["O"])


def test_wrong_scale_fails(case):
    wl, X, Wr, Q, K, V, out = case
    bad = oracle.moga_forward(X, Wr, Q, K, V, wl.M, scale=1 / math.sqrt(wl.d_model))
    _fails(bf16_round(bad["O"]), out["O"])


def test_one_token_rerouted_fails(case):
    wl, X, Wr, Q, K, V, out = case
    g = out["group_id"].copy()
    n = 17
    g[n] = (g[n] + 1) % wl.M
    rows = np.arange(X.shape[0])
    bad = oracle.moga_output_rows(X, Wr, Q, K, V, wl.M, rows, routed=(g, out["gate"]))
    _fails(bf16_round(bad), out["O"])


def test_boundary_off_by_one_fails(case):
    wl, X, Wr, Q, K, V, out = case
    perm, cu = out["perm"], out["cu_seqlens"].copy()
    cu[1] += 1
    Qp, Kp, Vp = (oracle.gather_rows(T, perm) for T in (Q, K, V))
    Op = oracle.group_attention(Qp, Kp, Vp, cu, 1 / math.sqrt(wl.D))
    bad = oracle.unpermute(Op, perm, out["gate"])
    _fails(bf16_round(bad), out["O"])


# ---------------------------------------------------------------------------
# Gradient bars (backward pass): the oracle's gradients rounded to bf16 pass,
# plausible mistakes fail
# ---------------------------------------------------------------------------

from parity import assert_grad_close  # noqa: E402


@pytest.fixture(scope="module")
def grads():
    wl = get_workload("tiny")
    inp = make_inputs(wl, device="cpu")
    X, Wr, Q, K, V = (to_numpy_f32(inp[k]) for k in ("X", "Wr", "Q", "K", "V"))
    dO = bf16_round(np.random.default_rng(3).standard_normal(Q.shape))
    ref = oracle.moga_backward(X, Wr, Q, K, V, wl.M, dO)
    return wl, X, Wr, Q, K, V, dO, ref


def _grad_fails(got, want, what):
    with pytest.raises(AssertionError):
        assert_grad_close(got, want, what)


def test_rounded_gradients_pass(grads):
    *_, ref = grads
    for k in ("dQ", "dK", "dV"):
        assert_grad_close(bf16_round(ref[k]), ref[k], k)


def test_gradient_without_delta_fails(grads):
    wl, X, Wr, Q, K, V, dO, ref = grads
    scale = 1 / math.sqrt(wl.D)
    bad = ref["dQ"].copy()
    perm, cu = ref["perm"], ref["cu_seqlens"]
    for i in range(wl.M):
        rows = perm[cu[i]:cu[i + 1]]
        for h in range(wl.H):
            P = np.exp(scale * Q[rows, h] @ K[rows, h].T - ref["lse"][h, cu[i]:cu[i + 1], None])
            bad[rows, h] += scale * (P * ref["delta"][h, cu[i]:cu[i + 1], None]) @ K[rows, h]
    _grad_fails(bf16_round(bad), ref["dQ"], "dQ without delta")


def test_gradient_missing_scale_fails(grads):
    wl, *_, ref = grads
    _grad_fails(bf16_round(ref["dK"] * math.sqrt(wl.D)), ref["dK"], "dK without scale")


def test_gradient_ungated_dv_fails(grads):
    wl, X, Wr, Q, K, V, dO, ref = grads
    bad = ref["dV"] / ref["gate"][:, None, None]   # dV of a row mixes the group's gates; this rescales it
    _grad_fails(bf16_round(bad), ref["dV"], "dV with the gate left out")


def test_router_gradient_mistakes_fail(grads):
    *_, ref = grads
    _grad_fails(-ref["dX"], ref["dX"], "dX sign")
    _grad_fails(ref["dWr"] / np.mean(ref["gate"]), ref["dWr"], "dWr without p_g")
    _grad_fails(ref["dgate"] * ref["gate"], ref["dgate"], "dgate of the gated output")
