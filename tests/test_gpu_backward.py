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


def _stage(moga, tr, extra, heads=None):
    """Give tr's attention backward the workspace that keeps dS of all heads
    (or of `heads` heads) for its groups, plus `extra` bytes (negative: too
    small by that much)."""
    need = moga.moga_attention_backward_staged_bytes(tr.cu_seqlens, tr.H)
    if heads is not None:
        need = 4096 + (need - 4096) // tr.H * heads
    tr.ws_bwd = torch.empty(need + extra, dtype=torch.uint8, device=DEV)
    return need


def _check(moga, X, Wr, Q, K, V, dO, bias=None, label="", staged=None):
    N, H, D = Q.shape
    M, d = Wr.shape
    print(f"[backward] {label} N={N} H={H} D={D} M={M} d={d} staged={staged}", flush=True)
    tr = moga.MogaTraining(N, d, H, D, M, DEV)
    tr.forward(X, Wr, Q, K, V, bias)
    if staged is not None:
        _stage(moga, tr, staged)
    grads = tr.backward(dO)
    torch.cuda.synchronize()
    if staged is not None:
        assert moga.moga_attention_backward_staged(tr.ws_bwd) == (H if staged >= 0 else H - 1)
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


def _sweep_shapes(seed, count):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 6001)), int(rng.integers(1, 4)), int(rng.choice([64, 128])),
             int(rng.integers(1, 33)), int(rng.choice([64, 128]))) for _ in range(count)]


@pytest.mark.parametrize("N,H,D,M,d", _sweep_shapes(2025, 5))
def test_backward_shape_sweep(moga, N, H, D, M, d):
    _check(moga, *_case("wan13b_21f", seed=N + M, N=N, H=H, D=D, M=M, d_model=d), label=f"sweep {N, H, D, M, d}")


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


def _unstaged(moga, tr):
    """The attention backward of tr's saved state with the minimum workspace."""
    return moga.moga_group_attention_backward(tr.Qp, tr.Kp, tr.Vp, tr.dOp, tr.lse, tr.delta, tr.cu_seqlens,
                                              tr.perm, 0.0)


@pytest.mark.parametrize("N,H,D,M,d", [
    (3001, 2, 128, 5, 256),   # ragged groups: partial key and query blocks, odd block counts
    (777, 3, 64, 3, 128),
    (1, 2, 128, 4, 128),      # one token: one block of one query and one key, plus the zero padding block
    (2000, 1, 64, 64, 128),   # many (and empty) groups
    (9000, 2, 128, 3, 128),   # groups of thousands: many 64-key tiles per dQ item
])
def test_backward_staged(moga, N, H, D, M, d):
    """dS kept in the workspace: gradients against the oracle; dK and dV
    bitwise those of the minimum-workspace call (same kernel arithmetic), dQ
    within float32 rounding of it."""
    X, Wr, Q, K, V, dO, _ = _case("wan13b_21f", seed=81 + N, N=N, H=H, D=D, M=M, d_model=d)
    tr, grads = _check(moga, X, Wr, Q, K, V, dO, label=f"staged {N, H, D, M, d}", staged=0)
    dQ, dK, dV = _unstaged(moga, tr)
    torch.cuda.synchronize()
    assert torch.equal(dK, grads["dK"]) and torch.equal(dV, grads["dV"])
    diff = (dQ.float() - grads["dQ"].float()).norm() / max(dQ.float().norm().item(), 1e-30)
    print(f"[backward] staged vs unstaged dQ rel_fro {diff.item():.2e} "
          f"(bitwise {torch.equal(dQ, grads['dQ'])})", flush=True)
    assert diff.item() <= 1e-2


def _staged_vs_unstaged(moga, sizes, H, D, seed, label):
    """The staged form against the minimum-workspace form on the same saved
    state (random Q, K, V, dO in permuted order, groups of the given sizes):
    dK and dV bitwise, dQ within float32 rounding."""
    N, M = sum(sizes), len(sizes)
    print(f"[backward] {label} D={D} H={H} sizes={sizes}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(seed)
    Qp, Kp, Vp, dO = (torch.randn(N, H, D, generator=g, device=DEV).bfloat16() for _ in range(4))
    cu = torch.tensor([0] + list(np.cumsum(sizes)), dtype=torch.int32, device=DEV)
    perm = torch.arange(N, dtype=torch.int32, device=DEV)
    gate = torch.ones(N, dtype=torch.float32, device=DEV)
    Op, lse = moga.moga_group_attention_train(Qp, Kp, Vp, cu)
    dOp, delta, _ = moga.moga_unpermute_backward(dO, Op, perm, gate)
    need = moga.moga_attention_backward_staged_bytes(cu, H)
    nb = [(n + 31) // 32 for n in sizes]
    assert need == 4096 + H * sum(b * (b + b % 2) for b in nb) * 2048
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    a = moga.moga_group_attention_backward(Qp, Kp, Vp, dOp, lse, delta, cu, perm, 0.0, ws=ws)
    b = moga.moga_group_attention_backward(Qp, Kp, Vp, dOp, lse, delta, cu, perm, 0.0)
    torch.cuda.synchronize()
    assert moga.moga_attention_backward_staged(ws) == H
    for t in a:
        assert torch.isfinite(t.float()).all()
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
    diff = (a[0].float() - b[0].float()).norm() / b[0].float().norm()
    print(f"[backward] {label} D={D}: dQ rel_fro vs unstaged {diff.item():.2e}", flush=True)
    assert diff.item() <= 1e-2


@pytest.mark.parametrize("D", [64, 128])
def test_backward_staged_block_edges(moga, D):
    """Group sizes at the 32-row block edges: odd and even block counts,
    partial key and query blocks, the zero padding block, one-row groups."""
    _staged_vs_unstaged(moga, [1, 31, 32, 33, 63, 64, 65, 255, 256, 257], 2, D, 91 + D, "staged block edges")


def _staged_sweep(seed, count):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        M = int(rng.integers(1, 33))
        sizes = rng.multinomial(int(rng.integers(1, 6001)), rng.dirichlet(np.full(M, 0.7))).tolist()
        out.append((sizes, int(rng.integers(1, 4)), int(rng.choice([64, 128]))))
    return out


@pytest.mark.parametrize("sizes,H,D", _staged_sweep(2026, 8))
def test_backward_staged_sweep(moga, sizes, H, D):
    """Seeded random group sizes (empty groups included), heads and widths."""
    if sum(sizes) == 0:
        sizes[0] = 1
    _staged_vs_unstaged(moga, sizes, H, D, 97 + sum(sizes), "staged sweep")


def test_backward_staged_partial(moga):
    """A workspace one byte short of all heads' dS: the device plan keeps the
    first H-1 heads; the last head's dQ is the minimum-workspace result bit
    for bit, dK and dV are bitwise equal for every head."""
    X, Wr, Q, K, V, dO, _ = _case("wan13b_21f", seed=83, N=3001, H=3, D=128, M=5, d_model=256)
    tr, grads = _check(moga, X, Wr, Q, K, V, dO, label="staged, one byte short", staged=-1)
    dQ, dK, dV = _unstaged(moga, tr)
    torch.cuda.synchronize()
    assert torch.equal(dK, grads["dK"]) and torch.equal(dV, grads["dV"])
    assert torch.equal(dQ[:, 2], grads["dQ"][:, 2])
    diff = (dQ[:, :2].float() - grads["dQ"][:, :2].float()).norm() / dQ[:, :2].float().norm()
    assert diff.item() <= 1e-2


def test_backward_staged_too_small(moga):
    """A workspace one byte short of a single head's dS: nothing is staged,
    bitwise the minimum-workspace result."""
    X, Wr, Q, K, V, dO, _ = _case("wan13b_21f", seed=85, N=3001, H=2, D=128, M=5, d_model=256)
    N, H, D = Q.shape
    tr = moga.MogaTraining(N, 256, H, D, 5, DEV)
    tr.forward(X, Wr, Q, K, V)
    _stage(moga, tr, -1, heads=1)
    grads = tr.backward(dO)
    torch.cuda.synchronize()
    assert moga.moga_attention_backward_staged(tr.ws_bwd) == 0
    dQ, dK, dV = _unstaged(moga, tr)
    torch.cuda.synchronize()
    assert torch.equal(dQ, grads["dQ"]) and torch.equal(dK, grads["dK"]) and torch.equal(dV, grads["dV"])


def test_backward_staged_deterministic(moga):
    X, Wr, Q, K, V, dO, _ = _case("wan13b_21f", seed=84, N=4000, H=2, D=128, M=4, d_model=128)
    tr = moga.MogaTraining(4000, 128, 2, 128, 4, DEV)
    tr.forward(X, Wr, Q, K, V)
    _stage(moga, tr, 4096)
    a = {k: v.clone() for k, v in tr.backward(dO).items()}
    b = tr.backward(dO)
    torch.cuda.synchronize()
    assert moga.moga_attention_backward_staged(tr.ws_bwd) == 2
    for k in a:
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("name,staged", [("wan13b_21f", False), ("clip30s_122f", False), ("clip30s_122f", True)])
def test_backward_full_size(moga, name, staged):
    """Full-size training backward in the configuration the bench times:
    sampled rows of dQ, dgate and the router's dX against the oracle row by
    row, and two group invariants over every row: a group's dV sums to its
    gated upstream gradient (softmax rows sum to 1) and its dK sums to zero
    (the row sums of dS vanish)."""
    from workloads import sample_rows
    wl = get_workload(name)
    print(f"[backward] full size {name} N={wl.N} H={wl.H} M={wl.M}", flush=True)
    inp = make_inputs(wl, device=DEV)
    X, Wr, Q, K, V = (inp[k] for k in ("X", "Wr", "Q", "K", "V"))
    g = torch.Generator(device=DEV).manual_seed(wl.seed)
    dO = torch.randn(Q.shape, generator=g, device=DEV).bfloat16()
    tr = moga.MogaTraining(wl.N, wl.d_model, wl.H, wl.D, wl.M, DEV)
    tr.forward(X, Wr, Q, K, V)
    if staged:
        print(f"[backward] full size {name}: staged dS workspace {_stage(moga, tr, 0) / 2**30:.1f} GiB", flush=True)
    grads = tr.backward(dO)
    torch.cuda.synchronize()
    assert moga.moga_attention_backward_staged(tr.ws_bwd) == (wl.H if staged else 0)
    Xn, Wn = _np(X), _np(Wr)
    g_ref, _, logits = oracle.route(Xn, Wn)
    np.testing.assert_array_equal(tr.group_id.cpu().numpy(), g_ref)
    rows = sample_rows(g_ref, wl.M, per_group=2, seed=wl.seed)
    ref = oracle.moga_backward_rows(Xn, Wn, _np(Q), _np(K), _np(V), wl.M, _np(dO), rows, routed=(g_ref, logits))
    idx = torch.from_numpy(rows).to(DEV)
    errs = {}
    for k in ("dQ", "dgate", "dX"):
        errs[k] = round(assert_grad_close(grads[k][idx].float().cpu().numpy(), ref[k], f"{name} {k}")["rel_fro"], 5)
    # group sums over all rows, in float64 on the device
    gid = tr.group_id.long()
    dA = tr.gate[:, None, None].double() * dO.double()
    sums = {}
    for k, t in (("dV", grads["dV"].double()), ("dK", grads["dK"].double()), ("dA", dA)):
        z = torch.zeros((wl.M,) + tuple(Q.shape[1:]), dtype=torch.float64, device=DEV)
        sums[k] = z.index_add_(0, gid, t).cpu().numpy()
    absum = {k: torch.zeros((wl.M,) + tuple(Q.shape[1:]), dtype=torch.float64, device=DEV)
             .index_add_(0, gid, grads[k].double().abs()).cpu().numpy() for k in ("dV", "dK")}
    v_err = np.abs(sums["dV"] - sums["dA"]).max() / absum["dV"].max()
    k_err = np.abs(sums["dK"]).max() / absum["dK"].max()
    print(f"[backward] full size {name}: {rows.size} rows rel_fro {errs}; group-sum errors dV {v_err:.2e} "
          f"dK {k_err:.2e}", flush=True)
    assert v_err <= 5e-3 and k_err <= 5e-3
