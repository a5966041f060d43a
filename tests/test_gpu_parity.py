"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Integer results (group ids, permutation, cu_seqlens, max_seqlen, gathered rows)
must be bit-exact; float32 gates within GATE_RTOL; bf16 outputs within the
max-abs / mean-abs / relative-Frobenius bars of tests/parity.py.
"""

import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
from parity import assert_gate_close, assert_output_close
from workloads import get_workload, make_inputs, make_shots, sample_rows
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


def _inputs(name, seed=None, device="cpu", **over):
    """Draw on the CPU (reproducible) and move to the GPU."""
    inp = make_inputs(get_workload(name), device=device, seed=seed, **over)
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def _full_check(moga, inp, bias=None, label=""):
    wl = inp["workload"]
    X, Wr, Q, K, V = (inp[k] for k in ("X", "Wr", "Q", "K", "V"))
    M = Wr.shape[0]
    print(f"[parity] {label} N={X.shape[0]} H={Q.shape[1]} D={Q.shape[2]} M={M}", flush=True)
    gid, gate = moga.moga_route(X, Wr, bias)
    p = moga.moga_permute(gid, M, Q, K, V)
    Op = moga.moga_group_attention(p["Qp"], p["Kp"], p["Vp"], p["cu_seqlens"])
    O = moga.moga_unpermute(Op, p["perm"], gate)
    torch.cuda.synchronize()

    Xn, Wn, Qn, Kn, Vn = (_np(t) for t in (X, Wr, Q, K, V))
    bn = None if bias is None else bias.cpu().numpy()
    ref = oracle.moga_forward(Xn, Wn, Qn, Kn, Vn, M, bias=bn)
    np.testing.assert_array_equal(gid.cpu().numpy(), ref["group_id"])
    assert_gate_close(gate.cpu().numpy(), ref["gate"])
    np.testing.assert_array_equal(p["perm"].cpu().numpy(), ref["perm"])
    np.testing.assert_array_equal(p["cu_seqlens"].cpu().numpy(), ref["cu_seqlens"])
    assert int(p["max_seqlen"].item()) == ref["max_seqlen"]
    perm = p["perm"].long()
    for a, b in ((p["Qp"], Q), (p["Kp"], K), (p["Vp"], V)):
        assert torch.equal(a, b[perm])
    e_attn = assert_output_close(_np(Op), ref["Op"], "Op")
    e_out = assert_output_close(_np(O), ref["O"], "O")
    Of = moga.moga_group_attention_unpermute(p["Qp"], p["Kp"], p["Vp"], p["cu_seqlens"], p["perm"], gate)
    torch.cuda.synchronize()
    assert_output_close(_np(Of), ref["O"], "O (fused attention + unpermute)")
    Og = moga.moga_group_attention_fused(Q, K, V, p["cu_seqlens"], p["perm"], gate)
    torch.cuda.synchronize()
    assert_output_close(_np(Og), ref["O"], "O (gather on load)")
    assert torch.equal(Og, Of)   # same rows, same key order, same arithmetic
    # transposed-V layout: the same gathered rows, V as [H, D, N]
    pv = moga.moga_permute_vt(gid, M, Q, K, V)
    assert torch.equal(pv["perm"], p["perm"]) and torch.equal(pv["cu_seqlens"], p["cu_seqlens"])
    assert torch.equal(pv["Qp"], p["Qp"]) and torch.equal(pv["Kp"], p["Kp"])
    N = X.shape[0]
    assert pv["Vt"].shape[2] == moga.moga_vt_row_length(N)
    assert torch.equal(pv["Vt"][:, :, :N], p["Vp"].permute(1, 2, 0))
    assert not pv["Vt"][:, :, N:].any()          # zero padding
    Ot = moga.moga_group_attention_unpermute_vt(pv["Qp"], pv["Kp"], pv["Vt"], pv["cu_seqlens"], pv["perm"], gate)
    torch.cuda.synchronize()
    assert_output_close(_np(Ot), ref["O"], "O (transposed V)")
    # without the Q copy: the attention reads query rows through perm
    pq = moga.moga_permute_vt(gid, M, None, K, V)
    assert pq["Qp"] is None
    assert torch.equal(pq["Kp"], pv["Kp"]) and torch.equal(pq["Vt"], pv["Vt"])
    Oq = moga.moga_group_attention_unpermute_vtq(Q, pq["Kp"], pq["Vt"], pq["cu_seqlens"], pq["perm"], gate)
    torch.cuda.synchronize()
    assert torch.equal(Oq, Ot)   # same query values, same arithmetic
    print(f"[parity] {label} Op {e_attn} O {e_out}", flush=True)
    return gid, gate, p, Op, O, ref


def test_tiny_workload(moga):
    _full_check(moga, _inputs("tiny"), label="tiny")


@pytest.mark.parametrize("N,H,D,M", [
    (6000, 4, 128, 8),      # several 128-query tiles and 64-key tiles, ragged tails
    (777, 2, 128, 1),       # one group: full attention
    (3001, 1, 64, 64),      # many small groups
    (1, 3, 128, 4),         # a single token
    (5, 2, 64, 3),          # fewer tokens than a tile
    (4097, 3, 128, 16),
    (700, 64, 128, 4),      # H * D = 8192, the widest supported token row
    (16000, 1, 64, 2),      # mean group 8,000 tokens: the default path's 128-query items
    (17000, 1, 128, 2),     # mean group 8,500 tokens: its 256-query items
])
def test_shapes(moga, N, H, D, M):
    _full_check(moga, _inputs("wan13b_21f", N=N, H=H, D=D, M=M, d_model=256), label=f"shape{N}")


def _sweep_shapes(seed, count):
    """Seeded random shapes: token counts from 1 to 9000, 1-4 heads of 64 or
    128, 1-64 groups, small model widths."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        N = int(rng.choice([int(rng.integers(1, 200)), int(rng.integers(200, 9001))]))
        out.append((N, int(rng.integers(1, 5)), int(rng.choice([64, 128])), int(rng.integers(1, 65)),
                    int(rng.choice([64, 128, 256]))))
    return out


@pytest.mark.parametrize("N,H,D,M,d", _sweep_shapes(2024, 10))
def test_shape_sweep(moga, N, H, D, M, d):
    _full_check(moga, _inputs("wan13b_21f", seed=N + M, N=N, H=H, D=D, M=M, d_model=d), label=f"sweep{N, H, D, M}")


_GUARD = 4096  # elements after every output that no call may touch


def _guarded(shape, dtype):
    """An output view at the start of a larger buffer; the buffer is filled
    with NaN (float types) or -7 (integers) so that an unwritten output
    element or a write past the end shows."""
    n = int(np.prod(shape))
    fill = float("nan") if dtype.is_floating_point else -7
    buf = torch.full((n + _GUARD,), fill, dtype=dtype, device=DEV)
    return buf[:n].view(shape), buf


def _guard_intact(buf, n):
    g = buf[n:]
    return bool(torch.isnan(g).all()) if g.dtype.is_floating_point else bool((g == -7).all())


@pytest.mark.parametrize("bias_on", [False, True])
def test_outputs_fully_written_and_guarded(moga, bias_on):
    """Every output element of the default path's calls is written (no NaN
    from the poison fill survives, and beta = 0 reads nothing), nothing is
    written past the end of an output, and with a bias that sends about 90%
    of the tokens to one group (skew stress) the result still matches."""
    N, H, D, M = 3001, 2, 128, 5
    inp = _inputs("wan13b_21f", N=N, H=H, D=D, M=M, d_model=256)
    X, Wr, Q, K, V = (inp[k] for k in ("X", "Wr", "Q", "K", "V"))
    bias = torch.tensor([0.0, 0.0, 3.5, 0.0, 0.0], device=DEV) if bias_on else None
    gid, gbuf = _guarded((N,), torch.int32)
    gate, gtbuf = _guarded((N,), torch.float32)
    moga.moga_route(X, Wr, bias, gid, gate)
    ldv = moga.moga_vt_row_length(N)
    Kp, kbuf = _guarded((N, H, D), torch.bfloat16)
    Vt, vbuf = _guarded((H, D, ldv), torch.bfloat16)
    perm, pbuf = _guarded((N,), torch.int32)
    cu, cbuf = _guarded((M + 1,), torch.int32)
    mx, mbuf = _guarded((1,), torch.int32)
    moga.moga_permute_vt(gid, M, None, K, V, None, Kp, Vt, perm, cu, mx)
    O, obuf = _guarded((N, H, D), torch.bfloat16)
    moga.moga_group_attention_unpermute_vtq(Q, Kp, Vt, cu, perm, gate, 0.0, 0.0, O)
    torch.cuda.synchronize()
    for name, t, buf in (("group_id", gid, gbuf), ("gate", gate, gtbuf), ("Kp", Kp, kbuf), ("Vt", Vt, vbuf),
                         ("perm", perm, pbuf), ("cu_seqlens", cu, cbuf), ("max_seqlen", mx, mbuf), ("O", O, obuf)):
        assert _guard_intact(buf, t.numel()), f"{name}: write past the end"
        if t.dtype.is_floating_point:
            assert not torch.isnan(t).any(), f"{name}: elements left unwritten"
        else:
            assert not (t == -7).any(), f"{name}: elements left unwritten"
    counts = np.bincount(gid.cpu().numpy(), minlength=M)
    if bias_on:
        assert counts.max() >= 0.85 * N, counts
    ref = oracle.moga_forward(*(_np(t) for t in (X, Wr, Q, K, V)), M,
                              bias=None if bias is None else bias.cpu().numpy())
    np.testing.assert_array_equal(gid.cpu().numpy(), ref["group_id"])
    assert_output_close(_np(O), ref["O"], "O (poison-filled outputs)")


def test_skewed_with_bias_and_empty_groups(moga):
    inp = _inputs("clip30s_122f", N=5000, H=2, D=128, M=6, d_model=512)
    # bias pushes most tokens into group 2 and empties group 5
    bias = torch.tensor([0.0, 0.0, 6.0, 0.0, 0.0, -60.0], device=DEV)
    gid, *_ = _full_check(moga, inp, bias=bias, label="skew")
    counts = np.bincount(gid.cpu().numpy(), minlength=6)
    assert counts[5] == 0 and counts[2] > 0.5 * 5000


@pytest.mark.parametrize("N,d_model,M", [
    (1000, 32, 5),      # no 128-channel step: the 32-channel tail only
    (1000, 96, 16),     # tail only, three 32-channel steps
    (1500, 160, 17),    # one step (no pipeline) + tail; 17..32 groups
    (2000, 288, 33),    # two steps (drain only) + tail; 33..48 groups
    (1200, 384, 48),    # three steps: drain with one step left over
    (3000, 640, 64),    # five steps; 49..64 groups
    (4098, 1024, 32),   # eight steps: the steady loop runs; ragged token tail
    (257, 1536, 16),    # one token past the first 256-token block
])
def test_route_loop_paths(moga, N, d_model, M):
    """Router kernel against the oracle over each path of its channel loop
    (tail only, unpipelined, drain, steady loop) and each group-count class."""
    inp = _inputs("clip30s_122f", N=N, H=1, D=64, M=M, d_model=d_model, n_components=M)
    X, Wr = inp["X"], inp["Wr"]
    bias = torch.linspace(-0.5, 0.5, M, device=DEV) if N % 2 else None
    print(f"[parity] route N={N} d_model={d_model} M={M} bias={bias is not None}", flush=True)
    gid, gate = moga.moga_route(X, Wr, bias)
    torch.cuda.synchronize()
    g_ref, gate_ref, _ = oracle.route(_np(X), _np(Wr), None if bias is None else bias.cpu().numpy())
    np.testing.assert_array_equal(gid.cpu().numpy(), g_ref)
    assert_gate_close(gate.cpu().numpy(), gate_ref)


def test_attention_deterministic(moga):
    inp = _inputs("wan13b_21f", N=3000, H=2, D=128, M=4, d_model=256)
    gid, gate = moga.moga_route(inp["X"], inp["Wr"])
    p = moga.moga_permute(gid, 4, inp["Q"], inp["K"], inp["V"])
    a = moga.moga_group_attention(p["Qp"], p["Kp"], p["Vp"], p["cu_seqlens"])
    b = moga.moga_group_attention(p["Qp"], p["Kp"], p["Vp"], p["cu_seqlens"])
    assert torch.equal(a, b)


def test_fused_unpermute_accumulates(moga):
    inp = _inputs("wan13b_21f", N=2600, H=2, D=128, M=5, d_model=256)
    gid, gate = moga.moga_route(inp["X"], inp["Wr"])
    p = moga.moga_permute(gid, 5, inp["Q"], inp["K"], inp["V"])
    prev = inp["V"].clone()
    O = moga.moga_group_attention_unpermute(p["Qp"], p["Kp"], p["Vp"], p["cu_seqlens"], p["perm"], gate,
                                            beta=0.5, O=prev)
    torch.cuda.synchronize()
    ref = oracle.moga_forward(*(_np(inp[k]) for k in ("X", "Wr", "Q", "K", "V")), 5)
    assert_output_close(_np(O), ref["O"] + 0.5 * _np(inp["V"]), "fused O + 0.5 V")


def test_gather_on_load_accumulates(moga):
    inp = _inputs("wan13b_21f", N=2600, H=2, D=128, M=5, d_model=256)
    gid, gate = moga.moga_route(inp["X"], inp["Wr"])
    p = moga.moga_permute(gid, 5)                       # sort only, no gathered copies
    assert p["Qp"] is None
    prev = inp["V"].clone()
    O = moga.moga_group_attention_fused(inp["Q"], inp["K"], inp["V"], p["cu_seqlens"], p["perm"], gate,
                                        beta=0.5, O=prev)
    torch.cuda.synchronize()
    ref = oracle.moga_forward(*(_np(inp[k]) for k in ("X", "Wr", "Q", "K", "V")), 5)
    assert_output_close(_np(O), ref["O"] + 0.5 * _np(inp["V"]), "gather-on-load O + 0.5 V")


@pytest.mark.parametrize("D", [128, 64])
def test_transposed_v_paths_accumulate(moga, D):
    inp = _inputs("wan13b_21f", N=2600, H=2, D=D, M=5, d_model=256)
    gid, gate = moga.moga_route(inp["X"], inp["Wr"])
    pv = moga.moga_permute_vt(gid, 5, inp["Q"], inp["K"], inp["V"])
    pq = moga.moga_permute_vt(gid, 5, None, inp["K"], inp["V"])
    Ot = moga.moga_group_attention_unpermute_vt(pv["Qp"], pv["Kp"], pv["Vt"], pv["cu_seqlens"], pv["perm"], gate,
                                                beta=0.5, O=inp["V"].clone())
    Oq = moga.moga_group_attention_unpermute_vtq(inp["Q"], pq["Kp"], pq["Vt"], pq["cu_seqlens"], pq["perm"], gate,
                                                 beta=0.5, O=inp["V"].clone())
    torch.cuda.synchronize()
    ref = oracle.moga_forward(*(_np(inp[k]) for k in ("X", "Wr", "Q", "K", "V")), 5)
    assert_output_close(_np(Oq), ref["O"] + 0.5 * _np(inp["V"]), "transposed-V, queries through perm: O + 0.5 V")
    assert torch.equal(Oq, Ot)


def test_unpermute_accumulate(moga):
    inp = _inputs("wan13b_21f", N=2500, H=2, D=64, M=5, d_model=128)
    gid, gate = moga.moga_route(inp["X"], inp["Wr"])
    p = moga.moga_permute(gid, 5, inp["Q"], inp["K"], inp["V"])
    prev = inp["V"].clone()
    O = moga.moga_unpermute(p["Qp"], p["perm"], gate, beta=0.5, O=prev)
    torch.cuda.synchronize()
    perm, g = p["perm"].cpu().numpy(), gate.cpu().numpy()
    ref = oracle.unpermute(_np(p["Qp"]), perm, g, 0.5, _np(inp["V"]))
    # float32 evaluation (rounding relative to each product) then one bf16 rounding
    terms = np.abs(oracle.unpermute(_np(p["Qp"]), perm, g)) + 0.5 * np.abs(_np(inp["V"]))
    err = np.abs(_np(O) - ref)
    assert (err <= 2.0 ** -8 * np.abs(ref) + 2.0 ** -22 * terms).all(), err.max()


@pytest.mark.parametrize("T,Hs,Ws,win_t,th,tw,H,D,alpha,beta", [
    (6, 6, 10, 3, 3, 5, 2, 128, 1.0, 0.0),     # groups of 45: one partial tile
    (4, 30, 52, 2, 30, 26, 1, 128, 0.5, 0.5),  # Wan-like frames, groups of 1560
    (3, 8, 8, 1, 8, 8, 2, 64, 1.0, 1.0),
    (6, 30, 52, 6, 30, 52, 1, 64, 1.0, 0.0),     # 9,360-key window: past the key-row table
    (5, 24, 32, 5, 24, 32, 2, 128, 1.0, 0.0),    # 3,840 keys: a full key-row table, 30 whole 128-query items
    (5, 30, 26, 5, 30, 26, 1, 64, 1.0, 1.0),     # 3,900 keys: just past the table
    (3, 30, 52, 3, 30, 26, 2, 128, 1.0, 1.0),    # the long-video windows (2,340 keys, a 36-query last item), accumulating
])
def test_stga(moga, T, Hs, Ws, win_t, th, tw, H, D, alpha, beta):
    N = T * Hs * Ws
    print(f"[parity] stga N={N} geo={T, Hs, Ws, win_t, th, tw} H={H} D={D}", flush=True)
    inp = _inputs("tiny", N=N, H=H, D=D, M=2)
    Q, K, V = inp["Q"], inp["K"], inp["V"]
    O = V.clone() if beta != 0 else None
    out = moga.moga_stga_attention(Q, K, V, T, Hs, Ws, win_t, th, tw, alpha=alpha, beta=beta, O=O)
    torch.cuda.synchronize()
    ref = oracle.stga_attention(_np(Q), _np(K), _np(V), T, Hs, Ws, win_t, th, tw, 1 / math.sqrt(D),
                                alpha=alpha, beta=beta, O_prev=_np(V))
    assert_output_close(_np(out), ref, "STGA")


def test_stga_deterministic(moga):
    """Every output row of an STGA window is written by one work item, so two
    calls on the same inputs agree bit for bit."""
    T, Hs, Ws = 3, 30, 52
    inp = _inputs("tiny", N=T * Hs * Ws, H=2, D=128, M=2)
    Q, K, V = inp["Q"], inp["K"], inp["V"]
    a = moga.moga_stga_attention(Q, K, V, T, Hs, Ws, 3, 30, 26)
    b = moga.moga_stga_attention(Q, K, V, T, Hs, Ws, 3, 30, 26)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("T,Hs,Ws,shots,win_t,th,tw,aug,H,D,alpha,beta", [
    (7, 6, 10, [0, 3, 4, 7], 2, 3, 5, 1, 2, 128, 1.0, 0.0),     # a one-frame shot, ragged windows
    (9, 30, 52, [0, 5, 9], 3, 30, 26, 1, 1, 128, 0.5, 0.5),     # Wan-like frames, 780-token tiles
    (8, 8, 8, [0, 2, 3, 8], 3, 4, 8, 0, 2, 64, 1.0, 1.0),       # no augmentation
    (6, 4, 4, [0, 6], 2, 4, 4, 1, 1, 64, 1.0, 0.0),             # one shot: plain windows
    (5, 4, 8, [0, 1, 2, 3, 4, 5], 4, 2, 4, 1, 2, 128, 1.0, 0.0),  # every frame its own shot
    (12, 6, 10, [0, 1, 5, 6, 12], 3, 6, 5, 2, 2, 128, 1.0, 0.0),  # two frames per side, clipped
    (10, 30, 52, [0, 4, 10], 3, 30, 26, 3, 1, 128, 1.0, 0.0),   # three per side, Wan-like tile
    (12, 30, 52, [0, 5, 12], 5, 30, 52, 1, 1, 64, 1.0, 0.0),    # 10,920-key windows: past the table
])
def test_stga_shot(moga, T, Hs, Ws, shots, win_t, th, tw, aug, H, D, alpha, beta):
    N = T * Hs * Ws
    print(f"[parity] stga-shot N={N} shots={shots} geo={win_t, th, tw} aug={aug} H={H} D={D}", flush=True)
    inp = _inputs("tiny", N=N, H=H, D=D, M=2)
    Q, K, V = inp["Q"], inp["K"], inp["V"]
    O = V.clone() if beta != 0 else None
    ss = torch.tensor(shots, dtype=torch.int32, device=DEV)
    out = moga.moga_stga_shot_attention(Q, K, V, T, Hs, Ws, ss, win_t, th, tw, augment=aug, alpha=alpha,
                                        beta=beta, O=O)
    torch.cuda.synchronize()
    ref = oracle.stga_shot_attention(_np(Q), _np(K), _np(V), T, Hs, Ws, shots, win_t, th, tw, 1 / math.sqrt(D),
                                     aug)
    ref = alpha * ref + beta * _np(V)
    assert_output_close(_np(out), ref, "shot STGA")


# ---------------------------------------------------------------------------
# Full workload sizes, in the launch configuration the benchmark times
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,path,seed", [("wan13b_21f", "fused_vt", None), ("clip30s_122f", "fused_vt", None),
                                            ("clip30s_122f", "fused_vtq", None), ("wan13b_21f", "fused_vtq", None),
                                            ("clip30s_122f", "fused_vtq", 4242),    # another draw of the recipe
                                            ("clip30s_122f", "fused_epilogue", None),
                                            ("clip30s_122f", "gather_on_load", None), ("clip30s_122f", "separate", None),
                                            ("wan14b_122f", "fused_vt", None), ("wan14b_122f", "fused_vtq", None),
                                            ("minute_372f", "fused_vtq", None), ("minute_372f", "fused_vt", None),
                                            ("minute_372f", "fused_epilogue", None),
                                            ("minute_372f", "gather_on_load", None)])
def test_full_size_sampled(moga, name, path, seed):
    wl = get_workload(name)
    if seed is not None:
        wl = dataclasses.replace(wl, seed=seed)
    print(f"[parity] full {name} path={path} seed={wl.seed} N={wl.N} d={wl.d_model} H={wl.H} M={wl.M}", flush=True)
    inp = make_inputs(wl, device=DEV)
    X, Wr, Q, K, V = (inp[k] for k in ("X", "Wr", "Q", "K", "V"))
    fwd = moga.MogaForward(wl.N, wl.d_model, wl.H, wl.D, wl.M, DEV, stga=wl.stga, path=path)
    O = fwd(X, Wr, Q, K, V)
    torch.cuda.synchronize()

    Xn, Wn = _np(X), _np(Wr)
    g_ref, gate_ref, _ = oracle.route(Xn, Wn)
    np.testing.assert_array_equal(fwd.group_id.cpu().numpy(), g_ref)
    assert_gate_close(fwd.gate.cpu().numpy(), gate_ref)
    perm_ref, cu_ref, mx_ref = oracle.permute(g_ref, wl.M)
    np.testing.assert_array_equal(fwd.perm.cpu().numpy(), perm_ref)
    np.testing.assert_array_equal(fwd.cu_seqlens.cpu().numpy(), cu_ref)
    assert int(fwd.max_seqlen.item()) == mx_ref

    # the headline configuration gets a denser sample (about 1,000 rows)
    rows = sample_rows(g_ref, wl.M, per_group=64 if name == "clip30s_122f" else 6, seed=wl.seed)
    # plus the queries on both sides of the first 32-query wave and 256-query
    # work-item boundaries of every group (permuted positions 31/32, 255/256)
    edges = [perm_ref[cu_ref[i] + j] for i in range(wl.M) for j in (31, 32, 255, 256)
             if cu_ref[i] + j < cu_ref[i + 1]]
    if wl.stga is not None:
        s = wl.stga
        ids = oracle.stga_group_ids(s["T"], s["Hs"], s["Ws"], s["win_t"], s["tile_h"], s["tile_w"])
        # the STGA windows are cut into 128-query work items: in the first and
        # last window, the queries on both sides of the first item boundary
        # and of the last (partial) item, in the window's own token order
        for win in (0, int(ids.max())):
            members = np.nonzero(ids == win)[0]
            b = members.size // 128 * 128
            edges += [int(members[j]) for j in sorted({0, 127, 128, b - 1, b, members.size - 1})
                      if 0 <= j < members.size]
    rows = np.unique(np.concatenate([rows, np.asarray(edges, dtype=np.int64)]))
    Qn, Kn, Vn = _np(Q), _np(K), _np(V)
    want = oracle.moga_output_rows(Xn, Wn, Qn, Kn, Vn, wl.M, rows, routed=(g_ref, gate_ref))
    if wl.stga is not None:
        want = want + oracle.stga_attention_rows(Qn, Kn, Vn, ids, 1 / math.sqrt(wl.D), rows)
    got = _np(O[torch.from_numpy(rows).to(DEV)])
    e = assert_output_close(got, want, f"{name} sampled O")
    print(f"[parity] full {name}: {rows.size} rows, {e}", flush=True)


def test_full_size_visual_block(moga):
    """Minute-scale clip with a seeded multi-shot layout: the visual output
    (MoGA + shot-aware STGA + per-frame attention) / 3 on sampled tokens,
    including every shot's first and last frame."""
    wl = get_workload("minute_372f")
    s = dict(wl.stga)
    shots = make_shots(s["T"], wl.seed)
    s["shot_start"] = shots
    print(f"[parity] visual block minute_372f shots={shots}", flush=True)
    inp = make_inputs(wl, device=DEV)
    X, Wr, Q, K, V = (inp[k] for k in ("X", "Wr", "Q", "K", "V"))
    fwd = moga.MogaForward(wl.N, wl.d_model, wl.H, wl.D, wl.M, DEV, stga=s)
    O = fwd(X, Wr, Q, K, V)
    torch.cuda.synchronize()
    Xn, Wn, Qn, Kn, Vn = _np(X), _np(Wr), _np(Q), _np(K), _np(V)
    g_ref, gate_ref, _ = oracle.route(Xn, Wn)
    np.testing.assert_array_equal(fwd.group_id.cpu().numpy(), g_ref)
    rows = sample_rows(g_ref, wl.M, per_group=2, seed=wl.seed)
    area = s["Hs"] * s["Ws"]
    edge = [f * area + o for t in shots[1:-1] for f in (t - 1, t) for o in (0, area - 1)]
    rows = np.unique(np.concatenate([rows, np.asarray(edge, dtype=np.int64)]))
    scale = 1 / math.sqrt(wl.D)
    want = oracle.moga_output_rows(Xn, Wn, Qn, Kn, Vn, wl.M, rows, routed=(g_ref, gate_ref))
    want = want + oracle.stga_shot_attention_rows(Qn, Kn, Vn, s["T"], s["Hs"], s["Ws"], shots, s["win_t"],
                                                  s["tile_h"], s["tile_w"], scale, rows)
    frame_ids = oracle.stga_group_ids(s["T"], s["Hs"], s["Ws"], 1, s["Hs"], s["Ws"])
    want = (want + oracle.stga_attention_rows(Qn, Kn, Vn, frame_ids, scale, rows)) / 3.0
    got = _np(O[torch.from_numpy(rows).to(DEV)])
    e = assert_output_close(got, want, "minute_372f visual block sampled O")
    print(f"[parity] visual block: {rows.size} rows, {e}", flush=True)


@pytest.mark.parametrize("late,label", [(4.0, "float32-overflow"), (2.0, "overflow-fallback"),
                                        (0.9, "fixed-offset")])
def test_attention_score_growth(moga, late, label):
    """Scores that grow far beyond a row's first keys (which fix the exponent
    offset): with late = 2, q.k jumps from 0 to ~512, about 65 in log2 units
    after scaling, so the denominator passes 2^64 and the exact recomputation
    must engage; with late = 4 (~130 log2 units) the weights themselves would
    overflow float32 without it; with late = 0.9 (~29 log2 units) the main
    path keeps the large weights and must still be exact."""
    print(f"[parity] score growth {label}", flush=True)
    N, H, D = 700, 2, 128
    g = torch.Generator().manual_seed(7)
    Q = torch.full((N, H, D), 2.0).bfloat16()
    K = torch.zeros((N, H, D))
    K[200:] = late + 0.25 * torch.randn((N - 200, H, D), generator=g)
    K = K.bfloat16()
    V = torch.randn((N, H, D), generator=g).bfloat16()
    cu = torch.tensor([0, 100, N], dtype=torch.int32)    # second group starts with zero keys
    Op = moga.moga_group_attention(Q.to(DEV), K.to(DEV), V.to(DEV), cu.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.group_attention(_np(Q), _np(K), _np(V), cu.numpy(), 1 / math.sqrt(D))
    assert_output_close(_np(Op), ref, f"Op ({label})")
    # the same through the transposed-V paths (their own fallback instantiations):
    # groups [0, 100) and [100, N) sort to the identity permutation, gate 1
    gid = torch.cat([torch.zeros(100, dtype=torch.int32), torch.ones(N - 100, dtype=torch.int32)]).to(DEV)
    gate = torch.ones(N, dtype=torch.float32, device=DEV)
    Qd, Kd, Vd = Q.to(DEV), K.to(DEV), V.to(DEV)
    pv = moga.moga_permute_vt(gid, 2, Qd, Kd, Vd)
    assert torch.equal(pv["perm"].cpu(), torch.arange(N, dtype=torch.int32))
    Ot = moga.moga_group_attention_unpermute_vt(pv["Qp"], pv["Kp"], pv["Vt"], pv["cu_seqlens"], pv["perm"], gate)
    Oq = moga.moga_group_attention_unpermute_vtq(Qd, pv["Kp"], pv["Vt"], pv["cu_seqlens"], pv["perm"], gate)
    # and the gather-on-load instantiation (keys fetched through perm), whose
    # recomputation re-fetches the first tiles' key rows
    Of = moga.moga_group_attention_fused(Qd, Kd, Vd, pv["cu_seqlens"], pv["perm"], gate)
    torch.cuda.synchronize()
    assert_output_close(_np(Ot), ref, f"O transposed V ({label})")
    assert torch.equal(Oq, Ot)
    assert_output_close(_np(Of), ref, f"O gather on load ({label})")


@pytest.mark.parametrize("path", ["group_attention", "vtq", "fused"])
def test_attention_large_values(moga, path):
    """Large but finite values with late score growth: |V| ~ 2^100 and scores
    that climb to ~49 log2 units past the first keys, so the float32 sum of
    weight x value overflows while the denominator (~2^58) stays below 2^64.
    The result must still be the softmax average (exact up to rounding), which
    is the plain-size result scaled by 2^100 (powers of two scale exactly)."""
    print(f"[parity] large values {path}", flush=True)
    N, H, D = 700, 2, 128
    g = torch.Generator().manual_seed(11)
    Q = torch.full((N, H, D), 2.0).bfloat16()
    K = torch.zeros((N, H, D))
    K[200:] = 1.5 + 0.25 * torch.randn((N - 200, H, D), generator=g)
    K = K.bfloat16()
    V = torch.randn((N, H, D), generator=g).bfloat16()
    big = 2.0 ** 100
    Vb = (V.float() * big).bfloat16()
    assert torch.equal(Vb.float() / big, V.float())
    cu = torch.tensor([0, 100, N], dtype=torch.int32)
    ref = oracle.group_attention(_np(Q), _np(K), _np(V), cu.numpy(), 1 / math.sqrt(D))
    Qd, Kd, Vd = Q.to(DEV), K.to(DEV), Vb.to(DEV)
    if path == "group_attention":
        out = moga.moga_group_attention(Qd, Kd, Vd, cu.to(DEV))
    else:
        gid = torch.cat([torch.zeros(100, dtype=torch.int32), torch.ones(N - 100, dtype=torch.int32)]).to(DEV)
        gate = torch.ones(N, dtype=torch.float32, device=DEV)
        pv = moga.moga_permute_vt(gid, 2, None, Kd, Vd)
        if path == "vtq":
            out = moga.moga_group_attention_unpermute_vtq(Qd, pv["Kp"], pv["Vt"], pv["cu_seqlens"], pv["perm"], gate)
        else:
            out = moga.moga_group_attention_fused(Qd, Kd, Vd, pv["cu_seqlens"], pv["perm"], gate)
    torch.cuda.synchronize()
    got = _np(out)
    assert np.isfinite(got).all(), "large-value output is not finite"
    assert_output_close(got / big, ref, f"large values ({path})")


@pytest.mark.parametrize("late", [0.9, 2.0, 4.0])
def test_stga_score_growth(moga, late):
    """Static and shot-aware windows whose later frames' keys score far above
    the first frame's (the exponent offset comes from a window's first 32
    keys): the index-map instantiations must engage their exact recomputation
    where needed and match the oracle."""
    T, Hs, Ws, win_t, th, tw, H, D = 6, 6, 10, 3, 6, 10, 2, 128
    N = T * Hs * Ws
    print(f"[parity] stga score growth late={late}", flush=True)
    g = torch.Generator().manual_seed(13)
    Q = torch.full((N, H, D), 2.0).bfloat16()
    K = torch.zeros((N, H, D))
    frame = torch.arange(N) // (Hs * Ws)
    lateK = (frame % win_t) > 0                     # every window's frames after its first
    K[lateK] = late + 0.25 * torch.randn((int(lateK.sum()), H, D), generator=g)
    K = K.bfloat16()
    V = torch.randn((N, H, D), generator=g).bfloat16()
    Qd, Kd, Vd = Q.to(DEV), K.to(DEV), V.to(DEV)
    out = moga.moga_stga_attention(Qd, Kd, Vd, T, Hs, Ws, win_t, th, tw)
    shots = [0, 3, 6]
    outs = moga.moga_stga_shot_attention(Qd, Kd, Vd, T, Hs, Ws, torch.tensor(shots, dtype=torch.int32, device=DEV),
                                         win_t, th, tw, augment=1)
    torch.cuda.synchronize()
    sc = 1 / math.sqrt(D)
    ref = oracle.stga_attention(_np(Q), _np(K), _np(V), T, Hs, Ws, win_t, th, tw, sc)
    refs = oracle.stga_shot_attention(_np(Q), _np(K), _np(V), T, Hs, Ws, shots, win_t, th, tw, sc, 1)
    assert_output_close(_np(out), ref, f"STGA growth {late}")
    assert_output_close(_np(outs), refs, f"shot STGA growth {late}")


@pytest.mark.parametrize("name,M", [("tiny", 4), ("clip30s_122f", 16), ("minute_372f", 32)])
def test_balance_stats(moga, name, M):
    """F_i, P_i and L_gb (Eq. 6) from the GPU route output, against the oracle's
    float64 statistics of the same group ids and gates; bitwise repeatable."""
    wl = get_workload(name)
    print(f"[parity] balance {name}", flush=True)
    inp = make_inputs(wl, device=DEV)
    gid, gate = moga.moga_route(inp["X"], inp["Wr"])
    F, P, loss = moga.moga_balance_stats(gid, gate, wl.M, alpha=0.1)
    F2, P2, loss2 = moga.moga_balance_stats(gid, gate, wl.M, alpha=0.1)
    torch.cuda.synchronize()
    Fr, Pr, Lr = oracle.balance_stats(gid.cpu().numpy(), gate.cpu().numpy(), wl.M, 0.1)
    np.testing.assert_allclose(F.cpu().numpy(), Fr, rtol=1e-6)
    np.testing.assert_allclose(P.cpu().numpy(), Pr, rtol=1e-5, atol=1e-9)
    assert abs(loss.item() - Lr) <= 1e-5 * Lr
    assert torch.equal(P, P2) and torch.equal(loss, loss2)


def test_graph_capture_replays(moga):
    """The whole layer pass (route, permute, attention with the gated
    unpermute, shot-aware STGA and the per-frame branch) captured once in a
    HIP graph: every replay, with eager work and synchronisations between
    them, must equal the eager result bit for bit.  No launch in the pass
    records a memset, and all scratch is preallocated by MogaForward."""
    T, Hs, Ws = 6, 6, 10
    N = T * Hs * Ws
    inp = _inputs("wan13b_21f", N=N, H=2, D=128, M=5, d_model=128)
    X, Wr, Q, K, V = (inp[k] for k in ("X", "Wr", "Q", "K", "V"))
    geo = dict(T=T, Hs=Hs, Ws=Ws, win_t=2, tile_h=3, tile_w=5, shot_start=[0, 2, 3, 6])
    fwd = moga.MogaForward(N, 128, 2, 128, 5, DEV, stga=geo)
    eager = fwd(X, Wr, Q, K, V).clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fwd(X, Wr, Q, K, V)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = fwd(X, Wr, Q, K, V)
    for rep in range(3):
        fwd.O.zero_()
        junk = (Q.float() * 2).sum()  # unrelated eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs"
        assert torch.isfinite(junk)
