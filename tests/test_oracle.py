"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Nothing here compares the oracle with itself: every check is a closed form, an
invariant, a hand-worked case, a brute-force loop on a tiny input, or a special
case that reduces to a library routine (torch's scaled_dot_product_attention
in float64 on the CPU).  The mutation tests at the end plant plausible mistakes
in the oracle and check that some pin catches each of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import moga_oracle as om

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _sdpa(Q, K, V, mask=None, scale=None):
    """Library attention in float64 on [N, H, D] arrays; mask[i, j] True = attend."""
    q = torch.from_numpy(np.ascontiguousarray(np.transpose(Q, (1, 0, 2)), dtype=np.float64))
    k = torch.from_numpy(np.ascontiguousarray(np.transpose(K, (1, 0, 2)), dtype=np.float64))
    v = torch.from_numpy(np.ascontiguousarray(np.transpose(V, (1, 0, 2)), dtype=np.float64))
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=scale)
    return np.transpose(o.numpy(), (1, 0, 2))


def _random_case(seed, N=96, d=24, M=4, H=2, D=16, bias=False):
    r = _rng(seed)
    X = r.standard_normal((N, d))
    Wr = r.standard_normal((M, d)) / math.sqrt(d)
    Q, K, V = (r.standard_normal((N, H, D)) for _ in range(3))
    b = r.standard_normal(M) if bias else None
    return X, Wr, Q, K, V, b


# ---------------------------------------------------------------------------
# Router pins
# ---------------------------------------------------------------------------

def check_route_closed_form():
    # d_model = M = 4 and W_r = 2 * (permutation matrix of a 3-cycle), so
    # r[n, i] = 2 * X[n, pi(i)] exactly; a transposed W_r would give pi^-1.
    pi = [1, 2, 0, 3]
    Wr = np.zeros((4, 4))
    for i, j in enumerate(pi):
        Wr[i, j] = 2.0
    X = np.array([[0.0, 1.5, 0.0, 0.0],     # r = (3, 0, 0, 0)    -> g = 0
                  [0.0, 0.0, 0.0, -1.0],    # r = (0, 0, 0, -2)   -> tie of 0,1,2 -> g = 0
                  [0.25, 0.0, 0.0, 0.5],    # r = (0, 0, 0.5, 1)  -> g = 3
                  [1.0, 0.0, 2.0, 0.0]])    # r = (0, 4, 2, 0)    -> g = 1
    r_expect = np.array([[3, 0, 0, 0], [0, 0, 0, -2], [0, 0, 0.5, 1], [0, 4, 2, 0]], dtype=float)
    g_expect = [0, 0, 3, 1]
    gate_expect = [math.exp(3) / (math.exp(3) + 3),
                   1.0 / (3 + math.exp(-2)),
                   math.exp(1) / (2 + math.exp(0.5) + math.exp(1)),
                   math.exp(4) / (2 + math.exp(2) + math.exp(4))]
    g, gate, r = oracle.route(X, Wr)
    np.testing.assert_array_equal(r, r_expect)
    np.testing.assert_array_equal(g, g_expect)
    np.testing.assert_allclose(gate, gate_expect, rtol=1e-6)


def test_route_closed_form():
    check_route_closed_form()


def test_route_single_group_gate_is_one():
    X, Wr, *_ = _random_case(1, M=1)
    g, gate, _ = oracle.route(X, Wr)
    assert (g == 0).all() and (gate == 1.0).all()


def test_route_softmax_shift_invariance():
    # adding the same constant to every score changes neither p nor argmax
    X, Wr, *_ = _random_case(2, M=7)
    g0, gate0, _ = oracle.route(X, Wr)
    g1, gate1, _ = oracle.route(X, Wr, bias=np.full(7, 0.375))
    np.testing.assert_array_equal(g0, g1)
    np.testing.assert_allclose(gate1, gate0, rtol=1e-6)


def test_route_bias_forces_group():
    X, Wr, *_ = _random_case(3, M=5)
    b = np.zeros(5)
    b[3] = 1e3
    g, gate, _ = oracle.route(X, Wr, bias=b)
    assert (g == 3).all()
    np.testing.assert_allclose(gate, 1.0, rtol=1e-7)


def check_route_bruteforce():
    X, Wr, *_ = _random_case(4, N=16, d=8, M=5)
    g, gate, _ = oracle.route(X, Wr)
    for n in range(16):
        r = [math.fsum(X[n, k] * Wr[i, k] for k in range(8)) for i in range(5)]
        best = max(range(5), key=lambda i: (r[i], -i))
        assert g[n] == best
        p = math.exp(r[best]) / math.fsum(math.exp(x) for x in r)
        assert abs(gate[n] - p) <= 1e-6 * p
        assert 1.0 / 5 - 1e-7 <= gate[n] <= 1.0 + 1e-7   # the top softmax probability


def test_route_bruteforce():
    check_route_bruteforce()


# ---------------------------------------------------------------------------
# Permutation pins (Algorithm 1 step 2)
# ---------------------------------------------------------------------------

def check_permute_hand_example():
    # groups: token 0->2, 1->0, 2->1, 3->0, 4->2, 5->2, 6->1; group 3 is empty
    g = np.array([2, 0, 1, 0, 2, 2, 1])
    perm, cu, mx = oracle.permute(g, 4)
    np.testing.assert_array_equal(perm, [1, 3, 2, 6, 0, 4, 5])
    np.testing.assert_array_equal(cu, [0, 2, 4, 7, 7])
    assert mx == 3


def test_permute_hand_example():
    check_permute_hand_example()


def check_permute_bruteforce(seed=5):
    r = _rng(seed)
    for M in (1, 3, 8, 64):
        g = r.integers(0, M, size=int(r.integers(1, 300)))
        if M > 2:
            g[g == 1] = 0                     # force an empty group
        perm, cu, mx = oracle.permute(g, M)
        want = [n for i in range(M) for n in range(g.size) if g[n] == i]
        np.testing.assert_array_equal(perm, want)
        counts = [int((g == i).sum()) for i in range(M)]
        np.testing.assert_array_equal(np.diff(cu), counts)
        assert cu[0] == 0 and cu[-1] == g.size and mx == max(counts)
        assert sorted(perm.tolist()) == list(range(g.size))   # bijection


def test_permute_bruteforce():
    check_permute_bruteforce()


# ---------------------------------------------------------------------------
# Attention pins (Eq. 1 inside groups; MoGA output equation)
# ---------------------------------------------------------------------------

def check_single_group_is_full_attention():
    X, Wr, Q, K, V, _ = _random_case(6, M=1)
    out = oracle.moga_forward(X, Wr, Q, K, V, M=1)
    np.testing.assert_allclose(out["O"], _sdpa(Q, K, V), atol=1e-12)


def test_single_group_is_full_attention():
    check_single_group_is_full_attention()


def check_moga_is_gated_masked_attention(seed=7, bias=False):
    X, Wr, Q, K, V, b = _random_case(seed, N=120, M=5, bias=bias)
    out = oracle.moga_forward(X, Wr, Q, K, V, M=5, bias=b)
    g = out["group_id"]
    mask = g[:, None] == g[None, :]
    ref = out["gate"].astype(np.float64)[:, None, None] * _sdpa(Q, K, V, mask)
    np.testing.assert_allclose(out["O"], ref, atol=1e-6)   # gate is float32


def test_moga_is_gated_masked_attention():
    check_moga_is_gated_masked_attention()
    check_moga_is_gated_masked_attention(seed=8, bias=True)


def test_closed_form_zero_query_is_group_mean():
    X, Wr, Q, K, V, _ = _random_case(9, M=3)
    out = oracle.moga_forward(X, Wr, np.zeros_like(Q), K, V, M=3)
    g, gate = out["group_id"], out["gate"].astype(np.float64)
    for n in range(X.shape[0]):
        mean = V[g == g[n]].mean(axis=0)
        np.testing.assert_allclose(out["O"][n], gate[n] * mean, atol=1e-12)


def test_closed_form_constant_value():
    X, Wr, Q, K, _, _ = _random_case(10, M=4)
    c = np.array([[0.5] * 16, [-1.25] * 16])
    V = np.broadcast_to(c, Q.shape).copy()
    out = oracle.moga_forward(X, Wr, Q, K, V, M=4)
    np.testing.assert_allclose(out["O"], out["gate"].astype(np.float64)[:, None, None] * c[None], atol=1e-12)


def test_closed_form_singleton_and_pair_groups():
    # bias routes token 0 alone to group 0, tokens 1 and 2 to group 1, the rest to group 2
    r = _rng(11)
    N, d, H, D = 10, 6, 2, 8
    X = np.zeros((N, d))
    X[0, 0] = 1.0
    X[1:3, 1] = 1.0
    X[3:, 2] = 1.0
    Wr = np.eye(3, d) * 5.0
    Q, K, V = (r.standard_normal((N, H, D)) for _ in range(3))
    out = oracle.moga_forward(X, Wr, Q, K, V, M=3)
    gate = out["gate"].astype(np.float64)
    np.testing.assert_allclose(out["O"][0], gate[0] * V[0], atol=1e-12)
    s = 1 / math.sqrt(D)
    for n, m in ((1, 2), (2, 1)):
        for h in range(H):
            a = 1.0 / (1.0 + math.exp(-(Q[n, h] @ K[n, h] - Q[n, h] @ K[m, h]) * s))  # weight on itself
            np.testing.assert_allclose(out["O"][n, h], gate[n] * (a * V[n, h] + (1 - a) * V[m, h]), atol=1e-12)


def check_bruteforce_loops(seed=12):
    X, Wr, Q, K, V, _ = _random_case(seed, N=14, d=6, M=3, H=2, D=4)
    out = oracle.moga_forward(X, Wr, Q, K, V, M=3)
    g, gate = out["group_id"], out["gate"]
    for n in range(14):
        for h in range(2):
            members = [m for m in range(14) if g[m] == g[n]]
            s = [math.fsum(Q[n, h, c] * K[m, h, c] for c in range(4)) / 2.0 for m in members]
            top = max(s)
            w = [math.exp(x - top) for x in s]
            z = math.fsum(w)
            for c in range(4):
                o = math.fsum(wi * V[m, h, c] for wi, m in zip(w, members)) / z
                assert abs(out["O"][n, h, c] - float(gate[n]) * o) < 1e-12


def test_bruteforce_loops():
    check_bruteforce_loops()


def test_permutation_equivariance():
    X, Wr, Q, K, V, _ = _random_case(13, N=80, M=4)
    sigma = _rng(14).permutation(80)
    a = oracle.moga_forward(X, Wr, Q, K, V, M=4)
    b = oracle.moga_forward(X[sigma], Wr, Q[sigma], K[sigma], V[sigma], M=4)
    np.testing.assert_array_equal(b["group_id"], a["group_id"][sigma])
    np.testing.assert_array_equal(b["gate"], a["gate"][sigma])
    np.testing.assert_array_equal(b["cu_seqlens"], a["cu_seqlens"])
    np.testing.assert_allclose(b["O"], a["O"][sigma], atol=1e-12)


def test_unpermute_inverts_permute():
    r = _rng(15)
    g = r.integers(0, 6, size=50)
    T = r.standard_normal((50, 3, 4))
    perm, _, _ = oracle.permute(g, 6)
    back = oracle.unpermute(oracle.gather_rows(T, perm), perm, np.ones(50, np.float32))
    np.testing.assert_array_equal(back, T)
    prev = r.standard_normal((50, 3, 4))
    gate = r.uniform(0.2, 1.0, 50).astype(np.float32)
    acc = oracle.unpermute(oracle.gather_rows(T, perm), perm, gate, beta=1.0, O_prev=prev)
    np.testing.assert_allclose(acc, prev + gate.astype(np.float64)[:, None, None] * T, atol=1e-15)


def test_rows_helpers_agree_with_full_pass():
    X, Wr, Q, K, V, _ = _random_case(16, N=100, M=4)
    out = oracle.moga_forward(X, Wr, Q, K, V, M=4)
    rows = np.array([0, 7, 50, 99])
    np.testing.assert_allclose(oracle.moga_output_rows(X, Wr, Q, K, V, 4, rows), out["O"][rows], atol=1e-13)
    Qp, Kp, Vp = (oracle.gather_rows(T, out["perm"]) for T in (Q, K, V))
    np.testing.assert_allclose(oracle.group_attention_rows(Qp, Kp, Vp, out["cu_seqlens"], 0.25, rows),
                               out["Op"][rows], atol=1e-13)


# ---------------------------------------------------------------------------
# STGA pins
# ---------------------------------------------------------------------------

def test_stga_ids_hand_example():
    # T=2 frames of 2 x 4 tokens, one-frame windows, 1 x 2 spatial tiles
    ids = oracle.stga_group_ids(2, 2, 4, 1, 1, 2)
    np.testing.assert_array_equal(ids, [0, 0, 1, 1, 2, 2, 3, 3, 4, 4, 5, 5, 6, 6, 7, 7])
    # T=4, Hs=2, Ws=2, two-frame windows, whole-frame tile: two groups of 8
    np.testing.assert_array_equal(oracle.stga_group_ids(4, 2, 2, 2, 2, 2), [0] * 8 + [1] * 8)
    # 2 x 2 spatial tiles on a 4 x 4 frame
    np.testing.assert_array_equal(oracle.stga_group_ids(1, 4, 4, 1, 2, 2),
                                  [0, 0, 1, 1, 0, 0, 1, 1, 2, 2, 3, 3, 2, 2, 3, 3])


def check_stga_is_window_masked_attention():
    r = _rng(17)
    T, Hs, Ws, H, D = 6, 4, 6, 2, 8
    N = T * Hs * Ws
    Q, K, V = (r.standard_normal((N, H, D)) for _ in range(3))
    out = oracle.stga_attention(Q, K, V, T, Hs, Ws, 3, 2, 3, 1 / math.sqrt(D))
    ids = oracle.stga_group_ids(T, Hs, Ws, 3, 2, 3)
    np.testing.assert_allclose(out, _sdpa(Q, K, V, ids[:, None] == ids[None, :]), atol=1e-12)
    full = oracle.stga_attention(Q, K, V, T, Hs, Ws, T, Hs, Ws, 1 / math.sqrt(D))
    np.testing.assert_allclose(full, _sdpa(Q, K, V), atol=1e-12)
    single = oracle.stga_attention(Q, K, V, T, Hs, Ws, 1, 1, 1, 1 / math.sqrt(D))
    np.testing.assert_allclose(single, V, atol=1e-15)


def test_stga_is_window_masked_attention():
    check_stga_is_window_masked_attention()


def test_moga_plus_stga_is_sum_of_branches():
    r = _rng(18)
    T, Hs, Ws, H, D, d, M = 3, 2, 4, 2, 8, 10, 3
    N = T * Hs * Ws
    X = r.standard_normal((N, d))
    Wr = r.standard_normal((M, d))
    Q, K, V = (r.standard_normal((N, H, D)) for _ in range(3))
    geo = dict(T=T, Hs=Hs, Ws=Ws, win_t=1, tile_h=2, tile_w=2)
    out = oracle.moga_forward(X, Wr, Q, K, V, M, stga=dict(geo, alpha=0.5, beta=0.5))
    g = out["group_id"]
    ids = oracle.stga_group_ids(T, Hs, Ws, 1, 2, 2)
    moga = out["gate"].astype(np.float64)[:, None, None] * _sdpa(Q, K, V, g[:, None] == g[None, :])
    stga = _sdpa(Q, K, V, ids[:, None] == ids[None, :])
    np.testing.assert_allclose(out["O"], 0.5 * moga + 0.5 * stga, atol=1e-6)


def test_shot_windows_hand_example():
    # 10 frames, shots [0,4) [4,5) [5,10), windows of 3 frames
    w = oracle.shot_windows([0, 4, 5, 10], 3)
    assert w == [(0, 3, [], []), (3, 1, [], [4]), (4, 1, [3], [5]), (5, 3, [4], []), (8, 2, [], [])]
    assert oracle.shot_windows([0, 4, 5, 10], 3, aug=False) == [(0, 3, [], []), (3, 1, [], []), (4, 1, [], []),
                                                                (5, 3, [], []), (8, 2, [], [])]
    # two frames per side, clipped to the one-frame middle shot
    assert oracle.shot_windows([0, 4, 5, 10], 3, aug=2) == [(0, 3, [], []), (3, 1, [], [4]), (4, 1, [2, 3], [5, 6]),
                                                            (5, 3, [4], []), (8, 2, [], [])]


def _shot_mask(T, Hs, Ws, shot_start, win_t, th, tw, aug=1):
    """Allowed (query, key) pairs restated token by token from the STGA rules."""
    N = T * Hs * Ws
    shot = np.zeros(T, int)
    for s_, (lo, hi) in enumerate(zip(shot_start[:-1], shot_start[1:])):
        shot[lo:hi] = s_
    def win(t):  # index of t's window inside its shot, and whether first/last
        lo, hi = shot_start[shot[t]], shot_start[shot[t] + 1]
        k = (t - lo) // win_t
        return k, k == 0, lo + (k + 1) * win_t >= hi
    mask = np.zeros((N, N), bool)
    for n in range(N):
        t, y, x = n // (Hs * Ws), (n // Ws) % Hs, n % Ws
        for m in range(N):
            u, yy, xx = m // (Hs * Ws), (m // Ws) % Hs, m % Ws
            if yy // th != y // th or xx // tw != x // tw:
                continue
            same = shot[u] == shot[t] and win(u)[0] == win(t)[0]
            k, first, last = win(t)
            prev = first and shot[u] == shot[t] - 1 and shot_start[shot[t]] - u <= aug
            nxt = last and shot[u] == shot[t] + 1 and u - shot_start[shot[t] + 1] < aug
            mask[n, m] = same or prev or nxt
    return mask


def check_stga_shot_masked():
    r = _rng(19)
    T, Hs, Ws, H, D = 7, 2, 4, 2, 8
    shots = [0, 3, 4, 7]
    N = T * Hs * Ws
    Q, K, V = (r.standard_normal((N, H, D)) for _ in range(3))
    for aug in (1, 2):
        out = oracle.stga_shot_attention(Q, K, V, T, Hs, Ws, shots, 2, 1, 2, 0.3, aug)
        ref = _sdpa(Q, K, V, _shot_mask(T, Hs, Ws, shots, 2, 1, 2, aug), scale=0.3)
        np.testing.assert_allclose(out, ref, atol=1e-12)
    # one shot and windows that tile it: the plain STGA windows
    plain = oracle.stga_shot_attention(Q, K, V, T, Hs, Ws, [0, T], 7, 2, 2, 0.3)
    np.testing.assert_allclose(plain, _sdpa(Q, K, V, oracle.stga_group_ids(T, Hs, Ws, 7, 2, 2)[:, None]
                                             == oracle.stga_group_ids(T, Hs, Ws, 7, 2, 2)[None, :], scale=0.3),
                               atol=1e-12)


def test_stga_shot_is_masked_attention():
    check_stga_shot_masked()


def test_stga_shot_rows_match_masked_attention():
    r = _rng(21)
    T, Hs, Ws, H, D = 6, 2, 2, 1, 4
    shots = [0, 1, 4, 6]
    N = T * Hs * Ws
    Q, K, V = (r.standard_normal((N, H, D)) for _ in range(3))
    for aug in (1, 2, 0):
        rows = oracle.stga_shot_attention_rows(Q, K, V, T, Hs, Ws, shots, 2, 2, 1, 0.7, np.arange(N), aug)
        mask = _shot_mask(T, Hs, Ws, shots, 2, 2, 1, aug)
        if not aug:
            wid = np.array([w for w, (t0, nt, _, _) in enumerate(oracle.shot_windows(shots, 2, False))
                            for _ in range(nt)])
            tok_t = np.arange(N) // (Hs * Ws)
            col = np.arange(N) % Ws
            mask = (wid[tok_t][:, None] == wid[tok_t][None, :]) & (col[:, None] == col[None, :])
        np.testing.assert_allclose(rows, _sdpa(Q, K, V, mask, scale=0.7), atol=1e-12)


def test_frame_attention_and_visual_mean():
    r = _rng(20)
    T, Hs, Ws, H, D, d, M = 4, 2, 3, 2, 8, 12, 3
    N = T * Hs * Ws
    X = r.standard_normal((N, d))
    Wr = r.standard_normal((M, d))
    Q, K, V = (r.standard_normal((N, H, D)) for _ in range(3))
    frame_ids = np.arange(N) // (Hs * Ws)
    fr = oracle.frame_attention(Q, K, V, T, Hs, Ws, 1 / math.sqrt(D))
    np.testing.assert_allclose(fr, _sdpa(Q, K, V, frame_ids[:, None] == frame_ids[None, :]), atol=1e-12)
    vb = oracle.visual_block_forward(X, Wr, Q, K, V, M, T, Hs, Ws, [0, 2, 4], 2, 1, 3)
    moga = oracle.moga_forward(X, Wr, Q, K, V, M)["O"]
    st = oracle.stga_shot_attention(Q, K, V, T, Hs, Ws, [0, 2, 4], 2, 1, 3, 1 / math.sqrt(D))
    np.testing.assert_allclose(vb, (moga + st + fr) / 3, atol=1e-12)


# ---------------------------------------------------------------------------
# Backward pass: pinned against float64 autograd of an independent dense
# formulation (same-group mask, router softmax, gate times attention)
# ---------------------------------------------------------------------------

def _autograd_grads(X, Wr, Q, K, V, dO, bias, g, scale):
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True)  # noqa: E731
    Xt, Wt, Qt, Kt, Vt = t(X), t(Wr), t(Q), t(K), t(V)
    bt = t(np.zeros(Wr.shape[0]) if bias is None else bias)
    gt = torch.tensor(np.asarray(g, dtype=np.int64))
    prob = torch.softmax(Xt @ Wt.T + bt, dim=1)
    p = prob[torch.arange(X.shape[0]), gt]
    mask = gt[:, None] == gt[None, :]
    outs = []
    for h in range(Q.shape[1]):
        S = scale * (Qt[:, h] @ Kt[:, h].T)
        S = S.masked_fill(~mask, float("-inf"))
        outs.append(torch.softmax(S, dim=1) @ Vt[:, h])
    O = p[:, None, None] * torch.stack(outs, dim=1)
    (O * torch.tensor(dO)).sum().backward()
    return {"dQ": Qt.grad.numpy(), "dK": Kt.grad.numpy(), "dV": Vt.grad.numpy(), "dX": Xt.grad.numpy(),
            "dWr": Wt.grad.numpy(), "dbias": bt.grad.numpy()}


def check_backward_autograd(seed=30, bias=True):
    X, Wr, Q, K, V, b = _random_case(seed, N=90, d=20, M=4, H=2, D=8, bias=bias)
    dO = _rng(seed + 100).standard_normal(Q.shape)
    out = oracle.moga_backward(X, Wr, Q, K, V, 4, dO, scale=0.4, bias=b)
    ref = _autograd_grads(X, Wr, Q, K, V, dO, b, out["group_id"], 0.4)
    for k, v in ref.items():
        np.testing.assert_allclose(out[k], v, rtol=1e-9, atol=1e-11, err_msg=k)


def test_backward_matches_autograd():
    check_backward_autograd()
    check_backward_autograd(seed=31, bias=False)


def test_backward_rows_match_full_backward():
    X, Wr, Q, K, V, b = _random_case(39, N=70, d=16, M=3, H=2, D=8, bias=True)
    dO = _rng(40).standard_normal(Q.shape)
    full = oracle.moga_backward(X, Wr, Q, K, V, 3, dO, bias=b)
    rows = np.array([0, 5, 33, 69])
    part = oracle.moga_backward_rows(X, Wr, Q, K, V, 3, dO, rows, bias=b)
    for k in ("dQ", "dgate", "dX"):
        np.testing.assert_allclose(part[k], full[k][rows], rtol=1e-10, atol=1e-12, err_msg=k)


def test_backward_group_sum_invariants():
    # rows of P sum to 1: a group's dV sums to its gated upstream gradient;
    # rows of dS sum to 0: a group's dK sums to zero
    X, Wr, Q, K, V, _ = _random_case(41, N=80, M=4)
    dO = _rng(42).standard_normal(Q.shape)
    out = oracle.moga_backward(X, Wr, Q, K, V, 4, dO)
    g, p = out["group_id"], out["gate"]
    for i in range(4):
        m = g == i
        if m.any():
            np.testing.assert_allclose(out["dV"][m].sum(axis=0), (p[m, None, None] * dO[m]).sum(axis=0), atol=1e-12)
            np.testing.assert_allclose(out["dK"][m].sum(axis=0), 0.0, atol=1e-12)


def test_backward_single_group_router_gradient_vanishes():
    # M = 1: p == 1 for every token and its derivative is zero
    X, Wr, Q, K, V, _ = _random_case(32, N=40, M=1)
    dO = _rng(33).standard_normal(Q.shape)
    out = oracle.moga_backward(X, Wr, Q, K, V, 1, dO)
    assert np.abs(out["dX"]).max() == 0 and np.abs(out["dWr"]).max() == 0 and np.abs(out["dbias"]).max() == 0


def test_backward_constant_values_give_no_query_key_gradient():
    # V rows equal inside a group: attention returns that row for any weights
    X, Wr, Q, K, _, _ = _random_case(34, N=50, M=3)
    V = np.broadcast_to(_rng(35).standard_normal((1, Q.shape[1], Q.shape[2])), Q.shape).copy()
    out = oracle.moga_backward(X, Wr, Q, K, V, 3, _rng(36).standard_normal(Q.shape))
    assert np.abs(out["dQ"]).max() < 1e-12 and np.abs(out["dK"]).max() < 1e-12


def test_backward_lse_and_delta_definitions():
    X, Wr, Q, K, V, _ = _random_case(37, N=30, M=2, H=1, D=4)
    dO = _rng(38).standard_normal(Q.shape)
    out = oracle.moga_backward(X, Wr, Q, K, V, 2, dO)
    perm, cu = out["perm"], out["cu_seqlens"]
    scale = 0.5
    j = int(cu[1])                     # first row of group 1
    grp = perm[cu[1]:cu[2]]
    n = perm[j]
    s = [math.fsum(Q[n, 0, c] * K[m, 0, c] for c in range(4)) * scale for m in grp]
    assert abs(out["lse"][0, j] - math.log(math.fsum(math.exp(x) for x in s))) < 1e-12
    assert abs(out["delta"][0, j] - out["gate"][n] * float(np.dot(dO[n, 0], out["Op"][j, 0]))) < 1e-12


# ---------------------------------------------------------------------------
# Group-balancing statistics (Eq. 6)
# ---------------------------------------------------------------------------

def check_balance_worked_example():
    """Eq. 6 by hand on six tokens with gates other than 1 (so that P_i and
    F_i differ): group ids 0, 2, 0, 1, 2, 2 and gates 0.9, 0.6, 0.7, 0.5,
    0.8, 0.6, M = 3, alpha = 0.1.  Counts 2, 1, 3 give F = 2/6, 1/6, 3/6; the
    gate sums 0.9 + 0.7 = 1.6, 0.5 and 0.6 + 0.8 + 0.6 = 2.0, each over N = 6,
    give P = 1.6/6, 0.5/6, 2.0/6; sum_i F_i P_i = (3.2 + 0.5 + 6.0) / 36 =
    9.7/36 and L_gb = 0.1 * 3 * 9.7/36 = 2.91/36."""
    g = np.array([0, 2, 0, 1, 2, 2])
    gate = np.array([0.9, 0.6, 0.7, 0.5, 0.8, 0.6])
    F, P, L = oracle.balance_stats(g, gate, 3, 0.1)
    np.testing.assert_allclose(F, [1 / 3, 1 / 6, 1 / 2], rtol=0, atol=1e-15)
    np.testing.assert_allclose(P, [1.6 / 6, 0.5 / 6, 2.0 / 6], rtol=0, atol=1e-15)
    assert abs(L - 2.91 / 36) < 1e-15


def test_balance_stats_worked_example():
    check_balance_worked_example()


def test_balance_stats_pages_values():
    with open(os.path.join(GOLDEN, "balance_loss_facts.json")) as f:
        facts = json.load(f)
    alpha, M = facts["alpha"], 8
    # uniform, fully confident routing: L_gb reaches its stated minimum alpha
    g = np.repeat(np.arange(M), 5)
    _, _, L = oracle.balance_stats(g, np.ones(g.size), M, alpha)
    assert abs(L - facts["uniform_confident_loss_over_alpha"] * alpha) < 1e-12
    # collapse onto one group: sum F_i P_i = 1, so L_gb = alpha * M
    _, _, L = oracle.balance_stats(np.zeros(40, int), np.ones(40), M, alpha)
    assert abs(L - alpha * M) < 1e-12


# ---------------------------------------------------------------------------
# Mutation tests: plant a mistake in the oracle (on the CPU) and check a pin fails
# ---------------------------------------------------------------------------

def _wrong_scale(S, V):
    S = S * 2.0
    S = S - S.max(axis=-1, keepdims=True)
    P = np.exp(S)
    return (P / P.sum(axis=-1, keepdims=True)) @ V


def _no_normalise(S, V):
    S = S - S.max(axis=-1, keepdims=True)
    return np.exp(S) @ V


def _transposed_router(X, Wr, bias=None):
    return np.asarray(X, float) @ np.asarray(Wr, float)


def _unstable_permute(group_id, M):
    perm, cu, mx = _orig_permute(group_id, M)
    g = np.asarray(group_id)
    out = perm.copy()
    for i in range(M):                      # reverse the order inside each group
        out[cu[i]:cu[i + 1]] = perm[cu[i]:cu[i + 1]][::-1]
    return out, cu, mx


def _ungated_unpermute(Op, perm, gate, beta=0.0, O_prev=None):
    return _orig_unpermute(Op, perm, np.ones_like(gate), beta, O_prev)


def _off_by_one_cu(group_id, M):
    perm, cu, mx = _orig_permute(group_id, M)
    cu = cu.copy()
    cu[1] += 1
    return perm, cu, mx


def _windows_ignore_shots(shot_start, win_t, aug=1):
    return _orig_shot_windows([shot_start[0], shot_start[-1]], win_t, aug)


def _augment_wrong_frames(shot_start, win_t, aug=1):
    # the adjacent frames taken one step too far into the neighbouring shots
    return [(t0, nt, [f - 1 for f in p], [f + 1 for f in n])
            for t0, nt, p, n in _orig_shot_windows(shot_start, win_t, aug)]


def _backward_no_delta(*a, **k):
    out = _orig_backward(*a, **k)   # dS = P * dP (delta term dropped) changes dQ and dK
    X, Wr, Q, K, V, M, dO = a[:7]
    scale = k.get("scale") or 1.0 / math.sqrt(Q.shape[2])
    perm, cu = out["perm"], out["cu_seqlens"]
    for i in range(M):
        rows = perm[cu[i]:cu[i + 1]]
        for h in range(Q.shape[1]):
            P = np.exp(scale * Q[rows, h] @ K[rows, h].T - out["lse"][h, cu[i]:cu[i + 1], None])
            out["dQ"][rows, h] += scale * (P * out["delta"][h, cu[i]:cu[i + 1], None]) @ K[rows, h]
    return out


def _backward_router_sign(*a, **k):
    out = _orig_backward(*a, **k)
    out["dX"], out["dWr"], out["dbias"] = -out["dX"], -out["dWr"], -out["dbias"]
    return out


def _backward_unscaled_dk(*a, **k):
    out = _orig_backward(*a, **k)
    out["dK"] = out["dK"] / (k.get("scale") or 1.0 / math.sqrt(a[2].shape[2]))
    return out


def _balance_gate_ignored(group_id, gate, M, alpha=0.1):
    # P_i taken as the token fraction, as if every gate were 1
    return _orig_balance(group_id, np.ones(np.asarray(gate).shape), M, alpha)


def _balance_per_group_mean(group_id, gate, M, alpha=0.1):
    # P_i as the average gate inside group i (the prose's reading, not Eq. 6's 1/N)
    F, P, _ = _orig_balance(group_id, gate, M, alpha)
    P = np.divide(P, F, out=np.zeros_like(P), where=F > 0)
    return F, P, alpha * M * float(np.sum(F * P))


_orig_balance = om.balance_stats
_orig_permute = om.permute
_orig_unpermute = om.unpermute
_orig_shot_windows = om.shot_windows
_orig_backward = om.moga_backward

MUTANTS = [
    ("_softmax_rows_times_v", _wrong_scale, [check_moga_is_gated_masked_attention, check_bruteforce_loops]),
    ("_softmax_rows_times_v", _no_normalise, [check_single_group_is_full_attention]),
    ("router_logits", _transposed_router, [check_route_closed_form]),
    ("permute", _unstable_permute, [check_permute_hand_example, check_permute_bruteforce]),
    ("permute", _off_by_one_cu, [check_moga_is_gated_masked_attention]),
    ("unpermute", _ungated_unpermute, [check_moga_is_gated_masked_attention, check_bruteforce_loops]),
    ("shot_windows", _windows_ignore_shots, [check_stga_shot_masked]),
    ("shot_windows", _augment_wrong_frames, [check_stga_shot_masked]),
    ("moga_backward", _backward_no_delta, [check_backward_autograd]),
    ("moga_backward", _backward_router_sign, [check_backward_autograd]),
    ("moga_backward", _backward_unscaled_dk, [check_backward_autograd]),
    ("balance_stats", _balance_gate_ignored, [check_balance_worked_example]),
    ("balance_stats", _balance_per_group_mean, [check_balance_worked_example]),
]


@pytest.mark.parametrize("name,mutant,checks", MUTANTS,
                         ids=[f"{m[0]}:{m[1].__name__}" for m in MUTANTS])
def test_pins_catch_planted_mistakes(monkeypatch, name, mutant, checks):
    monkeypatch.setattr(om, name, mutant)
    monkeypatch.setattr(oracle, name, mutant, raising=False)
    for check in checks:
        with pytest.raises((AssertionError, IndexError, ValueError)):
            check()


# ---------------------------------------------------------------------------
# Property tests: random sizes, including empty groups, one group holding
# every token and fewer tokens than a tile
# ---------------------------------------------------------------------------

from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

_sizes = st.tuples(st.integers(1, 300), st.integers(1, 64), st.sampled_from([1, 2, 3]), st.sampled_from([64, 128]),
                   st.integers(0, 2**31 - 1), st.booleans())


@settings(max_examples=25, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(_sizes)
def test_property_forward(case):
    N, M, H, D, seed, one_group = case
    r = _rng(seed)
    d = 16
    X = r.standard_normal((N, d))
    Wr = r.standard_normal((M, d)) / math.sqrt(d)
    b = np.zeros(M)
    if one_group:
        b[M - 1] = 1e3                     # every token routed to the last group
    Q, K, V = (r.standard_normal((N, H, D)) for _ in range(3))
    out = oracle.moga_forward(X, Wr, Q, K, V, M=M, bias=b)
    g, perm, cu = out["group_id"], out["perm"], out["cu_seqlens"]
    # every token in exactly one group; counts add up; empty groups repeat cu
    assert g.shape == (N,) and g.min() >= 0 and g.max() < M
    assert cu[0] == 0 and cu[-1] == N and np.all(np.diff(cu) >= 0)
    np.testing.assert_array_equal(np.diff(cu), np.bincount(g, minlength=M))
    assert out["max_seqlen"] == np.diff(cu).max()
    # perm is a bijection, contiguous by group in group order, stable inside
    np.testing.assert_array_equal(np.sort(perm), np.arange(N))
    key = g[perm].astype(np.int64) * N + perm
    assert np.all(np.diff(key) > 0)
    if one_group:
        assert np.all(g == M - 1)
    # the gate is the softmax probability of the chosen group
    r_logits = X @ Wr.T + b
    p = np.exp(r_logits - r_logits.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    np.testing.assert_allclose(out["gate"], p[np.arange(N), g], rtol=1e-5)
    # output: gated attention masked to the token's own group (library routine)
    mask = g[:, None] == g[None, :]
    ref = out["gate"].astype(np.float64)[:, None, None] * _sdpa(Q, K, V, mask, scale=1 / math.sqrt(D))
    np.testing.assert_allclose(out["O"], ref, atol=1e-6)
