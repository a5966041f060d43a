"""Plain, slow, obviously-correct CPU oracle for the MoGA forward hot path.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Source of every definition: the page "MoGA: Mixture-of-Groups Attention for
End-to-End Long Video Generation" (architecture explainer of arXiv 2510.18692),
sections "Vanilla Self-Attention and Its Computational Barrier in Video DiTs"
(Eq. 1), "MoGA Router: Learned Per-Token Group Assignment" (routing scores,
softmax gating Eq. 3, hard argmax assignment), "Grouped Attention: Computing
Self-Attention Within Assigned Groups" (MoGA output equation),
"MoGA Pseudocode and Kernel Integration" (Algorithm 1, steps 1-4),
"Group Balancing Loss: Preventing Router Collapse" (Eq. 6 with F_i and P_i) and
"Spatial-Temporal Group Attention (STGA): Complementary Local Attention".

Precision: every floating-point step is evaluated in float64 from the exact
input values (callers pass float arrays that hold bf16 values).  The single
exception is the router's argmax, which is taken on the float32 rounding of
the exact float64 logits, because that is the precision the GPU kernel decides
in; inputs are generated so that the top-1 margin is far above that rounding.

Readings of points the pages leave open:
  * softmax scale is 1/sqrt(D) with D the per-head dimension;
  * group ids are 0-based; argmax ties go to the lowest index;
  * inside a group, tokens keep their original order (stable permutation);
  * one routing decision per token, shared by every head;
  * empty groups are allowed and produce no rows;
  * the MoGA gate multiplies the attention output once, at unpermute time;
  * STGA groups are fixed (t // win_t, y // tile_h, x // tile_w) windows over
    frame-major tokens n = (t * Hs + y) * Ws + x, with no gate;
  * shot-aware STGA: windows restart at every shot start; the keys and values
    (never the queries) of a shot's first window also hold the previous
    shot's last frame(s), those of its last window the next shot's first
    frame(s), each restricted to the same spatial tile (shot_windows);
  * the visual output is the plain mean of MoGA, shot-aware STGA and
    per-frame attention.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "router_logits",
    "route",
    "permute",
    "gather_rows",
    "group_attention",
    "group_attention_rows",
    "unpermute",
    "stga_group_ids",
    "stga_attention",
    "stga_attention_rows",
    "moga_forward",
    "moga_output_rows",
    "balance_stats",
    "moga_backward",
    "moga_backward_rows",
    "shot_windows",
    "stga_shot_attention",
    "stga_shot_attention_rows",
    "frame_attention",
    "visual_block_forward",
]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# Step 1: router ("MoGA Router" section; Algorithm 1 step 1)
# ---------------------------------------------------------------------------

def router_logits(X, Wr, bias=None) -> np.ndarray:
    """Routing scores r = x W_r (+ optional bias), one row per token.

    "MoGA Router" section, routing-score equation: a single linear map from the
    hidden dimension to M scores.  ``Wr`` is stored as [M, d_model] (one
    prototype per row), so r[n, i] = sum_k X[n, k] * Wr[i, k].
    Evaluated in float64; products of bf16 values are exact there.
    """
    r = _f64(X) @ _f64(Wr).T
    if bias is not None:
        r = r + _f64(bias)[None, :]
    return r


def route(X, Wr, bias=None):
    """Hard group assignment and gate for every token.

    "MoGA Router" section: p(i|x) = softmax(r)_i (Eq. 3) and
    g(x) = argmax_i p(i|x).  Because softmax is strictly increasing in each
    score, the argmax of p is the argmax of r.  The gate used by the MoGA
    output equation ("Grouped Attention" section) is p(g(x)|x)
    = 1 / sum_j exp(r_j - r_g).

    Returns (group_id int32[N], gate float32[N], logits float64[N, M]).
    """
    r64 = router_logits(X, Wr, bias)
    # decision in float32, ties -> lowest index (numpy argmax convention)
    g = np.argmax(r64.astype(np.float32), axis=1).astype(np.int32)
    r_top = r64[np.arange(r64.shape[0]), g]
    denom = np.exp(r64 - r_top[:, None]).sum(axis=1)
    gate = (1.0 / denom).astype(np.float32)
    return g, gate, r64


# ---------------------------------------------------------------------------
# Step 2: permutation by group ("MoGA Pseudocode", Algorithm 1 step 2)
# ---------------------------------------------------------------------------

def permute(group_id, M: int):
    """Order tokens so group 0 comes first, then group 1, and so on.

    Algorithm 1 step 2: the permuted sequence holds every token of group 0,
    then every token of group 1, ...; cu_seqlens marks the group boundaries,
    max_seqlen is the largest group and the permute index maps permuted
    positions back to original tokens.  Within a group the original token
    order is kept (a stable sort; the pages do not fix this order).

    Returns (perm int32[N] with perm[j] = original token at permuted row j,
             cu_seqlens int32[M+1], max_seqlen int).
    """
    g = np.asarray(group_id).astype(np.int64)
    if g.size and (g.min() < 0 or g.max() >= M):
        raise ValueError("group id out of range")
    counts = np.bincount(g, minlength=M)
    cu = np.zeros(M + 1, dtype=np.int64)
    cu[1:] = np.cumsum(counts)
    perm = np.argsort(g, kind="stable").astype(np.int32)
    max_seqlen = int(counts.max()) if M > 0 else 0
    return perm, cu.astype(np.int32), max_seqlen


def gather_rows(T, perm) -> np.ndarray:
    """Permuted copy T_hat[j] = T[perm[j]] (Algorithm 1 step 2 applied to Q, K, V)."""
    return np.asarray(T)[np.asarray(perm)]


# ---------------------------------------------------------------------------
# Step 3: self-attention inside every group (Eq. 1 per group; Algorithm 1 step 3)
# ---------------------------------------------------------------------------

def _softmax_rows_times_v(S, V):
    """softmax over the last axis of S (float64), then times V (Eq. 1)."""
    S = S - S.max(axis=-1, keepdims=True)
    P = np.exp(S)
    P /= P.sum(axis=-1, keepdims=True)
    return P @ V


def _group_of_rows(cu_seqlens, rows):
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    # group i holds permuted rows cu[i] .. cu[i+1]-1; empty groups never match
    return np.searchsorted(cu, np.asarray(rows, dtype=np.int64), side="right") - 1


def group_attention_rows(Qp, Kp, Vp, cu_seqlens, scale, rows, heads=None):
    """Attention output of selected permuted rows, every head unless ``heads``.

    For permuted row j in group i and head h (Eq. 1 restricted to the group,
    Algorithm 1 step 3): O[j, h] = softmax(q_jh . K_ih^T * scale) V_ih, where
    K_ih, V_ih are rows cu[i] .. cu[i+1]-1 of head h.  Non-causal; the token
    attends to itself.  Returns float64 [len(rows), H_sel, D].
    """
    rows = np.asarray(rows, dtype=np.int64)
    Hn = Qp.shape[1]
    heads = np.arange(Hn) if heads is None else np.asarray(heads, dtype=np.int64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    out = np.zeros((rows.size, heads.size, Qp.shape[2]), dtype=np.float64)
    grp = _group_of_rows(cu, rows)
    for i in np.unique(grp):
        sel = np.nonzero(grp == i)[0]
        lo, hi = cu[i], cu[i + 1]
        for a, h in enumerate(heads):
            q = _f64(Qp[rows[sel], h, :])
            k = _f64(Kp[lo:hi, h, :])
            v = _f64(Vp[lo:hi, h, :])
            out[sel, a, :] = _softmax_rows_times_v((q @ k.T) * scale, v)
    return out


def group_attention(Qp, Kp, Vp, cu_seqlens, scale, row_block: int = 2048):
    """Attention of every permuted row within its group (float64 [N, H, D]).

    Rows are evaluated ``row_block`` at a time only to bound memory; each row's
    softmax is independent of the others, so this is the same definition.
    """
    N = Qp.shape[0]
    out = np.zeros((N, Qp.shape[1], Qp.shape[2]), dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    for i in range(cu.size - 1):
        lo, hi = int(cu[i]), int(cu[i + 1])
        for s in range(lo, hi, row_block):
            r = np.arange(s, min(hi, s + row_block))
            out[r] = group_attention_rows(Qp, Kp, Vp, cu, scale, r)
    return out


# ---------------------------------------------------------------------------
# Step 4: gate and unpermute ("Grouped Attention" output equation; Algorithm 1 step 4)
# ---------------------------------------------------------------------------

def unpermute(Op, perm, gate, beta: float = 0.0, O_prev=None):
    """O[perm[j]] = beta * O_prev[perm[j]] + gate[perm[j]] * Op[j].

    The MoGA output equation multiplies the in-group attention of token x by
    p(g(x)|x); Algorithm 1 step 4 returns rows to their original positions.
    ``beta`` = 0 overwrites, 1 adds onto ``O_prev`` (used to sum with STGA).
    """
    perm = np.asarray(perm, dtype=np.int64)
    g64 = _f64(gate)
    out = np.zeros(Op.shape, dtype=np.float64)
    out[perm] = g64[perm][:, None, None] * _f64(Op)
    if beta != 0.0:
        out += beta * _f64(O_prev)
    return out


# ---------------------------------------------------------------------------
# STGA branch ("Spatial-Temporal Group Attention (STGA)" section)
# ---------------------------------------------------------------------------

def stga_group_ids(T, Hs, Ws, win_t, tile_h, tile_w) -> np.ndarray:
    """Static group of every frame-major token n = (t*Hs + y)*Ws + x.

    STGA section: the latent grid is split into fixed spatial windows and
    frames are grouped along time.  Here the spatial windows are tile_h x
    tile_w and the temporal groups are consecutive runs of win_t frames.
    Group id = ((t // win_t) * (Hs // tile_h) + y // tile_h) * (Ws // tile_w)
               + x // tile_w.
    """
    if T % win_t or Hs % tile_h or Ws % tile_w:
        raise ValueError("STGA windows must tile the latent grid")
    ids = np.empty((T, Hs, Ws), dtype=np.int64)
    for t in range(T):
        for y in range(Hs):
            for x in range(Ws):
                ids[t, y, x] = ((t // win_t) * (Hs // tile_h) + y // tile_h) * (Ws // tile_w) + x // tile_w
    return ids.reshape(-1)


def stga_attention_rows(Q, K, V, ids, scale, rows):
    """STGA output of selected original rows: softmax attention over the
    tokens that share the row's static group (float64 [len(rows), H, D])."""
    rows = np.asarray(rows, dtype=np.int64)
    ids = np.asarray(ids)
    out = np.zeros((rows.size, Q.shape[1], Q.shape[2]), dtype=np.float64)
    for gid in np.unique(ids[rows]):
        sel = np.nonzero(ids[rows] == gid)[0]
        members = np.nonzero(ids == gid)[0]
        for h in range(Q.shape[1]):
            q = _f64(Q[rows[sel], h, :])
            k = _f64(K[members, h, :])
            v = _f64(V[members, h, :])
            out[sel, h, :] = _softmax_rows_times_v((q @ k.T) * scale, v)
    return out


def stga_attention(Q, K, V, T, Hs, Ws, win_t, tile_h, tile_w, scale,
                   alpha: float = 1.0, beta: float = 0.0, O_prev=None):
    """O = beta * O_prev + alpha * STGA(Q, K, V) over every token (float64)."""
    ids = stga_group_ids(T, Hs, Ws, win_t, tile_h, tile_w)
    if ids.size != Q.shape[0]:
        raise ValueError("T*Hs*Ws must equal N")
    out = alpha * stga_attention_rows(Q, K, V, ids, scale, np.arange(Q.shape[0]))
    if beta != 0.0:
        out += beta * _f64(O_prev)
    return out


# ---------------------------------------------------------------------------
# Shot-aware STGA, per-frame attention and the visual block (STGA section)
# ---------------------------------------------------------------------------

def shot_windows(shot_start, win_t, aug=1):
    """Temporal windows of the shot-aware STGA.

    STGA section: frames are grouped along time and frames of different shots
    never share a temporal group; keys and values (not queries) of a group are
    augmented with latent frames from the adjacent shots.  Reading used: each
    shot [a_s, a_{s+1}) is cut into consecutive windows of win_t frames (the
    last one may be shorter); the first window of a shot (other than the first
    shot) also takes the last ``aug`` frames of the previous shot as keys, and
    the last window of a shot (other than the last shot) the first ``aug``
    frames of the next shot, each clipped to that shot's length.  aug = 1
    gives two augmentation frames for a shot held in one window (one from
    each side); aug = 0 (or False) turns augmentation off.
    Returns a list of (t0, nt, prev_frames, next_frames).
    """
    aug = int(aug)
    a = [int(x) for x in shot_start]
    out = []
    for sh in range(len(a) - 1):
        lo, hi = a[sh], a[sh + 1]
        starts = list(range(lo, hi, win_t))
        for k, t0 in enumerate(starts):
            nt = min(win_t, hi - t0)
            prev = list(range(max(a[sh - 1], lo - aug), lo)) if (k == 0 and sh > 0) else []
            nxt = list(range(hi, min(a[sh + 2], hi + aug))) if (k == len(starts) - 1 and sh < len(a) - 2) else []
            out.append((t0, nt, prev, nxt))
    return out


def stga_shot_attention(Q, K, V, T, Hs, Ws, shot_start, win_t, tile_h, tile_w, scale, aug=1):
    """Shot-aware STGA over frame-major tokens (float64 [N, H, D]): for each
    window and spatial tile, the window's tokens in the tile attend to those
    same tokens plus, as extra keys, the tile's tokens in the augmentation
    frames (shot_windows)."""
    if Hs % tile_h or Ws % tile_w:
        raise ValueError("spatial tiles must tile the frame")
    def tokens(frames, y0, x0):
        return np.array([(t * Hs + y) * Ws + x for t in frames
                         for y in range(y0, y0 + tile_h) for x in range(x0, x0 + tile_w)], dtype=np.int64)
    out = np.zeros(Q.shape, dtype=np.float64)
    for t0, nt, prev, nxt in shot_windows(shot_start, win_t, aug):
        extra = prev + nxt
        for y0 in range(0, Hs, tile_h):
            for x0 in range(0, Ws, tile_w):
                q_tok = tokens(range(t0, t0 + nt), y0, x0)
                k_tok = np.concatenate([q_tok, tokens(extra, y0, x0)]) if extra else q_tok
                for h in range(Q.shape[1]):
                    q = _f64(Q[q_tok, h, :])
                    k = _f64(K[k_tok, h, :])
                    v = _f64(V[k_tok, h, :])
                    out[q_tok, h, :] = _softmax_rows_times_v((q @ k.T) * scale, v)
    return out


def stga_shot_attention_rows(Q, K, V, T, Hs, Ws, shot_start, win_t, tile_h, tile_w, scale, rows, aug=1):
    """Shot-aware STGA output of selected tokens only (float64 [len(rows), H, D]);
    the same windows and key sets as stga_shot_attention."""
    area = tile_h * tile_w
    wins = shot_windows(shot_start, win_t, aug)
    frame_win = {}
    for t0, nt, prev, nxt in wins:
        for t in range(t0, t0 + nt):
            frame_win[t] = (t0, nt, prev, nxt)
    out = np.zeros((len(rows), Q.shape[1], Q.shape[2]), dtype=np.float64)
    for a, n in enumerate(np.asarray(rows, dtype=np.int64)):
        t, y, x = int(n) // (Hs * Ws), (int(n) // Ws) % Hs, int(n) % Ws
        t0, nt, prev, nxt = frame_win[t]
        y0, x0 = y // tile_h * tile_h, x // tile_w * tile_w
        frames = list(range(t0, t0 + nt)) + prev + nxt
        k_tok = np.array([(f * Hs + yy) * Ws + xx for f in frames
                          for yy in range(y0, y0 + tile_h) for xx in range(x0, x0 + tile_w)], dtype=np.int64)
        assert k_tok.size == len(frames) * area
        for h in range(Q.shape[1]):
            q = _f64(Q[n, h, :])[None, :]
            out[a, h, :] = _softmax_rows_times_v((q @ _f64(K[k_tok, h, :]).T) * scale, _f64(V[k_tok, h, :]))[0]
    return out


def frame_attention(Q, K, V, T, Hs, Ws, scale):
    """Per-frame attention (STGA section): every latent frame is one group."""
    return stga_attention(Q, K, V, T, Hs, Ws, 1, Hs, Ws, scale)


def visual_block_forward(X, Wr, Q, K, V, M, T, Hs, Ws, shot_start, win_t, tile_h, tile_w, scale=None, aug=1):
    """Visual attention output of the STGA section: the arithmetic mean of the
    MoGA, shot-aware STGA and per-frame attention outputs (float64)."""
    D = Q.shape[2]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    moga = moga_forward(X, Wr, Q, K, V, M, scale)["O"]
    stga = stga_shot_attention(Q, K, V, T, Hs, Ws, shot_start, win_t, tile_h, tile_w, scale, aug)
    frame = frame_attention(Q, K, V, T, Hs, Ws, scale)
    return (moga + stga + frame) / 3.0


# ---------------------------------------------------------------------------
# Whole forward path (Algorithm 1 steps 1-4, plus the optional STGA sum)
# ---------------------------------------------------------------------------

def moga_forward(X, Wr, Q, K, V, M: int, scale=None, bias=None, stga=None):
    """Full MoGA forward on original token order.

    ``stga`` is None or a dict with T, Hs, Ws, win_t, tile_h, tile_w and the
    weights alpha (STGA) / beta (MoGA); the result is then
    beta * MoGA + alpha * STGA.  Returns a dict with every intermediate.
    """
    D = Q.shape[2]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    g, gate, r = route(X, Wr, bias)
    perm, cu, max_seqlen = permute(g, M)
    Qp, Kp, Vp = gather_rows(Q, perm), gather_rows(K, perm), gather_rows(V, perm)
    Op = group_attention(Qp, Kp, Vp, cu, scale)
    O = unpermute(Op, perm, gate)
    if stga is not None:
        S = stga_attention(Q, K, V, stga["T"], stga["Hs"], stga["Ws"], stga["win_t"],
                           stga["tile_h"], stga["tile_w"], scale)
        O = stga.get("beta", 1.0) * O + stga.get("alpha", 1.0) * S
    return {"group_id": g, "gate": gate, "logits": r, "perm": perm, "cu_seqlens": cu,
            "max_seqlen": max_seqlen, "Op": Op, "O": O}


def moga_output_rows(X, Wr, Q, K, V, M: int, rows, scale=None, bias=None, routed=None):
    """MoGA output at selected ORIGINAL token rows, without the full pass.

    For token n in group g: O[n] = gate_n * SA(q_n, K_g, V_g) (MoGA output
    equation).  ``routed`` may pass a precomputed (group_id, gate) pair.
    Returns float64 [len(rows), H, D].
    """
    D = Q.shape[2]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    if routed is None:
        g, gate, _ = route(X, Wr, bias)
    else:
        g, gate = routed
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, Q.shape[1], D), dtype=np.float64)
    for grp in np.unique(g[rows]):
        sel = np.nonzero(g[rows] == grp)[0]
        members = np.nonzero(g == grp)[0]  # original order; attention is order-free
        for h in range(Q.shape[1]):
            q = _f64(Q[rows[sel], h, :])
            k = _f64(K[members, h, :])
            v = _f64(V[members, h, :])
            out[sel, h, :] = _softmax_rows_times_v((q @ k.T) * scale, v)
    out *= _f64(gate)[rows][:, None, None]
    return out


# ---------------------------------------------------------------------------
# Group-balancing statistics ("Group Balancing Loss" section, Eq. 6)
# ---------------------------------------------------------------------------

def balance_stats(group_id, gate, M: int, alpha: float = 0.1):
    """F_i, P_i and L_gb = alpha * M * sum_i F_i P_i.

    F_i = (1/N) * #{x : g(x) = i};  P_i = (1/N) * sum over tokens with
    g(x) = i of p(g(x)|x), taking the equation's 1/N literally (the prose
    beside it speaks of a per-group average; that reading is not used).
    """
    g = np.asarray(group_id, dtype=np.int64)
    N = g.size
    F = np.bincount(g, minlength=M).astype(np.float64) / N
    P = np.bincount(g, weights=_f64(gate), minlength=M) / N
    return F, P, alpha * M * float(np.sum(F * P))


# ---------------------------------------------------------------------------
# Backward pass ("Grouped Attention" section: the gate p(g|x) is the gradient
# path to the router; Eq. 1 and Eq. 3 differentiated by the chain rule)
# ---------------------------------------------------------------------------

def moga_backward(X, Wr, Q, K, V, M: int, dO, scale=None, bias=None):
    """Gradients of L = sum(O * dO) for the MoGA output O[n] = p_n * SA_n,
    with p_n = softmax(r_n)[g_n], r_n = X_n W_r^T (+ b) and the hard choice
    g_n = argmax r_n held fixed (it has no gradient).  Everything in float64.

    Written out from the chain rule:
      dgate_n   = <dO_n, SA_n>                    (over heads and channels)
      dSA_n     = p_n * dO_n
      per group and head, with P = softmax(scale Q K^T) and A = P V:
        dV = P^T dA,  dP = dA V^T,  dS = P * (dP - rowsum(dA * A)),
        dQ = scale dS K,  dK = scale dS^T Q
      dr_nj     = dgate_n * p_n * ([j == g_n] - softmax(r_n)_j)
      dX = dr W_r,  dW_r = dr^T X,  db = sum_n dr_n.
    Returns a dict with dQ, dK, dV [N, H, D], dX [N, d_model], dWr [M, d_model],
    dbias [M], dgate [N], plus the forward pieces the GPU backward consumes
    (permuted SA output Op, per-row log-sum-exp lse [H, N] of the scaled scores,
    and delta [H, N] = rowsum(dSA * SA) in permuted order).
    """
    X, Wr, Q, K, V, dO = (_f64(a) for a in (X, Wr, Q, K, V, dO))
    N, H, D = Q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    r = router_logits(X, Wr, bias)
    g = np.argmax(r.astype(np.float32), axis=1)
    e = np.exp(r - r.max(axis=1, keepdims=True))
    prob = e / e.sum(axis=1, keepdims=True)
    p = prob[np.arange(N), g]
    perm, cu, _ = permute(g, M)
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    Op = np.zeros((N, H, D))
    lse = np.zeros((H, N))
    delta = np.zeros((H, N))
    dgate = np.zeros(N)
    for i in range(M):
        rows = perm[cu[i]:cu[i + 1]]
        if rows.size == 0:
            continue
        for h in range(H):
            q, k, v = Q[rows, h], K[rows, h], V[rows, h]
            S = scale * (q @ k.T)
            mx = S.max(axis=1, keepdims=True)
            P = np.exp(S - mx)
            den = P.sum(axis=1, keepdims=True)
            P /= den
            A = P @ v
            dA = p[rows, None] * dO[rows, h]
            dgate[rows] += np.sum(dO[rows, h] * A, axis=1)
            dV[rows, h] = P.T @ dA
            dP = dA @ v.T
            dl = np.sum(dA * A, axis=1, keepdims=True)
            dS = P * (dP - dl)
            dQ[rows, h] = scale * (dS @ k)
            dK[rows, h] = scale * (dS.T @ q)
            Op[cu[i]:cu[i + 1], h] = A
            lse[h, cu[i]:cu[i + 1]] = (mx + np.log(den))[:, 0]
            delta[h, cu[i]:cu[i + 1]] = dl[:, 0]
    onehot = np.zeros_like(prob)
    onehot[np.arange(N), g] = 1.0
    dr = (dgate * p)[:, None] * (onehot - prob)
    return {"dQ": dQ, "dK": dK, "dV": dV, "dX": dr @ _f64(Wr), "dWr": dr.T @ X, "dbias": dr.sum(axis=0),
            "dgate": dgate, "dlogits": dr, "group_id": g.astype(np.int32), "gate": p, "perm": perm,
            "cu_seqlens": cu, "Op": Op, "lse": lse, "delta": delta}


def moga_backward_rows(X, Wr, Q, K, V, M: int, dO, rows, scale=None, bias=None, routed=None):
    """The per-token gradients of moga_backward for selected ORIGINAL rows
    only, each from its own group (the same chain rule, the selected queries
    of a group at a time): dQ[rows] (float64 [len, H, D]), dgate[rows] and
    the router's dX[rows].  ``routed`` may pass a precomputed
    (group_id, logits) pair."""
    X, Wr, dO = _f64(X), _f64(Wr), _f64(dO)
    N, H, D = Q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    if routed is None:
        r = router_logits(X, Wr, bias)
        g = np.argmax(r.astype(np.float32), axis=1)
    else:
        g, r = routed
        r = _f64(r)
    rows = np.asarray(rows, dtype=np.int64)
    e = np.exp(r[rows] - r[rows].max(axis=1, keepdims=True))
    prob = e / e.sum(axis=1, keepdims=True)
    pg = prob[np.arange(rows.size), g[rows]]
    dQ = np.zeros((rows.size, H, D))
    dgate = np.zeros(rows.size)
    for grp in np.unique(g[rows]):
        sel = np.nonzero(g[rows] == grp)[0]
        members = np.nonzero(g == grp)[0]
        for h in range(H):
            q, k, v = _f64(Q[rows[sel], h]), _f64(K[members, h]), _f64(V[members, h])
            S = scale * (q @ k.T)
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            A = P @ v
            dA = pg[sel, None] * dO[rows[sel], h]
            dgate[sel] += np.sum(dO[rows[sel], h] * A, axis=1)
            dS = P * (dA @ v.T - np.sum(dA * A, axis=1, keepdims=True))
            dQ[sel, h] = scale * (dS @ k)
    onehot = np.zeros((rows.size, M))
    onehot[np.arange(rows.size), g[rows]] = 1.0
    dX = ((dgate * pg)[:, None] * (onehot - prob)) @ Wr
    return {"dQ": dQ, "dgate": dgate, "dX": dX}
