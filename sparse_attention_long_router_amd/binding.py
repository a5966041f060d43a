"""Python entry points with the names of the C ABI (include/moga.h).

Each function checks tensor placement, dtype and shape, allocates missing
outputs with torch (device memory is all torch provides here) and calls the
library on the current HIP stream.  No arithmetic of the method happens in
Python.
"""

from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import (MOGA_OP_ATTENTION_BACKWARD, MOGA_OP_BALANCE_STATS, MOGA_OP_GROUP_ATTENTION, MOGA_OP_PERMUTE,
                   MOGA_OP_ROUTE_BACKWARD, check, ptr, stream_handle)

BF16 = torch.bfloat16


def _need(t, name, dtype=None, ndim=None, shape=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def moga_workspace_bytes(op: int, N: int, M: int, H: int = 1, D: int = 64) -> int:
    return _lib.workspace_bytes(op, N, M, H, D)


def _workspace(op, N, M, H, D, ws, device):
    need = moga_workspace_bytes(op, N, M, H, D)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    _need(ws, "ws")
    return ws, ws.numel() * ws.element_size()


def moga_route(X, Wr, bias=None, group_id=None, gate=None):
    """group_id int32 [N], gate float32 [N] from X [N, d] and W_r [M, d] (bf16)."""
    _need(X, "X", BF16, 2)
    M, d = Wr.shape
    _need(Wr, "Wr", BF16, 2, (M, X.shape[1]))
    if bias is not None:
        _need(bias, "bias", torch.float32, 1, (M,))
    N = X.shape[0]
    group_id = torch.empty(N, dtype=torch.int32, device=X.device) if group_id is None else group_id
    gate = torch.empty(N, dtype=torch.float32, device=X.device) if gate is None else gate
    _need(group_id, "group_id", torch.int32, 1, (N,))
    _need(gate, "gate", torch.float32, 1, (N,))
    check(_lib.LIB.moga_route(ptr(X), ptr(Wr), ptr(bias), N, d, M, ptr(group_id), ptr(gate), None, 0,
                              stream_handle()),
          "moga_route")
    return group_id, gate


def moga_permute(group_id, M, Q=None, K=None, V=None, Qp=None, Kp=None, Vp=None, perm=None, cu_seqlens=None,
                 max_seqlen=None, ws=None):
    """Stable group permutation; gathers Q/K/V when given.  Returns a dict."""
    _need(group_id, "group_id", torch.int32, 1)
    N = group_id.shape[0]
    dev = group_id.device
    rows = Q is not None
    H = D = 1
    if rows:
        _need(Q, "Q", BF16, 3)
        H, D = Q.shape[1], Q.shape[2]
        for name, t in (("K", K), ("V", V)):
            _need(t, name, BF16, 3, Q.shape)
        if Q.shape[0] != N:
            raise ValueError("Q rows must match group_id")
        Qp = torch.empty_like(Q) if Qp is None else Qp
        Kp = torch.empty_like(K) if Kp is None else Kp
        Vp = torch.empty_like(V) if Vp is None else Vp
        for name, t in (("Qp", Qp), ("Kp", Kp), ("Vp", Vp)):
            _need(t, name, BF16, 3, Q.shape)
    perm = torch.empty(N, dtype=torch.int32, device=dev) if perm is None else perm
    cu_seqlens = torch.empty(M + 1, dtype=torch.int32, device=dev) if cu_seqlens is None else cu_seqlens
    max_seqlen = torch.empty(1, dtype=torch.int32, device=dev) if max_seqlen is None else max_seqlen
    _need(perm, "perm", torch.int32, 1, (N,))
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1, (M + 1,))
    _need(max_seqlen, "max_seqlen", torch.int32, 1, (1,))
    ws, nbytes = _workspace(MOGA_OP_PERMUTE, N, M, H, D, ws, dev)
    check(_lib.LIB.moga_permute(ptr(group_id), ptr(Q), ptr(K), ptr(V), N, H, D, M, ptr(Qp), ptr(Kp), ptr(Vp),
                                ptr(perm), ptr(cu_seqlens), ptr(max_seqlen), ptr(ws), nbytes, stream_handle()),
          "moga_permute")
    return {"Qp": Qp, "Kp": Kp, "Vp": Vp, "perm": perm, "cu_seqlens": cu_seqlens, "max_seqlen": max_seqlen}


def moga_group_attention(Qp, Kp, Vp, cu_seqlens, softmax_scale=0.0, Op=None, ws=None):
    """Attention inside each group of the permuted Q/K/V (bf16 [N, H, D])."""
    _need(Qp, "Qp", BF16, 3)
    N, H, D = Qp.shape
    _need(Kp, "Kp", BF16, 3, Qp.shape)
    _need(Vp, "Vp", BF16, 3, Qp.shape)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    M = cu_seqlens.shape[0] - 1
    Op = torch.empty_like(Qp) if Op is None else Op
    _need(Op, "Op", BF16, 3, Qp.shape)
    ws, nbytes = _workspace(MOGA_OP_GROUP_ATTENTION, N, M, H, D, ws, Qp.device)
    check(_lib.LIB.moga_group_attention(ptr(Qp), ptr(Kp), ptr(Vp), ptr(cu_seqlens), N, H, D, M,
                                        float(softmax_scale), ptr(Op), ptr(ws), nbytes, stream_handle()),
          "moga_group_attention")
    return Op


def moga_group_attention_unpermute(Qp, Kp, Vp, cu_seqlens, perm, gate, softmax_scale=0.0, beta=0.0, O=None,
                                   ws=None):
    """Group attention with the gated unpermute fused in: O[perm[j]] = beta*O + gate*Attn(j)."""
    _need(Qp, "Qp", BF16, 3)
    N, H, D = Qp.shape
    _need(Kp, "Kp", BF16, 3, Qp.shape)
    _need(Vp, "Vp", BF16, 3, Qp.shape)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _need(perm, "perm", torch.int32, 1, (N,))
    _need(gate, "gate", torch.float32, 1, (N,))
    M = cu_seqlens.shape[0] - 1
    if O is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs an existing O")
        O = torch.empty_like(Qp)
    _need(O, "O", BF16, 3, Qp.shape)
    ws, nbytes = _workspace(MOGA_OP_GROUP_ATTENTION, N, M, H, D, ws, Qp.device)
    check(_lib.LIB.moga_group_attention_unpermute(ptr(Qp), ptr(Kp), ptr(Vp), ptr(cu_seqlens), ptr(perm), ptr(gate),
                                                  N, H, D, M, float(softmax_scale), float(beta), ptr(O), ptr(ws),
                                                  nbytes, stream_handle()),
          "moga_group_attention_unpermute")
    return O


def moga_vt_row_length(N):
    """Tokens per channel row of the transposed-V layout: N rounded up to a
    multiple of 64, plus 64 (the padding is zeros)."""
    return (N + 63) // 64 * 64 + 64


def _permute_vt_outputs(group_id, M, Q, K, V, Qp, Kp, Vt, perm, cu_seqlens, max_seqlen):
    """Checks and (where missing) allocates the outputs of the transposed-V permute."""
    _need(group_id, "group_id", torch.int32, 1)
    N = group_id.shape[0]
    dev = group_id.device
    _need(K, "K", BF16, 3)
    H, D = K.shape[1], K.shape[2]
    _need(V, "V", BF16, 3, K.shape)
    if K.shape[0] != N:
        raise ValueError("K rows must match group_id")
    if Q is not None:
        _need(Q, "Q", BF16, 3, K.shape)
        Qp = torch.empty_like(Q) if Qp is None else Qp
        _need(Qp, "Qp", BF16, 3, K.shape)
    elif Qp is not None:
        raise ValueError("Qp given without Q")
    Kp = torch.empty_like(K) if Kp is None else Kp
    ldv = moga_vt_row_length(N)
    Vt = torch.empty((H, D, ldv), dtype=BF16, device=dev) if Vt is None else Vt
    _need(Kp, "Kp", BF16, 3, K.shape)
    _need(Vt, "Vt", BF16, 3, (H, D, ldv))
    perm = torch.empty(N, dtype=torch.int32, device=dev) if perm is None else perm
    cu_seqlens = torch.empty(M + 1, dtype=torch.int32, device=dev) if cu_seqlens is None else cu_seqlens
    max_seqlen = torch.empty(1, dtype=torch.int32, device=dev) if max_seqlen is None else max_seqlen
    _need(perm, "perm", torch.int32, 1, (N,))
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1, (M + 1,))
    _need(max_seqlen, "max_seqlen", torch.int32, 1, (1,))
    return {"Qp": Qp, "Kp": Kp, "Vt": Vt, "perm": perm, "cu_seqlens": cu_seqlens, "max_seqlen": max_seqlen}


def moga_permute_vt(group_id, M, Q, K, V, Qp=None, Kp=None, Vt=None, perm=None, cu_seqlens=None,
                    max_seqlen=None, ws=None):
    """moga_permute with V written transposed per head: Vt bf16 [H, D, ldv]
    (ldv = moga_vt_row_length(N)), Vt[h, d, j] = V[perm[j], h, d] for j < N,
    zeros after.  Q = None skips the Q gather (for
    moga_group_attention_unpermute_vtq, which reads Q through perm).  Returns
    a dict (Qp, Kp, Vt, perm, cu_seqlens, max_seqlen); Qp is None without Q."""
    out = _permute_vt_outputs(group_id, M, Q, K, V, Qp, Kp, Vt, perm, cu_seqlens, max_seqlen)
    N, H, D = K.shape
    ws, nbytes = _workspace(MOGA_OP_PERMUTE, N, M, H, D, ws, group_id.device)
    check(_lib.LIB.moga_permute_vt(ptr(group_id), ptr(Q), ptr(K), ptr(V), N, H, D, M, ptr(out["Qp"]),
                                   ptr(out["Kp"]), ptr(out["Vt"]), ptr(out["perm"]), ptr(out["cu_seqlens"]),
                                   ptr(out["max_seqlen"]), ptr(ws), nbytes, stream_handle()),
          "moga_permute_vt")
    return out


def moga_permute_vt_noalloc(group_id, M, Q, K, V, Qp=None, Kp=None, Vt=None, perm=None, cu_seqlens=None,
                            max_seqlen=None):
    """moga_permute_vt without a workspace: the library keeps the sort's
    scratch in a fixed per-GPU device array (see include/moga.h).  Pass every
    output to have no allocation at all; missing ones are allocated here."""
    out = _permute_vt_outputs(group_id, M, Q, K, V, Qp, Kp, Vt, perm, cu_seqlens, max_seqlen)
    N, H, D = K.shape
    check(_lib.LIB.moga_permute_vt_noalloc(ptr(group_id), ptr(Q), ptr(K), ptr(V), N, H, D, M, ptr(out["Qp"]),
                                           ptr(out["Kp"]), ptr(out["Vt"]), ptr(out["perm"]),
                                           ptr(out["cu_seqlens"]), ptr(out["max_seqlen"]), stream_handle()),
          "moga_permute_vt_noalloc")
    return out


def moga_group_attention_unpermute_vt(Qp, Kp, Vt, cu_seqlens, perm, gate, softmax_scale=0.0, beta=0.0, O=None,
                                      ws=None):
    """moga_group_attention_unpermute with V transposed per head (Vt bf16
    [H, D, moga_vt_row_length(N)] from moga_permute_vt)."""
    _need(Qp, "Qp", BF16, 3)
    N, H, D = Qp.shape
    _need(Kp, "Kp", BF16, 3, Qp.shape)
    _need(Vt, "Vt", BF16, 3, (H, D, moga_vt_row_length(N)))
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _need(perm, "perm", torch.int32, 1, (N,))
    _need(gate, "gate", torch.float32, 1, (N,))
    M = cu_seqlens.shape[0] - 1
    if O is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs an existing O")
        O = torch.empty_like(Qp)
    _need(O, "O", BF16, 3, Qp.shape)
    ws, nbytes = _workspace(MOGA_OP_GROUP_ATTENTION, N, M, H, D, ws, Qp.device)
    check(_lib.LIB.moga_group_attention_unpermute_vt(ptr(Qp), ptr(Kp), ptr(Vt), ptr(cu_seqlens), ptr(perm),
                                                     ptr(gate), N, H, D, M, float(softmax_scale), float(beta),
                                                     ptr(O), ptr(ws), nbytes, stream_handle()),
          "moga_group_attention_unpermute_vt")
    return O


def moga_group_attention_unpermute_vtq(Q, Kp, Vt, cu_seqlens, perm, gate, softmax_scale=0.0, beta=0.0, O=None,
                                       ws=None):
    """moga_group_attention_unpermute_vt with Q in original token order (read
    through perm inside the kernel); Kp and Vt from moga_permute_vt."""
    _need(Q, "Q", BF16, 3)
    N, H, D = Q.shape
    _need(Kp, "Kp", BF16, 3, Q.shape)
    _need(Vt, "Vt", BF16, 3, (H, D, moga_vt_row_length(N)))
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _need(perm, "perm", torch.int32, 1, (N,))
    _need(gate, "gate", torch.float32, 1, (N,))
    M = cu_seqlens.shape[0] - 1
    if O is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs an existing O")
        O = torch.empty_like(Q)
    _need(O, "O", BF16, 3, Q.shape)
    ws, nbytes = _workspace(MOGA_OP_GROUP_ATTENTION, N, M, H, D, ws, Q.device)
    check(_lib.LIB.moga_group_attention_unpermute_vtq(ptr(Q), ptr(Kp), ptr(Vt), ptr(cu_seqlens), ptr(perm),
                                                      ptr(gate), N, H, D, M, float(softmax_scale), float(beta),
                                                      ptr(O), ptr(ws), nbytes, stream_handle()),
          "moga_group_attention_unpermute_vtq")
    return O


def moga_group_attention_fused(Q, K, V, cu_seqlens, perm, gate, softmax_scale=0.0, beta=0.0, O=None, ws=None):
    """Gated group attention on the original-order Q/K/V (rows read through
    perm): O[n] = beta*O[n] + gate[n]*Attn(n)."""
    _need(Q, "Q", BF16, 3)
    N, H, D = Q.shape
    _need(K, "K", BF16, 3, Q.shape)
    _need(V, "V", BF16, 3, Q.shape)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _need(perm, "perm", torch.int32, 1, (N,))
    _need(gate, "gate", torch.float32, 1, (N,))
    M = cu_seqlens.shape[0] - 1
    if O is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs an existing O")
        O = torch.empty_like(Q)
    _need(O, "O", BF16, 3, Q.shape)
    for name, t in (("Q", Q), ("K", K), ("V", V)):
        if O.data_ptr() == t.data_ptr():
            raise ValueError(f"O must not alias {name}")
    ws, nbytes = _workspace(MOGA_OP_GROUP_ATTENTION, N, M, H, D, ws, Q.device)
    check(_lib.LIB.moga_group_attention_fused(ptr(Q), ptr(K), ptr(V), ptr(cu_seqlens), ptr(perm), ptr(gate), N, H, D,
                                              M, float(softmax_scale), float(beta), ptr(O), ptr(ws), nbytes,
                                              stream_handle()),
          "moga_group_attention_fused")
    return O


def moga_unpermute(Op, perm, gate, beta=0.0, O=None):
    """O[perm[j]] = beta * O[perm[j]] + gate[perm[j]] * Op[j]."""
    _need(Op, "Op", BF16, 3)
    N, H, D = Op.shape
    _need(perm, "perm", torch.int32, 1, (N,))
    _need(gate, "gate", torch.float32, 1, (N,))
    if O is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs an existing O")
        O = torch.empty_like(Op)
    _need(O, "O", BF16, 3, Op.shape)
    check(_lib.LIB.moga_unpermute(ptr(Op), ptr(perm), ptr(gate), N, H, D, float(beta), ptr(O), stream_handle()),
          "moga_unpermute")
    return O


def moga_stga_attention(Q, K, V, T, Hs, Ws, win_t, tile_h, tile_w, softmax_scale=0.0, alpha=1.0, beta=0.0,
                        O=None):
    """Static window attention over frame-major tokens; O = beta*O + alpha*STGA."""
    _need(Q, "Q", BF16, 3)
    N, H, D = Q.shape
    _need(K, "K", BF16, 3, Q.shape)
    _need(V, "V", BF16, 3, Q.shape)
    if O is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs an existing O")
        O = torch.empty_like(Q)
    _need(O, "O", BF16, 3, Q.shape)
    if T * Hs * Ws != N:
        raise ValueError("T*Hs*Ws must equal N")
    check(_lib.LIB.moga_stga_attention(ptr(Q), ptr(K), ptr(V), T, Hs, Ws, win_t, tile_h, tile_w, H, D,
                                       float(softmax_scale), float(alpha), float(beta), ptr(O), None, 0,
                                       stream_handle()),
          "moga_stga_attention")
    return O


def moga_stga_shot_workspace_bytes(T: int, n_shots: int, win_t: int) -> int:
    return int(_lib.LIB.moga_stga_shot_workspace_bytes(T, n_shots, win_t))


def moga_stga_shot_attention(Q, K, V, T, Hs, Ws, shot_start, win_t, tile_h, tile_w, augment=1,
                             softmax_scale=0.0, alpha=1.0, beta=0.0, O=None, ws=None):
    """Shot-aware window attention over frame-major tokens; O = beta*O + alpha*STGA.
    shot_start: int32 GPU tensor [n_shots + 1] (0, ..., T); augment: frames
    taken from each adjacent shot as extra keys (0: none; True counts as 1)."""
    _need(Q, "Q", BF16, 3)
    N, H, D = Q.shape
    _need(K, "K", BF16, 3, Q.shape)
    _need(V, "V", BF16, 3, Q.shape)
    _need(shot_start, "shot_start", torch.int32, 1)
    n_shots = shot_start.shape[0] - 1
    if O is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs an existing O")
        O = torch.empty_like(Q)
    _need(O, "O", BF16, 3, Q.shape)
    if T * Hs * Ws != N:
        raise ValueError("T*Hs*Ws must equal N")
    if n_shots < 1:
        raise ValueError("shot_start needs at least two entries")
    need = moga_stga_shot_workspace_bytes(T, n_shots, win_t)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=Q.device)
    _need(ws, "ws")
    check(_lib.LIB.moga_stga_shot_attention(ptr(Q), ptr(K), ptr(V), T, Hs, Ws, ptr(shot_start), n_shots, win_t,
                                            tile_h, tile_w, int(augment), H, D, float(softmax_scale),
                                            float(alpha), float(beta), ptr(O), ptr(ws),
                                            ws.numel() * ws.element_size(), stream_handle()),
          "moga_stga_shot_attention")
    return O


def moga_balance_stats(group_id, gate, M, alpha=0.1, ws=None):
    """F [M], P [M] and the loss alpha*M*sum(F*P) (float32 device tensors)."""
    _need(group_id, "group_id", torch.int32, 1)
    N = group_id.shape[0]
    _need(gate, "gate", torch.float32, 1, (N,))
    dev = group_id.device
    F = torch.empty(M, dtype=torch.float32, device=dev)
    P = torch.empty(M, dtype=torch.float32, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    ws, nbytes = _workspace(MOGA_OP_BALANCE_STATS, N, M, 1, 64, ws, dev)
    check(_lib.LIB.moga_balance_stats(ptr(group_id), ptr(gate), N, M, float(alpha), ptr(F), ptr(P), ptr(loss),
                                      ptr(ws), nbytes, stream_handle()),
          "moga_balance_stats")
    return F, P, loss


class MogaForward:
    """Preallocated buffers for one MoGA layer pass and, when ``stga``
    geometry is given, the STGA branch.  ``__call__`` launches the library
    calls back to back on the current stream and allocates nothing.

    ``path`` selects how the group attention meets the permutation:
      "fused_vtq" (default): a gathered K copy and V gathered transposed per
        head; the attention reads each query row through perm and applies
        the gated unpermute in its epilogue (moga_permute_vt without Q,
        moga_group_attention_unpermute_vtq; N <= 2^23 - 128);
      "fused_vt": as "fused_vtq" with a gathered Q copy
        (moga_group_attention_unpermute_vt);
      "fused_epilogue": as "fused_vt" with V in row layout
        (moga_permute, moga_group_attention_unpermute);
      "gather_on_load": sort only, then moga_group_attention_fused reads
        Q/K/V rows through perm -- no gathered copies (3*N*H*D bf16 less
        device memory) at about the same step time (the gather pass saved is
        spent again on indirect row reads inside the attention);
      "separate": gathered copies, moga_group_attention, moga_unpermute.

    ``stga``: dict with T, Hs, Ws, win_t, tile_h, tile_w and optionally
    ``shot_start`` (a list of shot start frames ending with T) and ``augment``
    (frames per adjacent shot, default 1).  Without shots the branch is the
    plain static-window STGA, added with ``stga_weight``.  With
    ``shot_start`` the pass computes the visual attention output of the STGA
    section: the mean of MoGA, shot-aware STGA and per-frame attention."""

    PATHS = ("fused_vtq", "fused_vt", "fused_epilogue", "gather_on_load", "separate")
    VT_MAX_TOKENS = (1 << 23) - 128

    def __init__(self, N, d_model, H, D, M, device, stga=None, path="fused_vtq"):
        if path not in self.PATHS:
            raise ValueError(f"path must be one of {self.PATHS}")
        if path in ("fused_vt", "fused_vtq") and N > self.VT_MAX_TOKENS:
            raise ValueError(f"path '{path}' takes at most {self.VT_MAX_TOKENS} tokens; use 'fused_epilogue'")
        self.N, self.d_model, self.H, self.D, self.M, self.stga = N, d_model, H, D, M, stga
        self.path = path
        e = lambda *s, dt=BF16: torch.empty(*s, dtype=dt, device=device)  # noqa: E731
        self.group_id = e(N, dt=torch.int32)
        self.gate = e(N, dt=torch.float32)
        self.O = e(N, H, D)
        copies = path != "gather_on_load"
        self.Qp, self.Kp, self.Vp = (e(N, H, D) if copies else None for _ in range(3))
        self.Vt = None
        if path in ("fused_vt", "fused_vtq"):
            self.Vp, self.Vt = None, e(H, D, moga_vt_row_length(N))
        if path == "fused_vtq":
            self.Qp = None
        self.Op = e(N, H, D) if path == "separate" else None
        self.perm = e(N, dt=torch.int32)
        self.cu_seqlens = e(M + 1, dt=torch.int32)
        self.max_seqlen = e(1, dt=torch.int32)
        self.ws_perm = e(max(moga_workspace_bytes(MOGA_OP_PERMUTE, N, M, H, D), 1), dt=torch.uint8)
        self.ws_attn = e(max(moga_workspace_bytes(MOGA_OP_GROUP_ATTENTION, N, M, H, D), 1), dt=torch.uint8)
        self.shot_start = None
        if stga is not None and stga.get("shot_start") is not None:
            shots = list(stga["shot_start"])
            self.shot_start = torch.tensor(shots, dtype=torch.int32).to(device)
            self.ws_shot = e(max(moga_stga_shot_workspace_bytes(stga["T"], len(shots) - 1, stga["win_t"]), 1),
                             dt=torch.uint8)

    def __call__(self, X, Wr, Q, K, V, bias=None, softmax_scale=0.0, stga_weight=1.0, moga_weight=1.0):
        """O = moga_weight * MoGA + stga_weight * STGA (the STGA term only with
        geometry); with shots, O = (MoGA + shot STGA + per-frame) / 3."""
        moga_route(X, Wr, bias, self.group_id, self.gate)
        if self.path == "gather_on_load":
            moga_permute(self.group_id, self.M, perm=self.perm, cu_seqlens=self.cu_seqlens,
                         max_seqlen=self.max_seqlen, ws=self.ws_perm)
            moga_group_attention_fused(Q, K, V, self.cu_seqlens, self.perm, self.gate, softmax_scale, 0.0, self.O,
                                       self.ws_attn)
        elif self.path == "fused_vt":
            moga_permute_vt(self.group_id, self.M, Q, K, V, self.Qp, self.Kp, self.Vt, self.perm, self.cu_seqlens,
                            self.max_seqlen, self.ws_perm)
            moga_group_attention_unpermute_vt(self.Qp, self.Kp, self.Vt, self.cu_seqlens, self.perm, self.gate,
                                              softmax_scale, 0.0, self.O, self.ws_attn)
        elif self.path == "fused_vtq":
            moga_permute_vt(self.group_id, self.M, None, K, V, None, self.Kp, self.Vt, self.perm, self.cu_seqlens,
                            self.max_seqlen, self.ws_perm)
            moga_group_attention_unpermute_vtq(Q, self.Kp, self.Vt, self.cu_seqlens, self.perm, self.gate,
                                               softmax_scale, 0.0, self.O, self.ws_attn)
        else:
            moga_permute(self.group_id, self.M, Q, K, V, self.Qp, self.Kp, self.Vp, self.perm, self.cu_seqlens,
                         self.max_seqlen, self.ws_perm)
        if self.path == "fused_epilogue":
            moga_group_attention_unpermute(self.Qp, self.Kp, self.Vp, self.cu_seqlens, self.perm, self.gate,
                                           softmax_scale, 0.0, self.O, self.ws_attn)
        elif self.path == "separate":
            moga_group_attention(self.Qp, self.Kp, self.Vp, self.cu_seqlens, softmax_scale, self.Op, self.ws_attn)
            moga_unpermute(self.Op, self.perm, self.gate, 0.0, self.O)
        g = self.stga
        if g is None:
            if moga_weight != 1.0:
                raise ValueError("moga_weight applies only together with an STGA branch")
        elif self.shot_start is not None:
            third = 1.0 / 3.0
            # O = MoGA  ->  (MoGA + shot STGA) / 3  ->  + per-frame / 3
            moga_stga_shot_attention(Q, K, V, g["T"], g["Hs"], g["Ws"], self.shot_start, g["win_t"], g["tile_h"],
                                     g["tile_w"], g.get("augment", 1), softmax_scale, third, third, self.O,
                                     self.ws_shot)
            moga_stga_attention(Q, K, V, g["T"], g["Hs"], g["Ws"], 1, g["Hs"], g["Ws"], softmax_scale, third, 1.0,
                                self.O)
        else:
            moga_stga_attention(Q, K, V, g["T"], g["Hs"], g["Ws"], g["win_t"], g["tile_h"], g["tile_w"],
                                softmax_scale, stga_weight, moga_weight, self.O)
        return self.O


# ---------------------------------------------------------------------------
# Backward pass
# ---------------------------------------------------------------------------

F32 = torch.float32


def moga_group_attention_train(Qp, Kp, Vp, cu_seqlens, softmax_scale=0.0, Op=None, lse=None, ws=None):
    """moga_group_attention that also returns lse float32 [H, N] (natural-log
    log-sum-exp of each row's scaled scores, permuted rows)."""
    _need(Qp, "Qp", BF16, 3)
    N, H, D = Qp.shape
    _need(Kp, "Kp", BF16, 3, Qp.shape)
    _need(Vp, "Vp", BF16, 3, Qp.shape)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    M = cu_seqlens.shape[0] - 1
    Op = torch.empty_like(Qp) if Op is None else Op
    lse = torch.empty((H, N), dtype=F32, device=Qp.device) if lse is None else lse
    _need(Op, "Op", BF16, 3, Qp.shape)
    _need(lse, "lse", F32, 2, (H, N))
    ws, nbytes = _workspace(MOGA_OP_GROUP_ATTENTION, N, M, H, D, ws, Qp.device)
    check(_lib.LIB.moga_group_attention_train(ptr(Qp), ptr(Kp), ptr(Vp), ptr(cu_seqlens), N, H, D, M,
                                              float(softmax_scale), ptr(Op), ptr(lse), ptr(ws), nbytes,
                                              stream_handle()),
          "moga_group_attention_train")
    return Op, lse


def moga_unpermute_backward(dO, Op, perm, gate, dOp=None, delta=None, dgate=None):
    """(dOp bf16 [N, H, D] permuted, delta float32 [H, N], dgate float32 [N])."""
    _need(dO, "dO", BF16, 3)
    N, H, D = dO.shape
    _need(Op, "Op", BF16, 3, dO.shape)
    _need(perm, "perm", torch.int32, 1, (N,))
    _need(gate, "gate", F32, 1, (N,))
    dOp = torch.empty_like(dO) if dOp is None else dOp
    delta = torch.empty((H, N), dtype=F32, device=dO.device) if delta is None else delta
    dgate = torch.empty(N, dtype=F32, device=dO.device) if dgate is None else dgate
    _need(dOp, "dOp", BF16, 3, dO.shape)
    _need(delta, "delta", F32, 2, (H, N))
    _need(dgate, "dgate", F32, 1, (N,))
    check(_lib.LIB.moga_unpermute_backward(ptr(dO), ptr(Op), ptr(perm), ptr(gate), N, H, D, ptr(dOp), ptr(delta),
                                           ptr(dgate), stream_handle()),
          "moga_unpermute_backward")
    return dOp, delta, dgate


def moga_group_attention_backward(Qp, Kp, Vp, dOp, lse, delta, cu_seqlens, perm, softmax_scale=0.0, dQ=None,
                                  dK=None, dV=None, ws=None):
    """dQ, dK, dV bf16 [N, H, D] in original token order (through perm)."""
    _need(Qp, "Qp", BF16, 3)
    N, H, D = Qp.shape
    for name, t in (("Kp", Kp), ("Vp", Vp), ("dOp", dOp)):
        _need(t, name, BF16, 3, Qp.shape)
    _need(lse, "lse", F32, 2, (H, N))
    _need(delta, "delta", F32, 2, (H, N))
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _need(perm, "perm", torch.int32, 1, (N,))
    M = cu_seqlens.shape[0] - 1
    dQ = torch.empty_like(Qp) if dQ is None else dQ
    dK = torch.empty_like(Qp) if dK is None else dK
    dV = torch.empty_like(Qp) if dV is None else dV
    for name, t in (("dQ", dQ), ("dK", dK), ("dV", dV)):
        _need(t, name, BF16, 3, Qp.shape)
    ws, nbytes = _workspace(MOGA_OP_ATTENTION_BACKWARD, N, M, H, D, ws, Qp.device)
    check(_lib.LIB.moga_group_attention_backward(ptr(Qp), ptr(Kp), ptr(Vp), ptr(dOp), ptr(lse), ptr(delta),
                                                 ptr(cu_seqlens), ptr(perm), N, H, D, M, float(softmax_scale),
                                                 ptr(dQ), ptr(dK), ptr(dV), ptr(ws), nbytes, stream_handle()),
          "moga_group_attention_backward")
    return dQ, dK, dV


def moga_attention_backward_staged_bytes(cu_seqlens, H: int) -> int:
    """Workspace of moga_group_attention_backward that keeps dS for these
    groups (cu_seqlens int32 [M + 1], copied to the host if on the device)."""
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor")
    host = cu_seqlens.detach().to("cpu").contiguous()
    M = host.shape[0] - 1
    n = int(_lib.LIB.moga_attention_backward_staged_bytes(ctypes.c_void_p(host.data_ptr()), M, int(H)))
    if n == 0:
        raise ValueError("moga_attention_backward_staged_bytes: invalid cu_seqlens or H")
    return n


STAGED_FLAG_OFFSET = 2560  # MOGA_BWD_STAGED_FLAG_OFFSET in include/moga.h


def moga_attention_backward_staged(ws) -> int:
    """Heads whose dS the last moga_group_attention_backward on this
    workspace kept (reads the count the call leaves in ws; synchronises)."""
    if ws.numel() * ws.element_size() <= 4096:
        return 0
    return int(ws.view(torch.uint8)[STAGED_FLAG_OFFSET:STAGED_FLAG_OFFSET + 4].view(torch.int32).item())


def moga_route_backward(X, Wr, group_id, dgate, bias=None, dX=None, dWr=None, dbias=None, ws=None):
    """Router gradients (dX float32 [N, d_model], dWr float32 [M, d_model],
    dbias float32 [M]) from dgate."""
    _need(X, "X", BF16, 2)
    M, d = Wr.shape
    _need(Wr, "Wr", BF16, 2, (M, X.shape[1]))
    N = X.shape[0]
    _need(group_id, "group_id", torch.int32, 1, (N,))
    _need(dgate, "dgate", F32, 1, (N,))
    if bias is not None:
        _need(bias, "bias", F32, 1, (M,))
    dX = torch.empty((N, d), dtype=F32, device=X.device) if dX is None else dX
    dWr = torch.empty((M, d), dtype=F32, device=X.device) if dWr is None else dWr
    dbias = torch.empty(M, dtype=F32, device=X.device) if dbias is None else dbias
    _need(dX, "dX", F32, 2, (N, d))
    _need(dWr, "dWr", F32, 2, (M, d))
    _need(dbias, "dbias", F32, 1, (M,))
    ws, nbytes = _workspace(MOGA_OP_ROUTE_BACKWARD, N, M, 1, d, ws, X.device)
    check(_lib.LIB.moga_route_backward(ptr(X), ptr(Wr), ptr(bias), ptr(group_id), ptr(dgate), N, d, M, ptr(dX),
                                       ptr(dWr), ptr(dbias), ptr(ws), nbytes, stream_handle()),
          "moga_route_backward")
    return dX, dWr, dbias


class MogaTraining:
    """One MoGA layer for training: ``forward`` runs route -> permute (with
    gathered copies) -> attention that saves Op and lse -> gated unpermute and
    keeps what the backward needs; ``backward(dO)`` runs the unpermute,
    attention and router backward and returns the gradients of sum(O * dO)
    w.r.t. Q, K, V (bf16, original order), the router's share of dX, dWr and
    dbias (float32), plus dgate.  Buffers are allocated once.

    ``ds_bytes`` > 0 gives the attention backward a workspace of that many
    bytes, in which it keeps dS for as many heads as fit (all of them with
    ``moga_attention_backward_staged_bytes``): five matrix products instead
    of seven for those heads, for about sum_g n_g^2 * 2 bytes of device
    memory per head."""

    def __init__(self, N, d_model, H, D, M, device, ds_bytes=0):
        self.N, self.d_model, self.H, self.D, self.M = N, d_model, H, D, M
        e = lambda *s, dt=BF16: torch.empty(*s, dtype=dt, device=device)  # noqa: E731
        self.group_id, self.gate = e(N, dt=torch.int32), e(N, dt=F32)
        self.Qp, self.Kp, self.Vp, self.Op, self.O = (e(N, H, D) for _ in range(5))
        self.lse = e(H, N, dt=F32)
        self.perm, self.cu_seqlens, self.max_seqlen = e(N, dt=torch.int32), e(M + 1, dt=torch.int32), e(1, dt=torch.int32)
        self.ws_perm = e(max(moga_workspace_bytes(MOGA_OP_PERMUTE, N, M, H, D), 1), dt=torch.uint8)
        self.ws_attn = e(max(moga_workspace_bytes(MOGA_OP_GROUP_ATTENTION, N, M, H, D), 1), dt=torch.uint8)
        self.ws_bwd = e(max(moga_workspace_bytes(MOGA_OP_ATTENTION_BACKWARD, N, M, H, D), int(ds_bytes), 1),
                        dt=torch.uint8)
        self.ws_rbwd = e(max(moga_workspace_bytes(MOGA_OP_ROUTE_BACKWARD, N, M, 1, d_model), 1), dt=torch.uint8)
        self.dOp, self.delta, self.dgate = e(N, H, D), e(H, N, dt=F32), e(N, dt=F32)
        self.dQ, self.dK, self.dV = (e(N, H, D) for _ in range(3))
        self.dX, self.dWr, self.dbias = e(N, d_model, dt=F32), e(M, d_model, dt=F32), e(M, dt=F32)
        self.saved = None

    def forward(self, X, Wr, Q, K, V, bias=None, softmax_scale=0.0):
        moga_route(X, Wr, bias, self.group_id, self.gate)
        moga_permute(self.group_id, self.M, Q, K, V, self.Qp, self.Kp, self.Vp, self.perm, self.cu_seqlens,
                     self.max_seqlen, self.ws_perm)
        moga_group_attention_train(self.Qp, self.Kp, self.Vp, self.cu_seqlens, softmax_scale, self.Op, self.lse,
                                   self.ws_attn)
        moga_unpermute(self.Op, self.perm, self.gate, 0.0, self.O)
        self.saved = (X, Wr, bias, softmax_scale)
        return self.O

    def backward(self, dO):
        if self.saved is None:
            raise RuntimeError("backward before forward")
        X, Wr, bias, softmax_scale = self.saved
        moga_unpermute_backward(dO, self.Op, self.perm, self.gate, self.dOp, self.delta, self.dgate)
        moga_group_attention_backward(self.Qp, self.Kp, self.Vp, self.dOp, self.lse, self.delta, self.cu_seqlens,
                                      self.perm, softmax_scale, self.dQ, self.dK, self.dV, self.ws_bwd)
        moga_route_backward(X, Wr, self.group_id, self.dgate, bias, self.dX, self.dWr, self.dbias, self.ws_rbwd)
        return {"dQ": self.dQ, "dK": self.dK, "dV": self.dV, "dX": self.dX, "dWr": self.dWr, "dbias": self.dbias,
                "dgate": self.dgate}
