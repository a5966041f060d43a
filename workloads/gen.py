"""Seeded synthetic inputs for the MoGA forward hot path (torch, any device).

Recipe:
  * W_r ~ N(0, 1/d_model) with shape [M, d_model]; W_q, W_k, W_v ~ N(0, 1/d_model)
    with shape [d_model, H*D].
  * Tokens: "none" -> x ~ N(0, I).  Mixtures -> x_n = gamma * w_hat[pi(k_n)]
    + mu_perp[k_n] + sqrt(sigma2) * eps_n, where w_hat[i] is router row i
    scaled to unit norm (a trained router's prototype sitting on a cluster),
    mu_perp[k] ~ N(0, (1 - sigma2) I) with its part inside the span of W_r's
    rows removed, eps_n ~ N(0, I), and the component k_n is drawn with weights
    proportional to k^-s ("zipf") or uniform ("equal", each component then
    pointing at a random group, so several can share one).
  * X is rounded to bf16; Q, K, V = bf16(X @ W_{q,k,v}) computed in float32.
  * Margin screen: every token's top-1 minus top-2 router score, computed in
    float64 from the bf16 values, must be at least 1e-4; tokens below it get a
    fresh noise draw until they pass.  This keeps the hard assignment a
    well-posed integer decision for any float32 summation order.

The generator draws random numbers and does this screening only; it holds no
routing decision, sort, attention or gate of the method itself.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

from .configs import Workload

MARGIN_MIN = 1e-4


def _gen(device, seed: int, stream: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + stream)
    return g


def top2_margin(Xb: torch.Tensor, Wr: torch.Tensor, chunk: int = 65536) -> torch.Tensor:
    """float64 top-1 minus top-2 router score per token (inf when M == 1)."""
    N, M = Xb.shape[0], Wr.shape[0]
    if M == 1:
        return torch.full((N,), math.inf, dtype=torch.float64, device=Xb.device)
    W = Wr.double()
    out = torch.empty(N, dtype=torch.float64, device=Xb.device)
    for s in range(0, N, chunk):
        r = Xb[s:s + chunk].double() @ W.T
        top = torch.topk(r, 2, dim=1).values
        out[s:s + chunk] = top[:, 0] - top[:, 1]
    return out


def _project(Xb: torch.Tensor, W: torch.Tensor, H: int, D: int, chunk: int = 32768) -> torch.Tensor:
    N = Xb.shape[0]
    out = torch.empty((N, H * D), dtype=torch.bfloat16, device=Xb.device)
    Wf = W.float()
    for s in range(0, N, chunk):
        out[s:s + chunk] = (Xb[s:s + chunk].float() @ Wf).bfloat16()
    return out.view(N, H, D)


def make_inputs(wl: Workload, device="cpu", seed: int | None = None, **overrides) -> dict:
    """Draw one workload's inputs.  ``overrides`` replace Workload fields
    (e.g. N=..., H=... for smaller cases of the same recipe).

    Returns torch tensors on ``device``: X [N, d_model], Wr [M, d_model],
    Q, K, V [N, H, D] (all bf16) and the mixture labels (int64 [N] or None).
    """
    if overrides:
        wl = dataclasses.replace(wl, **overrides)
    seed = wl.seed if seed is None else seed
    N, d, H, D, M = wl.N, wl.d_model, wl.H, wl.D, wl.M
    dev = torch.device(device)
    sd = 1.0 / math.sqrt(d)

    Wr = (torch.randn(M, d, generator=_gen(dev, seed, 1), device=dev) * sd).bfloat16()
    Wq = (torch.randn(d, H * D, generator=_gen(dev, seed, 2), device=dev) * sd).bfloat16()
    Wk = (torch.randn(d, H * D, generator=_gen(dev, seed, 3), device=dev) * sd).bfloat16()
    Wv = (torch.randn(d, H * D, generator=_gen(dev, seed, 4), device=dev) * sd).bfloat16()

    labels = None
    sig = math.sqrt(wl.sigma2)
    if wl.mixture == "none":
        base = torch.zeros((1, d), device=dev)
        X = torch.randn(N, d, generator=_gen(dev, seed, 5), device=dev)
        noise_scale = 1.0
    else:
        Kc = wl.n_components
        if wl.mixture == "zipf":
            w = torch.arange(1, Kc + 1, dtype=torch.float64, device=dev) ** (-wl.zipf_s)
            pi = torch.arange(Kc, device=dev) % M
        elif wl.mixture == "equal":
            w = torch.ones(Kc, dtype=torch.float64, device=dev)
            pi = torch.randint(0, M, (Kc,), generator=_gen(dev, seed, 6), device=dev)
        else:
            raise ValueError(f"unknown mixture {wl.mixture!r}")
        W64 = Wr.double()
        mu = torch.randn(Kc, d, generator=_gen(dev, seed, 7), device=dev).double() * math.sqrt(1.0 - wl.sigma2)
        # remove the part of each content mean that lies in the span of W_r's rows
        coef = torch.linalg.solve(W64 @ W64.T, W64 @ mu.T)          # [M, Kc]
        mu = mu - (W64.T @ coef).T
        w_hat = W64 / W64.norm(dim=1, keepdim=True)
        centers = (wl.gamma * w_hat[pi] + mu).float()                  # [Kc, d]
        labels = torch.multinomial((w / w.sum()).float(), N, replacement=True,
                                   generator=_gen(dev, seed, 8))
        base = centers
        X = torch.randn(N, d, generator=_gen(dev, seed, 9), device=dev) * sig
        X += centers[labels]
        noise_scale = sig
    Xb = X.bfloat16()
    del X

    # margin screen: redraw the noise of tokens whose top-1 margin is too small
    for attempt in range(1, 64):
        bad = torch.nonzero(top2_margin(Xb, Wr) < MARGIN_MIN).flatten()
        if bad.numel() == 0:
            break
        fresh = torch.randn(bad.numel(), d, generator=_gen(dev, seed, 100 + attempt), device=dev) * noise_scale
        fresh += base[labels[bad]] if labels is not None else base
        Xb[bad] = fresh.bfloat16()
    else:
        raise RuntimeError("margin screen did not converge")

    Q = _project(Xb, Wq, H, D)
    K = _project(Xb, Wk, H, D)
    V = _project(Xb, Wv, H, D)
    return {"X": Xb, "Wr": Wr, "Q": Q, "K": K, "V": V, "labels": labels, "workload": wl, "seed": seed}


def make_shots(T: int, seed: int, min_len: int = 12, max_len: int = 60) -> list:
    """Seeded multi-shot layout of T latent frames: shot lengths drawn
    uniformly from [min_len, max_len] latent frames (about 2 to 10 seconds at
    the 4x temporal compression of a 24 fps video), the last shot cut at T.
    Returns the shot start frames followed by T (n_shots + 1 values)."""
    rng = np.random.default_rng(seed * 1000 + 11)
    starts = [0]
    while starts[-1] < T:
        starts.append(min(T, starts[-1] + int(rng.integers(min_len, max_len + 1))))
    return starts


def to_numpy_f32(t: torch.Tensor) -> np.ndarray:
    """Exact float32 copy of a bf16/float tensor on the host."""
    return t.detach().float().cpu().numpy()


def sample_rows(group_id: np.ndarray, M: int, per_group: int, seed: int) -> np.ndarray:
    """Stratified sample of ORIGINAL token rows: in every non-empty group the
    first and last token plus up to ``per_group`` random ones (sorted, unique)."""
    rng = np.random.default_rng(seed)
    g = np.asarray(group_id)
    picks = []
    for i in range(M):
        members = np.nonzero(g == i)[0]
        if members.size == 0:
            continue
        picks += [members[0], members[-1]]
        k = min(per_group, members.size)
        picks += list(rng.choice(members, size=k, replace=False))
    return np.unique(np.asarray(picks, dtype=np.int64))
