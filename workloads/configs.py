"""The five synthetic workloads of the MoGA forward hot path.

Shapes follow the pages' workloads: Wan2.1 latent frames of 30 x 52 = 1560
tokens (480x832 video, VAE (4,8,8) and patchify (1,2,2), "Vanilla
Self-Attention" section of the MoGA explainer page), Wan2.1-1.3B attention
(d_model 1536, 12 heads of 128) and Wan2.1-14B attention (d_model 5120, 40
heads of 128), with 30-second (~190k tokens) and minute-scale (~580k tokens)
contexts.  Group counts, the mixture recipe and the STGA tile are those of the
workload definitions below.
"""

from __future__ import annotations

from dataclasses import dataclass, field

FRAME_H, FRAME_W = 30, 52  # latent tokens per frame: 30 x 52 = 1560


@dataclass(frozen=True)
class Workload:
    name: str
    N: int
    d_model: int
    H: int
    D: int
    M: int
    mixture: str            # "none", "equal" (equal weights, random targets) or "zipf"
    n_components: int
    zipf_s: float = 1.1
    gamma: float = 0.0      # strength of the router-prototype direction in a token
    sigma2: float = 0.5     # per-token noise variance (content mean gets 1 - sigma2)
    stga: dict | None = field(default=None)
    seed: int = 1000
    bf16: bool = True

    @property
    def frames(self) -> int:
        return self.N // (FRAME_H * FRAME_W)


# gamma: calibrated once on the 30-second workload so that the largest group is
# about 4x the mean group size, then kept for the other Zipf workloads.
GAMMA_ZIPF = 1.75
GAMMA_EQUAL = 1.75

WORKLOADS = {
    "tiny": Workload("tiny", N=2048, d_model=128, H=2, D=64, M=4, mixture="none",
                     n_components=0, seed=1001),
    "wan13b_21f": Workload("wan13b_21f", N=21 * 1560, d_model=1536, H=12, D=128, M=8,
                           mixture="equal", n_components=16, gamma=GAMMA_EQUAL, seed=1002),
    "clip30s_122f": Workload("clip30s_122f", N=122 * 1560, d_model=1536, H=12, D=128, M=16,
                             mixture="zipf", n_components=16, gamma=GAMMA_ZIPF, seed=1003),
    "wan14b_122f": Workload("wan14b_122f", N=122 * 1560, d_model=5120, H=40, D=128, M=16,
                            mixture="zipf", n_components=16, gamma=GAMMA_ZIPF, seed=1004),
    "minute_372f": Workload("minute_372f", N=372 * 1560, d_model=1536, H=12, D=128, M=32,
                            mixture="zipf", n_components=32, gamma=GAMMA_ZIPF, seed=1005,
                            stga=dict(T=372, Hs=FRAME_H, Ws=FRAME_W, win_t=3, tile_h=30, tile_w=26)),
}

# The workload the benchmark line is quoted on (N ~ 190k, Wan2.1-1.3B shape).
BENCH_WORKLOAD = "clip30s_122f"


def get_workload(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; choose from {sorted(WORKLOADS)}") from None
