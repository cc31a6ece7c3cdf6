"""Workload descriptions: shapes, input kind and the selection rule's parameters.

Selection parameters are stored the way the method states them (a keep
fraction, a threshold), never as integer counts: each side turns a fraction
into a count itself.
"""

from dataclasses import dataclass
from fractions import Fraction
from typing import Optional, Tuple


@dataclass(frozen=True)
class Spec:
    """One synthetic workload.

    cfg_id  seeds every random stream of the workload (see generate.py)
    B, H, N, d, block   batch, heads, tokens, head dim, block (tile) size
    kind    "iid" (Q, K, V drawn N(0,1)) or "fourier" (low-frequency fields
            over a (t, y, x) token grid plus 0.3 N(0,1) noise)
    grid    (T, Y, X) with T*Y*X == N, tokens in raster order; fourier only
    mode    "topk" | "cdf" | "sla3" | "maskin"
    keep    critical fraction of key blocks per query block (topk, sla3, maskin)
    marg    fraction of key blocks that are marginal, taken right after the
            critical ones in score order (sla3, maskin); None when no linear branch
    thr     NABLA threshold; blocks are kept until the pooled-softmax mass
            reaches 1 - thr (cdf)
    """

    cfg_id: int
    name: str
    B: int
    H: int
    N: int
    d: int
    block: int
    kind: str
    grid: Optional[Tuple[int, int, int]] = None
    mode: str = "topk"
    keep: Optional[Fraction] = None
    marg: Optional[Fraction] = None
    thr: Optional[float] = None

    def __post_init__(self):
        if self.kind not in ("iid", "fourier"):
            raise ValueError(f"unknown kind {self.kind!r}")
        if self.kind == "fourier":
            if self.grid is None or self.grid[0] * self.grid[1] * self.grid[2] != self.N:
                raise ValueError("fourier inputs need a (T, Y, X) grid with T*Y*X == N")
        if self.mode not in ("topk", "cdf", "sla3", "maskin"):
            raise ValueError(f"unknown mode {self.mode!r}")

    @property
    def nb(self) -> int:
        return -(-self.N // self.block)


F = Fraction

CONFIGS = {
    # 1024-token toy: i.i.d. N(0,1), 16x16 block grid, top 4 key blocks (25%).
    "tiny": Spec(1, "tiny", B=1, H=2, N=1024, d=64, block=64, kind="iid",
                 mode="topk", keep=F(1, 4)),
    # Short video latent, 4 x 32 x 64 tokens, NABLA cut with thr = 0.1.
    "short_video": Spec(2, "short_video", B=1, H=12, N=8192, d=64, block=64, kind="fourier",
                        grid=(4, 32, 64), mode="cdf", thr=0.1),
    # Wan-1.3B-like layer, 21 x 30 x 52 tokens: top 5% critical, next 15% marginal.
    "wan1p3b": Spec(3, "wan1p3b", B=1, H=12, N=32760, d=128, block=128, kind="fourier",
                    grid=(21, 30, 52), mode="sla3", keep=F(5, 100), marg=F(15, 100)),
    # Wan-14B-like layer, 21 x 45 x 80 tokens, top-k key tiles at 95% sparsity.
    "wan14b": Spec(4, "wan14b", B=1, H=40, N=75600, d=128, block=128, kind="fourier",
                   grid=(21, 45, 80), mode="topk", keep=F(5, 100)),
    # Long clip, 60 x 64 x 64 tokens, mask given as input: per-head top-k at
    # 95% (a) and 90% (b) sparsity, plus the next 5% of tiles on the linear
    # branch.  Both variants use the same data (same cfg_id).
    "long_clip_95": Spec(5, "long_clip_95", B=1, H=40, N=245760, d=128, block=128, kind="fourier",
                         grid=(60, 64, 64), mode="maskin", keep=F(5, 100), marg=F(5, 100)),
    "long_clip_90": Spec(5, "long_clip_90", B=1, H=40, N=245760, d=128, block=128, kind="fourier",
                         grid=(60, 64, 64), mode="maskin", keep=F(10, 100), marg=F(5, 100)),
}


def spec_for(name: str) -> Spec:
    return CONFIGS[name]
