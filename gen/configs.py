"""Workload configurations (shapes, mask parameters, generator recipe).

The five layer shapes below are synthetic stand-ins for attention layers of the
video DiTs named on the pages (CogVideoX-5B and Wan2.1-1.3B in the BLADE
abstract; a 720p Wan-like layer for long sequences).  The pages print no model
shapes, so the sizes are specification choices, not page values.

This module holds only numbers.  It contains none of the method's arithmetic:
the oracle and the HIP path each compute the mask and the attention themselves.

Mask-source ids and adaptive modes use the same integer codes as the C ABI
(``include/asa.h``); both sides define them on their own.
"""
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

# pattern ids (Sparse-vDiT, "四种注意力模式" table: M0 full, M1 skip, M2 diagonal,
# M3 multi-diagonal, M4 vertical stripe; 0 = the adaptive ASA source)
ADAPTIVE, FULL, SKIP, DIAG, MULTIDIAG, VSTRIPE, FRAME_TILE = 0, 1, 2, 3, 4, 5, 6
TOPK, TAU = 0, 1


@dataclass
class Config:
    name: str
    seed: int
    B: int
    H: int
    N: int
    d: int
    blk: int
    dtype: str                      # "f32" or "bf16" (input dtype)
    frames: int
    Hs: int                         # latent frame height (tokens)
    Ws: int                         # latent frame width (tokens)
    n_text: int = 0                 # leading text tokens (noise only)
    structure: str = "none"         # "none" | "lowrank" | "smooth"
    # mask
    kind: str = "adaptive"          # "adaptive" | "static"
    mode: int = TOPK
    k: int = 0
    tau: float = 0.0
    k_cap: int = 0
    keep_diag: int = 1
    patterns: Optional[List[Tuple[int, int]]] = None   # per head (id, param)
    target_density: Optional[float] = None              # for tuned top-k
    # per-head multipliers of the generated Q and V (None = 1 for every head); they spread
    # the heads over the regimes the pattern search tells apart
    q_head_scale: Optional[List[float]] = None
    v_head_scale: Optional[List[float]] = None
    notes: str = ""

    @property
    def Nb(self) -> int:
        return (self.N + self.blk - 1) // self.blk

    def head_patterns(self) -> List[Tuple[int, int]]:
        if self.patterns is None:
            return [(ADAPTIVE, 0)] * self.H
        return list(self.patterns)


# Config 1: tiny adaptive case, fp32, finishes in well under a second on the oracle.
TINY = Config(
    name="tiny_asa_fp32", seed=1, B=1, H=2, N=1024, d=64, blk=64, dtype="f32",
    frames=4, Hs=16, Ws=16, structure="none",
    kind="adaptive", mode=TOPK, k=4, keep_diag=1,
    notes="Q,K,V ~ N(0,1); top-4 of 16 key blocks plus the diagonal",
)

# Config 2: static Sparse-vDiT patterns, one per head pair.
STATIC = Config(
    name="static_patterns_bf16", seed=2, B=1, H=8, N=8192, d=64, blk=128, dtype="bf16",
    frames=8, Hs=32, Ws=32, structure="lowrank",
    kind="static",
    patterns=[(DIAG, 0), (DIAG, 0), (MULTIDIAG, 1024), (MULTIDIAG, 1024),
              (VSTRIPE, 2), (VSTRIPE, 2), (FULL, 0), (SKIP, 0)],
    notes="stride 1024 tokens = one 32x32 frame; vertical stripe = first 2 key blocks",
)

# Config 3: CogVideoX-5B-shaped layer: 226 text tokens + 13 frames of 30x45.
COGVIDEOX = Config(
    name="cogvideox5b_layer", seed=3, B=1, H=48, N=17776, d=64, blk=128, dtype="bf16",
    frames=13, Hs=30, Ws=45, n_text=226, structure="smooth",
    kind="adaptive", mode=TAU, tau=0.9, k_cap=34, keep_diag=1,
    notes="cumulative-mass 0.9, adaptive prefix capped at floor(0.25*139)=34 blocks, text rows/cols kept",
)

# Config 4: Wan2.1-1.3B-shaped layer: 21 frames of 30x52 (the metric workload).
# k is the top-k whose realized density (top-k plus diagonal, oracle mask at
# seed 4) is closest to 10 %; a CPU test recomputes it from the oracle.
WAN = Config(
    name="wan21_1p3b_layer", seed=4, B=1, H=12, N=32760, d=128, blk=128, dtype="bf16",
    frames=21, Hs=30, Ws=52, structure="smooth",
    kind="adaptive", mode=TOPK, k=26, keep_diag=1, target_density=0.10,
    notes="top-k tuned to 10% density",
)

# Config 5: long 720p-like layer: 21 frames of 45x80; adaptive at 5 % combined with
# a multi-diagonal static mask of stride 3600 tokens (one frame); heads 22-23 skipped.
LONG720 = Config(
    name="long720p_layer", seed=5, B=1, H=24, N=75600, d=128, blk=128, dtype="bf16",
    frames=21, Hs=45, Ws=80, structure="smooth",
    kind="adaptive", mode=TOPK, k=30, keep_diag=1, target_density=0.05,
    patterns=[(MULTIDIAG, 3600)] * 22 + [(SKIP, 0), (SKIP, 0)],
    notes="adaptive density measured before the multi-diagonal union",
)

ALL = [TINY, STATIC, COGVIDEOX, WAN, LONG720]
BY_NAME = {c.name: c for c in ALL}
