"""Seeded synthetic Q, K, V generators shared by the oracle side and the HIP side.

Both sides receive exactly the tensors produced here (the HIP side as bf16/fp32
device tensors, the oracle as the same values upcast to float64).  Nothing in
this module computes any part of the attention or the mask rule.

Recipe (seed = config number, NumPy PCG64 via ``default_rng``):

1. Q, K, V noise: three draws of ``standard_normal((B,H,N,d), float32)`` in that
   order.
2. Structure, added identically to Q, K and V on the video tokens (text tokens,
   the first ``n_text`` positions, get noise only):

   * ``lowrank``: per (b, h, frame) a rank-4 term ``U[F x 4] @ W[4 x d] / 2`` with
     U and W standard normal (F = tokens per frame).
   * ``smooth``: per (b, h, frame) a standard-normal field ``[Hs, Ws, d]`` blurred
     by a Gaussian of sigma 3 tokens over the two spatial axes (reflect borders,
     truncated at 4 sigma), rescaled per channel to unit standard deviation over
     the frame, then multiplied by 2.
3. Optional per-head multipliers (``q_head_scale``, ``v_head_scale``) scale head h of
   Q and of V after step 2, in float32.
4. Tokens are laid out as text first, then frames in raster order (row-major
   over ``Hs x Ws``).
5. bf16 configs round the float32 values to bf16 with round-to-nearest-even
   (``torch.Tensor.to(torch.bfloat16)``).
"""
from dataclasses import replace
from typing import Dict, Optional

import numpy as np
import torch
from scipy.ndimage import gaussian_filter

from .configs import Config


def scaled(cfg: Config, *, H: Optional[int] = None, frames: Optional[int] = None,
           n_text: Optional[int] = None, Hs: Optional[int] = None,
           Ws: Optional[int] = None, name_suffix: str = "_scaled") -> Config:
    """Return a smaller copy of ``cfg`` (fewer heads / frames / pixels)."""
    H = cfg.H if H is None else H
    frames = cfg.frames if frames is None else frames
    n_text = cfg.n_text if n_text is None else n_text
    Hs = cfg.Hs if Hs is None else Hs
    Ws = cfg.Ws if Ws is None else Ws
    N = n_text + frames * Hs * Ws
    pats = cfg.patterns
    if pats is not None and len(pats) != H:
        # keep the per-head pattern list proportional: cycle the original list
        pats = [cfg.patterns[(h * len(cfg.patterns)) // H] for h in range(H)]
    return replace(cfg, name=cfg.name + name_suffix, H=H, frames=frames,
                   n_text=n_text, Hs=Hs, Ws=Ws, N=N, patterns=pats)


def _structure(cfg: Config, rng: np.random.Generator) -> Optional[np.ndarray]:
    """Per-frame structured component, shape [B, H, frames*Hs*Ws, d] float32."""
    B, H, d = cfg.B, cfg.H, cfg.d
    F = cfg.Hs * cfg.Ws
    if cfg.structure == "none":
        return None
    if cfg.structure == "lowrank":
        U = rng.standard_normal((B, H, cfg.frames, F, 4), dtype=np.float32)
        W = rng.standard_normal((B, H, cfg.frames, 4, d), dtype=np.float32)
        comp = np.matmul(U, W) * np.float32(0.5)
        return comp.reshape(B, H, cfg.frames * F, d)
    if cfg.structure == "smooth":
        out = np.empty((B, H, cfg.frames, cfg.Hs, cfg.Ws, d), dtype=np.float32)
        for b in range(B):
            for h in range(H):
                fld = rng.standard_normal((cfg.frames, cfg.Hs, cfg.Ws, d), dtype=np.float32)
                fld = gaussian_filter(fld, sigma=(0, 3, 3, 0), mode="reflect", truncate=4.0)
                std = fld.std(axis=(1, 2), keepdims=True, dtype=np.float64)
                out[b, h] = (fld / std.astype(np.float32)) * np.float32(2.0)
        return out.reshape(B, H, cfg.frames * F, d)
    raise ValueError(f"unknown structure {cfg.structure!r}")


def make_inputs(cfg: Config) -> Dict[str, torch.Tensor]:
    """Q, K, V as contiguous CPU torch tensors [B,H,N,d] in the config's dtype."""
    assert cfg.N == cfg.n_text + cfg.frames * cfg.Hs * cfg.Ws, "token count mismatch"
    rng = np.random.default_rng(cfg.seed)
    shape = (cfg.B, cfg.H, cfg.N, cfg.d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    comp = _structure(cfg, rng)
    if comp is not None:
        t0 = cfg.n_text
        q[:, :, t0:] += comp
        k[:, :, t0:] += comp
        v[:, :, t0:] += comp
        del comp
    if cfg.q_head_scale is not None:
        q *= np.asarray(cfg.q_head_scale, dtype=np.float32)[None, :, None, None]
    if cfg.v_head_scale is not None:
        v *= np.asarray(cfg.v_head_scale, dtype=np.float32)[None, :, None, None]
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    return {name: torch.from_numpy(a).to(tdt).contiguous()
            for name, a in (("q", q), ("k", k), ("v", v))}


def as_float64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a bf16/fp32 CPU tensor to a float64 NumPy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()
