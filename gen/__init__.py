"""Seeded synthetic inputs and workload configurations (no method arithmetic)."""
from .configs import (ADAPTIVE, FULL, SKIP, DIAG, MULTIDIAG, VSTRIPE, FRAME_TILE, TOPK, TAU,
                      Config, TINY, STATIC, COGVIDEOX, WAN, LONG720, ALL, BY_NAME)
from .inputs import make_inputs, as_float64, scaled
