"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no attention arithmetic: it only draws random numbers and
arranges them into the shapes the attention path consumes.  Both the fp64
oracle and the HIP library receive the very same bf16 bytes from here.

Recipe: ``torch.Generator`` seeded with ``seed``, ``randn`` in fp32, rounded
to bf16 (round to nearest even, torch's conversion).  Q, K and V entries are
i.i.d. N(0, 1).  Sequence b of a configuration with seed s uses seed
``s * 16 + b``.  Within one sequence the draws happen in a fixed order: K
stream, V stream, then queries.
"""
from __future__ import annotations

import numpy as np
import torch

HQ, HKV, D, WINDOW = 32, 2, 128, 2048


def gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def randn_bf16(shape, seed=None, device="cpu", generator=None):
    """i.i.d. N(0,1) drawn in fp32 then rounded to bf16."""
    g = generator if generator is not None else gen(seed, device)
    return torch.randn(*shape, generator=g, device=device,
                       dtype=torch.float32).to(torch.bfloat16)


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def from_bits(a: np.ndarray) -> torch.Tensor:
    """numpy uint16 bit patterns -> bf16 tensor (host)."""
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)


def seq_seed(config_seed: int, b: int) -> int:
    return int(config_seed) * 16 + int(b)


def stream(seed: int, n: int, device="cpu"):
    """A logical K/V stream of n positions for one sequence and one layer:
    (k [n, HKV, D], v [n, HKV, D]) bf16, row r = position r."""
    g = gen(seed, device)
    k = randn_bf16((n, HKV, D), generator=g, device=device)
    v = randn_bf16((n, HKV, D), generator=g, device=device)
    return k, v


def queries(seed: int, n: int, hq=HQ, device="cpu"):
    """n query tokens [n, hq, D] bf16."""
    return randn_bf16((n, hq, D), seed=seed, device=device)


# --------------------------------------------------------------------------
# structured inputs for special cases (values chosen by hand, no arithmetic
# of the method)

def zeros_bf16(shape, device="cpu"):
    return torch.zeros(*shape, dtype=torch.bfloat16, device=device)


def constant_bf16(shape, value, device="cpu"):
    return torch.full(shape, float(value), dtype=torch.bfloat16, device=device)


def needle_stream(seed: int, n: int, needle_pos, direction_seed: int,
                  magnitude=8.0, device="cpu"):
    """A stream of small random keys plus, at each position in needle_pos,
    a key equal to ``magnitude`` times a fixed unit-ish direction u (per KV
    head).  Returns (k, v, u) with u [HKV, D] bf16; queries built from u
    score the needle keys far above the rest."""
    k, v = stream(seed, n, device)
    k = (k.float() * 0.05).to(torch.bfloat16)
    u = randn_bf16((HKV, D), seed=direction_seed, device=device)
    u = (u.float() / u.float().norm(dim=-1, keepdim=True) * 2.0).to(torch.bfloat16)
    for p in needle_pos:
        k[p] = (u.float() * magnitude).to(torch.bfloat16)
    return k, v, u
