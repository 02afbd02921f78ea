"""Seeded synthetic workloads shared by the tests, the bench and the smoke check.

This module only draws and rounds inputs; it holds none of the attention
arithmetic.  Every array is produced on the host with numpy's PCG64, so the
GPU path and the fp64 oracle consume bit-identical values:

* q and k are standard-normal draws, L2-normalised per row in fp64 (the
  caller-side prerequisite), then rounded to the working dtype;
* v is standard normal, rounded to the working dtype;
* "bf16" inputs are rounded fp64 -> fp32 (round-to-nearest-even) -> bf16
  (round-to-nearest-even), which is what ``torch.Tensor.to(torch.bfloat16)``
  does to an fp32 tensor.

The oracle receives the fp64 upcast of the *rounded* values.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Tuple

import numpy as np


# ---------------------------------------------------------------------------
# dtype rounding
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    NaN maps to a quiet NaN; +-Inf and finite overflow behave as IEEE RNE.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r = r.copy()
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp32 values."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Rounded:
    """One input tensor in its working dtype plus its exact fp64 value.

    ``device`` is what goes to the GPU: float32 array, or uint16 bf16 bits.
    ``exact`` is the fp64 upcast of the rounded value (what the oracle eats).
    """
    dtype: str
    device: np.ndarray
    exact: np.ndarray


def round_to(x64: np.ndarray, dtype: str) -> Rounded:
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return Rounded("f32", x32, x32.astype(np.float64))
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x32)
        return Rounded("bf16", bits, bf16_bits_to_f32(bits).astype(np.float64))
    raise ValueError(f"unknown dtype {dtype!r}")


def l2_normalise(x: np.ndarray) -> np.ndarray:
    """Row-wise L2 normalisation in fp64 (the caller-side precondition)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


# ---------------------------------------------------------------------------
# Draws
# ---------------------------------------------------------------------------

def draw_qkv(seed, B: int, H: int, N: int, dk: int, dv: int, dtype: str,
             normalise: bool = True) -> Tuple[Rounded, Rounded, Rounded]:
    """q, then k, then v, each standard normal in its full shape; q and k
    L2-normalised per row; all rounded to ``dtype``."""
    g = np.random.Generator(np.random.PCG64(seed))
    q = g.standard_normal((B, H, N, dk))
    k = g.standard_normal((B, H, N, dk))
    v = g.standard_normal((B, H, N, dv))
    if normalise:
        q, k = l2_normalise(q), l2_normalise(k)
    return round_to(q, dtype), round_to(k, dtype), round_to(v, dtype)


def draw_prefix_kv(b: int, h: int, N: int, dk: int, dv: int, part: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Decode-workload prefix of one (b, h): k then v, PCG64([2, b, h])
    (PCG64([2, b, h, part]) for a further part of the prefix, part >= 1);
    k normalised; both rounded to fp32 and returned as fp64 values."""
    g = np.random.Generator(np.random.PCG64([2, b, h] if part == 0 else [2, b, h, part]))
    k = l2_normalise(g.standard_normal((N, dk)))
    v = g.standard_normal((N, dv))
    return (k.astype(np.float32).astype(np.float64),
            v.astype(np.float32).astype(np.float64))


def draw_decode_token(t: int, B: int, H: int, dk: int, dv: int, dtype: str = "f32"
                      ) -> Tuple[Rounded, Rounded, Rounded]:
    """Inputs of decode step t for all (b, h): PCG64([2, 1<<20, t]); q, k, v."""
    g = np.random.Generator(np.random.PCG64([2, 1 << 20, t]))
    q = l2_normalise(g.standard_normal((B, H, dk)))
    k = l2_normalise(g.standard_normal((B, H, dk)))
    v = g.standard_normal((B, H, dv))
    return round_to(q, dtype), round_to(k, dtype), round_to(v, dtype)


def draw_split_points(N: int, count: int = 7, seed=(4, 7)) -> List[int]:
    """``count`` distinct cut points drawn uniformly from 1 .. N-1, sorted."""
    g = np.random.Generator(np.random.PCG64(list(seed)))
    cuts = g.choice(np.arange(1, N), size=count, replace=False)
    return sorted(int(c) for c in cuts)


# ---------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill" or "decode"
    B: int
    H: int
    N: int               # prefill length, or prefix length for decode
    dk: int
    dv: int
    n: int
    chunk: int
    dtype: str           # GPU input dtype: "f32" or "bf16"
    seed: int
    steps: int = 0       # decode steps
    extra: Dict = field(default_factory=dict)

    @property
    def tol(self) -> Tuple[str, float]:
        """("rel", 1e-5) on fp32 paths, ("abs", 5e-3) on bf16-input paths."""
        return ("rel", 1e-5) if self.dtype == "f32" else ("abs", 5e-3)


WORKLOADS: Dict[str, Workload] = {
    # single sequence, one head; the oracle finishes in seconds
    "tiny": Workload("tiny N256 dk16 dv64 n3 f32", "prefill", 1, 1, 256, 16, 64, 3, 64, "f32", 0),
    # the prefill workload the headline tokens/s is quoted on
    "prefill": Workload("prefill B4 H8 N8192 dk16 dv64 n3 bf16", "prefill", 4, 8, 8192, 16, 64, 3, 64, "bf16", 1),
    # the decode workload the headline us/step is quoted on
    "decode": Workload("decode B64 H32 dk16 dv64 n3 f32 prefix65536 x256 steps", "decode",
                       64, 32, 65536, 16, 64, 3, 0, "f32", 2, steps=256),
    "order5": Workload("prefill B1 H16 N16384 dk16 dv64 n5 f32", "prefill", 1, 16, 16384, 16, 64, 5, 64, "f32", 3),
    "wide": Workload("prefill B1 H16 N65536 dk64 dv64 n3 bf16", "prefill", 1, 16, 65536, 64, 64, 3, 64, "bf16", 4,
                     extra={"splits": 8}),
}
