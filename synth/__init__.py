"""Seeded synthetic inputs for the Graph Machine sparse-layer path.

This module only draws random inputs.  It holds none of the arithmetic of
sparse edge referral (SER) or sparse edge attention (SEA): both the oracle and
the HIP path receive what it returns and compute on their own.

Recipe (page "Graph Machine: Towards Better Pretraining via Edges", ai.info,
sections "Key Contributions" 2-3 and "Methodology in Plain English"; the
pages publish no activations or edge tensors, so the shapes follow a
Qwen3-0.6B-like layer and the distributions are plain readings):

* Edge tensors are ``idx[B, n, Hkv, s]`` int32 and ``w[B, n, Hkv, s]`` fp32,
  one row of ``s`` slots per (sequence, token, KV head).  Every index is
  causal: ``0 <= idx[b, i, h, t] <= i``.
* ``mode="uniform"``: every slot is uniform on ``{0..i}`` (token 0 points to
  itself).
* ``mode="mixed"``: even slots are "local", uniform on the preceding
  ``window`` positions ``{max(0, i-window) .. i-1}`` (0 for token 0); odd
  slots are "far", uniform on ``{0..i}``.
* Weights are the softmax over the ``s`` slots of N(0, 2^2) logits, computed
  in float64 and stored as fp32, so every weight is positive and a row sums
  to 1 (up to the fp32 rounding).
* q, k, v and the upstream gradient are N(0, 1).  bf16 tensors are the
  round-to-nearest-even bf16 of an fp32 sample.

Streams: every tensor has its own numpy ``PCG64`` stream keyed by
``(seed, tensor id + 16 * layer)``; on a GPU device torch's seeded Philox
generator is used instead (only for shapes too large to draw on the host
quickly; the oracle then receives the downloaded tensor).
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

BASE_SEED = 20260902
TENSOR_ID = {"q": 1, "k": 2, "v": 3, "dout": 4, "idx": 5, "wlogit": 6}
LAYER_STRIDE = 16


def _stream(seed: int, name: str, layer: int) -> list[int]:
    return [int(seed), TENSOR_ID[name] + LAYER_STRIDE * int(layer)]


def edges(seed: int, B: int, n: int, hkv: int, s: int, mode: str = "mixed",
          layer: int = 0, window: int = 64, logit_std: float = 2.0):
    """Return ``(idx int32 [B,n,hkv,s], w float32 [B,n,hkv,s])`` as numpy."""
    if mode not in ("uniform", "mixed"):
        raise ValueError(f"unknown edge mode {mode!r}")
    rng = np.random.default_rng(_stream(seed, "idx", layer))
    i = np.arange(n, dtype=np.int64).reshape(1, n, 1, 1)
    u = rng.random((B, n, hkv, s))
    far = np.floor(u * (i + 1)).astype(np.int64)          # uniform on {0..i}
    far = np.minimum(far, i)
    if mode == "uniform":
        idx = far
    else:
        span = np.minimum(i, window)                        # |{max(0,i-w)..i-1}|
        local = i - 1 - np.floor(u * span).astype(np.int64)
        local = np.where(i == 0, 0, np.clip(local, np.maximum(i - window, 0), i))
        slot = np.arange(s).reshape(1, 1, 1, s)
        idx = np.where(slot % 2 == 0, local, far)
    wr = np.random.default_rng(_stream(seed, "wlogit", layer))
    logits = wr.standard_normal((B, n, hkv, s)) * logit_std
    logits -= logits.max(axis=-1, keepdims=True)
    e = np.exp(logits)
    w = (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)
    return idx.astype(np.int32), w


def normal(seed: int, name: str, shape, dtype=torch.float32, layer: int = 0,
           device="cpu") -> torch.Tensor:
    """N(0,1) tensor of ``shape`` in ``dtype`` (bf16 = RNE of an fp32 draw)."""
    device = torch.device(device)
    if device.type == "cpu":
        rng = np.random.default_rng(_stream(seed, name, layer))
        x = torch.from_numpy(rng.standard_normal(tuple(shape), dtype=np.float32))
    else:
        g = torch.Generator(device=device)
        s = _stream(seed, name, layer)
        g.manual_seed((s[0] * 1_000_003 + s[1]) & ((1 << 63) - 1))
        x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return x.to(dtype)


@dataclasses.dataclass(frozen=True)
class Preset:
    """One named workload: shapes, edge recipe and which stages run."""
    name: str
    B: int
    n: int
    hq: int
    hkv: int
    d: int
    dtype: torch.dtype
    s1: int
    s2: int
    s3: int
    mode: str
    seed: int
    ser: bool          # run SER (A' = Sparsify_s1(A A)) before SEA
    backward: bool     # run SEA and SER backward
    layers: int = 1    # sparse layers in a stack (edges carried between them)
    ser_steps: int = 1 # chained SER steps per layer

    @property
    def units(self) -> int:
        return self.B * self.n * self.hkv

    @property
    def s_in(self) -> int:
        """Width of the stored edge rows fed to the first stage."""
        return self.s2 if self.ser else self.s1


PRESETS = {
    p.name: p for p in [
        # batch 1, n=64, 4 q / 2 KV heads, d=16, fp32, s1=s2=s3=2, every slot
        # uniform on [0, i]; one SER step then SEA forward and backward.
        Preset("tiny", 1, 64, 4, 2, 16, torch.float32, 2, 2, 2, "uniform",
               BASE_SEED + 0, ser=True, backward=True),
        # SEA forward only, Qwen3-0.6B-like layer, s1=2, local/far mix.
        Preset("sea2", 8, 4096, 16, 8, 128, torch.bfloat16, 2, 2, 2, "mixed",
               BASE_SEED + 1, ser=False, backward=False),
        # SER (top-4 of 16 two-hop candidates) then SEA forward.
        Preset("ser_sea4", 8, 4096, 16, 8, 128, torch.bfloat16, 4, 4, 4, "mixed",
               BASE_SEED + 2, ser=True, backward=False),
        # 21 sparse layers, each two chained SER steps then SEA forward.
        Preset("stack21", 32, 4096, 16, 8, 128, torch.bfloat16, 4, 4, 4, "mixed",
               BASE_SEED + 3, ser=True, backward=False, layers=21, ser_steps=2),
        # long context forward + backward.
        Preset("long64k", 1, 65536, 16, 8, 128, torch.bfloat16, 4, 4, 4, "mixed",
               BASE_SEED + 4, ser=True, backward=True),
        # the measured layer pass: ser_sea4's shape plus both backwards.
        Preset("metric", 8, 4096, 16, 8, 128, torch.bfloat16, 4, 4, 4, "mixed",
               BASE_SEED + 2, ser=True, backward=True),
        # the narrower budget (s1, s2, s3) = (2, 4, 4): top-2 of 16 two-hop
        # candidates, then SEA at s1 = 2; the metric pass's shape otherwise.
        Preset("theia", 8, 4096, 16, 8, 128, torch.bfloat16, 2, 4, 4, "mixed",
               BASE_SEED + 5, ser=True, backward=True),
        # the measured pass at other head shapes and in fp32 (the general
        # SEA kernels: rows other than 256 bytes)
        Preset("d64", 8, 4096, 16, 8, 64, torch.bfloat16, 4, 4, 4, "mixed",
               BASE_SEED + 6, ser=True, backward=True),
        Preset("d256", 8, 4096, 16, 8, 256, torch.bfloat16, 4, 4, 4, "mixed",
               BASE_SEED + 7, ser=True, backward=True),
        Preset("fp32", 8, 4096, 16, 8, 128, torch.float32, 4, 4, 4, "mixed",
               BASE_SEED + 8, ser=True, backward=True),
    ]
}
