"""Seeded synthetic inputs for the SageBwd attention path.

This module only draws random numbers and rounds them to bfloat16. It holds
none of the attention method's arithmetic, so both the HIP path (through its
tests and the benchmark) and the CPU oracle can take their inputs from here
without sharing any computation.

Workloads stand in for the ones the SageBwd pages measure on (Llama-1B
training at 8K/16K tokens, a ~400M pretraining model, CogVideoX layers); the
datasets and checkpoints themselves are not used. Shapes and distributions:

  tiny        B1 H2  N128   non-causal  Q,K,V,dO ~ N(0,1)
  pretrain    B8 H16 N2048  causal      Q,K ~ N(0,1) then per-token RMS norm
                                        (QK-norm, unit gain, eps 1e-6); V,dO ~ N(0,1)
  llama8k     B1 H32 N8192  causal      Q,V,dO ~ N(0,1); K ~ N(0,1) + a per-(b,h,
                                        channel) bias of variance 4 shared by tokens
  llama16k    B1 H32 N16384 causal      as llama8k
  video       B2 H30 N17776 non-causal  Q,K ~ N(0,1) plus +-8 on 4 random channels
                                        per (tensor, b, h); V,dO ~ N(0,1)

  rowscale    (custom shapes, for the fused QK-norm) Q, K ~ N(0,1), each token
                                        row scaled by exp(U(ln 0.05, ln 20)), i.e.
                                        un-normalized activations; V,dO ~ N(0,1)

Seeds: every (tensor, batch b, head h) has its own numpy PCG64 stream seeded by
SeedSequence([1000*k + tensor index, b, h]) with tensor index Q 0, K 1, V 2,
dO 3, K-bias 4, outlier channels 6, row scales 7 (K's with head 1000 + h),
and k = 1..5 in the order above.  Draws are
float32, rounded to bfloat16 with round-to-nearest-even; the bf16 bit patterns
(uint16) are what both sides receive.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import numpy as np

D = 64


@dataclass(frozen=True)
class Workload:
    name: str
    k: int            # seed family
    B: int
    H: int
    N: int
    causal: bool
    smooth_k: bool
    smooth_q: bool
    dist: str         # "normal" | "qknorm" | "kbias" | "outlier" | "rowscale"
    d: int = D

    @property
    def bh(self) -> int:
        return self.B * self.H


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 2, 128, False, True, False, "normal"),
    "pretrain": Workload("pretrain", 2, 8, 16, 2048, True, True, False, "qknorm"),
    "llama8k": Workload("llama8k", 3, 1, 32, 8192, True, True, True, "kbias"),
    "llama16k": Workload("llama16k", 4, 1, 32, 16384, True, True, True, "kbias"),
    "video": Workload("video", 5, 2, 30, 17776, False, True, True, "outlier"),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _gen(seed: int, b: int, h: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, b, h])))


def make_head(w: Workload, b: int, h: int, seed_family: int | None = None) -> dict:
    """Inputs of one (batch, head): {"q","k","v","do"} as uint16 bf16 bits [N, d].
    Each tensor of each head has its own PCG64 stream seeded by
    SeedSequence([1000*k + tensor index, b, h])."""
    k = w.k if seed_family is None else seed_family
    shape = (w.N, w.d)
    q = _gen(1000 * k + 0, b, h).standard_normal(shape, dtype=np.float32)
    kk = _gen(1000 * k + 1, b, h).standard_normal(shape, dtype=np.float32)
    v = _gen(1000 * k + 2, b, h).standard_normal(shape, dtype=np.float32)
    do = _gen(1000 * k + 3, b, h).standard_normal(shape, dtype=np.float32)
    if w.dist == "qknorm":
        # input preparation only: the model-side QK-norm that produces such inputs
        for x in (q, kk):
            ms = np.mean(x * x, axis=-1, keepdims=True, dtype=np.float32)
            x /= np.sqrt(ms + np.float32(1e-6), dtype=np.float32)
    elif w.dist == "kbias":
        kk += _gen(1000 * k + 4, b, h).standard_normal((1, w.d), dtype=np.float32) * np.float32(2.0)
    elif w.dist == "outlier":
        for ti, x in enumerate((q, kk)):
            rng = _gen(1000 * k + 6, b, 1000 * ti + h)
            ch = rng.choice(w.d, size=4, replace=False)
            sign = rng.choice(np.array([-1.0, 1.0], dtype=np.float32), size=4)
            x[:, ch] += (np.float32(8.0) * sign)[None, :]
    elif w.dist == "rowscale":
        for ti, x in enumerate((q, kk)):
            u = _gen(1000 * k + 7, b, 1000 * ti + h).uniform(np.log(0.05), np.log(20.0), (w.N, 1))
            x *= np.exp(u).astype(np.float32)
    elif w.dist != "normal":
        raise ValueError(w.dist)
    return {n: f32_to_bf16_bits(a) for n, a in (("q", q), ("k", kk), ("v", v), ("do", do))}


def make_inputs(w: Workload, seed_family: int | None = None, threads: int = 8) -> dict:
    """Return {"q","k","v","do"} as uint16 bf16 bit arrays of shape [B,H,N,d]."""
    from concurrent.futures import ThreadPoolExecutor
    out = {n: np.empty((w.B, w.H, w.N, w.d), np.uint16) for n in ("q", "k", "v", "do")}

    def one(bh):
        b, h = divmod(bh, w.H)
        for n, a in make_head(w, b, h, seed_family).items():
            out[n][b, h] = a

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(one, range(w.B * w.H)))
    return out


def custom(B: int, H: int, N: int, causal: bool, smooth_k: bool = True, smooth_q: bool = False,
           dist: str = "normal", seed_family: int = 77) -> Workload:
    """An ad-hoc workload (edge cases: ragged N, tiny N, other flags)."""
    return Workload(f"custom_B{B}H{H}N{N}", seed_family, B, H, N, causal, smooth_k, smooth_q, dist)
