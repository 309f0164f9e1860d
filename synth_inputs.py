"""Seeded synthetic workloads for the MoE token path (layout -> dispatch -> combine).

This module only draws inputs. It holds none of the method's arithmetic, and both
the CPU oracle and the HIP path are fed from it (the arrays are made once on the
host and, for the GPU side, copied to device memory unchanged).

Workloads (one per named shape; `seed` fixes every draw):

  tiny  : 16 tokens, hidden 2048, 8 experts in 8 groups of 1, top-2, uniform routing
  t256  : 256 tokens, hidden 7168, 256 experts in 8 groups of 32, top-8, uniform
  t4096 : 4096 tokens, hidden 7168, 256 experts in 8 groups of 32, top-8, uniform
          (the headline dispatch/combine bandwidth shape)
  skew  : 4096 tokens, hidden 4096, 128 experts in 8 groups of 16, top-8,
          Zipf(s=1.2) expert popularity over a seeded expert permutation,
          sampled without replacement per token
  fp8   : the t4096 shape, dispatched with FP8 e4m3 per-128-block quantisation

These stand in for the AMD Developer Challenge 2025 All-to-All problem sizes
(8-256 experts, top 2-8, hidden 2048-7168, 16-256 tokens) and for the
DeepSeek-V3-style EP8 shape (hidden 7168, top-8, 256 experts over 8 ranks)
that the mori IntraNode dispatch pull request measures.

Recipe (per workload, numpy Generator(PCG64(seed)), draws in this order):
  1. x       : standard_normal float32 [T, H], rounded to bf16 by torch's CPU
               cast (round to nearest even); kept as raw uint16 bits.
  2. routing : uniform -> per token, the first K entries of a stable argsort of
               E uniform keys (a uniform K-subset, in draw order);
               zipf    -> p(rank r) ~ r^-s over a seeded permutation of the
               experts; Gumbel-top-K of log p (successive sampling without
               replacement), taken in descending key order.
  3. weights : softmax over K of standard_normal float32 logits [T, K],
               computed in float32 with the row max subtracted.
"""
from __future__ import annotations

import dataclasses

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_inputs", "make_workload"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    E: int
    G: int
    K: int
    routing: str = "uniform"   # "uniform" | "zipf"
    zipf_s: float = 1.2
    fp8: bool = False
    seed: int = 1

    def describe(self) -> str:
        r = self.routing if self.routing == "uniform" else f"zipf(s={self.zipf_s})"
        d = "fp8-e4m3/128" if self.fp8 else "bf16"
        return (f"{self.name}: T={self.T} H={self.H} E={self.E} G={self.G} K={self.K} "
                f"routing={r} dispatch={d} seed={self.seed}")


WORKLOADS = {
    "tiny": Workload("tiny", T=16, H=2048, E=8, G=8, K=2, seed=1),
    "t256": Workload("t256", T=256, H=7168, E=256, G=8, K=8, seed=2),
    "t4096": Workload("t4096", T=4096, H=7168, E=256, G=8, K=8, seed=3),
    "skew": Workload("skew", T=4096, H=4096, E=128, G=8, K=8, routing="zipf",
                     zipf_s=1.2, seed=4),
    "fp8": Workload("fp8", T=4096, H=7168, E=256, G=8, K=8, fp8=True, seed=5),
}


def _bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    import torch  # CPU cast only
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _uniform_routing(rng: np.random.Generator, T: int, E: int, K: int) -> np.ndarray:
    out = np.empty((T, K), dtype=np.int32)
    chunk = max(1, (1 << 22) // max(E, 1))
    for t0 in range(0, T, chunk):
        keys = rng.random((min(chunk, T - t0), E))
        out[t0:t0 + keys.shape[0]] = np.argsort(keys, axis=1, kind="stable")[:, :K]
    return out


def _zipf_routing(rng: np.random.Generator, T: int, E: int, K: int, s: float) -> np.ndarray:
    perm = rng.permutation(E)
    p_rank = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    p = np.empty(E, dtype=np.float64)
    p[perm] = p_rank / p_rank.sum()
    logp = np.log(p)
    out = np.empty((T, K), dtype=np.int32)
    chunk = max(1, (1 << 22) // max(E, 1))
    for t0 in range(0, T, chunk):
        n = min(chunk, T - t0)
        keys = logp[None, :] + rng.gumbel(size=(n, E))
        out[t0:t0 + n] = np.argsort(-keys, axis=1, kind="stable")[:, :K]
    return out


def _softmax_weights(rng: np.random.Generator, T: int, K: int) -> np.ndarray:
    logits = rng.standard_normal((T, K), dtype=np.float32)
    z = logits - logits.max(axis=1, keepdims=True)
    ez = np.exp(z, dtype=np.float32)
    return (ez / ez.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)


def make_inputs(T: int, H: int, E: int, K: int, *, seed: int, routing: str = "uniform",
                zipf_s: float = 1.2) -> dict:
    """Draw x (bf16 bits, uint16 [T,H]), topk_idx (int32 [T,K]) and topk_w (fp32 [T,K])."""
    if K > E:
        raise ValueError("top-k larger than the expert count")
    rng = np.random.Generator(np.random.PCG64(seed))
    x = _bf16_bits(rng.standard_normal((T, H), dtype=np.float32)) if T * H else \
        np.zeros((T, H), dtype=np.uint16)
    if routing == "uniform":
        idx = _uniform_routing(rng, T, E, K)
    elif routing == "zipf":
        idx = _zipf_routing(rng, T, E, K, zipf_s)
    else:
        raise ValueError(f"unknown routing {routing!r}")
    w = _softmax_weights(rng, T, K)
    return {"x": x, "topk_idx": idx, "topk_w": w}


def make_workload(wl: Workload | str) -> dict:
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    d = make_inputs(wl.T, wl.H, wl.E, wl.K, seed=wl.seed, routing=wl.routing,
                    zipf_s=wl.zipf_s)
    d["workload"] = wl
    return d
