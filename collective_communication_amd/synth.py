"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the collectives: it only draws numbers.
Floating inputs are drawn in fp32 with numpy's PCG64 generator and narrowed
to bf16 / fp16 by torch's own CPU casts (round to nearest even), so neither
the oracle nor the HIP path contributes to its own inputs.

Workload recipe (shapes and distributions of the pages' workloads):

* AllReduce R=4, 1-D bf16 [81920] (160 KiB, four owner segments), N(0, 1).
* TP decode AllReduce R=8, bf16 [64, 7168], N(0, 0.02^2) (second argument of
  N is a variance); message sweep 8 KiB .. 64 MiB per rank, same law.
* Sequence-parallel ReduceScatter then AllGather, R=8, bf16 [8192, 4096], N(0,1).
* Gather of vocab-sharded logits, R=8, fp32 [256, 19008], N(0, 4) (sigma 2);
  Broadcast of int32 [256] uniform in [0, 152064) from root 7.
* MoE dispatch/combine, R=8, 4096 tokens x hidden 7168 bf16 N(0,1) per rank;
  256 experts, top-8 routing from Zipf(1.2)-skewed expert logits with
  Gumbel noise (Gumbel-top-k draws k experts without replacement with
  probabilities proportional to expert popularity), fp32 softmax gate weights.
"""
from __future__ import annotations

import numpy as np


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _narrow(x32: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 -> storage of ``dtype`` via torch's CPU cast (bf16 as uint16 bits)."""
    if dtype == "fp32":
        return x32
    if dtype == "fp16":
        return x32.astype(np.float16)
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(np.ascontiguousarray(x32)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def gaussian(shape, sigma: float, seed: int, dtype: str = "bf16") -> np.ndarray:
    """i.i.d. N(0, sigma^2) drawn in fp32, narrowed to ``dtype``."""
    x = rng(seed).standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x = x * np.float32(sigma)
    return _narrow(x, dtype)


def small_integers(shape, lim: int, seed: int, dtype: str) -> np.ndarray:
    """Integers uniform in [-lim, lim] stored as ``dtype`` (exact in all)."""
    x = rng(seed).integers(-lim, lim + 1, size=shape).astype(np.float32)
    if dtype == "int32":
        return x.astype(np.int32)
    return _narrow(x, dtype)


def uniform_int32(shape, lo: int, hi: int, seed: int) -> np.ndarray:
    """int32 uniform in [lo, hi)."""
    return rng(seed).integers(lo, hi, size=shape, dtype=np.int64).astype(np.int32)


def random_bits(shape, nbytes_per_elem: int, seed: int) -> np.ndarray:
    """Arbitrary bit patterns (copy primitives are dtype-agnostic)."""
    g = rng(seed)
    if nbytes_per_elem == 2:
        return g.integers(0, 1 << 16, size=shape, dtype=np.uint32).astype(np.uint16)
    if nbytes_per_elem == 4:
        return g.integers(0, 1 << 32, size=shape, dtype=np.uint64).astype(np.uint32)
    return g.integers(0, 256, size=shape, dtype=np.uint32).astype(np.uint8)


def zipf_routing(tokens: int, experts: int, topk: int, seed: int,
                 s: float = 1.2, permute_seed: int | None = None):
    """Top-k expert ids and fp32 gate weights for ``tokens`` tokens.

    Expert popularity p_e is proportional to (e + 1)^-s (over the expert index,
    or over a seeded permutation of it when ``permute_seed`` is given).  Logits
    are ln p_e plus standard Gumbel noise; the k largest logits (ties to the
    lower expert id) give the ids in descending-logit order, and the gate
    weights are the fp32 softmax of those k logits, max-subtracted.
    Returns (ids int32 [T, K], w fp32 [T, K]).
    """
    g = rng(seed)
    rank = np.arange(experts, dtype=np.float64)
    if permute_seed is not None:
        rank = rng(permute_seed).permutation(experts).astype(np.float64)
    logp = (-s * np.log(rank + 1.0)).astype(np.float32)
    u = g.random(size=(tokens, experts), dtype=np.float32)
    u = np.clip(u, np.float32(1e-30), np.float32(1.0) - np.float32(2.0 ** -24))
    gumbel = -np.log(-np.log(u))
    logits = (logp[None, :] + gumbel).astype(np.float32)
    order = np.argsort(-logits, axis=1, kind="stable")[:, :topk]
    ids = order.astype(np.int32)
    sel = np.take_along_axis(logits, order, axis=1)
    z = np.exp(sel - sel[:, :1])
    w = (z / z.sum(axis=1, keepdims=True)).astype(np.float32)
    return np.ascontiguousarray(ids), np.ascontiguousarray(w)
