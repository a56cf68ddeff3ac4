"""Seeded synthetic inputs for the Gemma 2 attention layer.

This module only draws random numbers and places them in the layouts the
library and the oracle consume.  It holds none of the attention arithmetic, so
the GPU path and the CPU oracle can both be fed from it.

Recipe (the same for every workload):
  * each tensor of a workload gets its own stream SeedSequence([seed, index]);
  * the tensor is drawn as float32 in fixed chunks of CHUNK elements of its
    flattened (row-major) form, chunk c from child c of that stream, so the
    values do not depend on how many threads draw them;
  * normal draws use numpy's standard_normal; Student-t draws use
    standard_t(nu) divided by sqrt(nu / (nu - 2)), the theoretical standard
    deviation (the 27B-shaped workload asks for unit variance);
  * the draw is multiplied by the workload's scale for that tensor, then rounded
    to the storage type (bf16 with round-to-nearest-even through torch, or kept
    in float32).

Shapes follow the model card's per-size table (H / KVH / head dim) and its
local window / global span; see WORKLOADS.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

CHUNK = 1 << 22

# Workloads: the five seeded configurations plus saturation variants.
#   q_mul/k_mul/v_mul multiply the unit draws; dist is "normal" or "t3".
WORKLOADS = {
    "tiny": dict(kind="prefill", B=1, T=256, S=256, H=4, KVH=2, d=64,
                 dtype="f32", query_scale=1.0 / 8.0, softcap=50.0, window=64,
                 seed=0, q_mul=4.0, k_mul=1.0, v_mul=1.0, dist="normal"),
    "tiny-sat": dict(kind="prefill", B=1, T=256, S=256, H=4, KVH=2, d=64,
                     dtype="f32", query_scale=1.0 / 8.0, softcap=50.0, window=64,
                     seed=0, q_mul=32.0, k_mul=1.0, v_mul=1.0, dist="normal"),
    "2b-8k": dict(kind="prefill", B=4, T=8192, S=8192, H=8, KVH=4, d=256,
                  dtype="bf16", query_scale=1.0 / 16.0, softcap=50.0, window=4096,
                  seed=1, q_mul=1.0, k_mul=1.0, v_mul=1.0, dist="normal"),
    "9b-8k": dict(kind="prefill", B=2, T=8192, S=8192, H=16, KVH=8, d=256,
                  dtype="bf16", query_scale=1.0 / 16.0, softcap=50.0, window=4096,
                  seed=2, q_mul=3.0, k_mul=3.0, v_mul=1.0, dist="normal"),
    "9b-8k-sat": dict(kind="prefill", B=2, T=8192, S=8192, H=16, KVH=8, d=256,
                      dtype="bf16", query_scale=1.0 / 16.0, softcap=50.0,
                      window=4096, seed=2, q_mul=5.5, k_mul=5.5, v_mul=1.0,
                      dist="normal"),
    "27b-8k": dict(kind="prefill", B=1, T=8192, S=8192, H=32, KVH=16, d=128,
                   dtype="bf16", query_scale=1.0 / 12.0, softcap=50.0,
                   window=4096, seed=3, q_mul=1.0, k_mul=1.0, v_mul=1.0,
                   dist="t3"),
    "9b-decode": dict(kind="decode", B=64, T=1, S=8192, H=16, KVH=8, d=256,
                      dtype="bf16", query_scale=1.0 / 16.0, softcap=50.0,
                      window=4096, seed=4, q_mul=1.0, k_mul=1.0, v_mul=1.0,
                      dist="normal", len_lo=4096, len_hi=8192),
}


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _draw_into(out_flat: torch.Tensor, seed: int, stream: int, dist: str,
               mul: float) -> None:
    """Fill a flat CPU tensor (bf16 or f32) with the seeded draw of one stream."""
    n = out_flat.numel()
    nchunks = max(1, (n + CHUNK - 1) // CHUNK)
    children = np.random.SeedSequence([seed, stream]).spawn(nchunks)

    def one(c: int) -> None:
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        rng = np.random.default_rng(children[c])
        if dist == "normal":
            x = rng.standard_normal(hi - lo, dtype=np.float32)
        elif dist == "t3":
            nu = 3.0
            x = (rng.standard_t(nu, size=hi - lo) / math.sqrt(nu / (nu - 2.0)))
            x = x.astype(np.float32)
        else:
            raise ValueError(f"unknown distribution {dist!r}")
        if mul != 1.0:
            x *= np.float32(mul)
        out_flat[lo:hi].copy_(torch.from_numpy(x))

    if nchunks == 1:
        one(0)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(one, range(nchunks)))


def torch_dtype(name: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def draw(shape, seed: int, stream: int, *, dtype: str = "bf16",
         dist: str = "normal", mul: float = 1.0) -> torch.Tensor:
    """One seeded tensor of the given shape on the CPU, in the storage type."""
    t = torch.empty(tuple(shape), dtype=torch_dtype(dtype))
    _draw_into(t.view(-1), seed, stream, dist, mul)
    return t


def prefill_inputs(cfg: dict):
    """q (B,T,H,d), k and v (B,S,KVH,d) of a prefill workload, CPU tensors.

    The local and the global layer of a pair read the same q, k, v.
    """
    B, T, S, H, KVH, d = (cfg[x] for x in ("B", "T", "S", "H", "KVH", "d"))
    dt, seed, dist = cfg["dtype"], cfg["seed"], cfg["dist"]
    q = draw((B, T, H, d), seed, 0, dtype=dt, dist=dist, mul=cfg["q_mul"])
    k = draw((B, S, KVH, d), seed, 1, dtype=dt, dist=dist, mul=cfg["k_mul"])
    v = draw((B, S, KVH, d), seed, 2, dtype="f32" if dt == "f32" else dt,
             dist="normal", mul=cfg["v_mul"])
    return q, k, v


def decode_lengths(cfg: dict) -> np.ndarray:
    """Per-sequence cache lengths L_b, uniform on [len_lo, len_hi]."""
    rng = np.random.default_rng(np.random.SeedSequence([cfg["seed"], 99]))
    return rng.integers(cfg["len_lo"], cfg["len_hi"] + 1, size=cfg["B"]).astype(np.int32)


def ring_from_linear(cache: torch.Tensor, lens: np.ndarray, slots: int,
                     fill=float("nan")) -> torch.Tensor:
    """Place the last `slots` positions of each sequence at slot p mod slots.

    cache: (B, S, KVH, d) linear cache holding position p at row p.  Positions
    older than L_b - slots are dropped, as a local layer's ring would; slots
    that hold no position (L_b < slots) are set to `fill`.
    """
    B = cache.shape[0]
    ring = torch.full((B, slots) + tuple(cache.shape[2:]), fill, dtype=cache.dtype)
    for b in range(B):
        L = int(lens[b])
        lo = max(0, L - slots)
        pos = torch.arange(lo, L)
        ring[b, pos % slots] = cache[b, lo:L]
    return ring


def poison_beyond(cache: torch.Tensor, lens: np.ndarray, fill=float("nan")) -> None:
    """Set rows at positions >= L_b of a linear cache to `fill` (in place)."""
    for b in range(cache.shape[0]):
        cache[b, int(lens[b]):] = fill


def decode_inputs(cfg: dict, *, poison: bool = False):
    """Inputs of the decode workload as CPU tensors.

    Returns q (B,1,H,d), the global layer's linear caches k_g, v_g (B,S,KVH,d),
    kv_lens (B,) int32, and the local layer's rings k_l, v_l (B,window,KVH,d)
    holding the same sequences' last `window` positions at slot p mod window.
    With poison=True every slot that holds no visible position is NaN.
    """
    B, S, H, KVH, d = (cfg[x] for x in ("B", "S", "H", "KVH", "d"))
    dt, seed = cfg["dtype"], cfg["seed"]
    q = draw((B, 1, H, d), seed, 0, dtype=dt, mul=cfg["q_mul"])
    k_g = draw((B, S, KVH, d), seed, 1, dtype=dt, mul=cfg["k_mul"])
    v_g = draw((B, S, KVH, d), seed, 2, dtype=dt, mul=cfg["v_mul"])
    lens = decode_lengths(cfg)
    W = cfg["window"]
    k_l = ring_from_linear(k_g, lens, W)
    v_l = ring_from_linear(v_g, lens, W)
    if poison:
        poison_beyond(k_g, lens)
        poison_beyond(v_g, lens)
    return q, k_g, v_g, lens, k_l, v_l


def paged_from_linear(cache: torch.Tensor, lens: np.ndarray, block_size: int, *,
                      seed: int, keep_last: int = 0, spare_blocks: int = 0,
                      fill=float("nan")):
    """Lay a linear cache out as a block pool and a block table.

    cache: (B, S, KVH, d) holding position p of sequence b at row p.  Logical
    block i of sequence b (positions i*block_size .. (i+1)*block_size - 1) is
    stored in a physical block chosen by a seeded random permutation.  Blocks
    at or past L_b are not allocated; with keep_last = W > 0, blocks holding
    none of the last W positions are not allocated either (dropped, as a
    serving runtime drops a local layer's old blocks).  Unallocated table
    entries are -1.  Rows of allocated blocks at positions >= L_b, and
    `spare_blocks` extra pool blocks, are set to `fill`.

    Returns pool (num_blocks, block_size, KVH, d) and table (B, max_blocks)
    int32 with max_blocks = ceil(S / block_size).
    """
    B, S = cache.shape[0], cache.shape[1]
    bs = block_size
    max_blocks = (S + bs - 1) // bs
    wanted = []
    for b in range(B):
        L = int(lens[b])
        first = max(0, L - keep_last) // bs if keep_last > 0 else 0
        last = (L - 1) // bs
        wanted.extend((b, i) for i in range(first, last + 1))
    n = len(wanted) + spare_blocks
    perm = np.random.default_rng(np.random.SeedSequence([seed, 7])).permutation(n)
    pool = torch.full((n, bs) + tuple(cache.shape[2:]), fill, dtype=cache.dtype)
    table = np.full((B, max_blocks), -1, np.int32)
    for (b, i), phys in zip(wanted, perm[:len(wanted)]):
        L = int(lens[b])
        lo, hi = i * bs, min((i + 1) * bs, L, S)
        table[b, i] = phys
        pool[phys, :hi - lo] = cache[b, lo:hi]
    return pool, table


def to_f32_numpy(t: torch.Tensor) -> np.ndarray:
    """Exact float32 copy of a CPU/GPU tensor holding bf16 or f32 values."""
    return t.detach().to("cpu", torch.float32).contiguous().numpy()
