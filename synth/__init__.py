"""Seeded synthetic inputs for the HGA hot path.

Both the GPU library's tests/benchmark and the CPU oracle draw their inputs
from here, and from nowhere else.  This module holds none of the method's
arithmetic: no RoPE, no summaries, no routing, no attention.  It only draws
normal samples with a fixed seed, quantises them to the input dtype, and (for
the needle workload) adds a fixed direction to chosen key rows.

Workloads (one per entry of ``CONFIGS``), all grouped-query attention inputs
of one layer, with K/V/Q ~ N(0, 1) before RoPE:

* ``tiny``       1 query / 1 KV head, d=64, fp32, 1024 tokens, theta=1e4,
                 C=64 in 4 groups of 16, 1 sink + 2 local chunks, top-2
                 chunks, top-4 groups; 8 decode queries at positions
                 1016..1023 (each routed on its own).
* ``decode4k``   32/4 heads, d=128, bf16, theta=1e6, 4096 tokens, 1 sink + 4
                 local chunks, top-8 chunks, top-16 groups, batch 1, one
                 decode token at 4095.
* ``prefill32k`` same layer at 32768 tokens; one 64-token query chunk (the
                 last chunk, positions 32704..32767); top-20 chunks, top-40
                 groups (1024 visible keys = 3.125 %); 16 planted needle
                 chunks.
* ``decode64k``  same layer at 65536 tokens, batch 8 independent sequences,
                 one decode token at 65535; top-52 chunks, top-104 groups
                 (2048 visible keys = 3.125 %).
* ``host64k``    as ``decode64k`` with batch 4; the caller keeps the full
                 pool in pinned host memory.
* ``prompt32k``  whole-prompt prefill of the ``prefill32k`` layer: queries for
                 all 32768 tokens (every 64-token chunk is a query chunk),
                 top-20 chunks, top-40 groups (1024 keys per query chunk once
                 20 chunks are candidates); no planted needles (one planted
                 direction cannot match the pooled queries of every chunk).

Seeds: sequence b of workload i (1-based, in the order above) draws from
``numpy.random.Generator(PCG64(1000*i + b))`` in the order K [Hkv][T][d],
V [Hkv][T][d], Q [Hq][lq][d], then the needle draws.  bf16 values are the
round-to-nearest-even of the float32 draws and are held as uint16 bit
patterns.

Needles (``prefill32k``): 16 chunk ids drawn without replacement from the
candidate range [n_sink, c_q - n_local).  For each KV head, u is the unit
vector of the mean raw query of that head's query heads over the query chunk,
restricted to ``needle_dims``; every key of a needle chunk gets kappa*u added
(kappa = 16) before rounding.  ``needle_dims`` are the last 8 pairs of each
half of the head (dims 56..63 and 120..127 at d=128): with theta=1e6 those
pairs turn by less than 0.2 rad over 32K positions, so the planted direction
stays aligned with the rotated query across the whole context.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

_LAYER = dict(head_dim=128, n_q_heads=32, n_kv_heads=4, dtype="bf16", rope_theta=1e6,
              chunk_size=64, groups_per_chunk=4, hf_wavelength=64.0)

CONFIGS: Dict[str, dict] = {
    "tiny": dict(index=1, head_dim=64, n_q_heads=1, n_kv_heads=1, dtype="f32", rope_theta=1e4,
                 chunk_size=64, groups_per_chunk=4, hf_wavelength=64.0, context=1024,
                 n_sink_chunks=1, n_local_chunks=2, topk_chunks=2, topk_groups=4, batch=1,
                 lq=8, query_pos0=1016, per_token_queries=True),
    "decode4k": dict(index=2, **_LAYER, context=4096, n_sink_chunks=1, n_local_chunks=4,
                     topk_chunks=8, topk_groups=16, batch=1, lq=1, query_pos0=4095),
    "prefill32k": dict(index=3, **_LAYER, context=32768, n_sink_chunks=1, n_local_chunks=4,
                       topk_chunks=20, topk_groups=40, batch=1, lq=64, query_pos0=32704,
                       needles=16, needle_kappa=16.0),
    "decode64k": dict(index=4, **_LAYER, context=65536, n_sink_chunks=1, n_local_chunks=4,
                      topk_chunks=52, topk_groups=104, batch=8, lq=1, query_pos0=65535),
    "host64k": dict(index=5, **_LAYER, context=65536, n_sink_chunks=1, n_local_chunks=4,
                    topk_chunks=52, topk_groups=104, batch=4, lq=1, query_pos0=65535),
    "prompt32k": dict(index=6, **_LAYER, context=32768, n_sink_chunks=1, n_local_chunks=4,
                      topk_chunks=20, topk_groups=40, batch=1, lq=32768, query_pos0=0,
                      whole_prompt=True),
}


def needle_dims(d: int) -> np.ndarray:
    h = d // 2
    return np.concatenate([np.arange(h - 8, h), np.arange(d - 8, d)])


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Inputs:
    name: str
    params: dict
    k: np.ndarray          # [B][Hkv][T][d]  uint16 (bf16 bits) or float32
    v: np.ndarray          # [B][Hkv][T][d]
    q: np.ndarray          # [B][Hq][lq][d]
    pos0: np.ndarray       # [B] int32, position of the first query token
    needle_chunks: Optional[np.ndarray] = None   # [B][n_needles]

    @property
    def is_bf16(self) -> bool:
        return self.params["dtype"] == "bf16"

    def f64(self, a: np.ndarray) -> np.ndarray:
        """Exact float64 view of an input array (bf16 bits or float32)."""
        if a.dtype == np.uint16:
            return bf16_to_f32(a).astype(np.float64)
        return a.astype(np.float64)


def _quant(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def generate(name: str, batch: Optional[int] = None, context: Optional[int] = None,
             seeds: Optional[List[int]] = None, overrides: Optional[dict] = None) -> Inputs:
    """Draw the inputs of workload ``name``.

    ``batch`` / ``context`` override the workload's sizes (smaller parity
    cases); the seed of sequence b stays 1000*index + b unless ``seeds``
    gives them explicitly.  With a shorter context the query moves to the
    end of it (the same offset from the end as in the full workload).
    ``overrides`` replaces other entries of the workload (head counts,
    head_dim, dtype, budgets, lq) for shape-coverage cases."""
    p = dict(CONFIGS[name])
    if overrides:
        p.update(overrides)
    B = p["batch"] if batch is None else int(batch)
    T = p["context"] if context is None else int(context)
    if p.get("whole_prompt"):  # every token is a query token
        p["context"], p["lq"], p["query_pos0"] = T, T, 0
    elif context is not None:
        p["query_pos0"] = p["query_pos0"] - p["context"] + T
        p["context"] = T
    p["batch"] = B
    d, hkv, hq, lq = p["head_dim"], p["n_kv_heads"], p["n_q_heads"], p["lq"]
    dt = p["dtype"]
    ks, vs, qs, needles = [], [], [], []
    for b in range(B):
        seed = (1000 * p["index"] + b) if seeds is None else int(seeds[b])
        rng = np.random.Generator(np.random.PCG64(seed))
        k = rng.standard_normal((hkv, T, d), dtype=np.float32)
        v = rng.standard_normal((hkv, T, d), dtype=np.float32)
        q = rng.standard_normal((hq, lq, d), dtype=np.float32)
        if p.get("needles"):
            C = p["chunk_size"]
            cq = p["query_pos0"] // C
            lo, hi = p["n_sink_chunks"], cq - p["n_local_chunks"]
            ids = np.sort(rng.choice(np.arange(lo, hi), size=p["needles"], replace=False))
            nd = needle_dims(d)
            hg = hq // hkv
            for h in range(hkv):
                qm = q[h * hg:(h + 1) * hg].astype(np.float64).mean(axis=(0, 1))[nd]
                u = (qm / np.linalg.norm(qm)).astype(np.float32)
                for c in ids:
                    k[h, c * C:(c + 1) * C][:, nd] += np.float32(p["needle_kappa"]) * u
            needles.append(ids)
        ks.append(_quant(k, dt))
        vs.append(_quant(v, dt))
        qs.append(_quant(q, dt))
    pos0 = np.full(B, p["query_pos0"], dtype=np.int32)
    return Inputs(name=name, params=p, k=np.stack(ks), v=np.stack(vs), q=np.stack(qs), pos0=pos0,
                  needle_chunks=np.stack(needles) if needles else None)
