"""Drives the HIP library through its C ABI on seeded synthetic inputs.

Used by the GPU parity tests, ``__graft_entry__.smoke`` and ``bench.py``.
Device memory and streams come from torch; every step runs in libhga.so.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

import long_context_hga_amd as hga
from synth import Inputs


def to_dev(a: np.ndarray, dev="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev)
    return torch.from_numpy(a).to(dev)


def dev_to_np_bf16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


@dataclasses.dataclass
class State:
    inp: Inputs
    cfg: hga.hga_config
    B: int
    T: int
    max_chunks: int
    max_sel: int
    k_raw: torch.Tensor
    v_raw: torch.Tensor
    q: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    chunk_sum: torch.Tensor
    group_sum: torch.Tensor
    ws: torch.Tensor
    pos0: torch.Tensor


def build_state(inp: Inputs, cfg_over: Optional[dict] = None, pool_on_host: bool = False,
                max_lq: Optional[int] = None) -> State:
    p = dict(inp.params)
    if cfg_over:
        p.update(cfg_over)
    cfg = hga.config_from(p)
    B, T = inp.k.shape[0], inp.k.shape[2]
    d, hkv = p["head_dim"], p["n_kv_heads"]
    max_chunks = T // p["chunk_size"]
    lq = inp.q.shape[2] if max_lq is None else max_lq
    max_sel = hga.hga_max_selected(cfg, lq)
    elt = torch.int16 if p["dtype"] == "bf16" else torch.float32
    k_raw = to_dev(inp.k)
    v_raw = to_dev(inp.v)
    q = to_dev(inp.q)
    if pool_on_host:
        k_pool = torch.empty((B, hkv, T, d), dtype=elt, pin_memory=True)
        v_pool = torch.empty((B, hkv, T, d), dtype=elt, pin_memory=True)
        # the append writes through the device mapping of the pinned pool
    else:
        k_pool = torch.empty((B, hkv, T, d), dtype=elt, device="cuda")
        v_pool = torch.empty((B, hkv, T, d), dtype=elt, device="cuda")
    chunk_sum = torch.zeros((B, hkv, max_chunks, d), dtype=torch.float32, device="cuda")
    group_sum = torch.zeros((B, hkv, max_chunks * p["groups_per_chunk"], d), dtype=torch.float32,
                            device="cuda")
    wsb = hga.hga_workspace_bytes(cfg, B, T, lq)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    pos0 = to_dev(inp.pos0.astype(np.int32))
    st = State(inp, cfg, B, T, max_chunks, max_sel, k_raw, v_raw, q, k_pool, v_pool, chunk_sum,
               group_sum, ws, pos0)
    if not pool_on_host:
        hga.hga_build_summaries(cfg, B, k_raw, v_raw, 0, T, k_pool, v_pool, T, chunk_sum, group_sum,
                                max_chunks)
    else:
        dk = torch.empty((B, hkv, T, d), dtype=elt, device="cuda")
        dv = torch.empty((B, hkv, T, d), dtype=elt, device="cuda")
        hga.hga_build_summaries(cfg, B, k_raw, v_raw, 0, T, dk, dv, T, chunk_sum, group_sum,
                                max_chunks)
        k_pool.copy_(dk)
        v_pool.copy_(dv)
        del dk, dv
    return st


@dataclasses.dataclass
class Step:
    sel: torch.Tensor
    n_sel: torch.Tensor
    scores: torch.Tensor
    out: torch.Tensor
    lse: torch.Tensor


def alloc_step(st: State, lq: int) -> Step:
    p = st.inp.params
    B, hkv, hq, d = st.B, p["n_kv_heads"], p["n_q_heads"], p["head_dim"]
    lists = hq if p.get("route_per_head") else hkv  # one list per query head or per KV head
    return Step(
        sel=torch.full((B, lists, st.max_sel), -7, dtype=torch.int32, device="cuda"),
        n_sel=torch.full((B, lists), -7, dtype=torch.int32, device="cuda"),
        scores=torch.full((B, lists, st.max_chunks), float("nan"), dtype=torch.float64,
                          device="cuda"),
        out=torch.full((B, hq, lq, d), float("nan"), dtype=torch.float32, device="cuda"),
        lse=torch.full((B, hq, lq), float("nan"), dtype=torch.float32, device="cuda"))


def route(st: State, q: torch.Tensor, lq: int, pos0: torch.Tensor, s: Step, with_scores=True):
    hga.hga_route(st.cfg, st.B, q, lq, pos0, st.chunk_sum, st.group_sum, st.max_chunks, s.sel,
                  s.n_sel, st.max_sel, s.scores if with_scores else None, st.ws)


def attend(st: State, q: torch.Tensor, lq: int, pos0: torch.Tensor, s: Step,
           part=hga.HGA_PART_ALL, k_src=None, v_src=None, layout=hga.HGA_SRC_POOL, out=None,
           lse=None):
    hga.hga_attend(st.cfg, st.B, q, lq, pos0, st.k_pool if k_src is None else k_src,
                   st.v_pool if v_src is None else v_src, layout, st.T, s.sel, s.n_sel,
                   st.max_sel, part, s.out if out is None else out, s.lse if lse is None else lse,
                   st.ws)


def v_token_view(v_pool: torch.Tensor) -> torch.Tensor:
    """View [B][H][T/16][16][d] of a V pool, whose 16-token groups are stored
    transposed ([d][16] blocks): element [b, h, g, t, e] is token 16g+t, dim e."""
    B, H, T, d = v_pool.shape
    return v_pool.view(B, H, T // 16, d, 16).transpose(3, 4)


def v_rows(v_pool: torch.Tensor) -> np.ndarray:
    """A V pool as token rows [B][H][T][d] (host copy)."""
    B, H, T, d = v_pool.shape
    return v_token_view(v_pool).cpu().numpy().reshape(B, H, T, d)


def query_slice(st: State, i: int) -> torch.Tensor:
    """Query token i of every head as its own lq=1 query [B][Hq][1][d]."""
    return st.q[:, :, i:i + 1, :].contiguous()
