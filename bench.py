"""Benchmark of the HGA decode hot path on one MI355X.

Workload (default): one decode step of a GQA attention layer (32 query / 4 KV
heads, head_dim 128, bf16, RoPE theta 1e6) at 65536 tokens of context, batch
8 independent sequences, query at position 65535.  C = 64 tokens per chunk in
4 groups of 16; 1 sink + 4 local chunks, top-52 chunks then top-104 groups,
so 2048 of 65536 keys (3.125 %) are attended per (sequence, KV head).

One step = the whole path for the new token of every sequence:
  1. hga_build_summaries: the token at 65535 completes chunk 1023, so the
     chunk's 64 raw keys are rotated into the pool and its chunk and group
     summaries are written;
  2. hga_route: pooled query, level-1 scores of 1018 candidate chunks,
     top-52, level-2 scores of 208 groups, top-104, window merge;
  3. hga_attend: exact softmax attention over the 128 selected groups with
     the gather fused into the loads.
Inputs are resident in HBM before timing.  The state (pool, summaries,
queries) is replicated R times at distinct addresses and the steps cycle
through the replicas, so the timed traffic comes from HBM and not from the
256 MB last-level cache.

Prints one JSON line.  ``value`` = decoded query tokens per second per layer
(B tokens per step).  ``roofline`` covers the dominant kernel (hga_attend):
algorithmic bytes per launch / its mean launch duration measured with HIP
events on the launch stream.  ``cpu_baseline`` times the fp64 CPU oracle on a
bounded sample (the same step, repeated for ~10 s) on this host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

HBM_PEAK_GBS = 8000.0


def algorithmic_bytes(p, B):
    """Bytes the method must move per step (per launch) at the decode workload."""
    d, hkv, hq = p["head_dim"], p["n_kv_heads"], p["n_q_heads"]
    g = p["chunk_size"] // p["groups_per_chunk"]
    max_sel = (p["n_sink_chunks"] + p["n_local_chunks"] + 1) * p["groups_per_chunk"] + p["topk_groups"]
    ct = p["query_pos0"] // p["chunk_size"]
    n_cand = ct - p["n_local_chunks"] - p["n_sink_chunks"]
    kv = max_sel * g * d * 2 * 2 * hkv           # selected K and V rows, bf16
    q = hq * d * 2
    o = hq * d * 4
    idx = hkv * max_sel * 4
    attend = B * (kv + q + o + idx)
    route = B * (n_cand * d * 4 * hkv + p["topk_chunks"] * p["groups_per_chunk"] * d * 4 * hkv + q + idx)
    refresh = B * hkv * p["chunk_size"] * d * 2 * 4 + B * hkv * (1 + p["groups_per_chunk"]) * d * 4
    return dict(attend=attend, route=route, refresh=refresh, total=attend + route + refresh)


def cpu_baseline(inp, cfg_params, min_seconds=10.0):
    """The fp64 C oracle doing the same step (chunk refresh + route + attend for
    every sequence of the batch), repeated for about min_seconds."""
    import numpy as np
    import oracle
    cfg = oracle.cfg_from(cfg_params)
    p = cfg_params
    d, hkv = p["head_dim"], p["n_kv_heads"]
    hg = p["n_q_heads"] // hkv
    B, T = inp.k.shape[0], inp.k.shape[2]
    pos = int(inp.pos0[0])
    c0 = (pos // 64) * 64
    U = B * hkv
    # untimed state: summaries of the completed chunks and the rotated pool
    cs = np.zeros((U, T // 64, d))
    gs = np.zeros((U, T // 16, d))
    kp = np.zeros((U, T, d))
    vp = np.zeros((U, T, d))
    kraw = []
    for b in range(B):
        for h in range(hkv):
            u = b * hkv + h
            kr = inp.f64(inp.k[b, h])
            a, g = oracle.summaries(cfg, kr[:c0])
            cs[u, :a.shape[0]] = a
            gs[u, :g.shape[0]] = g
            kp[u] = oracle.pool(cfg, kr, 0)
            vp[u] = inp.f64(inp.v[b, h])
            kraw.append(kr[c0:c0 + 64].copy())
    q = np.stack([inp.f64(inp.q[b, h * hg:(h + 1) * hg, 0:1]) for b in range(B) for h in range(hkv)])
    max_sel = (p["n_sink_chunks"] + p["n_local_chunks"] + 1) * 4 + p["topk_groups"]
    times = []
    t_start = time.perf_counter()
    while len(times) < 5 or time.perf_counter() - t_start < min_seconds:
        t0 = time.perf_counter()
        for u in range(U):  # refresh of the chunk the new token completes
            kp[u, c0:c0 + 64] = oracle.pool(cfg, kraw[u], c0)
            cs[u, c0 // 64] = oracle.span_summary(cfg, kraw[u], c0)
            for i in range(4):
                gs[u, c0 // 16 + i] = oracle.span_summary(cfg, kraw[u][16 * i:16 * i + 16], c0 + 16 * i)
        oracle.step(cfg, q, np.full(U, pos), cs, gs, kp, vp, max_sel)
        times.append(time.perf_counter() - t0)
    med = float(np.median(times))
    return {"value": B / med, "unit": "tokens/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"the full step: all {B} sequences x {hkv} KV heads, chunk refresh + route + "
                      f"attend of one decode token at position {pos} (context {T}); fp64 C oracle, "
                      f"OpenMP over the {U} units; median of {len(times)} runs "
                      f"({med * 1e3:.1f} ms each, {time.perf_counter() - t_start:.1f} s total)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the decode path is "
              "per-GPU and this build has no multi-GPU leg", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gpu_harness as gh
    import long_context_hga_amd as hga
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    name = "decode64k"
    t_gen = time.time()
    inp = synth.generate(name)
    p = inp.params
    B, T = p["batch"], p["context"]
    st = gh.build_state(inp)
    torch.cuda.synchronize()
    print(f"[bench] state built in {time.time() - t_gen:.1f}s", file=sys.stderr, flush=True)

    pos = int(inp.pos0[0])
    c0 = (pos // 64) * 64
    q = gh.query_slice(st, 0)
    # raw K/V of the chunk that the new token completes (kept by the caller)
    kc = st.k_raw[:, :, c0:c0 + 64].contiguous()
    vc = st.v_raw[:, :, c0:c0 + 64].contiguous()
    R = max(1, args.replicas)
    reps = []
    for r in range(R):
        reps.append(dict(
            k_pool=st.k_pool if r == 0 else st.k_pool.clone(),
            v_pool=st.v_pool if r == 0 else st.v_pool.clone(),
            chunk_sum=st.chunk_sum if r == 0 else st.chunk_sum.clone(),
            group_sum=st.group_sum if r == 0 else st.group_sum.clone(),
            q=q if r == 0 else q.clone(), kc=kc if r == 0 else kc.clone(),
            vc=vc if r == 0 else vc.clone(), ws=torch.zeros_like(st.ws),
            s=gh.alloc_step(st, 1)))
    del st.k_raw, st.v_raw
    torch.cuda.synchronize()
    cfg = st.cfg
    stream = torch.cuda.current_stream()

    def step(r, ev=None):
        x = reps[r]
        hga.hga_build_summaries(cfg, B, x["kc"], x["vc"], c0, 64, x["k_pool"], x["v_pool"], T,
                                x["chunk_sum"], x["group_sum"], st.max_chunks, stream)
        s = x["s"]
        hga.hga_route(cfg, B, x["q"], 1, st.pos0, x["chunk_sum"], x["group_sum"], st.max_chunks,
                      s.sel, s.n_sel, st.max_sel, None, x["ws"], stream)
        if ev is not None:
            ev[0].record(stream)
        hga.hga_attend(cfg, B, x["q"], 1, st.pos0, x["k_pool"], x["v_pool"], hga.HGA_SRC_POOL, T,
                       s.sel, s.n_sel, st.max_sel, hga.HGA_PART_ALL, s.out, s.lse, x["ws"], stream)
        if ev is not None:
            ev[1].record(stream)

    for i in range(args.warmup):
        step(i % R)
    torch.cuda.synchronize()
    # whole-step timing
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        step(i % R)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_total = t0.elapsed_time(t1)
    ms_step = ms_total / args.steps
    # per-launch duration of the dominant kernel, events on its stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i in range(args.steps):
        step(i % R, evs[i])
    torch.cuda.synchronize()
    attend_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    s0 = reps[0]["s"]
    assert (s0.n_sel == st.max_sel).all().item() and torch.isfinite(s0.out).all().item()

    ab = algorithmic_bytes(p, B)
    achieved = ab["attend"] / (attend_ms * 1e-3) / 1e9
    out = {
        "metric": "routed-attention query tokens/s per layer at 64K ctx; achieved HBM GB/s vs peak",
        "value": B / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V, pre-RoPE)",
        "config": {"workload": "decode64k: GQA 32q/4kv heads, d=128, bf16, theta 1e6, ctx 65536, "
                               "batch 8 decode at t=65535, C=64 (4x16), 1 sink + 4 local chunks, "
                               "top-52 chunks, top-104 groups (2048 keys, 3.125%), pool in HBM",
                   "batch": B, "context": T, "replicas": R,
                   "step_bytes_algorithmic": ab["total"],
                   "step_GBps_algorithmic": ab["total"] / (ms_step * 1e-3) / 1e9},
        "roofline": {"kernel": "hga_attend (attend_decode_kernel)", "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "bytes_per_launch": ab["attend"], "launch_ms": attend_ms},
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(inp, p)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
