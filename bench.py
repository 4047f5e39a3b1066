"""Benchmark of the HGA decode hot path on one MI355X.

Workload: one decode step of a GQA attention layer (32 query / 4 KV heads,
head_dim 128, bf16, RoPE theta 1e6) at 65536 tokens of context, batch 8
independent sequences, query at position 65535.  C = 64 tokens per chunk in
4 groups of 16; 1 sink + 4 local chunks, top-52 chunks then top-104 groups,
so 2048 of 65536 keys (3.125 %) are attended per (sequence, KV head).

One step = the whole path for the new token of every sequence, one
hga_decode_step call on one stream (four launches):
  - the new token at 65535 is rotated into the pool, its raw key joins the
    chunk staging rows, and chunk 1023, which it completes, gets its chunk
    and group summaries (read by routing from the next step on);
  - routing: pooled query, level-1 scores of 1018 candidate chunks, top-52,
    level-2 scores of 208 groups, top-104, window merge;
  - exact softmax attention over the 128 selected groups with the gather
    fused into the loads, then the split merge.
Inputs are resident in HBM before timing.  The state (pool, summaries,
queries) is replicated R times at distinct addresses and the steps cycle
through the replicas, so the timed traffic comes from HBM and not from the
256 MB last-level cache.  The timed region replays a HIP graph holding R
consecutive steps.

Prints one JSON line.  ``value`` = decoded query tokens per second per layer
(B tokens per step), over exactly --steps graph-replayed steps;
``timing_distribution`` gives the per-step median, p10 and p90 over at least
1000 further replays (each between two events).  ``roofline`` covers the
dominant call, the longer of the routing call (tile + selection kernels) and
the attention call (split + merge kernels): algorithmic bytes per launch / its
mean launch duration, measured with HIP events around the calls on the launch
stream (the step run through the separate entry points) while a spin kernel
keeps the queue filled ahead (so host launch latency does not enter);
``roofline_other_call`` the other one; ``roofline_step`` the whole step's
algorithmic bytes over its graph-timed duration.  ``summary_build`` times the
bulk build of the whole context and the refresh of one completed chunk.
``cpu_baseline`` times the fp64 CPU oracle doing the same step, repeated for
about 10 s, on this host's cores, and on one thread (``single_thread``), with
the host CPU model.

``--workload prefill32k`` runs the chunked-prefill leg instead: one 64-token
query chunk at 32K context (append + summaries of the chunk, routing with the
pooled query, MFMA attention; one hga_prefill_step call), reported as query
tokens/s with the attention call's achieved TFLOP/s against the bf16 dense
MFMA peak.  ``--sweep`` prints one line per decode sweep point (context 4K to
64K, batch 8 to 32 at 64K) instead of the benchmark line.
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

# HBM traffic of the attention entry point (its split kernel plus its merge
# kernel), from two rocprofv3 --pmc passes over this bench (FETCH_SIZE, then
# WRITE_SIZE; KiB per dispatch, summed over the two kernels) and scaled by
# what the same counters read for a plain device copy of known size
# (bench.py --calibrate-copy).  Valid only for the kernel source it was taken
# on: if hga_attend.hip or hga_decode.hip has changed since, traffic is
# reported as null.
ATTEND_TRAFFIC = dict(
    source_sha256="cc38ba742d4ea0f51728196b44e428741e9ca90e81376bd039f78dec69db21e8",
    fetch_kib=16752.70 + 1448.19, write_kib=2080.02 + 136.00, fetch_scale=2.0, write_scale=1.0)


# The same for the routing entry point (its tile kernel plus its selection
# kernel), valid for the routing sources it was taken on.
ROUTE_TRAFFIC = dict(
    source_sha256="9e3ab9994fd6827c5c8a7759439521fe496c7511c2222ed124de0c7042b058c1",
    fetch_kib=8490.04 + 1957.72, write_kib=319.00 + 17.00, fetch_scale=2.0, write_scale=1.0)


def algorithmic_bytes(p, B):
    """Bytes the method must move per step at the decode workload."""
    d, hkv, hq = p["head_dim"], p["n_kv_heads"], p["n_q_heads"]
    g = p["chunk_size"] // p["groups_per_chunk"]
    max_sel = (p["n_sink_chunks"] + p["n_local_chunks"] + 1) * p["groups_per_chunk"] + p["topk_groups"]
    ct = p["query_pos0"] // p["chunk_size"]
    n_cand = ct - p["n_local_chunks"] - p["n_sink_chunks"]
    lists = hq if p.get("route_per_head") else hkv  # selected lists per sequence
    row = d + 4 if p.get("pool_dtype") == 1 else d * 2  # bytes per K (or V) row: FP8 + scale, or bf16
    kv = max_sel * g * row * 2 * lists           # selected K and V rows of every list
    q = hq * d * 2
    o = hq * d * 4
    idx = lists * max_sel * 4
    attend = B * (kv + q + o + idx)
    # level-1 rows of every list, level-2 rows of its kept chunks
    route = B * (n_cand * d * 4 * lists + p["topk_chunks"] * p["groups_per_chunk"] * d * 4 * lists
                 + q + idx)
    # new token: raw K, V in, rotated K, V out; refresh: 64 raw keys in, 1 + G rows out
    refresh = B * hkv * (4 * d * 2 + p["chunk_size"] * d * 2 + (1 + p["groups_per_chunk"]) * d * 4)
    return dict(attend=attend, route=route, refresh=refresh, total=attend + route + refresh)


def attend_source_sha():
    """sha256 of the decode attention sources (split kernel + merge kernel)."""
    import hashlib
    h = hashlib.sha256()
    for name in ("hga_attend.hip", "hga_decode.hip"):
        with open(os.path.join(ROOT, "long_context_hga_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def attend_traffic():
    """HBM bytes per hga_attend call from the stored counter figures, or None."""
    t = ATTEND_TRAFFIC
    if t is None or t["source_sha256"] != attend_source_sha():
        return None
    return t["fetch_kib"] * 1024 * t["fetch_scale"] + t["write_kib"] * 1024 * t["write_scale"]


def route_source_sha():
    """sha256 of the routing sources (tile and selection kernels)."""
    import hashlib
    h = hashlib.sha256()
    for name in ("hga_route.hip", "hga_topk.h"):
        with open(os.path.join(ROOT, "long_context_hga_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def route_traffic():
    """HBM bytes per hga_route call from the stored counter figures, or None."""
    t = ROUTE_TRAFFIC
    if t is None or t["source_sha256"] != route_source_sha():
        return None
    return t["fetch_kib"] * 1024 * t["fetch_scale"] + t["write_kib"] * 1024 * t["write_scale"]


def calibrate_copy(n_bytes=512 << 20, reps=4):
    """A plain device-to-device copy of known size, for scaling the FETCH_SIZE
    and WRITE_SIZE counters: each dispatch reads and writes n_bytes."""
    import torch
    src = torch.ones(n_bytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read_per_dispatch": n_bytes,
                      "bytes_written_per_dispatch": n_bytes, "dispatches": reps}), flush=True)


def calibrate_copy_rate(reps=50):
    """Read + write rate of plain device-to-device copies (calibration
    library kernels in five shapes, and torch's copy_) at the gather's size
    (the decode64k lists: 33.5 MB each way) and at 512 MiB: the ceiling a
    copy reaches on this device, next to the published 8 TB/s."""
    import ctypes
    import torch
    torch.cuda.init()
    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    lib = ctypes.CDLL(os.path.join(ROOT, "long_context_hga_amd", "libhga_calib.so"))
    f = lib.hga_calib_copy_rate
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    names = ["1 uint4 per thread", "4 uint4 per thread, loads first",
             "4 uint4 per thread, non-temporal", "8 uint4 per thread, loads first",
             "grid-stride, 8 workgroups per CU"]
    for n_bytes in (33554432, 512 << 20):
        src = torch.ones(n_bytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for v, name in enumerate(names):
            gb, ms = ctypes.c_double(), ctypes.c_double()
            rc = f(src.data_ptr(), dst.data_ptr(), n_bytes, v, reps, n_cus, ctypes.byref(gb),
                   ctypes.byref(ms))
            assert rc == 0, rc
            print(json.dumps({"calibration": "device copy rate", "kernel": name, "bytes": n_bytes,
                              "ms": ms.value, "GBps_read_plus_write": gb.value,
                              "frac_of_8TBps": gb.value / HBM_PEAK_GBS}), flush=True)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        dst.copy_(src)
        ev[0].record()
        for _ in range(reps):
            dst.copy_(src)
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / reps
        print(json.dumps({"calibration": "device copy rate", "kernel": "torch copy_", "bytes": n_bytes,
                          "ms": ms, "GBps_read_plus_write": 2 * n_bytes / (ms * 1e-3) / 1e9,
                          "frac_of_8TBps": 2 * n_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}),
              flush=True)
        del src, dst
    # what one CU pulls from HBM: few workgroups, each reading its own 1 MiB,
    # a fresh slice of a 2 GiB buffer per launch (no cache reuse)
    import numpy as np
    g = lib.hga_calib_cu_read_rate
    g.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                  ctypes.c_int, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    per = 1 << 20
    src = torch.ones(2048 * per, dtype=torch.uint8, device="cuda")
    out = torch.empty(256 * 1024, dtype=torch.int32, device="cuda")
    for n_wg, thr in ((32, 1024), (32, 256), (64, 1024), (256, 256)):
        ts = []
        for r in range(1, 2048 // n_wg):
            gb, ms = ctypes.c_double(), ctypes.c_double()
            rc = g(src.data_ptr() + r * n_wg * per, per, n_wg, thr, out.data_ptr(), 1,
                   ctypes.byref(gb), ctypes.byref(ms))
            assert rc == 0, rc
            ts.append(ms.value)
        t = float(np.median(ts))
        print(json.dumps({"calibration": "per-workgroup HBM read rate", "workgroups": n_wg,
                          "threads": thr, "bytes_per_workgroup": per, "launches": len(ts),
                          "us_median": t * 1e3, "GBps_per_workgroup": per / (t * 1e-3) / 1e9,
                          "GBps_total": n_wg * per / (t * 1e-3) / 1e9}), flush=True)
    del src, out


def calibrate_mfma(rounds=2500):
    """Dense bf16 rate that v_mfma_f32_16x16x32_bf16 and
    v_mfma_f32_32x32x16_bf16 reach on this device (all CUs, 1, 2 and 4 waves
    per SIMD), from the calibration library."""
    import ctypes
    import torch
    torch.cuda.init()
    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    lib = ctypes.CDLL(os.path.join(ROOT, "long_context_hga_amd", "libhga_calib.so"))
    f = lib.hga_calib_mfma_rate_shape
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    for shape, name in ((0, "v_mfma_f32_16x16x32_bf16"), (1, "v_mfma_f32_32x32x16_bf16"),
                        (2, "v_mfma_f32_16x16x32_bf16, distinct operands, 8 accumulators"),
                        (3, "v_mfma_f32_16x16x32_bf16, distinct operands, 16 accumulators")):
        for w in (1, 2, 4):
            tf, ms = ctypes.c_double(), ctypes.c_double()
            rc = f(n_cus, w, rounds, shape, ctypes.byref(tf), ctypes.byref(ms))
            assert rc == 0, rc
            print(json.dumps({"calibration": f"{name} issue rate", "cus": n_cus,
                              "waves_per_simd": w, "tflops": tf.value, "ms": ms.value,
                              "published_peak_tflops": 2500.0}), flush=True)


def calibrate_valu_decode(reps=200):
    """The decode attention split on the vector ALUs (a calibration kernel of
    libhga_calib.so, not part of the library) against the library's
    matrix-core split, on the same decode64k lists: the two outputs compared,
    both calls (split + merge) event-timed with the queue filled ahead.  The
    calls alternate on one state, so each reads the selected K/V under the
    same cache conditions as the other."""
    import ctypes
    import math
    import numpy as np
    import torch
    import gpu_harness as gh
    import synth
    torch.cuda.init()
    inp = synth.generate("decode64k")
    st = gh.build_state(inp)
    p = inp.params
    B, T, d, hkv, hq = st.B, st.T, p["head_dim"], p["n_kv_heads"], p["n_q_heads"]
    q = gh.query_slice(st, 0)
    s = gh.alloc_step(st, 1)
    gh.route(st, q, 1, st.pos0, s)
    gh.attend(st, q, 1, st.pos0, s)
    torch.cuda.synchronize()
    vrows = gh.v_token_view(st.v_pool).contiguous()  # token rows [B][Hkv][T/16][16][d]
    assert vrows.numel() == B * hkv * T * d
    omega = (ctypes.c_double * (d // 2))(*[p["rope_theta"] ** (-2.0 * j / d) for j in range(d // 2)])
    splits = (st.max_sel + 7) // 8
    part = torch.empty(B * hkv * splits * (16 + 8 * d), dtype=torch.float32, device="cuda")
    out = torch.full((B, hq, d), float("nan"), dtype=torch.float32, device="cuda")
    lib = ctypes.CDLL(os.path.join(ROOT, "long_context_hga_amd", "libhga_calib.so"))
    f = lib.hga_calib_valu_decode
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, ctypes.POINTER(ctypes.c_double), ctypes.c_float, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p]
    qscale = math.log2(math.e) / math.sqrt(d)

    def valu():
        rc = f(q.data_ptr(), st.pos0.data_ptr(), st.k_pool.data_ptr(), vrows.data_ptr(), T,
               s.sel.data_ptr(), s.n_sel.data_ptr(), st.max_sel, B, hq, hkv, omega, qscale,
               part.data_ptr(), out.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert rc == 0, rc

    def mfma():
        gh.attend(st, q, 1, st.pos0, s)

    valu()
    torch.cuda.synchronize()
    ref = s.out[:, :, 0, :]
    assert torch.isfinite(out).all().item()
    diff = (out - ref).abs().max().item()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
    torch.cuda._sleep(int(2e8))
    for e in ev:
        e[0].record()
        mfma()
        e[1].record()
        valu()
        e[2].record()
    torch.cuda.synchronize()
    t_mfma = float(np.median([e[0].elapsed_time(e[1]) for e in ev]))
    t_valu = float(np.median([e[1].elapsed_time(e[2]) for e in ev]))
    kv_bytes = int(s.n_sel.sum().item()) * 16 * d * 2 * 2
    print(json.dumps({"calibration": "decode attention split + merge: vector ALUs vs matrix cores",
                      "workload": "decode64k lists (batch 8, 2048 selected keys per sequence and KV head)",
                      "max_abs_diff_vs_library": diff, "selected_kv_bytes": kv_bytes,
                      "mfma_call_ms": t_mfma, "valu_call_ms": t_valu,
                      "mfma_GBps": kv_bytes / (t_mfma * 1e-3) / 1e9,
                      "valu_GBps": kv_bytes / (t_valu * 1e-3) / 1e9, "reps": reps}), flush=True)
    assert diff < 1e-4, diff


def cpu_baseline(inp, cfg_params, min_seconds=10.0):
    """The fp64 C oracle doing the same step (append + chunk refresh + route +
    attend for every sequence of the batch), repeated for about min_seconds."""
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
    t_sum = 0.0  # the summary builds of the completed chunks, timed (one thread each)
    for b in range(B):
        for h in range(hkv):
            u = b * hkv + h
            kr = inp.f64(inp.k[b, h])
            t0 = time.perf_counter()
            a, g = oracle.summaries(cfg, kr[:c0])
            t_sum += time.perf_counter() - t0
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
        for u in range(U):  # append of the new token, refresh of the chunk it completes
            kp[u, pos] = oracle.pool(cfg, kraw[u][pos - c0:pos - c0 + 1], pos)[0]
            cs[u, c0 // 64] = oracle.span_summary(cfg, kraw[u], c0)
            for i in range(4):
                gs[u, c0 // 16 + i] = oracle.span_summary(cfg, kraw[u][16 * i:16 * i + 16], c0 + 16 * i)
        oracle.step(cfg, q, np.full(U, pos), cs, gs, kp, vp, max_sel)
        times.append(time.perf_counter() - t0)
    med = float(np.median(times))
    total = time.perf_counter() - t_start
    # the same step on one thread (route + attend of every unit; fewer runs)
    threads = oracle.max_threads()
    oracle.set_threads(1)
    t1s = []
    t_one = time.perf_counter()
    try:
        while len(t1s) < 2 or time.perf_counter() - t_one < min_seconds / 2:
            t0 = time.perf_counter()
            oracle.step(cfg, q, np.full(U, pos), cs, gs, kp, vp, max_sel)
            t1s.append(time.perf_counter() - t0)
    finally:
        oracle.set_threads(threads)
    med1 = float(np.median(t1s))
    return {"value": B / med, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "host_cpu": host_cpu_model(),
            "sample": f"the full step: all {B} sequences x {hkv} KV heads, append + chunk refresh + "
                      f"route + attend of one decode token at position {pos} (context {T}); fp64 C "
                      f"oracle, OpenMP over the {U} units; median of {len(times)} runs "
                      f"({med * 1e3:.1f} ms each, {total:.1f} s total)",
            "single_thread": {"value": B / med1, "unit": "tokens/s", "cores": 1,
                              "sample": f"route + attend of the same {U} units on one thread "
                                        f"(no append or refresh); median of {len(t1s)} runs "
                                        f"({med1 * 1e3:.1f} ms each)"},
            "summary_build": {"value": U * c0 / t_sum / 1e6, "unit": "M token rows/s", "cores": 1,
                              "sample": f"chunk and group summaries of the {c0} completed tokens "
                                        f"of each of the {U} units, one thread ({t_sum:.2f} s in "
                                        f"all)"}}


def host_cpu_model():
    """The host CPU's model name and logical CPU count, from /proc/cpuinfo."""
    try:
        names = [l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo")
                 if l.startswith("model name")]
        return f"{names[0]} ({len(names)} logical CPUs visible)" if names else None
    except OSError:
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--workload", default="decode64k",
                    choices=["decode64k", "prefill32k", "host64k", "prompt32k"],
                    help="decode64k (default): the batch-8 64K decode step; prefill32k: one "
                         "64-token query chunk at 32K context (MFMA attention); host64k: "
                         "batch-4 64K decode with the pool in pinned host memory")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--replays", type=int, default=1000,
                    help="graph replays of the per-step timing distribution (at least)")
    ap.add_argument("--profile-calls", type=int, default=0, metavar="N",
                    help="decode64k: only run N steps through the separate entry points "
                         "(append, hga_route, hga_attend, chunk refresh, hga_gather), no "
                         "graphs and no spin kernels, for hardware-counter runs")
    ap.add_argument("--fp8", action="store_true",
                    help="host64k: the K/V pool (host, windows, working sets, cache) in FP8")
    ap.add_argument("--sweep", action="store_true",
                    help="decode sweep over context 4K..64K and batch 8..32 (one JSON line "
                         "per point) instead of the benchmark line")
    ap.add_argument("--calibrate-mfma", action="store_true",
                    help="only measure the dense bf16 rate of v_mfma_f32_16x16x32_bf16 at 1, 2 and 4 "
                         "waves per SIMD")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 512 MiB device copy (counter calibration)")
    ap.add_argument("--calibrate-copy-rate", action="store_true",
                    help="only measure plain device copies (the copy ceiling of the gather)")
    ap.add_argument("--calibrate-valu-decode", action="store_true",
                    help="only compare the decode attention on the vector ALUs (calibration "
                         "kernel) with the library's matrix-core decode on the decode64k lists")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the decode path is "
              "per-GPU and this build has no multi-GPU leg", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.calibrate_copy_rate:
        calibrate_copy_rate()
        return
    if args.calibrate_mfma:
        calibrate_mfma()
        return
    if args.calibrate_valu_decode:
        calibrate_valu_decode()
        return
    if args.sweep:
        run_sweep(args)
        return
    if args.workload == "prefill32k":
        run_prefill32k(args)
    elif args.workload == "prompt32k":
        run_prompt32k(args)
    elif args.workload == "host64k":
        run_host64k(args)
    else:
        run_decode64k(args)


def run_decode64k(args):
    out, inp = measure_decode(args, "decode64k")
    if out is None:  # --profile-calls
        return
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(inp, inp.params)
    print(json.dumps(out), flush=True)


def measure_decode(args, name, batch=None, context=None, overrides=None, replicas=None):
    """Time the fused decode step of workload ``name`` (optionally resized)
    as a replayed HIP graph, and the attend / route calls with events.
    Returns the result line (without cpu_baseline, None with
    --profile-calls) and the inputs."""
    import numpy as np
    import torch

    import gpu_harness as gh
    import long_context_hga_amd as hga
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    t_gen = time.time()
    inp = synth.generate(name, batch=batch, context=context, overrides=overrides)
    p = inp.params
    B, T = p["batch"], p["context"]
    st = gh.build_state(inp)
    torch.cuda.synchronize()
    print(f"[bench] state built in {time.time() - t_gen:.1f}s", file=sys.stderr, flush=True)

    pos = int(inp.pos0[0])
    c0 = (pos // 64) * 64
    # selected lists per sequence: one per query head when routing per head;
    # a working set holds max_sel groups of every list
    lists = p["n_q_heads"] if p.get("route_per_head") else p["n_kv_heads"]
    q = gh.query_slice(st, 0)
    # raw K/V of the new token; raw keys of the chunk it completes (the
    # staging rows of the fused step, and the chunk input of the separate
    # summary call)
    kt = st.k_raw[:, :, pos:pos + 1].contiguous()
    vt = st.v_raw[:, :, pos:pos + 1].contiguous()
    kc = st.k_raw[:, :, c0:c0 + 64].contiguous()
    if p.get("pool_dtype") == 1:  # the FP8 pool: codes then row scales, built from the raw K/V
        nbytes = B * p["n_kv_heads"] * T * (p["head_dim"] + 4)
        st.k_pool = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        st.v_pool = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        hga.hga_build_summaries(st.cfg, B, st.k_raw, st.v_raw, 0, T, st.k_pool, st.v_pool, T, None,
                                None, st.max_chunks)
        torch.cuda.synchronize()
    R = max(1, args.replicas if replicas is None else replicas)
    reps = []
    for r in range(R):
        reps.append(dict(
            k_pool=st.k_pool if r == 0 else st.k_pool.clone(),
            v_pool=st.v_pool if r == 0 else st.v_pool.clone(),
            chunk_sum=st.chunk_sum if r == 0 else st.chunk_sum.clone(),
            group_sum=st.group_sum if r == 0 else st.group_sum.clone(),
            q=q if r == 0 else q.clone(), kt=kt if r == 0 else kt.clone(),
            vt=vt if r == 0 else vt.clone(), kc=kc if r == 0 else kc.clone(),
            stage=kc.clone(), ws=torch.zeros_like(st.ws), s=gh.alloc_step(st, 1)))
    del st.k_raw, st.v_raw
    torch.cuda.synchronize()
    cfg = st.cfg

    def step(r):
        # The fused decode step (four launches): level-1 scores; selection
        # with the token's pool append and the completed chunk's summaries
        # in extra workgroups; attention; split merge.  stream=None: the
        # binding enqueues on torch's current stream (the capture stream
        # inside torch.cuda.graph).
        x = reps[r]
        s = x["s"]
        hga.hga_decode_step(cfg, B, x["q"], x["kt"], x["vt"], st.pos0, x["k_pool"], x["v_pool"], T,
                            x["stage"], x["chunk_sum"], x["group_sum"], st.max_chunks, s.sel,
                            s.n_sel, st.max_sel, s.out, s.lse, x["ws"])

    def step_parts(r, ev):
        # The same step through the separate entry points, with events around
        # the route and attend calls (per-call durations).
        x = reps[r]
        s = x["s"]
        hga.hga_build_summaries(cfg, B, x["kt"], x["vt"], pos, 1, x["k_pool"], x["v_pool"], T,
                                None, None, st.max_chunks)
        if ev:
            ev[0].record()
        hga.hga_route(cfg, B, x["q"], 1, st.pos0, x["chunk_sum"], x["group_sum"], st.max_chunks,
                      s.sel, s.n_sel, st.max_sel, None, x["ws"])
        if ev:
            ev[1].record()
        hga.hga_attend(cfg, B, x["q"], 1, st.pos0, x["k_pool"], x["v_pool"], hga.HGA_SRC_POOL, T,
                       s.sel, s.n_sel, st.max_sel, hga.HGA_PART_ALL, s.out, s.lse, x["ws"])
        if ev:
            ev[2].record()
        hga.hga_build_summaries(cfg, B, x["kc"], None, c0, 64, None, None, T, x["chunk_sum"],
                                x["group_sum"], st.max_chunks)

    if args.profile_calls:
        # counter runs: only the separate-entry calls, synchronised once
        kw = torch.empty((B, lists, st.max_sel * 16, p["head_dim"]),
                         dtype=reps[0]["k_pool"].dtype, device="cuda")
        vw = torch.empty_like(kw)
        assert kw.numel() == B * reps[0]["s"].sel.shape[1] * st.max_sel * 16 * p["head_dim"]
        for i in range(args.profile_calls):
            x = reps[i % R]
            step_parts(i % R, None)
            hga.hga_gather(cfg, B, x["k_pool"], x["v_pool"], T, 0, x["s"].sel, x["s"].n_sel,
                           st.max_sel, st.pos0, hga.HGA_PART_ALL, kw, vw)
        torch.cuda.synchronize()
        print(f"[bench] {args.profile_calls} separate-entry steps + gathers done", file=sys.stderr,
              flush=True)
        return None, inp

    for i in range(max(args.warmup, R)):
        step(i % R)
    torch.cuda.synchronize()
    eager_out = [x["s"].out.clone() for x in reps]

    # whole-step throughput: HIP graphs of consecutive steps (one per
    # replica); the timed region replays them for exactly --steps steps, then
    # the per-step distribution over many more replays
    ms_step, steps_timed, dist = time_graph_exact(step, R, args, min_replays=args.replays)
    for r, x in enumerate(reps):  # graph replays reproduce the eager results
        assert torch.equal(x["s"].out, eager_out[r]), "graph replay differs from eager run"

    # per-launch kernel durations: events on the launch stream around each
    # call, with the queue filled ahead (a spin kernel holds the GPU while
    # the host enqueues) so host launch latency does not enter the figures
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda._sleep(int(2e8))
    for i in range(args.steps):
        step_parts(i % R, evs[i])
    torch.cuda.synchronize()
    route_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    attend_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    for r, x in enumerate(reps):  # the separate calls give the fused step's bits
        assert torch.equal(x["s"].out, eager_out[r]), "separate calls differ from the fused step"
    s0 = reps[0]["s"]
    assert (s0.n_sel == st.max_sel).all().item() and torch.isfinite(s0.out).all().item()

    # hga_gather from the HBM pool into a working set (the same lists): its
    # own copy rate, read + write (bf16 pool)
    gather_ms, gather_bytes, copy_ms = float("nan"), 0, float("nan")
    if p.get("pool_dtype", 0) == 0:
        kw = torch.empty((B, lists, st.max_sel * 16, p["head_dim"]),
                         dtype=reps[0]["k_pool"].dtype, device="cuda")
        vw = torch.empty_like(kw)
        # the gather writes max_sel groups of every list of every sequence
        assert kw.numel() == B * reps[0]["s"].sel.shape[1] * st.max_sel * 16 * p["head_dim"]
        gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(20)]
        for x in reps:  # first launches (code load, caches) stay out of the timing
            hga.hga_gather(cfg, B, x["k_pool"], x["v_pool"], T, 0, x["s"].sel, x["s"].n_sel,
                           st.max_sel, st.pos0, hga.HGA_PART_ALL, kw, vw)
        torch.cuda.synchronize()
        torch.cuda._sleep(int(1e8))
        for i, (e0, e1) in enumerate(gev):
            x = reps[i % R]
            e0.record()
            hga.hga_gather(cfg, B, x["k_pool"], x["v_pool"], T, 0, x["s"].sel, x["s"].n_sel,
                           st.max_sel, st.pos0, hga.HGA_PART_ALL, kw, vw)
            e1.record()
        torch.cuda.synchronize()
        gather_ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in gev]))
        gather_bytes = 2 * int(reps[0]["s"].n_sel.sum().item()) * 16 * p["head_dim"] * 2 * 2
        del kw, vw
        copy_ms = copy_rate_ms(gather_bytes // 2)

    # summary build: the bulk build of the whole context (every unit's pool
    # and summaries) and the refresh of one completed chunk, event-timed
    build_ms, chunk_ms = float("nan"), float("nan")
    if p.get("pool_dtype", 0) == 0:
        x = reps[0]
        shape = (B, p["n_kv_heads"], T, p["head_dim"])
        kraw = torch.randn(shape, device="cuda").to(torch.bfloat16).view(x["kc"].dtype)
        vraw = torch.randn(shape, device="cuda").to(torch.bfloat16).view(x["kc"].dtype)
        be = [torch.cuda.Event(enable_timing=True) for _ in range(3)]

        def bulk():
            hga.hga_build_summaries(cfg, B, kraw, vraw, 0, T, x["k_pool"], x["v_pool"], T,
                                    x["chunk_sum"], x["group_sum"], st.max_chunks)
        bulk()  # warm
        torch.cuda.synchronize()
        torch.cuda._sleep(int(1e8))
        be[0].record()
        bulk()
        be[1].record()
        for _ in range(20):
            hga.hga_build_summaries(cfg, B, x["kc"], None, c0, 64, None, None, T, x["chunk_sum"],
                                    x["group_sum"], st.max_chunks)
        be[2].record()
        torch.cuda.synchronize()
        build_ms = be[0].elapsed_time(be[1])
        chunk_ms = be[1].elapsed_time(be[2]) / 20
        del kraw

    ab = algorithmic_bytes(p, B)
    calls = {
        "hga_route call (tile + selection kernels)": (route_ms, ab["route"]),
        "hga_attend call (split + merge kernels)": (attend_ms, ab["attend"]),
    }
    dom = max(calls, key=lambda k: calls[k][0])  # the call that takes longest
    def roof(name, traffic):
        ms, nb = calls[name]
        ach = nb / (ms * 1e-3) / 1e9
        return {"kernel": name, "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": ach / HBM_PEAK_GBS, "traffic": traffic,
                "bytes_per_launch": nb, "launch_ms": ms}
    traffic = {"hga_attend call (split + merge kernels)": attend_traffic(),
               "hga_route call (tile + selection kernels)": route_traffic()}
    step_gbs = ab["total"] / (ms_step * 1e-3) / 1e9
    out = {
        "metric": "routed-attention query tokens/s per layer at 64K ctx; achieved HBM GB/s vs peak",
        "value": B / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps_timed,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V, pre-RoPE)",
        "config": {"workload": f"{name}: GQA {p['n_q_heads']}q/{p['n_kv_heads']}kv heads, "
                               f"d={p['head_dim']}, bf16, theta {p['rope_theta']:g}, ctx {T}, "
                               f"batch {B} decode at t={pos}, C=64 (4x16), "
                               f"{p['n_sink_chunks']} sink + {p['n_local_chunks']} local chunks, "
                               f"top-{p['topk_chunks']} chunks, top-{p['topk_groups']} groups "
                               f"({st.max_sel * 16} keys, {100.0 * st.max_sel * 16 / T:.3g}%), "
                               + ("one list per query head, " if p.get("route_per_head") else "")
                               + ("FP8 pool (E4M3FN + row scales) " if p.get("pool_dtype") == 1 else "")
                               + "pool in HBM",
                   "batch": B, "context": T, "replicas": R,
                   "timing": "HIP graph of R steps, replayed",
                   "step_bytes_algorithmic": ab["total"],
                   "step_GBps_algorithmic": ab["total"] / (ms_step * 1e-3) / 1e9},
        "timing_distribution": dist,
        "roofline": roof(dom, traffic[dom]),
        "roofline_other_call": [roof(k, traffic[k]) for k in calls if k != dom][0],
        "roofline_step": {"scope": "whole fused step (graph-timed), algorithmic bytes of the "
                                   "append, chunk refresh, routing and attention",
                          "bound": "hbm", "achieved": step_gbs, "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": step_gbs / HBM_PEAK_GBS,
                          "bytes_per_step": ab["total"], "ms_per_step": ms_step},
        "summary_build": {"bulk_ms": build_ms, "bulk_tokens": B * p["n_kv_heads"] * T,
                          "bulk_Mtokens_per_s": B * p["n_kv_heads"] * T / (build_ms * 1e-3) / 1e6,
                          "chunk_refresh_ms": chunk_ms,
                          "note": "bulk: hga_build_summaries over the whole context of every "
                                  "unit (rotated K and V pool rows, summaries of every chunk); "
                                  "chunk: the summaries of one completed 64-token chunk of "
                                  "every unit"},
        "gather_hbm": {"kernel": "hga_gather, HBM pool -> HBM working set (same lists)",
                       "launch_ms": gather_ms, "bytes_read_and_written": gather_bytes,
                       "achieved_GBps": gather_bytes / (gather_ms * 1e-3) / 1e9,
                       "frac_of_8TBps": gather_bytes / (gather_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                       "device_copy_GBps": gather_bytes / (copy_ms * 1e-3) / 1e9,
                       "frac_of_device_copy": copy_ms / gather_ms,
                       "device_copy_note": "a contiguous device-to-device copy of the same "
                                           "bytes (torch copy_, event-timed): the rate a plain "
                                           "read + write stream reaches on this device"},
    }
    del reps, st
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out, inp


# Decode sweep: context 4K..64K and batch 8..32 at 64K.  4K is the 4K decode
# workload as defined (batch 1, top-8 chunks, top-16 groups); 8K and 16K keep
# its budget at batch 8 (the windows alone are 384 tokens, above 3.125 % of
# 8K); 32K and 64K use the 3.125 % budgets of the 32K and 64K workloads.  Then
# one point routes per query head (one list per head instead of per KV head)
# and two read the FP8 pool (E4M3FN codes with row scales).
SWEEP = [
    ("decode4k", None, None, None),
    ("decode64k", 8, 8192, dict(topk_chunks=8, topk_groups=16)),
    ("decode64k", 8, 16384, dict(topk_chunks=8, topk_groups=16)),
    ("decode64k", 8, 32768, dict(topk_chunks=20, topk_groups=40)),
    ("decode64k", 8, 65536, None),
    ("decode64k", 16, 65536, None),
    ("decode64k", 32, 65536, None),
    ("decode64k", 8, 65536, dict(route_per_head=1)),
    ("decode64k", 8, 65536, dict(pool_dtype=1)),
    ("decode64k", 32, 65536, dict(pool_dtype=1)),
]


def run_sweep(args):
    """One JSON line per sweep point: whole-step tokens/s and the attention
    call's achieved GB/s against the HBM peak."""
    for name, batch, context, over in SWEEP:
        B = batch or 1
        R = args.replicas if B <= 8 else max(2, args.replicas * 8 // B)
        print(f"[sweep] {name} batch {batch} context {context} {over or ''} replicas {R}",
              file=sys.stderr, flush=True)
        out, _ = measure_decode(args, name, batch=batch, context=context, overrides=over,
                                replicas=R)
        c = out["config"]
        calls = (out["roofline"], out["roofline_other_call"])
        r = [x for x in calls if x["kernel"].startswith("hga_attend")][0]
        rr = [x for x in calls if x["kernel"].startswith("hga_route")][0]
        print(json.dumps({"sweep": "decode", "workload": c["workload"], "context": c["context"],
                          "batch": c["batch"], "tokens_per_s": out["value"],
                          "ms_per_step": out["ms_per_step"],
                          "median_us": out["timing_distribution"]["median_us"],
                          "step_GBps_algorithmic": c["step_GBps_algorithmic"],
                          "attend_ms": r["launch_ms"], "attend_bytes": r["bytes_per_launch"],
                          "attend_GBps": r["achieved"], "attend_frac_of_8TBps": r["frac"],
                          "route_ms": rr["launch_ms"]}), flush=True)


def prefill_algorithmic(p):
    """Algorithmic flops and bytes of attending one query chunk (lq = C
    tokens of chunk c_q) over its selected set, per the method: QK^T and PV
    over the visible keys (all window and routed keys; current-chunk keys
    up to each token)."""
    d, hq, hkv = p["head_dim"], p["n_q_heads"], p["n_kv_heads"]
    C, G = p["chunk_size"], p["groups_per_chunk"]
    g = C // G
    n_sel = (p["n_sink_chunks"] + p["n_local_chunks"] + 1) * G + p["topk_groups"]
    prior = (n_sel - G) * g              # keys before the query chunk
    visits = C * prior + C * (C + 1) // 2  # (query, key) pairs per head
    flops = hq * visits * d * 2 * 2
    kv = hkv * n_sel * g * d * 2 * 2
    q = hq * C * d * 2
    o = hq * C * d * 4
    return dict(flops=flops, attend_bytes=kv + q + o + hkv * n_sel * 4, n_sel=n_sel)


def cpu_baseline_prefill(inp, cfg_params, min_seconds=10.0):
    """The fp64 C oracle doing the prefill step: the query chunk's pool append
    and summaries, then routing and attention of its 64 tokens, for every KV
    head, repeated for about min_seconds."""
    import numpy as np
    import oracle
    cfg = oracle.cfg_from(cfg_params)
    p = cfg_params
    d, hkv = p["head_dim"], p["n_kv_heads"]
    hg = p["n_q_heads"] // hkv
    B, T, lq = inp.k.shape[0], inp.k.shape[2], inp.q.shape[2]
    pos = int(inp.pos0[0])
    U = B * hkv
    cs = np.zeros((U, T // 64, d))
    gs = np.zeros((U, T // 16, d))
    kp = np.zeros((U, T, d))
    vp = np.zeros((U, T, d))
    kraw = []
    for b in range(B):
        for h in range(hkv):
            u = b * hkv + h
            kr = inp.f64(inp.k[b, h])
            a, g = oracle.summaries(cfg, kr[:pos])
            cs[u, :a.shape[0]] = a
            gs[u, :g.shape[0]] = g
            kp[u, :pos] = oracle.pool(cfg, kr[:pos], 0)
            vp[u] = inp.f64(inp.v[b, h])
            kraw.append(kr[pos:pos + lq].copy())
    q = np.stack([inp.f64(inp.q[b, h * hg:(h + 1) * hg]) for b in range(B) for h in range(hkv)])
    max_sel = (p["n_sink_chunks"] + p["n_local_chunks"] + 1) * 4 + p["topk_groups"]
    times = []
    t_start = time.perf_counter()
    while len(times) < 5 or time.perf_counter() - t_start < min_seconds:
        t0 = time.perf_counter()
        for u in range(U):
            kp[u, pos:pos + lq] = oracle.pool(cfg, kraw[u], pos)
            cs[u, pos // 64] = oracle.span_summary(cfg, kraw[u], pos)
            for i in range(4):
                gs[u, pos // 16 + i] = oracle.span_summary(cfg, kraw[u][16 * i:16 * i + 16], pos + 16 * i)
        oracle.step(cfg, q, np.full(U, pos), cs, gs, kp, vp, max_sel)
        times.append(time.perf_counter() - t0)
    med = float(np.median(times))
    return {"value": B * lq / med, "unit": "tokens/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"the full prefill step: {hkv} KV heads, append + summaries of the {lq}-token "
                      f"query chunk at {pos}, route + attend of its {lq} tokens (context {T}); "
                      f"fp64 C oracle, OpenMP over the {U} units; median of {len(times)} runs "
                      f"({med * 1e3:.1f} ms each, {time.perf_counter() - t_start:.1f} s total)"}


def run_prefill32k(args):
    import numpy as np
    import torch

    import gpu_harness as gh
    import long_context_hga_amd as hga
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    inp = synth.generate("prefill32k")
    p = inp.params
    B, T = p["batch"], p["context"]
    pos = int(inp.pos0[0])
    lq = inp.q.shape[2]
    st = gh.build_state(inp)
    torch.cuda.synchronize()
    kc = st.k_raw[:, :, pos:pos + lq].contiguous()
    vc = st.v_raw[:, :, pos:pos + lq].contiguous()
    R = max(1, args.replicas)
    reps = []
    for r in range(R):
        reps.append(dict(
            k_pool=st.k_pool if r == 0 else st.k_pool.clone(),
            v_pool=st.v_pool if r == 0 else st.v_pool.clone(),
            chunk_sum=st.chunk_sum if r == 0 else st.chunk_sum.clone(),
            group_sum=st.group_sum if r == 0 else st.group_sum.clone(),
            q=st.q if r == 0 else st.q.clone(), kc=kc if r == 0 else kc.clone(),
            vc=vc if r == 0 else vc.clone(), stage=torch.zeros_like(kc),
            ws=torch.zeros_like(st.ws), s=gh.alloc_step(st, lq)))
    del st.k_raw, st.v_raw
    torch.cuda.synchronize()
    cfg = st.cfg

    def step(r, ev=None):
        # the query chunk's K/V enter the pool (and its summaries are built),
        # then its 64 tokens are routed (pooled query) and attended: one
        # hga_prefill_step (four launches); with events, the same work through
        # the separate entry points, timing the route and attend calls
        x = reps[r]
        s = x["s"]
        if ev is None:
            hga.hga_prefill_step(cfg, B, x["q"], lq, x["kc"], x["vc"], st.pos0, x["k_pool"],
                                 x["v_pool"], T, x["stage"], x["chunk_sum"], x["group_sum"],
                                 st.max_chunks, s.sel, s.n_sel, st.max_sel, s.out, s.lse, x["ws"])
            return
        hga.hga_build_summaries(cfg, B, x["kc"], x["vc"], pos, lq, x["k_pool"], x["v_pool"], T,
                                x["chunk_sum"], x["group_sum"], st.max_chunks)
        ev[0].record()
        hga.hga_route(cfg, B, x["q"], lq, st.pos0, x["chunk_sum"], x["group_sum"], st.max_chunks,
                      s.sel, s.n_sel, st.max_sel, None, x["ws"])
        ev[1].record()
        hga.hga_attend(cfg, B, x["q"], lq, st.pos0, x["k_pool"], x["v_pool"], hga.HGA_SRC_POOL, T,
                       s.sel, s.n_sel, st.max_sel, hga.HGA_PART_ALL, s.out, s.lse, x["ws"])
        ev[2].record()

    ms_step, steps_timed = time_graph(step, R, args)
    fused_out = [x["s"].out.clone() for x in reps]
    route_ms, attend_ms = time_launches(step, R, args)
    for r, x in enumerate(reps):  # the separate calls give the fused step's bits
        assert torch.equal(x["s"].out, fused_out[r]), "separate calls differ from the fused step"
    s0 = reps[0]["s"]
    assert torch.isfinite(s0.out).all().item()
    alg = prefill_algorithmic(p)
    achieved = alg["flops"] / (attend_ms * 1e-3) / 1e12
    out = {
        "metric": "routed-attention query tokens/s per layer, chunked prefill at 32K ctx; "
                  "MFMA utilisation",
        "value": B * lq / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps_timed,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V, pre-RoPE, 16 planted needle chunks)",
        "config": {"workload": "prefill32k: GQA 32q/4kv heads, d=128, bf16, theta 1e6, ctx 32768, "
                               "query chunk 511 (64 tokens at 32704..32767), 1 sink + 4 local "
                               "chunks, top-20 chunks, top-40 groups (1024 keys, 3.125%)",
                   "batch": B, "context": T, "query_tokens": lq, "replicas": R,
                   "timing": "HIP graph of R hga_prefill_step calls, replayed"},
        "roofline": {"kernel": "hga_attend (MFMA prefill split + merge kernels)", "bound": "mfma",
                     "achieved": achieved, "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": achieved / 2500.0, "traffic": None,
                     "flops_per_launch": alg["flops"], "launch_ms": attend_ms,
                     "hbm_bytes_per_launch": alg["attend_bytes"],
                     "route_launch_ms": route_ms},
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline_prefill(inp, p)
    print(json.dumps(out), flush=True)


def prompt_flops(n_sel, sel, p):
    """Algorithmic flops of attending every query chunk of the prompt over its
    list: QK^T and PV over the visible (query, key) pairs (every key of a
    group before the chunk; keys up to each token inside it)."""
    import numpy as np
    d, hq, hkv = p["head_dim"], p["n_q_heads"], p["n_kv_heads"]
    C, g = p["chunk_size"], p["chunk_size"] // p["groups_per_chunk"]
    hg = hq // hkv
    B, nq = n_sel.shape[0], n_sel.shape[1]
    pairs = 0
    for b in range(B):
        for qc in range(nq):
            for h in range(hkv):
                gids = sel[b, qc, h, :n_sel[b, qc, h]]
                cur = gids[gids // (C // g) == qc]          # groups of the query chunk
                prior = len(gids) - len(cur)
                pairs += prior * g * C
                for gid in cur:                             # key p visible to tau >= p
                    first = int(gid) * g - qc * C
                    pairs += sum(C - (first + i) for i in range(g))
    return int(pairs) * hg * d * 2 * 2


def cpu_baseline_prompt(inp, cfg_params, chunks=(508, 509, 510, 511)):
    """The fp64 C oracle doing the whole-prompt prefill: the pool append and
    summaries of the whole prompt (timed once), route + attend of a sample of
    query chunks (all KV heads), scaled to tokens per second of the prompt."""
    import numpy as np
    import oracle
    cfg = oracle.cfg_from(cfg_params)
    p = cfg_params
    d, hkv = p["head_dim"], p["n_kv_heads"]
    hg = p["n_q_heads"] // hkv
    B, T = inp.k.shape[0], inp.k.shape[2]
    U = B * hkv
    t0 = time.perf_counter()
    cs = np.zeros((U, T // 64, d))
    gs = np.zeros((U, T // 16, d))
    kp = np.zeros((U, T, d))
    vp = np.zeros((U, T, d))
    for b in range(B):
        for h in range(hkv):
            u = b * hkv + h
            kr = inp.f64(inp.k[b, h])
            cs[u], gs[u] = oracle.summaries(cfg, kr)
            kp[u] = oracle.pool(cfg, kr, 0)
            vp[u] = inp.f64(inp.v[b, h])
    t_append = time.perf_counter() - t0
    max_sel = (p["n_sink_chunks"] + p["n_local_chunks"] + 1) * 4 + p["topk_groups"]
    t0 = time.perf_counter()
    for qc in chunks:
        q = np.stack([inp.f64(inp.q[b, h * hg:(h + 1) * hg, qc * 64:(qc + 1) * 64])
                      for b in range(B) for h in range(hkv)])
        oracle.step(cfg, q, np.full(U, qc * 64), cs, gs, kp, vp, max_sel)
    t_chunks = time.perf_counter() - t0
    per_token = t_append / T + t_chunks / (len(chunks) * 64)
    return {"value": 1.0 / per_token * B, "unit": "tokens/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"pool append + summaries of the whole {T}-token prompt ({t_append:.1f} s, "
                      f"{hkv} KV heads) plus route + attend of query chunks "
                      f"{chunks[0]}..{chunks[-1]} (full budget, {t_chunks:.1f} s), scaled per "
                      f"token; fp64 C oracle, OpenMP over the {U} units"}


def run_prompt32k(args):
    """Whole-prompt chunked prefill of a 32K prompt: one hga_prefill_prompt call
    appends the prompt (pool + summaries), routes its 512 query chunks and
    attends them on the matrix cores."""
    import numpy as np
    import torch

    import gpu_harness as gh
    import long_context_hga_amd as hga
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    inp = synth.generate("prompt32k")
    p = inp.params
    B, T = p["batch"], p["context"]
    nq = T // 64
    st = gh.build_state(inp, max_lq=64)
    cfg, hkv = st.cfg, p["n_kv_heads"]
    kp, vp = torch.zeros_like(st.k_pool), torch.zeros_like(st.v_pool)
    cs, gs = torch.zeros_like(st.chunk_sum), torch.zeros_like(st.group_sum)
    sel = torch.zeros((B, nq, hkv, st.max_sel), dtype=torch.int32, device="cuda")
    n_sel = torch.zeros((B, nq, hkv), dtype=torch.int32, device="cuda")
    out = torch.empty((B, p["n_q_heads"], T, p["head_dim"]), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, p["n_q_heads"], T), dtype=torch.float32, device="cuda")
    ws = torch.zeros(hga.hga_prompt_workspace_bytes(cfg, B, T, st.max_chunks), dtype=torch.uint8,
                     device="cuda")

    def call(phases):
        hga.hga_prefill_prompt(cfg, B, T, st.q, st.k_raw, st.v_raw, kp, vp, T, cs, gs,
                               st.max_chunks, sel, n_sel, st.max_sel, out, lse, ws, phases=phases)

    def timed(phases, n):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        torch.cuda._sleep(int(2e8))  # the queue fills ahead: no host launch latency
        for e0, e1 in evs:
            e0.record()
            call(phases)
            e1.record()
        torch.cuda.synchronize()
        return float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))

    for _ in range(max(3, args.warmup // 4)):
        call(hga.HGA_PROMPT_ALL)
    torch.cuda.synchronize()
    n = max(5, args.steps // 10)
    ms_prompt = timed(hga.HGA_PROMPT_ALL, n)
    ms_append = timed(hga.HGA_PROMPT_APPEND, n)
    ms_route = timed(hga.HGA_PROMPT_ROUTE, n)
    ms_attend = timed(hga.HGA_PROMPT_ATTEND, n)
    assert torch.equal(kp, st.k_pool) and torch.isfinite(out).all().item()
    flops = prompt_flops(n_sel.cpu().numpy(), sel.cpu().numpy(), p)
    achieved = flops / (ms_attend * 1e-3) / 1e12
    res = {
        "metric": "whole-prompt chunked prefill tokens/s per layer at 32K; MFMA utilisation",
        "value": B * T / (ms_prompt * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": n,
        "warmup": args.warmup,
        "ms_per_step": ms_prompt,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V, pre-RoPE)",
        "config": {"workload": "prompt32k: GQA 32q/4kv heads, d=128, bf16, theta 1e6, a "
                               "32768-token prompt, all 512 query chunks of 64 tokens; 1 sink + 4 "
                               "local chunks, top-20 chunks, top-40 groups (1024 keys per chunk "
                               "at full budget)",
                   "batch": B, "context": T, "query_chunks": nq,
                   "timing": "events around each hga_prefill_prompt call (one step = one "
                             "prompt), queue filled ahead",
                   "phase_ms": {"append": ms_append, "route": ms_route, "attend": ms_attend}},
        "roofline": {"kernel": "attend_prompt_kernel (the attend phase, one launch)",
                     "bound": "mfma", "achieved": achieved, "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": achieved / 2500.0, "traffic": None, "flops_per_launch": flops,
                     "launch_ms": ms_attend},
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline_prompt(inp, p)
    print(json.dumps(res), flush=True)


def run_host64k(args):
    """Decode at 64K with the full K/V pool in pinned host memory: per step the
    new token is appended (device window pool and host pool), routed on the
    device summaries, and attended by hga_attend_tiered (routed groups copied
    over PCIe while the windows are attended from device memory: in one launch
    on one stream, or on a second stream), then the completed chunk's
    summaries are rebuilt.  Both forms are timed eagerly (events on the main
    stream around each step); the faster is the reported value."""
    import numpy as np
    import torch

    import gpu_harness as gh
    import long_context_hga_amd as hga
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    fp8 = bool(args.fp8)
    inp = synth.generate("host64k", overrides=dict(pool_dtype=1) if fp8 else None)
    p = inp.params
    B, T = p["batch"], p["context"]
    st = gh.build_state(inp)
    if fp8:  # the FP8 pool: codes then row scales, built from the raw K/V
        nbytes = B * p["n_kv_heads"] * T * (p["head_dim"] + 4)
        st.k_pool = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        st.v_pool = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        hga.hga_build_summaries(st.cfg, B, st.k_raw, st.v_raw, 0, T, st.k_pool, st.v_pool, T, None,
                                None, st.max_chunks)
        torch.cuda.synchronize()
    k_cold = torch.empty(st.k_pool.shape, dtype=st.k_pool.dtype, pin_memory=True)
    v_cold = torch.empty(st.v_pool.shape, dtype=st.v_pool.dtype, pin_memory=True)
    k_cold.copy_(st.k_pool)
    v_cold.copy_(st.v_pool)
    torch.cuda.synchronize()
    pos = int(inp.pos0[0])
    c0 = (pos // 64) * 64
    # selected lists per sequence: one per query head when routing per head;
    # a working set holds max_sel groups of every list
    lists = p["n_q_heads"] if p.get("route_per_head") else p["n_kv_heads"]
    q = gh.query_slice(st, 0)
    kt = st.k_raw[:, :, pos:pos + 1].contiguous()
    vt = st.v_raw[:, :, pos:pos + 1].contiguous()
    kc = st.k_raw[:, :, c0:c0 + 64].contiguous()
    del st.k_raw, st.v_raw
    cfg = st.cfg
    hkv, d = p["n_kv_heads"], p["head_dim"]
    if fp8:  # working set: codes then row scales
        kw = torch.zeros(B * hkv * st.max_sel * 16 * (d + 4), dtype=torch.uint8, device="cuda")
    else:
        kw = torch.zeros((B, hkv, st.max_sel * 16, d), dtype=st.k_pool.dtype, device="cuda")
    vw = torch.zeros_like(kw)
    s = gh.alloc_step(st, 1)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    tier_events = (torch.cuda.Event(), torch.cuda.Event())  # fork / join of the two-stream form

    def step(second):
        # the new token goes to the device window pool and, over PCIe, to the host pool
        hga.hga_build_summaries(cfg, B, kt, vt, pos, 1, st.k_pool, st.v_pool, T, None, None,
                                st.max_chunks)
        hga.hga_build_summaries(cfg, B, kt, vt, pos, 1, k_cold, v_cold, T, None, None,
                                st.max_chunks)
        hga.hga_route(cfg, B, q, 1, st.pos0, st.chunk_sum, st.group_sum, st.max_chunks, s.sel,
                      s.n_sel, st.max_sel, None, st.ws)
        hga.hga_attend_tiered(cfg, B, q, 1, st.pos0, st.k_pool, st.v_pool, T, k_cold, v_cold, T,
                              s.sel, s.n_sel, st.max_sel, kw, vw, s.out, s.lse, st.ws,
                              stream_a=main, stream_b=second,
                              events=tier_events if second is not None else None)
        hga.hga_build_summaries(cfg, B, kc, None, c0, 64, None, None, T, st.chunk_sum,
                                st.group_sum, st.max_chunks)

    def time_steps(second):
        for _ in range(args.warmup):
            step(second)
        torch.cuda.synchronize()
        # reference: the same step with the whole list attended from the device pool
        out_dev = torch.empty_like(s.out)
        lse_dev = torch.empty_like(s.lse)
        hga.hga_attend(cfg, B, q, 1, st.pos0, st.k_pool, st.v_pool, hga.HGA_SRC_POOL, T, s.sel,
                       s.n_sel, st.max_sel, hga.HGA_PART_ALL, out_dev, lse_dev, st.ws)
        torch.cuda.synchronize()
        assert (s.out - out_dev).abs().max().item() <= 1e-5
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(n):
            step(second)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / n

    n = max(1, args.steps)
    # the two forms of the host tier: the window attention and the PCIe copy
    # in one launch on one stream, or on two streams joined by events
    ms_one = time_steps(None)
    ms_two = time_steps(side)
    ms_step = min(ms_one, ms_two)

    def timed(fn, reps, stream=None):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream or main):
            fn()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    # warm tier: the same step with the routed groups fetched through an LRU
    # cache of n_warm groups per (sequence, KV head) in device memory, over a
    # sequence of queries that drift (q <- (q + eps z) / sqrt(1 + eps^2), z
    # ~ N(0, 1), seeded): consecutive steps route to overlapping groups
    n_warm, eps, n_warm_steps = 2 * p["topk_groups"], 0.25, max(32, n // 4)
    if fp8:  # cache slots: codes then row scales
        k_warm = torch.zeros(B * hkv * n_warm * 16 * (d + 4), dtype=torch.uint8, device="cuda")
    else:
        k_warm = torch.zeros((B, hkv, n_warm, 16, d), dtype=st.k_pool.dtype, device="cuda")
    v_warm = torch.zeros_like(k_warm)
    w_tags = torch.full((B, hkv, n_warm), -1, dtype=torch.int32, device="cuda")
    w_used = torch.zeros((B, hkv, n_warm), dtype=torch.int32, device="cuda")
    w_hits = torch.zeros((B, hkv), dtype=torch.int32, device="cuda")
    wsw = torch.zeros(hga.hga_warm_workspace_bytes(cfg, B, st.max_sel), dtype=torch.uint8,
                      device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(5000)
    qf = q.view(torch.bfloat16).float()
    qs = []
    for _ in range(n_warm_steps + args.warmup):
        qs.append(qf.to(torch.bfloat16).view(torch.int16).contiguous())
        z = torch.randn(qf.shape, generator=gen, device="cuda")
        qf = (qf + eps * z) / float((1 + eps * eps) ** 0.5)
    oa, la = torch.empty_like(s.out), torch.empty_like(s.lse)
    ob, lb = torch.empty_like(s.out), torch.empty_like(s.lse)
    ws_b = torch.zeros_like(st.ws)
    hit_counts = []

    def warm_step(i, stamp):
        qi = qs[i]
        hga.hga_build_summaries(cfg, B, kt, vt, pos, 1, st.k_pool, st.v_pool, T, None, None,
                                st.max_chunks)
        hga.hga_build_summaries(cfg, B, kt, vt, pos, 1, k_cold, v_cold, T, None, None,
                                st.max_chunks)
        hga.hga_route(cfg, B, qi, 1, st.pos0, st.chunk_sum, st.group_sum, st.max_chunks, s.sel,
                      s.n_sel, st.max_sel, None, st.ws)
        hga.hga_warm_gather(cfg, B, k_cold, v_cold, T, s.sel, s.n_sel, st.max_sel, st.pos0,
                            k_warm, v_warm, w_tags, w_used, n_warm, stamp, kw, vw, w_hits, wsw)
        hga.hga_attend(cfg, B, qi, 1, st.pos0, st.k_pool, st.v_pool, hga.HGA_SRC_POOL, T, s.sel,
                       s.n_sel, st.max_sel, hga.HGA_PART_WINDOWS, oa, la, st.ws)
        hga.hga_attend(cfg, B, qi, 1, st.pos0, kw, vw, hga.HGA_SRC_WORKING_SET, T, s.sel, s.n_sel,
                       st.max_sel, hga.HGA_PART_ROUTED, ob, lb, ws_b)
        hga.hga_merge_partials(cfg, B, 1, oa, la, ob, lb, s.out, s.lse)
        hga.hga_build_summaries(cfg, B, kc, None, c0, 64, None, None, T, st.chunk_sum,
                                st.group_sum, st.max_chunks)

    stamp = 0
    for i in range(args.warmup):
        stamp += 1
        warm_step(i, stamp)
    torch.cuda.synchronize()
    w0 = torch.cuda.Event(enable_timing=True)
    w1 = torch.cuda.Event(enable_timing=True)
    hit_total = torch.zeros((), dtype=torch.int64, device="cuda")
    # a spin kernel holds the GPU while the host queues every step (a dozen
    # binding calls per step would otherwise leave the GPU waiting on Python)
    torch.cuda._sleep(int(4e8))
    w0.record()
    for i in range(args.warmup, args.warmup + n_warm_steps):
        stamp += 1
        warm_step(i, stamp)
        hit_total += w_hits.sum()
    w1.record()
    torch.cuda.synchronize()
    ms_warm = w0.elapsed_time(w1) / n_warm_steps
    routed_per_step = int((s.n_sel.cpu().numpy() - (p["n_sink_chunks"] + p["n_local_chunks"] + 1)
                           * p["groups_per_chunk"]).sum())
    hit_rate = float(hit_total.item()) / (routed_per_step * n_warm_steps)
    # the same drifting queries without the cache: every routed group over PCIe
    c0e = torch.cuda.Event(enable_timing=True)
    c1e = torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(4e8))
    c0e.record()
    for i in range(args.warmup, args.warmup + n_warm_steps):
        qi = qs[i]
        hga.hga_build_summaries(cfg, B, kt, vt, pos, 1, st.k_pool, st.v_pool, T, None, None,
                                st.max_chunks)
        hga.hga_build_summaries(cfg, B, kt, vt, pos, 1, k_cold, v_cold, T, None, None,
                                st.max_chunks)
        hga.hga_route(cfg, B, qi, 1, st.pos0, st.chunk_sum, st.group_sum, st.max_chunks, s.sel,
                      s.n_sel, st.max_sel, None, st.ws)
        hga.hga_attend_tiered(cfg, B, qi, 1, st.pos0, st.k_pool, st.v_pool, T, k_cold, v_cold, T,
                              s.sel, s.n_sel, st.max_sel, kw, vw, s.out, s.lse, st.ws,
                              stream_a=main, stream_b=None)
        hga.hga_build_summaries(cfg, B, kc, None, c0, 64, None, None, T, st.chunk_sum,
                                st.group_sum, st.max_chunks)
    c1e.record()
    torch.cuda.synchronize()
    ms_cold = c0e.elapsed_time(c1e) / n_warm_steps

    reps = max(5, n // 4)
    ws2 = torch.zeros_like(st.ws)
    ob, lb = torch.empty_like(s.out), torch.empty_like(s.lse)
    t_gather = timed(lambda: hga.hga_gather(cfg, B, k_cold, v_cold, T, 1, s.sel, s.n_sel,
                                            st.max_sel, st.pos0, hga.HGA_PART_ROUTED, kw, vw), reps)
    t_routed = timed(lambda: (hga.hga_gather(cfg, B, k_cold, v_cold, T, 1, s.sel, s.n_sel,
                                             st.max_sel, st.pos0, hga.HGA_PART_ROUTED, kw, vw),
                              hga.hga_attend(cfg, B, q, 1, st.pos0, kw, vw,
                                             hga.HGA_SRC_WORKING_SET, T, s.sel, s.n_sel,
                                             st.max_sel, hga.HGA_PART_ROUTED, ob, lb, ws2)), reps)
    t_windows = timed(lambda: hga.hga_attend(cfg, B, q, 1, st.pos0, st.k_pool, st.v_pool,
                                             hga.HGA_SRC_POOL, T, s.sel, s.n_sel, st.max_sel,
                                             hga.HGA_PART_WINDOWS, ob, lb, ws2), reps)
    t_tiered = timed(lambda: hga.hga_attend_tiered(cfg, B, q, 1, st.pos0, st.k_pool, st.v_pool, T,
                                                   k_cold, v_cold, T, s.sel, s.n_sel, st.max_sel,
                                                   kw, vw, s.out, s.lse, st.ws, stream_a=main,
                                                   stream_b=side, events=tier_events), reps)
    t_tiered_one = timed(lambda: hga.hga_attend_tiered(cfg, B, q, 1, st.pos0, st.k_pool, st.v_pool,
                                                       T, k_cold, v_cold, T, s.sel, s.n_sel,
                                                       st.max_sel, kw, vw, s.out, s.lse, st.ws,
                                                       stream_a=main, stream_b=None), reps)
    # pinned host -> device copy peak (256 MiB)
    hbuf = torch.empty(256 << 20, dtype=torch.uint8, pin_memory=True)
    dbuf = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    t_h2d = timed(lambda: dbuf.copy_(hbuf, non_blocking=True), 5)
    h2d_gbs = (256 << 20) / (t_h2d * 1e-3) / 1e9
    routed_groups = int((s.n_sel.cpu().numpy() - (p["n_sink_chunks"] + p["n_local_chunks"] + 1)
                         * p["groups_per_chunk"]).sum())
    routed_bytes = routed_groups * 16 * ((d + 4) if fp8 else d * 2) * 2
    pcie_gbs = routed_bytes / (t_gather * 1e-3) / 1e9
    def overlap_of(t):
        return 1.0 - (t - max(t_routed, t_windows)) / min(t_routed, t_windows)
    out = {
        "metric": "routed-attention query tokens/s per layer at 64K ctx, pool in pinned host "
                  "memory (including transfer)",
        "value": B / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": n,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V, pre-RoPE)",
        "config": {"workload": "host64k: GQA 32q/4kv heads, d=128, bf16, ctx 65536, batch 4 decode "
                               "at t=65535, top-52 chunks, top-104 groups; full K/V pool in pinned "
                               "host memory, windows and summaries in HBM"
                               + ("; FP8 pool (E4M3FN codes + power-of-two row scales)" if fp8
                                  else ""),
                   "pool": "fp8" if fp8 else "bf16",
                   "batch": B, "context": T, "timing": "eager, events around each step",
                   "tier_form": "one launch" if ms_one <= ms_two else "two streams",
                   "ms_per_step_one_launch": ms_one, "ms_per_step_two_streams": ms_two},
        "pcie": {"routed_bytes_per_step": routed_bytes, "gather_ms": t_gather,
                 "achieved_GBps": pcie_gbs, "pinned_h2d_copy_GBps": h2d_gbs,
                 "frac_of_h2d": pcie_gbs / h2d_gbs},
        "warm_tier": {"slots_per_unit": n_warm, "query_drift_eps": eps, "steps": n_warm_steps,
                      "hit_rate": hit_rate,
                      "pcie_bytes_per_step": (1.0 - hit_rate) * routed_bytes,
                      "ms_per_step": ms_warm, "tokens_per_s": B / (ms_warm * 1e-3),
                      "ms_per_step_without_cache_same_queries": ms_cold,
                      "timing": "events around all steps, queue filled ahead by a spin kernel"},
        "overlap": {"routed_part_alone_ms": t_routed, "windows_part_alone_ms": t_windows,
                    "tiered_call_one_launch_ms": t_tiered_one,
                    "overlap_fraction_one_launch": overlap_of(t_tiered_one),
                    "tiered_call_two_streams_ms": t_tiered,
                    "overlap_fraction_two_streams": overlap_of(t_tiered)},
    }
    print(json.dumps(out), flush=True)


def copy_rate_ms(n_bytes, reps=20):
    """Median duration (ms) of a contiguous device copy of n_bytes (read
    n_bytes, write n_bytes), event-timed."""
    import numpy as np
    import torch
    src = torch.ones(n_bytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    torch.cuda._sleep(int(5e7))
    ev[0].record()
    for i in range(reps):
        dst.copy_(src)
        ev[i + 1].record()
    torch.cuda.synchronize()
    t = float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]))
    del src, dst
    return t


def time_graph_exact(step, R, args, min_replays=1000):
    """Step time over exactly args.steps steps, and its distribution.

    One HIP graph holds R consecutive steps (replicas 0..R-1), a second the
    remaining args.steps % R.  The timed region (bracketed by device
    synchronisation) replays the first args.steps // R times and the second
    once: exactly args.steps steps; returns their mean (ms).  Then at least
    min_replays replays of the first graph, each between two events on the
    launch stream with the queue filled ahead (a spin kernel holds the GPU
    while the host enqueues), give the per-step distribution (replay / R):
    median, p10, p90 in microseconds."""
    import numpy as np
    import torch
    K = max(1, args.steps)
    for i in range(max(args.warmup, R)):
        step(i % R)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for r in range(R):
            step(r)
    g_tail = None
    if K % R:
        g_tail = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_tail):
            for r in range(K % R):
                step(r)
    for _ in range(max(1, args.warmup // R)):
        g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(K // R):
        g.replay()
    if g_tail is not None:
        g_tail.replay()
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / K
    # distribution: per-replay events, queue filled ahead in batches
    n = max(min_replays, (K + R - 1) // R)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    per = []
    batch = 250
    for b0 in range(0, n, batch):
        b1 = min(n, b0 + batch)
        torch.cuda._sleep(int(5e7))
        ev[b0].record()
        for i in range(b0, b1):
            g.replay()
            ev[i + 1].record()
        torch.cuda.synchronize()
        per += [ev[i].elapsed_time(ev[i + 1]) * 1e3 / R for i in range(b0, b1)]
    per = np.asarray(per)
    dist = {"replays": int(n), "steps_per_replay": R, "steps": int(n * R),
            "median_us": float(np.median(per)), "p10_us": float(np.percentile(per, 10)),
            "p90_us": float(np.percentile(per, 90)), "mean_us": float(per.mean())}
    return ms_step, K, dist


def time_graph(step, R, args):
    """Mean step time (ms) over exactly args.steps graph-replayed steps."""
    ms_step, K, _ = time_graph_exact(step, R, args, min_replays=0)
    return ms_step, K


def time_launches(step, R, args):
    """Mean durations (ms) of the route and attend calls: events on the launch
    stream around each call, with the queue filled ahead by a spin kernel so
    host launch latency does not enter."""
    import numpy as np
    import torch
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda._sleep(int(2e8))
    for i in range(args.steps):
        step(i % R, evs[i])
    torch.cuda.synchronize()
    route_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    attend_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    return route_ms, attend_ms


if __name__ == "__main__":
    main()
