"""HGA reference oracle: TEST INFRASTRUCTURE ONLY.

Thin ctypes wrapper around ``hga_oracle.c``: a plain fp64 CPU implementation
of the Hierarchical Global Attention hot path (chunk/group RoPE-aware key
summaries, two-level routing with sink/local/current windows, exact softmax
attention over the selected token K/V), following the HGA technical summary
on gist.science, section "Kernmechanisme", items 1-4.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never does, and this
package imports nothing from it.  All arrays here are float64 numpy arrays;
the conversion from the seeded bf16/fp32 inputs to float64 is exact.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hga_oracle.c")
_LIB = os.path.join(_HERE, "libhga_oracle.so")

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int)
_lp = ctypes.POINTER(ctypes.c_long)


class OraCfg(ctypes.Structure):
    _fields_ = [
        ("d", ctypes.c_int),
        ("hq", ctypes.c_int),
        ("hkv", ctypes.c_int),
        ("C", ctypes.c_int),
        ("G", ctypes.c_int),
        ("n_sink", ctypes.c_int),
        ("n_local", ctypes.c_int),
        ("topk_c", ctypes.c_int),
        ("topk_g", ctypes.c_int),
        ("theta", ctypes.c_double),
        ("hf_wavelength", ctypes.c_double),
        ("pool_bf16", ctypes.c_int),
        ("rep_integer", ctypes.c_int),
        ("rope_interleaved", ctypes.c_int),
        ("route_max", ctypes.c_int),
    ]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, no FP contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
             "-std=gnu11", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        c = ctypes.POINTER(OraCfg)
        L.ora_omega.argtypes = [c, ctypes.c_int]
        L.ora_omega.restype = ctypes.c_double
        L.ora_is_hf.argtypes = [c, ctypes.c_int]
        L.ora_is_hf.restype = ctypes.c_int
        L.ora_rope.argtypes = [c, _dp, ctypes.c_double, _dp]
        L.ora_span_summary.argtypes = [c, _dp, ctypes.c_long, ctypes.c_int, _dp]
        L.ora_summaries.argtypes = [c, _dp, ctypes.c_long, _dp, _dp]
        L.ora_round_bf16.argtypes = [ctypes.c_double]
        L.ora_round_bf16.restype = ctypes.c_double
        L.ora_round_bf16_vec.argtypes = [_dp, ctypes.c_long, _dp]
        L.ora_pool.argtypes = [c, _dp, ctypes.c_long, ctypes.c_long, _dp]
        L.ora_fp8_scale.argtypes = [ctypes.c_double]
        L.ora_fp8_scale.restype = ctypes.c_double
        L.ora_fp8_encode.argtypes = [ctypes.c_double]
        L.ora_fp8_encode.restype = ctypes.c_int
        L.ora_fp8_decode.argtypes = [ctypes.c_int]
        L.ora_fp8_decode.restype = ctypes.c_double
        L.ora_fp8_rows.argtypes = [_dp, ctypes.c_long, ctypes.c_int, _ip, _dp, _dp]
        L.ora_pool_fp8.argtypes = [c, _dp, ctypes.c_long, ctypes.c_long, _ip, _dp, _dp]
        L.ora_windows.argtypes = [c, ctypes.c_long, _lp, _lp, _lp]
        L.ora_windows.restype = ctypes.c_int
        L.ora_pooled_query.argtypes = [c, _dp, ctypes.c_int, ctypes.c_int, ctypes.c_long, _dp]
        L.ora_group_scores.argtypes = [c, _dp, ctypes.c_int, ctypes.c_long, _dp, ctypes.c_long,
                                       _dp]
        L.ora_select.argtypes = [c, _dp, ctypes.c_int, ctypes.c_long, _dp, _dp, _ip, ctypes.c_int,
                                 _dp, _dp]
        L.ora_select.restype = ctypes.c_int
        L.ora_attend.argtypes = [c, _dp, ctypes.c_int, ctypes.c_long, _dp, _dp, _ip, ctypes.c_int,
                                 _dp, _dp]
        L.ora_merge.argtypes = [ctypes.c_int, ctypes.c_long, _dp, _dp, _dp, _dp, _dp, _dp]
        L.ora_gather.argtypes = [c, _dp, _ip, ctypes.c_int, _dp]
        L.ora_warm_step.argtypes = [ctypes.c_int, _ip, _ip, _ip, ctypes.c_int, ctypes.c_int, _ip,
                                    _ip]
        L.ora_warm_step.restype = ctypes.c_int
        L.ora_step.argtypes = [c, ctypes.c_int, _dp, ctypes.c_int, _lp, _dp, _dp, ctypes.c_long,
                               _dp, _dp, ctypes.c_long, _ip, _ip, ctypes.c_int, _dp]
        L.ora_step.restype = ctypes.c_int
        L.ora_max_threads.restype = ctypes.c_int
        L.ora_set_threads.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def _d(a):
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(_dp)


def _i(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(_ip)


def make_cfg(d, hq, hkv, C, G, n_sink, n_local, topk_c, topk_g, theta, hf_wavelength,
             pool_bf16=True, rep_integer=False, rope_interleaved=False,
             route_max=False) -> OraCfg:
    return OraCfg(d, hq, hkv, C, G, n_sink, n_local, topk_c, topk_g, float(theta),
                  float(hf_wavelength), int(bool(pool_bf16)), int(bool(rep_integer)),
                  int(bool(rope_interleaved)), int(bool(route_max)))


def cfg_from(p: dict) -> OraCfg:
    """Build the oracle config from a plain dict (keys as in ``synth.CONFIGS``;
    ``rep_position`` 1 selects the representative position a + n/2,
    ``rope_style`` 1 interleaved RoPE pairs, ``route_pool`` 1 the max-pooled
    routing query)."""
    return make_cfg(p["head_dim"], p["n_q_heads"], p["n_kv_heads"], p["chunk_size"],
                    p["groups_per_chunk"], p["n_sink_chunks"], p["n_local_chunks"],
                    p["topk_chunks"], p["topk_groups"], p["rope_theta"], p["hf_wavelength"],
                    p["dtype"] == "bf16", p.get("rep_position", 0) == 1,
                    p.get("rope_style", 0) == 1, p.get("route_pool", 0) == 1)


def omega(cfg, j):
    return lib().ora_omega(ctypes.byref(cfg), j)


def is_hf(cfg, j):
    return bool(lib().ora_is_hf(ctypes.byref(cfg), j))


def rope(cfg, x, pos):
    x, xp = _d(x)
    out = np.empty(cfg.d)
    lib().ora_rope(ctypes.byref(cfg), xp, float(pos), out.ctypes.data_as(_dp))
    return out


def span_summary(cfg, kraw, a):
    kraw, kp = _d(kraw)
    out = np.empty(cfg.d)
    lib().ora_span_summary(ctypes.byref(cfg), kp, int(a), kraw.shape[0], out.ctypes.data_as(_dp))
    return out


def summaries(cfg, kraw):
    """kraw [T][d] of one (sequence, KV head) -> (chunk_sum [T/C][d], group_sum [T/g][d])."""
    kraw, kp = _d(kraw)
    T = kraw.shape[0]
    nch = T // cfg.C
    cs = np.empty((nch, cfg.d))
    gs = np.empty((nch * cfg.G, cfg.d))
    lib().ora_summaries(ctypes.byref(cfg), kp, T, cs.ctypes.data_as(_dp), gs.ctypes.data_as(_dp))
    return cs, gs


def round_bf16(x):
    x = np.asarray(x, dtype=np.float64)
    xc, xp = _d(x)
    out = np.empty_like(xc)
    lib().ora_round_bf16_vec(xp, xc.size, out.ctypes.data_as(_dp))
    return out.reshape(x.shape)


def pool(cfg, kraw, pos0=0):
    """Rotated, rounded pool keys for raw keys kraw [n][d] at positions pos0.."""
    kraw, kp = _d(kraw)
    out = np.empty_like(kraw)
    lib().ora_pool(ctypes.byref(cfg), kp, int(pos0), kraw.shape[0], out.ctypes.data_as(_dp))
    return out


def fp8_scale(amax):
    return lib().ora_fp8_scale(float(amax))


def fp8_encode(y):
    return lib().ora_fp8_encode(float(y))


def fp8_decode(code):
    return lib().ora_fp8_decode(int(code))


def fp8_rows(x):
    """Rows x [n][d] -> (codes int32 [n][d], scales [n], dequantised [n][d])."""
    x, xp = _d(x)
    n, d = x.shape
    codes = np.zeros((n, d), dtype=np.int32)
    scales = np.zeros(n)
    deq = np.zeros((n, d))
    lib().ora_fp8_rows(xp, n, d, codes.ctypes.data_as(_ip), scales.ctypes.data_as(_dp),
                       deq.ctypes.data_as(_dp))
    return codes, scales, deq


def pool_fp8(cfg, kraw, pos0=0):
    """FP8 pool keys for raw keys kraw [n][d] at positions pos0..: (codes,
    scales, dequantised rows)."""
    kraw, kp = _d(kraw)
    n, d = kraw.shape
    codes = np.zeros((n, d), dtype=np.int32)
    scales = np.zeros(n)
    deq = np.zeros((n, d))
    lib().ora_pool_fp8(ctypes.byref(cfg), kp, int(pos0), n, codes.ctypes.data_as(_ip),
                       scales.ctypes.data_as(_dp), deq.ctypes.data_as(_dp))
    return codes, scales, deq


def windows(cfg, ct):
    win = np.zeros(max(int(ct), 1), dtype=np.int64)
    lo = ctypes.c_long()
    hi = ctypes.c_long()
    n = lib().ora_windows(ctypes.byref(cfg), int(ct), win.ctypes.data_as(_lp), ctypes.byref(lo),
                          ctypes.byref(hi))
    return win[:n].copy(), lo.value, hi.value


def pooled_query(cfg, q, pos0):
    """q [hg][lq][d] raw -> mean rotated query [d]."""
    q, qp = _d(q)
    out = np.empty(cfg.d)
    lib().ora_pooled_query(ctypes.byref(cfg), qp, q.shape[0], q.shape[1], int(pos0),
                           out.ctypes.data_as(_dp))
    return out


def select(cfg, q, pos0, chunk_sum, group_sum, max_sel=1 << 16):
    """Two-level selection for one unit.

    q [hg][lq][d] raw.  Returns (sel_groups int32 array, margins[2],
    candidate scores in chunk order)."""
    q, qp = _d(q)
    cs, csp = _d(chunk_sum)
    gs, gsp = _d(group_sum)
    sel = np.zeros(max_sel, dtype=np.int32)
    margins = np.zeros(2)
    ct = int(pos0) // cfg.C
    ncand = max(0, ct - cfg.n_local - cfg.n_sink)
    scores = np.zeros(max(ncand, 1))
    n = lib().ora_select(ctypes.byref(cfg), qp, q.shape[1], int(pos0), csp, gsp,
                         sel.ctypes.data_as(_ip), max_sel, margins.ctypes.data_as(_dp),
                         scores.ctypes.data_as(_dp))
    if n < 0:
        raise ValueError("max_sel too small")
    return sel[:n].copy(), margins, scores[:ncand].copy()


def group_scores(cfg, q, pos0, group_sum):
    """Level-2 score of every group id before the query chunk: the pooled
    routing query of q [hg][lq][d] (raw, at positions pos0..) dotted with
    group_sum [n][d], over sqrt(d)."""
    q, qp = _d(q)
    gs, gsp = _d(group_sum)
    n = min(gs.shape[0], (int(pos0) // cfg.C) * cfg.G)
    out = np.zeros(max(n, 1))
    lib().ora_group_scores(ctypes.byref(cfg), qp, q.shape[1], int(pos0), gsp, n,
                           out.ctypes.data_as(_dp))
    return out[:n].copy()


def attend(cfg, q, pos0, kpool, vpool, sel_groups):
    """q [hg][lq][d] raw; kpool/vpool [T][d].  Returns (out [hg][lq][d], lse [hg][lq])."""
    q, qp = _d(q)
    kp_, kpp = _d(kpool)
    vp_, vpp = _d(vpool)
    sel, selp = _i(sel_groups)
    hg, lq = q.shape[0], q.shape[1]
    out = np.empty((hg, lq, cfg.d))
    lse = np.empty((hg, lq))
    lib().ora_attend(ctypes.byref(cfg), qp, lq, int(pos0), kpp, vpp, selp, sel.size,
                     out.ctypes.data_as(_dp), lse.ctypes.data_as(_dp))
    return out, lse


def merge(oa, la, ob, lb):
    oa, oap = _d(oa)
    ob, obp = _d(ob)
    la, lap = _d(la)
    lb, lbp = _d(lb)
    d = oa.shape[-1]
    n = la.size
    out = np.empty_like(oa)
    lse = np.empty_like(la)
    lib().ora_merge(d, n, oap, lap, obp, lbp, out.ctypes.data_as(_dp), lse.ctypes.data_as(_dp))
    return out, lse


def gather(cfg, pool_, sel_groups):
    p, pp = _d(pool_)
    sel, selp = _i(sel_groups)
    g = cfg.C // cfg.G
    out = np.empty((sel.size * g, cfg.d))
    lib().ora_gather(ctypes.byref(cfg), pp, selp, sel.size, out.ctypes.data_as(_dp))
    return out


def warm_step(tags, used, routed, step_no):
    """One call of the warm-tier LRU policy for one unit.  tags, used: int
    arrays [n_warm] (copies are updated and returned); routed: the distinct
    routed group ids in list order.  Returns (tags, used, slot [n], hit [n],
    n_hits)."""
    tags, tp = _i(np.array(tags, dtype=np.int32, copy=True))
    used, up = _i(np.array(used, dtype=np.int32, copy=True))
    routed, rp = _i(np.asarray(routed, dtype=np.int32))
    n = routed.size
    slot = np.zeros(max(n, 1), dtype=np.int32)
    hit = np.zeros(max(n, 1), dtype=np.int32)
    nh = lib().ora_warm_step(tags.size, tp, up, rp, n, int(step_no), slot.ctypes.data_as(_ip),
                             hit.ctypes.data_as(_ip))
    if nh < 0:
        raise ValueError("more misses than free slots")
    return tags, used, slot[:n].copy(), hit[:n].copy(), nh


def step(cfg, q, pos0, chunk_sum, group_sum, kpool, vpool, max_sel):
    """Batched selection + attention over independent units (OpenMP).

    q [U][hg][lq][d]; pos0 [U]; chunk_sum [U][nch][d]; group_sum
    [U][nch*G][d]; kpool/vpool [U][T][d].  Returns (sel [U][max_sel],
    nsel [U], out [U][hg][lq][d])."""
    q, qp = _d(q)
    cs, csp = _d(chunk_sum)
    gs, gsp = _d(group_sum)
    kp_, kpp = _d(kpool)
    vp_, vpp = _d(vpool)
    pos = np.ascontiguousarray(pos0, dtype=np.int64)
    U, hg, lq, d = q.shape
    sel = np.zeros((U, max_sel), dtype=np.int32)
    nsel = np.zeros(U, dtype=np.int32)
    out = np.empty((U, hg, lq, d))
    bad = lib().ora_step(ctypes.byref(cfg), U, qp, lq, pos.ctypes.data_as(_lp), csp, gsp,
                         cs.shape[1], kpp, vpp, kp_.shape[1], sel.ctypes.data_as(_ip),
                         nsel.ctypes.data_as(_ip), max_sel, out.ctypes.data_as(_dp))
    if bad:
        raise ValueError("max_sel too small")
    return sel, nsel, out


def max_threads() -> int:
    return lib().ora_max_threads()


def set_threads(n: int) -> None:
    """Threads of step()'s parallel loop (timing only)."""
    lib().ora_set_threads(int(n))
