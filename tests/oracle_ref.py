"""Per-unit oracle references and the comparison rules of the GPU parity tests.

Comparison rules (written here once, used by every GPU test):
  * pool keys: each element equals the oracle's fp64 rotation rounded once to
    the pool dtype; at most 1 ulp apart, and differing elements are rarer
    than 1e-6 (both sides rotate in fp64; only an fp64 value within ~1e-16
    of a rounding midpoint can round differently).
  * pool values: bit-exact copy.
  * summaries: fp32 results within 1 fp32 ulp of the fp64 oracle, plus an
    absolute 2e-10: at positions up to 65535 the fp64 angle p*omega itself
    carries up to ~1.5e-11 rad of rounding, and the two sides may round it
    differently (per-token product vs. fp64 angle stepping); on a span mean
    of keys of size ~4 that is < 1e-10, far below the 1e-6 score margin.
  * selections: where the oracle's level-1 and level-2 score gaps at the
    cut both exceed 1e-6, the GPU list equals the oracle list exactly.
    Otherwise the unit is reported "unpinned" and the GPU list must still be a
    valid two-level top-k within 1e-6: the windows are present, the routed
    count matches, the level-1 set it came from is the oracle's when the
    level-1 gap exceeds 1e-6 (else any set that keeps every chunk scoring
    above the k-th by more than 1e-6 and fills up with chunks within 1e-6 of
    it), and over the groups of that set the routed groups contain every group
    scoring above the k_g-th by more than 1e-6 and none scoring below it by
    more than 1e-6.
  * attention outputs: the oracle attends over the GPU's own selection;
    max-abs difference <= 2e-3 (bf16 inputs, fp32 accumulation).
"""
from __future__ import annotations

import itertools
import math

import numpy as np

import oracle
from synth import Inputs

MARGIN = 1e-6
ATOL_OUT = 2e-3


class UnitCache:
    """Oracle state of (sequence b, KV head h): summaries and rotated pool."""

    def __init__(self, inp: Inputs, cfg):
        self.inp = inp
        self.cfg = cfg
        self._c = {}

    def get(self, b, h, need_pool=True):
        key = (b, h, need_pool)
        if key not in self._c:
            kraw = self.inp.f64(self.inp.k[b, h])
            cs, gs = oracle.summaries(self.cfg, kraw)
            kp = oracle.pool(self.cfg, kraw, 0) if need_pool else None
            v = self.inp.f64(self.inp.v[b, h]) if need_pool else None
            self._c[key] = (cs, gs, kp, v)
        return self._c[key]


def q_unit(inp: Inputs, cfg, b, h, tok0, lq):
    hg = cfg.hq // cfg.hkv
    return inp.f64(inp.q[b, h * hg:(h + 1) * hg, tok0:tok0 + lq])


def window_groups(cfg, pos0, lq):
    ct = pos0 // cfg.C
    last = pos0 + lq - 1
    win, lo, hi = oracle.windows(cfg, ct)
    g = [c * cfg.G + j for c in win for j in range(cfg.G)]
    g += list(range(ct * cfg.G, last // (cfg.C // cfg.G) + 1))
    return set(g), lo, hi


def check_selection(cfg, gpu_sel, ora_sel, margins, ora_scores, pos0, lq, gscores):
    """Returns True if the unit was pinned (exact match required).

    ora_scores: the oracle's level-1 scores of the candidate chunks (chunk
    order); gscores: its level-2 score of every group id before the query
    chunk (oracle.group_scores)."""
    pinned = margins[0] > MARGIN and margins[1] > MARGIN
    if pinned:
        assert list(gpu_sel) == list(ora_sel), (list(gpu_sel), list(ora_sel), margins)
        return True
    wins, lo, hi = window_groups(cfg, pos0, lq)
    gs = set(int(x) for x in gpu_sel)
    assert wins <= gs
    assert len(gpu_sel) == len(ora_sel)
    assert list(gpu_sel) == sorted(gs)
    routed = gs - wins
    n_cand = hi - lo
    k1 = min(cfg.topk_c, n_cand)
    if k1 == 0:
        assert not routed
        return False
    s1 = np.asarray(ora_scores, dtype=np.float64)
    kth1 = np.sort(s1)[::-1][k1 - 1]
    sure = [lo + i for i in range(n_cand) if s1[i] > kth1 + MARGIN]
    near = [lo + i for i in range(n_cand) if abs(s1[i] - kth1) <= MARGIN]
    if margins[0] > MARGIN:  # the level-1 set is unique: the k1 chunks scoring >= the k-th
        fills = [()]
        sure = [lo + i for i in range(n_cand) if s1[i] >= kth1]
        assert len(sure) == k1
    else:
        need = k1 - len(sure)
        assert 0 <= need <= len(near), (need, len(near))
        fills = list(itertools.islice(itertools.combinations(near, need), 4096))
    k2 = min(cfg.topk_g, k1 * cfg.G)
    g_sc = np.asarray(gscores, dtype=np.float64)
    for fill in fills:  # some admissible level-1 set must explain the routed groups
        chunks = sorted(set(sure) | set(fill))
        cand = [c * cfg.G + j for c in chunks for j in range(cfg.G)]
        if not routed <= set(cand):
            continue
        kth2 = np.sort(g_sc[cand])[::-1][k2 - 1]
        must = {gid for gid in cand if g_sc[gid] > kth2 + MARGIN}
        may = {gid for gid in cand if g_sc[gid] >= kth2 - MARGIN}
        if must <= routed <= may:
            return False
    raise AssertionError(f"routed groups {sorted(routed)} are no two-level top-k within {MARGIN} "
                         f"(margins {margins})")


def check_pool_keys(gpu_vals: np.ndarray, ora_vals: np.ndarray, bf16: bool):
    diff = np.abs(gpu_vals - ora_vals)
    ulp = np.abs(ora_vals) * (2.0 ** -7 if bf16 else 2.0 ** -23) + 1e-38
    assert np.all(diff <= ulp), float(np.max(diff / ulp))
    assert np.count_nonzero(diff) <= max(1, int(1e-6 * diff.size))


def check_summaries(gpu: np.ndarray, ora: np.ndarray):
    tol = np.abs(ora) * 2.0 ** -23 + 2e-10
    bad = np.abs(gpu.astype(np.float64) - ora) > tol
    assert not bad.any(), (np.argwhere(bad)[:5], gpu[bad][:5], ora[bad][:5])


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))
