"""GPU checks of the warm tier (hga_warm_gather): a bounded LRU cache in
device memory of recently routed groups in front of the pinned host pool.

Over a sequence of decode steps whose queries drift, every step's cache state
(tags, stamps) and hit counts must equal the oracle's warm-tier policy
(oracle.warm_step: hits renew their stamp; the i-th miss in list order takes
the i-th least recently used non-hit slot, stamp order, ties by slot index,
empty slots first), and the working set must hold the oracle's gather of its
own pool for the routed groups (values bit-exact, keys within the pool-key
rule) as well as exactly what hga_gather (HGA_PART_ROUTED) copies.  The
attention through the cache is compared with the oracle's attention over the
list and with the device path."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth
from oracle_ref import ATOL_OUT, UnitCache, check_pool_keys, max_abs, q_unit, window_groups

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import long_context_hga_amd as hga  # noqa: E402
import gpu_harness as gh  # noqa: E402


def pinned_copy(t):
    h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    h.copy_(t)
    return h


@pytest.mark.parametrize("n_warm,drift", [(208, 0.25), (104, 0.5)])
def test_warm_cache_matches_gather_and_lru_model(n_warm, drift):
    inp = synth.generate("host64k", batch=2, context=8192)
    st = gh.build_state(inp)
    cfg = oracle.cfg_from(inp.params)
    B, hkv, T, max_sel = st.B, 4, st.T, st.max_sel
    kc, vc = pinned_copy(st.k_pool), pinned_copy(st.v_pool)
    k_warm = torch.zeros((B, hkv, n_warm, 16, 128), dtype=st.k_pool.dtype, device="cuda")
    v_warm = torch.zeros_like(k_warm)
    tags = torch.full((B, hkv, n_warm), -1, dtype=torch.int32, device="cuda")
    used = torch.zeros((B, hkv, n_warm), dtype=torch.int32, device="cuda")
    hits = torch.zeros((B, hkv), dtype=torch.int32, device="cuda")
    wsw = torch.zeros(hga.hga_warm_workspace_bytes(st.cfg, B, max_sel), dtype=torch.uint8,
                      device="cuda")
    kw = torch.zeros((B, hkv, max_sel * 16, 128), dtype=st.k_pool.dtype, device="cuda")
    vw = torch.zeros_like(kw)
    kref, vref = torch.zeros_like(kw), torch.zeros_like(vw)
    m_tags = np.full((B, hkv, n_warm), -1, dtype=np.int32)
    m_used = np.zeros((B, hkv, n_warm), dtype=np.int32)
    uc = UnitCache(inp, cfg)
    pos = int(inp.pos0[0])
    wins, _, _ = window_groups(cfg, pos, 1)
    rng = np.random.default_rng(77)
    q = st.q[:, :, :1].view(torch.bfloat16).float()  # the queries' bf16 bit patterns as values
    total_hits = 0
    for step in range(1, 9):
        qb = q.to(torch.bfloat16).view(torch.int16).contiguous()
        s = gh.alloc_step(st, 1)
        gh.route(st, qb, 1, st.pos0, s)
        hga.hga_warm_gather(st.cfg, B, kc, vc, T, s.sel, s.n_sel, max_sel, st.pos0, k_warm, v_warm,
                            tags, used, n_warm, step, kw, vw, hits, wsw)
        hga.hga_gather(st.cfg, B, kc, vc, T, 1, s.sel, s.n_sel, max_sel, st.pos0,
                       hga.HGA_PART_ROUTED, kref, vref)
        torch.cuda.synchronize()
        sel, nsel = s.sel.cpu().numpy(), s.n_sel.cpu().numpy()
        for b in range(B):
            for h in range(hkv):
                lst = [int(g) for g in sel[b, h, :nsel[b, h]]]
                routed = [g for g in lst if g not in wins]
                slots = [i for i, g in enumerate(lst) if g not in wins]
                rows = np.concatenate([np.arange(16 * i, 16 * i + 16) for i in slots])
                rows_t = torch.tensor(rows, device="cuda")
                assert torch.equal(kw[b, h, rows_t], kref[b, h, rows_t]), (step, b, h)
                assert torch.equal(vw[b, h, rows_t], vref[b, h, rows_t]), (step, b, h)
                m_tags[b, h], m_used[b, h], _, _, n_hit = oracle.warm_step(
                    m_tags[b, h], m_used[b, h], routed, step)
                assert int(hits[b, h]) == n_hit, (step, b, h, int(hits[b, h]), n_hit)
                total_hits += n_hit
                if step in (1, 8):  # the working set against the oracle's gather of its pool
                    _, _, kpo, vpo = uc.get(b, h)
                    kr = inp.f64(gh.dev_to_np_bf16(kw[b, h, rows_t]))
                    check_pool_keys(kr, oracle.gather(cfg, kpo, routed), True)
                    vr = inp.f64(gh.v_rows(vw[b:b + 1, h:h + 1])[0, 0][rows].view(np.uint16))
                    np.testing.assert_array_equal(vr, oracle.gather(cfg, vpo, routed))
        np.testing.assert_array_equal(tags.cpu().numpy(), m_tags)
        np.testing.assert_array_equal(used.cpu().numpy(), m_used)
        # the next query drifts from this one
        z = torch.tensor(rng.standard_normal(tuple(q.shape)), dtype=torch.float32, device="cuda")
        q = (q + drift * z) / float(np.sqrt(1 + drift * drift))
    assert total_hits > 0  # correlated queries reuse cached groups


def test_warm_then_attend_equals_device_path():
    """The working set filled through the cache, attended with the windows
    from the device pool and merged, equals attention over the whole list."""
    inp = synth.generate("host64k", batch=2, context=8192)
    st = gh.build_state(inp)
    B, max_sel = st.B, st.max_sel
    cfg = oracle.cfg_from(inp.params)
    uc = UnitCache(inp, cfg)
    kc, vc = pinned_copy(st.k_pool), pinned_copy(st.v_pool)
    k_warm = torch.zeros((B, 4, 128, 16, 128), dtype=st.k_pool.dtype, device="cuda")
    v_warm = torch.zeros_like(k_warm)
    tags = torch.full((B, 4, 128), -1, dtype=torch.int32, device="cuda")
    used = torch.zeros((B, 4, 128), dtype=torch.int32, device="cuda")
    wsw = torch.zeros(hga.hga_warm_workspace_bytes(st.cfg, B, max_sel), dtype=torch.uint8,
                      device="cuda")
    kw = torch.zeros((B, 4, max_sel * 16, 128), dtype=st.k_pool.dtype, device="cuda")
    vw = torch.zeros_like(kw)
    q = gh.query_slice(st, 0)
    s = gh.alloc_step(st, 1)
    gh.route(st, q, 1, st.pos0, s)
    gh.attend(st, q, 1, st.pos0, s)
    for step in (1, 2):  # all misses, then all hits
        hga.hga_warm_gather(st.cfg, B, kc, vc, st.T, s.sel, s.n_sel, max_sel, st.pos0, k_warm,
                            v_warm, tags, used, 128, step, kw, vw, None, wsw)
        oa, la = torch.empty_like(s.out), torch.empty_like(s.lse)
        ob, lb = torch.empty_like(s.out), torch.empty_like(s.lse)
        gh.attend(st, q, 1, st.pos0, s, part=hga.HGA_PART_WINDOWS, out=oa, lse=la)
        gh.attend(st, q, 1, st.pos0, s, part=hga.HGA_PART_ROUTED, k_src=kw, v_src=vw,
                  layout=hga.HGA_SRC_WORKING_SET, out=ob, lse=lb)
        om, lm = torch.empty_like(oa), torch.empty_like(la)
        hga.hga_merge_partials(st.cfg, B, 1, oa, la, ob, lb, om, lm)
        torch.cuda.synchronize()
        assert (om - s.out).abs().max().item() <= 1e-5, step
        assert (lm - s.lse).abs().max().item() <= 1e-5, step
        out = om.cpu().numpy()
        sel, nsel = s.sel.cpu().numpy(), s.n_sel.cpu().numpy()
        pos = int(inp.pos0[0])
        for b in range(B):
            for h in range(4):
                _, _, kpo, vpo = uc.get(b, h)
                o_ref, _ = oracle.attend(cfg, q_unit(inp, cfg, b, h, 0, 1), pos, kpo, vpo,
                                         sel[b, h, :nsel[b, h]])
                assert max_abs(out[b, h * 8:(h + 1) * 8], o_ref) <= ATOL_OUT, (step, b, h)
