"""GPU parity of the routing / summary variants against the fp64 oracle with
the same switches: the high-frequency threshold at the group length
(lambda_hf = g = 16 instead of C = 64), the representative position a + n/2
instead of the midpoint a + (n-1)/2, interleaved RoPE pairs, and routing per
query head (tests/oracle_ref.py rules:
summaries within 1 fp32 ulp, selections exact where the margins allow,
outputs within the attention tolerance)."""
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth
from oracle_ref import ATOL_OUT, UnitCache, check_selection, check_summaries, max_abs, q_unit

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import gpu_harness as gh  # noqa: E402

VARIANTS = [dict(hf_wavelength=16.0), dict(rep_position=1),
            dict(hf_wavelength=16.0, rep_position=1), dict(rope_style=1),
            dict(rope_style=1, rep_position=1)]


def vid(v):
    return "-".join(f"{k}={v[k]}" for k in sorted(v))


@pytest.mark.parametrize("variant", VARIANTS, ids=vid)
def test_variant_summaries_route_attend(variant):
    """Summaries of a 4K context, then decode (1 and 7 query tokens) and a
    64-token prefill chunk routed and attended, all against the oracle run
    with the same variant."""
    inp = synth.generate("prefill32k", batch=2, context=4096, overrides=dict(variant, needles=0))
    st = gh.build_state(inp)
    cfg = oracle.cfg_from(inp.params)
    uc = UnitCache(inp, cfg)
    B, hkv = st.B, inp.k.shape[1]
    hg = cfg.hq // cfg.hkv
    cs_gpu, gs_gpu = st.chunk_sum.cpu().numpy(), st.group_sum.cpu().numpy()
    for b in range(B):
        for h in range(hkv):
            cs, gs, _, _ = uc.get(b, h)
            check_summaries(cs_gpu[b, h, :cs.shape[0]], cs)
            check_summaries(gs_gpu[b, h, :gs.shape[0]], gs)
    for pos, lq in ((4095, 1), (3000, 7), (4032, 64)):
        q = st.q[:, :, :lq].contiguous()
        pos_t = torch.full((B,), pos, dtype=torch.int32, device="cuda")
        s = gh.alloc_step(st, lq)
        gh.route(st, q, lq, pos_t, s)
        gh.attend(st, q, lq, pos_t, s)
        torch.cuda.synchronize()
        sel, nsel, out = s.sel.cpu().numpy(), s.n_sel.cpu().numpy(), s.out.cpu().numpy()
        for b in range(B):
            for h in range(hkv):
                cs, gs, kp, v = uc.get(b, h)
                qu = q_unit(inp, cfg, b, h, 0, lq)
                g = sel[b, h, :nsel[b, h]]
                osel, margins, oscores = oracle.select(cfg, qu, pos, cs, gs)
                check_selection(cfg, g, osel, margins, oscores, pos, lq,
                                oracle.group_scores(cfg, qu, pos, gs))
                o_ref, _ = oracle.attend(cfg, qu, pos, kp, v, g)
                assert max_abs(out[b, h * hg:(h + 1) * hg], o_ref) <= ATOL_OUT, (pos, lq, b, h)


def test_variants_change_the_summaries():
    """The switches reach the kernels: each variant's summaries differ from
    the default ones (LF pairs rotated elsewhere, or pairs reclassified)."""
    base = gh.build_state(synth.generate("prefill32k", context=1024, overrides=dict(needles=0)))
    for v in VARIANTS:
        st = gh.build_state(synth.generate("prefill32k", context=1024, overrides=dict(v, needles=0)))
        assert not torch.equal(st.chunk_sum, base.chunk_sum), v
        assert not torch.equal(st.group_sum, base.group_sum), v
        if "rope_style" not in v:  # the pool depends only on the pairing
            assert torch.equal(st.k_pool, base.k_pool)
        else:
            assert not torch.equal(st.k_pool, base.k_pool)


@pytest.mark.parametrize("hq,hkv", [(32, 4), (8, 4)])
def test_route_per_query_head(hq, hkv):
    """One list per query head, routed with that head's own rotated query
    (the oracle run with a single query head per unit), attended over its KV
    head: decode (1 and 7 query tokens) and a 64-token prefill chunk; the
    fused decode step gives the bits of the separate calls; the gather copies
    each head's list."""
    import long_context_hga_amd as hga
    over = dict(n_q_heads=hq, n_kv_heads=hkv, route_per_head=1, needles=0)
    inp = synth.generate("prefill32k", batch=2, context=4096, overrides=over)
    st = gh.build_state(inp)
    p1 = dict(inp.params, n_q_heads=1, n_kv_heads=1)
    ocfg = oracle.cfg_from(p1)          # one query head per routing unit
    ucfg = oracle.cfg_from(inp.params)  # summaries / pool (independent of the routing)
    uc = UnitCache(inp, ucfg)
    B, hg, max_sel = st.B, hq // hkv, st.max_sel
    for pos, lq in ((4095, 1), (3000, 7), (4032, 64)):
        q = st.q[:, :, :lq].contiguous()
        pos_t = torch.full((B,), pos, dtype=torch.int32, device="cuda")
        sel = torch.full((B, hq, max_sel), -7, dtype=torch.int32, device="cuda")
        n_sel = torch.full((B, hq), -7, dtype=torch.int32, device="cuda")
        out = torch.full((B, hq, lq, 128), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((B, hq, lq), float("nan"), dtype=torch.float32, device="cuda")
        ws = torch.zeros(hga.hga_workspace_bytes(st.cfg, B, st.T, lq), dtype=torch.uint8,
                         device="cuda")
        hga.hga_route(st.cfg, B, q, lq, pos_t, st.chunk_sum, st.group_sum, st.max_chunks, sel,
                      n_sel, max_sel, None, ws)
        hga.hga_attend(st.cfg, B, q, lq, pos_t, st.k_pool, st.v_pool, hga.HGA_SRC_POOL, st.T,
                       sel, n_sel, max_sel, hga.HGA_PART_ALL, out, lse, ws)
        torch.cuda.synchronize()
        sel_h, nsel_h, out_h = sel.cpu().numpy(), n_sel.cpu().numpy(), out.cpu().numpy()
        lists_differ = False
        for b in range(B):
            for qh in range(hq):
                cs, gs, kp, v = uc.get(b, qh // hg)
                qu = inp.f64(inp.q[b, qh:qh + 1, :lq])
                g = sel_h[b, qh, :nsel_h[b, qh]]
                osel, margins, oscores = oracle.select(ocfg, qu, pos, cs, gs)
                check_selection(ocfg, g, osel, margins, oscores, pos, lq,
                                oracle.group_scores(ocfg, qu, pos, gs))
                o_ref, _ = oracle.attend(ocfg, qu, pos, kp, v, g)
                assert max_abs(out_h[b, qh:qh + 1], o_ref) <= ATOL_OUT, (pos, lq, b, qh)
                if qh % hg and not (g.size == sel_h[b, qh - 1, :nsel_h[b, qh - 1]].size and
                                    (g == sel_h[b, qh - 1, :nsel_h[b, qh - 1]]).all()):
                    lists_differ = True
        assert lists_differ  # the heads of a KV head do route differently
        if lq == 1:
            # gather of every head's list == the pool rows it names
            kw = torch.zeros((B, hq, max_sel * 16, 128), dtype=st.k_pool.dtype, device="cuda")
            vw = torch.zeros_like(kw)
            hga.hga_gather(st.cfg, B, st.k_pool, st.v_pool, st.T, 0, sel, n_sel, max_sel, pos_t,
                           hga.HGA_PART_ALL, kw, vw)
            out2 = torch.full_like(out, float("nan"))
            hga.hga_attend(st.cfg, B, q, lq, pos_t, kw, vw, hga.HGA_SRC_WORKING_SET, st.T, sel,
                           n_sel, max_sel, hga.HGA_PART_ALL, out2, None, ws)
            torch.cuda.synchronize()
            assert torch.equal(out2, out)
            b, qh = 1, hq - 1
            gid = int(sel[b, qh, 5])
            assert torch.equal(kw[b, qh, 5 * 16:6 * 16], st.k_pool[b, qh // hg, gid * 16:gid * 16 + 16])
            # the fused step (append + refresh of the chunk the token ends + route +
            # attend) gives the same bits
            stage = st.k_raw[:, :, pos // 64 * 64:pos // 64 * 64 + 64].contiguous()
            sel3 = torch.full_like(sel, -7)
            n3 = torch.full_like(n_sel, -7)
            out3 = torch.full_like(out, float("nan"))
            kp3, vp3 = st.k_pool.clone(), st.v_pool.clone()
            cs3, gs3 = st.chunk_sum.clone(), st.group_sum.clone()
            hga.hga_decode_step(st.cfg, B, q, st.k_raw[:, :, pos].contiguous(),
                                st.v_raw[:, :, pos].contiguous(), pos_t, kp3, vp3, st.T, stage,
                                cs3, gs3, st.max_chunks, sel3, n3, max_sel, out3, None,
                                torch.zeros_like(ws))
            torch.cuda.synchronize()
            assert torch.equal(n3, n_sel) and torch.equal(out3, out)
            assert torch.equal(kp3, st.k_pool) and torch.equal(cs3, st.chunk_sum)


def test_interleaved_whole_prompt_and_fused_step():
    """Interleaved RoPE pairs through the whole-prompt prefill (every chunk of
    a 512-token prompt against the oracle) and the fused decode step (the
    bits of the separate calls)."""
    import long_context_hga_amd as hga
    inp = synth.generate("prompt32k", context=512, overrides=dict(rope_style=1))
    st = gh.build_state(inp, max_lq=64)
    cfg = oracle.cfg_from(inp.params)
    uc = UnitCache(inp, cfg)
    T, nq, hg = st.T, st.T // 64, 8
    sel = torch.full((1, nq, 4, st.max_sel), -7, dtype=torch.int32, device="cuda")
    n_sel = torch.full((1, nq, 4), -7, dtype=torch.int32, device="cuda")
    out = torch.full((1, 32, T, 128), float("nan"), dtype=torch.float32, device="cuda")
    kp, vp = torch.zeros_like(st.k_pool), torch.zeros_like(st.v_pool)
    cs, gs = torch.zeros_like(st.chunk_sum), torch.zeros_like(st.group_sum)
    ws = torch.zeros(hga.hga_prompt_workspace_bytes(st.cfg, 1, T, st.max_chunks),
                     dtype=torch.uint8, device="cuda")
    hga.hga_prefill_prompt(st.cfg, 1, T, st.q, st.k_raw, st.v_raw, kp, vp, T, cs, gs,
                           st.max_chunks, sel, n_sel, st.max_sel, out, None, ws)
    torch.cuda.synchronize()
    sel_h, nsel_h, out_h = sel.cpu().numpy(), n_sel.cpu().numpy(), out.cpu().numpy()
    for qc in range(nq):
        for h in range(4):
            cs_, gs_, kpo, vpo = uc.get(0, h)
            qu = q_unit(inp, cfg, 0, h, qc * 64, 64)
            g = sel_h[0, qc, h, :nsel_h[0, qc, h]]
            osel, margins, oscores = oracle.select(cfg, qu, qc * 64, cs_, gs_)
            check_selection(cfg, g, osel, margins, oscores, qc * 64, 64,
                            oracle.group_scores(cfg, qu, qc * 64, gs_))
            o_ref, _ = oracle.attend(cfg, qu, qc * 64, kpo, vpo, g)
            assert max_abs(out_h[0, h * hg:(h + 1) * hg, qc * 64:(qc + 1) * 64], o_ref) <= ATOL_OUT
    # fused decode step at the last position == route + attend
    dinp = synth.generate("decode64k", batch=2, context=2048, overrides=dict(rope_style=1))
    dst = gh.build_state(dinp)
    q = gh.query_slice(dst, 0)
    s1 = gh.alloc_step(dst, 1)
    gh.route(dst, q, 1, dst.pos0, s1)
    gh.attend(dst, q, 1, dst.pos0, s1)
    pos = int(dinp.pos0[0])
    stage = dst.k_raw[:, :, pos // 64 * 64:pos // 64 * 64 + 64].contiguous()
    s2 = gh.alloc_step(dst, 1)
    hga.hga_decode_step(dst.cfg, 2, q, dst.k_raw[:, :, pos].contiguous(),
                        dst.v_raw[:, :, pos].contiguous(), dst.pos0, dst.k_pool, dst.v_pool, dst.T,
                        stage, dst.chunk_sum, dst.group_sum, dst.max_chunks, s2.sel, s2.n_sel,
                        dst.max_sel, s2.out, s2.lse, torch.zeros_like(dst.ws))
    torch.cuda.synchronize()
    assert torch.equal(s1.n_sel, s2.n_sel) and torch.equal(s1.out, s2.out)


def _route_attend_check(inp, st, cfg, uc, pos, lq, units, q=None):
    """Route + attend lq query tokens at pos; selections and outputs of the
    given (b, h) units against the oracle run with cfg.  Returns the lists."""
    B, hg = st.B, cfg.hq // cfg.hkv
    q = st.q[:, :, :lq].contiguous() if q is None else q
    pos_t = torch.full((B,), pos, dtype=torch.int32, device="cuda")
    s = gh.alloc_step(st, lq)
    gh.route(st, q, lq, pos_t, s)
    gh.attend(st, q, lq, pos_t, s)
    torch.cuda.synchronize()
    sel, nsel, out = s.sel.cpu().numpy(), s.n_sel.cpu().numpy(), s.out.cpu().numpy()
    lists = {}
    for b, h in units:
        cs, gs, kp, v = uc.get(b, h)
        qu = q_unit(inp, cfg, b, h, 0, lq)
        g = sel[b, h, :nsel[b, h]]
        osel, margins, oscores = oracle.select(cfg, qu, pos, cs, gs)
        check_selection(cfg, g, osel, margins, oscores, pos, lq,
                        oracle.group_scores(cfg, qu, pos, gs))
        o_ref, _ = oracle.attend(cfg, qu, pos, kp, v, g)
        assert max_abs(out[b, h * hg:(h + 1) * hg], o_ref) <= ATOL_OUT, (pos, lq, b, h)
        lists[b, h] = g.copy()
    return lists, s


def test_max_pooled_routing_query():
    """Max pooling of the routing query (route_pool = 1: each query head's
    token-mean query, a candidate scoring the largest head score): decode (1
    and 7 query tokens) and a 64-token prefill chunk at 4K against the oracle
    run with max pooling; the lists differ from mean pooling; the fused
    decode step gives the bits of the separate calls."""
    import long_context_hga_amd as hga
    inp = synth.generate("prefill32k", batch=2, context=4096, overrides=dict(route_pool=1, needles=0))
    st = gh.build_state(inp)
    cfg = oracle.cfg_from(inp.params)
    assert cfg.route_max == 1
    uc = UnitCache(inp, cfg)
    units = [(b, h) for b in range(st.B) for h in range(4)]
    differ = 0
    for pos, lq in ((4095, 1), (3000, 7), (4032, 64)):
        lists, _ = _route_attend_check(inp, st, cfg, uc, pos, lq, units)
        mean_cfg = oracle.cfg_from(dict(inp.params, route_pool=0))
        for (b, h), g in lists.items():
            cs, gs, _, _ = uc.get(b, h, need_pool=False)
            gm, _, _ = oracle.select(mean_cfg, q_unit(inp, mean_cfg, b, h, 0, lq), pos, cs, gs)
            differ += int(len(gm) != len(g) or (gm != g).any())
    assert differ > 0  # the switch reaches the kernels
    # fused decode step == separate calls, with max pooling
    B, T = st.B, st.T
    pos = 4000
    pos_t = torch.full((B,), pos, dtype=torch.int32, device="cuda")
    q = gh.query_slice(st, 0)
    c0 = pos // 64 * 64
    kt = st.k_raw[:, :, pos:pos + 1].contiguous()
    vt = st.v_raw[:, :, pos:pos + 1].contiguous()
    sa = gh.alloc_step(st, 1)
    gh.route(st, q, 1, pos_t, sa)
    gh.attend(st, q, 1, pos_t, sa)
    sb = gh.alloc_step(st, 1)
    stage = st.k_raw[:, :, c0:c0 + 64].contiguous()
    hga.hga_decode_step(st.cfg, B, q, kt, vt, pos_t, st.k_pool.clone(), st.v_pool.clone(), T,
                        stage, st.chunk_sum.clone(), st.group_sum.clone(), st.max_chunks, sb.sel,
                        sb.n_sel, st.max_sel, sb.out, sb.lse, torch.zeros_like(st.ws))
    torch.cuda.synchronize()
    assert torch.equal(sa.sel, sb.sel) and torch.equal(sa.out, sb.out)


@pytest.mark.parametrize("context", [65536, 131072])
def test_max_pooled_routing_long_contexts(context):
    """Max pooling at 64K (1018 candidates: the fast selection) and 128K
    (2042: the streaming selection), one sequence, every KV head against the
    oracle."""
    inp = synth.generate("decode64k", batch=1, context=context, overrides=dict(route_pool=1))
    st = gh.build_state(inp)
    cfg = oracle.cfg_from(inp.params)
    uc = UnitCache(inp, cfg)
    print(f"[max pooling] context {context}", flush=True)
    _route_attend_check(inp, st, cfg, uc, int(inp.pos0[0]), 1, [(0, h) for h in range(4)],
                        q=gh.query_slice(st, 0))


def test_max_pooled_routing_whole_prompt():
    """The whole-prompt prefill with max pooling (the pooled query once per
    query chunk and head): sampled chunks of a 2K prompt against the oracle."""
    import long_context_hga_amd as hga
    inp = synth.generate("prompt32k", context=2048, overrides=dict(route_pool=1))
    st = gh.build_state(inp, max_lq=64)
    cfg = oracle.cfg_from(inp.params)
    uc = UnitCache(inp, cfg)
    B, T, ms = st.B, st.T, st.max_sel
    nq = T // 64
    sel = torch.full((B, nq, 4, ms), -7, dtype=torch.int32, device="cuda")
    n_sel = torch.full((B, nq, 4), -7, dtype=torch.int32, device="cuda")
    out = torch.full((B, 32, T, 128), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.zeros(hga.hga_prompt_workspace_bytes(st.cfg, B, T, st.max_chunks),
                     dtype=torch.uint8, device="cuda")
    hga.hga_prefill_prompt(st.cfg, B, T, st.q, st.k_raw, st.v_raw, st.k_pool.clone(),
                           st.v_pool.clone(), T, st.chunk_sum.clone(), st.group_sum.clone(),
                           st.max_chunks, sel, n_sel, ms, out, None, ws)
    torch.cuda.synchronize()
    sl, ns, o = sel.cpu().numpy(), n_sel.cpu().numpy(), out.cpu().numpy()
    for b in range(B):
        for h in range(4):
            cs, gs, kp, v = uc.get(b, h)
            for qc in (6, 19, 31):
                p0 = qc * 64
                qu = q_unit(inp, cfg, b, h, p0, 64)
                g = sl[b, qc, h, :ns[b, qc, h]]
                osel, margins, oscores = oracle.select(cfg, qu, p0, cs, gs)
                check_selection(cfg, g, osel, margins, oscores, p0, 64,
                                oracle.group_scores(cfg, qu, p0, gs))
                o_ref, _ = oracle.attend(cfg, qu, p0, kp, v, g)
                assert max_abs(o[b, h * 8:(h + 1) * 8, p0:p0 + 64], o_ref) <= ATOL_OUT, (b, h, qc)
