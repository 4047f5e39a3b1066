"""GPU parity on head shapes beyond the benchmark layer: every supported
query-heads-per-KV-head ratio (1, 2, 4, 8) at head_dim 128 and 64, bf16, for
decode (1 and several query tokens) and, at head_dim 128, chunked prefill,
whole-prompt prefill and the fused prefill step;
checked against the fp64 oracle on the GPU's own selection, and the
selection itself against the oracle's (tests/oracle_ref.py rules)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth
from oracle_ref import ATOL_OUT, UnitCache, check_selection, max_abs, q_unit

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import gpu_harness as gh  # noqa: E402

SHAPES = [dict(n_q_heads=4, n_kv_heads=4, head_dim=128),
          dict(n_q_heads=8, n_kv_heads=4, head_dim=128),
          dict(n_q_heads=16, n_kv_heads=4, head_dim=128),
          dict(n_q_heads=8, n_kv_heads=1, head_dim=128),
          dict(n_q_heads=32, n_kv_heads=4, head_dim=64),
          dict(n_q_heads=8, n_kv_heads=2, head_dim=64),
          dict(n_q_heads=2, n_kv_heads=2, head_dim=64)]


def run(inp, st, pos, lq):
    cfg = oracle.cfg_from(inp.params)
    uc = UnitCache(inp, cfg)
    B, hkv = inp.k.shape[0], inp.k.shape[1]
    hg = cfg.hq // cfg.hkv
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


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"hq{s['n_q_heads']}-hkv{s['n_kv_heads']}-d{s['head_dim']}")
def test_decode_shapes(shape):
    inp = synth.generate("prefill32k", batch=2, context=2048, overrides=dict(shape, needles=0))
    st = gh.build_state(inp)
    for pos, lq in ((2047, 1), (1500, 1), (1003, 5), (640, 15), (70, 3)):
        run(inp, st, pos, lq)


@pytest.mark.parametrize("shape", [s for s in SHAPES if s["head_dim"] == 128],
                         ids=lambda s: f"hq{s['n_q_heads']}-hkv{s['n_kv_heads']}")
def test_prefill_shapes(shape):
    inp = synth.generate("prefill32k", batch=2, context=2048, overrides=dict(shape, needles=0))
    st = gh.build_state(inp)
    for pos, lq in ((1984, 64), (1200, 16), (705, 40)):
        run(inp, st, pos, lq)


@pytest.mark.parametrize("shape", [s for s in SHAPES if s["head_dim"] == 128],
                         ids=lambda s: f"hq{s['n_q_heads']}-hkv{s['n_kv_heads']}")
def test_prompt_shapes(shape):
    """Whole-prompt prefill at every head ratio (the one-head workgroup form
    at ratio 1, head pairs otherwise): every query chunk of a 1K prompt and
    B = 2, against the oracle."""
    import long_context_hga_amd as hga
    inp = synth.generate("prompt32k", batch=2, context=1024, overrides=dict(shape))
    st = gh.build_state(inp, max_lq=64)
    cfg = oracle.cfg_from(inp.params)
    uc = UnitCache(inp, cfg)
    B, hkv, T = st.B, inp.k.shape[1], st.T
    hq, hg, nq = cfg.hq, cfg.hq // cfg.hkv, T // 64
    sel = torch.full((B, nq, hkv, st.max_sel), -7, dtype=torch.int32, device="cuda")
    n_sel = torch.full((B, nq, hkv), -7, dtype=torch.int32, device="cuda")
    out = torch.full((B, hq, T, 128), float("nan"), dtype=torch.float32, device="cuda")
    kp, vp = torch.zeros_like(st.k_pool), torch.zeros_like(st.v_pool)
    cs, gs = torch.zeros_like(st.chunk_sum), torch.zeros_like(st.group_sum)
    ws = torch.zeros(hga.hga_prompt_workspace_bytes(st.cfg, B, T, st.max_chunks),
                     dtype=torch.uint8, device="cuda")
    hga.hga_prefill_prompt(st.cfg, B, T, st.q, st.k_raw, st.v_raw, kp, vp, T, cs, gs,
                           st.max_chunks, sel, n_sel, st.max_sel, out, None, ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    sel_h, nsel_h, out_h = sel.cpu().numpy(), n_sel.cpu().numpy(), out.cpu().numpy()
    for b in range(B):
        for qc in range(nq):
            pos = qc * 64
            for h in range(hkv):
                cs_, gs_, kpo, vpo = uc.get(b, h)
                qu = q_unit(inp, cfg, b, h, pos, 64)
                g = sel_h[b, qc, h, :nsel_h[b, qc, h]]
                osel, margins, oscores = oracle.select(cfg, qu, pos, cs_, gs_)
                check_selection(cfg, g, osel, margins, oscores, pos, 64,
                                oracle.group_scores(cfg, qu, pos, gs_))
                o_ref, _ = oracle.attend(cfg, qu, pos, kpo, vpo, g)
                err = max_abs(out_h[b, h * hg:(h + 1) * hg, pos:pos + 64], o_ref)
                assert err <= ATOL_OUT, (b, qc, h, err)


@pytest.mark.parametrize("shape", [s for s in SHAPES if s["head_dim"] == 128][:3] +
                         [s for s in SHAPES if s["head_dim"] == 64][:1],
                         ids=lambda s: f"hq{s['n_q_heads']}-hkv{s['n_kv_heads']}-d{s['head_dim']}")
def test_prefill_step_shapes(shape):
    """The fused chunked-prefill step at other head ratios and head_dim 64
    (decode-kernel shapes there), bit-identical to the separate calls."""
    import long_context_hga_amd as hga
    inp = synth.generate("prefill32k", batch=2, context=2048, overrides=dict(shape, needles=0))
    st = gh.build_state(inp)
    B, T = st.B, st.T
    lq = 64 if shape["head_dim"] == 128 else 12
    pos = 20 * 64 + (0 if lq == 64 else 52)  # a whole chunk, or the tail that ends it
    c0 = pos // 64 * 64
    q = st.q[:, :, :lq].contiguous()
    kn = st.k_raw[:, :, pos:pos + lq].contiguous()
    vn = st.v_raw[:, :, pos:pos + lq].contiguous()
    pos_t = torch.full((B,), pos, dtype=torch.int32, device="cuda")

    def fresh():
        kp = torch.zeros_like(st.k_pool)
        vp = torch.zeros_like(st.v_pool)
        cs = torch.zeros_like(st.chunk_sum)
        gs = torch.zeros_like(st.group_sum)
        hga.hga_build_summaries(st.cfg, B, st.k_raw[:, :, :pos].contiguous(),
                                st.v_raw[:, :, :pos].contiguous(), 0, pos, kp, vp, T, cs, gs,
                                st.max_chunks)
        return kp, vp, cs, gs

    ka, va, csa, gsa = fresh()
    sa = gh.alloc_step(st, lq)
    hga.hga_build_summaries(st.cfg, B, kn, vn, pos, lq, ka, va, T, None, None, st.max_chunks)
    hga.hga_build_summaries(st.cfg, B, st.k_raw[:, :, c0:c0 + 64].contiguous(), None, c0, 64,
                            None, None, T, csa, gsa, st.max_chunks)
    hga.hga_route(st.cfg, B, q, lq, pos_t, csa, gsa, st.max_chunks, sa.sel, sa.n_sel, st.max_sel,
                  None, st.ws)
    hga.hga_attend(st.cfg, B, q, lq, pos_t, ka, va, hga.HGA_SRC_POOL, T, sa.sel, sa.n_sel,
                   st.max_sel, hga.HGA_PART_ALL, sa.out, sa.lse, st.ws)
    kb, vb, csb, gsb = fresh()
    stage = torch.zeros_like(st.k_raw[:, :, :64])
    stage[:, :, :pos - c0] = st.k_raw[:, :, c0:pos]
    sb = gh.alloc_step(st, lq)
    hga.hga_prefill_step(st.cfg, B, q, lq, kn, vn, pos_t, kb, vb, T, stage, csb, gsb,
                         st.max_chunks, sb.sel, sb.n_sel, st.max_sel, sb.out, sb.lse,
                         torch.zeros_like(st.ws))
    torch.cuda.synchronize()
    assert torch.equal(sa.n_sel, sb.n_sel)
    assert torch.equal(sa.out, sb.out) and torch.equal(sa.lse, sb.lse)
    assert torch.equal(ka, kb) and torch.equal(va, vb)
    assert torch.equal(csa, csb) and torch.equal(gsa, gsb)
