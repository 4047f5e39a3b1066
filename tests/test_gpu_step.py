"""GPU parity of the fused decode step (hga_decode_step) against the separate
entry points it fuses (hga_build_summaries, hga_route, hga_attend) and
against the fp64 oracle, over consecutive positions that cross a chunk end."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth
from oracle_ref import ATOL_OUT, UnitCache, max_abs, q_unit

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import long_context_hga_amd as hga  # noqa: E402
import gpu_harness as gh  # noqa: E402


def fresh(st, p_start):
    """Pools and summaries built for positions 0 .. p_start-1 only."""
    B, hkv, T, d = st.k_pool.shape
    kp = torch.zeros_like(st.k_pool)
    vp = torch.zeros_like(st.v_pool)
    cs = torch.zeros_like(st.chunk_sum)
    gs = torch.zeros_like(st.group_sum)
    hga.hga_build_summaries(st.cfg, B, st.k_raw[:, :, :p_start].contiguous(),
                            st.v_raw[:, :, :p_start].contiguous(), 0, p_start, kp, vp, T, cs, gs,
                            st.max_chunks)
    return kp, vp, cs, gs


@pytest.mark.parametrize("name,B,T,p_start,n_steps", [("decode64k", 2, 4096, 4026, 12),
                                                      ("host64k", 1, 8192, 8127, 65),
                                                      ("tiny", 1, 1024, 1016, 8)])
def test_decode_step_equals_separate_calls(name, B, T, p_start, n_steps):
    inp = synth.generate(name, batch=B, context=T)
    st = gh.build_state(inp, max_lq=1)
    q = gh.query_slice(st, 0)
    ka, va, csa, gsa = fresh(st, p_start)
    kb, vb, csb, gsb = fresh(st, p_start)
    c0 = p_start // 64 * 64
    stage = torch.zeros_like(st.k_raw[:, :, :64])
    stage[:, :, :p_start - c0] = st.k_raw[:, :, c0:p_start]
    wsb = torch.zeros_like(st.ws)
    cfg = st.cfg
    for i in range(n_steps):
        p = p_start + i
        pos_t = torch.full((B,), p, dtype=torch.int32, device="cuda")
        kt = st.k_raw[:, :, p:p + 1].contiguous()
        vt = st.v_raw[:, :, p:p + 1].contiguous()
        # separate calls
        sa = gh.alloc_step(st, 1)
        hga.hga_build_summaries(cfg, B, kt, vt, p, 1, ka, va, T, None, None, st.max_chunks)
        if p % 64 == 63:
            hga.hga_build_summaries(cfg, B, st.k_raw[:, :, p - 63:p + 1].contiguous(), None, p - 63,
                                    64, None, None, T, csa, gsa, st.max_chunks)
        hga.hga_route(cfg, B, q, 1, pos_t, csa, gsa, st.max_chunks, sa.sel, sa.n_sel, st.max_sel,
                      None, st.ws)
        hga.hga_attend(cfg, B, q, 1, pos_t, ka, va, hga.HGA_SRC_POOL, T, sa.sel, sa.n_sel,
                       st.max_sel, hga.HGA_PART_ALL, sa.out, sa.lse, st.ws)
        # fused step
        sb = gh.alloc_step(st, 1)
        hga.hga_decode_step(cfg, B, q, kt, vt, pos_t, kb, vb, T, stage, csb, gsb, st.max_chunks,
                            sb.sel, sb.n_sel, st.max_sel, sb.out, sb.lse, wsb)
        torch.cuda.synchronize()
        assert torch.equal(sa.n_sel, sb.n_sel), p
        for b in range(B):
            for h in range(st.k_pool.shape[1]):
                n = int(sa.n_sel[b, h])
                assert torch.equal(sa.sel[b, h, :n], sb.sel[b, h, :n]), (p, b, h)
        assert torch.equal(sa.out, sb.out) and torch.equal(sa.lse, sb.lse), p
    assert torch.equal(ka, kb) and torch.equal(va, vb)
    assert torch.equal(csa, csb) and torch.equal(gsa, gsb)
    assert torch.equal(stage[:, :, (p_start + n_steps - 1) % 64],
                       st.k_raw[:, :, p_start + n_steps - 1])
    # the last step against the oracle
    ocfg = oracle.cfg_from(inp.params)
    uc = UnitCache(inp, ocfg)
    hg = ocfg.hq // ocfg.hkv
    out = sb.out.cpu().numpy()
    for b in range(B):
        for h in range(st.k_pool.shape[1]):
            _, _, kpo, vpo = uc.get(b, h)
            g = sb.sel[b, h, :int(sb.n_sel[b, h])].cpu().numpy()
            o_ref, _ = oracle.attend(ocfg, q_unit(inp, ocfg, b, h, 0, 1), p, kpo, vpo, g)
            assert max_abs(out[b, h * hg:(h + 1) * hg], o_ref) <= ATOL_OUT


def test_decode_step_invalid_position_writes_nothing():
    inp = synth.generate("decode64k", batch=1, context=2048)
    st = gh.build_state(inp, max_lq=1)
    q = gh.query_slice(st, 0)
    kp0, vp0 = st.k_pool.clone(), st.v_pool.clone()
    cs0, gs0 = st.chunk_sum.clone(), st.group_sum.clone()
    stage = torch.zeros_like(st.k_raw[:, :, :64])
    s = gh.alloc_step(st, 1)
    for bad in (-1, 2048, 1 << 20):
        pos_t = torch.full((1,), bad, dtype=torch.int32, device="cuda")
        hga.hga_decode_step(st.cfg, 1, q, st.k_raw[:, :, :1].contiguous(),
                            st.v_raw[:, :, :1].contiguous(), pos_t, st.k_pool, st.v_pool, st.T,
                            stage, st.chunk_sum, st.group_sum, st.max_chunks, s.sel, s.n_sel,
                            st.max_sel, s.out, s.lse, st.ws)
        torch.cuda.synchronize()
        assert (s.n_sel == -1).all() and torch.isnan(s.out).all()
    assert torch.equal(st.k_pool, kp0) and torch.equal(st.v_pool, vp0)
    assert torch.equal(st.chunk_sum, cs0) and torch.equal(st.group_sum, gs0)
    assert not stage.any()


def test_step_position_beyond_pool_writes_nothing():
    """Summary tables longer than the pool: a step whose tokens do not fit the
    pool is unusable (n_sel = -1, NaN outputs) and writes nothing, while the
    last position that fits works."""
    inp = synth.generate("decode64k", batch=1, context=2048)
    st = gh.build_state(inp, max_lq=10)
    cap = 1008  # 63 groups; the summary tables hold 32 chunks (2048 tokens)
    kp = st.k_pool[:, :, :cap].contiguous()
    vp = st.v_pool[:, :, :cap].contiguous()
    kp0, vp0 = kp.clone(), vp.clone()
    cs0, gs0 = st.chunk_sum.clone(), st.group_sum.clone()
    stage = torch.zeros_like(st.k_raw[:, :, :64])
    for bad, lq in ((1008, 1), (1500, 1), (2047, 1), (1000, 10)):
        print(f"[beyond pool] pos {bad} lq {lq}", flush=True)
        s = gh.alloc_step(st, lq)
        pos_t = torch.full((1,), bad, dtype=torch.int32, device="cuda")
        q = st.q[:, :, :1].repeat(1, 1, lq, 1).contiguous()  # the workload holds one token
        hga.hga_prefill_step(st.cfg, 1, q, lq,
                             st.k_raw[:, :, :lq].contiguous(), st.v_raw[:, :, :lq].contiguous(),
                             pos_t, kp, vp, cap, stage, st.chunk_sum, st.group_sum, st.max_chunks,
                             s.sel, s.n_sel, st.max_sel, s.out, s.lse, st.ws)
        torch.cuda.synchronize()
        assert (s.n_sel == -1).all() and torch.isnan(s.out).all(), bad
    assert torch.equal(kp, kp0) and torch.equal(vp, vp0)
    assert torch.equal(st.chunk_sum, cs0) and torch.equal(st.group_sum, gs0)
    assert not stage.any()
    s = gh.alloc_step(st, 1)
    pos_t = torch.full((1,), cap - 1, dtype=torch.int32, device="cuda")
    hga.hga_decode_step(st.cfg, 1, gh.query_slice(st, 0), st.k_raw[:, :, cap - 1].contiguous(),
                        st.v_raw[:, :, cap - 1].contiguous(), pos_t, kp, vp, cap, stage,
                        st.chunk_sum, st.group_sum, st.max_chunks, s.sel, s.n_sel, st.max_sel,
                        s.out, s.lse, st.ws)
    torch.cuda.synchronize()
    assert (s.n_sel > 0).all() and torch.isfinite(s.out).all()


@pytest.mark.parametrize("B,T,pos,lq", [(1, 4096, 4032, 64),       # the whole last chunk
                                        (2, 4096, 40 * 64, 64),    # a whole chunk mid-context
                                        (2, 4096, 30 * 64 + 47, 17),  # ends its chunk
                                        (2, 4096, 30 * 64 + 3, 20),   # inside a chunk
                                        (2, 4096, 20 * 64 + 59, 5),   # decode kernel, ends its chunk
                                        (1, 2048, 7 * 64 + 16, 48)])
def test_prefill_step_equals_separate_calls(B, T, pos, lq):
    """hga_prefill_step (append + chunk summaries + route + attend of lq query
    tokens in four launches) gives the bits of the separate calls; its output
    matches the oracle's attention over the selection."""
    inp = synth.generate("prefill32k", batch=B, context=T)
    st = gh.build_state(inp)
    cfg = st.cfg
    q = st.q[:, :, :lq].contiguous()
    pos_t = torch.full((B,), pos, dtype=torch.int32, device="cuda")
    kn = st.k_raw[:, :, pos:pos + lq].contiguous()
    vn = st.v_raw[:, :, pos:pos + lq].contiguous()
    c0 = pos // 64 * 64
    ends = pos + lq == c0 + 64
    print(f"[prefill step] B {B} T {T} pos {pos} lq {lq}", flush=True)
    # separate calls
    ka, va, csa, gsa = fresh(st, pos)
    sa = gh.alloc_step(st, lq)
    hga.hga_build_summaries(cfg, B, kn, vn, pos, lq, ka, va, T, None, None, st.max_chunks)
    if ends:
        hga.hga_build_summaries(cfg, B, st.k_raw[:, :, c0:c0 + 64].contiguous(), None, c0, 64,
                                None, None, T, csa, gsa, st.max_chunks)
    hga.hga_route(cfg, B, q, lq, pos_t, csa, gsa, st.max_chunks, sa.sel, sa.n_sel, st.max_sel,
                  None, st.ws)
    hga.hga_attend(cfg, B, q, lq, pos_t, ka, va, hga.HGA_SRC_POOL, T, sa.sel, sa.n_sel, st.max_sel,
                   hga.HGA_PART_ALL, sa.out, sa.lse, st.ws)
    # fused step
    kb, vb, csb, gsb = fresh(st, pos)
    stage = torch.zeros_like(st.k_raw[:, :, :64])
    stage[:, :, :pos - c0] = st.k_raw[:, :, c0:pos]
    sb = gh.alloc_step(st, lq)
    wsb = torch.zeros_like(st.ws)
    hga.hga_prefill_step(cfg, B, q, lq, kn, vn, pos_t, kb, vb, T, stage, csb, gsb, st.max_chunks,
                         sb.sel, sb.n_sel, st.max_sel, sb.out, sb.lse, wsb)
    torch.cuda.synchronize()
    assert torch.equal(sa.n_sel, sb.n_sel)
    assert (sb.n_sel > 0).all()
    for b in range(B):
        for h in range(st.k_pool.shape[1]):
            n = int(sa.n_sel[b, h])
            assert torch.equal(sa.sel[b, h, :n], sb.sel[b, h, :n]), (b, h)
    assert torch.equal(sa.out, sb.out) and torch.equal(sa.lse, sb.lse)
    assert torch.equal(ka, kb) and torch.equal(va, vb)
    assert torch.equal(csa, csb) and torch.equal(gsa, gsb)
    assert torch.equal(stage[:, :, pos - c0:pos - c0 + lq], kn)
    if ends:  # the chunk's summaries exist now
        assert csb[:, :, pos // 64].abs().sum().item() > 0
    ocfg = oracle.cfg_from(inp.params)
    uc = UnitCache(inp, ocfg)
    hg = ocfg.hq // ocfg.hkv
    out = sb.out.cpu().numpy()
    for b in range(B):
        for h in range(st.k_pool.shape[1]):
            _, _, kpo, vpo = uc.get(b, h)
            g = sb.sel[b, h, :int(sb.n_sel[b, h])].cpu().numpy()
            o_ref, _ = oracle.attend(ocfg, q_unit(inp, ocfg, b, h, 0, lq), pos, kpo, vpo, g)
            assert max_abs(out[b, h * hg:(h + 1) * hg], o_ref) <= ATOL_OUT


def test_prefill_step_unusable_position_writes_nothing():
    inp = synth.generate("prefill32k", batch=1, context=2048)
    st = gh.build_state(inp)
    q = st.q[:, :, :20].contiguous()
    kp0, vp0 = st.k_pool.clone(), st.v_pool.clone()
    cs0, gs0 = st.chunk_sum.clone(), st.group_sum.clone()
    stage = torch.zeros_like(st.k_raw[:, :, :64])
    s = gh.alloc_step(st, 20)
    for bad in (-5, 10 * 64 + 50, 2048 - 10, 1 << 20):  # negative, crossing a chunk end, beyond
        pos_t = torch.full((1,), bad, dtype=torch.int32, device="cuda")
        hga.hga_prefill_step(st.cfg, 1, q, 20, st.k_raw[:, :, :20].contiguous(),
                             st.v_raw[:, :, :20].contiguous(), pos_t, st.k_pool, st.v_pool, st.T,
                             stage, st.chunk_sum, st.group_sum, st.max_chunks, s.sel, s.n_sel,
                             st.max_sel, s.out, s.lse, st.ws)
        torch.cuda.synchronize()
        assert (s.n_sel == -1).all() and torch.isnan(s.out).all(), bad
    assert torch.equal(st.k_pool, kp0) and torch.equal(st.v_pool, vp0)
    assert torch.equal(st.chunk_sum, cs0) and torch.equal(st.group_sum, gs0)
    assert not stage.any()
