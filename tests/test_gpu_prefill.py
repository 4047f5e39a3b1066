"""GPU parity of chunked-prefill attention (16..64 query tokens of one chunk,
the MFMA kernel) against the fp64 oracle, through the C ABI.

Comparison rules: tests/oracle_ref.py.  Inputs: the prefill32k workload
(32/4 heads, d=128, bf16, 16 planted needle chunks) at its full size and at
reduced contexts, with query chunks of ragged lengths and offsets.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth
from oracle_ref import ATOL_OUT, UnitCache, check_selection, max_abs, q_unit

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import long_context_hga_amd as hga  # noqa: E402
import gpu_harness as gh  # noqa: E402


def say(*a):
    print(*a, flush=True)


def ora_cfg(inp, **over):
    p = dict(inp.params)
    p.update(over)
    return oracle.cfg_from(p)


def run_prefill(inp, st, pos, lq, tok0=0, cfg_over=None, check_sel=True, uc=None):
    """Route + attend the query tokens tok0..tok0+lq-1 placed at positions
    pos..pos+lq-1 for every unit; compare with the oracle.  Returns the worst
    output error and the step."""
    cfg = ora_cfg(inp, **(cfg_over or {}))
    uc = uc or UnitCache(inp, cfg)
    B, hkv = inp.k.shape[0], inp.k.shape[1]
    hg = cfg.hq // cfg.hkv
    q = st.q[:, :, tok0:tok0 + lq].contiguous()
    pos_t = torch.full((B,), pos, dtype=torch.int32, device="cuda")
    s = gh.alloc_step(st, lq)
    gh.route(st, q, lq, pos_t, s)
    gh.attend(st, q, lq, pos_t, s)
    torch.cuda.synchronize()
    sel, nsel = s.sel.cpu().numpy(), s.n_sel.cpu().numpy()
    out, lse = s.out.cpu().numpy(), s.lse.cpu().numpy()
    worst = 0.0
    for b in range(B):
        for h in range(hkv):
            cs, gs, kp, v = uc.get(b, h)
            qu = q_unit(inp, cfg, b, h, tok0, lq)
            g = sel[b, h, :nsel[b, h]]
            if check_sel:
                osel, margins, oscores = oracle.select(cfg, qu, pos, cs, gs)
                check_selection(cfg, g, osel, margins, oscores, pos, lq,
                                oracle.group_scores(cfg, qu, pos, gs))
            o_ref, l_ref = oracle.attend(cfg, qu, pos, kp, v, g)
            err = max_abs(out[b, h * hg:(h + 1) * hg], o_ref)
            worst = max(worst, err)
            assert err <= ATOL_OUT, (pos, lq, b, h, err)
            assert max_abs(lse[b, h * hg:(h + 1) * hg], l_ref) <= 1e-3
    return worst, s


def test_prefill32k_full_attend():
    """The prefill workload at full size: last chunk of a 32K context, 1024
    selected keys per KV head, all 32 heads x 64 tokens against the oracle."""
    inp = synth.generate("prefill32k")
    st = gh.build_state(inp)
    pos = int(inp.pos0[0])
    say(f"[prefill32k] pos {pos}")
    worst, s = run_prefill(inp, st, pos, 64)
    assert (s.n_sel == 64).all()
    chunks = set(int(x) // 4 for x in s.sel[0].flatten().cpu().numpy())
    assert set(int(c) for c in inp.needle_chunks[0]) <= chunks
    say(f"[prefill32k] worst |out - oracle| = {worst:.2e}")


@pytest.mark.parametrize("chunk,off,lq", [(63, 0, 64), (63, 0, 16), (62, 5, 17), (40, 16, 48),
                                          (50, 31, 33), (33, 1, 63), (20, 47, 17), (7, 0, 64),
                                          (5, 0, 40), (1, 10, 54), (0, 0, 16), (0, 32, 32)])
def test_prefill_ragged_query_chunks(chunk, off, lq):
    """Query chunks of 16..64 tokens at any offset inside their chunk, from
    the first chunk (windows only) to the last one of a 4K context; B = 2."""
    inp = synth.generate("prefill32k", batch=2, context=4096)
    st = gh.build_state(inp)
    pos = chunk * 64 + off
    say(f"[prefill ragged] pos {pos} lq {lq}")
    run_prefill(inp, st, pos, lq)


def test_prefill_select_all_equals_dense():
    """Budgets above the candidate count select every chunk: the output is
    dense causal attention over 0..tau for each query token."""
    T = 2048
    inp = synth.generate("prefill32k", context=T)
    over = dict(topk_chunks=40, topk_groups=160)
    st = gh.build_state(inp, cfg_over=over)
    cfg = ora_cfg(inp, **over)
    pos = T - 64
    q = st.q.contiguous()
    s = gh.alloc_step(st, 64)
    gh.route(st, q, 64, st.pos0, s)
    gh.attend(st, q, 64, st.pos0, s)
    torch.cuda.synchronize()
    assert (s.n_sel == T // 16).all()
    hg = 8
    out = s.out.cpu().numpy()
    for h in range(4):
        kp = oracle.pool(cfg, inp.f64(inp.k[0, h]), 0)
        v = inp.f64(inp.v[0, h])
        qu = q_unit(inp, cfg, 0, h, 0, 64)
        o_ref, _ = oracle.attend(cfg, qu, pos, kp, v, np.arange(T // 16))
        assert max_abs(out[0, h * hg:(h + 1) * hg], o_ref) <= ATOL_OUT


def test_prefill_parts_merge_and_working_set():
    """windows + routed parts merged == all; the working-set source gives the
    same bits as the pool source."""
    inp = synth.generate("prefill32k", batch=2, context=8192)
    st = gh.build_state(inp)
    q = st.q.contiguous()
    s = gh.alloc_step(st, 64)
    gh.route(st, q, 64, st.pos0, s)
    gh.attend(st, q, 64, st.pos0, s)
    out_all, lse_all = s.out.clone(), s.lse.clone()
    oa, la = torch.empty_like(s.out), torch.empty_like(s.lse)
    ob, lb = torch.empty_like(s.out), torch.empty_like(s.lse)
    gh.attend(st, q, 64, st.pos0, s, part=hga.HGA_PART_WINDOWS, out=oa, lse=la)
    gh.attend(st, q, 64, st.pos0, s, part=hga.HGA_PART_ROUTED, out=ob, lse=lb)
    om, lm = torch.empty_like(oa), torch.empty_like(la)
    hga.hga_merge_partials(st.cfg, st.B, 64, oa, la, ob, lb, om, lm)
    kw = torch.zeros((st.B, 4, st.max_sel * 16, 128), dtype=torch.int16, device="cuda")
    vw = torch.zeros_like(kw)
    hga.hga_gather(st.cfg, st.B, st.k_pool, st.v_pool, st.T, 0, s.sel, s.n_sel, st.max_sel,
                   st.pos0, hga.HGA_PART_ALL, kw, vw)
    ow, lw = torch.empty_like(s.out), torch.empty_like(s.lse)
    gh.attend(st, q, 64, st.pos0, s, k_src=kw, v_src=vw, layout=hga.HGA_SRC_WORKING_SET, out=ow,
              lse=lw)
    torch.cuda.synchronize()
    assert (om - out_all).abs().max().item() <= 1e-5
    assert (lm - lse_all).abs().max().item() <= 1e-5
    assert torch.equal(ow, out_all) and torch.equal(lw, lse_all)


def test_unwritten_rows_after_the_query_are_ignored():
    """Pool rows after the last query token (not yet appended) may hold any
    bits, NaN included: prefill and decode outputs stay equal to the oracle."""
    inp = synth.generate("prefill32k", context=4096)
    st = gh.build_state(inp)
    cfg = ora_cfg(inp)
    uc = UnitCache(inp, cfg)
    pos, lq = 30 * 64 + 3, 20
    nan_bits = torch.tensor([0x7FC0], dtype=torch.int32).to(torch.int16).item()
    st.k_pool[:, :, pos + lq:] = nan_bits
    vt = gh.v_token_view(st.v_pool)  # V groups are stored transposed
    p1 = pos + lq
    vt[:, :, p1 // 16, p1 % 16:] = nan_bits
    vt[:, :, p1 // 16 + 1:] = nan_bits
    run_prefill(inp, st, pos, lq, check_sel=False, uc=uc)
    # decode: token 5 of the query chunk at position pos + 7
    p1 = pos + 7
    q = st.q[:, :, 5:6].contiguous()
    pos_t = torch.full((1,), p1, dtype=torch.int32, device="cuda")
    s = gh.alloc_step(st, 1)
    gh.route(st, q, 1, pos_t, s)
    gh.attend(st, q, 1, pos_t, s)
    torch.cuda.synchronize()
    out = s.out.cpu().numpy()
    assert np.isfinite(out).all()
    for h in range(4):
        _, _, kp, v = uc.get(0, h)
        g = s.sel[0, h, :int(s.n_sel[0, h])].cpu().numpy()
        o_ref, _ = oracle.attend(cfg, q_unit(inp, cfg, 0, h, 5, 1), p1, kp, v, g)
        assert max_abs(out[0, h * 8:(h + 1) * 8], o_ref) <= ATOL_OUT


def test_prefill_invalid_position_is_loud():
    inp = synth.generate("prefill32k", context=4096)
    st = gh.build_state(inp)
    q = st.q[:, :, :32].contiguous()
    s = gh.alloc_step(st, 32)
    for bad in (-64, 4096 * 4, 40 * 64 + 40):  # negative, beyond capacity, crossing a chunk end
        pos_t = torch.full((1,), bad, dtype=torch.int32, device="cuda")
        gh.route(st, q, 32, pos_t, s)
        gh.attend(st, q, 32, pos_t, s)
        torch.cuda.synchronize()
        assert (s.n_sel == -1).all()
        assert torch.isnan(s.out).all()


def test_prefill_determinism_bitwise():
    inp = synth.generate("prefill32k", context=8192)
    st = gh.build_state(inp)
    q = st.q.contiguous()
    res = []
    for _ in range(3):
        s = gh.alloc_step(st, 64)
        gh.route(st, q, 64, st.pos0, s)
        gh.attend(st, q, 64, st.pos0, s)
        torch.cuda.synchronize()
        res.append((s.out.clone(), s.lse.clone()))
    for r in res[1:]:
        assert torch.equal(r[0], res[0][0]) and torch.equal(r[1], res[0][1])


@pytest.mark.parametrize("chunk,off,lq", [(63, 62, 2), (40, 5, 3), (33, 57, 7), (20, 0, 15),
                                          (0, 1, 15), (2, 49, 15)])
def test_multi_token_decode(chunk, off, lq):
    """2..15 query tokens of one chunk (several 16-row column blocks of
    (head, token) rows on the decode kernel) against the oracle."""
    inp = synth.generate("prefill32k", batch=2, context=4096)
    st = gh.build_state(inp)
    say(f"[multi-token decode] pos {chunk * 64 + off} lq {lq}")
    run_prefill(inp, st, chunk * 64 + off, lq)
