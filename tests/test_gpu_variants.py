"""GPU parity of the routing / summary variants against the fp64 oracle with
the same switches: the high-frequency threshold at the group length
(lambda_hf = g = 16 instead of C = 64) and the representative position
a + n/2 instead of the midpoint a + (n-1)/2 (tests/oracle_ref.py rules:
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
            dict(hf_wavelength=16.0, rep_position=1)]


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
                check_selection(cfg, g, osel, margins, oscores, pos, lq)
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
        assert torch.equal(st.k_pool, base.k_pool)  # the pool does not depend on them
