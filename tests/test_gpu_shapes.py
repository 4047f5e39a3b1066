"""GPU parity on head shapes beyond the benchmark layer: every supported
query-heads-per-KV-head ratio (1, 2, 4, 8) at head_dim 128 and 64, bf16, for
decode (1 and several query tokens) and, at head_dim 128, chunked prefill;
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
            check_selection(cfg, g, osel, margins, oscores, pos, lq)
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
