"""GPU parity of the whole-prompt chunked prefill (hga_prefill_prompt): every
64-token query chunk of a prompt routed and attended in one call, against the
fp64 oracle (selection under the margin rule, outputs within the tolerance)
and against the per-chunk entry points (hga_route bit-exact, hga_attend to
fp32 rounding).  Inputs: the prompt32k workload (queries for every token of
the prefill32k layer) at 2K and at its full 32K size."""
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


class Prompt:
    """Buffers of one hga_prefill_prompt call over the inputs of ``inp``."""

    def __init__(self, inp, st):
        p = inp.params
        self.B, self.T = st.B, st.T
        self.nq = self.T // 64
        hkv, hq, d = p["n_kv_heads"], p["n_q_heads"], p["head_dim"]
        self.cfg = st.cfg
        self.max_sel = st.max_sel
        self.max_chunks = st.max_chunks
        self.k_pool = torch.zeros_like(st.k_pool)
        self.v_pool = torch.zeros_like(st.v_pool)
        self.chunk_sum = torch.zeros_like(st.chunk_sum)
        self.group_sum = torch.zeros_like(st.group_sum)
        self.sel = torch.full((self.B, self.nq, hkv, self.max_sel), -7, dtype=torch.int32,
                              device="cuda")
        self.n_sel = torch.full((self.B, self.nq, hkv), -7, dtype=torch.int32, device="cuda")
        self.out = torch.full((self.B, hq, self.T, d), float("nan"), dtype=torch.float32,
                              device="cuda")
        self.lse = torch.full((self.B, hq, self.T), float("nan"), dtype=torch.float32,
                              device="cuda")
        wsb = hga.hga_prompt_workspace_bytes(self.cfg, self.B, self.T, self.max_chunks)
        self.ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")

    def run(self, st, phases=hga.HGA_PROMPT_ALL):
        hga.hga_prefill_prompt(self.cfg, self.B, self.T, st.q, st.k_raw, st.v_raw, self.k_pool,
                               self.v_pool, self.T, self.chunk_sum, self.group_sum,
                               self.max_chunks, self.sel, self.n_sel, self.max_sel, self.out,
                               self.lse, self.ws, phases=phases)


def check_chunks(inp, pr, chunks):
    """Selections and outputs of the given query chunks against the oracle."""
    cfg = oracle.cfg_from(inp.params)
    uc = UnitCache(inp, cfg)
    hg = cfg.hq // cfg.hkv
    sel, nsel = pr.sel.cpu().numpy(), pr.n_sel.cpu().numpy()
    out, lse = pr.out.cpu().numpy(), pr.lse.cpu().numpy()
    worst = 0.0
    for b in range(pr.B):
        for qc in chunks:
            pos = qc * 64
            for h in range(cfg.hkv):
                cs, gs, kp, v = uc.get(b, h)
                qu = q_unit(inp, cfg, b, h, pos, 64)
                g = sel[b, qc, h, :nsel[b, qc, h]]
                osel, margins, oscores = oracle.select(cfg, qu, pos, cs, gs)
                check_selection(cfg, g, osel, margins, oscores, pos, 64,
                                oracle.group_scores(cfg, qu, pos, gs))
                o_ref, l_ref = oracle.attend(cfg, qu, pos, kp, v, g)
                got = out[b, h * hg:(h + 1) * hg, pos:pos + 64]
                err = max_abs(got, o_ref)
                worst = max(worst, err)
                assert err <= ATOL_OUT, (b, qc, h, err)
                assert max_abs(lse[b, h * hg:(h + 1) * hg, pos:pos + 64], l_ref) <= 1e-3
    return worst


def test_prompt_2k_every_chunk_against_oracle():
    """Every query chunk of a 2K prompt (32 chunks, from windows only to
    routed), 4 KV heads x 8 query heads, against the oracle; the append phase
    writes the same pool and summaries as hga_build_summaries."""
    inp = synth.generate("prompt32k", context=2048)
    st = gh.build_state(inp, max_lq=64)
    pr = Prompt(inp, st)
    pr.run(st)
    torch.cuda.synchronize()
    assert torch.equal(pr.k_pool, st.k_pool) and torch.equal(pr.v_pool, st.v_pool)
    assert torch.equal(pr.chunk_sum, st.chunk_sum) and torch.equal(pr.group_sum, st.group_sum)
    assert torch.isfinite(pr.out).all()
    worst = check_chunks(inp, pr, range(pr.nq))
    say(f"[prompt 2k] worst |out - oracle| = {worst:.2e}")


def test_prompt_phases_and_per_chunk_calls():
    """The phases run one at a time give the bits of one call; each chunk's
    list equals hga_route for that chunk alone, its output hga_attend's."""
    inp = synth.generate("prompt32k", batch=2, context=4096)
    st = gh.build_state(inp, max_lq=64)
    pr_all = Prompt(inp, st)
    pr_all.run(st)
    pr = Prompt(inp, st)
    for ph in (hga.HGA_PROMPT_APPEND, hga.HGA_PROMPT_ROUTE, hga.HGA_PROMPT_ATTEND):
        pr.run(st, phases=ph)
    torch.cuda.synchronize()
    assert torch.equal(pr.sel, pr_all.sel) and torch.equal(pr.n_sel, pr_all.n_sel)
    assert torch.equal(pr.out, pr_all.out) and torch.equal(pr.lse, pr_all.lse)
    for qc in (0, 5, 6, 17, 40, 63):
        pos = qc * 64
        q = st.q[:, :, pos:pos + 64].contiguous()
        pos_t = torch.full((st.B,), pos, dtype=torch.int32, device="cuda")
        s = gh.alloc_step(st, 64)
        gh.route(st, q, 64, pos_t, s)
        gh.attend(st, q, 64, pos_t, s)
        torch.cuda.synchronize()
        assert torch.equal(s.n_sel, pr.n_sel[:, qc]), qc
        for b in range(st.B):
            for h in range(4):
                n = int(s.n_sel[b, h])
                assert torch.equal(s.sel[b, h, :n], pr.sel[b, qc, h, :n]), (qc, b, h)
        diff = (s.out - pr.out[:, :, pos:pos + 64]).abs().max().item()
        assert diff <= 1e-5, (qc, diff)
        assert (s.lse - pr.lse[:, :, pos:pos + 64]).abs().max().item() <= 1e-5


def test_prompt_32k_sampled_chunks():
    """The full 32K prompt (512 query chunks in one call); sampled chunks
    against the oracle, every output finite, the full budget selected."""
    inp = synth.generate("prompt32k")
    st = gh.build_state(inp, max_lq=64)
    pr = Prompt(inp, st)
    pr.run(st)
    torch.cuda.synchronize()
    assert torch.isfinite(pr.out).all()
    assert (pr.n_sel[:, 25:] == st.max_sel).all()  # full budget once 20 chunks are candidates
    worst = check_chunks(inp, pr, [0, 7, 100, 511])
    say(f"[prompt 32k] worst |out - oracle| = {worst:.2e}")


def test_prompt_unusable_list_is_loud():
    """A list length outside 0..max_sel (never written by the route phase)
    gives NaN outputs for its query chunk, and only for it."""
    inp = synth.generate("prompt32k", context=1024)
    st = gh.build_state(inp, max_lq=64)
    pr = Prompt(inp, st)
    pr.run(st, phases=hga.HGA_PROMPT_APPEND | hga.HGA_PROMPT_ROUTE)
    pr.n_sel[0, 9, 2] = -1
    pr.run(st, phases=hga.HGA_PROMPT_ATTEND)
    torch.cuda.synchronize()
    hg = 8
    bad = pr.out[0, 2 * hg:3 * hg, 9 * 64:10 * 64]
    assert torch.isnan(bad).all()
    pr.out[0, 2 * hg:3 * hg, 9 * 64:10 * 64] = 0.0
    assert torch.isfinite(pr.out).all()
