"""GPU parity of the host-tier attention (hga_attend_tiered): windows from the
device pool on one stream, routed groups copied over PCIe from a pinned host
pool and attended on a second stream, merged exactly.  Checked against
hga_attend over the whole list and against the fp64 oracle."""
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


def pinned_copy(t):
    h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    h.copy_(t)
    return h


def run_tiered(st, kc, vc, q, lq, pos_t, side):
    s = gh.alloc_step(st, lq)
    gh.route(st, q, lq, pos_t, s)
    gh.attend(st, q, lq, pos_t, s)  # reference: the whole list from the device pool
    kw = torch.zeros((st.B, st.k_pool.shape[1], st.max_sel * 16, st.k_pool.shape[3]),
                     dtype=st.k_pool.dtype, device="cuda")
    vw = torch.zeros_like(kw)
    out = torch.full_like(s.out, float("nan"))
    lse = torch.full_like(s.lse, float("nan"))
    ws2 = torch.zeros_like(st.ws)
    hga.hga_attend_tiered(st.cfg, st.B, q, lq, pos_t, st.k_pool, st.v_pool, st.T, kc, vc, st.T,
                          s.sel, s.n_sel, st.max_sel, kw, vw, out, lse, ws2, stream_b=side,
                          events=(torch.cuda.Event(), torch.cuda.Event()))
    torch.cuda.synchronize()
    return s, out, lse


@pytest.mark.parametrize("B,T,form", [(2, 8192, "two streams"), (1, 4096, "two streams"),
                                      (2, 8192, "one launch"), (1, 4096, "one launch")])
def test_tiered_decode_equals_device_path_and_oracle(B, T, form):
    """Both forms: two streams (copy + routed attention on the second), and
    one stream with the window attention and the copy in one launch."""
    inp = synth.generate("host64k", batch=B, context=T)
    st = gh.build_state(inp)
    kc, vc = pinned_copy(st.k_pool), pinned_copy(st.v_pool)
    side = torch.cuda.Stream() if form == "two streams" else None
    q = gh.query_slice(st, 0)
    s, out, lse = run_tiered(st, kc, vc, q, 1, st.pos0, side)
    assert (out - s.out).abs().max().item() <= 1e-5
    assert (lse - s.lse).abs().max().item() <= 1e-5
    cfg = oracle.cfg_from(inp.params)
    uc = UnitCache(inp, cfg)
    pos = int(inp.pos0[0])
    o = out.cpu().numpy()
    for b in range(B):
        for h in range(4):
            _, _, kp, v = uc.get(b, h)
            g = s.sel[b, h, :int(s.n_sel[b, h])].cpu().numpy()
            o_ref, _ = oracle.attend(cfg, q_unit(inp, cfg, b, h, 0, 1), pos, kp, v, g)
            assert max_abs(o[b, h * 8:(h + 1) * 8], o_ref) <= ATOL_OUT


def test_tiered_reads_only_window_rows_of_the_device_pool():
    """Rows of the device pool outside the windows are never read: filling
    them with NaN leaves the result unchanged."""
    inp = synth.generate("host64k", batch=1, context=8192)
    st = gh.build_state(inp)
    kc, vc = pinned_copy(st.k_pool), pinned_copy(st.v_pool)
    side = torch.cuda.Stream()
    q = gh.query_slice(st, 0)
    s0, out0, _ = run_tiered(st, kc, vc, q, 1, st.pos0, side)
    pos = int(inp.pos0[0])
    ct = pos // 64
    nan_bits = torch.tensor([0x7FC0], dtype=torch.int32).to(torch.int16).item()
    lo, hi = 64 * 1, 64 * (ct - 4)  # between the sink chunk and the local window
    st.k_pool[:, :, lo:hi] = nan_bits
    gh.v_token_view(st.v_pool)[:, :, lo // 16:hi // 16] = nan_bits
    kw = torch.zeros((1, 4, st.max_sel * 16, 128), dtype=st.k_pool.dtype, device="cuda")
    vw = torch.zeros_like(kw)
    out = torch.full_like(out0, float("nan"))
    hga.hga_attend_tiered(st.cfg, 1, q, 1, st.pos0, st.k_pool, st.v_pool, st.T, kc, vc, st.T,
                          s0.sel, s0.n_sel, st.max_sel, kw, vw, out, None, st.ws, stream_b=side,
                          events=(torch.cuda.Event(), torch.cuda.Event()))
    torch.cuda.synchronize()
    assert torch.equal(out, out0)


@pytest.mark.parametrize("form", ["two streams", "one stream"])
def test_tiered_prefill_chunk(form):
    """A 64-token query chunk through the host tier (MFMA attention for both
    parts) equals the device path."""
    inp = synth.generate("prefill32k", context=4096)
    st = gh.build_state(inp)
    kc, vc = pinned_copy(st.k_pool), pinned_copy(st.v_pool)
    side = torch.cuda.Stream() if form == "two streams" else None
    q = st.q.contiguous()
    s, out, lse = run_tiered(st, kc, vc, q, 64, st.pos0, side)
    assert torch.isfinite(out).all()
    assert (out - s.out).abs().max().item() <= 1e-5
    assert (lse - s.lse).abs().max().item() <= 1e-5


def test_tiered_forms_give_the_same_bits():
    """The one-launch front (window attention beside the copy) and the
    two-stream form write identical outputs; several decode tokens in a row
    through the same buffers."""
    inp = synth.generate("host64k", batch=2, context=8192)
    st = gh.build_state(inp)
    kc, vc = pinned_copy(st.k_pool), pinned_copy(st.v_pool)
    side = torch.cuda.Stream()
    q = gh.query_slice(st, 0)
    for p in (8191, 8190, 8128):
        pos_t = torch.full((st.B,), p, dtype=torch.int32, device="cuda")
        _, out2, lse2 = run_tiered(st, kc, vc, q, 1, pos_t, side)
        _, out1, lse1 = run_tiered(st, kc, vc, q, 1, pos_t, None)
        assert torch.isfinite(out1).all(), p
        assert torch.equal(out1, out2) and torch.equal(lse1, lse2), p


def test_append_into_pinned_host_pool_equals_device_append():
    """hga_build_summaries writes a pinned host pool over PCIe with the same
    bits as a device pool (one-token appends and a bulk range)."""
    inp = synth.generate("host64k", batch=2, context=2048)
    st = gh.build_state(inp)
    kc = torch.zeros(st.k_pool.shape, dtype=st.k_pool.dtype, pin_memory=True)
    vc = torch.zeros(st.v_pool.shape, dtype=st.v_pool.dtype, pin_memory=True)
    hga.hga_build_summaries(st.cfg, st.B, st.k_raw[:, :, :2000].contiguous(),
                            st.v_raw[:, :, :2000].contiguous(), 0, 2000, kc, vc, st.T, None, None,
                            st.max_chunks)
    for p in range(2000, 2048):
        hga.hga_build_summaries(st.cfg, st.B, st.k_raw[:, :, p:p + 1].contiguous(),
                                st.v_raw[:, :, p:p + 1].contiguous(), p, 1, kc, vc, st.T, None,
                                None, st.max_chunks)
    torch.cuda.synchronize()
    assert torch.equal(kc, st.k_pool.cpu()) and torch.equal(vc, st.v_pool.cpu())
