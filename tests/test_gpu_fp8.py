"""GPU checks of the FP8 pool variant (pool_dtype = 1): every (token, KV head)
row of the rotated keys and of the values as OCP E4M3FN codes times a
power-of-two row scale.

The append is compared with the oracle's quantiser (values exact: the same
codes and scales; keys: the same scales and codes except where the two fp64
rotations fall on either side of a rounding tie, which must stay rare and one
code apart).  Decode, chunked-prefill, whole-prompt and host-tier attention
on the FP8 pool are compared with the oracle run on its own FP8 pool
(tests/oracle_ref.py tolerance); the gather and the warm tier copy codes and
row scales bit for bit; attention over an FP8 working set equals attention
over the pool, and the fused steps equal the separate calls (bit-identical)."""
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

FP8_VALUES = np.array([oracle.fp8_decode(c) for c in range(256)])


class Fp8Pool:
    """Codes then row scales, for K and for V (V in transposed group blocks)."""

    def __init__(self, B, hkv, T, d):
        self.B, self.hkv, self.T, self.d = B, hkv, T, d
        n = B * hkv * T * d + B * hkv * T * 4
        self.k = torch.zeros(n, dtype=torch.uint8, device="cuda")
        self.v = torch.zeros(n, dtype=torch.uint8, device="cuda")

    def split(self, buf):
        B, hkv, T, d = self.B, self.hkv, self.T, self.d
        h = buf.cpu().numpy()
        codes = h[:B * hkv * T * d].reshape(B, hkv, T, d)
        scales = h[B * hkv * T * d:].view(np.float32).reshape(B, hkv, T)
        return codes, scales

    def k_rows(self, b, h):
        codes, scales = self.split(self.k)
        return codes[b, h].astype(np.int64), scales[b, h].astype(np.float64)

    def v_rows(self, b, h):
        """Token rows [T][d] of the transposed V groups."""
        codes, scales = self.split(self.v)
        c = codes[b, h].reshape(self.T // 16, self.d, 16).transpose(0, 2, 1).reshape(self.T, self.d)
        return c.astype(np.int64), scales[b, h].astype(np.float64)

    def deq(self, b, h):
        kc, ks = self.k_rows(b, h)
        vc, vs = self.v_rows(b, h)
        return FP8_VALUES[kc] * ks[:, None], FP8_VALUES[vc] * vs[:, None]


def fp8_state(name="decode64k", batch=2, context=4096, max_lq=None):
    inp = synth.generate(name, batch=batch, context=context, overrides=dict(pool_dtype=1))
    st = gh.build_state(inp, max_lq=max_lq)  # bf16 pool (unused) and the summaries
    pool = Fp8Pool(st.B, 4, st.T, 128)
    hga.hga_build_summaries(st.cfg, st.B, st.k_raw, st.v_raw, 0, st.T, pool.k, pool.v, st.T, None,
                            None, st.max_chunks)
    torch.cuda.synchronize()
    return inp, st, pool


def test_fp8_append_matches_oracle_quantiser():
    inp, st, pool = fp8_state(batch=2, context=2048)
    cfg = oracle.cfg_from(inp.params)
    for b in range(st.B):
        for h in range(4):
            kraw = inp.f64(inp.k[b, h])
            ocodes, oscales, _ = oracle.pool_fp8(cfg, kraw, 0)
            kc, ks = pool.k_rows(b, h)
            np.testing.assert_array_equal(ks, oscales)
            diff = kc != ocodes
            assert diff.sum() <= max(1, int(1e-4 * diff.size)), int(diff.sum())
            if diff.any():  # one code apart: neighbouring values of the same sign
                assert np.all(np.abs((kc[diff] & 0x7F) - (ocodes[diff] & 0x7F)) == 1)
            vcodes, vscales, _ = oracle.fp8_rows(inp.f64(inp.v[b, h]))
            vc, vs = pool.v_rows(b, h)
            np.testing.assert_array_equal(vs, vscales)
            np.testing.assert_array_equal(vc, vcodes)


@pytest.mark.parametrize("lq", [1, 5])
def test_fp8_decode_attention_against_oracle(lq):
    inp, st, pool = fp8_state(batch=2, context=4096, max_lq=lq)
    cfg = oracle.cfg_from(inp.params)
    uc = UnitCache(inp, cfg)
    q = gh.query_slice(st, 0) if lq == 1 else st.q[:, :, :1].repeat(1, 1, lq, 1).contiguous()
    deq = {}
    for pos in (4095 - lq + 1, 3000, 1280):
        pos_t = torch.full((st.B,), pos, dtype=torch.int32, device="cuda")
        s = gh.alloc_step(st, lq)
        gh.route(st, q, lq, pos_t, s)
        hga.hga_attend(st.cfg, st.B, q, lq, pos_t, pool.k, pool.v, hga.HGA_SRC_POOL, st.T, s.sel,
                       s.n_sel, st.max_sel, hga.HGA_PART_ALL, s.out, s.lse, st.ws)
        torch.cuda.synchronize()
        sel, nsel, out = s.sel.cpu().numpy(), s.n_sel.cpu().numpy(), s.out.cpu().numpy()
        qh = q.cpu().numpy().view(np.uint16)  # bf16 bit patterns
        for b in range(st.B):
            for h in range(4):
                cs, gs, _, _ = uc.get(b, h, need_pool=False)
                qu = inp.f64(qh[b, h * 8:(h + 1) * 8])
                g = sel[b, h, :nsel[b, h]]
                osel, margins, oscores = oracle.select(cfg, qu, pos, cs, gs)
                check_selection(cfg, g, osel, margins, oscores, pos, lq,
                                oracle.group_scores(cfg, qu, pos, gs))
                if (b, h) not in deq:  # the oracle's own FP8 pool
                    deq[b, h] = (oracle.pool_fp8(cfg, inp.f64(inp.k[b, h]), 0)[2],
                                 oracle.fp8_rows(inp.f64(inp.v[b, h]))[2])
                kd, vd = deq[b, h]
                o_ref, _ = oracle.attend(cfg, qu, pos, kd, vd, g)
                assert max_abs(out[b, h * 8:(h + 1) * 8], o_ref) <= ATOL_OUT, (pos, b, h)


def test_fp8_decode_step_equals_separate_calls():
    inp, st, _ = fp8_state(batch=2, context=4096)
    B, T = st.B, st.T
    p_start = 4026
    q = gh.query_slice(st, 0)

    def fresh():
        pool = Fp8Pool(B, 4, T, 128)
        cs, gs = torch.zeros_like(st.chunk_sum), torch.zeros_like(st.group_sum)
        hga.hga_build_summaries(st.cfg, B, st.k_raw[:, :, :p_start].contiguous(),
                                st.v_raw[:, :, :p_start].contiguous(), 0, p_start, pool.k, pool.v, T,
                                cs, gs, st.max_chunks)
        return pool, cs, gs

    pa, csa, gsa = fresh()
    pb, csb, gsb = fresh()
    c0 = p_start // 64 * 64
    stage = torch.zeros_like(st.k_raw[:, :, :64])
    stage[:, :, :p_start - c0] = st.k_raw[:, :, c0:p_start]
    for p in range(p_start, p_start + 12):  # crosses the end of chunk 62
        pos_t = torch.full((B,), p, dtype=torch.int32, device="cuda")
        kt = st.k_raw[:, :, p:p + 1].contiguous()
        vt = st.v_raw[:, :, p:p + 1].contiguous()
        sa = gh.alloc_step(st, 1)
        hga.hga_build_summaries(st.cfg, B, kt, vt, p, 1, pa.k, pa.v, T, None, None, st.max_chunks)
        if p % 64 == 63:
            hga.hga_build_summaries(st.cfg, B, st.k_raw[:, :, p - 63:p + 1].contiguous(), None,
                                    p - 63, 64, None, None, T, csa, gsa, st.max_chunks)
        hga.hga_route(st.cfg, B, q, 1, pos_t, csa, gsa, st.max_chunks, sa.sel, sa.n_sel,
                      st.max_sel, None, st.ws)
        hga.hga_attend(st.cfg, B, q, 1, pos_t, pa.k, pa.v, hga.HGA_SRC_POOL, T, sa.sel, sa.n_sel,
                       st.max_sel, hga.HGA_PART_ALL, sa.out, sa.lse, st.ws)
        sb = gh.alloc_step(st, 1)
        hga.hga_decode_step(st.cfg, B, q, kt, vt, pos_t, pb.k, pb.v, T, stage, csb, gsb,
                            st.max_chunks, sb.sel, sb.n_sel, st.max_sel, sb.out, sb.lse,
                            torch.zeros_like(st.ws))
        torch.cuda.synchronize()
        assert torch.equal(sa.n_sel, sb.n_sel) and torch.equal(sa.out, sb.out), p
    assert torch.equal(pa.k, pb.k) and torch.equal(pa.v, pb.v)
    assert torch.equal(csa, csb) and torch.equal(gsa, gsb)


@pytest.mark.parametrize("pos,lq", [(20 * 64 + 59, 5), (30 * 64 + 3, 15), (2047, 1)])
def test_fp8_prefill_step_equals_separate_calls(pos, lq):
    """hga_prefill_step with 1..15 query tokens on the FP8 pool appends every
    one of its tokens (the same codes and scales as hga_build_summaries over
    those tokens) and gives the bits of the separate calls."""
    inp, st, _ = fp8_state(batch=2, context=4096, max_lq=lq)
    B, T = st.B, st.T
    q = st.q[:, :, :1].repeat(1, 1, lq, 1).contiguous()  # the workload holds one query token
    pos_t = torch.full((B,), pos, dtype=torch.int32, device="cuda")
    kn = st.k_raw[:, :, pos:pos + lq].contiguous()
    vn = st.v_raw[:, :, pos:pos + lq].contiguous()
    c0 = pos // 64 * 64
    ends = pos + lq == c0 + 64
    print(f"[fp8 prefill step] pos {pos} lq {lq}", flush=True)

    def fresh():
        pool = Fp8Pool(B, 4, T, 128)
        cs, gs = torch.zeros_like(st.chunk_sum), torch.zeros_like(st.group_sum)
        hga.hga_build_summaries(st.cfg, B, st.k_raw[:, :, :pos].contiguous(),
                                st.v_raw[:, :, :pos].contiguous(), 0, pos, pool.k, pool.v, T, cs,
                                gs, st.max_chunks)
        return pool, cs, gs

    pa, csa, gsa = fresh()
    sa = gh.alloc_step(st, lq)
    hga.hga_build_summaries(st.cfg, B, kn, vn, pos, lq, pa.k, pa.v, T, None, None, st.max_chunks)
    if ends:
        hga.hga_build_summaries(st.cfg, B, st.k_raw[:, :, c0:c0 + 64].contiguous(), None, c0, 64,
                                None, None, T, csa, gsa, st.max_chunks)
    hga.hga_route(st.cfg, B, q, lq, pos_t, csa, gsa, st.max_chunks, sa.sel, sa.n_sel, st.max_sel,
                  None, st.ws)
    hga.hga_attend(st.cfg, B, q, lq, pos_t, pa.k, pa.v, hga.HGA_SRC_POOL, T, sa.sel, sa.n_sel,
                   st.max_sel, hga.HGA_PART_ALL, sa.out, sa.lse, st.ws)
    pb, csb, gsb = fresh()
    stage = torch.zeros_like(st.k_raw[:, :, :64])
    stage[:, :, :pos - c0] = st.k_raw[:, :, c0:pos]
    sb = gh.alloc_step(st, lq)
    hga.hga_prefill_step(st.cfg, B, q, lq, kn, vn, pos_t, pb.k, pb.v, T, stage, csb, gsb,
                         st.max_chunks, sb.sel, sb.n_sel, st.max_sel, sb.out, sb.lse,
                         torch.zeros_like(st.ws))
    torch.cuda.synchronize()
    assert (sb.n_sel > 0).all()
    assert torch.equal(sa.n_sel, sb.n_sel) and torch.equal(sa.sel, sb.sel)
    assert torch.equal(sa.out, sb.out) and torch.equal(sa.lse, sb.lse)
    assert torch.equal(pa.k, pb.k) and torch.equal(pa.v, pb.v)
    assert torch.equal(csa, csb) and torch.equal(gsa, gsb)
    # every appended row holds the oracle quantiser's scale
    cfg = oracle.cfg_from(inp.params)
    for b in range(B):
        for h in range(4):
            _, oscales, _ = oracle.pool_fp8(cfg, inp.f64(inp.k[b, h, pos:pos + lq]), pos)
            _, ks = pb.k_rows(b, h)
            np.testing.assert_array_equal(ks[pos:pos + lq], oscales)
            _, vscales, _ = oracle.fp8_rows(inp.f64(inp.v[b, h, pos:pos + lq]))
            _, vs = pb.v_rows(b, h)
            np.testing.assert_array_equal(vs[pos:pos + lq], vscales)


def fp8_ws(B, lists, max_sel, d=128):
    """An FP8 working set: codes [B][lists][max_sel*16][d], then row scales."""
    n = B * lists * max_sel * 16 * (d + 4)
    return (torch.zeros(n, dtype=torch.uint8, device="cuda"),
            torch.zeros(n, dtype=torch.uint8, device="cuda"))


def split_ws(buf, B, lists, max_sel, d=128):
    h = buf.cpu().numpy()
    nc = B * lists * max_sel * 16 * d
    return (h[:nc].reshape(B, lists, max_sel, 16 * d),
            h[nc:].view(np.float32).reshape(B, lists, max_sel, 16))


def pool_groups(buf, B, hkv, T, d=128):
    h = buf.cpu().numpy()
    nc = B * hkv * T * d
    return (h[:nc].reshape(B, hkv, T // 16, 16 * d),
            h[nc:].view(np.float32).reshape(B, hkv, T // 16, 16))


def pinned(t):
    h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    h.copy_(t)
    return h


@pytest.mark.parametrize("host", [False, True])
def test_fp8_gather_copies_codes_and_scales(host):
    """hga_gather from the FP8 pool (device memory, or pinned host memory over
    PCIe) copies each listed group's 16 code rows and 16 row scales of K and
    V into its working-set slot, bit for bit; HGA_PART_ROUTED copies the routed
    slots only."""
    inp, st, pool = fp8_state(batch=2, context=4096)
    B, T, ms = st.B, st.T, st.max_sel
    q = gh.query_slice(st, 0)
    s = gh.alloc_step(st, 1)
    gh.route(st, q, 1, st.pos0, s)
    kp, vp = (pinned(pool.k), pinned(pool.v)) if host else (pool.k, pool.v)
    kw, vw = fp8_ws(B, 4, ms)
    hga.hga_gather(st.cfg, B, kp, vp, T, int(host), s.sel, s.n_sel, ms, st.pos0,
                   hga.HGA_PART_ALL, kw, vw)
    kr, vr = fp8_ws(B, 4, ms)
    hga.hga_gather(st.cfg, B, kp, vp, T, int(host), s.sel, s.n_sel, ms, st.pos0,
                   hga.HGA_PART_ROUTED, kr, vr)
    torch.cuda.synchronize()
    sel, nsel = s.sel.cpu().numpy(), s.n_sel.cpu().numpy()
    for buf, wbuf, rbuf in ((pool.k, kw, kr), (pool.v, vw, vr)):
        pc, psc = pool_groups(buf, B, 4, T)
        wc, wsc = split_ws(wbuf, B, 4, ms)
        rc, rsc = split_ws(rbuf, B, 4, ms)
        for b in range(B):
            for h in range(4):
                n = nsel[b, h]
                g = sel[b, h, :n]
                np.testing.assert_array_equal(wc[b, h, :n], pc[b, h, g])
                np.testing.assert_array_equal(wsc[b, h, :n], psc[b, h, g])
                routed = slice(4, n - 4 * 4 - 4)  # sink | routed | local | current (pos 4095)
                np.testing.assert_array_equal(rc[b, h, routed], pc[b, h, g[routed]])
                np.testing.assert_array_equal(rsc[b, h, routed], psc[b, h, g[routed]])
                assert not rc[b, h, :4].any() and not rc[b, h, n - 20:n].any()


def test_fp8_attend_working_set_equals_pool():
    """Decode attention over an FP8 working set gives the bits of the same
    attention over the FP8 pool."""
    inp, st, pool = fp8_state(batch=2, context=4096, max_lq=5)
    B, T, ms = st.B, st.T, st.max_sel
    for lq in (1, 5):
        q = gh.query_slice(st, 0) if lq == 1 else st.q[:, :, :1].repeat(1, 1, lq, 1).contiguous()
        pos_t = torch.full((B,), 3000, dtype=torch.int32, device="cuda")
        s = gh.alloc_step(st, lq)
        gh.route(st, q, lq, pos_t, s)
        hga.hga_attend(st.cfg, B, q, lq, pos_t, pool.k, pool.v, hga.HGA_SRC_POOL, T, s.sel,
                       s.n_sel, ms, hga.HGA_PART_ALL, s.out, s.lse, st.ws)
        kw, vw = fp8_ws(B, 4, ms)
        hga.hga_gather(st.cfg, B, pool.k, pool.v, T, 0, s.sel, s.n_sel, ms, pos_t,
                       hga.HGA_PART_ALL, kw, vw)
        ow, lw = torch.empty_like(s.out), torch.empty_like(s.lse)
        hga.hga_attend(st.cfg, B, q, lq, pos_t, kw, vw, hga.HGA_SRC_WORKING_SET, 0, s.sel,
                       s.n_sel, ms, hga.HGA_PART_ALL, ow, lw, st.ws)
        torch.cuda.synchronize()
        assert torch.equal(ow, s.out) and torch.equal(lw, s.lse), lq


@pytest.mark.parametrize("form", ["two streams", "one launch"])
def test_fp8_tiered_against_device_path_and_oracle(form):
    """The host tier on the FP8 pool: windows from the device pool, routed
    groups copied from the pinned host pool (codes and scales) and attended
    from the working set, merged exactly.  Equal to hga_attend over the whole
    list within the merge's rounding, and to the oracle run on its own FP8
    pool within the decode tolerance."""
    inp, st, pool = fp8_state(batch=2, context=8192)
    B, T, ms = st.B, st.T, st.max_sel
    cfg = oracle.cfg_from(inp.params)
    kc, vc = pinned(pool.k), pinned(pool.v)
    q = gh.query_slice(st, 0)
    s = gh.alloc_step(st, 1)
    gh.route(st, q, 1, st.pos0, s)
    hga.hga_attend(st.cfg, B, q, 1, st.pos0, pool.k, pool.v, hga.HGA_SRC_POOL, T, s.sel, s.n_sel,
                   ms, hga.HGA_PART_ALL, s.out, s.lse, st.ws)
    kw, vw = fp8_ws(B, 4, ms)
    out = torch.full_like(s.out, float("nan"))
    lse = torch.full_like(s.lse, float("nan"))
    side = torch.cuda.Stream() if form == "two streams" else None
    hga.hga_attend_tiered(st.cfg, B, q, 1, st.pos0, pool.k, pool.v, T, kc, vc, T, s.sel, s.n_sel,
                          ms, kw, vw, out, lse, torch.zeros_like(st.ws), stream_b=side,
                          events=(torch.cuda.Event(), torch.cuda.Event()))
    torch.cuda.synchronize()
    assert (out - s.out).abs().max().item() <= 1e-5
    assert (lse - s.lse).abs().max().item() <= 1e-5
    pos = int(inp.pos0[0])
    o = out.cpu().numpy()
    qh = q.cpu().numpy().view(np.uint16)
    for b in range(B):
        for h in range(4):
            kd = oracle.pool_fp8(cfg, inp.f64(inp.k[b, h]), 0)[2]
            vd = oracle.fp8_rows(inp.f64(inp.v[b, h]))[2]
            g = s.sel[b, h, :int(s.n_sel[b, h])].cpu().numpy()
            o_ref, _ = oracle.attend(cfg, inp.f64(qh[b, h * 8:(h + 1) * 8]), pos, kd, vd, g)
            assert max_abs(o[b, h * 8:(h + 1) * 8], o_ref) <= ATOL_OUT, (b, h)


def test_fp8_warm_tier_equals_gather():
    """The warm tier on the FP8 pool: over drifting decode steps the working
    set's routed slots (codes and row scales) equal what hga_gather copies
    from the pinned host pool, and the attention through the cache equals the
    device path within the merge's rounding."""
    inp, st, pool = fp8_state(batch=2, context=8192)
    B, T, ms, n_warm = st.B, st.T, st.max_sel, 208
    kc, vc = pinned(pool.k), pinned(pool.v)
    units = B * 4
    k_warm = torch.zeros(units * n_warm * 16 * (128 + 4), dtype=torch.uint8, device="cuda")
    v_warm = torch.zeros_like(k_warm)
    tags = torch.full((B, 4, n_warm), -1, dtype=torch.int32, device="cuda")
    used = torch.zeros((B, 4, n_warm), dtype=torch.int32, device="cuda")
    hits = torch.zeros((B, 4), dtype=torch.int32, device="cuda")
    wsw = torch.zeros(hga.hga_warm_workspace_bytes(st.cfg, B, ms), dtype=torch.uint8,
                      device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(11)
    qf = gh.query_slice(st, 0).view(torch.bfloat16).float()
    total_hits = 0
    for step in range(1, 7):
        q = qf.to(torch.bfloat16).view(torch.int16).contiguous()
        s = gh.alloc_step(st, 1)
        gh.route(st, q, 1, st.pos0, s)
        kw, vw = fp8_ws(B, 4, ms)
        hga.hga_warm_gather(st.cfg, B, kc, vc, T, s.sel, s.n_sel, ms, st.pos0, k_warm, v_warm,
                            tags, used, n_warm, step, kw, vw, hits, wsw)
        kr, vr = fp8_ws(B, 4, ms)
        hga.hga_gather(st.cfg, B, kc, vc, T, 1, s.sel, s.n_sel, ms, st.pos0,
                       hga.HGA_PART_ROUTED, kr, vr)
        oa, la = torch.empty_like(s.out), torch.empty_like(s.lse)
        ob, lb = torch.empty_like(s.out), torch.empty_like(s.lse)
        hga.hga_attend(st.cfg, B, q, 1, st.pos0, pool.k, pool.v, hga.HGA_SRC_POOL, T, s.sel,
                       s.n_sel, ms, hga.HGA_PART_WINDOWS, oa, la, st.ws)
        hga.hga_attend(st.cfg, B, q, 1, st.pos0, kw, vw, hga.HGA_SRC_WORKING_SET, 0, s.sel,
                       s.n_sel, ms, hga.HGA_PART_ROUTED, ob, lb, torch.zeros_like(st.ws))
        out, lse = torch.empty_like(s.out), torch.empty_like(s.lse)
        hga.hga_merge_partials(st.cfg, B, 1, oa, la, ob, lb, out, lse)
        hga.hga_attend(st.cfg, B, q, 1, st.pos0, pool.k, pool.v, hga.HGA_SRC_POOL, T, s.sel,
                       s.n_sel, ms, hga.HGA_PART_ALL, s.out, s.lse, st.ws)
        torch.cuda.synchronize()
        assert torch.equal(kw, kr) and torch.equal(vw, vr), step
        assert (out - s.out).abs().max().item() <= 1e-5, step
        total_hits += int(hits.sum().item())
        qf = (qf + 0.25 * torch.randn(qf.shape, generator=gen, device="cuda")) / (1 + 0.0625) ** 0.5
    assert total_hits > 0  # the drifting queries reuse cached groups


def fp8_oracle_pool(inp, cfg, b, h):
    """The oracle's own FP8 pool of unit (b, h), dequantised: keys, values."""
    return (oracle.pool_fp8(cfg, inp.f64(inp.k[b, h]), 0)[2],
            oracle.fp8_rows(inp.f64(inp.v[b, h]))[2])


def test_fp8_prefill_chunk_against_oracle_and_working_set():
    """A 64-token query chunk (the MFMA prefill kernel) on the FP8 pool
    against the oracle run on its own FP8 pool; the same attention over an
    FP8 working set gives the same bits."""
    inp = synth.generate("prefill32k", context=4096, overrides=dict(pool_dtype=1))
    st = gh.build_state(inp)
    B, T, ms = st.B, st.T, st.max_sel
    pool = Fp8Pool(B, 4, T, 128)
    hga.hga_build_summaries(st.cfg, B, st.k_raw, st.v_raw, 0, T, pool.k, pool.v, T, None, None,
                            st.max_chunks)
    cfg = oracle.cfg_from(inp.params)
    pos = int(inp.pos0[0])
    q = st.q.contiguous()
    lq = q.shape[2]
    s = gh.alloc_step(st, lq)
    gh.route(st, q, lq, st.pos0, s)
    hga.hga_attend(st.cfg, B, q, lq, st.pos0, pool.k, pool.v, hga.HGA_SRC_POOL, T, s.sel, s.n_sel,
                   ms, hga.HGA_PART_ALL, s.out, s.lse, st.ws)
    kw, vw = fp8_ws(B, 4, ms)
    hga.hga_gather(st.cfg, B, pool.k, pool.v, T, 0, s.sel, s.n_sel, ms, st.pos0, hga.HGA_PART_ALL,
                   kw, vw)
    ow, lw = torch.empty_like(s.out), torch.empty_like(s.lse)
    hga.hga_attend(st.cfg, B, q, lq, st.pos0, kw, vw, hga.HGA_SRC_WORKING_SET, 0, s.sel, s.n_sel,
                   ms, hga.HGA_PART_ALL, ow, lw, st.ws)
    torch.cuda.synchronize()
    assert torch.equal(ow, s.out) and torch.equal(lw, s.lse)
    out, lse = s.out.cpu().numpy(), s.lse.cpu().numpy()
    for b in range(B):
        for h in range(4):
            kd, vd = fp8_oracle_pool(inp, cfg, b, h)
            g = s.sel[b, h, :int(s.n_sel[b, h])].cpu().numpy()
            o_ref, l_ref = oracle.attend(cfg, q_unit(inp, cfg, b, h, 0, lq), pos, kd, vd, g)
            assert max_abs(out[b, h * 8:(h + 1) * 8], o_ref) <= ATOL_OUT, (b, h)
            assert max_abs(lse[b, h * 8:(h + 1) * 8], l_ref) <= 1e-3, (b, h)


def test_fp8_prefill_step_64_tokens_equals_separate_calls():
    """hga_prefill_step with a whole 64-token chunk on the FP8 pool: the
    chunk's tokens appended, its summaries built, routed and attended by the
    MFMA kernel; the bits of the separate calls."""
    inp, st, _ = fp8_state(batch=2, context=4096, max_lq=64)
    B, T, lq, pos = st.B, st.T, 64, 20 * 64
    q = st.q[:, :, :1].repeat(1, 1, lq, 1).contiguous()
    pos_t = torch.full((B,), pos, dtype=torch.int32, device="cuda")
    kn = st.k_raw[:, :, pos:pos + lq].contiguous()
    vn = st.v_raw[:, :, pos:pos + lq].contiguous()

    def fresh():
        pool = Fp8Pool(B, 4, T, 128)
        cs, gs = torch.zeros_like(st.chunk_sum), torch.zeros_like(st.group_sum)
        hga.hga_build_summaries(st.cfg, B, st.k_raw[:, :, :pos].contiguous(),
                                st.v_raw[:, :, :pos].contiguous(), 0, pos, pool.k, pool.v, T, cs,
                                gs, st.max_chunks)
        return pool, cs, gs

    pa, csa, gsa = fresh()
    sa = gh.alloc_step(st, lq)
    hga.hga_build_summaries(st.cfg, B, kn, vn, pos, lq, pa.k, pa.v, T, csa, gsa, st.max_chunks)
    hga.hga_route(st.cfg, B, q, lq, pos_t, csa, gsa, st.max_chunks, sa.sel, sa.n_sel, st.max_sel,
                  None, st.ws)
    hga.hga_attend(st.cfg, B, q, lq, pos_t, pa.k, pa.v, hga.HGA_SRC_POOL, T, sa.sel, sa.n_sel,
                   st.max_sel, hga.HGA_PART_ALL, sa.out, sa.lse, st.ws)
    pb, csb, gsb = fresh()
    sb = gh.alloc_step(st, lq)
    hga.hga_prefill_step(st.cfg, B, q, lq, kn, vn, pos_t, pb.k, pb.v, T,
                         torch.zeros_like(st.k_raw[:, :, :64]), csb, gsb, st.max_chunks, sb.sel,
                         sb.n_sel, st.max_sel, sb.out, sb.lse, torch.zeros_like(st.ws))
    torch.cuda.synchronize()
    assert torch.equal(sa.n_sel, sb.n_sel) and torch.equal(sa.sel, sb.sel)
    assert torch.equal(sa.out, sb.out) and torch.equal(sa.lse, sb.lse)
    assert torch.equal(pa.k, pb.k) and torch.equal(pa.v, pb.v)
    assert torch.equal(csa, csb) and torch.equal(gsa, gsb)


def test_fp8_tiered_prefill_chunk_equals_device_path():
    """A 64-token query chunk through the host tier on the FP8 pool (both
    parts on the MFMA prefill kernel) equals the device path within the
    merge's rounding."""
    inp = synth.generate("prefill32k", context=4096, overrides=dict(pool_dtype=1))
    st = gh.build_state(inp)
    B, T, ms = st.B, st.T, st.max_sel
    pool = Fp8Pool(B, 4, T, 128)
    hga.hga_build_summaries(st.cfg, B, st.k_raw, st.v_raw, 0, T, pool.k, pool.v, T, None, None,
                            st.max_chunks)
    kc, vc = pinned(pool.k), pinned(pool.v)
    q = st.q.contiguous()
    lq = q.shape[2]
    s = gh.alloc_step(st, lq)
    gh.route(st, q, lq, st.pos0, s)
    hga.hga_attend(st.cfg, B, q, lq, st.pos0, pool.k, pool.v, hga.HGA_SRC_POOL, T, s.sel, s.n_sel,
                   ms, hga.HGA_PART_ALL, s.out, s.lse, st.ws)
    for side in (torch.cuda.Stream(), None):
        kw, vw = fp8_ws(B, 4, ms)
        out = torch.full_like(s.out, float("nan"))
        lse = torch.full_like(s.lse, float("nan"))
        hga.hga_attend_tiered(st.cfg, B, q, lq, st.pos0, pool.k, pool.v, T, kc, vc, T, s.sel,
                              s.n_sel, ms, kw, vw, out, lse, torch.zeros_like(st.ws),
                              stream_b=side, events=(torch.cuda.Event(), torch.cuda.Event()))
        torch.cuda.synchronize()
        assert (out - s.out).abs().max().item() <= 1e-5
        assert (lse - s.lse).abs().max().item() <= 1e-5


def test_fp8_prompt_against_oracle():
    """The whole-prompt prefill on the FP8 pool (2K prompt): the append phase
    writes the FP8 pool hga_build_summaries writes, and sampled query chunks
    (windows only up to routed) match the oracle run on its own FP8 pool."""
    inp = synth.generate("prompt32k", context=2048, overrides=dict(pool_dtype=1))
    st = gh.build_state(inp, max_lq=64)
    B, T, ms = st.B, st.T, st.max_sel
    nq = T // 64
    ref = Fp8Pool(B, 4, T, 128)
    hga.hga_build_summaries(st.cfg, B, st.k_raw, st.v_raw, 0, T, ref.k, ref.v, T, None, None,
                            st.max_chunks)
    pool = Fp8Pool(B, 4, T, 128)
    cs, gs = torch.zeros_like(st.chunk_sum), torch.zeros_like(st.group_sum)
    sel = torch.full((B, nq, 4, ms), -7, dtype=torch.int32, device="cuda")
    n_sel = torch.full((B, nq, 4), -7, dtype=torch.int32, device="cuda")
    out = torch.full((B, 32, T, 128), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, 32, T), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.zeros(hga.hga_prompt_workspace_bytes(st.cfg, B, T, st.max_chunks),
                     dtype=torch.uint8, device="cuda")
    hga.hga_prefill_prompt(st.cfg, B, T, st.q, st.k_raw, st.v_raw, pool.k, pool.v, T, cs, gs,
                           st.max_chunks, sel, n_sel, ms, out, lse, ws)
    torch.cuda.synchronize()
    assert torch.equal(pool.k, ref.k) and torch.equal(pool.v, ref.v)
    assert torch.equal(cs, st.chunk_sum) and torch.equal(gs, st.group_sum)
    assert torch.isfinite(out).all()
    cfg = oracle.cfg_from(inp.params)
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    sl, ns = sel.cpu().numpy(), n_sel.cpu().numpy()
    for b in range(B):
        for h in range(4):
            kd, vd = fp8_oracle_pool(inp, cfg, b, h)
            for qc in (0, 3, 11, 31):
                p0 = qc * 64
                g = sl[b, qc, h, :ns[b, qc, h]]
                o_ref, l_ref = oracle.attend(cfg, q_unit(inp, cfg, b, h, p0, 64), p0, kd, vd, g)
                assert max_abs(o[b, h * 8:(h + 1) * 8, p0:p0 + 64], o_ref) <= ATOL_OUT, (b, h, qc)
                assert max_abs(l[b, h * 8:(h + 1) * 8, p0:p0 + 64], l_ref) <= 1e-3, (b, h, qc)
