"""GPU checks of the FP8 pool variant (pool_dtype = 1): every (token, KV head)
row of the rotated keys and of the values as OCP E4M3FN codes times a
power-of-two row scale.

The append is compared with the oracle's quantiser (values exact: the same
codes and scales; keys: the same scales and codes except where the two fp64
rotations fall on either side of a rounding tie, which must stay rare and one
code apart).  Decode attention on the FP8 pool is compared with the oracle
run on the GPU's own dequantised pool (tests/oracle_ref.py tolerance), and
the fused decode step with the separate calls (bit-identical)."""
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
                check_selection(cfg, g, osel, margins, oscores, pos, lq)
                kd, vd = pool.deq(b, h)
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
