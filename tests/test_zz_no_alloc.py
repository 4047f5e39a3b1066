"""hga_decode_step_noalloc (scratch in the library's static per-GPU array, no
workspace argument) against hga_decode_step with a caller workspace: two
calls in a row, the second on a smaller input, each bit-identical to the
workspace form in lists, outputs, LSE, pools and summaries."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import long_context_hga_amd as hga  # noqa: E402
import gpu_harness as gh  # noqa: E402


def one_call(batch, context):
    inp = synth.generate("decode64k", batch=batch, context=context)
    st = gh.build_state(inp)
    B, T = st.B, st.T
    pos = T - 1
    c0 = pos // 64 * 64
    q = gh.query_slice(st, 0)
    kt = st.k_raw[:, :, pos].contiguous()
    vt = st.v_raw[:, :, pos].contiguous()
    state = [dict(kp=st.k_pool.clone(), vp=st.v_pool.clone(), cs=st.chunk_sum.clone(),
                  gs=st.group_sum.clone(), stage=st.k_raw[:, :, c0:c0 + 64].contiguous(),
                  s=gh.alloc_step(st, 1)) for _ in range(2)]
    a, b = state
    print(f"[noalloc] batch {B} context {T}: workspace form", flush=True)
    hga.hga_decode_step(st.cfg, B, q, kt, vt, st.pos0, a["kp"], a["vp"], T, a["stage"], a["cs"],
                        a["gs"], st.max_chunks, a["s"].sel, a["s"].n_sel, st.max_sel, a["s"].out,
                        a["s"].lse, st.ws)
    print(f"[noalloc] batch {B} context {T}: static scratch", flush=True)
    hga.hga_decode_step_noalloc(st.cfg, B, q, kt, vt, st.pos0, b["kp"], b["vp"], T, b["stage"],
                                b["cs"], b["gs"], st.max_chunks, b["s"].sel, b["s"].n_sel,
                                st.max_sel, b["s"].out, b["s"].lse)
    torch.cuda.synchronize()
    sa, sb = a["s"], b["s"]
    assert (sb.n_sel == st.max_sel).all()
    assert torch.isfinite(sb.out).all()
    assert torch.equal(sa.n_sel, sb.n_sel) and torch.equal(sa.sel, sb.sel)
    assert torch.equal(sa.out, sb.out) and torch.equal(sa.lse, sb.lse)
    for key in ("kp", "vp", "cs", "gs", "stage"):
        assert torch.equal(a[key], b[key]), key


def test_noalloc_equals_workspace_form_twice():
    one_call(8, 16384)
    one_call(2, 4096)  # smaller: the scratch still holds the first call's data


def test_noalloc_rejects_batch_beyond_scratch():
    inp = synth.generate("decode64k", batch=1, context=4096)
    st = gh.build_state(inp)
    big = hga.hga_workspace_bytes(st.cfg, 512, st.T, 1)
    assert big > hga.HGA_NOALLOC_SCRATCH_BYTES
    s = gh.alloc_step(st, 1)
    with pytest.raises(hga.HgaError) as e:
        hga.hga_decode_step_noalloc(st.cfg, 512, st.q, st.k_raw, st.v_raw, st.pos0, st.k_pool,
                                    st.v_pool, st.T, st.k_raw, st.chunk_sum, st.group_sum,
                                    st.max_chunks, s.sel, s.n_sel, st.max_sel, s.out, s.lse)
    assert e.value.status == hga.HGA_ERR_WORKSPACE_TOO_SMALL
