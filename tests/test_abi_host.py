"""Host-only checks of the C ABI: the library loads, exports every symbol
include/hga.h declares, and validation rejects bad arguments before any
launch (so none of these calls needs a GPU)."""
import ctypes
import os
import re

import pytest

import long_context_hga_amd as hga
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "hga.h")).read()
    return sorted(set(re.findall(r"^\s*(?:hga_status|const char\*|int32_t)\s+(hga_\w+)\(", src,
                                 re.M)))


def test_exports_every_declared_symbol():
    L = hga.lib()
    names = declared_symbols()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(hga.EXPORTED)


def test_version_and_status_strings():
    assert hga.hga_version() == 1
    for s in range(6):
        assert hga.hga_status_string(s)


def cfg(**over):
    return hga.config_from(synth.CONFIGS["decode64k"], **over)


def test_validate():
    assert hga.hga_validate(cfg()) == hga.HGA_OK
    assert hga.hga_validate(hga.config_from(synth.CONFIGS["tiny"])) == hga.HGA_OK
    bad = [dict(head_dim=127), dict(n_q_heads=30), dict(groups_per_chunk=3), dict(rope_theta=1.0),
           dict(topk_chunks=-1), dict(hf_wavelength=float("nan")), dict(qkv_dtype=7),
           dict(rep_position=2), dict(route_per_head=-1), dict(rope_style=3),
           dict(pool_dtype=2), dict(route_pool=2)]
    for b in bad:
        assert hga.hga_validate(cfg(**b)) == hga.HGA_ERR_INVALID_ARGUMENT, b
    unsup = [dict(head_dim=96), dict(chunk_size=128), dict(groups_per_chunk=8),
             dict(n_q_heads=64, n_kv_heads=4)]
    for u in unsup:
        assert hga.hga_validate(cfg(**u)) == hga.HGA_ERR_UNSUPPORTED, u
    assert hga.lib().hga_validate(None) == hga.HGA_ERR_INVALID_ARGUMENT


def test_sizes():
    c = cfg()
    assert hga.hga_max_selected(c, 1) == (1 + 4 + 1) * 4 + 104
    n = hga.hga_workspace_bytes(c, 8, 65536, 1)
    assert n >= (1 << 20) + 8 * 4 * 1023 * 8
    with pytest.raises(hga.HgaError):
        hga.hga_workspace_bytes(c, 0, 65536, 1)


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def test_build_summaries_rejects():
    c = ctypes.byref(cfg())
    L = hga.lib()
    f = L.hga_build_summaries
    ok = (c, 1, FAKE, FAKE, 0, 64, FAKE, FAKE, 64, FAKE, FAKE, 1, None)
    assert f(*ok[:2], None, *ok[3:]) == hga.HGA_ERR_INVALID_ARGUMENT
    assert f(c, 1, FAKE, FAKE, 0, 65, FAKE, FAKE, 64, FAKE, FAKE, 1, None) == hga.HGA_ERR_OUT_OF_RANGE
    assert f(c, 1, FAKE, FAKE, 0, 128, FAKE, FAKE, 128, FAKE, FAKE, 1, None) == hga.HGA_ERR_OUT_OF_RANGE
    assert f(c, 1, FAKE, FAKE, 0, 64, FAKE, None, 64, FAKE, FAKE, 1, None) == hga.HGA_ERR_INVALID_ARGUMENT
    assert f(c, 1, FAKE, FAKE, -1, 64, FAKE, FAKE, 64, FAKE, FAKE, 1, None) == hga.HGA_ERR_INVALID_ARGUMENT
    assert f(c, 1, FAKE, FAKE, 0, 64, None, None, 0, None, None, 0, None) == hga.HGA_OK  # no-op


def test_route_rejects():
    c = ctypes.byref(cfg())
    f = hga.lib().hga_route
    args = [c, 8, FAKE, 1, FAKE, FAKE, FAKE, 1024, FAKE, FAKE, 128, None, FAKE, 1 << 30, None]
    a = list(args); a[10] = 127
    assert f(*a) == hga.HGA_ERR_OUT_OF_RANGE
    a = list(args); a[13] = 1000
    assert f(*a) == hga.HGA_ERR_WORKSPACE_TOO_SMALL
    a = list(args); a[2] = None
    assert f(*a) == hga.HGA_ERR_INVALID_ARGUMENT
    a = list(args); a[3] = 65
    assert f(*a) == hga.HGA_ERR_INVALID_ARGUMENT
    a = list(args); a[7] = 100000
    assert f(*a) == hga.HGA_ERR_UNSUPPORTED  # candidate table beyond the LDS budget


def test_attend_rejects():
    c = ctypes.byref(cfg())
    f = hga.lib().hga_attend
    args = [c, 8, FAKE, 1, FAKE, FAKE, FAKE, 0, 65536, FAKE, FAKE, 128, 0, FAKE, None, FAKE,
            1 << 30, None]
    a = list(args); a[7] = 5
    assert f(*a) == hga.HGA_ERR_INVALID_ARGUMENT
    a = list(args); a[12] = 3
    assert f(*a) == hga.HGA_ERR_INVALID_ARGUMENT
    a = list(args); a[16] = 4096
    assert f(*a) == hga.HGA_ERR_WORKSPACE_TOO_SMALL
    a = list(args); a[8] = 0
    assert f(*a) == hga.HGA_ERR_INVALID_ARGUMENT
    a = list(args); a[13] = None
    assert f(*a) == hga.HGA_ERR_INVALID_ARGUMENT
    a = list(args); a[3] = 65  # more query tokens than a chunk
    assert f(*a) == hga.HGA_ERR_INVALID_ARGUMENT
    # 16..64 query tokens (MFMA prefill) need head_dim 128 and bf16
    for over in (dict(qkv_dtype=hga.HGA_F32), dict(head_dim=64)):
        a = list(args); a[0] = ctypes.byref(cfg(**over)); a[3] = 32
        assert f(*a) == hga.HGA_ERR_UNSUPPORTED, over


def test_attend_tiered_rejects():
    c = ctypes.byref(cfg())
    f = hga.lib().hga_attend_tiered
    args = [c, 4, FAKE, 1, FAKE, FAKE, FAKE, 65536, FAKE, FAKE, 65536, FAKE, FAKE, 128, FAKE, FAKE,
            FAKE, None, FAKE, 1 << 30, None, None, None, None]
    a = list(args); a[8] = None  # no cold pool
    assert f(*a) == hga.HGA_ERR_INVALID_ARGUMENT
    a = list(args); a[14] = None  # no working set
    assert f(*a) == hga.HGA_ERR_INVALID_ARGUMENT
    a = list(args); a[19] = 4096
    assert f(*a) == hga.HGA_ERR_WORKSPACE_TOO_SMALL
    a = list(args); a[13] = 300
    assert f(*a) == hga.HGA_ERR_UNSUPPORTED
    a = list(args); a[0] = ctypes.byref(cfg(qkv_dtype=hga.HGA_F32)); a[3] = 32
    assert f(*a) == hga.HGA_ERR_UNSUPPORTED
    # the two-stream form needs the caller's two distinct events
    n = hga.hga_workspace_bytes(cfg(), 4, 65536, 1)
    for ev in ((None, None), (FAKE, None), (None, FAKE), (FAKE, FAKE)):
        a = list(args); a[19] = n; a[21] = FAKE; a[22], a[23] = ev
        assert f(*a) == hga.HGA_ERR_INVALID_ARGUMENT, ev
    # hga_workspace_bytes covers the tiered call: with that size the call gets
    # past the workspace check and rejects the cold pool, which is not pinned
    n = hga.hga_workspace_bytes(cfg(), 4, 65536, 1)
    a = list(args); a[19] = n
    assert f(*a) == hga.HGA_ERR_INVALID_ARGUMENT


def test_fused_steps_reject():
    c = ctypes.byref(cfg())
    f = hga.lib().hga_prefill_step
    # cfg, B, q, lq, k_new, v_new, pos, k_pool, v_pool, cap, stage, cs, gs, max_chunks, sel,
    # n_sel, max_sel, out, lse, ws, ws_bytes, stream
    args = [c, 8, FAKE, 64, FAKE, FAKE, FAKE, FAKE, FAKE, 65536, FAKE, FAKE, FAKE, 1024, FAKE,
            FAKE, 128, FAKE, None, FAKE, 1 << 30, None]
    for lq in (0, 65):
        a = list(args); a[3] = lq
        assert f(*a) == hga.HGA_ERR_INVALID_ARGUMENT, lq
    a = list(args); a[10] = None  # no staging rows
    assert f(*a) == hga.HGA_ERR_INVALID_ARGUMENT
    a = list(args); a[20] = 4096
    assert f(*a) == hga.HGA_ERR_WORKSPACE_TOO_SMALL
    a = list(args); a[16] = 10  # list shorter than the windows + top-k_g
    assert f(*a) == hga.HGA_ERR_OUT_OF_RANGE
    for over in (dict(qkv_dtype=hga.HGA_F32), dict(head_dim=64)):
        a = list(args); a[0] = ctypes.byref(cfg(**over))
        assert f(*a) == hga.HGA_ERR_UNSUPPORTED, over
    d = hga.lib().hga_decode_step
    dargs = [c, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 65536, FAKE, FAKE, FAKE, 1024, FAKE, FAKE,
             128, FAKE, None, FAKE, 1 << 30, None]
    a = list(dargs); a[9] = None
    assert d(*a) == hga.HGA_ERR_INVALID_ARGUMENT
    a = list(dargs); a[19] = 4096
    assert d(*a) == hga.HGA_ERR_WORKSPACE_TOO_SMALL


def test_prefill_prompt_rejects():
    c = ctypes.byref(cfg())
    n = hga.hga_prompt_workspace_bytes(cfg(), 1, 32768, 512)
    assert n >= 4 * 512 * (511 + 128) * 8
    ws_size = ctypes.c_size_t()
    w = hga.lib().hga_prompt_workspace_bytes
    assert w(c, 1, 1000, 512, ctypes.byref(ws_size)) == hga.HGA_ERR_INVALID_ARGUMENT  # T % C
    assert w(c, 1, 32768, 100, ctypes.byref(ws_size)) == hga.HGA_ERR_INVALID_ARGUMENT
    f = hga.lib().hga_prefill_prompt
    # cfg, B, T, q, k_raw, v_raw, k_pool, v_pool, cap, cs, gs, max_chunks, sel, n_sel, max_sel,
    # out, lse, phases, ws, ws_bytes, stream
    args = [c, 1, 32768, FAKE, FAKE, FAKE, FAKE, FAKE, 32768, FAKE, FAKE, 512, FAKE, FAKE, 128,
            FAKE, None, hga.HGA_PROMPT_ALL, FAKE, 1 << 30, None]
    a = list(args); a[2] = 1000  # not a multiple of the chunk size
    assert f(*a) == hga.HGA_ERR_INVALID_ARGUMENT
    for ph in (0, 8, -1):
        a = list(args); a[17] = ph
        assert f(*a) == hga.HGA_ERR_INVALID_ARGUMENT, ph
    a = list(args); a[4] = None  # append phase without raw keys
    assert f(*a) == hga.HGA_ERR_INVALID_ARGUMENT
    a = list(args); a[15] = None  # attend phase without an output
    assert f(*a) == hga.HGA_ERR_INVALID_ARGUMENT
    a = list(args); a[8] = 16384  # prompt longer than the pool
    assert f(*a) == hga.HGA_ERR_OUT_OF_RANGE
    a = list(args); a[14] = 10
    assert f(*a) == hga.HGA_ERR_OUT_OF_RANGE
    a = list(args); a[19] = 4096
    assert f(*a) == hga.HGA_ERR_WORKSPACE_TOO_SMALL
    for over in (dict(qkv_dtype=hga.HGA_F32), dict(head_dim=64)):
        a = list(args); a[0] = ctypes.byref(cfg(**over))
        assert f(*a) == hga.HGA_ERR_UNSUPPORTED, over


def test_fp8_pool_limits():
    """The FP8 pool needs bf16 inputs and head_dim 128; its gather checks its
    arguments like the bf16 one (no call here reaches a launch)."""
    assert hga.hga_validate(cfg(pool_dtype=1)) == hga.HGA_OK
    assert hga.hga_validate(cfg(pool_dtype=1, qkv_dtype=hga.HGA_F32)) == hga.HGA_ERR_UNSUPPORTED
    assert hga.hga_validate(cfg(pool_dtype=1, head_dim=64)) == hga.HGA_ERR_UNSUPPORTED
    c = ctypes.byref(cfg(pool_dtype=1))
    g = hga.lib().hga_gather
    assert g(c, 8, FAKE, FAKE, 65536, 0, FAKE, FAKE, 128, None, 2, FAKE, FAKE, None) == \
        hga.HGA_ERR_INVALID_ARGUMENT  # part needs positions
    assert g(c, 8, FAKE, FAKE, 65535, 0, FAKE, FAKE, 128, None, 0, FAKE, FAKE, None) == \
        hga.HGA_ERR_INVALID_ARGUMENT  # pool_cap not a multiple of 16


def test_warm_gather_rejects():
    c = ctypes.byref(cfg())
    f = hga.lib().hga_warm_gather
    # cfg, B, k_cold, v_cold, cap, sel, n_sel, max_sel, pos, k_warm, v_warm, tags, used, n_warm,
    # step, k_ws, v_ws, hits, ws, ws_bytes, stream
    args = [c, 4, FAKE, FAKE, 65536, FAKE, FAKE, 128, FAKE, FAKE, FAKE, FAKE, FAKE, 256, 1, FAKE,
            FAKE, None, FAKE, 1 << 30, None]
    a = list(args); a[13] = 50  # fewer slots than topk_groups
    assert f(*a) == hga.HGA_ERR_OUT_OF_RANGE
    a = list(args); a[13] = 2048
    assert f(*a) == hga.HGA_ERR_OUT_OF_RANGE
    a = list(args); a[14] = 0  # the step stamp must be positive
    assert f(*a) == hga.HGA_ERR_INVALID_ARGUMENT
    a = list(args); a[11] = None
    assert f(*a) == hga.HGA_ERR_INVALID_ARGUMENT
    a = list(args); a[19] = 16
    assert f(*a) == hga.HGA_ERR_WORKSPACE_TOO_SMALL
    # valid sizes reach the pinned-pool check: FAKE is not pinned host memory
    assert f(*args) == hga.HGA_ERR_INVALID_ARGUMENT
    assert hga.hga_warm_workspace_bytes(cfg(), 4, 128) >= 2 * 4 * 4 * 128 * 4


def test_gather_and_merge_reject():
    c = ctypes.byref(cfg())
    g = hga.lib().hga_gather
    assert g(c, 8, FAKE, FAKE, 65536, 0, FAKE, FAKE, 128, None, 2, FAKE, FAKE, None) == \
        hga.HGA_ERR_INVALID_ARGUMENT  # part needs positions
    assert g(c, 8, None, FAKE, 65536, 0, FAKE, FAKE, 128, None, 0, FAKE, FAKE, None) == \
        hga.HGA_ERR_INVALID_ARGUMENT
    m = hga.lib().hga_merge_partials
    assert m(c, 8, 1, FAKE, None, FAKE, FAKE, FAKE, None, None) == hga.HGA_ERR_INVALID_ARGUMENT
