"""Python binding of the HGA C ABI (``libhga.so``, declared in ``include/hga.h``).

Argument marshalling only: every step of the hot path runs in the HIP
kernels of the library.  Tensor arguments may be torch tensors (their
``data_ptr()`` is passed), raw integer addresses, or ``None`` for nullable
pointers.  ``stream`` defaults to torch's current HIP stream.  A status other
than ``HGA_OK`` raises :class:`HgaError`.  There is no fallback: if the
library is not built, importing the functions raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhga.so")

HGA_OK = 0
HGA_ERR_INVALID_ARGUMENT = 1
HGA_ERR_UNSUPPORTED = 2
HGA_ERR_WORKSPACE_TOO_SMALL = 3
HGA_ERR_OUT_OF_RANGE = 4
HGA_ERR_HIP = 5

HGA_F32 = 0
HGA_BF16 = 1
HGA_SRC_POOL = 0
HGA_SRC_WORKING_SET = 1
HGA_PART_ALL = 0
HGA_PART_WINDOWS = 1
HGA_PART_ROUTED = 2
HGA_PROMPT_APPEND = 1
HGA_PROMPT_ROUTE = 2
HGA_PROMPT_ATTEND = 4
HGA_PROMPT_ALL = 7

EXPORTED = ("hga_validate", "hga_max_selected", "hga_workspace_bytes", "hga_workspace_reset",
            "hga_build_summaries", "hga_route", "hga_gather", "hga_attend", "hga_decode_step",
            "hga_prefill_step", "hga_prompt_workspace_bytes", "hga_prefill_prompt",
            "hga_attend_tiered", "hga_warm_workspace_bytes", "hga_warm_gather",
            "hga_merge_partials", "hga_status_string", "hga_version", "hga_decode_step_noalloc")


class HgaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class hga_config(ctypes.Structure):
    _fields_ = [
        ("head_dim", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("chunk_size", ctypes.c_int32),
        ("groups_per_chunk", ctypes.c_int32),
        ("n_sink_chunks", ctypes.c_int32),
        ("n_local_chunks", ctypes.c_int32),
        ("topk_chunks", ctypes.c_int32),
        ("topk_groups", ctypes.c_int32),
        ("rope_theta", ctypes.c_double),
        ("hf_wavelength", ctypes.c_double),
        ("qkv_dtype", ctypes.c_int32),
        ("rep_position", ctypes.c_int32),
        ("route_per_head", ctypes.c_int32),
        ("rope_style", ctypes.c_int32),
        ("pool_dtype", ctypes.c_int32),
        ("route_pool", ctypes.c_int32),
    ]


def config_from(p: dict, **over) -> hga_config:
    """hga_config from a plain dict with the field names above (``dtype`` may
    be given as "bf16"/"f32" instead of ``qkv_dtype``; ``rep_position``,
    ``route_per_head``, ``rope_style``, ``pool_dtype`` and ``route_pool``
    default to 0)."""
    q = dict(p)
    q.update(over)
    dt = q.get("qkv_dtype", HGA_BF16 if q.get("dtype") == "bf16" else HGA_F32)
    return hga_config(int(q["head_dim"]), int(q["n_q_heads"]), int(q["n_kv_heads"]),
                      int(q["chunk_size"]), int(q["groups_per_chunk"]), int(q["n_sink_chunks"]),
                      int(q["n_local_chunks"]), int(q["topk_chunks"]), int(q["topk_groups"]),
                      float(q["rope_theta"]), float(q["hf_wavelength"]), int(dt),
                      int(q.get("rep_position", 0)), int(q.get("route_per_head", 0)),
                      int(q.get("rope_style", 0)), int(q.get("pool_dtype", 0)),
                      int(q.get("route_pool", 0)))


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32
_C = ctypes.POINTER(hga_config)


def lib() -> ctypes.CDLL:
    """Load libhga.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "hga_validate": [_C],
            "hga_max_selected": [_C, _I, ctypes.POINTER(_I)],
            "hga_workspace_bytes": [_C, _I, _I, _I, ctypes.POINTER(ctypes.c_size_t)],
            "hga_workspace_reset": [_P, ctypes.c_size_t, _P],
            "hga_build_summaries": [_C, _I, _P, _P, _I, _I, _P, _P, _I, _P, _P, _I, _P],
            "hga_route": [_C, _I, _P, _I, _P, _P, _P, _I, _P, _P, _I, _P, _P, ctypes.c_size_t, _P],
            "hga_gather": [_C, _I, _P, _P, _I, _I, _P, _P, _I, _P, _I, _P, _P, _P],
            "hga_attend": [_C, _I, _P, _I, _P, _P, _P, _I, _I, _P, _P, _I, _I, _P, _P, _P,
                           ctypes.c_size_t, _P],
            "hga_decode_step": [_C, _I, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _I, _P, _P, _I,
                                _P, _P, _P, ctypes.c_size_t, _P],
            "hga_decode_step_noalloc": [_C, _I, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _I, _P,
                                        _P, _I, _P, _P, _P],
            "hga_prefill_step": [_C, _I, _P, _I, _P, _P, _P, _P, _P, _I, _P, _P, _P, _I, _P, _P,
                                 _I, _P, _P, _P, ctypes.c_size_t, _P],
            "hga_prompt_workspace_bytes": [_C, _I, _I, _I, ctypes.POINTER(ctypes.c_size_t)],
            "hga_prefill_prompt": [_C, _I, _I, _P, _P, _P, _P, _P, _I, _P, _P, _I, _P, _P, _I, _P,
                                   _P, _I, _P, ctypes.c_size_t, _P],
            "hga_attend_tiered": [_C, _I, _P, _I, _P, _P, _P, _I, _P, _P, _I, _P, _P, _I, _P, _P,
                                  _P, _P, _P, ctypes.c_size_t, _P, _P, _P, _P],
            "hga_warm_workspace_bytes": [_C, _I, _I, ctypes.POINTER(ctypes.c_size_t)],
            "hga_warm_gather": [_C, _I, _P, _P, _I, _P, _P, _I, _P, _P, _P, _P, _P, _I, _I, _P,
                                _P, _P, _P, ctypes.c_size_t, _P],
            "hga_merge_partials": [_C, _I, _I, _P, _P, _P, _P, _P, _P, _P],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.hga_status_string.argtypes = [ctypes.c_int]
        L.hga_status_string.restype = ctypes.c_char_p
        L.hga_version.argtypes = []
        L.hga_version.restype = ctypes.c_int32
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().hga_status_string(int(s)).decode()


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _event(e):
    """hipEvent_t of a torch.cuda.Event (torch creates its event on the first
    record, so an unused one is recorded once on the current stream) or a raw
    handle."""
    if isinstance(e, int):
        return e
    if not e.cuda_event:
        e.record()
    return e.cuda_event


def _check(st: int, where: str):
    if st != HGA_OK:
        raise HgaError(st, where)


def _cfg(cfg):
    return ctypes.byref(cfg if isinstance(cfg, hga_config) else config_from(cfg))


def hga_validate(cfg) -> int:
    return lib().hga_validate(_cfg(cfg))


def hga_version() -> int:
    return lib().hga_version()


def hga_status_string(s: int) -> str:
    return status_string(s)


def hga_max_selected(cfg, max_lq: int = 1) -> int:
    out = _I()
    _check(lib().hga_max_selected(_cfg(cfg), max_lq, ctypes.byref(out)), "hga_max_selected")
    return out.value


def hga_workspace_bytes(cfg, B: int, max_ctx: int, max_lq: int = 1) -> int:
    out = ctypes.c_size_t()
    _check(lib().hga_workspace_bytes(_cfg(cfg), B, max_ctx, max_lq, ctypes.byref(out)),
           "hga_workspace_bytes")
    return out.value


def hga_workspace_reset(ws, stream=None):
    _check(lib().hga_workspace_reset(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "hga_workspace_reset")


def hga_build_summaries(cfg, B, k_raw, v_new, pos0, n_tok, k_pool, v_pool, pool_cap, chunk_sum,
                        group_sum, max_chunks, stream=None):
    _check(lib().hga_build_summaries(_cfg(cfg), B, _ptr(k_raw), _ptr(v_new), pos0, n_tok,
                                     _ptr(k_pool), _ptr(v_pool), pool_cap, _ptr(chunk_sum),
                                     _ptr(group_sum), max_chunks, _stream(stream)),
           "hga_build_summaries")


def hga_route(cfg, B, q_raw, lq, q_pos0, chunk_sum, group_sum, max_chunks, sel_groups, n_sel,
              max_sel, chunk_scores, ws, stream=None):
    _check(lib().hga_route(_cfg(cfg), B, _ptr(q_raw), lq, _ptr(q_pos0), _ptr(chunk_sum),
                           _ptr(group_sum), max_chunks, _ptr(sel_groups), _ptr(n_sel), max_sel,
                           _ptr(chunk_scores), _ptr(ws), ws.numel() * ws.element_size(),
                           _stream(stream)),
           "hga_route")


def hga_gather(cfg, B, k_pool, v_pool, pool_cap, pool_is_host, sel_groups, n_sel, max_sel,
               q_pos0, part, k_ws, v_ws, stream=None):
    _check(lib().hga_gather(_cfg(cfg), B, _ptr(k_pool), _ptr(v_pool), pool_cap, int(pool_is_host),
                            _ptr(sel_groups), _ptr(n_sel), max_sel, _ptr(q_pos0), part, _ptr(k_ws),
                            _ptr(v_ws), _stream(stream)),
           "hga_gather")


def hga_attend(cfg, B, q_raw, lq, q_pos0, k_src, v_src, src_layout, src_cap, sel_groups, n_sel,
               max_sel, part, out, lse, ws, stream=None):
    _check(lib().hga_attend(_cfg(cfg), B, _ptr(q_raw), lq, _ptr(q_pos0), _ptr(k_src), _ptr(v_src),
                            src_layout, src_cap, _ptr(sel_groups), _ptr(n_sel), max_sel, part,
                            _ptr(out), _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(),
                            _stream(stream)),
           "hga_attend")


def hga_decode_step(cfg, B, q_raw, k_new, v_new, q_pos0, k_pool, v_pool, pool_cap, k_stage,
                    chunk_sum, group_sum, max_chunks, sel_groups, n_sel, max_sel, out, lse_opt, ws,
                    stream=None):
    _check(lib().hga_decode_step(_cfg(cfg), B, _ptr(q_raw), _ptr(k_new), _ptr(v_new), _ptr(q_pos0),
                                 _ptr(k_pool), _ptr(v_pool), pool_cap, _ptr(k_stage),
                                 _ptr(chunk_sum), _ptr(group_sum), max_chunks, _ptr(sel_groups),
                                 _ptr(n_sel), max_sel, _ptr(out), _ptr(lse_opt), _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(stream)),
           "hga_decode_step")


HGA_NOALLOC_SCRATCH_BYTES = 16 << 20


def hga_decode_step_noalloc(cfg, B, q_raw, k_new, v_new, q_pos0, k_pool, v_pool, pool_cap,
                            k_stage, chunk_sum, group_sum, max_chunks, sel_groups, n_sel, max_sel,
                            out, lse_opt, stream=None):
    """hga_decode_step with the library's static per-GPU scratch instead of a
    workspace (for callers that cannot allocate); calls on one GPU must not
    overlap."""
    _check(lib().hga_decode_step_noalloc(_cfg(cfg), B, _ptr(q_raw), _ptr(k_new), _ptr(v_new),
                                         _ptr(q_pos0), _ptr(k_pool), _ptr(v_pool), pool_cap,
                                         _ptr(k_stage), _ptr(chunk_sum), _ptr(group_sum),
                                         max_chunks, _ptr(sel_groups), _ptr(n_sel), max_sel,
                                         _ptr(out), _ptr(lse_opt), _stream(stream)),
           "hga_decode_step_noalloc")


def hga_prefill_step(cfg, B, q_raw, lq, k_new, v_new, q_pos0, k_pool, v_pool, pool_cap, k_stage,
                     chunk_sum, group_sum, max_chunks, sel_groups, n_sel, max_sel, out, lse_opt, ws,
                     stream=None):
    _check(lib().hga_prefill_step(_cfg(cfg), B, _ptr(q_raw), lq, _ptr(k_new), _ptr(v_new),
                                  _ptr(q_pos0), _ptr(k_pool), _ptr(v_pool), pool_cap,
                                  _ptr(k_stage), _ptr(chunk_sum), _ptr(group_sum), max_chunks,
                                  _ptr(sel_groups), _ptr(n_sel), max_sel, _ptr(out), _ptr(lse_opt),
                                  _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "hga_prefill_step")


def hga_prompt_workspace_bytes(cfg, B: int, T: int, max_chunks: int) -> int:
    out = ctypes.c_size_t()
    _check(lib().hga_prompt_workspace_bytes(_cfg(cfg), B, T, max_chunks, ctypes.byref(out)),
           "hga_prompt_workspace_bytes")
    return out.value


def hga_prefill_prompt(cfg, B, T, q_raw, k_raw, v_raw, k_pool, v_pool, pool_cap, chunk_sum,
                       group_sum, max_chunks, sel_groups, n_sel, max_sel, out, lse_opt, ws,
                       phases=HGA_PROMPT_ALL, stream=None):
    _check(lib().hga_prefill_prompt(_cfg(cfg), B, T, _ptr(q_raw), _ptr(k_raw), _ptr(v_raw),
                                    _ptr(k_pool), _ptr(v_pool), pool_cap, _ptr(chunk_sum),
                                    _ptr(group_sum), max_chunks, _ptr(sel_groups), _ptr(n_sel),
                                    max_sel, _ptr(out), _ptr(lse_opt), phases, _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream)),
           "hga_prefill_prompt")


def hga_attend_tiered(cfg, B, q_raw, lq, q_pos0, k_hot, v_hot, hot_cap, k_cold, v_cold, cold_cap,
                      sel_groups, n_sel, max_sel, k_ws, v_ws, out, lse_opt, ws, stream_a=None,
                      stream_b=None, events=None):
    """Windows from the device pool on stream_a, routed groups copied from the
    pinned host pool and attended on stream_b, merged on stream_a.  stream_a
    defaults to the current stream; stream_b=None selects the one-stream form
    (the window attention and the copy share one launch on stream_a).  With
    stream_b, ``events`` is a pair of torch.cuda.Event (fork, join) that the
    call records; they are created once by the caller and reused."""
    ev = (None, None)
    if stream_b is not None:
        if events is None or len(events) != 2:
            raise ValueError("hga_attend_tiered with stream_b needs events=(fork, join)")
        ev = tuple(_event(e) for e in events)
    _check(lib().hga_attend_tiered(_cfg(cfg), B, _ptr(q_raw), lq, _ptr(q_pos0), _ptr(k_hot),
                                   _ptr(v_hot), hot_cap, _ptr(k_cold), _ptr(v_cold), cold_cap,
                                   _ptr(sel_groups), _ptr(n_sel), max_sel, _ptr(k_ws), _ptr(v_ws),
                                   _ptr(out), _ptr(lse_opt), _ptr(ws), ws.numel() * ws.element_size(),
                                   _stream(stream_a), None if stream_b is None else _stream(stream_b),
                                   ev[0], ev[1]),
           "hga_attend_tiered")


def hga_warm_workspace_bytes(cfg, B: int, max_sel: int) -> int:
    out = ctypes.c_size_t()
    _check(lib().hga_warm_workspace_bytes(_cfg(cfg), B, max_sel, ctypes.byref(out)),
           "hga_warm_workspace_bytes")
    return out.value


def hga_warm_gather(cfg, B, k_cold, v_cold, cold_cap, sel_groups, n_sel, max_sel, q_pos0, k_warm,
                    v_warm, warm_tags, warm_used, n_warm, step, k_ws, v_ws, hits_opt, ws,
                    stream=None):
    _check(lib().hga_warm_gather(_cfg(cfg), B, _ptr(k_cold), _ptr(v_cold), cold_cap,
                                 _ptr(sel_groups), _ptr(n_sel), max_sel, _ptr(q_pos0),
                                 _ptr(k_warm), _ptr(v_warm), _ptr(warm_tags), _ptr(warm_used),
                                 n_warm, step, _ptr(k_ws), _ptr(v_ws), _ptr(hits_opt), _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(stream)),
           "hga_warm_gather")


def hga_merge_partials(cfg, B, lq, out_a, lse_a, out_b, lse_b, out, lse_out=None, stream=None):
    _check(lib().hga_merge_partials(_cfg(cfg), B, lq, _ptr(out_a), _ptr(lse_a), _ptr(out_b),
                                    _ptr(lse_b), _ptr(out), _ptr(lse_out), _stream(stream)),
           "hga_merge_partials")
