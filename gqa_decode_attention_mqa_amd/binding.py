"""Thin ctypes binding of ``libmqa_decode.so`` for torch tensors.

Argument marshalling only: shapes and dtypes are checked, device pointers and
torch's current HIP stream are handed to the C ABI (``include/mqa_decode.h``),
and every step of the computation runs in the library's kernels.  There is no
fallback: if the library is missing or a call fails, an exception says so.
"""
from __future__ import annotations

import ctypes
import math
import re
from pathlib import Path

import torch

import os

_PKG = Path(__file__).resolve().parent
# MQA_DECODE_LIB names another build of the library (e.g. the host-sanitizer
# build, _build/libmqa_decode_asan.so); by default the in-tree build is loaded.
LIB_PATH = Path(os.environ["MQA_DECODE_LIB"]) if os.environ.get("MQA_DECODE_LIB") else _PKG / "libmqa_decode.so"
HEADER_PATH = _PKG.parent / "include" / "mqa_decode.h"

MQA_OK = 0
VARIANTS = {"auto": 0, "valu": 1, "mfma": 2}
VARIANT_NAMES = {v: k for k, v in VARIANTS.items()}
COMBINE = {"auto": 0, "separate": 1, "fused": 2}
SCHEDULES = {None: 0, "auto": 0, "per_item": 1, "persistent": 2}
KV_FORMATS = {"bf16": 0, "fp8": 1, "int8": 2}


class MqaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__("%s failed with status %d: %s" % (where, status, detail))


class DecodeOpts(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int), ("chunk", ctypes.c_int), ("combine", ctypes.c_int),
                ("ev_main_begin", ctypes.c_void_p), ("ev_main_end", ctypes.c_void_p),
                ("window", ctypes.c_int), ("kv_format", ctypes.c_int),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("ev_combine_begin", ctypes.c_void_p), ("ev_combine_end", ctypes.c_void_p),
                ("host_seq_lens", ctypes.c_void_p), ("schedule", ctypes.c_int)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int), ("chunk", ctypes.c_int), ("max_splits", ctypes.c_int),
                ("combine", ctypes.c_int), ("head_blocks", ctypes.c_int),
                ("grid_main", ctypes.c_longlong), ("block_main", ctypes.c_int),
                ("grid_combine", ctypes.c_longlong), ("workspace_bytes", ctypes.c_size_t),
                ("persistent", ctypes.c_int)]


_lib = None


def load_library():
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise ImportError("libmqa_decode.so is not built at %s; run "
                          "`python -m gqa_decode_attention_mqa_amd.build` (or __graft_entry__.build())" % LIB_PATH)
    lib = ctypes.CDLL(str(LIB_PATH))
    vp, i32p, f32p = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    ints = [ctypes.c_int] * 5
    lib.mqa_decode_attention.argtypes = [vp, vp, vp, i32p, f32p] + ints + [ctypes.c_float, vp]
    lib.mqa_decode_attention.restype = ctypes.c_int
    lib.mqa_decode_attention_paged.argtypes = [vp, vp, vp, i32p, i32p, f32p] + [ctypes.c_int] * 7 + \
        [ctypes.c_float, vp, ctypes.POINTER(DecodeOpts)]
    lib.mqa_decode_attention_paged.restype = ctypes.c_int
    lib.mqa_decode_attention_window.argtypes = [vp, vp, vp, i32p, f32p] + ints + [ctypes.c_int, ctypes.c_float, vp]
    lib.mqa_decode_attention_window.restype = ctypes.c_int
    lib.mqa_decode_attention_quant.argtypes = [vp, vp, vp, vp, vp, i32p, f32p] + ints + \
        [ctypes.c_int, ctypes.c_float, vp, ctypes.POINTER(DecodeOpts)]
    lib.mqa_decode_attention_quant.restype = ctypes.c_int
    lib.mqa_decode_attention_multi.argtypes = [vp, vp, vp, i32p, f32p] + [ctypes.c_int] * 6 + \
        [ctypes.c_float, vp, ctypes.POINTER(DecodeOpts)]
    lib.mqa_decode_attention_multi.restype = ctypes.c_int
    lib.mqa_decode_attention_ex.argtypes = [vp, vp, vp, i32p, f32p] + ints + \
        [ctypes.c_float, vp, ctypes.POINTER(DecodeOpts)]
    lib.mqa_decode_attention_ex.restype = ctypes.c_int
    lib.mqa_decode_attention_noalloc.argtypes = [vp, vp, vp, i32p, f32p] + ints + \
        [ctypes.c_float, vp, ctypes.POINTER(DecodeOpts)]
    lib.mqa_decode_attention_noalloc.restype = ctypes.c_int
    lib.mqa_prefill_attention.argtypes = [vp, vp, vp, i32p, f32p] + ints + [ctypes.c_float, vp]
    lib.mqa_prefill_attention.restype = ctypes.c_int
    lib.mqa_decode_plan.argtypes = ints + [ctypes.c_float, ctypes.POINTER(DecodeOpts), ctypes.POINTER(PlanInfo)]
    lib.mqa_decode_plan.restype = ctypes.c_int
    lib.mqa_decode_plan_multi.argtypes = [ctypes.c_int] * 6 + [ctypes.c_float, ctypes.POINTER(DecodeOpts),
                                                              ctypes.POINTER(PlanInfo)]
    lib.mqa_decode_plan_multi.restype = ctypes.c_int
    lib.mqa_prefill_plan.argtypes = [ctypes.c_int] * 5 + [ctypes.c_float, ctypes.POINTER(PlanInfo),
                                                          ctypes.POINTER(ctypes.c_int)]
    lib.mqa_prefill_plan.restype = ctypes.c_int
    lib.mqa_status_string.argtypes = [ctypes.c_int]
    lib.mqa_status_string.restype = ctypes.c_char_p
    lib.mqa_last_error.argtypes = []
    lib.mqa_last_error.restype = ctypes.c_char_p
    lib.mqa_release_workspaces.argtypes = []
    lib.mqa_release_workspaces.restype = None
    lib.mqa_stream_read_probe.argtypes = [vp, ctypes.c_size_t, ctypes.c_int, vp, vp, vp, vp]
    lib.mqa_stream_read_probe.restype = ctypes.c_int
    lib.mqa_version.argtypes = []
    lib.mqa_version.restype = ctypes.c_int
    _lib = lib
    return lib


def declared_functions() -> list[str]:
    """Names of the functions ``include/mqa_decode.h`` declares."""
    text = HEADER_PATH.read_text()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(mqa_\w+)\s*\(", text, flags=re.M)))


def _check(status: int, where: str):
    if status != MQA_OK:
        lib = load_library()
        raise MqaError(status, where, "%s (%s)" % (lib.mqa_status_string(status).decode(),
                                                   lib.mqa_last_error().decode()))


def _host_lens(host_seq_lens):
    """A contiguous host int32 copy of the lengths (kept alive by the caller's opts), or None."""
    if host_seq_lens is None:
        return None
    t = torch.as_tensor(host_seq_lens)
    if t.device.type != "cpu":
        raise ValueError("host_seq_lens must be in host memory")
    return t.to(torch.int32).contiguous()


def _checked_lens(host_seq_lens, B):
    if host_seq_lens is None:
        return None
    t = _host_lens(host_seq_lens)
    if t.dim() != 1 or t.numel() != B:
        raise ValueError("host_seq_lens must hold B = %d lengths, got shape %s" % (B, tuple(t.shape)))
    return t


def make_opts(variant=None, chunk=None, combine=None, ev_begin=None, ev_end=None, window=None,
              kv_format=None, k_scale=None, v_scale=None, ev_combine_begin=None, ev_combine_end=None,
              host_seq_lens=None, schedule=None) -> DecodeOpts:
    """Options of a decode call.  ``host_seq_lens``: an optional host copy of the lengths, used by
    the planner only to pick the chunk size (see mqa_decode_opts.host_seq_lens).  ``schedule``:
    None / "auto", "per_item" or "persistent" (see mqa_decode_opts.schedule)."""
    o = DecodeOpts()
    o.schedule = SCHEDULES[schedule] if isinstance(schedule, str) or schedule is None else int(schedule)
    o._host_lens = _host_lens(host_seq_lens)
    o.host_seq_lens = o._host_lens.data_ptr() if o._host_lens is not None else None
    o.ev_combine_begin = ev_combine_begin
    o.ev_combine_end = ev_combine_end
    o.window = int(window or 0)
    o.kv_format = KV_FORMATS[kv_format] if isinstance(kv_format, str) else int(kv_format or 0)
    o.k_scale = k_scale
    o.v_scale = v_scale
    o.variant = VARIANTS[variant] if isinstance(variant, str) else int(variant or 0)
    o.chunk = int(chunk or 0)
    o.combine = COMBINE[combine] if isinstance(combine, str) else int(combine or 0)
    o.ev_main_begin = ev_begin
    o.ev_main_end = ev_end
    return o


def plan(B, Hq, Hkv, D, Lmax, scale=None, variant=None, chunk=None, combine=None, window=None,
         kv_format=None, tokens=1, host_seq_lens=None, schedule=None) -> dict:
    """The library's launch plan for a decode call of this shape (host only);
    ``tokens`` > 1 plans a multi-token call."""
    lib = load_library()
    info = PlanInfo()
    opts = make_opts(variant, chunk, combine, window=window, kv_format=kv_format, host_seq_lens=host_seq_lens,
                     schedule=schedule)
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib.mqa_decode_plan_multi(B, int(tokens), Hq, Hkv, D, Lmax, sc, ctypes.byref(opts), ctypes.byref(info)),
           "mqa_decode_plan")
    return {"variant": VARIANT_NAMES.get(info.variant, info.variant), "chunk": info.chunk,
            "max_splits": info.max_splits, "combine": info.combine, "head_blocks": info.head_blocks,
            "grid_main": info.grid_main, "block_main": info.block_main,
            "grid_combine": info.grid_combine, "workspace_bytes": info.workspace_bytes,
            "persistent": bool(info.persistent)}


def prefill_plan(B, Hq, Hkv, D, Lmax, scale=None) -> dict:
    """The library's launch plan for a mqa_prefill_attention call (host only);
    ``rows_per_block`` is the number of query rows (position, head of the group)
    one workgroup serves."""
    lib = load_library()
    info = PlanInfo()
    rows = ctypes.c_int(0)
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib.mqa_prefill_plan(B, Hq, Hkv, D, Lmax, sc, ctypes.byref(info), ctypes.byref(rows)),
           "mqa_prefill_plan")
    return {"variant": VARIANT_NAMES.get(info.variant, info.variant), "chunk": info.chunk,
            "max_splits": info.max_splits, "combine": info.combine, "head_blocks": info.head_blocks,
            "grid_main": info.grid_main, "block_main": info.block_main,
            "grid_combine": info.grid_combine, "workspace_bytes": info.workspace_bytes,
            "rows_per_block": rows.value}


def _stream_ptr(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _require(t: torch.Tensor, name: str, dtype, ndim: int, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.dim() != ndim:
        raise ValueError("%s must have %d dims, got shape %s" % (name, ndim, tuple(t.shape)))
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, seq_lens: torch.Tensor,
           scale: float | None = None, out: torch.Tensor | None = None, variant=None, chunk=None,
           combine=None, events=None, window=None, host_seq_lens=None, schedule=None) -> torch.Tensor:
    """One decode step.  q [B,Hq,D] bf16, caches [B,Lmax,Hkv,D] bf16, seq_lens [B] int32 -> fp32 [B,Hq,D].

    Runs on torch's current stream of q's device.  ``events`` = (begin, end)
    torch.cuda.Event pair recorded around the split-K kernel alone.  ``window``
    (> 0) restricts each sequence to its last ``window`` positions.
    """
    if q.device.type != "cuda":
        raise ValueError("decode runs on the GPU; q is on %s" % q.device)
    dev = q.device
    _require(q, "q", torch.bfloat16, 3, dev)
    _require(k_cache, "k_cache", torch.bfloat16, 4, dev)
    _require(v_cache, "v_cache", torch.bfloat16, 4, dev)
    _require(seq_lens, "seq_lens", torch.int32, 1, dev)
    B, Hq, D = q.shape
    Bk, Lmax, Hkv, Dk = k_cache.shape
    if v_cache.shape != k_cache.shape or Bk != B or Dk != D or seq_lens.shape[0] != B:
        raise ValueError("shape mismatch: q %s, k %s, v %s, seq_lens %s" % (
            tuple(q.shape), tuple(k_cache.shape), tuple(v_cache.shape), tuple(seq_lens.shape)))
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    _require(out, "out", torch.float32, 3, dev)
    if tuple(out.shape) != (B, Hq, D):
        raise ValueError("out must have shape %s" % ((B, Hq, D),))
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    ev_b = ev_e = None
    if events is not None:
        ev_b, ev_e = events[0].cuda_event, events[1].cuda_event
    opts = make_opts(variant, chunk, combine, ev_b, ev_e, window,
                     host_seq_lens=_checked_lens(host_seq_lens, B), schedule=schedule)
    lib = load_library()
    st = lib.mqa_decode_attention_ex(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                     seq_lens.data_ptr(), out.data_ptr(), B, Hq, Hkv, D, Lmax,
                                     sc, _stream_ptr(dev), ctypes.byref(opts))
    _check(st, "mqa_decode_attention")
    return out


def decode_paged(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor, block_table: torch.Tensor,
                 seq_lens: torch.Tensor, scale: float | None = None, out: torch.Tensor | None = None,
                 variant=None, chunk=None, combine=None, events=None, window=None, kv_format=None,
                 k_scale=None, v_scale=None, host_seq_lens=None, schedule=None) -> torch.Tensor:
    """One decode step over a paged cache.  q [B,Hq,D] bf16, pages [num_pages,page_size,Hkv,D] bf16,
    block_table [B,max_blocks] int32, seq_lens [B] int32 -> fp32 [B,Hq,D].  With ``kv_format``
    "fp8" or "int8" the pages hold 8-bit codes (uint8) and ``k_scale`` / ``v_scale`` are fp32
    [num_pages, Hkv, page_size]."""
    if q.device.type != "cuda":
        raise ValueError("decode_paged runs on the GPU; q is on %s" % q.device)
    dev = q.device
    _require(q, "q", torch.bfloat16, 3, dev)
    fmt = KV_FORMATS[kv_format] if isinstance(kv_format, str) else int(kv_format or 0)
    _require(k_pages, "k_pages", torch.uint8 if fmt else torch.bfloat16, 4, dev)
    _require(v_pages, "v_pages", torch.uint8 if fmt else torch.bfloat16, 4, dev)
    sk = sv = None
    if fmt:
        _require(k_scale, "k_scale", torch.float32, 3, dev)
        _require(v_scale, "v_scale", torch.float32, 3, dev)
        if tuple(k_scale.shape) != (k_pages.shape[0], k_pages.shape[2], k_pages.shape[1]) or \
                v_scale.shape != k_scale.shape:
            raise ValueError("scales must have shape [num_pages, Hkv, page_size]")
        sk, sv = k_scale.data_ptr(), v_scale.data_ptr()
    _require(block_table, "block_table", torch.int32, 2, dev)
    _require(seq_lens, "seq_lens", torch.int32, 1, dev)
    B, Hq, D = q.shape
    num_pages, page_size, Hkv, Dk = k_pages.shape
    if v_pages.shape != k_pages.shape or Dk != D or seq_lens.shape[0] != B or block_table.shape[0] != B:
        raise ValueError("shape mismatch: q %s, pages %s, block_table %s, seq_lens %s" % (
            tuple(q.shape), tuple(k_pages.shape), tuple(block_table.shape), tuple(seq_lens.shape)))
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    _require(out, "out", torch.float32, 3, dev)
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    ev_b = ev_e = None
    if events is not None:
        ev_b, ev_e = events[0].cuda_event, events[1].cuda_event
    opts = make_opts(variant, chunk, combine, ev_b, ev_e, window, fmt, sk, sv,
                     host_seq_lens=_checked_lens(host_seq_lens, B), schedule=schedule)
    lib = load_library()
    st = lib.mqa_decode_attention_paged(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(),
                                        block_table.data_ptr(), seq_lens.data_ptr(), out.data_ptr(),
                                        B, Hq, Hkv, D, num_pages, page_size, block_table.shape[1],
                                        sc, _stream_ptr(dev), ctypes.byref(opts))
    _check(st, "mqa_decode_attention_paged")
    return out


def decode_quant(q: torch.Tensor, k_codes: torch.Tensor, v_codes: torch.Tensor, k_scale: torch.Tensor,
                 v_scale: torch.Tensor, seq_lens: torch.Tensor, kv_format: str, scale: float | None = None,
                 out: torch.Tensor | None = None, variant=None, chunk=None, combine=None, events=None,
                 window=None, host_seq_lens=None, schedule=None) -> torch.Tensor:
    """One decode step against an 8-bit cache through ``mqa_decode_attention_quant``.
    q [B,Hq,D] bf16; codes [B,Lmax,Hkv,D] uint8 (E4M3 for "fp8", two's complement for
    "int8"); scales [B,Hkv,Lmax] fp32; seq_lens [B] int32 -> fp32 [B,Hq,D]."""
    if q.device.type != "cuda":
        raise ValueError("decode_quant runs on the GPU; q is on %s" % q.device)
    dev = q.device
    _require(q, "q", torch.bfloat16, 3, dev)
    _require(k_codes, "k_codes", torch.uint8, 4, dev)
    _require(v_codes, "v_codes", torch.uint8, 4, dev)
    _require(k_scale, "k_scale", torch.float32, 3, dev)
    _require(v_scale, "v_scale", torch.float32, 3, dev)
    _require(seq_lens, "seq_lens", torch.int32, 1, dev)
    B, Hq, D = q.shape
    Bk, Lmax, Hkv, Dk = k_codes.shape
    if v_codes.shape != k_codes.shape or Bk != B or Dk != D or seq_lens.shape[0] != B or \
            tuple(k_scale.shape) != (B, Hkv, Lmax) or v_scale.shape != k_scale.shape:
        raise ValueError("shape mismatch: q %s, codes %s, scales %s, seq_lens %s" % (
            tuple(q.shape), tuple(k_codes.shape), tuple(k_scale.shape), tuple(seq_lens.shape)))
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    _require(out, "out", torch.float32, 3, dev)
    if tuple(out.shape) != (B, Hq, D):
        raise ValueError("out must have shape %s" % ((B, Hq, D),))
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    ev_b = ev_e = None
    if events is not None:
        ev_b, ev_e = events[0].cuda_event, events[1].cuda_event
    opts = make_opts(variant, chunk, combine, ev_b, ev_e, window,
                     host_seq_lens=_checked_lens(host_seq_lens, B), schedule=schedule)
    lib = load_library()
    st = lib.mqa_decode_attention_quant(q.data_ptr(), k_codes.data_ptr(), v_codes.data_ptr(), k_scale.data_ptr(),
                                        v_scale.data_ptr(), seq_lens.data_ptr(), out.data_ptr(), B, Hq, Hkv, D,
                                        Lmax, KV_FORMATS[kv_format], sc, _stream_ptr(dev), ctypes.byref(opts))
    _check(st, "mqa_decode_attention_quant")
    return out


def decode_multi(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, seq_lens: torch.Tensor,
                 scale: float | None = None, out: torch.Tensor | None = None, variant=None, chunk=None,
                 combine=None, events=None, kv_format=None, k_scale=None, v_scale=None, host_seq_lens=None, schedule=None) -> torch.Tensor:
    """T new tokens per sequence through ``mqa_decode_attention_multi``: q [B,T,Hq,D] bf16
    -> fp32 [B,T,Hq,D]; token i attends positions 0 .. seq_lens[b] - T + i.  Caches as for
    :func:`decode` (bf16), or 8-bit codes with ``kv_format`` and scales as for :func:`decode_quant`."""
    if q.device.type != "cuda":
        raise ValueError("decode_multi runs on the GPU; q is on %s" % q.device)
    dev = q.device
    _require(q, "q", torch.bfloat16, 4, dev)
    fmt = KV_FORMATS[kv_format] if isinstance(kv_format, str) else int(kv_format or 0)
    _require(k_cache, "k_cache", torch.uint8 if fmt else torch.bfloat16, 4, dev)
    _require(v_cache, "v_cache", torch.uint8 if fmt else torch.bfloat16, 4, dev)
    _require(seq_lens, "seq_lens", torch.int32, 1, dev)
    B, T, Hq, D = q.shape
    Bk, Lmax, Hkv, Dk = k_cache.shape
    if v_cache.shape != k_cache.shape or Bk != B or Dk != D or seq_lens.shape[0] != B:
        raise ValueError("shape mismatch: q %s, k %s, v %s, seq_lens %s" % (
            tuple(q.shape), tuple(k_cache.shape), tuple(v_cache.shape), tuple(seq_lens.shape)))
    sk = sv = None
    if fmt:
        _require(k_scale, "k_scale", torch.float32, 3, dev)
        _require(v_scale, "v_scale", torch.float32, 3, dev)
        if tuple(k_scale.shape) != (B, Hkv, Lmax) or v_scale.shape != k_scale.shape:
            raise ValueError("scales must have shape [B, Hkv, Lmax]")
        sk, sv = k_scale.data_ptr(), v_scale.data_ptr()
    if out is None:
        out = torch.empty((B, T, Hq, D), dtype=torch.float32, device=dev)
    _require(out, "out", torch.float32, 4, dev)
    if tuple(out.shape) != (B, T, Hq, D):
        raise ValueError("out must have shape %s" % ((B, T, Hq, D),))
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    ev_b = ev_e = None
    if events is not None:
        ev_b, ev_e = events[0].cuda_event, events[1].cuda_event
    opts = make_opts(variant, chunk, combine, ev_b, ev_e, None, fmt, sk, sv,
                     host_seq_lens=_checked_lens(host_seq_lens, B), schedule=schedule)
    lib = load_library()
    st = lib.mqa_decode_attention_multi(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(),
                                        out.data_ptr(), B, T, Hq, Hkv, D, Lmax, sc, _stream_ptr(dev),
                                        ctypes.byref(opts))
    _check(st, "mqa_decode_attention_multi")
    return out


def decode_window(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, seq_lens: torch.Tensor,
                  window: int, scale: float | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """One decode step with a sliding window through ``mqa_decode_attention_window``:
    sequence b attends its last ``window`` positions.  Shapes as :func:`decode`."""
    if q.device.type != "cuda":
        raise ValueError("decode_window runs on the GPU; q is on %s" % q.device)
    dev = q.device
    _require(q, "q", torch.bfloat16, 3, dev)
    _require(k_cache, "k_cache", torch.bfloat16, 4, dev)
    _require(v_cache, "v_cache", torch.bfloat16, 4, dev)
    _require(seq_lens, "seq_lens", torch.int32, 1, dev)
    B, Hq, D = q.shape
    Bk, Lmax, Hkv, Dk = k_cache.shape
    if v_cache.shape != k_cache.shape or Bk != B or Dk != D or seq_lens.shape[0] != B:
        raise ValueError("shape mismatch: q %s, k %s, v %s, seq_lens %s" % (
            tuple(q.shape), tuple(k_cache.shape), tuple(v_cache.shape), tuple(seq_lens.shape)))
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    _require(out, "out", torch.float32, 3, dev)
    if tuple(out.shape) != (B, Hq, D):
        raise ValueError("out must have shape %s" % ((B, Hq, D),))
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    lib = load_library()
    st = lib.mqa_decode_attention_window(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                         seq_lens.data_ptr(), out.data_ptr(), B, Hq, Hkv, D, Lmax,
                                         int(window), sc, _stream_ptr(dev))
    _check(st, "mqa_decode_attention_window")
    return out


def prefill(q_seq: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, seq_lens: torch.Tensor,
            scale: float | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """Causal attention with no cache: q_seq [B,Lmax,Hq,D] bf16 -> fp32 [B,Lmax,Hq,D]."""
    if q_seq.device.type != "cuda":
        raise ValueError("prefill runs on the GPU; q_seq is on %s" % q_seq.device)
    dev = q_seq.device
    _require(q_seq, "q_seq", torch.bfloat16, 4, dev)
    _require(k_cache, "k_cache", torch.bfloat16, 4, dev)
    _require(v_cache, "v_cache", torch.bfloat16, 4, dev)
    _require(seq_lens, "seq_lens", torch.int32, 1, dev)
    B, Lmax, Hq, D = q_seq.shape
    if k_cache.shape[:2] != (B, Lmax) or k_cache.shape[3] != D or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch between q_seq and the caches")
    Hkv = k_cache.shape[2]
    if out is None:
        out = torch.empty((B, Lmax, Hq, D), dtype=torch.float32, device=dev)
    _require(out, "out", torch.float32, 4, dev)
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    lib = load_library()
    st = lib.mqa_prefill_attention(q_seq.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                   seq_lens.data_ptr(), out.data_ptr(), B, Hq, Hkv, D, Lmax, sc,
                                   _stream_ptr(dev))
    _check(st, "mqa_prefill_attention")
    return out


def release_workspaces():
    load_library().mqa_release_workspaces()


def stream_read_probe(buf: torch.Tensor, workgroups: int, sink: torch.Tensor, events=None):
    """Streaming-read calibration over all of ``buf`` (contiguous device memory) with
    ``workgroups`` workgroups; ``sink`` int32 or uint32 [>= workgroups]; ``events`` =
    (begin, end) torch.cuda.Event pair recorded by the kernel's own dispatch."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be contiguous device memory")
    if sink.device != buf.device or sink.numel() < workgroups or sink.element_size() != 4:
        raise ValueError("sink must hold at least `workgroups` 4-byte words on buf's device")
    ev_b = ev_e = None
    if events is not None:
        ev_b, ev_e = events[0].cuda_event, events[1].cuda_event
    lib = load_library()
    st = lib.mqa_stream_read_probe(buf.data_ptr(), buf.numel() * buf.element_size(), int(workgroups),
                                   sink.data_ptr(), _stream_ptr(buf.device), ev_b, ev_e)
    _check(st, "mqa_stream_read_probe")
