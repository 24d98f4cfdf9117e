"""CPU fp64 oracle for one MQA/GQA decode step (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and it imports nothing
from the product package: the two sides meet only through the seeded input
generator, which holds none of the method's arithmetic.

The arithmetic lives in ``decode_oracle.c`` (plain C, OpenMP over
(sequence, head) pairs, double precision, no fast-math).  This module compiles
it with gcc when the shared object is missing and marshals arrays through
ctypes.  See the C file's header for the definition it follows and the
passages of the source pages it restates.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "decode_oracle.c"
_LIB_PATH = _HERE / "liboracle.so"
_lib = None


def build(force: bool = False) -> Path:
    """Compile ``liboracle.so`` with gcc (-O2, OpenMP, strict IEEE math)."""
    if force or not _LIB_PATH.exists() or _LIB_PATH.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB_PATH.with_suffix(".so.tmp%d" % os.getpid())
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-fno-fast-math", "-ffp-contract=off",
               str(_SRC), "-o", str(tmp), "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(str(_LIB_PATH))
        u16p = ctypes.POINTER(ctypes.c_uint16)
        i32p = ctypes.POINTER(ctypes.c_int32)
        f64p = ctypes.POINTER(ctypes.c_double)
        lib.oracle_decode.argtypes = [u16p, u16p, u16p, i32p] + [ctypes.c_int] * 5 + \
            [ctypes.c_double, f64p, f64p]
        lib.oracle_decode.restype = ctypes.c_int
        lib.oracle_causal_prefill.argtypes = [u16p, u16p, u16p, i32p] + [ctypes.c_int] * 5 + \
            [ctypes.c_double, f64p]
        lib.oracle_decode_paged.argtypes = [u16p, u16p, u16p, i32p, i32p] + [ctypes.c_int] * 7 + \
            [ctypes.c_double, f64p]
        lib.oracle_decode_paged.restype = ctypes.c_int
        lib.oracle_causal_prefill.restype = ctypes.c_int
        lib.oracle_decode_window.argtypes = [u16p, u16p, u16p, i32p] + [ctypes.c_int] * 6 + \
            [ctypes.c_double, f64p]
        lib.oracle_local_prefill.argtypes = [u16p, u16p, u16p, i32p] + [ctypes.c_int] * 6 + \
            [ctypes.c_double, f64p]
        u8p = ctypes.POINTER(ctypes.c_uint8)
        f32p = ctypes.POINTER(ctypes.c_float)
        lib.oracle_decode_quant.argtypes = [u16p, u8p, u8p, f32p, f32p, i32p] + [ctypes.c_int] * 6 + \
            [ctypes.c_double, f64p]
        lib.oracle_fp8_e4m3_value.argtypes = [ctypes.c_uint8]
        lib.oracle_fp8_e4m3_value.restype = ctypes.c_double
        lib.oracle_decode_multi.argtypes = [u16p, u16p, u16p, i32p] + [ctypes.c_int] * 6 + \
            [ctypes.c_double, f64p]
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_threads.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _bits(x) -> np.ndarray:
    """bfloat16 data as a C-contiguous uint16 array of its bit patterns."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            if x.dtype != torch.bfloat16:
                raise TypeError("oracle expects bfloat16 tensors, got %s" % x.dtype)
            x = x.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)
    except ImportError:  # pragma: no cover - torch is always present here
        pass
    a = np.ascontiguousarray(x)
    if a.dtype != np.uint16:
        raise TypeError("oracle expects bf16 bit patterns as uint16, got %s" % a.dtype)
    return a


def _lens(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu").numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def set_threads(n: int) -> int:
    """Set the OpenMP thread count; returns the count now in effect."""
    return _load().oracle_set_threads(int(n))


def max_threads() -> int:
    return _load().oracle_max_threads()


def decode(q, k_cache, v_cache, seq_lens, scale: float, return_lse: bool = False):
    """fp64 decode step.  Shapes: q [B,Hq,D], caches [B,Lmax,Hkv,D], seq_lens [B].

    Returns ``out`` [B,Hq,D] float64 (and the natural-log LSE [B,Hq] when
    ``return_lse``).
    """
    qb, kb, vb = _bits(q), _bits(k_cache), _bits(v_cache)
    lens = _lens(seq_lens)
    B, Hq, D = qb.shape
    Bk, Lmax, Hkv, Dk = kb.shape
    if vb.shape != kb.shape or Bk != B or Dk != D or lens.shape != (B,):
        raise ValueError("inconsistent shapes q%s k%s v%s lens%s" % (qb.shape, kb.shape, vb.shape, lens.shape))
    out = np.empty((B, Hq, D), dtype=np.float64)
    lse = np.empty((B, Hq), dtype=np.float64) if return_lse else None
    rc = _load().oracle_decode(_ptr(qb, ctypes.c_uint16), _ptr(kb, ctypes.c_uint16),
                               _ptr(vb, ctypes.c_uint16), _ptr(lens, ctypes.c_int32),
                               B, Hq, Hkv, D, Lmax, float(scale), _ptr(out, ctypes.c_double),
                               _ptr(lse, ctypes.c_double) if lse is not None else None)
    if rc != 0:
        raise ValueError("oracle_decode rejected its arguments (code %d)" % rc)
    return (out, lse) if return_lse else out


def decode_paged(q, k_pages, v_pages, block_table, seq_lens, scale: float):
    """fp64 decode step over a paged cache.  q [B,Hq,D], pages [num_pages,page_size,Hkv,D],
    block_table [B,max_blocks] int32, seq_lens [B].  Returns ``out`` [B,Hq,D] float64."""
    qb, kb, vb = _bits(q), _bits(k_pages), _bits(v_pages)
    lens = _lens(seq_lens)
    table = _lens(block_table)
    B, Hq, D = qb.shape
    num_pages, page_size, Hkv, Dk = kb.shape
    if vb.shape != kb.shape or Dk != D or lens.shape != (B,) or table.ndim != 2 or table.shape[0] != B:
        raise ValueError("inconsistent shapes q%s pages%s table%s lens%s" % (qb.shape, kb.shape, table.shape,
                                                                           lens.shape))
    out = np.empty((B, Hq, D), dtype=np.float64)
    rc = _load().oracle_decode_paged(_ptr(qb, ctypes.c_uint16), _ptr(kb, ctypes.c_uint16),
                                     _ptr(vb, ctypes.c_uint16), _ptr(table, ctypes.c_int32),
                                     _ptr(lens, ctypes.c_int32), B, Hq, Hkv, D, num_pages, page_size,
                                     table.shape[1], float(scale), _ptr(out, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle_decode_paged rejected its arguments (code %d)" % rc)
    return out


def causal_prefill(q_seq, k_cache, v_cache, seq_lens, scale: float):
    """fp64 causal attention with no cache.  q_seq [B,Lmax,Hq,D] -> [B,Lmax,Hq,D]."""
    qb, kb, vb = _bits(q_seq), _bits(k_cache), _bits(v_cache)
    lens = _lens(seq_lens)
    B, Lmax, Hq, D = qb.shape
    Bk, Lk, Hkv, Dk = kb.shape
    if vb.shape != kb.shape or (Bk, Lk, Dk) != (B, Lmax, D) or lens.shape != (B,):
        raise ValueError("inconsistent shapes")
    out = np.empty((B, Lmax, Hq, D), dtype=np.float64)
    rc = _load().oracle_causal_prefill(_ptr(qb, ctypes.c_uint16), _ptr(kb, ctypes.c_uint16),
                                       _ptr(vb, ctypes.c_uint16), _ptr(lens, ctypes.c_int32),
                                       B, Hq, Hkv, D, Lmax, float(scale), _ptr(out, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle_causal_prefill rejected its arguments (code %d)" % rc)
    return out


def decode_window(q, k_cache, v_cache, seq_lens, window: int, scale: float):
    """fp64 decode step with a sliding window: sequence b attends positions
    max(0, n - window) .. n - 1.  Shapes as :func:`decode`.  Returns ``out`` [B,Hq,D]."""
    qb, kb, vb = _bits(q), _bits(k_cache), _bits(v_cache)
    lens = _lens(seq_lens)
    B, Hq, D = qb.shape
    Bk, Lmax, Hkv, Dk = kb.shape
    if vb.shape != kb.shape or Bk != B or Dk != D or lens.shape != (B,):
        raise ValueError("inconsistent shapes q%s k%s v%s lens%s" % (qb.shape, kb.shape, vb.shape, lens.shape))
    out = np.empty((B, Hq, D), dtype=np.float64)
    rc = _load().oracle_decode_window(_ptr(qb, ctypes.c_uint16), _ptr(kb, ctypes.c_uint16),
                                      _ptr(vb, ctypes.c_uint16), _ptr(lens, ctypes.c_int32),
                                      B, Hq, Hkv, D, Lmax, int(window), float(scale),
                                      _ptr(out, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle_decode_window rejected its arguments (code %d)" % rc)
    return out


def local_prefill(q_seq, k_cache, v_cache, seq_lens, window: int, scale: float):
    """fp64 sliding-window causal attention with no cache (row i attends
    i - window < j <= i).  q_seq [B,Lmax,Hq,D] -> [B,Lmax,Hq,D]."""
    qb, kb, vb = _bits(q_seq), _bits(k_cache), _bits(v_cache)
    lens = _lens(seq_lens)
    B, Lmax, Hq, D = qb.shape
    Bk, Lk, Hkv, Dk = kb.shape
    if vb.shape != kb.shape or (Bk, Lk, Dk) != (B, Lmax, D) or lens.shape != (B,):
        raise ValueError("inconsistent shapes")
    out = np.empty((B, Lmax, Hq, D), dtype=np.float64)
    rc = _load().oracle_local_prefill(_ptr(qb, ctypes.c_uint16), _ptr(kb, ctypes.c_uint16),
                                      _ptr(vb, ctypes.c_uint16), _ptr(lens, ctypes.c_int32),
                                      B, Hq, Hkv, D, Lmax, int(window), float(scale),
                                      _ptr(out, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle_local_prefill rejected its arguments (code %d)" % rc)
    return out


KV_FORMATS = {"fp8": 1, "int8": 2}


def fp8_e4m3_value(code: int) -> float:
    """Value of one E4M3 code (0..255) as the oracle decodes it."""
    return _load().oracle_fp8_e4m3_value(int(code))


def _codes(x) -> np.ndarray:
    """8-bit codes (uint8, int8 or float8 tensors, or arrays) as a C-contiguous uint8 array."""
    import torch
    if isinstance(x, torch.Tensor):
        x = x.detach().to("cpu").contiguous()
        if x.element_size() != 1:
            raise TypeError("oracle expects 8-bit codes, got %s" % x.dtype)
        return np.ascontiguousarray(x.view(torch.uint8).numpy())
    a = np.ascontiguousarray(np.asarray(x))
    if a.itemsize != 1:
        raise TypeError("oracle expects 8-bit codes, got %s" % a.dtype)
    return a.view(np.uint8)


def _scales(x) -> np.ndarray:
    import torch
    if isinstance(x, torch.Tensor):
        x = x.detach().to("cpu").numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def decode_quant(q, k_codes, v_codes, k_scale, v_scale, seq_lens, kv_format: str, scale: float):
    """fp64 decode step against an 8-bit cache.  q [B,Hq,D] bf16; codes [B,Lmax,Hkv,D]
    (uint8 bits; E4M3 for "fp8", two's complement for "int8"); scales [B,Hkv,Lmax] fp32.
    Returns ``out`` [B,Hq,D] float64."""
    qb, kc, vc = _bits(q), _codes(k_codes), _codes(v_codes)
    ks, vs = _scales(k_scale), _scales(v_scale)
    lens = _lens(seq_lens)
    B, Hq, D = qb.shape
    Bk, Lmax, Hkv, Dk = kc.shape
    if vc.shape != kc.shape or Bk != B or Dk != D or lens.shape != (B,) or \
            ks.shape != (B, Hkv, Lmax) or vs.shape != ks.shape:
        raise ValueError("inconsistent shapes q%s codes%s scales%s lens%s" % (qb.shape, kc.shape, ks.shape,
                                                                            lens.shape))
    out = np.empty((B, Hq, D), dtype=np.float64)
    rc = _load().oracle_decode_quant(_ptr(qb, ctypes.c_uint16), _ptr(kc, ctypes.c_uint8), _ptr(vc, ctypes.c_uint8),
                                     _ptr(ks, ctypes.c_float), _ptr(vs, ctypes.c_float), _ptr(lens, ctypes.c_int32),
                                     B, Hq, Hkv, D, Lmax, KV_FORMATS[kv_format], float(scale),
                                     _ptr(out, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle_decode_quant rejected its arguments (code %d)" % rc)
    return out


def decode_multi(q, k_cache, v_cache, seq_lens, scale: float):
    """fp64 decode of T tokens per sequence, causal among themselves: token i of
    sequence b attends positions 0 .. seq_lens[b] - T + i.  q [B,T,Hq,D] ->
    ``out`` [B,T,Hq,D] float64."""
    qb, kb, vb = _bits(q), _bits(k_cache), _bits(v_cache)
    lens = _lens(seq_lens)
    B, T, Hq, D = qb.shape
    Bk, Lmax, Hkv, Dk = kb.shape
    if vb.shape != kb.shape or Bk != B or Dk != D or lens.shape != (B,):
        raise ValueError("inconsistent shapes q%s k%s v%s lens%s" % (qb.shape, kb.shape, vb.shape, lens.shape))
    out = np.empty((B, T, Hq, D), dtype=np.float64)
    rc = _load().oracle_decode_multi(_ptr(qb, ctypes.c_uint16), _ptr(kb, ctypes.c_uint16),
                                     _ptr(vb, ctypes.c_uint16), _ptr(lens, ctypes.c_int32),
                                     B, T, Hq, Hkv, D, Lmax, float(scale), _ptr(out, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle_decode_multi rejected its arguments (code %d)" % rc)
    return out
