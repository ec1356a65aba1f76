"""CPU oracle for paged decode attention (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The library in
``paged_kv_cache_301_amd`` never imports it, and it never imports the library.

``decode`` wraps the plain fp64 C implementation in ``pa_oracle.c`` (gather the
sequence's blocks through the block table into contiguous K / V, then standard
max-subtracted softmax attention; see that file's header for the passages it
follows).  ``build`` compiles it with gcc.  ``write_kv`` stores new tokens'
rows into their slots; ``block_manager`` holds the free-list / reference-count
/ copy-on-write bookkeeping and the whole-block copy, in plain Python.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
LIB_PATH = os.path.join(_HERE, "libpa_oracle.so")

# Element-type codes understood by the C oracle.
F32, F16, BF16 = 0, 1, 2

_lib = None


def build(verbose: bool = False) -> str:
    """Compile ``pa_oracle.c`` into ``libpa_oracle.so`` (gcc, OpenMP, no fast-math)."""
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
           _SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) or (
                os.path.getmtime(LIB_PATH) < os.path.getmtime(_SRC)):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        lib.oracle_decode.restype = ctypes.c_int
        lib.oracle_decode.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_double, ctypes.c_void_p,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
        lib.oracle_half_to_double.restype = ctypes.c_double
        lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_double.restype = ctypes.c_double
        lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_prefill.restype = ctypes.c_int
        lib.oracle_prefill.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_double, ctypes.c_void_p,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
            ctypes.c_int]
        lib.oracle_write_kv.restype = ctypes.c_longlong
        lib.oracle_write_kv.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 6
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        _lib = lib
    return _lib


def num_threads() -> int:
    """Threads the oracle's OpenMP loop uses."""
    return _load().oracle_num_threads()


def half_to_double(bits: int) -> float:
    return _load().oracle_half_to_double(bits)


def bf16_to_double(bits: int) -> float:
    return _load().oracle_bf16_to_double(bits)


def _dtype_code(t) -> int:
    import torch
    return {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}[t.dtype]


def _host(t):
    """A contiguous CPU tensor (copies device tensors to the host)."""
    return t.detach().to("cpu").contiguous()


def write_kv(key, value, slot_mapping, key_cache, value_cache, inplace=False):
    """Store new tokens' K / V rows into their cache slots (copies of the host
    caches are returned and the inputs are not modified, unless ``inplace``:
    then the caches must be contiguous CPU tensors and are written directly).

    key, value [T,Hkv,D]; slot_mapping [T] int32 (block * B + offset, negative
    to skip); key_cache / value_cache [NB,Hkv,B,D].  Returns
    (new_key_cache, new_value_cache, tokens_written).
    """
    import torch
    k, v = _host(key), _host(value)
    sm = _host(slot_mapping).to(torch.int32)
    if inplace:
        kc, vc = key_cache, value_cache
        if kc.device.type != "cpu" or not (kc.is_contiguous() and vc.is_contiguous()):
            raise ValueError("inplace needs contiguous host caches")
    else:
        kc, vc = _host(key_cache).clone(), _host(value_cache).clone()
    T, Hkv, D = k.shape
    NB, Hkv2, B, D2 = kc.shape
    if (Hkv2, D2) != (Hkv, D) or v.shape != k.shape or vc.shape != kc.shape:
        raise ValueError("shapes do not match")
    if not (k.dtype == v.dtype == kc.dtype == vc.dtype):
        raise TypeError("one element type expected")
    n = _load().oracle_write_kv(k.data_ptr(), v.data_ptr(), sm.data_ptr(), kc.data_ptr(),
                                vc.data_ptr(), T, Hkv, D, B, NB, k.element_size())
    return kc, vc, int(n)


def prefill(query, key_cache, value_cache, block_tables, seq_lens, query_start,
            scale: float, rows=None) -> np.ndarray:
    """fp64 causal attention of several new tokens per sequence.

    query [T,Hq,D] (rows grouped by sequence); query_start [S+1] int32; the
    other arguments as in ``decode`` (seq_lens count the new tokens).  Row
    query_start[s] + k attends tokens 0 .. seq_lens[s] - n_s + k.  Returns
    float64 [T,Hq,D], or [len(rows),D] for flat (t * Hq + h) ``rows``.
    """
    import torch
    q, kc, vc = _host(query), _host(key_cache), _host(value_cache)
    bt = _host(block_tables).to(torch.int32)
    sl = _host(seq_lens).to(torch.int32)
    qs = _host(query_start).to(torch.int32)
    if not (q.dtype == kc.dtype == vc.dtype):
        raise TypeError("query, key_cache and value_cache must share one dtype")
    T, Hq, D = q.shape
    NB, Hkv, B, D2 = kc.shape
    S = sl.shape[0]
    if D2 != D or vc.shape != kc.shape or qs.shape != (S + 1,):
        raise ValueError("shapes do not match")
    max_blocks = bt.shape[1] if bt.dim() == 2 else 0
    if rows is None:
        rows_arr, nrows = None, T * Hq
    else:
        rows_arr = np.ascontiguousarray(np.asarray(list(rows), dtype=np.int32))
        nrows = int(rows_arr.size)
    out = np.zeros((nrows, D), dtype=np.float64)
    rc = _load().oracle_prefill(
        q.data_ptr(), kc.data_ptr(), vc.data_ptr(), bt.data_ptr(), sl.data_ptr(),
        qs.data_ptr(), float(scale), out.ctypes.data, S, T, Hq, Hkv, D, B, NB,
        max_blocks, _dtype_code(q),
        None if rows_arr is None else rows_arr.ctypes.data, nrows)
    if rc != 0:
        raise ValueError(f"oracle_prefill rejected its arguments (code {rc})")
    return out.reshape(T, Hq, D) if rows is None else out


def decode(query, key_cache, value_cache, block_tables, seq_lens, scale: float,
           rows=None) -> np.ndarray:
    """fp64 paged decode attention.

    query [S,Hq,D]; key_cache / value_cache [NB,Hkv,B,D] (fp32, fp16 or bf16,
    all the same type); block_tables [S,max_blocks] int32; seq_lens [S] int32.
    ``rows``: optional iterable of flat (s * Hq + h) row indices to compute.
    Returns float64 numpy array [S,Hq,D], or [len(rows),D] when ``rows`` given.
    Tensors may live on any device; they are copied to the host.
    """
    import torch
    q, kc, vc = _host(query), _host(key_cache), _host(value_cache)
    bt = _host(block_tables).to(torch.int32)
    sl = _host(seq_lens).to(torch.int32)
    if not (q.dtype == kc.dtype == vc.dtype):
        raise TypeError("query, key_cache and value_cache must share one dtype")
    S, Hq, D = q.shape
    NB, Hkv, B, D2 = kc.shape
    if D2 != D or vc.shape != kc.shape:
        raise ValueError("cache shapes do not match the query")
    max_blocks = bt.shape[1] if bt.dim() == 2 else 0
    if rows is None:
        rows_arr = None
        nrows = S * Hq
    else:
        rows_arr = np.ascontiguousarray(np.asarray(list(rows), dtype=np.int32))
        nrows = int(rows_arr.size)
    out = np.zeros((nrows, D), dtype=np.float64)
    rc = _load().oracle_decode(
        q.data_ptr(), kc.data_ptr(), vc.data_ptr(), bt.data_ptr(), sl.data_ptr(),
        float(scale), out.ctypes.data, S, Hq, Hkv, D, B, NB, max_blocks,
        _dtype_code(q),
        None if rows_arr is None else rows_arr.ctypes.data, nrows)
    if rc != 0:
        raise ValueError(f"oracle_decode rejected its arguments (code {rc})")
    return out.reshape(S, Hq, D) if rows is None else out
