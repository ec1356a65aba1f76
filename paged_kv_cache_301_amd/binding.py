"""Python binding of libpa_decode.so (argument marshalling only).

Every step of the computation runs in the library's HIP kernels; this module
checks tensor shapes and types, passes device pointers and the current HIP
stream, and allocates the split plan's workspace with torch when the caller
does not bring one.  It raises if the library is not built: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpa_decode.so")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
HEADER = os.path.join(INCLUDE, "pa_decode.h")

# pa_dtype
PA_F32, PA_F16, PA_BF16 = 0, 1, 2
# pa_status
(PA_OK, PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP,
 PA_ERR_NO_BLOCKS, PA_ERR_BAD_ID, PA_ERR_DEVICE_CHECK, PA_ERR_SCRATCH) = range(10)
# bytes of the static device scratch of pa_decode_noalloc (PA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20
# pa_kernel
KERNEL_AUTO, KERNEL_GENERIC, KERNEL_VALU, KERNEL_MFMA = range(4)
KERNELS = {"auto": KERNEL_AUTO, "generic": KERNEL_GENERIC, "valu": KERNEL_VALU, "mfma": KERNEL_MFMA}
# stages
STAGE_PARTITIONS, STAGE_COMBINE, STAGE_ALL = 1, 2, 3

_TORCH_TO_PA = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}


class PaConfig(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int), ("partition_tokens", ctypes.c_int),
                ("stages", ctypes.c_int), ("kv_reuse", ctypes.c_int), ("check", ctypes.c_int),
                ("token_waves", ctypes.c_int)]


class PaPlan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int), ("partition_tokens", ctypes.c_int),
                ("max_partitions", ctypes.c_int), ("split", ctypes.c_int),
                ("workspace_bytes", ctypes.c_size_t), ("token_waves", ctypes.c_int)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class PaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lib = None

_INT = ctypes.c_int
_PTR = ctypes.c_void_p
_SHAPE = [_INT] * 7 + [_INT, _INT]       # S Hq Hkv D B NB max_blocks dtype out_dtype


def load():
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_301_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.pa_decode_plan.restype = _INT
    lib.pa_decode_plan.argtypes = _SHAPE + [ctypes.POINTER(PaConfig), ctypes.POINTER(PaPlan)]
    lib.pa_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.pa_decode_workspace_bytes.argtypes = list(_SHAPE)
    tensors = [_PTR, _PTR, _PTR, _PTR, _PTR, ctypes.c_float, _PTR]
    lib.pa_decode.restype = _INT
    lib.pa_decode.argtypes = tensors + _SHAPE + [_PTR, ctypes.c_size_t, _PTR]
    lib.pa_decode_ex.restype = _INT
    lib.pa_decode_ex.argtypes = tensors + _SHAPE + [ctypes.POINTER(PaConfig), _PTR,
                                                    ctypes.c_size_t, _PTR]
    lib.pa_write_kv.restype = _INT
    lib.pa_write_kv.argtypes = [_PTR] * 5 + [_INT] * 6 + [_PTR]
    lib.pa_append_kv.restype = _INT
    lib.pa_append_kv.argtypes = [_PTR] * 6 + [_INT] * 7 + [_PTR]
    mq_shape = [_INT] * 9 + [_INT, _INT]  # S T Hq Hkv D B NB max_blocks max_query_len dtype out_dtype
    lib.pa_prefill_plan.restype = _INT
    lib.pa_prefill_plan.argtypes = mq_shape + [ctypes.POINTER(PaConfig), ctypes.POINTER(PaPlan)]
    lib.pa_prefill.restype = _INT
    lib.pa_prefill.argtypes = ([_PTR] * 6 + [ctypes.c_float, _PTR] + mq_shape +
                               [ctypes.POINTER(PaConfig), _PTR, ctypes.c_size_t, _PTR])
    lib.pa_decode_noalloc.restype = _INT
    lib.pa_decode_noalloc.argtypes = tensors + _SHAPE + [ctypes.POINTER(PaConfig), _PTR]
    lib.pa_check_inputs.restype = _INT
    lib.pa_check_inputs.argtypes = [_PTR, _PTR] + [_INT] * 4 + [_PTR, _PTR]
    lib.pa_get_device_error.restype = _INT
    lib.pa_get_device_error.argtypes = [_PTR, ctypes.POINTER(ctypes.c_int32)]
    lib.pa_copy_blocks.restype = _INT
    lib.pa_copy_blocks.argtypes = [_PTR] * 3 + [_INT] * 6 + [_PTR]
    lib.pa_read_bytes.restype = _INT
    lib.pa_read_bytes.argtypes = [_PTR, ctypes.c_size_t, _PTR, _PTR]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_status_string.argtypes = [_INT]
    # host block pool
    P, I32P = _PTR, ctypes.POINTER(ctypes.c_int32)
    IP = ctypes.POINTER(_INT)
    for name, res, args in [
            ("pa_pool_create", _INT, [_INT, _INT, I32P, ctypes.POINTER(_PTR)]),
            ("pa_pool_destroy", None, [P]),
            ("pa_pool_num_free", _INT, [P]),
            ("pa_pool_refcount", _INT, [P, _INT]),
            ("pa_seq_create", _INT, [P, IP]),
            ("pa_seq_fork", _INT, [P, _INT, IP]),
            ("pa_seq_append", _INT, [P, _INT, _INT, I32P, I32P, I32P]),
            ("pa_seq_append_batch", _INT, [P, IP, _INT, I32P, I32P, IP]),
            ("pa_seq_release", _INT, [P, _INT]),
            ("pa_seq_length", _INT, [P, _INT]),
            ("pa_seq_num_blocks", _INT, [P, _INT]),
            ("pa_pool_export", _INT, [P, IP, _INT, _INT, ctypes.c_int32, I32P, I32P])]:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def header_functions():
    """Names of the functions the headers under include/ declare."""
    import glob
    names = set()
    for path in sorted(glob.glob(os.path.join(INCLUDE, "*.h"))):
        text = open(path).read()
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(pa_\w+)\s*\(", text, re.M))
    return sorted(names)


def status_string(status: int) -> str:
    return load().pa_status_string(status).decode()


class InputCheckError(PaError, ValueError):
    """The library's device check found lengths or block-table entries that
    violate the documented preconditions; nothing was launched."""


def _check(status: int):
    if status == PA_ERR_DEVICE_CHECK:
        raise InputCheckError(status, status_string(status))
    if status != PA_OK:
        raise PaError(status, status_string(status))


def _check_flag(check) -> int:
    """pa_config.check: None leaves it to the PA_CHECK environment variable
    (read by the library at every call), True / False force it."""
    return 0 if check is None else (1 if check else -1)


def _config(kernel="auto", partition_tokens=0, stages=0, kv_reuse=False, check=None,
            token_waves=None) -> PaConfig:
    """The C config.  Choices left to the library (kernel "auto", partition 0)
    take the PA_KERNEL (auto / generic / valu / mfma) and PA_PARTITION_TOKENS
    environment variables when those are set, and decode token-waves (None)
    PA_TOKEN_WAVES; explicit arguments win.  The multi-token calls pass
    token_waves=0."""
    if isinstance(kernel, str) and kernel == "auto":
        kernel = os.environ.get("PA_KERNEL", "auto") or "auto"
    if not partition_tokens:
        partition_tokens = int(os.environ.get("PA_PARTITION_TOKENS", "0") or 0)
    if token_waves is None:
        token_waves = int(os.environ.get("PA_TOKEN_WAVES", "0") or 0)
    if isinstance(kernel, str) and kernel not in KERNELS:
        raise ValueError(f"unknown kernel {kernel!r} (one of {sorted(KERNELS)})")
    k = KERNELS[kernel] if isinstance(kernel, str) else int(kernel)
    return PaConfig(k, int(partition_tokens), int(stages), int(bool(kv_reuse)), _check_flag(check),
                    int(token_waves))


def _shape_args(query, key_cache, block_tables, out_dtype):
    S, Hq, D = query.shape
    NB, Hkv, B, D2 = key_cache.shape
    if D2 != D:
        raise ValueError("query and cache head sizes differ")
    max_blocks = block_tables.shape[1]
    return (S, Hq, Hkv, D, B, NB, max_blocks, _TORCH_TO_PA[query.dtype], _TORCH_TO_PA[out_dtype])


def plan(S, Hq, Hkv, D, B, NB, max_blocks, dtype, out_dtype=None, *, kernel="auto",
         partition_tokens=0, stages=0, kv_reuse=False, token_waves=None) -> dict:
    """Resolve the plan for a shape (host only; no GPU needed)."""
    dt = _TORCH_TO_PA.get(dtype, dtype)
    odt = dt if out_dtype is None else _TORCH_TO_PA.get(out_dtype, out_dtype)
    p = PaPlan()
    cfg = _config(kernel, partition_tokens, stages, kv_reuse, token_waves=token_waves)
    _check(load().pa_decode_plan(S, Hq, Hkv, D, B, NB, max_blocks, dt, odt,
                                 ctypes.byref(cfg), ctypes.byref(p)))
    return p.as_dict()


def decode(query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
           block_tables: torch.Tensor, seq_lens: torch.Tensor, scale: float,
           out: Optional[torch.Tensor] = None, *, out_dtype: Optional[torch.dtype] = None,
           kernel="auto", partition_tokens: int = 0, stages: int = 0, kv_reuse: bool = False,
           workspace: Optional[torch.Tensor] = None, stream=None,
           check: Optional[bool] = None, token_waves: Optional[int] = None) -> torch.Tensor:
    """Paged decode attention: out[S,Hq,D] from query[S,Hq,D], K/V pools
    [NB,Hkv,B,D], block_tables[S,max_blocks] int32 and seq_lens[S] int32.

    All tensors must be contiguous and on the same GPU.  Asynchronous on
    ``stream`` (default: torch's current stream); ``out`` and the workspace,
    when this function allocates them, are allocated on that stream.
    ``check`` (default None: the library follows the PA_CHECK environment
    variable) makes the library verify the lengths and table entries on the
    device first; it raises InputCheckError instead of launching (the checked
    call synchronises the stream).
    """
    lib = load()
    for name, t in (("query", query), ("key_cache", key_cache), ("value_cache", value_cache),
                    ("block_tables", block_tables), ("seq_lens", seq_lens)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_tables and seq_lens must be int32")
    if not (query.dtype == key_cache.dtype == value_cache.dtype):
        raise TypeError("query, key_cache and value_cache must share one dtype")
    if value_cache.shape != key_cache.shape:
        raise ValueError("key_cache and value_cache shapes differ")
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else query.dtype
    if out is not None and (out.shape != query.shape or out.dtype != out_dtype
                            or not out.is_contiguous()):
        raise ValueError("out must be a contiguous [S,Hq,D] tensor of out_dtype")
    shape = _shape_args(query, key_cache, block_tables, out_dtype)
    if seq_lens.shape != (shape[0],) or block_tables.shape[0] != shape[0]:
        raise ValueError("seq_lens / block_tables do not match the batch size")
    cfg = _config(kernel, partition_tokens, stages, kv_reuse, check, token_waves)
    p = PaPlan()
    _check(lib.pa_decode_plan(*shape, ctypes.byref(cfg), ctypes.byref(p)))
    tstream = _torch_stream(stream, query.device)
    with torch.cuda.stream(tstream):
        # allocated on the launch stream: the caching allocator then orders
        # any reuse of these blocks after the kernels that use them
        if out is None:
            out = torch.empty(query.shape, dtype=out_dtype, device=query.device)
        if p.workspace_bytes and workspace is None:
            workspace = torch.empty(p.workspace_bytes, dtype=torch.uint8, device=query.device)
    ws_ptr, ws_bytes = None, 0
    if p.workspace_bytes:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    st = tstream.cuda_stream
    _check(lib.pa_decode_ex(query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
                            block_tables.data_ptr(), seq_lens.data_ptr(), float(scale),
                            out.data_ptr(), *shape, ctypes.byref(cfg), ws_ptr, ws_bytes, st))
    return out


def decode_noalloc(query, key_cache, value_cache, block_tables, seq_lens, scale, out, *,
                   kernel="auto", partition_tokens=0, stages=0, kv_reuse=False, stream=None,
                   check: Optional[bool] = None, token_waves: Optional[int] = None) -> torch.Tensor:
    """``decode`` through pa_decode_noalloc: the split plan's partial results
    go to the library's static device scratch, and nothing is allocated here
    either (``out`` must be given).  Calls that overlap on one GPU race for
    the scratch."""
    lib = load()
    for name, t in (("query", query), ("key_cache", key_cache), ("value_cache", value_cache),
                    ("block_tables", block_tables), ("seq_lens", seq_lens), ("out", out)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_tables and seq_lens must be int32")
    if not (query.dtype == key_cache.dtype == value_cache.dtype):
        raise TypeError("query, key_cache and value_cache must share one dtype")
    if value_cache.shape != key_cache.shape or out.shape != query.shape:
        raise ValueError("cache or output shapes do not match")
    shape = _shape_args(query, key_cache, block_tables, out.dtype)
    if seq_lens.shape != (shape[0],) or block_tables.shape[0] != shape[0]:
        raise ValueError("seq_lens / block_tables do not match the batch size")
    cfg = _config(kernel, partition_tokens, stages, kv_reuse, check, token_waves)
    _check(lib.pa_decode_noalloc(query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
                                 block_tables.data_ptr(), seq_lens.data_ptr(), float(scale),
                                 out.data_ptr(), *shape, ctypes.byref(cfg),
                                 _stream_handle(stream, query.device)))
    return out


def plan_prefill(S, T, Hq, Hkv, D, B, NB, max_blocks, max_query_len, dtype, out_dtype=None, *,
                 kernel="auto", partition_tokens=0, stages=0, kv_reuse=False) -> dict:
    """Resolve the plan of a multi-token causal call (host only)."""
    dt = _TORCH_TO_PA.get(dtype, dtype)
    odt = dt if out_dtype is None else _TORCH_TO_PA.get(out_dtype, out_dtype)
    p = PaPlan()
    cfg = _config(kernel, partition_tokens, stages, kv_reuse, token_waves=0)
    _check(load().pa_prefill_plan(S, T, Hq, Hkv, D, B, NB, max_blocks, max_query_len, dt, odt,
                                  ctypes.byref(cfg), ctypes.byref(p)))
    return p.as_dict()


def prefill(query, key_cache, value_cache, block_tables, seq_lens, query_start, scale,
            out=None, *, max_query_len: Optional[int] = None, out_dtype=None, kernel="auto",
            partition_tokens: int = 0, stages: int = 0, kv_reuse: bool = False,
            workspace=None, stream=None, check: Optional[bool] = None) -> torch.Tensor:
    """Causal attention of several new tokens per sequence: out[T,Hq,D] from
    query[T,Hq,D] (rows grouped by sequence, query_start[S+1] int32), the
    paged K/V pools and block_tables / seq_lens (lengths count the new
    tokens).  ``max_query_len`` (the largest n_s) is read back from
    query_start when not given, which synchronises the stream.  ``check`` as
    in ``decode``; ``out`` and the workspace, when allocated here, are
    allocated on the launch stream."""
    lib = load()
    for name, t in (("query", query), ("key_cache", key_cache), ("value_cache", value_cache),
                    ("block_tables", block_tables), ("seq_lens", seq_lens),
                    ("query_start", query_start)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    for t in (block_tables, seq_lens, query_start):
        if t.dtype != torch.int32:
            raise TypeError("block_tables, seq_lens and query_start must be int32")
    if not (query.dtype == key_cache.dtype == value_cache.dtype):
        raise TypeError("query, key_cache and value_cache must share one dtype")
    if value_cache.shape != key_cache.shape:
        raise ValueError("key_cache and value_cache shapes differ")
    S = seq_lens.shape[0]
    if query_start.shape != (S + 1,) or block_tables.shape[0] != S:
        raise ValueError("query_start / block_tables do not match seq_lens")
    T, Hq, D = query.shape
    NB, Hkv, B, D2 = key_cache.shape
    if D2 != D:
        raise ValueError("query and cache head sizes differ")
    if max_query_len is None:
        max_query_len = int((query_start[1:] - query_start[:-1]).max().item()) if S else 0
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else query.dtype
    if out is not None and (out.shape != query.shape or out.dtype != out_dtype
                            or not out.is_contiguous()):
        raise ValueError("out must be a contiguous [T,Hq,D] tensor of out_dtype")
    shape = (S, T, Hq, Hkv, D, B, NB, block_tables.shape[1], int(max_query_len),
             _TORCH_TO_PA[query.dtype], _TORCH_TO_PA[out_dtype])
    cfg = _config(kernel, partition_tokens, stages, kv_reuse, check, 0)
    p = PaPlan()
    _check(lib.pa_prefill_plan(*shape, ctypes.byref(cfg), ctypes.byref(p)))
    tstream = _torch_stream(stream, query.device)
    with torch.cuda.stream(tstream):
        if out is None:
            out = torch.empty(query.shape, dtype=out_dtype, device=query.device)
        if p.workspace_bytes and workspace is None:
            workspace = torch.empty(p.workspace_bytes, dtype=torch.uint8, device=query.device)
    ws_ptr, ws_bytes = None, 0
    if p.workspace_bytes:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check(lib.pa_prefill(query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
                          block_tables.data_ptr(), seq_lens.data_ptr(), query_start.data_ptr(),
                          float(scale), out.data_ptr(), *shape, ctypes.byref(cfg), ws_ptr,
                          ws_bytes, tstream.cuda_stream))
    return out


def prefill_workload(pw, **kw) -> torch.Tensor:
    """``prefill`` on a PrefillWorkload (see workloads.make_prefill_workload)."""
    w = pw.base
    return prefill(pw.query, w.key_cache, w.value_cache, w.block_tables, w.seq_lens,
                   pw.query_start, w.scale, max_query_len=pw.max_query_len, **kw)


def check_inputs(block_tables, seq_lens, num_blocks: int, block_size: int, stream=None):
    """Run the device check of lengths and used table entries; returns
    (number of offending sequences, smallest offending index or None).
    Synchronises the stream."""
    lib = load()
    if not (block_tables.is_cuda and seq_lens.is_cuda):
        raise ValueError("tensors must be on the GPU")
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_tables and seq_lens must be int32")
    if not (block_tables.is_contiguous() and seq_lens.is_contiguous()):
        raise ValueError("tensors must be contiguous")
    S = seq_lens.shape[0]
    if block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must be [S, max_blocks]")
    report = torch.empty(2, dtype=torch.int32, device=seq_lens.device)
    st = _stream_handle(stream, seq_lens.device)
    _check(lib.pa_check_inputs(block_tables.data_ptr(), seq_lens.data_ptr(), S,
                               block_tables.shape[1], block_size, num_blocks,
                               report.data_ptr(), st))
    bad, first = report.cpu().tolist()
    return bad, (first if bad else None)


def device_error(stream=None):
    """The library's sticky device-check result on the stream's device:
    (status, smallest offending sequence or None).  Reading clears it;
    synchronises the stream."""
    first = ctypes.c_int32(-1)
    st = load().pa_get_device_error(_stream_handle(stream, None), ctypes.byref(first))
    if st not in (PA_OK, PA_ERR_DEVICE_CHECK):
        _check(st)
    return st, (first.value if first.value >= 0 else None)


def _torch_stream(stream, device):
    """A torch stream object for ``stream`` (None: the current stream of
    ``device``; a raw hipStream_t handle is wrapped as an external stream)."""
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def _stream_handle(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check_kv_pair(key, value, key_cache, value_cache):
    for name, t in (("key", key), ("value", value), ("key_cache", key_cache),
                    ("value_cache", value_cache)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if not (key.dtype == value.dtype == key_cache.dtype == value_cache.dtype):
        raise TypeError("key, value and the caches must share one dtype")
    if key.shape != value.shape or key_cache.shape != value_cache.shape:
        raise ValueError("key/value or cache shapes differ")
    if key.dim() != 3 or key_cache.dim() != 4 or key.shape[1:] != (key_cache.shape[1], key_cache.shape[3]):
        raise ValueError("key must be [T,Hkv,D] and the caches [NB,Hkv,B,D]")


def write_kv(key, value, slot_mapping, key_cache, value_cache, stream=None):
    """Store key/value [T,Hkv,D] into their cache slots (slot_mapping [T] int32:
    block * B + offset, negative to skip).  In place on the caches."""
    lib = load()
    _check_kv_pair(key, value, key_cache, value_cache)
    if slot_mapping.dtype != torch.int32 or slot_mapping.shape != (key.shape[0],) or not slot_mapping.is_cuda:
        raise ValueError("slot_mapping must be a GPU int32 tensor [T]")
    T, Hkv, D = key.shape
    NB, _, B, _ = key_cache.shape
    _check(lib.pa_write_kv(key.data_ptr(), value.data_ptr(), slot_mapping.data_ptr(),
                           key_cache.data_ptr(), value_cache.data_ptr(), T, Hkv, D, B, NB,
                           _TORCH_TO_PA[key.dtype], _stream_handle(stream, key.device)))


def append_kv(key, value, block_tables, seq_lens, key_cache, value_cache, stream=None):
    """Decode-step write: sequence s's new token (the last of its seq_lens[s]
    tokens) from key/value [S,Hkv,D] into its slot.  In place on the caches."""
    lib = load()
    _check_kv_pair(key, value, key_cache, value_cache)
    S, Hkv, D = key.shape
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_tables and seq_lens must be int32")
    if block_tables.shape[0] != S or seq_lens.shape != (S,):
        raise ValueError("block_tables / seq_lens do not match the batch")
    NB, _, B, _ = key_cache.shape
    _check(lib.pa_append_kv(key.data_ptr(), value.data_ptr(), block_tables.data_ptr(),
                            seq_lens.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
                            S, Hkv, D, B, NB, block_tables.shape[1], _TORCH_TO_PA[key.dtype],
                            _stream_handle(stream, key.device)))


def copy_blocks(key_cache, value_cache, pairs, stream=None):
    """Copy whole blocks src -> dst in both caches (pairs: GPU int32 [n,2]).
    In place on the caches."""
    lib = load()
    if key_cache.shape != value_cache.shape or key_cache.dtype != value_cache.dtype:
        raise ValueError("key_cache and value_cache must match")
    if not (key_cache.is_cuda and value_cache.is_cuda and pairs.is_cuda):
        raise ValueError("tensors must be on the GPU")
    if key_cache.dim() != 4 or not (key_cache.is_contiguous() and value_cache.is_contiguous()):
        raise ValueError("caches must be contiguous [NB,Hkv,B,D]")
    if pairs.dtype != torch.int32 or pairs.dim() != 2 or pairs.shape[1] != 2 or not pairs.is_contiguous():
        raise ValueError("pairs must be a contiguous int32 [n,2] tensor")
    NB, Hkv, B, D = key_cache.shape
    _check(lib.pa_copy_blocks(key_cache.data_ptr(), value_cache.data_ptr(), pairs.data_ptr(),
                              pairs.shape[0], Hkv, D, B, NB, _TORCH_TO_PA[key_cache.dtype],
                              _stream_handle(stream, key_cache.device)))


def read_bytes(buf: torch.Tensor, sink: torch.Tensor, stream=None):
    """Stream the bytes of a contiguous GPU tensor through the library's plain
    read kernel once (the achievable-read reference); sink: a GPU tensor of at
    least 4 bytes that the kernel may write."""
    lib = load()
    if not (buf.is_cuda and sink.is_cuda):
        raise ValueError("tensors must be on the GPU")
    if not buf.is_contiguous() or sink.numel() * sink.element_size() < 4:
        raise ValueError("buf must be contiguous and sink at least 4 bytes")
    _check(lib.pa_read_bytes(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(),
                             _stream_handle(stream, buf.device)))


class BlockPool:
    """Host block pool of the library (free stack, reference counts, block
    tables, copy-on-write).  Thin wrapper: every operation is one C call."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        self._lib = load()
        h = ctypes.c_void_p()
        order = None
        if free_order is not None:
            if len(free_order) != num_blocks:
                raise ValueError("free_order must list every block once")
            order = (ctypes.c_int32 * num_blocks)(*[int(b) for b in free_order])
        _check(self._lib.pa_pool_create(num_blocks, block_size, order, ctypes.byref(h)))
        self._h = h
        self.num_blocks, self.block_size = num_blocks, block_size

    def close(self):
        if self._h:
            self._lib.pa_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def num_free(self) -> int:
        return self._lib.pa_pool_num_free(self._h)

    def refcount(self, block: int) -> int:
        return self._lib.pa_pool_refcount(self._h, block)

    def create(self) -> int:
        sid = ctypes.c_int()
        _check(self._lib.pa_seq_create(self._h, ctypes.byref(sid)))
        return sid.value

    def fork(self, parent: int) -> int:
        sid = ctypes.c_int()
        _check(self._lib.pa_seq_fork(self._h, parent, ctypes.byref(sid)))
        return sid.value

    def append(self, seq: int, n: int = 1):
        """Slots for the next n tokens and the copy-on-write pair (or None)."""
        slots = (ctypes.c_int32 * max(n, 1))()
        src, dst = ctypes.c_int32(), ctypes.c_int32()
        _check(self._lib.pa_seq_append(self._h, seq, n, slots, ctypes.byref(src), ctypes.byref(dst)))
        return list(slots[:n]), (None if src.value < 0 else (src.value, dst.value))

    def append_batch(self, seqs):
        """One new token per sequence: (slots, [(src, dst), ...])."""
        n = len(seqs)
        ids = (ctypes.c_int * max(n, 1))(*seqs)
        slots = (ctypes.c_int32 * max(n, 1))()
        pairs = (ctypes.c_int32 * max(2 * n, 2))()
        npairs = ctypes.c_int()
        _check(self._lib.pa_seq_append_batch(self._h, ids, n, slots, pairs, ctypes.byref(npairs)))
        k = npairs.value
        return list(slots[:n]), [(pairs[2 * i], pairs[2 * i + 1]) for i in range(k)]

    def release(self, seq: int):
        _check(self._lib.pa_seq_release(self._h, seq))

    def length(self, seq: int) -> int:
        return self._lib.pa_seq_length(self._h, seq)

    def num_blocks_of(self, seq: int) -> int:
        return self._lib.pa_seq_num_blocks(self._h, seq)

    def export(self, seqs, max_blocks: int, pad: int = 0):
        """Block tables [n][max_blocks] and lengths [n] (host int32 tensors)."""
        n = len(seqs)
        tables = torch.empty((n, max_blocks), dtype=torch.int32)
        lens = torch.empty((n,), dtype=torch.int32)
        ids = (ctypes.c_int * max(n, 1))(*seqs)
        I32P = ctypes.POINTER(ctypes.c_int32)
        _check(self._lib.pa_pool_export(self._h, ids, n, max_blocks, pad,
                                        ctypes.cast(tables.data_ptr(), I32P),
                                        ctypes.cast(lens.data_ptr(), I32P)))
        return tables, lens


class PreparedCall:
    """A decode call with every argument marshalled once, for tight loops
    (benchmarks, graph-free serving loops): calling it only crosses the C ABI.

    The tensors passed to ``prepare`` must stay alive and unmoved."""

    def __init__(self, fn, args):
        self._fn = fn
        self._args = args

    def __call__(self):
        _check(self._fn(*self._args))


def prepare(query, key_cache, value_cache, block_tables, seq_lens, scale, out, *,
            kernel="auto", partition_tokens=0, stages=0, kv_reuse=False, workspace=None,
            stream=None, check: Optional[bool] = None,
            token_waves: Optional[int] = None) -> PreparedCall:
    """Validate once (by running the same checks as ``decode`` on a plan) and
    return a PreparedCall that launches the configured stage(s).  ``check``
    as in ``decode``: the library's device check then runs at every call."""
    lib = load()
    shape = _shape_args(query, key_cache, block_tables, out.dtype)
    cfg = _config(kernel, partition_tokens, stages, kv_reuse, check, token_waves)
    p = PaPlan()
    _check(lib.pa_decode_plan(*shape, ctypes.byref(cfg), ctypes.byref(p)))
    if p.workspace_bytes and workspace is None:
        raise ValueError("this plan needs a workspace")
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if stream is None:
        stream = torch.cuda.current_stream(query.device)
    st = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    args = (query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
            block_tables.data_ptr(), seq_lens.data_ptr(), ctypes.c_float(scale),
            out.data_ptr(), *shape, ctypes.pointer(cfg), ws_ptr, ctypes.c_size_t(ws_bytes), st)
    return PreparedCall(lib.pa_decode_ex, args)


def decode_workload(w, out_dtype=None, **kw) -> torch.Tensor:
    """decode() on a ``workloads.Workload``."""
    return decode(w.query, w.key_cache, w.value_cache, w.block_tables, w.seq_lens, w.scale,
                  out_dtype=out_dtype, **kw)
