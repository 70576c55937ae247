"""Thin Python binding of the C ABI in include/gqa_attn.h (ctypes).

Only argument marshalling lives here: torch tensors are turned into
``gqa_tensor_t`` views (pointer, dtype code, shape, strides) and handed to
``libgqa_attn.so``; every step of the computation runs in the library's HIP
kernels.  PyTorch provides device memory and the current stream.  If the
library has not been built, every call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # imported before the library so both share one HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libgqa_attn.so")

GQA_OK, GQA_ERR_INVALID_ARG, GQA_ERR_UNSUPPORTED, GQA_ERR_WORKSPACE, GQA_ERR_HIP = range(5)
DTYPES = {
    torch.float16: 0,
    torch.bfloat16: 1,
    torch.float8_e4m3fn: 2,
    torch.float32: 3,
    torch.bool: 4,
    torch.uint8: 4,
}
FORMS = {"padded_bhnd": 0, "packed_nhd": 1, "paged": 2}
CAUSAL = {"none": 0, "upper_left": 1, "lower_right": 2}
NORM = {"softmax": 0, "none": 1}
QDQ = {None: 0, "off": 0, "fp8": 1, "int8": 2}


class GqaTensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("ndim", ctypes.c_int32),
        ("shape", ctypes.c_int64 * 4),
        ("stride", ctypes.c_int64 * 4),
    ]


class GqaArgs(ctypes.Structure):
    _fields_ = [
        ("q", GqaTensor),
        ("k", GqaTensor),
        ("v", GqaTensor),
        ("attn_mask", GqaTensor),
        ("out", GqaTensor),
        ("query_lengths", ctypes.c_void_p),
        ("kv_lengths", ctypes.c_void_p),
        ("batch", ctypes.c_int32),
        ("query_form", ctypes.c_int32),
        ("kv_form", ctypes.c_int32),
        ("causal_kind", ctypes.c_int32),
        ("norm", ctypes.c_int32),
        ("qdq", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("qscale", ctypes.c_float),
        ("k_descale", ctypes.c_float),
        ("v_descale", ctypes.c_float),
        ("num_heads", ctypes.c_int32),
        ("kv_num_heads", ctypes.c_int32),
        ("tree_parents", ctypes.c_void_p),
        ("kv_page_table", ctypes.c_void_p),
        ("kv_max_pages", ctypes.c_int32),
    ]


class GqaKvUpdateArgs(ctypes.Structure):
    """gqa_kv_update_args_t (include/gqa_kv_cache.h)."""
    _fields_ = [
        ("past_cache", GqaTensor),
        ("update", GqaTensor),
        ("out", GqaTensor),
        ("write_indices", ctypes.c_void_p),
        ("update_lengths", ctypes.c_void_p),
        ("update_form", ctypes.c_int32),
    ]


class GqaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"gqa_attn: {status_str(status)} ({status}): {detail}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libgqa_attn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -c 'import __graft_entry__ as g; g.build()')")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(GqaArgs)
        lib.gqa_attn_validate.argtypes = [P]
        lib.gqa_attn_validate.restype = ctypes.c_int
        lib.gqa_attn_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
        lib.gqa_attn_workspace_size.restype = ctypes.c_int
        lib.gqa_attn_forward.argtypes = [P, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        lib.gqa_attn_forward.restype = ctypes.c_int
        lib.gqa_attn_status_str.argtypes = [ctypes.c_int]
        lib.gqa_attn_status_str.restype = ctypes.c_char_p
        lib.gqa_attn_last_error.argtypes = []
        lib.gqa_attn_last_error.restype = ctypes.c_char_p
        lib.gqa_attn_last_hip_error.argtypes = []
        lib.gqa_attn_last_hip_error.restype = ctypes.c_int
        lib.gqa_attn_abi_version.argtypes = []
        lib.gqa_attn_abi_version.restype = ctypes.c_int
        lib.gqa_attn_forward_noalloc.argtypes = [P, ctypes.c_void_p]
        lib.gqa_attn_forward_noalloc.restype = ctypes.c_int
        I32 = ctypes.POINTER(ctypes.c_int32)
        lib.gqa_attn_check_lengths.argtypes = [P, I32, I32, I32]
        lib.gqa_attn_check_lengths.restype = ctypes.c_int
        lib.gqa_attn_timer_start.argtypes = [ctypes.c_int]
        lib.gqa_attn_timer_start.restype = ctypes.c_int
        lib.gqa_attn_timer_stop.argtypes = [ctypes.POINTER(ctypes.c_double),
                                            ctypes.POINTER(ctypes.c_int)]
        lib.gqa_attn_timer_stop.restype = ctypes.c_int
        K = ctypes.POINTER(GqaKvUpdateArgs)
        lib.gqa_kv_cache_update_validate.argtypes = [K]
        lib.gqa_kv_cache_update_validate.restype = ctypes.c_int
        lib.gqa_kv_cache_update.argtypes = [K, ctypes.c_void_p]
        lib.gqa_kv_cache_update.restype = ctypes.c_int
        _lib = lib
    return _lib


def status_str(status: int) -> str:
    return load().gqa_attn_status_str(status).decode()


def last_error() -> str:
    return load().gqa_attn_last_error().decode()


def timer_start(max_launches: int) -> int:
    """Open the library's main-kernel timing window (gqa_attn_timer_start)."""
    return load().gqa_attn_timer_start(int(max_launches))


def timer_stop():
    """Close the window: (status, summed main-kernel ms, timed calls)."""
    ms, n = ctypes.c_double(0.0), ctypes.c_int(0)
    st = load().gqa_attn_timer_stop(ctypes.byref(ms), ctypes.byref(n))
    return st, ms.value, n.value


def tensor_view(t: Optional[torch.Tensor]) -> GqaTensor:
    """gqa_tensor_t describing t (an absent tensor when t is None)."""
    v = GqaTensor()
    if t is None:
        v.data = None
        v.ndim = 0
        return v
    if t.dim() > 4:
        raise ValueError("tensors have rank <= 4")
    v.data = t.data_ptr()
    v.dtype = DTYPES[t.dtype]
    v.ndim = t.dim()
    for d in range(t.dim()):
        v.shape[d] = t.shape[d]
        v.stride[d] = t.stride(d)
    return v


def make_args(q, k, v, attn_mask=None, out=None, *, query_lengths=None, kv_lengths=None,
              batch=None, query_form="padded_bhnd", kv_form="padded_bhnd", causal_kind="none",
              norm="softmax", qdq=None, qscale=1.0, scale=1.0, k_descale=1.0, v_descale=1.0,
              num_heads=None, kv_num_heads=None, tree_parents=None,
              kv_page_table=None) -> GqaArgs:
    """Fill a gqa_attn_args_t from tensors (no copies, no checks)."""
    a = GqaArgs()
    a.q, a.k, a.v = tensor_view(q), tensor_view(k), tensor_view(v)
    a.attn_mask = tensor_view(attn_mask)
    a.out = tensor_view(out)
    for name, t in (("query_lengths", query_lengths), ("kv_lengths", kv_lengths),
                    ("tree_parents", tree_parents), ("kv_page_table", kv_page_table)):
        if t is not None and t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32")
        setattr(a, name, None if t is None else t.data_ptr())
    if batch is None:
        if query_form == "padded_bhnd":
            batch = q.shape[0]
        elif kv_form == "padded_bhnd":
            batch = k.shape[0]
        else:
            batch = query_lengths.numel() - 1
    a.batch = batch
    a.kv_max_pages = 0 if kv_page_table is None else kv_page_table.shape[-1]
    a.query_form = FORMS[query_form]
    a.kv_form = FORMS[kv_form]
    a.causal_kind = CAUSAL[causal_kind]
    a.norm = NORM[norm]
    a.qdq = QDQ[qdq]
    a.scale = scale
    a.qscale = qscale
    a.k_descale = k_descale
    a.v_descale = v_descale
    a.num_heads = q.shape[1] if num_heads is None else num_heads
    a.kv_num_heads = k.shape[1] if kv_num_heads is None else kv_num_heads
    return a


def gqa_attn_validate(args: GqaArgs) -> int:
    return load().gqa_attn_validate(ctypes.byref(args))


def gqa_attn_check_lengths(args: GqaArgs, query_lengths=None, kv_lengths=None,
                           kv_page_table=None) -> int:
    """gqa_attn_check_lengths over host copies (numpy int32 arrays or None)
    of the call's length arrays; returns the status code."""
    import numpy as np
    keep = []

    def ptr(x):
        if x is None:
            return None
        a = np.ascontiguousarray(np.asarray(x, dtype=np.int32))
        keep.append(a)
        return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))

    return load().gqa_attn_check_lengths(ctypes.byref(args), ptr(query_lengths), ptr(kv_lengths),
                                         ptr(kv_page_table))


def gqa_attn_workspace_size(args: GqaArgs) -> int:
    n = ctypes.c_size_t(0)
    st = load().gqa_attn_workspace_size(ctypes.byref(args), ctypes.byref(n))
    if st != GQA_OK:
        raise GqaError(st, last_error())
    return n.value


def gqa_attn_forward(args: GqaArgs, workspace: Optional[torch.Tensor], stream) -> None:
    ws_ptr = None if workspace is None else workspace.data_ptr()
    ws_n = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().gqa_attn_forward(ctypes.byref(args), ws_ptr, ws_n, stream)
    if st != GQA_OK:
        raise GqaError(st, last_error())


def gqa_attn_forward_noalloc(args: GqaArgs, stream) -> None:
    """The forward call whose workspace is the library's static buffer."""
    st = load().gqa_attn_forward_noalloc(ctypes.byref(args), stream)
    if st != GQA_OK:
        raise GqaError(st, last_error())


def out_dtype_for(q_dtype: torch.dtype) -> torch.dtype:
    return torch.float16 if q_dtype == torch.float8_e4m3fn else q_dtype


def attn_forward(q, k, v, attn_mask=None, *, out=None, workspace=None, stream=None, **kw):
    """Y = attention(q, k, v, ...) on the current torch stream.

    Keyword arguments are those of make_args.  ``out`` (optional) must have
    q's shape; it is allocated with torch.empty otherwise -- rows that are
    not valid are left as they were.  ``workspace`` is allocated when the
    call needs one and none is given.
    """
    if not q.is_cuda:
        raise ValueError("attn_forward runs on the GPU: pass device tensors")
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype_for(q.dtype), device=q.device)
    args = make_args(q, k, v, attn_mask, out, **kw)
    n = gqa_attn_workspace_size(args)
    if n and (workspace is None or workspace.numel() * workspace.element_size() < n):
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    gqa_attn_forward(args, workspace if n else None, stream)
    return out


# ------------------------------------------------------------ KV-cache update
def make_kv_update_args(past_cache, update, out=None, *, write_indices=None, update_lengths=None,
                        update_form="padded_bhnd") -> GqaKvUpdateArgs:
    """gqa_kv_update_args_t for torch tensors (out = past_cache: in place)."""
    a = GqaKvUpdateArgs()
    a.past_cache = tensor_view(past_cache)
    a.update = tensor_view(update)
    a.out = tensor_view(past_cache if out is None else out)
    a.write_indices = None if write_indices is None else write_indices.data_ptr()
    a.update_lengths = None if update_lengths is None else update_lengths.data_ptr()
    a.update_form = FORMS[update_form]
    a._keep = (past_cache, update, out, write_indices, update_lengths)
    return a


def gqa_kv_cache_update_validate(args: GqaKvUpdateArgs) -> int:
    return load().gqa_kv_cache_update_validate(ctypes.byref(args))


def gqa_kv_cache_update(args: GqaKvUpdateArgs, stream) -> None:
    st = load().gqa_kv_cache_update(ctypes.byref(args), stream)
    if st != GQA_OK:
        raise GqaError(st, last_error())


def kv_cache_update(past_cache, update, *, out=None, write_indices=None, update_lengths=None,
                    update_form="padded_bhnd", stream=None):
    """Y = TRT_KVCacheUpdate(past_cache, update, ...) on the current torch
    stream; in place (Y is past_cache) unless ``out`` is given."""
    if not past_cache.is_cuda:
        raise ValueError("kv_cache_update runs on the GPU: pass device tensors")
    args = make_kv_update_args(past_cache, update, out, write_indices=write_indices,
                               update_lengths=update_lengths, update_form=update_form)
    if stream is None:
        stream = torch.cuda.current_stream(past_cache.device).cuda_stream
    gqa_kv_cache_update(args, stream)
    return past_cache if out is None else out
