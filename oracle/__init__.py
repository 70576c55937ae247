"""CPU oracle for the fused ragged GQA attention operator -- test infrastructure.

Only the test-suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package.  The product library never does,
and this package imports nothing from the product.

The arithmetic lives in ``gqa_oracle.c`` (plain C, fp64, OpenMP over output
rows); this module only compiles it with gcc and marshals host tensors.
The operator follows the onnx-tensorrt "TensorRT Custom Operator Schemas"
page, sections TRT_Attention and TRT_QuantizedAttention.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gqa_oracle.c")
_LIB = os.path.join(_HERE, "_build", "liboracle.so")

# dtype codes private to the oracle (mirror the enum in gqa_oracle.c)
_DT = {
    torch.float16: 0,
    torch.bfloat16: 1,
    torch.float8_e4m3fn: 2,
    torch.float32: 3,
    torch.bool: 4,
    torch.uint8: 4,
    torch.float64: 5,
}
FORMS = {"padded_bhnd": 0, "packed_nhd": 1, "paged": 2}
CAUSAL = {"none": 0, "upper_left": 1, "lower_right": 2}
NORM = {"softmax": 0, "none": 1}
QDQ = {None: 0, "off": 0, "fp8": 1, "int8": 2}


class _Tensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("ndim", ctypes.c_int32),
        ("shape", ctypes.c_int64 * 4),
        ("stride", ctypes.c_int64 * 4),
    ]


class _Args(ctypes.Structure):
    _fields_ = [
        ("q", _Tensor),
        ("k", _Tensor),
        ("v", _Tensor),
        ("mask", _Tensor),
        ("query_form", ctypes.c_int32),
        ("kv_form", ctypes.c_int32),
        ("query_lengths", ctypes.c_void_p),
        ("kv_lengths", ctypes.c_void_p),
        ("batch", ctypes.c_int32),
        ("causal_kind", ctypes.c_int32),
        ("norm", ctypes.c_int32),
        ("qdq", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("qscale", ctypes.c_float),
        ("k_descale", ctypes.c_float),
        ("v_descale", ctypes.c_float),
        ("num_heads", ctypes.c_int32),
        ("kv_num_heads", ctypes.c_int32),
        ("amb_rel", ctypes.c_double),
        ("tree_parents", ctypes.c_void_p),
        ("kv_page_table", ctypes.c_void_p),
        ("kv_max_pages", ctypes.c_int32),
    ]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into oracle/_build/liboracle.so."""
    os.makedirs(os.path.dirname(_LIB), exist_ok=True)
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        lib.oracle_rows.restype = ctypes.c_int
        lib.oracle_rows.argtypes = [
            ctypes.POINTER(_Args), ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ]
        lib.oracle_count_rows.restype = ctypes.c_int64
        lib.oracle_count_rows.argtypes = [ctypes.POINTER(_Args)]
        lib.oracle_list_rows.restype = ctypes.c_int64
        lib.oracle_list_rows.argtypes = [ctypes.POINTER(_Args), ctypes.c_void_p, ctypes.c_int64]
        lib.oracle_decode.restype = ctypes.c_double
        lib.oracle_decode.argtypes = [ctypes.c_int32, ctypes.c_uint32]
        lib.oracle_quantize.restype = ctypes.c_double
        lib.oracle_quantize.argtypes = [
            ctypes.c_int32, ctypes.c_double, ctypes.c_double, ctypes.POINTER(ctypes.c_double)
        ]
        _lib = lib
    return _lib


def _tensor(t: torch.Tensor | None, keep: list) -> _Tensor:
    out = _Tensor()
    if t is None:
        out.data = None
        out.ndim = 0
        return out
    if t.device.type != "cpu":
        raise ValueError("oracle inputs must be host tensors")
    if t.dim() > 4:
        raise ValueError("rank > 4")
    keep.append(t)
    out.data = t.data_ptr()
    out.dtype = _DT[t.dtype]
    out.ndim = t.dim()
    for d in range(t.dim()):
        out.shape[d] = t.shape[d]
        out.stride[d] = t.stride(d)
    return out


@dataclass
class OracleResult:
    rows: np.ndarray      # [R, 3] int32 (b, h, i)
    out: np.ndarray       # [R, D] float64
    amb: np.ndarray       # [R, D] float64 ambiguity bound
    nallowed: np.ndarray  # [R] int64


def _args(q, k, v, mask, query_lengths, kv_lengths, batch, query_form, kv_form, causal_kind,
          norm, qdq, qscale, scale, k_descale, v_descale, num_heads, kv_num_heads, amb_rel, keep):
    a = _Args()
    a.q, a.k, a.v = _tensor(q, keep), _tensor(k, keep), _tensor(v, keep)
    a.mask = _tensor(mask, keep)
    a.query_form = FORMS[query_form]
    a.kv_form = FORMS[kv_form]
    for name in ("query_lengths", "kv_lengths"):
        t = query_lengths if name == "query_lengths" else kv_lengths
        if t is None:
            setattr(a, name, None)
        else:
            t = t.to("cpu", torch.int32).contiguous()
            keep.append(t)
            setattr(a, name, t.data_ptr())
    if batch is None:
        if query_form == "padded_bhnd":
            batch = q.shape[0]
        elif kv_form == "padded_bhnd":
            batch = k.shape[0]
        else:
            batch = query_lengths.numel() - 1
    a.batch = batch
    a.causal_kind = CAUSAL[causal_kind]
    a.norm = NORM[norm]
    a.qdq = QDQ[qdq]
    a.scale = scale
    a.qscale = qscale
    a.k_descale = k_descale
    a.v_descale = v_descale
    a.num_heads = num_heads
    a.kv_num_heads = kv_num_heads
    a.amb_rel = amb_rel
    a.tree_parents = None
    a.kv_page_table = None
    a.kv_max_pages = 0
    return a


def list_rows(q, k, v, *, query_lengths=None, kv_lengths=None, batch=None,
              query_form="padded_bhnd", kv_form="padded_bhnd", num_heads=None,
              kv_num_heads=None) -> np.ndarray:
    """Every valid output row (b, h, i) of the operator, as an [R, 3] int32 array."""
    keep: list = []
    a = _args(q, k, v, None, query_lengths, kv_lengths, batch, query_form, kv_form, "none",
              "softmax", None, 1.0, 1.0, 1.0, 1.0, num_heads, kv_num_heads, 0.0, keep)
    lib = _load()
    n = lib.oracle_count_rows(ctypes.byref(a))
    rows = np.zeros((max(n, 1), 3), dtype=np.int32)
    lib.oracle_list_rows(ctypes.byref(a), rows.ctypes.data, n)
    return rows[:n]


def attention(q, k, v, mask=None, *, query_lengths=None, kv_lengths=None, batch=None,
              query_form="padded_bhnd", kv_form="padded_bhnd", causal_kind="none",
              norm="softmax", qdq=None, qscale=1.0, scale=1.0, k_descale=1.0, v_descale=1.0,
              num_heads=None, kv_num_heads=None, rows=None, amb_rel=1e-5,
              tree_parents=None, kv_page_table=None) -> OracleResult:
    """Evaluate the operator on host tensors (raw storage dtypes).

    ``rows`` selects output rows (b, h, i); default is every valid row.
    ``num_heads`` / ``kv_num_heads`` default to Q's / K's head dimension.
    ``tree_parents``: int32 parent index of each query row's draft token
    (token-aligned with Q's rows: [T_q] packed, [B, N_q] padded), or None.
    ``kv_page_table``: int32 [B, 2, max_pages] for kv_form "paged" (K and V
    are then page pools [P, H_kv, page_size, D]).
    """
    if num_heads is None:
        num_heads = q.shape[1]
    if kv_num_heads is None:
        kv_num_heads = k.shape[1]
    keep: list = []
    a = _args(q, k, v, mask, query_lengths, kv_lengths, batch, query_form, kv_form, causal_kind,
              norm, qdq, qscale, scale, k_descale, v_descale, num_heads, kv_num_heads, amb_rel,
              keep)
    if tree_parents is not None:
        tp = torch.as_tensor(tree_parents).to("cpu", torch.int32).contiguous()
        keep.append(tp)
        a.tree_parents = tp.data_ptr()
    if kv_page_table is not None:
        pt = torch.as_tensor(kv_page_table).to("cpu", torch.int32).contiguous()
        keep.append(pt)
        a.kv_page_table = pt.data_ptr()
        a.kv_max_pages = pt.shape[-1]
    lib = _load()
    if rows is None:
        n = lib.oracle_count_rows(ctypes.byref(a))
        rows = np.zeros((max(n, 1), 3), dtype=np.int32)
        lib.oracle_list_rows(ctypes.byref(a), rows.ctypes.data, n)
        rows = rows[:n]
    rows = np.ascontiguousarray(rows, dtype=np.int32).reshape(-1, 3)
    D = q.shape[-1]
    out = np.zeros((rows.shape[0], D), dtype=np.float64)
    amb = np.zeros((rows.shape[0], D), dtype=np.float64)
    nal = np.zeros((rows.shape[0],), dtype=np.int64)
    rc = lib.oracle_rows(ctypes.byref(a), rows.ctypes.data, rows.shape[0], out.ctypes.data,
                         amb.ctypes.data, nal.ctypes.data)
    if rc != 0:
        raise ValueError("oracle rejected the arguments (code %d)" % rc)
    return OracleResult(rows=rows, out=out, amb=amb, nallowed=nal)


def decode(dtype: torch.dtype, bits: int) -> float:
    """Exact value of one storage code (f16 / bf16 / e4m3fn)."""
    return _load().oracle_decode(_DT[dtype], bits)


def quantize(kind: str, x: float, amb_rel: float = 0.0):
    """(value, delta) of the Q/DQ rounding of x ('fp8' or 'int8')."""
    d = ctypes.c_double(0.0)
    r = _load().oracle_quantize(QDQ[kind], x, amb_rel, ctypes.byref(d))
    return r, d.value
