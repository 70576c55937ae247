"""The C-ABI library on the host (no GPU needed): it loads, exports every
function include/gqa_attn.h declares, and its host-only entry points
(validate, workspace_size, status strings) behave as documented.  No call
here touches device memory: descriptors carry fake, aligned pointers."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

from gqa_attention_ragged_amd import capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

F16, BF16, FP8, F32, BOOL = 0, 1, 2, 3, 4
PADDED, PACKED = 0, 1


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gqa_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function():
    lib = capi.load()
    names = declared_functions()
    assert len(names) >= 9, names
    assert "gqa_kv_cache_update" in names and "gqa_kv_cache_update_validate" in names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.gqa_attn_abi_version() == 6
    assert "gqa_attn_check_lengths" in names


_addr = [0x100000]


def fake(shape, dtype=F16, strides=None):
    t = capi.GqaTensor()
    _addr[0] += 0x1000000
    t.data = _addr[0]
    t.dtype = dtype
    t.ndim = len(shape)
    if strides is None:
        strides, s = [], 1
        for n in reversed(shape):
            strides.insert(0, s)
            s *= n
    for d, (n, st) in enumerate(zip(shape, strides)):
        t.shape[d] = n
        t.stride[d] = st
    return t


def base_args(qf=PADDED, kf=PADDED, B=2, hq=8, hkv=2, nq=64, nkv=80, D=128, dt=F16, kvdt=None):
    a = capi.GqaArgs()
    kvdt = dt if kvdt is None else kvdt
    a.q = fake([B, hq, nq, D] if qf == PADDED else [B * nq, hq, D], dt)
    a.k = fake([B, hkv, nkv, D] if kf == PADDED else [B * nkv, hkv, D], kvdt)
    a.v = fake([B, hkv, nkv, D] if kf == PADDED else [B * nkv, hkv, D], kvdt)
    a.out = fake([B, hq, nq, D] if qf == PADDED else [B * nq, hq, D], F16 if dt == FP8 else dt)
    a.attn_mask = capi.GqaTensor()
    a.query_lengths = 0x7000000 if qf == PACKED else None
    a.kv_lengths = 0x7100000 if kf == PACKED else None
    a.batch = B
    a.query_form, a.kv_form = qf, kf
    a.scale, a.qscale, a.k_descale, a.v_descale = 0.125, 1.0, 1.0, 1.0
    a.num_heads, a.kv_num_heads = hq, hkv
    return a


def st(a):
    return capi.gqa_attn_validate(a)


def test_valid_forms_pass():
    for qf in (PADDED, PACKED):
        for kf in (PADDED, PACKED):
            for dt in (F16, BF16):
                assert st(base_args(qf, kf, dt=dt)) == capi.GQA_OK, capi.last_error()


def test_status_strings():
    for s in range(5):
        assert capi.status_str(s)
    assert capi.status_str(99) == "unknown status"


@pytest.mark.parametrize("mutate,code", [
    (lambda a: setattr(a, "num_heads", 7), capi.GQA_ERR_INVALID_ARG),
    (lambda a: setattr(a, "kv_num_heads", 3), capi.GQA_ERR_INVALID_ARG),
    (lambda a: setattr(a, "batch", 3), capi.GQA_ERR_INVALID_ARG),
    (lambda a: setattr(a, "query_form", 5), capi.GQA_ERR_INVALID_ARG),
    (lambda a: setattr(a, "causal_kind", 3), capi.GQA_ERR_INVALID_ARG),
    (lambda a: setattr(a, "qdq", 7), capi.GQA_ERR_INVALID_ARG),
    (lambda a: setattr(a.q, "data", None), capi.GQA_ERR_INVALID_ARG),
    (lambda a: setattr(a.q, "ndim", 3), capi.GQA_ERR_INVALID_ARG),
    (lambda a: a.k.stride.__setitem__(3, 2), capi.GQA_ERR_INVALID_ARG),
    (lambda a: setattr(a.v, "dtype", BF16), capi.GQA_ERR_INVALID_ARG),
    (lambda a: setattr(a.out, "dtype", BF16), capi.GQA_ERR_INVALID_ARG),
    (lambda a: a.out.shape.__setitem__(2, 63), capi.GQA_ERR_INVALID_ARG),
    (lambda a: a.v.shape.__setitem__(2, 81), capi.GQA_ERR_INVALID_ARG),
    (lambda a: setattr(a.q, "data", a.q.data + 2), capi.GQA_ERR_UNSUPPORTED),
    (lambda a: a.q.stride.__setitem__(2, 130), capi.GQA_ERR_UNSUPPORTED),
])
def test_invalid_arguments(mutate, code):
    a = base_args()
    mutate(a)
    assert st(a) == code, capi.last_error()
    assert capi.last_error()


def test_packed_requires_lengths():
    a = base_args(PACKED, PADDED)
    a.query_lengths = None
    assert st(a) == capi.GQA_ERR_INVALID_ARG
    assert "query_lengths" in capi.last_error()
    a = base_args(PADDED, PACKED)
    a.kv_lengths = None
    assert st(a) == capi.GQA_ERR_INVALID_ARG
    assert "kv_lengths" in capi.last_error()


def test_head_size_and_dtype_support():
    assert st(base_args(D=96)) == capi.GQA_ERR_UNSUPPORTED
    assert st(base_args(D=64)) == capi.GQA_OK
    a = base_args(dt=FP8)  # fp8 Q/K/V needs fp8 Q/DQ of the scores
    assert st(a) == capi.GQA_ERR_UNSUPPORTED
    a.qdq, a.qscale = 1, 1 / 448
    assert st(a) == capi.GQA_OK, capi.last_error()
    a.qscale = 0.0
    assert st(a) == capi.GQA_ERR_INVALID_ARG
    # fp8 KV cache with f16 Q: decode and prefill with softmax, no Q/DQ
    assert st(base_args(kvdt=FP8)) == capi.GQA_OK, capi.last_error()
    assert st(base_args(nq=1, kvdt=FP8)) == capi.GQA_OK, capi.last_error()
    a = base_args(kvdt=FP8)
    a.qdq, a.qscale = 1, 1 / 448
    assert st(a) == capi.GQA_ERR_UNSUPPORTED
    a = base_args(kvdt=FP8)
    a.norm = 1  # "none"
    assert st(a) == capi.GQA_ERR_UNSUPPORTED


def test_mask_validation():
    a = base_args()
    a.attn_mask = fake([2, 1, 64, 80], BOOL)
    assert st(a) == capi.GQA_OK, capi.last_error()
    a.attn_mask = fake([64, 80], F32)
    assert st(a) == capi.GQA_OK
    a.attn_mask = fake([3, 1, 64, 80], BOOL)
    assert st(a) == capi.GQA_ERR_INVALID_ARG
    a.attn_mask = fake([2, 5, 64, 80], BOOL)
    assert st(a) == capi.GQA_ERR_INVALID_ARG
    a.attn_mask = fake([2, 1, 64, 79], F16)  # shorter than N_kv with no kv_lengths
    assert st(a) == capi.GQA_ERR_INVALID_ARG
    a.attn_mask = fake([2, 1, 64, 80], FP8)
    assert st(a) == capi.GQA_ERR_INVALID_ARG


def test_workspace_sizes():
    # prefill: the per-workgroup records of the tile map, 32 bytes per
    # workgroup (the opt-in persistent kernel: its claim counters instead,
    # under 1 KiB); the decode step (N_q = 1) needs split partials
    n0 = capi.gqa_attn_workspace_size(base_args())
    if os.environ.get("GQA_ATTN_PERSIST") == "1":
        assert 0 < n0 <= 1024
    else:
        assert n0 == 0  # 8 workgroups: each builds the map itself
    m = base_args()
    m.attn_mask = fake([2, 1, 64, 80], BOOL)
    assert capi.gqa_attn_workspace_size(m) == 0
    # 64 x 512 rows x 8 head groups = 8192 workgroups: records
    big = base_args(B=64, hq=32, hkv=8, nq=512)
    big.attn_mask = fake([64, 1, 512, 80], BOOL)
    n_wg = 64 * (512 // 32) * (32 // math.gcd(32 // 8, 4))
    assert capi.gqa_attn_workspace_size(big) == (n_wg * 32 + 255) // 256 * 256 + 256
    # more than 64 sequences: the workgroups build the map themselves
    assert capi.gqa_attn_workspace_size(base_args(B=65, hq=32, hkv=8, nq=512)) == 0
    a = base_args(B=128, hq=32, hkv=8, nq=1, nkv=32768)
    n = capi.gqa_attn_workspace_size(a)
    assert n > 128 * 32 * 130 * 4
    assert n < 1 << 30


def test_empty_batch_is_valid():
    a = base_args(B=0)
    assert st(a) == capi.GQA_OK
    a = base_args(PACKED, PACKED, B=2)
    a.q.shape[0] = 0
    a.out.shape[0] = 0
    assert st(a) == capi.GQA_OK


# ------------------------------------------------------------ KV-cache update
def kv_args(form=PADDED, B=2, H=4, N=64, D=128, nu=8, T=10, dt=F16, in_place=True):
    a = capi.GqaKvUpdateArgs()
    a.past_cache = fake([B, H, N, D], dt)
    a.update = fake([B, H, nu, D] if form == PADDED else [T, H, D], dt)
    a.out = a.past_cache if in_place else fake([B, H, N, D], dt)
    a.write_indices = 0x7000
    a.update_lengths = 0x8000
    a.update_form = form
    return a


@pytest.mark.parametrize("form", [PADDED, PACKED])
@pytest.mark.parametrize("dt", [F16, BF16, FP8])
@pytest.mark.parametrize("in_place", [True, False])
def test_kv_update_validate_accepts(form, dt, in_place):
    a = kv_args(form=form, dt=dt, in_place=in_place)
    assert capi.gqa_kv_cache_update_validate(a) == 0, capi.last_error()


def test_kv_update_validate_rejects():
    a = kv_args(form=PACKED)
    a.update_lengths = None
    assert capi.gqa_kv_cache_update_validate(a) == 1  # packed needs lengths
    a = kv_args()
    a.update.dtype = BF16
    assert capi.gqa_kv_cache_update_validate(a) == 1  # dtype mismatch
    a = kv_args()
    a.update.shape[1] = 3
    assert capi.gqa_kv_cache_update_validate(a) == 1  # head count mismatch
    a = kv_args(in_place=False)
    a.out.shape[2] = 63
    assert capi.gqa_kv_cache_update_validate(a) == 1  # out shape
    a = kv_args(dt=FP8, D=8)
    assert capi.gqa_kv_cache_update_validate(a) == 2  # 8-byte rows
    a = kv_args()
    a.out = fake([2, 4, 64, 128], F16)
    a.out.data = a.past_cache.data
    a.out.stride[0] = a.past_cache.stride[0] * 2
    assert capi.gqa_kv_cache_update_validate(a) == 1  # aliasing with other strides
    a = kv_args(dt=F32)
    assert capi.gqa_kv_cache_update_validate(a) == 1  # dtype


def test_tree_parents_validation():
    """Tree decoding resolves up to 128 drafts per sequence: padded Q with
    N_q > 128 is rejected on the host; packed Q (checked on the device) and
    N_q <= 128 pass."""
    a = base_args(nq=128, nkv=140)
    a.tree_parents = 0x7200000
    assert st(a) == capi.GQA_OK, capi.last_error()
    a = base_args(nq=129, nkv=140)
    a.tree_parents = 0x7200000
    assert st(a) == capi.GQA_ERR_UNSUPPORTED
    assert "tree_parents" in capi.last_error()
    a = base_args(PACKED, PADDED, nq=200, nkv=220)
    a.tree_parents = 0x7200000
    assert st(a) == capi.GQA_OK, capi.last_error()


def _paged_args(nq=1, ps=64, P=40, pages=8, qdq=0):
    a = base_args(nq=nq)
    a.kv_form = 2
    a.k = fake([P, 2, ps, 128], F16)
    a.v = fake([P, 2, ps, 128], F16)
    a.kv_lengths = 0x7100000
    a.kv_page_table = 0x7300000
    a.kv_max_pages = pages
    a.qdq = qdq
    return a


def test_paged_kv_validation():
    assert st(_paged_args(nq=1, ps=32)) == capi.GQA_OK, capi.last_error()      # decode
    assert st(_paged_args(nq=64, ps=64)) == capi.GQA_OK, capi.last_error()     # prefill
    assert st(_paged_args(nq=64, ps=32)) == capi.GQA_ERR_UNSUPPORTED           # prefill pages < 64
    assert st(_paged_args(nq=1, ps=48)) == capi.GQA_ERR_UNSUPPORTED            # not a power of two
    assert st(_paged_args(nq=1, ps=16)) == capi.GQA_ERR_UNSUPPORTED            # < 32
    a = _paged_args(nq=64, ps=64, qdq=2)
    a.qscale = 1 / 64
    assert st(a) == capi.GQA_ERR_UNSUPPORTED                                   # Q/DQ
    a = _paged_args()
    a.kv_page_table = None
    assert st(a) == capi.GQA_ERR_INVALID_ARG
    a = _paged_args()
    a.kv_lengths = None
    assert st(a) == capi.GQA_ERR_INVALID_ARG
    a = _paged_args()
    a.kv_max_pages = 0
    assert st(a) == capi.GQA_ERR_INVALID_ARG
    a = base_args()
    a.kv_page_table = 0x7300000
    assert st(a) == capi.GQA_ERR_INVALID_ARG                                   # table without paging
    a = _paged_args()
    a.kv_form = 3
    assert st(a) == capi.GQA_ERR_INVALID_ARG
    # fp8 KV in pages: prefill (with a mask or a tree too) and decode
    a = _paged_args(nq=64)
    a.k.dtype = a.v.dtype = FP8
    assert st(a) == capi.GQA_OK, capi.last_error()
    a.attn_mask = fake([2, 1, 64, 8 * 64], BOOL)
    assert st(a) == capi.GQA_OK, capi.last_error()
    a = _paged_args(nq=64)
    a.k.dtype = a.v.dtype = FP8
    a.tree_parents = 0x7200000
    assert st(a) == capi.GQA_OK, capi.last_error()
    a = _paged_args(nq=1)
    a.k.dtype = a.v.dtype = FP8
    assert st(a) == capi.GQA_OK, capi.last_error()


# ------------------------------------------------------------ 32-bit windows
def test_negative_strides_rejected():
    a = base_args()
    a.k.stride[2] = -128
    assert st(a) == capi.GQA_ERR_UNSUPPORTED
    assert "negative stride" in capi.last_error()
    a = base_args()
    a.attn_mask = fake([2, 1, 64, 80], BOOL, strides=[5120, 5120, -80, 1])
    assert st(a) == capi.GQA_ERR_UNSUPPORTED


def test_window_spans_below_4gib():
    """A key tile / decode split (8704 rows) and a query tile (32 rows) are
    read through 32-bit windows with 64-bit bases: the row stride times that
    many rows must stay below 4 GiB, however long the whole sequence is."""
    # a 262144-token packed KV of 64 heads x 128 f16 spans 4 GiB per tensor
    # but 8704 rows of it only 138 MB: accepted
    a = base_args(PACKED, PACKED, B=1, hq=64, hkv=64, nq=262144, nkv=262144)
    assert st(a) == capi.GQA_OK, capi.last_error()
    # a row stride of 512 KiB (f16: 262144 elements): 8704 rows reach 4 GiB
    big = 262144
    a = base_args(PADDED, PACKED, B=1, nkv=100)
    a.k = fake([100, 2, 128], F16, strides=[big, 128, 1])
    a.v = fake([100, 2, 128], F16, strides=[big, 128, 1])
    assert st(a) == capi.GQA_ERR_UNSUPPORTED
    assert "4 GiB" in capi.last_error()
    # just below: 8704 rows of 256 KiB stride minus a row: 2.2 GB, accepted
    a.k = fake([100, 2, 128], F16, strides=[big // 2, 128, 1])
    a.v = fake([100, 2, 128], F16, strides=[big // 2, 128, 1])
    assert st(a) == capi.GQA_OK, capi.last_error()
    # Q: 32 rows of a 160 MiB stride
    a = base_args()
    q_stride = 80 << 20  # elements (f16): 160 MiB per row, 31 rows > 4 GiB
    a.q = fake([2, 8, 64, 128], F16, strides=[64 * q_stride, 128, q_stride, 1])
    assert st(a) == capi.GQA_ERR_UNSUPPORTED


# ------------------------------------------------- device-side preconditions
def _lens_args(qf=PACKED, kf=PADDED, B=3, nq=50, nkv=80, mask=None, tree=False, paged=False):
    a = base_args(qf, kf, B=B, nq=nq, nkv=nkv)
    if qf == PADDED:
        a.query_lengths = 0x7000000
    if kf == PADDED:
        a.kv_lengths = 0x7100000
    if mask is not None:
        a.attn_mask = fake(mask, BOOL)
    if tree:
        a.tree_parents = 0x7200000
    if paged:
        a.kv_form = 2
        a.k = fake([12, 2, 64, 128], F16)
        a.v = fake([12, 2, 64, 128], F16)
        a.kv_page_table = 0x7300000
        a.kv_max_pages = 2
    return a


def _chk(a, ql=None, kl=None, pt=None):
    return capi.gqa_attn_check_lengths(a, ql, kl, pt)


def test_check_lengths_accepts_valid():
    a = _lens_args()                                  # packed Q (T = 150), padded KV [B]
    assert _chk(a, [0, 50, 50, 150], [60, 0, 80]) == capi.GQA_OK, capi.last_error()
    a = _lens_args(PACKED, PACKED)                    # both packed: T_kv = 240
    assert _chk(a, [0, 1, 2, 3], [0, 100, 100, 240]) == capi.GQA_OK, capi.last_error()
    a = _lens_args(PADDED, PADDED)                    # padded Q with lengths
    assert _chk(a, [0, 50, 99, 100], [80, 1, 0]) == capi.GQA_OK, capi.last_error()


@pytest.mark.parametrize("case,ql,kl,needle", [
    ("ql0", [1, 50, 50, 150], [60, 0, 80], "query_lengths[0]"),
    ("ql_order", [0, 50, 40, 150], [60, 0, 80], "non-decreasing"),
    ("ql_range", [0, 50, 50, 151], [60, 0, 80], "exceed q"),
    ("kl_neg", [0, 50, 50, 150], [60, -1, 80], "kv_lengths"),
    ("kl_range", [0, 50, 50, 150], [60, 0, 81], "exceed k/v"),
])
def test_check_lengths_rejects(case, ql, kl, needle):
    a = _lens_args()
    assert _chk(a, ql, kl) == capi.GQA_ERR_INVALID_ARG, case
    assert needle in capi.last_error(), (case, capi.last_error())


def test_check_lengths_packed_kv_and_padded_q():
    a = _lens_args(PACKED, PACKED)
    assert _chk(a, [0, 1, 2, 3], [2, 100, 100, 240]) == capi.GQA_ERR_INVALID_ARG
    assert _chk(a, [0, 1, 2, 3], [0, 100, 90, 240]) == capi.GQA_ERR_INVALID_ARG
    assert _chk(a, [0, 1, 2, 3], [0, 100, 100, 241]) == capi.GQA_ERR_INVALID_ARG
    a = _lens_args(PADDED, PADDED)
    assert _chk(a, [0, 51, 60, 70], [1, 1, 1]) == capi.GQA_ERR_INVALID_ARG  # q_len 51 > N_q 50


def test_check_lengths_mask_tree_pages():
    a = _lens_args(mask=[3, 1, 40, 80])               # mask rows cover 40 queries only
    assert _chk(a, [0, 40, 40, 80], [60, 0, 80]) == capi.GQA_OK, capi.last_error()
    assert _chk(a, [0, 41, 41, 81], [60, 0, 80]) == capi.GQA_ERR_INVALID_ARG
    assert "attn_mask" in capi.last_error()
    a = _lens_args(mask=[1, 1, 1, 70])                # broadcast rows, 70 keys
    assert _chk(a, [0, 41, 41, 81], [70, 0, 5]) == capi.GQA_OK, capi.last_error()
    assert _chk(a, [0, 41, 41, 81], [71, 0, 5]) == capi.GQA_ERR_INVALID_ARG
    a = _lens_args(B=2, nq=200, nkv=300, tree=True)   # 128 drafts resolved per sequence
    assert _chk(a, [0, 128, 200], [130, 300]) == capi.GQA_OK, capi.last_error()
    assert _chk(a, [0, 129, 200], [130, 300]) == capi.GQA_ERR_INVALID_ARG
    assert "drafts" in capi.last_error()
    a = _lens_args(B=2, nq=4, paged=True)             # pools of 12 pages
    pt = np.array([[[0, 9], [11, 3]], [[5, 5], [0, 0]]], dtype=np.int32)
    assert _chk(a, [0, 4, 8], [128, 64], pt) == capi.GQA_OK, capi.last_error()
    assert _chk(a, [0, 4, 8], [129, 64], pt) == capi.GQA_ERR_INVALID_ARG   # beyond 2 pages
    bad = pt.copy()
    bad[1, 0, 0] = 12                                  # K page 12 of a 12-page pool
    assert _chk(a, [0, 4, 8], [128, 64], bad) == capi.GQA_ERR_INVALID_ARG
    assert "page" in capi.last_error()
    bad = pt.copy()
    bad[1, 1, 1] = -1                                  # unused entry (64 keys = 1 page): ignored
    assert _chk(a, [0, 4, 8], [128, 64], bad) == capi.GQA_OK, capi.last_error()


def test_check_lengths_needs_host_copies():
    a = _lens_args()
    assert _chk(a, None, [60, 0, 80]) == capi.GQA_ERR_INVALID_ARG
    assert "host copy" in capi.last_error()


def test_split_kv_planning():
    """Key slices for prefill: a padded-Q grid that fills 3/4 to one round of
    the 512 workgroup slots takes none (tree decoding shape: 32 sequences x 64
    drafts x 8 head groups = 512 workgroups); half a round, or a packed grid
    (an upper bound), over long keys takes slices (the workspace holds their
    fp32 partials)."""
    full = base_args(PADDED, PADDED, B=32, hq=32, hkv=8, nq=64, nkv=8192)
    assert capi.gqa_attn_workspace_size(full) == 0
    half = base_args(PADDED, PADDED, B=16, hq=32, hkv=8, nq=64, nkv=8192)
    assert capi.gqa_attn_workspace_size(half) > 16 * 64 * 32 * 2 * 128 * 4
    # 24 sequences: padded, 384 workgroups (3/4 of a round): none; packed, an
    # upper bound of 576 workgroups: slices
    assert capi.gqa_attn_workspace_size(
        base_args(PADDED, PADDED, B=24, hq=32, hkv=8, nq=64, nkv=8192)) == 0
    packed = base_args(PACKED, PADDED, B=24, hq=32, hkv=8, nq=64, nkv=8192)
    assert capi.gqa_attn_workspace_size(packed) > 24 * 64 * 32 * 2 * 128 * 4


def test_timer_argument_errors():
    # the main-kernel timer's host-side checks (no HIP call is made): a
    # window needs a positive size, a stop needs an open window and outputs
    lib = capi.load()
    assert capi.timer_start(0) == capi.GQA_ERR_INVALID_ARG
    assert capi.timer_start(-3) == capi.GQA_ERR_INVALID_ARG
    st, ms, n = capi.timer_stop()
    assert st == capi.GQA_ERR_INVALID_ARG and "no timing window" in capi.last_error()
    assert lib.gqa_attn_timer_stop(None, None) == capi.GQA_ERR_INVALID_ARG
