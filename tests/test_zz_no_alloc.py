"""The allocation-free forward call (gqa_attn_forward_noalloc, static device
workspace) against the caller-workspace call (gqa_attn_forward), through the
C ABI: two calls in a row on the decode step (split-KV partials in the
workspace), the second smaller, then two split-KV prefill calls, the second
smaller; each output equal to the caller-workspace output within the parity
tolerance (the same kernels and plan: bit for bit in practice) and checked
against the oracle on the smaller call.  Then a call whose workspace would
exceed the static buffer is rejected before any launch."""
import ctypes

import numpy as np
import pytest
import torch

from gqa_attention_ragged_amd import capi, synth
from tests import parity

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _both(c):
    """(caller-workspace output, static-workspace output) of one case."""
    a = synth.sentinel_like(c.q.shape, c.out_dtype, DEV)
    b = synth.sentinel_like(c.q.shape, c.out_dtype, DEV)
    stream = torch.cuda.current_stream().cuda_stream
    args_a = capi.make_args(c.q, c.k, c.v, c.mask, a, **c.kwargs())
    n = capi.gqa_attn_workspace_size(args_a)
    assert n > 0  # the case uses a workspace
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    capi.gqa_attn_forward(args_a, ws, stream)
    args_b = capi.make_args(c.q, c.k, c.v, c.mask, b, **c.kwargs())
    capi.gqa_attn_forward_noalloc(args_b, stream)
    torch.cuda.synchronize()
    return a, b


def _check_pair(c, a, b):
    tol = parity.tolerance(c)
    n = int(np.sum(c.q_lens)) if c.query_form == "packed_nhd" else None
    x = (a[:n] if n is not None else a).float()
    y = (b[:n] if n is not None else b).float()
    assert torch.all(torch.isfinite(y))
    assert float((x - y).abs().max()) <= tol
    if n is not None:  # the packed slack rows keep the sentinel in both
        assert torch.equal(a[n:].view(torch.int16), b[n:].view(torch.int16))


def test_noalloc_decode_two_calls_second_smaller():
    big = synth.generate(seed=8100, q_lens=np.ones(24, int),
                         kv_lens=np.random.default_rng(8100).integers(1000, 20000, size=24),
                         num_heads=32, kv_num_heads=8, head_dim=128, n_q=1, n_kv=20000,
                         dtype=torch.float16, pass_query_lengths=False, device=DEV,
                         name="noalloc-decode-big")
    a, b = _both(big)
    _check_pair(big, a, b)
    small = synth.generate(seed=8101, q_lens=np.ones(3, int), kv_lens=[700, 1, 4000],
                           num_heads=8, kv_num_heads=2, head_dim=64, n_q=1, n_kv=4000,
                           dtype=torch.bfloat16, pass_query_lengths=False, device=DEV,
                           name="noalloc-decode-small")
    a, b = _both(small)
    _check_pair(small, a, b)
    parity.compare(small, b)


def test_noalloc_prefill_split_two_calls_second_smaller():
    big = synth.generate(seed=8200, q_lens=[200, 37, 64], kv_lens=[6000, 3000, 4500],
                         num_heads=32, kv_num_heads=8, head_dim=128, query_form="packed_nhd",
                         kv_form="padded_bhnd", n_kv=6016, q_slack=2, dtype=torch.float16,
                         causal_kind="lower_right", mask_kind="f16", mask_p=0.1, device=DEV,
                         name="noalloc-prefill-big")
    a, b = _both(big)
    _check_pair(big, a, b)
    small = synth.generate(seed=8201, q_lens=[37, 5], kv_lens=[2900, 700], num_heads=8,
                           kv_num_heads=2, head_dim=128, query_form="packed_nhd",
                           kv_form="packed_nhd", q_slack=2, kv_slack=2, dtype=torch.bfloat16,
                           causal_kind="lower_right", device=DEV, name="noalloc-prefill-small")
    a, b = _both(small)
    _check_pair(small, a, b)
    parity.compare(small, b)


def test_noalloc_prefill_records_two_calls_second_smaller():
    # at least 1024 workgroups and no key slices: the static buffer holds the
    # tile-map records, and the second, smaller call rewrites fewer of them
    rng = np.random.default_rng(8300)
    ql = rng.integers(64, 400, size=64)
    kl = ql + rng.integers(0, 40, size=64)
    big = synth.generate(seed=8300, q_lens=ql, kv_lens=kl, num_heads=32, kv_num_heads=8,
                         head_dim=128, query_form="packed_nhd", kv_form="packed_nhd",
                         q_slack=2, kv_slack=2, dtype=torch.bfloat16, causal_kind="lower_right",
                         device=DEV, name="noalloc-records-big")
    a, b = _both(big)
    _check_pair(big, a, b)
    ql2 = rng.integers(100, 300, size=40)
    small = synth.generate(seed=8301, q_lens=ql2, kv_lens=ql2 + 7, num_heads=32,
                           kv_num_heads=8, head_dim=128, query_form="packed_nhd",
                           kv_form="padded_bhnd", n_kv=int(ql2.max()) + 9, q_slack=2,
                           dtype=torch.float16, causal_kind="none", device=DEV,
                           name="noalloc-records-small")
    a, b = _both(small)
    _check_pair(small, a, b)
    parity.compare(small, b)


def test_noalloc_rejects_beyond_static_buffer():
    # 512 sequences x 32 heads x 32 key splits of partials: more than 128 MiB
    # of workspace.  K / V are stride-0 views of one row (the call is
    # rejected on the host, before any launch, so nothing reads them).
    B, hq, hkv, n_kv, D = 512, 32, 8, 131072, 128
    q = torch.zeros((B, hq, 1, D), dtype=torch.float16, device=DEV)
    row = torch.zeros((1, 1, 1, D), dtype=torch.float16, device=DEV)
    k = row.expand(B, hkv, n_kv, D)
    v = row.expand(B, hkv, n_kv, D)
    out = synth.sentinel_like(q.shape, torch.float16, DEV)
    kv_lengths = torch.ones(B, dtype=torch.int32, device=DEV)
    args = capi.make_args(q, k, v, None, out, kv_lengths=kv_lengths, scale=0.088)
    assert capi.gqa_attn_workspace_size(args) > (128 << 20)
    st = capi.load().gqa_attn_forward_noalloc(ctypes.byref(args),
                                              torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == capi.GQA_ERR_WORKSPACE
    assert "static scratch" in capi.last_error()
    assert torch.all(out.view(torch.int16) == synth.SENTINEL_BITS[torch.float16])
