"""GPU parity of prefill over an fp8 (E4M3FN) KV cache with 16-bit Q.

TensorRT Edge-LLM "TensorRT Plugins Guide", AttentionPlugin: the plugin keeps
an FP16 or FP8 KV cache for prefill (normal and chunked) and decode.  K / V
are stored as E4M3FN codes with per-tensor fp32 descales (k_descale,
v_descale); the scores are scale * k_descale * (q . k8) and the output
v_descale * sum P v8.  The prefill kernels copy the codes into LDS and
convert each tile once to Q's 16-bit type (exact: every E4M3FN value is an
f16 / bf16 value).  Every valid row is compared with the oracle element by
element, and padding rows of the output must keep their sentinel bits.
"""
import numpy as np
import pytest
import torch

from gqa_attention_ragged_amd import capi, synth
from tests import parity
from tests.test_gpu_parity import FORMS, _case

pytestmark = pytest.mark.gpu

DEV = "cuda"
FP8 = torch.float8_e4m3fn


@pytest.mark.parametrize("qf,kf", [(a, b) for a in FORMS for b in FORMS])
@pytest.mark.parametrize("causal", ["none", "upper_left", "lower_right"])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_kv8_forms_causal(qf, kf, causal, dtype):
    seed = 5000 + FORMS.index(qf) * 2 + FORMS.index(kf) + 4 * ["none", "upper_left",
                                                                 "lower_right"].index(causal)
    c = _case(seed, qf=qf, kf=kf, causal=causal, dtype=dtype, kv_fp8=True)
    parity.compare(c, parity.run_gpu(c))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("heads", [(8, 2), (8, 1), (4, 4), (12, 4)])
def test_kv8_head_sizes_and_groups(D, heads):
    hq, hkv = heads
    c = _case(5100 + D + hq * 3 + hkv, qf="packed_nhd", kf="padded_bhnd", causal="lower_right",
              dtype=torch.bfloat16 if hkv % 2 else torch.float16, D=D, hq=hq, hkv=hkv,
              kv_fp8=True)
    parity.compare(c, parity.run_gpu(c))


@pytest.mark.parametrize("mask", ["bool", "f16", "f32"])
@pytest.mark.parametrize("causal", ["none", "lower_right"])
def test_kv8_masks(mask, causal):
    # masks over an fp8 cache are read per lane (no LDS staging)
    c = _case(5200 + ["bool", "f16", "f32"].index(mask) * 2 + (causal != "none"),
              qf="packed_nhd", kf="packed_nhd", causal=causal, mask=mask, kv_fp8=True)
    parity.compare(c, parity.run_gpu(c))


def test_kv8_ragged_with_empty_sequences():
    c = _case(5250, qf="packed_nhd", kf="packed_nhd", causal="lower_right", zero=True, B=6,
              kv_fp8=True)
    parity.compare(c, parity.run_gpu(c))


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_kv8_chunked_context_split(dtype):
    # few query rows over a long context: the split-KV path and its merge
    rng = np.random.default_rng(5300)
    ql = rng.integers(1, 200, size=3)
    kl = ql + rng.integers(3000, 6000, size=3)
    c = synth.generate(seed=5300, q_lens=ql, kv_lens=kl, num_heads=8, kv_num_heads=2,
                       head_dim=128, query_form="packed_nhd", kv_form="padded_bhnd", dtype=dtype,
                       n_kv=int(kl.max()) + 3, causal_kind="lower_right", mask_kind="f16",
                       mask_p=0.1, mask_diag_true=True, kv_fp8_from=torch.float16, kv_dtype=FP8,
                       device=DEV, name=f"kv8-chunked-{dtype}")
    args = capi.make_args(c.q, c.k, c.v, c.mask, torch.empty_like(c.q), **c.kwargs())
    assert capi.gqa_attn_workspace_size(args) > 0  # the split path is taken
    parity.compare(c, parity.run_gpu(c))


@pytest.mark.parametrize("qf", FORMS)
def test_kv8_tree(qf):
    rng = np.random.default_rng(5400)
    ql = rng.integers(1, 65, size=3)
    kl = ql + rng.integers(0, 400, size=3)
    n_q = int(ql.max()) if qf == "packed_nhd" else int(ql.max()) + 3
    c = synth.generate(seed=5400 + (qf == "packed_nhd"), q_lens=ql, kv_lens=kl, num_heads=8,
                       kv_num_heads=2, head_dim=128, query_form=qf, kv_form="padded_bhnd",
                       dtype=torch.float16, n_q=n_q, n_kv=int(kl.max()) + 5,
                       pass_query_lengths=True, tree="spec", kv_fp8_from=torch.float16,
                       kv_dtype=FP8, device=DEV, name=f"kv8-tree-{qf}")
    parity.compare(c, parity.run_gpu(c))


@pytest.mark.parametrize("ps", [64, 128])
@pytest.mark.parametrize("causal,mask", [("lower_right", None), ("none", None), ("none", "bool"),
                                         ("upper_left", "f16")])
def test_kv8_paged_prefill(ps, causal, mask):
    rng = np.random.default_rng(5500 + ps)
    ql = rng.integers(1, 150, size=3)
    kl = ql + rng.integers(0, 500, size=3)
    c = synth.generate(seed=5500 + ps + (mask is not None), q_lens=ql, kv_lens=kl, num_heads=8,
                       kv_num_heads=2, head_dim=128, query_form="packed_nhd", kv_form="paged",
                       dtype=torch.bfloat16, n_kv=int(kl.max()) + 5, pass_query_lengths=True,
                       mask_kind=mask, mask_p=0.2, mask_diag_true=True, causal_kind=causal,
                       page_size=ps, kv_fp8_from=torch.bfloat16, kv_dtype=FP8, device=DEV,
                       name=f"kv8-paged-{ps}-{causal}-{mask}")
    parity.compare(c, parity.run_gpu(c))


def test_kv8_paged_tree():
    rng = np.random.default_rng(5560)
    ql = rng.integers(1, 65, size=3)
    kl = ql + rng.integers(0, 400, size=3)
    c = synth.generate(seed=5560, q_lens=ql, kv_lens=kl, num_heads=8, kv_num_heads=2,
                       head_dim=128, query_form="packed_nhd", kv_form="paged",
                       dtype=torch.float16, n_kv=int(kl.max()) + 5, pass_query_lengths=True,
                       tree="spec", page_size=64, kv_fp8_from=torch.float16, kv_dtype=FP8,
                       device=DEV, name="kv8-paged-tree")
    parity.compare(c, parity.run_gpu(c))


def test_kv8_rejects_qdq_and_none():
    c = _case(5600, qf="packed_nhd", kf="packed_nhd", kv_fp8=True)
    out = torch.empty_like(c.q)
    kw = c.kwargs()
    for extra in ({"qdq": "fp8", "qscale": 1 / 448.0}, {"norm": "none"}):
        args = capi.make_args(c.q, c.k, c.v, c.mask, out, **{**kw, **extra})
        assert capi.gqa_attn_validate(args) == capi.GQA_ERR_UNSUPPORTED
