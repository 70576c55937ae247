"""GPU parity of tree (speculative) decoding through the C ABI against the
CPU oracle (TensorRT Edge-LLM "TensorRT Plugins Guide", AttentionPlugin:
tree decoding attention).  Each sequence's query rows are draft tokens whose
keys are the last q_len keys; a row attends the context and its ancestor
drafts.  Small cases compare every valid row and check that padding rows of
the output keep their sentinel bits; the full-size workload compares sampled
rows."""
import numpy as np
import pytest
import torch

from gqa_attention_ragged_amd import capi, synth
from tests import parity

pytestmark = pytest.mark.gpu

DEV = "cuda"
FORMS = ["padded_bhnd", "packed_nhd"]


def _tree_case(seed, *, qf, kf, tree, causal="none", mask=None, dtype=torch.float16, D=128,
               hq=8, hkv=2, norm="softmax", qdq=None, B=3, qmax=64, ctx_max=300, ctx_min=0):
    rng = np.random.default_rng(seed)
    ql = rng.integers(1, qmax + 1, size=B)
    kl = ql + rng.integers(ctx_min, ctx_max + 1, size=B)
    pass_ql = qf == "packed_nhd" or seed % 2 == 1
    n_q = int(ql.max()) if qf == "packed_nhd" else min(64, int(ql.max()) + 3)
    if not pass_ql:
        ql = np.full(B, n_q)
        kl = ql + rng.integers(ctx_min, ctx_max + 1, size=B)
    return synth.generate(
        seed=seed, q_lens=ql, kv_lens=kl, num_heads=hq, kv_num_heads=hkv, head_dim=D,
        query_form=qf, kv_form=kf, dtype=dtype, n_q=n_q, n_kv=int(kl.max()) + 5, q_slack=3,
        kv_slack=2, pass_query_lengths=pass_ql, mask_kind=mask, mask_p=0.2,
        mask_diag_true=True, causal_kind=causal, norm=norm, qdq=qdq,
        qscale=float(np.float32(1 / 448.0)) if qdq == "fp8" else 1 / 64.0,
        dist="round_normal" if dtype == torch.float8_e4m3fn else "normal", tree=tree,
        device=DEV, name=f"tree{seed}-{qf[:3]}-{kf[:3]}-{tree}-{causal}-{mask}-{dtype}-{D}")


@pytest.mark.parametrize("qf,kf", [(a, b) for a in FORMS for b in FORMS])
@pytest.mark.parametrize("tree", ["spec", "random", "chain", "star", "bad"])
def test_tree_forms(qf, kf, tree):
    seed = 3000 + FORMS.index(qf) * 2 + FORMS.index(kf) + 10 * ["spec", "random", "chain",
                                                                 "star", "bad"].index(tree)
    c = _tree_case(seed, qf=qf, kf=kf, tree=tree)
    parity.compare(c, parity.run_gpu(c))


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float16, 64),
                                     (torch.bfloat16, 64)])
@pytest.mark.parametrize("causal,mask", [("none", None), ("lower_right", None),
                                         ("upper_left", None), ("none", "bool"),
                                         ("lower_right", "f16")])
def test_tree_dtypes_masks(dtype, D, causal, mask):
    seed = 3100 + D + ["none", "lower_right", "upper_left"].index(causal) * 7 + (mask is not None)
    c = _tree_case(seed, qf="packed_nhd", kf="padded_bhnd", tree="spec", causal=causal,
                   mask=mask, dtype=dtype, D=D)
    parity.compare(c, parity.run_gpu(c))


def test_tree_chain_equals_lower_right():
    """A chain of drafts is lower_right causal attention; the GPU results of
    the two formulations agree to the output tolerance."""
    c = _tree_case(3200, qf="packed_nhd", kf="packed_nhd", tree="chain")
    a = parity.run_gpu(c)
    kw = c.kwargs()
    kw.update(tree_parents=None, causal_kind="lower_right")
    b = capi.attn_forward(c.q, c.k, c.v, c.mask, out=synth.sentinel_like(c.q.shape, c.out_dtype, DEV),
                          **kw)
    torch.cuda.synchronize()
    n = int(np.sum(c.q_lens))
    assert torch.allclose(a[:n].float(), b[:n].float(), atol=2e-3, rtol=0)


@pytest.mark.parametrize("norm,qdq,dtype", [("softmax", "fp8", torch.float8_e4m3fn),
                                            ("softmax", "int8", torch.float16),
                                            ("none", None, torch.float16)])
def test_tree_quantized_and_none(norm, qdq, dtype):
    c = _tree_case(3300 + ["fp8", "int8", None].index(qdq), qf="padded_bhnd", kf="padded_bhnd",
                   tree="spec", norm=norm, qdq=qdq, dtype=dtype)
    parity.compare(c, parity.run_gpu(c), amb_rel=1e-4 if dtype != torch.float8_e4m3fn else 1e-5)


def test_tree_split_kv():
    """Few draft rows over long contexts: the keys of each query tile are
    split over several workgroups and merged (the tree tile is in one slice)."""
    c = _tree_case(3400, qf="padded_bhnd", kf="padded_bhnd", tree="spec", B=2, ctx_min=3000,
                   ctx_max=6000, hq=8, hkv=2)
    parity.compare(c, parity.run_gpu(c))


def test_tree_long_packed_rows():
    """Packed sequences of up to 100 drafts with a star tree (every draft
    hangs off the context): each row sees the context and itself."""
    c = _tree_case(3500, qf="packed_nhd", kf="packed_nhd", tree="star", qmax=100, B=2)
    parity.compare(c, parity.run_gpu(c))


def test_tree_workload_sampled():
    c = synth.make_config("tree", device=DEV)
    out = parity.run_gpu(c)
    rows = parity.sample_rows(c, n_per_seq=2, seed=6)
    st = parity.compare(c, out, rows=rows)
    assert st["rows"] > 0
    assert not torch.isnan(out.float()).any()
