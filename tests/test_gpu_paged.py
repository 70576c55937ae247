"""GPU parity of paged KV (TensorRT Edge-LLM "TensorRT Plugins Guide",
AttentionPlugin decoder tensor contract: kv_page_table [N, 2,
max_pages_per_sequence]) through the C ABI against the CPU oracle: decode
(query length 1, 16-bit and fp8 pools), chunked prefill with causal kinds and
masks, tree decoding, split-KV, and the same data as padded KV giving
bitwise-identical outputs.  Pools carry NaN spare pages and NaN rows past
each length, and unused table entries point at a NaN page, so a wrong page or
row shows up as NaN in a valid row."""
import numpy as np
import pytest
import torch

from gqa_attention_ragged_amd import synth
from tests import parity

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _decode_case(seed, ps, dtype=torch.float16, kv_fp8=False, kv_form="paged", B=6, D=128,
                 hq=8, hkv=2, kvmax=3000):
    rng = np.random.default_rng(seed)
    kl = rng.integers(0, kvmax + 1, size=B)
    kl[0] = ps  # exactly one page
    kl[1] = 1   # one key
    if B > 2:
        kl[2] = 0  # empty sequence
    return synth.generate(
        seed=seed, q_lens=np.ones(B, dtype=np.int64), kv_lens=kl, num_heads=hq, kv_num_heads=hkv,
        head_dim=D, n_q=1, n_kv=int(kl.max()) + 1, dtype=dtype, kv_form=kv_form, page_size=ps,
        pass_query_lengths=False, kv_fp8_from=dtype if kv_fp8 else None,
        kv_dtype=torch.float8_e4m3fn if kv_fp8 else None, device=DEV,
        name=f"pdec{seed}-{ps}-{dtype}-{kv_fp8}-{D}")


@pytest.mark.parametrize("ps", [32, 64, 256])
@pytest.mark.parametrize("dtype,kv_fp8,D", [(torch.float16, False, 128), (torch.bfloat16, False, 64),
                                            (torch.float16, True, 128), (torch.bfloat16, True, 128)])
def test_paged_decode(ps, dtype, kv_fp8, D):
    c = _decode_case(4000 + ps + D + 7 * kv_fp8, ps, dtype, kv_fp8, D=D)
    parity.compare(c, parity.run_gpu(c))


def _prefill_case(seed, ps, *, qf="packed_nhd", causal="lower_right", mask=None, tree=None,
                  dtype=torch.float16, kv_form="paged", B=3, D=128, qmax=150, ctx=400):
    rng = np.random.default_rng(seed)
    ql = rng.integers(1, qmax + 1, size=B)
    kl = ql + rng.integers(0, ctx + 1, size=B)
    if tree:
        ql = np.minimum(ql, 64)
        kl = ql + rng.integers(0, ctx + 1, size=B)
    n_q = int(ql.max()) if qf == "packed_nhd" else int(ql.max()) + 2
    return synth.generate(
        seed=seed, q_lens=ql, kv_lens=kl, num_heads=8, kv_num_heads=2, head_dim=D,
        query_form=qf, kv_form=kv_form, dtype=dtype, n_q=n_q, n_kv=int(kl.max()) + 5,
        q_slack=2, pass_query_lengths=True, mask_kind=mask, mask_p=0.2, mask_diag_true=True,
        causal_kind=causal, tree=tree, page_size=ps, device=DEV,
        name=f"ppre{seed}-{ps}-{qf[:3]}-{causal}-{mask}-{tree}-{dtype}-{D}")


@pytest.mark.parametrize("ps", [64, 128])
@pytest.mark.parametrize("qf", ["padded_bhnd", "packed_nhd"])
@pytest.mark.parametrize("causal,mask", [("lower_right", None), ("none", None),
                                         ("upper_left", "bool"), ("lower_right", "f16")])
def test_paged_prefill(ps, qf, causal, mask):
    seed = 4100 + ps + (qf == "packed_nhd") * 3 + ["lower_right", "none", "upper_left"].index(causal) * 11 \
        + (mask is not None)
    c = _prefill_case(seed, ps, qf=qf, causal=causal, mask=mask,
                      dtype=torch.bfloat16 if seed % 2 else torch.float16, D=64 if seed % 3 == 0 else 128)
    parity.compare(c, parity.run_gpu(c))


def test_paged_tree():
    c = _prefill_case(4200, 64, tree="spec", causal="none")
    parity.compare(c, parity.run_gpu(c))


def test_paged_split_kv():
    # few query rows over long keys: split-KV slices through the page table
    c = _prefill_case(4300, 128, qmax=40, ctx=6000, B=2)
    parity.compare(c, parity.run_gpu(c))


@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_paged_equals_padded_bitwise(kind):
    """Drawn from one seed, the paged case holds the padded case's K/V rows on
    shuffled pages: the kernels read the same values in the same order, so the
    outputs are bitwise equal."""
    if kind == "decode":
        a = _decode_case(4400, 64, kv_form="padded_bhnd")
        b = _decode_case(4400, 64)
    else:
        a = _prefill_case(4401, 64, kv_form="padded_bhnd")
        b = _prefill_case(4401, 64)
    ya, yb = parity.run_gpu(a), parity.run_gpu(b)
    assert torch.equal(ya.view(torch.int16), yb.view(torch.int16))


def test_paged_decode_workload_sampled():
    c = synth.make_config("4p", device=DEV)
    out = parity.run_gpu(c)
    rows = parity.sample_rows(c, n_per_seq=1, seed=4)
    st = parity.compare(c, out, rows=rows)
    assert st["rows"] > 0
    assert not torch.isnan(out.float()).any()
