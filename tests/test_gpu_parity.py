"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small cases compare every valid row element by element and check that no
padding row of the output was written; full-size workload cases compare
sampled rows the oracle computes one by one.  Inputs are seeded and
synthetic (gqa_attention_ragged_amd.synth); padding is NaN-poisoned, so a
kernel that reads it produces NaN in a valid row.
"""
import dataclasses
import itertools

import numpy as np
import pytest
import torch

from gqa_attention_ragged_amd import capi, synth
from tests import parity

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _lens(rng, B, lo, hi):
    return rng.integers(lo, hi + 1, size=B)


def _case(seed, *, qf, kf, causal="none", mask=None, dtype=torch.float16, D=128, hq=8, hkv=2,
          norm="softmax", qdq=None, B=3, qmax=150, kvmax=170, zero=False, n_q_pad=None,
          kv_fp8=False, mask_heads=1, qscale=None, scale=None):
    rng = np.random.default_rng(seed)
    ql = _lens(rng, B, 0 if zero else 1, qmax)
    kl = _lens(rng, B, 0 if zero else 1, kvmax)
    if causal == "lower_right" and not zero:
        kl = np.maximum(kl, ql)
    pass_ql = qf == "packed_nhd" or seed % 2 == 1
    n_q = int(ql.max()) + 5 if n_q_pad is None else n_q_pad
    if not pass_ql:
        ql = np.full(B, n_q)
        if causal == "lower_right":
            kl = np.maximum(kl, ql)
    return synth.generate(
        seed=seed, q_lens=ql, kv_lens=kl, num_heads=hq, kv_num_heads=hkv, head_dim=D,
        query_form=qf, kv_form=kf, dtype=dtype, n_q=n_q, n_kv=int(kl.max()) + 7, q_slack=3,
        kv_slack=2, pass_query_lengths=pass_ql, mask_kind=mask, mask_heads=mask_heads,
        mask_p=0.2, mask_value=-4.0 if seed % 3 else -float("inf"), mask_diag_true=True,
        causal_kind=causal, norm=norm, qdq=qdq, scale=scale,
        qscale=qscale if qscale is not None else (
            float(np.float32(1 / 448.0)) if qdq == "fp8" else 1 / 64.0),
        kv_fp8_from=torch.float16 if kv_fp8 else None,
        kv_dtype=torch.float8_e4m3fn if kv_fp8 else None,
        dist="round_normal" if dtype == torch.float8_e4m3fn else "normal",
        device=DEV, name=f"s{seed}-{qf[:3]}-{kf[:3]}-{causal}-{mask}-{dtype}-{D}-{hq}/{hkv}")


FORMS = ["padded_bhnd", "packed_nhd"]


def test_config1_full():
    c = synth.make_config("1", device=DEV)
    out = parity.run_gpu(c)
    st = parity.compare(c, out)
    assert st["rows"] == 2 * 4 * 128


@pytest.mark.parametrize("qf,kf", list(itertools.product(FORMS, FORMS)))
@pytest.mark.parametrize("causal", ["none", "upper_left", "lower_right"])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_forms_causal(qf, kf, causal, dtype):
    seed = 100 + FORMS.index(qf) * 10 + FORMS.index(kf) * 5 + ["none", "upper_left",
                                                              "lower_right"].index(causal)
    c = _case(seed, qf=qf, kf=kf, causal=causal, dtype=dtype)
    parity.compare(c, parity.run_gpu(c))


@pytest.mark.parametrize("mask", ["bool", "f16", "bf16", "f32"])
@pytest.mark.parametrize("causal", ["none", "lower_right"])
@pytest.mark.parametrize("mask_heads", [1, 8])
def test_masks(mask, causal, mask_heads):
    seed = 200 + ["bool", "f16", "bf16", "f32"].index(mask) * 4 + (causal == "none") * 2 + (
        mask_heads == 8)
    c = _case(seed, qf="packed_nhd", kf="padded_bhnd", causal=causal, mask=mask,
              mask_heads=mask_heads)
    parity.compare(c, parity.run_gpu(c))



@pytest.mark.parametrize("mask", ["bool", "f16", "bf16"])
@pytest.mark.parametrize("causal", ["none", "lower_right", "upper_left"])
@pytest.mark.parametrize("row_bcast", [False, True])
def test_head_broadcast_masks_ragged_tails(mask, causal, row_bcast):
    # Head-broadcast masks whose rows are whole 16-byte chunks (the kernel
    # stages their tiles through LDS) with key lengths that end inside a
    # chunk, and the last query row of each sequence at varied positions
    # within a 32-row tile; row_bcast: one mask row shared by all queries.
    seed = 250 + ["bool", "f16", "bf16"].index(mask) * 6 + ["none", "lower_right",
                                                         "upper_left"].index(causal) * 2 + row_bcast
    rng = np.random.default_rng(seed)
    ql = np.array([31, 1, 70, 33, 17])
    kl = rng.integers(1, 300, size=5) * 2 + 1  # odd lengths
    if causal == "lower_right":
        kl = np.maximum(kl, ql)
    c = synth.generate(seed=seed, q_lens=ql, kv_lens=kl, num_heads=8, kv_num_heads=2,
                       head_dim=128, query_form="packed_nhd", kv_form="padded_bhnd",
                       n_kv=640, q_slack=2, kv_slack=0, dtype=torch.float16, mask_kind=mask,
                       mask_p=0.2, mask_value=-3.0, mask_diag_true=True, causal_kind=causal,
                       device=DEV, name=f"staged-mask-{mask}-{causal}-{row_bcast}")
    if row_bcast:
        c = dataclasses.replace(c, mask=c.mask[:, :, :1, :].contiguous())
    parity.compare(c, parity.run_gpu(c))

@pytest.mark.parametrize("scale", [-0.0883, 0.0])
@pytest.mark.parametrize("kind", ["plain", "staged_bool", "f32_mask", "none", "fp8_qdq"])
def test_non_positive_scale(scale, kind):
    # A negative or zero score scale: the scores change sign or all become 0
    # (softmax then spreads evenly over the allowed keys).
    seed = 470 + ["plain", "staged_bool", "f32_mask", "none", "fp8_qdq"].index(kind) * 2 + (
        scale == 0.0)
    if kind == "staged_bool":
        ql = np.array([31, 1, 70, 33, 17])
        kl = np.array([101, 40, 333, 77, 9])
        c = synth.generate(seed=seed, q_lens=ql, kv_lens=np.maximum(kl, ql), num_heads=8,
                           kv_num_heads=2, head_dim=128, query_form="packed_nhd",
                           kv_form="padded_bhnd", n_kv=640, q_slack=2, kv_slack=0,
                           dtype=torch.float16, mask_kind="bool", mask_p=0.2,
                           mask_diag_true=True, causal_kind="lower_right", scale=scale,
                           device=DEV, name=f"scale{scale}-staged")
    elif kind == "fp8_qdq":
        c = _case(seed, qf="padded_bhnd", kf="padded_bhnd", causal="upper_left", mask="bool",
                  dtype=torch.float8_e4m3fn, qdq="fp8", qmax=120, kvmax=140, scale=scale)
    else:
        c = _case(seed, qf="packed_nhd", kf="packed_nhd",
                  causal="none" if kind == "none" else "lower_right",
                  mask="f32" if kind == "f32_mask" else None,
                  norm="none" if kind == "none" else "softmax", scale=scale)
    parity.compare(c, parity.run_gpu(c))


@pytest.mark.parametrize("mask", ["bool", "f16", "bf16"])
@pytest.mark.parametrize("norm,qdq", [("softmax", "fp8"), ("none", "fp8")])
def test_fp8_staged_masks(mask, norm, qdq):
    # fp8 kernels stage head-broadcast masks as fp32 raw-score biases that
    # initialize the score accumulators: bool (0 / -inf), additive f16 / bf16
    # values (some -inf), under each normalization.
    seed = 280 + ["bool", "f16", "bf16"].index(mask) * 2 + ["softmax", "none"].index(norm)
    ql = np.array([31, 1, 70, 33, 17])
    kl = np.array([301, 40, 333, 77, 19])
    c = synth.generate(seed=seed, q_lens=ql, kv_lens=np.maximum(kl, ql), num_heads=8,
                       kv_num_heads=2, head_dim=128, query_form="packed_nhd",
                       kv_form="padded_bhnd", n_kv=640, q_slack=2, kv_slack=0,
                       dtype=torch.float8_e4m3fn, dist="round_normal", mask_kind=mask,
                       mask_p=0.2, mask_value=-3.0 if seed % 2 else -float("inf"),
                       mask_diag_true=True, causal_kind="lower_right", norm=norm, qdq=qdq,
                       qscale=float(np.float32(1 / 448.0)), device=DEV,
                       name=f"fp8-staged-{mask}-{norm}-{qdq}")
    parity.compare(c, parity.run_gpu(c))


@pytest.mark.parametrize("D,qscale", [(64, 1 / 448.0), (64, 1 / 2000.0), (128, 1 / 2000.0)])
def test_fp8_bool_mask_kernels(D, qscale):
    # fp8 kernels with a staged bool mask (bool known at compile time, three
    # workgroups per CU) in both Q/DQ variants: a small qscale keeps the
    # quantizer's clamp, 1/448 takes the clamp-free one; ragged rows and
    # keys, a mask with rows of no allowed key besides the forced diagonal.
    seed = 290 + D + int(1 / qscale) % 13
    ql = np.array([45, 1, 96, 0, 33, 64])
    kl = np.array([301, 40, 333, 19, 77, 64])
    c = synth.generate(seed=seed, q_lens=ql, kv_lens=np.maximum(kl, ql), num_heads=8,
                       kv_num_heads=2, head_dim=D, query_form="packed_nhd",
                       kv_form="padded_bhnd", n_kv=352, q_slack=2, kv_slack=0,
                       dtype=torch.float8_e4m3fn, dist="round_normal", mask_kind="bool",
                       mask_p=0.35, mask_diag_true=True, causal_kind="lower_right",
                       norm="softmax", qdq="fp8", qscale=float(np.float32(qscale)),
                       device=DEV, name=f"fp8-bool-D{D}-{int(1 / qscale)}")
    parity.compare(c, parity.run_gpu(c), amb_rel=1e-4)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("heads", [(4, 4), (8, 4), (8, 2), (8, 1), (12, 4), (6, 2)])
def test_head_groups_and_head_size(D, heads):
    hq, hkv = heads
    c = _case(300 + D + hq * 3 + hkv, qf="packed_nhd", kf="packed_nhd", causal="lower_right",
              D=D, hq=hq, hkv=hkv, dtype=torch.bfloat16)
    parity.compare(c, parity.run_gpu(c))


@pytest.mark.parametrize("B", [13, 20, 32, 40, 64])
def test_dispatch_map_batch_sizes(B):
    # The row-tile map sorts the sequences over 16, 32 or 64 lanes depending
    # on the batch: every size class, with empty sequences and ties in KV
    # length, each output row written exactly once.
    rng = np.random.default_rng(4000 + B)
    ql = rng.integers(0, 70, size=B)
    kl = rng.choice([0, 1, 40, 96, 97, 150], size=B)
    kl = np.maximum(kl, ql)
    c = synth.generate(seed=4000 + B, q_lens=ql, kv_lens=kl, num_heads=8, kv_num_heads=2,
                       head_dim=64, query_form="packed_nhd",
                       kv_form="padded_bhnd" if B % 2 else "packed_nhd",
                       causal_kind="lower_right", q_slack=3, kv_slack=3, device=DEV,
                       name=f"map-B{B}")
    parity.compare(c, parity.run_gpu(c))


def test_ragged_with_empty_sequences():
    c = synth.generate(seed=401, q_lens=[0, 5, 0, 64, 1, 33], kv_lens=[3, 0, 0, 70, 1, 200],
                       num_heads=8, kv_num_heads=2, head_dim=128, query_form="packed_nhd",
                       kv_form="packed_nhd", causal_kind="lower_right", q_slack=4, kv_slack=4,
                       device=DEV, name="empties")
    out = parity.run_gpu(c)
    parity.compare(c, out)


@pytest.mark.parametrize("norm,qdq", [("none", None), ("none", "fp8"), ("none", "int8"),
                                      ("softmax", "fp8"), ("softmax", "int8")])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_norm_and_qdq_16bit(norm, qdq, dtype):
    seed = 500 + ["none", "softmax"].index(norm) * 10 + [None, "fp8", "int8"].index(qdq)
    c = _case(seed, qf="padded_bhnd", kf="packed_nhd", causal="upper_left", mask="bool",
              dtype=dtype, norm=norm, qdq=qdq, qmax=90, kvmax=120)
    parity.compare(c, parity.run_gpu(c), amb_rel=1e-4)


@pytest.mark.parametrize("causal,mask", [("upper_left", None), ("upper_left", "bool"),
                                         ("none", None), ("lower_right", "f16")])
@pytest.mark.parametrize("D", [64, 128])
def test_fp8_quantized(causal, mask, D):
    seed = 600 + D + ["upper_left", "none", "lower_right"].index(causal) * 3 + (mask is not None)
    c = _case(seed, qf="padded_bhnd", kf="padded_bhnd", causal=causal, mask=mask,
              dtype=torch.float8_e4m3fn, D=D, qdq="fp8", qmax=200, kvmax=200)
    parity.compare(c, parity.run_gpu(c))


@pytest.mark.parametrize("dtype,qdq,qscale", [
    (torch.float8_e4m3fn, "fp8", 1 / 2000.0), (torch.float16, "fp8", 1 / 1000.0),
    (torch.bfloat16, "int8", 1 / 400.0), (torch.float8_e4m3fn, "fp8", 1 / 460.0)])
def test_qdq_saturating_scales(dtype, qdq, qscale):
    # small qscale: P / qscale exceeds the format's range on the largest
    # probabilities and the quantizer saturates (the kernel keeps its clamp);
    # 1/460 is the largest range the clamp-free variant accepts
    seed = 650 + int(1 / qscale) % 97
    c = _case(seed, qf="padded_bhnd", kf="padded_bhnd", causal="upper_left", dtype=dtype,
              qdq=qdq, qscale=float(np.float32(qscale)), qmax=120, kvmax=120, B=2)
    parity.compare(c, parity.run_gpu(c), amb_rel=1e-4)


@pytest.mark.parametrize("kv", ["f16", "bf16", "fp8"])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_small(kv, D):
    rng = np.random.default_rng(700 + D)
    B = 5
    kl = rng.integers(1, 3000, size=B)
    kl[1] = 1
    dtype = torch.bfloat16 if kv == "bf16" else torch.float16
    c = synth.generate(seed=700 + D, q_lens=np.ones(B, int), kv_lens=kl, num_heads=8,
                       kv_num_heads=2, head_dim=D, n_q=1, n_kv=int(kl.max()) + 9, dtype=dtype,
                       pass_query_lengths=False,
                       kv_fp8_from=torch.float16 if kv == "fp8" else None,
                       kv_dtype=torch.float8_e4m3fn if kv == "fp8" else None, device=DEV,
                       name=f"decode-{kv}-{D}")
    parity.compare(c, parity.run_gpu(c))


def test_decode_with_query_lengths_skips_rows():
    c = synth.generate(seed=710, q_lens=[1, 0, 1], kv_lens=[40, 50, 0], num_heads=4,
                       kv_num_heads=1, head_dim=128, n_q=1, n_kv=64, pass_query_lengths=True,
                       device=DEV, name="decode-ql")
    parity.compare(c, parity.run_gpu(c))


def test_packed_equals_padded_bitwise_and_deterministic():
    c = _case(801, qf="padded_bhnd", kf="padded_bhnd", causal="lower_right", mask="f16",
              dtype=torch.bfloat16, n_q_pad=None)
    a = parity.run_gpu(c)
    a2 = parity.run_gpu(c)
    assert torch.equal(a.view(torch.int16), a2.view(torch.int16))
    ql = np.concatenate([[0], np.cumsum(c.q_lens)]).astype(np.int32)
    kl = np.concatenate([[0], np.cumsum(c.kv_lens)]).astype(np.int32)
    qp = torch.cat([c.q[b, :, :c.q_lens[b]].transpose(0, 1) for b in range(c.batch)]).contiguous()
    kp = torch.cat([c.k[b, :, :c.kv_lens[b]].transpose(0, 1) for b in range(c.batch)]).contiguous()
    vp = torch.cat([c.v[b, :, :c.kv_lens[b]].transpose(0, 1) for b in range(c.batch)]).contiguous()
    kw = c.kwargs()
    kw.update(query_form="packed_nhd", kv_form="packed_nhd",
              query_lengths=torch.from_numpy(ql).to(DEV), kv_lengths=torch.from_numpy(kl).to(DEV))
    b2 = capi.attn_forward(qp, kp, vp, c.mask, **kw)
    torch.cuda.synchronize()
    for b in range(c.batch):
        x = a[b, :, :c.q_lens[b]].transpose(0, 1)
        y = b2[ql[b]:ql[b + 1]]
        assert torch.equal(x.contiguous().view(torch.int16), y.view(torch.int16)), b


# ---------------------------------------------------------------- full sizes
@pytest.mark.parametrize("cfg", ["2", "3", "4a", "4b", "5a", "5b"])
def test_workload_sampled(cfg):
    c = synth.make_config(cfg, device=DEV)
    out = parity.run_gpu(c)
    rows = parity.sample_rows(c, n_per_seq=6 if c.batch <= 16 else 1, seed=int(cfg[0]))
    st = parity.compare(c, out, rows=rows)
    assert st["rows"] > 0
    # no NaN anywhere in the valid rows of the output (padding poisoned with NaN)
    if c.query_form == "packed_nhd":
        assert not torch.isnan(out[: int(np.sum(c.q_lens))].float()).any()
    else:
        assert not torch.isnan(out.float()).any()


# ------------------------------------------------------------- split-KV prefill
@pytest.mark.parametrize("heads", [(8, 4), (4, 4), (6, 2)])
def test_split_kv_prefill_row_tiles(heads):
    # split-KV with 64- and 128-row workgroups (group sizes 2 and 1) and a
    # group of 3 heads: the merge walks every row of the larger row tiles
    hq, hkv = heads
    seed = 960 + hq * 3 + hkv
    rng = np.random.default_rng(seed)
    ql = np.array([130, 3, 70])
    kl = np.maximum(np.array([3000, 900, 2100]) + rng.integers(0, 64, size=3), ql)
    c = synth.generate(seed=seed, q_lens=ql, kv_lens=kl, num_heads=hq, kv_num_heads=hkv,
                       head_dim=128, query_form="packed_nhd", kv_form="packed_nhd",
                       q_slack=2, kv_slack=2, dtype=torch.float16, causal_kind="lower_right",
                       device=DEV, name=f"splitkv-rows-{hq}/{hkv}")
    args = capi.make_args(c.q, c.k, c.v, c.mask, c.q, **c.kwargs())
    assert capi.gqa_attn_workspace_size(args) > 0  # the split path is taken
    parity.compare(c, parity.run_gpu(c))


@pytest.mark.parametrize("causal,mask", [("lower_right", None), ("lower_right", "f16"),
                                         ("none", "bool"), ("upper_left", None)])
@pytest.mark.parametrize("dtype,D", [(torch.float16, 128), (torch.bfloat16, 64)])
def test_split_kv_prefill(causal, mask, dtype, D):
    # few query rows over long keys: the host splits the keys of each query
    # tile over several workgroups and merges the partials
    seed = 900 + D + ["lower_right", "none", "upper_left"].index(causal) * 3 + (mask is not None)
    rng = np.random.default_rng(seed)
    ql = np.array([37, 0, 5, 64])
    kl = np.array([2900, 100, 5, 1500]) + rng.integers(0, 64, size=4)
    if causal == "lower_right":
        kl = np.maximum(kl, ql)
    c = synth.generate(seed=seed, q_lens=ql, kv_lens=kl, num_heads=8, kv_num_heads=2,
                       head_dim=D, query_form="packed_nhd", kv_form="padded_bhnd",
                       n_kv=int(kl.max()) + 3, q_slack=2, dtype=dtype, mask_kind=mask,
                       mask_p=0.2, mask_diag_true=True, causal_kind=causal, device=DEV,
                       name=f"splitkv-{causal}-{mask}-{D}")
    args = capi.make_args(c.q, c.k, c.v, c.mask, c.q, **c.kwargs())
    assert capi.gqa_attn_workspace_size(args) > 0  # the split path is taken
    parity.compare(c, parity.run_gpu(c))

