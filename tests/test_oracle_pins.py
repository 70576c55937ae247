"""Pins of the CPU oracle against things other than itself (CPU only).

- storage formats: every f16 / bf16 / E4M3FN code against torch's casts;
- the Q/DQ rounding: dense fp32 sweeps against torch's E4M3FN cast and
  numpy's round-half-even, plus the saturation reading;
- the whole operator: a dense numpy brute force (tests/bruteforce.py) on
  tiny inputs over every feature combination;
- a library special case: torch's scaled_dot_product_attention in float64;
- invariants and closed forms (rows sum to one, GQA = MHA on repeated KV,
  packed = padded, upper_left = lower_right when lengths match, one-key
  rows echo V, Q = 0 gives the mean of the allowed V);
- hand-derived golden cases under tests/golden/.
"""
import itertools
import json
import math
import os
import zlib

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from gqa_attention_ragged_amd import synth
from tests.bruteforce import dense

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- formats
@pytest.mark.parametrize("dt", [torch.float16, torch.bfloat16])
def test_decode_16bit_all_codes(oracle_mod, dt):
    codes = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    ref = codes.view(dt).double().numpy()
    got = np.array([oracle_mod.decode(dt, c) for c in range(65536)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def test_decode_e4m3_all_codes(oracle_mod):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).float().double().numpy()
    got = np.array([oracle_mod.decode(torch.float8_e4m3fn, c) for c in range(256)])
    nan = np.isnan(ref)
    assert nan.sum() == 2  # S.1111.111 only
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def _fp8_sweep():
    vals = torch.arange(127, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    vals = vals.float().numpy().astype(np.float64)
    mids = 0.5 * (vals[:-1] + vals[1:])
    rng = np.random.default_rng(0)
    rand = rng.uniform(0, 448, 20000)
    near = np.concatenate([np.nextafter(mids.astype(np.float32), np.float32(0)),
                           np.nextafter(mids.astype(np.float32), np.float32(1000))])
    x = np.concatenate([vals, mids, rand, near]).astype(np.float32)
    return np.concatenate([x, -x])


def test_quantize_fp8_matches_torch_in_range(oracle_mod):
    x = _fp8_sweep()
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).float().double().numpy()
    got = np.array([oracle_mod.quantize("fp8", float(v))[0] for v in x])
    assert np.array_equal(ref, got)


def test_quantize_fp8_saturates_and_flags_midpoints(oracle_mod):
    for v in (448.0, 460.0, 464.0, 500.0, 1e6):
        assert oracle_mod.quantize("fp8", v)[0] == 448.0
        assert oracle_mod.quantize("fp8", -v)[0] == -448.0
    # exact midpoint between 1.0 and 1.125 -> even code (1.0), gap flagged
    r, d = oracle_mod.quantize("fp8", 1.0625, 1e-6)
    assert r == 1.0 and d == 0.125
    # between 1.125 and 1.25: tie goes to the even code 1.25
    r, d = oracle_mod.quantize("fp8", 1.1875, 1e-6)
    assert r == 1.25 and d == 0.125
    r, d = oracle_mod.quantize("fp8", 1.1, 1e-6)
    assert r == 1.125 and d == 0.0


def test_quantize_int8_matches_numpy(oracle_mod):
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.uniform(-300, 300, 20000), np.arange(-200, 200) + 0.5,
                        np.arange(-200, 200).astype(np.float64)])
    ref = np.clip(np.rint(x), -128, 127)
    got = np.array([oracle_mod.quantize("int8", float(v))[0] for v in x])
    assert np.array_equal(ref, got)
    assert oracle_mod.quantize("int8", 2.5, 1e-6) == (2.0, 1.0)


# ---------------------------------------------------------- brute force
def _run_oracle(oracle_mod, c, amb_rel=1e-6):
    res = oracle_mod.attention(c.q, c.k, c.v, c.mask, amb_rel=amb_rel, **c.kwargs())
    return res


def _compare_dense(oracle_mod, c, atol=1e-12):
    res = _run_oracle(oracle_mod, c)
    Y, valid = dense(c)
    b, h, i = res.rows[:, 0], res.rows[:, 1], res.rows[:, 2]
    assert len(res.rows) == int(valid.sum())
    ref = Y[b, h, i]
    err = np.abs(res.out - ref)
    lim = atol * (1 + np.abs(ref)) + res.amb
    assert np.all(err <= lim), (c.name, float(err.max()))
    return res


def _tiny_case(seed, qf, kf, causal, mask, norm, qdq, hq, hkv, dtype, zero_lengths=True):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 4))
    ql = rng.integers(0 if zero_lengths else 1, 12, size=B)
    kl = rng.integers(0 if zero_lengths else 1, 14, size=B)
    if causal == "lower_right":
        kl = np.maximum(kl, ql)  # keep most rows non-empty; empties covered elsewhere
    D = 8 if seed % 2 else 16
    kind = {None: None, "bool": "bool", "add": ["f16", "bf16", "f32"][seed % 3]}[mask]
    n_q = int(ql.max()) + 2
    pass_ql = True if qf == "packed_nhd" else bool(seed % 2)
    if not pass_ql:
        ql = np.full(B, n_q)  # padded Q without query_lengths: every row is valid
        if causal == "lower_right":
            kl = np.maximum(kl, ql)
    return synth.generate(
        seed=seed, q_lens=ql, kv_lens=kl, num_heads=hq, kv_num_heads=hkv, head_dim=D,
        query_form=qf, kv_form=kf, dtype=dtype, n_q=n_q, n_kv=int(kl.max()) + 3,
        q_slack=2, kv_slack=1, pass_query_lengths=pass_ql,
        mask_kind=kind, mask_heads=hq if seed % 2 else 1, mask_p=0.3,
        mask_value=-3.0 if seed % 5 else -float("inf"), causal_kind=causal, norm=norm, qdq=qdq,
        qscale=float(np.float32(1 / 448.0)) if qdq == "fp8" else (1 / 64.0 if qdq else 1.0),
        scale=0.3 + 0.05 * (seed % 7), name=f"tiny{seed}")


FORMS = ["padded_bhnd", "packed_nhd"]


@pytest.mark.parametrize("qf,kf", list(itertools.product(FORMS, FORMS)))
@pytest.mark.parametrize("causal", ["none", "upper_left", "lower_right"])
@pytest.mark.parametrize("mask", [None, "bool", "add"])
def test_oracle_vs_bruteforce_forms_causal_mask(oracle_mod, qf, kf, causal, mask):
    for s in range(3):
        seed = zlib.crc32(repr((qf, kf, causal, mask, s)).encode()) % 100000
        hq, hkv = [(1, 1), (4, 2), (8, 2), (4, 1)][seed % 4]
        c = _tiny_case(seed, qf, kf, causal, mask, "softmax", None, hq, hkv, torch.float16)
        _compare_dense(oracle_mod, c)


@pytest.mark.parametrize("norm", ["softmax", "none"])
@pytest.mark.parametrize("qdq", [None, "fp8", "int8"])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16, torch.float8_e4m3fn])
def test_oracle_vs_bruteforce_norm_qdq_dtype(oracle_mod, norm, qdq, dtype):
    for s in range(3):
        seed = 17 * s + 3 + (7 if norm == "none" else 0)
        qf, kf = FORMS[s % 2], FORMS[(s // 2) % 2]
        causal = ["none", "upper_left", "lower_right"][s]
        mask = [None, "bool", "add"][(s + 1) % 3]
        c = _tiny_case(seed, qf, kf, causal, mask, norm, qdq, 4, 2, dtype)
        _compare_dense(oracle_mod, c)


def test_oracle_vs_bruteforce_fp8_kv_descale(oracle_mod):
    c = synth.generate(seed=11, q_lens=[1, 1, 1], kv_lens=[5, 17, 9], num_heads=8,
                       kv_num_heads=2, head_dim=16, n_q=1, n_kv=20, dtype=torch.float16,
                       kv_dtype=torch.float8_e4m3fn, kv_fp8_from=torch.float16)
    assert c.k_descale != 1.0 and c.v_descale != 1.0
    _compare_dense(oracle_mod, c)


def test_padding_rows_not_listed(oracle_mod):
    c = _tiny_case(5, "padded_bhnd", "packed_nhd", "none", None, "softmax", None, 4, 2,
                   torch.float16)
    rows = oracle_mod.list_rows(c.q, c.k, c.v, **{k: c.kwargs()[k] for k in (
        "query_lengths", "kv_lengths", "batch", "query_form", "kv_form", "num_heads",
        "kv_num_heads")})
    assert len(rows) == int(np.sum(c.q_lens)) * c.num_heads
    for b, h, i in rows:
        assert i < c.q_lens[b]


# -------------------------------------------------- library special case
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("mask", [None, "bool", "add"])
@pytest.mark.parametrize("heads", [(4, 4), (8, 2)])
def test_oracle_vs_torch_sdpa(oracle_mod, causal, mask, heads):
    hq, hkv = heads
    c = synth.generate(seed=21, q_lens=[24, 24], kv_lens=[24, 24], num_heads=hq,
                       kv_num_heads=hkv, head_dim=32, dtype=torch.float16,
                       causal_kind="upper_left" if causal else "none",
                       mask_kind=None if mask is None else ("bool" if mask == "bool" else "f32"),
                       mask_heads=hq, mask_p=0.2, mask_value=-2.5, mask_diag_true=True,
                       pass_kv_lengths=False, scale=0.2)
    res = oracle_mod.attention(c.q, c.k, c.v, c.mask, **c.kwargs())
    am = None
    if c.mask is not None:
        am = c.mask if c.mask.dtype == torch.bool else c.mask.double()
    ref = F.scaled_dot_product_attention(
        c.q.double(), c.k.double(), c.v.double(), attn_mask=am, is_causal=causal,
        scale=float(np.float32(c.scale)), enable_gqa=hq != hkv).numpy()
    b, h, i = res.rows.T
    assert np.allclose(res.out, ref[b, h, i], rtol=0, atol=1e-12)


# ------------------------------------------------- invariants / closed forms
def test_rows_sum_to_one_with_unit_v(oracle_mod):
    c = _tiny_case(31, "packed_nhd", "padded_bhnd", "lower_right", "add", "softmax", None, 4, 2,
                   torch.float16, zero_lengths=False)
    c.v = torch.ones_like(c.v)
    res = _run_oracle(oracle_mod, c)
    has = res.nallowed > 0
    assert has.any()
    assert np.allclose(res.out[has], 1.0, rtol=0, atol=1e-13)
    assert np.all(res.out[~has] == 0.0)


def test_none_norm_with_unit_v_sums_scores(oracle_mod):
    c = synth.generate(seed=32, q_lens=[6], kv_lens=[9], num_heads=2, kv_num_heads=1,
                       head_dim=16, causal_kind="lower_right", norm="none", scale=0.25)
    c.v = torch.ones_like(c.v)
    res = _run_oracle(oracle_mod, c)
    S = (c.q.double()[0] @ c.k.double()[0, 0].T) * float(np.float32(0.25))  # [2, 6, 9]
    for r, (b, h, i) in enumerate(res.rows):
        lim = i + (9 - 6)
        assert math.isclose(res.out[r, 0], float(S[h, i, :lim + 1].sum()), abs_tol=1e-12)


def test_gqa_equals_mha_on_repeated_kv(oracle_mod):
    c = _tiny_case(41, "packed_nhd", "packed_nhd", "lower_right", "bool", "softmax", None, 8, 2,
                   torch.bfloat16)
    a = _run_oracle(oracle_mod, c).out
    c2 = c.to_host()
    c2.k = c.k.repeat_interleave(4, dim=1)
    c2.v = c.v.repeat_interleave(4, dim=1)
    c2.kv_num_heads = 8
    b = _run_oracle(oracle_mod, c2).out
    assert np.array_equal(a, b)


def test_packed_equals_padded(oracle_mod):
    c = _tiny_case(43, "padded_bhnd", "padded_bhnd", "lower_right", "add", "softmax", "fp8", 4, 2,
                   torch.float16)
    ref = _run_oracle(oracle_mod, c)
    ql = np.concatenate([[0], np.cumsum(c.q_lens)])
    kl = np.concatenate([[0], np.cumsum(c.kv_lens)])
    qp = torch.cat([c.q[b, :, :c.q_lens[b]].transpose(0, 1) for b in range(c.batch)])
    kp = torch.cat([c.k[b, :, :c.kv_lens[b]].transpose(0, 1) for b in range(c.batch)])
    vp = torch.cat([c.v[b, :, :c.kv_lens[b]].transpose(0, 1) for b in range(c.batch)])
    c2 = c.to_host()
    c2.q, c2.k, c2.v = qp, kp, vp
    c2.query_form = c2.kv_form = "packed_nhd"
    c2.query_lengths = torch.from_numpy(ql.astype(np.int32))
    c2.kv_lengths = torch.from_numpy(kl.astype(np.int32))
    got = _run_oracle(oracle_mod, c2)
    assert np.array_equal(ref.rows, got.rows)
    assert np.array_equal(ref.out, got.out)


def test_upper_left_equals_lower_right_when_lengths_match(oracle_mod):
    c = synth.generate(seed=44, q_lens=[7, 13, 1], kv_lens=[7, 13, 1], num_heads=4,
                       kv_num_heads=2, head_dim=8, query_form="packed_nhd", kv_form="packed_nhd",
                       causal_kind="upper_left")
    a = _run_oracle(oracle_mod, c).out
    c.causal_kind = "lower_right"
    b = _run_oracle(oracle_mod, c).out
    assert np.array_equal(a, b)


def test_one_key_rows_echo_v_and_zero_q_gives_mean(oracle_mod):
    c = synth.generate(seed=45, q_lens=[5], kv_lens=[5], num_heads=2, kv_num_heads=1,
                       head_dim=8, causal_kind="upper_left")
    res = _run_oracle(oracle_mod, c)
    v = c.v.double().numpy()
    for r, (b, h, i) in enumerate(res.rows):
        if i == 0:
            assert np.array_equal(res.out[r], v[b, 0, 0])
    c.q = torch.zeros_like(c.q)
    res = _run_oracle(oracle_mod, c)
    for r, (b, h, i) in enumerate(res.rows):
        assert np.allclose(res.out[r], v[b, 0, :i + 1].mean(axis=0), rtol=0, atol=1e-14)


def test_fully_masked_rows_are_zero(oracle_mod):
    # lower_right with kv_len < q_len leaves the first rows without a key;
    # an empty KV sequence leaves every row of that sequence without a key.
    c = synth.generate(seed=46, q_lens=[6, 3], kv_lens=[2, 0], num_heads=2, kv_num_heads=2,
                       head_dim=8, n_kv=4, causal_kind="lower_right")
    res = _run_oracle(oracle_mod, c)
    for r, (b, h, i) in enumerate(res.rows):
        expect_empty = (b == 1) or (i + 2 - 6 < 0)
        assert (res.nallowed[r] == 0) == expect_empty
        if expect_empty:
            assert np.all(res.out[r] == 0.0)


# ----------------------------------------------------------- golden cases
def _load_golden():
    out = []
    for fn in sorted(os.listdir(GOLDEN)):
        if fn.startswith("attention") and fn.endswith(".json"):
            with open(os.path.join(GOLDEN, fn)) as f:
                for case in json.load(f)["cases"]:
                    out.append(pytest.param(case, id=f"{fn[:-5]}:{case['name']}"))
    return out


@pytest.mark.parametrize("g", _load_golden())
def test_golden(oracle_mod, g):
    dt = {"f16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[g["dtype"]]
    q = torch.tensor(g["q"], dtype=torch.float32).to(dt)
    k = torch.tensor(g["k"], dtype=torch.float32).to(dt)
    v = torch.tensor(g["v"], dtype=torch.float32).to(dt)
    mask = None
    if "mask" in g:
        mask = torch.tensor(g["mask"], dtype=torch.bool if g["mask_dtype"] == "bool"
                            else torch.float32)
    kw = dict(query_form=g.get("query_form", "padded_bhnd"),
              kv_form=g.get("kv_form", "padded_bhnd"), causal_kind=g.get("causal", "none"),
              norm=g.get("norm", "softmax"), qdq=g.get("qdq"),
              qscale=g.get("qscale", 1.0), scale=g.get("scale", 1.0))
    if "query_lengths" in g:
        kw["query_lengths"] = torch.tensor(g["query_lengths"], dtype=torch.int32)
    if "kv_lengths" in g:
        kw["kv_lengths"] = torch.tensor(g["kv_lengths"], dtype=torch.int32)
    res = oracle_mod.attention(q, k, v, mask, **kw)
    exp = np.array(g["expected"], dtype=np.float64)
    assert res.out.shape == exp.shape
    assert np.allclose(res.out, exp, rtol=g.get("rtol", 0.0), atol=g.get("atol", 1e-15)), (
        res.out, exp)
