"""Pins of the oracle's tree-decoding rule (TensorRT Edge-LLM "TensorRT
Plugins Guide", AttentionPlugin: tree decoding attention) on the CPU:
hand-derived golden cases, a chain tree equals lower_right causal, and the
whole operator against the dense brute force, which builds the rule as a
reachability closure instead of the oracle's parent walk."""
import json
import os
import zlib

import numpy as np
import pytest
import torch

from gqa_attention_ragged_amd import synth
from bruteforce import dense

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tree_decoding.json")
FORMS = ["padded_bhnd", "packed_nhd"]


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_golden(oracle_mod, case):
    D = 8
    q = torch.zeros((1, 1, 3, D), dtype=torch.float16)
    k = torch.zeros((1, 1, 5, D), dtype=torch.float16)
    v = torch.zeros((1, 1, 5, D), dtype=torch.float16)
    v[0, 0, :, 0] = torch.tensor([0.0, 3.0, 6.0, 9.0, 12.0])
    res = oracle_mod.attention(q, k, v, kv_lengths=torch.tensor([5], dtype=torch.int32),
                               tree_parents=torch.tensor(case["parents"], dtype=torch.int32),
                               scale=1.0)
    assert np.allclose(res.out[:, 0], case["expect_channel0"], rtol=0, atol=1e-12)
    assert np.all(res.out[:, 1:] == 0)


def _tree_case(seed, qf, kf, causal, mask, tree, dtype=torch.float16, hq=4, hkv=2):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 4))
    ql = rng.integers(0, 12, size=B)
    kl = ql + rng.integers(0, 9, size=B)  # the drafts are the last q_len keys
    D = 8 if seed % 2 else 16
    n_q = int(ql.max()) + 2
    pass_ql = True if qf == "packed_nhd" else bool(seed % 2)
    if not pass_ql:
        ql = np.full(B, n_q)
        kl = ql + rng.integers(0, 9, size=B)
    return synth.generate(
        seed=seed, q_lens=ql, kv_lens=kl, num_heads=hq, kv_num_heads=hkv, head_dim=D,
        query_form=qf, kv_form=kf, dtype=dtype, n_q=n_q, n_kv=int(kl.max()) + 3, q_slack=2,
        kv_slack=1, pass_query_lengths=pass_ql, mask_kind=mask, mask_p=0.3,
        causal_kind=causal, scale=0.3 + 0.05 * (seed % 7), tree=tree, name=f"tree{seed}")


def _compare_dense(oracle_mod, c):
    res = oracle_mod.attention(c.q, c.k, c.v, c.mask, **c.kwargs())
    Y, valid = dense(c)
    b, h, i = res.rows[:, 0], res.rows[:, 1], res.rows[:, 2]
    assert len(res.rows) == int(valid.sum())
    ref = Y[b, h, i]
    assert np.all(np.abs(res.out - ref) <= 1e-12 * (1 + np.abs(ref))), c.name


@pytest.mark.parametrize("qf,kf", [(a, b) for a in FORMS for b in FORMS])
@pytest.mark.parametrize("tree", ["random", "spec", "star", "bad"])
@pytest.mark.parametrize("causal,mask", [("none", None), ("upper_left", None), ("none", "bool"),
                                         ("lower_right", "f16")])
def test_tree_vs_bruteforce(oracle_mod, qf, kf, tree, causal, mask):
    for s in range(2):
        seed = zlib.crc32(repr((qf, kf, tree, causal, mask, s)).encode()) % 100000
        _compare_dense(oracle_mod, _tree_case(seed, qf, kf, causal, mask, tree))


@pytest.mark.parametrize("qf", FORMS)
def test_chain_tree_is_lower_right(oracle_mod, qf):
    """A single path of drafts is ordinary lower_right causal attention: the
    allowed sets coincide, so the fp64 results are identical."""
    for s in range(4):
        c = _tree_case(100 + s, qf, "packed_nhd", "none", None, "chain")
        a = oracle_mod.attention(c.q, c.k, c.v, c.mask, **c.kwargs())
        kw = c.kwargs()
        kw.update(tree_parents=None, causal_kind="lower_right")
        b = oracle_mod.attention(c.q, c.k, c.v, c.mask, **kw)
        assert np.array_equal(a.rows, b.rows)
        assert np.array_equal(a.out, b.out)
        assert np.array_equal(a.nallowed, b.nallowed)


def test_tree_allowed_counts(oracle_mod):
    """Row i attends kv_len - q_len context keys plus depth(i) + 1 drafts."""
    c = _tree_case(7, "packed_nhd", "packed_nhd", "none", None, "spec", hq=1, hkv=1)
    res = oracle_mod.attention(c.q, c.k, c.v, c.mask, **c.kwargs())
    tp = c.tree_parents.numpy()
    starts = np.concatenate([[0], np.cumsum(c.q_lens)])
    for (b, h, i), n in zip(res.rows, res.nallowed):
        par = tp[starts[b]:starts[b] + c.q_lens[b]]
        depth, u = 0, i
        while 0 <= par[u] < u:
            u, depth = par[u], depth + 1
        assert n == c.kv_lens[b] - c.q_lens[b] + depth + 1
