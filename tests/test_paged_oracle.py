"""Pins of the oracle's paged-KV addressing (TensorRT Edge-LLM "TensorRT
Plugins Guide", AttentionPlugin decoder tensor contract: kv_page_table
[N, 2, max_pages_per_sequence]) on the CPU: the same data as padded KV and as
page pools give identical results, and the whole operator matches the dense
brute force, which un-pages with its own gather."""
import zlib

import numpy as np
import pytest
import torch

from gqa_attention_ragged_amd import synth
from bruteforce import dense


def _paged_case(seed, qf, causal, mask, ps, kv_form="paged", tree=None, dtype=torch.float16):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 4))
    ql = rng.integers(0, 10, size=B)
    kl = rng.integers(0, 3 * ps + 5, size=B)
    if causal == "lower_right" or tree:
        kl = np.maximum(kl, ql)
    D = 8 if seed % 2 else 16
    return synth.generate(
        seed=seed, q_lens=ql, kv_lens=kl, num_heads=4, kv_num_heads=2, head_dim=D,
        query_form=qf, kv_form=kv_form, dtype=dtype, n_q=int(ql.max()) + 2,
        n_kv=int(kl.max()) + 3, q_slack=1, pass_query_lengths=True, mask_kind=mask, mask_p=0.3,
        causal_kind=causal,
        scale=0.4, page_size=ps, tree=tree, name=f"paged{seed}")


@pytest.mark.parametrize("qf", ["padded_bhnd", "packed_nhd"])
@pytest.mark.parametrize("causal,mask", [("none", None), ("lower_right", None), ("upper_left", "bool"),
                                         ("none", "f16")])
@pytest.mark.parametrize("ps", [4, 8, 16])
def test_paged_vs_bruteforce(oracle_mod, qf, causal, mask, ps):
    for s in range(2):
        seed = zlib.crc32(repr((qf, causal, mask, ps, s)).encode()) % 100000
        c = _paged_case(seed, qf, causal, mask, ps)
        res = oracle_mod.attention(c.q, c.k, c.v, c.mask, **c.kwargs())
        Y, valid = dense(c)
        b, h, i = res.rows[:, 0], res.rows[:, 1], res.rows[:, 2]
        assert len(res.rows) == int(valid.sum())
        ref = Y[b, h, i]
        assert np.all(np.abs(res.out - ref) <= 1e-12 * (1 + np.abs(ref))), c.name


@pytest.mark.parametrize("ps", [4, 16])
def test_paged_equals_padded(oracle_mod, ps):
    """Drawn from the same seed, the paged case holds exactly the padded
    case's K/V rows, scattered over pages: the fp64 results are identical."""
    for s in range(3):
        seed = 500 + 10 * ps + s
        a = _paged_case(seed, "packed_nhd", "lower_right", None, ps, kv_form="padded_bhnd")
        b = _paged_case(seed, "packed_nhd", "lower_right", None, ps)
        assert b.kv_form == "paged" and b.kv_page_table is not None
        ra = oracle_mod.attention(a.q, a.k, a.v, a.mask, **a.kwargs())
        rb = oracle_mod.attention(b.q, b.k, b.v, b.mask, **b.kwargs())
        assert np.array_equal(ra.rows, rb.rows)
        assert np.array_equal(ra.out, rb.out)


def test_paged_tree_vs_bruteforce(oracle_mod):
    for s in range(3):
        c = _paged_case(700 + s, "packed_nhd", "none", None, 8, tree="spec")
        res = oracle_mod.attention(c.q, c.k, c.v, c.mask, **c.kwargs())
        Y, _ = dense(c)
        ref = Y[res.rows[:, 0], res.rows[:, 1], res.rows[:, 2]]
        assert np.all(np.abs(res.out - ref) <= 1e-12 * (1 + np.abs(ref)))


def test_paged_prefix_means(oracle_mod):
    """Closed form: Q = 0 makes every allowed score equal, so a lower_right
    causal row i of a sequence with q_len = kv_len is the mean of V over keys
    0..i, wherever the pages of those keys sit in the pool."""
    c = _paged_case(900, "padded_bhnd", "lower_right", None, 4)
    c.q = torch.zeros_like(c.q)
    res = oracle_mod.attention(c.q, c.k, c.v, c.mask, **c.kwargs())
    tab = c.kv_page_table.numpy()
    vp = c.v.double().numpy()
    ps = c.v.shape[2]
    for (b, h, i), o in zip(res.rows, res.out):
        diag = int(c.kv_lens[b]) - int(c.q_lens[b])
        keys = range(0, min(int(c.kv_lens[b]), i + diag + 1))
        if not len(keys):
            assert np.all(o == 0)
            continue
        g = h // 2
        rows = np.stack([vp[tab[b, 1, j // ps], g, j % ps] for j in keys])
        assert np.allclose(o, rows.mean(axis=0), rtol=0, atol=1e-12)
