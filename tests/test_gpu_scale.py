"""GPU parity at sizes and shapes the other suites do not reach: more than
64 sequences (the tile map's index-order path), a long causal sequence, a
long decode context, multi-query attention with 32 query heads per KV head
(beyond the decode kernel's 16, so it runs the prefill kernel with one query
row), and group sizes 8 and 16 in the decode kernel.  Sampled rows are
compared with the oracle computed row by row; inputs are seeded and
synthetic."""
import numpy as np
import pytest
import torch

from gqa_attention_ragged_amd import synth
from tests import parity

pytestmark = pytest.mark.gpu

DEV = "cuda"


def test_many_sequences_prefill():
    # 150 ragged sequences (more than the 64 the sorted tile map handles)
    rng = np.random.default_rng(5001)
    L = rng.integers(1, 200, size=150)
    L[::17] = 0
    c = synth.generate(seed=5001, q_lens=L, kv_lens=L, num_heads=8, kv_num_heads=2,
                       head_dim=128, query_form="packed_nhd", kv_form="packed_nhd",
                       dtype=torch.bfloat16, causal_kind="lower_right", q_slack=3, kv_slack=3,
                       device=DEV, name="many-seqs")
    out = parity.run_gpu(c)
    parity.compare(c, out, rows=parity.sample_rows(c, n_per_seq=1, seed=1))
    n = int(np.sum(L))
    assert not torch.isnan(out[:n].float()).any()


def test_long_causal_sequence():
    # one 32768-token causal sequence (512 row tiles per head group)
    c = synth.generate(seed=5002, q_lens=[32768], kv_lens=[32768], num_heads=8, kv_num_heads=2,
                       head_dim=128, query_form="packed_nhd", kv_form="packed_nhd",
                       dtype=torch.bfloat16, causal_kind="lower_right", device=DEV,
                       name="long-causal")
    out = parity.run_gpu(c)
    rows = np.array([(0, h, i) for h in (0, 7) for i in (0, 1, 63, 64, 4095, 20000, 32767)],
                    dtype=np.int32)
    parity.compare(c, out, rows=rows)


def test_long_decode_context():
    # 131072 keys per sequence: 32 splits of 4096 keys
    c = synth.generate(seed=5003, q_lens=[1, 1], kv_lens=[131072, 70001], num_heads=8,
                       kv_num_heads=2, head_dim=128, n_q=1, n_kv=131072, dtype=torch.float16,
                       pass_query_lengths=False, device=DEV, name="long-decode")
    parity.compare(c, parity.run_gpu(c))


@pytest.mark.parametrize("hq,hkv", [(32, 1), (16, 1), (64, 8)])
def test_decode_large_groups(hq, hkv):
    rng = np.random.default_rng(5004 + hq)
    kl = rng.integers(1, 5000, size=3)
    c = synth.generate(seed=5004 + hq, q_lens=np.ones(3, int), kv_lens=kl, num_heads=hq,
                       kv_num_heads=hkv, head_dim=128, n_q=1, n_kv=int(kl.max()) + 3,
                       dtype=torch.bfloat16, pass_query_lengths=False, device=DEV,
                       name=f"decode-g{hq // hkv}")
    parity.compare(c, parity.run_gpu(c))


def test_mqa_prefill_group_32():
    c = synth.generate(seed=5005, q_lens=[70, 1, 130], kv_lens=[200, 90, 130], num_heads=32,
                       kv_num_heads=1, head_dim=64, query_form="packed_nhd",
                       kv_form="padded_bhnd", n_kv=210, dtype=torch.float16,
                       causal_kind="lower_right", device=DEV, name="mqa-prefill")
    parity.compare(c, parity.run_gpu(c))
