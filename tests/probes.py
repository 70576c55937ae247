"""Exact-gather probes for the ragged indexing (test helper, no tests).

One-hot keys (key j of every sequence and KV head has a 1 in dimension j)
and a query row holding A = 64 in dimension t make the row's score 64 on key
t and 0 on every other allowed key, so softmax weighs key t by 1 and the
others by e^-64 (below the rounding of any output format).  V rows are
exactly representable in f16 and bf16 and differ for every sequence, KV
head, key and d % 4, so each output row must equal the V row of its picked
key bit for bit: which row that is depends on every ragged offset, the head
map and the causal alignment (onnx-tensorrt "TensorRT Custom Operator
Schemas", TRT_Attention: tensor format notation, causal_kind).
"""
from __future__ import annotations

import numpy as np
import torch

from gqa_attention_ragged_amd import synth

A = 64.0


def allowed_keys(causal: str, i: int, q_len: int, kv_len: int) -> int:
    """Number of keys (a prefix 0..n-1) row i may see."""
    if causal == "none":
        return kv_len
    if causal == "upper_left":
        return min(kv_len, i + 1)
    return max(0, min(kv_len, i + kv_len - q_len + 1))


def gather_probe(seed, qf, kf, causal, dtype, D=128, hq=8, hkv=2, device="cpu"):
    """(case, expect, kv_starts): expect[(b, h, i)] = (kv head, key) whose V
    row the output row must equal, or None for a row with no allowed key."""
    rng = np.random.default_rng(seed)
    B = 4
    ql = rng.integers(1, 100, size=B)
    kl = rng.integers(1, D + 1, size=B)  # every key its own one-hot dimension
    ql[0], kl[0] = 37, 64
    G = hq // hkv
    nq, nk = int(ql.max()) + 3, int(kl.max()) + 5
    qs = np.concatenate([[0], np.cumsum(ql)])
    ks = np.concatenate([[0], np.cumsum(kl)])

    def alloc(form, heads, n, lens):
        if form == "packed_nhd":
            return torch.full((int(np.sum(lens)) + 2, heads, D), float("nan"))
        return torch.full((B, heads, n, D), float("nan"))

    def row(t, form, starts, b, h, i):
        return t[int(starts[b]) + i, h] if form == "packed_nhd" else t[b, h, i]

    q, k, v = alloc(qf, hq, nq, ql), alloc(kf, hkv, nk, kl), alloc(kf, hkv, nk, kl)
    d_idx = torch.arange(D)
    expect = {}
    for b in range(B):
        for g in range(hkv):
            # (j + 1) * 2^e, e from d % 4, the KV head and the sequence
            scale = torch.pow(2.0, ((d_idx % 4) + 2 * g + 3 * (b % 3) - 8).float())
            for j in range(int(kl[b])):
                kr = torch.zeros(D)
                kr[j] = 1.0
                row(k, kf, ks, b, g, j)[:] = kr
                row(v, kf, ks, b, g, j)[:] = (j + 1) * scale
        for h in range(hq):
            for i in range(int(ql[b])):
                n = allowed_keys(causal, i, int(ql[b]), int(kl[b]))
                qr = torch.zeros(D)
                if n > 0:
                    t = int(rng.integers(0, n))
                    qr[t] = A
                    expect[(b, h, i)] = (h // G, t)
                else:
                    expect[(b, h, i)] = None
                row(q, qf, qs, b, h, i)[:] = qr
    to = lambda t: t.to(dtype).to(device)
    kv_lengths = ks if kf == "packed_nhd" else kl
    case = synth.Case(
        name=f"probe-{qf[:3]}-{kf[:3]}-{causal}-{dtype}", q=to(q), k=to(k), v=to(v), mask=None,
        query_lengths=torch.from_numpy(qs.astype(np.int32)).to(device),
        kv_lengths=torch.from_numpy(np.asarray(kv_lengths).astype(np.int32)).to(device),
        batch=B, query_form=qf, kv_form=kf, causal_kind=causal, norm="softmax", qdq=None,
        qscale=1.0, scale=1.0, k_descale=1.0, v_descale=1.0, num_heads=hq, kv_num_heads=hkv,
        q_lens=ql, kv_lens=kl, out_dtype=dtype)
    return case, expect, ks
