"""Dense brute-force evaluation of the attention operator for tiny inputs.

An independent formulation used only to pin the oracle: it decodes every
tensor with torch's own dtype conversions, unpacks packed forms into a
dense padded layout, materialises the full score matrix, the causal,
length and mask predicates as dense boolean arrays, and evaluates the
operator with numpy float64 matrix products.  It shares nothing with the
oracle's C code.  Follows the onnx-tensorrt "TensorRT Custom Operator
Schemas" page, sections TRT_Attention and TRT_QuantizedAttention, under
the same readings the oracle documents.
"""
from __future__ import annotations

import numpy as np
import torch


def _f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.float8_e4m3fn:
        return t.float().double().numpy()
    return t.double().numpy()


def _tree_allowed(case, b: int, L: int, kv: int, nq: int, nk: int) -> np.ndarray:
    """[nq, nk] bool: the tree-decoding rule for sequence b (TensorRT
    Edge-LLM "TensorRT Plugins Guide", AttentionPlugin, tree decoding).
    Formulated as a reachability closure instead of a parent walk: E[u, p]
    marks the edge draft u -> parent p (p in [0, u-1]); R = (I + E)^(L)
    under boolean matrix products gives R[i, t] = t is draft i or one of its
    ancestors.  Context keys (j < kv - L) are always allowed."""
    tp = case.tree_parents.cpu().numpy().astype(np.int64)
    row0 = int(np.sum(case.q_lens[:b])) if case.query_form == "packed_nhd" else b * case.q.shape[2]
    par = tp[row0:row0 + L]
    E = np.zeros((L, L), dtype=np.int64)
    for u in range(L):
        if 0 <= par[u] < u:
            E[u, par[u]] = 1
    R = np.eye(L, dtype=np.int64)
    step = np.eye(L, dtype=np.int64) + E
    for _ in range(max(L, 1)):
        R = np.minimum(R @ step, 1)
    out = np.ones((nq, nk), dtype=bool)
    base = kv - L
    for jj in range(max(base, 0), min(kv, nk)):
        t = jj - base
        out[:L, jj] = R[:, t].astype(bool)
    return out


def dense(case) -> tuple[np.ndarray, np.ndarray]:
    """(Y [B, Hq, Nq, D] float64, valid [B, Hq, Nq] bool) for a host Case."""
    B, Hq, Hkv = case.batch, case.num_heads, case.kv_num_heads
    ql, kl = np.asarray(case.q_lens), np.asarray(case.kv_lens)
    nq = max(1, int(ql.max(initial=0)))
    nk = max(1, int(kl.max(initial=0)))
    q = _f64(case.q)
    k = _f64(case.k) * case.k_descale
    v = _f64(case.v) * case.v_descale
    D = q.shape[-1]

    def unpack(x, form, lens, n):
        out = np.zeros((B, x.shape[1] if form == "packed_nhd" else x.shape[1], n, D))
        if form == "packed_nhd":
            starts = np.concatenate([[0], np.cumsum(lens)])
            for b in range(B):
                L = int(lens[b])
                out[b, :, :L] = np.transpose(x[starts[b]:starts[b] + L], (1, 0, 2))
        else:
            for b in range(B):
                L = int(lens[b])
                out[b, :, :L] = x[b, :, :L]
        return out

    def unpage(x, w):
        # paged KV: key j of sequence b is row j % ps of page table[b, w, j // ps]
        ps = x.shape[2]
        tab = case.kv_page_table.cpu().numpy()
        out = np.zeros((B, x.shape[1], nk, D))
        for b in range(B):
            for jj in range(int(kl[b])):
                out[b, :, jj] = x[tab[b, w, jj // ps], :, jj % ps]
        return out

    Q = unpack(q, case.query_form, ql, nq)                 # [B, Hq, nq, D]
    if case.kv_form == "paged":
        K, V = unpage(k, 0), unpage(v, 1)
    else:
        K = unpack(k, case.kv_form, kl, nk)                # [B, Hkv, nk, D]
        V = unpack(v, case.kv_form, kl, nk)
    G = Hq // Hkv
    K = np.repeat(K, G, axis=1)
    V = np.repeat(V, G, axis=1)
    S = np.float64(np.float32(case.scale)) * (Q @ np.swapaxes(K, -1, -2))   # [B,Hq,nq,nk]

    i = np.arange(nq)[:, None]
    j = np.arange(nk)[None, :]
    allowed = np.zeros((B, Hq, nq, nk), dtype=bool)
    for b in range(B):
        a = (j < kl[b]) & (i < ql[b])
        if case.causal_kind == "upper_left":
            a &= j <= i
        elif case.causal_kind == "lower_right":
            a &= j <= i + (kl[b] - ql[b])
        if case.tree_parents is not None:
            a &= _tree_allowed(case, b, int(ql[b]), int(kl[b]), nq, nk)
        allowed[b] = a

    if case.mask is not None:
        m = case.mask
        m = m.numpy() if m.dtype == torch.bool else m.double().numpy()
        m = m.reshape((1,) * (4 - m.ndim) + m.shape)
        m = np.broadcast_to(m, (B, Hq, max(m.shape[2], 1), max(m.shape[3], 1)))
        # pad / crop the query and key axes to the dense size
        mq = np.zeros((B, Hq, nq, nk), dtype=m.dtype)
        if m.shape[2] == 1:
            m = np.broadcast_to(m, (B, Hq, nq, m.shape[3]))
        if m.shape[3] == 1:
            m = np.broadcast_to(m, (B, Hq, m.shape[2], nk))
        r, c = min(nq, m.shape[2]), min(nk, m.shape[3])
        mq[:, :, :r, :c] = m[:, :, :r, :c]
        if case.mask.dtype == torch.bool:
            allowed &= mq.astype(bool)
        else:
            allowed &= ~np.isneginf(mq)
            S = S + np.where(allowed, mq, 0.0)

    has_any = allowed.any(axis=-1, keepdims=True)
    if case.norm == "softmax":
        Sm = np.where(allowed, S, -np.inf)
        mx = np.where(has_any, Sm.max(axis=-1, keepdims=True), 0.0)
        E = np.where(allowed, np.exp(Sm - mx), 0.0)
        den = E.sum(axis=-1, keepdims=True)
        P = np.where(has_any, E / np.where(den == 0, 1.0, den), 0.0)
    else:
        P = np.where(allowed, S, 0.0)

    if case.qdq is not None:
        qs = np.float64(np.float32(case.qscale))
        x = P / qs
        if case.qdq == "fp8":
            xs = np.clip(x, -448.0, 448.0)
            c = torch.from_numpy(xs).to(torch.float8_e4m3fn).double().numpy()
        else:
            c = np.clip(np.rint(x), -128.0, 127.0)
        P = np.where(allowed, c * qs, 0.0)

    Y = P @ V
    valid = np.zeros((B, Hq, nq), dtype=bool)
    for b in range(B):
        valid[b, :, :ql[b]] = True
    return Y, valid
