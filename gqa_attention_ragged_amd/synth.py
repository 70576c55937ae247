"""Seeded synthetic inputs for the ragged GQA attention operator.

This module only draws inputs; it holds none of the operator's arithmetic.
Both the GPU library's tests and the CPU oracle consume what it produces.

Draw order (reproducible): a numpy PCG64 generator seeded with ``seed``
draws the lengths first and then the mask; a torch generator on the target
device, seeded with ``seed``, draws the Q/K/V values, sequence by sequence.

Padding is poisoned so that any read of it shows up: rows of a padded
tensor beyond a sequence's valid length, and rows of a packed tensor beyond
the last cumulative length, hold NaN.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

FP8 = torch.float8_e4m3fn
NAN_BITS = {torch.float16: 0x7E00, torch.bfloat16: 0x7FC0}
# Output sentinel: a NaN payload no arithmetic produces, so untouched rows
# can be recognised bit for bit.
SENTINEL_BITS = {torch.float16: 0x7E01, torch.bfloat16: 0x7FC1, torch.float32: 0x7FC00001}


@dataclass
class Case:
    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    mask: Optional[torch.Tensor]
    query_lengths: Optional[torch.Tensor]   # int32 cumulative [B+1] or None
    kv_lengths: Optional[torch.Tensor]      # int32 cumulative [B+1] (packed) / [B] (padded) / None
    batch: int
    query_form: str
    kv_form: str
    causal_kind: str
    norm: str
    qdq: Optional[str]
    qscale: float
    scale: float
    k_descale: float
    v_descale: float
    num_heads: int
    kv_num_heads: int
    q_lens: np.ndarray                      # per-batch valid query lengths
    kv_lens: np.ndarray                     # per-batch valid KV lengths
    out_dtype: torch.dtype
    meta: dict = field(default_factory=dict)
    tree_parents: Optional[torch.Tensor] = None  # int32, token-aligned with Q's rows, or None
    kv_page_table: Optional[torch.Tensor] = None  # int32 [B, 2, max_pages] (kv_form "paged")

    def kwargs(self) -> dict:
        """Operator arguments shared by the GPU binding and the oracle."""
        return dict(
            query_lengths=self.query_lengths, kv_lengths=self.kv_lengths, batch=self.batch,
            query_form=self.query_form, kv_form=self.kv_form, causal_kind=self.causal_kind,
            norm=self.norm, qdq=self.qdq, qscale=self.qscale, scale=self.scale,
            k_descale=self.k_descale, v_descale=self.v_descale, num_heads=self.num_heads,
            kv_num_heads=self.kv_num_heads, tree_parents=self.tree_parents,
            kv_page_table=self.kv_page_table,
        )

    def to_host(self) -> "Case":
        """Same case with every tensor copied to host memory."""
        c = Case(**{k: getattr(self, k) for k in self.__dataclass_fields__})
        for k in ("q", "k", "v", "mask", "query_lengths", "kv_lengths", "tree_parents",
                  "kv_page_table"):
            t = getattr(self, k)
            if t is not None:
                setattr(c, k, t.cpu())
        return c


def sentinel_like(shape, dtype, device) -> torch.Tensor:
    """A tensor filled with the output sentinel bit pattern."""
    if dtype == torch.float32:
        t = torch.empty(shape, dtype=torch.int32, device=device)
        t.fill_(SENTINEL_BITS[dtype])
        return t.view(torch.float32)
    t = torch.empty(shape, dtype=torch.int16, device=device)
    t.fill_(SENTINEL_BITS[dtype])
    return t.view(dtype)


def _nan_fill(shape, dtype, device) -> torch.Tensor:
    if dtype == FP8:
        t = torch.empty(shape, dtype=torch.uint8, device=device)
        t.fill_(0x7F)
        return t.view(FP8)
    if dtype == torch.float32:
        return torch.full(shape, float("nan"), dtype=dtype, device=device)
    t = torch.empty(shape, dtype=torch.int16, device=device)
    t.fill_(NAN_BITS[dtype])
    return t.view(dtype)


def _values(gen, shape, dtype, dist, device) -> torch.Tensor:
    x = torch.randn(shape, generator=gen, dtype=torch.float32, device=device)
    if dist == "round_normal":
        x = torch.round(x)
    return x.to(dtype)


def generate(*, seed: int, q_lens, kv_lens, num_heads: int, kv_num_heads: int, head_dim: int,
             query_form: str = "padded_bhnd", kv_form: str = "padded_bhnd",
             dtype=torch.float16, kv_dtype=None, n_q=None, n_kv=None, q_slack: int = 0,
             kv_slack: int = 0, pass_query_lengths=None, pass_kv_lengths=None,
             mask_kind: Optional[str] = None, mask_heads: int = 1, mask_p: float = 0.1,
             mask_value: float = -10000.0, mask_rank: int = 4, mask_diag_true: bool = False,
             causal_kind: str = "none", norm: str = "softmax", qdq: Optional[str] = None,
             qscale: float = 1.0, scale: Optional[float] = None, dist: str = "normal",
             kv_fp8_from: Optional[torch.dtype] = None, device="cpu", name="case",
             nan_padding: bool = True, tree: Optional[str] = None, page_size: int = 64,
             spare_pages: int = 3) -> Case:
    """Draw one operator instance.

    q_lens / kv_lens: per-sequence valid lengths (sequences of ints).
    n_q / n_kv: padded sizes (default: the max length).
    q_slack / kv_slack: extra NaN rows after the last packed row.
    mask_kind: None, 'bool', or an additive dtype name 'f16' | 'bf16' | 'f32'.
    kv_fp8_from: draw K/V in this dtype, then store them as E4M3FN with a
      per-tensor fp32 descale s = amax / 448 (the stored code is x / s).
    tree: draft-token parents for tree decoding, token-aligned with Q's rows
      (see ``tree_parents``); None for ordinary attention.
    kv_form "paged": K and V are drawn as padded [B, H_kv, n_kv, D], then
      scattered into two pools of pages [P, H_kv, page_size, D] in a random
      page order (separate for K and V), with ``spare_pages`` extra NaN
      pages; rows of a last page past the length are NaN, and page-table
      entries past a sequence's pages point at a NaN page.
    """
    kv_dtype = kv_dtype or dtype
    q_lens = np.asarray(q_lens, dtype=np.int64)
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    B = len(q_lens)
    assert len(kv_lens) == B
    D = head_dim
    n_q = int(n_q if n_q is not None else max(1, int(q_lens.max(initial=0))))
    n_kv = int(n_kv if n_kv is not None else max(1, int(kv_lens.max(initial=0))))
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    rng = np.random.Generator(np.random.PCG64(seed + 1_000_003))

    src_kv_dtype = kv_fp8_from if kv_fp8_from is not None else kv_dtype

    # Q
    if query_form == "packed_nhd":
        tq = int(q_lens.sum()) + q_slack
        q = _nan_fill((tq, num_heads, D), dtype, device) if nan_padding else torch.zeros(
            (tq, num_heads, D), dtype=dtype, device=device)
        off = 0
        for b in range(B):
            L = int(q_lens[b])
            if L:
                q[off:off + L] = _values(gen, (L, num_heads, D), dtype, dist, device)
            off += L
    else:
        q = _nan_fill((B, num_heads, n_q, D), dtype, device) if nan_padding else torch.zeros(
            (B, num_heads, n_q, D), dtype=dtype, device=device)
        for b in range(B):
            L = int(q_lens[b])
            if L:
                q[b, :, :L] = _values(gen, (num_heads, L, D), dtype, dist, device)

    # K, V (drawn in src dtype)
    def kv_tensor():
        if kv_form == "packed_nhd":
            tk = int(kv_lens.sum()) + kv_slack
            t = _nan_fill((tk, kv_num_heads, D), src_kv_dtype, device)
            off = 0
            for b in range(B):
                L = int(kv_lens[b])
                if L:
                    t[off:off + L] = _values(gen, (L, kv_num_heads, D), src_kv_dtype, dist, device)
                off += L
        else:
            t = _nan_fill((B, kv_num_heads, n_kv, D), src_kv_dtype, device)
            for b in range(B):
                L = int(kv_lens[b])
                if L:
                    t[b, :, :L] = _values(gen, (kv_num_heads, L, D), src_kv_dtype, dist, device)
        return t

    paged = kv_form == "paged"
    if paged:
        kv_form = "padded_bhnd"
        n_kv = -(-n_kv // page_size) * page_size  # whole pages
    k = kv_tensor()
    v = kv_tensor()
    k_descale = v_descale = 1.0
    if kv_fp8_from is not None:
        k, k_descale = _to_fp8_per_tensor(k, kv_form, kv_lens)
        v, v_descale = _to_fp8_per_tensor(v, kv_form, kv_lens)

    if query_form == "padded_bhnd" and pass_query_lengths is False:
        assert np.all(q_lens == n_q), "padded Q without query_lengths: every row is valid"
    if kv_form == "padded_bhnd" and pass_kv_lengths is False:
        assert np.all(kv_lens == n_kv), "padded KV without kv_lengths: every key is valid"

    # lengths
    ql_cum = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    kl_cum = np.concatenate([[0], np.cumsum(kv_lens)]).astype(np.int32)
    if pass_query_lengths is None:
        pass_query_lengths = query_form == "packed_nhd"
    if pass_kv_lengths is None:
        pass_kv_lengths = True
    query_lengths = torch.from_numpy(ql_cum).to(device) if pass_query_lengths else None
    kv_page_table = None
    if paged:
        k, v, kv_page_table = _to_pages(k, v, kv_lens, page_size, spare_pages, rng)
        kv_form = "paged"
        pass_kv_lengths = True
    if kv_form == "packed_nhd":
        kv_lengths = torch.from_numpy(kl_cum).to(device)
    else:
        kv_lengths = torch.from_numpy(kv_lens.astype(np.int32)).to(device) if pass_kv_lengths else None

    # mask
    mask = None
    if mask_kind is not None:
        full = (B, mask_heads, n_q if query_form == "padded_bhnd" else max(1, int(q_lens.max(initial=0))),
                n_kv if kv_form != "packed_nhd" else max(1, int(kv_lens.max(initial=0))))
        draw = rng.random(full)
        if mask_kind == "bool":
            m = draw >= mask_p  # True = may attend
            if mask_diag_true:
                n = min(full[2], full[3])
                idx = np.arange(n)
                m[:, :, idx, idx] = True
            mask = torch.from_numpy(m)
        else:
            mdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[mask_kind]
            m = np.where(draw < mask_p, np.float32(mask_value), np.float32(0.0))
            mask = torch.from_numpy(m).to(mdt)
        if mask_rank < 4:
            mask = mask.reshape(full[4 - mask_rank:]) if all(
                s == 1 for s in full[:4 - mask_rank]) else mask
        mask = mask.to(device)

    tree_parents = None
    if tree is not None:
        rows = int(q_lens.sum()) + q_slack if query_form == "packed_nhd" else B * n_q
        par = np.full(rows, -1, dtype=np.int32)
        for b in range(B):
            L = int(q_lens[b])
            row0 = int(ql_cum[b]) if query_form == "packed_nhd" else b * n_q
            par[row0:row0 + L] = tree_parents_for(rng, L, tree)
        tree_parents = torch.from_numpy(par).to(device)

    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out_dtype = torch.float16 if dtype == FP8 else dtype
    return Case(name=name, q=q, k=k, v=v, mask=mask, query_lengths=query_lengths,
                kv_lengths=kv_lengths, batch=B, query_form=query_form, kv_form=kv_form,
                causal_kind=causal_kind, norm=norm, qdq=qdq, qscale=float(qscale),
                scale=float(scale), k_descale=float(k_descale), v_descale=float(v_descale),
                num_heads=num_heads, kv_num_heads=kv_num_heads, q_lens=q_lens, kv_lens=kv_lens,
                out_dtype=out_dtype, meta=dict(seed=seed), tree_parents=tree_parents,
                kv_page_table=kv_page_table)


def _to_pages(k, v, kv_lens, ps: int, spare: int, rng):
    """Scatter padded K / V [B, H, n, D] (n a multiple of ps) into page pools
    [P, H, ps, D]: sequence b uses ceil(kv_len_b / ps) pages, K and V in
    independent random page orders; spare pages and the rows past a length
    stay NaN.  Returns (k_pool, v_pool, table [B, 2, max_pages] int32 on K's
    device)."""
    B, H, n, D = k.shape
    assert n % ps == 0
    npages = np.array([(int(L) + ps - 1) // ps for L in kv_lens], dtype=np.int64)
    used = int(npages.sum())
    P = used + spare
    max_pages = max(1, n // ps)
    poison = used  # first spare page: every unused table entry points at it
    table = np.full((B, 2, max_pages), poison, dtype=np.int32)
    b_idx = np.repeat(np.arange(B), npages)
    p_idx = np.concatenate([np.arange(c) for c in npages]) if used else np.zeros(0, np.int64)
    pools = []
    for w, src in enumerate((k, v)):
        pool = _nan_fill((P, H, ps, D), src.dtype, src.device)
        order = rng.permutation(used)
        table[b_idx, w, p_idx] = order
        if used:
            pages = src.view(B, H, n // ps, ps, D)
            bi = torch.from_numpy(b_idx).to(src.device)
            pi = torch.from_numpy(p_idx).to(src.device)
            flat = pool.view(torch.uint8) if src.dtype == FP8 else pool
            srcv = pages.view(torch.uint8) if src.dtype == FP8 else pages
            flat[torch.from_numpy(order).to(src.device)] = srcv[bi, :, pi]
        pools.append(pool)
    return pools[0], pools[1], torch.from_numpy(table).to(k.device)


def tree_parents_for(rng, n: int, kind: str) -> np.ndarray:
    """Parents of n draft tokens in topological order (parent < child; -1 =
    attached to the committed context).
      chain:  t - 1 (a single path: the ordinary causal case);
      star:   -1 for every token;
      random: uniform in [-1, t - 1];
      spec:   levels of growing width (1, 2, 4, 8, then 16 per level), each
              token's parent drawn from the previous level -- the shape of a
              speculative-decoding draft tree;
      bad:    random, with some parents out of range (>= t or < -1)."""
    t = np.arange(n)
    if kind == "chain":
        return (t - 1).astype(np.int32)
    if kind == "star":
        return np.full(n, -1, dtype=np.int32)
    if kind in ("random", "bad"):
        par = np.array([int(rng.integers(-1, i)) if i > 0 else -1 for i in range(n)], dtype=np.int32)
        if kind == "bad" and n:
            pick = rng.random(n) < 0.3
            junk = rng.integers(-5, n + 5, size=n).astype(np.int32)
            par = np.where(pick, junk, par).astype(np.int32)
        return par
    if kind == "spec":
        par = np.full(n, -1, dtype=np.int32)
        prev, start, width = [-1], 0, 1
        while start < n:
            level = list(range(start, min(n, start + width)))
            for i in level:
                par[i] = prev[int(rng.integers(0, len(prev)))]
            prev, start, width = level, start + len(level), min(16, width * 2)
        return par
    raise ValueError(kind)


def _to_fp8_per_tensor(x: torch.Tensor, form: str, lens) -> tuple[torch.Tensor, float]:
    """Store x as E4M3FN codes of x / s with s = fp32(amax(|x_valid|) / 448)."""
    amax = 0.0
    if form == "packed_nhd":
        n = int(np.sum(lens))
        if n:
            amax = float(x[:n].float().abs().max())
    else:
        for b, L in enumerate(lens):
            if L:
                amax = max(amax, float(x[b, :, :int(L)].float().abs().max()))
    s = float(np.float32(amax / 448.0)) if amax > 0 else 1.0
    out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    out.fill_(0x7F)  # NaN code in the padding
    out = out.view(FP8)
    if form == "packed_nhd":
        n = int(np.sum(lens))
        if n:
            out[:n] = (x[:n].float() / s).to(FP8)
    else:
        for b, L in enumerate(lens):
            L = int(L)
            if L:
                out[b, :, :L] = (x[b, :, :L].float() / s).to(FP8)
    return out, s


# --------------------------------------------------------------------------
# The five workload configurations (LLM-shaped prefill, chunked context,
# decode and quantized attention), at their full sizes.
# --------------------------------------------------------------------------
CONFIGS = ("1", "2", "3", "4a", "4b", "4p", "5a", "5b", "tree")

DESCRIPTIONS = {
    "1": "tiny padded MHA fp16 B=2 H=4 N=128 D=64",
    "2": "packed ragged causal GQA prefill bf16 B=16 L~U[64,2048] Hq=32 Hkv=8 D=128",
    "3": "packed Q / padded KV chunked context fp16 B=8 q~U[1,512] Nkv=8192 + additive mask",
    "4a": "decode fp16 KV B=128 Nkv=32768 kv~U[512,32768] Hq=32 Hkv=8 D=128",
    "4b": "decode fp8 e4m3 KV (per-tensor fp32 descale) B=128 Nkv=32768 Hq=32 Hkv=8 D=128",
    "4p": "decode fp16 KV in 64-key pages (paged KV) B=128 kv~U[512,32768] Hq=32 Hkv=8 D=128",
    "5a": "quantized attention fp8 Q/K/V B=4 N=4096 Hq=32 Hkv=8 D=128 causal, P fp8 Q/DQ 1/448",
    "5b": "quantized attention as 5a plus bool mask [4,1,4096,4096] 90% true",
    "tree": ("tree (speculative) decoding fp16 B=32, 64 draft tokens per sequence in a "
             "1-2-4-8-16-wide tree, context U[1024,8192], Hq=32 Hkv=8 D=128"),
}


def config_lengths(cfg: str):
    """(q_lens, kv_lens) of a configuration (drawn first from its seed)."""
    seed = {"1": 1, "2": 2, "3": 3, "4a": 4, "4b": 4, "4p": 4, "5a": 5, "5b": 5, "tree": 6}[cfg]
    rng = np.random.Generator(np.random.PCG64(seed))
    if cfg == "1":
        return np.full(2, 128), np.full(2, 128)
    if cfg == "2":
        L = rng.integers(64, 2049, size=16)
        return L, L.copy()
    if cfg == "3":
        q = rng.integers(1, 513, size=8)
        kv = np.array([rng.integers(int(a), 8193) for a in q])
        return q, kv
    if cfg in ("4a", "4b", "4p"):
        kv = rng.integers(512, 32769, size=128)
        return np.ones(128, dtype=np.int64), kv
    if cfg == "tree":
        ctx = rng.integers(1024, 8193, size=32)
        return np.full(32, 64), ctx + 64
    return np.full(4, 4096), np.full(4, 4096)


def make_config(cfg: str, device="cpu") -> Case:
    """One of the workload configurations, at full size, on ``device``."""
    q_lens, kv_lens = config_lengths(cfg)
    if cfg == "1":
        return generate(seed=1, q_lens=q_lens, kv_lens=kv_lens, num_heads=4, kv_num_heads=4,
                        head_dim=64, dtype=torch.float16, scale=1.0 / 8.0, pass_kv_lengths=False,
                        device=device, name="cfg1")
    if cfg == "2":
        return generate(seed=2, q_lens=q_lens, kv_lens=kv_lens, num_heads=32, kv_num_heads=8,
                        head_dim=128, query_form="packed_nhd", kv_form="packed_nhd",
                        dtype=torch.bfloat16, causal_kind="lower_right", device=device,
                        name="cfg2")
    if cfg == "3":
        return generate(seed=3, q_lens=q_lens, kv_lens=kv_lens, num_heads=32, kv_num_heads=8,
                        head_dim=128, query_form="packed_nhd", kv_form="padded_bhnd", n_kv=8192,
                        dtype=torch.float16, causal_kind="lower_right", mask_kind="f16",
                        mask_p=0.1, mask_value=-10000.0, device=device, name="cfg3")
    if cfg == "tree":
        # the 64 drafts' keys are the last 64 valid KV rows of each sequence
        return generate(seed=6, q_lens=q_lens, kv_lens=kv_lens, num_heads=32, kv_num_heads=8,
                        head_dim=128, n_q=64, n_kv=8192 + 64, dtype=torch.float16,
                        tree="spec", device=device, name="cfgtree")
    if cfg == "4p":
        return generate(seed=4, q_lens=q_lens, kv_lens=kv_lens, num_heads=32, kv_num_heads=8,
                        head_dim=128, n_q=1, n_kv=32768, dtype=torch.float16, kv_form="paged",
                        page_size=64, pass_query_lengths=False, device=device, name="cfg4p")
    if cfg in ("4a", "4b"):
        return generate(seed=4, q_lens=q_lens, kv_lens=kv_lens, num_heads=32, kv_num_heads=8,
                        head_dim=128, n_q=1, n_kv=32768, dtype=torch.float16,
                        kv_fp8_from=torch.float16 if cfg == "4b" else None,
                        kv_dtype=FP8 if cfg == "4b" else None, pass_query_lengths=False,
                        device=device, name="cfg" + cfg)
    return generate(seed=5, q_lens=q_lens, kv_lens=kv_lens, num_heads=32, kv_num_heads=8,
                    head_dim=128, dtype=FP8, dist="round_normal", causal_kind="upper_left",
                    qdq="fp8", qscale=float(np.float32(1.0 / 448.0)), pass_kv_lengths=False,
                    mask_kind="bool" if cfg == "5b" else None, mask_p=0.1, mask_diag_true=True,
                    device=device, name="cfg" + cfg)


# ------------------------------------------------------------ KV-cache update
@dataclass
class KvUpdateCase:
    name: str
    past_cache: torch.Tensor            # [B, H, N, D]
    update: torch.Tensor                # padded [B, H, N_u, D] or packed [T, H, D]
    write_indices: Optional[torch.Tensor]
    update_lengths: Optional[torch.Tensor]
    update_form: str
    counts: np.ndarray                  # rows each sequence writes (before dropping)
    starts: np.ndarray                  # write index of each sequence

    def kwargs(self) -> dict:
        return dict(write_indices=self.write_indices, update_lengths=self.update_lengths,
                    update_form=self.update_form)


def kv_update_case(*, seed: int, B: int, H: int, N: int, D: int, counts, starts=None,
                   update_form: str = "padded_bhnd", dtype=torch.float16, pass_lengths=True,
                   pass_indices=True, n_u=None, slack: int = 0, device="cpu",
                   name: str = "kvu") -> KvUpdateCase:
    """A seeded cache and update: counts[b] rows for sequence b written from
    starts[b] (drawn in [0, N - counts[b]] when None).  Padded updates carry
    NaN-free random rows everywhere (rows past counts[b] must not be used);
    packed updates carry `slack` extra rows at the end."""
    rng = np.random.default_rng(seed)
    counts = np.asarray(counts, dtype=np.int64)
    if starts is None:
        starts = np.array([int(rng.integers(0, max(N - c, 0) + 1)) for c in counts], dtype=np.int64)
    starts = np.asarray(starts, dtype=np.int64)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)

    def rand(shape):
        x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        return x.to(dtype)

    cache = rand((B, H, N, D))
    if update_form == "packed_nhd":
        upd = rand((int(counts.sum()) + slack, H, D))
    else:
        nu = int(counts.max(initial=0)) if n_u is None else n_u
        upd = rand((B, H, nu, D))
    ul = None
    if pass_lengths or update_form == "packed_nhd":
        ul = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device=device)
    wi = torch.tensor(starts, dtype=torch.int32, device=device) if pass_indices else None
    return KvUpdateCase(name=name, past_cache=cache, update=upd, write_indices=wi, update_lengths=ul,
                        update_form=update_form, counts=counts,
                        starts=starts if pass_indices else np.zeros(B, np.int64))


KV_UPDATE_DESCRIPTION = ("KV-cache update, packed bf16 rows of 16 sequences L~U[64,2048] written "
                         "in place into a padded [16, 8, 4096, 128] cache at random offsets")


def make_kv_update_workload(device="cpu") -> KvUpdateCase:
    """The prefill workload's K written into a cache: 16 sequences, lengths of
    the prefill workload, H=8, D=128, bf16, cache length 4096."""
    q_lens, _ = config_lengths("2")
    return kv_update_case(seed=21, B=16, H=8, N=4096, D=128, counts=q_lens,
                          update_form="packed_nhd", dtype=torch.bfloat16, device=device,
                          name="kvu")
