"""GPU-vs-oracle comparison helpers used by the GPU tests, the smoke check and
the bench.  The oracle runs on host copies of exactly the bytes the GPU read.

Parity rule (per output element of a valid row):
    |Y_gpu - O| <= max(tol, ulp_out(|O|)) + A
with O the oracle's fp64 value, A its Q/DQ ambiguity bound, tol 2e-3 for an
f16 output, 1e-2 for bf16, 3e-2 whenever the scores are quantized, and
ulp_out the spacing of the output dtype at |O| (output rounding alone can
exceed tol for large |O|; the number of elements that needed it is
reported).  Rows that are not valid must keep the output's sentinel bits.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from gqa_attention_ragged_amd import capi, synth

TOL = {torch.float16: 2e-3, torch.bfloat16: 1e-2}
QDQ_TOL = 3e-2


def tolerance(case) -> float:
    return QDQ_TOL if case.qdq else TOL[case.out_dtype]


def run_gpu(case, out=None, sentinel=True):
    """Run the HIP path on a device case; returns the output tensor."""
    if out is None:
        out = synth.sentinel_like(case.q.shape, case.out_dtype, case.q.device) if sentinel else None
    out = capi.attn_forward(case.q, case.k, case.v, case.mask, out=out, **case.kwargs())
    torch.cuda.synchronize()
    return out


def subcase(case, bs):
    """Host copy of the case restricted to the sequences in bs (re-packed)."""
    c = case
    bs = list(bs)

    def take(t, form, lens):
        if form == "packed_nhd":
            starts = np.concatenate([[0], np.cumsum(lens)])
            return torch.cat([t[int(starts[b]):int(starts[b] + lens[b])].cpu() for b in bs])
        return torch.stack([t[b].cpu() for b in bs])

    q = take(c.q, c.query_form, c.q_lens)
    table = None
    if c.kv_form == "paged":
        # the sequences' own pages only, renumbered in a compact pool
        ps = c.k.shape[2]
        tab = c.kv_page_table.cpu()
        table = torch.zeros((len(bs), 2, tab.shape[2]), dtype=torch.int32)
        pools = []
        for w, src in enumerate((c.k, c.v)):
            ids = []
            for n, b in enumerate(bs):
                cnt = (int(c.kv_lens[b]) + ps - 1) // ps
                table[n, w, :cnt] = torch.arange(len(ids), len(ids) + cnt, dtype=torch.int32)
                ids += [int(x) for x in tab[b, w, :cnt]]
            if not ids:
                ids = [0]
            pools.append(src[torch.tensor(ids, device=src.device)].cpu())
        k, v = pools
    else:
        k = take(c.k, c.kv_form, c.kv_lens)
        v = take(c.v, c.kv_form, c.kv_lens)
    mask = None
    if c.mask is not None:
        m = c.mask
        if m.dim() == 4 and m.shape[0] != 1:
            mask = torch.stack([m[b].cpu() for b in bs])
        else:
            mask = m.cpu()
    ql = np.asarray([c.q_lens[b] for b in bs])
    kl = np.asarray([c.kv_lens[b] for b in bs])
    query_lengths = None
    if c.query_lengths is not None:
        query_lengths = torch.from_numpy(np.concatenate([[0], np.cumsum(ql)]).astype(np.int32))
    kv_lengths = None
    if c.kv_form == "packed_nhd":
        kv_lengths = torch.from_numpy(np.concatenate([[0], np.cumsum(kl)]).astype(np.int32))
    elif c.kv_lengths is not None:
        kv_lengths = torch.from_numpy(kl.astype(np.int32))
    tree = None
    if c.tree_parents is not None:  # token-aligned with Q's rows
        tp = c.tree_parents.cpu()
        if c.query_form == "packed_nhd":
            starts = np.concatenate([[0], np.cumsum(c.q_lens)])
            tree = torch.cat([tp[int(starts[b]):int(starts[b] + c.q_lens[b])] for b in bs])
        else:
            n_q = c.q.shape[2]
            tree = torch.cat([tp[b * n_q:(b + 1) * n_q] for b in bs])
    sub = synth.Case(**{f: getattr(c, f) for f in c.__dataclass_fields__})
    sub.q, sub.k, sub.v, sub.mask = q, k, v, mask
    sub.tree_parents = tree
    sub.kv_page_table = table
    sub.query_lengths, sub.kv_lengths = query_lengths, kv_lengths
    sub.batch = len(bs)
    sub.q_lens, sub.kv_lens = ql, kl
    return sub


def _ulp(x: np.ndarray, dtype) -> np.ndarray:
    ax = np.abs(x)
    if dtype == torch.float16:
        return np.spacing(ax.astype(np.float16)).astype(np.float64)
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def gpu_rows(case, out_host: torch.Tensor, rows: np.ndarray) -> np.ndarray:
    """Output rows (b, h, i) of a host copy of the GPU output, as float64."""
    b, h, i = rows[:, 0], rows[:, 1], rows[:, 2]
    if case.query_form == "packed_nhd":
        starts = np.concatenate([[0], np.cumsum(case.q_lens)]).astype(np.int64)
        return out_host[torch.from_numpy(starts[b] + i), torch.from_numpy(h)].double().numpy()
    return out_host[torch.from_numpy(b), torch.from_numpy(h), torch.from_numpy(i)].double().numpy()


def sample_rows(case, n_per_seq: int, seed: int = 0) -> np.ndarray:
    """Valid rows (b, h, i): per sequence the first and last row plus random ones."""
    rng = np.random.default_rng(seed)
    out = []
    for b in range(case.batch):
        L = int(case.q_lens[b])
        if L == 0:
            continue
        cand = {0, L - 1, L // 2}
        cand |= set(int(x) for x in rng.integers(0, L, size=n_per_seq))
        for i in sorted(cand):
            out.append((b, int(rng.integers(0, case.num_heads)), i))
            out.append((b, case.num_heads - 1, i))
    return np.asarray(out, dtype=np.int32).reshape(-1, 3)


def compare(case, out: torch.Tensor, rows=None, amb_rel=1e-5, check_untouched=True):
    """Check a GPU output against the oracle.  rows=None checks every valid
    row (small cases); otherwise only the given rows (b, h, i).  Returns a
    dict of statistics; raises AssertionError on any violation."""
    out_host = out.cpu()
    if rows is None:
        host = case.to_host()
        res = oracle.attention(host.q, host.k, host.v, host.mask, amb_rel=amb_rel, **host.kwargs())
        rows_all = res.rows
        ref, amb = res.out, res.amb
    else:
        rows_all = np.asarray(rows, dtype=np.int32)
        ref = np.zeros((len(rows_all), case.q.shape[-1]))
        amb = np.zeros_like(ref)
        for b in np.unique(rows_all[:, 0]):
            sel = rows_all[:, 0] == b
            sub = subcase(case, [int(b)])
            r = rows_all[sel].copy()
            r[:, 0] = 0
            res = oracle.attention(sub.q, sub.k, sub.v, sub.mask, amb_rel=amb_rel, **sub.kwargs(),
                                   rows=r)
            ref[sel], amb[sel] = res.out, res.amb
    got = gpu_rows(case, out_host, rows_all)
    tol = tolerance(case)
    lim = np.maximum(tol, _ulp(ref, case.out_dtype)) + amb
    err = np.abs(got - ref)
    bad = ~(err <= lim)  # NaN counts as bad
    stats = dict(rows=int(len(rows_all)), max_err=float(np.nanmax(err)) if err.size else 0.0,
                 tol=tol, ulp_relaxed=int(np.sum((err > tol) & ~bad)),
                 amb_elems=int(np.sum(amb > 0)))
    if bad.any():
        k = np.argwhere(bad)[0]
        raise AssertionError(
            f"{case.name}: {int(bad.sum())} elements out of tolerance; first at row "
            f"{rows_all[k[0]].tolist()} d={k[1]}: gpu={got[k[0], k[1]]!r} oracle={ref[k[0], k[1]]!r} "
            f"lim={lim[k[0], k[1]]!r} stats={stats}")
    if check_untouched and rows is None:
        stats["untouched_ok"] = untouched_ok(case, out_host, rows_all)
        assert stats["untouched_ok"], f"{case.name}: a padding row of the output was written"
    return stats


def untouched_ok(case, out_host: torch.Tensor, rows: np.ndarray) -> bool:
    """Every output row that is not valid still holds the sentinel bits."""
    bits = synth.SENTINEL_BITS[case.out_dtype]
    raw = out_host.view(torch.int16 if case.out_dtype != torch.float32 else torch.int32)
    raw = raw.to(torch.int64) & 0xFFFF
    written = torch.zeros(raw.shape[:-1], dtype=torch.bool)
    b, h, i = (torch.from_numpy(rows[:, c].astype(np.int64)) for c in range(3))
    if case.query_form == "packed_nhd":
        starts = torch.from_numpy(np.concatenate([[0], np.cumsum(case.q_lens)]).astype(np.int64))
        written[starts[b] + i, h] = True
    else:
        written[b, h, i] = True
    untouched = raw[~written]
    return bool(torch.all(untouched == bits))
