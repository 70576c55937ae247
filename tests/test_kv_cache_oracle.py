"""Pins of the KV-cache update oracle (oracle/kv_cache.py) on the CPU:
hand-derived golden cases, an independent gather formulation on random
shapes, packed = padded, and the no-op / out-of-range cases."""
import json
import os

import numpy as np
import pytest

from oracle import kv_cache as kvo

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_cache_update.json")


def _cache(B, H, N, D):
    b, h, n, d = np.meshgrid(np.arange(B), np.arange(H), np.arange(N), np.arange(D), indexing="ij")
    return (1000 * b + 100 * h + 10 * n + d).astype(np.int32)


def _update(B, H, Nu, D):
    return -_cache(B, H, Nu, D) - 1


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_golden(case):
    B, H, N, D = case["B"], case["H"], case["N"], case["D"]
    nu = int(case["update_padded"].split("shape [")[1].split(",")[2])
    cache, upd = _cache(B, H, N, D), _update(B, H, nu, D)
    wi = None if case["write_indices"] is None else np.array(case["write_indices"], np.int32)
    ul = None if case["update_lengths"] is None else np.array(case["update_lengths"], np.int32)
    y = kvo.kv_cache_update(cache, upd, write_indices=wi, update_lengths=ul)
    expect = cache.copy()
    for b, pos, t in case["overwritten"]:
        expect[b, :, pos, :] = upd[b, :, t, :]
    assert np.array_equal(y, expect)
    # the packed form of the same update gives the same cache
    if ul is not None:
        rows = [upd[b, :, t, :] for b in range(B) for t in range(int(ul[b + 1] - ul[b]))]
        packed = np.stack(rows) if rows else np.zeros((0, H, D), np.int32)
        yp = kvo.kv_cache_update(cache, packed, write_indices=wi, update_lengths=ul,
                                 update_form="packed_nhd")
        assert np.array_equal(yp, expect)


def _gather_reference(cache, upd, wi, counts, firsts, packed):
    """Y by gathering: for every (b, n) the source row index t = n - w_b
    selects the update when 0 <= t < L_b, else the cache."""
    B, H, N, D = cache.shape
    y = np.empty_like(cache)
    for b in range(B):
        t = np.arange(N) - (0 if wi is None else int(wi[b]))
        take = (t >= 0) & (t < counts[b])
        y[b] = cache[b]
        if take.any():
            src = upd[firsts[b] + t[take]].transpose(1, 0, 2) if packed else upd[b][:, t[take], :]
            y[b][:, take, :] = src
    return y


@pytest.mark.parametrize("seed", range(8))
def test_matches_gather_formulation(seed):
    rng = np.random.default_rng(1000 + seed)
    B, H, N, D = int(rng.integers(1, 5)), int(rng.integers(1, 4)), int(rng.integers(1, 12)), 3
    cache = rng.integers(-2**15, 2**15, size=(B, H, N, D)).astype(np.int16)
    counts = rng.integers(0, N + 3, size=B)
    ul = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    wi = rng.integers(-3, N + 2, size=B).astype(np.int32)
    packed_upd = rng.integers(-2**15, 2**15, size=(int(ul[-1]), H, D)).astype(np.int16)
    y = kvo.kv_cache_update(cache, packed_upd, write_indices=wi, update_lengths=ul,
                            update_form="packed_nhd")
    assert np.array_equal(y, _gather_reference(cache, packed_upd, wi, counts, ul[:-1], True))
    nu = int(counts.max(initial=0))
    pad = rng.integers(-2**15, 2**15, size=(B, H, nu, D)).astype(np.int16)
    for b in range(B):
        pad[b, :, :counts[b], :] = packed_upd[ul[b]:ul[b + 1]].transpose(1, 0, 2)
    yp = kvo.kv_cache_update(cache, pad, write_indices=wi, update_lengths=ul)
    assert np.array_equal(yp, y)


def test_empty_update_is_identity():
    rng = np.random.default_rng(7)
    cache = rng.integers(0, 255, size=(3, 2, 6, 4)).astype(np.uint8)
    ul = np.zeros(4, np.int32)
    y = kvo.kv_cache_update(cache, np.zeros((0, 2, 4), np.uint8), write_indices=np.array([0, 2, 5]),
                            update_lengths=ul, update_form="packed_nhd")
    assert np.array_equal(y, cache)


def test_torch_fp8_bits_are_copied_exactly():
    import torch
    c = torch.randn(2, 2, 4, 8).to(torch.float8_e4m3fn)
    u = torch.randn(2, 2, 1, 8).to(torch.float8_e4m3fn)
    y = kvo.kv_cache_update(c, u, write_indices=np.array([3, 0], np.int32))
    assert y.dtype == np.uint8
    cb, ub = c.view(torch.uint8).numpy(), u.view(torch.uint8).numpy()
    assert np.array_equal(y[0, :, 3], ub[0, :, 0]) and np.array_equal(y[1, :, 0], ub[1, :, 0])
    assert np.array_equal(y[0, :, :3], cb[0, :, :3]) and np.array_equal(y[1, :, 1:], cb[1, :, 1:])
