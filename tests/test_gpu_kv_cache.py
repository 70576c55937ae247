"""GPU parity of the KV-cache update (TRT_KVCacheUpdate) through the C ABI:
bit-exact against the CPU oracle (oracle/kv_cache.py) on the whole cache,
in place and out of place, padded and packed updates, every element type,
ragged and empty lengths, rows that fall outside the cache, strided caches."""
import numpy as np
import pytest
import torch

from gqa_attention_ragged_amd import capi, synth
from oracle import kv_cache as kvo

pytestmark = pytest.mark.gpu
DEV = "cuda"
DTYPES = [torch.float16, torch.bfloat16, torch.float8_e4m3fn]


def _bits(t):
    es = t.element_size()
    return t.detach().cpu().contiguous().view({1: torch.uint8, 2: torch.int16}[es]).numpy()


def _run(c, in_place=True):
    before = c.past_cache.clone()
    out = None if in_place else torch.empty_like(c.past_cache)
    y = capi.kv_cache_update(c.past_cache, c.update, out=out, **c.kwargs())
    torch.cuda.synchronize()
    expect = kvo.kv_cache_update(before, c.update, **{k: (None if v is None else v.cpu()) if k != "update_form" else v
                                                      for k, v in c.kwargs().items()})
    assert np.array_equal(_bits(y), expect)
    if not in_place:  # the cache itself is left as it was
        assert torch.equal(c.past_cache.view(torch.uint8), before.view(torch.uint8))
    return y


@pytest.mark.parametrize("form", ["padded_bhnd", "packed_nhd"])
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("in_place", [True, False])
def test_ragged_update(form, dtype, in_place):
    seed = 3000 + DTYPES.index(dtype) * 4 + (form == "packed_nhd") * 2 + in_place
    rng = np.random.default_rng(seed)
    counts = rng.integers(0, 40, size=5)
    counts[1] = 0
    c = synth.kv_update_case(seed=seed, B=5, H=3, N=96, D=128, counts=counts, update_form=form,
                             dtype=dtype, slack=3, device=DEV, name=f"ragged-{form}")
    _run(c, in_place)


@pytest.mark.parametrize("dtype", DTYPES)
def test_rows_outside_the_cache_are_dropped(dtype):
    counts = [10, 7, 4, 1]
    starts = [90, -3, 95, 99]  # N = 100: tails and heads fall outside
    c = synth.kv_update_case(seed=3100 + DTYPES.index(dtype), B=4, H=2, N=100, D=64, counts=counts,
                             starts=starts, update_form="packed_nhd", dtype=dtype, device=DEV)
    _run(c)


def test_no_indices_no_lengths_whole_padded_update():
    c = synth.kv_update_case(seed=3200, B=3, H=4, N=50, D=128, counts=[6, 6, 6], starts=[0, 0, 0],
                             pass_lengths=False, pass_indices=False, device=DEV)
    _run(c)


def test_decode_step_one_token_per_sequence():
    rng = np.random.default_rng(3300)
    B, N = 64, 2048
    counts = np.ones(B, dtype=np.int64)
    starts = rng.integers(0, N, size=B)
    c = synth.kv_update_case(seed=3300, B=B, H=8, N=N, D=128, counts=counts, starts=starts,
                             dtype=torch.bfloat16, device=DEV)
    _run(c)


def test_strided_cache_view():
    # the cache is a view into a longer buffer (sequence stride > N * D)
    c = synth.kv_update_case(seed=3400, B=3, H=2, N=40, D=64, counts=[5, 9, 0], device=DEV)
    big = torch.zeros(3, 2, 48, 64, dtype=c.past_cache.dtype, device=DEV)
    big[:, :, :40] = c.past_cache
    c.past_cache = big[:, :, :40]
    _run(c)
    assert torch.count_nonzero(big[:, :, 40:].float()) == 0  # outside the view untouched


def test_workload_full():
    c = synth.make_kv_update_workload(device=DEV)
    _run(c)
