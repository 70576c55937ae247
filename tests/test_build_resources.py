"""Resources of the built kernels (from the compiler's per-kernel report,
recorded by the build): no kernel uses scratch memory.  The key loops wait
for their direct-to-LDS tile copies with hand-placed vmcnt waits; scratch
loads would share that counter, and a spilled kernel state once produced
wrong results that way, so scratch is kept out of every kernel."""
import json
import os

import pytest

from gqa_attention_ragged_amd import build


def _resources():
    if not os.path.exists(build.RESOURCES):
        pytest.fail("build the library first (its kernel resource report is missing)")
    with open(build.RESOURCES) as f:
        return json.load(f)


def test_every_kernel_is_reported():
    ks = _resources()
    names = {k["kernel"] for k in ks}
    assert any("prefill_kernel" in n for n in names)
    assert any("decode_split_kernel" in n for n in names)
    assert any("length_check_kernel" in n for n in names)
    assert len(ks) >= 100, len(ks)


def test_no_kernel_uses_scratch():
    bad = [(k["kernel"], k.get("scratch"), k.get("vgpr_spill"), k.get("sgpr_spill"))
           for k in _resources() if k.get("scratch", 0) != 0 or k.get("vgpr_spill", 0) != 0]
    assert not bad, bad
